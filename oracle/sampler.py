"""Oracle for the temperature sampler that follows a decode step.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check and
the CPU-baseline leg of the benchmark may call this module.

P1 = "13. 读一个最小推理引擎：nano-vllm", "它省略了什么" and "第一站：主循环": the
sampler uses temperature only (no top-k / top-p; temperature 0 is not
allowed) and draws a token as the argmax of the probabilities divided by
independent Exp(1) noise, which has the distribution of a multinomial draw
from those probabilities.

Two functions:

* ``sample_exact``: the definition, in fp64: argmax_j softmax(l / T)_j / E_j.
* ``sample_decision``: the same choice made the way the kernel makes it, in
  fp32, from the equivalent log form (the Gumbel-max form: log of a softmax
  differs from l / T by a per-row constant, and -ln E_j is the noise):
      key_j = fp32( fp32(l_j * fp32(1 / T)) + g_j ),   g_j = -ln E_j,
  token = the smallest j with the largest key. Every operation is a single
  correctly rounded fp32 operation, so numpy reproduces the kernel's keys
  bit for bit and the integer decision is taken in the same precision on
  both sides. The noise g is an input (random draws are passed in).

Pins (tests/test_sampler.py): the two functions agree except where the two
best fp64 keys are closer than fp32 rounding can resolve; with the noise
drawn many times the token frequencies follow softmax(l / T); zero noise
gives the plain argmax; a very small temperature gives the plain argmax.
"""

from __future__ import annotations

import numpy as np


def sample_exact(logits, temperatures, exp_noise) -> np.ndarray:
    """argmax_j softmax(l / T)_j / E_j per row, all in fp64."""
    l = np.asarray(logits, dtype=np.float64)
    t = np.asarray(temperatures, dtype=np.float64)[:, None]
    z = l / t
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    return np.argmax(p / np.asarray(exp_noise, dtype=np.float64), axis=1).astype(np.int32)


def decision_keys(logits, temperatures, gumbel) -> np.ndarray:
    """fp32 keys fp32(fp32(l * fp32(1 / T)) + g)."""
    l = np.asarray(logits, dtype=np.float32)
    inv = (np.float32(1.0) / np.asarray(temperatures, dtype=np.float32))[:, None]
    prod = (l * inv).astype(np.float32)
    return (prod + np.asarray(gumbel, dtype=np.float32)).astype(np.float32)


def sample_decision(logits, temperatures, gumbel) -> np.ndarray:
    """Smallest index of the largest fp32 key per row (np.argmax returns the first maximum)."""
    return np.argmax(decision_keys(logits, temperatures, gumbel), axis=1).astype(np.int32)
