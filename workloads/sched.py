"""Configuration 5 inputs: seeded request lengths and the replay's sizes.

256 token-free requests whose prompt and output lengths are drawn uniformly
from [100, 1024]; the scheduler that turns them into steps is part of the
path (the library's native scheduler) and has its own oracle. This module
holds only the seeded draws, the configuration's limits and the random-stream
id of each (step, layer)'s q/k/v.
"""

from __future__ import annotations

import numpy as np

from . import SEEDS

MAX_NUM_SEQS = 512
MAX_BATCHED_TOKENS = 16384
NUM_LAYERS = 28
NUM_REQUESTS = 256
POOL_BLOCKS = 800  # per layer; small enough that the replay preempts (23 times at seed 4)


def requests(seed: int = SEEDS[5], num_requests: int = NUM_REQUESTS, lo: int = 100, hi: int = 1024):
    """(prompt_lens, output_lens), each int array of num_requests draws in [lo, hi]."""
    rng = np.random.default_rng(seed)
    prompts = rng.integers(lo, hi + 1, size=num_requests)
    outputs = rng.integers(lo, hi + 1, size=num_requests)
    return prompts, outputs


def step_stream(step: int, layer: int) -> int:
    """Random-stream id of a (step, layer) pair's q/k/v."""
    return 1_000_000 + step * 64 + layer
