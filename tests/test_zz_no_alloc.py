"""paged_attn_decode_noalloc (the decode call on the library's own scratch
array, for callers that cannot allocate) against paged_attn_decode with a
caller workspace: identical bits on two calls in a row, the second with a
smaller batch (the scratch then still holds the first call's partials), and
the oracle on both; with 64 query heads (eight per KV head) the first call
runs on the row-tile kernel (its partials in the scratch) and the second on
the MFMA tile form, split over the keys with its partials in the scratch. (A launch needing more than the scratch is rejected on the
host; on a 256-CU GPU no supported shape does: the row-wide kernel needs at
most about 34 MB with 32 query heads, the tile form's partials about 6.5 MB.)"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from paged_kv_attention_28_amd import binding as B
from paged_kv_attention_28_amd import harness as H
from tests import oracle_side as O
from tests.test_gpu_parity import assert_close, custom

pytestmark = pytest.mark.gpu


def _decode_case(lens, hq, seed):
    w = custom(lens, [L - 1 for L in lens], hq=hq, kind="decode", seed=seed)
    dw = H.DeviceWorkload(w).build()
    p = w.passes[0]
    q, m = dw.pass_inputs(p)
    return w, dw, p, q, m


def _both(w, dw, q, m):
    ws = H.decode_workspace(w, q.shape[0], m.max_context_len)
    ref = torch.full_like(q, float("nan"))
    B.paged_attn_decode(ref, q, dw.k_cache, dw.v_cache, m.block_tables, m.context_lens, w.scale, m.max_context_len,
                        ws)
    got = torch.full_like(q, float("nan"))
    B.paged_attn_decode_noalloc(got, q, dw.k_cache, dw.v_cache, m.block_tables, m.context_lens, w.scale,
                                m.max_context_len)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("hq", [16, 32, 64])
def test_noalloc_matches_workspace_call_twice(hq):
    rng = np.random.default_rng(60 + hq)
    big = [int(x) for x in rng.integers(1, 3000, size=300)]
    small = [1, 700, 2049, 5000, 33]
    first = _decode_case(big, hq, seed=61)
    print(f"[noalloc] H_q {hq}: first call, {len(big)} sequences", flush=True)
    w, dw, p, q, m = first
    ref, got = _both(w, dw, q, m)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "first call differs"
    kc, vc = O.build_caches(w, device="cuda")
    assert_close(got, O.run_pass(w, p, kc, vc, q=q), None, f"noalloc H_q {hq}")
    del dw
    print(f"[noalloc] H_q {hq}: second call, {len(small)} sequences", flush=True)
    w, dw, p, q, m = _decode_case(small, hq, seed=62)
    ref, got = _both(w, dw, q, m)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "second (smaller) call differs"
    kc, vc = O.build_caches(w, device="cuda")
    assert_close(got, O.run_pass(w, p, kc, vc, q=q), None, f"noalloc H_q {hq}, small batch")
