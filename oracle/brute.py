"""Scalar brute-force attention for tiny inputs (pure Python floats and math.exp).

TEST INFRASTRUCTURE. An independent second form of the oracle's attention: no
numpy, no vectorisation, explicit loops over sequences, heads, queries, keys
and dimensions, with the block table walked one position at a time. It exists
to pin ``oracle.paged`` on tiny shapes (generic block size, head dim and head
counts); it is too slow for anything else.

Page references: P1 = "13. 读一个最小推理引擎：nano-vllm" ("第二站" for
num_cached_tokens, "第五站" for the slot formula, "第六站" for reading the
context through the block table).
"""

from __future__ import annotations

import math
import struct


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def brute_paged_attention(q_bits, q_pos, seq_of_query, cache_k_bits, cache_v_bits,
                          tables, block_size, num_q_heads, num_kv_heads, head_dim,
                          scale):
    """Return nested lists out[i][h][d] for every query row i.

    q_bits[i][h][d]: bf16 bits of query row i; q_pos[i]: its absolute
    position; seq_of_query[i]: its sequence. cache_*_bits[blk][off][g][d]:
    bf16 bits. tables[b]: physical blocks of sequence b.
    """
    group = num_q_heads // num_kv_heads
    out = []
    for i in range(len(q_bits)):
        b = seq_of_query[i]
        p = q_pos[i]
        row = []
        for h in range(num_q_heads):
            g = h // group
            scores = []
            for j in range(p + 1):
                blk = tables[b][j // block_size]
                off = j % block_size
                acc = 0.0
                for d in range(head_dim):
                    acc += _bf16(q_bits[i][h][d]) * _bf16(cache_k_bits[blk][off][g][d])
                scores.append(scale * acc)
            top = max(scores)
            weights = [math.exp(s - top) for s in scores]
            total = sum(weights)
            vec = []
            for d in range(head_dim):
                acc = 0.0
                for j in range(p + 1):
                    blk = tables[b][j // block_size]
                    off = j % block_size
                    acc += weights[j] * _bf16(cache_v_bits[blk][off][g][d])
                vec.append(acc / total)
            row.append(vec)
        out.append(row)
    return out
