"""Brute-force attention for tiny inputs: numpy fp64, pure-Python loops over tokens.

TEST INFRASTRUCTURE ONLY (part of the oracle; see ``oracle/__init__.py``).

An implementation separate from ``pa_oracle.c``: it widens stored values with numpy's own
casts instead of decoding bit fields, walks the block table position by position, and
takes the softmax with ``scipy.special.softmax``.  It follows the same definition (plain
attention over the logical sequence, a sliding window keeping the last W positions, query
head h reading KV head h // (Hq / Hkv)).
"""
from __future__ import annotations

import numpy as np
from scipy.special import softmax


def widen_np(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def paged_attention(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype, num_q_heads,
                    query_start_loc=None, window=0):
    kc = widen_np(k_cache, dtype)
    vc = widen_np(v_cache, dtype)
    qd = widen_np(q, dtype)
    nb, hkv, bs, d = kc.shape
    grp = num_q_heads // hkv
    B = len(seq_lens)
    out = np.zeros((q.shape[0], num_q_heads, d))
    for s in range(B):
        L = int(seq_lens[s])
        r0 = s if query_start_loc is None else int(query_start_loc[s])
        n = 1 if query_start_loc is None else int(query_start_loc[s + 1]) - r0
        for r in range(n):
            p = L - n + r
            positions = [t for t in range(0, p + 1) if window <= 0 or t > p - window]
            if not positions:
                continue
            for h in range(num_q_heads):
                g = h // grp
                K = np.stack([kc[block_tables[s][t // bs], g, t % bs] for t in positions])
                V = np.stack([vc[block_tables[s][t // bs], g, t % bs] for t in positions])
                w = softmax(float(scale) * (K @ qd[r0 + r, h]))
                out[r0 + r, h] = w @ V
    return out
