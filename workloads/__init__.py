"""Seeded synthetic inputs for paged KV-cache decode attention.

This module only *draws* inputs: sequence lengths, query-row counts, the order in which
physical blocks leave the free pool, a script of block-ledger operations, and the q/K/V
values.  It holds none of the method's arithmetic: it never maps a position to a block or
a slot and never computes attention.  The CPU oracle and the HIP library both consume what
it returns, each with its own code.

Workload shapes follow the pages' examples:
  * block size 16 and the block-table indirection ("PagedAttention deep dive", donmain.dev,
    section on splitting the KV cache into blocks);
  * OPT-13B (40 heads x 128, fp16, 2048-token maximum) from the KV-size section of the
    SOSP'23 notes (ghkdgus29.github.io);
  * Qwen3-8B / Mistral-7B GQA shapes (8 KV heads x 128) and Gemma-3-4B sliding-window
    layers (4 KV heads x 256, window 1024) from the per-model KV-cache measurements
    (sotaaz.com, sections "1. Full attention" and "2. Sliding window");
  * a shared system-prompt prefix ("PagedAttention deep dive", section on block sharing)
    and chunked prefill mixed with decodes (duolabs.co.kr, section on paging-based KV
    management).
The traffic traces the pages measure on (ShareGPT) are not available; only their shape is
imitated through the length distributions below.

Values are N(0, 1) drawn as float32 from numpy's PCG64 and rounded to the cache dtype with
round-to-nearest-even.  Big arrays are drawn in fixed 4 Mi-element chunks, chunk i from the
i-th child of a SeedSequence, so the result depends only on the seed, never on the number
of threads used to fill it.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "DTYPES", "Append", "SharePrefix", "Fork", "Flush", "SwapOut", "SwapIn", "Free",
    "SetWindow", "Workload",
    "make", "CONFIG_NAMES", "normal", "to_storage", "nan_bits", "ACT", "act_dtype",
]

# storage dtype per cache dtype name: (numpy storage type, bytes per element)
DTYPES = {"f32": (np.float32, 4), "f16": (np.float16, 2), "bf16": (np.uint16, 2)}
# 8-bit caches (one 16-bit scale per 32 values): the activations (q, new k / v) keep a
# 16-bit type; these names give that type
ACT = {"q8_f16": "f16", "q8_bf16": "bf16"}


def act_dtype(dtype: str) -> str:
    """Type of q and of the new k / v rows for a cache dtype name."""
    return ACT.get(dtype, dtype)

_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(seed: int, stream: int, n: int) -> np.ndarray:
    """n float32 N(0,1) values, deterministic in (seed, stream)."""
    out = np.empty(n, np.float32)
    nch = (n + _CHUNK - 1) // _CHUNK
    kids = np.random.SeedSequence(entropy=seed, spawn_key=(stream,)).spawn(nch)

    def fill(i):
        lo = i * _CHUNK
        hi = min(n, lo + _CHUNK)
        np.random.default_rng(kids[i]).standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nch <= 1:
        for i in range(nch):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the cache dtype (RNE) and return its storage array.

    bf16 is returned as its uint16 bit pattern (numpy has no bf16 type).  Inputs are finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    dtype = act_dtype(dtype)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x.reshape(-1).view(np.uint32)
    out = np.empty(u.size, np.uint16)
    nch = (u.size + _CHUNK - 1) // _CHUNK

    def conv(i):
        lo = i * _CHUNK
        hi = min(u.size, lo + _CHUNK)
        w = u[lo:hi]
        r = (w >> 16) & 1
        r += 0x7FFF
        r += w
        r >>= 16
        out[lo:hi] = r

    if nch <= 1:
        for i in range(nch):
            conv(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(conv, range(nch)))
    return out.reshape(x.shape)


def nan_bits(dtype: str):
    """A quiet-NaN storage value for the dtype (used to poison bytes nobody may read)."""
    return {"f32": np.float32(np.nan), "f16": np.float16(np.nan),
            "bf16": np.uint16(0x7FC0)}[act_dtype(dtype)]


# ---------------------------------------------------------------- ledger script entries
@dataclass(frozen=True)
class Append:
    """Append ``n`` tokens to ``seq``.  Values are supplied for the last ``nv`` of them,
    rows ``off .. off+nv`` of ``Workload.k`` / ``Workload.v`` (the earlier ones, if any,
    fall out of a sliding window and are never stored)."""
    seq: int
    n: int
    nv: int
    off: int


@dataclass(frozen=True)
class SharePrefix:
    """``dst`` (new, empty) starts with the first ``n_tokens`` tokens of ``src``,
    pointing at the same physical blocks."""
    dst: int
    src: int
    n_tokens: int


@dataclass(frozen=True)
class Fork:
    """``dst`` (new, empty) becomes a second sample of ``src``: same length, same window,
    same physical blocks (each one reference more)."""
    dst: int
    src: int


@dataclass(frozen=True)
class Flush:
    """End of a step: the block copies and slot writes recorded since the previous Flush are
    carried out (copies first, then writes) before anything later."""


@dataclass(frozen=True)
class SwapOut:
    """Evict ``seq`` (None: the resident sequence that arrived last) to host blocks."""
    seq: int | None = None


@dataclass(frozen=True)
class SwapIn:
    """Bring swapped-out ``seq`` back into device blocks."""
    seq: int


@dataclass(frozen=True)
class Free:
    seq: int


@dataclass(frozen=True)
class SetWindow:
    """``seq`` keeps only its last ``window`` tokens."""
    seq: int
    window: int


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int          # pool size; the last id is a reserved never-allocated block
    seq_lens: np.ndarray     # int32 [B]: context length of each batch sequence, this step included
    q_rows: np.ndarray       # int32 [B]: query rows of each sequence (1 = decode)
    window: int              # 0 = full attention
    scale: np.float32
    n_layers: int
    free_order: np.ndarray   # int32 [num_blocks-1]: order in which free blocks are handed out
    script: list             # ledger operations, in order
    k: np.ndarray            # [N][Hkv][d] storage dtype: values referenced by Append.off
    v: np.ndarray
    q: np.ndarray            # [R][Hq][d] storage dtype, R = sum(q_rows)
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.size)

    @property
    def reserved_block(self) -> int:
        return self.num_blocks - 1

    @property
    def total_q_rows(self) -> int:
        return int(self.q_rows.sum())

    @property
    def elem_bytes(self) -> float:
        """Cache bytes per stored K (or V) element, scales included (17/16 for 8-bit)."""
        if self.dtype in ACT:
            return 1.0 + 2.0 / 32
        return DTYPES[self.dtype][1]

    @property
    def act(self) -> str:
        """Type of q and of the new k / v rows."""
        return act_dtype(self.dtype)

    def query_start_loc(self) -> np.ndarray:
        """Row offsets [B+1] (a plain running sum over ``q_rows``)."""
        out = np.zeros(self.num_seqs + 1, np.int32)
        np.cumsum(self.q_rows, out=out[1:])
        return out


CONFIG_NAMES = ("tiny", "opt13b", "gqa", "prefix_mixed", "swa", "parallel_sampling", "swap")


def _values(seed, n_tok, hkv, d, dtype, stream_k=2, stream_v=3):
    k = to_storage(normal(seed, stream_k, n_tok * hkv * d), dtype).reshape(n_tok, hkv, d)
    v = to_storage(normal(seed, stream_v, n_tok * hkv * d), dtype).reshape(n_tok, hkv, d)
    return k, v


def _queries(seed, rows, hq, d, dtype):
    return to_storage(normal(seed, 1, rows * hq * d), dtype).reshape(rows, hq, d)


def _pool_size(blocks_needed: int) -> int:
    # needed blocks plus 10% free, plus one reserved block
    return int(math.ceil(1.1 * blocks_needed)) + 1


def _plain(name, seed, dtype, hq, hkv, d, lens, n_layers, rng, last_token_apart=False, bs=16):
    """Decode batch: each sequence appends its context; with ``last_token_apart`` the
    context minus one token first, then the new token of every sequence."""
    lens = np.asarray(lens, np.int32)
    B = lens.size
    need = int(sum(-(-int(L) // bs) for L in lens))
    nb = _pool_size(need)
    free_order = rng.permutation(nb - 1).astype(np.int32)
    script = []
    off = 0
    if last_token_apart:
        for s in range(B):
            n = int(lens[s]) - 1
            if n > 0:
                script.append(Append(s, n, n, off))
                off += n
        for s in range(B):
            script.append(Append(s, 1, 1, off))
            off += 1
    else:
        for s in range(B):
            n = int(lens[s])
            script.append(Append(s, n, n, off))
            off += n
    k, v = _values(seed, off, hkv, d, dtype)
    q = _queries(seed, B, hq, d, dtype)
    return Workload(name, seed, dtype, hq, hkv, d, bs, nb, lens, np.ones(B, np.int32), 0,
                    np.float32(1.0 / math.sqrt(d)), n_layers, free_order, script, k, v, q)


def make(name: str, seed: int | None = None, **over) -> Workload:
    """Build one of the named workloads (CONFIG_NAMES, plus "rows" for free-shape tests).

    Keyword overrides shrink a workload for fast parity runs while keeping its structure:
      batch=, lo=, hi= (length range), median= / sigma= (log-normal), prefix=, chunks=,
      chunk_rows=, chunk_lo=, chunk_hi=, window=, prompts= / samples= / plens=, victims= /
      finishers= / grow_hi=, dtype= (including the 8-bit cache names "q8_f16" and "q8_bf16").
    """
    if name == "tiny":
        seed = 1 if seed is None else seed
        rng = np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(0,)))
        lens = over.get("lens", [1, 17, 100, 33])
        # a 64-block pool: 63 hand-out blocks + the reserved one
        w = _plain("tiny", seed, over.get("dtype", "f32"), over.get("hq", 4), over.get("hkv", 4),
                   over.get("d", 64), lens, 1, rng, last_token_apart=True)
        nb = max(64, w.num_blocks)
        w.num_blocks = nb
        w.free_order = rng.permutation(nb - 1).astype(np.int32)
        return w

    if name == "opt13b":
        seed = 2 if seed is None else seed
        rng = np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(0,)))
        B = over.get("batch", 64)
        lens = rng.integers(over.get("lo", 64), over.get("hi", 2048) + 1, size=B)
        return _plain("opt13b", seed, over.get("dtype", "f16"), 40, 40, 128, lens, 40, rng,
                      bs=over.get("block_size", 16))

    if name == "gqa":
        seed = 3 if seed is None else seed
        rng = np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(0,)))
        B = over.get("batch", 256)
        med = over.get("median", 1024)
        sig = over.get("sigma", 1.0)
        x = rng.lognormal(math.log(med), sig, size=B)
        lens = np.clip(np.rint(x), over.get("lo", 16), over.get("hi", 32768)).astype(np.int32)
        return _plain("gqa", seed, over.get("dtype", "bf16"), over.get("hq", 32),
                      over.get("hkv", 8), over.get("d", 128), lens, 36, rng,
                      bs=over.get("block_size", 16))

    if name == "prefix_mixed":
        seed = 4 if seed is None else seed
        rng = np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(0,)))
        bs = 16
        nd = over.get("batch", 128)
        prefix = over.get("prefix", 512)
        suffix = rng.integers(1, over.get("suffix_hi", 512) + 1, size=nd)
        nc = over.get("chunks", 4)
        crow = over.get("chunk_rows", 512)
        clen = rng.integers(over.get("chunk_lo", 1024), over.get("chunk_hi", 4096) + 1, size=nc)
        lens = np.concatenate([prefix + suffix, clen]).astype(np.int32)
        rows = np.concatenate([np.ones(nd, np.int32), np.full(nc, crow, np.int32)])
        need = -(-prefix // bs) + int(sum(-(-int(s) // bs) + 1 for s in suffix)) \
            + int(sum(-(-int(L) // bs) for L in clen))
        nb = _pool_size(need)
        free_order = rng.permutation(nb - 1).astype(np.int32)
        holder = 1_000_000           # a sequence that only holds the prefix, then leaves
        script = [Append(holder, prefix, prefix, 0)]
        off = prefix
        for s in range(nd):
            script.append(SharePrefix(s, holder, prefix))
        script.append(Free(holder))
        for s in range(nd):
            n = int(suffix[s])
            script.append(Append(s, n, n, off))
            off += n
        for c in range(nc):
            n = int(clen[c])
            script.append(Append(nd + c, n, n, off))
            off += n
        k, v = _values(seed, off, 8, 128, over.get("dtype", "bf16"))
        q = _queries(seed, int(rows.sum()), 32, 128, over.get("dtype", "bf16"))
        w = Workload("prefix_mixed", seed, over.get("dtype", "bf16"), 32, 8, 128, bs, nb, lens,
                     rows, over.get("window", 0), np.float32(1.0 / math.sqrt(128)), 36,
                     free_order, script, k, v, q)
        w.meta.update(prefix_tokens=prefix, prefix_sharers=nd, holder=holder)
        return w

    if name == "swa":
        seed = 5 if seed is None else seed
        rng = np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(0,)))
        bs = 16
        B = over.get("batch", 32)
        W = over.get("window", 1024)
        lens = rng.integers(over.get("lo", 4096), over.get("hi", 131072) + 1, size=B).astype(np.int32)
        # only blocks that intersect each window are ever held
        need = B * (-(-W // bs) + 1)
        nb = _pool_size(need)
        free_order = rng.permutation(nb - 1).astype(np.int32)
        script = []
        off = 0
        for s in range(B):
            script.append(SetWindow(s, W))
        for s in range(B):
            n = int(lens[s])
            nv = min(n, W)
            script.append(Append(s, n, nv, off))
            off += nv
        dt = over.get("dtype", "f16")
        hq, hkv, d = over.get("hq", 8), over.get("hkv", 4), over.get("d", 256)
        k, v = _values(seed, off, hkv, d, dt)
        q = _queries(seed, B, hq, d, dt)
        return Workload("swa", seed, dt, hq, hkv, d, bs, nb, lens, np.ones(B, np.int32), W,
                        np.float32(1.0 / math.sqrt(d)), 29, free_order, script, k, v, q)

    if name == "parallel_sampling":
        # OPT-13B shape; every prompt is prefilled, then forked into `samples` samples that
        # each append their own first token (the first decode step after the fork)
        seed = 7 if seed is None else seed
        rng = np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(0,)))
        bs = 16
        P = over.get("prompts", 16)
        n = over.get("samples", 4)
        hq, hkv, d = over.get("hq", 40), over.get("hkv", 40), over.get("d", 128)
        plen = rng.integers(over.get("lo", 64), over.get("hi", 2048) + 1, size=P)
        if "plens" in over:
            plen = np.asarray(over["plens"], np.int64)
            P = plen.size
        B = P * n
        # every sample may take one block of its own (a copy or a new block)
        need = int(sum(-(-int(L) // bs) for L in plen)) + B
        nb = _pool_size(need)
        free_order = rng.permutation(nb - 1).astype(np.int32)
        script, off = [], 0
        for p in range(P):
            script.append(Append(p * n, int(plen[p]), int(plen[p]), off))
            off += int(plen[p])
        script.append(Flush())
        for p in range(P):
            for j in range(1, n):
                script.append(Fork(p * n + j, p * n))
        for s in range(B):
            script.append(Append(s, 1, 1, off))
            off += 1
        script.append(Flush())
        dt = over.get("dtype", "f16")
        k, v = _values(seed, off, hkv, d, dt)
        q = _queries(seed, B, hq, d, dt)
        lens = (np.repeat(plen, n) + 1).astype(np.int32)
        w = Workload("parallel_sampling", seed, dt, hq, hkv, d, bs, nb, lens,
                     np.ones(B, np.int32), 0, np.float32(1.0 / math.sqrt(d)),
                     over.get("layers", 40), free_order, script, k, v, q)
        w.meta.update(prompts=P, samples=n)
        return w

    if name == "swap":
        # OPT-13B shape under memory pressure ("vLLM and PagedAttention" notes, scheduling):
        # `batch` sequences and `finishers` short-lived requests are prefilled, the
        # short-lived ones spread among the first arrivals.  The `victims` batch sequences
        # that arrived last are swapped out.  While they are away no new request is taken:
        # the residents go on decoding (U{1..grow_hi} tokens each) into the freed blocks and
        # the short-lived requests finish and leave.  Then the victims come back (earliest
        # arrival first) and every batch sequence appends its next token.
        seed = 8 if seed is None else seed
        rng = np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(0,)))
        bs = 16
        B = over.get("batch", 64)
        V = over.get("victims", 8)
        F = over.get("finishers", V)
        hq, hkv, d = over.get("hq", 40), over.get("hkv", 40), over.get("d", 128)
        lo, hi = over.get("lo", 64), over.get("hi", 2048)
        lens = rng.integers(lo, hi + 1, size=B)
        flens = rng.integers(lo, hi + 1, size=F)
        # creation order: residents with the short-lived requests spread among them, then
        # the victims
        order = list(range(B - V))
        for k in range(F):
            order.insert((k + 1) * (B - V) // (F + 1) + k, B + k)
        order += list(range(B - V, B))
        plen = {s_: int(lens[s_]) for s_ in range(B)}
        plen.update({B + k: int(flens[k]) for k in range(F)})
        residents = [s_ for s_ in order if not B - V <= s_ < B]
        grow = dict(zip(residents, rng.integers(1, over.get("grow_hi", 32) + 1,
                                                size=len(residents)).tolist()))
        need = (sum(-(-n // bs) for n in plen.values())
                + sum(-(-g // bs) + 1 for g in grow.values()) + B)
        nb = _pool_size(need)
        free_order = rng.permutation(nb - 1).astype(np.int32)
        script, off = [], 0
        for s_ in order:
            script.append(Append(s_, plen[s_], plen[s_], off))
            off += plen[s_]
        script.append(Flush())
        for _ in range(V):
            script.append(SwapOut(None))
        script.append(Flush())
        for s_ in residents:
            script.append(Append(s_, grow[s_], grow[s_], off))
            off += grow[s_]
        script.append(Flush())
        for k in range(F):
            script.append(Free(B + k))
        script.append(Flush())
        for k in range(V):
            script.append(SwapIn(B - V + k))
        script.append(Flush())
        for s_ in range(B):
            script.append(Append(s_, 1, 1, off))
            off += 1
        script.append(Flush())
        dt = over.get("dtype", "f16")
        k_, v_ = _values(seed, off, hkv, d, dt)
        q = _queries(seed, B, hq, d, dt)
        final = np.array([plen[s_] + grow.get(s_, 0) + 1 for s_ in range(B)], np.int32)
        host = int(sum(-(-int(L) // bs) for L in lens[B - V:]))
        w = Workload("swap", seed, dt, hq, hkv, d, bs, nb, final,
                     np.ones(B, np.int32), 0, np.float32(1.0 / math.sqrt(d)),
                     over.get("layers", 40), free_order, script, k_, v_, q)
        w.meta.update(host_blocks=host, victims=V, finishers=F)
        return w

    if name == "rows":
        # test-sized mixed batch with free shapes: sequence s has lens[s] context tokens and
        # rows[s] query rows (1 = decode, more = a chunk of the last rows[s] positions)
        seed = 6 if seed is None else seed
        rng = np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(0,)))
        bs = 16
        lens = np.asarray(over["lens"], np.int32)
        rows = np.asarray(over["rows"], np.int32)
        hq, hkv, d = over.get("hq", 8), over.get("hkv", 2), over.get("d", 128)
        dt = over.get("dtype", "bf16")
        need = int(sum(-(-int(L) // bs) for L in lens))
        nb = _pool_size(need)
        free_order = rng.permutation(nb - 1).astype(np.int32)
        script, off = [], 0
        for s in range(lens.size):
            n = int(lens[s])
            if n:
                script.append(Append(s, n, n, off))
                off += n
        k, v = _values(seed, off, hkv, d, dt)
        q = _queries(seed, int(rows.sum()), hq, d, dt)
        return Workload("rows", seed, dt, hq, hkv, d, bs, nb, lens, rows, over.get("window", 0),
                        np.float32(1.0 / math.sqrt(d)), 1, free_order, script, k, v, q)

    raise ValueError(f"unknown workload {name!r}")
