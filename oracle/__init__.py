"""CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The HIP library never imports, links or runs
anything here, and nothing here imports the library: the two share only the seeded input
generators in ``workloads``.

Pieces:
  * ``ledger``   - block ledger model (on-demand blocks, reference counts, copy-on-write,
    windows); ``copy_block`` carries out one recorded copy on host caches;
  * ``pa_oracle.c`` (built into ``liboracle.so``) - fp64 slot write and attention, paged
    and contiguous;
  * ``brute``    - an independent numpy version of the attention definition for tiny
    inputs;
  * ``q8``       - the 8-bit cache: quantizer, tile layout, copies, decoding;
  * ``kv_bytes_per_token`` / ``kv_read_bytes`` - the pages' KV byte accounting.
Every function is pinned by ``tests/test_oracle_pins.py`` to what the pages and plain
mathematics fix.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

from . import q8  # noqa: F401
from .ledger import (AdmissionClosed, Ledger, LedgerError, OutOfBlocks, SharedBlock,  # noqa: F401
                     run_script)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_DT = {"f32": 0, "f16": 1, "bf16": 2}
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_write_kv.argtypes = [P, P, P, i64, P, P, i32, i32, i32, i32, i32]
    lib.oracle_paged_attention.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, P, i32, P, P,
                                           i32, i32, f64, i32, i32]
    lib.oracle_contiguous_attention.argtypes = [P, P, P, P, i32, i32, i32, P, P, P, P, i32,
                                                i32, f64, i32, i32]
    lib.oracle_widen.argtypes = [P, P, i64, i32]
    for f in ("oracle_write_kv", "oracle_paged_attention", "oracle_contiguous_attention",
              "oracle_widen"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _bind(_LIB)
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Run the oracle's C part from another build of ``pa_oracle.c`` (tests use this to
    plant a mistake and check that a pin catches it)."""
    global _lib
    old = _load()
    _lib = _bind(path)
    try:
        yield
    finally:
        _lib = old


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _threads(n):
    if n:
        return int(n)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# --------------------------------------------------------------------------- kernels
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored cache elements -> float64, decoded from their bit fields."""
    x = np.ascontiguousarray(x)
    out = np.empty(x.size, np.float64)
    rc = _load().oracle_widen(_p(out), _p(x), x.size, _DT[dtype])
    assert rc == 0
    return out.reshape(x.shape)


def write_kv(k, v, slots, k_cache, v_cache, block_size: int, dtype: str) -> None:
    """Scatter k/v [T][Hkv][d] into the caches [NB][Hkv][bs][d] in place."""
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    slots = np.ascontiguousarray(slots, np.int64)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    nb, hkv, bs, d = k_cache.shape
    assert bs == block_size and k.shape[1:] == (hkv, d) and slots.size == k.shape[0]
    rc = _load().oracle_write_kv(_p(k), _p(v), _p(slots), slots.size, _p(k_cache), _p(v_cache),
                                 nb, hkv, d, bs, _DT[dtype])
    if rc != 0:
        raise ValueError(f"oracle_write_kv failed ({rc})")


def copy_block(k_cache, v_cache, src: int, dst: int, n: int) -> None:
    """Copy-on-write of one block: the first n entries of physical block src, for every KV
    head, of K and of V, become those of block dst ("vLLM and PagedAttention" notes,
    ghkdgus29.github.io, section on parallel sampling).  Entries n.. of dst are left as
    they are: the sequence that now owns dst writes them itself."""
    k_cache[dst, :, :n] = k_cache[src, :, :n]
    v_cache[dst, :, :n] = v_cache[src, :, :n]


def paged_attention(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype: str, num_q_heads,
                    query_start_loc=None, window: int = 0, threads: int = 0) -> np.ndarray:
    """fp64 attention through block tables. q [R][Hq][d]; returns [R][Hq][d] float64."""
    q = np.ascontiguousarray(q)
    bt = np.ascontiguousarray(block_tables, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    qsl = None if query_start_loc is None else np.ascontiguousarray(query_start_loc, np.int32)
    nb, hkv, bs, d = k_cache.shape
    out = np.zeros((q.shape[0], num_q_heads, d), np.float64)
    rc = _load().oracle_paged_attention(_p(out), _p(q), _p(k_cache), _p(v_cache), _DT[dtype], nb,
                                        hkv, d, bs, _p(bt), bt.shape[1], _p(sl), _p(qsl), sl.size,
                                        num_q_heads, float(scale), int(window), _threads(threads))
    if rc != 0:
        raise ValueError(f"oracle_paged_attention failed ({rc})")
    return out


def contiguous_attention(q, k_log, v_log, tok_off, first_pos, seq_lens, scale, dtype: str,
                         num_q_heads, query_start_loc=None, window: int = 0,
                         threads: int = 0) -> np.ndarray:
    """fp64 attention over logical arrays [N][Hkv][d]; token t of seq s is row
    tok_off[s] + t - first_pos[s].  No block table involved."""
    q = np.ascontiguousarray(q)
    k_log = np.ascontiguousarray(k_log)
    v_log = np.ascontiguousarray(v_log)
    to = np.ascontiguousarray(tok_off, np.int64)
    fp = np.ascontiguousarray(first_pos, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    qsl = None if query_start_loc is None else np.ascontiguousarray(query_start_loc, np.int32)
    hkv, d = k_log.shape[1:]
    out = np.zeros((q.shape[0], num_q_heads, d), np.float64)
    rc = _load().oracle_contiguous_attention(_p(out), _p(q), _p(k_log), _p(v_log), _DT[dtype],
                                             hkv, d, _p(to), _p(fp), _p(sl), _p(qsl), sl.size,
                                             num_q_heads, float(scale), int(window),
                                             _threads(threads))
    if rc != 0:
        raise ValueError(f"oracle_contiguous_attention failed ({rc})")
    return out


# ------------------------------------------------------------------ byte accounting
def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int,
                       scale_group: int = 0) -> int:
    """KV cache bytes one token takes: K and V, per KV head, per layer.

    The SOSP'23 notes write it as 2 x H x L x B with H the hidden size (KV-size section,
    ghkdgus29.github.io); per-model pages write 2 x KV heads x head size x bytes per layer
    (sotaaz.com, section on layer kinds).  With H = KV heads x head size the two agree.
    With scale_group = g > 0 (an 8-bit cache), every g values also carry one 2-byte scale
    (sotaaz.com, KV-cache measurements, planning notes of the full-attention section)."""
    row = head_dim * elem_bytes + (2 * (head_dim // scale_group) if scale_group else 0)
    return 2 * num_layers * num_kv_heads * row


def tokens_read(seq_len: int, q_rows: int, window: int) -> int:
    """Distinct context positions one sequence's rows attend to (each read once)."""
    last = seq_len - 1
    first_row_pos = seq_len - q_rows
    lo = max(0, first_row_pos - window + 1) if window > 0 else 0
    return max(0, last - lo + 1)


def kv_read_bytes(seq_lens, q_rows, window, num_kv_heads, head_dim, elem_bytes,
                  scale_group: int = 0) -> int:
    """Algorithmic KV bytes one layer of attention reads (each attended token once)."""
    n = sum(tokens_read(int(L), int(r), window) for L, r in zip(seq_lens, q_rows))
    return kv_bytes_per_token(1, num_kv_heads, head_dim, elem_bytes, scale_group) * n


# ------------------------------------------------------------------ whole workload
class Reference:
    """The oracle's view of a workload: its tables, slots, caches and outputs."""

    def __init__(self, w, threads: int = 0, poison: bool = True):
        from workloads import ACT, DTYPES, Append, SwapIn, SwapOut, nan_bits

        self.w = w
        led = Ledger(w.free_order, w.block_size, w.meta.get("host_blocks", 0))
        self.slots, self.copies, self.swaps = run_script(led, w.script)
        self.ledger = led
        B = w.num_seqs
        self.max_blocks = max(1, max(len(led.block_table(s)) for s in range(B)))
        fill = w.reserved_block
        self.block_tables = np.full((B, self.max_blocks), fill, np.int32)
        for s in range(B):
            t = led.block_table(s)
            row = np.array(t, np.int32)
            row[row < 0] = fill
            self.block_tables[s, :len(t)] = row
        self.q8 = w.dtype in ACT
        shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        if self.q8:
            # tile pools of codes and scales; poison 0xFF decodes to NaN
            self.k_cache = q8.empty_cache(*shape[:2], w.head_dim, w.block_size,
                                          0xFF if poison else 0)
            self.v_cache = q8.empty_cache(*shape[:2], w.head_dim, w.block_size,
                                          0xFF if poison else 0)
        else:
            st, _ = DTYPES[w.dtype]
            self.k_cache = np.full(shape, nan_bits(w.dtype) if poison else 0, st)
            self.v_cache = np.full(shape, nan_bits(w.dtype) if poison else 0, st)
        # host swap space: tiles laid out like the device pool's
        nh = w.meta.get("host_blocks", 0)
        self.host_k = np.zeros((nh,) + self.k_cache.shape[1:], self.k_cache.dtype)
        self.host_v = np.zeros((nh,) + self.v_cache.shape[1:], self.v_cache.dtype)
        for i, op in enumerate(w.script):
            if isinstance(op, SwapOut):
                for b, h in self.swaps[i][1]:
                    self.host_k[h], self.host_v[h] = self.k_cache[b], self.v_cache[b]
                continue
            if isinstance(op, SwapIn):
                for h, b in self.swaps[i][1]:
                    self.k_cache[b], self.v_cache[b] = self.host_k[h], self.host_v[h]
                continue
            if not isinstance(op, Append):
                continue
            for src, dst, n in self.copies[i]:
                (q8.copy_block if self.q8 else copy_block)(self.k_cache, self.v_cache, src, dst, n)
            if op.nv > 0:
                sl = np.asarray(self.slots[i][-op.nv:], np.int64)
                kr, vr = w.k[op.off:op.off + op.nv], w.v[op.off:op.off + op.nv]
                if self.q8:
                    q8.write_kv(widen(kr, w.act).astype(np.float32),
                                widen(vr, w.act).astype(np.float32), sl, self.k_cache,
                                self.v_cache)
                else:
                    write_kv(kr, vr, sl, self.k_cache, self.v_cache, w.block_size, w.dtype)
        self.threads = threads
        self._decoded = None

    def attention_inputs(self, q):
        """(q, k_cache, v_cache, dtype) for the attention definition.  An 8-bit cache is
        decoded to float32 (exactly) and q widened to float32 (exactly)."""
        if not self.q8:
            return q, self.k_cache, self.v_cache, self.w.dtype
        if self._decoded is None:
            self._decoded = (q8.dequantize_cache(self.k_cache), q8.dequantize_cache(self.v_cache))
        return (widen(q, self.w.act).astype(np.float32), *self._decoded, "f32")

    def write_batches(self):
        """(slots, k, v) triples in script order, exactly what the GPU side must write."""
        from workloads import Append

        for i, op in enumerate(self.w.script):
            if isinstance(op, Append) and op.nv > 0:
                yield (np.asarray(self.slots[i][-op.nv:], np.int64),
                       self.w.k[op.off:op.off + op.nv], self.w.v[op.off:op.off + op.nv])

    def attention(self, seqs=None) -> np.ndarray:
        w = self.w
        qsl = w.query_start_loc()
        if seqs is None:
            q, kc, vc, dt = self.attention_inputs(w.q)
            return paged_attention(q, kc, vc, self.block_tables, w.seq_lens, w.scale, dt,
                                   w.num_q_heads, qsl, w.window, self.threads)
        seqs = np.asarray(seqs)
        rows = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in seqs])
        sub_qsl = np.zeros(seqs.size + 1, np.int32)
        np.cumsum(w.q_rows[seqs], out=sub_qsl[1:])
        q, kc, vc, dt = self.attention_inputs(w.q[rows])
        return paged_attention(q, kc, vc, self.block_tables[seqs], w.seq_lens[seqs], w.scale,
                               dt, w.num_q_heads, sub_qsl, w.window, self.threads)
