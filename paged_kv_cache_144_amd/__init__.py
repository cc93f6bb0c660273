"""Paged KV-cache attention for AMD MI355X (gfx950): thin Python binding over ``libpa.so``.

Every step of the path runs in the HIP library; this module only marshals arguments
(device pointers from torch tensors, the current HIP stream) and wraps the host block
ledger.  The library must be built (``python -m paged_kv_cache_144_amd._build``); importing
works without it, but every call then raises - there is no CPU fallback.

The C ABI is declared in ``include/pa.h``; the names below mirror it:
  write_kv  -> pa_write_kv        decode -> pa_decode (+ pa_decode_workspace_size)
  copy_blocks -> pa_copy_blocks    Pool   -> pa_pool_* / pa_seq_*

An 8-bit cache (one fp16 scale per 32 values) is a uint8 tensor [NB][Hkv][17][d]
(``q8_cache``); its queries and new rows are fp16 or bf16, which selects PA_Q8_F16 or
PA_Q8_BF16.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_F32, PA_F16, PA_BF16, PA_Q8_F16, PA_Q8_BF16 = 0, 1, 2, 3, 4
STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_DTYPE",
          -4: "PA_ERR_UNSUPPORTED", -5: "PA_ERR_WORKSPACE", -6: "PA_ERR_LAUNCH",
          -7: "PA_ERR_OUT_OF_BLOCKS", -8: "PA_ERR_SHARED_BLOCK", -9: "PA_ERR_BAD_SEQ",
          -10: "PA_ERR_ADMISSION"}
BLOCK_SIZE = 16

# every symbol include/pa.h declares
EXPORTS = ("pa_write_kv", "pa_copy_blocks", "pa_swap_blocks", "pa_decode_workspace_size", "pa_decode_kernel_name",
           "pa_decode", "pa_decode_write_attend", "pa_decode_noalloc", "pa_decode_plan",
           "pa_decode_attend", "pa_set_decode_profile_events", "pa_set_chunk_profile_events",
           "pa_stream_read", "pa_status_string",
           "pa_pool_create", "pa_pool_destroy", "pa_seq_set_window", "pa_seq_append",
           "pa_seq_share_prefix", "pa_seq_free", "pa_seq_block_table", "pa_pool_block_tables",
           "pa_seq_len", "pa_pool_num_free", "pa_block_refcount", "pa_seq_fork",
           "pa_pool_take_copies", "pa_pool_num_pending_copies", "pa_pool_set_host_blocks",
           "pa_pool_num_host_free", "pa_pool_latest_resident", "pa_seq_swap_out",
           "pa_seq_swap_in")


class PAError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)}")


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_lib = None


def load():
    """Load libpa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_144_amd._build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    D = ctypes.POINTER(CacheDesc)
    sig = {
        "pa_write_kv": (i32, [P, P, P, i32, P, P, D, P]),
        "pa_copy_blocks": (i32, [P, P, D, P, i32, P, P]),
        "pa_swap_blocks": (i32, [P, P, P, P, D, i32, i32, P, i32, P, P]),
        "pa_decode_workspace_size": (ctypes.c_size_t, [D, i32, i32, i32, i32]),
        "pa_decode_kernel_name": (ctypes.c_char_p, [D, i32, i32, i32]),
        "pa_decode": (i32, [P, i32, P, P, P, D, P, i32, P, P, i32, i32, i32, i32, f32, i32, P,
                            ctypes.c_size_t, P]),
        "pa_decode_write_attend": (i32, [P, i32, P, P, P, P, P, D, P, i32, P, i32, i32, i32, f32,
                                         i32, P, ctypes.c_size_t, P]),
        "pa_decode_noalloc": (i32, [P, i32, P, P, P, D, P, i32, P, P, i32, i32, i32, i32, f32,
                                    i32, P]),
        "pa_decode_plan": (i32, [D, P, i32, P, P, i32, i32, i32, i32, i32, P, ctypes.c_size_t,
                                 P]),
        "pa_decode_attend": (i32, [P, i32, P, P, P, D, P, i32, P, P, i32, i32, i32, i32, f32,
                                   i32, P, ctypes.c_size_t, P]),
        "pa_set_decode_profile_events": (None, [P, P]),
        "pa_set_chunk_profile_events": (None, [P, P]),
        "pa_stream_read": (i32, [P, ctypes.c_size_t, P, P]),
        "pa_status_string": (ctypes.c_char_p, [i32]),
        "pa_pool_create": (i32, [i32, i32, P, i32, ctypes.POINTER(P)]),
        "pa_pool_destroy": (None, [P]),
        "pa_seq_set_window": (i32, [P, i64, i32]),
        "pa_seq_append": (i32, [P, i64, i32, P]),
        "pa_seq_share_prefix": (i32, [P, i64, i64, i32]),
        "pa_seq_free": (i32, [P, i64]),
        "pa_seq_block_table": (i32, [P, i64, P, i32, ctypes.POINTER(i32)]),
        "pa_pool_block_tables": (i32, [P, P, i32, i32, i32, P]),
        "pa_seq_len": (i32, [P, i64]),
        "pa_pool_num_free": (i32, [P]),
        "pa_block_refcount": (i32, [P, i32]),
        "pa_seq_fork": (i32, [P, i64, i64]),
        "pa_pool_take_copies": (i32, [P, P, i32, ctypes.POINTER(i32)]),
        "pa_pool_num_pending_copies": (i32, [P]),
        "pa_pool_set_host_blocks": (i32, [P, i32]),
        "pa_pool_num_host_free": (i32, [P]),
        "pa_pool_latest_resident": (i32, [P, ctypes.POINTER(i64)]),
        "pa_seq_swap_out": (i32, [P, i64, P, i32, ctypes.POINTER(i32)]),
        "pa_seq_swap_in": (i32, [P, i64, P, i32, ctypes.POINTER(i32)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(code, what):
    if code != 0:
        raise PAError(code, what)


# ------------------------------------------------------------------ torch marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    m = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _dev_ptr(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def cache_desc(k_cache, act=None) -> CacheDesc:
    """Pool description.  For an 8-bit (uint8) cache, `act` is the torch dtype of its
    queries and new rows (fp16 unless given)."""
    torch = _torch()
    nb, hkv, rows, d = k_cache.shape
    if k_cache.dtype == torch.uint8:
        if rows != BLOCK_SIZE + 1:
            raise ValueError("an 8-bit cache is [NB][Hkv][17][d]")
        code = PA_Q8_BF16 if act == torch.bfloat16 else PA_Q8_F16
        return CacheDesc(nb, BLOCK_SIZE, hkv, d, code)
    return CacheDesc(nb, rows, hkv, d, _dtype_code(k_cache))


def q8_cache(num_blocks, num_kv_heads, head_dim, device="cuda", fill=0xFF):
    """An empty 8-bit cache tensor (every byte `fill`; 0xFF decodes to NaN)."""
    torch = _torch()
    return torch.full((num_blocks, num_kv_heads, BLOCK_SIZE + 1, head_dim), fill,
                      dtype=torch.uint8, device=device)


def _check_act(t, k_cache, what):
    torch = _torch()
    if k_cache.dtype == torch.uint8:
        if t.dtype not in (torch.float16, torch.bfloat16):
            raise TypeError(f"{what} must be fp16 or bf16 for an 8-bit cache")
    elif t.dtype != k_cache.dtype:
        raise TypeError(f"{what} must have the cache dtype")


def write_kv(k, v, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """pa_write_kv: k, v [T][Hkv][d]; slot_mapping int64 [T]; caches [NB][Hkv][16][d]."""
    torch = _torch()
    lib = load()
    if k.shape != v.shape or k.dim() != 3 or k_cache.shape != v_cache.shape:
        raise ValueError("shape mismatch")
    _check_act(k, k_cache, "k")
    if v.dtype != k.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("k and v, and the two caches, must share their dtypes")
    if k.shape[1:] != (k_cache.shape[1], k_cache.shape[3]) or slot_mapping.numel() != k.shape[0]:
        raise ValueError("k/v rows do not match the cache or the slot count")
    desc = cache_desc(k_cache, k.dtype)
    rc = lib.pa_write_kv(_dev_ptr(k, "k"), _dev_ptr(v, "v"),
                         _dev_ptr(slot_mapping, "slot_mapping", torch.int64), k.shape[0],
                         _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                         ctypes.byref(desc), _stream(stream))
    _check(rc, "pa_write_kv")


def stream_read(buf, sink, stream=None) -> None:
    """pa_stream_read: read the whole contiguous device tensor `buf` once (its byte size a
    multiple of 16); `sink` is a device int32/uint32 word written only in a negligible case."""
    torch = _torch()
    lib = load()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink.dtype not in (torch.int32, torch.uint32) or not sink.is_cuda or sink.numel() < 1:
        raise ValueError("sink must be a device int32 word")
    rc = lib.pa_stream_read(ctypes.c_void_p(buf.data_ptr()),
                            buf.numel() * buf.element_size(), ctypes.c_void_p(sink.data_ptr()),
                            _stream(stream))
    _check(rc, "pa_stream_read")


def copy_blocks(k_cache, v_cache, copies, error_word=None, stream=None) -> None:
    """pa_copy_blocks: copies int32 [n][3] device tensor of (src, dst, entries) triples;
    error_word an optional int32 device tensor of one element."""
    torch = _torch()
    lib = load()
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype or k_cache.dim() != 4:
        raise ValueError("k_cache and v_cache must match")
    if copies.dim() != 2 or copies.shape[1] != 3:
        raise ValueError("copies must be [n][3]")
    if error_word is not None and error_word.numel() < 1:
        raise ValueError("error_word must hold one int32")
    desc = cache_desc(k_cache)
    n = copies.shape[0]
    rc = lib.pa_copy_blocks(_dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                            ctypes.byref(desc),
                            _dev_ptr(copies, "copies", torch.int32) if n else None, n,
                            _dev_ptr(error_word, "error_word", torch.int32), _stream(stream))
    _check(rc, "pa_copy_blocks")


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs, error_word=None, stream=None) -> None:
    """pa_swap_blocks: whole blocks src -> dst for int32 [n][2] (src, dst) device pairs.
    Either pool may be a pinned host tensor (pin_memory=True) of the same tile shape."""
    torch = _torch()
    lib = load()
    if (src_k.shape[1:] != dst_k.shape[1:] or src_k.shape != src_v.shape
            or dst_k.shape != dst_v.shape or src_k.dtype != dst_k.dtype):
        raise ValueError("the two pools must have one tile shape and dtype")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n][2]")
    for t, name in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v")):
        if not t.is_contiguous() or not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a contiguous device or pinned host tensor")
    desc = cache_desc(src_k)
    n = pairs.shape[0]
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.pa_swap_blocks(p(src_k), p(src_v), p(dst_k), p(dst_v), ctypes.byref(desc),
                            src_k.shape[0], dst_k.shape[0],
                            _dev_ptr(pairs, "pairs", torch.int32) if n else None, n,
                            _dev_ptr(error_word, "error_word", torch.int32), _stream(stream))
    _check(rc, "pa_swap_blocks")


def workspace_size(k_cache, num_seqs, total_q_rows, num_q_heads, max_seq_len,
                   q_dtype=None) -> int:
    desc = cache_desc(k_cache, q_dtype)
    n = load().pa_decode_workspace_size(ctypes.byref(desc), num_seqs, total_q_rows, num_q_heads,
                                        max_seq_len)
    if n == 0:
        raise PAError(-4, "pa_decode_workspace_size")
    return int(n)


def decode_kernel_name(k_cache, num_q_heads, q_dtype=None, num_seqs=0, window=0) -> str:
    """pa_decode_kernel_name: the decode kernel pa_decode launches for a batch of num_seqs
    decode rows of this pool and head count under `window` ("decode_mfma_kernel",
    "decode_group_kernel" or "decode_kernel")."""
    desc = cache_desc(k_cache, q_dtype)
    name = load().pa_decode_kernel_name(ctypes.byref(desc), num_q_heads, num_seqs, window)
    if name is None:
        raise PAError(-4, "pa_decode_kernel_name")
    return name.decode()


def alloc_workspace(k_cache, num_seqs, total_q_rows, num_q_heads, max_seq_len, q_dtype=None):
    torch = _torch()
    n = workspace_size(k_cache, num_seqs, total_q_rows, num_q_heads, max_seq_len, q_dtype)
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(n, dtype=torch.uint8, device=k_cache.device)


def decode(q, k_cache, v_cache, block_tables, seq_lens, scale, *, max_seq_len,
           query_start_loc=None, window=0, out=None, out_dtype=None, workspace=None,
           stream=None, step="both"):
    """pa_decode: q [R][Hq][d]; block_tables int32 [B][MB]; seq_lens int32 [B];
    query_start_loc int32 [B+1] or None (one row per sequence).  Returns out [R][Hq][d].

    step="plan" calls pa_decode_plan only, step="attend" pa_decode_attend only (reusing the
    plan in `workspace`), step="both" pa_decode."""
    torch = _torch()
    lib = load()
    if q.dim() != 3 or k_cache.dim() != 4 or block_tables.dim() != 2:
        raise ValueError("q is [R][Hq][d], the caches [NB][Hkv][rows][d], block_tables [B][MB]")
    R, hq, d = q.shape
    B, mb = block_tables.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache in shape and dtype")
    if d != k_cache.shape[3]:
        raise ValueError(f"q has head_dim {d}, the cache {k_cache.shape[3]}")
    if hq % k_cache.shape[1]:
        raise ValueError(f"{hq} query heads are not a multiple of {k_cache.shape[1]} KV heads")
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache"), (block_tables, "block_tables"),
                    (seq_lens, "seq_lens"), (query_start_loc, "query_start_loc"),
                    (workspace, "workspace"), (out, "out")):
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if seq_lens.numel() != B:
        raise ValueError("seq_lens length")
    if query_start_loc is not None and query_start_loc.numel() != B + 1:
        raise ValueError("query_start_loc length")
    _check_act(q, k_cache, "q")
    if out is not None:
        if tuple(out.shape) != (R, hq, d):
            raise ValueError(f"out must be [{R}][{hq}][{d}], got {list(out.shape)}")
        _dtype_code(out)
        if out_dtype is not None and out.dtype != out_dtype:
            raise TypeError(f"out is {out.dtype}, out_dtype {out_dtype}")
    if out is None:
        out = torch.empty((R, hq, d), dtype=out_dtype or torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(k_cache, B, R, hq, max_seq_len, q.dtype)
    desc = cache_desc(k_cache, q.dtype)
    bt = _dev_ptr(block_tables, "block_tables", torch.int32)
    sl = _dev_ptr(seq_lens, "seq_lens", torch.int32)
    qs = _dev_ptr(query_start_loc, "query_start_loc", torch.int32)
    ws = _dev_ptr(workspace, "workspace", torch.uint8)
    st = _stream(stream)
    if step == "plan":
        rc = lib.pa_decode_plan(ctypes.byref(desc), bt, mb, sl, qs, B, R, int(max_seq_len), hq,
                                int(window), ws, workspace.numel(), st)
        _check(rc, "pa_decode_plan")
        return out
    fn = lib.pa_decode if step == "both" else lib.pa_decode_attend
    rc = fn(_dev_ptr(out, "out"), _dtype_code(out), _dev_ptr(q, "q"),
            _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"), ctypes.byref(desc), bt,
            mb, sl, qs, B, R, int(max_seq_len), hq, float(scale), int(window), ws,
            workspace.numel(), st)
    _check(rc, "pa_decode" if step == "both" else "pa_decode_attend")
    return out


def decode_write_attend(q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, scale, *,
                        max_seq_len, workspace, window=0, out=None, out_dtype=None,
                        stream=None):
    """pa_decode_write_attend: write each sequence's new token (k_new / v_new row s, into
    the slot of position seq_lens[s] - 1) and attend, in one launch.  One query row per
    sequence; `workspace` must hold the plan (decode(..., step="plan") with the same tables,
    lengths and window).  Returns out [B][Hq][d]."""
    torch = _torch()
    lib = load()
    if q.dim() != 3 or k_cache.dim() != 4 or block_tables.dim() != 2:
        raise ValueError("q [B][Hq][d], caches [NB][Hkv][bs][d], block_tables [B][MB]")
    B, hq, d = q.shape
    if block_tables.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("one query row per sequence")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache in shape and dtype")
    if d != k_cache.shape[3]:
        raise ValueError(f"q has head_dim {d}, the cache {k_cache.shape[3]}")
    want = (B, k_cache.shape[1], d)
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        if tuple(t.shape) != want:
            raise ValueError(f"{name} must be {list(want)}")
        _check_act(t, k_cache, name)
    _check_act(q, k_cache, "q")
    if out is None:
        out = torch.empty((B, hq, d), dtype=out_dtype or torch.float32, device=q.device)
    elif tuple(out.shape) != (B, hq, d):
        raise ValueError(f"out must be [{B}][{hq}][{d}]")
    desc = cache_desc(k_cache, q.dtype)
    rc = lib.pa_decode_write_attend(
        _dev_ptr(out, "out"), _dtype_code(out), _dev_ptr(q, "q"), _dev_ptr(k_new, "k_new"),
        _dev_ptr(v_new, "v_new"), _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
        ctypes.byref(desc), _dev_ptr(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev_ptr(seq_lens, "seq_lens", torch.int32), B,
        int(max_seq_len), hq, float(scale), int(window),
        _dev_ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    _check(rc, "pa_decode_write_attend")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20      # PA_NOALLOC_SCRATCH_BYTES


def decode_noalloc(q, k_cache, v_cache, block_tables, seq_lens, scale, *, max_seq_len, out,
                   query_start_loc=None, window=0, stream=None):
    """pa_decode_noalloc: pa_decode with the library's fixed device workspace; `out` is the
    caller's [R][Hq][d] tensor (nothing is allocated on this path).  Calls that overlap on
    one device race on that workspace."""
    torch = _torch()
    lib = load()
    if q.dim() != 3 or k_cache.dim() != 4 or block_tables.dim() != 2 or out is None:
        raise ValueError("q [R][Hq][d], caches [NB][Hkv][rows][d], block_tables [B][MB], out")
    R, hq, d = q.shape
    B, mb = block_tables.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache in shape and dtype")
    if d != k_cache.shape[3] or tuple(out.shape) != (R, hq, d):
        raise ValueError("q, the cache and out disagree on their shapes")
    if seq_lens.numel() != B or (query_start_loc is not None
                                 and query_start_loc.numel() != B + 1):
        raise ValueError("seq_lens / query_start_loc length")
    _check_act(q, k_cache, "q")
    desc = cache_desc(k_cache, q.dtype)
    rc = lib.pa_decode_noalloc(
        _dev_ptr(out, "out"), _dtype_code(out), _dev_ptr(q, "q"), _dev_ptr(k_cache, "k_cache"),
        _dev_ptr(v_cache, "v_cache"), ctypes.byref(desc),
        _dev_ptr(block_tables, "block_tables", torch.int32), mb,
        _dev_ptr(seq_lens, "seq_lens", torch.int32),
        _dev_ptr(query_start_loc, "query_start_loc", torch.int32), B, R, int(max_seq_len), hq,
        float(scale), int(window), _stream(stream))
    _check(rc, "pa_decode_noalloc")
    return out


def _ev(e):
    return None if e is None else ctypes.c_void_p(e.cuda_event)


def set_decode_profile_events(before=None, after=None) -> None:
    """pa_set_decode_profile_events with torch.cuda.Event objects (recorded once already so
    that their handles exist), or None to switch the hook off."""
    load().pa_set_decode_profile_events(_ev(before), _ev(after))


def set_chunk_profile_events(before=None, after=None) -> None:
    """pa_set_chunk_profile_events (see set_decode_profile_events)."""
    load().pa_set_chunk_profile_events(_ev(before), _ev(after))


def device_error_bits(workspace) -> int:
    """Error bits the last pa_decode on this workspace left (synchronizes)."""
    return int(workspace[:4].cpu().view(_torch().int32)[0])


# ------------------------------------------------------------------ host block ledger
class Pool:
    """pa_pool: host ledger of one pool's blocks (first-in first-out free queue)."""

    def __init__(self, num_blocks, block_size=BLOCK_SIZE, free_order=None):
        lib = load()
        self._lib = lib
        h = ctypes.c_void_p()
        fo = None if free_order is None else np.ascontiguousarray(free_order, np.int32)
        rc = lib.pa_pool_create(num_blocks, block_size,
                                None if fo is None else fo.ctypes.data_as(ctypes.c_void_p),
                                0 if fo is None else fo.size, ctypes.byref(h))
        _check(rc, "pa_pool_create")
        self._h = h
        self.block_size = block_size
        self.num_blocks = num_blocks

    def close(self):
        if self._h:
            self._lib.pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover
            pass

    def set_window(self, seq, window):
        _check(self._lib.pa_seq_set_window(self._h, seq, window), "pa_seq_set_window")

    def append(self, seq, n) -> np.ndarray:
        slots = np.empty(max(0, n), np.int64)
        _check(self._lib.pa_seq_append(self._h, seq, n, slots.ctypes.data_as(ctypes.c_void_p)),
               "pa_seq_append")
        return slots

    def share_prefix(self, dst, src, n_tokens):
        _check(self._lib.pa_seq_share_prefix(self._h, dst, src, n_tokens), "pa_seq_share_prefix")

    def fork(self, dst, src):
        _check(self._lib.pa_seq_fork(self._h, dst, src), "pa_seq_fork")

    def num_pending_copies(self) -> int:
        return int(self._lib.pa_pool_num_pending_copies(self._h))

    def take_copies(self) -> np.ndarray:
        """End the copy batch; its (src, dst, entries) triples as int32 [n][3]."""
        n = ctypes.c_int32()
        out = np.empty((max(1, self.num_pending_copies()), 3), np.int32)
        _check(self._lib.pa_pool_take_copies(self._h, out.ctypes.data_as(ctypes.c_void_p),
                                             out.shape[0], ctypes.byref(n)),
               "pa_pool_take_copies")
        return out[:n.value].copy()

    def free(self, seq):
        _check(self._lib.pa_seq_free(self._h, seq), "pa_seq_free")

    def set_host_blocks(self, n):
        _check(self._lib.pa_pool_set_host_blocks(self._h, n), "pa_pool_set_host_blocks")

    def num_host_free(self) -> int:
        return int(self._lib.pa_pool_num_host_free(self._h))

    def latest_resident(self):
        s = ctypes.c_int64()
        rc = self._lib.pa_pool_latest_resident(self._h, ctypes.byref(s))
        if rc == -9:
            return None
        _check(rc, "pa_pool_latest_resident")
        return int(s.value)

    def _swap(self, fn, seq, what):
        n = ctypes.c_int32()
        rc = fn(self._h, seq, None, 0, ctypes.byref(n))
        if rc not in (0, -2):
            _check(rc, what)
        out = np.empty((max(1, n.value), 2), np.int32)
        if rc == -2:
            _check(fn(self._h, seq, out.ctypes.data_as(ctypes.c_void_p), out.shape[0],
                      ctypes.byref(n)), what)
        return out[:n.value].copy()

    def swap_out(self, seq) -> np.ndarray:
        """Evict seq: its (device block, host block) pairs, int32 [n][2]."""
        return self._swap(self._lib.pa_seq_swap_out, seq, "pa_seq_swap_out")

    def swap_in(self, seq) -> np.ndarray:
        """Bring seq back: its (host block, device block) pairs, int32 [n][2]."""
        return self._swap(self._lib.pa_seq_swap_in, seq, "pa_seq_swap_in")

    def block_table(self, seq) -> list:
        n = ctypes.c_int32()
        rc = self._lib.pa_seq_block_table(self._h, seq, None, 0, ctypes.byref(n))
        if rc not in (0, -2):
            _check(rc, "pa_seq_block_table")
        out = np.empty(n.value, np.int32)
        _check(self._lib.pa_seq_block_table(self._h, seq, out.ctypes.data_as(ctypes.c_void_p),
                                            n.value, ctypes.byref(n)), "pa_seq_block_table")
        return out.tolist()

    def block_tables(self, seqs, max_blocks, fill) -> np.ndarray:
        s = np.ascontiguousarray(seqs, np.int64)
        out = np.empty((s.size, max_blocks), np.int32)
        _check(self._lib.pa_pool_block_tables(self._h, s.ctypes.data_as(ctypes.c_void_p), s.size,
                                              max_blocks, fill,
                                              out.ctypes.data_as(ctypes.c_void_p)),
               "pa_pool_block_tables")
        return out

    def seq_len(self, seq) -> int:
        return int(self._lib.pa_seq_len(self._h, seq))

    def num_free(self) -> int:
        return int(self._lib.pa_pool_num_free(self._h))

    def refcount(self, block) -> int:
        return int(self._lib.pa_block_refcount(self._h, block))
