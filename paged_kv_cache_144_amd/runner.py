"""Drive a synthetic workload through the library: ledger script -> block tables, slots and
copy batches (host ``Pool``), then copies and values -> KV pool (``pa_copy_blocks``,
``pa_write_kv``), then ``pa_decode``.

Used by the benchmark, the smoke check and the GPU tests.  Only torch device memory and
copies happen here; the per-token work is in the HIP kernels.
"""
from __future__ import annotations

import numpy as np

from . import Pool, alloc_workspace, copy_blocks, decode, q8_cache, swap_blocks, write_kv

TORCH_DTYPES = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def _act(dtype: str) -> str:
    # 8-bit caches keep their queries and new rows in a 16-bit type
    return {"q8_f16": "f16", "q8_bf16": "bf16"}.get(dtype, dtype)


def to_device(a: np.ndarray, dtype: str, device):
    """Storage array (float32 / float16 / bf16 bits as uint16) -> torch tensor on device."""
    import torch
    if _act(dtype) == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def to_storage_np(t, dtype: str) -> np.ndarray:
    """Device tensor -> storage numpy array (bit pattern preserved)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.uint8:
        return t.numpy()
    if _act(dtype) == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DeviceWorkload:
    """Device state of one layer of a workload."""

    def __init__(self, w, device="cuda", poison=True, write=True):
        import torch
        from workloads import Append, Flush, Fork, Free, SetWindow, SharePrefix, SwapIn, SwapOut

        self.w = w
        self.device = device
        pool = Pool(w.num_blocks, w.block_size, w.free_order)
        nh = int(w.meta.get("host_blocks", 0))
        if nh:
            pool.set_host_blocks(nh)
        slots_all = np.full(w.k.shape[0], -1, np.int64)
        # batches of (swap-out pairs, copies, swap-in pairs, slots of the tokens written);
        # the device carries out each batch in that order
        batches = []
        cur = np.full(w.k.shape[0], -1, np.int64)
        outs, ins = [], []

        def end_batch():
            nonlocal cur, outs, ins
            copies = pool.take_copies()
            o = np.concatenate(outs) if outs else np.zeros((0, 2), np.int32)
            i = np.concatenate(ins) if ins else np.zeros((0, 2), np.int32)
            if copies.size or o.size or i.size or (cur >= 0).any():
                batches.append((o, copies, i, cur))
            cur = np.full(w.k.shape[0], -1, np.int64)
            outs, ins = [], []

        for op in w.script:
            if isinstance(op, Append):
                s = pool.append(op.seq, op.n)
                if op.nv:
                    slots_all[op.off:op.off + op.nv] = s[op.n - op.nv:]
                    cur[op.off:op.off + op.nv] = s[op.n - op.nv:]
            elif isinstance(op, Flush):
                end_batch()
            elif isinstance(op, SwapOut):
                seq = pool.latest_resident() if op.seq is None else op.seq
                outs.append(pool.swap_out(seq))
            elif isinstance(op, SwapIn):
                ins.append(pool.swap_in(op.seq))
            elif isinstance(op, Fork):
                pool.fork(op.dst, op.src)
            elif isinstance(op, SharePrefix):
                pool.share_prefix(op.dst, op.src, op.n_tokens)
            elif isinstance(op, Free):
                pool.free(op.seq)
            elif isinstance(op, SetWindow):
                pool.set_window(op.seq, op.window)
            else:  # pragma: no cover
                raise TypeError(op)
        end_batch()
        self.pool = pool
        self.slots = slots_all
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device) if a.size else None
        self.batches = [(dev(o), dev(c), dev(i), torch.from_numpy(sl).to(device))
                        for o, c, i, sl in batches]
        # copies of the last batch (the step that follows a fork), or None
        self.step_copies = self.batches[-1][1] if self.batches else None
        B = w.num_seqs
        self.max_blocks = max(1, max(len(pool.block_table(s)) for s in range(B)))
        self.block_tables_np = pool.block_tables(np.arange(B), self.max_blocks, w.reserved_block)
        shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        if w.dtype in ("q8_f16", "q8_bf16"):
            # every byte 0xFF: codes -1 with NaN scales
            fill8 = 0xFF if poison else 0
            self.k_cache = q8_cache(w.num_blocks, w.num_kv_heads, w.head_dim, device, fill8)
            self.v_cache = q8_cache(w.num_blocks, w.num_kv_heads, w.head_dim, device, fill8)
        else:
            tdt = getattr(torch, TORCH_DTYPES[w.dtype])
            fill = float("nan") if poison else 0.0
            self.k_cache = torch.full(shape, fill, dtype=tdt, device=device)
            self.v_cache = torch.full(shape, fill, dtype=tdt, device=device)
        self.block_tables = torch.from_numpy(self.block_tables_np).to(device)
        self.seq_lens = torch.from_numpy(np.ascontiguousarray(w.seq_lens, np.int32)).to(device)
        self.qsl = torch.from_numpy(w.query_start_loc()).to(device)
        self.q = to_device(w.q, w.dtype, device)
        self.max_seq_len = int(w.seq_lens.max()) if B else 0
        # host swap space: pinned tiles shaped like the device pool's
        hshape = (nh,) + tuple(self.k_cache.shape[1:])
        self.host_k = torch.zeros(hshape, dtype=self.k_cache.dtype, pin_memory=nh > 0)
        self.host_v = torch.zeros(hshape, dtype=self.k_cache.dtype, pin_memory=nh > 0)
        self.k_new = to_device(w.k, w.dtype, device)
        self.v_new = to_device(w.v, w.dtype, device)
        self.slot_mapping = torch.from_numpy(slots_all).to(device)
        if write:
            self.write()
        self.workspace = alloc_workspace(self.k_cache, B, w.total_q_rows, w.num_q_heads,
                                         self.max_seq_len, self.q.dtype)

    @property
    def uses_rows(self) -> bool:
        return bool((self.w.q_rows != 1).any())

    def write(self, stream=None):
        """Carry out every batch in order: swap-outs, copies, swap-ins, slot writes."""
        for outs, copies, ins, slots in self.batches:
            if outs is not None:
                swap_blocks(self.k_cache, self.v_cache, self.host_k, self.host_v, outs,
                            stream=stream)
            if copies is not None:
                copy_blocks(self.k_cache, self.v_cache, copies, stream=stream)
            if ins is not None:
                swap_blocks(self.host_k, self.host_v, self.k_cache, self.v_cache, ins,
                            stream=stream)
            write_kv(self.k_new, self.v_new, slots, self.k_cache, self.v_cache, stream)

    def decode(self, out=None, out_dtype=None, k_cache=None, v_cache=None, stream=None, **kw):
        w = self.w
        return decode(self.q, self.k_cache if k_cache is None else k_cache,
                      self.v_cache if v_cache is None else v_cache, self.block_tables,
                      self.seq_lens, float(w.scale), max_seq_len=self.max_seq_len,
                      query_start_loc=self.qsl if self.uses_rows else None, window=w.window,
                      out=out, out_dtype=out_dtype, workspace=self.workspace, stream=stream,
                      **kw)
