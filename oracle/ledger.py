"""Oracle model of the KV block ledger (pure Python, slow and plain).

TEST INFRASTRUCTURE ONLY: this package is the CPU oracle.  Only the tests, the smoke check
and the CPU-baseline leg of the benchmark may import it; the library never does.

What the pages fix, and where:
  * the KV cache is cut into fixed-size blocks (16 tokens by default); a sequence takes a
    physical block only when its last block is full, so its 17th token opens a second
    block, and any free block will do ("PagedAttention deep dive", donmain.dev, section on
    splitting the KV cache into blocks);
  * only the last block can be partly empty: a 100-token sequence uses 7 blocks and leaves
    12 slots empty (same page, section on waste falling under 4%);
  * the manager records how many entries each block holds, appends new tokens after the
    prompt's, and frees every block when the request ends (ghkdgus29.github.io, "vLLM and
    PagedAttention", section on basic decoding, block size 4 walk-through);
  * blocks shared by several sequences carry a reference count (same notes, section on
    parallel sampling: two samples share physical blocks 7 and 1, each with count 2);
  * when samples that share a partly filled block each write a different token into it,
    that block is copied and the count drops; fully shared earlier blocks stay shared
    (same section; "PagedAttention deep dive", donmain.dev, section on block sharing:
    copy-on-write at the point where sequences diverge);
  * eviction is all-or-nothing per sequence (same notes, scheduling section);
  * a sliding-window layer only keeps the most recent W tokens (sotaaz.com, section on
    layer kinds).

Readings where the pages are silent (each listed in the design notes):
  * free blocks are handed out first-in first-out, starting from a given order; a block
    whose count drops to zero goes to the back of that queue, in logical-block order;
  * an append that needs more blocks than are free fails and takes nothing;
  * copy-on-write: an append that writes into the partly filled last block while another
    sequence also references it first takes a fresh block (before any new block of the
    same append), records the copy (old block, new block, entries held) and gives the old
    block one reference less; the last remaining holder writes in place;
  * copies are carried out in batches, all pairs of a batch at once, copies before the
    batch's slot writes (``take_copies`` ends a batch).  A copy therefore may not read a
    block that received slots or a copy in the same batch: such an append is refused
    (SharedBlock) and takes nothing;
  * with a window W, after an append of n tokens to a sequence of length c, positions
    before c+n-W are not kept: their slot is -1, a block lying wholly before that point is
    released (table entry -1) and one never allocated stays -1.
"""
from __future__ import annotations

from collections import deque


class LedgerError(Exception):
    pass


class OutOfBlocks(LedgerError):
    pass


class SharedBlock(LedgerError):
    pass


class Ledger:
    def __init__(self, free_order, block_size: int = 16):
        self.bs = int(block_size)
        self.free = deque(int(b) for b in free_order)
        self.ref: dict[int, int] = {}
        self.table: dict[int, list[int]] = {}
        self.length: dict[int, int] = {}
        self.window: dict[int, int] = {}
        self.pending: list[tuple[int, int, int]] = []   # copies not yet taken
        self.touched: set[int] = set()     # blocks given slots or copies since the last take

    # -- queries -------------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, block: int) -> int:
        return self.ref.get(int(block), 0)

    def block_table(self, seq: int) -> list[int]:
        return list(self.table.get(seq, []))

    def seq_len(self, seq: int) -> int:
        return self.length.get(seq, 0)

    def filled(self, seq: int) -> list[int]:
        """Entries held by each logical block of ``seq`` (last one may be partial)."""
        n = self.length.get(seq, 0)
        out = []
        for i in range(len(self.table.get(seq, []))):
            out.append(max(0, min(self.bs, n - i * self.bs)))
        return out

    # -- operations ----------------------------------------------------------------
    def set_window(self, seq: int, window: int) -> None:
        self.table.setdefault(seq, [])
        self.length.setdefault(seq, 0)
        self.window[seq] = int(window)

    def take_copies(self) -> list[tuple[int, int, int]]:
        """End the batch: return its copies (src block, dst block, entries) in order."""
        out, self.pending = self.pending, []
        self.touched.clear()
        return out

    def _release(self, block: int) -> None:
        self.ref[block] -= 1
        if self.ref[block] == 0:
            del self.ref[block]
            self.free.append(block)

    def append(self, seq: int, n: int) -> list[int]:
        """Append n tokens; return the slot of each (block * bs + offset, or -1)."""
        tab = self.table.setdefault(seq, [])
        cur = self.length.setdefault(seq, 0)
        end = cur + n
        win = self.window.get(seq, 0)
        keep_from = max(0, end - win) if win > 0 else 0
        # first logical block that still holds a kept position
        first_kept_blk = keep_from // self.bs
        n_blk_after = -(-end // self.bs)
        # blocks to release: currently held blocks lying wholly before keep_from
        release = [i for i in range(min(first_kept_blk, len(tab))) if tab[i] >= 0]
        # new logical blocks to open
        new_blks = [i for i in range(len(tab), n_blk_after) if i >= first_kept_blk]
        # appending into the current partial last block while another sequence holds it:
        # that block is copied first
        cow = None
        if n > 0 and cur % self.bs != 0:
            last = cur // self.bs
            if last >= first_kept_blk and tab[last] >= 0 and self.ref[tab[last]] > 1:
                if tab[last] in self.touched:
                    raise SharedBlock(f"seq {seq}: shared block {tab[last]} has writes pending")
                cow = last
        need = len(new_blks) + (cow is not None)
        if need > len(self.free) + sum(1 for i in release if self.ref[tab[i]] == 1):
            raise OutOfBlocks(f"seq {seq}: needs {need} blocks, {len(self.free)} free")
        for i in release:
            self._release(tab[i])
            tab[i] = -1
        if cow is not None:
            old = tab[cow]
            b = self.free.popleft()
            self.ref[b] = 1
            self.ref[old] -= 1
            tab[cow] = b
            self.pending.append((old, b, cur - cow * self.bs))
            self.touched.add(b)
        for i in range(len(tab), n_blk_after):
            if i in new_blks:
                b = self.free.popleft()
                self.ref[b] = 1
                tab.append(b)
            else:
                tab.append(-1)
        self.length[seq] = end
        slots = []
        for p in range(cur, end):
            if p < keep_from:
                slots.append(-1)
            else:
                b = tab[p // self.bs]
                slots.append(b * self.bs + p % self.bs)
                self.touched.add(b)
        return slots

    def fork(self, dst: int, src: int) -> None:
        """``dst`` (new) becomes a copy of ``src``: its length, window and physical blocks."""
        if self.table.get(dst) or self.length.get(dst, 0):
            raise LedgerError(f"seq {dst} is not empty")
        if src not in self.table or src == dst:
            raise LedgerError(f"unknown sequence {src}")
        tab = list(self.table[src])
        for b in tab:
            if b >= 0:
                self.ref[b] += 1
        self.table[dst] = tab
        self.length[dst] = self.length[src]
        if src in self.window:
            self.window[dst] = self.window[src]

    def share_prefix(self, dst: int, src: int, n_tokens: int) -> None:
        """``dst`` (new) begins with the first n_tokens of ``src``, sharing its blocks."""
        if self.table.get(dst):
            raise LedgerError(f"seq {dst} is not empty")
        if n_tokens > self.length.get(src, 0):
            raise LedgerError("prefix longer than source")
        nblk = -(-n_tokens // self.bs)
        blocks = self.table[src][:nblk]
        if any(b < 0 for b in blocks):
            raise LedgerError("prefix holds released blocks")
        for b in blocks:
            self.ref[b] += 1
        self.table[dst] = list(blocks)
        self.length[dst] = n_tokens

    def free_seq(self, seq: int) -> None:
        for b in self.table.pop(seq, []):
            if b >= 0:
                self._release(b)
        self.length.pop(seq, None)
        self.window.pop(seq, None)


def run_script(ledger: Ledger, script):
    """Apply a workload's ledger script.  Returns ({Append index: slots},
    {Append index: copies that append recorded}); a Flush ends a batch."""
    from workloads import Append, Flush, Fork, Free, SetWindow, SharePrefix

    slots, copies = {}, {}
    for i, op in enumerate(script):
        if isinstance(op, Append):
            before = len(ledger.pending)
            slots[i] = ledger.append(op.seq, op.n)
            copies[i] = list(ledger.pending[before:])
        elif isinstance(op, Flush):
            ledger.take_copies()
        elif isinstance(op, Fork):
            ledger.fork(op.dst, op.src)
        elif isinstance(op, SharePrefix):
            ledger.share_prefix(op.dst, op.src, op.n_tokens)
        elif isinstance(op, Free):
            ledger.free_seq(op.seq)
        elif isinstance(op, SetWindow):
            ledger.set_window(op.seq, op.window)
        else:  # pragma: no cover
            raise TypeError(op)
    return slots, copies
