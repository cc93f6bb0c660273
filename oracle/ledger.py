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
  * eviction is all-or-nothing per sequence, the victim is the sequence that arrived last,
    and swapping moves an evicted sequence's blocks to CPU memory until GPU memory frees
    up (same notes, scheduling section);
  * while sequences sit in CPU memory no new request is taken; once finished requests free
    GPU memory, the swapped sequences come back first (same section, Swapping under the
    restoring strategies);
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
  * batches: the device carries out a batch's work in the order swap-outs, copies,
    swap-ins, slot writes, the pairs of each kind all at once; ``take_copies`` ends a
    batch.  Hence (a) a copy or a swap-out may not read a block that has writes pending in
    the batch (slots, a copy or a swap-in into it): such a call is refused (SharedBlock)
    and takes nothing; (b) a block, or a host block, freed while work on it is pending in
    the batch joins its free queue only when the batch ends;
  * swapping: the host swap space is a pool of host blocks handed out first-in first-out;
    a swap-out moves only the blocks the sequence holds alone (a block it shares stays on
    the device, still referenced); it needs a host block for each, all or nothing, and
    leaves the sequence unusable (no append, fork or share) until its swap-in, which needs
    a free device block for each host block, all or nothing;
  * arrival: a sequence arrives when it is first created (append, fork, share or window);
    the victim is the resident sequence holding device blocks that arrived last;
  * admission: while any sequence is swapped out, a call that would create a sequence for
    a new request (append, share_prefix or set_window on an unknown id) is refused
    (AdmissionClosed) and changes nothing; a fork is a further sample of a request already
    taken, not a new request, and stays allowed; admission reopens as soon as no sequence
    is swapped out (the last swap-in, or the swapped sequence being dropped);
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


class AdmissionClosed(LedgerError):
    """A new request while sequences are swapped out."""


class Ledger:
    def __init__(self, free_order, block_size: int = 16, host_blocks: int = 0):
        self.bs = int(block_size)
        self.free = deque(int(b) for b in free_order)
        self.ref: dict[int, int] = {}
        self.table: dict[int, list[int]] = {}
        self.length: dict[int, int] = {}
        self.window: dict[int, int] = {}
        self.arrival: dict[int, int] = {}
        self._clock = 0
        # the current batch
        self.pending: list[tuple[int, int, int]] = []   # copies not yet taken
        self.touched: set[int] = set()     # blocks with writes pending (slots, copy, swap-in)
        self.copy_src: set[int] = set()    # blocks a pending copy reads
        self.quarantine: list[int] = []    # freed with work pending: free at the batch end
        # host swap space
        self.host_free = deque(range(int(host_blocks)))
        self.host_quarantine: list[int] = []
        self.swapped: dict[int, list[int]] = {}   # seq -> host block per logical block, or -1

    # -- queries -------------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def num_host_free(self) -> int:
        return len(self.host_free)

    def refcount(self, block: int) -> int:
        return self.ref.get(int(block), 0)

    def block_table(self, seq: int) -> list[int]:
        """Device block per logical block; -1 where released or swapped out."""
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

    def latest_resident(self):
        """The victim: the resident sequence holding device blocks that arrived last."""
        best = None
        for s, tab in self.table.items():
            if s in self.swapped or not any(b >= 0 for b in tab):
                continue
            if best is None or self.arrival[s] > self.arrival[best]:
                best = s
        return best

    # -- operations ----------------------------------------------------------------
    def _create(self, seq: int) -> None:
        if seq not in self.table:
            self.table[seq] = []
            self.length[seq] = 0
            self._clock += 1
            self.arrival[seq] = self._clock

    def _resident(self, seq: int) -> None:
        if seq in self.swapped:
            raise LedgerError(f"seq {seq} is swapped out")

    def _admit(self, seq: int) -> None:
        """A new request waits while any sequence is swapped out."""
        if self.swapped and seq not in self.table:
            raise AdmissionClosed(f"seq {seq}: {len(self.swapped)} sequence(s) swapped out")

    def set_window(self, seq: int, window: int) -> None:
        self._admit(seq)
        self._create(seq)
        self.window[seq] = int(window)

    def take_copies(self) -> list[tuple[int, int, int]]:
        """End the batch: return its copies (src block, dst block, entries) in order."""
        out, self.pending = self.pending, []
        self.touched.clear()
        self.copy_src.clear()
        self.free.extend(self.quarantine)
        self.quarantine = []
        self.host_free.extend(self.host_quarantine)
        self.host_quarantine = []
        return out

    def _busy(self, block: int) -> bool:
        return block in self.touched or block in self.copy_src

    def _release(self, block: int) -> None:
        self.ref[block] -= 1
        if self.ref[block] == 0:
            del self.ref[block]
            (self.quarantine if self._busy(block) else self.free).append(block)

    def append(self, seq: int, n: int) -> list[int]:
        """Append n tokens; return the slot of each (block * bs + offset, or -1)."""
        self._resident(seq)
        self._admit(seq)
        self._create(seq)
        tab = self.table[seq]
        cur = self.length[seq]
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
        freed_now = sum(1 for i in release if self.ref[tab[i]] == 1 and not self._busy(tab[i]))
        if need > len(self.free) + freed_now:
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
            self.copy_src.add(old)
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

    def share_prefix(self, dst: int, src: int, n_tokens: int) -> None:
        """``dst`` (new) begins with the first n_tokens of ``src``, sharing its blocks."""
        self._resident(src)
        if self.table.get(dst) or dst in self.swapped:
            raise LedgerError(f"seq {dst} is not empty")
        self._admit(dst)
        if n_tokens > self.length.get(src, 0):
            raise LedgerError("prefix longer than source")
        nblk = -(-n_tokens // self.bs)
        blocks = self.table[src][:nblk]
        if any(b < 0 for b in blocks):
            raise LedgerError("prefix holds released blocks")
        for b in blocks:
            self.ref[b] += 1
        self._create(dst)
        self.table[dst] = list(blocks)
        self.length[dst] = n_tokens

    def fork(self, dst: int, src: int) -> None:
        """``dst`` (new) becomes a copy of ``src``: its length, window and physical blocks."""
        if self.table.get(dst) or self.length.get(dst, 0) or dst in self.swapped:
            raise LedgerError(f"seq {dst} is not empty")
        if src not in self.table or src == dst:
            raise LedgerError(f"unknown sequence {src}")
        self._resident(src)
        tab = list(self.table[src])
        for b in tab:
            if b >= 0:
                self.ref[b] += 1
        self._create(dst)
        self.table[dst] = tab
        self.length[dst] = self.length[src]
        if src in self.window:
            self.window[dst] = self.window[src]

    def swap_out(self, seq: int) -> list[tuple[int, int]]:
        """Move the blocks ``seq`` holds alone to host blocks; (device, host) pairs."""
        if seq not in self.table:
            raise LedgerError(f"unknown sequence {seq}")
        self._resident(seq)
        tab = self.table[seq]
        alone = [i for i, b in enumerate(tab) if b >= 0 and self.ref[b] == 1]
        if any(tab[i] in self.touched for i in alone):
            raise SharedBlock(f"seq {seq}: a block has writes pending")
        if len(alone) > len(self.host_free):
            raise OutOfBlocks(f"seq {seq}: needs {len(alone)} host blocks")
        where = [-1] * len(tab)
        pairs = []
        for i in alone:
            h = self.host_free.popleft()
            pairs.append((tab[i], h))
            where[i] = h
            self._release(tab[i])
            tab[i] = -1
        self.swapped[seq] = where
        return pairs

    def swap_in(self, seq: int) -> list[tuple[int, int]]:
        """Bring a swapped sequence back into free device blocks; (host, device) pairs."""
        if seq not in self.swapped:
            raise LedgerError(f"seq {seq} is not swapped out")
        where = self.swapped[seq]
        need = sum(1 for h in where if h >= 0)
        if need > len(self.free):
            raise OutOfBlocks(f"seq {seq}: needs {need} blocks, {len(self.free)} free")
        tab = self.table[seq]
        pairs = []
        for i, h in enumerate(where):
            if h >= 0:
                b = self.free.popleft()
                self.ref[b] = 1
                tab[i] = b
                pairs.append((h, b))
                self.touched.add(b)
                self.host_quarantine.append(h)
        del self.swapped[seq]
        return pairs

    def free_seq(self, seq: int) -> None:
        for b in self.table.pop(seq, []):
            if b >= 0:
                self._release(b)
        for h in self.swapped.pop(seq, []):
            if h >= 0:
                self.host_quarantine.append(h)
        self.length.pop(seq, None)
        self.window.pop(seq, None)
        self.arrival.pop(seq, None)


def run_script(ledger: Ledger, script):
    """Apply a workload's ledger script.  Returns ({Append index: slots},
    {Append index: copies that append recorded}, {SwapOut / SwapIn index: block pairs});
    a Flush ends a batch."""
    from workloads import Append, Flush, Fork, Free, SetWindow, SharePrefix, SwapIn, SwapOut

    slots, copies, swaps = {}, {}, {}
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
        elif isinstance(op, SwapOut):
            seq = ledger.latest_resident() if op.seq is None else op.seq
            swaps[i] = (seq, ledger.swap_out(seq))
        elif isinstance(op, SwapIn):
            swaps[i] = (op.seq, ledger.swap_in(op.seq))
        else:  # pragma: no cover
            raise TypeError(op)
    return slots, copies, swaps
