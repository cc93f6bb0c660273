"""Pins for the CPU oracle: checks against what the pages and plain mathematics fix.

Each ``pin_*`` function takes the oracle module and raises AssertionError on a mismatch.
``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py`` runs them on
copies of the oracle with a planted mistake and requires that some pin fails.
"""
import math
import os

import numpy as np

import workloads
from helpers import contiguous_inputs, logical_rows

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


# ------------------------------------------------------------------ byte accounting
def pin_kv_bytes(orc):
    for model, layers, hkv, d, e, want in _rows("kv_bytes.txt"):
        got = orc.kv_bytes_per_token(int(layers), int(hkv), int(d), int(e))
        assert got == int(want), (model, got, want)
    # the KV-size notes also give about 1.6 GB for a full 2048-token OPT-13B request
    (tok, gb, tol), = _rows("opt13b_request.txt")
    per = orc.kv_bytes_per_token(40, 40, 128, 2)
    assert abs(per * int(tok) / 1e9 - float(gb)) <= float(tol)


def pin_kv_totals(orc):
    shapes = {"qwen3_8b": (8, 128), "mistral_7b": (8, 128), "gemma3_4b": (4, 256)}
    for model, ctx, full, sliding, win, mib in _rows("kv_totals_mib.txt"):
        hkv, d = shapes[model]
        ctx, full, sliding, win = int(ctx), int(full), int(sliding), int(win)
        # a sliding layer holds only its window; a full layer holds the whole context
        total = orc.kv_bytes_per_token(full, hkv, d, 2) * ctx \
            + orc.kv_bytes_per_token(sliding, hkv, d, 2) * orc.tokens_read(ctx, 1, win)
        assert total == int(mib) * 2**20, (model, ctx, total / 2**20, mib)


def pin_kv_q8_bytes(orc):
    # 32 one-byte codes plus one 2-byte scale per 32 values: 34/64 of a 16-bit cache
    for case, m16, m8, exact in _rows("kv_q8_mib.txt"):
        if int(exact):
            # Qwen3-8B: 36 layers, 8 KV heads, head_dim 128, 32K tokens
            b16 = orc.kv_bytes_per_token(36, 8, 128, 2) * 32768
            b8 = orc.kv_bytes_per_token(36, 8, 128, 1, scale_group=32) * 32768
            assert (b16, b8) == (int(m16) * 2**20, int(m8) * 2**20), case
            assert round(100 * b8 / b16, 1) == 53.1
        else:
            for d in (128, 256, 576):
                ratio = orc.kv_bytes_per_token(1, 1, d, 1, 32) / orc.kv_bytes_per_token(1, 1, d, 2)
                assert round(int(m16) * ratio) == int(m8), (case, d)
    assert orc.kv_read_bytes([100, 4096], [1, 1], 1024, 4, 256, 1, 32) == 2 * 4 * 272 * 1124


def pin_kv_read_bytes(orc):
    # one decode row reads every context token once; a window caps it at W
    assert orc.tokens_read(100, 1, 0) == 100
    assert orc.tokens_read(100, 1, 1024) == 100
    assert orc.tokens_read(4096, 1, 1024) == 1024
    # chunk rows: the union of their ranges is the whole context
    assert orc.tokens_read(3000, 512, 0) == 3000
    assert orc.kv_read_bytes([100, 4096], [1, 1], 1024, 4, 256, 2) == 4096 * (100 + 1024)


# ------------------------------------------------------------------ the 8-bit cache
def pin_q8_grid(orc):
    # values already on a group's grid (scale a power of two, largest |code| 127) come back
    # exactly, with that scale; each group has its own scale
    rng = np.random.default_rng(5)
    codes = rng.integers(-127, 128, size=(6, 128)).astype(np.int8)
    codes[:, ::32] = np.where(rng.random((6, 4)) < 0.5, 127, -127)
    exps = rng.integers(-12, 6, size=(6, 4))
    scales = np.ldexp(1.0, exps).astype(np.float16)
    x = (codes.reshape(6, 4, 32) * scales[..., None].astype(np.float32)).reshape(6, 128)
    c, s = orc.q8.quantize(x.astype(np.float32))
    assert np.array_equal(c, codes) and np.array_equal(s, scales)
    assert np.array_equal(orc.q8.dequantize(c, s), x.astype(np.float64))


def pin_q8_rounding(orc):
    rng = np.random.default_rng(6)
    # magnitudes whose scales are normal fp16 numbers (>= 2^-14)
    x = (rng.standard_normal((200, 64)) * np.exp(rng.uniform(-4, 6, (200, 1)))).astype(np.float32)
    c, s = orc.q8.quantize(x)
    sf = s.astype(np.float64)
    err = np.abs(orc.q8.dequantize(c, s) - x).reshape(200, 2, 32)
    # nearest code: at most half a step away (plus the fp32 rounding of x / s)
    assert np.all(err <= sf[..., None] * (0.5 + 1e-5))
    # the scale is the group's largest |x| / 127 rounded to fp16, so the largest code is 127
    assert np.all(np.abs(c.reshape(200, 2, 32)).max(-1) == 127)
    amax = np.abs(x.reshape(200, 2, 32)).max(-1)
    assert np.all(np.abs(sf - amax / 127) <= amax / 127 * 2.0**-11)
    # symmetric, half-way cases to even, zero groups, saturation
    c2, s2 = orc.q8.quantize(-x)
    assert np.array_equal(c2, -c) and np.array_equal(s2, s)
    half = np.zeros((1, 32), np.float32)
    half[0, :4] = [127.0, 2.5, -3.5, 0.5]
    assert orc.q8.quantize(half)[0][0, :4].tolist() == [127, 2, -4, 0]
    z = orc.q8.quantize(np.zeros((2, 32), np.float32))
    assert not z[0].any() and not z[1].astype(np.float32).any()
    # subnormal scales are coarser (codes may saturate), but stay close to the value
    tiny = (rng.standard_normal((20, 32)) * 1e-4).astype(np.float32)
    ct, st = orc.q8.quantize(tiny)
    amx = np.abs(tiny).max(-1, keepdims=True)
    assert float(st.max()) < 2.0**-14
    assert np.all(np.abs(orc.q8.dequantize(ct, st) - tiny) <= 0.25 * amx)
    big = np.full((1, 32), 1e9, np.float32)
    cb, sb = orc.q8.quantize(big)
    assert float(sb[0, 0]) == 65504.0 and np.all(cb == 127)


def pin_q8_paged(orc):
    # paged attention over the 8-bit pool equals plain attention over each token's own
    # quantized-then-decoded rows (no table, no tile): the tile layout, the scatter and the
    # copy-on-write of codes and scales; free and unused slots decode to NaN
    cases = [("tiny", dict(dtype="q8_f16", d=64)), ("tiny", dict(dtype="q8_bf16", d=128)),
             ("swa", dict(batch=3, lo=50, hi=120, window=40, dtype="q8_f16")),
             ("parallel_sampling", dict(plens=[7, 16, 21, 40], samples=3, hq=4, hkv=2, d=64,
                                        dtype="q8_bf16"))]
    for name, kw in cases:
        w = workloads.make(name, **kw)
        got = orc.Reference(w).attention()
        k, v, off, first = contiguous_inputs(w)
        kd = np.stack([orc.q8.dequantize(*orc.q8.quantize(orc.widen(r, w.act).astype(np.float32)))
                       for r in k]).astype(np.float32) if len(k) else k
        vd = np.stack([orc.q8.dequantize(*orc.q8.quantize(orc.widen(r, w.act).astype(np.float32)))
                       for r in v]).astype(np.float32) if len(v) else v
        q = orc.widen(w.q, w.act).astype(np.float32)
        want = orc.contiguous_attention(q, kd, vd, off, first, w.seq_lens, w.scale, "f32",
                                        w.num_q_heads, w.query_start_loc(), w.window)
        assert np.isfinite(got).all(), name
        assert np.array_equal(got, want), name


# ------------------------------------------------------------------ the block ledger
def pin_blocks_and_waste(orc):
    for tok, blocks, empty in _rows("blocks_and_waste.txt"):
        led = orc.Ledger(range(64), 16)
        slots = led.append(0, int(tok))
        tab = led.block_table(0)
        assert len(tab) == int(blocks), (tok, tab)
        assert len(tab) * 16 - int(tok) == int(empty)
        assert led.num_free() == 64 - int(blocks)
        assert sorted(slots) == sorted(set(slots)) and len(slots) == int(tok)
        # each token's slot lies in the block its table entry names
        for p, s in enumerate(slots):
            assert s // 16 == tab[p // 16] and s % 16 == p % 16
    # the 17th token, appended on its own, opens a second block from anywhere in the pool
    led = orc.Ledger([5, 40, 2], 16)
    led.append(0, 16)
    assert led.block_table(0) == [5]
    (s17,) = led.append(0, 1)
    assert led.block_table(0) == [5, 40] and s17 == 40 * 16


def pin_walkthrough(orc):
    led = orc.Ledger(range(16), 4)
    for op, n, filled in _rows("walkthrough_bs4.txt"):
        if op == "append":
            led.append(0, int(n))
            assert led.filled(0) == [int(x) for x in filled.split(",")], led.filled(0)
            led.take_copies()               # each step's writes are done before the next
        else:
            led.free_seq(0)
            assert led.num_free() == 16 and led.block_table(0) == []


def pin_parallel_sampling(orc):
    led = orc.Ledger([7, 1, 3, 4, 5], 4)
    led.append("A1", 7)                    # "Four score and seven years ago our"
    led.fork("A2", "A1")
    for blk, ref in _rows("parallel_sampling_bs4.txt"):
        assert led.refcount(int(blk)) == int(ref)
    assert led.block_table("A1") == led.block_table("A2") == [7, 1]
    # the prompt's slots are written before the samples diverge
    assert led.take_copies() == []
    s1 = led.append("A1", 1)               # "fathers"
    s2 = led.append("A2", 1)               # "mothers"
    t1, t2 = led.block_table("A1"), led.block_table("A2")
    for lb, shared, before, ref in _rows("parallel_sampling_cow_bs4.txt"):
        lb, shared, before, ref = int(lb), int(shared), int(before), int(ref)
        assert (t1[lb] == t2[lb]) == bool(shared)
        assert led.refcount(before) == ref
        if shared:
            assert t1[lb] == t2[lb] == before
    # readings: the first writer copies into the next free block; the last holder writes
    # in place; the copy carries the 3 prompt entries of logical block 1
    assert t1 == [7, 3] and t2 == [7, 1]
    assert led.take_copies() == [(1, 3, 3)]
    assert s1 == [3 * 4 + 3] and s2 == [1 * 4 + 3]
    assert led.refcount(3) == 1
    # freeing one sample drops the counts; freeing both returns every block
    led.free_seq("A2")
    assert led.refcount(7) == 1 and led.refcount(1) == 0 and led.num_free() == 3
    led.free_seq("A1")
    assert led.num_free() == 5


def pin_cow_rules(orc):
    # a fork at a block boundary: the next token opens a block, nothing is copied
    led = orc.Ledger(range(8), 4)
    led.append(0, 8)
    led.fork(1, 0)
    led.take_copies()
    led.append(1, 1)
    assert led.take_copies() == [] and led.refcount(0) == 2 and led.refcount(1) == 2
    assert led.block_table(1) == [0, 1, 2]
    # a copy whose source block got slots in the same batch is refused and takes nothing
    led = orc.Ledger(range(8), 4)
    led.append(0, 6)
    led.fork(1, 0)
    before = (led.num_free(), led.block_table(1), led.refcount(1))
    try:
        led.append(1, 1)
    except orc.SharedBlock:
        pass
    else:
        raise AssertionError("copy from a block with pending writes accepted")
    assert (led.num_free(), led.block_table(1), led.refcount(1)) == before
    assert led.take_copies() == []
    led.append(1, 3)                       # now allowed: copy, then a new block
    assert led.block_table(1) == [0, 2, 3] and led.take_copies() == [(1, 2, 2)]
    # all or nothing: the copy needs a free block too
    led = orc.Ledger(range(2), 4)
    led.append(0, 6)
    led.fork(1, 0)
    led.take_copies()
    try:
        led.append(1, 1)
    except orc.OutOfBlocks:
        pass
    else:
        raise AssertionError("copy without a free block accepted")
    assert led.refcount(1) == 2 and led.take_copies() == [] and led.block_table(1) == [0, 1]


def pin_cow_attention(orc):
    # every sample attends over the prompt plus its own token, as a private sequence would;
    # the unused slots of every block hold NaN, so a missing or short copy shows
    w = workloads.make("parallel_sampling", plens=[7, 16, 21, 40], samples=3, hq=4, hkv=2, d=64)
    ref = orc.Reference(w)
    got = ref.attention()
    k_log, v_log, off, first = contiguous_inputs(w)
    want = orc.contiguous_attention(w.q, k_log, v_log, off, first, w.seq_lens, w.scale, w.dtype,
                                    w.num_q_heads, w.query_start_loc(), w.window)
    assert np.isfinite(got).all()
    assert np.array_equal(got, want)
    # samples of one prompt share its full blocks and no longer share the partial one
    for p, L in enumerate([7, 16, 21, 40]):
        tabs = [list(ref.block_tables[p * 3 + j]) for j in range(3)]
        full = L // 16
        assert all(t[:full] == tabs[0][:full] for t in tabs)
        assert len({t[full] for t in tabs}) == 3
        for b in tabs[0][:full]:
            assert ref.ledger.refcount(b) == 3


def pin_swap_ledger(orc):
    # eviction: all of a sequence or none of it, the latest arrival first, to host blocks
    led = orc.Ledger(range(12), 4, host_blocks=3)
    led.append("a", 9)                     # 3 blocks
    led.append("b", 5)                     # 2 blocks
    led.append("c", 4)                     # 1 block
    led.take_copies()
    assert led.latest_resident() == "c"
    assert led.swap_out("c") == [(5, 0)]
    assert led.latest_resident() == "b" and led.block_table("c") == [-1]
    assert led.num_free() == 7 and led.num_host_free() == 2
    # not enough host blocks: refused, nothing moves
    before = (led.block_table("a"), led.num_free(), led.num_host_free())
    try:
        led.swap_out("a")
    except orc.OutOfBlocks:
        pass
    else:
        raise AssertionError("partial eviction accepted")
    assert (led.block_table("a"), led.num_free(), led.num_host_free()) == before
    # a swapped sequence can do nothing until it is back
    for call in (lambda: led.append("c", 1), lambda: led.fork("d", "c")):
        try:
            call()
        except orc.LedgerError:
            pass
        else:
            raise AssertionError("swapped sequence used")
    # back into the first free blocks; its host block waits for the batch end
    assert led.swap_in("c") == [(0, 6)] and led.block_table("c") == [6]
    assert led.num_host_free() == 2
    led.take_copies()
    assert led.num_host_free() == 3
    # writes pending in the batch block an eviction
    led.append("b", 1)
    try:
        led.swap_out("b")
    except orc.SharedBlock:
        pass
    else:
        raise AssertionError("eviction with pending writes accepted")
    led.take_copies()
    # a block shared with another sequence stays on the device, still referenced
    led.fork("d", "a")
    led.take_copies()
    assert led.latest_resident() == "d" and led.swap_out("d") == []
    assert all(led.refcount(x) == 2 for x in led.block_table("a"))
    assert led.swap_in("d") == []
    # swap-in needs a free device block per host block, all or nothing; a resident
    # sequence ("c", one full block) takes every free block first
    led.swap_out("b")
    led.take_copies()
    led.append("c", 4 * led.num_free())
    try:
        led.swap_in("b")
    except orc.OutOfBlocks:
        pass
    else:
        raise AssertionError("swap-in without free blocks accepted")
    led.free_seq("c")
    led.take_copies()
    assert len(led.swap_in("b")) == 2


def pin_swap_admission(orc):
    # "vLLM and PagedAttention" notes, scheduling, Swapping: while sequences evicted to CPU
    # memory are away, no new request is taken; when finished requests free GPU memory the
    # evicted sequences come back first
    led = orc.Ledger(range(10), 4, host_blocks=4)
    led.append("a", 5)                     # blocks 0, 1
    led.append("b", 3)                     # block 2
    led.append("c", 6)                     # blocks 3, 4
    led.take_copies()
    assert led.swap_out(led.latest_resident()) == [(3, 0), (4, 1)]     # "c" leaves
    led.take_copies()
    state = lambda: (led.num_free(), led.num_host_free(), led.block_table("a"),
                     led.block_table("b"), led.latest_resident())
    before = state()
    refused = 0
    for call in (lambda: led.append("n", 1), lambda: led.append("n", 0),
                 lambda: led.share_prefix("n", "a", 4), lambda: led.set_window("n", 4)):
        try:
            call()
        except orc.AdmissionClosed:
            refused += 1
    assert refused == 4 and state() == before
    assert led.block_table("n") == [] and led.seq_len("n") == 0
    # admitted requests go on: a resident appends and a further sample is forked
    led.append("a", 3)
    led.fork("a2", "a")
    led.take_copies()
    # a resident finishes; the evicted sequence comes back before anyone new
    led.free_seq("b")
    led.take_copies()
    assert len(led.swap_in("c")) == 2
    led.append("n", 2)                     # admission has reopened
    assert led.latest_resident() == "n"
    # dropping the only swapped-out sequence reopens admission as well
    led.take_copies()
    led.swap_out("n")
    try:
        led.append("m", 1)
    except orc.AdmissionClosed:
        pass
    else:
        raise AssertionError("new request taken while a sequence is swapped out")
    led.free_seq("n")
    led.append("m", 1)
    assert led.block_table("m") != []


def pin_batch_reuse(orc):
    # a block freed while a copy still has to read it is not handed out in the same batch
    led = orc.Ledger([0, 1, 2, 3], 4)
    led.append("x", 6)                     # blocks 0, 1
    led.fork("y", "x")
    led.take_copies()
    led.append("x", 1)                     # copies block 1 -> 2
    led.free_seq("y")                      # block 1 has no holder left
    assert led.num_free() == 1             # block 3 only; block 1 waits
    led.append("z", 4)
    assert led.block_table("z") == [3]
    try:
        led.append("w", 1)
    except orc.OutOfBlocks:
        pass
    else:
        raise AssertionError("a block with a pending copy was handed out")
    assert led.take_copies() == [(1, 2, 2)]
    led.append("w", 1)
    assert led.block_table("w") == [1]


def pin_swap_attention(orc):
    # after evictions, residents growing into the freed blocks, finished requests leaving
    # and swap-ins, every sequence attends over exactly its own tokens (unwritten and free
    # slots hold NaN)
    w = workloads.make("swap", batch=10, victims=3, lo=5, hi=70, hq=4, hkv=2, d=64)
    ref = orc.Reference(w)
    got = ref.attention()
    k, v, off, first = contiguous_inputs(w)
    want = orc.contiguous_attention(w.q, k, v, off, first, w.seq_lens, w.scale, w.dtype,
                                    w.num_q_heads, w.query_start_loc(), w.window)
    assert np.isfinite(got).all() and np.array_equal(got, want)
    # the victims were the three last arrivals and came back to other blocks
    outs = [ref.swaps[i] for i in sorted(ref.swaps) if isinstance(w.script[i], workloads.SwapOut)]
    assert [s for s, _ in outs] == [9, 8, 7]


def pin_block_sizes(orc):
    # the block size changes where tokens sit, never what a row attends to; internal waste
    # stays below one block per sequence ("vLLM and PagedAttention" notes, section on the
    # block size; "PagedAttention deep dive", section on waste under 4%)
    for name, kw in [("opt13b", dict(batch=4, lo=20, hi=150)),
                     ("gqa", dict(batch=5, median=60, lo=16, hi=300))]:
        outs = []
        for bs in (4, 8, 16, 32):
            w = workloads.make(name, block_size=bs, **kw)
            ref = orc.Reference(w)
            outs.append(ref.attention())
            for s, L in enumerate(w.seq_lens):
                held = len(ref.ledger.block_table(s))
                assert held == -(-int(L) // bs) and 0 <= held * bs - int(L) < bs
        k, v, off, first = contiguous_inputs(w)
        want = orc.contiguous_attention(w.q, k, v, off, first, w.seq_lens, w.scale, w.dtype,
                                        w.num_q_heads, w.query_start_loc(), w.window)
        for o in outs:
            assert np.array_equal(o, want), name


def pin_all_or_nothing(orc):
    led = orc.Ledger(range(4), 16)
    led.append(0, 40)                       # 3 blocks
    before = (led.num_free(), led.block_table(0), led.seq_len(0))
    try:
        led.append(1, 33)                   # needs 3, 1 free
    except orc.OutOfBlocks:
        pass
    else:
        raise AssertionError("over-allocation accepted")
    assert (led.num_free(), led.block_table(0), led.seq_len(0)) == before
    assert led.block_table(1) == [] and led.seq_len(1) == 0


def pin_window_ledger(orc):
    # a sliding sequence keeps only blocks that hold one of its last W positions
    led = orc.Ledger(range(100), 16)
    led.set_window(0, 32)
    slots = led.append(0, 100)              # keeps positions 68..99 -> blocks 4, 5, 6
    tab = led.block_table(0)
    assert len(tab) == 7 and tab[:4] == [-1] * 4 and all(b >= 0 for b in tab[4:])
    assert slots[:68] == [-1] * 68 and all(s >= 0 for s in slots[68:])
    assert led.num_free() == 97
    led.take_copies()                       # the step's writes are done
    led.append(0, 30)                       # now 130: keeps 98..129 -> blocks 6, 7, 8
    tab = led.block_table(0)
    assert tab[:6] == [-1] * 6 and all(b >= 0 for b in tab[6:]) and led.num_free() == 97
    # within one batch, released blocks that still have writes pending wait for its end
    led = orc.Ledger(range(100), 16)
    led.set_window(0, 32)
    led.append(0, 100)
    led.append(0, 30)
    assert led.num_free() == 95
    led.take_copies()
    assert led.num_free() == 97


# ------------------------------------------------------------------ element widening
def pin_widen(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.widen(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # a few values fixed by the binary16 definition
    for b, x in [(0x3C00, 1.0), (0xC000, -2.0), (0x7BFF, 65504.0), (0x0001, 2.0**-24),
                 (0x0400, 2.0**-14), (0x3555, 0.333251953125)]:
        assert orc.widen(np.array([b], np.uint16), "f16")[0] == x
    got = orc.widen(bits, "bf16")
    with np.errstate(invalid="ignore"):
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], ref[~nan])
    assert orc.widen(np.array([0x3F80, 0x4049], np.uint16), "bf16").tolist() == [1.0, 3.140625]
    x = np.array([1.5, -0.1, 3e-39], np.float32)
    assert orc.widen(x, "f32").tolist() == x.astype(np.float64).tolist()


# ------------------------------------------------------------------ slot write
def pin_write_kv(orc):
    nb, hkv, bs, d = 4, 2, 16, 8
    kc = np.zeros((nb, hkv, bs, d), np.float32)
    vc = np.zeros_like(kc)
    k = np.arange(3 * hkv * d, dtype=np.float32).reshape(3, hkv, d) + 1
    v = -k
    orc.write_kv(k, v, np.array([35, -1, 16], np.int64), kc, vc, bs, "f32")
    # slot 35 = block 2, offset 3; slot 16 = block 1, offset 0; -1 is skipped
    assert np.array_equal(kc[2, :, 3], k[0]) and np.array_equal(vc[2, :, 3], v[0])
    assert np.array_equal(kc[1, :, 0], k[2]) and np.array_equal(vc[1, :, 0], v[2])
    assert np.count_nonzero(kc) == 2 * hkv * d and np.count_nonzero(vc) == 2 * hkv * d


# ------------------------------------------------------------------ attention values
def _tiny(**kw):
    return workloads.make("tiny", **kw)


def pin_one_token(orc):
    # a 1-token context attends to itself only: the output is that token's V
    w = _tiny()
    ref = orc.Reference(w)
    out = ref.attention()
    lr = logical_rows(w)
    s = int(np.nonzero(w.seq_lens == 1)[0][0])
    v0 = orc.widen(w.v[lr[s][0]], w.dtype)
    for h in range(w.num_q_heads):
        assert np.array_equal(out[s, h], v0[h // (w.num_q_heads // w.num_kv_heads)])


def pin_uniform(orc):
    # equal scores (q = 0, or scale = 0) weight every attended token equally: mean of V
    w = _tiny()
    lr = logical_rows(w)
    for mode in ("q0", "scale0"):
        if mode == "q0":
            w.q[:] = 0
        else:
            w = _tiny()
            w.scale = np.float32(0.0)
        out = orc.Reference(w).attention()
        for s in range(w.num_seqs):
            vals = orc.widen(w.v[lr[s]], w.dtype)        # [L][Hkv][d]
            mean = vals.mean(axis=0)
            np.testing.assert_allclose(out[s], mean, rtol=0, atol=1e-13)


def pin_two_tokens(orc):
    # scores ln 3 and 0 give weights 3/4 and 1/4
    w = _tiny(lens=[2], hq=2, hkv=1, d=4)
    w.scale = np.float32(0.5)
    lr = logical_rows(w)[0]
    k = np.zeros((2, 1, 4), np.float32)
    k[0, 0, 0] = 2.0
    w.k[lr] = k
    w.q[:] = 0
    w.q[0, :, 0] = np.float32(math.log(3.0))
    out = orc.Reference(w).attention()
    v = orc.widen(w.v[lr], w.dtype)[:, 0]
    # the float32 query rounds ln 3; the weights follow the rounded score
    x = 0.5 * 2.0 * float(np.float32(math.log(3.0)))
    a = math.exp(x) / (math.exp(x) + 1.0)
    np.testing.assert_allclose(out[0, 0], a * v[0] + (1 - a) * v[1], rtol=0, atol=1e-15)
    assert abs(a - 0.75) < 1e-7


def needle_case(w, s, tau, c=800.0):
    """K = 0 except K_tau = c e_0 for sequence s; q = e_0 for every head."""
    lr = logical_rows(w)
    w.k[lr[s]] = 0
    w.k[lr[s][tau], :, 0] = c
    w.q[:] = 0
    w.q[:, :, 0] = 1.0


def pin_needle(orc):
    # with the needle's score far above the rest, the output is the needle's V bit for bit;
    # every position of every sequence is tried, so a wrong block or offset shows up
    base = _tiny()
    lr = logical_rows(base)
    grp = base.num_q_heads // base.num_kv_heads
    for s in range(base.num_seqs):
        for tau in range(int(base.seq_lens[s])):
            w = _tiny()
            needle_case(w, s, tau)
            out = orc.Reference(w).attention(seqs=[s])
            v = orc.widen(w.v[lr[s][tau]], w.dtype)
            for h in range(w.num_q_heads):
                assert np.array_equal(out[0, h], v[h // grp]), (s, tau, h)


def pin_contiguous(orc):
    for name, kw in [("tiny", {}), ("opt13b", dict(batch=3, lo=20, hi=90)),
                     ("gqa", dict(batch=4, median=40, lo=16, hi=200)),
                     ("prefix_mixed", dict(batch=3, prefix=32, suffix_hi=20, chunks=2,
                                           chunk_rows=5, chunk_lo=20, chunk_hi=60)),
                     ("swa", dict(batch=3, lo=50, hi=120, window=40))]:
        w = workloads.make(name, **kw)
        paged = orc.Reference(w).attention()
        k, v, off, first = contiguous_inputs(w)
        cont = orc.contiguous_attention(w.q, k, v, off, first, w.seq_lens, w.scale, w.dtype,
                                        w.num_q_heads, w.query_start_loc(), w.window)
        assert np.array_equal(paged, cont), name


def pin_permutation(orc):
    # placement is arbitrary: any free order gives the same output bit for bit
    w1 = workloads.make("opt13b", batch=3, lo=20, hi=90)
    w2 = workloads.make("opt13b", batch=3, lo=20, hi=90)
    w2.free_order = np.random.default_rng(99).permutation(w2.free_order)
    r1, r2 = orc.Reference(w1), orc.Reference(w2)
    assert not np.array_equal(r1.block_tables, r2.block_tables)
    assert np.array_equal(r1.attention(), r2.attention())


def _sdpa(w):
    import torch
    k, v, off, first = contiguous_inputs(w)
    from oracle.brute import widen_np
    kd, vd, qd = widen_np(k, w.dtype), widen_np(v, w.dtype), widen_np(w.q, w.dtype)
    qsl = w.query_start_loc()
    out = np.zeros(qd.shape)
    for s in range(w.num_seqs):
        L, n, f = int(w.seq_lens[s]), int(w.q_rows[s]), int(first[s])
        K = torch.from_numpy(kd[off[s]:off[s] + L - f]).permute(1, 0, 2)[None].contiguous()
        V = torch.from_numpy(vd[off[s]:off[s] + L - f]).permute(1, 0, 2)[None].contiguous()
        Q = torch.from_numpy(qd[qsl[s]:qsl[s + 1]]).permute(1, 0, 2)[None].contiguous()
        pos = torch.arange(f, L)
        rowp = torch.arange(L - n, L)[:, None]
        mask = pos[None, :] <= rowp
        if w.window > 0:
            mask &= pos[None, :] > rowp - w.window
        o = torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, attn_mask=mask, scale=float(w.scale), enable_gqa=True)
        out[qsl[s]:qsl[s + 1]] = o[0].permute(1, 0, 2).numpy()
    return out


def pin_sdpa(orc):
    # a library routine (torch's math attention in float64, its own GQA head mapping and
    # boolean masks) on the logical data
    for name, kw in [("tiny", {}), ("gqa", dict(batch=4, median=40, lo=16, hi=200)),
                     ("prefix_mixed", dict(batch=3, prefix=32, suffix_hi=20, chunks=2,
                                           chunk_rows=7, chunk_lo=20, chunk_hi=60)),
                     ("swa", dict(batch=3, lo=50, hi=120, window=40))]:
        w = workloads.make(name, **kw)
        got = orc.Reference(w).attention()
        np.testing.assert_allclose(got, _sdpa(w), rtol=0, atol=1e-12, err_msg=name)


def pin_brute(orc):
    from oracle import brute
    for name, kw in [("tiny", {}), ("gqa", dict(batch=3, median=30, lo=16, hi=70)),
                     ("prefix_mixed", dict(batch=2, prefix=16, suffix_hi=20, chunks=1,
                                           chunk_rows=4, chunk_lo=20, chunk_hi=40)),
                     ("swa", dict(batch=2, lo=50, hi=90, window=24))]:
        w = workloads.make(name, **kw)
        ref = orc.Reference(w)
        got = ref.attention()
        want = brute.paged_attention(w.q, ref.k_cache, ref.v_cache, ref.block_tables,
                                     w.seq_lens, w.scale, w.dtype, w.num_q_heads,
                                     w.query_start_loc(), w.window)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12, err_msg=name)


def pin_window(orc):
    # W >= L is full attention; a window equals full attention over the last W tokens
    w = workloads.make("opt13b", batch=3, lo=30, hi=90)
    full = orc.Reference(w).attention()
    w.window = 4096
    assert np.array_equal(orc.Reference(w).attention(), full)
    W = 20
    w.window = W
    win = orc.Reference(w).attention()
    k, v, off, first = contiguous_inputs(w)
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        lo = off[s] + L - W
        trunc = orc.contiguous_attention(w.q[s:s + 1], k[lo:lo + W], v[lo:lo + W], [0], [0],
                                         [W], w.scale, w.dtype, w.num_q_heads)
        assert np.array_equal(trunc[0], win[s]), s


def pin_chunk_rows(orc):
    # chunk row r (position L - n + r) equals a one-row decode at length L - n + r + 1
    w = workloads.make("prefix_mixed", batch=1, prefix=16, suffix_hi=8, chunks=2, chunk_rows=6,
                       chunk_lo=30, chunk_hi=50)
    ref = orc.Reference(w)
    out = ref.attention()
    qsl = w.query_start_loc()
    for s in range(w.num_seqs):
        n, L = int(w.q_rows[s]), int(w.seq_lens[s])
        for r in range(n):
            one = orc.paged_attention(w.q[qsl[s] + r:qsl[s] + r + 1], ref.k_cache, ref.v_cache,
                                      ref.block_tables[s:s + 1], [L - n + r + 1], w.scale,
                                      w.dtype, w.num_q_heads)
            assert np.array_equal(one[0], out[qsl[s] + r]), (s, r)
    # rows see strictly more context as r grows: the first row ignores the last token
    s = w.num_seqs - 1
    k2 = ref.k_cache.copy()
    blk = ref.block_tables[s][(int(w.seq_lens[s]) - 1) // 16]
    k2[blk, :, (int(w.seq_lens[s]) - 1) % 16] = workloads.to_storage(np.float32([7.0]), w.dtype)[0]
    alt = orc.paged_attention(w.q, k2, ref.v_cache, ref.block_tables, w.seq_lens, w.scale,
                              w.dtype, w.num_q_heads, qsl, 0)
    assert np.array_equal(alt[qsl[s]], out[qsl[s]]) and not np.array_equal(alt[qsl[s + 1] - 1],
                                                                           out[qsl[s + 1] - 1])


def pin_shared_prefix(orc):
    # sharing prefix blocks gives the same output as private copies of the same values
    w = workloads.make("prefix_mixed", batch=4, prefix=48, suffix_hi=30, chunks=1, chunk_rows=3,
                       chunk_lo=20, chunk_hi=40)
    ref = orc.Reference(w)
    shared = ref.attention()
    for b in set(ref.block_tables[:4, :3].ravel().tolist()):
        assert ref.ledger.refcount(b) == 4
    # rebuild with every sequence holding its own prefix copy
    from workloads import Append, Free, SharePrefix
    script = []
    holder = w.meta["holder"]
    pre = next(op for op in w.script if isinstance(op, Append) and op.seq == holder)
    for op in w.script:
        if isinstance(op, SharePrefix):
            script.append(Append(op.dst, pre.n, pre.nv, pre.off))
        elif isinstance(op, Free) or (isinstance(op, Append) and op.seq == holder):
            continue
        else:
            script.append(op)
    w.script = script
    w.num_blocks *= 2                     # private copies need more blocks than sharing
    w.free_order = np.arange(w.num_blocks - 1, dtype=np.int32)
    priv = orc.Reference(w)
    assert len(set(priv.block_tables[:4, 0].tolist())) == 4
    assert np.array_equal(priv.attention(), shared)


def pin_gqa_mapping(orc):
    # with V constant g on KV head g, query head h reads KV head h // (Hq / Hkv)
    w = workloads.make("gqa", batch=2, median=30, lo=16, hi=60)
    w.v[:] = 0
    for g in range(w.num_kv_heads):
        w.v[:, g, :] = workloads.to_storage(np.float32([g]), w.dtype)[0]
    out = orc.Reference(w).attention()
    grp = w.num_q_heads // w.num_kv_heads
    for h in range(w.num_q_heads):
        np.testing.assert_allclose(out[:, h], h // grp, rtol=0, atol=1e-12)


def pin_nan_isolation(orc):
    # free slots, tails of last blocks and the reserved block all hold NaN; none is read
    for name, kw in [("tiny", {}), ("swa", dict(batch=3, lo=50, hi=120, window=40))]:
        w = workloads.make(name, **kw)
        out = orc.Reference(w, poison=True).attention()
        assert np.isfinite(out).all()
        out0 = orc.Reference(w, poison=False).attention()
        assert np.array_equal(out, out0)


ALL = [pin_kv_bytes, pin_kv_totals, pin_kv_q8_bytes, pin_kv_read_bytes, pin_q8_grid,
       pin_q8_rounding, pin_q8_paged, pin_blocks_and_waste, pin_walkthrough,
       pin_parallel_sampling, pin_cow_rules, pin_cow_attention, pin_swap_ledger,
       pin_swap_admission, pin_batch_reuse, pin_swap_attention, pin_block_sizes, pin_all_or_nothing, pin_window_ledger, pin_widen, pin_write_kv,
       pin_one_token, pin_uniform, pin_two_tokens, pin_needle, pin_contiguous, pin_permutation,
       pin_sdpa, pin_brute, pin_window, pin_chunk_rows, pin_shared_prefix, pin_gqa_mapping,
       pin_nan_isolation]
