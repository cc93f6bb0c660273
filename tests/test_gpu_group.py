"""Group mode (sliding-window decode batches: each (row, KV head) pair split among S
workgroups whose wavefronts combine in LDS, the last workgroup to arrive combining the S
parts) against the oracle and against the wave split, on the GPU.

Required, for every case:
  * pa_decode_kernel_name names the group kernel exactly where group mode applies (the
    per-lane kernel with 16-token blocks, windows of at most 64 blocks per wavefront, at
    most 8 workgroups per pair);
  * the output meets the oracle within the attention tolerance, and stays within 1e-5 of
    the wave split's output (PA_GROUP_MODE=0) on the same inputs;
  * no device error bits; rows with an empty context are zeros; a bad block id sets the
    error bit without disturbing other rows;
  * the one-launch step (pa_decode_write_attend) in group mode writes the newest slots bit
    for bit and meets the oracle.
"""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


def say(*a):
    print("[gpu-group]", *a, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def pa(torch):
    import paged_kv_cache_144_amd as pa
    pa.load()
    return pa


def check_close(got, ref, what):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got - ref)
    rel = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)
    say(f"{what}: max|d|={d.max():.3e} rel_l2={rel:.3e}")
    assert d.max() <= ATOL, f"{what}: max abs {d.max()}"
    assert rel <= RTOL, f"{what}: rel {rel}"


def device(w):
    from paged_kv_cache_144_amd.runner import DeviceWorkload
    return DeviceWorkload(w, "cuda")


def kernel_name(pa, dw, w):
    return pa.decode_kernel_name(dw.k_cache, w.num_q_heads, dw.q.dtype, w.num_seqs, w.window)


# (workload overrides, group mode expected).  Small batches split each pair among up to 8
# workgroups, a batch of 256 pairs keeps one workgroup per pair, tiny windows keep one.
CASES = [
    (dict(batch=5, lo=1500, hi=6000, window=1024), True),                      # f16 g2 d256
    (dict(batch=5, lo=1500, hi=6000, window=1024, dtype="f32"), True),         # 4 wavefronts
    (dict(batch=7, lo=100, hi=5000, window=700, hq=8, hkv=8, d=128, dtype="bf16"), True),
    (dict(batch=6, lo=100, hi=5000, window=2000, hq=32, hkv=4, d=128, dtype="f32"), True),
    (dict(batch=9, lo=16, hi=3000, window=2048, hq=4, hkv=4, d=64, dtype="f16"), True),
    (dict(batch=4, lo=20, hi=200, window=17, dtype="f16"), True),
    (dict(batch=4, lo=20, hi=400, window=1, dtype="bf16"), True),
    (dict(batch=5, lo=1500, hi=6000, window=1024, dtype="q8_f16"), True),
    (dict(batch=5, lo=500, hi=6000, window=1000, hq=16, hkv=8, d=128, dtype="q8_bf16"), True),
    # matrix-core shapes keep their kernel
    (dict(batch=5, lo=1500, hi=6000, window=1000, hq=32, hkv=4, d=128, dtype="bf16"), False),
    # wide windows: the split is raised until a wavefront's share fits 64 blocks
    (dict(batch=3, lo=7000, hi=9000, window=6000, dtype="f32"), True),
    (dict(batch=2, lo=17000, hi=20000, window=16400, hq=8, hkv=8, d=64, dtype="f16"), True),
    # windows past 64 x 4 x 8 blocks keep the wave split
    (dict(batch=2, lo=100, hi=3000, window=33000, hq=8, hkv=8, d=64, dtype="f16"), False),
    # 256 pairs: one workgroup per pair
    (dict(batch=64, lo=1100, hi=3000, window=1024), True),
]


@pytest.mark.parametrize("kw,group", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_group_mode_parity(torch, pa, orc, monkeypatch, kw, group):
    say("case", kw)
    w = workloads.make("swa", **kw)
    dw = device(w)
    name = kernel_name(pa, dw, w)
    assert (name == "decode_group_kernel") == group, name
    ref = orc.Reference(w).attention()
    out = dw.decode().cpu().numpy()
    assert pa.device_error_bits(dw.workspace) == 0
    check_close(out, ref, f"group={group} {kw}")
    monkeypatch.setenv("PA_GROUP_MODE", "0")
    assert kernel_name(pa, dw, w) != "decode_group_kernel"
    base = dw.decode().cpu().numpy()
    monkeypatch.delenv("PA_GROUP_MODE")
    assert np.abs(out - base).max() < 1e-5, "group mode and the wave split disagree"
    if group:
        # a repeated call gives the same bits (each pair's combine order is fixed)
        again = dw.decode().cpu().numpy()
        assert np.array_equal(out, again)


@pytest.mark.parametrize("kw", [
    dict(batch=5, lo=1500, hi=6000, window=1024),
    dict(batch=4, lo=300, hi=5000, window=2000, hq=16, hkv=8, d=128, dtype="q8_f16"),
], ids=["f16", "q8"])
def test_every_split(torch, pa, orc, monkeypatch, kw):
    """Every split from 1 to 8 workgroups per pair (PA_GROUP_SPLIT) meets the oracle, stays
    within 1e-5 of the wave split, and repeats bit for bit (the last workgroup to arrive
    combines the parts in a fixed order)."""
    w = workloads.make("swa", **kw)
    dw = device(w)
    ref = orc.Reference(w).attention()
    monkeypatch.setenv("PA_GROUP_MODE", "0")
    base = dw.decode().cpu().numpy()
    monkeypatch.delenv("PA_GROUP_MODE")
    for s in range(1, 9):
        monkeypatch.setenv("PA_GROUP_SPLIT", str(s))
        assert kernel_name(pa, dw, w) == "decode_group_kernel"
        out = dw.decode().cpu().numpy()
        assert pa.device_error_bits(dw.workspace) == 0
        check_close(out, ref, f"split {s} {kw}")
        assert np.abs(out - base).max() < 1e-5, f"split {s}"
        for _ in range(3):
            assert np.array_equal(out, dw.decode().cpu().numpy()), f"split {s} repeat"
    monkeypatch.delenv("PA_GROUP_SPLIT")


def test_group_mode_empty_rows_and_bad_ids(torch, pa, orc):
    w = workloads.make("swa", batch=6, lo=1500, hi=6000, window=1024)
    dw = device(w)
    assert kernel_name(pa, dw, w) == "decode_group_kernel"
    ref = orc.Reference(w).attention()
    dw.seq_lens[1] = 0
    dw.seq_lens[4] = 0
    out = dw.decode().cpu().numpy()
    assert pa.device_error_bits(dw.workspace) == 0
    for s in (1, 4):
        assert np.array_equal(out[s], np.zeros_like(out[s]))
    for s in (0, 2, 3, 5):
        check_close(out[s], ref[s], f"seq {s}")
    dw.seq_lens[1] = int(w.seq_lens[1])
    dw.seq_lens[4] = int(w.seq_lens[4])
    # a block id past the pool inside sequence 2's window
    L = int(w.seq_lens[2])
    j = (L - 1) // w.block_size - 3
    keep = int(dw.block_tables[2, j])
    dw.block_tables[2, j] = w.num_blocks + 7
    out = dw.decode().cpu().numpy()
    assert pa.device_error_bits(dw.workspace) & 1
    assert np.isfinite(out).all()
    for s in (0, 1, 3, 4, 5):
        check_close(out[s], ref[s], f"untouched seq {s}")
    dw.block_tables[2, j] = keep
    out = dw.decode().cpu().numpy()
    assert pa.device_error_bits(dw.workspace) == 0
    check_close(out, ref, "restored")


@pytest.mark.parametrize("kw", [
    dict(batch=5, lo=1500, hi=6000, window=1024, dtype="f32"),
    dict(batch=7, lo=100, hi=5000, window=700, hq=8, hkv=8, d=128, dtype="bf16"),
    dict(batch=4, lo=20, hi=400, window=1, dtype="f16"),
], ids=["f32-4waves", "bf16-8waves", "window1"])
def test_group_mode_write_attend(torch, pa, orc, kw):
    from test_gpu_fused import Step, check_close as fused_close
    say("write-attend", kw)
    w = workloads.make("swa", **kw)
    st = Step(torch, pa, w)
    dw = st.dw
    assert kernel_name(pa, dw, w) == "decode_group_kernel"
    out = st.run(pa).cpu().numpy()
    torch.cuda.synchronize()
    assert torch.equal(dw.k_cache.view(torch.uint8), st.k_full.view(torch.uint8)), "k pool"
    assert torch.equal(dw.v_cache.view(torch.uint8), st.v_full.view(torch.uint8)), "v pool"
    fused_close(out, orc.Reference(w).attention(), f"write-attend {kw}")
    assert pa.device_error_bits(dw.workspace) == 0


@pytest.mark.parametrize("plan_mode,attend_mode", [("1", "0"), ("0", "1")],
                         ids=["group-plan-wave-attend", "wave-plan-group-attend"])
def test_plan_for_the_other_mode_computes_nothing(torch, pa, monkeypatch, plan_mode,
                                                  attend_mode):
    """An attend call given a plan made for the other decode mode leaves the output alone
    and sets error bit 4 (its kernels check the mode the plan recorded before they read a
    wavefront record)."""
    w = workloads.make("swa", batch=5, lo=1500, hi=6000, window=1024)
    dw = device(w)
    common = dict(max_seq_len=dw.max_seq_len, window=w.window, workspace=dw.workspace)
    args = (dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.seq_lens, float(w.scale))
    monkeypatch.setenv("PA_GROUP_MODE", plan_mode)
    pa.decode(*args, step="plan", **common)
    monkeypatch.setenv("PA_GROUP_MODE", attend_mode)
    out = torch.full(tuple(dw.q.shape), 7.0, dtype=torch.float32, device="cuda")
    pa.decode(*args, step="attend", out=out, **common)
    assert pa.device_error_bits(dw.workspace) & 4
    assert bool((out == 7.0).all())
    # planned again in the attend call's mode, the same workspace computes normally
    pa.decode(*args, step="plan", **common)
    pa.decode(*args, step="attend", out=out, **common)
    assert pa.device_error_bits(dw.workspace) == 0
    assert bool(torch.isfinite(out).all()) and not bool((out == 7.0).all())
