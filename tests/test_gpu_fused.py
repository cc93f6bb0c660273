"""The one-launch decode step (pa_decode_write_attend) against the oracle, on the GPU.

Each case first builds the workload's pool as the oracle does, then puts NaN back into every
sequence's newest slot (as if this step's token had not been written), plans, and calls
pa_decode_write_attend with the step's new rows.  Required:
  * the pool afterwards equals the oracle's scattered pool bit for bit (the newest slots
    written, nothing else touched);
  * the output meets the oracle within the attention tolerance;
  * on the matrix-core kernel the new row enters the same arithmetic as a written one, so the
    output equals pa_decode's on the written pool bit for bit;
  * a needle placed on the newest token (or on an older one) gives that token's V exactly.
"""
import numpy as np
import pytest

import workloads
from helpers import logical_rows

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


def say(*a):
    print("[gpu-fused]", *a, flush=True)


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


def uses_matrix_cores(w):
    g = w.num_q_heads // w.num_kv_heads
    return g in (4, 8) and w.dtype in ("f16", "bf16") and w.block_size == 16


class Step:
    """A workload on the device with its newest tokens taken out of the pool again."""

    def __init__(self, torch, pa, w):
        import bench
        from paged_kv_cache_144_amd.runner import DeviceWorkload
        assert (w.q_rows == 1).all()
        self.w = w
        dw = DeviceWorkload(w, "cuda")
        self.dw = dw
        self.k_full = dw.k_cache.clone()
        self.v_full = dw.v_cache.clone()
        rows = torch.from_numpy(bench.step_rows(w)).cuda()
        self.k_new = dw.k_new.index_select(0, rows).contiguous()
        self.v_new = dw.v_new.index_select(0, rows).contiguous()
        self.slots = dw.slot_mapping.index_select(0, rows).contiguous()
        self.poison()

    def poison(self):
        import paged_kv_cache_144_amd as pa
        nan = self.k_new.clone().fill_(float("nan"))
        pa.write_kv(nan, nan, self.slots, self.dw.k_cache, self.dw.v_cache)

    def run(self, pa, out=None):
        dw, w = self.dw, self.w
        pa.decode(dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.seq_lens, float(w.scale),
                  max_seq_len=dw.max_seq_len, window=w.window, workspace=dw.workspace,
                  step="plan")
        return pa.decode_write_attend(dw.q, self.k_new, self.v_new, dw.k_cache, dw.v_cache,
                                      dw.block_tables, dw.seq_lens, float(w.scale),
                                      max_seq_len=dw.max_seq_len, window=w.window,
                                      workspace=dw.workspace, out=out)


CASES = [
    ("tiny", {}),
    ("tiny", dict(dtype="f16")),
    ("tiny", dict(dtype="bf16", hq=4, hkv=2, d=128)),
    ("tiny", dict(dtype="bf16", hq=8, hkv=1, d=256)),
    ("tiny", dict(dtype="f16", hq=16, hkv=4, d=64)),        # matrix cores, groups of 4
    ("tiny", dict(dtype="bf16", hq=16, hkv=2, d=128)),      # matrix cores, groups of 8
    ("tiny", dict(dtype="f16", hq=16, hkv=2, d=256)),
    ("opt13b", dict(batch=6, lo=64, hi=700)),
    ("opt13b", dict(batch=6, lo=64, hi=700, dtype="f32")),
    ("gqa", dict(batch=12, median=300, lo=16, hi=3000)),
    ("gqa", dict(batch=9, median=400, lo=16, hi=5000, dtype="f16")),
    ("swa", dict(batch=5, lo=1500, hi=6000, window=1024)),
    ("swa", dict(batch=5, lo=1500, hi=6000, window=1000, hq=32, hkv=4, d=128, dtype="bf16")),
    ("swa", dict(batch=4, lo=20, hi=200, window=17, dtype="f16")),
    ("opt13b", dict(batch=6, lo=64, hi=700, block_size=8)),
    ("opt13b", dict(batch=6, lo=64, hi=700, block_size=32)),
    ("gqa", dict(batch=12, median=300, lo=16, hi=3000, block_size=8)),
    ("gqa", dict(batch=12, median=300, lo=16, hi=3000, block_size=32)),
    ("parallel_sampling", dict(plens=[7, 16, 21, 40, 100, 255], samples=3, hq=4, hkv=2, d=64,
                               dtype="f32")),
    ("parallel_sampling", dict(prompts=4, samples=4, lo=64, hi=700)),
    ("parallel_sampling", dict(prompts=3, samples=5, hq=8, hkv=2, d=256, dtype="bf16", lo=20,
                               hi=300)),
    ("swap", dict(batch=12, victims=4, lo=64, hi=700)),
    ("swap", dict(batch=10, victims=3, lo=5, hi=70, hq=16, hkv=4, d=64, dtype="bf16")),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_write_attend_parity(torch, pa, orc, name, kw):
    check_write_attend(torch, pa, orc, name, kw)


# The workloads the benchmark times with the one-launch step (one query row per sequence),
# at their full sizes.
FULL = [("opt13b", {}), ("gqa", {}), ("swa", {}), ("parallel_sampling", {})]


@pytest.mark.slow
@pytest.mark.parametrize("name,kw", FULL, ids=[n for n, _ in FULL])
def test_write_attend_full_size(torch, pa, orc, name, kw):
    """The one-launch step at the workloads' full sizes, in the launch configuration the
    benchmark times: the same requirements as the smaller cases above."""
    check_write_attend(torch, pa, orc, name, kw)


def check_write_attend(torch, pa, orc, name, kw):
    say("case", name, kw)
    w = workloads.make(name, **kw)
    st = Step(torch, pa, w)
    dw = st.dw
    out = st.run(pa).cpu().numpy()
    torch.cuda.synchronize()
    # the newest slots now hold the new rows, and nothing else changed
    assert torch.equal(dw.k_cache.view(torch.uint8), st.k_full.view(torch.uint8)), "k pool"
    assert torch.equal(dw.v_cache.view(torch.uint8), st.v_full.view(torch.uint8)), "v pool"
    ref = orc.Reference(w)
    check_close(out, ref.attention(), f"{name} {kw}")
    assert pa.device_error_bits(dw.workspace) == 0
    if uses_matrix_cores(w):
        # the new row takes the place of the written one in the same arithmetic
        base = dw.decode().cpu().numpy()
        assert np.array_equal(out, base), "matrix-core output differs from pa_decode's"


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("tiny", dict(dtype="bf16", hq=16, hkv=2, d=128)),
    ("opt13b", dict(batch=6, lo=30, hi=400, block_size=8)),
    ("gqa", dict(batch=10, median=300, lo=16, hi=3000)),
    ("swa", dict(batch=4, lo=3000, hi=9000, window=1024)),
])
def test_write_attend_needle(torch, pa, orc, name, kw):
    """A needle on the newest token (taken from the new rows) or on an older one (from the
    pool) gives that token's V bit for bit."""
    say("needle", name, kw)
    w = workloads.make(name, **kw)
    st = Step(torch, pa, w)
    dw = st.dw
    lr = logical_rows(w)
    grp = w.num_q_heads // w.num_kv_heads
    bs = w.block_size
    B = w.num_seqs
    rng = np.random.default_rng(5)
    c = 2048.0
    dw.q.zero_()
    dw.q[:, :, 0] = 1.0
    for newest in (True, False):
        taus = {}
        k_new = torch.zeros_like(st.k_new)
        kc = st.k_full.clone()
        for s in range(B):
            L = int(w.seq_lens[s])
            lo = max(0, L - w.window) if w.window > 0 else 0
            tau = L - 1 if newest or L - 1 == lo else int(rng.integers(lo, L - 1))
            taus[s] = tau
            pos = np.arange(lo, L)
            bt = dw.block_tables_np[s]
            sl = torch.from_numpy(bt[pos // bs].astype(np.int64) * bs + pos % bs).cuda()
            kc[sl // bs, :, sl % bs, :] = 0
            if tau == L - 1:
                k_new[s, :, 0] = c
            else:
                kc[int(bt[tau // bs]), :, tau % bs, 0] = c
        dw.k_cache.copy_(kc)
        dw.v_cache.copy_(st.v_full)
        st.k_new_saved, st.k_new = st.k_new, k_new
        st.poison()
        out = st.run(pa).cpu().numpy()
        st.k_new = st.k_new_saved
        for s, tau in taus.items():
            v = orc.widen(w.v[lr[s][tau]], w.dtype).astype(np.float32)
            for h in range(w.num_q_heads):
                if not np.array_equal(out[s, h], v[h // grp]):
                    raise AssertionError(f"needle newest={newest} seq {s} tau {tau} head {h}: "
                                         f"{out[s, h][:4]} vs {v[h // grp][:4]}")
    assert pa.device_error_bits(dw.workspace) == 0


def test_write_attend_refuses_8bit_caches(torch, pa):
    w = workloads.make("tiny", dtype="q8_f16")
    from paged_kv_cache_144_amd.runner import DeviceWorkload
    dw = DeviceWorkload(w, "cuda")
    k_new = torch.zeros((w.num_seqs, w.num_kv_heads, w.head_dim), dtype=torch.float16,
                        device="cuda")
    with pytest.raises(pa.PAError) as e:
        pa.decode_write_attend(dw.q, k_new, k_new, dw.k_cache, dw.v_cache, dw.block_tables,
                               dw.seq_lens, float(w.scale), max_seq_len=dw.max_seq_len,
                               workspace=dw.workspace)
    assert e.value.code == -4
