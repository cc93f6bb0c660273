"""Host checks run inside the sanitizer build (started by tests/test_sanitizers.py in a
process of its own, with the sanitizer runtime preloaded).

    python sanitize_run.py <libpa host build> <oracle build>

It loads the instrumented host half of libpa.so (ledger, argument checks, kernel selection
and workspace layout, with the device half stubbed) and the instrumented C oracle, then
runs on them what the CPU suite runs on the normal builds: the ledger pins, the C++ ledger
against the oracle ledger on every workload script and on random scripts, the argument
checks of every entry point, workspace sizing and plan checks for every workload shape,
and every oracle pin.  Any sanitizer report aborts the process with a non-zero status.
"""
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import paged_kv_cache_144_amd as pa  # noqa: E402
import pins  # noqa: E402
import test_host  # noqa: E402
import workloads  # noqa: E402


def say(*a):
    print("[sanitize]", *a, flush=True)


def decode_host_paths(lib):
    """pa_decode_workspace_size / pa_decode_plan / pa_decode on every workload's shape, with
    fake device addresses (the stubbed launches never touch them), and the refusals."""
    fake = ctypes.c_void_p(0x10000)
    launches = lib.pa_stub_launches
    launches.restype = ctypes.c_int
    codes = {"f32": pa.PA_F32, "f16": pa.PA_F16, "bf16": pa.PA_BF16, "q8_f16": pa.PA_Q8_F16,
             "q8_bf16": pa.PA_Q8_BF16}
    shapes = [("tiny", {}), ("opt13b", {}), ("gqa", {}), ("swa", {}),
              ("prefix_mixed", dict(chunk_lo=1024, chunk_hi=1100)), ("parallel_sampling", {}),
              ("gqa", dict(dtype="q8_bf16")), ("opt13b", dict(block_size=8)),
              ("gqa", dict(block_size=32))]
    for name, kw in shapes:
        w = workloads.make(name, **kw)
        desc = pa.CacheDesc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                            codes[w.dtype])
        B, R = w.num_seqs, w.total_q_rows
        mx = int(w.seq_lens.max())
        n = lib.pa_decode_workspace_size(ctypes.byref(desc), B, R, w.num_q_heads, mx)
        assert n > 0, name
        kname = lib.pa_decode_kernel_name(ctypes.byref(desc), w.num_q_heads, B, w.window)
        assert kname in (b"decode_kernel", b"decode_mfma_kernel", b"decode_group_kernel"), name
        assert (kname == b"decode_group_kernel") == (name == "swa"), (name, kname)
        qsl = fake if (w.q_rows != 1).any() else None
        mb = -(-mx // w.block_size)
        out_dt = pa.PA_F32
        before = launches()
        rc = lib.pa_decode(fake, out_dt, fake, fake, fake, ctypes.byref(desc), fake, mb, fake,
                           qsl, B, R, mx, w.num_q_heads, ctypes.c_float(w.scale), w.window,
                           fake, n, None)
        assert rc == 0 and launches() > before, (name, rc)
        # refusals launch nothing: a short workspace (the size covers chunk rows as well, so
        # only a much smaller one is short for a decode-only batch), a misaligned one, a
        # head count that is no multiple of the KV heads
        before = launches()
        assert lib.pa_decode(fake, out_dt, fake, fake, fake, ctypes.byref(desc), fake, mb,
                             fake, qsl, B, R, mx, w.num_q_heads, ctypes.c_float(w.scale),
                             w.window, fake, 1024, None) == -5
        assert lib.pa_decode(fake, out_dt, fake, fake, fake, ctypes.byref(desc), fake, mb,
                             fake, qsl, B, R, mx, w.num_q_heads, ctypes.c_float(w.scale),
                             w.window, ctypes.c_void_p(0x10008), n, None) == -5
        assert lib.pa_decode(fake, out_dt, fake, fake, fake, ctypes.byref(desc), fake, mb,
                             fake, qsl, B, R, mx, w.num_q_heads + 1, ctypes.c_float(w.scale),
                             w.window, fake, n, None) in (-2, -4)
        assert launches() == before, name
        # the entry point without a workspace argument: same launches, or a refusal
        # when the shape needs more than its fixed workspace
        before = launches()
        rc = lib.pa_decode_noalloc(fake, out_dt, fake, fake, fake, ctypes.byref(desc), fake, mb,
                                   fake, qsl, B, R, mx, w.num_q_heads, ctypes.c_float(w.scale),
                                   w.window, None)
        assert (rc == 0 and launches() > before) or (rc == -5 and launches() == before), name
        say("decode host path", name, kw, "workspace", n)


def main():
    libpa, liboracle = sys.argv[1], sys.argv[2]
    pa.LIB_PATH = libpa
    lib = pa.load()
    say("loaded", libpa)

    # the C++ ledger: pins, workload scripts, random scripts, errors
    shim = test_host._PoolAsOracle(pa)
    for pin in (pins.pin_blocks_and_waste, pins.pin_walkthrough, pins.pin_parallel_sampling,
                pins.pin_cow_rules, pins.pin_swap_ledger, pins.pin_swap_admission,
                pins.pin_batch_reuse, pins.pin_all_or_nothing, pins.pin_window_ledger):
        pin(shim)
        say("ledger pin", pin.__name__)
    orc = oracle
    for name, kw in [("tiny", {}), ("opt13b", {}), ("gqa", {}),
                     ("prefix_mixed", dict(chunk_lo=1024, chunk_hi=1100)),
                     ("swa", dict(batch=6)), ("parallel_sampling", {}), ("swap", {})]:
        test_host.test_pool_matches_oracle_ledger(pa, orc, name, kw)
        say("ledger script", name)
    for seed in range(8):
        test_host.test_pool_random_scripts_match_oracle(pa, orc, seed)
    say("random ledger scripts")
    test_host.test_pool_errors(pa)
    test_host.test_status_strings(pa)
    test_host.test_host_validation_without_gpu(pa)
    say("argument checks")
    decode_host_paths(lib)

    # the C oracle
    with oracle.using_library(liboracle):
        for pin in pins.ALL:
            pin(oracle)
            say("oracle pin", pin.__name__)
    say("clean")


if __name__ == "__main__":
    main()
