"""Planted mistakes in copies of the oracle must each fail at least one pin (CPU only).

Each mutant is a textual change to a copy of ``oracle/pa_oracle.c``, ``oracle/ledger.py`` or
``oracle/q8.py``:
a dropped term, a wrong sign or index, a transposed operand.  The real oracle is untouched.
"""
import importlib.util
import os
import subprocess

import pytest

import pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

C_MUTANTS = {
    "drop_scale": ("x[t] = scale * acc;", "x[t] = acc;"),
    "exp_sign": ("double w = exp(x[t] - m);", "double w = exp(m - x[t]);"),
    "no_normalise": ("out[i] /= den;", "(void)den;"),
    "block_index": ("int64_t lb = t / block_size;", "int64_t lb = (t + 1) / block_size;"),
    "block_offset": ("(size_t)(t % block_size)) * d;", "(size_t)((t + 1) % block_size)) * d;"),
    "gqa_modulo": ("const int g = h / group;", "const int g = h % num_kv_heads;"),
    "window_off_by_one": ("if (window > 0 && p - window + 1 > 0) lo = p - window + 1;",
                          "if (window > 0 && p - window > 0) lo = p - window;"),
    "k_v_swapped": ("kr[t - lo] = (const char *)kbase + idx * esz;",
                    "kr[t - lo] = (const char *)vbase + idx * esz;"),
    "chunk_rows_reversed": ("const int64_t p = (int64_t)L - nrows + r;",
                            "const int64_t p = (int64_t)L - 1 - r;"),
    "f16_bias": ("v = ldexp((double)(f | 0x400), e - 25);", "v = ldexp((double)(f | 0x400), e - 24);"),
    "scatter_offset": ("int64_t blk = s / block_size, off = s % block_size;",
                       "int64_t blk = s / block_size, off = (s + 1) % block_size;"),
    "max_only_first": ("if (x[t] > m) m = x[t];", "if (t == 0) m = x[t];"),
    "q_row": ("const size_t qrow = ((size_t)(r0 + r) * num_q_heads + h) * d;",
              "const size_t qrow = ((size_t)(r0) * num_q_heads + h) * d;"),
}

PY_MUTANTS = {
    "ceil_to_floor": ("n_blk_after = -(-end // self.bs)", "n_blk_after = end // self.bs + (1 if end % self.bs > 1 else 0)"),
    "share_no_ref": ("            self.ref[b] += 1\n", "            pass\n"),
    "free_lost": ("(self.quarantine if self._busy(block) else self.free).append(block)", "pass"),
    "slot_offset": ("slots.append(b * self.bs + p % self.bs)", "slots.append(b * self.bs + (p + 1) % self.bs)"),
    "keep_off_by_one": ("keep_from = max(0, end - win) if win > 0 else 0",
                        "keep_from = max(0, end - win + 1) if win > 0 else 0"),
    "partial_alloc": ("        if need > len(self.free) +", "        if need > 10**9 +"),
    "shared_write_ok": ("and self.ref[tab[last]] > 1:", "and self.ref[tab[last]] > 2:"),
    "cow_no_copy": ("            self.pending.append((old, b, cur - cow * self.bs))\n",
                    "            pass\n"),
    "cow_short_copy": ("cur - cow * self.bs))", "cur - cow * self.bs - 1))"),
    "cow_no_decref": ("            self.ref[old] -= 1\n", "            pass\n"),
    "cow_pending_ignored": ("if tab[last] in self.touched:", "if False:"),
    "victim_first_arrival": ("self.arrival[s] > self.arrival[best]", "self.arrival[s] < self.arrival[best]"),
    "swap_shared_too": ("alone = [i for i, b in enumerate(tab) if b >= 0 and self.ref[b] == 1]",
                        "alone = [i for i, b in enumerate(tab) if b >= 0]"),
    "swap_in_unchecked": ("        if need > len(self.free):\n            raise OutOfBlocks(f\"seq {seq}: needs {need} blocks, {len(self.free)} free\")\n        tab = self.table[seq]",
                          "        tab = self.table[seq]"),
    "swap_pending_ok": ("        if any(tab[i] in self.touched for i in alone):\n", "        if False:\n"),
    "no_quarantine": ("(self.quarantine if self._busy(block) else self.free)", "self.free"),
    "host_reuse_now": ("                self.host_quarantine.append(h)\n        del self.swapped[seq]",
                       "                self.host_free.append(h)\n        del self.swapped[seq]"),
    "admit_while_swapped": ("if self.swapped and seq not in self.table:", "if False:"),
    "fork_no_ref": ("                self.ref[b] += 1\n        self._create(dst)\n        self.table[dst] = tab",
                    "                pass\n        self._create(dst)\n        self.table[dst] = tab"),
}


Q8_MUTANTS = {
    "q8_qmax": ("QMAX = 127\n", "QMAX = 126\n"),
    "q8_truncate": ("np.rint(r.astype(np.float32))", "np.trunc(r.astype(np.float32))"),
    "q8_signed_max": ("amax = np.abs(g).max(axis=-1)", "amax = g.max(axis=-1)"),
    "q8_scale_slot": ("cache[blk, :, bs, off * w:(off + 1) * w] = sb",
                      "cache[blk, :, bs, (bs - 1 - off) * w:(bs - off) * w] = sb"),
    "q8_copy_no_scales": ("        cache[dst, :, bs, :n * w] = cache[src, :, bs, :n * w]\n", ""),
    "q8_group_order": ("c.reshape(*c.shape[:-1], d // GROUP, GROUP) * s[..., None]",
                       "c.reshape(*c.shape[:-1], GROUP, d // GROUP) * s[..., None, :]"),
}


def _fails_some_pin(orc):
    failed = []
    for pin in pins.ALL:
        try:
            pin(orc)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(e).__name__))
    return failed


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mutant_caught(orc, tmp_path, name):
    old, new = C_MUTANTS[name]
    src = open(os.path.join(ORACLE_DIR, "pa_oracle.c")).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so),
                    str(mut), "-lm"], check=True)
    with orc.using_library(str(so)):
        failed = _fails_some_pin(orc)
    assert failed, f"planted mistake {name} passed every pin"


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_ledger_mutant_caught(orc, tmp_path, monkeypatch, name):
    old, new = PY_MUTANTS[name]
    src = open(os.path.join(ORACLE_DIR, "ledger.py")).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = tmp_path / "ledger_mut.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("ledger_mut", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    for attr in ("Ledger", "SharedBlock", "OutOfBlocks", "LedgerError", "AdmissionClosed",
                 "run_script"):
        monkeypatch.setattr(orc, attr, getattr(mod, attr))
    failed = _fails_some_pin(orc)
    assert failed, f"planted mistake {name} passed every pin"


@pytest.mark.parametrize("name", sorted(Q8_MUTANTS))
def test_q8_mutant_caught(orc, tmp_path, monkeypatch, name):
    old, new = Q8_MUTANTS[name]
    src = open(os.path.join(ORACLE_DIR, "q8.py")).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = tmp_path / "q8_mut.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("q8_mut", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    monkeypatch.setattr(orc, "q8", mod)
    failed = _fails_some_pin(orc)
    assert failed, f"planted mistake {name} passed every pin"
