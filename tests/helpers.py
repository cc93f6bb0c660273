"""Test-side bookkeeping over a workload's script (no paging arithmetic here).

``logical_rows`` replays the script's lengths only: it records, for every batch sequence and
every context position, which row of ``w.k`` / ``w.v`` holds that token's values (or -1 when
the token was never stored, e.g. before a sliding window).
"""
import numpy as np

from workloads import Append, Flush, Fork, Free, SetWindow, SharePrefix


def logical_rows(w):
    rows = {}
    for op in w.script:
        if isinstance(op, Append):
            r = rows.setdefault(op.seq, [])
            missing = op.n - op.nv
            r.extend([-1] * missing)
            r.extend(range(op.off, op.off + op.nv))
        elif isinstance(op, SharePrefix):
            rows[op.dst] = list(rows[op.src][:op.n_tokens])
        elif isinstance(op, Fork):
            rows[op.dst] = list(rows[op.src])
        elif isinstance(op, (Free, Flush)):
            pass
        elif isinstance(op, SetWindow):
            rows.setdefault(op.seq, [])
    return [np.asarray(rows.get(s, []), np.int64) for s in range(w.num_seqs)]


def contiguous_inputs(w):
    """Per-sequence logical K/V stacked: (k_log, v_log, tok_off, first_pos)."""
    lr = logical_rows(w)
    first = np.zeros(w.num_seqs, np.int32)
    off = np.zeros(w.num_seqs, np.int64)
    parts = []
    total = 0
    for s, r in enumerate(lr):
        stored = np.nonzero(r >= 0)[0]
        f = int(stored[0]) if stored.size else len(r)
        assert np.all(r[f:] >= 0)
        first[s] = f
        off[s] = total
        parts.append(r[f:])
        total += len(r) - f
    idx = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    return w.k[idx], w.v[idx], off, first
