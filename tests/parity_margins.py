"""Error margins of the GPU parity checks, collected over a test session.

Every comparison against the oracle records its errors here; ``conftest.py``
prints them at the end of the session (after the pass/fail dots, so they stay
visible under ``pytest -q``): one line per full-size workload, and one summary
line with the smallest margin over all the other comparisons.

A margin is bar / error: 1.0 means the error sits exactly on its bar.
"""
from __future__ import annotations

ROWS = []   # (tag, full_size, out_maxabs, out_rel, fin_rel or None, fin_bar or None, worst_head or None)


def record(tag, full_size, out_maxabs, out_rel, fin_rel=None, fin_bar=None, worst_head=None):
    ROWS.append((tag, bool(full_size), float(out_maxabs), float(out_rel),
                 None if fin_rel is None else float(fin_rel), fin_bar, worst_head))


def _margin(err, bar):
    return float('inf') if err <= 0 else bar / err


def lines(out_maxabs_bar, out_rel_bar):
    """The summary as text lines (empty if nothing was recorded)."""
    if not ROWS:
        return []
    out = [f"{'check':<34} {'out max-abs':>11} {'out rel-L2':>10} {'final rel':>9} {'margin':>6}  worst head"]

    def row_margin(r):
        _, _, mae, rel, frel, fbar, _ = r
        m = min(_margin(mae, out_maxabs_bar), _margin(rel, out_rel_bar))
        if frel is not None:
            m = min(m, _margin(frel, fbar))
        return m

    for r in ROWS:
        if not r[1]:
            continue
        tag, _, mae, rel, frel, fbar, wh = r
        fs = f"{frel:9.2e}" if frel is not None else f"{'-':>9}"
        out.append(f"{tag[:34]:<34} {mae:11.2e} {rel:10.2e} {fs} {row_margin(r):6.2f}  {wh or ''}")
    small = [r for r in ROWS if not r[1]]
    if small:
        worst = min(small, key=row_margin)
        out.append(f"other checks: {len(small)}, smallest margin {row_margin(worst):.2f} ({worst[0][:40]})")
    out.append(f"bars: out max-abs {out_maxabs_bar:g}, out rel-L2 {out_rel_bar:g}, "
               "final rel-L2 2e-3 (fp32 state) / 5e-3 (bf16 state)")
    return out
