"""Comparison rules shared by the GPU parity tests.

Tolerances (fixed by the method's statement of accuracy for this path):
  * fp32 outputs: per row (one head of one query, or one compressed entry),
    max |gpu - oracle| <= 1e-5 * max |oracle|;
  * bf16 outputs: elementwise |gpu - oracle| <= 2e-2 + 1e-2 |oracle|;
  * top-k sets: bit-exact, except entries whose oracle score lies within
    1e-3 of the oracle's k-th score (near ties, where fp32 and fp64 may
    legitimately order differently); ties of exactly equal scores are never
    exempt: within every group of equal scores the lower indices go first.
"""
from __future__ import annotations

import numpy as np
import torch

EXEMPT = 1e-3


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_rows_rel(gpu, ref, tol=1e-5, what=""):
    g = np.asarray(gpu, np.float64).reshape(-1, np.asarray(gpu).shape[-1])
    r = np.asarray(ref, np.float64).reshape(-1, g.shape[-1])
    err = np.abs(g - r).max(axis=1)
    scale = np.abs(r).max(axis=1)
    bad = err > tol * np.maximum(scale, 1e-30)
    bad &= ~((scale == 0) & (err == 0))
    assert not bad.any(), "%s: %d rows over %.1e row-relative; worst %.3e (row %d)" % (
        what, bad.sum(), tol, (err / np.maximum(scale, 1e-30)).max(), int(np.argmax(bad)))


def assert_bf16_close(gpu, ref, what=""):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    lim = 2e-2 + 1e-2 * np.abs(r)
    err = np.abs(g - r)
    bad = ~(err <= lim)
    assert not bad.any(), "%s: %d / %d elements outside 2e-2 + 1e-2|r|; worst excess %.3e" % (
        what, bad.sum(), bad.size, float((err - lim).max()))


def check_topk_row(gpu_idx, all_scores, k, n_vis, what=""):
    """gpu_idx: [k] int; all_scores: oracle scores of the row ([>= n_vis])."""
    gpu_idx = np.asarray(gpu_idx)
    nsel = min(k, n_vis)
    sel = gpu_idx[:nsel]
    assert (gpu_idx[nsel:] == -1).all(), "%s: padding not -1" % what
    assert (sel >= 0).all() and (sel < n_vis).all(), "%s: index outside [0, n_vis)" % what
    assert (np.diff(sel) > 0).all(), "%s: not strictly ascending" % what
    if nsel == 0 or nsel == n_vis:
        assert np.array_equal(sel, np.arange(nsel)), "%s: all-visible row" % what
        return 0
    s = np.asarray(all_scores[:n_vis], np.float64)
    order = np.lexsort((np.arange(n_vis), -s))
    tau = s[order[nsel - 1]]
    chosen = np.zeros(n_vis, bool)
    chosen[sel] = True
    must = s > tau + EXEMPT
    never = s < tau - EXEMPT
    assert chosen[must].all(), "%s: missed %d clear winners" % (what, (~chosen[must]).sum())
    assert not chosen[never].any(), "%s: took %d clear losers" % (what, chosen[never].sum())
    # exact ties (equal oracle scores) resolve toward the lower index
    ref = np.zeros(n_vis, bool)
    ref[order[:nsel]] = True
    diff = np.nonzero(chosen != ref)[0]
    for j in diff:
        assert abs(s[j] - tau) <= EXEMPT, what
    # exact ties: entries with equal nonzero oracle scores (identical key rows)
    # get equal scores on the device too, so whichever of them the device
    # takes must be the lowest indices of the group - for every such group,
    # whether other near-ties surround it or not
    band = np.nonzero((np.abs(s - tau) <= EXEMPT) & (s != 0))[0]
    vals, counts = np.unique(s[band], return_counts=True)
    for v in vals[counts > 1]:
        grp = np.nonzero(s == v)[0]            # ascending indices
        c = int(chosen[grp].sum())
        assert chosen[grp[:c]].all(), "%s: exact ties not taken lowest index first" % what
    return diff.size


def dev_i64(vals, device="cuda"):
    return torch.tensor(np.asarray(vals, np.int64).reshape(-1), dtype=torch.int64, device=device)


def dev_i32(vals, device="cuda"):
    return torch.tensor(np.asarray(vals, np.int32).reshape(-1), dtype=torch.int32, device=device)
