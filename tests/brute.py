"""Library-routine references used to pin the CPU oracle.

Nothing here restates the oracle's loops: attention goes through torch's
``scaled_dot_product_attention`` (float64, CPU) with an explicit boolean
mask built from the visibility rules, and selection goes through numpy's
``lexsort``.  Test infrastructure only.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def decode_bits(a):
    """Stored bits -> float64 through torch's own dtype conversions."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()
    if a.dtype == np.uint8:
        return torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    raise TypeError(a.dtype)


def sdpa_masked(q, keys, vals, mask, scale):
    """q [T, H, D], keys/vals [N, D] (one shared head), mask [T, N] bool.
    Returns out [T, H, D] and lse [T, H] via torch SDPA / logsumexp in float64."""
    qt = torch.as_tensor(q, dtype=torch.float64).permute(1, 0, 2)        # H, T, D
    H = qt.shape[0]
    k = torch.as_tensor(keys, dtype=torch.float64).unsqueeze(0).expand(H, -1, -1)
    v = torch.as_tensor(vals, dtype=torch.float64).unsqueeze(0).expand(H, -1, -1)
    m = torch.as_tensor(mask, dtype=torch.bool)
    out = F.scaled_dot_product_attention(qt, k, v, attn_mask=m.unsqueeze(0), scale=scale)
    logits = torch.einsum("htd,hnd->htn", qt, k) * scale
    logits = logits.masked_fill(~m.unsqueeze(0), float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)
    return out.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


def csa_mask(T, q_pos, idx_row_sets, Nc, R, raw_base, window):
    """Boolean [T, Nc + R]: selected compressed entries, then the raw window
    rows [max(0, t - W + 1), t] that the raw buffer holds."""
    mask = np.zeros((T, Nc + R), bool)
    for t in range(T):
        pos = q_pos + t
        for j in idx_row_sets[t]:
            if 0 <= j < Nc:
                mask[t, j] = True
        if window > 0:
            for tok in range(max(0, pos - window + 1), pos + 1):
                r = tok - raw_base
                if 0 <= r < R:
                    mask[t, Nc + r] = True
    return mask


def select_lexsort(scores, k):
    """Indices of the k best scores under (score desc, index asc), ascending."""
    scores = np.asarray(scores, np.float64)
    order = np.lexsort((np.arange(scores.size), -scores))
    return np.sort(order[:k])
