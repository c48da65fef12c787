"""Oracle for stage 2: ragged packing of the scheduled verify rows and tier rounding.

TEST INFRASTRUCTURE (see the package docstring): never imported by the product path.
"""

from __future__ import annotations

import numpy as np


def pack_ragged(windows, context_lens, tiers, src=None, max_rows=None):
    """Pack each request's window rows end to end and round the total up to a tier.

    [SGL] "Ragged verify under full CUDA graphs" and [CSDN] section 3: the scheduled
    verify tokens are laid out back to back in one [total_tokens, hidden] buffer with
    cu_seqlens-style segment starts; the total is rounded up to the nearest captured
    graph size.  Reading for what the pages leave open: rows between the packed total M
    and the tier are zero (they belong to no request); a total above the largest tier is
    an error.

    windows [B] (anchor-inclusive, 1..gamma), context_lens [B], tiers ascending,
    src [B, gamma, ...] or None.  Returns dict(cu_seqlens [B+1], M, tier, dst
    [max_rows, ...] or None, row_req [max_rows], row_pos [max_rows]) where row_req is the
    owning request (-1 for rows that belong to none) and row_pos the absolute sequence
    position of the row's token, ``context_lens[b] + i`` for window row i (-1 otherwise).
    """
    windows = [int(w) for w in windows]
    B = len(windows)
    cu = [0]
    for w in windows:
        cu.append(cu[-1] + w)
    M = cu[-1]
    tier = None
    for t in tiers:
        if t >= M:
            tier = int(t)
            break
    if tier is None:
        raise ValueError("packed total exceeds the largest tier")
    if max_rows is None:
        max_rows = tier
    row_req = np.full(max_rows, -1, dtype=np.int32)
    row_pos = np.full(max_rows, -1, dtype=np.int32)
    for b in range(B):
        for i in range(windows[b]):
            row_req[cu[b] + i] = b
            row_pos[cu[b] + i] = int(context_lens[b]) + i
    dst = None
    if src is not None:
        src = np.asarray(src)
        dst = np.zeros((max_rows,) + src.shape[2:], dtype=src.dtype)
        for b in range(B):
            for i in range(windows[b]):
                dst[cu[b] + i] = src[b, i]
    return {"cu_seqlens": np.asarray(cu, dtype=np.int32), "M": M, "tier": tier, "dst": dst,
            "row_req": row_req, "row_pos": row_pos}
