"""Token-to-expert permutation and group offsets.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages: each token uses 8 of 384 experts ("Thinking Machines' Inkling 2
Small Trains a 594B Model in 68 Hours", hermes-ai, section "594B weights, 17B
at work", routing row of the specification table), and tokens travel to their
routed experts already in NVFP4 ("Inkling 2 Small uses four-bit training ...",
ai-primer, section "Quantized NVLink and BBBK", dispatch). On one GPU the
dispatch reduces to grouping the routed (token, slot) pairs by local expert
and gathering each token's NVFP4 row.

Reading: the routed pairs of local expert g are ordered by their flat index
t*k + j ascending (a stable grouping), so the result is unique. Pairs routed
to experts outside [e0, e0 + n_local) are not local and are dropped.
"""

import numpy as np

from .mxfp8 import padded_offsets_from_offsets


def permute(topk_ids, e0, n_local):
    """Returns (offsets [n_local+1] int64, padded_offsets [n_local+1] int64,
    row_token [M] int32, row_slot [M] int32) with M = offsets[-1]."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    local_pos = np.nonzero((flat >= e0) & (flat < e0 + n_local))[0]
    le = flat[local_pos] - e0
    order = local_pos[np.argsort(le, kind="stable")]
    counts = np.bincount(le, minlength=n_local)[:n_local]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    padded = padded_offsets_from_offsets(offsets)
    return offsets, padded, (order // k).astype(np.int32), (order % k).astype(np.int32)


def gather_rows(row_token, *arrays):
    """Rows of each array (codes, scales, per-token outer) in permuted order."""
    idx = np.asarray(row_token, dtype=np.int64)
    return tuple(np.asarray(a)[idx] for a in arrays)
