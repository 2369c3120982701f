"""Comparison rules between the GPU library and the fp64 oracle.

Indices, counts, permutation and drop mask are compared bit for bit.  A token
whose oracle top-k logit margin z_(k) - z_(k+1) is below 1e-5 is a near tie:
either side of the tie is a correct selection, so such a token's expert set
is only checked to be a valid top-k, and it (plus, under a capacity limit,
every token sharing an expert whose ranks it could shift) is left out of the
element-wise comparisons.  Outputs must satisfy
max|y - y_ref| / max|y_ref| <= 1e-5 (fp32) or 2e-2 (bf16, fp32 accumulation).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

import oracle as O

NEAR_TIE = 1e-5
TOL = {"f32": 1e-5, "bf16": 2e-2}
# fp32 router on the GPU vs fp64: combine weights agree to a few fp32 ulps of
# the logits' dot-product error.
W_TOL = {"f32": 1e-6, "bf16": 2e-5}


def compare_routing(cfg, gpu_idx: np.ndarray, ref: Dict) -> Dict:
    """Check the GPU's top-k against the oracle's.  Returns the mask of tokens
    whose selection is identical (usable for element-wise comparisons) and the
    set of experts whose capacity ranks a near-tie flip could shift."""
    T, k = cfg.T, cfg.k
    gi = gpu_idx.reshape(T, k).astype(np.int64)
    oi = ref["idx"]
    z = ref["z"]
    zs = -np.sort(-z, axis=1)
    near = ref["margin"] < NEAR_TIE
    same = np.ones(T, dtype=bool)
    affected = set()
    for t in range(T):
        if np.array_equal(gi[t], oi[t]):
            continue
        gaps = zs[t, :k - 1] - zs[t, 1:k] if k > 1 else np.array([])
        inner_tie = gaps.size and gaps.min() < NEAR_TIE
        if not near[t]:
            # Only the order inside S_t may differ, and only across an inner tie.
            assert inner_tie and set(gi[t]) == set(oi[t]), (t, gi[t], oi[t])
            continue
        # Near tie at the boundary: the GPU set must still be a valid top-k.
        assert len(set(gi[t])) == k
        assert np.all(z[t, gi[t]] >= zs[t, k - 1] - NEAR_TIE), (t, gi[t], oi[t])
        same[t] = False
        affected |= set(gi[t]) ^ set(oi[t])
    return {"same": same, "affected": affected, "near": int(near.sum()),
            "flipped": int((~same).sum())}


def usable_tokens(cfg, ref, routing) -> np.ndarray:
    """Tokens whose output is uniquely determined given any near-tie flips."""
    ok = routing["same"].copy()
    if routing["affected"] and cfg.capacity_factor is not None:
        for t in range(cfg.T):
            if set(ref["idx"][t]) & routing["affected"]:
                ok[t] = False
    return ok


def compare_dispatch(gpu: Dict[str, np.ndarray], ref_disp: Dict[str, np.ndarray]) -> None:
    for key in ("counts", "offsets", "kept_offsets", "perm", "row_of", "drop"):
        g = np.asarray(gpu[key]).astype(np.int64)
        r = np.asarray(ref_disp[key]).astype(np.int64)
        assert g.shape == r.shape, key
        bad = np.nonzero(g != r)[0]
        assert bad.size == 0, f"{key}: {bad.size} mismatches, first at {bad[:5]}"


def rel_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    return O.relative_error(y_gpu, y_ref)
