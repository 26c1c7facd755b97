"""Acceptance rule for top-k results (test infrastructure only).

Several top-k answers can be correct when logits tie or nearly tie within the
floating-point tolerance, so a result is compared on what is unique and
checked for validity elsewhere.  With c the tolerance coefficient and
tol(v) = c * A[b][v] (A = sum of |r_i * e_i|, from the oracle), a GPU answer
G with scores S is accepted against the oracle's ordered answer O iff

1. G holds k distinct ids in [0, V);
2. |S_j - L[G_j]| <= tol(G_j) for every j;
3. S is non-increasing;
4. |L[G_j] - L[O_j]| <= tol(G_j) + tol(O_j) for every position j.

When every gap between consecutive oracle logits near the top exceeds twice
the tolerance, these force G == O exactly.
"""
from __future__ import annotations

import numpy as np

# |delta| <= c * sum|r_i e_i|: bf16 and Q8_0 tables (f32 accumulation) and f32 tables.
# f16 tables have no stated bound; they run the f32 tables' arithmetic (every
# binary16 value is exact in f32, then f32 FMAs), so they take the f32 bound.
TOL_BF16_Q8 = 2e-3
TOL_F32 = 1e-5


def tol_coeff(dtype: int) -> float:
    return TOL_F32 if dtype in (0, 3) else TOL_BF16_Q8


def check_row(gids, gscores, V: int, c: float, L_at_g, A_at_g, L_at_o=None, A_at_o=None):
    """Returns a list of failure strings (empty = accepted) for one batch row.

    L_at_g / A_at_g: oracle logit and |product| sum at the GPU's ids.
    L_at_o / A_at_o: the same at the oracle's own top-k ids (None: skip rule 4).
    """
    fails = []
    gids = np.asarray(gids, dtype=np.int64)
    gs = np.asarray(gscores, dtype=np.float64)
    k = gids.size
    if np.any(gids < 0) or np.any(gids >= V):
        fails.append(f"ids out of range: {gids.tolist()}")
        return fails
    if np.unique(gids).size != k:
        fails.append(f"duplicate ids: {gids.tolist()}")
    Lg = np.asarray(L_at_g, dtype=np.float64)
    Ag = np.asarray(A_at_g, dtype=np.float64)
    err = np.abs(gs - Lg)
    bad = np.nonzero(err > c * Ag)[0]
    if bad.size:
        j = int(bad[0])
        fails.append(f"score {j} (id {gids[j]}): |{gs[j]!r} - {Lg[j]!r}| > {c * Ag[j]!r}")
    if np.any(np.diff(gs) > 0):
        fails.append(f"scores not non-increasing: {gs.tolist()}")
    if L_at_o is not None:
        Lo = np.asarray(L_at_o, dtype=np.float64)
        Ao = np.asarray(A_at_o, dtype=np.float64)
        gap = np.abs(Lg - Lo)
        bad = np.nonzero(gap > c * (Ag + Ao))[0]
        if bad.size:
            j = int(bad[0])
            fails.append(f"position {j}: gpu id {gids[j]} logit {Lg[j]!r} vs oracle logit {Lo[j]!r}"
                         f" beyond {c * (Ag[j] + Ao[j])!r}")
    return fails


# Probabilities (softmax of L / T over the vocabulary).  With S_j within tol(G_j)
# of the exact logit and every logit within its tol, the log-partition moves by
# at most max_v tol(v) / T (it is 1-Lipschitz in the max norm of L / T), so
#   |ln P_j - ln p(G_j)| <= (tol(G_j) + max_v tol(v)) / T + slack,
# slack covering the f32 arithmetic of the probabilities themselves: exp2 and
# log2 to a few ulps, sums of at most a few hundred rounded non-negative terms
# (relative error <= 2^-24 each) and the rounding of exponent arguments
# (<= 2^-22 |ln p| in all).
PROB_SLACK_ABS = 5e-5
PROB_SLACK_REL = 2.0 ** -20
# Below this the f32 probability may underflow; such entries only need to be tiny.
PROB_LN_FLOOR = -80.0


def check_probs(gids, gprobs, T: float, c: float, L, A):
    """Failure strings for GPU probabilities of the GPU's ids, against the oracle's
    full [B, V] logits L and sums A at temperature T."""
    import oracle
    gids = np.asarray(gids, dtype=np.int64)
    gp = np.asarray(gprobs, dtype=np.float64)
    B, V = L.shape
    ref = oracle.probs_at(L, np.clip(gids, 0, V - 1).astype(np.int32), T)
    fails = []
    for b in range(B):
        tmax = c * float(np.max(A[b]))
        for j in range(gids.shape[1]):
            v = int(gids[b, j])
            lnp = float(np.log(ref[b, j])) if ref[b, j] > 0 else -np.inf
            if not 0.0 <= gp[b, j] <= 1.0:
                fails.append(f"row {b} pos {j}: probability {gp[b, j]!r} outside [0, 1]")
                continue
            if lnp < PROB_LN_FLOOR:
                if gp[b, j] > 1e-30:
                    fails.append(f"row {b} pos {j}: probability {gp[b, j]!r} for ln p = {lnp!r}")
                continue
            lim = (c * float(A[b, v]) + tmax) / T + PROB_SLACK_ABS + PROB_SLACK_REL * abs(lnp)
            err = abs(np.log(gp[b, j]) - lnp) if gp[b, j] > 0 else np.inf
            if err > lim:
                fails.append(f"row {b} pos {j} (id {v}): |ln {gp[b, j]!r} - ({lnp!r})| > {lim!r}")
    return fails


def check_full(gids, gscores, L, A, oids, c: float):
    """All rows, with the oracle's full [B, V] logits L, sums A and top-k ids oids."""
    gids = np.asarray(gids)
    B, V = L.shape
    fails = []
    for b in range(B):
        g = gids[b].astype(np.int64)
        o = np.asarray(oids[b], dtype=np.int64)
        gi = np.clip(g, 0, V - 1)
        f = check_row(g, gscores[b], V, c, L[b, gi], A[b, gi], L[b, o], A[b, o])
        fails += [f"row {b}: {s}" for s in f]
    return fails
