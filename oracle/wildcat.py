"""fp64 CPU oracle of the WildCat hot path (per head).  Test infrastructure only.

Sources (the pages, cited by title and section):
  * "WildCat: Near-Linear Attention in Theory and Practice", gist.science/de/paper/2602.10056,
    section "Methodik": part 1 (coreset selection by randomly pivoted Cholesky on the kernel
    matrix H = exp(beta K K^T), pivot drawn from the diagonal of the residual kernel matrix),
    part 2 (Nystroem weights W = h(K_S, K_S)^+ h(K_S, K), value compression V_S = W V).
    The French mirror gist.science/fr/paper/2602.10056, "Methodologie", states the same.
  * The abstract (gptget.net/papers/2602.10056, "Abstract"): attend only over a small weighted
    coreset chosen by randomly pivoted Cholesky and weighted optimally.

Where the pages leave a step open, the reading is:
  * beta = 1/sqrt(d) (softmax kernel exp(<x, y>/sqrt(d))).
  * One bin: r sequential pivot steps over all n keys of a head (forward); B contiguous bins
    with r/B steps each, then Nystroem weights over the union of the bins' pivots
    (forward_binned, see there; per-bin weights as an option).
  * The pseudo-inverse of H_SS over such a union is taken by a Cholesky in slot order that
    leaves out every point whose residual is at most DEPENDENT_TOL times its diagonal entry
    (numerically in the span of the earlier points; weight row zero).  For distinct keys
    nothing is left out and it is the inverse.
  * Step t: p = max(diag, 0); C = running sum of p (sequential, fp64); T = C[n-1];
    s = min{i : C_i > u_t T}; g = H[:, s] - F[:, :t] F[s, :t]^T; F[:, t] = g / sqrt(g[s]);
    diag -= F[:, t]^2; diag[s] = 0.  Breakdown (T <= 0, g[s] <= 0 or either not finite)
    stops the loop with rank = t.
  * Weights in the r x (dv+1) form W = H_SS^{-1} H_{S,:} [V, 1]: the pages' V_S with the
    all-ones column appended, which carries the softmax normaliser.  H_SS is solved by
    Cholesky (it is positive definite for distinct keys, so the pseudo-inverse the pages
    write coincides with the inverse).
  * Output O = Y[:, :dv] / Y[:, dv] with Y = exp(beta Q K_S^T) W; no shift is applied.
  * Key centring, when asked for, replaces K by center_keys(K) before every step.

Every function here is plain numpy/scipy in float64.  Inputs given in fp32 or bf16 are
upcast exactly.  Nothing in this package is shared with, or imported by, the HIP path.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import cho_factor, cho_solve

FLAG_BREAKDOWN = 1  # rank < r: the residual vanished (T <= 0) or a pivot's g[s] <= 0
FLAG_NONFINITE = 2  # a non-finite value reached the pivot loop
FLAG_DENOM = 4      # some query row had a Nystroem denominator Y[:, dv] <= 0
FLAG_DEPENDENT = 8  # union weights left out a coreset point numerically dependent on earlier ones

# Relative residual g_j / H_jj at or below which a point of a union coreset counts as dependent:
# 2^-12, above the fp32 rounding of the residual (about r 2^-24 at r = 4096) and far below the
# residuals of distinct keys under bounded inputs.
DEPENDENT_TOL = 2.0 ** -12


def beta_of(d: int) -> float:
    """beta = 1/sqrt(d): the softmax kernel exp(<x, y>/sqrt(d))."""
    return 1.0 / np.sqrt(d)


def kernel(X, Y, beta):
    """Softmax kernel block h(X, Y) = exp(beta X Y^T) ("Methodik" part 1, matrix H)."""
    return np.exp(beta * (np.asarray(X, np.float64) @ np.asarray(Y, np.float64).T))


def initial_residual(K, beta):
    """diag(H) = exp(beta |k_i|^2): the residual diagonal before the first pivot."""
    K = np.asarray(K, np.float64)
    return np.exp(beta * np.einsum("ij,ij->i", K, K))


def sample_pivot(diag, u):
    """Inverse-CDF draw from the residual diagonal ("Methodik" part 1, pivoting rule).

    Returns (s, T, C): s = min{i : C_i > u T} over the running sum C of max(diag, 0),
    or s = -1 when the total T is not positive and finite.  If rounding puts u T at or
    beyond C[n-1], the last index with positive mass is taken.
    """
    p = np.maximum(np.asarray(diag, np.float64), 0.0)
    C = np.cumsum(p)
    T = C[-1] if len(C) else 0.0
    if not (np.isfinite(T) and T > 0.0):
        return -1, T, C
    s = int(np.searchsorted(C, float(u) * T, side="right"))
    if s >= len(C):
        s = int(np.nonzero(p > 0.0)[0][-1])
    return s, T, C


def rpcholesky(K, r, uniforms, beta=None):
    """Randomly pivoted partial Cholesky of H = exp(beta K K^T) with r pivots.

    ``uniforms``: r values u_t in [0, 1) (forced, or the Philox draws of oracle.philox).
    Returns dict with pivots [r] (-1 after rank), F [n, r] (zero after rank),
    diag [n] (final residual diagonal), trace [r + 1] (T_t = sum max(diag, 0) before
    step t, T_r after the last step; zero after rank), rank, flags.
    """
    K = np.asarray(K, np.float64)
    n, d = K.shape
    beta = beta_of(d) if beta is None else beta
    if not 1 <= r <= n:
        raise ValueError("need 1 <= r <= n")
    diag = initial_residual(K, beta)
    F = np.zeros((n, r))
    pivots = -np.ones(r, np.int64)
    trace = np.zeros(r + 1)
    rank, flags = r, 0
    if not np.all(np.isfinite(K)):
        flags |= FLAG_NONFINITE
    for t in range(r):
        s, T, _ = sample_pivot(diag, uniforms[t])
        trace[t] = T if np.isfinite(T) else 0.0
        if s < 0:
            rank, flags = t, flags | FLAG_BREAKDOWN | (0 if np.isfinite(T) else FLAG_NONFINITE)
            break
        h = np.exp(beta * (K @ K[s]))          # column s of H
        g = h - F[:, :t] @ F[s, :t]            # minus what the first t pivots explain
        if not (np.isfinite(g[s]) and g[s] > 0.0):
            rank, flags = t, flags | FLAG_BREAKDOWN | (0 if np.isfinite(g[s]) else FLAG_NONFINITE)
            break
        F[:, t] = g / np.sqrt(g[s])
        diag = diag - F[:, t] ** 2
        diag[s] = 0.0
        pivots[t] = s
    else:
        trace[r] = np.cumsum(np.maximum(diag, 0.0))[-1]
    return dict(pivots=pivots, F=F, diag=diag, trace=trace, rank=rank, flags=flags)


def rpcholesky_follow(K, pivots, uniforms, beta=None):
    """The pivot loop of rpcholesky driven by a given pivot sequence instead of its own draws.

    At step t the residual diagonal is that of the given pivots before t; the step records the
    running-sum interval [C_{s-1}, C_s) of the given pivot s, the total T_t, and the index the
    draw u_t itself selects there (sample_pivot), then eliminates s as rpcholesky does.  With
    the loop's own pivots every u_t T_t lies in its interval; where another implementation's
    pivots part from the draws, the intervals tell how far u_t T_t lies from the choice made.
    Returns dict(lo, hi, T [len(pivots)] (fp64), chosen [len(pivots)] (the draw's own index),
    F [n, len(pivots)]).  Stops early (arrays cut) when a given pivot has no residual left.
    """
    K = np.asarray(K, np.float64)
    n, d = K.shape
    beta = beta_of(d) if beta is None else beta
    pivots = np.asarray(pivots, np.int64)
    r = len(pivots)
    diag = initial_residual(K, beta)
    F = np.zeros((n, r))
    lo, hi, T, chosen = np.zeros(r), np.zeros(r), np.zeros(r), -np.ones(r, np.int64)
    for t in range(r):
        s = int(pivots[t])
        own, Tt, C = sample_pivot(diag, uniforms[t])
        T[t], chosen[t] = Tt, own
        lo[t] = C[s - 1] if s > 0 else 0.0
        hi[t] = C[s]
        g = np.exp(beta * (K @ K[s])) - F[:, :t] @ F[s, :t]
        if not (np.isfinite(g[s]) and g[s] > 0.0):
            return dict(lo=lo[:t], hi=hi[:t], T=T[:t], chosen=chosen[:t], F=F[:, :t])
        F[:, t] = g / np.sqrt(g[s])
        diag = diag - F[:, t] ** 2
        diag[s] = 0.0
    return dict(lo=lo, hi=hi, T=T, chosen=chosen, F=F)


BLOCK_DRAWS = 4  # candidates drawn per pivot slot at most, in block pivot selection


def round_candidates(diag, uniforms, margins=None):
    """Candidates of one round of block pivot selection: drawn one after the other from the
    residual diagonal at the start of the round without replacement, i.e. candidate j is the
    inverse-CDF draw (sample_pivot) from the masses with the round's earlier candidates set to
    zero.  Stops early when no mass is left.  ``margins``: if given, a list that receives, per
    draw, the distance from u T to the nearer end of the chosen interval, over T."""
    p = np.maximum(np.asarray(diag, np.float64), 0.0)
    S = []
    for u in uniforms:
        q = p.copy()
        q[S] = 0.0
        s, T, C = sample_pivot(q, u)
        if s < 0:
            break
        if margins is not None:
            lo = C[s - 1] if s > 0 else 0.0
            margins.append(min(float(u) * T - lo, C[s] - float(u) * T) / T)
        S.append(s)
    return S


def rpcholesky_block(K, r, uniforms, b, beta=None, tol=DEPENDENT_TOL):
    """Randomly pivoted Cholesky with b candidate pivots per round.

    The pages name the sequential pivot selection as a limitation that oversampling could
    lift (future work, gist.science/de/paper/2602.10056, "Bedeutung und Ansprueche").  Reading
    taken: the block variant of randomly pivoted Cholesky, oversampled until the slots are
    full.  Round k draws b candidates from the residual diagonal at the start of the round,
    without replacement (round_candidates, u = uniforms[k b + j]); their kernel columns minus what the
    factor already explains are formed together, G = H[:, S] - F F[S, :]^T; then the
    candidates are taken in order like single pivots: candidate j's residual column g removes
    the round's earlier accepted candidates, and it is accepted into the next free slot when
    g[s] > tol H_ss (one dependent on the accepted ones has a negligible residual and is
    passed over).  After the round diag = diag - sum of the new
    columns squared, 0 at the accepted indices.  Rounds go on until the r slots are full or
    BLOCK_DRAWS r candidates are drawn (``uniforms`` holds that many); a round that finds no
    mass, or running out of draws, stops the loop with rank < r (breakdown).  Pivots fill
    slots 0 .. rank-1 in order, so F[S, :] is lower triangular as for single pivots; trace[t]
    is the total before the round that started with t slots full (other entries zero), and
    trace[r] the total after the last one.  Also returned: ``margins`` [BLOCK_DRAWS r], per
    draw the distance from u T to the nearer end of the interval it selects over T (nan for
    draws never made), and ``slot_round`` [r], the round that filled each slot (-1 if none).
    """
    K = np.asarray(K, np.float64)
    n, d = K.shape
    beta = beta_of(d) if beta is None else beta
    if not 1 <= r <= n:
        raise ValueError("need 1 <= r <= n")
    Hd = initial_residual(K, beta)
    diag = Hd.copy()
    F = np.zeros((n, r))
    pivots = -np.ones(r, np.int64)
    trace = np.zeros(r + 1)
    margins = np.full(BLOCK_DRAWS * r, np.nan)
    slot_round = -np.ones(r, np.int64)
    filled, flags = 0, 0
    if not np.all(np.isfinite(K)):
        flags |= FLAG_NONFINITE
    for k in range(BLOCK_DRAWS * r // b):
        if filled == r:
            break
        mk = []
        S = round_candidates(diag, uniforms[k * b:(k + 1) * b], mk)
        margins[k * b:k * b + len(mk)] = mk
        T = np.cumsum(np.maximum(diag, 0.0))[-1]
        trace[filled] = T if np.isfinite(T) else 0.0
        if not S:
            flags |= FLAG_BREAKDOWN | (0 if np.isfinite(T) else FLAG_NONFINITE)
            break
        f0 = filled
        G = kernel(K, K[S], beta) - F[:, :f0] @ F[S, :f0].T
        for j, s in enumerate(S):
            if filled == r:
                break
            g = G[:, j] - F[:, f0:filled] @ F[s, f0:filled]
            if not (np.isfinite(g[s]) and g[s] > tol * Hd[s]):
                continue
            F[:, filled] = g / np.sqrt(g[s])
            pivots[filled] = s
            slot_round[filled] = k
            filled += 1
        diag = diag - np.sum(F[:, f0:filled] ** 2, axis=1)
        diag[pivots[f0:filled]] = 0.0
    if filled == r:
        trace[r] = np.cumsum(np.maximum(diag, 0.0))[-1]
    else:
        flags |= FLAG_BREAKDOWN
    return dict(pivots=pivots, F=F, diag=diag, trace=trace, rank=filled, flags=flags, margins=margins,
                slot_round=slot_round)


def snap_uniforms_block(K, r, b, raw_uniforms, beta=None, tol=DEPENDENT_TOL):
    """Forced-uniform mode of rpcholesky_block: each candidate's u moves to the centre of the
    interval of the round-start running sum it selects (as snap_uniforms does per step).
    ``raw_uniforms`` and the result hold BLOCK_DRAWS r values; draws of rounds that never run
    stay as they are."""
    K = np.asarray(K, np.float64)
    beta = beta_of(K.shape[1]) if beta is None else beta
    u = np.asarray(raw_uniforms, np.float64).copy()
    out = u.astype(np.float32)
    Hd = initial_residual(K, beta)
    diag = Hd.copy()
    F = np.zeros((K.shape[0], r))
    filled = 0
    for k in range(BLOCK_DRAWS * r // b):
        if filled == r:
            break
        S = []
        p = np.maximum(diag, 0.0)
        for j in range(b):
            q = p.copy()
            q[S] = 0.0
            s, T, C = sample_pivot(q, u[k * b + j])
            if s < 0:
                break
            lo = C[s - 1] if s > 0 else 0.0
            v = np.round((lo + 0.5 * (C[s] - lo)) / T * 2.0 ** 24) * 2.0 ** -24
            v = min(max(v, 0.0), 1.0 - 2.0 ** -24)
            if sample_pivot(q, v)[0] != s:
                raise RuntimeError("snapping moved a candidate")
            out[k * b + j] = v
            S.append(s)
        if not S:
            return out
        # the round itself, as rpcholesky_block runs it
        f0 = filled
        G = kernel(K, K[S], beta) - F[:, :f0] @ F[S, :f0].T
        piv = []
        for j, s in enumerate(S):
            if filled == r:
                break
            g = G[:, j] - F[:, f0:filled] @ F[s, f0:filled]
            if not (np.isfinite(g[s]) and g[s] > tol * Hd[s]):
                continue
            F[:, filled] = g / np.sqrt(g[s])
            piv.append(s)
            filled += 1
        diag = diag - np.sum(F[:, f0:filled] ** 2, axis=1)
        diag[piv] = 0.0
    return out


def snap_uniforms(K, r, raw_uniforms, beta=None, with_pivots=False):
    """Forced-uniform mode: move each u_t to the middle of the CDF interval it selects.

    Runs the pivot loop with the raw draws; at step t the selected index s keeps its
    interval [C_{s-1}, C_s) of the oracle's running sum, and u_t becomes the centre of that
    interval divided by T, rounded to a multiple of 2^-24 (exact in fp32).  Any other
    implementation whose running sum is within half the interval of the oracle's then picks
    the same pivot.  Returns (snapped [r] float32, margin [r]): margin_t is the distance
    from u_t T to the nearer interval end, over T.  Steps after a breakdown keep u = 0.
    With ``with_pivots`` the pivots of the run (-1 after a breakdown) come third.
    """
    K = np.asarray(K, np.float64)
    n, d = K.shape
    beta = beta_of(d) if beta is None else beta
    snapped = np.zeros(r, np.float32)
    margin = np.zeros(r)
    piv = -np.ones(r, np.int64)
    diag = initial_residual(K, beta)
    F = np.zeros((n, r))
    for t in range(r):
        s, T, C = sample_pivot(diag, raw_uniforms[t])
        if s < 0:
            break
        lo = C[s - 1] if s > 0 else 0.0
        u = np.round((lo + 0.5 * (C[s] - lo)) / T * 2.0 ** 24) * 2.0 ** -24
        u = min(max(u, 0.0), 1.0 - 2.0 ** -24)
        s2, _, _ = sample_pivot(diag, u)
        if s2 != s:
            raise RuntimeError(f"snapping moved pivot at step {t}: {s} -> {s2}")
        snapped[t] = u
        margin[t] = min(u * T - lo, C[s] - u * T) / T
        h = np.exp(beta * (K @ K[s]))
        g = h - F[:, :t] @ F[s, :t]
        if not (np.isfinite(g[s]) and g[s] > 0.0):
            break
        F[:, t] = g / np.sqrt(g[s])
        diag = diag - F[:, t] ** 2
        diag[s] = 0.0
        piv[t] = s
    return (snapped, margin, piv) if with_pivots else (snapped, margin)


def weights(K, V, pivots, beta=None):
    """Nystroem weights W = H_SS^{-1} H_{S,:} [V, 1]  (r x (dv+1)).

    "Methodik" part 2: W_pages = h(K_S, K_S)^+ h(K_S, K) and V_S = W_pages V; the returned
    matrix is [V_S, W_pages 1].  ``pivots`` holds the rank valid pivots.
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    beta = beta_of(K.shape[1]) if beta is None else beta
    S = np.asarray(pivots, np.int64)
    KS = K[S]
    H_SS = kernel(KS, KS, beta)
    V1 = np.hstack([V, np.ones((V.shape[0], 1))])
    B = kernel(KS, K, beta) @ V1
    return cho_solve(cho_factor(H_SS, lower=True), B)


def attend(Q, K, pivots, W, beta=None):
    """Attention of every query over the weighted coreset.

    Y = exp(beta Q K_S^T) W and O = Y[:, :dv] / Y[:, dv].  Returns (O, denom, kappa) where
    denom = Y[:, dv] and kappa = sum |P| |W[:, dv]| / |Y[:, dv]| is the row's condition
    number for the normaliser (large kappa: the output row is ill-conditioned).
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    beta = beta_of(K.shape[1]) if beta is None else beta
    S = np.asarray(pivots, np.int64)
    dv = W.shape[1] - 1
    P = kernel(Q, K[S], beta)
    Y = P @ W
    denom = Y[:, dv]
    with np.errstate(divide="ignore", invalid="ignore"):
        O = Y[:, :dv] / denom[:, None]
        kappa = (np.abs(P) @ np.abs(W[:, dv])) / np.abs(denom)
    return O, denom, kappa


def forward(Q, K, V, r, uniforms, beta=None):
    """One head of the WildCat forward: pivots -> weights -> attend."""
    K = np.asarray(K, np.float64)
    beta = beta_of(K.shape[1]) if beta is None else beta
    rpc = rpcholesky(K, r, uniforms, beta)
    S = rpc["pivots"][: rpc["rank"]]
    W = weights(K, V, S, beta)
    O, denom, kappa = attend(Q, K, S, W, beta)
    flags = rpc["flags"] | (FLAG_DENOM if np.any(~(denom > 0.0)) else 0)
    return dict(O=O, W=W, denom=denom, kappa=kappa, pivots=rpc["pivots"], rank=rpc["rank"],
                flags=flags, F=rpc["F"], diag=rpc["diag"], trace=rpc["trace"])


def bin_bounds(n, r, B):
    """Bins of the divide-and-conquer selection: bin b holds the keys [b n/B, (b+1) n/B) and the
    pivot slots [b r/B, (b+1) r/B).  B must divide n and r."""
    if n % B or r % B:
        raise ValueError("the number of bins must divide n and r")
    nb, rb = n // B, r // B
    return [(b * nb, (b + 1) * nb, b * rb, (b + 1) * rb) for b in range(B)]


def independent_slots(H_SS, tol=DEPENDENT_TOL):
    """Which points of a coreset to keep for the pseudo-inverse of H_SS.

    Cholesky of H_SS in slot order, one column at a time: point j's residual is
    g_j = H_jj - sum over the kept earlier points c of L[j, c]^2.  If g_j > tol H_jj the point
    is kept and column j of L is the residual column over sqrt(g_j); otherwise it is left out
    (column j of L stays zero).  A slot whose diagonal entry is zero (an empty slot) is never
    kept.  Returns a boolean mask.
    """
    H = np.asarray(H_SS, np.float64)
    r = H.shape[0]
    L = np.zeros((r, r))
    keep = np.zeros(r, bool)
    for j in range(r):
        g = H[j:, j] - L[j:, :j] @ L[j, :j]
        if g[0] > tol * H[j, j]:
            keep[j] = True
            L[j:, j] = g / np.sqrt(g[0])
    return keep


def weights_union(K, V, slots, beta=None, tol=DEPENDENT_TOL):
    """Nystroem weights over a coreset given slot by slot, W = H_SS^+ H_{S,:} [V, 1].

    "Methodik" part 2 with the union of the bins' pivots as K_S.  ``slots`` holds key indices,
    -1 for an empty slot.  The pseudo-inverse is taken on the points independent_slots keeps:
    W[kept] solves H[kept, kept] W = H[kept, :] [V, 1] (Cholesky), every other row is zero.
    Returns (W [r, dv+1], kept mask [r]).
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    beta = beta_of(K.shape[1]) if beta is None else beta
    slots = np.asarray(slots, np.int64)
    r, dv = len(slots), V.shape[1]
    idx = np.nonzero(slots >= 0)[0]
    KS = K[slots[idx]]
    keep_v = independent_slots(kernel(KS, KS, beta), tol)
    kept = np.zeros(r, bool)
    kept[idx[keep_v]] = True
    W = np.zeros((r, dv + 1))
    if kept.any():
        S = slots[kept]
        V1 = np.hstack([V, np.ones((V.shape[0], 1))])
        W[kept] = cho_solve(cho_factor(kernel(K[S], K[S], beta), lower=True), kernel(K[S], K, beta) @ V1)
    return W, kept


def forward_binned(Q, K, V, r, B, uniforms, beta=None, weights_mode="union", pivot_block=1):
    """One head of divide-and-conquer WildCat with B bins.

    "Methodik" part 1 (efficiency): the input is split into B bins that are processed in
    parallel, at O(n r^2 / B^3 + n r d / B^2), i.e. n/B keys and r/B pivots per bin; part 2:
    once the coreset K_S is chosen, its Nystroem weights.  Readings taken where the pages are
    silent: the bins are contiguous blocks of keys; each bin runs the pivot loop on its own
    keys with slots [b r/B, (b+1) r/B) of ``uniforms``; K_S is the union of the bins' pivots in
    slot order, and
      * weights_mode "union": W = H_SS^+ H_{S,:} [V, 1] over all keys (weights_union);
      * weights_mode "bin": each bin's keys get their own weights on that bin's coreset,
        W_b = H_{S_b S_b}^{-1} H_{S_b, bin b} [V_b, 1]  (a block-diagonal stand-in, cheaper);
    every query attends over the union, Y = exp(beta Q K_S^T) W, O = Y[:, :dv] / Y[:, dv].
    Pivots are returned as key indices of the head, bin by bin; a slot left empty by a
    breakdown in its bin holds -1 and a zero row of W.  pivot_block = b > 1: each bin selects
    with rpcholesky_block (b candidates per round), bin b drawing from uniforms
    [BLOCK_DRAWS s0, BLOCK_DRAWS s1) for its slots [s0, s1).
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n, d = K.shape
    dv = V.shape[1]
    beta = beta_of(d) if beta is None else beta
    if weights_mode not in ("union", "bin"):
        raise ValueError("weights_mode is 'union' or 'bin'")
    pivots = -np.ones(r, np.int64)
    W = np.zeros((r, dv + 1))
    rank, flags = 0, 0
    for k0, k1, s0, s1 in bin_bounds(n, r, B):
        if pivot_block > 1:
            # bin b draws from its own stretch of BLOCK_DRAWS r / B uniforms
            ub = uniforms[BLOCK_DRAWS * s0:BLOCK_DRAWS * s1]
            rpc = rpcholesky_block(K[k0:k1], s1 - s0, ub, pivot_block, beta)
        else:
            rpc = rpcholesky(K[k0:k1], s1 - s0, uniforms[s0:s1], beta)
        rb = rpc["rank"]
        Sb = rpc["pivots"][:rb]
        if rb and weights_mode == "bin":
            W[s0:s0 + rb] = weights(K[k0:k1], V[k0:k1], Sb, beta)
        pivots[s0:s0 + rb] = Sb + k0
        rank += rb
        flags |= rpc["flags"]
    kept = pivots >= 0
    if weights_mode == "union":
        W, kept = weights_union(K, V, pivots, beta)
        if np.any(kept != (pivots >= 0)):
            flags |= FLAG_DEPENDENT
    valid = pivots >= 0
    O, denom, kappa = attend(Q, K, pivots[valid], W[valid], beta)
    flags |= FLAG_DENOM if np.any(~(denom > 0.0)) else 0
    return dict(O=O, W=W, denom=denom, kappa=kappa, pivots=pivots, rank=rank, flags=flags,
                kept=kept)


def snap_uniforms_binned(K, r, B, raw_uniforms, beta=None, pivot_block=1):
    """snap_uniforms (or snap_uniforms_block) applied bin by bin (bin b snaps its slots on its
    own keys).  With pivot_block > 1 the uniforms are BLOCK_DRAWS r long."""
    K = np.asarray(K, np.float64)
    if pivot_block > 1:
        out = np.zeros(BLOCK_DRAWS * r, np.float32)
        for k0, k1, s0, s1 in bin_bounds(K.shape[0], r, B):
            c0, c1 = BLOCK_DRAWS * s0, BLOCK_DRAWS * s1
            out[c0:c1] = snap_uniforms_block(K[k0:k1], s1 - s0, pivot_block, raw_uniforms[c0:c1], beta)
        return out
    out = np.zeros(r, np.float32)
    for k0, k1, s0, s1 in bin_bounds(K.shape[0], r, B):
        out[s0:s1] = snap_uniforms(K[k0:k1], s1 - s0, raw_uniforms[s0:s1], beta)[0]
    return out


def round_bf16(x):
    """fp32 -> bf16 with round-to-nearest-even (finite inputs), returned as float32."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def center_keys(K, dtype="f32"):
    """Key centring ("Methodik" part 3: softmax attention is invariant under a global shift of
    the keys, K <- K - mean of the keys).  Reading for the stored precision: the shifted keys
    are formed in fp64 and stored in the input precision, fp32 (round to nearest) or bf16 by
    way of fp32 (round to nearest even each time).  Returns them as float64 values."""
    K = np.asarray(K, np.float64)
    Kc = (K - K.mean(axis=0)).astype(np.float32)
    if dtype == "bf16":
        Kc = round_bf16(Kc)
    return Kc.astype(np.float64)


def compress(K, V, r, uniforms, B=1, beta=None, weights_mode="union"):
    """COMPRESSKV ("Zentrale Beitraege": the KV cache shrinks from Theta(n d) to O(r d)): the
    rows of a compressed cache for one head, from the keys and values of a prefix.

    The coreset keys K_S and their weight rows W are those of the forward (one bin) or the
    divide-and-conquer forward (B bins); an empty slot (pivot -1) becomes a zero key with a
    zero weight row, so that the cache always holds r rows.  Returns (KR [r, d], WR [r, dv+1],
    pivots, rank, flags).
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Q0 = np.zeros((0, K.shape[1]))
    if B == 1:
        out = forward(Q0, K, V, r, uniforms, beta)
    else:
        out = forward_binned(Q0, K, V, r, B, uniforms, beta, weights_mode)
    piv = out["pivots"]
    valid = piv >= 0
    KR = np.zeros((r, K.shape[1]))
    KR[valid] = K[piv[valid]]
    WR = np.zeros((r, V.shape[1] + 1))
    WR[: len(out["W"])] = out["W"]   # rows of empty slots are zero in W already
    return KR, WR, piv, out["rank"], out["flags"]


def exact_rows(K, V):
    """Cache rows that hold keys exactly: key k_j with weight row [v_j, 1], so that its
    contribution exp(beta q k_j) [v_j, 1] is that of exact softmax attention (numerator and
    normaliser)."""
    V = np.asarray(V, np.float64)
    return np.asarray(K, np.float64), np.hstack([V, np.ones((V.shape[0], 1))])


def decode(Q, KR, WR, beta=None):
    """Attention of decode queries over the rows of a cache: Y = exp(beta Q KR^T) WR,
    O = Y[:, :dv] / Y[:, dv] (compressed rows and exact rows alike)."""
    Q = np.asarray(Q, np.float64)
    KR = np.asarray(KR, np.float64)
    beta = beta_of(KR.shape[1]) if beta is None else beta
    Y = kernel(Q, KR, beta) @ np.asarray(WR, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        return Y[:, :-1] / Y[:, -1:]


def exact_attention(Q, K, V, beta=None):
    """Exact softmax attention softmax(beta Q K^T) V, with a row-max shift."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    beta = beta_of(K.shape[1]) if beta is None else beta
    L = beta * (Q @ K.T)
    L -= L.max(axis=1, keepdims=True)
    E = np.exp(L)
    return (E @ V) / E.sum(axis=1, keepdims=True)


def factor_rows_given_pivots(K, pivots, rows, beta=None):
    """Rows of the partial Cholesky factor F determined by a fixed pivot sequence.

    With L the Cholesky factor of H_SS (pivots in order), F[i, :] = L^{-1} H[S, i]; this is
    what the pivot loop produces for any row once the pivots are fixed, so rows of a large
    factor can be checked one by one.  Returns (F_rows [len(rows), r], diag_rows).
    """
    from scipy.linalg import solve_triangular

    K = np.asarray(K, np.float64)
    beta = beta_of(K.shape[1]) if beta is None else beta
    S = np.asarray(pivots, np.int64)
    KS = K[S]
    L = np.linalg.cholesky(kernel(KS, KS, beta))
    Hr = kernel(KS, K[rows], beta)                  # [r, len(rows)]
    Fr = solve_triangular(L, Hr, lower=True).T
    diag_rows = initial_residual(K[rows], beta) - np.einsum("ij,ij->i", Fr, Fr)
    return Fr, diag_rows


def rel_fro(a, b):
    """Relative Frobenius error |a - b|_F / |b|_F."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))
