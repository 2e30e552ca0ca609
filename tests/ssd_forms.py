"""Independent fp64 forms of the SSD layer, used to pin the oracle.

These are written from the pages' other descriptions of the same operator, not
from the recurrence the oracle implements, so agreement is evidence for both:

* ``dual_form`` -- the quadratic (attention-like) form Y = (L o C B^T) X with
  L[t, s] = a_t a_{t-1} ... a_{s+1} for t >= s and 0 above the diagonal
  ("Transformers are SSMs" paper card, Method 2 and Method 3, paper sections
  5.1-5.3; the Chinese wiki note on the same paper, section "对偶形式", gives
  L_ij = a_i x ... x a_{j+1}). Built by brute force: every entry of L is an
  explicit product of decays, and the final state is the weighted sum of the
  rank-one inputs x_s B_s^T.
* ``chunked_form`` -- the block structure of M = L o C B^T cut into chunks
  (paper card Method 3 and Method 5, paper sections 5.2 and 6): within a
  chunk, M is used as it is; between an earlier chunk k' and a later chunk k
  every block of M is a rank-N product left(k) * decay(k' -> k) * right(k')^T,
  with the decays taken from a cumulative log decay over the whole row. Y is
  the sum of those block products over all chunk pairs, computed pair by pair
  with no state carried from chunk to chunk; the state at each chunk's end from
  a zero start and the state entering each chunk are read off the same
  factors. It accepts chunk lengths that do not divide T.
"""
from __future__ import annotations

import numpy as np


def _group_of(h: int, H: int, G: int) -> int:
    return h // (H // G)


def dual_form(X, la, B, C):
    """Brute-force quadratic form for one row: X [T,H,P], la [T,H], B, C [T,G,N].

    Returns (Y [T,H,P], final [H,P,N]).
    """
    X = np.asarray(X, np.float64)
    la = np.asarray(la, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    T, H, P = X.shape
    G, N = B.shape[1], B.shape[2]
    a = np.exp(la)
    Y = np.zeros((T, H, P))
    final = np.zeros((H, P, N))
    for h in range(H):
        g = _group_of(h, H, G)
        L = np.zeros((T, T))
        for t in range(T):
            for s in range(t + 1):
                prod = 1.0
                for k in range(s + 1, t + 1):
                    prod *= a[k, h]
                L[t, s] = prod
        CB = C[:, g, :] @ B[:, g, :].T          # (C_t . B_s)
        Y[:, h, :] = (L * CB) @ X[:, h, :]
        for s in range(T):
            w = 1.0
            for k in range(s + 1, T):
                w *= a[k, h]
            final[h] += w * np.outer(X[s, h, :], B[s, g, :])
    return Y, final


def chunked_form(X, la, B, C, Q: int, init=None):
    """Chunk-pair block factorisation for one row: X [T,H,P], la [T,H], B, C [T,G,N].

    Returns (Y [T,H,P], final [H,P,N], start_states [K,H,P,N], chunk_states [K,H,P,N]).
    """
    X = np.asarray(X, np.float64)
    la = np.asarray(la, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    T, H, P = X.shape
    G, N = B.shape[1], B.shape[2]
    edges = list(range(0, T, Q)) + [T]
    K = len(edges) - 1
    # Whole-row cumulative log decay with a leading zero: the decay from just
    # after position s to position t (s < t) is exp(g[t+1] - g[s+1]); before
    # the first token g = 0, the state the initial state decays from.
    g = np.concatenate([np.zeros((1, H)), np.cumsum(la, axis=0)], axis=0)    # [T+1, H]
    Y = np.zeros((T, H, P))
    chunk_states = np.zeros((K, H, P, N))
    start_states = np.zeros((K, H, P, N))
    h0 = None if init is None else np.asarray(init, np.float64)
    for h in range(H):
        grp = _group_of(h, H, G)
        Bg, Cg = B[:, grp, :], C[:, grp, :]
        # left(k):  rows i of chunk k, C_i scaled by the decay from the chunk's start
        # right(k): rows j of chunk k, B_j scaled by the decay from j to the chunk's end
        left, right = [], []
        for k in range(K):
            b, e = edges[k], edges[k + 1]
            left.append(np.exp(g[b + 1:e + 1, h] - g[b, h])[:, None] * Cg[b:e])
            right.append(np.exp(g[e, h] - g[b + 1:e + 1, h])[:, None] * Bg[b:e])
        for k in range(K):
            b, e = edges[k], edges[k + 1]
            # the block of M on the diagonal, entry by entry
            idx = np.arange(b, e)
            decay = np.exp(g[idx + 1, h][:, None] - g[idx + 1, h][None, :])
            blk = np.tril(decay) * (Cg[b:e] @ Bg[b:e].T)
            Y[b:e, h] += blk @ X[b:e, h]
            # the state at this chunk's end from a zero start: (right factor)^T x
            chunk_states[k, h] = X[b:e, h].T @ right[k]
            # every earlier chunk k2 < k: the rank-N block product, and its share of the
            # state entering chunk k
            for k2 in range(k):
                e2 = edges[k2 + 1]
                between = np.exp(g[b, h] - g[e2, h])          # decay from the end of k2 to the start of k
                Y[b:e, h] += between * (left[k] @ (right[k2].T @ X[edges[k2]:e2, h]))
                start_states[k, h] += between * chunk_states[k2, h]
            if h0 is not None:
                # the initial state, decayed over every token before chunk k
                start_states[k, h] += np.exp(g[b, h]) * h0[h]
                Y[b:e, h] += left[k] @ (np.exp(g[b, h]) * h0[h]).T
    final = np.zeros((H, P, N))
    for h in range(H):
        for k in range(K):
            final[h] += np.exp(g[T, h] - g[edges[k + 1], h]) * chunk_states[k, h]
        if h0 is not None:
            final[h] += np.exp(g[T, h]) * h0[h]
    return Y, final, start_states, chunk_states
