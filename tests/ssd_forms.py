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
* ``chunked_form`` -- the four-term block decomposition (paper card Method 5,
  paper section 6: diagonal blocks, right factors, centre factors, left
  factors), written fresh from the mathematics with numpy einsums. It accepts
  chunk lengths that do not divide T (the last chunk is short).
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
    """Chunked block decomposition for one row: X [T,H,P], la [T,H], B, C [T,G,N].

    Returns (Y [T,H,P], final [H,P,N], start_states [K,H,P,N], chunk_states [K,H,P,N]).
    """
    X = np.asarray(X, np.float64)
    la = np.asarray(la, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    T, H, P = X.shape
    G, N = B.shape[1], B.shape[2]
    heads_g = np.array([_group_of(h, H, G) for h in range(H)])
    Bh = B[:, heads_g, :]                      # [T,H,N] per-head view
    Ch = C[:, heads_g, :]
    bounds = [(c0, min(c0 + Q, T)) for c0 in range(0, T, Q)]
    K = len(bounds)
    Y = np.zeros((T, H, P))
    chunk_states = np.zeros((K, H, P, N))
    chunk_total = np.zeros((K, H))
    css = []
    for k, (c0, c1) in enumerate(bounds):
        cs = np.cumsum(la[c0:c1], axis=0)               # [q,H], restarted per chunk
        css.append(cs)
        q = c1 - c0
        # Diagonal block: exp(segsum) masked below the diagonal before the exp.
        diff = cs[:, None, :] - cs[None, :, :]           # [i,j,H] = cs_i - cs_j
        lower = np.tril(np.ones((q, q), bool))
        seg = np.where(lower[:, :, None], diff, -np.inf)
        Lm = np.exp(seg)                                 # zero above the diagonal
        S = np.einsum("ihn,jhn->ijh", Ch[c0:c1], Bh[c0:c1])
        Y[c0:c1] += np.einsum("ijh,ijh,jhp->ihp", Lm, S, X[c0:c1])
        # Right factor: state at the chunk end from a zero start.
        to_end = np.exp(cs[-1][None, :] - cs)            # [q,H]
        chunk_states[k] = np.einsum("jh,jhp,jhn->hpn", to_end, X[c0:c1], Bh[c0:c1])
        chunk_total[k] = cs[-1]
    # Centre factor: scalar recurrence over chunk states.
    state = np.zeros((H, P, N)) if init is None else np.array(init, np.float64)
    start_states = np.zeros((K, H, P, N))
    for k in range(K):
        start_states[k] = state
        state = np.exp(chunk_total[k])[:, None, None] * state + chunk_states[k]
    # Left factor: carried-in state seen through exp(cumsum) at each position.
    for k, (c0, c1) in enumerate(bounds):
        from_start = np.exp(css[k])                      # [q,H]
        Y[c0:c1] += np.einsum("ih,ihn,hpn->ihp", from_start, Ch[c0:c1], start_states[k])
    return Y, state, start_states, chunk_states
