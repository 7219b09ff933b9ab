"""fp64 definitions of the chunk coefficients of the per-token recurrence (test infrastructure).

Derived from the momentum / forgetting recurrence (titans-pytorch-mlx README, Core
Equations, Eq. 13-14) with every gradient of a chunk taken at the chunk-start weights
("ATLAS ... | Summary", section 3.3).  Unrolling C steps of
    S_t = eta_t S_{t-1} - theta_t g_t,   W_t = (1 - alpha_t) W_{t-1} + S_t
gives S_end = P S_0 - sum_j cS_j g_j and W_end = beta W_0 + a_S S_0 - sum_j cW_j g_j with
    cS_j = theta_j prod_{l>j} eta_l
    cW_j = theta_j sum_{u>=j} prod_{l>u} (1 - alpha_l) prod_{j<l<=u} eta_l
    P = prod eta,  beta = prod (1 - alpha),  a_S = sum_u prod_{l>u} (1 - alpha_l) prod_{l<=u} eta_l
written out here as plain products and sums (no scan).  With an Omega window c the step-t
gradient is sum_{i=t-c+1..t} gamma_i g_i (ATLAS summary, section 3.2), so g_i's coefficient
is gamma_i times the sum of the step coefficients of the steps t in [i, i+c-1] inside the chunk.
Pinned against the literal recurrence in the oracle tests.
"""

from __future__ import annotations

import numpy as np


def chunk_coefficients(theta, eta, alpha):
    """One chunk's per-token gates -> (cW [C], cS [C], (P, beta, a_S))."""
    th = np.asarray(theta, dtype=np.float64)
    et = np.asarray(eta, dtype=np.float64)
    om = 1.0 - np.asarray(alpha, dtype=np.float64)
    C = len(th)
    cS = np.array([th[j] * np.prod(et[j + 1:]) for j in range(C)])
    cW = np.array([th[j] * sum(np.prod(om[u + 1:]) * np.prod(et[j + 1:u + 1]) for u in range(j, C))
                   for j in range(C)])
    P = float(np.prod(et))
    beta = float(np.prod(om))
    aS = float(sum(np.prod(om[u + 1:]) * np.prod(et[:u + 1]) for u in range(C)))
    return cW, cS, (P, beta, aS)


def sequence_coefficients(theta, eta, alpha, chunk):
    """Per-token gates of a whole call [T] -> cW [T], cS [T], scalars [T/chunk, 3]."""
    T = len(theta)
    cW = np.zeros(T)
    cS = np.zeros(T)
    sc = np.zeros((T // chunk, 3))
    for k in range(T // chunk):
        s = slice(k * chunk, (k + 1) * chunk)
        cW[s], cS[s], sc[k] = chunk_coefficients(theta[s], eta[s], alpha[s])
    return cW, cS, sc


def omega_coefficients(cW, cS, gamma, chunk, window, gamma_hist=None):
    """Row r of chunk k is token i = k*chunk - (window-1) + r; its coefficient is gamma_i times the
    sum of cW_t (cS_t) over t in [max(i, k*chunk), min(i+window-1, (k+1)*chunk-1)].  Tokens before
    the call take gamma from gamma_hist (the window-1 previous tokens, oldest first), or 0."""
    T = len(cW)
    c = window
    R = chunk + c - 1
    oW = np.zeros((T // chunk, R))
    oS = np.zeros((T // chunk, R))
    for k in range(T // chunk):
        s = k * chunk
        for r in range(R):
            i = s - (c - 1) + r
            if i >= 0:
                g = gamma[i]
            elif gamma_hist is not None:
                g = gamma_hist[(c - 1) + i]
            else:
                g = 0.0
            ts = range(max(i, s), min(i + c - 1, s + chunk - 1) + 1)
            oW[k, r] = g * sum(cW[t] for t in ts)
            oS[k, r] = g * sum(cS[t] for t in ts)
    return oW, oS
