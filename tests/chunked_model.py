"""Chunked form of the KDA recurrence in float64 numpy: the algebra the HIP kernels
evaluate, written plainly so each step can be compared with the sequential oracle.
Test infrastructure (imports nothing from the library or the oracle).

Derivation (from the recurrence S_r = (I - b_r k_r k_r^T) D_r S_{r-1} + b_r k_r v_r^T,
D_r = Diag(exp g_r)). Inside a chunk entered with state S, with G_r = sum_{j<=r} g_j
per key channel:
    U' = (I + A)^{-1} diag(b) (V - Kbar S),  Kbar = K * exp(G),
    A[r, j] = b_r sum_c k_r[c] exp(G_r[c] - G_j[c]) k_j[c]   for j < r,
    O = (Q * exp(G)) S + LowerIncl(Aqk) U',  Aqk[r, j] = sum_c q_r[c] exp(G_r[c] - G_j[c]) k_j[c],
    S_next = Diag(exp G_C) S + (K * exp(G_C - G))^T U'.
The C x C matrices hold exp(G_r - G_j) in factored form. Splitting each chunk into
16-token tiles and measuring the factor from the state before row tile a
(ref_a = G at the last token of tile a-1) keeps both factors finite: the row factor
exp(G_r - ref_a) is in [e^-80, 1] and the column factor exp(ref_a - G_j) is <= 1 off the
diagonal and in [1, e^80] on it, because each step's log-decay is >= -5 (the orkas.ai
Kimi K3 page, "Eine Untergrenze, die einen GPU-Codepfad beseitigte"). So diagonal tiles
are the same dense product as the others.
"""
import numpy as np

TILE = 16


def chunk_matrices(qc, kc, gc, tile=TILE, factor_dtype=np.float64, single_reference=False):
    """Akk, Aqk (C x C, lower incl. diagonal) for one chunk of one head via tile-factored
    products. With single_reference the chunk start is the reference for every tile (the
    path the decay floor does not make safe); factors are computed in factor_dtype."""
    C, dk = kc.shape
    G = np.cumsum(gc, axis=0)
    Akk = np.zeros((C, C))
    Aqk = np.zeros((C, C))
    with np.errstate(over="ignore", invalid="ignore"):
        for a in range(0, C, tile):
            ref = np.zeros(dk) if (a == 0 or single_reference) else G[a - 1]
            rows = slice(a, min(a + tile, C))
            cols = slice(0, min(a + tile, C))
            rf = np.exp((G[rows] - ref).astype(factor_dtype))
            cf = np.exp((ref - G[cols]).astype(factor_dtype))
            kr = kc[rows] * rf
            qr = qc[rows] * rf
            kcol = kc[cols] * cf
            Akk[rows, cols] = kr @ kcol.T
            Aqk[rows, cols] = qr @ kcol.T
    return np.tril(Akk), np.tril(Aqk), G


def chunked_forward(q, k, v, g, beta, S0=None, cu_seqlens=None, chunk=64, tile=TILE,
                    trace=None):
    """Same interface and layout as the oracle ([B, T, H, d]); returns (o, S_T) in float64.
    trace, if a list, receives per-chunk intermediates of head 0 of sequence 0."""
    q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        seqs = [(0, int(a), int(e)) for a, e in zip(cu_seqlens[:-1], cu_seqlens[1:])]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((len(seqs), H, dk, dv))
    for n, (b, t0, t1) in enumerate(seqs):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[n, h], np.float64)
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                qc, kc, vc, gc = (a[b, c0:c1, h] for a in (q, k, v, g))
                bc = beta[b, c0:c1, h]
                Akk, Aqk, G = chunk_matrices(qc, kc, gc, tile)
                C = c1 - c0
                A = np.tril(bc[:, None] * Akk, -1)
                Tinv = np.linalg.solve(np.eye(C) + A, np.eye(C))
                Kbar = kc * np.exp(G)
                Up = Tinv @ (bc[:, None] * (vc - Kbar @ S))
                O = (qc * np.exp(G)) @ S + Aqk @ Up
                if trace is not None and n == 0 and h == 0:
                    trace.append(dict(G=G, A=A, Aqk=Aqk, Tinv=Tinv, U=Up, S_in=S.copy()))
                S = np.exp(G[-1])[:, None] * S + (kc * np.exp(G[-1] - G)).T @ Up
                o[b, c0:c1, h] = O
            S_T[n, h] = S
    return o, S_T
