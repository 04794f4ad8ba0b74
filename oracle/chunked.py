"""Chunk-wise (WY) evaluation of the gated delta rule in float64 NumPy
(test infrastructure only; shares no code with ``recurrent`` or the GPU path).

The coverage-matrix page ("FLA operator-kernel correctness testing and
coverage matrix", section 2) quotes the DeltaNet chunk form: within a chunk the
state after row r is S^r = P^r S^0 + H^r, where P^r, the running product of
generalised Householder transitions, has the WY form P^r = I - sum_{i<=r}
k^i w^{i T}.  With a gate the same derivation gives, for a chunk of L rows
entering with state S0 (G = chunk-local inclusive cumsum of g, a scalar or a
K-vector per row):

    A[r, j] = beta_r * sum_d k_rd k_jd exp(G_rd - G_jd)      j < r   (else 0)
    T       = (I + A)^-1                   (unit lower triangular)
    W       = T (beta * exp(G) * K)        U = T (beta * V)
    E       = U - W S0                     (per-row corrected values, "v_new")
    O       = scale * [ (exp(G) * Q) S0 + Aqk E ],
              Aqk[r, j] = sum_d q_rd k_jd exp(G_rd - G_jd)   j <= r
    S_next  = diag(exp(G_L)) S0 + sum_j (exp(G_L - G_j) * k_j) e_j^T

and, inside the chunk, P^r = diag(exp(G_r)) - sum_{j<=r} diag(exp(G_r - G_j))
k_j w_j^T and H^r = sum_{j<=r} diag(exp(G_r - G_j)) k_j u_j^T (``wy_factors``);
at g = 0 this is the page's formula.  T is formed by explicit forward
substitution, row by row.

Chunks restart at every sequence start and the last chunk of a sequence may be
partial (the varlen chunk-boundary example on the KCP page, "flash-linear-
attention KCP precision-failure root-cause manual", section "why per-chunk
comparison lies under varlen KCP"); ``chunk_table`` enumerates them by brute
force.
"""
from __future__ import annotations

import numpy as np
import torch

EPS = 1e-6


def _np64(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def sequence_bounds(B: int, T: int, cu_seqlens) -> list:
    """(start, end) of each sequence in the flattened [B*T] token order."""
    if cu_seqlens is None:
        return [(b * T, (b + 1) * T) for b in range(B)]
    cu = [int(c) for c in cu_seqlens]
    return [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def chunk_table(B: int, T: int, cu_seqlens, C: int):
    """Brute-force chunk enumeration.

    Returns (idx int32 [NT, 3] of (sequence, first token in the flattened
    token order, length), off int32 [N+1] with off[n] = first chunk of
    sequence n and off[N] = NT)."""
    idx, off = [], [0]
    for n, (s, e) in enumerate(sequence_bounds(B, T, cu_seqlens)):
        t = s
        while t < e:
            idx.append((n, t, min(C, e - t)))
            t += C
        off.append(len(idx))
    return np.array(idx, dtype=np.int32).reshape(-1, 3), np.array(off, dtype=np.int32)


def _normalise_rows(x):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + EPS)


def forward_substitution(A: np.ndarray) -> np.ndarray:
    """(I + A)^-1 for strictly lower-triangular A (batched over leading
    dims): row r of T is e_r - sum_{j<r} A[r, j] T[j]."""
    L = A.shape[-1]
    Tm = np.zeros_like(A)
    for r in range(L):
        row = np.zeros(A.shape[:-2] + (L,))
        row[..., r] = 1.0
        if r:
            # sum_{j<r} A[r, j] T[j] as one (batched) vector-matrix product
            row = row - (A[..., r:r + 1, :r] @ Tm[..., :r, :])[..., 0, :]
        Tm[..., r, :] = row
    return Tm


def _chunk(qc, kc, vc, Gc, bc, S0, scale, per_channel):
    """One chunk for all value heads.  qc, kc [L,HV,K]; vc [L,HV,V];
    Gc [L,HV(,K)] (inclusive cumsum); bc [L,HV]; S0 [HV,K,V]."""
    L = kc.shape[0]
    qh = np.transpose(qc, (1, 0, 2))            # [HV,L,K]
    kh = np.transpose(kc, (1, 0, 2))
    vh = np.transpose(vc, (1, 0, 2))            # [HV,L,V]
    bh = bc.T                                   # [HV,L]
    if per_channel:
        Gh = np.transpose(Gc, (1, 0, 2))        # [HV,L,K]
        # pairwise decays exp(G_r - G_j) per channel, only where j <= r
        diff = Gh[:, :, None, :] - Gh[:, None, :, :]           # [HV,r,j,K]
        low = np.tril(np.ones((L, L)))[None, :, :, None] > 0
        dec = np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)
        kk = np.einsum("hrd,hjd,hrjd->hrj", kh, kh, dec)
        qk = np.einsum("hrd,hjd,hrjd->hrj", qh, kh, dec)
        gam = np.exp(Gh)                                       # [HV,L,K]
        kg_in = gam * kh                                       # exp(G_j) * k_j
        q_in = gam * qh
        last = np.exp(Gh[:, -1:, :] - Gh)                      # exp(G_L - G_j) [HV,L,K]
        k_out = last * kh
        decay_L = np.exp(Gh[:, -1, :])                         # [HV,K]
    else:
        Gh = Gc.T                                              # [HV,L]
        diff = Gh[:, :, None] - Gh[:, None, :]
        low = np.tril(np.ones((L, L)))[None] > 0
        dec = np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)
        kk = (kh @ np.transpose(kh, (0, 2, 1))) * dec
        qk = (qh @ np.transpose(kh, (0, 2, 1))) * dec
        gam = np.exp(Gh)[:, :, None]
        kg_in = gam * kh
        q_in = gam * qh
        k_out = np.exp(Gh[:, -1:] - Gh)[:, :, None] * kh
        decay_L = np.exp(Gh[:, -1])[:, None] * np.ones((1, kh.shape[-1]))
    A = bh[:, :, None] * np.tril(kk, -1)
    Tm = forward_substitution(A)
    W = Tm @ (bh[:, :, None] * kg_in)
    U = Tm @ (bh[:, :, None] * vh)
    E = U - W @ S0
    O = scale * (q_in @ S0 + qk @ E)           # qk already holds j <= r only
    S1 = decay_L[:, :, None] * S0 + np.transpose(k_out, (0, 2, 1)) @ E
    return dict(A=A, T=Tm, W=W, U=U, E=E, O=O, S_next=S1, QK=scale * qk, QG=scale * q_in, KT=k_out,
                DL=decay_L)


def chunked_fwd(q, k, v, g, beta, *, scale=1.0, h0=None, cu_seqlens=None,
                use_qk_l2norm=False, chunk_size=64, intermediates=False):
    """Chunk-wise forward.  Same layouts as the per-token oracle; returns
    (o [B,T,HV,V], ht [N,HV,K,V]) as float64 NumPy arrays and, when
    ``intermediates`` is set, a dict of per-chunk tensors indexed by the
    global chunk number of ``chunk_table``:
      G [NT,HV,C(,K)], A and T [NT,HV,C,C], W [NT,HV,C,K], U and E
      [NT,HV,C,V] (rows past a partial chunk's end are zero) and
      h [NT,HV,K,V] (the state entering each chunk); also the output's own
      operands QK = scale (Q K^T o decay mask) [NT,HV,C,C], QG = scale
      exp(G) q [NT,HV,C,K], and the state update's KT = exp(G_L - G) k
      [NT,HV,C,K] and DL = exp(G_L) [NT,HV,K]."""
    q, k, v, g, beta, h0 = (_np64(x) for x in (q, k, v, g, beta, h0))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    Gs = HV // H
    C = int(chunk_size)
    per_channel = g.ndim == 4
    if use_qk_l2norm:
        q, k = _normalise_rows(q), _normalise_rows(k)
    q = np.repeat(q, Gs, axis=2).reshape(B * T, HV, K)
    k = np.repeat(k, Gs, axis=2).reshape(B * T, HV, K)
    v = v.reshape(B * T, HV, V)
    g = g.reshape((B * T, HV, K) if per_channel else (B * T, HV))
    beta = beta.reshape(B * T, HV)
    idx, off = chunk_table(B, T, cu_seqlens, C)
    N = len(off) - 1
    NT = len(idx)
    o = np.zeros((B * T, HV, V))
    ht = np.zeros((N, HV, K, V))
    inter = None
    if intermediates:
        gshape = (NT, HV, C, K) if per_channel else (NT, HV, C)
        inter = dict(G=np.zeros(gshape), A=np.zeros((NT, HV, C, C)), T=np.zeros((NT, HV, C, C)),
                     W=np.zeros((NT, HV, C, K)), U=np.zeros((NT, HV, C, V)),
                     E=np.zeros((NT, HV, C, V)), h=np.zeros((NT, HV, K, V)),
                     QK=np.zeros((NT, HV, C, C)), QG=np.zeros((NT, HV, C, K)), KT=np.zeros((NT, HV, C, K)),
                     DL=np.zeros((NT, HV, K)))
    for n in range(N):
        S = h0[n].copy() if h0 is not None else np.zeros((HV, K, V))
        for c in range(off[n], off[n + 1]):
            _, t0, L = (int(x) for x in idx[c])
            sl = slice(t0, t0 + L)
            Gc = np.cumsum(g[sl], axis=0)
            r = _chunk(q[sl], k[sl], v[sl], Gc, beta[sl], S, scale, per_channel)
            if inter is not None:
                inter["h"][c] = S
                inter["G"][c, :, :L] = np.moveaxis(Gc, 0, 1)
                inter["A"][c, :, :L, :L] = r["A"]
                inter["T"][c, :, :L, :L] = r["T"]
                inter["W"][c, :, :L] = r["W"]
                inter["U"][c, :, :L] = r["U"]
                inter["E"][c, :, :L] = r["E"]
                inter["QK"][c, :, :L, :L] = r["QK"]
                inter["QG"][c, :, :L] = r["QG"]
                inter["KT"][c, :, :L] = r["KT"]
                inter["DL"][c] = r["DL"]
            o[sl] = np.transpose(r["O"], (1, 0, 2))
            S = r["S_next"]
        ht[n] = S
    o = o.reshape(B, T, HV, V)
    if intermediates:
        inter["idx"], inter["off"] = idx, off
        return o, ht, inter
    return o, ht


def wy_factors(k, beta, g, w, u):
    """P^r and H^r of one chunk of one head from its W and U rows.

    k [L,K] (already normalised), beta [L], g [L] or [L,K], w [L,K], u [L,V].
    Returns P [L,K,K] and Hs [L,K,V] with S_r = P[r] S0 + Hs[r]."""
    k, beta, g, w, u = (_np64(x) for x in (k, beta, g, w, u))
    L, K = k.shape
    G = np.cumsum(g, axis=0)
    if G.ndim == 1:
        G = G[:, None] * np.ones((1, K))
    P = np.zeros((L, K, K))
    Hs = np.zeros((L, K, u.shape[1]))
    for r in range(L):
        P[r] = np.diag(np.exp(G[r]))
        for j in range(r + 1):
            dk = np.exp(G[r] - G[j]) * k[j]
            P[r] -= np.outer(dk, w[j])
            Hs[r] += np.outer(dk, u[j])
    return P, Hs


# --------------------------------------------------------------------------
# Chunk-wise backward (float64, NumPy).  Gradients of the chunk form above,
# derived by matrix calculus for one chunk and written for the general
# per-channel gate (a scalar gate is the case G_rd = G_r for every d; its dg
# is the sum over d).  Per chunk, with S0 the entering state, dS1 the gradient
# of the leaving state and Kt = exp(G_L - G) * K, Kg = exp(G) * K,
# Qg = exp(G) * Q:
#   dE  = scale P^T dO + Kt dS1                      (P: gated q.k, j <= r)
#   dS0 = scale Qg^T dO + exp(G_L) * dS1 - W^T dE     (passed to the previous chunk)
#   dP  = scale dO E^T,   dW = -dE S0^T,   dU = dE
#   dT  = dW (beta Kg)^T + dU (beta V)^T,  dA = -T^T dT T^T (strictly lower)
#   dV  = beta T^T dU,    dKg = beta T^T dW
# then the gated bilinear forms A (k.k), P (q.k), Qg, Kg, Kt give dq, dk and
# the per-channel gate gradient dG, and dg is the reverse cumsum of dG within
# the chunk.  Pinned against the per-token backward in the tests.
# --------------------------------------------------------------------------

def _gated_pair(a, b, G, lower_strict):
    """D[r, j] = sum_d a_rd b_jd exp(G_rd - G_jd) on the (strict) lower
    triangle; a, b [HV,L,K], G [HV,L,K].  Returns D and the mask."""
    L = a.shape[1]
    low = np.tril(np.ones((L, L)), -1 if lower_strict else 0)[None, :, :, None] > 0
    diff = G[:, :, None, :] - G[:, None, :, :]
    ex = np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)       # [HV,r,j,K]
    return np.einsum("hrd,hjd,hrjd->hrj", a, b, ex), ex


def _gated_pair_grads(dD, a, b, ex):
    """Gradients of D[r,j] = sum_d a_rd b_jd ex_rjd w.r.t. a, b and G
    (ex = exp(G_r - G_j) on the mask): returns da, db, dG."""
    da = np.einsum("hrj,hjd,hrjd->hrd", dD, b, ex)
    db = np.einsum("hrj,hrd,hrjd->hjd", dD, a, ex)
    dG = a * da - b * db
    return da, db, dG


def _chunk_bwd(qc, kc, vc, Gc, bc, S0, dO, dS1, scale):
    """One chunk, all value heads; shapes as in _chunk plus dO [L,HV,V],
    dS1 [HV,K,V].  G is per channel here ([L,HV,K]).  Returns a dict."""
    q = np.transpose(qc, (1, 0, 2))
    k = np.transpose(kc, (1, 0, 2))
    v = np.transpose(vc, (1, 0, 2))
    G = np.transpose(Gc, (1, 0, 2))
    b = bc.T
    do = np.transpose(dO, (1, 0, 2))
    L = k.shape[1]
    HV = k.shape[0]
    # forward recompute
    Abar, exA = _gated_pair(k, k, G, True)
    A = b[:, :, None] * Abar
    Tm = forward_substitution(A)
    eG = np.exp(G)
    Kg, Qg = eG * k, eG * q
    GL = G[:, -1:, :]
    Kt = np.exp(GL - G) * k
    W = Tm @ (b[:, :, None] * Kg)
    U = Tm @ (b[:, :, None] * v)
    E = U - W @ S0
    P, exP = _gated_pair(q, k, G, False)
    tr = lambda x: np.transpose(x, (0, 2, 1))
    # backward
    dE = scale * tr(P) @ do + Kt @ dS1
    dS0 = scale * tr(Qg) @ do + np.exp(GL[:, 0, :])[:, :, None] * dS1 - tr(W) @ dE
    dP = scale * do @ tr(E)
    dQg = scale * do @ tr(S0)
    dKt = E @ tr(dS1)
    dW = -dE @ tr(S0)
    dU = dE
    dT = dW @ tr(b[:, :, None] * Kg) + dU @ tr(b[:, :, None] * v)
    TtdW = tr(Tm) @ dW
    TtdU = tr(Tm) @ dU
    dKg = b[:, :, None] * TtdW
    dv = b[:, :, None] * TtdU
    dA = np.tril(-tr(Tm) @ dT @ tr(Tm), -1)
    dbeta = (Kg * TtdW).sum(-1) + (v * TtdU).sum(-1) + (dA * Abar).sum(-1)
    dAbar = b[:, :, None] * dA
    dk1, dk2, dG_A = _gated_pair_grads(dAbar, k, k, exA)
    dq_P, dk_P, dG_P = _gated_pair_grads(dP, q, k, exP)
    dq = dq_P + eG * dQg
    dk = dk1 + dk2 + dk_P + eG * dKg + np.exp(GL - G) * dKt
    dG = dG_A + dG_P + Qg * dQg + Kg * dKg - Kt * dKt
    dG[:, -1, :] += (Kt * dKt).sum(1) + np.exp(GL[:, 0, :]) * (S0 * dS1).sum(-1)
    dg = np.flip(np.cumsum(np.flip(dG, 1), 1), 1)           # reverse cumsum over rows
    return dict(dq=dq, dk=dk, dv=dv, dbeta=dbeta, dg=dg, dS0=dS0, dE=dE,
                dEi=scale * tr(P) @ do, E=E)


def chunked_bwd(q, k, v, g, beta, do, dht=None, *, scale=1.0, h0=None, cu_seqlens=None,
                use_qk_l2norm=False, chunk_size=64, intermediates=False):
    """Chunk-wise backward of L = (o * do).sum() + (ht * dht).sum().
    Returns dict dq, dk [B,T,H,K]; dv [B,T,HV,V]; dg like g; dbeta like beta;
    dh0 [N,HV,K,V] (float64 NumPy).  With ``intermediates``: per-chunk dh
    [NT,HV,K,V] (gradient of the state leaving the chunk), dE and dEi
    [NT,HV,C,V] (dEi = scale P^T dO, the chunk-local part of dE)."""
    q, k, v, g, beta, h0, do, dht = (_np64(x) for x in (q, k, v, g, beta, h0, do, dht))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    Gs = HV // H
    C = int(chunk_size)
    per_channel = g.ndim == 4
    if use_qk_l2norm:
        nq = np.sqrt((q * q).sum(-1, keepdims=True) + EPS)
        nk = np.sqrt((k * k).sum(-1, keepdims=True) + EPS)
        qh, kh = q / nq, k / nk
    else:
        qh, kh = q, k
    qe = np.repeat(qh, Gs, axis=2).reshape(B * T, HV, K)
    ke = np.repeat(kh, Gs, axis=2).reshape(B * T, HV, K)
    vv = v.reshape(B * T, HV, V)
    gg = g.reshape(B * T, HV, K) if per_channel else np.repeat(g.reshape(B * T, HV, 1), K, axis=2)
    bb = beta.reshape(B * T, HV)
    dov = do.reshape(B * T, HV, V)
    idx, off = chunk_table(B, T, cu_seqlens, C)
    N, NT = len(off) - 1, len(idx)
    dqe = np.zeros((B * T, HV, K))
    dke = np.zeros((B * T, HV, K))
    dv = np.zeros((B * T, HV, V))
    dG = np.zeros((B * T, HV, K))
    dbeta = np.zeros((B * T, HV))
    dh0 = np.zeros((N, HV, K, V))
    inter = dict(dh=np.zeros((NT, HV, K, V)), dE=np.zeros((NT, HV, C, V)),
                 dEi=np.zeros((NT, HV, C, V))) if intermediates else None
    for n in range(N):
        # forward pass over the chunks to get the entering states
        S = h0[n].copy() if h0 is not None else np.zeros((HV, K, V))
        states = []
        for c in range(off[n], off[n + 1]):
            _, t0, L = (int(x) for x in idx[c])
            sl = slice(t0, t0 + L)
            states.append(S)
            Gc = np.cumsum(gg[sl], axis=0)
            r = _chunk(qe[sl], ke[sl], vv[sl], Gc, bb[sl], S, scale, True)
            S = r["S_next"]
        dS = dht[n].copy() if dht is not None else np.zeros((HV, K, V))
        for i, c in reversed(list(enumerate(range(off[n], off[n + 1])))):
            _, t0, L = (int(x) for x in idx[c])
            sl = slice(t0, t0 + L)
            if inter is not None:
                inter["dh"][c] = dS
            Gc = np.cumsum(gg[sl], axis=0)
            r = _chunk_bwd(qe[sl], ke[sl], vv[sl], Gc, bb[sl], states[i], dov[sl], dS, scale)
            dqe[sl] = np.transpose(r["dq"], (1, 0, 2))
            dke[sl] = np.transpose(r["dk"], (1, 0, 2))
            dv[sl] = np.transpose(r["dv"], (1, 0, 2))
            dbeta[sl] = r["dbeta"].T
            dG[sl] = np.transpose(r["dg"], (1, 0, 2))
            if inter is not None:
                inter["dE"][c, :, :L] = r["dE"]
                inter["dEi"][c, :, :L] = r["dEi"]
            dS = r["dS0"]
        dh0[n] = dS
    dqh = dqe.reshape(B, T, H, Gs, K).sum(3)
    dkh = dke.reshape(B, T, H, Gs, K).sum(3)
    if use_qk_l2norm:
        dq = (dqh - qh * (qh * dqh).sum(-1, keepdims=True)) / nq
        dk = (dkh - kh * (kh * dkh).sum(-1, keepdims=True)) / nk
    else:
        dq, dk = dqh, dkh
    dg = dG.reshape(B, T, HV, K)
    if not per_channel:
        dg = dg.sum(-1)
    out = dict(dq=dq, dk=dk, dv=dv.reshape(B, T, HV, V), dg=dg, dbeta=dbeta.reshape(B, T, HV), dh0=dh0)
    if intermediates:
        inter["idx"], inter["off"] = idx, off
        out["inter"] = inter
    return out
