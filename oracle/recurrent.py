"""Per-token gated delta-rule recurrence in float64 (test infrastructure only).

This is the plain definition of the operator, one token at a time, written
with PyTorch CPU ops so that autograd can differentiate it.  The operator
family is the one the coverage-matrix page ("FLA operator-kernel correctness
testing and coverage matrix", section 1 and section 3) lists as GDN / KDA /
DeltaNet; its per-token update, in the K x V orientation the page's chunk
form ``S^r = P^r S^0 + H^r`` fixes (section 2), is

    S' = D_t S_{t-1}                        D_t = diag(exp(g_t))  (decay first)
    e_t = beta_t (v_t - S'^T k_t)           the corrected value ("v_new")
    S_t = S' + k_t e_t^T                    == (I - beta k k^T) D_t S_{t-1} + beta k v^T
    o_t = scale * S_t^T q_t                 (uses the updated state)

with k, q optionally L2-normalised per row (x / sqrt(sum x^2 + 1e-6), the
``use_qk_l2norm_in_kernel`` axis of the same page, section 3), g a scalar per
(token, value head) or a K-vector per (token, value head) for the per-channel
(KDA) gate, and value head j reading q/k head j // (HV / H) (the GVA axis,
section 3).  Sequences are the rows of a dense batch or the ``cu_seqlens``
segments of a varlen batch (B == 1); each starts from h0[n] (or zeros) and
ends in ht[n].

``recurrent_bwd`` is the reverse of that recurrence derived by hand; it is
checked against autograd and finite differences in the tests, never trusted on
its own.  The joint loss ``(o * do).sum() + (ht * dht).sum()`` is the one the
contributor guide's delta-rule test uses ("Flash Linear Attention contributor
guide", section on tests).
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

EPS = 1e-6


def l2norm(x: torch.Tensor) -> torch.Tensor:
    """Row L2 normalisation over the last dim: x / sqrt(sum(x^2) + 1e-6)."""
    return x / torch.sqrt((x * x).sum(-1, keepdim=True) + EPS)


def sequences(B: int, T: int, cu_seqlens) -> list:
    """List of (batch_row, start, end) token ranges, one per sequence."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(c) for c in cu_seqlens]
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def _f64(x):
    return None if x is None else x.detach().to(torch.float64) if not x.requires_grad else x.to(torch.float64)


def _expand_heads(x: torch.Tensor, HV: int) -> torch.Tensor:
    """q/k head h serves value heads h*G .. h*G+G-1 (G = HV / H)."""
    H = x.shape[2]
    return x.repeat_interleave(HV // H, dim=2)


def _decay(S: torch.Tensor, gt: torch.Tensor, per_channel: bool) -> torch.Tensor:
    # S [..., HV, K, V]; gt [..., HV] or [..., HV, K]
    d = torch.exp(gt)
    return S * (d[..., :, None] if per_channel else d[..., None, None])


def _scan(q, k, v, g, beta, S, scale, per_channel):
    """Run one group of equal-length sequences.  Shapes: q,k [n,L,HV,K],
    v [n,L,HV,V], g [n,L,HV(,K)], beta [n,L,HV], S [n,HV,K,V].  Returns
    (o [n,L,HV,V], S_final)."""
    outs = []
    for t in range(q.shape[1]):
        S = _decay(S, g[:, t], per_channel)
        kt = k[:, t]
        pred = torch.einsum("nhkv,nhk->nhv", S, kt)
        e = beta[:, t, :, None] * (v[:, t] - pred)
        S = S + kt[..., :, None] * e[..., None, :]
        outs.append(scale * torch.einsum("nhkv,nhk->nhv", S, q[:, t]))
    o = torch.stack(outs, 1) if outs else q.new_zeros(q.shape[0], 0, v.shape[2], v.shape[3])
    return o, S


def recurrent_fwd(q, k, v, g, beta, *, scale: float = 1.0, h0=None, cu_seqlens=None,
                  use_qk_l2norm: bool = False, seqs: Optional[Sequence[int]] = None,
                  heads: Optional[Sequence[int]] = None):
    """Per-token forward.  Inputs follow the library layout (q, k [B,T,H,K];
    v [B,T,HV,V]; g [B,T,HV] or [B,T,HV,K]; beta [B,T,HV]; h0 [N,HV,K,V]).

    Returns (o [B,T,HV,V], ht [N,HV,K,V]) in float64.  ``seqs`` / ``heads``
    restrict the work to some sequences / value heads (outputs elsewhere are
    left at zero), for sampled checks of large batches.
    """
    q, k, v, g, beta, h0 = (_f64(x) for x in (q, k, v, g, beta, h0))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    per_channel = g.dim() == 4
    if use_qk_l2norm:
        q, k = l2norm(q), l2norm(k)
    q, k = _expand_heads(q, HV), _expand_heads(k, HV)
    segs = sequences(B, T, cu_seqlens)
    N = len(segs)
    hsel = list(range(HV)) if heads is None else list(heads)
    nsel = list(range(N)) if seqs is None else list(seqs)

    o_rows = {}
    ht = torch.zeros(N, HV, K, V, dtype=torch.float64)
    ht_list = {}
    if cu_seqlens is None and seqs is None:
        groups = [list(range(N))]           # all dense rows together
    else:
        groups = [[n] for n in nsel]
    for grp in groups:
        rows = [segs[n][0] for n in grp]
        s, e = segs[grp[0]][1], segs[grp[0]][2]
        sl = (rows, slice(s, e))
        qs, ks = q[sl][:, :, hsel], k[sl][:, :, hsel]
        vs, gs, bs = v[sl][:, :, hsel], g[sl][:, :, hsel], beta[sl][:, :, hsel]
        if h0 is not None:
            S0 = h0[grp][:, hsel]
        else:
            S0 = torch.zeros(len(grp), len(hsel), K, V, dtype=torch.float64)
        o_g, S_g = _scan(qs, ks, vs, gs, bs, S0, scale, per_channel)
        for i, n in enumerate(grp):
            o_rows[n] = o_g[i]
            ht_list[n] = S_g[i]
    # assemble (keeps autograd intact: no in-place writes into leaves)
    o_full = []
    for b in range(B):
        pieces = []
        cursor = 0
        for n, (bb, s, e) in enumerate(segs):
            if bb != b:
                continue
            if s > cursor:
                pieces.append(torch.zeros(s - cursor, HV, V, dtype=torch.float64))
            if n in o_rows:
                blk = o_rows[n]
                if len(hsel) != HV:
                    full = torch.zeros(e - s, HV, V, dtype=torch.float64)
                    full[:, hsel] = blk
                    blk = full
                pieces.append(blk)
            else:
                pieces.append(torch.zeros(e - s, HV, V, dtype=torch.float64))
            cursor = e
        if cursor < T:
            pieces.append(torch.zeros(T - cursor, HV, V, dtype=torch.float64))
        o_full.append(torch.cat(pieces, 0) if pieces else torch.zeros(T, HV, V, dtype=torch.float64))
    o = torch.stack(o_full, 0)
    hts = []
    for n in range(N):
        if n in ht_list:
            blk = ht_list[n]
            if len(hsel) != HV:
                full = torch.zeros(HV, K, V, dtype=torch.float64)
                full[hsel] = blk
                blk = full
            hts.append(blk)
        else:
            hts.append(torch.zeros(HV, K, V, dtype=torch.float64))
    ht = torch.stack(hts, 0) if hts else ht
    return o, ht


def autograd_bwd(q, k, v, g, beta, do, dht=None, *, scale=1.0, h0=None, cu_seqlens=None,
                 use_qk_l2norm=False):
    """Gradients of L = (o*do).sum() + (ht*dht).sum() by autograd over the
    per-token forward.  Returns dict dq, dk, dv, dg, dbeta, dh0 (float64)."""
    leaves = {n: x.detach().to(torch.float64).requires_grad_(True)
              for n, x in dict(q=q, k=k, v=v, g=g, beta=beta).items()}
    h0l = h0.detach().to(torch.float64).requires_grad_(True) if h0 is not None else None
    o, ht = recurrent_fwd(leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                          scale=scale, h0=h0l, cu_seqlens=cu_seqlens, use_qk_l2norm=use_qk_l2norm)
    loss = (o * do.to(torch.float64)).sum()
    if dht is not None:
        loss = loss + (ht * dht.to(torch.float64)).sum()
    loss.backward()
    out = {"d" + n: x.grad if x.grad is not None else torch.zeros_like(x) for n, x in leaves.items()}
    out["dh0"] = h0l.grad if h0l is not None else None
    return out


def _l2norm_bwd(x: torch.Tensor, dxh: torch.Tensor) -> torch.Tensor:
    """Backward of x -> x / n, n = sqrt(sum x^2 + eps):
    dx = (dxh - xh * (xh . dxh)) / n."""
    n = torch.sqrt((x * x).sum(-1, keepdim=True) + EPS)
    xh = x / n
    return (dxh - xh * (xh * dxh).sum(-1, keepdim=True)) / n


def recurrent_bwd(q, k, v, g, beta, do, dht=None, *, scale=1.0, h0=None, cu_seqlens=None,
                  use_qk_l2norm=False, ckpt: int = 64, seqs=None, heads=None):
    """Hand-derived reverse of the per-token recurrence (float64).

    For each sequence the forward is replayed with a stored state every
    ``ckpt`` tokens; segments are then recomputed and walked backwards:

        dS   += scale q_t do_t^T            (o_t = scale S_t^T q_t)
        dq_t  = scale S_t do_t
        de    = dS^T k_t                    (S_t = S' + k e^T)
        dk_t  = dS e_t - beta S' de         (both places k_t appears)
        dv_t  = beta de ;  dbeta_t = de . (v_t - S'^T k_t)
        dS'   = dS - beta k_t de^T
        dg_t  = sum(dS' o S') over V (and over K for a scalar gate)
        dS    = D_t dS'                     (S' = D_t S_{t-1})

    then dh0 = dS, the L2-norm backward, and a sum of dq / dk over each GVA
    group.  ``seqs`` / ``heads`` restrict the work (outputs elsewhere zero;
    dq / dk then only hold the selected value heads' contributions).
    Returns dict dq, dk, dv, dg, dbeta, dh0.
    """
    q, k, v, g, beta, h0, do, dht = (None if x is None else x.detach().to(torch.float64)
                                     for x in (q, k, v, g, beta, h0, do, dht))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    per_channel = g.dim() == 4
    qh = l2norm(q) if use_qk_l2norm else q
    kh = l2norm(k) if use_qk_l2norm else k
    qe, ke = _expand_heads(qh, HV), _expand_heads(kh, HV)
    segs = sequences(B, T, cu_seqlens)
    N = len(segs)
    hsel = list(range(HV)) if heads is None else list(heads)
    nsel = list(range(N)) if seqs is None else list(seqs)

    dqe = torch.zeros(B, T, HV, K, dtype=torch.float64)
    dke = torch.zeros(B, T, HV, K, dtype=torch.float64)
    dv = torch.zeros(B, T, HV, V, dtype=torch.float64)
    dg = torch.zeros_like(g)
    dbeta = torch.zeros_like(beta)
    dh0 = torch.zeros(N, HV, K, V, dtype=torch.float64)

    def dec(x, gt):
        return _decay(x, gt, per_channel)

    for n in nsel:
        b, s, e = segs[n]
        L = e - s
        hs = hsel
        S = h0[n][hs].clone() if h0 is not None else torch.zeros(len(hs), K, V, dtype=torch.float64)
        # forward replay with checkpoints of the state *before* token s + c*ckpt
        cps = []
        for t in range(L):
            if t % ckpt == 0:
                cps.append(S.clone())
            tt = s + t
            S = dec(S, g[b, tt, hs])
            kt = ke[b, tt, hs]
            ev = beta[b, tt, hs][:, None] * (v[b, tt, hs] - torch.einsum("hkv,hk->hv", S, kt))
            S = S + kt[:, :, None] * ev[:, None, :]
        dS = dht[n][hs].clone() if dht is not None else torch.zeros(len(hs), K, V, dtype=torch.float64)
        nseg = (L + ckpt - 1) // ckpt
        for c in reversed(range(nseg)):
            t0, t1 = c * ckpt, min(L, (c + 1) * ckpt)
            # recompute S' (decayed) and S_t for the segment
            Sc = cps[c]
            Sp, St, E = [], [], []
            for t in range(t0, t1):
                tt = s + t
                Sd = dec(Sc, g[b, tt, hs])
                kt = ke[b, tt, hs]
                ev = beta[b, tt, hs][:, None] * (v[b, tt, hs] - torch.einsum("hkv,hk->hv", Sd, kt))
                Sc = Sd + kt[:, :, None] * ev[:, None, :]
                Sp.append(Sd)
                St.append(Sc)
                E.append(ev)
            for i in reversed(range(t1 - t0)):
                tt = s + t0 + i
                qt, kt = qe[b, tt, hs], ke[b, tt, hs]
                dot = do[b, tt, hs]
                dS = dS + scale * qt[:, :, None] * dot[:, None, :]
                dqe[b, tt, hs] = scale * torch.einsum("hkv,hv->hk", St[i], dot)
                de = torch.einsum("hkv,hk->hv", dS, kt)
                bt = beta[b, tt, hs]
                pred = torch.einsum("hkv,hk->hv", Sp[i], kt)
                dke[b, tt, hs] = (torch.einsum("hkv,hv->hk", dS, E[i])
                                  - bt[:, None] * torch.einsum("hkv,hv->hk", Sp[i], de))
                dv[b, tt, hs] = bt[:, None] * de
                dbeta[b, tt, hs] = (de * (v[b, tt, hs] - pred)).sum(-1)
                dSp = dS - bt[:, None, None] * kt[:, :, None] * de[:, None, :]
                if per_channel:
                    dg[b, tt, hs] = (dSp * Sp[i]).sum(-1)
                else:
                    dg[b, tt, hs] = (dSp * Sp[i]).sum((-1, -2))
                dS = dec(dSp, g[b, tt, hs])
        dh0[n, hs] = dS
    # GVA: q/k head h gathers the gradients of its G value heads
    dqh = dqe.reshape(B, T, H, G, K).sum(3)
    dkh = dke.reshape(B, T, H, G, K).sum(3)
    if use_qk_l2norm:
        dq, dk = _l2norm_bwd(q, dqh), _l2norm_bwd(k, dkh)
    else:
        dq, dk = dqh, dkh
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dh0=dh0 if h0 is not None else dh0)


def transition(k, g, beta, *, cu_seqlens=None, use_qk_l2norm: bool = False):
    """Transition of every sequence (or segment): the product of its per-token
    maps A_t = (I - beta_t k_t k_t^T) D_t, last token leftmost, so that the
    recurrence above gives S_end = M S_start + (the end state from a zero
    start).  This is the matrix the KCP page's pre-process hands to the merge
    ("flash-linear-attention KCP precision-failure root-cause manual",
    pre-process and merge sections); at g = 0 over one chunk it is the page
    "FLA operator-kernel correctness testing and coverage matrix" section 2's
    P^r.  Returns M [N,HV,K,K] in float64."""
    k, g, beta = (_f64(x) for x in (k, g, beta))
    B, T, H, K = k.shape
    HV = beta.shape[2]
    per_channel = g.dim() == 4
    if use_qk_l2norm:
        k = l2norm(k)
    k = _expand_heads(k, HV)
    segs = sequences(B, T, cu_seqlens)
    M = torch.zeros(len(segs), HV, K, K, dtype=torch.float64)
    eye = torch.eye(K, dtype=torch.float64)
    for n, (b, s, e) in enumerate(segs):
        for j in range(HV):
            P = eye.clone()
            for t in range(s, e):
                d = torch.exp(g[b, t, j])
                D = torch.diag(d) if per_channel else d * eye
                kt = k[b, t, j]
                A = (eye - beta[b, t, j] * torch.outer(kt, kt)) @ D
                P = A @ P
            M[n, j] = P
    return M


def simple_gla_fwd(q, k, v, g, *, scale: float = 1.0, h0=None, cu_seqlens=None, use_qk_l2norm: bool = False):
    """Simple GLA, per token (the variant the coverage-matrix page lists beside
    the delta rule, "FLA operator-kernel correctness testing and coverage
    matrix", section 2): a scalar per-token gate and no delta correction,

        S_t = exp(g_t) S_{t-1} + k_t v_t^T,    o_t = scale * S_t^T q_t,

    with the same layouts, L2 norm, GVA mapping and sequences as
    ``recurrent_fwd``.  Returns (o [B,T,HV,V], ht [N,HV,K,V]) in float64."""
    q, k, v, g, h0 = (_f64(x) for x in (q, k, v, g, h0))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if use_qk_l2norm:
        q, k = l2norm(q), l2norm(k)
    q, k = _expand_heads(q, HV), _expand_heads(k, HV)
    segs = sequences(B, T, cu_seqlens)
    o = torch.zeros(B, T, HV, V, dtype=torch.float64)
    ht = torch.zeros(len(segs), HV, K, V, dtype=torch.float64)
    for n, (b, s, e) in enumerate(segs):
        S = h0[n].clone() if h0 is not None else torch.zeros(HV, K, V, dtype=torch.float64)
        for t in range(s, e):
            S = torch.exp(g[b, t])[:, None, None] * S + k[b, t][:, :, None] * v[b, t][:, None, :]
            o[b, t] = scale * torch.einsum("hkv,hk->hv", S, q[b, t])
        ht[n] = S
    return o, ht
