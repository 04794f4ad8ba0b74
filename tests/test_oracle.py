"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: closed forms of the
recurrence, a textbook routine, the explicit product of Householder
transitions (the WY identity on the coverage-matrix page, section 2), the
chunk-boundary example printed on the KCP page, invariants, and finite
differences.  They are chosen so that a dropped term, a wrong sign, a wrong
index or a transposed operand in either oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import chunked, recurrent
import workloads
from oracle.metrics import err_ratio

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
f64 = torch.float64


def rnd(*shape, seed=0, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return scale * torch.randn(*shape, generator=g, dtype=f64)


def problem(B=1, T=20, H=2, HV=2, K=8, V=6, per_channel=False, seed=0, slow=False, l2=True):
    g_ = torch.Generator().manual_seed(seed)
    q = torch.randn(B, T, H, K, generator=g_, dtype=f64)
    k = torch.randn(B, T, H, K, generator=g_, dtype=f64)
    if l2:
        q, k = F.normalize(q, dim=-1), F.normalize(k, dim=-1)
    v = torch.randn(B, T, HV, V, generator=g_, dtype=f64)
    gs = (B, T, HV, K) if per_channel else (B, T, HV)
    g = F.logsigmoid(torch.randn(*gs, generator=g_, dtype=f64) + (4.0 if slow else 0.0))
    beta = torch.sigmoid(torch.randn(B, T, HV, generator=g_, dtype=f64))
    return q, k, v, g, beta


# ---------------------------------------------------------------- chunk table

def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            out[key] = [int(x) for x in vals]
    return out


def test_chunk_table_page_example():
    gd = _read_golden("chunk_boundaries_400_624_c64.txt")
    lengths, C = gd["lengths"], gd["chunk_size"][0]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    idx, off = chunked.chunk_table(1, int(cu[-1]), cu, C)
    seq1 = idx[off[1]:off[2]]
    starts = list(seq1[:, 1])
    assert starts[:4] == gd["seq1_first_chunk_starts"]
    # every chunk lies inside its sequence, chunks tile each sequence exactly
    for n, L in enumerate(lengths):
        rows = idx[off[n]:off[n + 1]]
        assert (rows[:, 0] == n).all()
        assert rows[:, 2].sum() == L
        assert rows[0, 1] == cu[n]
        assert (np.diff(rows[:, 1]) == C).all()
        assert (rows[:-1, 2] == C).all() and 0 < rows[-1, 2] <= C
    assert off[-1] == math.ceil(400 / 64) + math.ceil(624 / 64)


def test_chunk_table_aligned_example():
    gd = _read_golden("chunk_boundaries_256_768_c64.txt")
    lengths, C = gd["lengths"], gd["chunk_size"][0]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    idx, off = chunked.chunk_table(1, int(cu[-1]), cu, C)
    assert (idx[:, 1] % gd["all_starts_multiple_of"][0] == 0).all()
    assert (idx[:, 2] == C).all() and len(idx) == (256 + 768) // 64


def test_chunk_table_dense_and_empty():
    idx, off = chunked.chunk_table(3, 100, None, 32)
    assert list(off) == [0, 4, 8, 12]
    assert list(idx[3]) == [0, 96, 4] and list(idx[4]) == [1, 100, 32]
    cu = np.array([0, 0, 5, 5, 70], np.int32)          # empty sequences allowed
    idx, off = chunked.chunk_table(1, 70, cu, 64)
    assert list(off) == [0, 0, 1, 1, 3]
    assert [tuple(r) for r in idx] == [(1, 0, 5), (3, 5, 64), (3, 69, 1)]


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("per_channel", [False, True])
def test_beta_zero_is_pure_decay(per_channel):
    q, k, v, g, beta = problem(T=17, K=5, V=4, per_channel=per_channel, seed=1)
    beta = torch.zeros_like(beta)
    h0 = rnd(1, 2, 5, 4, seed=2)
    o, ht = recurrent.recurrent_fwd(q, k, v, g, beta, scale=0.7, h0=h0)
    Gabs = torch.cumsum(g, 1)                                 # from the sequence start
    for t in range(17):
        for j in range(2):
            d = torch.exp(Gabs[0, t, j])
            dq = (d * q[0, t, j]) if per_channel else d * q[0, t, j]
            ref = 0.7 * dq @ h0[0, j]
            assert torch.allclose(o[0, t, j], ref, rtol=1e-12, atol=1e-14)
    for j in range(2):
        d = torch.exp(Gabs[0, -1, j])
        ref = (d[:, None] * h0[0, j]) if per_channel else d * h0[0, j]
        assert torch.allclose(ht[0, j], ref, rtol=1e-12, atol=1e-14)
    oc, hc = chunked.chunked_fwd(q, k, v, g, beta, scale=0.7, h0=h0, chunk_size=8)
    assert np.allclose(oc, o.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(hc, ht.numpy(), rtol=1e-12, atol=1e-14)


def test_single_token_from_zero_state():
    q, k, v, g, beta = problem(T=1, K=6, V=3, seed=3, l2=False)
    o, ht = recurrent.recurrent_fwd(q, k, v, g, beta, scale=1.3)
    for j in range(2):
        S = beta[0, 0, j] * torch.outer(k[0, 0, j], v[0, 0, j])
        assert torch.allclose(ht[0, j], S, rtol=1e-13)
        ref = 1.3 * beta[0, 0, j] * (q[0, 0, j] @ k[0, 0, j]) * v[0, 0, j]
        assert torch.allclose(o[0, 0, j], ref, rtol=1e-13)


@pytest.mark.parametrize("per_channel", [False, True])
def test_unit_keys_beta_one_recall_value(per_channel):
    """With beta = 1 and |k| = 1, S_t^T k_t = v_t for any gate and any state,
    so o_t = v_t when q_t = k_t and scale = 1.  Fails if the decay is applied
    after the correction, if the correction has the wrong sign, or if o uses
    the state before the update."""
    q, k, v, g, beta = problem(T=40, K=8, V=5, per_channel=per_channel, seed=4)
    beta = torch.ones_like(beta)
    h0 = rnd(1, 2, 8, 5, seed=5)
    o, _ = recurrent.recurrent_fwd(k, k, v, g, beta, scale=1.0, h0=h0)
    assert torch.allclose(o, v, rtol=1e-11, atol=1e-12)
    oc, _ = chunked.chunked_fwd(k, k, v, g, beta, scale=1.0, h0=h0, chunk_size=16)
    assert np.allclose(oc, v.numpy(), rtol=1e-11, atol=1e-12)


def test_orthonormal_keys_accumulate():
    """Standard-basis keys, g = 0, h0 = 0: the correction never fires and
    S_t = sum_{s<=t} beta_s e_s v_s^T (plain outer-product memory)."""
    T, K, V = 6, 8, 4
    k = torch.zeros(1, T, 1, K, dtype=f64)
    for t in range(T):
        k[0, t, 0, t] = 1.0
    q = rnd(1, T, 1, K, seed=6)
    v = rnd(1, T, 1, V, seed=7)
    beta = torch.sigmoid(rnd(1, T, 1, seed=8))
    g = torch.zeros(1, T, 1, dtype=f64)
    o, ht = recurrent.recurrent_fwd(q, k, v, g, beta, scale=0.5)
    S = torch.zeros(K, V, dtype=f64)
    for t in range(T):
        S = S + beta[0, t, 0] * torch.outer(k[0, t, 0], v[0, t, 0])
        assert torch.allclose(o[0, t, 0], 0.5 * q[0, t, 0] @ S, rtol=1e-13)
    assert torch.allclose(ht[0, 0], S, rtol=1e-13)


def test_householder_product_form():
    """The per-token recurrence equals the transition-matrix form
    S_t = (I - b k k^T) D_t S_{t-1} + b k v^T built from explicit K x K
    matrices (scalar and per-channel gates)."""
    for per_channel in (False, True):
        q, k, v, g, beta = problem(T=9, H=1, HV=1, K=5, V=3, per_channel=per_channel, seed=9)
        h0 = rnd(1, 1, 5, 3, seed=10)
        o, ht = recurrent.recurrent_fwd(q, k, v, g, beta, scale=1.0, h0=h0)
        S = h0[0, 0].clone()
        I = torch.eye(5, dtype=f64)
        for t in range(9):
            kt = k[0, t, 0]
            D = torch.diag(torch.exp(g[0, t, 0])) if per_channel else torch.exp(g[0, t, 0]) * I
            S = (I - beta[0, t, 0] * torch.outer(kt, kt)) @ D @ S + beta[0, t, 0] * torch.outer(kt, v[0, t, 0])
            assert torch.allclose(o[0, t, 0], S.T @ q[0, t, 0], rtol=1e-12)
        assert torch.allclose(ht[0, 0], S, rtol=1e-12)


# ------------------------------------------------------------- invariants

def test_linear_in_v_and_h0():
    q, k, v, g, beta = problem(T=15, seed=11)
    v2 = rnd(*v.shape, seed=12)
    h0a, h0b = rnd(1, 2, 8, 6, seed=13), rnd(1, 2, 8, 6, seed=14)
    oa, ha = recurrent.recurrent_fwd(q, k, v, g, beta, h0=h0a)
    ob, hb = recurrent.recurrent_fwd(q, k, v2, g, beta, h0=h0b)
    oc, hc = recurrent.recurrent_fwd(q, k, 2 * v - 3 * v2, g, beta, h0=2 * h0a - 3 * h0b)
    assert torch.allclose(oc, 2 * oa - 3 * ob, rtol=1e-11, atol=1e-12)
    assert torch.allclose(hc, 2 * ha - 3 * hb, rtol=1e-11, atol=1e-12)


def test_scale_is_linear_in_output_only():
    q, k, v, g, beta = problem(T=12, seed=15)
    o1, h1 = recurrent.recurrent_fwd(q, k, v, g, beta, scale=1.0)
    o2, h2 = recurrent.recurrent_fwd(q, k, v, g, beta, scale=0.25)
    assert torch.allclose(o2, 0.25 * o1, rtol=1e-13) and torch.equal(h1, h2)


def test_gva_equals_repeated_heads():
    q, k, v, g, beta = problem(T=14, H=2, HV=6, seed=16)
    h0 = rnd(1, 6, 8, 6, seed=17)
    o, ht = recurrent.recurrent_fwd(q, k, v, g, beta, h0=h0, use_qk_l2norm=True)
    qr, kr = q.repeat_interleave(3, 2), k.repeat_interleave(3, 2)
    o2, ht2 = recurrent.recurrent_fwd(qr, kr, v, g, beta, h0=h0, use_qk_l2norm=True)
    assert torch.allclose(o, o2, rtol=1e-14) and torch.allclose(ht, ht2, rtol=1e-14)
    # value head 4 must use q/k head 1 (= 4 // 3), not head 0
    o3, _ = recurrent.recurrent_fwd(q[:, :, 1:2], k[:, :, 1:2], v[:, :, 4:5], g[:, :, 4:5],
                                    beta[:, :, 4:5], h0=h0[:, 4:5], use_qk_l2norm=True)
    assert torch.allclose(o[:, :, 4:5], o3, rtol=1e-14)


def test_equal_channels_equal_scalar_gate():
    q, k, v, g, beta = problem(T=13, seed=18)
    gpc = g[..., None].expand(*g.shape, 8).contiguous()
    h0 = rnd(1, 2, 8, 6, seed=19)
    o1, h1 = recurrent.recurrent_fwd(q, k, v, g, beta, h0=h0)
    o2, h2 = recurrent.recurrent_fwd(q, k, v, gpc, beta, h0=h0)
    assert torch.allclose(o1, o2, rtol=1e-13) and torch.allclose(h1, h2, rtol=1e-13)


@pytest.mark.parametrize("split", [1, 7, 32, 33])
def test_state_passing_split(split):
    q, k, v, g, beta = problem(T=50, seed=20, slow=True)
    h0 = rnd(1, 2, 8, 6, seed=21)
    o, ht = recurrent.recurrent_fwd(q, k, v, g, beta, h0=h0)
    s = slice(0, split)
    r = slice(split, None)
    oa, ha = recurrent.recurrent_fwd(q[:, s], k[:, s], v[:, s], g[:, s], beta[:, s], h0=h0)
    ob, hb = recurrent.recurrent_fwd(q[:, r], k[:, r], v[:, r], g[:, r], beta[:, r], h0=ha)
    assert torch.allclose(torch.cat([oa, ob], 1), o, rtol=1e-12, atol=1e-13)
    assert torch.allclose(hb, ht, rtol=1e-12, atol=1e-13)


def test_varlen_equals_dense_per_sequence():
    lengths = [5, 0, 23, 64, 1]
    T = sum(lengths)
    q, k, v, g, beta = problem(T=T, seed=22)
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32)
    h0 = rnd(len(lengths), 2, 8, 6, seed=23)
    o, ht = recurrent.recurrent_fwd(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
    for n, L in enumerate(lengths):
        s, e = int(cu[n]), int(cu[n + 1])
        on, hn = recurrent.recurrent_fwd(q[:, s:e], k[:, s:e], v[:, s:e], g[:, s:e], beta[:, s:e],
                                         h0=h0[n:n + 1])
        assert torch.allclose(o[:, s:e], on, rtol=1e-14)
        assert torch.allclose(ht[n], hn[0], rtol=1e-14)
    assert torch.equal(ht[1], h0[1])                  # empty sequence: ht = h0


# ----------------------------------------------------------- chunked / WY

def test_forward_substitution_matches_solve():
    A = np.tril(np.random.default_rng(0).standard_normal((3, 12, 12)), -1) * 0.3
    Tm = chunked.forward_substitution(A)
    ref = np.linalg.solve(np.eye(12)[None] + A, np.broadcast_to(np.eye(12), A.shape))
    assert np.allclose(Tm, ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("per_channel", [False, True])
def test_wy_identity(per_channel):
    """P^r and H^r built from the chunk's W and U equal the explicit product of
    gated Householder transitions (coverage-matrix page, section 2); at g = 0
    this is the page's P^r = I - sum k^i w^i^T."""
    q, k, v, g, beta = problem(T=7, H=1, HV=1, K=6, V=4, per_channel=per_channel, seed=24)
    for gate in (g, torch.zeros_like(g)):
        _, _, it = chunked.chunked_fwd(q, k, v, gate, beta, chunk_size=8, intermediates=True)
        L = 7
        W, U = it["W"][0, 0, :L], it["U"][0, 0, :L]
        P, Hs = chunked.wy_factors(k[0, :, 0], beta[0, :, 0], gate[0, :, 0], W, U)
        Pm = torch.eye(6, dtype=f64)
        Hm = torch.zeros(6, 4, dtype=f64)
        I = torch.eye(6, dtype=f64)
        for r in range(L):
            kt = k[0, r, 0]
            gr = gate[0, r, 0]
            D = torch.diag(torch.exp(gr)) if per_channel else torch.exp(gr) * I
            M = (I - beta[0, r, 0] * torch.outer(kt, kt)) @ D
            Pm = M @ Pm
            Hm = M @ Hm + beta[0, r, 0] * torch.outer(kt, v[0, r, 0])
            assert np.allclose(P[r], Pm.numpy(), rtol=1e-11, atol=1e-12)
            assert np.allclose(Hs[r], Hm.numpy(), rtol=1e-11, atol=1e-12)
        if not bool(gate.abs().sum()):
            Wy = np.eye(6) - sum(np.outer(k[0, j, 0].numpy(), W[j]) for j in range(L))
            assert np.allclose(Wy, P[-1], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("C", [1, 2, 7, 32, 64])
@pytest.mark.parametrize("per_channel", [False, True])
def test_chunked_equals_recurrent(C, per_channel):
    q, k, v, g, beta = problem(B=2, T=100, H=2, HV=4, K=8, V=6, per_channel=per_channel,
                               seed=25, slow=True, l2=False)
    h0 = rnd(2, 4, 8, 6, seed=26)
    o, ht = recurrent.recurrent_fwd(q, k, v, g, beta, scale=0.9, h0=h0, use_qk_l2norm=True)
    oc, hc = chunked.chunked_fwd(q, k, v, g, beta, scale=0.9, h0=h0, use_qk_l2norm=True, chunk_size=C)
    assert err_ratio(oc, o) < 1e-12 and err_ratio(hc, ht) < 1e-12


def test_chunked_equals_recurrent_varlen():
    lengths = [70, 3, 0, 129, 64]
    T = sum(lengths)
    q, k, v, g, beta = problem(T=T, H=1, HV=2, K=8, V=5, seed=27, slow=True, l2=False)
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32)
    h0 = rnd(len(lengths), 2, 8, 5, seed=28)
    o, ht = recurrent.recurrent_fwd(q, k, v, g, beta, h0=h0, cu_seqlens=cu, use_qk_l2norm=True)
    oc, hc, it = chunked.chunked_fwd(q, k, v, g, beta, h0=h0, cu_seqlens=cu, use_qk_l2norm=True,
                                     chunk_size=32, intermediates=True)
    assert err_ratio(oc, o) < 1e-12 and err_ratio(hc, ht) < 1e-12
    # h[c] is the state entering chunk c: it equals the per-token state at that token
    for c in (it["off"][3], it["off"][3] + 2):
        n, t0, _ = (int(x) for x in it["idx"][c])
        s = int(cu[n])
        _, hpart = recurrent.recurrent_fwd(q[:, s:t0], k[:, s:t0], v[:, s:t0], g[:, s:t0],
                                           beta[:, s:t0], h0=h0[n:n + 1], use_qk_l2norm=True)
        assert np.allclose(it["h"][c], hpart[0].numpy(), rtol=1e-11, atol=1e-13)


def test_chunk_of_one_is_the_recurrence():
    """With C = 1: T = 1, w = beta exp(g) k, u = beta v, and e = u - w S0
    equals beta (v - (D S0)^T k) of the per-token form term by term."""
    q, k, v, g, beta = problem(T=5, H=1, HV=1, K=4, V=3, seed=29)
    h0 = rnd(1, 1, 4, 3, seed=30)
    _, _, it = chunked.chunked_fwd(q, k, v, g, beta, h0=h0, chunk_size=1, intermediates=True)
    S = h0[0, 0].numpy()
    for t in range(5):
        kt, bt = k[0, t, 0].numpy(), float(beta[0, t, 0])
        d = math.exp(float(g[0, t, 0]))
        assert np.allclose(it["W"][t, 0, 0], bt * d * kt, rtol=1e-14)
        assert np.allclose(it["U"][t, 0, 0], bt * v[0, t, 0].numpy(), rtol=1e-14)
        e = bt * (v[0, t, 0].numpy() - (d * S).T @ kt)
        assert np.allclose(it["E"][t, 0, 0], e, rtol=1e-12)
        S = d * S + np.outer(kt, e)


# -------------------------------------------------------------- backward

def _bwd_inputs(per_channel, seed, T=11, H=1, HV=2, K=4, V=3):
    q, k, v, g, beta = problem(T=T, H=H, HV=HV, K=K, V=V, per_channel=per_channel, seed=seed,
                               slow=True, l2=False)
    h0 = rnd(1, HV, K, V, seed=seed + 100)
    do = rnd(1, T, HV, V, seed=seed + 200)
    dht = rnd(1, HV, K, V, seed=seed + 300)
    return q, k, v, g, beta, h0, do, dht


@pytest.mark.parametrize("per_channel", [False, True])
def test_gradcheck_per_token(per_channel):
    """Autograd of the per-token forward against central differences."""
    q, k, v, g, beta, h0, do, dht = _bwd_inputs(per_channel, 31, T=6, K=3, V=2)

    def f(q_, k_, v_, g_, b_, h_):
        o, ht = recurrent.recurrent_fwd(q_, k_, v_, g_, b_, scale=0.8, h0=h_, use_qk_l2norm=True)
        return (o * do).sum() + (ht * dht).sum()

    args = [x.clone().requires_grad_(True) for x in (q, k, v, g, beta, h0)]
    assert torch.autograd.gradcheck(f, args, eps=1e-6, atol=1e-8, rtol=1e-6)


@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("l2", [False, True])
def test_hand_backward_equals_autograd(per_channel, l2):
    q, k, v, g, beta, h0, do, dht = _bwd_inputs(per_channel, 32, T=19, H=2, HV=4)
    kw = dict(scale=0.6, h0=h0, use_qk_l2norm=l2)
    ref = recurrent.autograd_bwd(q, k, v, g, beta, do, dht, **kw)
    got = recurrent.recurrent_bwd(q, k, v, g, beta, do, dht, ckpt=4, **kw)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert err_ratio(got[n], ref[n]) < 1e-12, n


def test_hand_backward_finite_differences_varlen():
    """Directional central differences of the loss, varlen batch, GVA."""
    lengths = [4, 0, 7]
    T = sum(lengths)
    q, k, v, g, beta, _, do, _ = _bwd_inputs(False, 33, T=T, H=1, HV=2)
    cu = torch.tensor([0, 4, 4, 11], dtype=torch.int32)
    h0 = rnd(3, 2, 4, 3, seed=34)
    dht = rnd(3, 2, 4, 3, seed=35)
    kw = dict(scale=1.1, h0=h0, cu_seqlens=cu, use_qk_l2norm=True)
    grads = recurrent.recurrent_bwd(q, k, v, g, beta, do, dht, ckpt=3, **kw)
    base = dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0)

    def loss(d):
        o, ht = recurrent.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=1.1,
                                        h0=d["h0"], cu_seqlens=cu, use_qk_l2norm=True)
        return float((o * do).sum() + (ht * dht).sum())

    for name in base:
        dirn = rnd(*base[name].shape, seed=hash(name) % 1000)
        eps = 1e-6
        plus = dict(base, **{name: base[name] + eps * dirn})
        minus = dict(base, **{name: base[name] - eps * dirn})
        fd = (loss(plus) - loss(minus)) / (2 * eps)
        an = float((grads["d" + name] * dirn).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), name


def test_beta_zero_dh0_closed_form():
    """beta = 0: dh0 = sum_t exp(Gabs_t) scale q_t do_t^T + exp(Gabs_T) dht."""
    q, k, v, g, beta, h0, do, dht = _bwd_inputs(False, 36, T=9, H=1, HV=1)
    beta = torch.zeros_like(beta)
    got = recurrent.recurrent_bwd(q, k, v, g, beta, do, dht, scale=0.5, h0=h0, ckpt=4)
    Gabs = torch.cumsum(g[0, :, 0], 0)
    ref = torch.exp(Gabs[-1]) * dht[0, 0]
    for t in range(9):
        ref = ref + torch.exp(Gabs[t]) * 0.5 * torch.outer(q[0, t, 0], do[0, t, 0])
    assert torch.allclose(got["dh0"][0, 0], ref, rtol=1e-12)
    assert float(got["dv"].abs().max()) == 0.0     # dv = beta de = 0


def test_err_ratio_definition():
    ref = np.array([3.0, 4.0])
    assert err_ratio(ref, ref) == 0.0
    assert abs(err_ratio(np.array([3.0, 4.0 + 0.5]), ref) - (0.5 / math.sqrt(2)) / (5 / math.sqrt(2))) < 1e-15
    with pytest.raises(AssertionError):
        err_ratio(np.array([np.nan, 1.0]), ref)


# -------------------------------------------------------- chunked backward

@pytest.mark.parametrize("C", [1, 3, 8, 32])
@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("l2", [False, True])
def test_chunked_backward_equals_per_token(C, per_channel, l2):
    q, k, v, g, beta, h0, do, dht = _bwd_inputs(per_channel, 40, T=37, H=2, HV=4, K=5, V=3)
    kw = dict(scale=0.7, h0=h0, use_qk_l2norm=l2)
    ref = recurrent.recurrent_bwd(q, k, v, g, beta, do, dht, ckpt=8, **kw)
    got = chunked.chunked_bwd(q, k, v, g, beta, do, dht, chunk_size=C, **kw)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert err_ratio(got[n], ref[n]) < 1e-11, n


def test_chunked_backward_varlen_and_state_gradients():
    lengths = [9, 0, 20, 1]
    T = sum(lengths)
    q, k, v, g, beta, _, do, _ = _bwd_inputs(False, 41, T=T, H=1, HV=2, K=4, V=3)
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32)
    h0 = rnd(4, 2, 4, 3, seed=42)
    dht = rnd(4, 2, 4, 3, seed=43)
    kw = dict(scale=1.2, h0=h0, cu_seqlens=cu, use_qk_l2norm=True)
    ref = recurrent.autograd_bwd(q, k, v, g, beta, do, dht, **kw)
    got = chunked.chunked_bwd(q, k, v, g, beta, do, dht, chunk_size=8, intermediates=True, **kw)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert err_ratio(got[n], ref[n]) < 1e-11, n
    # dh[c] is the gradient w.r.t. the state leaving chunk c: for the last chunk
    # of a sequence it is dht
    it = got["inter"]
    for n in range(4):
        if lengths[n]:
            last = it["off"][n + 1] - 1
            assert np.allclose(it["dh"][last], dht[n].numpy())
    # dE is the gradient w.r.t. E = T (beta V - ...) taken as a free output, so
    # dv = beta T^T dE per chunk (T from the forward oracle), and with dS1 = 0,
    # dE reduces to its chunk-local part dEi for the last chunk of a sequence
    # whose dht is zero
    _, _, fi = chunked.chunked_fwd(q, k, v, g, beta, chunk_size=8, intermediates=True, **kw)
    for c in range(len(it["idx"])):
        _, t0, L = (int(x) for x in it["idx"][c])
        dv_c = got["dv"][0, t0:t0 + L]                       # [L,HV,V]
        be = beta[0, t0:t0 + L].numpy()[:, :, None]
        TtdE = np.transpose(fi["T"][c, :, :L, :L], (0, 2, 1)) @ it["dE"][c, :, :L]
        assert np.allclose(dv_c, be * np.transpose(TtdE, (1, 0, 2)), atol=1e-12)
    got0 = chunked.chunked_bwd(q, k, v, g, beta, do, torch.zeros_like(dht), chunk_size=8,
                               intermediates=True, **kw)
    for n in range(4):
        if lengths[n]:
            last = got0["inter"]["off"][n + 1] - 1
            assert np.allclose(got0["inter"]["dE"][last], got0["inter"]["dEi"][last], atol=1e-14)


@pytest.mark.parametrize("pc", [False, True])
def test_transition_chains_segments(pc):
    """The segment transition M is pinned by the property that defines it:
    for any start state S0, running the per-token recurrence over the segment
    from S0 ends in M S0 + (the end state from zero).  Checked on random S0
    for two unaligned segments of a GVA batch, and M of the concatenation is
    the product of the two segments' transitions."""
    w = workloads.Workload("tr", B=1, T=0, H=1, HV=2, K=8, V=5, chunk_size=64, dtype="fp32",
                           per_channel_gate=pc, l2norm_in_kernel=True, slow_decay=True)
    inp = workloads.make_inputs(w, lengths=[9, 14])
    q, k, v, g, beta = (inp[n] for n in ("q", "k", "v", "g", "beta"))
    cu = inp["cu_seqlens"]
    M = recurrent.transition(k, g, beta, cu_seqlens=cu, use_qk_l2norm=True)
    S0 = torch.randn(2, 2, 8, 5, generator=torch.Generator().manual_seed(3), dtype=torch.float64)
    _, ht = recurrent.recurrent_fwd(q, k, v, g, beta, h0=S0, cu_seqlens=cu, use_qk_l2norm=True)
    _, ht0 = recurrent.recurrent_fwd(q, k, v, g, beta, h0=None, cu_seqlens=cu, use_qk_l2norm=True)
    np.testing.assert_allclose((M @ S0 + ht0).numpy(), ht.numpy(), rtol=1e-12, atol=1e-12)
    whole = torch.tensor([0, 23], dtype=torch.int32)
    Mw = recurrent.transition(k, g, beta, cu_seqlens=whole, use_qk_l2norm=True)
    np.testing.assert_allclose(Mw[0].numpy(), (M[1] @ M[0]).numpy(), rtol=1e-12, atol=1e-12)


def test_transition_at_zero_gate_is_the_wy_product():
    """At g = 0 the transition of one chunk is the page's P^r = I - sum_i k^i w^i^T
    with w from the chunked oracle's WY factors (a separate code path)."""
    w = workloads.Workload("trwy", B=1, T=12, H=1, HV=1, K=6, V=4, chunk_size=64, dtype="fp32",
                           host_l2norm=True)
    inp = workloads.make_inputs(w)
    g0 = torch.zeros_like(inp["g"])
    M = recurrent.transition(inp["k"], g0, inp["beta"])
    _, _, it = chunked.chunked_fwd(inp["q"], inp["k"], inp["v"], g0, inp["beta"], chunk_size=64,
                                   intermediates=True)
    kk = inp["k"][0, :, 0].double().numpy()
    W = it["W"][0, 0][:12]
    P = np.eye(6) - kk.T @ W
    np.testing.assert_allclose(M[0, 0].numpy(), P, rtol=1e-12, atol=1e-12)


def test_simple_gla_matches_its_parallel_form():
    """The per-token simple GLA oracle against its closed (attention) form,
    written out independently: o_t = scale [exp(G_t) q_t^T S0 +
    sum_{s<=t} exp(G_t - G_s) (q_t . k_s) v_s] and
    ht = exp(G_T) S0 + sum_s exp(G_T - G_s) k_s v_s^T, G the inclusive cumsum,
    on a varlen GVA batch with an empty sequence."""
    w = workloads.Workload("gla", B=1, T=0, H=1, HV=2, K=5, V=3, chunk_size=64, dtype="fp32",
                           l2norm_in_kernel=True, slow_decay=True, scale=0.7)
    inp = workloads.make_inputs(w, lengths=[7, 0, 11])
    q, k, v, g, h0, cu = (inp[n] for n in ("q", "k", "v", "g", "h0", "cu_seqlens"))
    o, ht = recurrent.simple_gla_fwd(q, k, v, g, scale=0.7, h0=h0, cu_seqlens=cu, use_qk_l2norm=True)
    qd, kd = q.double(), k.double()
    qn = qd / torch.sqrt((qd * qd).sum(-1, keepdim=True) + 1e-6)
    kn = kd / torch.sqrt((kd * kd).sum(-1, keepdim=True) + 1e-6)
    for n in range(3):
        s, e = int(cu[n]), int(cu[n + 1])
        for j in range(2):
            G = torch.cumsum(g[0, s:e, j].double(), 0)
            L = e - s
            for t in range(L):
                ref = torch.exp(G[t]) * (h0[n, j].double().T @ qn[0, s + t, 0])
                for u in range(t + 1):
                    ref = ref + torch.exp(G[t] - G[u]) * (qn[0, s + t, 0] @ kn[0, s + u, 0]) * v[0, s + u, j].double()
                np.testing.assert_allclose(o[0, s + t, j].numpy(), 0.7 * ref.numpy(), rtol=1e-12, atol=1e-12)
            Gt = G[-1] if L else torch.tensor(0.0, dtype=torch.float64)
            hr = torch.exp(Gt) * h0[n, j].double()
            for u in range(L):
                hr = hr + torch.exp(Gt - G[u]) * torch.outer(kn[0, s + u, 0], v[0, s + u, j].double())
            np.testing.assert_allclose(ht[n, j].numpy(), hr.numpy(), rtol=1e-12, atol=1e-12)


def test_beta_logits_chain_rule():
    """The beta-logits mode (beta = sigmoid(x), the beta-mode axis of the
    coverage-matrix page, section 3) composes the oracle with a sigmoid; the
    gradient with respect to x is dbeta * beta * (1 - beta).  Pinned by
    autograd through the per-token oracle with the sigmoid inside."""
    w = workloads.Workload("bl", B=1, T=13, H=1, HV=2, K=6, V=4, chunk_size=64, dtype="fp32",
                           l2norm_in_kernel=True, slow_decay=True, backward=True)
    inp = workloads.make_inputs(w)
    x = torch.logit(inp["beta"]).double().requires_grad_(True)
    o, ht = recurrent.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], torch.sigmoid(x), h0=inp["h0"],
                                    use_qk_l2norm=True)
    ((o * inp["do"].double()).sum() + (ht * inp["dht"].double()).sum()).backward()
    b = torch.sigmoid(x.detach())
    ref = chunked.chunked_bwd(inp["q"], inp["k"], inp["v"], inp["g"], b, inp["do"], inp["dht"], h0=inp["h0"],
                              use_qk_l2norm=True, chunk_size=8)
    np.testing.assert_allclose(x.grad.numpy(), ref["dbeta"] * (b * (1 - b)).numpy(), rtol=1e-9, atol=1e-12)
