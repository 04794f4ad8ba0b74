"""GPU parity of the backward path (K0-K3 recompute, B1 de_local, B2 reverse
state-gradient scan, B3 fused gradients) against the float64 chunk-wise
backward oracle, which is itself pinned to the per-token backward, autograd and
finite differences (tests/test_oracle.py).

Tolerances as for the forward: err_ratio = RMS(diff) / RMS(ref) <= 1e-4 for
float32 and <= 5e-3 for bf16 on every gradient (the per-gradient acceptance
line of the KCP page, "flash-linear-attention KCP precision-failure root-cause
manual", acceptance section) and on the intermediates de_local and dh.
"""
import numpy as np
import pytest
import torch

import chunked_gated_delta_06_amd as gdr
import workloads
from oracle import chunked, recurrent
from fwd_helpers import TOL, check, dev, f64, slice_inputs

pytestmark = pytest.mark.gpu

W = workloads.Workload
GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def mk(name="b", B=2, T=200, H=2, HV=2, K=64, V=64, C=64, dtype="bf16", l2=True, h0=True,
       slow=False, lengths=None, scale=1.0, seed=11, host_l2=False, pc=False):
    w = W(name, B=B, T=T, H=H, HV=HV, K=K, V=V, chunk_size=C, dtype=dtype, per_channel_gate=pc,
          l2norm_in_kernel=l2, host_l2norm=host_l2, h0=h0, slow_decay=slow, scale=scale, backward=True)
    return w, workloads.make_inputs(w, seed=seed, lengths=lengths)


def gpu_bwd(inp, *, h0=True, dht=True, workspace=None, out=None):
    """Library backward; returns (dict of gradients as CPU float64 arrays or
    None, workspace views, raw device outputs)."""
    res = gdr.chunk_bwd(
        dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]), dev(inp["do"]),
        dev(inp["dht"]) if dht else None, scale=inp["scale"], chunk_size=inp["chunk_size"],
        cu_seqlens=dev(inp["cu_seqlens"]), initial_state=dev(inp["h0"]) if h0 else None,
        use_qk_l2norm_in_kernel=inp["use_qk_l2norm"], workspace=workspace, return_workspace=True,
        out=out)
    torch.cuda.synchronize()
    *grads, ws = res
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=inp["chunk_size"],
                         cu_seqlens=inp["cu_seqlens"], use_qk_l2norm=inp["use_qk_l2norm"],
                         scale=inp["scale"])
    views = gdr.bwd_workspace_views(p, ws)
    got = {n: (None if t is None else f64(t)) for n, t in zip(GRADS, grads)}
    return got, views, grads


def oracle_bwd(inp, *, h0=True, dht=True, intermediates=False):
    return chunked.chunked_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["do"],
                               inp["dht"] if dht else None, scale=inp["scale"],
                               h0=inp["h0"] if h0 else None, cu_seqlens=inp["cu_seqlens"],
                               use_qk_l2norm=inp["use_qk_l2norm"], chunk_size=inp["chunk_size"],
                               intermediates=intermediates)


def compare(got, ref, tol, names=GRADS):
    out = {}
    for n in names:
        if got.get(n) is None:
            continue
        out[n] = check(n, got[n], ref[n], tol)
    return out


# ------------------------------------------------------------------ stages

STAGE_CASES = [
    dict(dtype="fp32", K=32, V=32, C=64),
    dict(dtype="fp32", K=128, V=64, C=32),
    dict(dtype="bf16", K=128, V=128, C=64),
    dict(dtype="bf16", K=64, V=32, C=64, H=1, HV=4),
    dict(dtype="bf16", K=128, V=256, C=32, l2=False, host_l2=True),
]


@pytest.mark.parametrize("case", range(len(STAGE_CASES)))
def test_bwd_stage_intermediates(case):
    kw = STAGE_CASES[case]
    w, inp = mk(**kw, slow=True)
    tol = TOL[w.dtype]
    got, views, _ = gpu_bwd(inp)
    ref = oracle_bwd(inp, intermediates=True)
    it = ref["inter"]
    NT = int(it["off"][-1])
    C = w.chunk_size
    # chunk table (recomputed by the backward)
    assert np.array_equal(views["chunk_idx"][:NT, :3].cpu().numpy(), it["idx"])
    # de_local = scale P^T dO, stored transposed per chunk
    de = f64(views["de_local"][:NT].transpose(-1, -2))
    check("de_local", de, it["dEi"], tol)
    # qscale = scale exp(G_r) / |q_r| on valid rows, 0 past the chunk end
    _, _, fi = chunked.chunked_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                   scale=inp["scale"], h0=inp["h0"], chunk_size=C,
                                   use_qk_l2norm=inp["use_qk_l2norm"], intermediates=True)
    q64 = inp["q"].double()
    rq = (1.0 / torch.sqrt((q64 * q64).sum(-1) + 1e-6)) if inp["use_qk_l2norm"] else torch.ones(q64.shape[:-1], dtype=torch.float64)
    rq = rq.reshape(-1, w.H).repeat_interleave(w.HV // w.H, dim=1).numpy()     # [B*T, HV]
    ref_qs = np.zeros((NT, w.HV, C))
    for c in range(NT):
        _, t0, L = (int(x) for x in it["idx"][c])
        ref_qs[c, :, :L] = inp["scale"] * np.exp(fi["G"][c, :, :L]) * rq[t0:t0 + L].T
    qs = f64(views["qscale"][:NT])
    check("qscale", qs, ref_qs, 1e-5)
    assert np.all(qs[ref_qs == 0] == 0)
    # dh: gradient of the state leaving each chunk (transposed per chunk)
    check("dh", f64(views["dh"][:NT].transpose(-1, -2)), it["dh"], tol)
    compare(got, ref, tol)


# ------------------------------------------------------------------ sweep

SWEEP = [
    dict(dtype="fp32", K=32, V=32, C=32),
    dict(dtype="fp32", K=64, V=128, C=64),
    dict(dtype="fp32", K=128, V=32, C=32, H=1, HV=2),
    dict(dtype="bf16", K=32, V=32, C=32),
    dict(dtype="bf16", K=32, V=64, C=32, H=2, HV=4),
    dict(dtype="bf16", K=64, V=64, C=64),
    dict(dtype="bf16", K=64, V=128, C=32),
    dict(dtype="bf16", K=128, V=64, C=32, H=2, HV=4),
    dict(dtype="bf16", K=128, V=128, C=64, l2=False, host_l2=True),
    dict(dtype="bf16", K=128, V=256, C=64, H=1, HV=2),
]


@pytest.mark.parametrize("case", range(len(SWEEP)))
def test_bwd_sweep(case):
    kw = SWEEP[case]
    w, inp = mk(**kw, scale=kw["K"] ** -0.5, seed=20 + case)
    got, _, _ = gpu_bwd(inp)
    compare(got, oracle_bwd(inp), TOL[w.dtype])


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_bwd_matches_per_token_backward(dtype):
    """End to end against the hand-derived per-token reverse recurrence."""
    w, inp = mk(dtype=dtype, B=1, T=150, K=32, V=32, C=32, slow=True, seed=3)
    got, _, _ = gpu_bwd(inp)
    ref = recurrent.recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["do"],
                                  inp["dht"], scale=inp["scale"], h0=inp["h0"],
                                  use_qk_l2norm=inp["use_qk_l2norm"])
    compare(got, {n: f64(t) if torch.is_tensor(t) else t for n, t in ref.items()}, TOL[dtype])


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_bwd_varlen_ragged(dtype):
    lengths = [0, 1, 63, 64, 65, 200, 0, 7, 130]
    w, inp = mk(dtype=dtype, B=1, T=sum(lengths), H=2, HV=4, K=64, V=32, C=64, lengths=lengths,
                seed=5)
    got, _, _ = gpu_bwd(inp)
    ref = oracle_bwd(inp)
    tol = TOL[dtype]
    compare(got, ref, tol)
    # every sequence on its own (per-sequence ratios, as on the KCP page)
    cu = inp["cu_seqlens"].numpy()
    for n in range(len(lengths)):
        s, e = int(cu[n]), int(cu[n + 1])
        if e - s < 16:
            continue
        for name in ("dq", "dk", "dv"):
            check(f"{name} seq {n}", got[name][:, s:e], ref[name][:, s:e], tol)
    check("dh0 of empty sequences", got["dh0"][[0, 6]], inp["dht"][[0, 6]].double().numpy(), 0.0)


@pytest.mark.parametrize("h0,dht", [(False, True), (True, False), (False, False)])
def test_bwd_optional_states(h0, dht):
    w, inp = mk(T=130, K=64, V=64, C=32, seed=9)
    got, _, _ = gpu_bwd(inp, h0=h0, dht=dht)
    compare(got, oracle_bwd(inp, h0=h0, dht=dht), TOL["bf16"])


def test_bwd_no_dh0_wanted():
    w, inp = mk(T=100, K=32, V=32, C=32, seed=13)
    res = gdr.chunk_bwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
                        dev(inp["do"]), dev(inp["dht"]), chunk_size=32, initial_state=dev(inp["h0"]),
                        use_qk_l2norm_in_kernel=True, want_dh0=False)
    torch.cuda.synchronize()
    assert res[5] is None
    ref = oracle_bwd(inp)
    for n, t in zip(GRADS[:5], res[:5]):
        check(n, f64(t), ref[n], TOL["bf16"])


def test_bwd_empty_batch():
    """T = 0: no token gradients; dh0 = dht for every sequence."""
    w, inp = mk(B=1, T=0, lengths=[0, 0, 0], K=32, V=32, C=64)
    got, _, _ = gpu_bwd(inp)
    assert np.array_equal(got["dh0"], inp["dht"].double().numpy())


def test_bwd_single_tokens():
    lengths = [1] * 9
    w, inp = mk(B=1, T=9, lengths=lengths, K=32, V=64, C=32, seed=17)
    got, _, _ = gpu_bwd(inp)
    compare(got, oracle_bwd(inp), TOL["bf16"])


def test_bwd_beta_zero_closed_form():
    """beta = 0: pure decay, dh0 = sum_t scale exp(Gabs_t) q^_t do_t^T + exp(Gabs_T) dht,
    dk = dv = 0 (a closed form independent of the chunk algebra)."""
    w, inp = mk(B=1, T=90, H=1, HV=1, K=32, V=32, C=32, dtype="fp32", seed=19)
    inp["beta"] = torch.zeros_like(inp["beta"])
    got, _, _ = gpu_bwd(inp)
    q = inp["q"].double()[0, :, 0]
    qh = q / torch.sqrt((q * q).sum(-1, keepdim=True) + 1e-6)
    Gabs = torch.cumsum(inp["g"].double()[0, :, 0], 0)
    do = inp["do"].double()[0, :, 0]
    ref = inp["scale"] * torch.einsum("t,tk,tv->kv", torch.exp(Gabs), qh, do) + torch.exp(Gabs[-1]) * inp["dht"].double()[0, 0]
    check("dh0 (beta=0)", got["dh0"][0, 0], ref.numpy(), 1e-4)
    assert np.abs(got["dk"]).max() == 0 and np.abs(got["dv"]).max() == 0


def test_bwd_deterministic_and_poisoned():
    """Two runs are bitwise equal; NaN-poisoned workspace and outputs are fully
    overwritten."""
    w, inp = mk(B=1, T=333, H=2, HV=4, K=128, V=64, C=64, seed=23)
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=64, use_qk_l2norm=True)
    lay = gdr.bwd_layout(p)
    ws = torch.empty(lay.total, dtype=torch.uint8, device="cuda")
    ws.view(torch.int8).fill_(-1)     # 0xFF bytes: NaN in bf16 and fp32
    outs = tuple(torch.full_like(dev(x), float("nan")) for x in
                 (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"]))
    dh0 = torch.full((1, 4, 128, 64), float("nan"), device="cuda")
    got1, _, raw1 = gpu_bwd(inp, workspace=ws, out=outs + (dh0,))
    for n in GRADS:
        assert np.isfinite(got1[n]).all(), n
    got2, _, _ = gpu_bwd(inp)
    for n in GRADS:
        assert np.array_equal(got1[n], got2[n]), n
    compare(got1, oracle_bwd(inp), TOL["bf16"])


@pytest.mark.parametrize("varlen", [False, True])
def test_bwd_reuses_saved_forward_states(varlen):
    """A forward with keep_states on the backward-sized workspace, then the
    backward with reuse_forward: the same gradients, bitwise, as the backward
    that recomputes the forward intermediates (the same kernels made them), and
    within tolerance of the oracle."""
    lengths = [70, 0, 129, 64] if varlen else None
    w, inp = mk(B=1 if varlen else 2, T=170, H=2, HV=4, K=128, V=64, slow=True, lengths=lengths)
    ref_got, _, _ = gpu_bwd(inp)
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=64, cu_seqlens=inp["cu_seqlens"],
                         use_qk_l2norm=True)
    lay = gdr.bwd_layout(p)
    ws = torch.full((lay.total,), 0xFF, dtype=torch.uint8, device="cuda")   # poisoned
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "do", "dht", "h0", "cu_seqlens")}
    o, ht = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                          initial_state=d["h0"], use_qk_l2norm_in_kernel=True, workspace=ws, keep_states=True)
    grads = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["dht"],
                          cu_seqlens=d["cu_seqlens"], initial_state=d["h0"], use_qk_l2norm_in_kernel=True,
                          workspace=ws, reuse_forward=True)
    torch.cuda.synchronize()
    for n, t in zip(GRADS, grads):
        assert np.array_equal(f64(t), ref_got[n]), n
    compare(ref_got, oracle_bwd(inp), TOL["bf16"])
    with pytest.raises(ValueError, match="reuse_forward"):
        gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["dht"], cu_seqlens=d["cu_seqlens"],
                      initial_state=d["h0"], use_qk_l2norm_in_kernel=True, reuse_forward=True)


def test_bwd_unsupported_shapes_raise():
    """K = 256 has no backward instantiation; a per-channel gate through the
    per-stage entry points (which take no gated rows) is refused too."""
    w, inp = mk(T=64, K=256, V=64, C=64)
    with pytest.raises(ValueError, match="backward supports"):
        gdr.chunk_bwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
                      dev(inp["do"]), None, chunk_size=64)
    w, inp = mk(T=64, K=64, V=64, C=32, pc=True)
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=32, use_qk_l2norm=True)
    x = torch.zeros(1024, device="cuda")
    with pytest.raises(ValueError, match="backward supports"):
        gdr.bwd_intra(p, dev(inp["q"]), dev(inp["k"]), dev(inp["g"]), dev(inp["do"]), x, x, x, x)


def test_bwd_varlen_equals_dense_rows():
    """A varlen batch of equal-length sequences gives bitwise the gradients of the
    dense batch with those rows."""
    w, inp = mk(B=3, T=150, K=64, V=64, C=64, seed=29)
    gd, _, _ = gpu_bwd(inp)
    vl = dict(inp)
    for n in ("q", "k", "v", "g", "beta", "do"):
        vl[n] = inp[n].reshape(1, 3 * 150, *inp[n].shape[2:]).contiguous()
    vl["cu_seqlens"] = torch.tensor([0, 150, 300, 450], dtype=torch.int32)
    gv, _, _ = gpu_bwd(vl)
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.array_equal(gv[n].reshape(gd[n].shape), gd[n]), n
    assert np.array_equal(gv["dh0"], gd["dh0"])


# ------------------------------------------------------------------ full-size workload

@pytest.mark.timeout(300)
def test_config_long_bf16_backward():
    """The long single-sequence workload (B=1, T=65536, H=HV=32, K=V=128,
    fwd+bwd) at full size on the GPU, checked on a sampled head against the
    chunk-wise oracle run on that head (H == HV, so the head's dq / dk have no
    other contributions)."""
    w = workloads.CONFIGS["long_bf16"]
    inp = workloads.make_inputs(w)
    res = gdr.chunk_bwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
                        dev(inp["do"]), dev(inp["dht"]), scale=inp["scale"], chunk_size=w.chunk_size,
                        initial_state=dev(inp["h0"]), use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    heads = [21]
    for n, t in zip(GRADS, res):
        assert bool(torch.isfinite(t).all()), n
    got = {n: f64(t[:, :, heads] if n != "dh0" else t[:, heads]) for n, t in zip(GRADS, res)}
    del res
    torch.cuda.empty_cache()
    ref = oracle_bwd(slice_inputs(inp, heads=heads))
    compare(got, ref, TOL[w.dtype])


@pytest.mark.timeout(300)
def test_config_long_bf16_gate_gradient_second_head():
    """The long single-sequence workload at full size again, with dg (the
    gradient the rounding reaches most) and dbeta checked on value head 5
    against the chunk-wise oracle of that head, at 4e-3."""
    w = workloads.CONFIGS["long_bf16"]
    inp = workloads.make_inputs(w)
    res = gdr.chunk_bwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
                        dev(inp["do"]), dev(inp["dht"]), scale=inp["scale"], chunk_size=w.chunk_size,
                        initial_state=dev(inp["h0"]), use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    heads = [5]
    got = {n: f64(t[:, :, heads]) for n, t in zip(GRADS, res) if n in ("dg", "dbeta")}
    del res
    torch.cuda.empty_cache()
    ref = oracle_bwd(slice_inputs(inp, heads=heads))
    compare(got, ref, 4e-3, names=("dg", "dbeta"))


def test_beta_logits_mode():
    """beta passed as logits (the kernels apply the sigmoid): forward (fused and
    separate stages, token by token) and backward against the oracle run on
    sigmoid(logits); the logits' gradient is dbeta * beta (1 - beta)."""
    w, inp = mk(B=2, T=150, H=2, HV=4, K=128, V=64, slow=True)
    x = torch.logit(inp["beta"])                     # the logits the kernels read
    b = torch.sigmoid(x.double())
    ref_inp = dict(inp, beta=b)
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "g", "do", "dht", "h0")}
    xd = dev(x.contiguous())
    ro, rht = chunked.chunked_fwd(inp["q"], inp["k"], inp["v"], inp["g"], b, h0=inp["h0"], use_qk_l2norm=True,
                                  chunk_size=64)
    for keep in (False, True):
        o, ht = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], xd, initial_state=d["h0"],
                              use_qk_l2norm_in_kernel=True, keep_states=keep, beta_logits=True)
        torch.cuda.synchronize()
        check(f"o keep={keep}", f64(o), ro, TOL["bf16"])
        check(f"ht keep={keep}", f64(ht), rht, TOL["bf16"])
    o, ht = gdr.fused_recurrent_fwd(d["q"], d["k"], d["v"], d["g"], xd, initial_state=d["h0"],
                                    use_qk_l2norm_in_kernel=True, beta_logits=True)
    torch.cuda.synchronize()
    check("o token-by-token", f64(o), ro, TOL["bf16"])
    grads = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], xd, d["do"], d["dht"], initial_state=d["h0"],
                          use_qk_l2norm_in_kernel=True, beta_logits=True)
    torch.cuda.synchronize()
    ref = oracle_bwd(ref_inp)
    ref["dbeta"] = ref["dbeta"] * (b * (1 - b)).numpy()
    compare({n: f64(t) for n, t in zip(GRADS, grads)}, ref, TOL["bf16"])


def test_beta_logits_persistent_backward():
    """beta as logits on the backward's persistent grid (bf16, chunk 64,
    K = 128, H = HV: one workgroup per compute unit looping over 260 (chunk,
    head) items, each fetching the next item's rows and beta during its own
    finish), ragged tail; every gradient against the oracle on sigmoid(logits)."""
    w, inp = mk(B=1, T=64 * 129 + 17, H=2, HV=2, K=128, V=128, slow=True)
    x = torch.logit(inp["beta"])
    b = torch.sigmoid(x.double())
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "g", "do", "dht", "h0")}
    grads = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], dev(x.contiguous()), d["do"], d["dht"],
                          initial_state=d["h0"], use_qk_l2norm_in_kernel=True, beta_logits=True)
    torch.cuda.synchronize()
    ref = oracle_bwd(dict(inp, beta=b))
    ref["dbeta"] = ref["dbeta"] * (b * (1 - b)).numpy()
    compare({n: f64(t) for n, t in zip(GRADS, grads)}, ref, TOL["bf16"])


@pytest.mark.parametrize("pc", [False, True], ids=["scalar", "per_channel"])
def test_bwd_int64_offsets(pc):
    """The backward on a varlen batch whose last sequence sits past 2^31
    elements of q / k / v / do, of the gradients and of the per-chunk state
    and state-gradient tensors (bf16, 16 heads; scalar gate at chunk 64 on the
    persistent B3, per-channel gate at chunk 32); only that sequence's
    gradients are checked, against the oracle on it alone."""
    H = HV = 16
    K = V = 128
    tail = 192
    s = (1 << 20) + 64          # the checked sequence starts past 2^31 elements
    T = s + tail
    assert s * H * K > 2 ** 31
    gen = torch.Generator().manual_seed(5)
    qt = torch.randn(1, tail, H, K, generator=gen).bfloat16()
    kt = torch.randn(1, tail, H, K, generator=gen).bfloat16()
    vt = torch.randn(1, tail, HV, V, generator=gen).bfloat16()
    dot = torch.randn(1, tail, HV, V, generator=gen).bfloat16()
    gw = (HV, K) if pc else (HV,)
    C = 32 if pc else 64
    gt = torch.nn.functional.logsigmoid(torch.randn(1, tail, *gw, generator=gen) + 4)
    bt = torch.sigmoid(torch.randn(1, tail, HV, generator=gen))
    h0 = 0.1 * torch.randn(2, HV, K, V, generator=gen)
    dht = torch.randn(2, HV, K, V, generator=gen)

    def full(x, width):
        y = torch.zeros(1, T, *width, dtype=x.dtype, device="cuda")
        y[:, s:] = x.cuda()
        return y

    cu = torch.tensor([0, s, T], dtype=torch.int32)
    grads = gdr.chunk_bwd(full(qt, (H, K)), full(kt, (H, K)), full(vt, (HV, V)), full(gt, gw),
                          full(bt, (HV,)), full(dot, (HV, V)), dev(dht), scale=1.0, chunk_size=C,
                          cu_seqlens=dev(cu), initial_state=dev(h0), use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    got = {n: f64(t[1:2] if n == "dh0" else t[:, s:]) for n, t in zip(GRADS, grads)}
    del grads
    torch.cuda.empty_cache()
    sub = dict(q=qt, k=kt, v=vt, g=gt, beta=bt, do=dot, dht=dht[1:2], h0=h0[1:2], cu_seqlens=None,
               scale=1.0, use_qk_l2norm=True, chunk_size=C)
    compare(got, oracle_bwd(sub), TOL["bf16"])


@pytest.mark.parametrize("cfg", [dict(B=2, T=512, H=2, HV=4, K=60, V=60),
                                 dict(B=1, T=130, H=1, HV=2, K=60, V=36, C=32, dtype="fp32"),
                                 dict(B=1, T=100, H=2, HV=2, K=100, V=20, C=32),
                                 dict(B=1, T=100, H=2, HV=2, K=100, V=20, C=32, dtype="fp32")],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_bwd_padded_head_dims(cfg):
    """The backward with head dims that run zero-padded (the page's D = 60, and
    K = 100 with a small V = 20); the padding adds only exact zeros to every
    contraction."""
    w, inp = mk(slow=True, **cfg)
    got, _, _ = gpu_bwd(inp)
    compare(got, oracle_bwd(inp), TOL[w.dtype])


@pytest.mark.parametrize("V", [20, 32, 128])
@pytest.mark.parametrize("seed", [11, 12, 13])
def test_bwd_bf16_gradient_margin(V, seed):
    """bf16 gradients keep a margin under the 5e-3 acceptance line on shapes
    where the gate gradient is most exposed to rounding (small V, slow decay,
    long-lived states, chunk 32, K = 100 zero-padded to 128): every gradient
    within 4e-3.  The bound rests on fp32 u (and its Tm diag(beta) operand as
    a hi + lo pair), fp32 dh and the scan's e operand as a hi + lo pair; with
    those intermediates in bf16 the gate gradient of these shapes reached
    5e-3 to 7e-3 (a float64 emulation of the rounding points, and one GPU
    measurement of 5.1e-3 at V = 20)."""
    w, inp = mk(B=1, T=100, H=2, HV=2, K=100, V=V, C=32, slow=True, seed=seed)
    got, _, _ = gpu_bwd(inp)
    compare(got, oracle_bwd(inp), 4e-3)


def test_bwd_fp32_k128_chunk64_runs_at_chunk32():
    """fp32 with K = 128 at chunk 64 has no backward instantiation; the library
    runs that backward at chunk 32 (the chunk form is exact at any chunk size)
    and matches the oracle at the fp32 bound."""
    w, inp = mk(B=1, T=150, H=2, HV=2, K=128, V=64, C=64, dtype="fp32", slow=True)
    got, _, _ = gpu_bwd(inp)
    compare(got, oracle_bwd(inp), TOL["fp32"])


# ------------------------------------------------------------------ per-channel gate (KDA-style)

PC_SWEEP = [
    dict(dtype="bf16", K=128, V=256, C=32, H=2, HV=2),
    dict(dtype="bf16", K=64, V=32, C=32, H=1, HV=4),
    dict(dtype="bf16", K=32, V=64, C=32, H=2, HV=2, l2=False, host_l2=True),
    dict(dtype="bf16", K=128, V=64, C=64, H=2, HV=4),                      # chunk 64 runs at 32
    dict(dtype="fp32", K=64, V=128, C=32, H=2, HV=2),
    dict(dtype="fp32", K=128, V=32, C=32, H=1, HV=2),
    dict(dtype="fp32", K=32, V=32, C=64, H=2, HV=2),
]


@pytest.mark.parametrize("case", range(len(PC_SWEEP)))
def test_bwd_per_channel_sweep(case):
    """The per-channel gate's backward (dg per channel, [B,T,HV,K]) on a ragged
    dense batch with slow decay and h0 / dht, against the chunk-wise oracle."""
    kw = PC_SWEEP[case]
    w, inp = mk(**kw, T=150, pc=True, slow=True, scale=kw["K"] ** -0.5, seed=40 + case)
    got, _, _ = gpu_bwd(inp)
    assert got["dg"].shape == tuple(inp["g"].shape)
    compare(got, oracle_bwd(inp), TOL[w.dtype])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bwd_per_channel_varlen(dtype):
    lengths = [0, 1, 31, 32, 33, 100, 0, 7, 70]
    w, inp = mk(dtype=dtype, B=1, T=sum(lengths), H=2, HV=4, K=64, V=64, C=32, lengths=lengths, pc=True,
                slow=True, seed=6)
    got, _, _ = gpu_bwd(inp)
    ref = oracle_bwd(inp)
    compare(got, ref, TOL[dtype])
    cu = inp["cu_seqlens"].numpy()
    for n in range(len(lengths)):
        s, e = int(cu[n]), int(cu[n + 1])
        if e - s < 16:
            continue
        for name in ("dq", "dk", "dv", "dg"):
            check(f"{name} seq {n}", got[name][:, s:e], ref[name][:, s:e], TOL[dtype])


def test_bwd_per_channel_intermediates():
    """The per-channel intra-chunk stage's de_local and the reverse scan's dh
    against the oracle's chunk-wise intermediates."""
    w, inp = mk(B=1, T=100, H=2, HV=2, K=64, V=64, C=32, pc=True, slow=True, seed=8)
    got, views, _ = gpu_bwd(inp)
    ref = oracle_bwd(inp, intermediates=True)
    it = ref["inter"]
    NT = int(it["off"][-1])
    check("de_local", f64(views["de_local"][:NT].transpose(-1, -2)), it["dEi"], TOL["bf16"])
    check("dh", f64(views["dh"][:NT].transpose(-1, -2)), it["dh"], TOL["bf16"])
    compare(got, ref, TOL["bf16"])


@pytest.mark.parametrize("pc", [False, True])
def test_bwd_reverse_scan_four_wave_grid(pc):
    """N * HV * V / 64 = 256 at chunk 32, K = 128, bf16: the reverse scan runs
    four compute waves (64 value columns) per workgroup.  A ragged tail, h0
    and slow decay, every gradient against the oracle on three heads."""
    w, inp = mk(B=2, T=77, H=32, HV=32, K=128, V=256, C=32, pc=pc, slow=True, seed=21, scale=128 ** -0.5)
    assert w.B * w.HV * (w.V // 64) >= 256
    heads = [0, 17, 31]
    res = gdr.chunk_bwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
                        dev(inp["do"]), dev(inp["dht"]), scale=inp["scale"], chunk_size=32,
                        initial_state=dev(inp["h0"]), use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    got = {n: f64(t[:, :, heads] if n != "dh0" else t[:, heads]) for n, t in zip(GRADS, res)}
    compare(got, oracle_bwd(slice_inputs(inp, heads=heads)), TOL["bf16"])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bwd_per_channel_wide_gate_span(dtype):
    """Per-channel gates of -9 per token on some channels (about 144 of decay
    inside a 16-row block, past the span below which the gated pair sums run
    on matrix cores, so those chunks take the exact per-term pass) and mild
    gates elsewhere in the batch, on a ragged dense batch: every gradient
    against the oracle."""
    w, inp = mk(dtype=dtype, B=2, T=100, H=2, HV=2, K=64, V=64, C=32, pc=True, seed=14)
    g = inp["g"].clone()
    g[0, :, :, ::3] = -9.0           # row 0: wide spans on every third channel
    g[0, 1::5, :, ::3] = -0.01
    inp["g"] = g.contiguous()
    got, _, _ = gpu_bwd(inp)
    for n in GRADS:
        assert bool(torch.isfinite(torch.as_tensor(got[n])).all()), n
    compare(got, oracle_bwd(inp), TOL[dtype])


def test_bwd_per_channel_gate_equal_channels_is_scalar():
    """A per-channel gate whose channels are all equal is the scalar gate: its
    dg summed over the channels equals the scalar backward's dg, and the other
    gradients agree, within the bf16 tolerance."""
    w, inp = mk(B=2, T=130, H=2, HV=2, K=64, V=64, C=32, slow=True, seed=12)
    got_s, _, _ = gpu_bwd(inp)
    pinp = dict(inp, g=inp["g"][..., None].expand(*inp["g"].shape, 64).contiguous())
    got_p, _, _ = gpu_bwd(pinp)
    for n in ("dq", "dk", "dv", "dbeta", "dh0"):
        check(n, got_p[n], got_s[n], TOL["bf16"])
    check("dg (channel sum)", got_p["dg"].sum(-1), got_s["dg"], TOL["bf16"])


@pytest.mark.timeout(300)
def test_config_kda_shaped_backward():
    """The KDA workload's shape (H = HV = 32, K = 128, V = 256, chunk 32, per-
    channel gate, host-normalised q / k, no h0) with 2 x 1024 tokens, do and
    dht ~ N(0, 1), against the chunk-wise oracle on two sampled heads."""
    base = workloads.CONFIGS["kda_bf16"]
    w = workloads.small(base, T=1024, backward=True)
    inp = workloads.make_inputs(w)
    res = gdr.chunk_bwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
                        dev(inp["do"]), dev(inp["dht"]), scale=inp["scale"], chunk_size=w.chunk_size,
                        initial_state=None, use_qk_l2norm_in_kernel=False)
    torch.cuda.synchronize()
    for n, t in zip(GRADS, res):
        assert bool(torch.isfinite(t).all()), n
    heads = [3, 30]
    got = {n: f64(t[:, :, heads] if n != "dh0" else t[:, heads]) for n, t in zip(GRADS, res)}
    sub = slice_inputs(inp, heads=heads)
    ref = chunked.chunked_bwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], sub["do"], sub["dht"],
                              scale=inp["scale"], h0=None, use_qk_l2norm=False, chunk_size=w.chunk_size)
    compare(got, ref, TOL[w.dtype])
