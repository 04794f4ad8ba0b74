"""GPU parity of the forward path (K0..K4) against the float64 oracle.

Tolerances: err_ratio = RMS(diff) / RMS(ref) <= 1e-4 for float32 and <= 5e-3
for bf16 on o, ht and the intermediates (the bf16 bound is the chunked-vs-
per-token noise level the KCP page's acceptance section names); integer chunk
tables are compared exactly.
"""
import ctypes

import numpy as np
import pytest
import torch

import chunked_gated_delta_06_amd as gdr
import workloads
from oracle import chunked, recurrent
from oracle.metrics import err_ratio
from fwd_helpers import TOL, check, dev, f64, gpu_fwd, oracle_fwd, slice_inputs

pytestmark = pytest.mark.gpu

W = workloads.Workload


def mk(name="t", B=2, T=200, H=2, HV=4, K=64, V=64, C=64, dtype="bf16", pc=False, l2=True, h0=True,
       slow=False, lengths=None, scale=1.0, seed=7, host_l2=False):
    w = W(name, B=B, T=T, H=H, HV=HV, K=K, V=V, chunk_size=C, dtype=dtype, per_channel_gate=pc,
          l2norm_in_kernel=l2, host_l2norm=host_l2, h0=h0, slow_decay=slow, scale=scale)
    return w, workloads.make_inputs(w, seed=seed, lengths=lengths)


# ------------------------------------------------------------------ K0

@pytest.mark.parametrize("case", ["dense", "page_example", "empty_seqs", "many_seqs", "config3"])
@pytest.mark.parametrize("C", [32, 64])
def test_chunk_table_bit_exact(case, C):
    rng = np.random.default_rng(0)
    if case == "dense":
        B, T, cu = 3, 100, None
    else:
        if case == "page_example":
            lengths = [400, 624]
        elif case == "empty_seqs":
            lengths = [0, 5, 0, 70, 64, 1, 0]
        elif case == "many_seqs":
            lengths = list(rng.integers(0, 200, size=3000))
        else:
            g = torch.Generator().manual_seed(workloads.SEED)
            lengths = workloads.draw_lengths(g, 24, 64, 2048)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        B, T = 1, int(cu[-1])
    N = B if cu is None else len(cu) - 1
    p = gdr.GdrProblem(B=B, T=T, H=1, HV=1, K=32, V=32, N=N, chunk_size=C, gate_per_channel=0,
                       use_qk_l2norm=0, dtype=0, scale=1.0)
    nt = gdr.fwd_layout(p).nt_max
    idx = torch.full((nt + 1, 4), -7, dtype=torch.int32, device="cuda")    # one canary row
    off = torch.full((N + 1,), -7, dtype=torch.int32, device="cuda")
    gdr.chunk_table(p, dev(torch.from_numpy(cu)) if cu is not None else None, idx, off)
    torch.cuda.synchronize()
    ref_idx, ref_off = chunked.chunk_table(B, T, cu, C)
    off_h = off.cpu().numpy()
    idx_h = idx.cpu().numpy()
    assert np.array_equal(off_h, ref_off)
    NT = int(ref_off[-1])
    assert np.array_equal(idx_h[:NT, :3], ref_idx)
    # chunk number inside the sequence
    assert np.array_equal(idx_h[:NT, 3], np.concatenate([np.arange(ref_off[n + 1] - ref_off[n])
                                                         for n in range(N)]).astype(np.int32)
                          if NT else np.zeros(0, np.int32))
    assert (idx_h[nt] == -7).all()
    assert nt >= NT


# ------------------------------------------------------------------ stages

STAGE_CASES = [
    dict(dtype="fp32", K=32, V=32, C=64),
    dict(dtype="fp32", K=64, V=128, C=32, pc=True),
    dict(dtype="bf16", K=128, V=128, C=64),
    dict(dtype="bf16", K=128, V=256, C=32, pc=True, l2=False, host_l2=True),
    dict(dtype="bf16", K=64, V=32, C=64, H=1, HV=4),
]


@pytest.mark.parametrize("cfg", STAGE_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_stage_intermediates(cfg):
    """K1 (Tm), K2 (w, u), K3 (h, v_new, ht) and K4 (o) each against the
    oracle's per-chunk quantities, on a ragged dense batch with slow decay."""
    w, inp = mk(T=150, slow=True, **cfg)
    tol = TOL[w.dtype]
    o, ht, ws = gpu_fwd(inp, keep_states=True)
    ro, rht, it = oracle_fwd(inp, intermediates=True)
    NT = int(it["off"][-1])
    assert np.array_equal(ws["chunk_idx"][:NT, :3].cpu().numpy(), it["idx"])
    check("Tm", f64(ws["Tm"][:NT]), it["T"], tol)
    check("w", f64(ws["w"][:NT]), it["W"], tol)
    check("u", f64(ws["u"][:NT]).transpose(0, 1, 3, 2), it["U"], tol)
    check("h", f64(ws["h"][:NT]).transpose(0, 1, 3, 2), it["h"], tol)
    check("v_new", f64(ws["v_new"][:NT]).transpose(0, 1, 3, 2), it["E"], tol)
    check("o", f64(o), ro, tol)
    check("ht", f64(ht), rht, tol)


# ------------------------------------------------------------------ per-channel fused scan + output

PC_FUSED_CASES = [
    # the per-channel workload's head dims (K = 128, V = 256), host-normalised q / k
    dict(K=128, V=256, pc=True, l2=False, host_l2=True),
    # in-kernel L2 norm, GVA
    dict(K=64, V=64, pc=True, H=1, HV=4),
    dict(K=32, V=128, pc=True),
]


@pytest.mark.parametrize("cfg", PC_FUSED_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_per_channel_fused_forward_intermediates(cfg):
    """Per-channel gate, bf16, chunk 32: the default forward runs the fused
    K1 + K2 (w, u, the scan's kt / dl, aqk and the gated queries qgs) and
    the per-channel fused scan + output.  Each of those regions against the
    oracle's per-chunk operands, Tm / h / v_new absent, o / ht against the
    oracle, on a ragged dense batch with slow decay and h0."""
    w, inp = mk(T=150, C=32, slow=True, scale=0.75, **cfg)
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=32, use_qk_l2norm=inp["use_qk_l2norm"])
    assert gdr.chunk_fwd_fused(p) == 2
    o, ht, ws = gpu_fwd(inp)
    ro, rht, it = oracle_fwd(inp, intermediates=True)
    NT = int(it["off"][-1])
    assert ws["Tm"] is None and ws["h"] is None and ws["v_new"] is None
    # aqk carries ~16 mantissa bits (hi + lo operands); the gated queries are
    # one bf16 rounding (or a hi + lo pair)
    check("aqk", f64(ws["aqk"][:NT]), it["QK"], 1e-4)
    qg_tol = 1e-4 if ws["qgs"].shape[2] == 2 else 2e-3
    check("qgs", f64(ws["qgs"][:NT]).sum(2), it["QG"], qg_tol)
    check("kt", f64(ws["kt"][:NT]), it["KT"], TOL["bf16"])
    check("dl", f64(ws["dl"][:NT]), it["DL"], 1e-5)
    check("w", f64(ws["w"][:NT]), it["W"], TOL["bf16"])
    assert ws["u"] is None      # u in the input dtype
    check("u", f64(ws["u_fused"][:NT]).transpose(0, 1, 3, 2), it["U"], TOL["bf16"])
    check("o", f64(o), ro, TOL["bf16"])
    check("ht", f64(ht), rht, TOL["bf16"])
    # the separate stages on the same inputs agree with it within the tolerance
    o2, ht2, _ = gpu_fwd(inp, keep_states=True)
    check("o (separate stages)", f64(o2), f64(o), TOL["bf16"])
    check("ht (separate stages)", f64(ht2), f64(ht), TOL["bf16"])


@pytest.mark.parametrize("keep", [False, True])
def test_per_channel_fused_forward_varlen_gva(keep):
    """The per-channel fused forward (and its kept-states form) on a varlen
    GVA batch at chunk 32: empty, one-token, chunk-aligned and ragged
    sequences, 2 value heads per q/k head, in-kernel L2 norm, h0; o and ht
    against the oracle, every sequence on its own."""
    lengths = [0, 1, 31, 32, 33, 100, 0, 7, 130]
    w, inp = mk(B=1, H=2, HV=4, K=128, V=128, C=32, pc=True, lengths=lengths, slow=True, scale=0.5)
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=32, cu_seqlens=inp["cu_seqlens"],
                         use_qk_l2norm=True, keep_states=keep)
    assert gdr.chunk_fwd_fused(p) == (0 if keep else 2)
    o, ht, ws = gpu_fwd(inp, keep_states=keep)
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, TOL["bf16"])
    check("ht", f64(ht), rht, TOL["bf16"])
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(lengths)):
        if lengths[n]:
            check(f"o[seq {n}]", f64(o)[:, cu[n]:cu[n + 1]], ro[:, cu[n]:cu[n + 1]], TOL["bf16"])
    if keep:
        assert ws["h"] is not None and ws["Tm"] is not None


def test_per_channel_fused_forward_extreme_gate_span():
    """Per-channel gates of -9 (about 144 of decay inside a 16-token block,
    above K1's exponential-safety limit, so its diagonal blocks take the
    per-element path for aqk as for A) with a few near-zero gates, on the
    per-channel fused forward (bf16, chunk 32, ragged tail)."""
    w, inp = mk(B=1, T=90, H=1, HV=2, K=64, V=64, C=32, pc=True)
    inp["g"] = inp["g"] * 0.0 - 9.0
    inp["g"][0, 1::3] = -0.01
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=32, use_qk_l2norm=True)
    assert gdr.chunk_fwd_fused(p) == 2
    o, ht, ws = gpu_fwd(inp)
    ro, rht, it = oracle_fwd(inp, intermediates=True)
    NT = int(it["off"][-1])
    check("aqk", f64(ws["aqk"][:NT]), it["QK"], 1e-4)
    check("o", f64(o), ro, TOL["bf16"])
    check("ht", f64(ht), rht, TOL["bf16"])


# ------------------------------------------------------------------ fused scan + output

FUSED_CASES = [
    # few value tiles: one compute wave (16 value columns) per workgroup
    dict(dtype="bf16", K=128, V=128, C=64),
    dict(dtype="bf16", K=64, V=256, C=32, H=1, HV=4),
    dict(dtype="fp32", K=64, V=64, C=64),
    dict(dtype="bf16", K=32, V=64, C=64, l2=False, host_l2=True),
    # >= 256 tiles of 32 value columns: two compute waves per workgroup (the
    # variant the full forward picks)
    dict(dtype="bf16", K=128, V=128, C=64, H=8, HV=32),
    dict(dtype="bf16", K=64, V=256, C=32, B=1, H=4, HV=32),
    dict(dtype="fp32", K=64, V=64, C=64, H=16, HV=64),
]


@pytest.mark.parametrize("cfg", FUSED_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_fused_stage_against_separate_stages(cfg):
    """gdr_fwd_h_o on the w, u and token factors of the fused K1 + K2 stage,
    beside the separate stages of a keep-states forward (whose scan reads the
    fp32 u of the separate WY stage and takes e as a hi + lo pair): both
    match the oracle, and each other within the tolerance."""
    w, inp = mk(T=150, slow=True, **cfg)
    tol = TOL[w.dtype]
    o_sep, ht_sep, ws = gpu_fwd(inp, keep_states=True)
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=inp["chunk_size"],
                         use_qk_l2norm=inp["use_qk_l2norm"], scale=inp["scale"])
    assert gdr.fwd_h_o_supported(p)
    o_f = torch.full_like(o_sep, float("nan"))
    ht_f = torch.full_like(ht_sep, float("nan"))
    gdr.fwd_kkt_wy(p, dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]), ws["chunk_idx"],
                   ws["chunk_off"], ws["w"], ws["u_fused"], ws["kscale"])
    gdr.fwd_h_o(p, dev(inp["q"]), dev(inp["k"]), ws["w"], ws["u_fused"], dev(inp["g"]), ws["kscale"],
                ws["chunk_idx"], ws["chunk_off"], dev(inp["h0"]), o_f, ht_f)
    torch.cuda.synchronize()
    ro, rht = oracle_fwd(inp)
    check("o fused", f64(o_f), ro, tol)
    check("o separate", f64(o_sep), ro, tol)
    check("ht fused", f64(ht_f), rht, tol)
    check("ht separate", f64(ht_sep), rht, tol)
    assert err_ratio(f64(o_f), f64(o_sep)) <= tol


KKT_WY_CASES = [
    dict(dtype="bf16", K=128, V=128, C=64),
    dict(dtype="bf16", K=256, V=64, C=64, H=1, HV=2),
    dict(dtype="bf16", K=64, V=256, C=32, H=1, HV=4),
    dict(dtype="bf16", K=32, V=32, C=32, l2=False, host_l2=True),
    dict(dtype="fp32", K=32, V=64, C=64),
    dict(dtype="fp32", K=128, V=128, C=32),
    dict(dtype="fp32", K=256, V=32, C=64, H=1, HV=1),
]


@pytest.mark.parametrize("cfg", KKT_WY_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_fused_kkt_wy_against_oracle(cfg):
    """gdr_fwd_kkt_wy (K1 + K2 in one kernel, Tm kept on chip) on a ragged
    dense GVA batch: w, u against the oracle's per-chunk W and U, the token
    factors against the separate K1's, and it leaves Tm's region alone."""
    w, inp = mk(T=150, slow=True, **cfg)
    tol = TOL[w.dtype]
    o_sep, ht_sep, ws = gpu_fwd(inp, keep_states=True)
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=inp["chunk_size"],
                         use_qk_l2norm=inp["use_qk_l2norm"], scale=inp["scale"])
    ro, rht, it = oracle_fwd(inp, intermediates=True)
    NT = int(it["off"][-1])
    wf = torch.full_like(ws["w"], float("nan"))
    uf = torch.full_like(ws["u_fused"], float("nan"))
    kf = torch.full_like(ws["kscale"], float("nan"))
    tm_before = ws["Tm"].clone()
    gdr.fwd_kkt_wy(p, dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]), ws["chunk_idx"],
                   ws["chunk_off"], wf, uf, kf)
    torch.cuda.synchronize()
    assert torch.equal(ws["Tm"], tm_before)
    check("w", f64(wf[:NT]), it["W"], tol)
    check("u", f64(uf[:NT]).transpose(0, 1, 3, 2), it["U"], tol)
    assert err_ratio(f64(wf[:NT]), f64(ws["w"][:NT])) <= tol
    assert not torch.isnan(kf[:NT]).any()
    np.testing.assert_allclose(f64(kf[:NT]), f64(ws["kscale"][:NT]), rtol=1e-5, atol=1e-6)
    # the fused stages end to end (the default forward) against the oracle
    o, ht, _ = gpu_fwd(inp)
    check("o", f64(o), ro, tol)
    check("ht", f64(ht), rht, tol)


def test_fused_default_uses_the_compact_workspace():
    """Without keep_states the forward takes the fused stages in the compact
    workspace layout (no Tm, h or v_new regions): o / ht match the oracle, and a
    workspace of exactly that size, inside guard bands, is enough and is not
    overrun; with keep_states the full layout is required."""
    w, inp = mk(B=2, T=170, H=8, HV=32, K=128, V=128, slow=True)
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=64, use_qk_l2norm=True)
    assert gdr.chunk_fwd_fused(p)
    lay = gdr.fwd_layout(p)
    full = gdr.fwd_layout(gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=64, use_qk_l2norm=True,
                                           keep_states=True))
    assert lay.Tm == lay.w and lay.h == lay.kscale and lay.total < full.total
    pad = 4096
    ws_full = torch.full((lay.total + 2 * pad,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = ws_full[pad:pad + lay.total]
    o, ht, views = gpu_fwd(inp, workspace=ws)
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, TOL["bf16"])
    check("ht", f64(ht), rht, TOL["bf16"])
    assert views["Tm"] is None and views["h"] is None and views["v_new"] is None
    assert (ws_full[:pad] == 0x5A).all() and (ws_full[pad + lay.total:] == 0x5A).all()
    # the C ABI refuses that workspace for the separate stages
    pk = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=64, use_qk_l2norm=True, keep_states=True)
    P = lambda t: ctypes.c_void_p(dev(t).data_ptr())
    st = gdr.lib().gdr_chunk_fwd(ctypes.byref(pk), P(inp["q"]), P(inp["k"]), P(inp["v"]), P(inp["g"]),
                                 P(inp["beta"]), None, None, ctypes.c_void_p(o.data_ptr()), None,
                                 ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(lay.total), None)
    assert st == 7   # GDR_ERR_WORKSPACE


# ------------------------------------------------------------------ sweep

SWEEP = []
for dtype in ("bf16", "fp32"):
    for C in (32, 64):
        for (K, V) in ((32, 64), (64, 64), (128, 128), (256, 64), (64, 256)):
            for pc in (False, True):
                if dtype == "fp32" and pc and K == 256 and C == 64:
                    continue
                SWEEP.append(dict(dtype=dtype, C=C, K=K, V=V, pc=pc))
                if not pc or (dtype == "bf16" and C == 32 and K <= 128):
                    # the separate scan and output stages too (the default is the
                    # fused stage wherever the shape has one)
                    SWEEP.append(dict(dtype=dtype, C=C, K=K, V=V, pc=pc, keep=True))


@pytest.mark.parametrize("cfg", SWEEP, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_forward_sweep(cfg):
    """Dense GVA batch with a ragged tail, in-kernel L2 norm, h0, slow decay."""
    cfg = dict(cfg)
    keep = cfg.pop("keep", False)
    w, inp = mk(B=2, T=137, H=2, HV=4, slow=True, scale=0.75, **cfg)
    o, ht, _ = gpu_fwd(inp, keep_states=keep)
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, TOL[w.dtype])
    check("ht", f64(ht), rht, TOL[w.dtype])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("pc", [False, True])
@pytest.mark.parametrize("l2", [False, True])
def test_forward_varlen(dtype, pc, l2):
    lengths = [1, 63, 64, 65, 0, 130, 7, 200]
    w, inp = mk(B=1, H=2, HV=4, K=64, V=128, dtype=dtype, pc=pc, l2=l2, lengths=lengths, slow=True,
                host_l2=not l2)
    o, ht, _ = gpu_fwd(inp)
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, TOL[dtype])
    check("ht", f64(ht), rht, TOL[dtype])
    # worst single sequence
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(lengths)):
        if lengths[n]:
            check(f"o[seq {n}]", f64(o)[:, cu[n]:cu[n + 1]], ro[:, cu[n]:cu[n + 1]], TOL[dtype])


def test_forward_matches_per_token_recurrence():
    """The GPU against the plain per-token oracle directly (not the chunked one)."""
    w, inp = mk(B=1, T=100, H=1, HV=2, K=64, V=64, dtype="fp32", slow=True)
    o, ht, _ = gpu_fwd(inp)
    ro, rht = recurrent.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], h0=inp["h0"],
                                      use_qk_l2norm=True)
    check("o", f64(o), ro, 1e-4)
    check("ht", f64(ht), rht, 1e-4)


# ------------------------------------------------------------------ edge cases

def test_empty_batch_and_no_state():
    w, inp = mk(B=2, T=0)
    o, ht, _ = gpu_fwd(inp)
    assert o.numel() == 0
    assert torch.equal(ht.cpu(), inp["h0"])


def test_single_token_sequences():
    w, inp = mk(B=1, lengths=[1, 1, 1, 2], dtype="fp32", K=32, V=32)
    o, ht, _ = gpu_fwd(inp)
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, 1e-4)
    check("ht", f64(ht), rht, 1e-4)


@pytest.mark.parametrize("scale", [1.0, 128 ** -0.5])
def test_largest_head_dims(scale):
    w, inp = mk(B=1, T=96, H=1, HV=2, K=256, V=256, scale=scale, slow=True)
    o, ht, _ = gpu_fwd(inp)
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, 5e-3)
    check("ht", f64(ht), rht, 5e-3)


def test_extreme_per_channel_gate_span():
    """Gate spans above the exponential-safety limit take the per-element path
    (diagonal blocks) and must still match."""
    w, inp = mk(B=1, T=64, H=1, HV=1, K=64, V=64, C=64, pc=True, dtype="fp32")
    inp["g"] = inp["g"] * 0.0 - 9.0          # ~144 of decay inside each 16-row block
    inp["g"][0, 1::3] = -0.01
    o, ht, _ = gpu_fwd(inp)
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, 1e-4)
    check("ht", f64(ht), rht, 1e-4)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_extreme_scalar_gate_span_fused_output(dtype):
    """Scalar gates of -9 per token (about 144 of decay inside a 16-token
    block, so every decay factor between blocks underflows), with a few
    near-zero gates, a ragged last chunk and the fused scan + output stage:
    the output's factored decays (row factor times column factor) must still
    match the plain exp(G_r - G_t)."""
    w, inp = mk(B=1, T=150, H=2, HV=2, K=128 if dtype == "bf16" else 64, V=64, C=64, dtype=dtype)
    inp["g"] = inp["g"] * 0.0 - 9.0
    inp["g"][0, 1::5] = -0.01
    o, ht, _ = gpu_fwd(inp)
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, TOL[dtype])
    check("ht", f64(ht), rht, TOL[dtype])


# ------------------------------------------------------------------ invariants (bitwise)

def test_varlen_equals_dense_per_sequence_bitwise():
    lengths = [130, 64, 1, 200]
    w, inp = mk(B=1, H=2, HV=4, K=128, V=128, lengths=lengths, slow=True)
    o, ht, _ = gpu_fwd(inp)
    cu = inp["cu_seqlens"].tolist()
    for n, L in enumerate(lengths):
        s, e = cu[n], cu[n + 1]
        sub = dict(inp, cu_seqlens=None, B=1, N=1, T=L)
        for key in ("q", "k", "v", "g", "beta"):
            sub[key] = inp[key][:, s:e].contiguous()
        sub["h0"] = inp["h0"][n:n + 1].contiguous()
        on, hn, _ = gpu_fwd(sub)
        assert torch.equal(o[:, s:e].cpu(), on.cpu()), f"o differs for sequence {n}"
        assert torch.equal(ht[n:n + 1].cpu(), hn.cpu()), f"ht differs for sequence {n}"


@pytest.mark.parametrize("split", [64, 192])
def test_split_handoff_bitwise(split):
    """Running [0, split) then [split, T) with ht -> h0 equals one pass, bit for
    bit, when the split sits on a chunk boundary (KCP page, step 4 of its
    playbook: a uniform single sequence must be bit-perfect)."""
    w, inp = mk(B=1, T=320, H=2, HV=2, K=128, V=128, slow=True)
    o, ht, _ = gpu_fwd(inp)
    a = dict(inp, T=split)
    b = dict(inp, T=320 - split)
    for key in ("q", "k", "v", "g", "beta"):
        a[key] = inp[key][:, :split].contiguous()
        b[key] = inp[key][:, split:].contiguous()
    oa, hta, _ = gpu_fwd(a)
    b["h0"] = hta.cpu()
    ob, htb, _ = gpu_fwd(b)
    assert torch.equal(torch.cat([oa, ob], 1).cpu(), o.cpu())
    assert torch.equal(htb.cpu(), ht.cpu())


def test_split_handoff_unaligned_within_tolerance():
    w, inp = mk(B=1, T=300, H=1, HV=2, K=64, V=64, slow=True)
    split = 111
    ro, rht = oracle_fwd(inp)
    a = dict(inp, T=split)
    b = dict(inp, T=300 - split)
    for key in ("q", "k", "v", "g", "beta"):
        a[key] = inp[key][:, :split].contiguous()
        b[key] = inp[key][:, split:].contiguous()
    oa, hta, _ = gpu_fwd(a)
    b["h0"] = hta.cpu()
    ob, htb, _ = gpu_fwd(b)
    check("o", f64(torch.cat([oa, ob], 1)), ro, 5e-3)
    check("ht", f64(htb), rht, 5e-3)


def test_gva_equals_repeated_heads_bitwise():
    w, inp = mk(B=2, T=150, H=2, HV=6, K=64, V=64)
    o, ht, _ = gpu_fwd(inp)
    rep = dict(inp, q=inp["q"].repeat_interleave(3, 2), k=inp["k"].repeat_interleave(3, 2))
    o2, ht2, _ = gpu_fwd(rep)
    assert torch.equal(o.cpu(), o2.cpu()) and torch.equal(ht.cpu(), ht2.cpu())


def test_h0_none_equals_zeros_bitwise():
    w, inp = mk(B=2, T=100)
    o1, ht1, _ = gpu_fwd(inp, h0=False)
    z = dict(inp, h0=torch.zeros_like(inp["h0"]))
    o2, ht2, _ = gpu_fwd(z)
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(ht1.cpu(), ht2.cpu())


def test_deterministic_and_nan_poison_and_canaries():
    """Run-to-run bitwise determinism; NaN-filled outputs and workspace on entry
    (the poisoning idea of the coverage-matrix page, section 7) leave no trace;
    guard bands around o, ht and the workspace are untouched."""
    w, inp = mk(B=2, T=170, H=2, HV=4, K=128, V=128, slow=True)
    o1, ht1, _ = gpu_fwd(inp)
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=64, use_qk_l2norm=True)
    lay = gdr.fwd_layout(p)
    pad = 4096
    ws_full = torch.full((lay.total + 2 * pad,), 0xFF, dtype=torch.uint8, device="cuda")
    ws = ws_full[pad:pad + lay.total]
    on = o1.numel()
    o_full = torch.full((on + 2 * pad,), float("nan"), dtype=o1.dtype, device="cuda")
    ht_full = torch.full((ht1.numel() + 2 * pad,), float("nan"), dtype=torch.float32, device="cuda")
    o = o_full[pad:pad + on].view(o1.shape)
    ht = ht_full[pad:pad + ht1.numel()].view(ht1.shape)
    o2, ht2, _ = gpu_fwd(inp, workspace=ws, out=(o, ht))
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(ht1.cpu(), ht2.cpu())
    assert not torch.isnan(o2).any() and not torch.isnan(ht2).any()
    assert torch.isnan(o_full[:pad]).all() and torch.isnan(o_full[pad + on:]).all()
    assert torch.isnan(ht_full[:pad]).all() and torch.isnan(ht_full[pad + ht1.numel():]).all()
    assert (ws_full[:pad] == 0xFF).all() and (ws_full[pad + lay.total:] == 0xFF).all()


@pytest.mark.parametrize("pc", [False, True], ids=["scalar", "per_channel"])
def test_int64_offsets(pc):
    """A varlen batch whose last sequence sits past 2^31 elements of q / k / v
    and of the per-chunk state tensor (per-channel gate: of g too, at chunk
    32); only that sequence is checked."""
    H = HV = 16
    K = V = 128
    tail = 192
    T_big = (1 << 20) + 64 + tail       # the checked sequence starts past 2^31 elements
    lengths = [T_big - tail, tail]
    gen = torch.Generator().manual_seed(3)
    T = T_big
    q = torch.zeros(1, T, H, K, dtype=torch.bfloat16)
    k = torch.zeros(1, T, H, K, dtype=torch.bfloat16)
    v = torch.zeros(1, T, HV, V, dtype=torch.bfloat16)
    gw = (HV, K) if pc else (HV,)
    g = torch.zeros(1, T, *gw)
    beta = torch.zeros(1, T, HV)
    s = T - tail
    q[:, s:] = torch.randn(1, tail, H, K, generator=gen).bfloat16()
    k[:, s:] = torch.randn(1, tail, H, K, generator=gen).bfloat16()
    v[:, s:] = torch.randn(1, tail, HV, V, generator=gen).bfloat16()
    g[:, s:] = torch.nn.functional.logsigmoid(torch.randn(1, tail, *gw, generator=gen) + 4)
    beta[:, s:] = torch.sigmoid(torch.randn(1, tail, HV, generator=gen))
    h0 = 0.1 * torch.randn(2, HV, K, V, generator=gen)
    assert s * H * K > 2 ** 31
    cu = torch.tensor([0, lengths[0], T], dtype=torch.int32)
    inp = dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, cu_seqlens=cu, scale=1.0, chunk_size=32 if pc else 64,
               use_qk_l2norm=True)
    sub = dict(inp, cu_seqlens=None, h0=h0[1:2])
    for key in ("q", "k", "v", "g", "beta"):
        sub[key] = inp[key][:, s:].contiguous()
    ro, rht = oracle_fwd(sub)
    for keep in (True, False):     # separate stages (h offsets past 2^31), then fused
        o, ht, ws = gpu_fwd(inp, keep_states=keep)
        check(f"o tail keep={keep}", f64(o[:, s:]), ro, 5e-3)
        check(f"ht tail keep={keep}", f64(ht[1:2]), rht, 5e-3)
        del o, ht, ws
        torch.cuda.empty_cache()


# ------------------------------------------------------------------ the five workloads

def _run_config(name, rows=None, heads=None):
    w = workloads.CONFIGS[name]
    inp = workloads.make_inputs(w)
    o, ht, _ = gpu_fwd(inp)
    sub = slice_inputs(inp, rows=rows, heads=heads)
    ro, rht = oracle_fwd(sub)
    og, htg = o, ht
    if rows is not None:
        og, htg = og[rows], htg[rows]
    if heads is not None:
        og, htg = og[:, :, heads], htg[:, heads]
    tol = TOL[w.dtype]
    r1 = check("o", f64(og), ro, tol)
    r2 = check("ht", f64(htg), rht, tol)
    print(f"{name}: err_ratio o={r1:.2e} ht={r2:.2e}")
    return inp, o, ht


def test_config_tiny_fp32():
    inp, o, ht = _run_config("tiny_fp32")
    ro, rht = recurrent.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], h0=inp["h0"])
    check("o (per-token)", f64(o), ro, 1e-4)


def test_config_gdn_dense_bf16():
    _run_config("gdn_dense_bf16")


def test_config_varlen_gva_bf16():
    inp, o, ht = _run_config("varlen_gva_bf16")
    assert any(L % 64 for L in np.diff(inp["cu_seqlens"].numpy()))


def test_config_kda_bf16():
    _run_config("kda_bf16", rows=slice(1, 2))


def test_config_kda_bf16_first_row():
    """The per-channel workload's other row (the two tests together check
    every output of the full-size forward)."""
    _run_config("kda_bf16", rows=slice(0, 1))


def test_config_long_bf16_forward():
    _run_config("long_bf16", heads=[0, 21])


# ------------------------------------------------------------------ head dims without an instantiation

PAD_CASES = [
    dict(B=2, T=512, H=2, HV=4, K=60, V=60, C=64),                        # the page's GVA shape with D = 60
    dict(B=1, T=150, H=2, HV=2, K=60, V=100, C=32, pc=True, l2=False, host_l2=True),
    dict(B=2, T=90, H=1, HV=2, K=60, V=36, C=64, dtype="fp32"),
    dict(B=1, T=70, H=2, HV=2, K=200, V=24, C=32),
]


@pytest.mark.parametrize("cfg", PAD_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_forward_padded_head_dims(cfg):
    """Non-power-of-two head dims run zero-padded to the next instantiated size;
    inputs sit between NaN guard bands (and a per-channel gate between 1e30
    bands, the page's right-padding trick) so a read past a tensor shows."""
    w, inp = mk(slow=True, scale=0.75, **cfg)
    pad = 4096

    def guarded(t, fill):
        flat = torch.full((t.numel() + 2 * pad,), fill, dtype=t.dtype, device="cuda")
        flat[pad:pad + t.numel()] = t.reshape(-1).cuda()
        return flat[pad:pad + t.numel()].view(t.shape)

    q, k, v = (guarded(inp[n], float("nan")) for n in ("q", "k", "v"))
    g = guarded(inp["g"], 1e30 if w.per_channel_gate else float("nan"))
    beta, h0 = guarded(inp["beta"], float("nan")), guarded(inp["h0"], float("nan"))
    o, ht = gdr.chunk_fwd(q, k, v, g, beta, scale=inp["scale"], chunk_size=w.chunk_size, initial_state=h0,
                          use_qk_l2norm_in_kernel=inp["use_qk_l2norm"])
    torch.cuda.synchronize()
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, TOL[w.dtype])
    check("ht", f64(ht), rht, TOL[w.dtype])
    if not w.per_channel_gate:
        o2, ht2, _ = gpu_fwd(inp, keep_states=True)
        check("o separate stages", f64(o2), ro, TOL[w.dtype])


def test_varlen_scan_order():
    """A varlen forward writes the sequences by decreasing chunk count (ties by
    index) into the workspace, the order the state scans start them in; the
    results stay those of the oracle (and equal, bitwise, a forward whose
    batch lists the sequences in that order: each sequence's arithmetic does
    not depend on where its workgroups run)."""
    lengths = [64, 2048, 0, 130, 640, 1, 700, 129]
    w, inp = mk(B=1, H=2, HV=4, K=64, V=64, lengths=lengths, slow=True)
    o, ht, ws = gpu_fwd(inp)
    cnt = [(L + 63) // 64 for L in lengths]
    want = sorted(range(len(lengths)), key=lambda n: (-cnt[n], n))
    assert ws["seq_order"].cpu().tolist() == want
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, TOL["bf16"])
    check("ht", f64(ht), rht, TOL["bf16"])


def test_padded_head_dims_varlen_without_states():
    """Zero-padded head dims (K = 60, V = 40) on a varlen batch with empty and
    one-token sequences, no h0 and no ht requested."""
    w, inp = mk(B=1, H=2, HV=4, K=60, V=40, lengths=[0, 1, 65, 0, 130], slow=True, h0=False)
    o, ht = gdr.chunk_fwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
                          cu_seqlens=dev(inp["cu_seqlens"]), output_final_state=False,
                          use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    assert ht is None
    ro, _ = oracle_fwd(inp, h0=False)
    check("o", f64(o), ro, TOL["bf16"])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_per_channel_scan_four_wave_grid(dtype):
    """Per-channel gate with N * HV * V / 64 = 256: the scan runs four waves
    (64 value columns) per workgroup. GVA (8 q/k heads, 64 value heads),
    a ragged tail (T = 77, chunk 32), h0 and slow decay."""
    w, inp = mk(B=2, T=77, H=8, HV=64, K=64, V=128, C=32, dtype=dtype, pc=True, slow=True, scale=0.5)
    assert w.B * w.HV * (w.V // 64) >= 256
    o, ht, _ = gpu_fwd(inp)
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, TOL[dtype])
    check("ht", f64(ht), rht, TOL[dtype])


def test_per_channel_fused_four_wave_grid_kept_states():
    """The per-channel fused scan + output on its four-compute-wave grid
    (N * HV * V / 64 = 256, bf16, chunk 32), whose four output waves split the
    chunk's token blocks and the 64 value columns: o and ht, and with kept
    states the h and v_new tiles those output waves store, against the oracle
    on a ragged GVA batch."""
    w, inp = mk(B=2, T=77, H=8, HV=64, K=64, V=128, C=32, pc=True, slow=True, scale=0.5)
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=32, use_qk_l2norm=True)
    assert gdr.chunk_fwd_fused(p) == 2
    ro, rht, it = oracle_fwd(inp, intermediates=True)
    NT = int(it["off"][-1])
    for keep in (False, True):
        o, ht, ws = gpu_fwd(inp, keep_states=keep)
        check(f"o (keep {keep})", f64(o), ro, TOL["bf16"])
        check(f"ht (keep {keep})", f64(ht), rht, TOL["bf16"])
        if keep:
            check("h", f64(ws["h"][:NT]).transpose(0, 1, 3, 2), it["h"], TOL["bf16"])
            check("v_new", f64(ws["v_new"][:NT]).transpose(0, 1, 3, 2), it["E"], TOL["bf16"])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_per_channel_scan_four_wave_grid_k32(dtype):
    """Per-channel gate, K = 32 at chunk 32 on a four-wave grid (B = 2, HV = 32,
    V = 256: N * HV * V / 64 = 256). A 32 x 32 key tile has 128 eight-element
    pieces, fewer than the workgroup's 256 threads, so only the first two waves
    fetch and stage the w and key tiles."""
    w, inp = mk(B=2, T=77, H=32, HV=32, K=32, V=256, C=32, dtype=dtype, pc=True, slow=True, scale=0.5)
    assert w.B * w.HV * (w.V // 64) >= 256
    o, ht, _ = gpu_fwd(inp)
    ro, rht = oracle_fwd(inp)
    check("o", f64(o), ro, TOL[dtype])
    check("ht", f64(ht), rht, TOL[dtype])


def test_stage_timing_reports_the_stages_each_call_runs():
    """gdr_stage_timing / gdr_stage_times: the stages of every call since
    timing was turned on, in launch order, with positive durations; nothing
    once it is off."""
    w, inp = mk(B=2, T=200, H=2, HV=2, K=128, V=128, C=64)
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "h0")}
    kw = dict(chunk_size=64, initial_state=d["h0"], use_qk_l2norm_in_kernel=True)
    gdr.stage_timing(True)
    try:
        for _ in range(2):
            gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], **kw)
        fused = gdr.stage_times()
        gdr.stage_timing(True)
        gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], keep_states=True, **kw)
        sep = gdr.stage_times()
    finally:
        gdr.stage_timing(False)
    assert [n for n, _ in fused] == ["kkt_wy", "fwd_h_o"] * 2
    assert [n for n, _ in sep] == ["chunk_table", "kkt_wy", "fwd_h_o"]
    assert all(ms > 0 for _, ms in fused + sep)
    gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], **kw)
    assert gdr.stage_times() == []
