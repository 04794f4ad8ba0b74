"""GPU parity of the token-by-token forward (gdr_fused_recurrent_fwd) against
the float64 per-token oracle.

The same tolerances as the chunked forward: err_ratio = RMS(diff) / RMS(ref)
<= 1e-4 for float32 and <= 5e-3 for bf16 on o and ht.  State hand-off across
calls (decoding one token at a time) is compared bitwise with one call over
the whole sequence: both keep the state in fp32 and the hand-off stores it
exactly.
"""
import numpy as np
import pytest
import torch

import chunked_gated_delta_06_amd as gdr
import workloads
from oracle import recurrent
from fwd_helpers import TOL, check, dev, f64, gpu_fwd

pytestmark = pytest.mark.gpu

W = workloads.Workload


def mk(B=2, T=137, H=2, HV=4, K=64, V=64, dtype="bf16", pc=False, l2=True, h0=True, slow=True,
       lengths=None, scale=0.75, seed=11):
    w = W("rec", B=B, T=T, H=H, HV=HV, K=K, V=V, chunk_size=64, dtype=dtype, per_channel_gate=pc,
          l2norm_in_kernel=l2, host_l2norm=not l2, h0=h0, slow_decay=slow, scale=scale)
    return w, workloads.make_inputs(w, seed=seed, lengths=lengths)


def gpu_rec(inp, h0=True, ht=True):
    o, htd = gdr.fused_recurrent_fwd(
        dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
        scale=inp["scale"], cu_seqlens=dev(inp["cu_seqlens"]),
        initial_state=dev(inp["h0"]) if h0 and inp["h0"] is not None else None,
        output_final_state=ht, use_qk_l2norm_in_kernel=inp["use_qk_l2norm"])
    torch.cuda.synchronize()
    return o, htd


def oracle(inp, h0=True):
    return recurrent.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                   scale=inp["scale"], h0=inp["h0"] if h0 else None,
                                   cu_seqlens=inp["cu_seqlens"], use_qk_l2norm=inp["use_qk_l2norm"])


SWEEP = [dict(dtype=dt, K=K, V=V, pc=pc)
         for dt in ("bf16", "fp32")
         for (K, V) in ((32, 64), (64, 64), (128, 128), (256, 64), (64, 256))
         for pc in (False, True)]


@pytest.mark.parametrize("cfg", SWEEP, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_recurrent_sweep(cfg):
    """Dense GVA batch, 137 tokens (a ragged 16-token block), in-kernel L2 norm,
    h0, slow decay so the state carries across the whole sequence."""
    w, inp = mk(**cfg)
    o, ht = gpu_rec(inp)
    ro, rht = oracle(inp)
    check("o", f64(o), ro, TOL[w.dtype])
    check("ht", f64(ht), rht, TOL[w.dtype])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("pc", [False, True])
@pytest.mark.parametrize("l2", [False, True])
def test_recurrent_varlen(dtype, pc, l2):
    lengths = [1, 15, 16, 17, 0, 130, 7, 0, 64]
    w, inp = mk(B=1, K=64, V=128, dtype=dtype, pc=pc, l2=l2, lengths=lengths)
    o, ht = gpu_rec(inp)
    ro, rht = oracle(inp)
    check("o", f64(o), ro, TOL[dtype])
    check("ht", f64(ht), rht, TOL[dtype])
    # empty sequences hand h0 straight through
    for n, L in enumerate(lengths):
        if L == 0:
            assert torch.equal(ht[n].cpu(), inp["h0"][n])


def test_recurrent_without_states():
    w, inp = mk(dtype="fp32", K=32, V=32)
    o, ht = gpu_rec(inp, h0=False, ht=False)
    assert ht is None
    ro, _ = oracle(inp, h0=False)
    check("o", f64(o), ro, 1e-4)
    # T = 0: nothing but the state hand-off
    w, inp = mk(T=0)
    o, ht = gpu_rec(inp)
    assert o.numel() == 0 and torch.equal(ht.cpu(), inp["h0"])


@pytest.mark.parametrize("pc", [False, True])
def test_decode_handoff_bitwise(pc):
    """Decoding token by token (each call hands its ht to the next as h0) is
    bitwise equal to one call over the whole sequence."""
    w, inp = mk(B=2, T=21, K=128, V=128, pc=pc)
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "h0")}
    o_all, ht_all = gdr.fused_recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=inp["scale"],
                                            initial_state=d["h0"], use_qk_l2norm_in_kernel=True)
    state = d["h0"]
    outs = []
    for t in range(w.T):
        sl = lambda x: x[:, t:t + 1].contiguous()
        o_t, state = gdr.fused_recurrent_fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]),
                                             scale=inp["scale"], initial_state=state,
                                             use_qk_l2norm_in_kernel=True)
        outs.append(o_t)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), o_all)
    assert torch.equal(state, ht_all)


def test_matches_chunked_path():
    """The two GPU forwards agree with each other and with the oracle on the
    dense bf16 GDN shape (one batch row, 16 heads)."""
    w, inp = mk(B=1, T=300, H=16, HV=16, K=128, V=128, scale=1.0, slow=False)
    o_r, ht_r = gpu_rec(inp)
    o_c, ht_c, _ = gpu_fwd(dict(inp, chunk_size=64))
    ro, rht = oracle(inp)
    check("o (recurrent)", f64(o_r), ro, 5e-3)
    check("o (chunked)", f64(o_c), ro, 5e-3)
    check("ht (recurrent)", f64(ht_r), rht, 5e-3)
    check("o recurrent vs chunked", f64(o_r), f64(o_c), 5e-3)


def test_decode_step_many_sequences():
    """One decoding step: 512 sequences of one token each (varlen), GVA 16 / 32
    heads, K = V = 128, bf16, each starting from its own state."""
    lengths = [1] * 512
    w, inp = mk(B=1, H=16, HV=32, K=128, V=128, lengths=lengths, scale=128 ** -0.5)
    o, ht = gpu_rec(inp)
    seqs = [0, 1, 255, 511]
    ro, rht = recurrent.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                      scale=inp["scale"], h0=inp["h0"], cu_seqlens=inp["cu_seqlens"],
                                      use_qk_l2norm=True, seqs=seqs)
    cu = inp["cu_seqlens"].tolist()
    idx = [cu[n] for n in seqs]
    check("o", f64(o)[:, idx], ro[:, idx], 5e-3)
    check("ht", f64(ht)[seqs], rht[seqs], 5e-3)


def test_recurrent_nan_poison_canaries_deterministic():
    """NaN-filled outputs on entry leave no trace, guard bands around o and ht
    stay untouched, and two runs agree bitwise."""
    w, inp = mk(B=3, T=45, K=128, V=128)
    o1, ht1 = gpu_rec(inp)
    pad = 4096
    on, hn = o1.numel(), ht1.numel()
    o_full = torch.full((on + 2 * pad,), float("nan"), dtype=o1.dtype, device="cuda")
    ht_full = torch.full((hn + 2 * pad,), float("nan"), dtype=torch.float32, device="cuda")
    o = o_full[pad:pad + on].view(o1.shape)
    ht = ht_full[pad:pad + hn].view(ht1.shape)
    gdr.fused_recurrent_fwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
                            scale=inp["scale"], initial_state=dev(inp["h0"]), use_qk_l2norm_in_kernel=True,
                            out=(o, ht))
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(ht, ht1)
    assert torch.isnan(o_full[:pad]).all() and torch.isnan(o_full[pad + on:]).all()
    assert torch.isnan(ht_full[:pad]).all() and torch.isnan(ht_full[pad + hn:]).all()


def test_recurrent_int64_offsets():
    """A varlen batch whose last sequence sits past 2^31 elements of q / k / v;
    only that sequence is checked against the oracle."""
    H = HV = 16
    K = V = 128
    tail = 40
    T = (1 << 20) + 64
    gen = torch.Generator().manual_seed(4)
    q = torch.zeros(1, T, H, K, dtype=torch.bfloat16)
    k = torch.zeros(1, T, H, K, dtype=torch.bfloat16)
    v = torch.zeros(1, T, HV, V, dtype=torch.bfloat16)
    g = torch.zeros(1, T, HV)
    beta = torch.zeros(1, T, HV)
    s = T - tail
    q[:, s:] = torch.randn(1, tail, H, K, generator=gen).bfloat16()
    k[:, s:] = torch.randn(1, tail, H, K, generator=gen).bfloat16()
    v[:, s:] = torch.randn(1, tail, HV, V, generator=gen).bfloat16()
    g[:, s:] = torch.nn.functional.logsigmoid(torch.randn(1, tail, HV, generator=gen) + 4)
    beta[:, s:] = torch.sigmoid(torch.randn(1, tail, HV, generator=gen))
    h0 = 0.1 * torch.randn(2, HV, K, V, generator=gen)
    assert (T - 1) * H * K > 2 ** 31
    cu = torch.tensor([0, s, T], dtype=torch.int32)
    o, ht = gdr.fused_recurrent_fwd(q.cuda(), k.cuda(), v.cuda(), g.cuda(), beta.cuda(), cu_seqlens=cu.cuda(),
                                    initial_state=h0.cuda(), use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    ro, rht = recurrent.recurrent_fwd(q[:, s:], k[:, s:], v[:, s:], g[:, s:], beta[:, s:], h0=h0[1:2],
                                      use_qk_l2norm=True)
    check("o tail", f64(o[:, s:]), ro.numpy(), 5e-3)
    check("ht tail", f64(ht[1:2]), rht.numpy(), 5e-3)
