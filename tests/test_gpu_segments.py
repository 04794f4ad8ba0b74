"""GPU parity of the single-device segment hand-off (gdr_chunk_fwd_segmented):
one sequence split into segments, each scanned on its own (local end state and
transition), the entering states merged along the segments, every segment
re-run from its entering state -- the KCP page's context-parallel forward with
the ranks replaced by the segments of one launch.

Against the float64 oracle: o and the final state of the whole sequence, the
state entering every segment (the oracle hands its own fp64 state from segment
to segment), and the transitions (the oracle's product of per-token maps).
Tolerances as the chunked forward: err_ratio <= 1e-4 (fp32), <= 5e-3 (bf16).
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


def mk(lengths, H=2, HV=4, K=64, V=64, C=64, dtype="bf16", pc=False, slow=True, h0=True, seed=5):
    w = W("seg", B=1, T=0, H=H, HV=HV, K=K, V=V, chunk_size=C, dtype=dtype, per_channel_gate=pc,
          l2norm_in_kernel=True, h0=h0, slow_decay=slow, scale=0.5)
    inp = workloads.make_inputs(w, seed=seed, lengths=lengths)
    # one sequence: the initial state is that of the first segment
    if inp["h0"] is not None:
        inp["h0"] = inp["h0"][:1].contiguous()
    return w, inp


def oracle_states(inp):
    """The oracle's state entering every segment and the end state, handing its
    own fp64 state from segment to segment."""
    cu = inp["cu_seqlens"].tolist()
    S = None if inp["h0"] is None else inp["h0"].double()
    states = [torch.zeros_like(inp["h0"], dtype=torch.float64) if S is None else S]
    for n in range(len(cu) - 1):
        sl = slice(cu[n], cu[n + 1])
        _, S = recurrent.recurrent_fwd(inp["q"][:, sl], inp["k"][:, sl], inp["v"][:, sl], inp["g"][:, sl],
                                       inp["beta"][:, sl], scale=inp["scale"], h0=states[-1],
                                       use_qk_l2norm=True)
        states.append(S)
    return torch.cat(states, 0).numpy()


CASES = [
    dict(dtype="bf16", K=64, V=64, C=64),
    dict(dtype="bf16", K=128, V=128, C=64),
    dict(dtype="bf16", K=64, V=128, C=32, pc=True),
    dict(dtype="fp32", K=32, V=64, C=64),
    dict(dtype="fp32", K=64, V=32, C=32, pc=True),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_segmented_forward(cfg):
    lengths = [64, 100, 1, 0, 135, 37]
    w, inp = mk(lengths, **cfg)
    tol = TOL[w.dtype]
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}
    o, ht, states, trans = gdr.chunk_fwd_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                                   scale=inp["scale"], chunk_size=w.chunk_size,
                                                   initial_state=d["h0"], use_qk_l2norm_in_kernel=True,
                                                   want_transitions=True)
    torch.cuda.synchronize()
    ro, rht = recurrent.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], scale=inp["scale"],
                                      h0=inp["h0"], use_qk_l2norm=True)
    check("o", f64(o), ro.numpy(), tol)
    check("ht", f64(ht), rht.numpy(), tol)
    rs = oracle_states(inp)
    check("segment states", f64(states), rs, tol)
    check("merged final state", f64(states[-1:]), rht.numpy(), tol)
    rM = recurrent.transition(inp["k"], inp["g"], inp["beta"], cu_seqlens=inp["cu_seqlens"], use_qk_l2norm=True)
    check("transitions", f64(trans), rM.numpy(), tol)
    # the empty segment hands its state straight through and has the identity transition
    assert torch.equal(states[3], states[4])
    assert torch.equal(trans[3].cpu(), torch.eye(w.K).expand(w.HV, w.K, w.K))
    # the single pass on the GPU agrees
    one = dict(inp, cu_seqlens=None)
    o1, ht1, _ = gpu_fwd(one)
    check("o vs single pass", f64(o), f64(o1), tol)


def test_segmented_long_sequence_fast_decay():
    """The long-sequence recipe (scalar gate logsigmoid(N(0,1)), K = V = 128,
    bf16) on 8 segments of 1024 tokens: against the GPU single pass, and the
    oracle on the first and last 256 tokens of two heads."""
    T, R = 8192, 8
    w, inp = mk([T // R] * R, H=4, HV=4, K=128, V=128, C=64, slow=False)
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}
    o, ht, states, _ = gdr.chunk_fwd_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                               scale=inp["scale"], initial_state=d["h0"],
                                               use_qk_l2norm_in_kernel=True)
    o1, ht1, _ = gpu_fwd(dict(inp, cu_seqlens=None))
    check("o vs single pass", f64(o), f64(o1), 5e-3)
    check("ht vs single pass", f64(ht), f64(ht1), 5e-3)
    hs = [0, 3]
    sub = {n: inp[n][:, :256][:, :, hs].contiguous() for n in ("q", "k", "v", "g", "beta")}
    ro, _ = recurrent.recurrent_fwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], scale=inp["scale"],
                                    h0=inp["h0"][:, hs], use_qk_l2norm=True)
    check("o first 256 tokens", f64(o)[:, :256][:, :, hs], ro.numpy(), 5e-3)
    # the last 256 tokens from the state the GPU merged into the last segment
    lo = T - 256
    sub = {n: inp[n][:, lo:][:, :, hs].contiguous() for n in ("q", "k", "v", "g", "beta")}
    _, S_lo = recurrent.recurrent_fwd(inp["q"][:, T - T // R:lo][:, :, hs].contiguous(),
                                      inp["k"][:, T - T // R:lo][:, :, hs].contiguous(),
                                      inp["v"][:, T - T // R:lo][:, :, hs].contiguous(),
                                      inp["g"][:, T - T // R:lo][:, :, hs].contiguous(),
                                      inp["beta"][:, T - T // R:lo][:, :, hs].contiguous(),
                                      scale=inp["scale"], h0=states[R - 1:R, hs].cpu(), use_qk_l2norm=True)
    ro, rht = recurrent.recurrent_fwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], scale=inp["scale"],
                                      h0=S_lo, use_qk_l2norm=True)
    check("o last 256 tokens", f64(o)[:, lo:][:, :, hs], ro.numpy(), 5e-3)
    check("ht", f64(ht)[:, hs], rht.numpy(), 5e-3)


def test_one_segment_is_the_single_pass():
    """One segment: the merge hands h0 through, the transition is that of the
    whole sequence, and o / ht match the oracle."""
    w, inp = mk([173], K=64, V=64)
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}
    o, ht, states, trans = gdr.chunk_fwd_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                                   scale=inp["scale"], initial_state=d["h0"],
                                                   use_qk_l2norm_in_kernel=True, want_transitions=True)
    torch.cuda.synchronize()
    assert torch.equal(states[0:1], d["h0"])
    ro, rht = recurrent.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], scale=inp["scale"],
                                      h0=inp["h0"], use_qk_l2norm=True)
    check("o", f64(o), ro.numpy(), 5e-3)
    check("ht", f64(ht), rht.numpy(), 5e-3)
    check("merged end state", f64(states[1:2]), rht.numpy(), 5e-3)
