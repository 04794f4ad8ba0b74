"""gdr_chunk_fwd_noalloc (the forward for callers that cannot allocate: no
workspace, the library's fixed per-device scratch) against gdr_chunk_fwd with
a workspace: the same kernels on the same inputs, so o and ht are bitwise
equal, and both within the tolerance of the chunked oracle.  Three calls in a
row, each smaller than the last (the scratch keeps the previous call's
contents), then a problem beyond the scratch, which is refused before any
launch."""
import pytest
import torch

import chunked_gated_delta_06_amd as gdr
import workloads
from fwd_helpers import TOL, check, dev, f64, oracle_fwd

pytestmark = pytest.mark.gpu

W = workloads.Workload

CALLS = [
    # fused path, dense GVA batch with a ragged tail (the larger call)
    dict(name="dense", B=2, T=300, H=2, HV=4, K=128, V=128, C=64, dtype="bf16", lengths=None),
    # separate stages (per-channel gate), varlen with an empty sequence
    dict(name="varlen_pc", B=1, T=0, H=2, HV=2, K=64, V=64, C=32, dtype="bf16", lengths=[70, 0, 33], pc=True),
    # zero-padded head dims in fp32 (padded copies after the compact layout), smallest
    dict(name="padded_fp32", B=1, T=40, H=1, HV=2, K=60, V=40, C=64, dtype="fp32", lengths=None),
]


def make(c):
    w = W(c["name"], B=c["B"], T=c["T"], H=c["H"], HV=c["HV"], K=c["K"], V=c["V"], chunk_size=c["C"],
          dtype=c["dtype"], per_channel_gate=c.get("pc", False), l2norm_in_kernel=True, h0=True,
          slow_decay=True, scale=0.5)
    return w, workloads.make_inputs(w, seed=31, lengths=c["lengths"])


def run_both(inp):
    d = {n: dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}
    kw = dict(scale=inp["scale"], chunk_size=inp["chunk_size"], cu_seqlens=d["cu_seqlens"],
              initial_state=d["h0"], use_qk_l2norm_in_kernel=True)
    o_ref, ht_ref = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], output_final_state=True, **kw)
    o = torch.full_like(o_ref, float("nan"))
    ht = torch.full_like(ht_ref, float("nan"))
    gdr.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], out=(o, ht), **kw)
    torch.cuda.synchronize()
    return o, ht, o_ref, ht_ref


def test_noalloc_forward_equals_workspace_forward():
    for c in CALLS:
        print(f"no-alloc call {c['name']}", flush=True)
        w, inp = make(c)
        o, ht, o_ref, ht_ref = run_both(inp)
        assert torch.equal(o, o_ref), c["name"]
        assert torch.equal(ht, ht_ref), c["name"]
        ro, rht = oracle_fwd(inp)
        check(f"o {c['name']}", f64(o), ro, TOL[w.dtype])
        check(f"ht {c['name']}", f64(ht), rht, TOL[w.dtype])


def test_noalloc_refuses_problems_beyond_the_scratch():
    """4 x 4096 tokens x 16 heads (bf16, K = V = 128) fit; 32768 tokens x 32
    heads (about 550 MB of w, u and token factors) do not, and come back as
    GDR_ERR_SCRATCH_LIMIT before any launch (o keeps its fill)."""
    T, Hh, K = 32768, 32, 128
    q = torch.zeros(1, T, Hh, K, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(1, T, Hh, device="cuda")
    o = torch.full((1, T, Hh, K), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="fixed scratch"):
        gdr.chunk_fwd_noalloc(q, q, q, g, g, out=(o, None))
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
