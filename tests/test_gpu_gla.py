"""GPU parity of the simple GLA forward (gdr_simple_gla_fwd: the chunked
stages with Tm = I, w = 0, u = v) against the float64 per-token oracle, which
is pinned to its closed attention form in tests/test_oracle.py.  Tolerances as
the chunked forward: err_ratio <= 1e-4 (fp32), <= 5e-3 (bf16)."""
import pytest
import torch

import chunked_gated_delta_06_amd as gdr
import workloads
from oracle import recurrent
from fwd_helpers import TOL, check, dev, f64

pytestmark = pytest.mark.gpu

W = workloads.Workload


def mk(B=2, T=150, H=2, HV=4, K=64, V=64, C=64, dtype="bf16", l2=True, slow=True, lengths=None, h0=True,
       scale=0.5):
    w = W("gla", B=B, T=T, H=H, HV=HV, K=K, V=V, chunk_size=C, dtype=dtype, l2norm_in_kernel=l2,
          host_l2norm=not l2, slow_decay=slow, h0=h0, scale=scale)
    return w, workloads.make_inputs(w, lengths=lengths, seed=9)


def run(inp, h0=True):
    o, ht = gdr.simple_gla_fwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), scale=inp["scale"],
                               chunk_size=inp["chunk_size"], cu_seqlens=dev(inp["cu_seqlens"]),
                               initial_state=dev(inp["h0"]) if h0 else None,
                               use_qk_l2norm_in_kernel=inp["use_qk_l2norm"])
    torch.cuda.synchronize()
    ro, rht = recurrent.simple_gla_fwd(inp["q"], inp["k"], inp["v"], inp["g"], scale=inp["scale"],
                                       h0=inp["h0"] if h0 else None, cu_seqlens=inp["cu_seqlens"],
                                       use_qk_l2norm=inp["use_qk_l2norm"])
    return o, ht, ro.numpy(), rht.numpy()


CASES = [dict(dtype=dt, C=C, K=K, V=V)
         for dt in ("bf16", "fp32") for C in (32, 64) for (K, V) in ((32, 64), (128, 128), (256, 64))]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_simple_gla_sweep(cfg):
    w, inp = mk(**cfg)
    o, ht, ro, rht = run(inp)
    check("o", f64(o), ro, TOL[w.dtype])
    check("ht", f64(ht), rht, TOL[w.dtype])


@pytest.mark.parametrize("l2", [False, True])
def test_simple_gla_varlen_and_no_state(l2):
    w, inp = mk(B=1, lengths=[1, 63, 0, 130, 64], l2=l2)
    o, ht, ro, rht = run(inp)
    check("o", f64(o), ro, 5e-3)
    check("ht", f64(ht), rht, 5e-3)
    assert torch.equal(ht[2].cpu(), inp["h0"][2])
    o, ht, ro, rht = run(inp, h0=False)
    check("o (h0 = 0)", f64(o), ro, 5e-3)


def test_simple_gla_dense_shape():
    """The dense bf16 GDN workload's shape (one batch row) with its gate recipe."""
    w, inp = mk(B=1, T=1024, H=16, HV=16, K=128, V=128, slow=False, scale=1.0)
    o, ht, ro, rht = run(inp)
    check("o", f64(o), ro, 5e-3)
    check("ht", f64(ht), rht, 5e-3)
