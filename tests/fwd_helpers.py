"""Helpers shared by the GPU parity tests: move seeded inputs to the GPU, run
the library forward, run the oracle on the same rounded inputs."""
import json
import os

import numpy as np
import torch

import chunked_gated_delta_06_amd as gdr
import workloads
from oracle import chunked
from oracle.metrics import err_ratio

TOL = {"bf16": 5e-3, "fp32": 1e-4}


def dev(x):
    return None if x is None else x.cuda()


def gpu_fwd(inp, *, h0=True, ht=True, workspace=None, out=None, keep_states=False):
    """Library forward on the inputs of ``workloads.make_inputs``; returns
    (o, ht, workspace views).  ``keep_states`` runs the separate scan and
    output stages (h and v_new kept in the workspace); otherwise the library
    picks the fused scan + output stage where the shape has one."""
    cu = dev(inp["cu_seqlens"])
    o, htd, ws = gdr.chunk_fwd(
        dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
        scale=inp["scale"], chunk_size=inp["chunk_size"], cu_seqlens=cu,
        initial_state=dev(inp["h0"]) if h0 else None, output_final_state=ht,
        use_qk_l2norm_in_kernel=inp["use_qk_l2norm"], workspace=workspace, return_workspace=True,
        out=out, keep_states=keep_states)
    torch.cuda.synchronize()
    p = gdr.make_problem(inp["q"], inp["v"], inp["g"], chunk_size=inp["chunk_size"],
                         cu_seqlens=inp["cu_seqlens"], use_qk_l2norm=inp["use_qk_l2norm"],
                         scale=inp["scale"], keep_states=keep_states)
    views = gdr.workspace_views(p, ws)
    return o, htd, views


def oracle_fwd(inp, h0=True, intermediates=False):
    return chunked.chunked_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                               scale=inp["scale"], h0=inp["h0"] if h0 else None,
                               cu_seqlens=inp["cu_seqlens"], use_qk_l2norm=inp["use_qk_l2norm"],
                               chunk_size=inp["chunk_size"], intermediates=intermediates)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def slice_inputs(inp, *, rows=None, heads=None):
    """Dense batch rows and/or value heads of a batch (H == HV only for heads)."""
    out = dict(inp)
    if rows is not None:
        for n in ("q", "k", "v", "g", "beta", "do"):
            if out.get(n) is not None:
                out[n] = out[n][rows]
        for n in ("h0", "dht"):
            if out.get(n) is not None:
                out[n] = out[n][rows]
        out["B"] = out["N"] = len(range(*rows.indices(inp["B"])))
    if heads is not None:
        for n in ("q", "k", "v", "g", "beta", "do"):
            if out.get(n) is not None:
                out[n] = out[n][:, :, heads].contiguous()
        for n in ("h0", "dht"):
            if out.get(n) is not None:
                out[n] = out[n][:, heads].contiguous()
    return out


def check(name, got, ref, tol):
    r = err_ratio(got, ref)
    log = os.environ.get("GDR_PARITY_LOG")
    if log:
        test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
        with open(log, "a") as f:
            f.write(json.dumps({"test": test, "tensor": name, "err_ratio": r, "tol": tol}) + "\n")
    assert r <= tol, f"{name}: err_ratio {r:.3e} > {tol:.1e}"
    return r
