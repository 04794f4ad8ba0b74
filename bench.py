#!/usr/bin/env python3
"""Throughput of the chunked gated delta-rule forward on one MI355X.

One step = one full forward (K0 chunk table, K1 kk^T + triangular inverse,
K2 WY recompute, K3 state scan, K4 output) over one batch of the workload,
inputs resident in HBM.  Prints one JSON line:

  value        tokens/s of the whole forward (B*T / seconds per step)
  roofline     the dominant kernel's algorithmic HBM bytes per launch / its
               average launch time (HIP events on the launch stream), against
               8 TB/s; traffic = measured HBM bytes per launch from rocprofv3
               counters (profiles/), null when the kernel changed since
  cpu_baseline the float64 per-token oracle timed on a bounded sample

The bench first checks a sample of its own output against the oracle and
refuses to report numbers when that check fails.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def stage_bytes_per_token_head(w, T_seq):
    """Algorithmic HBM bytes per (token, value head) of each forward stage:
    every tensor counted once when written and once per reading stage, at the
    library's storage dtypes (q/k/v/o/intermediates in the input dtype, g and
    beta in fp32, h0/ht fp32)."""
    e = 2 if w.dtype == "bf16" else 4
    r = w.H / w.HV
    K, V, C = w.K, w.V, w.chunk_size
    gb = 4 * K if w.per_channel_gate else 4
    return {
        "kkt_solve": r * K * e + gb + 4 + e * C,
        "wy": r * K * e + V * e + e * C + gb + 4 + e * K + e * V,
        "fwd_h": e * K + e * V + r * K * e + gb + e * V + e * K * V / C + 8 * K * V / T_seq,
        "fwd_o": 2 * r * K * e + gb + e * V + e * K * V / C + V * e,
    }


def kernel_source_hash(stage):
    fname = {"kkt_solve": "k1_kkt_solve.hip", "wy": "k2_wy.hip", "fwd_h": "k3_fwd_h.hip",
             "fwd_o": "k4_fwd_o.hip"}[stage]
    h = hashlib.sha256()
    for f in (fname, "gdr_device.h"):
        with open(os.path.join(ROOT, "chunked_gated_delta_06_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(stage, workload):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{stage}:{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(stage):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, inp, budget_s=12.0):
    """The per-token float64 oracle on a bounded sample of the workload: the
    first sequence, all value heads, as many tokens as fit the time budget."""
    import torch
    from oracle import recurrent
    threads = torch.get_num_threads()
    T = inp["T"] if inp["cu_seqlens"] is None else int(inp["cu_seqlens"][1])
    tokens, spent = 0, 0.0
    step = 256
    S0 = inp["h0"][0:1] if inp["h0"] is not None else None
    while spent < budget_s and tokens < T:
        n = min(step, T - tokens)
        sl = slice(tokens, tokens + n)
        t0 = time.perf_counter()
        _, S0 = recurrent.recurrent_fwd(inp["q"][0:1, sl], inp["k"][0:1, sl], inp["v"][0:1, sl],
                                        inp["g"][0:1, sl], inp["beta"][0:1, sl], scale=inp["scale"],
                                        h0=S0, use_qk_l2norm=inp["use_qk_l2norm"])
        spent += time.perf_counter() - t0
        tokens += n
    return {"value": tokens / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"per-token float64 recurrence, sequence 0, all {w.HV} value heads, "
                      f"first {tokens} tokens ({spent:.1f} s)"}


def parity_gate(w, inp, o, ht):
    """Sequence 0 (all heads) of the GPU output against the chunked oracle."""
    import torch
    from oracle import chunked
    from oracle.metrics import err_ratio
    if inp["cu_seqlens"] is None:
        sl = slice(0, 1)
        sub = {k: (inp[k][sl] if inp.get(k) is not None else None) for k in ("q", "k", "v", "g", "beta", "h0")}
        go, ght = o[sl], (ht[sl] if ht is not None else None)
    else:
        e = int(inp["cu_seqlens"][1])
        sub = {k: inp[k][:, :e] for k in ("q", "k", "v", "g", "beta")}
        sub["h0"] = inp["h0"][0:1] if inp["h0"] is not None else None
        go, ght = o[:, :e], (ht[0:1] if ht is not None else None)
    ro, rht = chunked.chunked_fwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], scale=inp["scale"],
                                  h0=sub["h0"], use_qk_l2norm=inp["use_qk_l2norm"],
                                  chunk_size=inp["chunk_size"])
    tol = 5e-3 if w.dtype == "bf16" else 1e-4
    eo = err_ratio(go, ro)
    eh = err_ratio(ght, rht) if ght is not None else 0.0
    return eo, eh, tol


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gdn_dense_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="per-stage times on stderr")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (known bytes, to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": n, "copies": 5}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the operator runs on a single device here "
              "(sequences and heads would shard across GPUs with no communication).", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunked_gated_delta_06_amd as gdr
    import workloads

    w = workloads.CONFIGS[args.workload]
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    d = {k: (inp[k].to(dev) if isinstance(inp.get(k), torch.Tensor) else inp.get(k))
         for k in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}
    kw = dict(scale=inp["scale"], chunk_size=inp["chunk_size"], cu_seqlens=d["cu_seqlens"],
              initial_state=d["h0"], output_final_state=True,
              use_qk_l2norm_in_kernel=inp["use_qk_l2norm"])
    o, ht, ws = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], return_workspace=True, **kw)
    torch.cuda.synchronize()
    eo, eh, tol = parity_gate(w, inp, o.cpu(), ht.cpu())
    print(f"parity gate ({args.workload}, sequence 0): err_ratio o={eo:.2e} ht={eh:.2e} (tol {tol:.0e})",
          file=sys.stderr, flush=True)
    if not (eo <= tol and eh <= tol):
        print("parity check failed: refusing to report throughput", file=sys.stderr)
        sys.exit(1)

    L = gdr.lib()
    p = gdr.make_problem(d["q"], d["v"], d["g"], chunk_size=inp["chunk_size"], cu_seqlens=d["cu_seqlens"],
                         use_qk_l2norm=inp["use_qk_l2norm"], scale=inp["scale"])
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    fwd_args = (ctypes.byref(p), P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["cu_seqlens"]),
                P(d["h0"]), P(o), P(ht), P(ws), ctypes.c_size_t(ws.numel()), sp)

    def step():
        st = L.gdr_chunk_fwd(*fwd_args)
        if st != 0:
            raise RuntimeError(L.gdr_status_string(st).decode())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    tokens = inp["B"] * inp["T"]
    value = tokens / (wall / args.steps)

    # per-stage launch times with events on the launch stream, same kernels and order
    views = gdr.workspace_views(p, ws)
    cidx, coff = views["chunk_idx"], views["chunk_off"]
    stages = {
        "chunk_table": lambda: gdr.chunk_table(p, d["cu_seqlens"], cidx, coff),
        "kkt_solve": lambda: gdr.fwd_kkt_solve(p, d["k"], d["g"], d["beta"], cidx, coff, views["Tm"],
                                               views["kscale"]),
        "wy": lambda: gdr.fwd_wy(p, d["k"], d["v"], d["g"], d["beta"], cidx, coff, views["Tm"], views["w"],
                                 views["u"]),
        "fwd_h": lambda: gdr.fwd_h(p, d["k"], views["w"], views["u"], d["g"], cidx, coff, d["h0"], views["h"],
                                   views["v_new"], ht, views["kscale"]),
        "fwd_o": lambda: gdr.fwd_o(p, d["q"], d["k"], views["v_new"], views["h"], d["g"], cidx, coff, o),
    }
    names = list(stages)
    acc = {n: 0.0 for n in names}
    reps = max(5, args.steps)
    for _ in range(2):
        for n in names:
            stages[n]()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(reps)]
    for r in range(reps):
        evs[r][0].record(stream)
        for i, n in enumerate(names):
            stages[n]()
            evs[r][i + 1].record(stream)
    torch.cuda.synchronize()
    for r in range(reps):
        for i, n in enumerate(names):
            acc[n] += evs[r][i].elapsed_time(evs[r][i + 1])
    avg_ms = {n: acc[n] / reps for n in names}
    if args.breakdown:
        print("per-stage ms: " + ", ".join(f"{n}={avg_ms[n]:.4f}" for n in names), file=sys.stderr)

    T_seq = inp["B"] * inp["T"] / inp["N"]
    per_unit = stage_bytes_per_token_head(w, T_seq)
    units = tokens * w.HV
    dom = max(per_unit, key=lambda n: avg_ms[n])
    alg_bytes = per_unit[dom] * units
    achieved = alg_bytes / (avg_ms[dom] * 1e-3) / 1e9
    traffic = measured_traffic(dom, w.name)
    fwd_bytes = sum(per_unit.values()) * units

    line = {
        "metric": "tokens/sec and % HBM/MFMA roofline, chunk GDN fwd (+bwd) on 1 MI355X",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) q/k/v, logsigmoid gates, sigmoid beta)",
        "config": {"workload": w.name, "B": inp["B"], "T": inp["T"], "H": w.H, "HV": w.HV, "K": w.K,
                   "V": w.V, "chunk_size": w.chunk_size, "pass": "forward",
                   "gate": "per-channel" if w.per_channel_gate else "scalar",
                   "l2norm_in_kernel": w.l2norm_in_kernel, "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "bytes_per_unit": per_unit[dom], "units": units, "avg_launch_ms": avg_ms[dom]},
        "stage_ms": avg_ms,
        "forward_hbm_frac": fwd_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "parity": {"o": eo, "ht": eh, "tol": tol},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
