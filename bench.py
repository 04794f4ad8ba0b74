#!/usr/bin/env python3
"""Throughput of the chunked gated delta-rule operator on one MI355X.

One step = one full forward (K0 chunk table, K1 kk^T + triangular inverse,
K2 WY recompute, K3 state scan, K4 output) over one batch of the workload,
inputs resident in HBM; for a workload with a backward (long_bf16) a step is
the forward, keeping its intermediates, plus the full backward reading them
(B1 de_local, B2 reverse state-gradient scan, B3 fused gradients); the record
also times the alternative that recomputes K0-K3 in the backward.

Timing: HIP events recorded on the launch stream around every whole call
(gdr_chunk_fwd, or gdr_chunk_fwd + gdr_chunk_bwd), after the warm-up calls;
the median over the timed calls is the step time.  The wall clock around the
same timed calls (one synchronisation on each side) is kept beside it.

Prints one JSON line for the dense GDN workload (the headline) with, for every
workload of the default run, a record under "configs":

  value / ms_per_step   tokens/s and the median step time (events)
  hbm_frac_four_stage   the four-stage byte model (every K1..K4 tensor once
                        written and once per reading stage) / time / 8 TB/s
  hbm_frac_moved        the bytes the timed path's own stages move (same
                        rules, only the stages that run) / time / 8 TB/s
  hbm_frac_operator_min operator inputs and outputs only / time / 8 TB/s
  mfma_frac             matrix-product FLOPs of the timed stages / time /
                        dense MFMA peak of the dtype (bf16 2.5 PF, fp32 157.3 TF)
  roofline              the dominant kernel's algorithmic HBM bytes per launch /
                        its average launch time (events), against 8 TB/s;
                        traffic = measured HBM bytes per launch from rocprofv3
                        counters (profiles/), null when the kernel changed since
  cpu_baseline          the float64 per-token oracle timed on a bounded sample

Each record first checks a sample of its own output against the oracle and
the bench refuses to report numbers when that check fails.
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
PEAK_MFMA_FLOPS = {"bf16": 2.5e15, "fp32": 157.3e12}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def stage_bytes_per_token_head(w, T_seq, pc_fused=False, keep=False):
    """Algorithmic HBM bytes per (token, value head) of each forward stage:
    every tensor counted once when written and once per reading stage, at the
    library's storage dtypes (q/k/v/o and the intermediates in the input dtype,
    except the separate WY stage's u, which is fp32; g and beta in fp32, h0/ht
    fp32).  ``pc_fused``: the per-channel fused forward (its fused K1 + K2 also
    writes aqk and the gated queries, read by the fused scan + output).
    ``keep``: a forward that keeps its states (its fused stages also write Tm,
    u in fp32, h and v_new)."""
    e = 2 if w.dtype == "bf16" else 4
    r = w.H / w.HV
    K, V, C = w.K, w.V, w.chunk_size
    gb = 4 * K if w.per_channel_gate else 4
    states = e * K * V / C + e * V          # h (per chunk) and v_new
    if w.per_channel_gate and K <= 128:
        # the WY stage also writes the scan's gated keys kt and decay dl, which
        # the scan reads in place of k and g
        kt_dl = e * K + 4 * K / C
        d = {
            "kkt_solve": r * K * e + gb + 4 + e * C,
            "wy": r * K * e + V * e + e * C + gb + 4 + e * K + 4 * V + kt_dl,
            # fused K1 + K2 (chunk 32): k, v, g, beta -> Tm, w, u, kt, dl
            "kkt_wy": r * K * e + V * e + gb + 4 + e * C + e * K + 4 * V + kt_dl,
            "fwd_h": e * K + 4 * V + kt_dl + e * V + e * K * V / C + 8 * K * V / T_seq,
            "fwd_o": 2 * r * K * e + gb + e * V + e * K * V / C + V * e,
        }
        if pc_fused or keep:
            # + q read; aqk (fp32) and the gated queries written (Tm only when
            # the states are kept; u in the input dtype otherwise)
            ue = 4 if keep else e
            d["kkt_wy"] += r * K * e + 4 * C + e * K - (0 if keep else e * C) - (4 - ue) * V
            # w, u, kt, dl, the gated queries, aqk -> o, ht (+ h, v_new when kept)
            d["fwd_h_o"] = (e * K + ue * V + kt_dl + e * K + 4 * C + e * V + 8 * K * V / T_seq
                            + (states if keep else 0))
        return d
    # K1's per-chunk token factors (scalar gate): 3C + 4 floats per chunk and
    # value head, of which the separate scan reads the first C + 4
    kf_row = 0 if w.per_channel_gate else 4 * (3 * C + 4) / C
    kf_scan = gb if w.per_channel_gate else 4 * (C + 4) / C
    ue = 4 if keep else e                   # u: fp32 when the states are kept
    return {
        "kkt_solve": r * K * e + gb + 4 + e * C + kf_row,
        "wy": r * K * e + V * e + e * C + gb + 4 + e * K + 4 * V,
        "fwd_h": e * K + 4 * V + r * K * e + kf_scan + e * V + e * K * V / C + 8 * K * V / T_seq,
        "fwd_o": 2 * r * K * e + gb + e * V + e * K * V / C + V * e,
        # fused K1 + K2: k, v, g, beta -> w, u, token factors (+ Tm when kept)
        "kkt_wy": r * K * e + V * e + gb + 4 + e * K + ue * V + kf_row + (e * C if keep else 0),
        # fused scan + output: w, u, k, q, token factors -> o, ht (+ h, v_new when kept)
        "fwd_h_o": e * K + ue * V + r * K * e + r * K * e + kf_row + e * V + 8 * K * V / T_seq
                   + (states if keep else 0),
    }


def four_stage_bytes_per_token_head(w, T_seq):
    """The four-stage byte model of the chunk method (K1 kk^T + inverse, K2
    WY, K3 state scan, K4 output), per (token, value head): every tensor the
    four stages materialise is counted once when written and once per reading
    stage, at the fixed storage dtypes (T, w, u, v_new, h in the input dtype;
    g, beta fp32; h0 / ht fp32).  It is independent of how this library fuses
    the stages."""
    e = 2 if w.dtype == "bf16" else 4
    r = w.H / w.HV
    K, V, C = w.K, w.V, w.chunk_size
    gb = 4 * K if w.per_channel_gate else 4
    k1 = r * K * e + gb + 4 + e * C
    k2 = r * K * e + V * e + e * C + gb + 4 + e * K + e * V
    k3 = e * K + e * V + r * K * e + gb + e * V + e * K * V / C + 8 * K * V / T_seq
    k4 = 2 * r * K * e + gb + e * V + e * K * V / C + V * e
    return k1 + k2 + k3 + k4


def operator_min_bytes_per_token_head(w, T_seq, backward=False):
    """The operator's own inputs and outputs only, per (token, value head):
    q, k (shared by a GVA group), v, g, beta, o, h0 / ht; the backward adds
    do, dht and the gradients dq, dk, dv, dg, dbeta, dh0."""
    e = 2 if w.dtype == "bf16" else 4
    r = w.H / w.HV
    K, V = w.K, w.V
    gb = 4 * K if w.per_channel_gate else 4
    fwd = 2 * r * K * e + 2 * V * e + gb + 4 + 8 * K * V / T_seq
    if not backward:
        return fwd
    # inputs q, k, v, g, beta, do, h0, dht; outputs dq, dk, dv, dg, dbeta, dh0
    return 2 * r * K * e + V * e + gb + 4 + V * e + 2 * r * K * e + V * e + gb + 4 + 12 * K * V / T_seq


def flops_per_token_head(w, part):
    """Matrix-product FLOPs per (token, value head) (2 per multiply-add,
    causal C x C products at half, the triangular inverse at C^2 / 3):
      forward  kk^T CK, inverse C^2/3, W CK, U CV, E = U - W S 2KV, state
               update 2KV, Q S0 2KV, Q K^T CK, P E CV
               = 3CK + 2CV + 6KV + C^2/3
      bwd      (B1..B3, the backward's own stages) P CK + P^T dO CV (B1);
               K dS, Q^T dO, W^T dE 6KV (B2); B3: P CK, P^T dO CV, K dS1 2KV,
               Y = T^T dE CV, dQg / T^T dW / dKt 6KV, dP CV, dA CV, and five
               C x C by C x K products (D K, D^T Q, kk^T, Dk K, Dk^T K) 5CK
               = 7CK + 5CV + 14KV"""
    K, V, C = w.K, w.V, w.chunk_size
    fwd = 3 * C * K + 2 * C * V + 6 * K * V + C * C / 3
    bwd = 7 * C * K + 5 * C * V + 14 * K * V
    if w.per_channel_gate:
        # the gated pair sums (P in the intra-chunk stage; dq, dk through P and
        # A in B3) run on the vector ALU and are not matrix-core FLOPs:
        # P^T dO CV (B1); 6KV (B2); Kt dS1 2KV, Y CV, dQg / TdW / dKt 6KV,
        # dP CV, dA CV (B3)
        bwd = 4 * C * V + 14 * K * V
    return {"forward": fwd, "bwd": bwd}[part]


def bwd_stage_bytes_per_token_head(w, T_seq):
    """Same accounting for the backward's own stages (the K1-K3 recompute is
    counted with the forward model, without the ht write)."""
    e = 2 if w.dtype == "bf16" else 4
    r = w.H / w.HV
    K, V, C = w.K, w.V, w.chunk_size
    fwd = stage_bytes_per_token_head(w, T_seq, keep=True)
    if w.per_channel_gate:
        return {
            "kkt_solve": fwd["kkt_solve"],
            "wy": fwd["wy"],
            "kkt_wy": fwd["kkt_wy"],
            "fwd_h": fwd["fwd_h"] - 4 * K * V / T_seq,
            # q, k, g, dO -> de_local, the gated rows kt, qg and the decay dl
            "bwd_intra": 2 * r * K * e + 4 * K + V * e + V * e + 2 * K * e + 4 * K / C,
            # kt, qg, w, dO, de_local, dl, dht -> dh (fp32), dh0
            "bwd_dh": 3 * K * e + 2 * V * e + 4 * K / C + 4 * K * V / C + 8 * K * V / T_seq,
            # q, k, v, g, beta, dO, Tm, h, v_new, dh (fp32), de_local, kt -> dq, dk, dv, dg, dbeta
            "bwd_dqkvg": 4 * r * K * e + 5 * V * e + 8 * K + 8 + e * C + e * K * V / C + 4 * K * V / C + K * e,
        }
    return {
        "kkt_solve": fwd["kkt_solve"],
        "wy": fwd["wy"],
        "kkt_wy": fwd["kkt_wy"],
        "fwd_h": fwd["fwd_h"] - 4 * K * V / T_seq,
        # q, k, g, dO -> de_local, qscale
        "bwd_intra": 2 * r * K * e + 4 + V * e + V * e + 4,
        # q, k, w, dO, de_local, qscale, kscale, dht -> dh (fp32), dh0
        "bwd_dh": 2 * r * K * e + K * e + 2 * V * e + 8 + 4 * K * V / C + 8 * K * V / T_seq,
        # q, k, v, g, beta, dO, Tm, h, v_new, dh (fp32) -> dq, dk, dv, dg, dbeta
        "bwd_dqkvg": 4 * r * K * e + 4 * V * e + 16 + e * C + e * K * V / C + 4 * K * V / C,
    }


def kernel_source_hash(stage):
    fname = {"kkt_solve": ("k1_kkt_solve.hip",), "wy": ("k2_wy.hip",), "fwd_h": ("k3_fwd_h.hip",),
             "fwd_o": ("k4_fwd_o.hip",), "fwd_h_o": ("k3_fwd_h.hip",),
             "kkt_wy": ("k12_kkt_wy.hip", "k12pc_kkt_wy.hip"), "bwd_intra": ("b1_bwd_intra.hip",),
             "bwd_dh": ("b2_bwd_dh.hip",), "bwd_dqkvg": ("b3_bwd_dqkvg.hip", "b3pc_bwd_dqkvg.hip"),
             "recurrent": ("k5_recurrent.hip",)}[stage]
    h = hashlib.sha256()
    for f in (*fname, "gdr_device.h"):
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


def cpu_baseline(w, inp, budget_s=20.0):
    """The per-token float64 oracle on a bounded sample of the workload: whole
    sequences in order, all value heads, until the time budget or the
    workload ends; the chunked/WY oracle is timed on the first sequence."""
    import torch
    from oracle import chunked, recurrent
    threads = torch.get_num_threads()
    B, N = inp["B"], inp["N"]
    cu = inp["cu_seqlens"]
    step = 512
    tokens, spent, seqs = 0, 0.0, 0
    for n in range(N):
        if spent >= budget_s:
            break
        if cu is None:
            b, s0, e0 = n, 0, inp["T"]
        else:
            b, s0, e0 = 0, int(cu[n]), int(cu[n + 1])
        S = inp["h0"][n:n + 1] if inp["h0"] is not None else None
        for s in range(s0, e0, step):
            if spent >= budget_s:
                break
            sl = slice(s, min(s + step, e0))
            t0 = time.perf_counter()
            _, S = recurrent.recurrent_fwd(inp["q"][b:b + 1, sl], inp["k"][b:b + 1, sl], inp["v"][b:b + 1, sl],
                                           inp["g"][b:b + 1, sl], inp["beta"][b:b + 1, sl], scale=inp["scale"],
                                           h0=S, use_qk_l2norm=inp["use_qk_l2norm"])
            spent += time.perf_counter() - t0
            tokens += sl.stop - sl.start
        seqs += 1
    # chunked/WY oracle on the first sequence (or its first 4096 tokens)
    if cu is None:
        b, s0, e0 = 0, 0, min(inp["T"], 4096)
    else:
        b, s0, e0 = 0, int(cu[0]), min(int(cu[1]), int(cu[0]) + 4096)
    sl = slice(s0, e0)
    t0 = time.perf_counter()
    chunked.chunked_fwd(inp["q"][b:b + 1, sl], inp["k"][b:b + 1, sl], inp["v"][b:b + 1, sl],
                        inp["g"][b:b + 1, sl], inp["beta"][b:b + 1, sl], scale=inp["scale"],
                        h0=inp["h0"][0:1] if inp["h0"] is not None else None,
                        use_qk_l2norm=inp["use_qk_l2norm"], chunk_size=inp["chunk_size"])
    tc = time.perf_counter() - t0
    return {"value": tokens / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"per-token float64 recurrence, {seqs} of {N} sequences in order (the last possibly "
                      f"cut at the {budget_s:.0f} s budget), all {w.HV} value heads, {tokens} tokens in "
                      f"{spent:.1f} s",
            "chunked_oracle_tokens_per_s": (e0 - s0) / tc,
            "chunked_oracle_sample": f"chunked/WY float64 evaluation, sequence 0, {e0 - s0} tokens, "
                                     f"all {w.HV} value heads, {tc:.1f} s"}


def cpu_baseline_bwd(w, inp, T=4096, heads=(0, 21)):
    """The per-token float64 oracle forward + hand-derived backward on the first
    T tokens of the given value heads, scaled to all value heads."""
    import torch
    from oracle import recurrent
    hs = list(heads)
    sub = {n: inp[n][:, :T][:, :, hs].contiguous() for n in ("q", "k", "v", "g", "beta", "do")}
    t0 = time.perf_counter()
    recurrent.recurrent_bwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], sub["do"],
                            inp["dht"][:, hs], scale=inp["scale"],
                            h0=inp["h0"][:, hs] if inp["h0"] is not None else None,
                            use_qk_l2norm=inp["use_qk_l2norm"])
    spent = time.perf_counter() - t0
    per_head_s = spent / len(hs)
    return {"value": T / (per_head_s * w.HV), "unit": "tokens/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"per-token float64 forward replay + reverse recurrence, first {T} tokens of value "
                      f"head(s) {hs} ({spent:.1f} s), rate scaled to all {w.HV} value heads"}


def parity_gate(w, inp, o, ht, max_tokens=2048, ht_heads=(0, -1)):
    """The first sequence against the chunked oracle: o on its first
    ``max_tokens`` tokens for every value head, and ht after the whole
    sequence (all heads when the sequence is no longer than max_tokens,
    otherwise the value heads ``ht_heads``, which needs H == HV)."""
    from oracle import chunked
    from oracle.metrics import err_ratio
    cu = inp["cu_seqlens"]
    s0, e0 = (0, inp["T"]) if cu is None else (int(cu[0]), int(cu[1]))
    Tp = min(e0 - s0, max_tokens)

    def run(t_end, heads):
        d = {}
        for n in ("q", "k", "v", "g", "beta"):
            x = inp[n][0:1, s0:t_end]
            d[n] = x if heads is None else x[:, :, heads].contiguous()
        h0 = inp["h0"]
        d["h0"] = None if h0 is None else (h0[0:1] if heads is None else h0[0:1, heads].contiguous())
        return chunked.chunked_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=inp["scale"], h0=d["h0"],
                                   use_qk_l2norm=inp["use_qk_l2norm"], chunk_size=inp["chunk_size"])

    ro, rht = run(s0 + Tp, None)
    eo = err_ratio(o[0:1, s0:s0 + Tp], ro)
    label_o = f"o (sequence 0, first {Tp} tokens, all heads)"
    if ht is None:
        return {label_o: eo}
    if Tp == e0 - s0:
        return {label_o: eo, "ht (sequence 0, all heads)": err_ratio(ht[0:1], rht)}
    assert w.H == w.HV, "a head subset of the final state needs H == HV"
    hs = sorted({h % w.HV for h in ht_heads})
    _, rht = run(e0, hs)
    return {label_o: eo, f"ht (sequence 0, heads {hs})": err_ratio(ht[0:1, hs], rht)}


def event_stage_ms(stream, stages, reps):
    """Average milliseconds per launch of each stage (HIP events recorded on
    the launch stream around every launch, stages run in order)."""
    import torch
    names = list(stages)
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
    acc = {n: 0.0 for n in names}
    for r in range(reps):
        for i, n in enumerate(names):
            acc[n] += evs[r][i].elapsed_time(evs[r][i + 1])
    return {n: acc[n] / reps for n in names}


def call_stage_ms(gdr, call, reps):
    """Average milliseconds per launch of each stage of a full library call,
    from the HIP events the library records on its launch stream after every
    stage (gdr_stage_timing), over ``reps`` calls run back to back after two
    untimed ones, so that each interval is the stage's own GPU time."""
    import torch
    call()
    call()
    torch.cuda.synchronize()
    gdr.stage_timing(True)
    try:
        for _ in range(reps):
            call()
        rec = gdr.stage_times()
    finally:
        gdr.stage_timing(False)
    acc, cnt = {}, {}
    for n, ms in rec:
        acc[n] = acc.get(n, 0.0) + ms
        cnt[n] = cnt.get(n, 0) + 1
    return {n: acc[n] / cnt[n] for n in acc}


def timed_calls(step, warmup, steps, stream):
    """Run ``warmup`` untimed steps, then ``steps`` timed steps with HIP events
    recorded on the launch stream around each whole step.  Returns the median
    and mean event time per step and the wall-clock time per step over the
    timed steps (one synchronisation on each side), in milliseconds."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    n = len(ms)
    med = ms[n // 2] if n % 2 else 0.5 * (ms[n // 2 - 1] + ms[n // 2])
    return {"median_ms": med, "mean_event_ms": sum(ms) / n, "wall_ms": wall, "min_ms": ms[0], "max_ms": ms[-1]}


def fractions(w, T_seq, units, ms, moved_per_unit, backward):
    """HBM and MFMA fractions of one step of ``ms`` milliseconds over ``units``
    (token, value head) pairs."""
    sec = ms * 1e-3
    out = {}
    if not backward:
        four = four_stage_bytes_per_token_head(w, T_seq)
        out["four_stage_bytes"] = four * units
        out["hbm_frac_four_stage"] = four * units / sec / (PEAK_HBM_GBS * 1e9)
        flops = flops_per_token_head(w, "forward") * units
    else:
        flops = (flops_per_token_head(w, "forward") + flops_per_token_head(w, "bwd")) * units
    out["moved_bytes"] = moved_per_unit * units
    out["hbm_frac_moved"] = moved_per_unit * units / sec / (PEAK_HBM_GBS * 1e9)
    omin = operator_min_bytes_per_token_head(w, T_seq, backward)
    out["operator_min_bytes"] = omin * units
    out["hbm_frac_operator_min"] = omin * units / sec / (PEAK_HBM_GBS * 1e9)
    out["flops"] = flops
    out["mfma_frac"] = flops / sec / PEAK_MFMA_FLOPS[w.dtype]
    return out


def roofline(per_unit, avg_ms, units, workload, stages):
    dom = max(stages, key=lambda n: avg_ms[n])
    alg_bytes = per_unit[dom] * units
    achieved = alg_bytes / (avg_ms[dom] * 1e-3) / 1e9
    return {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(dom, workload),
            "bytes_per_unit": per_unit[dom], "units": units, "avg_launch_ms": avg_ms[dom]}


def to_dev(inp, dev, names):
    import torch
    return {k: (inp[k].to(dev) if isinstance(inp.get(k), torch.Tensor) else inp.get(k)) for k in names}


def bwd_parity_gate(gdr, w, inp, dev, o, T=2048, heads=(0, 21)):
    """The timed forward's o on the first T tokens of two value heads, and the
    backward (same kernels, same per-head shapes) run on those tokens and
    heads, against the chunk-wise oracle."""
    import torch
    from oracle import chunked
    from oracle.metrics import err_ratio
    hs = list(heads)
    sub = {n: inp[n][:, :T][:, :, hs].contiguous() for n in ("q", "k", "v", "g", "beta", "do")}
    sub["h0"] = inp["h0"][:, hs].contiguous() if inp["h0"] is not None else None
    sub["dht"] = inp["dht"][:, hs].contiguous()
    d = to_dev(sub, dev, list(sub))
    res = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["dht"], scale=inp["scale"],
                        chunk_size=inp["chunk_size"], initial_state=d["h0"],
                        use_qk_l2norm_in_kernel=inp["use_qk_l2norm"])
    torch.cuda.synchronize()
    ref = chunked.chunked_bwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], sub["do"], sub["dht"],
                              scale=inp["scale"], h0=sub["h0"], use_qk_l2norm=inp["use_qk_l2norm"],
                              chunk_size=inp["chunk_size"])
    errs = {n: err_ratio(t.cpu(), ref[n]) for n, t in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), res)}
    ro, _ = chunked.chunked_fwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], scale=inp["scale"],
                                h0=sub["h0"], use_qk_l2norm=inp["use_qk_l2norm"], chunk_size=inp["chunk_size"])
    errs["o"] = err_ratio(o[:, :T][:, :, hs].cpu(), ro)
    return errs, (5e-3 if w.dtype == "bf16" else 1e-4)


def measure(gdr, w, steps, warmup, breakdown, label):
    """Time one workload; returns the fields of its JSON record."""
    import torch
    dev = torch.device("cuda:0")
    inp = workloads_inputs(w)
    backward = bool(w.backward)
    d = to_dev(inp, dev, ("q", "k", "v", "g", "beta", "h0", "cu_seqlens", "do", "dht"))
    kw = dict(scale=inp["scale"], chunk_size=inp["chunk_size"], cu_seqlens=d["cu_seqlens"],
              initial_state=d["h0"], output_final_state=True,
              use_qk_l2norm_in_kernel=inp["use_qk_l2norm"])
    # the same forward path the timed step runs (fused scan + output where the
    # shape has it); the workspace still holds the K0-K2 intermediates the
    # per-stage timing below reads
    o, ht, ws = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], return_workspace=True,
                              keep_states=False, **kw)
    torch.cuda.synchronize()
    if backward:
        errs, tol = bwd_parity_gate(gdr, w, inp, dev, o)
        parity = {**{f"{n} (first 2048 tokens, heads 0 and 21)": v for n, v in errs.items()}, "tol": tol}
        ok = all(v <= tol for v in errs.values())
    else:
        tol = 5e-3 if w.dtype == "bf16" else 1e-4
        parity = {**parity_gate(w, inp, o.cpu(), ht.cpu()), "tol": tol}
        ok = all(v <= tol for k, v in parity.items() if k != "tol")
    print(f"parity gate ({label}): " + ", ".join(f"{k}={v:.2e}" for k, v in parity.items()),
          file=sys.stderr, flush=True)
    if not ok:
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
    if backward:
        blay = gdr.bwd_layout(p)
        bws = torch.empty(blay.total, dtype=torch.uint8, device=dev)
        grads = [torch.empty_like(d[n]) for n in ("q", "k", "v", "g", "beta")]
        dh0 = torch.empty(inp["N"], w.HV, w.K, w.V, dtype=torch.float32, device=dev)
        bwd_args = (ctypes.byref(p), P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]),
                    P(d["cu_seqlens"]), P(d["h0"]), P(d["do"]), P(d["dht"]), *[P(t) for t in grads], P(dh0),
                    P(bws), ctypes.c_size_t(bws.numel()), sp)

        # a training step keeps the forward's intermediates for the backward:
        # the forward runs its separate stages into the backward's workspace
        # and the backward skips its recompute of K0-K3
        pk = gdr.make_problem(d["q"], d["v"], d["g"], chunk_size=inp["chunk_size"], cu_seqlens=d["cu_seqlens"],
                              use_qk_l2norm=inp["use_qk_l2norm"], scale=inp["scale"], keep_states=True)
        fwd_keep_args = (ctypes.byref(pk), *fwd_args[1:10], P(bws), ctypes.c_size_t(bws.numel()), sp)
        bwd_keep_args = (ctypes.byref(pk), *bwd_args[1:])

    def check_st(st):
        if st != 0:
            raise RuntimeError(L.gdr_status_string(st).decode())

    def step():
        if backward:
            check_st(L.gdr_chunk_fwd(*fwd_keep_args))
            check_st(L.gdr_chunk_bwd(*bwd_keep_args))
        else:
            check_st(L.gdr_chunk_fwd(*fwd_args))

    def step_recompute():
        check_st(L.gdr_chunk_fwd(*fwd_args))
        check_st(L.gdr_chunk_bwd(*bwd_args))

    timing = timed_calls(step, warmup, steps, stream)
    ms_per_step = timing["median_ms"]
    recompute = timed_calls(step_recompute, warmup, steps, stream) if backward else None
    tokens = inp["B"] * inp["T"]
    value = tokens / (ms_per_step * 1e-3)

    # per-stage launch times: the library's own HIP events on the launch
    # stream, inside the same calls the step makes
    reps = max(5, min(steps, 50))
    fwd_call = (lambda: check_st(L.gdr_chunk_fwd(*fwd_keep_args))) if backward else \
        (lambda: check_st(L.gdr_chunk_fwd(*fwd_args)))
    fwd_ms = call_stage_ms(gdr, fwd_call, reps)
    T_seq = inp["B"] * inp["T"] / inp["N"]
    units = tokens * w.HV
    pc_fused = not backward and gdr.chunk_fwd_fused(p) == 2
    per_unit = {k: v for k, v in stage_bytes_per_token_head(w, T_seq, pc_fused, keep=backward).items()
                if k in fwd_ms}
    rec = {"value": value, "ms_per_step": ms_per_step, "tokens": tokens,
           "timing": {**timing, "what": "HIP events around each whole call on the launch stream; "
                                        "ms_per_step = median_ms; wall_ms = wall clock per step"},
           "stage_ms": {"forward": fwd_ms}, "parity": parity}
    if not backward:
        rec.update(fractions(w, T_seq, units, ms_per_step, sum(per_unit.values()), False))
    rec["roofline"] = roofline(per_unit, fwd_ms, units, w.name, list(per_unit))
    if backward:
        # the backward's own stages (the step's forward leaves K0-K3's
        # intermediates in this workspace)
        bwd_ms = call_stage_ms(gdr, lambda: check_st(L.gdr_chunk_bwd(*bwd_keep_args)), reps)
        bper = {k: v for k, v in bwd_stage_bytes_per_token_head(w, T_seq).items() if k in bwd_ms}
        rec["stage_ms"]["backward"] = bwd_ms
        bwd_total_ms = sum(bwd_ms.values())
        rec["backward_hbm_frac"] = sum(bper.values()) * units / (bwd_total_ms * 1e-3) / 1e9 / PEAK_HBM_GBS
        rec["backward_ms"] = bwd_total_ms
        rec["recompute_ms_per_step"] = recompute["median_ms"]
        rec.update(fractions(w, T_seq, units, ms_per_step, sum(per_unit.values()) + sum(bper.values()), True))
        rec["step"] = ("forward with its intermediates kept (separate stages) + backward reading them; "
                       "recompute_ms_per_step: fused forward + backward that recomputes K0-K3")
        # the dominant kernel of a forward + backward step is taken among the
        # backward's own stages (the forward's stages are reported separately)
        rec["roofline"] = roofline(bper, bwd_ms, units, w.name, [n for n in bper if n.startswith("bwd_")])
        rec["forward_roofline"] = roofline(per_unit, fwd_ms, units, w.name, list(per_unit))
    if breakdown:
        for part, ms in rec["stage_ms"].items():
            print(f"{label} {part} per-stage ms: " + ", ".join(f"{n}={v:.4f}" for n, v in ms.items()),
                  file=sys.stderr)
    return rec, inp


def decode_bytes_per_token_head(w):
    """Algorithmic HBM bytes per (token, value head) of the token-by-token
    kernel over one decoding step (T tokens per sequence): q, k (shared by the
    value heads of a group), v, g, beta and o per token, plus the fp32 state
    read from h0 and written to ht once per sequence."""
    e = 2 if w.dtype == "bf16" else 4
    r = w.H / w.HV
    gb = 4 * w.K if w.per_channel_gate else 4
    return 2 * r * w.K * e + w.V * e + gb + 4 + w.V * e + 8 * w.K * w.V / w.T


def measure_decode(gdr, w, steps, warmup):
    """Time one decoding step of the token-by-token forward
    (gdr_fused_recurrent_fwd) on workload ``w``; returns its JSON record."""
    import torch
    from oracle import recurrent
    from oracle.metrics import err_ratio
    dev = torch.device("cuda:0")
    inp = workloads_inputs(w)
    d = to_dev(inp, dev, ("q", "k", "v", "g", "beta", "h0", "cu_seqlens"))
    kw = dict(scale=inp["scale"], cu_seqlens=d["cu_seqlens"], initial_state=d["h0"],
              use_qk_l2norm_in_kernel=inp["use_qk_l2norm"])
    o, ht = gdr.fused_recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], **kw)
    torch.cuda.synchronize()
    seqs = [0, 1, inp["N"] // 2, inp["N"] - 1]
    ro, rht = recurrent.recurrent_fwd(inp["q"][seqs], inp["k"][seqs], inp["v"][seqs], inp["g"][seqs],
                                      inp["beta"][seqs], scale=inp["scale"], h0=inp["h0"][seqs],
                                      use_qk_l2norm=inp["use_qk_l2norm"])
    tol = 5e-3 if w.dtype == "bf16" else 1e-4
    parity = {"o (4 sequences, all heads)": err_ratio(o[seqs].cpu(), ro),
              "ht (4 sequences, all heads)": err_ratio(ht[seqs].cpu(), rht), "tol": tol}
    print(f"parity gate ({w.name}): " + ", ".join(f"{k}={v:.2e}" for k, v in parity.items()),
          file=sys.stderr, flush=True)
    if not all(v <= tol for k, v in parity.items() if k != "tol"):
        print("parity check failed: refusing to report throughput", file=sys.stderr)
        sys.exit(1)
    L = gdr.lib()
    p = gdr.make_problem(d["q"], d["v"], d["g"], cu_seqlens=d["cu_seqlens"],
                         use_qk_l2norm=inp["use_qk_l2norm"], scale=inp["scale"])
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = torch.cuda.current_stream(dev)
    args = (ctypes.byref(p), P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["cu_seqlens"]),
            P(d["h0"]), P(o), P(ht), ctypes.c_void_p(stream.cuda_stream))

    def step():
        st = L.gdr_fused_recurrent_fwd(*args)
        if st != 0:
            raise RuntimeError(L.gdr_status_string(st).decode())

    timing = timed_calls(step, warmup, steps, stream)
    ms_per_step = timing["median_ms"]
    ev_ms = event_stage_ms(stream, {"recurrent": step}, max(5, min(steps, 50)))
    tokens = inp["B"] * inp["T"]
    units = tokens * w.HV
    per_unit = {"recurrent": decode_bytes_per_token_head(w)}
    rec = {"value": tokens / (ms_per_step * 1e-3), "ms_per_step": ms_per_step, "tokens": tokens,
           "timing": timing, "stage_ms": {"forward": ev_ms}, "parity": parity,
           "roofline": roofline(per_unit, ev_ms, units, w.name, ["recurrent"])}
    return rec, inp


def measure_segmented(gdr, w, R, steps, warmup):
    """The long sequence of ``w`` split into R equal segments and run as the
    single-device segment hand-off (gdr_chunk_fwd_segmented: local end states
    and transitions, merge, re-run), beside the single pass over the whole
    sequence (gdr_chunk_fwd).  Parity: o and ht against the single pass, and o
    on the first 2048 tokens of two heads against the chunked oracle."""
    import torch
    from oracle import chunked
    from oracle.metrics import err_ratio
    dev = torch.device("cuda:0")
    inp = workloads_inputs(w)
    T = inp["T"]
    cu = torch.arange(0, T + 1, T // R, dtype=torch.int32)
    d = to_dev(inp, dev, ("q", "k", "v", "g", "beta", "h0"))
    d["cu"] = cu.to(dev)
    o, ht, states, _ = gdr.chunk_fwd_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"],
                                               scale=inp["scale"], chunk_size=inp["chunk_size"],
                                               initial_state=d["h0"],
                                               use_qk_l2norm_in_kernel=inp["use_qk_l2norm"])
    o1, ht1, ws1 = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=inp["scale"],
                                 chunk_size=inp["chunk_size"], initial_state=d["h0"],
                                 use_qk_l2norm_in_kernel=inp["use_qk_l2norm"], return_workspace=True)
    torch.cuda.synchronize()
    hs = [0, w.HV // 2]
    sub = {n: inp[n][:, :2048][:, :, hs].contiguous() for n in ("q", "k", "v", "g", "beta")}
    ro, _ = chunked.chunked_fwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], scale=inp["scale"],
                                h0=inp["h0"][:, hs], use_qk_l2norm=inp["use_qk_l2norm"],
                                chunk_size=inp["chunk_size"])
    tol = 5e-3 if w.dtype == "bf16" else 1e-4
    parity = {"o vs single pass": err_ratio(o.cpu(), o1.cpu()), "ht vs single pass": err_ratio(ht.cpu(), ht1.cpu()),
              "o (first 2048 tokens, 2 heads) vs oracle": err_ratio(o[:, :2048][:, :, hs].cpu(), ro), "tol": tol}
    print(f"parity gate ({w.name}, {R} segments): " + ", ".join(f"{k}={v:.2e}" for k, v in parity.items()),
          file=sys.stderr, flush=True)
    if not all(v <= tol for k, v in parity.items() if k != "tol"):
        print("parity check failed: refusing to report throughput", file=sys.stderr)
        sys.exit(1)
    L = gdr.lib()
    p = gdr.make_problem(d["q"], d["v"], d["g"], chunk_size=inp["chunk_size"], cu_seqlens=d["cu"],
                         use_qk_l2norm=inp["use_qk_l2norm"], scale=inp["scale"])
    lay = gdr.seg_layout(p)
    ws = torch.empty(lay.total, dtype=torch.uint8, device=dev)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = (ctypes.byref(p), P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["cu"]), P(d["h0"]),
            P(o), P(ht), P(states), None, P(ws), ctypes.c_size_t(ws.numel()), sp)
    p1 = gdr.make_problem(d["q"], d["v"], d["g"], chunk_size=inp["chunk_size"],
                          use_qk_l2norm=inp["use_qk_l2norm"], scale=inp["scale"])
    args1 = (ctypes.byref(p1), P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), None, P(d["h0"]),
             P(o1), P(ht1), P(ws1), ctypes.c_size_t(ws1.numel()), sp)

    def seg_step():
        st = L.gdr_chunk_fwd_segmented(*args)
        if st != 0:
            raise RuntimeError(L.gdr_status_string(st).decode())

    def one_step():
        st = L.gdr_chunk_fwd(*args1)
        if st != 0:
            raise RuntimeError(L.gdr_status_string(st).decode())

    stream = torch.cuda.current_stream(dev)
    ms = timed_calls(seg_step, warmup, steps, stream)["median_ms"]
    ms1 = timed_calls(one_step, warmup, steps, stream)["median_ms"]
    return {"workload": w.name, "pass": f"forward, one sequence as {R} segments (segment hand-off on one GPU)",
            "B": 1, "T": T, "H": w.H, "HV": w.HV, "K": w.K, "V": w.V, "chunk_size": w.chunk_size, "segments": R,
            "tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms, "single_pass_ms_per_step": ms1,
            "parity": parity}


def measure_simple_gla(gdr, w, steps, warmup):
    """The simple GLA forward (gdr_simple_gla_fwd) on workload ``w``'s inputs
    (beta unused): parity of the first sequence's first 512 tokens on two
    heads against the per-token oracle, then the timed call."""
    import torch
    from oracle import recurrent
    from oracle.metrics import err_ratio
    dev = torch.device("cuda:0")
    inp = workloads_inputs(w)
    d = to_dev(inp, dev, ("q", "k", "v", "g", "h0", "cu_seqlens"))
    kw = dict(scale=inp["scale"], chunk_size=inp["chunk_size"], cu_seqlens=d["cu_seqlens"], initial_state=d["h0"],
              use_qk_l2norm_in_kernel=inp["use_qk_l2norm"])
    o, ht = gdr.simple_gla_fwd(d["q"], d["k"], d["v"], d["g"], **kw)
    torch.cuda.synchronize()
    hs = [0, w.HV - 1]
    sub = {n: inp[n][:1, :512][:, :, hs].contiguous() for n in ("q", "k", "v", "g")}
    ro, _ = recurrent.simple_gla_fwd(sub["q"], sub["k"], sub["v"], sub["g"], scale=inp["scale"],
                                     h0=inp["h0"][:1, hs], use_qk_l2norm=inp["use_qk_l2norm"])
    tol = 5e-3 if w.dtype == "bf16" else 1e-4
    parity = {"o (sequence 0, first 512 tokens, 2 heads)": err_ratio(o[:1, :512][:, :, hs].cpu(), ro), "tol": tol}
    print(f"parity gate ({w.name}, simple GLA): " + ", ".join(f"{k}={v:.2e}" for k, v in parity.items()),
          file=sys.stderr, flush=True)
    if not all(v <= tol for k, v in parity.items() if k != "tol"):
        print("parity check failed: refusing to report throughput", file=sys.stderr)
        sys.exit(1)
    L = gdr.lib()
    p = gdr.make_problem(d["q"], d["v"], d["g"], chunk_size=inp["chunk_size"], cu_seqlens=d["cu_seqlens"],
                         use_qk_l2norm=inp["use_qk_l2norm"], scale=inp["scale"])
    lay = gdr.fwd_layout(p)
    ws = torch.empty(lay.total, dtype=torch.uint8, device=dev)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = (ctypes.byref(p), P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["cu_seqlens"]), P(d["h0"]), P(o),
            P(ht), P(ws), ctypes.c_size_t(ws.numel()), sp)

    def step():
        st = L.gdr_simple_gla_fwd(*args)
        if st != 0:
            raise RuntimeError(L.gdr_status_string(st).decode())

    ms = timed_calls(step, warmup, steps, torch.cuda.current_stream(dev))["median_ms"]
    tokens = inp["B"] * inp["T"]
    return {"workload": w.name, "pass": "simple GLA forward (same chunked stages, w = 0, u = v)",
            "tokens_per_s": tokens / (ms * 1e-3), "ms_per_step": ms, "parity": parity}


def config_record(w, inp, rec):
    """One workload's record: its dimensions, then the measured fields."""
    return {"workload": w.name,
            "pass": ("forward+backward" if w.backward else
                     "token-by-token forward (one decoding step)" if w.T == 1 else "forward"),
            "B": inp["B"], "T": inp["T"], "N": inp["N"], "H": w.H, "HV": w.HV, "K": w.K, "V": w.V,
            "chunk_size": w.chunk_size, "dtype": w.dtype,
            "gate": "per-channel" if w.per_channel_gate else "scalar",
            "tokens_per_s": rec["value"], "ms_per_step": rec["ms_per_step"],
            **{k: v for k, v in rec.items() if k not in ("value", "ms_per_step")}}


def workloads_inputs(w):
    import workloads
    return workloads.make_inputs(w)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="gdn_dense_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the long-sequence forward + backward record of the default run")
    ap.add_argument("--breakdown", action="store_true", help="per-stage times on stderr")
    ap.add_argument("--segments", type=int, default=0, metavar="R",
                    help="only time the workload's first sequence as R segments (segment hand-off) "
                         "beside its single pass, print that record and exit")
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
    if args.segments:
        print(json.dumps(measure_segmented(gdr, w, args.segments, args.steps, args.warmup)))
        return
    if w.T == 1:
        rec, inp = measure_decode(gdr, w, args.steps, args.warmup)
    else:
        rec, inp = measure(gdr, w, args.steps, args.warmup, args.breakdown, w.name)
    line = {
        "metric": "tokens/sec and % HBM/MFMA roofline, chunk GDN fwd (+bwd) on 1 MI355X",
        "value": rec["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) q/k/v, logsigmoid gates, sigmoid beta)",
        "config": {"workload": w.name, "B": inp["B"], "T": inp["T"], "H": w.H, "HV": w.HV, "K": w.K,
                   "V": w.V, "chunk_size": w.chunk_size,
                   "pass": ("forward+backward" if w.backward else
                            "token-by-token forward (one decoding step)" if w.T == 1 else "forward"),
                   "gate": "per-channel" if w.per_channel_gate else "scalar",
                   "l2norm_in_kernel": w.l2norm_in_kernel, "parallelism": "single GPU"},
    }
    line.update({k: v for k, v in rec.items() if k not in ("value", "ms_per_step", "tokens")})
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp)
    del inp
    if not w.backward and not args.no_backward and w.T > 1 and not w.per_channel_gate:
        line["simple_gla"] = measure_simple_gla(gdr, w, args.steps, args.warmup)
    if not args.no_backward and w.name == "gdn_dense_bf16":
        # every other configuration of the operator: forward records for the
        # tiny fp32, varlen GVA and per-channel (KDA) workloads, the long
        # sequence's forward + backward step, and a forward + backward step on
        # the KDA workload's shape (median of 50 event-timed calls after 10
        # warm-ups each, the workload's own parity gate first)
        line["configs"] = {}
        for name in ("tiny_fp32", "varlen_gva_bf16", "kda_bf16", "long_bf16", "kda_train_bf16"):
            torch.cuda.empty_cache()
            wc = workloads.CONFIGS[name]
            crec, cinp = measure(gdr, wc, 50, 10, args.breakdown, wc.name)
            line["configs"][name] = config_record(wc, cinp, crec)
            if wc.backward and not args.no_cpu_baseline:
                line["configs"][name]["cpu_baseline"] = cpu_baseline_bwd(wc, cinp)
            del cinp
        torch.cuda.empty_cache()
        wb = workloads.CONFIGS["long_bf16"]
        line["segmented"] = measure_segmented(gdr, wb, 8, 20, 5)
        torch.cuda.empty_cache()
        wd = workloads.CONFIGS["decode_gva_bf16"]
        drec, dinp = measure_decode(gdr, wd, 50, 10)
        line["decode"] = config_record(wd, dinp, drec)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
