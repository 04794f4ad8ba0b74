// Host side of the C ABI declared in include/gdr.h: argument checks, the
// workspace plan and the launch sequence of the forward stages.  Nothing here
// allocates, frees or synchronises; every launch goes to the caller's stream.
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "gdr_internal.h"

namespace gdr {

bool bwd_shape_ok(const gdr_problem& p) {
  if (p.K != 32 && p.K != 64 && p.K != 128) return false;
  if (p.gate_per_channel)
    return p.chunk_size == 32 && bwd_scan_pc_fits(p.dtype, (int)p.K) && bwd_pc_fits(p.dtype, (int)p.K);
  return bwd_scan_fits(p.dtype, p.chunk_size, (int)p.K) && bwd_fused_fits(p.dtype, p.chunk_size, (int)p.K);
}

int64_t nt_max(const gdr_problem& p) {
  const int64_t C = p.chunk_size;
  if (p.T <= 0 || C <= 0) return 0;
  if (p.N == p.B && p.B > 1) return p.B * ((p.T + C - 1) / C);
  // dense B = 1 and varlen use the same bound; for a single dense row it is exact
  return (p.N == 1) ? (p.T + C - 1) / C : p.T / C + p.N;
}

}  // namespace gdr

using gdr::Args;

namespace {

// ---- stage timing (measurement only, off by default; gdr_stage_timing): the
// full forward and backward record a HIP event on their stream before their
// first launch and after each stage, per host thread, into events created on
// first use and kept; gdr_stage_times reads every stage interval recorded
// since timing was (re)enabled.  names[i] is the stage that ends at event i,
// or NULL where event i starts a call.
constexpr size_t kMaxTimedEvents = 8192;
struct StageTimer {
  bool on = false;
  std::vector<hipEvent_t> ev;
  std::vector<const char*> names;
  size_t used = 0;
};
thread_local StageTimer t_timer;

bool timer_record(hipStream_t s, const char* name) {
  if (t_timer.used == kMaxTimedEvents) return false;
  if (t_timer.used == t_timer.ev.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return false;
    t_timer.ev.push_back(e);
    t_timer.names.push_back(nullptr);
  }
  if (hipEventRecord(t_timer.ev[t_timer.used], s) != hipSuccess) return false;
  t_timer.names[t_timer.used++] = name;
  return true;
}
void timer_start(hipStream_t s) {
  if (t_timer.on) timer_record(s, nullptr);
}
// the stage that ends here (after a successful launch)
void timer_mark(hipError_t e, const char* name, hipStream_t s) {
  if (t_timer.on && e == hipSuccess && t_timer.used > 0) timer_record(s, name);
}

bool head_dim_ok(int64_t d) { return d == 32 || d == 64 || d == 128 || d == 256; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x) { return (x + 255) & ~size_t(255); }

size_t elem_size(const gdr_problem& p) { return p.dtype == GDR_BF16 ? 2 : 4; }

// Checks shared by the chunked and the token-by-token paths (chunk_size is
// not read here).
// Head dims the full forward / backward take by zero padding: any size up to
// 256 runs as the next instantiated one.
int64_t pad_dim(int64_t d) { return d <= 32 ? 32 : d <= 64 ? 64 : d <= 128 ? 128 : 256; }
bool pad_dims_ok(int64_t d) { return d >= 1 && d <= 256; }
bool needs_pad(const gdr_problem& p) { return !head_dim_ok(p.K) || !head_dim_ok(p.V); }
gdr_problem padded_problem(const gdr_problem& p) {
  gdr_problem r = p;
  r.K = pad_dim(p.K);
  r.V = pad_dim(p.V);
  return r;
}

gdr_status check_dims(const gdr_problem* p, bool varlen, bool allow_pad = false) {
  if (p == nullptr) return GDR_ERR_NULL_ARG;
  if (p->dtype != GDR_BF16 && p->dtype != GDR_FP32) return GDR_ERR_DTYPE;
  if (p->N < 1) return varlen ? GDR_ERR_VARLEN : GDR_ERR_SHAPE;
  if (p->B < 1 || p->T < 0 || p->H < 1 || p->HV < 1) return GDR_ERR_SHAPE;
  if (p->HV % p->H != 0) return GDR_ERR_SHAPE;
  if (allow_pad ? !(pad_dims_ok(p->K) && pad_dims_ok(p->V)) : !(head_dim_ok(p->K) && head_dim_ok(p->V)))
    return GDR_ERR_SHAPE;
  if (!std::isfinite(p->scale)) return GDR_ERR_SHAPE;
  if (varlen) {
    if (p->B != 1) return GDR_ERR_VARLEN;
  } else if (p->N != p->B) {
    return GDR_ERR_VARLEN;
  }
  return GDR_OK;
}

gdr_status check(const gdr_problem* p, bool varlen, bool allow_pad = false) {
  if (p == nullptr) return GDR_ERR_NULL_ARG;
  if (p->chunk_size != 32 && p->chunk_size != 64) return GDR_ERR_CHUNK_SIZE;
  const gdr_status st = check_dims(p, varlen, allow_pad);
  if (st != GDR_OK) return st;
  // fp32 with a per-channel gate at K = 256, chunk 64 does not fit one workgroup's LDS
  if (p->dtype == GDR_FP32 && p->gate_per_channel && pad_dim(p->K) == 256 && p->chunk_size == 64)
    return GDR_ERR_SHAPE;
  // token indices are int32 in the chunk table
  if (p->B * p->T >= (int64_t(1) << 31)) return GDR_ERR_SHAPE;
  return GDR_OK;
}

gdr::Args make_args(const gdr_problem& p) {
  Args a;
  std::memset(&a, 0, sizeof(a));
  a.B = p.B;
  a.T = p.T;
  a.H = p.H;
  a.HV = p.HV;
  a.K = p.K;
  a.V = p.V;
  a.N = p.N;
  a.NTmax = gdr::nt_max(p);
  a.C = p.chunk_size;
  a.per_channel = p.gate_per_channel ? 1 : 0;
  a.l2norm = p.use_qk_l2norm ? 1 : 0;
  a.beta_logits = p.beta_logits ? 1 : 0;
  a.dtype = p.dtype;
  a.scale = p.scale;
  return a;
}

// pc_regions: with a per-channel gate, reserve the WY stage's gated keys and
// decay for the warp-specialised scan (the backward keeps its own; the
// segmented forward runs the other per-channel scan).  pc_fused: the
// per-channel fused K1 + K2 and fused scan + output run, so Tm, h and v_new
// get no bytes and the aqk and gated-query regions do.
gdr_fwd_layout layout_of(const gdr_problem& p, bool pc_regions = true, bool pc_fused = false) {
  gdr_fwd_layout l;
  const int64_t nt = gdr::nt_max(p);
  const size_t es = elem_size(p);
  const size_t C = (size_t)p.chunk_size, HV = (size_t)p.HV, K = (size_t)p.K, V = (size_t)p.V;
  size_t off = 0;
  l.nt_max = nt;
  l.chunk_idx = off;
  off = round_up(off + (size_t)nt * 4 * sizeof(int32_t));
  l.chunk_off = off;
  off = round_up(off + ((size_t)p.N + 1) * sizeof(int32_t));
  l.seq_order = off;
  off = round_up(off + (size_t)p.N * sizeof(int32_t));
  l.Tm = off;
  off = round_up(off + (pc_fused ? 0 : (size_t)nt * HV * C * C * es));
  l.w = off;
  off = round_up(off + (size_t)nt * HV * C * K * es);
  l.u = off;   // fp32 from the separate WY stage, input dtype from the fused stages
  off = round_up(off + (size_t)nt * HV * V * C * (pc_fused ? es : sizeof(float)));
  l.h = off;
  off = round_up(off + (pc_fused ? 0 : (size_t)nt * HV * V * K * es));
  l.v_new = off;
  off = round_up(off + (pc_fused ? 0 : (size_t)nt * HV * V * C * es));
  l.kscale = off;
  off = round_up(off + (p.gate_per_channel ? 0 : (size_t)nt * HV * gdr::kscale_pitch(C) * sizeof(float)));
  const bool pcs = pc_regions && p.gate_per_channel && gdr::fwd_pc_scan_fits(p.dtype, (int)C, (int)K);
  // the fused per-channel K1 + K2 and scan + output (the kept-states forward
  // runs them too, storing h and v_new as well)
  const Args pa = make_args(p);
  const bool pco = pc_fused || (pcs && gdr::kkt_wy_pc_supported(pa) && gdr::fwd_h_o_pc_supported(pa));
  l.kt = off;
  off = round_up(off + (pcs || pc_fused ? (size_t)nt * HV * C * K * es : 0));
  l.dl = off;
  off = round_up(off + (pcs || pc_fused ? (size_t)nt * HV * K * sizeof(float) : 0));
  l.aqk = off;
  off = round_up(off + (pco ? (size_t)nt * HV * C * C * sizeof(float) : 0));
  l.qgs = off;
  off = round_up(off + (pco ? (size_t)nt * HV * gdr::kQgsTiles * C * K * es : 0));
  l.total = off;
  return l;
}

// The regions the fused path touches (chunk tables, w, u in the input dtype,
// kscale): Tm, h and v_new get no bytes (their offsets are the next region's).
gdr_fwd_layout fused_layout_of(const gdr_problem& p) {
  gdr_fwd_layout l;
  const int64_t nt = gdr::nt_max(p);
  const size_t es = elem_size(p);
  const size_t C = (size_t)p.chunk_size, HV = (size_t)p.HV, K = (size_t)p.K, V = (size_t)p.V;
  size_t off = 0;
  l.nt_max = nt;
  l.chunk_idx = off;
  off = round_up(off + (size_t)nt * 4 * sizeof(int32_t));
  l.chunk_off = off;
  off = round_up(off + ((size_t)p.N + 1) * sizeof(int32_t));
  l.seq_order = off;
  off = round_up(off + (size_t)p.N * sizeof(int32_t));
  l.Tm = off;
  l.w = off;
  off = round_up(off + (size_t)nt * HV * C * K * es);
  l.u = off;
  off = round_up(off + (size_t)nt * HV * V * C * es);
  l.h = off;
  l.v_new = off;
  l.kscale = off;
  off = round_up(off + (size_t)nt * HV * gdr::kscale_pitch(C) * sizeof(float));
  l.kt = off;
  l.dl = off;
  l.aqk = off;
  l.qgs = off;
  l.total = off;
  return l;
}

// Which fused forward gdr_chunk_fwd runs for the (padded) problem: 1 = fused
// K1 + K2 and fused scan + output (scalar gate), 2 = the per-channel fused
// K1 + K2 and fused scan + output, 0 = the separate stages.
int fused_kind(const gdr_problem& pp) {
  if (pp.keep_states) return 0;
  const Args a = make_args(pp);
  if (gdr::fwd_h_o_preferred(a)) return 1;
  if (gdr::fwd_h_o_pc_preferred(a) && gdr::kkt_wy_pc_supported(a)) return 2;
  return 0;
}

// The layout gdr_chunk_fwd works in: the compact one when the fused stages run
// (no keep_states and a shape with a fused scan + output stage), else the
// full one with Tm, h and v_new.
gdr_fwd_layout fwd_layout_for(const gdr_problem& pp) {
  switch (fused_kind(pp)) {
    case 1: return fused_layout_of(pp);
    case 2: return layout_of(pp, true, true);
  }
  return layout_of(pp);
}

gdr_status hip_status(hipError_t e) { return e == hipSuccess ? GDR_OK : GDR_ERR_HIP; }

gdr_bwd_layout bwd_layout_of(const gdr_problem& p) {
  gdr_bwd_layout l;
  l.fwd = layout_of(p, false);
  l.chunk_size = p.chunk_size;
  const int64_t nt = l.fwd.nt_max;
  const size_t es = elem_size(p);
  const size_t C = (size_t)p.chunk_size, HV = (size_t)p.HV, K = (size_t)p.K, V = (size_t)p.V;
  size_t off = l.fwd.total;
  l.de_local = off;
  off = round_up(off + (size_t)nt * HV * V * C * es);
  l.qscale = off;
  off = round_up(off + (size_t)nt * HV * C * sizeof(float));
  l.dh = off;  // fp32
  off = round_up(off + (size_t)nt * HV * V * K * sizeof(float));
  // per-channel gate: the chunk's gated rows and decay for the reverse scan
  const size_t pc = p.gate_per_channel ? 1 : 0;
  l.kt = off;
  off = round_up(off + pc * (size_t)nt * HV * C * K * es);
  l.qg = off;
  off = round_up(off + pc * (size_t)nt * HV * C * K * es);
  l.dl = off;
  off = round_up(off + pc * (size_t)nt * HV * K * sizeof(float));
  l.total = off;
  return l;
}

gdr_seg_layout seg_layout_of(const gdr_problem& p) {
  gdr_seg_layout l;
  l.fwd = layout_of(p, false);
  const int64_t nt = l.fwd.nt_max;
  const size_t es = elem_size(p);
  const size_t C = (size_t)p.chunk_size, HV = (size_t)p.HV, K = (size_t)p.K, V = (size_t)p.V, N = (size_t)p.N;
  size_t off = l.fwd.total;
  l.u_zero = off;   // read as the WY stage's u (fp32 with a per-channel gate)
  off = round_up(off + (size_t)nt * HV * K * C * sizeof(float));
  l.h_tr = off;
  off = round_up(off + (size_t)nt * HV * K * K * es);
  l.v_tr = off;
  off = round_up(off + (size_t)nt * HV * K * C * es);
  l.eye = off;
  off = round_up(off + N * HV * K * K * sizeof(float));
  l.s_ext = off;
  off = round_up(off + N * HV * K * V * sizeof(float));
  l.trans = off;
  off = round_up(off + N * HV * K * K * sizeof(float));
  l.s_in = off;
  off = round_up(off + (N + 1) * HV * K * V * sizeof(float));
  l.total = off;
  return l;
}

// The problem the full backward runs: padded head dims, and chunk 32 where the
// requested chunk 64 has no instantiation of the backward kernels (fp32 with
// K = 128).  The chunk form is exact at any chunk size, so the gradients are
// the same up to rounding; a saved-state backward (keep_states) cannot switch,
// because the forward's intermediates were chunked as requested.
gdr_problem bwd_problem(const gdr_problem& p) {
  gdr_problem r = padded_problem(p);
  if (!gdr::bwd_shape_ok(r) && r.chunk_size == 64 && !r.keep_states) {
    gdr_problem c32 = r;
    c32.chunk_size = 32;
    if (gdr::bwd_shape_ok(c32)) return c32;
  }
  return r;
}

gdr_status check_bwd(const gdr_problem* p, bool varlen, bool allow_pad = false) {
  const gdr_status st = check(p, varlen, allow_pad);
  if (st != GDR_OK) return st;
  return gdr::bwd_shape_ok(allow_pad ? bwd_problem(*p) : *p) ? GDR_OK : GDR_ERR_UNSUPPORTED;
}

// Padded copies of the inputs and outputs of a problem whose head dims are not
// instantiated, placed after the padded problem's own workspace (base).
struct PadLayout {
  size_t q, k, v, g, h0, o, ht, d_o, dht, dq, dk, dv, dh0, dg, total;
};

PadLayout pad_layout(const gdr_problem& p, size_t base, bool bwd) {
  PadLayout l;
  const gdr_problem pp = padded_problem(p);
  const size_t es = elem_size(p);
  const size_t BT = (size_t)(p.B * p.T), H = (size_t)p.H, HV = (size_t)p.HV, N = (size_t)p.N;
  const size_t Kp = (size_t)pp.K, Vp = (size_t)pp.V;
  size_t off = base;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes);
    return at;
  };
  l.q = take(BT * H * Kp * es);
  l.k = take(BT * H * Kp * es);
  l.v = take(BT * HV * Vp * es);
  l.g = take(p.gate_per_channel ? BT * HV * Kp * sizeof(float) : 0);
  l.h0 = take(N * HV * Kp * Vp * sizeof(float));
  l.o = take(bwd ? 0 : BT * HV * Vp * es);
  l.ht = take(bwd ? 0 : N * HV * Kp * Vp * sizeof(float));
  l.d_o = take(bwd ? BT * HV * Vp * es : 0);
  l.dht = take(bwd ? N * HV * Kp * Vp * sizeof(float) : 0);
  l.dq = take(bwd ? BT * H * Kp * es : 0);
  l.dk = take(bwd ? BT * H * Kp * es : 0);
  l.dv = take(bwd ? BT * HV * Vp * es : 0);
  l.dh0 = take(bwd ? N * HV * Kp * Vp * sizeof(float) : 0);
  l.dg = take(bwd && p.gate_per_channel ? BT * HV * Kp * sizeof(float) : 0);
  l.total = off;
  return l;
}

// K1 and K2 into Tm, w and u (fp32), and with a per-channel gate the scan's
// kt / dl when a.kt / a.dl are set: one fused stage (the scalar gate's
// kept-states fused K1 + K2, or the per-channel one where the shape has it),
// else the two stages.  The kept-states forward and the backward's recompute
// both come here, so they produce the same Tm, w and u.
hipError_t kkt_and_wy(const Args& a, hipError_t e, hipStream_t s) {
  if (!a.per_channel && a.u_f32 && !a.gla) {
    if (e == hipSuccess) e = gdr::launch_kkt_wy(a, s);
    timer_mark(e, "kkt_wy", s);
    return e;
  }
  if (a.per_channel && a.kt != nullptr && a.dl != nullptr && gdr::kkt_wy_pc_supported(a)) {
    if (e == hipSuccess) e = gdr::launch_kkt_wy_pc(a, s);
    timer_mark(e, "kkt_wy", s);
    return e;
  }
  if (e == hipSuccess) e = gdr::launch_kkt_solve(a, s);
  timer_mark(e, "kkt_solve", s);
  if (e == hipSuccess) e = gdr::launch_wy(a, s);
  timer_mark(e, "wy", s);
  return e;
}

// The forward's launch sequence for a problem with instantiated head dims;
// the intermediates go to the workspace at the offsets of l.
hipError_t fwd_run(const gdr_problem& p, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, const int32_t* cu_seqlens, const float* h0, void* o, float* ht, char* ws,
                   const gdr_fwd_layout& l, hipStream_t s) {
  Args a = make_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.cu = cu_seqlens;
  a.h0 = h0;
  a.chunk_idx = reinterpret_cast<int32_t*>(ws + l.chunk_idx);
  a.chunk_off = reinterpret_cast<int32_t*>(ws + l.chunk_off);
  a.seq_order = (a.cu != nullptr && a.N <= gdr::kMaxOrdered) ? reinterpret_cast<int32_t*>(ws + l.seq_order) : nullptr;
  a.Tm = ws + l.Tm;
  a.w = ws + l.w;
  a.u = ws + l.u;
  a.h = ws + l.h;
  a.v_new = ws + l.v_new;
  a.kscale = p.gate_per_channel ? nullptr : reinterpret_cast<float*>(ws + l.kscale);
  if (p.gate_per_channel && l.dl > l.kt) {
    // the WY stage writes the gated keys and decay the scan reads
    a.kt = ws + l.kt;
    a.dl = reinterpret_cast<float*>(ws + l.dl);
  }
  a.o = o;
  a.ht = ht;
  hipError_t e = hipSuccess;
  const int kind = fused_kind(p);
  if (kind == 2 && l.qgs > l.aqk) {
    // per-channel gate: the fused K1 + K2 also writes aqk and the gated query
    // pair, and the fused scan + output reads them (Tm, h and v_new stay on
    // chip; u in the input dtype, as in the scalar-gate fused stages)
    a.u_f32 = 0;
    a.Tm = nullptr;
    a.h = nullptr;
    a.v_new = nullptr;
    a.aqk = reinterpret_cast<float*>(ws + l.aqk);
    a.qgs = ws + l.qgs;
    e = gdr::launch_chunk_table(a, s);
    timer_mark(e, "chunk_table", s);
    if (e == hipSuccess) e = gdr::launch_kkt_wy_pc(a, s);
    timer_mark(e, "kkt_wy", s);
    if (e == hipSuccess) e = gdr::launch_fwd_h_o_pc(a, s);
    timer_mark(e, "fwd_h_o", s);
  } else if (kind == 1) {
    // fused K1 + K2 (Tm stays on chip) and fused scan + output (h and v_new
    // stay on chip); for a dense batch the first writes the chunk table too
    if (cu_seqlens == nullptr && a.NTmax > 0) {
      a.table_from_dims = 1;
    } else {
      e = gdr::launch_chunk_table(a, s);
      timer_mark(e, "chunk_table", s);
    }
    if (e == hipSuccess) e = gdr::launch_kkt_wy(a, s);
    timer_mark(e, "kkt_wy", s);
    a.table_from_dims = 0;
    if (e == hipSuccess) e = gdr::launch_fwd_h_o(a, s);
    timer_mark(e, "fwd_h_o", s);
  } else {
    a.u_f32 = 1;   // u in fp32 (what the backward reads)
    e = gdr::launch_chunk_table(a, s);
    timer_mark(e, "chunk_table", s);
    if (p.keep_states && !p.gate_per_channel && gdr::fwd_h_o_keep_supported(a)) {
      // kept states, scalar gate: the fused K1 + K2 writing Tm and an fp32 u,
      // and the fused scan + output storing h and v_new as well
      e = kkt_and_wy(a, e, s);
      if (e == hipSuccess) e = gdr::launch_fwd_h_o_keep(a, s);
      timer_mark(e, "fwd_h_o", s);
    } else if (p.keep_states && l.qgs > l.aqk && a.kt != nullptr && gdr::kkt_wy_pc_supported(a) &&
               gdr::fwd_h_o_pc_supported(a)) {
      // kept states, per-channel gate: the fused K1 + K2 writing Tm and the
      // output's operands, and the fused scan + output storing h and v_new
      a.aqk = reinterpret_cast<float*>(ws + l.aqk);
      a.qgs = ws + l.qgs;
      if (e == hipSuccess) e = gdr::launch_kkt_wy_pc(a, s);
      timer_mark(e, "kkt_wy", s);
      if (e == hipSuccess) e = gdr::launch_fwd_h_o_pc(a, s);
      timer_mark(e, "fwd_h_o", s);
    } else {
      e = kkt_and_wy(a, e, s);
      if (e == hipSuccess) e = gdr::launch_fwd_h(a, s);
      timer_mark(e, "fwd_h", s);
      if (e == hipSuccess) e = gdr::launch_fwd_o(a, s);
      timer_mark(e, "fwd_o", s);
    }
  }
  return e;
}

// The backward's launch sequence for a problem with instantiated head dims.
hipError_t bwd_run(const gdr_problem& p, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, const int32_t* cu_seqlens, const float* h0, const void* d_o, const float* dht,
                   void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0, char* ws,
                   const gdr_bwd_layout& l, hipStream_t s) {
  Args a = make_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.cu = cu_seqlens;
  a.h0 = h0;
  a.chunk_idx = reinterpret_cast<int32_t*>(ws + l.fwd.chunk_idx);
  a.chunk_off = reinterpret_cast<int32_t*>(ws + l.fwd.chunk_off);
  a.seq_order = (a.cu != nullptr && a.N <= gdr::kMaxOrdered) ? reinterpret_cast<int32_t*>(ws + l.fwd.seq_order) : nullptr;
  a.Tm = ws + l.fwd.Tm;
  a.w = ws + l.fwd.w;
  a.u = ws + l.fwd.u;
  a.h = ws + l.fwd.h;
  a.v_new = ws + l.fwd.v_new;
  a.kscale = reinterpret_cast<float*>(ws + l.fwd.kscale);
  a.ht = nullptr;
  a.d_o = d_o;
  a.dht = dht;
  a.de_local = ws + l.de_local;
  a.qscale = reinterpret_cast<float*>(ws + l.qscale);
  a.dh = ws + l.dh;
  a.dh0 = dh0;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dg;
  a.dbeta = dbeta;
  a.u_f32 = 1;   // u from the separate WY stage (recomputed here, or kept by the forward)
  if (p.gate_per_channel) {
    a.kscale = nullptr;
    a.qscale = nullptr;
    a.kt = ws + l.kt;
    a.qg = ws + l.qg;
    a.dl = reinterpret_cast<float*>(ws + l.dl);
  }
  hipError_t e = hipSuccess;
  if (!p.keep_states) {
    // recompute the forward's chunk tables, Tm, w, u, kscale, h and v_new
    e = gdr::launch_chunk_table(a, s);
    timer_mark(e, "chunk_table", s);
    e = kkt_and_wy(a, e, s);
    if (e == hipSuccess) e = gdr::launch_fwd_h(a, s);
    timer_mark(e, "fwd_h", s);
  }
  if (e == hipSuccess) e = gdr::launch_bwd_intra(a, s);
  timer_mark(e, "bwd_intra", s);
  if (e == hipSuccess) e = gdr::launch_bwd_dh(a, s);
  timer_mark(e, "bwd_dh", s);
  if (e == hipSuccess) e = p.gate_per_channel ? gdr::launch_bwd_dqkvg_pc(a, s) : gdr::launch_bwd_dqkvg(a, s);
  timer_mark(e, "bwd_dqkvg", s);
  return e;
}

// Argument checks of the full forward (everything but the workspace).
gdr_status check_fwd_args(const gdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const int32_t* cu_seqlens, const float* h0, const void* o,
                          const float* ht) {
  const gdr_status st = check(p, cu_seqlens != nullptr, true);
  if (st != GDR_OK) return st;
  if (p->T != 0 && (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr || o == nullptr))
    return GDR_ERR_NULL_ARG;
  const void* ptrs[] = {q, k, v, g, beta, cu_seqlens, h0, o, ht};
  for (const void* ptr : ptrs)
    if (ptr != nullptr && !aligned16(ptr)) return GDR_ERR_ALIGNMENT;
  return GDR_OK;
}

// ---- fixed scratch of the no-allocation forward (gdr_chunk_fwd_noalloc).
// One array per device, created with the code object and held until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels and copies get the per-device address that
// hipGetSymbolAddress returns, fetched once per device with that device
// current.
constexpr size_t kScratchBytes = GDR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device (looked up on the first call there).
gdr_status scratch_on_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return GDR_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return GDR_OK;
}

// The full forward on workspace `ws` laid out as `l` (the padded problem's
// layout; zero-padded copies of the inputs and outputs follow it when the head
// dims have no instantiation).
gdr_status chunk_fwd_run(const gdr_problem& p0, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int32_t* cu_seqlens, const float* h0, void* o, float* ht,
                         char* ws, const gdr_fwd_layout& l, hipStream_t s) {
  const gdr_problem* p = &p0;
  const gdr_problem pp = padded_problem(*p);
  timer_start(s);
  if (!needs_pad(*p)) return hip_status(fwd_run(*p, q, k, v, g, beta, cu_seqlens, h0, o, ht, ws, l, s));
  const PadLayout pl = pad_layout(*p, l.total, false);
  // head dims without an instantiation: zero-padded copies in, padded problem, copies out
  const int es = (int)elem_size(*p);
  const int64_t BT = p->B * p->T, H = p->H, HV = p->HV, N = p->N, K = p->K, V = p->V, Kp = pp.K, Vp = pp.V;
  hipError_t e = gdr::launch_pad(q, ws + pl.q, BT * H, 1, K, 1, Kp, es, s);
  if (e == hipSuccess) e = gdr::launch_pad(k, ws + pl.k, BT * H, 1, K, 1, Kp, es, s);
  if (e == hipSuccess) e = gdr::launch_pad(v, ws + pl.v, BT * HV, 1, V, 1, Vp, es, s);
  if (e == hipSuccess && p->gate_per_channel) e = gdr::launch_pad(g, ws + pl.g, BT * HV, 1, K, 1, Kp, 4, s);
  if (e == hipSuccess && h0 != nullptr) e = gdr::launch_pad(h0, ws + pl.h0, N * HV, K, V, Kp, Vp, 4, s);
  timer_mark(e, "pad", s);
  if (e == hipSuccess)
    e = fwd_run(pp, ws + pl.q, ws + pl.k, ws + pl.v,
                p->gate_per_channel ? reinterpret_cast<const float*>(ws + pl.g) : g, beta, cu_seqlens,
                h0 != nullptr ? reinterpret_cast<const float*>(ws + pl.h0) : nullptr, ws + pl.o,
                ht != nullptr ? reinterpret_cast<float*>(ws + pl.ht) : nullptr, ws, l, s);
  if (e == hipSuccess) e = gdr::launch_unpad(ws + pl.o, o, BT * HV, 1, V, 1, Vp, es, s);
  if (e == hipSuccess && ht != nullptr) e = gdr::launch_unpad(ws + pl.ht, ht, N * HV, K, V, Kp, Vp, 4, s);
  timer_mark(e, "unpad", s);
  return hip_status(e);
}


}  // namespace

extern "C" {

int gdr_abi_version(void) { return 6; }

gdr_status gdr_stage_timing(int enable) {
  t_timer.on = enable != 0;
  t_timer.used = 0;
  return GDR_OK;
}

int gdr_stage_times(const char** names, float* ms, int max_stages) {
  if (!t_timer.on || t_timer.used < 2 || names == nullptr || ms == nullptr) return 0;
  if (hipEventSynchronize(t_timer.ev[t_timer.used - 1]) != hipSuccess) return -1;
  int n = 0;
  for (size_t i = 1; i < t_timer.used && n < max_stages; ++i) {
    if (t_timer.names[i] == nullptr) continue;   // a call starts here
    float x = 0.f;
    if (hipEventElapsedTime(&x, t_timer.ev[i - 1], t_timer.ev[i]) != hipSuccess) return -1;
    names[n] = t_timer.names[i];
    ms[n++] = x;
  }
  return n;
}

const char* gdr_status_string(gdr_status s) {
  switch (s) {
    case GDR_OK: return "ok";
    case GDR_ERR_NULL_ARG: return "a required pointer is NULL";
    case GDR_ERR_CHUNK_SIZE: return "chunk_size must be either 32 or 64";
    case GDR_ERR_SHAPE:
      return "unsupported shape (dims < 1, HV % H != 0, K/V outside 1..256, or, for a single stage, "
             "K/V not in {32,64,128,256})";
    case GDR_ERR_VARLEN: return "cu_seqlens requires B == 1 and N >= 1; a dense batch requires N == B";
    case GDR_ERR_DTYPE: return "dtype must be GDR_BF16 or GDR_FP32";
    case GDR_ERR_ALIGNMENT: return "every pointer must be 16-byte aligned";
    case GDR_ERR_WORKSPACE: return "workspace missing or too small";
    case GDR_ERR_HIP: return "HIP launch failed";
    case GDR_ERR_CU_SEQLENS: return "cu_seqlens must start at 0, be non-decreasing and end at T";
    case GDR_ERR_SCRATCH_LIMIT:
      return "gdr_chunk_fwd_noalloc: the problem needs more than the fixed scratch of GDR_NOALLOC_SCRATCH_BYTES "
             "(use gdr_chunk_fwd with a workspace)";
    case GDR_ERR_UNSUPPORTED:
      return "backward supports K in {32, 64, 128} (a per-channel gate, and fp32 with K = 128, run at chunk_size "
             "32, so a saved-state backward there needs a chunk_size 32 forward; the per-stage backward entry "
             "points take a scalar gate only)";
  }
  return "unknown status";
}

gdr_status gdr_check_problem(const gdr_problem* p) {
  if (p == nullptr) return GDR_ERR_NULL_ARG;
  return check(p, p->N != p->B, true);
}

gdr_status gdr_validate_cu_seqlens(const int32_t* cu, int64_t N, int64_t T) {
  if (cu == nullptr) return GDR_ERR_NULL_ARG;
  if (N < 1 || cu[0] != 0 || cu[N] != T) return GDR_ERR_CU_SEQLENS;
  for (int64_t i = 0; i < N; ++i)
    if (cu[i + 1] < cu[i]) return GDR_ERR_CU_SEQLENS;
  return GDR_OK;
}

gdr_status gdr_fwd_workspace_layout(const gdr_problem* p, gdr_fwd_layout* out) {
  if (p == nullptr || out == nullptr) return GDR_ERR_NULL_ARG;
  const gdr_status st = check(p, p->N != p->B, true);
  if (st != GDR_OK) return st;
  *out = fwd_layout_for(padded_problem(*p));
  if (needs_pad(*p)) out->total = pad_layout(*p, out->total, false).total;
  return GDR_OK;
}

gdr_status gdr_fwd_workspace_bytes(const gdr_problem* p, size_t* bytes) {
  gdr_fwd_layout l;
  const gdr_status st = gdr_fwd_workspace_layout(p, &l);
  if (st != GDR_OK) return st;
  if (bytes == nullptr) return GDR_ERR_NULL_ARG;
  *bytes = l.total;
  return GDR_OK;
}

gdr_status gdr_chunk_fwd(const gdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int32_t* cu_seqlens, const float* h0, void* o, float* ht,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const gdr_status st = check_fwd_args(p, q, k, v, g, beta, cu_seqlens, h0, o, ht);
  if (st != GDR_OK) return st;
  if (workspace != nullptr && !aligned16(workspace)) return GDR_ERR_ALIGNMENT;
  const gdr_problem pp = padded_problem(*p);
  const gdr_fwd_layout l = fwd_layout_for(pp);
  const size_t need = needs_pad(*p) ? pad_layout(*p, l.total, false).total : l.total;
  if (workspace == nullptr || workspace_bytes < need) return GDR_ERR_WORKSPACE;
  return chunk_fwd_run(*p, q, k, v, g, beta, cu_seqlens, h0, o, ht, static_cast<char*>(workspace), l,
                       static_cast<hipStream_t>(stream));
}

gdr_status gdr_chunk_fwd_noalloc(const gdr_problem* p, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const int32_t* cu_seqlens, const float* h0,
                                 void* o, float* ht, void* stream) {
  const gdr_status st = check_fwd_args(p, q, k, v, g, beta, cu_seqlens, h0, o, ht);
  if (st != GDR_OK) return st;
  // the fused path touches only the chunk tables, w, u and kscale
  const gdr_problem pp = padded_problem(*p);
  const gdr_fwd_layout l = fwd_layout_for(pp);
  const size_t need = needs_pad(*p) ? pad_layout(*p, l.total, false).total : l.total;
  if (need > kScratchBytes) return GDR_ERR_SCRATCH_LIMIT;
  char* ws = nullptr;
  const gdr_status sst = scratch_on_current_device(&ws);
  if (sst != GDR_OK) return sst;
  return chunk_fwd_run(*p, q, k, v, g, beta, cu_seqlens, h0, o, ht, ws, l, static_cast<hipStream_t>(stream));
}

gdr_status gdr_chunk_table(const gdr_problem* p, const int32_t* cu_seqlens, int32_t* chunk_idx,
                           int32_t* chunk_off, void* stream) {
  gdr_status st = check(p, cu_seqlens != nullptr);
  if (st != GDR_OK) return st;
  if (chunk_off == nullptr || (gdr::nt_max(*p) > 0 && chunk_idx == nullptr)) return GDR_ERR_NULL_ARG;
  if (!aligned16(chunk_idx) || !aligned16(chunk_off) || !aligned16(cu_seqlens)) return GDR_ERR_ALIGNMENT;
  Args a = make_args(*p);
  a.cu = cu_seqlens;
  a.chunk_idx = chunk_idx;
  a.chunk_off = chunk_off;
  return hip_status(gdr::launch_chunk_table(a, static_cast<hipStream_t>(stream)));
}

namespace {
gdr_status stage_common(const gdr_problem* p, std::initializer_list<const void*> ptrs) {
  gdr_status st = check(p, p ? p->N != p->B : false);
  if (st != GDR_OK) return st;
  for (const void* ptr : ptrs) {
    if (ptr == nullptr) return GDR_ERR_NULL_ARG;
    if (!aligned16(ptr)) return GDR_ERR_ALIGNMENT;
  }
  return GDR_OK;
}
}  // namespace

gdr_status gdr_fwd_kkt_solve(const gdr_problem* p, const void* k, const float* g, const float* beta,
                             const int32_t* chunk_idx, const int32_t* chunk_off, void* Tm, float* kscale,
                             void* stream) {
  gdr_status st = stage_common(p, {k, g, beta, chunk_idx, chunk_off, Tm});
  if (st != GDR_OK) return st;
  if (!p->gate_per_channel && kscale == nullptr) return GDR_ERR_NULL_ARG;
  if (kscale != nullptr && !aligned16(kscale)) return GDR_ERR_ALIGNMENT;
  Args a = make_args(*p);
  a.k = k;
  a.g = g;
  a.beta = beta;
  a.chunk_idx = const_cast<int32_t*>(chunk_idx);
  a.chunk_off = const_cast<int32_t*>(chunk_off);
  a.Tm = Tm;
  a.kscale = p->gate_per_channel ? nullptr : kscale;
  return hip_status(gdr::launch_kkt_solve(a, static_cast<hipStream_t>(stream)));
}

gdr_status gdr_fwd_wy(const gdr_problem* p, const void* k, const void* v, const float* g, const float* beta,
                      const int32_t* chunk_idx, const int32_t* chunk_off, const void* Tm, void* w, void* u,
                      void* stream) {
  gdr_status st = stage_common(p, {k, v, g, beta, chunk_idx, chunk_off, Tm, w, u});
  if (st != GDR_OK) return st;
  Args a = make_args(*p);
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.chunk_idx = const_cast<int32_t*>(chunk_idx);
  a.chunk_off = const_cast<int32_t*>(chunk_off);
  a.Tm = const_cast<void*>(Tm);
  a.w = w;
  a.u = u;
  return hip_status(gdr::launch_wy(a, static_cast<hipStream_t>(stream)));
}

gdr_status gdr_fwd_kkt_wy(const gdr_problem* p, const void* k, const void* v, const float* g, const float* beta,
                          const int32_t* chunk_idx, const int32_t* chunk_off, void* w, void* u, float* kscale,
                          void* stream) {
  gdr_status st = stage_common(p, {k, v, g, beta, chunk_idx, chunk_off, w, u, kscale});
  if (st != GDR_OK) return st;
  if (p->gate_per_channel) return GDR_ERR_UNSUPPORTED;
  Args a = make_args(*p);
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.chunk_idx = const_cast<int32_t*>(chunk_idx);
  a.chunk_off = const_cast<int32_t*>(chunk_off);
  a.w = w;
  a.u = u;
  a.kscale = kscale;
  return hip_status(gdr::launch_kkt_wy(a, static_cast<hipStream_t>(stream)));
}

gdr_status gdr_fwd_h(const gdr_problem* p, const void* k, const void* w, const void* u, const float* g,
                     const float* kscale, const int32_t* chunk_idx, const int32_t* chunk_off, const float* h0,
                     void* h, void* v_new, float* ht, void* stream) {
  gdr_status st = stage_common(p, {k, w, u, chunk_idx, chunk_off, h, v_new});
  if (st != GDR_OK) return st;
  if (p->gate_per_channel ? g == nullptr : kscale == nullptr) return GDR_ERR_NULL_ARG;
  if ((g && !aligned16(g)) || (kscale && !aligned16(kscale))) return GDR_ERR_ALIGNMENT;
  if ((h0 && !aligned16(h0)) || (ht && !aligned16(ht))) return GDR_ERR_ALIGNMENT;
  Args a = make_args(*p);
  a.k = k;
  a.w = const_cast<void*>(w);
  a.u = const_cast<void*>(u);
  a.g = g;
  a.kscale = const_cast<float*>(kscale);
  a.chunk_idx = const_cast<int32_t*>(chunk_idx);
  a.chunk_off = const_cast<int32_t*>(chunk_off);
  a.h0 = h0;
  a.h = h;
  a.v_new = v_new;
  a.ht = ht;
  a.u_f32 = 1;   // u as gdr_fwd_wy writes it
  return hip_status(gdr::launch_fwd_h(a, static_cast<hipStream_t>(stream)));
}

int gdr_chunk_fwd_fused(const gdr_problem* p) {
  if (check(p, p ? p->N != p->B : false, true) != GDR_OK) return 0;
  return fused_kind(padded_problem(*p));
}

int gdr_fwd_h_o_supported(const gdr_problem* p) {
  if (check(p, p ? p->N != p->B : false) != GDR_OK) return 0;
  return gdr::fwd_h_o_supported(make_args(*p)) ? 1 : 0;
}

gdr_status gdr_fwd_h_o(const gdr_problem* p, const void* q, const void* k, const void* w, const void* u,
                       const float* g, const float* kscale, const int32_t* chunk_idx, const int32_t* chunk_off,
                       const float* h0, void* o, float* ht, void* stream) {
  gdr_status st = stage_common(p, {q, k, w, u, g, kscale, chunk_idx, chunk_off, o});
  if (st != GDR_OK) return st;
  if ((h0 && !aligned16(h0)) || (ht && !aligned16(ht))) return GDR_ERR_ALIGNMENT;
  Args a = make_args(*p);
  if (!gdr::fwd_h_o_supported(a)) return GDR_ERR_UNSUPPORTED;
  a.q = q;
  a.k = k;
  a.w = const_cast<void*>(w);
  a.u = const_cast<void*>(u);
  a.g = g;
  a.kscale = const_cast<float*>(kscale);
  a.chunk_idx = const_cast<int32_t*>(chunk_idx);
  a.chunk_off = const_cast<int32_t*>(chunk_off);
  a.h0 = h0;
  a.o = o;
  a.ht = ht;
  return hip_status(gdr::launch_fwd_h_o(a, static_cast<hipStream_t>(stream)));
}

gdr_status gdr_fwd_o(const gdr_problem* p, const void* q, const void* k, const void* v_new, const void* h,
                     const float* g, const int32_t* chunk_idx, const int32_t* chunk_off, void* o, void* stream) {
  gdr_status st = stage_common(p, {q, k, v_new, h, g, chunk_idx, chunk_off, o});
  if (st != GDR_OK) return st;
  Args a = make_args(*p);
  a.q = q;
  a.k = k;
  a.v_new = const_cast<void*>(v_new);
  a.h = const_cast<void*>(h);
  a.g = g;
  a.chunk_idx = const_cast<int32_t*>(chunk_idx);
  a.chunk_off = const_cast<int32_t*>(chunk_off);
  a.o = o;
  return hip_status(gdr::launch_fwd_o(a, static_cast<hipStream_t>(stream)));
}


gdr_status gdr_fused_recurrent_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                                   const float* g, const float* beta, const int32_t* cu_seqlens,
                                   const float* h0, void* o, float* ht, void* stream) {
  const gdr_status st = check_dims(p, cu_seqlens != nullptr);
  if (st != GDR_OK) return st;
  if (p->T > 0 && (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr || o == nullptr))
    return GDR_ERR_NULL_ARG;
  const void* ptrs[] = {q, k, v, g, beta, cu_seqlens, h0, o, ht};
  for (const void* ptr : ptrs)
    if (ptr != nullptr && !aligned16(ptr)) return GDR_ERR_ALIGNMENT;
  if (p->T == 0 && ht == nullptr) return GDR_OK;
  Args a = make_args(*p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.cu = cu_seqlens;
  a.h0 = h0;
  a.o = o;
  a.ht = ht;
  return hip_status(gdr::launch_recurrent(a, static_cast<hipStream_t>(stream)));
}

gdr_status gdr_simple_gla_fwd(const gdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                              const int32_t* cu_seqlens, const float* h0, void* o, float* ht, void* workspace,
                              size_t workspace_bytes, void* stream) {
  gdr_status st = check(p, cu_seqlens != nullptr);
  if (st != GDR_OK) return st;
  if (p->gate_per_channel) return GDR_ERR_UNSUPPORTED;
  if (p->T > 0 && (q == nullptr || k == nullptr || v == nullptr || g == nullptr || o == nullptr))
    return GDR_ERR_NULL_ARG;
  const void* ptrs[] = {q, k, v, g, cu_seqlens, h0, o, ht, workspace};
  for (const void* ptr : ptrs)
    if (ptr != nullptr && !aligned16(ptr)) return GDR_ERR_ALIGNMENT;
  // the same layout rule as gdr_fwd_workspace_layout (simple GLA runs the fused
  // scan + output stage wherever the shape has it)
  const gdr_fwd_layout l = gdr::fwd_h_o_supported(make_args(*p)) ? fused_layout_of(*p) : layout_of(*p);
  if (workspace == nullptr || workspace_bytes < l.total) return GDR_ERR_WORKSPACE;

  Args a = make_args(*p);
  char* ws = static_cast<char*>(workspace);
  a.gla = 1;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = nullptr;
  a.cu = cu_seqlens;
  a.h0 = h0;
  a.chunk_idx = reinterpret_cast<int32_t*>(ws + l.chunk_idx);
  a.chunk_off = reinterpret_cast<int32_t*>(ws + l.chunk_off);
  a.seq_order = (a.cu != nullptr && a.N <= gdr::kMaxOrdered) ? reinterpret_cast<int32_t*>(ws + l.seq_order) : nullptr;
  a.w = ws + l.w;
  a.u = ws + l.u;
  a.h = ws + l.h;
  a.v_new = ws + l.v_new;
  a.kscale = reinterpret_cast<float*>(ws + l.kscale);
  a.o = o;
  a.ht = ht;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (cu_seqlens == nullptr && a.NTmax > 0) {
    a.table_from_dims = 1;
  } else {
    e = gdr::launch_chunk_table(a, s);
  }
  if (e == hipSuccess) e = gdr::launch_kkt_wy(a, s);
  a.table_from_dims = 0;
  a.gla = 0;   // the scan and output stages see an ordinary w / u pair
  if (gdr::fwd_h_o_supported(a)) {
    if (e == hipSuccess) e = gdr::launch_fwd_h_o(a, s);
  } else {
    if (e == hipSuccess) e = gdr::launch_fwd_h(a, s);
    if (e == hipSuccess) e = gdr::launch_fwd_o(a, s);
  }
  return hip_status(e);
}

gdr_status gdr_segmented_workspace_layout(const gdr_problem* p, gdr_seg_layout* out) {
  if (p == nullptr || out == nullptr) return GDR_ERR_NULL_ARG;
  const gdr_status st = check(p, true);
  if (st != GDR_OK) return st;
  *out = seg_layout_of(*p);
  return GDR_OK;
}

gdr_status gdr_segmented_workspace_bytes(const gdr_problem* p, size_t* bytes) {
  gdr_seg_layout l;
  const gdr_status st = gdr_segmented_workspace_layout(p, &l);
  if (st != GDR_OK) return st;
  if (bytes == nullptr) return GDR_ERR_NULL_ARG;
  *bytes = l.total;
  return GDR_OK;
}

gdr_status gdr_chunk_fwd_segmented(const gdr_problem* p, const void* q, const void* k, const void* v,
                                   const float* g, const float* beta, const int32_t* cu_seqlens,
                                   const float* h0, void* o, float* ht, float* seg_states, float* transitions,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (cu_seqlens == nullptr) return GDR_ERR_NULL_ARG;
  gdr_status st = check(p, true);
  if (st != GDR_OK) return st;
  if (p->T > 0 && (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr || o == nullptr))
    return GDR_ERR_NULL_ARG;
  const void* ptrs[] = {q, k, v, g, beta, cu_seqlens, h0, o, ht, seg_states, transitions, workspace};
  for (const void* ptr : ptrs)
    if (ptr != nullptr && !aligned16(ptr)) return GDR_ERR_ALIGNMENT;
  const gdr_seg_layout l = seg_layout_of(*p);
  if (workspace == nullptr || workspace_bytes < l.total) return GDR_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  const int64_t HV = p->HV, K = p->K, V = p->V, N = p->N;
  float* s_ext = reinterpret_cast<float*>(ws + l.s_ext);
  float* trans = transitions ? transitions : reinterpret_cast<float*>(ws + l.trans);
  float* s_in = seg_states ? seg_states : reinterpret_cast<float*>(ws + l.s_in);
  hipStream_t s = static_cast<hipStream_t>(stream);

  Args a = make_args(*p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.cu = cu_seqlens;
  a.chunk_idx = reinterpret_cast<int32_t*>(ws + l.fwd.chunk_idx);
  a.chunk_off = reinterpret_cast<int32_t*>(ws + l.fwd.chunk_off);
  a.seq_order = (a.cu != nullptr && a.N <= gdr::kMaxOrdered) ? reinterpret_cast<int32_t*>(ws + l.fwd.seq_order) : nullptr;
  a.Tm = ws + l.fwd.Tm;
  a.w = ws + l.fwd.w;
  a.u = ws + l.fwd.u;
  a.h = ws + l.fwd.h;
  a.v_new = ws + l.fwd.v_new;
  a.kscale = p->gate_per_channel ? nullptr : reinterpret_cast<float*>(ws + l.fwd.kscale);
  // u from the fused K1 + K2 stage (scalar gate, input dtype) or the separate WY stage (fp32)
  a.u_f32 = p->gate_per_channel ? 1 : 0;

  // chunk tables over the segments, then w, u (and the token factors)
  hipError_t e = gdr::launch_chunk_table(a, s);
  if (!p->gate_per_channel) {
    if (e == hipSuccess) e = gdr::launch_kkt_wy(a, s);
  } else {
    if (e == hipSuccess) e = gdr::launch_kkt_solve(a, s);
    if (e == hipSuccess) e = gdr::launch_wy(a, s);
  }
  // pre-process 1: every segment's local end state from a zero state
  Args pre = a;
  pre.h0 = nullptr;
  pre.ht = s_ext;
  // the warp-specialised scan skips h and v_new when they are not wanted
  // (the other variants write them to the workspace regardless)
  if (gdr::fwd_h_states_optional(pre)) pre.h = pre.v_new = nullptr;
  if (e == hipSuccess) e = gdr::launch_fwd_h(pre, s);
  // pre-process 2: every segment's transition, the same scan over the K x K
  // identity with no values (u = 0): S <- diag(e^{G_L}) S - K'^T (W S)
  Args tr = a;
  tr.V = K;
  tr.u = ws + l.u_zero;
  tr.h = ws + l.h_tr;
  tr.v_new = ws + l.v_tr;
  tr.h0 = reinterpret_cast<float*>(ws + l.eye);
  tr.ht = trans;
  const bool tr_states_only = gdr::fwd_h_states_optional(tr);
  if (tr_states_only) {
    tr.h = tr.v_new = nullptr;
    tr.u = nullptr;   // u = 0: neither read nor staged
  } else if (e == hipSuccess) {
    e = gdr::launch_zero(ws + l.u_zero, l.h_tr - l.u_zero, s);
  }
  if (e == hipSuccess) e = gdr::launch_identity(N * HV, K, reinterpret_cast<float*>(ws + l.eye), s);
  if (e == hipSuccess) e = gdr::launch_fwd_h(tr, s);
  // merge along the segments
  if (e == hipSuccess) e = gdr::launch_merge(N, HV, K, V, trans, s_ext, h0, s_in, s);
  // re-run every segment from its entering state; the last segment's end state is ht
  Args re = a;
  re.h0 = s_in;
  re.o = o;
  re.ht = s_ext;
  if (gdr::fwd_h_o_supported(re)) {
    if (e == hipSuccess) e = gdr::launch_fwd_h_o(re, s);
  } else {
    if (e == hipSuccess) e = gdr::launch_fwd_h(re, s);
    if (e == hipSuccess) e = gdr::launch_fwd_o(re, s);
  }
  if (e == hipSuccess && ht != nullptr)
    e = hipMemcpyAsync(ht, s_ext + (N - 1) * HV * K * V, (size_t)(HV * K * V) * sizeof(float),
                       hipMemcpyDeviceToDevice, s);
  return hip_status(e);
}

gdr_status gdr_bwd_workspace_layout(const gdr_problem* p, gdr_bwd_layout* out) {
  if (p == nullptr || out == nullptr) return GDR_ERR_NULL_ARG;
  const gdr_status st = check_bwd(p, p->N != p->B, true);
  if (st != GDR_OK) return st;
  *out = bwd_layout_of(bwd_problem(*p));
  if (needs_pad(*p)) out->total = pad_layout(*p, out->total, true).total;
  return GDR_OK;
}

gdr_status gdr_bwd_workspace_bytes(const gdr_problem* p, size_t* bytes) {
  gdr_bwd_layout l;
  const gdr_status st = gdr_bwd_workspace_layout(p, &l);
  if (st != GDR_OK) return st;
  if (bytes == nullptr) return GDR_ERR_NULL_ARG;
  *bytes = l.total;
  return GDR_OK;
}

gdr_status gdr_chunk_bwd(const gdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int32_t* cu_seqlens, const float* h0, const void* d_o,
                         const float* dht, void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                         void* workspace, size_t workspace_bytes, void* stream) {
  gdr_status st = check_bwd(p, cu_seqlens != nullptr, true);
  if (st != GDR_OK) return st;
  if (p->T > 0) {
    const void* req[] = {q, k, v, g, beta, d_o, dq, dk, dv, dg, dbeta};
    for (const void* ptr : req)
      if (ptr == nullptr) return GDR_ERR_NULL_ARG;
  }
  const void* ptrs[] = {q, k, v, g, beta, cu_seqlens, h0, d_o, dht, dq, dk, dv, dg, dbeta, dh0, workspace};
  for (const void* ptr : ptrs)
    if (ptr != nullptr && !aligned16(ptr)) return GDR_ERR_ALIGNMENT;
  const gdr_problem pp = bwd_problem(*p);
  const gdr_bwd_layout l = bwd_layout_of(pp);
  const bool pad = needs_pad(*p);
  const PadLayout pl = pad_layout(*p, l.total, true);
  if (workspace == nullptr || workspace_bytes < (pad ? pl.total : l.total)) return GDR_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  timer_start(s);
  if (!pad)
    return hip_status(bwd_run(pp, q, k, v, g, beta, cu_seqlens, h0, d_o, dht, dq, dk, dv, dg, dbeta, dh0, ws, l, s));

  // head dims without an instantiation: zero-padded copies in, padded problem, copies out
  const int es = (int)elem_size(*p);
  const int64_t BT = p->B * p->T, H = p->H, HV = p->HV, N = p->N, K = p->K, V = p->V, Kp = pp.K, Vp = pp.V;
  hipError_t e = gdr::launch_pad(q, ws + pl.q, BT * H, 1, K, 1, Kp, es, s);
  if (e == hipSuccess) e = gdr::launch_pad(k, ws + pl.k, BT * H, 1, K, 1, Kp, es, s);
  if (e == hipSuccess) e = gdr::launch_pad(v, ws + pl.v, BT * HV, 1, V, 1, Vp, es, s);
  if (e == hipSuccess) e = gdr::launch_pad(d_o, ws + pl.d_o, BT * HV, 1, V, 1, Vp, es, s);
  if (e == hipSuccess && h0 != nullptr) e = gdr::launch_pad(h0, ws + pl.h0, N * HV, K, V, Kp, Vp, 4, s);
  if (e == hipSuccess && dht != nullptr) e = gdr::launch_pad(dht, ws + pl.dht, N * HV, K, V, Kp, Vp, 4, s);
  const bool pc = p->gate_per_channel != 0;
  if (e == hipSuccess && pc) e = gdr::launch_pad(g, ws + pl.g, BT * HV, 1, K, 1, Kp, 4, s);
  timer_mark(e, "pad", s);
  if (e == hipSuccess)
    e = bwd_run(pp, ws + pl.q, ws + pl.k, ws + pl.v, pc ? reinterpret_cast<const float*>(ws + pl.g) : g, beta,
                cu_seqlens, h0 != nullptr ? reinterpret_cast<const float*>(ws + pl.h0) : nullptr, ws + pl.d_o,
                dht != nullptr ? reinterpret_cast<const float*>(ws + pl.dht) : nullptr, ws + pl.dq, ws + pl.dk,
                ws + pl.dv, pc ? reinterpret_cast<float*>(ws + pl.dg) : dg, dbeta,
                dh0 != nullptr ? reinterpret_cast<float*>(ws + pl.dh0) : nullptr, ws, l, s);
  if (e == hipSuccess && pc) e = gdr::launch_unpad(ws + pl.dg, dg, BT * HV, 1, K, 1, Kp, 4, s);
  if (e == hipSuccess) e = gdr::launch_unpad(ws + pl.dq, dq, BT * H, 1, K, 1, Kp, es, s);
  if (e == hipSuccess) e = gdr::launch_unpad(ws + pl.dk, dk, BT * H, 1, K, 1, Kp, es, s);
  if (e == hipSuccess) e = gdr::launch_unpad(ws + pl.dv, dv, BT * HV, 1, V, 1, Vp, es, s);
  if (e == hipSuccess && dh0 != nullptr) e = gdr::launch_unpad(ws + pl.dh0, dh0, N * HV, K, V, Kp, Vp, 4, s);
  timer_mark(e, "unpad", s);
  return hip_status(e);
}

namespace {
gdr_status bwd_stage_common(const gdr_problem* p, std::initializer_list<const void*> ptrs) {
  gdr_status st = check_bwd(p, p ? p->N != p->B : false);
  if (st != GDR_OK) return st;
  for (const void* ptr : ptrs) {
    if (ptr == nullptr) return GDR_ERR_NULL_ARG;
    if (!aligned16(ptr)) return GDR_ERR_ALIGNMENT;
  }
  return GDR_OK;
}
}  // namespace

gdr_status gdr_bwd_intra(const gdr_problem* p, const void* q, const void* k, const float* g, const void* d_o,
                         const int32_t* chunk_idx, const int32_t* chunk_off, void* de_local, float* qscale,
                         void* stream) {
  gdr_status st = bwd_stage_common(p, {q, k, g, d_o, chunk_idx, chunk_off, de_local, qscale});
  if (st != GDR_OK) return st;
  if (p->gate_per_channel) return GDR_ERR_UNSUPPORTED;
  Args a = make_args(*p);
  a.q = q;
  a.k = k;
  a.g = g;
  a.d_o = d_o;
  a.chunk_idx = const_cast<int32_t*>(chunk_idx);
  a.chunk_off = const_cast<int32_t*>(chunk_off);
  a.de_local = de_local;
  a.qscale = qscale;
  return hip_status(gdr::launch_bwd_intra(a, static_cast<hipStream_t>(stream)));
}

gdr_status gdr_bwd_dh(const gdr_problem* p, const void* q, const void* k, const void* w, const void* d_o,
                      const void* de_local, const float* qscale, const float* kscale, const int32_t* chunk_idx,
                      const int32_t* chunk_off, const float* dht, void* dh, float* dh0, void* stream) {
  gdr_status st = bwd_stage_common(p, {q, k, w, d_o, de_local, qscale, kscale, chunk_idx, chunk_off, dh});
  if (st != GDR_OK) return st;
  if (p->gate_per_channel) return GDR_ERR_UNSUPPORTED;
  if ((dht && !aligned16(dht)) || (dh0 && !aligned16(dh0))) return GDR_ERR_ALIGNMENT;
  Args a = make_args(*p);
  a.q = q;
  a.k = k;
  a.w = const_cast<void*>(w);
  a.d_o = d_o;
  a.de_local = const_cast<void*>(de_local);
  a.qscale = const_cast<float*>(qscale);
  a.kscale = const_cast<float*>(kscale);
  a.chunk_idx = const_cast<int32_t*>(chunk_idx);
  a.chunk_off = const_cast<int32_t*>(chunk_off);
  a.dht = dht;
  a.dh = dh;
  a.dh0 = dh0;
  return hip_status(gdr::launch_bwd_dh(a, static_cast<hipStream_t>(stream)));
}

gdr_status gdr_bwd_dqkvg(const gdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const void* d_o, const void* Tm, const void* h, const void* v_new,
                         const void* dh, const int32_t* chunk_idx, const int32_t* chunk_off, void* dq, void* dk,
                         void* dv, float* dg, float* dbeta, void* stream) {
  gdr_status st = bwd_stage_common(
      p, {q, k, v, g, beta, d_o, Tm, h, v_new, dh, chunk_idx, chunk_off, dq, dk, dv, dg, dbeta});
  if (st != GDR_OK) return st;
  if (p->gate_per_channel) return GDR_ERR_UNSUPPORTED;
  Args a = make_args(*p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.d_o = d_o;
  a.Tm = const_cast<void*>(Tm);
  a.h = const_cast<void*>(h);
  a.v_new = const_cast<void*>(v_new);
  a.dh = const_cast<void*>(dh);
  a.chunk_idx = const_cast<int32_t*>(chunk_idx);
  a.chunk_off = const_cast<int32_t*>(chunk_off);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dg;
  a.dbeta = dbeta;
  return hip_status(gdr::launch_bwd_dqkvg(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
