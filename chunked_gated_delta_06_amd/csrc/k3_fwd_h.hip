// K3: inter-chunk state scan (chunk_fwd_h).
//
// For each sequence n, value head j and chunk c in order, with S the K x V
// state (fp32) entering the chunk:
//   h[c]   = S                                  (state at the chunk start, the
//            convention of the KCP page, "flash-linear-attention KCP
//            precision-failure root-cause manual", section "h and dh
//            cross-rank semantics")
//   e      = u - w S                            (corrected values, "v_new")
//   S      <- diag(exp(G_L)) S + sum_t (exp(G_L - G_t) k^_t) e_t^T
// which is S^L = P^L S^0 + H^L of the chunk form on the coverage-matrix page
// ("FLA operator-kernel correctness testing and coverage matrix", section 2).
//
// gfx950 mapping: one workgroup per (sequence, value head, BV = 16 NW value
// columns; the scalar-gate scan below uses 32, or 16 when that fills the chip
// better); wave w owns 16 columns of S as K/16 16x16 fp32 MFMA accumulators
// that never leave registers.
//  * The chunk loop is software-pipelined: every chunk's w / k / u / gate data
//    is fetched into registers two chunk steps before it is used (two register
//    payloads, loop unrolled by two), then staged into one of two LDS buffers,
//    so the global-load latency overlaps two steps of MFMA work instead of
//    stalling the sequential scan.
//  * e = u - w S on bf16 MFMA, with S fed as the B operand directly from its
//    accumulator layout (the "chained" contraction map); the S update k^T e
//    reads k^T from LDS with ds_read_b64_tr_b16 and takes e from the previous
//    MFMA's accumulators.
//  * A scalar gate and the key norm scale the rows of e in fp32, keeping the
//    raw keys exact; a per-channel gate scales the staged key tile.
//  * u written by the separate WY stage is fp32; the S update takes its e
//    operand as a bf16 hi + lo pair (two MFMAs), so the state, and the h,
//    v_new and gradients the backward derives from it, carry about 16
//    mantissa bits of e instead of 8.  The fused scan + output stage keeps
//    the single bf16 operand and the input-dtype u of the fused K1 + K2 stage.
//  * h is written transposed (h^T, four features per lane) for the output
//    kernel; e is written per-chunk transposed (v_new).
//  * Consecutive workgroups of one head are mapped to one XCD so the shared
//    w / k tiles are served from the same L2.
#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

template <typename T, int C, int K, bool PC, int NW>
struct K3 {
  static constexpr int NT = 64 * NW;            // threads per workgroup
  static constexpr int NE = C / 16;             // token blocks of e
  static constexpr int NS = K / 16;             // feature blocks of S
  static constexpr int KSK = K / 32;            // feature slabs
  static constexpr int KSC = C / 32;            // token slabs
  static constexpr int CPR = K / 8;             // 8-element pieces per key row
  static constexpr int NPW = C * CPR;           // 8-element pieces of a C x K tile
  static constexpr int NLD = (NPW + NT - 1) / NT;   // pieces per thread (the last round may be partial)
  static constexpr int WP = K + 16 / sizeof(T); // LDS pitch of w rows (+16 B)
  static constexpr int KP = K + 32 / sizeof(T); // LDS pitch of key rows (+32 B, transposed reads)
  static constexpr int GP = K + 1;
  static constexpr int NG = PC ? C * K / 4 / NT : 1;   // float4 pieces of a per-channel gate tile
  static_assert(!PC || NG * NT == C * K / 4, "every thread stages whole gate pieces");
  static constexpr size_t tile_bytes = (size_t)C * (WP + KP) * sizeof(T) + (PC ? K * 4 : 0);
  static constexpr size_t fixed_bytes = PC ? (size_t)C * GP * 4 : 0;
  static constexpr int NBUF = (2 * tile_bytes + fixed_bytes <= 160 * 1024) ? 2 : 1;
  static constexpr bool fits = NBUF * tile_bytes + fixed_bytes <= 160 * 1024;

  // one chunk's global data, held in registers between fetch and staging
  struct Regs {
    Frag<T> w[NLD], k[NLD];
    f32x4 u[NE];       // u (fp32, from the separate WY stage)
    f32x4 ks[NE];      // scalar gate: exp(G_L - G_t) / |k_t| for this lane's rows of e
    f32x4 gc[NG];      // per-channel gate tile piece
    float gl;          // scalar gate: exp(G_L)
    int64_t t0;
    int L;
  };

  struct Smem {
    T w[NBUF][C * WP];
    T k[NBUF][C * KP];
    float dec[NBUF][PC ? K : 1];   // exp(G_L,d) (per-channel gate)
    float gc[PC ? C * GP : 1];     // per-channel cumsum scratch
  };
};

template <typename T, int C, int K, bool PC, int NW>
__global__ __launch_bounds__(64 * NW) void k3_fwd_h(Args a) {
  using Cfg = K3<T, C, K, PC, NW>;
  using Regs = typename Cfg::Regs;
  constexpr int NT = Cfg::NT, NE = Cfg::NE, NS = Cfg::NS, KSK = Cfg::KSK, KSC = Cfg::KSC;
  constexpr int CPR = Cfg::CPR, NLD = Cfg::NLD, NPW = Cfg::NPW, WP = Cfg::WP, KP = Cfg::KP, GP = Cfg::GP;
  constexpr int NG = Cfg::NG, NBUF = Cfg::NBUF;
  constexpr int BV = 16 * NW;
  __shared__ __attribute__((aligned(16))) typename Cfg::Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const int64_t H = a.H, HV = a.HV, V = a.V, N = a.N;
  const int64_t nvt = V / BV;
  const ScanUnit su = scan_unit(a.seq_order, N, HV, nvt);
  const int64_t vt = su.vt, j = su.j, n = su.n;
  if (n >= N) return;
  const int64_t h = j / (HV / H);
  const int64_t v0 = vt * BV + 16 * wv;     // this wave's first value column
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ wbase = static_cast<const T*>(a.w);
  const float* __restrict__ ubase = static_cast<const float*>(a.u);
  T* __restrict__ hbase = static_cast<T*>(a.h);
  T* __restrict__ vnbase = static_cast<T*>(a.v_new);
  const float* __restrict__ gp = a.g;

  // ---- fetch chunk c into registers (no waiting here)
  // Addresses are a wave-uniform 64-bit base plus a 32-bit per-lane offset.
  // token range of the sequence, read once (see k3_scan)
  const int64_t c_begin = a.chunk_off[n];
  const int nc = a.chunk_off[n + 1] - (int)c_begin;
  const int64_t c_last = c_begin + (nc > 0 ? nc - 1 : 0);
  const int64_t seq_t0 = nc > 0 ? a.chunk_idx[4 * c_begin + 1] : 0;
  const int64_t seq_end = nc > 0 ? a.chunk_idx[4 * c_last + 1] + a.chunk_idx[4 * c_last + 2] : 0;
  auto fetch = [&](Regs& R, int64_t c) {
    R.t0 = seq_t0 + (c - c_begin) * C;
    R.L = (int)((seq_end - R.t0) < C ? (seq_end - R.t0) : C);
    const T* wp = wbase + (c * HV + j) * (int64_t)(C * K);
    const T* krow = kp + (R.t0 * H + h) * K;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      // pieces past the tile (K = 32 with four waves) load piece 0 and are never staged
      const int idx = ((NPW % NT == 0) || tid + NT * i < NPW) ? tid + NT * i : 0;
      const int t = idx / CPR, d8 = (idx % CPR) * 8;
      const int tc = t < R.L ? t : R.L - 1;
      R.k[i] = ld8(krow + (tc * (int)(H * K) + d8));   // rows past L: zeroed when staged
      R.w[i] = ld8(wp + 8 * idx);
    }
    const float* up = ubase + ((c * HV + j) * V + v0) * (int64_t)C;
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) R.u[eb] = ld4raw(up + (r16 * C + 16 * eb + 4 * g4));
    if constexpr (PC) {
      const float* grow = gp + (R.t0 * HV + j) * K;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int idx = tid + NT * i, t = idx / (K / 4), d4 = (idx % (K / 4)) * 4;
        const int tc = t < R.L ? t : R.L - 1;
        R.gc[i] = *reinterpret_cast<const f32x4*>(grow + (tc * (int)(HV * K) + d4));
      }
    } else {
      const float* ksp = a.kscale + (c * HV + j) * kscale_pitch(C);
#pragma unroll
      for (int eb = 0; eb < NE; ++eb) R.ks[eb] = *reinterpret_cast<const f32x4*>(ksp + 16 * eb + 4 * g4);
      R.gl = ksp[C];
    }
  };

  f32x4 ucur[NE];     // u of the chunk being computed (accumulator layout)
  f32x4 kscur[NE];    // its row factors for e (scalar gate)
  float glcur = 0.f;  // exp(G_L) (scalar gate)

  // ---- stage registers into LDS buffer b (waits for the fetch to land)
  auto stage = [&](const Regs& R, int b) {
    if constexpr (PC) {
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int idx = tid + NT * i, t = idx / (K / 4), d4 = (idx % (K / 4)) * 4;
        const f32x4 gr = (t < R.L) ? R.gc[i] : zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.gc[t * GP + d4 + e] = gr[e];
      }
      lds_barrier();
      // chunk-local cumsum down each feature column: all C reads issued
      // first, the running sum in registers, then the writes
      for (int d = tid; d < K; d += NT) {
        float col[C];
#pragma unroll
        for (int t = 0; t < C; ++t) col[t] = sm.gc[t * GP + d];
#pragma unroll
        for (int t = 1; t < C; ++t) col[t] += col[t - 1];
#pragma unroll
        for (int t = 0; t < C; ++t) sm.gc[t * GP + d] = col[t];
        sm.dec[b][d] = __expf(col[C - 1]);
      }
      lds_barrier();
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      if (NPW % NT != 0 && idx >= NPW) continue;
      st8(&sm.w[b][t * WP + d8], R.w[i]);
      const Frag<T> kr = (t < R.L) ? R.k[i] : frag_zero<T>();
      if constexpr (PC) {
        f32x8 x = kr.f32();
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sq += x[e] * x[e];
        sq = lanes_sum(sq, CPR);
        const float rn = a.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
        const float* Gl = &sm.gc[(C - 1) * GP];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= rn * __expf(Gl[d8 + e] - sm.gc[t * GP + d8 + e]);
        st8(&sm.k[b][t * KP + d8], Frag<T>::make(x));
      } else {
        st8(&sm.k[b][t * KP + d8], kr);
      }
    }
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) {
      ucur[eb] = R.u[eb];
      if constexpr (!PC) kscur[eb] = R.ks[eb];
    }
    if constexpr (!PC) glcur = R.gl;
  };

  // S: rows 16 mb + 4 g4 + i, column v0 + r16
  f32x4 S[NS];
#pragma unroll
  for (int mb = 0; mb < NS; ++mb) {
    if (a.h0 != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mb][i] = a.h0[((n * HV + j) * K + 16 * mb + 4 * g4 + i) * V + v0 + r16];
    } else {
      S[mb] = zero4();
    }
  }

  // ---- one chunk step from LDS buffer b
  auto compute = [&](int64_t c, int b) {
    // h[c] = S (transposed, 4 features per lane)
    T* hp = hbase + ((c * HV + j) * V + v0) * (int64_t)K;
#pragma unroll
    for (int mb = 0; mb < NS; ++mb) st4(hp + (r16 * K + 16 * mb + 4 * g4), S[mb]);
    // e = u - w S
    f32x4 E[NE];
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) E[eb] = ucur[eb];
    Frag<T> nS[KSK];
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks) nS[ks] = frag_from_halves<T>(-S[2 * ks], -S[2 * ks + 1]);
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) {
      const T* row = &sm.w[b][(16 * eb + r16) * WP];
#pragma unroll
      for (int ks = 0; ks < KSK; ++ks)
        mma(E[eb], ld_chain(row + 32 * ks + 4 * g4, row + 32 * ks + 16 + 4 * g4), nS[ks]);
    }
    // v_new = e (transposed per chunk)
    T* vnp = vnbase + ((c * HV + j) * V + v0) * (int64_t)C;
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) st4(vnp + (r16 * C + 16 * eb + 4 * g4), E[eb]);
    // S <- diag(exp(G_L)) S + k^T diag(s) e  (e as a hi + lo pair)
    SplitFrag<T> Ef[KSC];
#pragma unroll
    for (int kt = 0; kt < KSC; ++kt) {
      f32x4 lo = E[2 * kt], hi = E[2 * kt + 1];
      if constexpr (!PC) {
        lo *= kscur[2 * kt];
        hi *= kscur[2 * kt + 1];
      }
      Ef[kt] = SplitFrag<T>::make(cat8(lo, hi));
    }
    if constexpr (PC) {
#pragma unroll
      for (int mb = 0; mb < NS; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mb][i] *= sm.dec[b][16 * mb + 4 * g4 + i];
    } else {
#pragma unroll
      for (int mb = 0; mb < NS; ++mb) S[mb] *= glcur;
    }
#pragma unroll
    for (int mb = 0; mb < NS; ++mb)
#pragma unroll
      for (int kt = 0; kt < KSC; ++kt)
        mma_split(S[mb], lds_tr_frag(&sm.k[b][0], KP, 32 * kt + 4 * g4, 32 * kt + 16 + 4 * g4, 16 * mb, lane), Ef[kt]);
  };

  // ---- pipelined chunk loop.  Fetches are unconditional (the chunk index is
  // clamped to the sequence's last chunk, so the load addresses stay valid and
  // extra copies are simply never computed): with an identical stream of
  // memory operations on every path the compiler can wait for exactly the
  // fetch it needs instead of draining all outstanding loads.
  if (nc > 0) {
    auto cl = [&](int64_t c) { return c < c_last ? c : c_last; };
    Regs Ra, Rb;
    fetch(Ra, c_begin);
    fetch(Rb, cl(c_begin + 1));
    stage(Ra, 0);
    lds_barrier();
    fetch(Ra, cl(c_begin + 2));
    int i = 0;
    for (; i + 1 < nc; i += 2) {
      compute(c_begin + i, 0);
      if constexpr (NBUF == 1) lds_barrier();
      stage(Rb, NBUF - 1);
      fetch(Rb, cl(c_begin + i + 3));
      lds_barrier();
      compute(c_begin + i + 1, NBUF - 1);
      if constexpr (NBUF == 1) lds_barrier();
      stage(Ra, 0);
      fetch(Ra, cl(c_begin + i + 4));
      lds_barrier();
    }
    if (i < nc) compute(c_begin + i, 0);
  }

  if (a.ht != nullptr) {
#pragma unroll
    for (int mb = 0; mb < NS; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.ht[((n * HV + j) * K + 16 * mb + 4 * g4 + i) * V + v0 + r16] = S[mb][i];
  }
}

// ---------------------------------------------------------------------------
// Scalar-gate scan with warp specialisation.  Waves 0..NWC-1 compute (each owns
// 16 value columns of S and runs only the MFMA chain of the step); waves
// NWC..NWC+NWL-1 are loaders: they fetch each chunk's w / k / u / kscale into
// registers three chunk steps ahead (three payloads, loop unrolled by three),
// stage it into one of two LDS buffers while the compute waves work on the
// other, and meet the compute waves at one LDS-only barrier per step.  The
// compute waves therefore carry no prefetch registers, so the state and the
// e tiles stay in architectural VGPRs next to the MFMAs.
template <typename T, int C, int K, int NWC, int NWL, int NWO = 0, typename UT = T, bool PC = false>
struct K3S {
  static constexpr int NTL = 64 * NWL;          // loader threads
  static constexpr int BV = 16 * NWC;           // value columns per workgroup
  static constexpr int NE = C / 16, NS = K / 16, KSK = K / 32, KSC = C / 32;
  static constexpr int CPR = K / 8;
  static constexpr int NPW = C * CPR;           // 8-element pieces of a w (or k) tile
  static constexpr int NPU = BV * C / 8;        // 8-element pieces of the u tile
  static constexpr int NLD = (NPW + NTL - 1) / NTL;   // w and k pieces per loader thread
  static constexpr int NLU = (NPU + NTL - 1) / NTL;   // u pieces per loader thread
  // float4 pieces of a kscale row, or (per-channel gate) of the decay exp(G_L)
  static constexpr int KSN = PC ? K : C + 4;
  static constexpr int NKS = KSN / 4;
  static constexpr int WP = K + 16 / sizeof(T);
  static constexpr int KP = K + 32 / sizeof(T);
  static constexpr int UP = C + 16 / sizeof(UT); // u rows (one per value column), +16 B
  static constexpr size_t buf_bytes = (size_t)C * (WP + KP) * sizeof(T) + (size_t)BV * UP * sizeof(UT) + KSN * 4;
  static constexpr bool fits = 2 * buf_bytes <= 160 * 1024 && NKS <= NTL;
  // Output staging: the compute waves leave h and e of a step in LDS and the
  // loader waves store them during the next step, so the compute waves issue
  // no vector-memory instructions at all (their stores would queue behind the
  // loaders' loads in the CU's memory pipeline and stall the MFMA chain).
  // Used when the two extra buffers fit next to the double-buffered tiles.
  // staged h rows (one per value column); the fused output reads them as
  // 16-byte row pieces, which a 32-byte pad keeps free of bank conflicts (bf16;
  // fp32 keeps 16 bytes so that its fused shapes still fit)
  static constexpr int HSP = K + (NWO > 0 && sizeof(T) == 2 ? 32 : 16) / sizeof(T);
  static constexpr int VSP = C + 16 / sizeof(T);  // staged e rows
  static constexpr size_t stg_bytes = (size_t)BV * (HSP + VSP) * sizeof(T);
  static constexpr bool STG = 2 * (buf_bytes + stg_bytes) <= 160 * 1024;
  static constexpr int NDH = (BV * K / 8 + NTL - 1) / NTL;   // staged h pieces per loader thread
  static constexpr int NDV = (BV * C / 8 + NTL - 1) / NTL;   // staged e pieces per loader thread
  // fused output: the loaders also stage each chunk's q tile and gates, or
  // (per-channel gate) the gated query tile(s) and the intra attention aqk
  // (fp32 rows)
  static constexpr bool OUT = NWO > 0;
  static constexpr bool PCO = OUT && PC;
  static constexpr int QP = K + (sizeof(T) == 2 ? 32 : 16) / sizeof(T);   // staged q rows, padded as h
  static constexpr int NQT = PCO ? kQgsTiles : 1;   // staged query tiles
  static constexpr int AP = C + 4;              // staged aqk rows
  static constexpr int NLA = PCO ? (C * C / 4 + NTL - 1) / NTL : 1;   // float4 pieces of aqk per loader thread
  static constexpr size_t q_bytes =
      OUT ? (size_t)NQT * C * QP * sizeof(T) + (PCO ? (size_t)C * AP * 4 : 3 * C * 4) : 0;
  static constexpr bool fits_out = STG && 2 * (buf_bytes + stg_bytes + q_bytes) <= 160 * 1024;

  struct Regs {
    Frag<T> w[NLD], k[NLD];
    Frag<T> q[OUT ? NQT * NLD : 1];
    f32x4 pa[NLA];            // aqk pieces (per-channel fused output)
    Frag<UT> u[NLU];
    f32x4 ks;
    float g2;                 // G_t (threads < C) or 1 / |k_t| (threads C .. 2C - 1)
    float rk2, gref;          // threads < C: 1 / |k_t| and G at the end of t's key block
    int64_t t0;
    int L;
  };
  struct Smem {
    T w[2][C * WP];
    T k[2][C * KP];
    UT u[2][BV * UP];
    __attribute__((aligned(16))) float ks[2][KSN];
    T hs[STG ? 2 : 1][STG ? BV * HSP : 8];
    T es[STG ? 2 : 1][STG ? BV * VSP : 8];
    T q[OUT ? 2 : 1][OUT ? NQT * C * QP : 8];
    // per token of the staged chunk: gate cumsum G_t in log2 units, 1 / |k_t|
    // and the column factor exp(G_e - G_t) / |k_t|, e the last token of t's
    // key block (zero past L)
    __attribute__((aligned(16))) float gq[OUT && !PC ? 2 : 1][OUT && !PC ? C : 4];
    __attribute__((aligned(16))) float rk[OUT && !PC ? 2 : 1][OUT && !PC ? C : 4];
    __attribute__((aligned(16))) float cf[OUT && !PC ? 2 : 1][OUT && !PC ? C : 4];
    __attribute__((aligned(16))) float pa[PCO ? 2 : 1][PCO ? C * AP : 4];
  };
};

// KEEP = false: a scan that only needs the end states (the segment hand-off's
// pre-process), or the fused scan + output of a forward that keeps no states,
// writes neither h nor v_new.  With output waves and KEEP, the staged h / e
// are stored one step later while the output waves read them: by the loaders
// (scalar gate) or by the output waves themselves (per-channel gate, whose
// output work is light and whose loaders carry the larger payload).  ZU: u is zero (the transition
// scan), so it is neither read nor staged.  UT: u's storage type (fp32 from
// the separate WY stage, the input dtype from the fused K1 + K2 stage).
// PC: per-channel gate, with the chunk's gated keys exp(G_L - G_t) k^_t and
// decay exp(G_L) from the WY stage in place of the raw keys and the token
// factors: S <- diag(exp(G_L)) S + Kt^T e.  With output waves as well (bf16),
// o = (scale exp(G) q^) h + aqk e from the gated queries and aqk of the
// fused per-channel K1 + K2, so the output waves apply no gate factor
// themselves.
template <typename T, int C, int K, int NWC, int NWL, int NWO, bool KEEP = true, bool ZU = false, typename UT = T,
          bool PC = false>
__global__ __launch_bounds__(64 * (NWC + NWO + NWL)) void k3_scan(Args a) {
  using Cfg = K3S<T, C, K, NWC, NWL, NWO, UT, PC>;
  static_assert(!PC || NWO == 0 || sizeof(T) == 2, "the per-channel fused output takes bf16 gated queries");
  using Regs = typename Cfg::Regs;
  constexpr int NTL = Cfg::NTL, BV = Cfg::BV, NE = Cfg::NE, NS = Cfg::NS, KSK = Cfg::KSK, KSC = Cfg::KSC;
  constexpr int CPR = Cfg::CPR, NLD = Cfg::NLD, NLU = Cfg::NLU, NKS = Cfg::NKS, NPW = Cfg::NPW, NPU = Cfg::NPU;
  constexpr int WP = Cfg::WP, KP = Cfg::KP, UP = Cfg::UP;
  constexpr bool STG = Cfg::STG;
  constexpr int HSP = Cfg::HSP, VSP = Cfg::VSP, NDH = Cfg::NDH, NDV = Cfg::NDV;
  __shared__ __attribute__((aligned(16))) typename Cfg::Smem sm;

  // fused output: NWO output waves compute o from the staged h / e, and
  // neither h nor v_new is written
  constexpr bool OUT = Cfg::OUT;
  constexpr int QP = Cfg::QP, AP = Cfg::AP, NLA = Cfg::NLA;
  static_assert(!OUT || (Cfg::fits_out && Cfg::NTL >= 2 * C), "the fused output reads the staged h / e / q");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const bool loader = wv >= NWC + NWO;
  const bool outw = !loader && wv >= NWC;
  const int oi = wv - NWC;                       // output wave index
  const int tl = tid - 64 * (NWC + NWO);         // loader thread index
  const int64_t H = a.H, HV = a.HV, V = a.V, N = a.N;
  const int64_t nvt = V / BV;
  const ScanUnit su = scan_unit(a.seq_order, N, HV, nvt);
  const int64_t vt = su.vt, j = su.j, n = su.n;
  if (n >= N) return;
  const int64_t h = j / (HV / H);
  const int64_t vw = vt * BV;                    // workgroup's first value column
  const int64_t v0 = vw + 16 * wv;               // compute wave's first value column
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ wbase = static_cast<const T*>(a.w);
  const UT* __restrict__ ubase = static_cast<const UT*>(a.u);
  T* __restrict__ hbase = static_cast<T*>(a.h);
  T* __restrict__ vnbase = static_cast<T*>(a.v_new);

  const int64_t c_begin = a.chunk_off[n];
  const int nc = a.chunk_off[n + 1] - (int)c_begin;
  const int64_t c_last = c_begin + (nc > 0 ? nc - 1 : 0);
  auto cl = [&](int64_t c) { return c < c_last ? c : c_last; };
  // token range of the sequence, read once: chunk c_begin + x starts at
  // seq_t0 + x C, so the loop never waits on a chunk-table load (vector-memory
  // waits complete in order and would drain the prefetched payloads)
  const int64_t seq_t0 = nc > 0 ? a.chunk_idx[4 * c_begin + 1] : 0;
  const int64_t seq_end = nc > 0 ? a.chunk_idx[4 * c_last + 1] + a.chunk_idx[4 * c_last + 2] : 0;

  // ---- loader side
  auto fetch = [&](Regs& R, int64_t c) {
    R.t0 = seq_t0 + (c - c_begin) * C;
    R.L = (int)((seq_end - R.t0) < C ? (seq_end - R.t0) : C);
    const T* wp = wbase + (c * HV + j) * (int64_t)(C * K);
    // scalar gate: the raw key rows of the input; per-channel: the chunk's gated rows
    const T* krow = PC ? static_cast<const T*>(a.kt) + (c * HV + j) * (int64_t)(C * K) : kp + (R.t0 * H + h) * K;
    const int kstride = PC ? K : (int)(H * K);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tl + NTL * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      const bool in = (NPW % NTL == 0) || idx < NPW;
      // Only loads here: nothing reads the payload until it is staged, so the
      // in-order vector-memory counter lets the later payloads stay in flight.
      // Rows past L load row L-1 (a valid address) and are zeroed when staged;
      // pieces past the tile load piece 0 and are never staged.
      const int tc = t < R.L ? t : R.L - 1;
      R.k[i] = ld8(krow + (tc * kstride + d8));
      R.w[i] = ld8(wp + 8 * (in ? idx : 0));
      if constexpr (OUT && PC) {
        // the chunk's gated query tiles (hi, then lo), zero past L
        const T* qs = static_cast<const T*>(a.qgs) + (c * HV + j) * (int64_t)(kQgsTiles * C * K);
        R.q[i] = ld8(qs + 8 * (in ? idx : 0));
        if constexpr (kQgsTiles == 2) R.q[NLD + i] = ld8(qs + C * K + 8 * (in ? idx : 0));
      } else if constexpr (OUT) {
        R.q[i] = ld8(static_cast<const T*>(a.q) + (R.t0 * H + h) * K + (tc * (int)(H * K) + d8));
      }
    }
    if constexpr (OUT && PC) {
      const float* ap = a.aqk + (c * HV + j) * (int64_t)(C * C);
#pragma unroll
      for (int i = 0; i < NLA; ++i) {
        const int idx = tl + NTL * i;
        R.pa[i] = *reinterpret_cast<const f32x4*>(ap + 4 * (((C * C / 4) % NTL == 0 || idx < C * C / 4) ? idx : 0));
      }
    }
    if constexpr (!ZU) {
      const UT* up = ubase + ((c * HV + j) * V + vw) * (int64_t)C;
#pragma unroll
      for (int i = 0; i < NLU; ++i) {
        const int idx = tl + NTL * i;
        R.u[i] = ld8(up + 8 * (((NPU % NTL == 0) || idx < NPU) ? idx : 0));
      }
    }
    const float* ksp = PC ? a.dl + (c * HV + j) * (int64_t)K : a.kscale + (c * HV + j) * kscale_pitch(C);
    R.ks = *reinterpret_cast<const f32x4*>(ksp + 4 * (tl < NKS ? tl : 0));
    // fused output: G_t and 1 / |k_t| of the chunk (K1's token factors), and
    // for the column factor G at the end of t's key block (the chunk's last
    // token when the block runs past it)
    if constexpr (OUT && !PC) {
      R.g2 = ksp[C + 4 + (tl < 2 * C ? tl : 0)];
      const int tc = tl < C ? tl : 0;
      const int te = (tc | 15) < R.L - 1 ? (tc | 15) : R.L - 1;
      R.rk2 = ksp[2 * C + 4 + tc];
      R.gref = ksp[C + 4 + te];
    }
  };
  auto stage = [&](const Regs& R, int b) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tl + NTL * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      if ((NPW % NTL == 0) || idx < NPW) {
        st8(&sm.w[b][t * WP + d8], R.w[i]);
        st8(&sm.k[b][t * KP + d8], t < R.L ? R.k[i] : frag_zero<T>());
        if constexpr (OUT && PC) {
          st8(&sm.q[b][t * QP + d8], R.q[i]);
          if constexpr (kQgsTiles == 2) st8(&sm.q[b][(C + t) * QP + d8], R.q[NLD + i]);
        } else if constexpr (OUT) {
          st8(&sm.q[b][t * QP + d8], t < R.L ? R.q[i] : frag_zero<T>());
        }
      }
    }
    if constexpr (OUT && PC) {
#pragma unroll
      for (int i = 0; i < NLA; ++i) {
        const int idx = tl + NTL * i, r = idx / (C / 4), t4 = (idx % (C / 4)) * 4;
        if ((C * C / 4) % NTL == 0 || idx < C * C / 4) *reinterpret_cast<f32x4*>(&sm.pa[b][r * AP + t4]) = R.pa[i];
      }
    } else if constexpr (OUT) {
      if (tl < C) {
        // past L: G of the chunk's last token, so every staged factor stays finite
        sm.gq[b][tl] = (tl < R.L ? R.g2 : R.gref) * kLog2e;
        sm.cf[b][tl] = tl < R.L ? R.rk2 * exp2_fast((R.gref - R.g2) * kLog2e) : 0.f;
      } else if (tl < 2 * C) {
        sm.rk[b][tl - C] = R.g2;
      }
    }
    if constexpr (!ZU) {
#pragma unroll
      for (int i = 0; i < NLU; ++i) {
        const int idx = tl + NTL * i, v = idx / (C / 8), t8 = (idx % (C / 8)) * 8;
        if ((NPU % NTL == 0) || idx < NPU) st8(&sm.u[b][v * UP + t8], R.u[i]);
      }
    }
    if (tl < NKS) *reinterpret_cast<f32x4*>(&sm.ks[b][4 * tl]) = R.ks;
  };

  // staged h / e of step x (buffer x % 2) to global memory, 16 contiguous
  // bytes per lane: h^T rows of K features and e^T rows of C tokens are
  // contiguous for the workgroup's BV value columns
  auto drain = [&](int x) {
    const int64_t c = c_begin + x;
    T* hp = hbase + ((c * HV + j) * V + vw) * (int64_t)K;
    T* vnp = vnbase + ((c * HV + j) * V + vw) * (int64_t)C;
    Frag<T> hv[NDH], ev[NDV];
#pragma unroll
    for (int i = 0; i < NDH; ++i) {
      const int idx = tl + NTL * i, v = idx / (K / 8), d8 = (idx % (K / 8)) * 8;
      if ((BV * K / 8) % NTL == 0 || idx < BV * K / 8) hv[i] = ld8(&sm.hs[x & 1][v * HSP + d8]);
    }
#pragma unroll
    for (int i = 0; i < NDV; ++i) {
      const int idx = tl + NTL * i, v = idx / (C / 8), t8 = (idx % (C / 8)) * 8;
      if ((BV * C / 8) % NTL == 0 || idx < BV * C / 8) ev[i] = ld8(&sm.es[x & 1][v * VSP + t8]);
    }
#pragma unroll
    for (int i = 0; i < NDH; ++i) {
      const int idx = tl + NTL * i;
      if ((BV * K / 8) % NTL == 0 || idx < BV * K / 8) st8(hp + 8 * idx, hv[i]);
    }
#pragma unroll
    for (int i = 0; i < NDV; ++i) {
      const int idx = tl + NTL * i;
      if ((BV * C / 8) % NTL == 0 || idx < BV * C / 8) st8(vnp + 8 * idx, ev[i]);
    }
  };

  // The loader and compute waves run separate loops with the same sequence of
  // barriers (one per chunk step), so neither carries the other's registers.
  // Chunk c_begin + x lives in register slot x % 3 and LDS buffer x % 2; at
  // step s the compute waves work on chunk s while the loaders stage chunk s + 1
  // and fetch chunk s + 4 (indices clamped to the last chunk; extra copies are
  // staged but never computed) and, with output staging, store the h / e that
  // step s - 1 left in LDS.
  if (loader) {
    if (nc > 0) {
      Regs R0, R1, R2;
      fetch(R0, c_begin);
      fetch(R1, cl(c_begin + 1));
      fetch(R2, cl(c_begin + 2));
      stage(R0, 0);
      fetch(R0, cl(c_begin + 3));
      lds_barrier();
      for (int s0 = 0; s0 < nc; s0 += 3) {
        stage(R1, (s0 + 1) & 1);
        fetch(R1, cl(c_begin + s0 + 4));
        if constexpr (STG && KEEP && !(OUT && PC)) {
          if (s0 > 0) drain(s0 - 1);
        }
        lds_barrier();
        stage(R2, (s0 + 2) & 1);
        fetch(R2, cl(c_begin + s0 + 5));
        if constexpr (STG && KEEP && !(OUT && PC)) {
          if (s0 < nc) drain(s0);
        }
        lds_barrier();
        stage(R0, (s0 + 3) & 1);
        fetch(R0, cl(c_begin + s0 + 6));
        if constexpr (STG && KEEP && !(OUT && PC)) {
          if (s0 + 1 < nc) drain(s0 + 1);
        }
        lds_barrier();
      }
      // the last step's output when the loop ended right after it
      if constexpr (STG && KEEP && !(OUT && PC)) {
        if (nc % 3 == 0) drain(nc - 1);
      }
    }
    return;
  }

  // ---- output waves (fused output).  During step x an output wave computes o
  // of chunk x - 1 from the h / e the compute waves staged in LDS during step
  // x - 1, then the P^T blocks of chunk x from the key tile staged for step x,
  // as the output stage does: O^T = scale (h^T Q^T diag(exp(G) / |q|) +
  // e^T P^T), P^T[t][r] = k^_t . q^_r exp(G_r - G_t) for t <= r.  q rows are
  // read straight into MFMA operand registers one step ahead; o leaves as
  // 16-byte stores of four consecutive value columns per lane and block pair.
  if (outw) {
    if constexpr (OUT) {
      constexpr int NB = C / 16;                 // token blocks of a chunk
      // Output waves split the chunk's token blocks into NTS groups and, when
      // there are more waves than token blocks, the value columns into NCS parts.
      constexpr int NTS = NWO < NB ? NWO : NB;
      constexpr int NCS = NWO / NTS;
      constexpr int TPW = NB / NTS;              // token blocks per output wave (1 or 2)
      constexpr int NVW = BV / 16 / NCS;         // value blocks per output wave
      static_assert(TPW >= 1 && TPW <= 2 && TPW * NTS == NB && NTS * NCS == NWO && NVW * NCS * 16 == BV,
                    "output-wave token / column split");
      // The wave index is a compile-time constant inside `run` (one
      // instantiation per output wave, selected by a scalar branch): every
      // causal-block condition below folds away, so the loops unroll without
      // branches and LDS reads and independent MFMA chains interleave.  (A
      // runtime condition would split the code into small blocks, and held in
      // a vector register it would become a lane mask, which an MFMA ignores.)
      auto run = [&](auto owc) {
      constexpr int OW = decltype(owc)::value;
      constexpr int OT = OW % NTS, OC = OW / NTS;   // token group, column part
      constexpr int VB0 = OC * NVW;                 // first value block of the wave
      // token blocks {OT, NB - 1 - OT}: equal causal work for both groups
      constexpr int TB0 = OT, TB1 = NB - 1 - OT;
      auto tbk = [](int m) constexpr { return m == 0 ? TB0 : TB1; };
      constexpr int tbmax = TPW == 1 ? TB0 : TB1;
      T* __restrict__ op = static_cast<T*>(a.o);
      // operands of one chunk's output, carried from its P^T step to its o step
      struct ORegs {
        Frag<T> q[TPW][KSK];        // q rows of this wave's token blocks (per-channel: gated, hi part)
        Frag<T> ql[PC && kQgsTiles == 2 ? TPW : 1][PC && kQgsTiles == 2 ? KSK : 1];   // lo part of a gated-row pair
        SplitFrag<T> f[TPW][KSC];   // P^T as the chained B operand
        float isc[TPW];             // scale exp(G_r) / |q_r| (scalar gate)
      };
      auto chunk_t0 = [&](int x) { return seq_t0 + (int64_t)x * C; };
      auto chunk_L = [&](int x) {
        const int64_t r = seq_end - chunk_t0(x);
        return (int)(r < C ? r : C);
      };
      // P^T blocks of chunk x from the staged keys, queries and gates
      // (buffer x % 2; rows past L are zero there).  On a diagonal block
      // exp(G_r - G_t) is taken directly; below it, it is the row factor
      // exp(G_r - G_e) times the staged column factor exp(G_e - G_t) / |k_t|,
      // e the last token of t's key block (for non-positive gates both are at
      // most 1).  |q_r|^2 is the diagonal of the block's Q Q^T product, and the
      // output scale rides on the row factors.  A column r >= L of P^T only
      // reaches row r of o, which is never stored.
      // Per-channel gate: the gated query rows and the aqk rows come staged,
      // so the phase only reads them into operand registers (aqk rows are zero
      // above the diagonal and past L).
      auto pphase_pc = [&](ORegs& P, int x) {
        const int b = x & 1;
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
          const int rr = 16 * tbk(m) + r16;
#pragma unroll
          for (int ks = 0; ks < KSK; ++ks) {
            P.q[m][ks] = ld8(&sm.q[b][rr * QP + 32 * ks + 8 * g4]);
            if constexpr (kQgsTiles == 2) P.ql[m][ks] = ld8(&sm.q[b][(C + rr) * QP + 32 * ks + 8 * g4]);
          }
          const float* prow = &sm.pa[b][rr * AP];
#pragma unroll
          for (int kt = 0; kt < KSC; ++kt) {
            if (2 * kt > tbk(m)) continue;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(prow + 32 * kt + 4 * g4);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(prow + 32 * kt + 16 + 4 * g4);
            P.f[m][kt] = SplitFrag<T>::make(cat8(lo, hi));
          }
          P.isc[m] = 1.f;
        }
      };
      auto pphase_sc = [&](ORegs& P, int x) {
        const int b = x & 1;
        float rs[TPW], Gr[TPW];      // scale / |q_r| and G_r (log2 units)
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
          const int rr = 16 * tbk(m) + r16;
          f32x4 d = zero4();
#pragma unroll
          for (int ks = 0; ks < KSK; ++ks) {
            P.q[m][ks] = ld8(&sm.q[b][rr * QP + 32 * ks + 8 * g4]);
            mma(d, P.q[m][ks], P.q[m][ks]);
          }
          // Q Q^T[i][r16] sits in lane r16 + 16 (i >> 2), element i & 3
          const float d01 = (r16 & 1) ? d[1] : d[0], d23 = (r16 & 1) ? d[3] : d[2];
          const float sq = __shfl((r16 & 2) ? d23 : d01, r16 + 16 * (r16 >> 2), 64);
          rs[m] = a.l2norm ? a.scale * __builtin_amdgcn_rsqf(sq + kL2Eps) : a.scale;
          Gr[m] = sm.gq[b][rr];
        }
        f32x4 Pt[TPW][NB];
#pragma unroll
        for (int m = 0; m < TPW; ++m)
#pragma unroll
          for (int jb = 0; jb < NB; ++jb) Pt[m][jb] = zero4();
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
          if (jb > tbmax) continue;
          Frag<T> kf[KSK];
#pragma unroll
          for (int ks = 0; ks < KSK; ++ks) kf[ks] = ld8(&sm.k[b][(16 * jb + r16) * KP + 32 * ks + 8 * g4]);
#pragma unroll
          for (int m = 0; m < TPW; ++m) {
            if (jb > tbk(m)) continue;
#pragma unroll
            for (int ks = 0; ks < KSK; ++ks) mma(Pt[m][jb], kf[ks], P.q[m][ks]);
          }
          // P^T[t][rr] with t = 16 jb + 4 g4 + i: the four tokens' factors in one read each
          bool below = false, diag = false;
#pragma unroll
          for (int m = 0; m < TPW; ++m) {
            below |= jb < tbk(m);
            diag |= jb == tbk(m);
          }
          if (below) {
            const f32x4 cf4 = *reinterpret_cast<const f32x4*>(&sm.cf[b][16 * jb + 4 * g4]);
            const float Ge = sm.gq[b][16 * jb + 15];
#pragma unroll
            for (int m = 0; m < TPW; ++m) {
              if (jb >= tbk(m)) continue;
              Pt[m][jb] *= cf4 * (rs[m] * exp2_fast(Gr[m] - Ge));
            }
          }
          if (diag) {
            const f32x4 rk4 = *reinterpret_cast<const f32x4*>(&sm.rk[b][16 * jb + 4 * g4]);
            const f32x4 G4 = *reinterpret_cast<const f32x4*>(&sm.gq[b][16 * jb + 4 * g4]);
#pragma unroll
            for (int m = 0; m < TPW; ++m) {
              if (jb != tbk(m)) continue;
#pragma unroll
              for (int i = 0; i < 4; ++i)
                Pt[m][jb][i] *= 4 * g4 + i <= r16 ? rs[m] * rk4[i] * exp2_fast(Gr[m] - G4[i]) : 0.f;
            }
          }
        }
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
#pragma unroll
          for (int kt = 0; kt < KSC; ++kt) P.f[m][kt] = SplitFrag<T>::make(cat8(Pt[m][2 * kt], Pt[m][2 * kt + 1]));
          P.isc[m] = rs[m] * exp2_fast(Gr[m]);
        }
      };
      auto pphase = [&](ORegs& P, int x) {
        if constexpr (PC) {
          pphase_pc(P, x);
        } else {
          pphase_sc(P, x);
        }
      };
      // o of chunk x from the staged h / e (buffer x % 2) and its P^T step's operands
      auto ophase = [&](const ORegs& P, int x) {
        const int64_t t0 = chunk_t0(x);
        const int L = chunk_L(x);
        const T* hsb = sm.hs[x & 1];
        const T* esb = sm.es[x & 1];
        // kept states with a per-channel gate: the waves of token group 0 store
        // the staged h^T rows of their value blocks and those of group 1 the
        // e^T rows, as they read them (the loaders' registers have no room for
        // the stores there)
        constexpr bool KEEP_H = PC && KEEP && OT == 0, KEEP_E = PC && KEEP && OT == 1;
        const int64_t cx = c_begin + x;
        f32x4 O[TPW][NVW];
#pragma unroll
        for (int ib = 0; ib < NVW; ++ib) {
          const int vb = VB0 + ib;
          Frag<T> hf[KSK];
#pragma unroll
          for (int ks = 0; ks < KSK; ++ks) hf[ks] = ld8(&hsb[(16 * vb + r16) * HSP + 32 * ks + 8 * g4]);
          const T* erow = &esb[(16 * vb + r16) * VSP];
          if constexpr (KEEP_H) {
            T* hrow = hbase + ((cx * HV + j) * V + vw + 16 * vb + r16) * (int64_t)K;
#pragma unroll
            for (int ks = 0; ks < KSK; ++ks) st8(hrow + 32 * ks + 8 * g4, hf[ks]);
          }
          if constexpr (KEEP_E) {
            T* vrow = vnbase + ((cx * HV + j) * V + vw + 16 * vb + r16) * (int64_t)C;
#pragma unroll
            for (int kt = 0; kt < KSC; ++kt) {
              using V4 = typename Vec<T>::v4;
              *reinterpret_cast<V4*>(vrow + 32 * kt + 4 * g4) = ld4raw(erow + 32 * kt + 4 * g4);
              *reinterpret_cast<V4*>(vrow + 32 * kt + 16 + 4 * g4) = ld4raw(erow + 32 * kt + 16 + 4 * g4);
            }
          }
#pragma unroll
          for (int m = 0; m < TPW; ++m) {
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < KSK; ++ks) {
              mma(acc, hf[ks], P.q[m][ks]);
              if constexpr (PC && kQgsTiles == 2) mma(acc, hf[ks], P.ql[m][ks]);
            }
            if constexpr (!PC) acc *= P.isc[m];
#pragma unroll
            for (int kt = 0; kt < KSC; ++kt) {
              if (2 * kt > tbk(m)) continue;
              mma_split(acc, ld_chain(erow + 32 * kt + 4 * g4, erow + 32 * kt + 16 + 4 * g4), P.f[m][kt]);
            }
            O[m][ib] = acc;
          }
        }
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
          const int rr = 16 * tbk(m) + r16;
          T* orow = op + ((t0 + rr) * HV + j) * V + vw + 16 * VB0;
          if (rr < L) {
            if constexpr (NVW % 2 == 0) {
#pragma unroll
              for (int pb = 0; pb < NVW / 2; ++pb) st_pair(orow + 32 * pb, O[m][2 * pb], O[m][2 * pb + 1], lane);
            } else {
#pragma unroll
              for (int vb = 0; vb < NVW; ++vb) st4(orow + 16 * vb + 4 * g4, O[m][vb]);
            }
          }
        }
      };

      // Same barrier sequence as the other roles: one per chunk step over
      // 3 ceil(nc / 3) steps.  Step x: o of chunk x - 1, then P^T of chunk x
      // (whose operands stay in registers for the next step's o).  (Merging
      // the two phases into one branch-free block, so that they interleave,
      // measured slower.)
      if (nc > 0) {
        ORegs P;
        lds_barrier();
        const int nsteps = 3 * ((nc + 2) / 3);
        for (int x = 0; x < nsteps; ++x) {
          if (x >= 1 && x - 1 < nc) ophase(P, x - 1);
          if (x < nc) pphase(P, x);
          lds_barrier();
        }
        // the last chunk's o when the loop ended right after its step
        if (nsteps == nc) ophase(P, nc - 1);
      }
      };
      const int oiu = __builtin_amdgcn_readfirstlane(oi);
      if constexpr (NWO == 2) {
        if (oiu == 0) {
          run(std::integral_constant<int, 0>{});
        } else {
          run(std::integral_constant<int, 1>{});
        }
      } else {
        static_assert(NWO == 4, "two or four output waves");
        if (oiu == 0) {
          run(std::integral_constant<int, 0>{});
        } else if (oiu == 1) {
          run(std::integral_constant<int, 1>{});
        } else if (oiu == 2) {
          run(std::integral_constant<int, 2>{});
        } else {
          run(std::integral_constant<int, 3>{});
        }
      }
    }
    return;
  }

  // ---- compute waves: S rows 16 mb + 4 g4 + i, column v0 + r16
  f32x4 S[NS];
#pragma unroll
  for (int mb = 0; mb < NS; ++mb) {
    if (a.h0 != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mb][i] = a.h0[((n * HV + j) * K + 16 * mb + 4 * g4 + i) * V + v0 + r16];
    } else {
      S[mb] = zero4();
    }
  }
  auto compute = [&](int64_t c, int b) {
    // every LDS fragment of the step is requested up front (w rows for e, k^T
    // columns for the S update), so the reads overlap the MFMA chain instead of
    // each MFMA waiting on its own read
    Frag<T> wf[KSK][NE], kf[KSC][NS];
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks)
#pragma unroll
      for (int eb = 0; eb < NE; ++eb) {
        const T* row = &sm.w[b][(16 * eb + r16) * WP];
        wf[ks][eb] = ld_chain(row + 32 * ks + 4 * g4, row + 32 * ks + 16 + 4 * g4);
      }
#pragma unroll
    for (int kt = 0; kt < KSC; ++kt)
#pragma unroll
      for (int mb = 0; mb < NS; ++mb)
        kf[kt][mb] = lds_tr_frag(&sm.k[b][0], KP, 32 * kt + 4 * g4, 32 * kt + 16 + 4 * g4, 16 * mb, lane);
    f32x4 E[NE];
    const UT* urow = &sm.u[b][(16 * wv + r16) * UP];
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) E[eb] = ZU ? zero4() : ld4f(urow + 16 * eb + 4 * g4);
    f32x4 sc[NE];
#pragma unroll
    for (int eb = 0; eb < NE; ++eb)
      sc[eb] = PC ? f32x4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4*>(&sm.ks[b][16 * eb + 4 * g4]);
    const float gl = PC ? 1.f : sm.ks[b][C];
    // h[c] = S (transposed): staged in LDS for the loaders, or stored directly
    // with feature blocks paired into 16-byte stores
    if constexpr (STG && (OUT || KEEP)) {
      T* hs = &sm.hs[b][(16 * wv + r16) * HSP];
#pragma unroll
      for (int mb = 0; mb < NS; ++mb) st4(hs + 16 * mb + 4 * g4, S[mb]);
    } else if constexpr (KEEP) {
      T* hp = hbase + ((c * HV + j) * V + v0) * (int64_t)K;
#pragma unroll
      for (int m = 0; m < NS / 2; ++m) st_pair(hp + (r16 * K + 32 * m), S[2 * m], S[2 * m + 1], lane);
    }
    // e = u - w S  (independent accumulators alternate between MFMAs)
    Frag<T> nS[KSK];
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks) nS[ks] = frag_from_halves<T>(-S[2 * ks], -S[2 * ks + 1]);
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks)
#pragma unroll
      for (int eb = 0; eb < NE; ++eb) mma(E[eb], wf[ks][eb], nS[ks]);
    // v_new = e (transposed per chunk)
    if constexpr (STG && (OUT || KEEP)) {
      T* es = &sm.es[b][(16 * wv + r16) * VSP];
#pragma unroll
      for (int eb = 0; eb < NE; ++eb) st4(es + 16 * eb + 4 * g4, E[eb]);
    } else if constexpr (KEEP) {
      T* vnp = vnbase + ((c * HV + j) * V + v0) * (int64_t)C;
#pragma unroll
      for (int m = 0; m < NE / 2; ++m) st_pair(vnp + (r16 * C + 32 * m), E[2 * m], E[2 * m + 1], lane);
    }
    // S <- exp(G_L) S + k^T diag(exp(G_L - G_t) / |k_t|) e: e as a hi + lo
    // pair except in the scalar-gate fused scan + output stage that keeps no
    // states
    if constexpr (PC) {
      // row d of S decays by exp(G_L,d)
#pragma unroll
      for (int mb = 0; mb < NS; ++mb) S[mb] *= *reinterpret_cast<const f32x4*>(&sm.ks[b][16 * mb + 4 * g4]);
    } else {
#pragma unroll
      for (int mb = 0; mb < NS; ++mb) S[mb] *= gl;
    }
    if constexpr (OUT && !PC && !KEEP) {
      Frag<T> Ef[KSC];
#pragma unroll
      for (int kt = 0; kt < KSC; ++kt) Ef[kt] = frag_from_halves<T>(E[2 * kt] * sc[2 * kt], E[2 * kt + 1] * sc[2 * kt + 1]);
#pragma unroll
      for (int kt = 0; kt < KSC; ++kt)
#pragma unroll
        for (int mb = 0; mb < NS; ++mb) mma(S[mb], kf[kt][mb], Ef[kt]);
    } else {
      SplitFrag<T> Ef[KSC];
#pragma unroll
      for (int kt = 0; kt < KSC; ++kt) Ef[kt] = SplitFrag<T>::make(cat8(E[2 * kt] * sc[2 * kt], E[2 * kt + 1] * sc[2 * kt + 1]));
#pragma unroll
      for (int kt = 0; kt < KSC; ++kt)
#pragma unroll
        for (int mb = 0; mb < NS; ++mb) mma_split(S[mb], kf[kt][mb], Ef[kt]);
    }
  };

  if (nc > 0) {
    lds_barrier();
    for (int s0 = 0; s0 < nc; s0 += 3) {
      compute(c_begin + s0, s0 & 1);
      lds_barrier();
      if (s0 + 1 < nc) compute(c_begin + s0 + 1, (s0 + 1) & 1);
      lds_barrier();
      if (s0 + 2 < nc) compute(c_begin + s0 + 2, s0 & 1);
      lds_barrier();
    }
  }
  if (a.ht != nullptr) {
#pragma unroll
    for (int mb = 0; mb < NS; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.ht[((n * HV + j) * K + 16 * mb + 4 * g4 + i) * V + v0 + r16] = S[mb][i];
  }
}

template <typename T, int C, int K, bool PC, int NW>
hipError_t launch_nw(const Args& a, hipStream_t s) {
  if constexpr (!K3<T, C, K, PC, NW>::fits) {
    return hipErrorInvalidValue;    // rejected on the host before any launch
  } else {
    const int64_t nblk = a.N * a.HV * (a.V / (16 * NW));
    hipLaunchKernelGGL((k3_fwd_h<T, C, K, PC, NW>), dim3((unsigned)nblk), dim3(64 * NW), 0, s, a);
    return hipGetLastError();
  }
}

// The warp-specialised scan reading u of type UT: 2 compute + 2 loader waves
// (4 loader waves when elements or u are fp32 or K = 256, to keep each
// loader's payload in registers), or 1 + NWL (below).
template <typename T, int C, int K, typename UT>
constexpr int scan_loaders() {
  return (sizeof(T) == 4 || sizeof(UT) == 4 || K == 256) ? 4 : 2;
}

template <typename T, int C, int K, typename UT>
hipError_t launch_keep(const Args& a, hipStream_t s) {
  constexpr int NWL = scan_loaders<T, C, K, UT>();
  if constexpr (!K3S<T, C, K, 2, NWL, 0, UT>::fits) {
    return hipErrorInvalidValue;
  } else {
    const int64_t nblk32 = a.N * a.HV * (a.V / 32);
    if (nblk32 < kNumCUs)
      hipLaunchKernelGGL((k3_scan<T, C, K, 1, NWL, 0, true, false, UT>), dim3((unsigned)(2 * nblk32)),
                         dim3(64 * (1 + NWL)), 0, s, a);
    else
      hipLaunchKernelGGL((k3_scan<T, C, K, 2, NWL, 0, true, false, UT>), dim3((unsigned)nblk32),
                         dim3(64 * (2 + NWL)), 0, s, a);
    return hipGetLastError();
  }
}

// Per-channel gate with the WY stage's gated keys and decay (a.kt, a.dl): the
// warp-specialised scan in its per-channel mode, u in fp32.
// (K = 256 keeps the other per-channel scan: its loaders' payload would spill)
template <typename T, int C, int K>
constexpr bool pc_scan_fits() {
  return K <= 128 && K3S<T, C, K, 2, scan_loaders<T, C, K, float>(), 0, float, true>::fits &&
         K3S<T, C, K, 1, scan_loaders<T, C, K, float>(), 0, float, true>::fits;
}

template <typename T, int C, int K>
hipError_t launch_keep_pc(const Args& a, hipStream_t s) {
  constexpr int NWL = scan_loaders<T, C, K, float>();
  if constexpr (!pc_scan_fits<T, C, K>()) {
    return hipErrorInvalidValue;
  } else {
    const int64_t nblk32 = a.N * a.HV * (a.V / 32);
    if (nblk32 < kNumCUs)
      hipLaunchKernelGGL((k3_scan<T, C, K, 1, NWL, 0, true, false, float, true>), dim3((unsigned)(2 * nblk32)),
                         dim3(64 * (1 + NWL)), 0, s, a);
    else
      hipLaunchKernelGGL((k3_scan<T, C, K, 2, NWL, 0, true, false, float, true>), dim3((unsigned)nblk32),
                         dim3(64 * (2 + NWL)), 0, s, a);
    return hipGetLastError();
  }
}

template <typename T, int C, int K, bool PC>
hipError_t launch_t(const Args& a, hipStream_t s) {
  if constexpr (PC && pc_scan_fits<T, C, K>()) {
    if (a.kt != nullptr && a.dl != nullptr && a.h != nullptr && a.u_f32) return launch_keep_pc<T, C, K>(a, s);
  }
  if constexpr (!PC) {
    // warp-specialised scan: 2 compute + 2 loader waves (4 loader waves when
    // elements are fp32 or K = 256, to keep each loader's payload in registers)
    constexpr int NWL = scan_loaders<T, C, K, T>();
    if constexpr (K3S<T, C, K, 2, NWL>::fits && K3S<T, C, K, 2, scan_loaders<T, C, K, float>(), 0, float>::fits) {
      // 32 value columns (two compute waves) per workgroup, or 16 (one) when
      // the 32-column grid would leave compute units idle: the scan's step
      // latency does not shrink with fewer columns, so more workgroups is the
      // only way to use the whole chip on few long sequences
      const int64_t nblk32 = a.N * a.HV * (a.V / 32);
      // h == NULL: end states only; u == NULL too: u is zero (transition scan)
      const bool keep = a.h != nullptr, zu = !keep && a.u == nullptr;
      if (keep) return a.u_f32 ? launch_keep<T, C, K, float>(a, s) : launch_keep<T, C, K, T>(a, s);
      if (nblk32 < kNumCUs) {
        const dim3 g((unsigned)(2 * nblk32)), b(64 * (1 + NWL));
        if (!zu)
          hipLaunchKernelGGL((k3_scan<T, C, K, 1, NWL, 0, false>), g, b, 0, s, a);
        else
          hipLaunchKernelGGL((k3_scan<T, C, K, 1, NWL, 0, false, true>), g, b, 0, s, a);
      } else {
        const dim3 g((unsigned)nblk32), b(64 * (2 + NWL));
        if (!zu)
          hipLaunchKernelGGL((k3_scan<T, C, K, 2, NWL, 0, false>), g, b, 0, s, a);
        else
          hipLaunchKernelGGL((k3_scan<T, C, K, 2, NWL, 0, false, true>), g, b, 0, s, a);
      }
      return hipGetLastError();
    }
  }
  // per-channel gate (and a scalar gate whose warp-specialised scan does not
  // fit): u comes from the separate WY stage, in fp32.  Each workgroup forms
  // the chunk's gate cumsum and decayed keys itself, so four waves (64 value
  // columns) share that work when the grid still gives every compute unit a
  // workgroup; otherwise (and for shapes whose double-buffered tiles exceed
  // LDS) two waves, 32 columns
  if (sizeof(T) == 2 && !a.u_f32 && a.u != nullptr) return hipErrorInvalidValue;
  if constexpr (PC && K3<T, C, K, PC, 4>::fits) {
    if (a.V % 64 == 0 && a.N * a.HV * (a.V / 64) >= kNumCUs) return launch_nw<T, C, K, PC, 4>(a, s);
  }
  return launch_nw<T, C, K, PC, 2>(a, s);
}

template <typename T, int C, bool PC>
hipError_t launch_k(const Args& a, hipStream_t s) {
  switch (a.K) {
    case 32: return launch_t<T, C, 32, PC>(a, s);
    case 64: return launch_t<T, C, 64, PC>(a, s);
    case 128: return launch_t<T, C, 128, PC>(a, s);
    case 256: return launch_t<T, C, 256, PC>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_c(const Args& a, hipStream_t s) {
  if (a.C == 32) return a.per_channel ? launch_k<T, 32, true>(a, s) : launch_k<T, 32, false>(a, s);
  return a.per_channel ? launch_k<T, 64, true>(a, s) : launch_k<T, 64, false>(a, s);
}

// ---- fused state scan + output (scalar gate): 1 or 2 compute waves, 2 output
// waves, 4 loader waves (the output waves' registers leave room for only half
// a loader payload per thread).  Shapes qualify when the staged h / e fit in
// LDS next to the double-buffered tiles and no role spills.
template <typename T, int C, int K>
constexpr bool fused_ok() {
  return K3S<T, C, K, 2, 4, 2>::fits && K3S<T, C, K, 2, 4, 2>::fits_out && K3S<T, C, K, 1, 4, 2>::fits_out &&
         K <= 128;
}
// the kept-states variant: u in fp32 from the kept-states fused K1 + K2, e as
// a hi + lo pair in the state update, h and v_new stored
template <typename T, int C, int K>
constexpr bool fused_keep_ok() {
  return K <= 128 && K3S<T, C, K, 2, 4, 2, float>::fits_out && K3S<T, C, K, 1, 4, 2, float>::fits_out;
}

template <typename T, int C, int K, bool KEEP>
hipError_t launch_fused_t(const Args& a, hipStream_t s) {
  using UT = typename std::conditional<KEEP, float, T>::type;
  constexpr bool ok = KEEP ? fused_keep_ok<T, C, K>() : fused_ok<T, C, K>();
  if constexpr (ok) {
    const int64_t nblk32 = a.N * a.HV * (a.V / 32);
    if (nblk32 < kNumCUs) {
      hipLaunchKernelGGL((k3_scan<T, C, K, 1, 4, 2, KEEP, false, UT>), dim3((unsigned)(2 * nblk32)), dim3(64 * 7),
                         0, s, a);
    } else {
      hipLaunchKernelGGL((k3_scan<T, C, K, 2, 4, 2, KEEP, false, UT>), dim3((unsigned)nblk32), dim3(64 * 8), 0, s,
                         a);
    }
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <typename T, int C, bool KEEP>
bool fused_ok_k(int64_t K) {
  switch (K) {
    case 32: return KEEP ? fused_keep_ok<T, C, 32>() : fused_ok<T, C, 32>();
    case 64: return KEEP ? fused_keep_ok<T, C, 64>() : fused_ok<T, C, 64>();
    case 128: return KEEP ? fused_keep_ok<T, C, 128>() : fused_ok<T, C, 128>();
    case 256: return KEEP ? fused_keep_ok<T, C, 256>() : fused_ok<T, C, 256>();
  }
  return false;
}

template <typename T, int C, bool KEEP>
hipError_t launch_fused_k(const Args& a, hipStream_t s) {
  switch (a.K) {
    case 32: return launch_fused_t<T, C, 32, KEEP>(a, s);
    case 64: return launch_fused_t<T, C, 64, KEEP>(a, s);
    case 128: return launch_fused_t<T, C, 128, KEEP>(a, s);
    case 256: return launch_fused_t<T, C, 256, KEEP>(a, s);
  }
  return hipErrorInvalidValue;
}

// ---- fused state scan + output, per-channel gate (bf16, chunk 32): the
// per-channel scan's compute and loader waves plus output waves on the aqk and
// gated queries of the fused per-channel K1 + K2.  64 value columns (4 compute
// waves, and 4 output waves that split the chunk's two token blocks and the
// columns in halves) per workgroup when that grid still gives every compute
// unit a workgroup, else 32 (2 compute and 2 output waves).
template <typename T, int C, int K>
constexpr bool pc_out_ok() {
  constexpr int NWL = scan_loaders<T, C, K, float>();
  return sizeof(T) == 2 && C == 32 && K <= 128 && K3S<T, C, K, 4, NWL, 4, float, true>::fits_out &&
         K3S<T, C, K, 2, NWL, 2, float, true>::fits_out;
}

// KEEP: h and v_new are stored as well (kept states), and u is the fp32 of
// the kept-states K1 + K2; otherwise u is in the input dtype
template <typename T, int C, int K, bool KEEP>
hipError_t launch_pc_out_t(const Args& a, hipStream_t s) {
  if constexpr (pc_out_ok<T, C, K>()) {
    using UT = typename std::conditional<KEEP, float, T>::type;
    constexpr int NWL = scan_loaders<T, C, K, float>();
    const int64_t nblk64 = a.N * a.HV * (a.V / 64);
    if (a.V % 64 == 0 && nblk64 >= kNumCUs) {
      hipLaunchKernelGGL((k3_scan<T, C, K, 4, NWL, 4, KEEP, false, UT, true>), dim3((unsigned)nblk64),
                         dim3(64 * (8 + NWL)), 0, s, a);
    } else {
      hipLaunchKernelGGL((k3_scan<T, C, K, 2, NWL, 2, KEEP, false, UT, true>),
                         dim3((unsigned)(a.N * a.HV * (a.V / 32))), dim3(64 * (4 + NWL)), 0, s, a);
    }
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

bool pc_out_ok_k(int64_t K) {
  switch (K) {
    case 32: return pc_out_ok<bf16, 32, 32>();
    case 64: return pc_out_ok<bf16, 32, 64>();
    case 128: return pc_out_ok<bf16, 32, 128>();
  }
  return false;
}

}  // namespace

namespace {
// the condition launch_t uses to pick the warp-specialised scan
template <typename T, int C, int K>
constexpr bool specialised_fits() {
  return K3S<T, C, K, 2, scan_loaders<T, C, K, T>()>::fits &&
         K3S<T, C, K, 2, scan_loaders<T, C, K, float>(), 0, float>::fits;
}
template <typename T, int C>
bool specialised_k(int64_t K) {
  switch (K) {
    case 32: return specialised_fits<T, C, 32>();
    case 64: return specialised_fits<T, C, 64>();
    case 128: return specialised_fits<T, C, 128>();
    case 256: return specialised_fits<T, C, 256>();
  }
  return false;
}
}  // namespace

bool fwd_pc_scan_fits(int dtype, int C, int K) {
  auto k = [&](auto tc, auto cc) {
    using TT = decltype(tc);
    constexpr int CC = decltype(cc)::value;
    switch (K) {
      case 32: return pc_scan_fits<TT, CC, 32>();
      case 64: return pc_scan_fits<TT, CC, 64>();
      case 128: return pc_scan_fits<TT, CC, 128>();
      case 256: return pc_scan_fits<TT, CC, 256>();
    }
    return false;
  };
  if (dtype == GDR_BF16)
    return C == 32 ? k(bf16{}, std::integral_constant<int, 32>{}) : k(bf16{}, std::integral_constant<int, 64>{});
  return C == 32 ? k(float{}, std::integral_constant<int, 32>{}) : k(float{}, std::integral_constant<int, 64>{});
}

bool fwd_h_states_optional(const Args& a) {
  if (a.per_channel) return false;
  if (a.dtype == GDR_BF16) return a.C == 32 ? specialised_k<bf16, 32>(a.K) : specialised_k<bf16, 64>(a.K);
  return a.C == 32 ? specialised_k<float, 32>(a.K) : specialised_k<float, 64>(a.K);
}

hipError_t launch_fwd_h(const Args& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  return a.dtype == GDR_BF16 ? launch_c<bf16>(a, s) : launch_c<float>(a, s);
}

bool fwd_h_o_supported(const Args& a) {
  if (a.per_channel) return false;
  if (a.dtype == GDR_BF16) return a.C == 32 ? fused_ok_k<bf16, 32, false>(a.K) : fused_ok_k<bf16, 64, false>(a.K);
  return a.C == 32 ? fused_ok_k<float, 32, false>(a.K) : fused_ok_k<float, 64, false>(a.K);
}

bool fwd_h_o_preferred(const Args& a) {
  // measured faster than the separate scan and output stages on both grid
  // shapes (one 16-column compute wave per workgroup on few long sequences:
  // 1.78 vs 1.95 ms; two compute waves on 4 x 16 heads: 145 vs 222 us)
  return fwd_h_o_supported(a);
}

bool fwd_h_o_pc_supported(const Args& a) {
  return a.per_channel && a.dtype == GDR_BF16 && a.C == 32 && pc_out_ok_k(a.K) && a.V % 32 == 0;
}

bool fwd_h_o_pc_preferred(const Args& a) { return fwd_h_o_pc_supported(a); }

hipError_t launch_fwd_h_o_pc(const Args& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  const bool keep = a.h != nullptr && a.v_new != nullptr;
  if (!fwd_h_o_pc_supported(a) || a.kt == nullptr || a.dl == nullptr || a.aqk == nullptr || a.qgs == nullptr ||
      a.u == nullptr || (a.u_f32 != 0) != keep)
    return hipErrorInvalidValue;
  switch (a.K) {
    case 32: return keep ? launch_pc_out_t<bf16, 32, 32, true>(a, s) : launch_pc_out_t<bf16, 32, 32, false>(a, s);
    case 64: return keep ? launch_pc_out_t<bf16, 32, 64, true>(a, s) : launch_pc_out_t<bf16, 32, 64, false>(a, s);
    case 128:
      return keep ? launch_pc_out_t<bf16, 32, 128, true>(a, s) : launch_pc_out_t<bf16, 32, 128, false>(a, s);
  }
  return hipErrorInvalidValue;
}

bool fwd_h_o_keep_supported(const Args& a) {
  if (a.per_channel) return false;
  if (a.dtype == GDR_BF16) return a.C == 32 ? fused_ok_k<bf16, 32, true>(a.K) : fused_ok_k<bf16, 64, true>(a.K);
  return a.C == 32 ? fused_ok_k<float, 32, true>(a.K) : fused_ok_k<float, 64, true>(a.K);
}

hipError_t launch_fwd_h_o_keep(const Args& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  if (!fwd_h_o_keep_supported(a) || a.h == nullptr || a.v_new == nullptr || !a.u_f32) return hipErrorInvalidValue;
  if (a.dtype == GDR_BF16)
    return a.C == 32 ? launch_fused_k<bf16, 32, true>(a, s) : launch_fused_k<bf16, 64, true>(a, s);
  return a.C == 32 ? launch_fused_k<float, 32, true>(a, s) : launch_fused_k<float, 64, true>(a, s);
}

hipError_t launch_fwd_h_o(const Args& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  if (a.dtype == GDR_BF16)
    return a.C == 32 ? launch_fused_k<bf16, 32, false>(a, s) : launch_fused_k<bf16, 64, false>(a, s);
  return a.C == 32 ? launch_fused_k<float, 32, false>(a, s) : launch_fused_k<float, 64, false>(a, s);
}

}  // namespace gdr
