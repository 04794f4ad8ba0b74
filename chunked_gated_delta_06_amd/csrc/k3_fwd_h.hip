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
//  * h is written transposed (h^T, four features per lane) for the output
//    kernel; e is written per-chunk transposed (v_new).
//  * Consecutive workgroups of one head are mapped to one XCD so the shared
//    w / k tiles are served from the same L2.
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
  static constexpr int NLD = C * CPR / NT;      // pieces of a C x K tile per thread
  static constexpr int WP = K + 16 / sizeof(T); // LDS pitch of w rows (+16 B)
  static constexpr int KP = K + 32 / sizeof(T); // LDS pitch of key rows (+32 B, transposed reads)
  static constexpr int GP = K + 1;
  static constexpr int NG = PC ? C * K / 4 / NT : 1;   // float4 pieces of a per-channel gate tile
  static constexpr size_t tile_bytes = (size_t)C * (WP + KP) * sizeof(T) + (PC ? K * 4 : 0);
  static constexpr size_t fixed_bytes = PC ? (size_t)C * GP * 4 : 0;
  static constexpr int NBUF = (2 * tile_bytes + fixed_bytes <= 160 * 1024) ? 2 : 1;
  static constexpr bool fits = NBUF * tile_bytes + fixed_bytes <= 160 * 1024;

  // one chunk's global data, held in registers between fetch and staging
  struct Regs {
    Frag<T> w[NLD], k[NLD];
    v4_t<T> u[NE];
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
  constexpr int CPR = Cfg::CPR, NLD = Cfg::NLD, WP = Cfg::WP, KP = Cfg::KP, GP = Cfg::GP;
  constexpr int NG = Cfg::NG, NBUF = Cfg::NBUF;
  constexpr int BV = 16 * NW;
  __shared__ __attribute__((aligned(16))) typename Cfg::Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const int64_t H = a.H, HV = a.HV, V = a.V, N = a.N;
  const int64_t nvt = V / BV;
  const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t vt = bid % nvt, j = (bid / nvt) % HV, n = bid / (nvt * HV);
  if (n >= N) return;
  const int64_t h = j / (HV / H);
  const int64_t v0 = vt * BV + 16 * wv;     // this wave's first value column
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ wbase = static_cast<const T*>(a.w);
  const T* __restrict__ ubase = static_cast<const T*>(a.u);
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
      const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      const int tc = t < R.L ? t : R.L - 1;
      const Frag<T> kr = ld8(krow + (tc * (int)(H * K) + d8));
      R.w[i] = ld8(wp + 8 * idx);
      R.k[i] = (t < R.L) ? kr : frag_zero<T>();
    }
    const T* up = ubase + ((c * HV + j) * V + v0) * (int64_t)C;
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) R.u[eb] = ld4raw(up + (r16 * C + 16 * eb + 4 * g4));
    if constexpr (PC) {
      const float* grow = gp + (R.t0 * HV + j) * K;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int idx = tid + NT * i, t = idx / (K / 4), d4 = (idx % (K / 4)) * 4;
        const int tc = t < R.L ? t : R.L - 1;
        const f32x4 gr = *reinterpret_cast<const f32x4*>(grow + (tc * (int)(HV * K) + d4));
        R.gc[i] = (t < R.L) ? gr : zero4();
      }
    } else {
      const float* ksp = a.kscale + (c * HV + j) * (int64_t)(C + 4);
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
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.gc[t * GP + d4 + e] = R.gc[i][e];
      }
      lds_barrier();
      for (int d = tid; d < K; d += NT) {
        float run = 0.f;
        for (int t = 0; t < C; ++t) {
          run += sm.gc[t * GP + d];
          sm.gc[t * GP + d] = run;
        }
        sm.dec[b][d] = __expf(run);
      }
      lds_barrier();
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      st8(&sm.w[b][t * WP + d8], R.w[i]);
      if constexpr (PC) {
        f32x8 x = R.k[i].f32();
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
        st8(&sm.k[b][t * KP + d8], R.k[i]);
      }
    }
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) {
      ucur[eb] = to_f32<T>(R.u[eb]);
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
    // S <- diag(exp(G_L)) S + k^T diag(s) e
    Frag<T> Ef[KSC];
#pragma unroll
    for (int kt = 0; kt < KSC; ++kt) {
      f32x4 lo = E[2 * kt], hi = E[2 * kt + 1];
      if constexpr (!PC) {
        lo *= kscur[2 * kt];
        hi *= kscur[2 * kt + 1];
      }
      Ef[kt] = frag_from_halves<T>(lo, hi);
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
        mma(S[mb], lds_tr_frag(&sm.k[b][0], KP, 32 * kt + 4 * g4, 32 * kt + 16 + 4 * g4, 16 * mb, lane), Ef[kt]);
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
template <typename T, int C, int K, int NWC, int NWL>
struct K3S {
  static constexpr int NTL = 64 * NWL;          // loader threads
  static constexpr int BV = 16 * NWC;           // value columns per workgroup
  static constexpr int NE = C / 16, NS = K / 16, KSK = K / 32, KSC = C / 32;
  static constexpr int CPR = K / 8;
  static constexpr int NPW = C * CPR;           // 8-element pieces of a w (or k) tile
  static constexpr int NPU = BV * C / 8;        // 8-element pieces of the u tile
  static constexpr int NLD = (NPW + NTL - 1) / NTL;   // w and k pieces per loader thread
  static constexpr int NLU = (NPU + NTL - 1) / NTL;   // u pieces per loader thread
  static constexpr int NKS = (C + 4) / 4;       // float4 pieces of a kscale row
  static constexpr int WP = K + 16 / sizeof(T);
  static constexpr int KP = K + 32 / sizeof(T);
  static constexpr int UP = C + 8 / sizeof(T);  // u rows (one per value column), +8 B
  static constexpr size_t buf_bytes = (size_t)C * (WP + KP) * sizeof(T) + (size_t)BV * UP * sizeof(T) + (C + 4) * 4;
  static constexpr bool fits = 2 * buf_bytes <= 160 * 1024 && NKS <= NTL;

  struct Regs {
    Frag<T> w[NLD], k[NLD];
    Frag<T> u[NLU];
    f32x4 ks;
    int64_t t0;
    int L;
  };
  struct Smem {
    T w[2][C * WP];
    T k[2][C * KP];
    T u[2][BV * UP];
    float ks[2][C + 4];
  };
};

template <typename T, int C, int K, int NWC, int NWL>
__global__ __launch_bounds__(64 * (NWC + NWL)) void k3_scan(Args a) {
  using Cfg = K3S<T, C, K, NWC, NWL>;
  using Regs = typename Cfg::Regs;
  constexpr int NTL = Cfg::NTL, BV = Cfg::BV, NE = Cfg::NE, NS = Cfg::NS, KSK = Cfg::KSK, KSC = Cfg::KSC;
  constexpr int CPR = Cfg::CPR, NLD = Cfg::NLD, NLU = Cfg::NLU, NKS = Cfg::NKS, NPW = Cfg::NPW, NPU = Cfg::NPU;
  constexpr int WP = Cfg::WP, KP = Cfg::KP, UP = Cfg::UP;
  __shared__ __attribute__((aligned(16))) typename Cfg::Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const bool loader = wv >= NWC;
  const int tl = tid - 64 * NWC;                 // loader thread index
  const int64_t H = a.H, HV = a.HV, V = a.V, N = a.N;
  const int64_t nvt = V / BV;
  const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t vt = bid % nvt, j = (bid / nvt) % HV, n = bid / (nvt * HV);
  if (n >= N) return;
  const int64_t h = j / (HV / H);
  const int64_t vw = vt * BV;                    // workgroup's first value column
  const int64_t v0 = vw + 16 * wv;               // compute wave's first value column
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ wbase = static_cast<const T*>(a.w);
  const T* __restrict__ ubase = static_cast<const T*>(a.u);
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
    const T* krow = kp + (R.t0 * H + h) * K;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tl + NTL * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      const bool in = (NPW % NTL == 0) || idx < NPW;
      // rows past L load row L-1 (a valid address) and are zeroed by a select
      const int tc = t < R.L ? t : R.L - 1;
      const Frag<T> kr = ld8(krow + (tc * (int)(H * K) + d8));
      R.w[i] = in ? ld8(wp + 8 * idx) : frag_zero<T>();
      R.k[i] = (in && t < R.L) ? kr : frag_zero<T>();
    }
    const T* up = ubase + ((c * HV + j) * V + vw) * (int64_t)C;
#pragma unroll
    for (int i = 0; i < NLU; ++i) {
      const int idx = tl + NTL * i;
      R.u[i] = ((NPU % NTL == 0) || idx < NPU) ? ld8(up + 8 * idx) : frag_zero<T>();
    }
    const float* ksp = a.kscale + (c * HV + j) * (int64_t)(C + 4);
    R.ks = (tl < NKS) ? *reinterpret_cast<const f32x4*>(ksp + 4 * tl) : zero4();
  };
  auto stage = [&](const Regs& R, int b) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tl + NTL * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      if ((NPW % NTL == 0) || idx < NPW) {
        st8(&sm.w[b][t * WP + d8], R.w[i]);
        st8(&sm.k[b][t * KP + d8], R.k[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < NLU; ++i) {
      const int idx = tl + NTL * i, v = idx / (C / 8), t8 = (idx % (C / 8)) * 8;
      if ((NPU % NTL == 0) || idx < NPU) st8(&sm.u[b][v * UP + t8], R.u[i]);
    }
    if (tl < NKS) *reinterpret_cast<f32x4*>(&sm.ks[b][4 * tl]) = R.ks;
  };

  // The loader and compute waves run separate loops with the same sequence of
  // barriers (one per chunk step), so neither carries the other's registers.
  // Chunk c_begin + x lives in register slot x % 3 and LDS buffer x % 2; at
  // step s the compute waves work on chunk s while the loaders stage chunk s + 1
  // and fetch chunk s + 4 (indices clamped to the last chunk; extra copies are
  // staged but never computed).
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
        lds_barrier();
        stage(R2, (s0 + 2) & 1);
        fetch(R2, cl(c_begin + s0 + 5));
        lds_barrier();
        stage(R0, (s0 + 3) & 1);
        fetch(R0, cl(c_begin + s0 + 6));
        lds_barrier();
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
    const T* urow = &sm.u[b][(16 * wv + r16) * UP];
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) E[eb] = ld4f(urow + 16 * eb + 4 * g4);
    f32x4 sc[NE];
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) sc[eb] = *reinterpret_cast<const f32x4*>(&sm.ks[b][16 * eb + 4 * g4]);
    const float gl = sm.ks[b][C];
    // h[c] = S (transposed, 4 features per lane)
    T* hp = hbase + ((c * HV + j) * V + v0) * (int64_t)K;
#pragma unroll
    for (int m = 0; m < NS / 2; ++m) st_pair(hp + (r16 * K + 32 * m), S[2 * m], S[2 * m + 1], lane);
    // e = u - w S  (independent accumulators alternate between MFMAs)
    Frag<T> nS[KSK];
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks) nS[ks] = frag_from_halves<T>(-S[2 * ks], -S[2 * ks + 1]);
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks)
#pragma unroll
      for (int eb = 0; eb < NE; ++eb) mma(E[eb], wf[ks][eb], nS[ks]);
    // v_new = e (transposed per chunk)
    T* vnp = vnbase + ((c * HV + j) * V + v0) * (int64_t)C;
#pragma unroll
    for (int m = 0; m < NE / 2; ++m) st_pair(vnp + (r16 * C + 32 * m), E[2 * m], E[2 * m + 1], lane);
    // S <- exp(G_L) S + k^T diag(exp(G_L - G_t) / |k_t|) e
    Frag<T> Ef[KSC];
#pragma unroll
    for (int kt = 0; kt < KSC; ++kt) Ef[kt] = frag_from_halves<T>(E[2 * kt] * sc[2 * kt], E[2 * kt + 1] * sc[2 * kt + 1]);
#pragma unroll
    for (int mb = 0; mb < NS; ++mb) S[mb] *= gl;
#pragma unroll
    for (int kt = 0; kt < KSC; ++kt)
#pragma unroll
      for (int mb = 0; mb < NS; ++mb) mma(S[mb], kf[kt][mb], Ef[kt]);
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

template <typename T, int C, int K, bool PC>
hipError_t launch_t(const Args& a, hipStream_t s) {
  if constexpr (!PC) {
    // warp-specialised scan: 2 compute + 2 loader waves (4 loader waves when
    // elements are fp32 or K = 256, to keep each loader's payload in registers)
    constexpr int NWL = (sizeof(T) == 4 || K == 256) ? 4 : 2;
    if constexpr (K3S<T, C, K, 2, NWL>::fits) {
      // 32 value columns (two compute waves) per workgroup, or 16 (one) when
      // the 32-column grid would leave compute units idle: the scan's step
      // latency does not shrink with fewer columns, so more workgroups is the
      // only way to use the whole chip on few long sequences
      const int64_t nblk32 = a.N * a.HV * (a.V / 32);
      if (nblk32 < kNumCUs) {
        hipLaunchKernelGGL((k3_scan<T, C, K, 1, NWL>), dim3((unsigned)(2 * nblk32)), dim3(64 * (1 + NWL)), 0, s, a);
      } else {
        hipLaunchKernelGGL((k3_scan<T, C, K, 2, NWL>), dim3((unsigned)nblk32), dim3(64 * (2 + NWL)), 0, s, a);
      }
      return hipGetLastError();
    }
  }
  // per-channel gate (and shapes whose double-buffered tiles exceed LDS):
  // two waves (32 value columns) per workgroup
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

}  // namespace

hipError_t launch_fwd_h(const Args& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  return a.dtype == GDR_BF16 ? launch_c<bf16>(a, s) : launch_c<float>(a, s);
}

}  // namespace gdr
