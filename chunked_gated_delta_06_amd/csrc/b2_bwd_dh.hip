// B2: reverse state-gradient scan (bwd_dhu).
//
// For each sequence n and value head j, dS (K x V, fp32) starts at dht (or 0)
// and runs over the chunks from last to first:
//   dh[c] = dS                                   (gradient of the state leaving
//            chunk c: the hand-off of the KCP page, "flash-linear-attention
//            KCP precision-failure root-cause manual", section "h and dh
//            cross-rank semantics", which passes dht back to the previous rank)
//   dE    = de_local + diag(kscale) K dS         (gradient of the chunk's e)
//   dS   <- exp(G_L) dS + Q^T diag(qscale) dO - W^T dE
// and dh0 = dS at the end, with kscale[t] = exp(G_L - G_t) / |k_t| and
// qscale[r] = scale exp(G_r) / |q_r|.  This is the transpose of the forward
// recursion S <- exp(G_L) S + K~^T (U - W S) of the chunk form on the
// coverage-matrix page ("FLA operator-kernel correctness testing and coverage
// matrix", section 2) plus the inter term of o.  dh is stored in fp32 for
// every input dtype: the gate gradient sums products of h and dh over whole
// K x V states, where a bf16 dh would cost it about a third of its error
// budget.
//
// gfx950 mapping (as the forward scan): one workgroup per (sequence, value
// head, 32 value columns, or 16 when that fills the chip better).  Each
// compute wave owns 16 columns of dS as
// K/16 fp32 MFMA accumulators; NWL loader waves fetch each chunk's k, q, w,
// dO, de_local and kscale into registers three steps ahead and stage them into
// LDS (two buffers when they fit, else one with a second barrier per step);
// dO is multiplied by qscale while it is staged.  dE = K dS takes dS straight
// from its accumulators as the B operand (chained contraction map); the dS
// update reads q^T and w^T with transposed LDS reads.
//
// Per-channel gate (PC): the chunk's gate enters every feature separately,
//   dE = de_local + Kt dS,   dS <- diag(exp(G_L)) dS + Qg^T dO - W^T dE,
// with the gated rows kt = exp(G_L - G_t) k^_t and qg = scale exp(G_t) q^_t and
// the decay dl = exp(G_L) that the intra-chunk stage wrote per chunk; they take
// the place of the raw rows and the row factors kscale / qscale.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

template <typename T, int C, int K, int NWC_, int NWL, bool PC = false>
struct B2S {
  static constexpr int NWC = NWC_;
  static constexpr int NTL = 64 * NWL;
  static constexpr int BV = 16 * NWC;
  static constexpr int NE = C / 16, NS = K / 16, KSK = K / 32, KSC = C / 32;
  static constexpr int CPR = K / 8;
  static constexpr int NPW = C * CPR;                   // 8-element pieces of a C x K tile
  static constexpr int NLD = (NPW + NTL - 1) / NTL;
  static constexpr int NPO = C * BV / 8;                // dO pieces
  static constexpr int NLO = (NPO + NTL - 1) / NTL;
  static constexpr int NPE = BV * C / 8;                // de_local pieces
  static constexpr int NLE = (NPE + NTL - 1) / NTL;
  static constexpr int NKS = PC ? K / 4 : (C + 4) / 4;   // float4 pieces of the row factors / decay
  static constexpr int KSN = PC ? K : C + 4;
  static constexpr int KR = K + 16 / sizeof(T);         // k rows (row reads)
  static constexpr int KP = K + 32 / sizeof(T);         // q, w rows (transposed reads)
  static constexpr int OP = BV + 32 / sizeof(T);        // scaled dO rows (transposed reads)
  static constexpr int EP = C + 8 / sizeof(T);          // de_local rows (one per value column)
  static constexpr size_t buf_bytes =
      ((size_t)C * (KR + 2 * KP) + (size_t)C * OP + (size_t)BV * EP) * sizeof(T) + KSN * 4;
  static constexpr int NBUF = 2 * buf_bytes <= 160 * 1024 ? 2 : 1;
  static constexpr bool fits = NBUF * buf_bytes <= 160 * 1024 && NKS <= NTL;
  // dh staging: the compute waves leave each step's dh (fp32, one row of K
  // features per value column) in one of two LDS buffers and the loader waves
  // store it during the next step, so the compute waves issue no
  // vector-memory instructions (stores behind the loaders' loads would stall
  // their MFMA chains).  Used for 16-bit inputs when both buffers fit beside
  // the tiles (the fp32 loaders have no registers to spare for it).
  // staged dh rows: K floats, unpadded; the 16-byte chunk c of row v sits at
  // chunk c ^ (v % 8), so the compute waves' 16-byte writes of 16 rows spread
  // over the banks
  static constexpr int HSP = K;
  static constexpr size_t stg_bytes = (size_t)BV * HSP * 4;
  static constexpr bool STG = sizeof(T) == 2 && NBUF == 2 && 2 * (buf_bytes + stg_bytes) <= 160 * 1024;
  static constexpr int NDH = (BV * K / 4 + NTL - 1) / NTL;   // staged float4 pieces per loader thread

  struct Regs {
    Frag<T> k[NLD], q[NLD], w[NLD];
    Frag<T> o[NLO];
    float qs[NLO];
    Frag<T> e[NLE];
    f32x4 ks;
    int L;
  };
  struct Smem {
    T k[NBUF][C * KR];
    T q[NBUF][C * KP];
    T w[NBUF][C * KP];
    T o[NBUF][C * OP];
    T e[NBUF][BV * EP];
    float ks[NBUF][KSN];
    __attribute__((aligned(16))) float hs[STG ? 2 : 1][STG ? BV * HSP : 4];
  };
};

template <typename T, int C, int K, int NWC_, int NWL, bool PC = false>
__global__ __launch_bounds__(64 * (NWC_ + NWL)) void b2_bwd_dh(Args a) {
  using Cfg = B2S<T, C, K, NWC_, NWL, PC>;
  using Regs = typename Cfg::Regs;
  constexpr int NWC = Cfg::NWC, NTL = Cfg::NTL, BV = Cfg::BV, NE = Cfg::NE, NS = Cfg::NS;
  constexpr int KSK = Cfg::KSK, KSC = Cfg::KSC, CPR = Cfg::CPR, NLD = Cfg::NLD, NLO = Cfg::NLO;
  constexpr int NLE = Cfg::NLE, NKS = Cfg::NKS, NPW = Cfg::NPW, NPO = Cfg::NPO, NPE = Cfg::NPE;
  constexpr int KR = Cfg::KR, KP = Cfg::KP, OP = Cfg::OP, EP = Cfg::EP, NBUF = Cfg::NBUF;
  constexpr bool STG = Cfg::STG;
  constexpr int HSP = Cfg::HSP, NDH = Cfg::NDH;
  __shared__ __attribute__((aligned(16))) typename Cfg::Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const bool loader = wv >= NWC;
  const int tl = tid - 64 * NWC;
  const int64_t H = a.H, HV = a.HV, V = a.V, N = a.N;
  const int64_t nvt = V / BV;
  const ScanUnit su = scan_unit(a.seq_order, N, HV, nvt);
  const int64_t vt = su.vt, j = su.j, n = su.n;
  if (n >= N) return;
  const int64_t h = j / (HV / H);
  const int64_t vw = vt * BV;
  const int64_t v0 = vw + 16 * wv;
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const T* __restrict__ wbase = static_cast<const T*>(a.w);
  const T* __restrict__ dop = static_cast<const T*>(a.d_o);
  const T* __restrict__ debase = static_cast<const T*>(a.de_local);
  float* __restrict__ dhbase = static_cast<float*>(a.dh);

  const int64_t c_begin = a.chunk_off[n];
  const int nc = a.chunk_off[n + 1] - (int)c_begin;
  const int64_t c_last = c_begin + (nc > 0 ? nc - 1 : 0);
  // step x works on chunk c_last - x; indices past the first chunk are clamped
  // to it (those copies are staged but never computed)
  auto chunk_at = [&](int x) -> int64_t { return x < nc ? c_last - x : c_begin; };
  const int64_t seq_t0 = nc > 0 ? a.chunk_idx[4 * c_begin + 1] : 0;
  const int64_t seq_end = nc > 0 ? a.chunk_idx[4 * c_last + 1] + a.chunk_idx[4 * c_last + 2] : 0;

  auto fetch = [&](Regs& R, int64_t c) {
    const int64_t t0 = seq_t0 + (c - c_begin) * C;
    const int L = (int)((seq_end - t0) < C ? (seq_end - t0) : C);
    const T* wp = wbase + (c * HV + j) * (int64_t)(C * K);
    // scalar gate: raw rows of the input; per-channel: the chunk's gated rows
    const T* krow = PC ? static_cast<const T*>(a.kt) + (c * HV + j) * (int64_t)(C * K) : kp + (t0 * H + h) * K;
    const T* qrow = PC ? static_cast<const T*>(a.qg) + (c * HV + j) * (int64_t)(C * K) : qp + (t0 * H + h) * K;
    const int rstride = PC ? K : (int)(H * K);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tl + NTL * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      const bool in = (NPW % NTL == 0) || idx < NPW;
      // Only loads here (the payload is first read when staged, so the
      // in-order vector-memory counter leaves the later payloads in flight);
      // rows past L load row L-1 and are zeroed when staged, pieces past the
      // tile load piece 0 and are never staged.
      const int tc = t < L ? t : L - 1;
      R.k[i] = ld8(krow + (tc * rstride + d8));
      R.q[i] = ld8(qrow + (tc * rstride + d8));
      R.w[i] = ld8(wp + 8 * (in ? idx : 0));
    }
    const T* orow = dop + (t0 * HV + j) * V + vw;
    const float* qsp = a.qscale + (c * HV + j) * (int64_t)C;
#pragma unroll
    for (int i = 0; i < NLO; ++i) {
      const int idx = tl + NTL * i, t = idx / (BV / 8), v8 = (idx % (BV / 8)) * 8;
      const bool in = (NPO % NTL == 0) || idx < NPO;
      const int tc = t < L ? t : L - 1;
      R.o[i] = ld8(orow + (tc * (int)(HV * V) + v8));
      R.qs[i] = PC ? 1.f : qsp[tc];
    }
    const T* ep = debase + ((c * HV + j) * V + vw) * (int64_t)C;
#pragma unroll
    for (int i = 0; i < NLE; ++i) {
      const int idx = tl + NTL * i;
      R.e[i] = ld8(ep + 8 * (((NPE % NTL == 0) || idx < NPE) ? idx : 0));
    }
    const float* ksp = PC ? a.dl + (c * HV + j) * (int64_t)K : a.kscale + (c * HV + j) * kscale_pitch(C);
    R.ks = *reinterpret_cast<const f32x4*>(ksp + 4 * (tl < NKS ? tl : 0));
    R.L = L;
  };
  auto stage = [&](const Regs& R, int b) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tl + NTL * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      if ((NPW % NTL == 0) || idx < NPW) {
        st8(&sm.k[b][t * KR + d8], t < R.L ? R.k[i] : frag_zero<T>());
        st8(&sm.q[b][t * KP + d8], t < R.L ? R.q[i] : frag_zero<T>());
        st8(&sm.w[b][t * KP + d8], R.w[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < NLO; ++i) {
      const int idx = tl + NTL * i, t = idx / (BV / 8), v8 = (idx % (BV / 8)) * 8;
      // rows past L: a zero row factor (the loaded row is a finite copy of row
      // L-1); per-channel: the gated q rows past L are zero instead
      const float qs = t < R.L ? R.qs[i] : 0.f;
      if ((NPO % NTL == 0) || idx < NPO) st8(&sm.o[b][t * OP + v8], PC ? R.o[i] : Frag<T>::make(R.o[i].f32() * qs));
    }
#pragma unroll
    for (int i = 0; i < NLE; ++i) {
      const int idx = tl + NTL * i, v = idx / (C / 8), t8 = (idx % (C / 8)) * 8;
      if ((NPE % NTL == 0) || idx < NPE) st8(&sm.e[b][v * EP + t8], R.e[i]);
    }
    if (tl < NKS) *reinterpret_cast<f32x4*>(&sm.ks[b][4 * tl]) = R.ks;
  };

  // staged dh of step x (buffer x % 2) to global memory: the workgroup's BV
  // rows of K features are contiguous in dh[c]
  auto drain = [&](int x) {
    float* hp = dhbase + ((chunk_at(x) * HV + j) * V + vw) * (int64_t)K;
    f32x4 hv[NDH];
#pragma unroll
    for (int i = 0; i < NDH; ++i) {
      const int idx = tl + NTL * i, v = idx / (K / 4), c4 = idx % (K / 4);
      if ((BV * K / 4) % NTL == 0 || idx < BV * K / 4)
        hv[i] = *reinterpret_cast<const f32x4*>(&sm.hs[x & 1][v * HSP + 4 * (c4 ^ (v & 7))]);
    }
#pragma unroll
    for (int i = 0; i < NDH; ++i) {
      const int idx = tl + NTL * i;
      if ((BV * K / 4) % NTL == 0 || idx < BV * K / 4) *reinterpret_cast<f32x4*>(hp + 4 * idx) = hv[i];
    }
  };

  // Loader and compute waves run separate loops with the same barrier
  // sequence.  Step x lives in register slot x % 3 and LDS buffer x % NBUF; at
  // step s the compute waves work on step s while the loaders stage step s + 1
  // (after a second barrier when there is one buffer), fetch step s + 4 and,
  // with dh staging, store the dh that step s - 1 left in LDS.
  if (loader) {
    if (nc > 0) {
      Regs R0, R1, R2;
      fetch(R0, chunk_at(0));
      fetch(R1, chunk_at(1));
      fetch(R2, chunk_at(2));
      stage(R0, 0);
      fetch(R0, chunk_at(3));
      lds_barrier();
      for (int s0 = 0; s0 < nc; s0 += 3) {
        if constexpr (NBUF == 1) lds_barrier();
        stage(R1, (s0 + 1) % NBUF);
        fetch(R1, chunk_at(s0 + 4));
        if constexpr (STG) {
          if (s0 > 0) drain(s0 - 1);
        }
        lds_barrier();
        if constexpr (NBUF == 1) lds_barrier();
        stage(R2, (s0 + 2) % NBUF);
        fetch(R2, chunk_at(s0 + 5));
        if constexpr (STG) drain(s0);
        lds_barrier();
        if constexpr (NBUF == 1) lds_barrier();
        stage(R0, (s0 + 3) % NBUF);
        fetch(R0, chunk_at(s0 + 6));
        if constexpr (STG) {
          if (s0 + 1 < nc) drain(s0 + 1);
        }
        lds_barrier();
      }
      // the last step's dh when the loop ended right after it
      if constexpr (STG) {
        if (nc % 3 == 0) drain(nc - 1);
      }
    }
    return;
  }

  // ---- compute waves: dS rows 16 mb + 4 g4 + i, column v0 + r16
  f32x4 S[NS];
#pragma unroll
  for (int mb = 0; mb < NS; ++mb) {
    if (a.dht != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mb][i] = a.dht[((n * HV + j) * K + 16 * mb + 4 * g4 + i) * V + v0 + r16];
    } else {
      S[mb] = zero4();
    }
  }
  auto compute = [&](int64_t c, int b) {
    Frag<T> kf[KSK][NE];
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks)
#pragma unroll
      for (int eb = 0; eb < NE; ++eb) {
        const T* row = &sm.k[b][(16 * eb + r16) * KR];
        kf[ks][eb] = ld_chain(row + 32 * ks + 4 * g4, row + 32 * ks + 16 + 4 * g4);
      }
    f32x4 sc[NE], dl[NE];
    const T* erow = &sm.e[b][(16 * wv + r16) * EP];
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) {
      sc[eb] = PC ? f32x4{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4*>(&sm.ks[b][16 * eb + 4 * g4]);
      dl[eb] = ld4f(erow + 16 * eb + 4 * g4);
    }
    const float gl = PC ? 1.f : sm.ks[b][C];
    // dh[c] = dS (fp32, transposed): staged for the loaders (buffer b = the
    // step's parity), or stored with feature blocks paired into 16-byte stores
    if constexpr (STG) {
      float* hs = &sm.hs[b][(16 * wv + r16) * HSP];
#pragma unroll
      for (int mb = 0; mb < NS; ++mb) *reinterpret_cast<f32x4*>(hs + 4 * ((4 * mb + g4) ^ (r16 & 7))) = S[mb];
    } else {
      float* hp = dhbase + ((c * HV + j) * V + v0) * (int64_t)K;
#pragma unroll
      for (int m = 0; m < NS / 2; ++m) st_pair(hp + (r16 * K + 32 * m), S[2 * m], S[2 * m + 1], lane);
    }
    // dE = de_local + diag(kscale) K dS
    Frag<T> Sf[KSK];
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks) Sf[ks] = frag_from_halves<T>(S[2 * ks], S[2 * ks + 1]);
    f32x4 E[NE];
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) E[eb] = zero4();
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks)
#pragma unroll
      for (int eb = 0; eb < NE; ++eb) mma(E[eb], kf[ks][eb], Sf[ks]);
    Frag<T> nE[KSC];
#pragma unroll
    for (int kt = 0; kt < KSC; ++kt)
      nE[kt] = frag_from_halves<T>(-(E[2 * kt] * sc[2 * kt] + dl[2 * kt]),
                                   -(E[2 * kt + 1] * sc[2 * kt + 1] + dl[2 * kt + 1]));
    // dS <- exp(G_L) dS + Q^T diag(qscale) dO - W^T dE (per-channel: row d of
    // dS decays by exp(G_Ld))
    if constexpr (PC) {
#pragma unroll
      for (int mb = 0; mb < NS; ++mb) S[mb] *= *reinterpret_cast<const f32x4*>(&sm.ks[b][16 * mb + 4 * g4]);
    } else {
#pragma unroll
      for (int mb = 0; mb < NS; ++mb) S[mb] *= gl;
    }
#pragma unroll
    for (int mb = 0; mb < NS; ++mb)
#pragma unroll
      for (int kt = 0; kt < KSC; ++kt) {
        const int r0 = 32 * kt + 4 * g4, r1 = 32 * kt + 16 + 4 * g4;
        mma(S[mb], lds_tr_frag(&sm.q[b][0], KP, r0, r1, 16 * mb, lane),
            lds_tr_frag(&sm.o[b][0], OP, r0, r1, 16 * wv, lane));
        mma(S[mb], lds_tr_frag(&sm.w[b][0], KP, r0, r1, 16 * mb, lane), nE[kt]);
      }
  };

  if (nc > 0) {
    lds_barrier();
    for (int s0 = 0; s0 < nc; s0 += 3) {
      compute(chunk_at(s0), s0 % NBUF);
      lds_barrier();
      if constexpr (NBUF == 1) lds_barrier();
      if (s0 + 1 < nc) compute(chunk_at(s0 + 1), (s0 + 1) % NBUF);
      lds_barrier();
      if constexpr (NBUF == 1) lds_barrier();
      if (s0 + 2 < nc) compute(chunk_at(s0 + 2), (s0 + 2) % NBUF);
      lds_barrier();
      if constexpr (NBUF == 1) lds_barrier();
    }
  }
  if (a.dh0 != nullptr) {
#pragma unroll
    for (int mb = 0; mb < NS; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.dh0[((n * HV + j) * K + 16 * mb + 4 * g4 + i) * V + v0 + r16] = S[mb][i];
  }
}

template <typename T, int C, int K>
constexpr int loader_waves() {
  // about 150 VGPRs of prefetch per loader thread (three payloads of three
  // C x K tiles)
  constexpr int x = (int)sizeof(T) * C * K / 4096;
  return x < 2 ? 2 : (x > 8 ? 8 : x);
}

template <typename T, int C, int K, bool PC = false>
hipError_t launch_t(const Args& a, hipStream_t s) {
  constexpr int NWL = loader_waves<T, C, K>();
  if constexpr (!B2S<T, C, K, 2, NWL, PC>::fits) {
    return hipErrorInvalidValue;    // rejected on the host before any launch
  } else {
    // 32 value columns per workgroup, or 16 when the 32-column grid would
    // leave compute units idle (as the forward scan), or 64 (four compute and
    // four loader waves, 16-bit inputs) when the 64-column grid still gives
    // every compute unit a workgroup and its tiles fit: the 32-column grid
    // would then run in two rounds of one workgroup per compute unit
    const int64_t nblk32 = a.N * a.HV * (a.V / 32);
    if constexpr (sizeof(T) == 2 && B2S<T, C, K, 4, 4, PC>::STG) {
      if (a.V % 64 == 0 && nblk32 / 2 >= kNumCUs && 2 * B2S<T, C, K, 2, NWL, PC>::buf_bytes +
                                                          2 * B2S<T, C, K, 2, NWL, PC>::stg_bytes > 80 * 1024) {
        hipLaunchKernelGGL((b2_bwd_dh<T, C, K, 4, 4, PC>), dim3((unsigned)(nblk32 / 2)), dim3(64 * 8), 0, s, a);
        return hipGetLastError();
      }
    }
    if (nblk32 < kNumCUs) {
      hipLaunchKernelGGL((b2_bwd_dh<T, C, K, 1, NWL, PC>), dim3((unsigned)(2 * nblk32)), dim3(64 * (1 + NWL)), 0, s,
                         a);
    } else {
      hipLaunchKernelGGL((b2_bwd_dh<T, C, K, 2, NWL, PC>), dim3((unsigned)nblk32), dim3(64 * (2 + NWL)), 0, s, a);
    }
    return hipGetLastError();
  }
}

template <typename T, int C>
hipError_t launch_k(const Args& a, hipStream_t s) {
  switch (a.K) {
    case 32: return launch_t<T, C, 32>(a, s);
    case 64: return launch_t<T, C, 64>(a, s);
    case 128: return launch_t<T, C, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

// per-channel gate: chunk 32 (the backward runs a chunk-64 problem at 32)
template <typename T>
hipError_t launch_pc(const Args& a, hipStream_t s) {
  if (a.C != 32) return hipErrorInvalidValue;
  switch (a.K) {
    case 32: return launch_t<T, 32, 32, true>(a, s);
    case 64: return launch_t<T, 32, 64, true>(a, s);
    case 128: return launch_t<T, 32, 128, true>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_c(const Args& a, hipStream_t s) {
  if (a.per_channel) return launch_pc<T>(a, s);
  return a.C == 32 ? launch_k<T, 32>(a, s) : launch_k<T, 64>(a, s);
}

}  // namespace

bool bwd_scan_fits(int dtype, int C, int K) {
  bool ok = false;
#define GDR_B2_FITS(TT, CC, KK) \
  if (C == CC && K == KK) ok = B2S<TT, CC, KK, 2, loader_waves<TT, CC, KK>()>::fits;
  if (dtype == GDR_BF16) {
    GDR_B2_FITS(bf16, 32, 32) GDR_B2_FITS(bf16, 32, 64) GDR_B2_FITS(bf16, 32, 128)
    GDR_B2_FITS(bf16, 64, 32) GDR_B2_FITS(bf16, 64, 64) GDR_B2_FITS(bf16, 64, 128)
  } else {
    GDR_B2_FITS(float, 32, 32) GDR_B2_FITS(float, 32, 64) GDR_B2_FITS(float, 32, 128)
    GDR_B2_FITS(float, 64, 32) GDR_B2_FITS(float, 64, 64) GDR_B2_FITS(float, 64, 128)
  }
#undef GDR_B2_FITS
  return ok;
}

bool bwd_scan_pc_fits(int dtype, int K) {
  if (dtype == GDR_BF16)
    return K == 32 ? B2S<bf16, 32, 32, 2, loader_waves<bf16, 32, 32>(), true>::fits
         : K == 64 ? B2S<bf16, 32, 64, 2, loader_waves<bf16, 32, 64>(), true>::fits
         : K == 128 ? B2S<bf16, 32, 128, 2, loader_waves<bf16, 32, 128>(), true>::fits : false;
  return K == 32 ? B2S<float, 32, 32, 2, loader_waves<float, 32, 32>(), true>::fits
       : K == 64 ? B2S<float, 32, 64, 2, loader_waves<float, 32, 64>(), true>::fits
       : K == 128 ? B2S<float, 32, 128, 2, loader_waves<float, 32, 128>(), true>::fits : false;
}

hipError_t launch_bwd_dh(const Args& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  return a.dtype == GDR_BF16 ? launch_c<bf16>(a, s) : launch_c<float>(a, s);
}

}  // namespace gdr
