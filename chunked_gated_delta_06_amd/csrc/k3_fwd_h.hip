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
// columns); wave w owns 16 columns of S as eight (K/16) 16x16 fp32 MFMA
// accumulators that never leave registers.  Per chunk:
//  * w and the raw keys are staged token-major in LDS (coalesced 16-byte
//    loads); u arrives straight from its per-chunk transposed layout;
//  * e = u - w S on bf16 MFMA, with S fed as the B operand directly from its
//    accumulator layout (the "chained" contraction map);
//  * the S update k^T e reads k^T from LDS with ds_read_b64_tr_b16 and takes e
//    from the previous MFMA's accumulators, again without a round trip;
//  * a scalar gate and the key norm scale the rows of e in fp32, keeping the
//    raw keys exact; a per-channel gate scales the key tile element-wise;
//  * h is written transposed (h^T, 8-byte stores of four features) for the
//    output kernel; e is written per-chunk transposed (v_new).
//  * consecutive workgroups of one head are mapped to one XCD so the shared
//    w / k tiles hit the same L2.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

template <typename T, int C, int K, bool PC, int NW>
__global__ __launch_bounds__(64 * NW) void k3_fwd_h(FwdArgs a) {
  constexpr int NE = C / 16;        // token blocks of e
  constexpr int NS = K / 16;        // feature blocks of S
  constexpr int KSK = K / 32;       // feature slabs
  constexpr int KSC = C / 32;       // token slabs
  constexpr int PADE = 16 / sizeof(T);
  constexpr int KP = K + PADE;
  constexpr int CPR = K / 8;
  constexpr int GP = K + 1;
  constexpr int BV = 16 * NW;
  __shared__ __attribute__((aligned(16))) T sW[C * KP];
  __shared__ __attribute__((aligned(16))) T sK[C * KP];
  __shared__ float sSc[C], sRn[C];
  __shared__ float sDec[PC ? K : 1];
  __shared__ float sGc[PC ? C * GP : 1];
  __shared__ float sGL;

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

  const int32_t c_begin = a.chunk_off[n], c_end = a.chunk_off[n + 1];
  for (int64_t c = c_begin; c < c_end; ++c) {
    const int64_t t0 = a.chunk_idx[4 * c + 1];
    const int L = a.chunk_idx[4 * c + 2];
    const T* wp = wbase + (c * HV + j) * (int64_t)(C * K);

    // ---- stage w, k and the gate factors of chunk c
    if constexpr (PC) {
      for (int idx = tid; idx < C * K; idx += 64 * NW) {
        const int t = idx / K, d = idx % K;
        sGc[t * GP + d] = (t < L) ? a.g[((t0 + t) * HV + j) * K + d] : 0.f;
      }
      __syncthreads();
      for (int d = tid; d < K; d += 64 * NW) {
        float run = 0.f;
        for (int t = 0; t < C; ++t) {
          run += sGc[t * GP + d];
          sGc[t * GP + d] = run;
        }
        sDec[d] = __expf(run);
      }
      __syncthreads();
    }
    for (int idx = tid; idx < C * CPR; idx += 64 * NW) {
      const int t = idx / CPR, d8 = (idx % CPR) * 8;
      st8(&sW[t * KP + d8], ld8(wp + t * K + d8));
      Frag<T> f = (t < L) ? ld8(kp + ((t0 + t) * H + h) * K + d8) : frag_zero<T>();
      f32x8 x = f.f32();
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += x[e] * x[e];
      sq = lanes_sum(sq, CPR);
      const float rn = a.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
      if (idx % CPR == 0) sRn[t] = rn;
      if constexpr (PC) {
        const float* Gl = &sGc[(C - 1) * GP];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= rn * __expf(Gl[d8 + e] - sGc[t * GP + d8 + e]);
        f = Frag<T>::make(x);
      }
      st8(&sK[t * KP + d8], f);
    }
    if (!PC && wv == 0) {
      const float gv = (lane < L) ? a.g[(t0 + lane) * HV + j] : 0.f;
      const float G = wave_incl_scan(gv, lane);
      const float GL = __shfl(G, 63, 64);        // padded rows add 0, so lane 63 holds G_L
      if (lane == 0) sGL = __expf(GL);
      if (lane < C) sSc[lane] = __expf(GL - G);
    }
    __syncthreads();

    // ---- h[c] = S (transposed, 4 features per lane)
    T* hp = hbase + ((c * HV + j) * V + v0 + r16) * (int64_t)K;
#pragma unroll
    for (int mb = 0; mb < NS; ++mb) st4(hp + 16 * mb + 4 * g4, S[mb]);

    // ---- e = u - w S
    const T* up = ubase + ((c * HV + j) * V + v0 + r16) * (int64_t)C;
    f32x4 E[NE];
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) E[eb] = ld4f(up + 16 * eb + 4 * g4);
    Frag<T> nS[KSK];
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks) nS[ks] = frag_from_halves<T>(-S[2 * ks], -S[2 * ks + 1]);
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) {
      const T* row = &sW[(16 * eb + r16) * KP];
#pragma unroll
      for (int ks = 0; ks < KSK; ++ks) {
        mma(E[eb], ld_chain(row + 32 * ks + 4 * g4, row + 32 * ks + 16 + 4 * g4), nS[ks]);
      }
    }

    // ---- v_new = e (transposed per chunk)
    T* vnp = vnbase + ((c * HV + j) * V + v0 + r16) * (int64_t)C;
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) st4(vnp + 16 * eb + 4 * g4, E[eb]);

    // ---- S <- diag(exp(G_L)) S + k^T diag(s) e
    Frag<T> Ef[KSC];
#pragma unroll
    for (int kt = 0; kt < KSC; ++kt) {
      f32x4 lo = E[2 * kt], hi = E[2 * kt + 1];
      if constexpr (!PC) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t_lo = 32 * kt + 4 * g4 + i, t_hi = t_lo + 16;
          lo[i] *= sSc[t_lo] * sRn[t_lo];
          hi[i] *= sSc[t_hi] * sRn[t_hi];
        }
      }
      Ef[kt] = frag_from_halves<T>(lo, hi);
    }
    if constexpr (PC) {
#pragma unroll
      for (int mb = 0; mb < NS; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mb][i] *= sDec[16 * mb + 4 * g4 + i];
    } else {
      const float dec = sGL;
#pragma unroll
      for (int mb = 0; mb < NS; ++mb) S[mb] *= dec;
    }
#pragma unroll
    for (int mb = 0; mb < NS; ++mb) {
#pragma unroll
      for (int kt = 0; kt < KSC; ++kt) {
        mma(S[mb], lds_tr_frag(sK, KP, 32 * kt + 4 * g4, 32 * kt + 16 + 4 * g4, 16 * mb, lane), Ef[kt]);
      }
    }
    __syncthreads();
  }

  if (a.ht != nullptr) {
#pragma unroll
    for (int mb = 0; mb < NS; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.ht[((n * HV + j) * K + 16 * mb + 4 * g4 + i) * V + v0 + r16] = S[mb][i];
  }
}

// LDS bytes of one workgroup (the per-channel gate tile dominates in fp32)
template <typename T, int C, int K, bool PC>
constexpr size_t lds_bytes() {
  return 2 * C * (K + 16 / sizeof(T)) * sizeof(T) + (PC ? C * (K + 1) * 4 + K * 4 : 0) + 3 * C * 4;
}

template <typename T, int C, int K, bool PC>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  if constexpr (lds_bytes<T, C, K, PC>() > 160 * 1024) {
    return hipErrorInvalidValue;    // rejected on the host before any launch
  } else if (a.V % 32 == 0) {
    // value columns per workgroup: 32 (two waves) when V allows it
    const int64_t nblk = a.N * a.HV * (a.V / 32);
    hipLaunchKernelGGL((k3_fwd_h<T, C, K, PC, 2>), dim3((unsigned)nblk), dim3(128), 0, s, a);
  } else {
    const int64_t nblk = a.N * a.HV * (a.V / 16);
    hipLaunchKernelGGL((k3_fwd_h<T, C, K, PC, 1>), dim3((unsigned)nblk), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T, int C, bool PC>
hipError_t launch_k(const FwdArgs& a, hipStream_t s) {
  switch (a.K) {
    case 32: return launch_t<T, C, 32, PC>(a, s);
    case 64: return launch_t<T, C, 64, PC>(a, s);
    case 128: return launch_t<T, C, 128, PC>(a, s);
    case 256: return launch_t<T, C, 256, PC>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_c(const FwdArgs& a, hipStream_t s) {
  if (a.C == 32) return a.per_channel ? launch_k<T, 32, true>(a, s) : launch_k<T, 32, false>(a, s);
  return a.per_channel ? launch_k<T, 64, true>(a, s) : launch_k<T, 64, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_h(const FwdArgs& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  return a.dtype == GDR_BF16 ? launch_c<bf16>(a, s) : launch_c<float>(a, s);
}

}  // namespace gdr
