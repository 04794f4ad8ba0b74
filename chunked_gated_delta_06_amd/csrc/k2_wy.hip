// K2: WY recompute.
//
// For one chunk and value head, from Tm = (I + A)^-1 (K1):
//   w = Tm (beta * exp(G) * k^)      u = Tm (beta * v)
// (u in fp32 for every input dtype, its operand Tm diag(beta) as a bf16 hi + lo
// pair: the state scan forms e = u - w S from it, and e is much smaller than u
// once the state predicts the values, so a bf16 rounding of u, or of Tm beta,
// lands in e, and from there in every gradient, at a large relative size)
// the WY factors of the DeltaNet chunk form P^r = I - sum_i k^i w^i^T on the
// coverage-matrix page ("FLA operator-kernel correctness testing and coverage
// matrix", section 2), with the gate folded into w.
//
// gfx950 mapping (4 waves per chunk and value head):
//  * the k and v tiles are staged token-major in LDS with coalesced 16-byte
//    loads and read back transposed with ds_read_b64_tr_b16, so both products
//    contract over tokens on bf16 MFMA without a transposing copy;
//  * w is computed as w^T = k^T (Tm diag(s))^T, so each lane ends with four
//    consecutive features of one token (an 8-byte token-major store), and u as
//    Tm diag(beta) v, so each lane ends with four consecutive tokens of one
//    value column (an 8-byte store into the per-chunk transposed u);
//  * with a scalar gate the per-token factor s_t = beta_t exp(G_t) / |k_t|
//    multiplies the columns of Tm, leaving the raw keys exact; a per-channel
//    gate multiplies the key tile element-wise by exp(G_td) <= 1, and (when
//    the caller gives a.kt / a.dl) the stage also writes the state scan's
//    gated keys exp(G_L - G_t) k^_t and decay exp(G_L), so the scan does not
//    form the chunk's gate cumsum in each of its workgroups;
//  * blocks above the diagonal of Tm are skipped (Tm is lower triangular);
//  * every global load of a chunk (keys, the first value pass, Tm rows, g,
//    beta) is issued before the first wait, so a workgroup pays one memory
//    round trip, not four.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

template <typename T, int C, int K, bool PC>
__global__ __launch_bounds__(256) void k2_wy(Args a) {
  constexpr int NW = 4;
  constexpr int NT = 256;
  constexpr int NB = C / 16;
  constexpr int KSC = C / 32;                       // token slabs
  constexpr int PADE = 16 / sizeof(T) * 1;          // 16 bytes of row padding
  constexpr int KP = K + PADE;
  constexpr int VT = sizeof(T) == 2 ? 128 : 64;     // value columns staged per pass
  constexpr int VP = VT + PADE;
  constexpr int GP = K + 1;
  constexpr int CPR = K / 8;                        // 8-element chunks per key row
  constexpr int NKP = (C * CPR + NT - 1) / NT;      // key pieces per thread
  constexpr int NVP = (C * VT / 8 + NT - 1) / NT;   // value pieces per thread and pass
  __shared__ __attribute__((aligned(16))) T sK[C * KP];
  // a per-channel gate's cumsum tile is dead once the decayed key tile is
  // staged, before the first value pass: the value tile reuses its bytes
  constexpr int kVBytes = C * VP * (int)sizeof(T), kGBytes = PC ? C * GP * 4 : 0;
  __shared__ __attribute__((aligned(16))) char sVG[kVBytes > kGBytes ? kVBytes : kGBytes];
  T* const sV = reinterpret_cast<T*>(sVG);
  float* const sGc = reinterpret_cast<float*>(sVG);
  __shared__ float sS[C], sB[C], sRn[C];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const ChunkHead ch = chunk_head(a.HV);
  const int64_t c = ch.c, j = ch.j;
  if (c >= a.chunk_off[a.N]) return;
  const int64_t t0 = a.chunk_idx[4 * c + 1];
  const int L = a.chunk_idx[4 * c + 2];
  const int64_t H = a.H, HV = a.HV, V = a.V, h = j / (HV / H);
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ vp = static_cast<const T*>(a.v);
  const T* __restrict__ Tp = static_cast<const T*>(a.Tm) + (c * HV + j) * (int64_t)(C * C);
  T* __restrict__ wp = static_cast<T*>(a.w) + (c * HV + j) * (int64_t)(C * K);
  float* __restrict__ up = static_cast<float*>(a.u) + (c * HV + j) * (int64_t)C * V;

  // ---- every global load of the chunk is issued up front (one round trip):
  //      key rows, the first value pass, the rows of Tm this lane feeds, g, beta
  Frag<T> kr[NKP], vr[NVP];
  auto fetch_v = [&](int64_t v0) {
    const int nv = (V - v0) < VT ? (int)(V - v0) : VT;
    const int vpr = nv / 8;
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int idx = tid + NT * i, t = idx / vpr, d8 = (idx % vpr) * 8;
      vr[i] = (idx < C * vpr && t < L) ? ld8(vp + ((t0 + t) * HV + j) * V + v0 + d8) : frag_zero<T>();
    }
  };
#pragma unroll
  for (int i = 0; i < NKP; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    kr[i] = (idx < C * CPR && t < L) ? ld8(kp + ((t0 + t) * H + h) * K + d8) : frag_zero<T>();
  }
  fetch_v(0);
  // rows of Tm this lane feeds: row 16 rb + r16, tokens 32 ks + 8 g4 + e
  Frag<T> tf[NB][KSC];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb)
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks)
      tf[rb][ks] = (2 * ks <= rb) ? ld8(Tp + (16 * rb + r16) * C + 32 * ks + 8 * g4) : frag_zero<T>();
  float gv = 0.f, bv = 0.f;
  if (wv == 0 && lane < L) {
    if (!PC) gv = a.g[(t0 + lane) * HV + j];
    bv = beta_value(a.beta[(t0 + lane) * HV + j], a.beta_logits);
  }

  if constexpr (PC) {
    for (int idx = tid; idx < C * K; idx += NT) {
      const int t = idx / K, d = idx % K;
      sGc[t * GP + d] = (t < L) ? a.g[((t0 + t) * HV + j) * K + d] : 0.f;
    }
    lds_barrier();
    // chunk-local cumsum down each feature column: all C reads first, the
    // running sum in registers (same order of additions), then the writes
    for (int d = tid; d < K; d += NT) {
      float col[C];
#pragma unroll
      for (int t = 0; t < C; ++t) col[t] = sGc[t * GP + d];
#pragma unroll
      for (int t = 1; t < C; ++t) col[t] += col[t - 1];
#pragma unroll
      for (int t = 0; t < C; ++t) sGc[t * GP + d] = col[t];
    }
    lds_barrier();
  }

  // key tile (token-major), row norms of the raw keys; with a per-channel gate
  // (and a.kt set) also the state scan's gated key rows exp(G_L - G_t) k^_t
  // (zero past L) and the decay exp(G_L), one float per feature
  T* __restrict__ ktp = (PC && a.kt != nullptr) ? static_cast<T*>(a.kt) + (c * HV + j) * (int64_t)(C * K) : nullptr;
#pragma unroll
  for (int i = 0; i < NKP; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    f32x8 x = kr[i].f32();
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sq += x[e] * x[e];
    sq = lanes_sum_t<CPR>(sq);
    if (idx < C * CPR) {
      const float rn = a.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
      if (d8 == 0) sRn[t] = rn;
      Frag<T> f = kr[i];
      if constexpr (PC) {
        if (ktp != nullptr) {
          f32x8 y;
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = x[e] * rn * __expf(sGc[(L - 1) * GP + d8 + e] - sGc[t * GP + d8 + e]);
          st8(ktp + t * K + d8, Frag<T>::make(y));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= __expf(sGc[t * GP + d8 + e]);
        f = Frag<T>::make(x);
      }
      st8(&sK[t * KP + d8], f);
    }
  }
  if constexpr (PC) {
    if (a.dl != nullptr)
      for (int d = tid; d < K; d += NT) a.dl[(c * HV + j) * K + d] = __expf(sGc[(L - 1) * GP + d]);
  }
  lds_barrier();
  if (wv == 0) {
    const float G = PC ? 0.f : wave_incl_scan(gv, lane);
    if (lane < C) {
      sB[lane] = bv;
      sS[lane] = bv * sRn[lane] * (PC ? 1.f : __expf(G));
    }
  }
  lds_barrier();

  // w^T = k^T (Tm diag(s))^T; with K / 32 feature pairs per wave or more, the
  // blocks (2 p, 2 p + 1) are computed together and leave as 16-byte stores
  auto w_block = [&](int fb, int rb) {
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      if (2 * ks > rb) continue;
      const Frag<T> ka = lds_tr_frag(sK, KP, 32 * ks + 8 * g4, 32 * ks + 8 * g4 + 4, 16 * fb, lane);
      f32x8 sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[e] = sS[32 * ks + 8 * g4 + e];
      mma(acc, ka, Frag<T>::make(tf[rb][ks].f32() * sc));
    }
    return acc;
  };
  if constexpr (K / 32 >= NW) {
    for (int fp = wv; fp < K / 32; fp += NW) {
#pragma unroll
      for (int rb = 0; rb < NB; ++rb)
        st_pair(wp + (16 * rb + r16) * K + 32 * fp, w_block(2 * fp, rb), w_block(2 * fp + 1, rb), lane);
    }
  } else {
    for (int fb = wv; fb < K / 16; fb += NW) {
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) st4(wp + (16 * rb + r16) * K + 16 * fb + 4 * g4, w_block(fb, rb));
    }
  }

  // u = Tm diag(beta) v, value columns staged VT at a time (the next pass's
  // loads are issued while this one is computed)
  for (int64_t v0 = 0; v0 < V; v0 += VT) {
    const int nv = (V - v0) < VT ? (int)(V - v0) : VT;
    const int vpr = nv / 8;
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int idx = tid + NT * i, t = idx / vpr, d8 = (idx % vpr) * 8;
      if (idx < C * vpr) st8(&sV[t * VP + d8], vr[i]);
    }
    lds_barrier();
    if (v0 + VT < V) fetch_v(v0 + VT);
    for (int vb = wv; vb < nv / 16; vb += NW) {
      f32x4 acc[NB];
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        acc[rb] = zero4();
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
          if (2 * ks > rb) continue;
          f32x8 sc;
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[e] = sB[32 * ks + 8 * g4 + e];
          const Frag<T> vbf = lds_tr_frag(sV, VP, 32 * ks + 8 * g4, 32 * ks + 8 * g4 + 4, 16 * vb, lane);
          // the scaled rows of Tm as a hi + lo pair: u keeps ~16 mantissa bits
          mma_split(acc[rb], SplitFrag<T>::make(tf[rb][ks].f32() * sc), vbf);
        }
      }
      // token blocks paired into 16-byte stores of the transposed fp32 u rows
#pragma unroll
      for (int m = 0; m < NB / 2; ++m)
        st_pair(up + (v0 + 16 * vb + r16) * C + 32 * m, acc[2 * m], acc[2 * m + 1], lane);
    }
  }
}

template <typename T, int C, int K, bool PC>
hipError_t launch_t(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL((k2_wy<T, C, K, PC>), dim3((unsigned)(a.NTmax * a.HV)), dim3(256), 0, s, a);
  return hipGetLastError();
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

hipError_t launch_wy(const Args& a, hipStream_t s) {
  if (a.NTmax == 0) return hipSuccess;
  return a.dtype == GDR_BF16 ? launch_c<bf16>(a, s) : launch_c<float>(a, s);
}

}  // namespace gdr
