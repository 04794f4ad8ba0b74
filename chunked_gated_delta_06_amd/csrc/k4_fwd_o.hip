// K4: chunk output (chunk_fwd_o).
//
// For one chunk (L rows) and value head j, with h the state entering the chunk
// (K3) and e its corrected values:
//   o_r = scale * [ (exp(G_r) q^_r)^T h + sum_{t<=r} (sum_d q^_rd k^_td exp(G_rd - G_td)) e_t ]
// i.e. O = scale (diag(exp(G)) Q h + (Q K^T o M) E), the output of the chunk
// form on the coverage-matrix page ("FLA operator-kernel correctness testing
// and coverage matrix", section 2) with the decay mask M folded in.
//
// gfx950 mapping: one workgroup per (chunk, value head), wave w owns output
// rows 16 w .. 16 w + 15 and all value columns.  The wave computes P^T blocks
// (K Q^T, causal blocks only) on bf16 MFMA from the raw q / k rows, scales
// them in fp32 (norms, gate, causal mask) and feeds the accumulators straight
// in as the B operand of O^T += e^T P^T ("chained" contraction map); the inter
// part O^T = h^T Q^T reads h^T and the per-chunk transposed e with plain
// 16-byte / 8-byte loads.  Producing O^T leaves each lane four consecutive
// value columns of one token, so o is written with 8-byte stores.  A
// per-channel gate uses a reference row per block so that every exponential
// factor stays <= 1 (diagonal blocks: the middle row, with a per-element
// fallback when the block's gate span is too wide).
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

constexpr float kSpanLimit = 80.f;

template <typename T, int C, int K, bool PC>
__global__ __launch_bounds__(C * 4) void k4_fwd_o(Args a) {
  constexpr int NB = C / 16;
  constexpr int NT = 64 * NB;
  constexpr int KSK = K / 32;
  constexpr int KSC = C / 32;
  constexpr int GP = K + 1;
  constexpr int CPR = K / 8;
  constexpr int VT = sizeof(T) == 2 ? 64 : (K == 256 ? 16 : 32);   // value columns staged per pass
  constexpr int HP = K + 16 / sizeof(T);          // LDS pitch of h^T rows
  constexpr int EP = C + 16 / sizeof(T);          // LDS pitch of e^T rows
  constexpr int KP = K + 16 / sizeof(T);          // LDS pitch of key rows
  constexpr int NHP = (VT * K / 8 + NT - 1) / NT;  // 8-element h pieces per thread
  constexpr int NEP = (VT * C / 8 + NT - 1) / NT;  // 8-element e pieces per thread
  constexpr int NKP = (C * CPR + NT - 1) / NT;     // 8-element key pieces per thread
  __shared__ float sG[C], sRq[C], sRk[C];
  // Per-channel gate: the key tile and the gate's cumsum tile are dead once
  // the P^T blocks and the q rows are in registers, so the h^T / e^T tiles of
  // the value loop reuse their bytes (chunk 32, K = 128: 26 KB of LDS instead
  // of 48 KB, 4 workgroups per CU instead of 3).  With a scalar gate the tiles
  // stay apart (sharing measured slower there).
  constexpr int kKBytes = C * KP * (int)sizeof(T), kGBytes = PC ? C * GP * 4 : 0;
  constexpr int kHBytes = VT * HP * (int)sizeof(T), kEBytes = VT * EP * (int)sizeof(T);
  constexpr int kPre = kKBytes + kGBytes, kLoop = kHBytes + kEBytes;
  constexpr int kBytes = PC ? (kPre > kLoop ? kPre : kLoop) : kLoop + kKBytes;
  __shared__ __attribute__((aligned(16))) char sBuf[kBytes];
  T* const sH = reinterpret_cast<T*>(sBuf);
  T* const sE = reinterpret_cast<T*>(sBuf + kHBytes);
  T* const sK = reinterpret_cast<T*>(sBuf + (PC ? 0 : kLoop));
  float* const sGc = reinterpret_cast<float*>(sBuf + kKBytes);   // per-channel gate only

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const ChunkHead ch = chunk_head(a.HV);
  const int64_t c = ch.c, j = ch.j;
  if (c >= a.chunk_off[a.N]) return;
  const int64_t t0 = a.chunk_idx[4 * c + 1];
  const int L = a.chunk_idx[4 * c + 2];
  const int64_t H = a.H, HV = a.HV, V = a.V, h = j / (HV / H);
  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ hp = static_cast<const T*>(a.h) + (c * HV + j) * V * (int64_t)K;
  const T* __restrict__ ep = static_cast<const T*>(a.v_new) + (c * HV + j) * V * (int64_t)C;
  T* __restrict__ op = static_cast<T*>(a.o);

  auto row8 = [&](const T* base, int row, int ks) -> Frag<T> {
    if (row < L) return ld8(base + ((t0 + row) * H + h) * K + 32 * ks + 8 * g4);
    return frag_zero<T>();
  };

  // ---- every global load the chunk needs before its first MFMA is issued up
  //      front, in the order it is consumed (vector-memory waits complete in
  //      order): the scalar gate, the key tile, this lane's q row, the first
  //      h^T / e^T tile
  const float gv = (!PC && wv == 0 && lane < L) ? a.g[(t0 + lane) * HV + j] : 0.f;
  Frag<T> kreg[NKP];
#pragma unroll
  for (int i = 0; i < NKP; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    kreg[i] = (idx < C * CPR && t < L) ? ld8(kp + ((t0 + t) * H + h) * K + d8) : frag_zero<T>();
  }
  const int rr = 16 * wv + r16;               // this lane's output row
  Frag<T> qf[KSK];
#pragma unroll
  for (int ks = 0; ks < KSK; ++ks) qf[ks] = row8(qp, rr, ks);

  // ---- h^T and e^T tiles of VT value columns: fetched into registers early,
  //      staged into LDS, then read as MFMA A operands
  Frag<T> hreg[NHP], ereg[NEP];
  auto fetch_tile = [&](int64_t v0) {
    const int nv = (V - v0) < VT ? (int)(V - v0) : VT;
    const T* hsrc = hp + v0 * K;
    const T* esrc = ep + v0 * C;
#pragma unroll
    for (int i = 0; i < NHP; ++i) {
      const int idx = tid + NT * i;
      hreg[i] = (idx < nv * K / 8) ? ld8(hsrc + 8 * idx) : frag_zero<T>();
    }
#pragma unroll
    for (int i = 0; i < NEP; ++i) {
      const int idx = tid + NT * i;
      ereg[i] = (idx < nv * C / 8) ? ld8(esrc + 8 * idx) : frag_zero<T>();
    }
  };
  auto stage_tile = [&]() {
#pragma unroll
    for (int i = 0; i < NHP; ++i) {
      const int idx = tid + NT * i;
      if (idx < VT * K / 8) st8(&sH[(idx / (K / 8)) * HP + (idx % (K / 8)) * 8], hreg[i]);
    }
#pragma unroll
    for (int i = 0; i < NEP; ++i) {
      const int idx = tid + NT * i;
      if (idx < VT * C / 8) st8(&sE[(idx / (C / 8)) * EP + (idx % (C / 8)) * 8], ereg[i]);
    }
  };
  fetch_tile(0);

  // ---- gates, norms, key tile
  if constexpr (PC) {
    for (int idx = tid; idx < C * K; idx += 64 * NB) {
      const int t = idx / K, d = idx % K;
      sGc[t * GP + d] = (t < L) ? a.g[((t0 + t) * HV + j) * K + d] : 0.f;
    }
    lds_barrier();
    // chunk-local cumsum down each feature column: all C reads first, the
    // running sum in registers (same order of additions), then the writes
    for (int d = tid; d < K; d += 64 * NB) {
      float col[C];
#pragma unroll
      for (int t = 0; t < C; ++t) col[t] = sGc[t * GP + d];
#pragma unroll
      for (int t = 1; t < C; ++t) col[t] += col[t - 1];
#pragma unroll
      for (int t = 0; t < C; ++t) sGc[t * GP + d] = col[t];
    }
  } else {
    if (wv == 0) {
      const float G = wave_incl_scan(gv, lane);
      if (lane < C) sG[lane] = G;
    }
  }
#pragma unroll
  for (int i = 0; i < NKP; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    const f32x8 x = kreg[i].f32();
    float sk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sk += x[e] * x[e];
    sk = lanes_sum_t<CPR>(sk);
    if (idx < C * CPR) {
      if (d8 == 0) sRk[t] = a.l2norm ? 1.f / sqrtf(sk + kL2Eps) : 1.f;
      st8(&sK[t * KP + d8], kreg[i]);
    }
  }
  {
    float sq = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks) {
      const f32x8 xq = qf[ks].f32();
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += xq[e] * xq[e];
    }
    sq = group4_sum(sq);
    if (g4 == 0) sRq[rr] = a.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
  }
  lds_barrier();
  auto krow8 = [&](int row, int ks) -> Frag<T> { return ld8(&sK[row * KP + 32 * ks + 8 * g4]); };

  // ---- P^T blocks (t-block jb, r-block wv), jb <= wv
  const float rq = sRq[rr];
  f32x4 Pt[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) {
    Pt[jb] = zero4();
    if (jb > wv) continue;
    if constexpr (!PC) {
#pragma unroll
      for (int ks = 0; ks < KSK; ++ks) mma(Pt[jb], krow8(16 * jb + r16, ks), qf[ks]);
    } else {
      bool direct = false;
      int m = 16 * jb + 15;
      if (jb == wv) {
        m = 16 * jb + 8;
        float span = 0.f;
        for (int d = lane; d < K; d += 64)
          span = fmaxf(span, sGc[(16 * jb) * GP + d] - sGc[(16 * jb + 15) * GP + d]);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) span = fmaxf(span, __shfl_xor(span, o, 64));
        direct = span > kSpanLimit;
      }
      if (!direct) {
        const int tk = 16 * jb + r16;
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks) {
          f32x8 xa = krow8(tk, ks).f32(), xb = qf[ks].f32();
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = 32 * ks + 8 * g4 + e;
            const float gm = sGc[m * GP + d];
            xa[e] *= __expf(gm - sGc[tk * GP + d]);
            xb[e] *= __expf(sGc[rr * GP + d] - gm);
          }
          mma_split(Pt[jb], SplitFrag<T>::make(xa), SplitFrag<T>::make(xb));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * jb + 4 * g4 + i;
          float s = 0.f;
          if (t <= rr && rr < L) {
            for (int d = 0; d < K; ++d)
              s += to_float(sK[t * KP + d]) * to_float(qp[((t0 + rr) * H + h) * K + d]) *
                   __expf(sGc[rr * GP + d] - sGc[t * GP + d]);
          }
          Pt[jb][i] = s;
        }
      }
    }
    // scale and mask: P^T[t][rr], t = 16 jb + 4 g4 + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * jb + 4 * g4 + i;
      float f = 0.f;
      if (t <= rr && rr < L) {
        f = rq * sRk[t];
        if (!PC) f *= __expf(sG[rr] - sG[t]);
      }
      Pt[jb][i] *= f;
    }
  }
  // P^T as the B operand of the intra product, kept as a bf16 hi + lo pair
  SplitFrag<T> Pf[KSC];
#pragma unroll
  for (int kt = 0; kt < KSC; ++kt) Pf[kt] = SplitFrag<T>::make(cat8(Pt[2 * kt], Pt[2 * kt + 1]));

  // q rows for the inter part: raw q (scalar gate, exact) or exp(G_r) q_r
  // (per-channel gate, as a hi + lo pair)
  SplitFrag<T> qi[KSK];
#pragma unroll
  for (int ks = 0; ks < KSK; ++ks) {
    f32x8 x = qf[ks].f32();
    if constexpr (PC) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= __expf(sGc[rr * GP + 32 * ks + 8 * g4 + e]);
      qi[ks] = SplitFrag<T>::make(x);
    } else {
      qi[ks].hi = qf[ks];
      qi[ks].lo = frag_zero<T>();
    }
  }
  const float inter_scale = rq * (PC ? 1.f : __expf(sG[rr]));
  const float sc = a.scale;

  // ---- O^T = h^T Q^T (scaled) + e^T P^T, 16 value columns at a time
  if constexpr (PC) lds_barrier();   // every wave's reads of the key and gate tiles are done
  for (int64_t v0 = 0; v0 < V; v0 += VT) {
  stage_tile();
  lds_barrier();
  if (v0 + VT < V) fetch_tile(v0 + VT);
  const int nvb = ((V - v0) < VT ? (int)(V - v0) : VT) / 16;
  auto o_block = [&](int vbl) {
    f32x4 acc = zero4();
    const T* hrow = &sH[(16 * vbl + r16) * HP];
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks) {
      if constexpr (PC) {
        mma_split(acc, ld8(hrow + 32 * ks + 8 * g4), qi[ks]);
      } else {
        mma(acc, ld8(hrow + 32 * ks + 8 * g4), qi[ks].hi);
      }
    }
    acc *= inter_scale;
    const T* erow = &sE[(16 * vbl + r16) * EP];
#pragma unroll
    for (int kt = 0; kt < KSC; ++kt) {
      if (2 * kt > wv) continue;
      mma_split(acc, ld_chain(erow + 32 * kt + 4 * g4, erow + 32 * kt + 16 + 4 * g4), Pf[kt]);
    }
    return acc * sc;
  };
  T* orow = op + ((t0 + rr) * HV + j) * V + v0;
  if constexpr (VT >= 32) {
    // value blocks paired into 16-byte stores (nvb is even: V is a multiple of 32)
    for (int vbl = 0; vbl < nvb; vbl += 2) {
      const f32x4 x = o_block(vbl), y = o_block(vbl + 1);
      if (rr < L) st_pair(orow + 16 * vbl, x, y, lane);
    }
  } else {
    for (int vbl = 0; vbl < nvb; ++vbl) {
      const f32x4 x = o_block(vbl);
      if (rr < L) st4(orow + 16 * vbl + 4 * g4, x);
    }
  }
  lds_barrier();
  }
}

template <typename T, int C, int K, bool PC>
hipError_t launch_t(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL((k4_fwd_o<T, C, K, PC>), dim3((unsigned)(a.NTmax * a.HV)), dim3(C * 4), 0, s, a);
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

hipError_t launch_fwd_o(const Args& a, hipStream_t s) {
  if (a.NTmax == 0) return hipSuccess;
  return a.dtype == GDR_BF16 ? launch_c<bf16>(a, s) : launch_c<float>(a, s);
}

}  // namespace gdr
