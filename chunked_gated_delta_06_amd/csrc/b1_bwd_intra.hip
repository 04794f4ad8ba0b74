// B1: chunk-local part of the value gradient (bwd, intra-chunk).
//
// Backward of o = scale [ diag(exp(G)) Q^ h + (Q^ K^T o M) E ] with respect to
// the corrected values E of the same chunk:
//   de_local = scale P^T dO,   P[r][t] = q^_r . k^_t exp(G_r - G_t)  (t <= r)
// and the row factors of the inter term that the reverse state scan needs:
//   qscale[r] = scale exp(G_r) / |q_r|          (0 past the chunk end)
// (chunk form of the coverage-matrix page, "FLA operator-kernel correctness
// testing and coverage matrix", section 2, differentiated through o).
//
// gfx950 mapping: one workgroup per (chunk, value head), wave w owns tokens
// t = 16 w .. 16 w + 15 of de_local.  The q and k tiles are read once per
// workgroup (all loads issued before the first wait) and staged in LDS; the
// wave computes its column blocks of P from the raw bf16 q / k rows on MFMA,
// applies norms, gate and causal mask in fp32 and feeds the accumulators as
// the A operand (rows t) of
// de_local = P^T dO in the "chained" contraction map, as a bf16 hi + lo pair;
// dO is staged through LDS 32 value columns at a time and read with
// transposed LDS reads.  The result leaves each lane four consecutive tokens
// of one value column, which is the transposed per-chunk layout of
// de_local, written with 8-byte stores.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

// largest diagonal-block gate span for the reference-row form of P
constexpr float kSpanLimit = 80.f;

template <typename T, int C, int K>
__global__ __launch_bounds__(C * 4) void b1_bwd_intra(Args a) {
  constexpr int NB = C / 16;
  constexpr int NT = 64 * NB;
  constexpr int KSK = K / 32;
  constexpr int KSC = C / 32;
  constexpr int CPR = K / 8;
  constexpr int VT = 32;                          // value columns per pass
  constexpr int DP = VT + 32 / sizeof(T);         // LDS pitch of dO rows
  constexpr int KP = K + 16 / sizeof(T);          // LDS pitch of q / k rows
  constexpr int NPD = VT * C / 8 / NT;            // 8-element dO pieces per thread (= 1)
  constexpr int NPK = (C * CPR + NT - 1) / NT;     // 8-element q / k pieces per thread
  static_assert(NPD * NT * 8 == VT * C, "dO tile pieces");
  __shared__ __attribute__((aligned(16))) float sG[C];
  __shared__ __attribute__((aligned(16))) float sRq[C];
  __shared__ __attribute__((aligned(16))) float sRk[C];
  __shared__ __attribute__((aligned(16))) T sDO[C * DP];
  __shared__ __attribute__((aligned(16))) T sQ[C * KP];
  __shared__ __attribute__((aligned(16))) T sK[C * KP];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const ChunkHead ch = chunk_head(a.HV);
  const int64_t c = ch.c, j = ch.j;
  if (c >= a.chunk_off[a.N]) return;
  const int64_t t0 = a.chunk_idx[4 * c + 1];
  const int L = a.chunk_idx[4 * c + 2];
  const int64_t H = a.H, HV = a.HV, V = a.V, h = j / (HV / H);
  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ dop = static_cast<const T*>(a.d_o);
  T* __restrict__ dep = static_cast<T*>(a.de_local) + (c * HV + j) * V * (int64_t)C;

  // ---- every global load of the chunk is issued up front: the gate, the q
  //      and k tiles (each read once, coalesced) and the first dO tile
  const float gv = (wv == 0 && lane < L) ? a.g[(t0 + lane) * HV + j] : 0.f;
  Frag<T> qreg[NPK], kreg[NPK];
#pragma unroll
  for (int i = 0; i < NPK; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    const bool in = idx < C * CPR && t < L;
    qreg[i] = in ? ld8(qp + ((t0 + t) * H + h) * K + d8) : frag_zero<T>();
    kreg[i] = in ? ld8(kp + ((t0 + t) * H + h) * K + d8) : frag_zero<T>();
  }
  // dO tile (rows t, VT value columns from v0)
  Frag<T> dreg[NPD];
  auto fetch_tile = [&](int64_t v0) {
#pragma unroll
    for (int i = 0; i < NPD; ++i) {
      const int idx = tid + NT * i, t = idx / (VT / 8), v8 = (idx % (VT / 8)) * 8;
      dreg[i] = (t < L) ? ld8(dop + ((t0 + t) * HV + j) * V + v0 + v8) : frag_zero<T>();
    }
  };
  auto stage_tile = [&]() {
#pragma unroll
    for (int i = 0; i < NPD; ++i) {
      const int idx = tid + NT * i, t = idx / (VT / 8), v8 = (idx % (VT / 8)) * 8;
      st8(&sDO[t * DP + v8], dreg[i]);
    }
  };
  fetch_tile(0);

  // ---- gate cumsum; q / k tiles into LDS with their row norms
  if (wv == 0) {
    const float G = wave_incl_scan(gv, lane);
    if (lane < C) sG[lane] = G;
  }
#pragma unroll
  for (int i = 0; i < NPK; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    const f32x8 xq = qreg[i].f32(), xk = kreg[i].f32();
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sq += xq[e] * xq[e];
      sk += xk[e] * xk[e];
    }
    sq = lanes_sum_t<CPR>(sq);
    sk = lanes_sum_t<CPR>(sk);
    if (idx < C * CPR) {
      st8(&sQ[t * KP + d8], qreg[i]);
      st8(&sK[t * KP + d8], kreg[i]);
      if (d8 == 0) {
        sRq[t] = a.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
        sRk[t] = a.l2norm ? 1.f / sqrtf(sk + kL2Eps) : 1.f;
      }
    }
  }
  lds_barrier();
  const int rr = 16 * wv + r16;
  if (g4 == 0)
    a.qscale[(c * HV + j) * C + rr] = (rr < L) ? a.scale * __expf(sG[rr]) * sRq[rr] : 0.f;

  // ---- P blocks (r-block rb, t-block wv) for rb >= wv: acc[i] = P[16 rb + 4 g + i][16 wv + l % 16]
  const int tt = 16 * wv + r16;           // this lane's token column of P
  const float rkt = sRk[tt], Gt = sG[tt];
  f32x4 Pa[NB];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    Pa[rb] = zero4();
    if (rb < wv) continue;
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks)
      mma(Pa[rb], ld8(&sQ[(16 * rb + r16) * KP + 32 * ks + 8 * g4]), ld8(&sK[tt * KP + 32 * ks + 8 * g4]));
    // the factors of the lane's four consecutive rows in one 16-byte read each
    const f32x4 Rq4 = *reinterpret_cast<const f32x4*>(&sRq[16 * rb + 4 * g4]);
    const f32x4 G4 = *reinterpret_cast<const f32x4*>(&sG[16 * rb + 4 * g4]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rb + 4 * g4 + i;
      Pa[rb][i] *= (tt <= r && r < L) ? Rq4[i] * rkt * __expf(G4[i] - Gt) : 0.f;
    }
  }
  // P^T rows t as A operands over the chained r map, as hi + lo pairs
  SplitFrag<T> Pf[KSC];
#pragma unroll
  for (int s = 0; s < KSC; ++s) Pf[s] = SplitFrag<T>::make(cat8(Pa[2 * s], Pa[2 * s + 1]));

  // ---- de_local^T[v][t] = scale sum_r P[r][t] dO[r][v]
  const float sc = a.scale;
  for (int64_t v0 = 0; v0 < V; v0 += VT) {
    stage_tile();
    lds_barrier();
    if (v0 + VT < V) fetch_tile(v0 + VT);
#pragma unroll
    for (int vb = 0; vb < VT / 16; ++vb) {
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        if (2 * s + 1 < wv) continue;     // r < 16 wv in the whole slab: P is zero
        mma_split(acc, Pf[s], lds_tr_frag(sDO, DP, 32 * s + 4 * g4, 32 * s + 16 + 4 * g4, 16 * vb, lane));
      }
      // acc[i] = de_local[16 wv + 4 g + i][v0 + 16 vb + l % 16]
      st4(dep + (v0 + 16 * vb + r16) * C + 16 * wv + 4 * g4, acc * sc);
    }
    lds_barrier();
  }
}

// Per-channel gate (chunk 32): the same de_local, with
//   P[r][t] = sum_d q^_rd k^_td exp(G_rd - G_td)        (t <= r)
// formed on MFMA with a reference row per 16 x 16 block (as the forward's
// per-channel K1 forms kk^T), and, for the reverse scan, the chunk's gated
// operand rows and decay
//   kt[t][d] = exp(G_Ld - G_td) k^_td      qg[t][d] = scale exp(G_td) q^_td
//   dl[d]    = exp(G_Ld)
// ([NT][HV][C][K] in the input dtype, zero past L; [NT][HV][K] fp32), which
// take the place of the raw rows and the row factors of the scalar gate.
// Four waves: P is split over the threads by (row, token group); de_local
// blocks (token block w % 2, value blocks (w / 2) + 2 i) on MFMA with P^T as a
// bf16 hi + lo pair.
template <typename T, int K>
__global__ __launch_bounds__(256) void b1_bwd_intra_pc(Args a) {
  constexpr int C = 32;
  constexpr int NT = 256;
  constexpr int CPR = K / 8;
  constexpr int VT = 32;
  constexpr int DP = VT + 32 / sizeof(T);
  constexpr int KP = K + 16 / sizeof(T);
  constexpr int GP = K + 1;
  constexpr int PP = C + 32 / sizeof(T);          // P^T rows (hi / lo tiles)
  constexpr int NPK = (C * CPR + NT - 1) / NT;
  constexpr int NPD = (VT * C / 8 + NT - 1) / NT;
  __shared__ float sRq[C], sRk[C];
  __shared__ __attribute__((aligned(16))) float sG[C * GP];
  __shared__ __attribute__((aligned(16))) T sQ[C * KP];
  __shared__ __attribute__((aligned(16))) T sK[C * KP];
  __shared__ __attribute__((aligned(16))) T sDO[C * DP];
  __shared__ __attribute__((aligned(16))) T sPT[2 * C * PP];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const ChunkHead ch = chunk_head(a.HV);
  const int64_t c = ch.c, j = ch.j;
  if (c >= a.chunk_off[a.N]) return;
  const int64_t t0 = a.chunk_idx[4 * c + 1];
  const int L = a.chunk_idx[4 * c + 2];
  const int64_t H = a.H, HV = a.HV, V = a.V, h = j / (HV / H);
  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ dop = static_cast<const T*>(a.d_o);
  T* __restrict__ dep = static_cast<T*>(a.de_local) + (c * HV + j) * V * (int64_t)C;
  T* __restrict__ ktp = static_cast<T*>(a.kt) + (c * HV + j) * (int64_t)(C * K);
  T* __restrict__ qgp = static_cast<T*>(a.qg) + (c * HV + j) * (int64_t)(C * K);
  float* __restrict__ dlp = a.dl + (c * HV + j) * (int64_t)K;
  const FTile<T> fPT = ftile<T, PP>(reinterpret_cast<char*>(sPT), C);

  // ---- loads: q, k rows, the gate tile, the first dO tile
  Frag<T> qreg[NPK], kreg[NPK];
#pragma unroll
  for (int i = 0; i < NPK; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    const bool in = idx < C * CPR && t < L;
    qreg[i] = in ? ld8(qp + ((t0 + t) * H + h) * K + d8) : frag_zero<T>();
    kreg[i] = in ? ld8(kp + ((t0 + t) * H + h) * K + d8) : frag_zero<T>();
  }
  for (int idx = tid; idx < C * K / 4; idx += NT) {
    const int t = idx / (K / 4), d4 = (idx % (K / 4)) * 4;
    const f32x4 gv = (t < L) ? *reinterpret_cast<const f32x4*>(a.g + ((t0 + t) * HV + j) * K + d4) : zero4();
#pragma unroll
    for (int e = 0; e < 4; ++e) sG[t * GP + d4 + e] = gv[e];
  }
  Frag<T> dreg[NPD];
  auto fetch_tile = [&](int64_t v0) {
#pragma unroll
    for (int i = 0; i < NPD; ++i) {
      const int idx = tid + NT * i, t = idx / (VT / 8), v8 = (idx % (VT / 8)) * 8;
      dreg[i] = (idx < VT * C / 8 && t < L) ? ld8(dop + ((t0 + t) * HV + j) * V + v0 + v8) : frag_zero<T>();
    }
  };
  fetch_tile(0);

  // ---- q / k tiles and their row norms; the gate cumsum down each column
#pragma unroll
  for (int i = 0; i < NPK; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    const f32x8 xq = qreg[i].f32(), xk = kreg[i].f32();
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sq += xq[e] * xq[e];
      sk += xk[e] * xk[e];
    }
    sq = lanes_sum_t<CPR>(sq);
    sk = lanes_sum_t<CPR>(sk);
    if (idx < C * CPR) {
      st8(&sQ[t * KP + d8], qreg[i]);
      st8(&sK[t * KP + d8], kreg[i]);
      if (d8 == 0) {
        sRq[t] = a.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
        sRk[t] = a.l2norm ? 1.f / sqrtf(sk + kL2Eps) : 1.f;
      }
    }
  }
  lds_barrier();
  for (int d = tid; d < K; d += NT) {
    float col[C];
#pragma unroll
    for (int t = 0; t < C; ++t) col[t] = sG[t * GP + d];
#pragma unroll
    for (int t = 1; t < C; ++t) col[t] += col[t - 1];
#pragma unroll
    for (int t = 0; t < C; ++t) sG[t * GP + d] = col[t];
  }
  lds_barrier();

  // ---- the reverse scan's operands: kt, qg (zero past L) and dl
  const float* GL = &sG[(L - 1) * GP];
#pragma unroll
  for (int i = 0; i < NPK; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    if (idx < C * CPR) {
      f32x8 xk = kreg[i].f32(), xq = qreg[i].f32();
      const float rk = sRk[t], rq = sRq[t] * a.scale;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gt = sG[t * GP + d8 + e];
        xk[e] = (t < L) ? xk[e] * rk * __expf(GL[d8 + e] - gt) : 0.f;
        xq[e] = (t < L) ? xq[e] * rq * __expf(gt) : 0.f;
      }
      st8(ktp + t * K + d8, Frag<T>::make(xk));
      st8(qgp + t * K + d8, Frag<T>::make(xq));
    }
  }
  for (int d = tid; d < K; d += NT) dlp[d] = __expf(GL[d]);

  // ---- P^T[t][r] = rq_r rk_t sum_d q_rd k_td exp(G_rd - G_td), t <= r < L:
  //      the lower-triangular 16 x 16 blocks (r block rb, t block cb <= rb)
  //      on MFMA, one per wave, with a reference row m per block so that both
  //      gated operands carry factors exp(+-(G - G_m)) <= 1 (off-diagonal: the
  //      last row of the t block; diagonal: the middle row while the block's
  //      gate span keeps every factor below e^80, else per-element
  //      exponentials); operands as bf16 hi + lo pairs.  The block above the
  //      diagonal is zero.
  {
    constexpr int NB = C / 16, KS = K / 32;
    int bi = 0;
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb, ++bi) {
        if (bi % 4 != wv) continue;
        f32x4 sp = zero4();
        if (cb <= rb) {
          bool direct = false;
          int m = 16 * cb + 15;
          if (cb == rb) {
            m = 16 * rb + 8;
            float span = 0.f;
            for (int d = lane; d < K; d += 64)
              span = fmaxf(span, sG[(16 * rb) * GP + d] - sG[(16 * rb + 15) * GP + d]);
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) span = fmaxf(span, __shfl_xor(span, o, 64));
            direct = span > kSpanLimit;
          }
          const int ra = 16 * rb + r16, rc = 16 * cb + r16;
          if (!direct) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              const int d0 = 32 * ks + 8 * g4;
              f32x8 xq = ld8(&sQ[ra * KP + d0]).f32(), xk = ld8(&sK[rc * KP + d0]).f32();
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float gm = sG[m * GP + d0 + e];
                xq[e] *= __expf(sG[ra * GP + d0 + e] - gm);
                xk[e] *= __expf(gm - sG[rc * GP + d0 + e]);
              }
              // element i of lane (r16, g4): row r = 16 rb + 4 g4 + i, token t = 16 cb + r16
              mma_split(sp, SplitFrag<T>::make(xq), SplitFrag<T>::make(xk));
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 16 * rb + 4 * g4 + i, t = 16 * cb + r16;
              float sum = 0.f;
              if (t <= r && r < L) {
                for (int d = 0; d < K; ++d)
                  sum += to_float(sQ[r * KP + d]) * to_float(sK[t * KP + d]) * __expf(sG[r * GP + d] - sG[t * GP + d]);
              }
              sp[i] = sum;
            }
          }
          const int t = 16 * cb + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * rb + 4 * g4 + i;
            sp[i] = (t <= r && r < L) ? sp[i] * sRq[r] * sRk[t] : 0.f;
          }
        }
        fPT.put4(16 * cb + r16, 16 * rb + 4 * g4, sp);
      }
    }
  }

  // ---- de_local^T[v][t] = scale sum_r P^T[t][r] dO[r][v]
  const int tb = wv & 1;
  const float sc = a.scale;
  for (int64_t v0 = 0; v0 < V; v0 += VT) {
#pragma unroll
    for (int i = 0; i < NPD; ++i) {
      const int idx = tid + NT * i, t = idx / (VT / 8), v8 = (idx % (VT / 8)) * 8;
      if (idx < VT * C / 8) st8(&sDO[t * DP + v8], dreg[i]);
    }
    lds_barrier();
    if (v0 + VT < V) fetch_tile(v0 + VT);
    {
      const int vb = wv >> 1;
      f32x4 acc = zero4();
      mma_split(acc, fPT.row(16 * tb + r16, 0, lane), lds_col8(sDO, DP, 0, 16 * vb, lane));
      st4(dep + (v0 + 16 * vb + r16) * C + 16 * tb + 4 * g4, acc * sc);
    }
    lds_barrier();
  }
}

template <typename T>
hipError_t launch_pc(const Args& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.NTmax * a.HV));
  switch (a.K) {
    case 32: hipLaunchKernelGGL((b1_bwd_intra_pc<T, 32>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((b1_bwd_intra_pc<T, 64>), grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((b1_bwd_intra_pc<T, 128>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int C>
hipError_t launch_k(const Args& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.NTmax * a.HV));
  switch (a.K) {
    case 32: hipLaunchKernelGGL((b1_bwd_intra<T, C, 32>), grid, dim3(C * 4), 0, s, a); break;
    case 64: hipLaunchKernelGGL((b1_bwd_intra<T, C, 64>), grid, dim3(C * 4), 0, s, a); break;
    case 128: hipLaunchKernelGGL((b1_bwd_intra<T, C, 128>), grid, dim3(C * 4), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_c(const Args& a, hipStream_t s) {
  return a.C == 32 ? launch_k<T, 32>(a, s) : launch_k<T, 64>(a, s);
}

}  // namespace

hipError_t launch_bwd_intra(const Args& a, hipStream_t s) {
  if (a.NTmax == 0) return hipSuccess;
  if (a.per_channel) {
    if (a.C != 32) return hipErrorInvalidValue;
    return a.dtype == GDR_BF16 ? launch_pc<bf16>(a, s) : launch_pc<float>(a, s);
  }
  return a.dtype == GDR_BF16 ? launch_c<bf16>(a, s) : launch_c<float>(a, s);
}

}  // namespace gdr
