// K1: intra-chunk kk^T and triangular inverse.
//
// For one chunk (L <= C rows) and one value head j, with G the chunk-local
// inclusive cumsum of the gate and k^ the (optionally L2-normalised) keys:
//   A[r][c] = beta_r * sum_d k^_rd k^_cd exp(G_rd - G_cd)   for c < r
//   Tm      = (I + A)^-1                                     (unit lower triangular)
// which is the first half of the WY construction of the DeltaNet chunk form
// on the coverage-matrix page ("FLA operator-kernel correctness testing and
// coverage matrix", section 2) with the gate folded in.
//
// gfx950 mapping (one wave per chunk):
//  * kk^T on bf16 MFMA (fp32 accumulate) with the raw input keys, which are
//    exact in bf16; the L2 norm, beta and a scalar gate enter afterwards as
//    fp32 row / column factors, so normalised keys are never rounded.  Under
//    GVA (HV > H) the raw kk^T is computed once per q/k head and reused for the
//    HV/H value heads of the group.
//  * Per-channel gates sit inside the contraction: each 16x16 block uses a
//    reference row m so both operands carry factors exp(+-(G - G_m)) <= 1
//    (off-diagonal: m = last row of the column block).  Diagonal blocks use
//    m = the block's middle row when the block's gate span keeps every factor
//    below e^80; otherwise that block falls back to per-element exponentials.
//  * (I + A)^-1 in fp32: the 16x16 diagonal blocks by forward substitution
//    (one lane per column, four blocks in parallel), then block forward
//    substitution T_ib = -T_ii sum_m A_im T_mb on fp32 MFMA, in place in LDS.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

constexpr float kSpanLimit = 80.f;

template <typename T, int C, int K, bool PC>
__global__ __launch_bounds__(64) void k1_kkt_solve(Args a) {
  constexpr int NB = C / 16;                 // 16-row blocks per chunk
  constexpr int KS = K / 32;                 // contraction slabs
  constexpr int NLB = NB * (NB + 1) / 2;     // lower-triangular blocks
  constexpr int GP = K + 1;                  // LDS pitch of the per-channel gate tile
  // A, then T, in fp32: only the lower-triangular 16 x 16 blocks are ever
  // touched, so they are stored packed (block (rb, cb <= rb) at index
  // rb (rb + 1) / 2 + cb, rows of 17 floats), which keeps the workgroup's LDS
  // small enough for more single-wave workgroups per CU
  // A per-channel gate's cumsum tile is last read by the kk^T products, and A
  // is held in registers until then, so A / T reuse the tile's bytes (one
  // value head per workgroup: the tile is never needed again)
  constexpr int kMFloats = NLB * 16 * 17, kGFloats = PC ? C * GP : 0;
  __shared__ float sMG[kMFloats > kGFloats ? kMFloats : kGFloats];
  float* const sM = sMG;
  float* const sGc = sMG;   // per-channel gate only
  // block (rb, cb) base; element (i, k) of a block at base + 17 i + k
  auto blk = [](int rb, int cb) { return (rb * (rb + 1) / 2 + cb) * (16 * 17); };
  __shared__ float sG[C], sBeta[C], sRn[C];

  const int lane = threadIdx.x, r16 = lane & 15, g4 = lane >> 4;
  const int64_t NG = PC ? a.HV : a.H;    // workgroups per chunk
  const ChunkHead ch = chunk_head(NG);
  const int64_t c = ch.c;
  if (c >= a.chunk_off[a.N]) return;
  const int64_t t0 = a.chunk_idx[4 * c + 1];
  const int L = a.chunk_idx[4 * c + 2];
  const int64_t H = a.H, HV = a.HV, GR = HV / H;
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  T* __restrict__ Tout = static_cast<T*>(a.Tm);

  // value heads handled by this workgroup: the whole GVA group (scalar gate) or one
  const int64_t jfirst = PC ? ch.j : ch.j * GR;
  const int64_t jcount = PC ? 1 : GR;
  const int64_t h = jfirst / GR;

  auto krow = [&](int row, int ks) -> Frag<T> {
    if (row < L) return ld8(kp + ((t0 + row) * H + h) * K + 32 * ks + 8 * g4);
    return frag_zero<T>();
  };

  // the first value head's gate and beta are requested together with the
  // keys, so their latency overlaps the kk^T products
  auto fetch_gb = [&](int64_t j, float& gv, float& bv) {
    gv = (!PC && lane < L) ? a.g[(t0 + lane) * HV + j] : 0.f;
    bv = (lane < L) ? beta_value(a.beta[(t0 + lane) * HV + j], a.beta_logits) : 0.f;
  };
  // (scalar gate: all key fragments at once; a per-channel gate re-reads the
  // keys block by block below and loads them per slab here)
  Frag<T> kf[PC ? 1 : KS][NB];
  if constexpr (!PC) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) kf[ks][rb] = krow(16 * rb + r16, ks);
  }
  float gnext, bnext;
  fetch_gb(jfirst, gnext, bnext);

  // ---- raw kk^T (scalar gate) and row norms
  f32x4 acc[NLB];
#pragma unroll
  for (int i = 0; i < NLB; ++i) acc[i] = zero4();
  float ss[NB];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) ss[rb] = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    Frag<T> f[NB];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      if constexpr (PC) {
        f[rb] = krow(16 * rb + r16, ks);
      } else {
        f[rb] = kf[ks][rb];
      }
      const f32x8 x = f[rb].f32();
#pragma unroll
      for (int e = 0; e < 8; ++e) ss[rb] += x[e] * x[e];
    }
    if constexpr (!PC) {
#pragma unroll
      for (int rb = 0; rb < NB; ++rb)
#pragma unroll
        for (int cb = 0; cb <= rb; ++cb) mma(acc[rb * (rb + 1) / 2 + cb], f[rb], f[cb]);
    }
  }
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const float tot = group4_sum(ss[rb]);
    if (g4 == 0) sRn[16 * rb + r16] = a.l2norm ? 1.f / sqrtf(tot + kL2Eps) : 1.f;
  }

  for (int64_t jj = 0; jj < jcount; ++jj) {
    const int64_t j = jfirst + jj;
    // ---- gates: chunk-local inclusive cumsum, one token per lane
    const float gv = gnext, bv = bnext;
    if (jj + 1 < jcount) fetch_gb(j + 1, gnext, bnext);
    const float Gc = PC ? 0.f : wave_incl_scan(gv, lane);
    if (lane < C) {
      sG[lane] = Gc;
      sBeta[lane] = bv;
    }
    if constexpr (PC) {
      // per-channel gate tile, then cumsum along the tokens of every channel
      for (int idx = lane; idx < C * K; idx += 64) {
        const int t = idx / K, d = idx % K;
        sGc[t * GP + d] = (t < L) ? a.g[((t0 + t) * HV + j) * K + d] : 0.f;
      }
      lds_barrier();
      // chunk-local cumsum down each feature column: all C reads first, the
      // running sum in registers (same order of additions), then the writes
      for (int d = lane; d < K; d += 64) {
        float col[C];
#pragma unroll
        for (int t = 0; t < C; ++t) col[t] = sGc[t * GP + d];
#pragma unroll
        for (int t = 1; t < C; ++t) col[t] += col[t - 1];
#pragma unroll
        for (int t = 0; t < C; ++t) sGc[t * GP + d] = col[t];
      }
      lds_barrier();
      // gated kk^T, block by block, with a reference row per block
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
        for (int cb = 0; cb <= rb; ++cb) {
          f32x4 s = zero4();
          bool direct = false;
          int m = 16 * cb + 15;
          if (cb == rb) {
            m = 16 * rb + 8;
            float span = 0.f;
            for (int d = lane; d < K; d += 64)
              span = fmaxf(span, sGc[(16 * rb) * GP + d] - sGc[(16 * rb + 15) * GP + d]);
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) span = fmaxf(span, __shfl_xor(span, o, 64));
            direct = span > kSpanLimit;
          }
          if (!direct) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              f32x8 xa = krow(16 * rb + r16, ks).f32(), xb = krow(16 * cb + r16, ks).f32();
              const int ra = 16 * rb + r16, rbw = 16 * cb + r16;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int d = 32 * ks + 8 * g4 + e;
                const float gm = sGc[m * GP + d];
                xa[e] *= __expf(sGc[ra * GP + d] - gm);
                xb[e] *= __expf(gm - sGc[rbw * GP + d]);
              }
              mma(s, Frag<T>::make(xa), Frag<T>::make(xb));
            }
          } else {
            // per-element exponentials for a block whose gate span is too wide
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 16 * rb + 4 * g4 + i, cc = 16 * cb + r16;
              float sum = 0.f;
              if (cc < r && r < L) {
                for (int d = 0; d < K; ++d)
                  sum += to_float(kp[((t0 + r) * H + h) * K + d]) * to_float(kp[((t0 + cc) * H + h) * K + d]) *
                         __expf(sGc[r * GP + d] - sGc[cc * GP + d]);
              }
              s[i] = sum;
            }
          }
          acc[rb * (rb + 1) / 2 + cb] = s;
        }
      }
    }
    lds_barrier();

    // ---- A into LDS (strictly lower, fp32)
#pragma unroll
    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
      for (int cb = 0; cb <= rb; ++cb) {
        const f32x4 s = acc[rb * (rb + 1) / 2 + cb];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rb + 4 * g4 + i, cc = 16 * cb + r16;
          float val = 0.f;
          if (cc < r && r < L) {
            val = sBeta[r] * s[i] * sRn[r] * sRn[cc];
            if (!PC) val *= __expf(sG[r] - sG[cc]);
          }
          sM[blk(rb, cb) + (4 * g4 + i) * 17 + r16] = val;
        }
      }
    lds_barrier();

    // ---- diagonal 16x16 inverses by forward substitution (lane = column)
    float x[16];
    const int db = g4;
    float* Md = sM + blk(db < NB ? db : 0, db < NB ? db : 0);
    if (db < NB) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = (r == r16) ? 1.f : 0.f;
#pragma unroll
        for (int q = 0; q < r; ++q) s -= Md[r * 17 + q] * x[q];
        x[r] = s;
      }
    }
    lds_barrier();
    if (db < NB) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Md[r * 17 + r16] = x[r];
    }
    lds_barrier();

    // ---- block forward substitution: T_ib = -T_ii * sum_{m=b}^{i-1} A_im T_mb
#pragma unroll
    for (int ib = 1; ib < NB; ++ib) {
      f32x4 res[NB > 1 ? NB - 1 : 1];
#pragma unroll
      for (int jb = 0; jb < ib; ++jb) {
        f32x4 X = zero4();
#pragma unroll
        for (int mb = jb; mb < ib; ++mb) {
          float av[4], bvv[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            av[s] = sM[blk(ib, mb) + r16 * 17 + 4 * g4 + s];
            bvv[s] = sM[blk(mb, jb) + (4 * g4 + s) * 17 + r16];
          }
          mma16_f32(X, av, bvv);
        }
        float tv[4], xv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          tv[s] = sM[blk(ib, ib) + r16 * 17 + 4 * g4 + s];
          xv[s] = X[s];
        }
        f32x4 Y = zero4();
        mma16_f32(Y, tv, xv);
        res[jb] = -Y;
      }
      lds_barrier();
#pragma unroll
      for (int jb = 0; jb < ib; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sM[blk(ib, jb) + (4 * g4 + i) * 17 + r16] = res[jb][i];
      lds_barrier();
    }

    // ---- per-token factors of the chunk (layout at kscale_pitch): the ones
    //      the state scan applies to the rows of e, kscale[t] = exp(G_L - G_t)
    //      / |k_t| and exp(G_L), then G_t and 1 / |k_t| for the fused output
    if constexpr (!PC) {
      if (a.kscale != nullptr) {
        float* ks = a.kscale + (c * HV + j) * kscale_pitch(C);
        const float GL = __shfl(Gc, 63, 64);     // padded lanes add 0, so lane 63 holds G_L
        if (lane < C) {
          ks[lane] = (lane < L) ? __expf(GL - Gc) * sRn[lane] : 0.f;
          ks[C + 4 + lane] = (lane < L) ? Gc : 0.f;
          ks[2 * C + 4 + lane] = (lane < L) ? sRn[lane] : 0.f;
        }
        if (lane < 4) ks[C + lane] = (lane == 0) ? __expf(GL) : 0.f;
      }
    }

    // ---- store Tm (rows / cols past L and the upper triangle are zero)
    T* dst = Tout + (c * HV + j) * (int64_t)(C * C);
    for (int idx = lane; idx < C * C / 8; idx += 64) {
      const int r = idx / (C / 8), c8 = (idx % (C / 8)) * 8;
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int cc = c8 + e;
        x[e] = (r < L && cc <= r) ? sM[blk(r >> 4, cc >> 4) + (r & 15) * 17 + (cc & 15)] : 0.f;
      }
      st8(dst + r * C + c8, Frag<T>::make(x));
    }
    lds_barrier();
  }
}

template <typename T, int C, int K, bool PC>
hipError_t launch_t(const Args& a, hipStream_t s) {
  const unsigned gy = (unsigned)(PC ? a.HV : a.H);
  hipLaunchKernelGGL((k1_kkt_solve<T, C, K, PC>), dim3((unsigned)(a.NTmax * gy)), dim3(64), 0, s, a);
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

hipError_t launch_kkt_solve(const Args& a, hipStream_t s) {
  if (a.NTmax == 0) return hipSuccess;
  return a.dtype == GDR_BF16 ? launch_c<bf16>(a, s) : launch_c<float>(a, s);
}

}  // namespace gdr
