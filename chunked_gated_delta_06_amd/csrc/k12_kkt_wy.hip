// K1 + K2 fused (scalar gate): intra-chunk kk^T, triangular inverse and the
// WY factors in one pass, with the inverse never leaving the chip.
//
// For one chunk (L <= C rows) and value head j, with G the chunk-local gate
// cumsum and k^ the (optionally L2-normalised) keys:
//   A[r][c] = beta_r (k^_r . k^_c) exp(G_r - G_c)    c < r
//   Tm      = (I + A)^-1
//   w = Tm (beta exp(G) k^)        u = Tm (beta v)
// the WY construction of the DeltaNet chunk form P^r = I - sum_i k^i w^i^T on
// the coverage-matrix page ("FLA operator-kernel correctness testing and
// coverage matrix", section 2) with the gate folded in.  Same results as the
// K1 and K2 stages up to rounding (Tm feeds w and u in fp32 here, not through
// its bf16 copy).  The fused forward's variant writes neither Tm nor a wide u;
// the kept-states variant (KEEP) writes Tm for the backward and u in fp32, its
// operand Tm diag(beta) as a hi + lo pair, as the separate WY stage does.  For simple
// GLA (no delta correction) it yields Tm = I, w = 0 and u = v, so the same scan
// and output stages evaluate S_t = exp(g_t) S_{t-1} + k_t v_t^T.
//
// gfx950 mapping (4 waves per chunk and value head):
//  * the key tile is staged token-major in LDS once (coalesced 16-byte loads)
//    and serves both the kk^T products (row fragments, bf16 MFMA on the raw
//    keys, which are exact) and the w products (transposed reads);
//  * the lower-triangular 16x16 blocks of kk^T are spread over the 4 waves;
//    beta, the norms and exp(G_r - G_c) <= 1 enter as fp32 factors;
//  * (I + A)^-1 in fp32 in LDS: the diagonal blocks by forward substitution
//    (one lane per column), then block forward substitution on fp32 MFMA with
//    the blocks of one block row spread over the waves;
//  * w and u as in K2, with the rows of Tm read from LDS in fp32 and scaled by
//    the per-token factors before the single rounding to the MFMA operand;
//  * every global load of the chunk (keys, first value pass, g, beta) is
//    issued before the first wait;
//  * the value tile shares its LDS with Tm: the rows of Tm go to registers
//    before the first value pass is staged, so with bf16 and chunk 64 a
//    workgroup holds 35 KB of LDS and 128 registers per lane, and four
//    workgroups share a CU (a dense batch's chunks run in whole rounds).
#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

template <typename T, int C, int K, bool KEEP>
__global__ __launch_bounds__(256, sizeof(T) == 2 && !KEEP ? 4 : 1) void k12_kkt_wy(Args a) {
  using UT = typename std::conditional<KEEP, float, T>::type;   // u's storage type
  constexpr int NW = 4;
  constexpr int NT = 256;
  constexpr int NB = C / 16;                        // 16-row blocks per chunk
  constexpr int NLB = NB * (NB + 1) / 2;            // lower-triangular blocks
  constexpr int KSC = C / 32;                       // token slabs
  constexpr int KS = K / 32;                        // feature slabs
  constexpr int PADE = 16 / sizeof(T);              // 16 bytes of row padding
  constexpr int KP = K + PADE;
  constexpr int VT = sizeof(T) == 2 ? 128 : 64;     // value columns staged per pass
  constexpr int VP = VT + PADE;
  constexpr int CPR = K / 8;                        // 8-element pieces per key row
  constexpr int NKP = (C * CPR + NT - 1) / NT;      // key pieces per thread
  constexpr int NVP = (C * VT / 8 + NT - 1) / NT;   // value pieces per thread and pass
  __shared__ __attribute__((aligned(16))) T sK[C * KP];
  // A, then Tm, in fp32: the lower-triangular blocks only, packed (block
  // (rb, cb <= rb) at rb (rb + 1) / 2 + cb, rows of MP floats); the value
  // tile reuses the same bytes once Tm is in registers
  // Rows of MP = 20 floats keep every row 16-byte aligned (T's rows leave as
  // 16-byte reads) and make the column-wise writes of a 64-lane block and the
  // 8-lane phases of those reads bank-conflict free; blocks start MB floats
  // apart, MB = 16 MP + 16, so the four diagonal blocks inverted side by side
  // sit on different banks.
  constexpr int MP = 20, MB = 16 * MP + 16;
  constexpr int kVBytes = C * VP * (int)sizeof(T), kMBytes = NLB * MB * 4;
  __shared__ __attribute__((aligned(16))) char sVM[kVBytes > kMBytes ? kVBytes : kMBytes];
  T* const sV = reinterpret_cast<T*>(sVM);
  float* const sM = reinterpret_cast<float*>(sVM);
  auto blk = [](int rb, int cb) { return (rb * (rb + 1) / 2 + cb) * MB; };
  __shared__ __attribute__((aligned(16))) float sS[C];
  __shared__ __attribute__((aligned(16))) float sB[C];
  __shared__ __attribute__((aligned(16))) float sRn[C];
  __shared__ __attribute__((aligned(16))) float sG[C];

  // the wave index is read into a scalar register, so every per-wave choice
  // below is a scalar branch around whole MFMA sequences
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ChunkHead ch = chunk_head(a.HV);
  const int64_t c = ch.c, j = ch.j;
  int64_t t0;
  int L;
  if (a.table_from_dims) {
    // dense batch: chunk c is chunk c % NC of row c / NC; the first value
    // head's workgroups also write the table for the stages that follow
    const int64_t NC = (a.T + C - 1) / C, n = c / NC, cl = c % NC;
    t0 = n * a.T + cl * C;
    L = (int)((a.T - cl * C) < C ? (a.T - cl * C) : C);
    if (j == 0 && tid == 0) {
      reinterpret_cast<int4*>(a.chunk_idx)[c] = int4{(int32_t)n, (int32_t)t0, L, (int32_t)cl};
      if (c == 0)
        for (int64_t b = 0; b <= a.B; ++b) a.chunk_off[b] = (int32_t)(b * NC);
    }
  } else {
    if (c >= a.chunk_off[a.N]) return;
    t0 = a.chunk_idx[4 * c + 1];
    L = a.chunk_idx[4 * c + 2];
  }
  const int64_t H = a.H, HV = a.HV, V = a.V, h = j / (HV / H);
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ vp = static_cast<const T*>(a.v);
  T* __restrict__ wp = static_cast<T*>(a.w) + (c * HV + j) * (int64_t)(C * K);
  UT* __restrict__ up = static_cast<UT*>(a.u) + (c * HV + j) * (int64_t)C * V;

  // ---- every global load of the chunk up front: key rows, the first value
  //      pass, g and beta
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
  float gv = 0.f, bv = 0.f;
  if (wv == 0 && lane < L) {
    gv = a.g[(t0 + lane) * HV + j];
    bv = a.gla ? 1.f : beta_value(a.beta[(t0 + lane) * HV + j], a.beta_logits);
  }

  // ---- key tile (token-major) and the row norms of the raw keys
#pragma unroll
  for (int i = 0; i < NKP; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    const f32x8 x = kr[i].f32();
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sq += x[e] * x[e];
    sq = lanes_sum_t<CPR>(sq);
    if (idx < C * CPR) {
      if (d8 == 0) sRn[t] = a.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
      st8(&sK[t * KP + d8], kr[i]);
    }
  }
  lds_barrier();

  // ---- gates (wave 0, one token per lane) and the per-token factors
  if (wv == 0) {
    const float Gc = wave_incl_scan(gv, lane);
    if (lane < C) {
      sG[lane] = Gc;
      // simple GLA: u = v (beta = 1 on the chunk's rows) and w = 0
      sB[lane] = a.gla ? (lane < L ? 1.f : 0.f) : bv;
      sS[lane] = a.gla ? 0.f : bv * sRn[lane] * __expf(Gc);
    }
    // kscale row of the chunk (the state scan's and the fused output's
    // factors): exp(G_L - G_t) / |k_t|, exp(G_L) and 3 zeros, G_t, 1 / |k_t|
    float* ks = a.kscale + (c * HV + j) * kscale_pitch(C);
    const float GL = __shfl(Gc, 63, 64);     // padded lanes add 0, so lane 63 holds G_L
    if (lane < C) {
      ks[lane] = (lane < L) ? __expf(GL - Gc) * sRn[lane] : 0.f;
      ks[C + 4 + lane] = (lane < L) ? Gc : 0.f;
      ks[2 * C + 4 + lane] = (lane < L) ? sRn[lane] : 0.f;
    }
    if (lane < 4) ks[C + lane] = (lane == 0) ? __expf(GL) : 0.f;
  }
  lds_barrier();

  // ---- A = beta (k^ k^T) exp(G_r - G_c), strictly lower, blocks over the waves
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
    for (int cb = 0; cb <= rb; ++cb) {
      if ((rb * (rb + 1) / 2 + cb) % NW != wv) continue;
      f32x4 s = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const Frag<T> fa = Frag<T>::raw(*reinterpret_cast<const v8_t<T>*>(&sK[(16 * rb + r16) * KP + 32 * ks + 8 * g4]));
        const Frag<T> fb = Frag<T>::raw(*reinterpret_cast<const v8_t<T>*>(&sK[(16 * cb + r16) * KP + 32 * ks + 8 * g4]));
        mma(s, fa, fb);
      }
      // the block's rows r = 16 rb + 4 g4 + i: their factors in one 16-byte
      // read each; the column's once
      const int r4 = 16 * rb + 4 * g4, cc = 16 * cb + r16;
      const f32x4 B4 = *reinterpret_cast<const f32x4*>(&sB[r4]);
      const f32x4 N4 = *reinterpret_cast<const f32x4*>(&sRn[r4]);
      const f32x4 G4 = *reinterpret_cast<const f32x4*>(&sG[r4]);
      const float nc = sRn[cc], gc = sG[cc];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r4 + i;
        const float val = (!a.gla && cc < r && r < L) ? B4[i] * s[i] * N4[i] * nc * __expf(G4[i] - gc) : 0.f;
        sM[blk(rb, cb) + (4 * g4 + i) * MP + r16] = val;
      }
    }
  }
  lds_barrier();

  // ---- diagonal 16x16 inverses by forward substitution (wave 0, lane = column)
  {
    float x[16];
    const int db = g4;
    float* Md = sM + blk(db < NB ? db : 0, db < NB ? db : 0);
    const bool act = wv == 0 && db < NB;
    if (act) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = (r == r16) ? 1.f : 0.f;
#pragma unroll
        for (int q = 0; q < r; ++q) s -= Md[r * MP + q] * x[q];
        x[r] = s;
      }
    }
    lds_barrier();
    if (act) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Md[r * MP + r16] = x[r];
    }
    lds_barrier();
  }

  // ---- block forward substitution T_ib = -T_ii sum_{m=b}^{i-1} A_im T_mb,
  //      block column jb of block row ib on wave jb
#pragma unroll
  for (int ib = 1; ib < NB; ++ib) {
    f32x4 res = zero4();
    const int jb = wv;
    if (jb < ib) {
      f32x4 X = zero4();
      for (int mb = jb; mb < ib; ++mb) {
        float av[4], bvv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          av[s] = sM[blk(ib, mb) + r16 * MP + 4 * g4 + s];
          bvv[s] = sM[blk(mb, jb) + (4 * g4 + s) * MP + r16];
        }
        mma16_f32(X, av, bvv);
      }
      float tv[4], xv[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        tv[s] = sM[blk(ib, ib) + r16 * MP + 4 * g4 + s];
        xv[s] = X[s];
      }
      f32x4 Y = zero4();
      mma16_f32(Y, tv, xv);
      res = -Y;
    }
    lds_barrier();
    if (jb < ib) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sM[blk(ib, jb) + (4 * g4 + i) * MP + r16] = res[i];
    }
    lds_barrier();
  }

  // ---- Tm itself (kept-states variant; rows / cols past L and the upper
  //      triangle zero)
  if constexpr (KEEP) {
    T* dst = static_cast<T*>(a.Tm) + (c * HV + j) * (int64_t)(C * C);
    for (int idx = tid; idx < C * C / 8; idx += NT) {
      const int r = idx / (C / 8), c8 = (idx % (C / 8)) * 8;
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int cc = c8 + e;
        x[e] = (r < L && cc <= r) ? sM[blk(r >> 4, cc >> 4) + (r & 15) * MP + (cc & 15)] : 0.f;
      }
      st8(dst + r * C + c8, Frag<T>::make(x));
    }
  }

  // ---- rows of Tm this lane feeds (fp32, from LDS): row 16 rb + r16, tokens
  //      32 ks + 8 g4 + e; blocks above the diagonal are zero
  f32x8 tf[NB][KSC];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb)
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      const int cb = 2 * ks + (g4 >> 1);
      const int cbs = cb <= rb ? cb : rb;
      const float* src = sM + blk(rb, cbs) + r16 * MP + 8 * (g4 & 1);
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(src), x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tf[rb][ks][e] = cb <= rb ? x0[e] : 0.f;
        tf[rb][ks][4 + e] = cb <= rb ? x1[e] : 0.f;
      }
    }

  // the first value pass goes to LDS now (its registers are free during the w
  // products); sV shares its LDS with Tm, whose rows every wave has read
  auto stage_v = [&](int64_t v0) {
    const int nv = (V - v0) < VT ? (int)(V - v0) : VT;
    const int vpr = nv / 8;
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int idx = tid + NT * i, t = idx / vpr, d8 = (idx % vpr) * 8;
      if (idx < C * vpr) st8(&sV[t * VP + d8], vr[i]);
    }
  };
  lds_barrier();
  stage_v(0);

  // w^T = k^T (Tm diag(s))^T, s_t = beta_t exp(G_t) / |k_t|
  auto w_block = [&](int fb, int rb) {
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      if (2 * ks > rb) continue;
      const Frag<T> ka = lds_tr_frag(sK, KP, 32 * ks + 8 * g4, 32 * ks + 8 * g4 + 4, 16 * fb, lane);
      f32x8 sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[e] = sS[32 * ks + 8 * g4 + e];
      mma(acc, ka, Frag<T>::make(tf[rb][ks] * sc));
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
    if (v0 > 0) {
      lds_barrier();
      stage_v(v0);
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
          if constexpr (KEEP) {
            mma_split(acc[rb], SplitFrag<T>::make(tf[rb][ks] * sc), vbf);
          } else {
            mma(acc[rb], Frag<T>::make(tf[rb][ks] * sc), vbf);
          }
        }
      }
      // token blocks paired into 16-byte stores of the transposed u rows
#pragma unroll
      for (int m = 0; m < NB / 2; ++m)
        st_pair(up + (v0 + 16 * vb + r16) * C + 32 * m, acc[2 * m], acc[2 * m + 1], lane);
    }
  }
}

template <typename T, int C, int K>
hipError_t launch_t(const Args& a, hipStream_t s) {
  if (a.u_f32)
    hipLaunchKernelGGL((k12_kkt_wy<T, C, K, true>), dim3((unsigned)(a.NTmax * a.HV)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k12_kkt_wy<T, C, K, false>), dim3((unsigned)(a.NTmax * a.HV)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int C>
hipError_t launch_k(const Args& a, hipStream_t s) {
  switch (a.K) {
    case 32: return launch_t<T, C, 32>(a, s);
    case 64: return launch_t<T, C, 64>(a, s);
    case 128: return launch_t<T, C, 128>(a, s);
    case 256: return launch_t<T, C, 256>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_kkt_wy(const Args& a, hipStream_t s) {
  if (a.NTmax == 0) return hipSuccess;
  if (a.dtype == GDR_BF16) return a.C == 32 ? launch_k<bf16, 32>(a, s) : launch_k<bf16, 64>(a, s);
  return a.C == 32 ? launch_k<float, 32>(a, s) : launch_k<float, 64>(a, s);
}

}  // namespace gdr
