// K1 + K2 fused, per-channel gate: the chunk's gate cumsum, kk^T and the
// triangular inverse, the WY factors and every per-chunk operand the
// per-channel state scan (and the fused scan + output) reads, in one pass.
//
// For one chunk (L <= C rows) and value head j, with G the chunk-local
// inclusive cumsum of the per-channel gate (G_td, one value per token and
// feature) and k^, q^ the (optionally L2-normalised) keys and queries:
//   A[r][c] = beta_r sum_d k^_rd k^_cd exp(G_rd - G_cd)      c < r
//   Tm      = (I + A)^-1                                       (unit lower triangular)
//   w = Tm (beta exp(G) k^)          u = Tm (beta v)
// the WY construction of the DeltaNet chunk form P^r = I - sum_i k^i w^i^T on
// the coverage-matrix page ("FLA operator-kernel correctness testing and
// coverage matrix", section 2) with the gate folded in, plus
//   kt_t = exp(G_L - G_t) k^_t,  dl = exp(G_L)                (the state update)
// and, for the fused scan + output (a.aqk / a.qgs set, bf16),
//   aqk[r][t] = scale sum_d q^_rd k^_td exp(G_rd - G_td)       t <= r
//   qgs_t     = scale exp(G_t) q^_t   (the output's inter term; one tile in the
//                                      input dtype, or a bf16 hi + lo pair)
// Same results as the K1 and K2 stages up to rounding (Tm feeds w and u here
// in fp32 instead of through its bf16 copy); Tm itself is written only when
// a.Tm is set (the backward reads it), and u is written in fp32 when a.u_f32
// is set (kept states), else in the input dtype (the fused forward).
//
// gfx950 mapping (4 waves per chunk and value head):
//  * every global load of the chunk (key and query rows, the gate tile as
//    16-byte pieces, beta, the first value pass) is issued before the first
//    wait; the gate tile is staged into LDS and summed down each feature
//    column there;
//  * the raw key and query tiles are staged token-major (288-byte rows, where
//    16-byte row reads are conflict-free); the lower-triangular 16 x 16 blocks
//    of kk^T (and of q k^T) are spread over the waves, each block with a
//    reference row m so that both gated operands carry factors exp(+-(G - G_m))
//    <= 1 (off-diagonal: the last row of the column block; diagonal: the
//    middle row while the block's gate span keeps every factor below e^80,
//    else per-element exponentials); kk^T takes single-rounded bf16 operands,
//    q k^T hi + lo pairs;
//  * the element-wise operands (k exp(G) for w, kt, the gated queries) come
//    from each thread's own key / query pieces, still in registers, with one
//    exponential per element shared between them;
//  * (I + A)^-1 in fp32 in LDS as in the fused scalar-gate stage; w and u as in
//    K2 with the rows of Tm taken from LDS in fp32.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

constexpr float kSpanLimit = 80.f;

template <typename T, int C, int K>
struct K12P {
  static constexpr int NW = 4, NT = 256;
  static constexpr int NB = C / 16;                      // 16-row blocks per chunk
  static constexpr int NLB = NB * (NB + 1) / 2;          // lower-triangular blocks
  static constexpr int KSC = C / 32;                     // token slabs
  static constexpr int KS = K / 32;                      // feature slabs
  static constexpr int KP = K + 32 / sizeof(T);          // raw key / query rows (row-fragment reads)
  static constexpr int KPT = K + 16 / sizeof(T);         // k exp(G) rows (transposed reads)
  static constexpr int GP = K + 4;                       // gate rows, fp32, 16-byte aligned
  static constexpr int VT = sizeof(T) == 2 ? 128 : 64;   // value columns staged per pass
  static constexpr int VP = VT + 16 / sizeof(T);
  static constexpr int CPR = K / 8;                      // 8-element pieces per key row
  static constexpr int NKP = (C * CPR + NT - 1) / NT;    // key / query pieces per thread
  static constexpr int NVP = (C * VT / 8 + NT - 1) / NT; // value pieces per thread and pass
  static constexpr int NGP = (C * K / 4 + NT - 1) / NT;  // 16-byte gate pieces per thread
  // A, then Tm, fp32, packed lower-triangular blocks with 20-float rows
  static constexpr int MP = 20, MB = 16 * MP + 16;
  static constexpr int kGBytes = C * GP * 4, kVBytes = C * VP * (int)sizeof(T);
  static constexpr int kGVBytes = kGBytes > kVBytes ? kGBytes : kVBytes;
  static constexpr size_t lds_bytes =
      (size_t)2 * C * KP * sizeof(T) + (size_t)C * KPT * sizeof(T) + kGVBytes + NLB * MB * 4 + 4 * C * 4;
  static constexpr bool fits = lds_bytes <= 64 * 1024;
};

template <typename T, int C, int K, typename UT>
__global__ __launch_bounds__(256) void k12pc_kkt_wy(Args a) {
  using Cfg = K12P<T, C, K>;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, NB = Cfg::NB, NLB = Cfg::NLB, KSC = Cfg::KSC, KS = Cfg::KS;
  constexpr int KP = Cfg::KP, KPT = Cfg::KPT, GP = Cfg::GP, VT = Cfg::VT, VP = Cfg::VP, CPR = Cfg::CPR;
  constexpr int NKP = Cfg::NKP, NVP = Cfg::NVP, NGP = Cfg::NGP, MP = Cfg::MP, MB = Cfg::MB;
  __shared__ __attribute__((aligned(16))) T sK[C * KP];
  __shared__ __attribute__((aligned(16))) T sQ[C * KP];
  __shared__ __attribute__((aligned(16))) T sKg[C * KPT];
  // the gate cumsum tile is dead once A, aqk and the element-wise operands are
  // formed, before the first value pass: the value tile reuses its bytes
  __shared__ __attribute__((aligned(16))) char sGV[Cfg::kGVBytes];
  float* const sGc = reinterpret_cast<float*>(sGV);
  T* const sV = reinterpret_cast<T*>(sGV);
  __shared__ __attribute__((aligned(16))) float sM[NLB * MB];
  __shared__ __attribute__((aligned(16))) float sB[C];
  __shared__ __attribute__((aligned(16))) float sRn[C];
  __shared__ __attribute__((aligned(16))) float sRq[C];
  __shared__ __attribute__((aligned(16))) float sS[C];
  auto blk = [](int rb, int cb) { return (rb * (rb + 1) / 2 + cb) * MB; };

  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ChunkHead ch = chunk_head(a.HV);
  const int64_t c = ch.c, j = ch.j;
  if (c >= a.chunk_off[a.N]) return;
  const int64_t t0 = a.chunk_idx[4 * c + 1];
  const int L = a.chunk_idx[4 * c + 2];
  const int64_t H = a.H, HV = a.HV, V = a.V, h = j / (HV / H);
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const T* __restrict__ vp = static_cast<const T*>(a.v);
  T* __restrict__ wp = static_cast<T*>(a.w) + (c * HV + j) * (int64_t)(C * K);
  UT* __restrict__ up = static_cast<UT*>(a.u) + (c * HV + j) * (int64_t)C * V;
  // intra attention and gated queries for the fused scan + output (bf16 only)
  const bool want_q = sizeof(T) == 2 && a.aqk != nullptr && a.qgs != nullptr;

  // ---- every global load of the chunk up front: key and query rows, the
  //      first value pass, the gate tile, beta
  Frag<T> kr[NKP], qr[NKP], vr[NVP];
  f32x4 gr[NGP];
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
    const bool in = idx < C * CPR && t < L;
    kr[i] = in ? ld8(kp + ((t0 + t) * H + h) * K + d8) : frag_zero<T>();
    qr[i] = (in && want_q) ? ld8(qp + ((t0 + t) * H + h) * K + d8) : frag_zero<T>();
  }
#pragma unroll
  for (int i = 0; i < NGP; ++i) {
    const int idx = tid + NT * i, t = idx / (K / 4), d4 = (idx % (K / 4)) * 4;
    gr[i] = (idx < C * K / 4 && t < L) ? *reinterpret_cast<const f32x4*>(a.g + ((t0 + t) * HV + j) * K + d4)
                                       : zero4();
  }
  fetch_v(0);
  const float bv = (tid < L) ? beta_value(a.beta[(t0 + tid) * HV + j], a.beta_logits) : 0.f;

  // ---- gate tile, raw key / query tiles, row norms, beta
#pragma unroll
  for (int i = 0; i < NGP; ++i) {
    const int idx = tid + NT * i, t = idx / (K / 4), d4 = (idx % (K / 4)) * 4;
    if (idx < C * K / 4) *reinterpret_cast<f32x4*>(&sGc[t * GP + d4]) = gr[i];
  }
  float rn[NKP], rq[NKP];
#pragma unroll
  for (int i = 0; i < NKP; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    const f32x8 x = kr[i].f32(), y = qr[i].f32();
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sk += x[e] * x[e];
      sq += y[e] * y[e];
    }
    sk = lanes_sum_t<CPR>(sk);
    sq = lanes_sum_t<CPR>(sq);
    rn[i] = a.l2norm ? 1.f / sqrtf(sk + kL2Eps) : 1.f;
    rq[i] = a.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
    if (idx < C * CPR) {
      if (d8 == 0) {
        sRn[t] = rn[i];
        sRq[t] = rq[i];
      }
      st8(&sK[t * KP + d8], kr[i]);
      st8(&sQ[t * KP + d8], qr[i]);
    }
  }
  if (tid < C) sB[tid] = bv;
  lds_barrier();
  // chunk-local cumsum down each feature column: all C reads first, the
  // running sum in registers, then the writes
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

  // ---- element-wise operands from this thread's own pieces: k exp(G) (the w
  //      products' tile), kt = exp(G_L - G_t) k^_t, the gated queries, dl
  T* __restrict__ ktp = a.kt != nullptr ? static_cast<T*>(a.kt) + (c * HV + j) * (int64_t)(C * K) : nullptr;
  T* __restrict__ qgp = want_q ? static_cast<T*>(a.qgs) + (c * HV + j) * (int64_t)(kQgsTiles * C * K) : nullptr;
#pragma unroll
  for (int i = 0; i < NKP; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    if (idx < C * CPR) {
      const float* Gt = &sGc[t * GP + d8];
      const float* Gl = &sGc[(L - 1) * GP + d8];
      const f32x8 G = cat8(*reinterpret_cast<const f32x4*>(Gt), *reinterpret_cast<const f32x4*>(Gt + 4));
      const f32x8 x = kr[i].f32();
      f32x8 ex;
#pragma unroll
      for (int e = 0; e < 8; ++e) ex[e] = __expf(G[e]);
      st8(&sKg[t * KPT + d8], Frag<T>::make(x * ex));
      if (ktp != nullptr) {
        const f32x8 GL = cat8(*reinterpret_cast<const f32x4*>(Gl), *reinterpret_cast<const f32x4*>(Gl + 4));
        f32x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[e] * rn[i] * __expf(GL[e] - G[e]);
        st8(ktp + t * K + d8, Frag<T>::make(y));
      }
      if (qgp != nullptr) {
        const SplitFrag<T> sp = SplitFrag<T>::make(qr[i].f32() * ex * (a.scale * rq[i]));
        st8(qgp + t * K + d8, sp.hi);
        if constexpr (kQgsTiles == 2) st8(qgp + (C + t) * K + d8, sp.lo);
      }
    }
  }
  if (a.dl != nullptr)
    for (int d = tid; d < K; d += NT) a.dl[(c * HV + j) * K + d] = __expf(sGc[(L - 1) * GP + d]);

  // ---- gated kk^T (and q k^T) blocks, spread over the waves
  auto grow8 = [&](int row, int d0) {
    const float* p = &sGc[row * GP + d0];
    return cat8(*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4));
  };
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
    for (int cb = 0; cb <= rb; ++cb) {
      if ((rb * (rb + 1) / 2 + cb) % NW != wv) continue;
      f32x4 s = zero4(), sqk = zero4();
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
      const int ra = 16 * rb + r16, rc = 16 * cb + r16;
      if (!direct) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int d0 = 32 * ks + 8 * g4;
          f32x8 xa = ld8(&sK[ra * KP + d0]).f32(), xb = ld8(&sK[rc * KP + d0]).f32();
          f32x8 xq = want_q ? ld8(&sQ[ra * KP + d0]).f32() : zero8();
          const f32x8 Gm = grow8(m, d0), Ga = grow8(ra, d0), Gb = grow8(rc, d0);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float fa = __expf(Ga[e] - Gm[e]);
            xa[e] *= fa;
            xq[e] *= fa;
            xb[e] *= __expf(Gm[e] - Gb[e]);
          }
          mma(s, Frag<T>::make(xa), Frag<T>::make(xb));
          // q k^T transposed: element i of lane (r16, g4) is row 16 rb + r16,
          // column 16 cb + 4 g4 + i
          if (want_q) mma_split(sqk, SplitFrag<T>::make(xb), SplitFrag<T>::make(xq));
        }
      } else {
        // per-element exponentials for a block whose gate span is too wide
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rb + 4 * g4 + i, cc = 16 * cb + r16;
          float sum = 0.f;
          if (cc < r && r < L) {
            for (int d = 0; d < K; ++d)
              sum += to_float(sK[r * KP + d]) * to_float(sK[cc * KP + d]) * __expf(sGc[r * GP + d] - sGc[cc * GP + d]);
          }
          s[i] = sum;
          const int tc = 16 * cb + 4 * g4 + i;
          float sq = 0.f;
          if (want_q && tc <= ra && ra < L) {
            for (int d = 0; d < K; ++d)
              sq += to_float(sQ[ra * KP + d]) * to_float(sK[tc * KP + d]) * __expf(sGc[ra * GP + d] - sGc[tc * GP + d]);
          }
          sqk[i] = sq;
        }
      }
      // A (strictly lower, fp32) into LDS; the factors of the lane's four
      // consecutive rows in one 16-byte read each, the column's once
      {
        const int r4 = 16 * rb + 4 * g4, cc = 16 * cb + r16;
        const f32x4 B4 = *reinterpret_cast<const f32x4*>(&sB[r4]);
        const f32x4 N4 = *reinterpret_cast<const f32x4*>(&sRn[r4]);
        const float nc = sRn[cc];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r4 + i;
          sM[blk(rb, cb) + (4 * g4 + i) * MP + r16] = (cc < r && r < L) ? B4[i] * s[i] * N4[i] * nc : 0.f;
        }
      }
      // aqk row ra: scale / (|q_r| |k_t|) on t <= r < L
      if (want_q) {
        const float fr = (ra < L) ? a.scale * sRq[ra] : 0.f;
        const f32x4 T4 = *reinterpret_cast<const f32x4*>(&sRn[16 * cb + 4 * g4]);
        f32x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tc = 16 * cb + 4 * g4 + i;
          o4[i] = tc <= ra ? sqk[i] * fr * T4[i] : 0.f;
        }
        *reinterpret_cast<f32x4*>(a.aqk + (c * HV + j) * (int64_t)(C * C) + ra * C + 16 * cb + 4 * g4) = o4;
      }
    }
  }
  // aqk blocks above the diagonal are zero
  if (want_q) {
#pragma unroll
    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
      for (int cb = rb + 1; cb < NB; ++cb) {
        if ((rb * NB + cb) % NW != wv) continue;
        *reinterpret_cast<f32x4*>(a.aqk + (c * HV + j) * (int64_t)(C * C) + (16 * rb + r16) * C + 16 * cb + 4 * g4) =
            zero4();
      }
  }
  if (tid < C) sS[tid] = sB[tid] * sRn[tid];
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
        for (int q = 0; q < 4; ++q) {
          av[q] = sM[blk(ib, mb) + r16 * MP + 4 * g4 + q];
          bvv[q] = sM[blk(mb, jb) + (4 * g4 + q) * MP + r16];
        }
        mma16_f32(X, av, bvv);
      }
      float tv[4], xv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        tv[q] = sM[blk(ib, ib) + r16 * MP + 4 * g4 + q];
        xv[q] = X[q];
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

  // ---- Tm (for the backward; rows / cols past L and the upper triangle zero)
  if (a.Tm != nullptr) {
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

  // ---- rows of Tm this lane feeds (fp32): row 16 rb + r16, tokens
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

  // the first value pass goes to LDS now, in the bytes of the gate tile
  auto stage_v = [&](int64_t v0) {
    const int nv = (V - v0) < VT ? (int)(V - v0) : VT;
    const int vpr = nv / 8;
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int idx = tid + NT * i, t = idx / vpr, d8 = (idx % vpr) * 8;
      if (idx < C * vpr) st8(&sV[t * VP + d8], vr[i]);
    }
  };
  stage_v(0);

  // w^T = (k exp(G))^T (Tm diag(beta / |k|))^T, feature blocks over the waves
  auto w_block = [&](int fb, int rb) {
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      if (2 * ks > rb) continue;
      const Frag<T> ka = lds_tr_frag(sKg, KPT, 32 * ks + 8 * g4, 32 * ks + 8 * g4 + 4, 16 * fb, lane);
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

  // u = Tm diag(beta) v (fp32 out, Tm diag(beta) as a hi + lo pair), value
  // columns staged VT at a time (the next pass's loads are issued while this
  // one is computed)
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
          mma_split(acc[rb], SplitFrag<T>::make(tf[rb][ks] * sc), vbf);
        }
      }
#pragma unroll
      for (int m2 = 0; m2 < NB / 2; ++m2)
        st_pair(up + (v0 + 16 * vb + r16) * C + 32 * m2, acc[2 * m2], acc[2 * m2 + 1], lane);
    }
  }
}

template <typename T, int C, int K>
hipError_t launch_t(const Args& a, hipStream_t s) {
  if constexpr (K12P<T, C, K>::fits) {
    // u in fp32 (kept states, which the backward reads) or in the input dtype
    // (the fused forward, whose scan + output takes it as the scalar-gate fused
    // stage does)
    if (a.u_f32)
      hipLaunchKernelGGL((k12pc_kkt_wy<T, C, K, float>), dim3((unsigned)(a.NTmax * a.HV)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k12pc_kkt_wy<T, C, K, T>), dim3((unsigned)(a.NTmax * a.HV)), dim3(256), 0, s, a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

}  // namespace

bool kkt_wy_pc_supported(const Args& a) {
  if (!a.per_channel || a.C != 32) return false;
  if (a.dtype == GDR_BF16) {
    switch (a.K) {
      case 32: return K12P<bf16, 32, 32>::fits;
      case 64: return K12P<bf16, 32, 64>::fits;
      case 128: return K12P<bf16, 32, 128>::fits;
    }
  }
  return false;
}

hipError_t launch_kkt_wy_pc(const Args& a, hipStream_t s) {
  if (a.NTmax == 0) return hipSuccess;
  if (!kkt_wy_pc_supported(a)) return hipErrorInvalidValue;
  switch (a.K) {
    case 32: return launch_t<bf16, 32, 32>(a, s);
    case 64: return launch_t<bf16, 32, 64>(a, s);
    case 128: return launch_t<bf16, 32, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdr
