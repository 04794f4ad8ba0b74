// B3 for a per-channel gate (KDA-style): every gradient of a chunk that the
// reverse state scan does not produce, for one chunk (L rows) and q/k head h,
// with the value heads j of its group processed in turn.
//
// With G the chunk-local gate cumsum per channel (C x K), S0 = h[c] (state
// entering the chunk), dS1 = dh[c] (gradient of the state leaving it), E =
// v_new, T = (I + A)^-1 and the chunk form on the coverage-matrix page ("FLA
// operator-kernel correctness testing and coverage matrix", section 2) with a
// diagonal gate per feature:
//   dE   = de_local + Kt dS1,          Kt[t][d] = exp(G_Ld - G_td) k^_td
//   Y    = T^T dE,   dv = diag(beta) Y
//   dQg  = scale dO S0^T,   TdW = -Y S0^T,   dKt = E dS1^T        (C x K)
//   dP   = scale dO E^T (t <= r),            dA = -Y E^T (t < r)  (C x C)
// The gated pair forms P[r][t] = sum_d q^_rd k^_td exp(G_rd - G_td) and
// Abar[r][t] = sum_d k^_rd k^_td exp(G_rd - G_td) give, per feature d,
//   dqP[r][d]  = sum_{t<=r} dP[r][t] k^_td exp(G_rd - G_td)
//   dkP[t][d]  = sum_{r>=t} dP[r][t] q^_rd exp(G_rd - G_td)
//   dkA1[r][d] = sum_{t<r}  dA[r][t] k^_td exp(G_rd - G_td)
//   dkA2[t][d] = sum_{r>t}  beta_r dA[r][t] k^_rd exp(G_rd - G_td)
// and then, with gam = exp(G_td), kap = exp(G_Ld - G_td):
//   dq^ = dqP + gam dQg
//   dk^ = beta dkA1 + dkA2 + dkP + beta gam TdW + kap dKt
//   dG  = q^ dqP - k^ dkP + beta k^ dkA1 - k^ dkA2 + gam q^ dQg
//         + beta gam k^ TdW - kap k^ dKt,
//   dG[L-1][d] += sum_t kap k^_td dKt[t][d] + exp(G_Ld) sum_v S0[d][v] dS1[d][v]
//   dbeta = sum_d gam k^ TdW + sum_v v Y + sum_d k^ dkA1
//   dg    = reverse cumsum of dG over the chunk, per feature
// (dbeta's last term is sum_m dA[t][m] Abar[t][m]); dq, dk are summed over the
// group and taken through the L2-norm backward.
//
// gfx950 mapping (chunk 32, four waves, one workgroup per chunk and q/k head):
// the dense products run on MFMA as in the scalar-gate stage, over value tiles
// of 32 columns, with dS1 and the fp32 intermediates (dE, Y) as bf16 hi + lo
// operand pairs.  The gated pair sums do not factor into one matrix product
// (their exponent depends on the row, the column and the feature), so they run
// on the vector ALU in the MFMA accumulator layout each wave already holds for
// dQg, TdW and dKt (lane: rows 16 rb + 4 g + e, feature 16 db + l % 16): one
// pass over the chunk's rows x serves all four, x < r feeding dqP / dkA1 and
// x > r feeding dkP / dkA2, with one exponential of the exact difference per
// term (G_rd - G_xd below the diagonal, G_xd - G_rd above it: <= 0 for a decay
// gate, so no factor exceeds 1 and no reference row is needed).
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

// largest 16-row gate span (max over features of G at the block's first row
// minus its last) for which the gated pair sums take the MFMA form
constexpr float kPairSpan = 40.f;

template <typename T, int K>
struct B3P {
  static constexpr int C = 32, NW = 4, NT = 256, VT = 32;
  static constexpr int EB = sizeof(T);
  static constexpr int CPR = K / 8;
  static constexpr int PK = K + 32 / EB;     // q, k, kt, h^T, dh^T, dq / dk out rows
  static constexpr int PCC = C + 32 / EB;    // T, e^T, de_local^T, dE^T rows
  static constexpr int PV = VT + 32 / EB;    // dO, v, Y rows
  static constexpr int GP = K + 1;           // gate cumsum rows (fp32)
  static constexpr int CP = C + 1;           // dP, dA rows (fp32)
  static constexpr int NRB = C / 16, NKB = K / 16, NVB = VT / 16, KSK = K / 32;
  static constexpr int NBK = NRB * NKB;
  static constexpr int SCK = (NBK + NW - 1) / NW;    // C x K blocks per wave
  static_assert(NW % NRB == 0 && NBK % NW == 0, "a wave owns one row block and whole slots");
  static constexpr int NPQ = (C * CPR + NT - 1) / NT;
  static constexpr int NPT = (C * C / 8 + NT - 1) / NT;
  static constexpr int NPH = (VT * CPR + NT - 1) / NT;
  static constexpr int NPO = (C * VT / 8 + NT - 1) / NT;
  static constexpr int NPE = (VT * C / 8 + NT - 1) / NT;
  // LDS (bytes)
  static constexpr size_t oQ = 0;
  static constexpr size_t oK = oQ + (size_t)C * PK * EB;
  static constexpr size_t oKt = oK + (size_t)C * PK * EB;
  static constexpr size_t oT = oKt + (size_t)C * PK * EB;
  static constexpr size_t oG = oT + (size_t)C * PCC * EB;
  static constexpr size_t oLoop = oG + (size_t)C * GP * 4;
  static constexpr int SPL = sizeof(T) == 2 ? 2 : 1;     // hi + lo tiles
  static constexpr size_t lH = 0;
  static constexpr size_t lDH = lH + (size_t)VT * PK * EB;
  static constexpr size_t lDO = lDH + (size_t)VT * PK * EB * SPL;
  static constexpr size_t lV = lDO + (size_t)C * PV * EB;
  static constexpr size_t lE = lV + (size_t)C * PV * EB;
  static constexpr size_t lDL = lE + (size_t)VT * PCC * EB;
  static constexpr size_t lDE = lDL + (size_t)VT * PCC * EB;
  static constexpr size_t lY = lDE + (size_t)VT * PCC * EB * SPL;
  static constexpr size_t loop_bytes = lY + (size_t)C * PV * EB * SPL;
  // after the value loop: dP, dA, the dG tile; at the end: the dq / dk rows
  static constexpr size_t pDP = 0, pDA = pDP + (size_t)C * CP * 4, pDG = pDA + (size_t)C * CP * 4;
  static constexpr size_t post_bytes = pDG + (size_t)C * GP * 4;
  static constexpr size_t fin_bytes = 2 * (size_t)C * PK * EB;
  static constexpr size_t region =
      loop_bytes > post_bytes ? (loop_bytes > fin_bytes ? loop_bytes : fin_bytes)
                              : (post_bytes > fin_bytes ? post_bytes : fin_bytes);
  static constexpr size_t oRows = oLoop + ((region + 15) & ~size_t(15));
  // rows: rq, rk, beta; per-wave dbeta, q.dq, k.dk partials; last-row column
  // extras per row block; lr per feature and its per-wave partials
  static constexpr size_t rows_floats = 3 * C + 3 * NW * C + NRB * K + K + NW * K;
  static constexpr size_t total = oRows + rows_floats * 4;
  static constexpr bool fits = total <= 160 * 1024;
};

template <typename T, int K>
__global__ __launch_bounds__(256) void b3pc_bwd_dqkvg(Args a) {
  using Cfg = B3P<T, K>;
  constexpr int C = Cfg::C, NW = Cfg::NW, NT = Cfg::NT, VT = Cfg::VT, CPR = Cfg::CPR;
  constexpr int PK = Cfg::PK, PCC = Cfg::PCC, PV = Cfg::PV, GP = Cfg::GP, CP = Cfg::CP;
  constexpr int NRB = Cfg::NRB, KSK = Cfg::KSK, NBK = Cfg::NBK, SCK = Cfg::SCK;
  constexpr int NPQ = Cfg::NPQ, NPT = Cfg::NPT, NPH = Cfg::NPH, NPO = Cfg::NPO, NPE = Cfg::NPE;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::total];

  auto body = [&](auto wvc) {
  constexpr int wv = decltype(wvc)::value;
  constexpr int rb = wv % NRB;          // this wave's row block
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const ChunkHead ch = chunk_head(a.H);
  const int64_t c = ch.c, h = ch.j;
  if (c >= a.chunk_off[a.N]) return;
  const int64_t t0 = a.chunk_idx[4 * c + 1];
  const int L = a.chunk_idx[4 * c + 2];
  const int64_t H = a.H, HV = a.HV, V = a.V;
  const int ng = (int)(HV / H);
  const float scale = a.scale;

  T* sQ = reinterpret_cast<T*>(smem + Cfg::oQ);
  T* sK = reinterpret_cast<T*>(smem + Cfg::oK);
  T* sKt = reinterpret_cast<T*>(smem + Cfg::oKt);
  T* sT = reinterpret_cast<T*>(smem + Cfg::oT);
  float* sG = reinterpret_cast<float*>(smem + Cfg::oG);
  char* loop = smem + Cfg::oLoop;
  T* sH = reinterpret_cast<T*>(loop + Cfg::lH);
  const FTile<T> fDH = ftile<T, PK>(loop + Cfg::lDH, VT);     // dS1^T [v][d]
  T* sDO = reinterpret_cast<T*>(loop + Cfg::lDO);
  T* sV = reinterpret_cast<T*>(loop + Cfg::lV);
  T* sE = reinterpret_cast<T*>(loop + Cfg::lE);               // e^T [v][t]
  T* sDL = reinterpret_cast<T*>(loop + Cfg::lDL);             // de_local^T [v][t]
  const FTile<T> fDE = ftile<T, PCC>(loop + Cfg::lDE, VT);    // dE^T [v][t]
  const FTile<T> fY = ftile<T, PV>(loop + Cfg::lY, C);        // Y [t][v]
  float* sDP = reinterpret_cast<float*>(loop + Cfg::pDP);     // scale dO E^T [r][t], t <= r < L
  float* sDA = reinterpret_cast<float*>(loop + Cfg::pDA);     // -Y E^T [r][t], t < r < L
  float* sDG = reinterpret_cast<float*>(loop + Cfg::pDG);     // dG [t][d]
  T* sOq = reinterpret_cast<T*>(loop);
  T* sOk = reinterpret_cast<T*>(loop + (size_t)C * PK * sizeof(T));
  float* sRq = reinterpret_cast<float*>(smem + Cfg::oRows);
  float* sRk = sRq + C;
  float* sB = sRk + C;
  float* sRowB = sB + C;               // [NW][C]
  float* sDotQ = sRowB + NW * C;       // [NW][C]
  float* sDotK = sDotQ + NW * C;       // [NW][C]
  float* sLast = sDotK + NW * C;       // [NRB][K]
  float* sLr = sLast + NRB * K;        // [K]
  float* sLrW = sLr + K;               // [NW][K]

  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ vp = static_cast<const T*>(a.v);
  const T* __restrict__ dop = static_cast<const T*>(a.d_o);

  // ---- q, k tiles (rows past L zero) and their row norms
  {
    Frag<T> qr[NPQ], kr[NPQ];
#pragma unroll
    for (int i = 0; i < NPQ; ++i) {
      const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      const bool in = idx < C * CPR && t < L;
      qr[i] = in ? ld8(qp + ((t0 + t) * H + h) * K + d8) : frag_zero<T>();
      kr[i] = in ? ld8(kp + ((t0 + t) * H + h) * K + d8) : frag_zero<T>();
    }
#pragma unroll
    for (int i = 0; i < NPQ; ++i) {
      const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      const f32x8 xq = qr[i].f32(), xk = kr[i].f32();
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq += xq[e] * xq[e];
        sk += xk[e] * xk[e];
      }
      sq = lanes_sum_t<CPR>(sq);
      sk = lanes_sum_t<CPR>(sk);
      if (idx < C * CPR) {
        st8(&sQ[t * PK + d8], qr[i]);
        st8(&sK[t * PK + d8], kr[i]);
        if (d8 == 0) {
          sRq[t] = a.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
          sRk[t] = a.l2norm ? 1.f / sqrtf(sk + kL2Eps) : 1.f;
        }
      }
    }
  }

  // this lane's C x K elements: slot i is block b = wv + NW i, rows
  // 16 rb + 4 g4 + e, feature 16 (b / NRB) + r16
  f32x4 sq_[SCK], sk_[SCK];       // dq^, dk^ summed over the group
#pragma unroll
  for (int i = 0; i < SCK; ++i) sq_[i] = sk_[i] = zero4();

  // value tiles: each tile's loads are issued one tile ahead, into
  // registers, and staged when the previous tile's products are done
  Frag<T> hr[NPH], orr[NPO], vr[NPO], er[NPE], dlr[NPE];
  Frag<float> dhr[NPH];
  auto fetch_tile = [&](int64_t j, int64_t v0) {
    const T* hb = static_cast<const T*>(a.h) + ((c * HV + j) * V + v0) * (int64_t)K;
    const float* dhb = static_cast<const float*>(a.dh) + ((c * HV + j) * V + v0) * (int64_t)K;
    const T* eb = static_cast<const T*>(a.v_new) + ((c * HV + j) * V + v0) * (int64_t)C;
    const T* db = static_cast<const T*>(a.de_local) + ((c * HV + j) * V + v0) * (int64_t)C;
#pragma unroll
    for (int i = 0; i < NPH; ++i) {
      const int idx = tid + NT * i;
      const bool in = idx < VT * CPR;
      hr[i] = in ? ld8(hb + 8 * idx) : frag_zero<T>();
      dhr[i] = in ? ld8(dhb + 8 * idx) : frag_zero<float>();
    }
#pragma unroll
    for (int i = 0; i < NPO; ++i) {
      const int idx = tid + NT * i, t = idx / (VT / 8), v8 = (idx % (VT / 8)) * 8;
      // rows past L load row 0 (a valid address) and are zeroed when staged
      const int tc = (idx < C * VT / 8 && t < L) ? t : 0;
      orr[i] = ld8(dop + ((t0 + tc) * HV + j) * V + v0 + v8);
      vr[i] = ld8(vp + ((t0 + tc) * HV + j) * V + v0 + v8);
    }
#pragma unroll
    for (int i = 0; i < NPE; ++i) {
      const int idx = tid + NT * i;
      const int ic = idx < VT * C / 8 ? idx : 0;
      er[i] = ld8(eb + 8 * ic);
      dlr[i] = ld8(db + 8 * ic);
    }
  };
  for (int jj = 0; jj < ng; ++jj) {
    const int64_t j = h * ng + jj;
    // ---- per-head tiles: the gate (cumsum below), beta, T, kt, then the
    //      head's first value tile.  The gate pieces are requested first and
    //      all at once, so staging them waits for nothing younger, and beta's
    //      sigmoid is taken after the last request, so no instruction needs a
    //      loaded value while the others are in flight.
    {
      constexpr int NPG = (C * K / 4 + NT - 1) / NT;   // float4 gate pieces per thread
      f32x4 gr[NPG];
#pragma unroll
      for (int i = 0; i < NPG; ++i) {
        const int idx = tid + NT * i, t = idx / (K / 4), d4 = (idx % (K / 4)) * 4;
        gr[i] = (idx < C * K / 4 && t < L) ? *reinterpret_cast<const f32x4*>(a.g + ((t0 + t) * HV + j) * K + d4)
                                           : zero4();
      }
      const float braw = (tid < L) ? a.beta[(t0 + tid) * HV + j] : 0.f;
      const T* tp = static_cast<const T*>(a.Tm) + (c * HV + j) * (int64_t)(C * C);
      const T* ktp = static_cast<const T*>(a.kt) + (c * HV + j) * (int64_t)(C * K);
      Frag<T> tr[NPT], ktr[NPQ];
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int idx = tid + NT * i;
        tr[i] = (idx < C * C / 8) ? ld8(tp + 8 * idx) : frag_zero<T>();
      }
#pragma unroll
      for (int i = 0; i < NPQ; ++i) {
        const int idx = tid + NT * i;
        ktr[i] = (idx < C * CPR) ? ld8(ktp + 8 * idx) : frag_zero<T>();
      }
      fetch_tile(j, 0);
#pragma unroll
      for (int i = 0; i < NPG; ++i) {
        const int idx = tid + NT * i, t = idx / (K / 4), d4 = (idx % (K / 4)) * 4;
        if (idx < C * K / 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sG[t * GP + d4 + e] = gr[i][e];
        }
      }
      const float bv = (tid < L) ? beta_value(braw, a.beta_logits) : 0.f;
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int idx = tid + NT * i, r = idx / (C / 8), c8 = (idx % (C / 8)) * 8;
        if (idx < C * C / 8) st8(&sT[r * PCC + c8], tr[i]);
      }
#pragma unroll
      for (int i = 0; i < NPQ; ++i) {
        const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
        if (idx < C * CPR) st8(&sKt[t * PK + d8], ktr[i]);
      }
      if (tid < C) sB[tid] = bv;
      for (int i = tid; i < NW * C; i += NT) sRowB[i] = 0.f;
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
    // sum_v S0[d][v] dS1[d][v] per feature, accumulated where the h and dh
    // pieces are staged: a thread's pieces all hold features d8 .. d8 + 7
    // (d8 = 8 (tid % CPR)), from the fp32 dh
    float lr8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) lr8[e] = 0.f;

    f32x4 dQg[SCK], TdW[SCK], dKt[SCK], dP = zero4(), dA = zero4();
#pragma unroll
    for (int i = 0; i < SCK; ++i) dQg[i] = TdW[i] = dKt[i] = zero4();


    for (int64_t v0 = 0; v0 < V; v0 += VT) {
      {
#pragma unroll
        for (int i = 0; i < NPH; ++i) {
          const int idx = tid + NT * i, v = idx / CPR, d8 = (idx % CPR) * 8;
          if (idx < VT * CPR) {
            st8(&sH[v * PK + d8], hr[i]);
            const f32x8 fy = dhr[i].f32();
            const Frag<T> hi = Frag<T>::make(fy);
            st8(&fDH.hi[v * PK + d8], hi);
            if constexpr (FTile<T>::kSplit) st8(&fDH.lo[v * PK + d8], Frag<T>::make(fy - hi.f32()));
            const f32x8 hx = hr[i].f32();
#pragma unroll
            for (int e = 0; e < 8; ++e) lr8[e] += hx[e] * fy[e];
          }
        }
#pragma unroll
        for (int i = 0; i < NPO; ++i) {
          const int idx = tid + NT * i, t = idx / (VT / 8), v8 = (idx % (VT / 8)) * 8;
          if (idx < C * VT / 8) {
            st8(&sDO[t * PV + v8], t < L ? orr[i] : frag_zero<T>());
            st8(&sV[t * PV + v8], t < L ? vr[i] : frag_zero<T>());
          }
        }
#pragma unroll
        for (int i = 0; i < NPE; ++i) {
          const int idx = tid + NT * i, v = idx / (C / 8), t8 = (idx % (C / 8)) * 8;
          if (idx < VT * C / 8) {
            st8(&sE[v * PCC + t8], er[i]);
            st8(&sDL[v * PCC + t8], dlr[i]);
          }
        }
      }
      if (v0 + VT < V) fetch_tile(j, v0 + VT);
      lds_barrier();

      // ---- dE^T[v][t] = de_local^T[v][t] + (Kt dS1)[t][v]; one 16 x 16 block per wave
      {
        constexpr int tb = wv % NRB, vb = wv / NRB;
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks)
          mma_split(acc, ld8(&sKt[(16 * tb + r16) * PK + 32 * ks + 8 * g4]), fDH.row(16 * vb + r16, 32 * ks, lane));
        const f32x4 dl4 = ld4f(&sDL[(16 * vb + r16) * PCC + 16 * tb + 4 * g4]);
        fDE.put4(16 * vb + r16, 16 * tb + 4 * g4, acc + dl4);
      }
      lds_barrier();

      // ---- Y^T[v][t] = (dE^T T)[v][t]; dv = beta Y; dbeta += v . Y
      {
        constexpr int vb = wv % 2, tb = wv / 2;
        f32x4 acc = zero4();
        mma_split(acc, fDE.row(16 * vb + r16, 0, lane), lds_col8(sT, PCC, 0, 16 * tb, lane));
        const int t = 16 * tb + r16, vc = 16 * vb + 4 * g4;
        if (t < L) st4(static_cast<T*>(a.dv) + ((t0 + t) * HV + j) * V + v0 + vc, acc * sB[t]);
        const f32x4 vv = ld4f(&sV[t * PV + vc]);
        const float p = group4_sum(acc[0] * vv[0] + acc[1] * vv[1] + acc[2] * vv[2] + acc[3] * vv[3]);
        if (g4 == 0) sRowB[wv * C + t] += p;
        fY.put4(t, vc, acc);
      }
      lds_barrier();

      // ---- products over this tile's 32 value columns
      {
        const Frag<T> aO = ld8(&sDO[(16 * rb + r16) * PV + 8 * g4]);
        const SplitFrag<T> aY = fY.row(16 * rb + r16, 0, lane);
        const Frag<T> aE = lds_col8(sE, PCC, 0, 16 * rb, lane);
#pragma unroll
        for (int i = 0; i < SCK; ++i) {
          const int db = (wv + NW * i) / NRB;
          const Frag<T> bS = lds_col8(sH, PK, 0, 16 * db, lane);
          const SplitFrag<T> bD = fDH.col(0, 16 * db, lane);
          mma(dQg[i], aO, bS);
          mma_split(TdW[i], aY, bS);
          mma_split(dKt[i], aE, bD);
        }
        constexpr int cb = wv / NRB;
        const Frag<T> bE = lds_col8(sE, PCC, 0, 16 * cb, lane);
        mma(dP, aO, bE);
        mma_split(dA, aY, bE);
      }
      lds_barrier();
    }

    // ---- dP, dA to LDS (masked); lr and the last-row extras
    {
      constexpr int cb = wv / NRB;
      const int t = 16 * cb + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rb + 4 * g4 + e;
        sDP[r * CP + t] = (t <= r && r < L) ? scale * dP[e] : 0.f;
        sDA[r * CP + t] = (t < r && r < L) ? -dA[e] : 0.f;
      }
    }
    // lr: the lanes holding the same features are CPR apart in a wave; one
    // partial per wave, summed in wave order below
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = lr8[e];
#pragma unroll
      for (int off = CPR; off < 64; off *= 2) x += __shfl_xor(x, off, 64);
      lr8[e] = x;
    }
    if (lane < CPR) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sLrW[wv * K + 8 * lane + e] = lr8[e];
    }
#pragma unroll
    for (int i = 0; i < SCK; ++i) {
      dQg[i] *= scale;
      TdW[i] = -TdW[i];
    }
    lds_barrier();
    for (int d = tid; d < K; d += NT) {
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) x += sLrW[w * K + d];
      sLr[d] = x;
    }

    // ---- the gated pair sums.  With every 16-row block's gate span below
    //      kPairSpan they run on MFMA with a reference row per block: for the
    //      wave's rows r (block R = rb) m = 16 R, for its rows t (block T = rb)
    //      m' = 16 T + 15, so that
    //        dqP[r]  = exp(G_r - G_m)   sum_t dP[r][t] (k^_t exp(G_m - G_t))
    //        dkP[t]  = exp(G_m' - G_t)  sum_r dP[r][t] (q^_r exp(G_r - G_m'))
    //      (dkA1, dkA2 alike with dA and beta dA^T): every outer factor is
    //      <= 1 and every inner one <= exp(span); rows outside the causal
    //      range are zeroed before their factor could overflow.  Operands go
    //      in as bf16 hi + lo pairs.  A wider span takes one pass over the
    //      chunk's rows x with the exact difference per term.
    f32x4 dqP[SCK], dkP[SCK], dkA1[SCK], dkA2[SCK], Gr[SCK];
#pragma unroll
    for (int i = 0; i < SCK; ++i) {
      dqP[i] = dkP[i] = dkA1[i] = dkA2[i] = zero4();
      const int d = 16 * ((wv + NW * i) / NRB) + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) Gr[i][e] = sG[(16 * rb + 4 * g4 + e) * GP + d];
    }
    float span = 0.f;
#pragma unroll
    for (int b = 0; b < NRB; ++b)
      for (int d = lane; d < K; d += 64) span = fmaxf(span, sG[(16 * b) * GP + d] - sG[(16 * b + 15) * GP + d]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) span = fmaxf(span, __shfl_xor(span, o, 64));
    if (span <= kPairSpan) {
      const int ra = 16 * rb + r16;
      f32x8 xp, xa, xpt, xat;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int x = 8 * g4 + e;
        xp[e] = sDP[ra * CP + x];
        xa[e] = sDA[ra * CP + x];
        xpt[e] = sDP[x * CP + ra];
        xat[e] = sB[x] * sDA[x * CP + ra];
      }
      const SplitFrag<T> aP = SplitFrag<T>::make(xp), aA = SplitFrag<T>::make(xa);
      const SplitFrag<T> aPT = SplitFrag<T>::make(xpt), aAT = SplitFrag<T>::make(xat);
      const int mR = 16 * rb, mT = 16 * rb + 15;
#pragma unroll
      for (int i = 0; i < SCK; ++i) {
        const int db = (wv + NW * i) / NRB, d = 16 * db + r16;
        const float GmR = sG[mR * GP + d], GmT = sG[mT * GP + d];
        const f32x8 kc = lds_col8(sK, PK, 0, 16 * db, lane).f32(), qc = lds_col8(sQ, PK, 0, 16 * db, lane).f32();
        f32x8 bK, bQ, bK2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int x = 8 * g4 + e;
          const float Gx = sG[x * GP + d];
          const float f = x <= mT ? __expf(GmR - Gx) : 0.f;     // t up to the end of block R
          const float hh = x >= mR ? __expf(Gx - GmT) : 0.f;    // r from the start of block T
          const float kx = kc[e] * sRk[x];
          bK[e] = kx * f;
          bQ[e] = qc[e] * sRq[x] * hh;
          bK2[e] = kx * hh;
        }
        const SplitFrag<T> fK = SplitFrag<T>::make(bK);
        f32x4 c1 = zero4(), c2 = zero4(), c3 = zero4(), c4 = zero4();
        mma_split(c1, aP, fK);
        mma_split(c2, aA, fK);
        mma_split(c3, aPT, SplitFrag<T>::make(bQ));
        mma_split(c4, aAT, SplitFrag<T>::make(bK2));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float e2 = __expf(Gr[i][e] - GmR), e1 = __expf(GmT - Gr[i][e]);
          dqP[i][e] = e2 * c1[e];
          dkA1[i][e] = e2 * c2[e];
          dkP[i][e] = e1 * c3[e];
          dkA2[i][e] = e1 * c4[e];
        }
      }
    } else {
      for (int x = 0; x < L; ++x) {
        const float bx = sB[x], rqx = sRq[x], rkx = sRk[x];
        float dpa[4], dpb[4], daa[4], dab[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rb + 4 * g4 + e;
          dpa[e] = sDP[r * CP + x];     // dP[r][x], x <= r
          daa[e] = sDA[r * CP + x];     // dA[r][x], x < r
          dpb[e] = sDP[x * CP + r];     // dP[x][r], x >= r
          dab[e] = bx * sDA[x * CP + r];
        }
#pragma unroll
        for (int i = 0; i < SCK; ++i) {
          const int d = 16 * ((wv + NW * i) / NRB) + r16;
          const float kx = to_float(sK[x * PK + d]) * rkx, qx = to_float(sQ[x * PK + d]) * rqx;
          const float gx = sG[x * GP + d];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * g4 + e;
            // exp(G_r - G_x) below the diagonal, exp(G_x - G_r) above it
            const float ex = __expf(x <= r ? Gr[i][e] - gx : gx - Gr[i][e]);
            if (x <= r) {
              dqP[i][e] += dpa[e] * kx * ex;
              dkA1[i][e] += daa[e] * kx * ex;
            }
            if (x >= r) {
              dkP[i][e] += dpb[e] * qx * ex;
              dkA2[i][e] += dab[e] * kx * ex;
            }
          }
        }
      }
    }

    // ---- per element: dq^, dk^ (group sums), dG; dbeta row parts; last-row extras
    {
      f32x4 rowb = zero4();
      // the wave's rows t = 16 rb + 4 g4 + e are the same in every slot: their
      // factors in one 16-byte read each, the raw q / k values in one
      // transposed read per slot
      const int r4 = 16 * rb + 4 * g4;
      const f32x4 B4 = *reinterpret_cast<const f32x4*>(&sB[r4]);
      const f32x4 RK4 = *reinterpret_cast<const f32x4*>(&sRk[r4]);
      const f32x4 RQ4 = *reinterpret_cast<const f32x4*>(&sRq[r4]);
#pragma unroll
      for (int i = 0; i < SCK; ++i) {
        const int db = (wv + NW * i) / NRB, d = 16 * db + r16;
        const float gl = sG[(L - 1) * GP + d];
        const f32x4 K4 = lds_rows4(sK, PK, r4, 16 * db, lane) * RK4;
        const f32x4 Q4 = lds_rows4(sQ, PK, r4, 16 * db, lane) * RQ4;
        float last = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = r4 + e;
          const bool ok = t < L;
          const float gt = sG[t * GP + d];
          const float gam = ok ? __expf(gt) : 0.f, kap = ok ? __expf(gl - gt) : 0.f;
          const float bt = B4[e];
          const float kv = K4[e], qv = Q4[e];
          const float dq = dqP[i][e] + gam * dQg[i][e];
          const float dk = bt * dkA1[i][e] + dkA2[i][e] + dkP[i][e] + bt * gam * TdW[i][e] + kap * dKt[i][e];
          const float dg = qv * dqP[i][e] - kv * dkP[i][e] + kv * bt * dkA1[i][e] - kv * dkA2[i][e] +
                           gam * qv * dQg[i][e] + bt * gam * kv * TdW[i][e] - kap * kv * dKt[i][e];
          sDG[t * GP + d] = ok ? dg : 0.f;
          sq_[i][e] += ok ? dq : 0.f;
          sk_[i][e] += ok ? dk : 0.f;
          rowb[e] += ok ? gam * kv * TdW[i][e] + kv * dkA1[i][e] : 0.f;
          last += kap * kv * dKt[i][e];
        }
        last = group4_sum(last);
        if (g4 == 0) sLast[rb * K + d] = last;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float s = lanes_sum_t<16>(rowb[e]);
        if (r16 == 0) sRowB[wv * C + 16 * rb + 4 * g4 + e] += s;
      }
    }
    lds_barrier();

    // ---- dg = reverse cumsum of dG per feature; dbeta
    for (int d = tid; d < K; d += NT) {
      float x = 0.f;
      for (int t = L - 1; t >= 0; --t) {
        x += sDG[t * GP + d];
        if (t == L - 1) {
          float ex = __expf(sG[(L - 1) * GP + d]) * sLr[d];
#pragma unroll
          for (int b = 0; b < NRB; ++b) ex += sLast[b * K + d];
          x += ex;
        }
        a.dg[((t0 + t) * HV + j) * K + d] = x;
      }
    }
    if (tid < L) {
      float db = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) db += sRowB[w * C + tid];
      a.dbeta[(t0 + tid) * HV + j] = a.beta_logits ? db * sB[tid] * (1.f - sB[tid]) : db;
    }
    lds_barrier();
  }

  // ---- L2-norm backward, dq / dk through LDS as 16-byte rows
  if (a.l2norm) {
    f32x4 qd = zero4(), kd = zero4();
#pragma unroll
    for (int i = 0; i < SCK; ++i) {
      const int db = (wv + NW * i) / NRB;
      qd += lds_rows4(sQ, PK, 16 * rb + 4 * g4, 16 * db, lane) * sq_[i];
      kd += lds_rows4(sK, PK, 16 * rb + 4 * g4, 16 * db, lane) * sk_[i];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rb + 4 * g4 + e;
      const float q1 = lanes_sum_t<16>(qd[e]), k1 = lanes_sum_t<16>(kd[e]);
      if (r16 == 0) {
        sDotQ[wv * C + r] = q1;
        sDotK[wv * C + r] = k1;
      }
    }
    lds_barrier();
  }
  {
    const int r4 = 16 * rb + 4 * g4;
    const f32x4 rq = *reinterpret_cast<const f32x4*>(&sRq[r4]), rk = *reinterpret_cast<const f32x4*>(&sRk[r4]);
    f32x4 cq = zero4(), ck = zero4();
    if (a.l2norm) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (w % NRB != rb) continue;
        cq += *reinterpret_cast<const f32x4*>(&sDotQ[w * C + r4]);
        ck += *reinterpret_cast<const f32x4*>(&sDotK[w * C + r4]);
      }
      cq *= rq * rq;
      ck *= rk * rk;
    }
#pragma unroll
    for (int i = 0; i < SCK; ++i) {
      const int db = (wv + NW * i) / NRB, d = 16 * db + r16;
      // dq^ is with respect to q^ = q rq; with the norm off rq = 1
      f32x4 oq = sq_[i], okv = sk_[i];
      if (a.l2norm) {
        oq = rq * (sq_[i] - cq * lds_rows4(sQ, PK, r4, 16 * db, lane));
        okv = rk * (sk_[i] - ck * lds_rows4(sK, PK, r4, 16 * db, lane));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sOq[(r4 + e) * PK + d] = (T)oq[e];
        sOk[(r4 + e) * PK + d] = (T)okv[e];
      }
    }
  }
  lds_barrier();
  T* dqp = static_cast<T*>(a.dq);
  T* dkp = static_cast<T*>(a.dk);
#pragma unroll
  for (int i = 0; i < NPQ; ++i) {
    const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
    if (idx < C * CPR && t < L) {
      st8(dqp + ((t0 + t) * H + h) * K + d8, ld8(&sOq[t * PK + d8]));
      st8(dkp + ((t0 + t) * H + h) * K + d8, ld8(&sOk[t * PK + d8]));
    }
  }
  };
  with_wave_index<4>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6), body);
}

template <typename T, int K>
hipError_t launch_t(const Args& a, hipStream_t s) {
  if constexpr (!B3P<T, K>::fits) {
    return hipErrorInvalidValue;    // rejected on the host before any launch
  } else {
    hipLaunchKernelGGL((b3pc_bwd_dqkvg<T, K>), dim3((unsigned)(a.NTmax * a.H)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
}

template <typename T>
hipError_t launch_k(const Args& a, hipStream_t s) {
  switch (a.K) {
    case 32: return launch_t<T, 32>(a, s);
    case 64: return launch_t<T, 64>(a, s);
    case 128: return launch_t<T, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool bwd_pc_fits(int dtype, int K) {
  if (dtype == GDR_BF16)
    return K == 32 ? B3P<bf16, 32>::fits : K == 64 ? B3P<bf16, 64>::fits : K == 128 ? B3P<bf16, 128>::fits : false;
  return K == 32 ? B3P<float, 32>::fits : K == 64 ? B3P<float, 64>::fits : K == 128 ? B3P<float, 128>::fits : false;
}

hipError_t launch_bwd_dqkvg_pc(const Args& a, hipStream_t s) {
  if (a.NTmax == 0) return hipSuccess;
  if (a.C != 32) return hipErrorInvalidValue;
  return a.dtype == GDR_BF16 ? launch_k<bf16>(a, s) : launch_k<float>(a, s);
}

}  // namespace gdr
