// B3: fused chunk-parallel backward (bwd_o + bwd_wy + bwd_dqk_intra).
//
// Per chunk (L rows), q/k head h and each value head j of its group, with S0 =
// h[c] (state entering the chunk), dS1 = dh[c] (gradient of the state leaving
// it), E = v_new, T = (I + A)^-1, gate G (chunk-local cumsum), gamma = exp(G),
// kappa = exp(G_L - G), row norms rq, rk and P[r][t] = q^_r . k^_t exp(G_r - G_t)
// (t <= r), the gradients of the chunk form on the coverage-matrix page ("FLA
// operator-kernel correctness testing and coverage matrix", section 2) are
//   dE   = scale P^T dO + diag(kappa) K^ dS1       (gradient of E)
//   Y    = T^T dE                                  dv = diag(beta) Y
//   dQg  = scale dO S0^T     T^T dW = -Y S0^T      dKt = E dS1^T
//   dP   = scale dO E^T      dA = -Y E^T (strictly lower)
// where dA = -T^T dT T^T collapses to -Y E^T because
// beta (V - diag(gamma) K^ S0) = (I + A) E, so the WY factors' gradient dT
// never has to be formed.  Then
//   dq^ = gamma dQg + D K^,               D[r][t] = dP[r][t] exp(G_r - G_t)
//   dk^ = kappa dKt + beta gamma T^T dW + D^T Q^ + Dk K^ + Dk^T K^,
//         Dk[t][m] = beta_t dA[t][m] exp(G_t - G_m)
//   dbeta_t = gamma_t k^_t . (T^T dW)_t + v_t . Y_t + sum_m dA[t][m] Abar[t][m]
//   dG (per row) from every exp(G) factor, dg = reverse cumsum of dG in the
//   chunk; finally the group sum over value heads (GVA) and the L2-norm
//   backward dx = (dx^ - x^ (x^ . dx^)) / |x|.
//
// gfx950 mapping: one workgroup (4 waves) per (chunk, q/k head); value heads
// of a GVA group run one after the other and sum dq^, dk^ in registers.
// Every operand sits in LDS as a row-major tile; MFMA fragments use the row
// contraction map and come from 16-byte row reads or ds_read_b64_tr_b16
// column reads, so any product (A or A^T times B or B^T) is one code path.
// fp32 intermediates that feed MFMAs (P, dE, Y, D, Dk, and dS1, which the
// reverse scan stores in fp32) are kept as bf16 hi + lo pairs.  The value dimension is streamed in tiles of 32 columns: per tile the
// kernel stages h^T, dh^T, dO, v and e^T, forms dE and Y (writing dv) and
// accumulates the C x K and C x C products above in registers; a wave owns a
// fixed set of 16 x 16 output blocks (one row block) for the whole chunk.  The
// next head's T tile, gate and beta are fetched into registers while the
// current head's last value tile is computed, and (one workgroup per CU) each
// value tile while the previous one is; dq and dk leave through an LDS tile
// as 16-byte row pieces.  Cross-lane sums use DPP row permutations.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

template <typename T, int C, int K, int NW>
struct B3 {
  static constexpr int NT = 64 * NW;
  static constexpr int VT = 32;
  static constexpr int EB = sizeof(T);
  static constexpr int CPR = K / 8;
  static constexpr int PK = K + 32 / EB;     // q, k, h^T, dh^T, dq / dk out rows
  static constexpr int PC = C + 32 / EB;     // T, e^T, P^T, D rows
  static constexpr int PV = VT + 32 / EB;    // dO, v, dE, Y rows
  static constexpr int NRB = C / 16, NKB = K / 16, NVB = VT / 16;
  static constexpr int KSK = K / 32, KSC = C / 32;
  static_assert(NW % NRB == 0, "a wave owns one row block");
  // 16 x 16 blocks per wave: block b = wave + NW * slot
  static constexpr int NBK = NRB * NKB, NBC = NRB * NRB, NBV = NRB * NVB;
  static constexpr int SCK = (NBK + NW - 1) / NW;
  static constexpr int SCC = (NBC + NW - 1) / NW;
  static constexpr int SCV = (NBV + NW - 1) / NW;
  // 8-element pieces per thread of the staged tiles
  static constexpr int NPQ = (C * CPR + NT - 1) / NT;        // q / k tiles
  static constexpr int NPT = (C * C / 8 + NT - 1) / NT;      // T tile
  static constexpr int NPH = (VT * CPR + NT - 1) / NT;       // h^T / dh^T tiles
  static constexpr int NPO = (C * VT / 8 + NT - 1) / NT;     // dO / v tiles
  static constexpr int NPE = (VT * C / 8 + NT - 1) / NT;     // e^T tile
  // LDS byte offsets
  static constexpr size_t oQ = 0;
  static constexpr size_t oK = oQ + (size_t)C * PK * EB;
  static constexpr size_t oT = oK + (size_t)C * PK * EB;
  static constexpr size_t oLoop = oT + (size_t)C * PC * EB;
  static constexpr size_t FCV = (size_t)C * PV * 4;     // fp32 operand tile C x PV (hi + lo)
  static_assert((size_t)VT * PC * (sizeof(T) == 2 ? 2 : 1) * sizeof(T) <= FCV, "dE^T (VT x PC) fits the dE slot");
  static_assert(C % 4 == 0, "16-byte row-factor reads");
  static constexpr size_t FCC = (size_t)C * PC * 4;     // fp32 operand tile C x PC
  static constexpr size_t lH = 0;
  static constexpr size_t lDH = lH + (size_t)VT * PK * EB;                    // dS1^T, hi (+ lo) tiles
  static constexpr size_t lDO = lDH + (size_t)VT * PK * EB * (sizeof(T) == 2 ? 2 : 1);
  static constexpr size_t lV = lDO + (size_t)C * PV * EB;
  static constexpr size_t lE = lV + (size_t)C * PV * EB;
  static constexpr size_t lDE = lE + (size_t)VT * PC * EB;
  static constexpr size_t lY = lDE + FCV;
  static constexpr size_t lPT = lY + FCV;
  static constexpr size_t loop_bytes = lPT + FCC;
  static constexpr size_t pD1 = 0, pD2 = FCC;
  static constexpr size_t pOq = 0, pOk = (size_t)C * PK * EB;
  static constexpr size_t post_bytes = 2 * FCC > 2 * pOk ? 2 * FCC : 2 * pOk;
  static constexpr size_t oRows = oLoop + (loop_bytes > post_bytes ? loop_bytes : post_bytes);
  // rows: G, rq, rk, beta; per-wave dG, dbeta, q.dq, k.dk partials; 2 NW scalars
  static constexpr size_t rows_floats = 4 * C + 4 * NW * C + 2 * NW;
  static constexpr size_t total = oRows + rows_floats * 4;
  static_assert(oRows % 16 == 0, "row factors start 16-byte aligned");
  static constexpr bool fits = total <= 160 * 1024;
  // the LDS holds the CU to one workgroup (four waves with 512 registers each)
  static constexpr bool one_per_cu = 2 * total > 160 * 1024;
  // Persistent workgroups (one per CU, each looping over items and requesting
  // the next item's rows during the current one's finish) where one workgroup
  // per CU runs anyway and no GVA group's registers compete; otherwise one
  // workgroup per item.
  template <bool GVA> static constexpr bool persistent() { return one_per_cu && !GVA; }
};

template <typename T, int C, int K, bool GVA, int NW>
__global__ __launch_bounds__(64 * NW) void b3_bwd_dqkvg(Args a) {
  using Cfg = B3<T, C, K, NW>;
  constexpr int NT = Cfg::NT, VT = Cfg::VT, PK = Cfg::PK, PC = Cfg::PC, PV = Cfg::PV, CPR = Cfg::CPR;
  constexpr int NRB = Cfg::NRB, NVB = Cfg::NVB, KSK = Cfg::KSK, KSC = Cfg::KSC;
  constexpr int NBK = Cfg::NBK, NBC = Cfg::NBC, NBV = Cfg::NBV;
  constexpr int SCK = Cfg::SCK, SCC = Cfg::SCC, SCV = Cfg::SCV;
  constexpr int NPQ = Cfg::NPQ, NPT = Cfg::NPT, NPH = Cfg::NPH, NPO = Cfg::NPO, NPE = Cfg::NPE;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::total];

  // the body below runs with its wave index as a compile-time constant
  // (with_wave_index): each wave's output-block slots and causal conditions
  // fold, so the MFMA loops unroll without runtime branches
  auto body = [&](auto wvc) {
  constexpr int wv = decltype(wvc)::value;
  // lane indices are re-read opaquely at the top of every item (below), so the
  // compiler recomputes addresses per item instead of hoisting them all out of
  // the item loop, where they would stay live across the whole item
  int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int64_t H = a.H, HV = a.HV, V = a.V;
  // Persistent workgroups: items (chunk, q/k head) blockIdx.x, blockIdx.x +
  // gridDim.x, ...; item i is chunk i / H, head i % H.
  struct Item {
    int64_t c, h, t0;
    int L;
  };
  const int64_t nitems = (int64_t)a.chunk_off[a.N] * H;
  auto item_at = [&](int64_t i) {
    Item it;
    it.c = i / H;
    it.h = i % H;
    it.t0 = a.chunk_idx[4 * it.c + 1];
    it.L = a.chunk_idx[4 * it.c + 2];
    return it;
  };
  int64_t item = blockIdx.x;
  if (item >= nitems) return;
  Item cur = item_at(item);
  const int ng = (int)(HV / H);
  const float scale = a.scale;

  T* sQ = reinterpret_cast<T*>(smem + Cfg::oQ);
  T* sK = reinterpret_cast<T*>(smem + Cfg::oK);
  T* sT = reinterpret_cast<T*>(smem + Cfg::oT);
  char* loop = smem + Cfg::oLoop;
  T* sH = reinterpret_cast<T*>(loop + Cfg::lH);
  const FTile<T> fDH = ftile<T, PK>(loop + Cfg::lDH, VT);   // dS1^T [v][d]
  T* sDO = reinterpret_cast<T*>(loop + Cfg::lDO);
  T* sV = reinterpret_cast<T*>(loop + Cfg::lV);
  T* sE = reinterpret_cast<T*>(loop + Cfg::lE);
  // fp32 operand tiles (bf16 hi + lo in LDS), stored in the orientation that
  // lets each lane write its accumulator's four consecutive elements as one
  // 8-byte store: fDE holds dE^T [v][t], fP holds P [r][t], fD1 / fD2 hold the
  // transposes of the D products' operands
  const FTile<T> fDE = ftile<T, PC>(loop + Cfg::lDE, VT);
  const FTile<T> fY = ftile<T, PV>(loop + Cfg::lY, C);
  const FTile<T> fP = ftile<T, PC>(loop + Cfg::lPT, C);
  const FTile<T> fD1 = ftile<T, PC>(loop + Cfg::pD1, C);
  const FTile<T> fD2 = ftile<T, PC>(loop + Cfg::pD2, C);
  T* sOq = reinterpret_cast<T*>(loop + Cfg::pOq);
  T* sOk = reinterpret_cast<T*>(loop + Cfg::pOk);
  float* sG = reinterpret_cast<float*>(smem + Cfg::oRows);
  float* sRq = sG + C;
  float* sRk = sRq + C;
  float* sB = sRk + C;
  float* sRowG = sB + C;           // [NW][C]
  float* sRowB = sRowG + NW * C;   // [NW][C]
  float* sDotQ = sRowB + NW * C;   // [NW][C]
  float* sDotK = sDotQ + NW * C;   // [NW][C]
  float* sRed = sDotK + NW * C;    // [2 NW]

  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ vp = static_cast<const T*>(a.v);
  const T* __restrict__ dop = static_cast<const T*>(a.d_o);

  // ---- global fetches into registers (staged into LDS later)
  struct HeadRegs {
    Frag<T> t[NPT];
    float g, b;
  };
  struct TileRegs {
    Frag<T> h[NPH], o[NPO], v[NPO], e[NPE];
    Frag<float> dh[NPH];     // dS1 (fp32)
  };
  auto fetch_head = [&](HeadRegs& R, const Item& I, int64_t j) {
    const int64_t c = I.c, t0 = I.t0;
    const int L = I.L;
    const T* tp = static_cast<const T*>(a.Tm) + (c * HV + j) * (int64_t)(C * C);
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int idx = tid + NT * i;
      R.t[i] = (idx < C * C / 8) ? ld8(tp + 8 * idx) : frag_zero<T>();
    }
    R.g = (tid < L) ? a.g[(t0 + tid) * HV + j] : 0.f;
    // raw beta (or logit): the sigmoid is taken where the row is staged, so
    // no instruction needs the loaded value (and waits for it and for every
    // load issued before it) while the fetch is in flight
    R.b = (tid < L) ? a.beta[(t0 + tid) * HV + j] : 0.f;
  };
  auto fetch_tile = [&](TileRegs& R, const Item& I, int64_t j, int64_t v0) {
    const int64_t c = I.c, t0 = I.t0;
    const int L = I.L;
    const T* hb = static_cast<const T*>(a.h) + ((c * HV + j) * V + v0) * (int64_t)K;
    const float* dhb = static_cast<const float*>(a.dh) + ((c * HV + j) * V + v0) * (int64_t)K;
    const T* eb = static_cast<const T*>(a.v_new) + ((c * HV + j) * V + v0) * (int64_t)C;
#pragma unroll
    for (int i = 0; i < NPH; ++i) {
      const int idx = tid + NT * i;
      const bool in = idx < VT * CPR;
      R.h[i] = in ? ld8(hb + 8 * idx) : frag_zero<T>();
      R.dh[i] = in ? ld8(dhb + 8 * idx) : frag_zero<float>();
    }
#pragma unroll
    for (int i = 0; i < NPO; ++i) {
      const int idx = tid + NT * i, t = idx / (VT / 8), v8 = (idx % (VT / 8)) * 8;
      const bool in = idx < C * VT / 8 && t < L;
      R.o[i] = in ? ld8(dop + ((t0 + t) * HV + j) * V + v0 + v8) : frag_zero<T>();
      R.v[i] = in ? ld8(vp + ((t0 + t) * HV + j) * V + v0 + v8) : frag_zero<T>();
    }
#pragma unroll
    for (int i = 0; i < NPE; ++i) {
      const int idx = tid + NT * i;
      R.e[i] = (idx < VT * C / 8) ? ld8(eb + 8 * idx) : frag_zero<T>();
    }
  };
  float lr = 0.f;     // sum of S0 o dS1 over the head (this thread's share)
  auto stage_tile = [&](const TileRegs& R) {
#pragma unroll
    for (int i = 0; i < NPH; ++i) {
      const int idx = tid + NT * i, v = idx / CPR, d8 = (idx % CPR) * 8;
      const f32x8 fx = R.h[i].f32(), fy = R.dh[i].f32();
      if (idx < VT * CPR) {
        st8(&sH[v * PK + d8], R.h[i]);
        const Frag<T> hi = Frag<T>::make(fy);
        st8(&fDH.hi[v * PK + d8], hi);
        if constexpr (FTile<T>::kSplit) st8(&fDH.lo[v * PK + d8], Frag<T>::make(fy - hi.f32()));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) lr += fx[e] * fy[e];
    }
#pragma unroll
    for (int i = 0; i < NPO; ++i) {
      const int idx = tid + NT * i, t = idx / (VT / 8), v8 = (idx % (VT / 8)) * 8;
      if (idx < C * VT / 8) {
        st8(&sDO[t * PV + v8], R.o[i]);
        st8(&sV[t * PV + v8], R.v[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < NPE; ++i) {
      const int idx = tid + NT * i, v = idx / (C / 8), t8 = (idx % (C / 8)) * 8;
      if (idx < VT * C / 8) st8(&sE[v * PC + t8], R.e[i]);
    }
  };

  HeadRegs HR;
  // The value tile's registers.  When the LDS already holds the CU to one
  // workgroup (whose four waves then have 512 registers each), each tile's
  // loads are issued one tile ahead -- the first head's first tile with the
  // q / k rows -- so their latency overlaps the previous tile's products
  // instead of stalling every tile; otherwise a tile is fetched where it is
  // staged, keeping two workgroups per CU.
  constexpr bool PF = Cfg::one_per_cu;
  TileRegs TN;
  // q, k rows of item I (rows past L are zero), and their staging with the
  // row norms
  Frag<T> qr[NPQ], kr[NPQ];
  auto fetch_qk = [&](const Item& I) {
#pragma unroll
    for (int i = 0; i < NPQ; ++i) {
      const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      const bool in = idx < C * CPR && t < I.L;
      qr[i] = in ? ld8(qp + ((I.t0 + t) * H + I.h) * K + d8) : frag_zero<T>();
      kr[i] = in ? ld8(kp + ((I.t0 + t) * H + I.h) * K + d8) : frag_zero<T>();
    }
  };
  auto stage_qk = [&]() {
#pragma unroll
    for (int i = 0; i < NPQ; ++i) {
      const int idx = tid + NT * i, t = idx / CPR, d8 = (idx % CPR) * 8;
      if (idx < C * CPR) {
        st8(&sQ[t * PK + d8], qr[i]);
        st8(&sK[t * PK + d8], kr[i]);
      }
      const f32x8 xq = qr[i].f32(), xk = kr[i].f32();
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq += xq[e] * xq[e];
        sk += xk[e] * xk[e];
      }
      sq = lanes_sum_t<CPR>(sq);
      sk = lanes_sum_t<CPR>(sk);
      if (idx < C * CPR && d8 == 0) {
        sRq[t] = a.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
        sRk[t] = a.l2norm ? 1.f / sqrtf(sk + kL2Eps) : 1.f;
      }
    }
    for (int i = tid; i < 2 * NW * C; i += NT) sDotQ[i] = 0.f;   // sDotQ and sDotK
  };
  // the first item's rows, with its first head's T tile, gate and beta (and
  // first value tile) already on the way
  fetch_qk(cur);
  fetch_head(HR, cur, cur.h * ng);
  if constexpr (PF) fetch_tile(TN, cur, cur.h * ng, 0);

  // a wave's fixed output blocks: slot i of a product is block b = wv + NW i,
  // row block b % NRB (= wv % NRB), column block b / NRB
  const int rb = wv % NRB;
  f32x4 dq[SCK], dk[SCK];          // dq^, dk^ of the current value head
  f32x4 sq_[GVA ? SCK : 1], sk_[GVA ? SCK : 1];

  for (;;) {
  asm volatile("" : "+v"(tid), "+v"(lane), "+v"(r16), "+v"(g4));
  const int64_t h = cur.h, t0 = cur.t0;
  const int L = cur.L;
  stage_qk();
  if constexpr (GVA) {
#pragma unroll
    for (int i = 0; i < SCK; ++i) sq_[i] = sk_[i] = zero4();
  }

  for (int jj = 0; jj < ng; ++jj) {
    const int64_t j = h * ng + jj;
    // ---- per-head rows and the T tile
    {
      const float G = wave_incl_scan(HR.g, lane);
      if (wv == 0 && lane < C) sG[lane] = G;
      if (tid < C) sB[tid] = tid < L ? beta_value(HR.b, a.beta_logits) : 0.f;
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int idx = tid + NT * i, r = idx / (C / 8), c8 = (idx % (C / 8)) * 8;
        if (idx < C * C / 8) st8(&sT[r * PC + c8], HR.t[i]);
      }
    }
    for (int i = tid; i < 2 * NW * C; i += NT) sRowG[i] = 0.f;     // sRowG and sRowB
    if (tid < 2 * NW) sRed[tid] = 0.f;
    lr = 0.f;
    lds_barrier();
    const float GL = sG[L - 1];
    // dE's row factors kappa_t rk_t for the wave's rows t = 16 rb + 4 g4 + e
    // (every dE slot of a wave has row block rb), formed once per head
    f32x4 kapE;
    {
      const int t4 = 16 * rb + 4 * g4;
      const f32x4 G4 = *reinterpret_cast<const f32x4*>(&sG[t4]);
      const f32x4 K4 = *reinterpret_cast<const f32x4*>(&sRk[t4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) kapE[e] = (t4 + e < L) ? __expf(GL - G4[e]) * K4[e] : 0.f;
    }

    // ---- P tile, P[r][t] (norms, gate, causal mask applied).  Slot i's block
    //      has key rows t in the wave's row block rb (tb = b % NRB = rb) and
    //      query rows r in block cb: the key fragments and the factors of the
    //      rows t are read once; blocks with rb > cb are zero.
    {
      const int r4 = 16 * rb + 4 * g4;
      const f32x4 Gt4 = *reinterpret_cast<const f32x4*>(&sG[r4]);
      const f32x4 Rkt4 = *reinterpret_cast<const f32x4*>(&sRk[r4]);
      Frag<T> kr[KSK];
#pragma unroll
      for (int ks = 0; ks < KSK; ++ks) kr[ks] = ld8(&sK[(16 * rb + r16) * PK + 32 * ks + 8 * g4]);
#pragma unroll
      for (int i = 0; i < SCC; ++i) {
        const int b = wv + NW * i, cb = b / NRB;
        if (b >= NBC) continue;
        const int r = 16 * cb + r16;
        f32x4 pv = zero4();
        if (rb <= cb) {
          f32x4 acc = zero4();
#pragma unroll
          for (int ks = 0; ks < KSK; ++ks) mma(acc, kr[ks], ld8(&sQ[r * PK + 32 * ks + 8 * g4]));
          const float Gr = sG[r], Rqr = sRq[r];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = r4 + e <= r && r < L;
            pv[e] = ok ? acc[e] * Rqr * Rkt4[e] * __expf(Gr - Gt4[e]) : 0.f;
          }
        }
        fP.put4(r, r4, pv);
      }
    }

    f32x4 dQg[SCK], TdW[SCK], dKt[SCK], dP[SCC], dA[SCC];
#pragma unroll
    for (int i = 0; i < SCK; ++i) dQg[i] = TdW[i] = dKt[i] = zero4();
#pragma unroll
    for (int i = 0; i < SCC; ++i) dP[i] = dA[i] = zero4();

    for (int64_t v0 = 0; v0 < V; v0 += VT) {
      if constexpr (!PF) fetch_tile(TN, cur, j, v0);
      stage_tile(TN);
      lds_barrier();
      if (v0 + VT >= V && jj + 1 < ng) fetch_head(HR, cur, j + 1);
      if constexpr (PF) {
        if (v0 + VT < V) {
          fetch_tile(TN, cur, j, v0 + VT);
        } else if (jj + 1 < ng) {
          fetch_tile(TN, cur, j + 1, 0);
        }
      }

      // ---- dE[t][v] = scale (P^T dO)[t][v] + kappa_t rk_t (K dS1)[t][v]
#pragma unroll
      for (int i = 0; i < SCV; ++i) {
        const int b = wv + NW * i, tb = b % NRB, vb = b / NRB;
        if (b >= NBV) continue;
        f32x4 a1 = zero4(), a2 = zero4();
#pragma unroll
        for (int s = 0; s < KSC; ++s) {
          if (32 * s + 31 < 16 * tb) continue;
          mma_split(a1, fP.col(32 * s, 16 * tb, lane), lds_col8(sDO, PV, 32 * s, 16 * vb, lane));
        }
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks)
          mma_split(a2, ld8(&sK[(16 * tb + r16) * PK + 32 * ks + 8 * g4]), fDH.row(16 * vb + r16, 32 * ks, lane));
        static_assert(NW % NRB == 0, "every dE slot of a wave has row block rb");
        const f32x4 dv4 = scale * a1 + kapE * a2;
        fDE.put4(16 * vb + r16, 16 * tb + 4 * g4, dv4);
      }
      lds_barrier();

      // ---- Y^T[v][t] = (dE^T T)[v][t]; dv = beta Y; dbeta += v . Y
#pragma unroll
      for (int i = 0; i < SCV; ++i) {
        const int b = wv + NW * i, vb = b % NVB, tb = b / NVB;
        if (b >= NBV) continue;
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < KSC; ++s) {
          if (32 * s + 31 < 16 * tb) continue;
          mma_split(acc, fDE.row(16 * vb + r16, 32 * s, lane), lds_col8(sT, PC, 32 * s, 16 * tb, lane));
        }
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
        const Frag<T> aE = lds_col8(sE, PC, 0, 16 * rb, lane);
#pragma unroll
        for (int i = 0; i < SCK; ++i) {
          const int b = wv + NW * i, db = b / NRB;
          if (b >= NBK) continue;
          const Frag<T> bS = lds_col8(sH, PK, 0, 16 * db, lane);
          mma(dQg[i], aO, bS);
          mma_split(TdW[i], aY, bS);
          mma_split(dKt[i], aE, fDH.col(0, 16 * db, lane));
        }
#pragma unroll
        for (int i = 0; i < SCC; ++i) {
          const int b = wv + NW * i, cb = b / NRB;
          if (b >= NBC) continue;
          const Frag<T> bE = lds_col8(sE, PC, 0, 16 * cb, lane);
          mma(dP[i], aO, bE);
          mma_split(dA[i], aY, bE);
        }
      }
      lds_barrier();
    }

    // ---- S0 . dS1 (for the exp(G_L) factor of the state hand-off)
    lr = lanes_sum_t<64>(lr);
    if (lane == 0) sRed[wv] = lr;

    // ---- D = dP o exp(G_r - G_t) (causal); dG from P.  The wave's rows
    //      r = 16 rb + 4 g4 + e are the same in every slot: their factors are
    //      read once and their sums over t stay in registers until one
    //      reduction after the slots; blocks above the diagonal are zero.
    const int r4 = 16 * rb + 4 * g4;
    const f32x4 Gr4 = *reinterpret_cast<const f32x4*>(&sG[r4]);
    const f32x4 Rq4 = *reinterpret_cast<const f32x4*>(&sRq[r4]);
    const f32x4 Rk4 = *reinterpret_cast<const f32x4*>(&sRk[r4]);
    const f32x4 B4 = *reinterpret_cast<const f32x4*>(&sB[r4]);
    f32x4 Dv[SCC];
    {
      f32x4 rowP = zero4();
#pragma unroll
      for (int i = 0; i < SCC; ++i) {
        const int b = wv + NW * i, cb = b / NRB;
        Dv[i] = zero4();
        if (b >= NBC || cb > rb) continue;
        const int t = 16 * cb + r16;
        const float Gt = sG[t];
        const f32x4 P4 = fP.get4(r4, 16 * cb, lane);
        float colsum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = t <= r4 + e && r4 + e < L;
          const float dps = scale * dP[i][e];
          Dv[i][e] = ok ? dps * __expf(Gr4[e] - Gt) : 0.f;
          const float pd = ok ? dps * P4[e] : 0.f;
          rowP[e] += pd;
          colsum += pd;
        }
        colsum = group4_sum(colsum);
        if (g4 == 0) sRowG[wv * C + t] -= colsum;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float rs = lanes_sum_t<16>(rowP[e]);
        if (r16 == 0) sRowG[wv * C + r4 + e] += rs;
      }
    }
    lds_barrier();     // P^T is dead: D tiles overlay it

    // ---- D tiles; row-dot terms of dG / dbeta; dq^, dk^ row-scaled parts
#pragma unroll
    for (int i = 0; i < SCC; ++i) {
      const int b = wv + NW * i, cb = b / NRB;
      if (b >= NBC) continue;
      const int t = 16 * cb + r16;
      fD1.put4(t, r4, Dv[i] * sRk[t]);
      fD2.put4(t, r4, Dv[i] * Rq4);
    }
    {
      f32x4 qd = zero4(), kw = zero4(), kk = zero4();
#pragma unroll
      for (int i = 0; i < SCK; ++i) {
        const int b = wv + NW * i, db = b / NRB;
        dQg[i] *= scale;
        TdW[i] = -TdW[i];
        if (b >= NBK) continue;
        const f32x4 q4 = lds_rows4(sQ, PK, r4, 16 * db, lane), k4 = lds_rows4(sK, PK, r4, 16 * db, lane);
        qd += q4 * dQg[i];
        kw += k4 * TdW[i];
        kk += k4 * dKt[i];
      }
      float last = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r4 + e;
        const float q1 = lanes_sum_t<16>(qd[e]), k1 = lanes_sum_t<16>(kw[e]), k2 = lanes_sum_t<16>(kk[e]);
        const bool ok = r < L;
        const float gam = __expf(Gr4[e]), kap = __expf(GL - Gr4[e]);
        const float tw = ok ? gam * Rk4[e] * k1 : 0.f;
        const float kt = ok ? kap * Rk4[e] * k2 : 0.f;
        if (r16 == 0) {
          sRowG[wv * C + r] += (ok ? gam * Rq4[e] * q1 : 0.f) + B4[e] * tw - kt;
          sRowB[wv * C + r] += tw;
        }
        last += kt;
#pragma unroll
        for (int i = 0; i < SCK; ++i) {
          dq[i][e] = gam * dQg[i][e];
          dk[i][e] = kap * dKt[i][e] + B4[e] * gam * TdW[i][e];
        }
      }
      last = group4_sum(last);
      if (lane == 0) sRed[NW + wv] = last;
    }
    lds_barrier();

    // ---- dq^ += D~ K (D~ = D rk_t), dk^ += D^^T Q (D^ = D rq_r)
#pragma unroll
    for (int i = 0; i < SCK; ++i) {
      const int b = wv + NW * i, db = b / NRB;
      if (b >= NBK) continue;
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        if (32 * s <= 16 * rb + 15)
          mma_split(dq[i], fD1.col(32 * s, 16 * rb, lane), lds_col8(sK, PK, 32 * s, 16 * db, lane));
        if (32 * s + 31 >= 16 * rb)
          mma_split(dk[i], fD2.row(16 * rb + r16, 32 * s, lane), lds_col8(sQ, PK, 32 * s, 16 * db, lane));
      }
    }
    lds_barrier();

    // ---- dA (strictly lower): dbeta, dG and the Dk tiles
    {
      f32x4 rowB = zero4(), rowG = zero4();
#pragma unroll
      for (int i = 0; i < SCC; ++i) {
        const int b = wv + NW * i, cb = b / NRB;
        if (b >= NBC) continue;
        const int m = 16 * cb + r16;
        f32x4 d1v = zero4(), d2v = zero4();
        if (cb <= rb) {
          f32x4 kk = zero4();
#pragma unroll
          for (int ks = 0; ks < KSK; ++ks)
            mma(kk, ld8(&sK[(16 * rb + r16) * PK + 32 * ks + 8 * g4]), ld8(&sK[(16 * cb + r16) * PK + 32 * ks + 8 * g4]));
          const float Gm = sG[m], Rkm = sRk[m];
          float colsum = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = r4 + e;
            const bool ok = m < t && t < L;
            const float da = -dA[i][e];
            const float ex = ok ? __expf(Gr4[e] - Gm) : 0.f;
            const float abar = Rk4[e] * Rkm * kk[e] * ex;
            const float dbp = ok ? da * abar : 0.f;
            const float dkv = ok ? B4[e] * da * ex : 0.f;
            const float ad = B4[e] * dbp;
            rowB[e] += dbp;
            rowG[e] += ad;
            colsum += ad;
            d1v[e] = dkv * Rkm;
            d2v[e] = dkv * Rk4[e];
          }
          colsum = group4_sum(colsum);
          if (g4 == 0) sRowG[wv * C + m] -= colsum;
        }
        fD1.put4(m, r4, d1v);
        fD2.put4(m, r4, d2v);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float rb1 = lanes_sum_t<16>(rowB[e]), rg = lanes_sum_t<16>(rowG[e]);
        if (r16 == 0) {
          sRowB[wv * C + r4 + e] += rb1;
          sRowG[wv * C + r4 + e] += rg;
        }
      }
    }
    lds_barrier();

    // ---- dk^ += Dk~ K + Dk^^T K
#pragma unroll
    for (int i = 0; i < SCK; ++i) {
      const int b = wv + NW * i, db = b / NRB;
      if (b >= NBK) continue;
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        if (32 * s <= 16 * rb + 15)
          mma_split(dk[i], fD1.col(32 * s, 16 * rb, lane), lds_col8(sK, PK, 32 * s, 16 * db, lane));
        if (32 * s + 31 >= 16 * rb)
          mma_split(dk[i], fD2.row(16 * rb + r16, 32 * s, lane), lds_col8(sK, PK, 32 * s, 16 * db, lane));
      }
    }
    if constexpr (GVA) {
#pragma unroll
      for (int i = 0; i < SCK; ++i) {
        sq_[i] += dq[i];
        sk_[i] += dk[i];
      }
    }
    lds_barrier();

    // ---- dg = reverse cumsum of dG over the chunk, dbeta
    if (wv == 0) {
      float lrt = 0.f, lst = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        lrt += sRed[w];
        lst += sRed[NW + w];
      }
      const int tr = C - 1 - lane;            // this lane's row, reversed
      float x = 0.f;
      if (lane < C && tr < L) {
#pragma unroll
        for (int w = 0; w < NW; ++w) x += sRowG[w * C + tr];
        if (tr == L - 1) x += lst + __expf(GL) * lrt;
      }
      const float y = wave_incl_scan(x, lane);
      if (lane < C && tr < L) a.dg[(t0 + tr) * HV + j] = y;
    }
    if (wv == 1) {      // dbeta beside wave 0's dg
      if (lane < L) {
        float db = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) db += sRowB[w * C + lane];
        // with logits, d/dx sigmoid(x) = beta (1 - beta)
        a.dbeta[(t0 + lane) * HV + j] = a.beta_logits ? db * sB[lane] * (1.f - sB[lane]) : db;
      }
    }
    lds_barrier();
  }

  // ---- group sums, L2-norm backward, dq / dk through LDS as 16-byte rows
  // (rows r4 + e of every slot: the raw q / k values in one transposed read per
  // slot and tile, the row factors in one read each)
  auto finish = [&](const f32x4 (&DQ)[SCK], const f32x4 (&DK)[SCK]) {
    const int r4 = 16 * rb + 4 * g4;
    if (a.l2norm) {
      f32x4 qd = zero4(), kd = zero4();
#pragma unroll
      for (int i = 0; i < SCK; ++i) {
        const int b = wv + NW * i, db = b / NRB;
        if (b >= NBK) continue;
        qd += lds_rows4(sQ, PK, r4, 16 * db, lane) * DQ[i];
        kd += lds_rows4(sK, PK, r4, 16 * db, lane) * DK[i];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float q1 = lanes_sum_t<16>(qd[e]), k1 = lanes_sum_t<16>(kd[e]);
        if (r16 == 0) {
          sDotQ[wv * C + r4 + e] = q1;
          sDotK[wv * C + r4 + e] = k1;
        }
      }
      lds_barrier();
    }
    const f32x4 rq = *reinterpret_cast<const f32x4*>(&sRq[r4]), rk = *reinterpret_cast<const f32x4*>(&sRk[r4]);
    f32x4 cq = zero4(), ck = zero4();
    if (a.l2norm) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        cq += *reinterpret_cast<const f32x4*>(&sDotQ[w * C + r4]);
        ck += *reinterpret_cast<const f32x4*>(&sDotK[w * C + r4]);
      }
      cq *= rq * rq;
      ck *= rk * rk;
    }
#pragma unroll
    for (int i = 0; i < SCK; ++i) {
      const int b = wv + NW * i, db = b / NRB, d = 16 * db + r16;
      if (b >= NBK) continue;
      f32x4 oq = DQ[i], okv = DK[i];
      if (a.l2norm) {
        oq = rq * (DQ[i] - cq * lds_rows4(sQ, PK, r4, 16 * db, lane));
        okv = rk * (DK[i] - ck * lds_rows4(sK, PK, r4, 16 * db, lane));
      }
      if constexpr (sizeof(T) == 2) {
        // adjacent columns pair up (DPP lane swap within each lane pair): the
        // even lane writes rows r4, r4 + 1 and the odd lane rows r4 + 2, r4 + 3,
        // each as one 4-byte (two-column) LDS write instead of four 2-byte ones
        const bool odd = r16 & 1;
        const int row0 = r4 + (odd ? 2 : 0), col = d - (odd ? 1 : 0);
        auto pair_store = [&](T* tile, const f32x4 x) {
          const float p0 = dpp_f<0xB1>(odd ? x[0] : x[2]), p1 = dpp_f<0xB1>(odd ? x[1] : x[3]);
          using P2 = T __attribute__((ext_vector_type(2)));
          *reinterpret_cast<P2*>(&tile[row0 * PK + col]) = P2{(T)(odd ? p0 : x[0]), (T)(odd ? x[2] : p0)};
          *reinterpret_cast<P2*>(&tile[(row0 + 1) * PK + col]) = P2{(T)(odd ? p1 : x[1]), (T)(odd ? x[3] : p1)};
        };
        pair_store(sOq, oq);
        pair_store(sOk, okv);
      } else {
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
  // the next item's rows, T tile, gate, beta and first value tile are
  // requested before this item's finish, which hides their latency (the value
  // tile's registers are free once this item's last tile is staged)
  const int64_t next = item + gridDim.x;
  const bool more = Cfg::template persistent<GVA>() && next < nitems;
  Item nx = cur;
  if (more) {
    nx = item_at(next);
    fetch_qk(nx);
    fetch_head(HR, nx, nx.h * ng);
    fetch_tile(TN, nx, nx.h * ng, 0);
  }
  if constexpr (GVA) {
    finish(sq_, sk_);
  } else {
    finish(dq, dk);
  }
  if constexpr (!Cfg::template persistent<GVA>()) break;
  if (!more) break;
  item = next;
  cur = nx;
  lds_barrier();      // the finish's LDS reads end before the next item's staging
  }   // items
  };
  with_wave_index<NW>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6), body);
}

// Four waves (one per SIMD): the kernel holds about 400 live registers per
// lane at chunk 64, which two waves per SIMD (256 each) cannot hold without
// spilling.
template <typename T, int C, int K>
constexpr int b3_waves() {
  return 4;
}

template <typename T, int C, int K>
hipError_t launch_t(const Args& a, hipStream_t s) {
  constexpr int NW = b3_waves<T, C, K>();
  if constexpr (!B3<T, C, K, NW>::fits) {
    return hipErrorInvalidValue;    // rejected on the host before any launch
  } else {
    // one workgroup per CU that loops over the items, or one per item
    using Cfg = B3<T, C, K, NW>;
    const int64_t items = a.NTmax * a.H;
    const bool pers = a.HV == a.H ? Cfg::template persistent<false>() : Cfg::template persistent<true>();
    const dim3 grid((unsigned)(pers && items > kNumCUs ? kNumCUs : items));
    if (a.HV == a.H)
      hipLaunchKernelGGL((b3_bwd_dqkvg<T, C, K, false, NW>), grid, dim3(64 * NW), 0, s, a);
    else
      hipLaunchKernelGGL((b3_bwd_dqkvg<T, C, K, true, NW>), grid, dim3(64 * NW), 0, s, a);
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

template <typename T>
hipError_t launch_c(const Args& a, hipStream_t s) {
  return a.C == 32 ? launch_k<T, 32>(a, s) : launch_k<T, 64>(a, s);
}

}  // namespace

bool bwd_fused_fits(int dtype, int C, int K) {
  bool ok = false;
#define GDR_B3_FITS(TT, CC, KK) \
  if (C == CC && K == KK) ok = B3<TT, CC, KK, b3_waves<TT, CC, KK>()>::fits;
  if (dtype == GDR_BF16) {
    GDR_B3_FITS(bf16, 32, 32) GDR_B3_FITS(bf16, 32, 64) GDR_B3_FITS(bf16, 32, 128)
    GDR_B3_FITS(bf16, 64, 32) GDR_B3_FITS(bf16, 64, 64) GDR_B3_FITS(bf16, 64, 128)
  } else {
    GDR_B3_FITS(float, 32, 32) GDR_B3_FITS(float, 32, 64) GDR_B3_FITS(float, 32, 128)
    GDR_B3_FITS(float, 64, 32) GDR_B3_FITS(float, 64, 64) GDR_B3_FITS(float, 64, 128)
  }
#undef GDR_B3_FITS
  return ok;
}

hipError_t launch_bwd_dqkvg(const Args& a, hipStream_t s) {
  if (a.NTmax == 0) return hipSuccess;
  return a.dtype == GDR_BF16 ? launch_c<bf16>(a, s) : launch_c<float>(a, s);
}

}  // namespace gdr
