// K5: token-by-token (fused recurrent) forward of the gated delta rule.
//
// For one sequence, value head j and a 16-column slice of the state, the
// recurrence is applied one token at a time with the state in registers:
//   S' = D_t S                     D_t = diag(exp(g_t)), scalar or per channel
//   e  = beta_t (v_t - S'^T k^_t)
//   S  = S' + k^_t e^T
//   o_t = scale * S^T q^_t
// This is the per-token form the chunk form of the coverage-matrix page
// ("FLA operator-kernel correctness testing and coverage matrix", sections 2
// and 3: the fused_recurrent entry point beside chunk) reorganises; it needs no
// chunk table and no workspace, which suits decoding and short sequences.
//
// gfx950 mapping (one wave per workgroup):
//  * lane l holds column vc = l / 4 of the slice and the K / 4 state rows
//    kq * K / 4 .. of kq = l % 4, so every row reduction (S'^T k, S^T q) is a
//    quad sum on DPP (two cross-lane adds inside a 16-lane row);
//  * tokens arrive in blocks of 16: the wave loads the next block's k, q, v,
//    g and beta into registers (coalesced 16-byte loads, issued before the
//    current block is computed) and stages them in LDS, with the key / query
//    row norms and the gate exponentials computed once per element there;
//  * rows past the end of the sequence are staged as zeros (g = beta = k = 0),
//    which would leave the state exactly unchanged; the unrolled token loop
//    still stops at the last valid row (a scalar branch), so a decoding step
//    of one token does one token's work;
//  * outputs of a block leave through an LDS tile, four consecutive columns
//    per lane.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

constexpr int kBV = 16;   // state columns per workgroup
constexpr int kTB = 16;   // tokens per staged block

template <typename T, int K, bool PC>
__global__ __launch_bounds__(64) void k5_recurrent(Args a) {
  constexpr int KR = K / 4;             // state rows per lane
  constexpr int KV8 = K / 8;            // 8-element pieces per key row
  constexpr int NKL = kTB * KV8 / 64;   // key (and query) pieces per lane per block
  constexpr int NGL = PC ? kTB * K / 4 / 64 : 1;   // per-channel gate quads per lane
  static_assert(NKL >= 1 && (kTB * KV8) % 64 == 0, "key pieces must tile the wave");

  // The state tile (h0 in, ht out) is live only before the first block is
  // staged and after the last one is computed, so it shares its LDS with the
  // key / query tiles: a one-wave workgroup then holds about 10 KB of LDS
  // (K = 128, bf16) and a CU keeps twice as many decoding waves resident.
  constexpr int kKQBytes = 2 * kTB * K * (int)sizeof(T);
  constexpr int kSBytes = K * kBV * 4;
  __shared__ __attribute__((aligned(16))) char sKQS[kKQBytes > kSBytes ? kKQBytes : kSBytes];
  T* const sK = reinterpret_cast<T*>(sKQS);
  T* const sQ = sK + kTB * K;
  float* const sS = reinterpret_cast<float*>(sKQS);
  __shared__ __attribute__((aligned(16))) float sG[PC ? kTB * K : kTB];   // exp(g)
  __shared__ __attribute__((aligned(16))) float sV[kTB * kBV];
  __shared__ __attribute__((aligned(16))) float sO[kTB * kBV];
  __shared__ float sB[kTB], sRk[kTB], sRq[kTB];

  const int lane = threadIdx.x, kq = lane & 3, vc = lane >> 2;
  const int64_t NVT = a.V / kBV;
  const int64_t bid = xcd_remap(blockIdx.x, (int64_t)gridDim.x);
  const int64_t vt = bid % NVT, j = (bid / NVT) % a.HV, n = bid / (NVT * a.HV);
  const int64_t H = a.H, HV = a.HV, V = a.V, hq = j / (HV / H);
  int64_t bos, len;
  if (a.cu != nullptr) {
    bos = a.cu[n];
    len = (int64_t)a.cu[n + 1] - bos;
  } else {
    bos = n * a.T;
    len = a.T;
  }
  const int64_t v0 = vt * kBV;
  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ vp = static_cast<const T*>(a.v);
  T* __restrict__ op = static_cast<T*>(a.o);

  // ---- block loads into registers (addresses clamped to the sequence; rows
  // past its end are zeroed when staged, never at the load)
  struct Blk {
    v8_t<T> k[NKL], q[NKL];
    f32x4 v;
    float gb;
    f32x4 gc[NGL];
  };
  auto load = [&](int64_t blk, Blk& b) {
    const int64_t last = len - 1 - blk * kTB;    // last valid row of the block
#pragma unroll
    for (int m = 0; m < NKL; ++m) {
      const int idx = lane + 64 * m, row = idx / KV8, piece = idx % KV8;
      const int64_t t = bos + blk * kTB + (row <= last ? row : last);
      const int64_t off = (t * H + hq) * K + 8 * piece;
      b.k[m] = ld8(kp + off).v;
      b.q[m] = ld8(qp + off).v;
    }
    {
      const int row = lane >> 2, c4 = 4 * (lane & 3);
      const int64_t t = bos + blk * kTB + (row <= last ? row : last);
      b.v = ld4f(vp + (t * HV + j) * V + v0 + c4);
    }
    {
      const int row = lane & (kTB - 1);
      const int64_t t = bos + blk * kTB + (row <= last ? row : last);
      if (lane < kTB) b.gb = PC ? 0.f : a.g[t * HV + j];
      else if (lane < 2 * kTB) b.gb = beta_value(a.beta[t * HV + j], a.beta_logits);
      else b.gb = 0.f;
    }
    if constexpr (PC) {
#pragma unroll
      for (int m = 0; m < NGL; ++m) {
        const int idx = lane + 64 * m, row = idx / (K / 4), c4 = 4 * (idx % (K / 4));
        const int64_t t = bos + blk * kTB + (row <= last ? row : last);
        b.gc[m] = *reinterpret_cast<const f32x4*>(a.g + (t * HV + j) * K + c4);
      }
    }
  };

  // ---- staging into LDS: zero rows past the end, row norms, gate exponentials
  auto stage = [&](int64_t blk, const Blk& b) {
    const int64_t nvalid = len - blk * kTB;
#pragma unroll
    for (int m = 0; m < NKL; ++m) {
      const int idx = lane + 64 * m, row = idx / KV8, piece = idx % KV8;
      const bool ok = row < nvalid;
      const f32x8 kf = ok ? to_f32<T>(b.k[m]) : zero8();
      const f32x8 qf = ok ? to_f32<T>(b.q[m]) : zero8();
      *reinterpret_cast<v8_t<T>*>(sK + row * K + 8 * piece) = cvt8<T>(kf);
      *reinterpret_cast<v8_t<T>*>(sQ + row * K + 8 * piece) = cvt8<T>(qf);
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sk = __builtin_fmaf(kf[e], kf[e], sk);
        sq = __builtin_fmaf(qf[e], qf[e], sq);
      }
      // a row's pieces sit in KV8 consecutive lanes
      sk = lanes_sum_t<KV8>(sk);
      sq = lanes_sum_t<KV8>(sq);
      if (piece == 0) {
        sRk[row] = a.l2norm ? 1.f / sqrtf(sk + kL2Eps) : 1.f;
        sRq[row] = a.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
      }
    }
    {
      const int row = lane >> 2, c4 = 4 * (lane & 3);
      *reinterpret_cast<f32x4*>(sV + row * kBV + c4) = row < nvalid ? b.v : zero4();
    }
    {
      const int row = lane & (kTB - 1);
      const bool ok = row < nvalid;
      if (lane < kTB) {
        if constexpr (!PC) sG[row] = ok ? __expf(b.gb) : 1.f;
      } else if (lane < 2 * kTB) {
        sB[row] = ok ? b.gb : 0.f;
      }
    }
    if constexpr (PC) {
#pragma unroll
      for (int m = 0; m < NGL; ++m) {
        const int idx = lane + 64 * m, row = idx / (K / 4), c4 = 4 * (idx % (K / 4));
        f32x4 x = f32x4{1.f, 1.f, 1.f, 1.f};
        if (row < nvalid) {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = __expf(b.gc[m][e]);
        }
        *reinterpret_cast<f32x4*>(sG + row * K + c4) = x;
      }
    }
  };

  // the first block's loads are issued before the state's, so a decoding
  // step pays one memory round trip for both
  const int64_t nblk = (len + kTB - 1) / kTB;
  Blk cur;
  if (nblk > 0) load(0, cur);

  // state: rows kq * KR + i, column v0 + vc, in fp32
  // h0 / ht pass through an LDS tile so that HBM sees 16-byte accesses (four
  // consecutive columns per lane, 64 contiguous bytes per row)
  constexpr int NSL = K * kBV / 4 / 64;   // state quads per lane
  const int64_t hbase = (n * HV + j) * K * V + v0;
  float S[KR];
  if (a.h0 != nullptr) {
    f32x4 hq4[NSL];
#pragma unroll
    for (int m = 0; m < NSL; ++m) {
      const int idx = lane + 64 * m, r = idx >> 2, c4 = 4 * (idx & 3);
      hq4[m] = *reinterpret_cast<const f32x4*>(a.h0 + hbase + (int64_t)r * V + c4);
    }
#pragma unroll
    for (int m = 0; m < NSL; ++m) {
      const int idx = lane + 64 * m, r = idx >> 2, c4 = 4 * (idx & 3);
      *reinterpret_cast<f32x4*>(sS + r * kBV + c4) = hq4[m];
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < KR; ++i) S[i] = sS[(kq * KR + i) * kBV + vc];
  } else {
#pragma unroll
    for (int i = 0; i < KR; ++i) S[i] = 0.f;
  }

  for (int64_t blk = 0; blk < nblk; ++blk) {
    lds_barrier();                 // the previous block's reads of LDS are done
    stage(blk, cur);
    if (blk + 1 < nblk) load(blk + 1, cur);
    lds_barrier();

    // rows past the end of the sequence are no-ops on the state; a partial
    // block (the last, or a decoding step's only one) skips them with a
    // scalar branch
    const int nv = (int)(len - blk * kTB < kTB ? len - blk * kTB : kTB);
#pragma unroll
    for (int tt = 0; tt < kTB; ++tt) {
      // Every operation is spelled out (no contraction left to the compiler),
      // so a token's arithmetic does not depend on its position in the
      // unrolled block: handing the state over between calls is exact.
      if (tt < nv) {
#pragma clang fp contract(off)
      // the lane's key / query rows are streamed from LDS in 8-element pieces
      auto kpc = [&](int p) { return to_f32<T>(*reinterpret_cast<const v8_t<T>*>(sK + tt * K + kq * KR + 8 * p)); };
      auto qpc = [&](int p) { return to_f32<T>(*reinterpret_cast<const v8_t<T>*>(sQ + tt * K + kq * KR + 8 * p)); };
      const float rk = sRk[tt], rq = sRq[tt], bt = sB[tt], vv = sV[tt * kBV + vc];
      float ks = 0.f;
      if constexpr (PC) {
#pragma unroll
        for (int p = 0; p < KR / 4; ++p) {
          const f32x4 gm = *reinterpret_cast<const f32x4*>(sG + tt * K + kq * KR + 4 * p);
#pragma unroll
          for (int e = 0; e < 4; ++e) S[4 * p + e] = S[4 * p + e] * gm[e];
        }
#pragma unroll
        for (int p = 0; p < KR / 8; ++p) {
          const f32x8 x = kpc(p);
#pragma unroll
          for (int e = 0; e < 8; ++e) ks = __builtin_fmaf(S[8 * p + e], x[e], ks);
        }
        ks = lanes_sum_t<4>(ks) * rk;
      } else {
        const float gm = sG[tt];
#pragma unroll
        for (int p = 0; p < KR / 8; ++p) {
          const f32x8 x = kpc(p);
#pragma unroll
          for (int e = 0; e < 8; ++e) ks = __builtin_fmaf(S[8 * p + e], x[e], ks);
        }
        ks = lanes_sum_t<4>(ks) * (gm * rk);
#pragma unroll
        for (int i = 0; i < KR; ++i) S[i] = S[i] * gm;
      }
      const float c = rk * (bt * (vv - ks));
      float os = 0.f;
#pragma unroll
      for (int p = 0; p < KR / 8; ++p) {
        const f32x8 x = kpc(p), y = qpc(p);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          S[8 * p + e] = __builtin_fmaf(x[e], c, S[8 * p + e]);
          os = __builtin_fmaf(S[8 * p + e], y[e], os);
        }
      }
      os = lanes_sum_t<4>(os) * (rq * a.scale);
      if (kq == 0) sO[tt * kBV + vc] = os;
      }
    }

    lds_barrier();
    {
      const int row = lane >> 2, c4 = 4 * (lane & 3);
      if (row < len - blk * kTB) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(sO + row * kBV + c4);
        st4(op + ((bos + blk * kTB + row) * HV + j) * V + v0 + c4, x);
      }
    }
  }

  if (a.ht != nullptr) {
    lds_barrier();
#pragma unroll
    for (int i = 0; i < KR; ++i) sS[(kq * KR + i) * kBV + vc] = S[i];
    lds_barrier();
#pragma unroll
    for (int m = 0; m < NSL; ++m) {
      const int idx = lane + 64 * m, r = idx >> 2, c4 = 4 * (idx & 3);
      *reinterpret_cast<f32x4*>(a.ht + hbase + (int64_t)r * V + c4) =
          *reinterpret_cast<const f32x4*>(sS + r * kBV + c4);
    }
  }
}

template <typename T, int K>
hipError_t launch_k(const Args& a, hipStream_t s) {
  const int64_t nblk = a.N * a.HV * (a.V / kBV);
  if (a.per_channel)
    hipLaunchKernelGGL((k5_recurrent<T, K, true>), dim3((unsigned)nblk), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((k5_recurrent<T, K, false>), dim3((unsigned)nblk), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const Args& a, hipStream_t s) {
  switch (a.K) {
    case 32: return launch_k<T, 32>(a, s);
    case 64: return launch_k<T, 64>(a, s);
    case 128: return launch_k<T, 128>(a, s);
    default: return launch_k<T, 256>(a, s);
  }
}

}  // namespace

hipError_t launch_recurrent(const Args& a, hipStream_t s) {
  if (a.N * a.HV * (a.V / kBV) == 0) return hipSuccess;
  return a.dtype == GDR_BF16 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace gdr
