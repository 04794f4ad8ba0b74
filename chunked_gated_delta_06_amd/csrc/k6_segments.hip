// Segment hand-off on one device: the context-parallel scheme of the KCP page
// ("flash-linear-attention KCP precision-failure root-cause manual", sections
// on the pre-process / merge kernels and "h and dh cross-rank semantics") run
// with every segment of one long sequence in the same launch instead of on its
// own rank.
//
// Each segment r is first scanned on its own from a zero state (its local end
// state S_ext[r]) and from the K x K identity with no values (its transition
// M[r], the product of the segment's per-token maps D_t (I - beta_t k_t k_t^T)),
// both with the chunk scan.  The merge below then chains the segments:
//   S_in[0] = h0,   S_in[r + 1] = M[r] S_in[r] + S_ext[r],
// and each segment is re-run from S_in[r].  This file holds the merge and two
// fills the host sequence needs; the scans are the library's own stages.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

constexpr int kMB = 16;    // state columns per merge workgroup
constexpr int kMT = 256;   // merge threads

// S_in for every segment boundary, for one value head and 16 state columns.
// The running state tile sits in LDS; thread t owns row k = t / (256 / K) and
// K / 16 consecutive columns of it, reads its row of M[r] as 16-byte vectors
// and the tile rows as broadcast LDS reads.  Output (k, c) of a step is
// S_ext[r][k][c] + sum_m M[r][k][m] S[m][c] in fp32, summed in order of m.
template <int K>
__global__ __launch_bounds__(kMT) void k6_merge(int64_t R, int64_t HV, int64_t V, const float* __restrict__ M,
                                                const float* __restrict__ Sext, const float* __restrict__ h0,
                                                float* __restrict__ Sin) {
  constexpr int TPR = kMT / K;        // threads per row
  constexpr int CPT = kMB / TPR;      // columns per thread
  __shared__ __attribute__((aligned(16))) float sX[K * kMB];
  const int tid = threadIdx.x, k = tid / TPR, c0 = (tid % TPR) * CPT;
  const int64_t nvt = V / kMB;
  const int64_t j = blockIdx.x / nvt, v0 = (blockIdx.x % nvt) * kMB;

  float x[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t off = (j * K + k) * V + v0 + c0 + c;
    x[c] = h0 != nullptr ? h0[off] : 0.f;
    sX[k * kMB + c0 + c] = x[c];
    Sin[off] = x[c];
  }
  for (int64_t r = 0; r < R; ++r) {
    __syncthreads();
    const float* Mrow = M + ((r * HV + j) * K + k) * (int64_t)K;
#pragma unroll
    for (int c = 0; c < CPT; ++c) x[c] = Sext[((r * HV + j) * K + k) * V + v0 + c0 + c];
    for (int mm = 0; mm < K; mm += 4) {
      const f32x4 m4 = *reinterpret_cast<const f32x4*>(Mrow + mm);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int c = 0; c < CPT; ++c) x[c] = __builtin_fmaf(m4[e], sX[(mm + e) * kMB + c0 + c], x[c]);
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      sX[k * kMB + c0 + c] = x[c];
      Sin[(((r + 1) * HV + j) * K + k) * V + v0 + c0 + c] = x[c];
    }
  }
}

// out[n][j] = I (K x K) for every segment and value head.
__global__ void k6_identity(int64_t total, int64_t K, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t e = i % (K * K);
  out[i] = (e / K == e % K) ? 1.f : 0.f;
}

// n16 16-byte words of zeros.
__global__ void k6_zero16(int64_t n16, f32x4* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) out[i] = zero4();
}

unsigned blocks(int64_t n, int t) { return (unsigned)((n + t - 1) / t); }

}  // namespace

hipError_t launch_identity(int64_t count, int64_t K, float* out, hipStream_t s) {
  const int64_t total = count * K * K;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k6_identity, dim3(blocks(total, 256)), dim3(256), 0, s, total, K, out);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(k6_zero16, dim3(blocks(n16, 256)), dim3(256), 0, s, n16, static_cast<f32x4*>(p));
  return hipGetLastError();
}

hipError_t launch_merge(int64_t R, int64_t HV, int64_t K, int64_t V, const float* M, const float* Sext,
                        const float* h0, float* Sin, hipStream_t s) {
  const dim3 grid((unsigned)(HV * (V / kMB)));
  switch (K) {
    case 32: hipLaunchKernelGGL(k6_merge<32>, grid, dim3(kMT), 0, s, R, HV, V, M, Sext, h0, Sin); break;
    case 64: hipLaunchKernelGGL(k6_merge<64>, grid, dim3(kMT), 0, s, R, HV, V, M, Sext, h0, Sin); break;
    case 128: hipLaunchKernelGGL(k6_merge<128>, grid, dim3(kMT), 0, s, R, HV, V, M, Sext, h0, Sin); break;
    case 256: hipLaunchKernelGGL(k6_merge<256>, grid, dim3(kMT), 0, s, R, HV, V, M, Sext, h0, Sin); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdr
