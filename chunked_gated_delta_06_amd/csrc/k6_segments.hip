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
// The running state sits in LDS; output (k, c) of a step is
// S_ext[r][k][c] + sum_m M[r][k][m] S[m][c] in fp32, summed in order of m.
template <int K>
__global__ __launch_bounds__(kMT) void k6_merge(int64_t R, int64_t HV, int64_t V, const float* __restrict__ M,
                                                const float* __restrict__ Sext, const float* __restrict__ h0,
                                                float* __restrict__ Sin) {
  constexpr int PER = K * kMB / kMT;   // outputs per thread
  __shared__ float sX[K * kMB];
  const int tid = threadIdx.x;
  const int64_t nvt = V / kMB;
  const int64_t j = blockIdx.x / nvt, v0 = (blockIdx.x % nvt) * kMB;

#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = tid + kMT * m, k = idx / kMB, c = idx % kMB;
    const int64_t off = (j * K + k) * V + v0 + c;
    const float x = h0 != nullptr ? h0[off] : 0.f;
    sX[idx] = x;
    Sin[off] = x;
  }
  for (int64_t r = 0; r < R; ++r) {
    __syncthreads();
    float acc[PER];
    const float* Mr = M + (r * HV + j) * K * K;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = tid + kMT * m, k = idx / kMB, c = idx % kMB;
      float s = Sext[((r * HV + j) * K + k) * V + v0 + c];
      for (int mm = 0; mm < K; ++mm) s = __builtin_fmaf(Mr[(int64_t)k * K + mm], sX[mm * kMB + c], s);
      acc[m] = s;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = tid + kMT * m, k = idx / kMB, c = idx % kMB;
      sX[idx] = acc[m];
      Sin[(((r + 1) * HV + j) * K + k) * V + v0 + c] = acc[m];
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
