// Zero padding of head dimensions at the library boundary.
//
// The chunked kernels are instantiated for head dims K, V in {32, 64, 128,
// 256}.  Other sizes (the coverage-matrix page's non-power-of-two D, "FLA
// operator-kernel correctness testing and coverage matrix", section 3) run
// padded: q, k, v (and a per-channel gate, h0, dO, dht) are copied into
// zero-filled tensors of the next supported size, the padded problem runs, and
// o, ht (dq, dk, dv, dh0) are copied back.  Zero key / query features change no
// norm and no dot product, a zero value column stays zero in every state, so
// the padded problem's results restricted to the original dims are exactly the
// unpadded operator's (up to the rounding order of the larger contractions).
//
// Both kernels copy a batch of M matrices, R x C inside Rp x Cp (element
// (m, i, j) at (m Rp + i) Cp + j), as raw 2- or 4-byte words; one thread per
// padded element, consecutive threads on consecutive columns.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

template <typename W>
__global__ void k7_pad(const W* __restrict__ src, W* __restrict__ dst, int64_t total, int64_t R, int64_t C,
                       int64_t Rp, int64_t Cp) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int64_t j = e % Cp, i = (e / Cp) % Rp, m = e / (Cp * Rp);
  dst[e] = (i < R && j < C) ? src[(m * R + i) * C + j] : W(0);
}

template <typename W>
__global__ void k7_unpad(const W* __restrict__ src, W* __restrict__ dst, int64_t total, int64_t R, int64_t C,
                         int64_t Rp, int64_t Cp) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int64_t j = e % C, i = (e / C) % R, m = e / (C * R);
  dst[e] = src[(m * Rp + i) * Cp + j];
}

unsigned nblocks(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_pad(const void* src, void* dst, int64_t M, int64_t R, int64_t C, int64_t Rp, int64_t Cp,
                      int esize, hipStream_t s) {
  const int64_t total = M * Rp * Cp;
  if (total == 0) return hipSuccess;
  if (esize == 2)
    hipLaunchKernelGGL(k7_pad<uint16_t>, dim3(nblocks(total)), dim3(256), 0, s, static_cast<const uint16_t*>(src),
                       static_cast<uint16_t*>(dst), total, R, C, Rp, Cp);
  else
    hipLaunchKernelGGL(k7_pad<uint32_t>, dim3(nblocks(total)), dim3(256), 0, s, static_cast<const uint32_t*>(src),
                       static_cast<uint32_t*>(dst), total, R, C, Rp, Cp);
  return hipGetLastError();
}

hipError_t launch_unpad(const void* src, void* dst, int64_t M, int64_t R, int64_t C, int64_t Rp, int64_t Cp,
                        int esize, hipStream_t s) {
  const int64_t total = M * R * C;
  if (total == 0) return hipSuccess;
  if (esize == 2)
    hipLaunchKernelGGL(k7_unpad<uint16_t>, dim3(nblocks(total)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), total, R, C, Rp, Cp);
  else
    hipLaunchKernelGGL(k7_unpad<uint32_t>, dim3(nblocks(total)), dim3(256), 0, s,
                       static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), total, R, C, Rp, Cp);
  return hipGetLastError();
}

}  // namespace gdr
