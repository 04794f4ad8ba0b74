// K0: chunk table of a dense or varlen batch.
//
// Chunks restart at every sequence start and the last chunk of a sequence may
// be partial, as in the varlen chunk-boundary example of the KCP page
// ("flash-linear-attention KCP precision-failure root-cause manual", section
// "why per-chunk comparison lies under varlen KCP").  Row c of the table is
// (sequence, first token in the flattened token order, length, chunk number
// inside the sequence); chunk_off[n] is the first chunk of sequence n and
// chunk_off[N] the number of chunks.  The table is built on the device so the
// host never waits for cu_seqlens; later stages size their grids to the bound
// NT_max = floor(T / C) + N and read chunk_off[N].
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

__global__ __launch_bounds__(256) void k0_dense(int32_t* __restrict__ idx, int32_t* __restrict__ off,
                                                int64_t B, int64_t T, int32_t C) {
  const int64_t NC = (T + C - 1) / C;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c < B * NC) {
    const int64_t n = c / NC, cl = c % NC;
    const int64_t start = cl * C;
    int4 row;
    row.x = (int32_t)n;
    row.y = (int32_t)(n * T + start);
    row.z = (int32_t)((T - start) < C ? (T - start) : C);
    row.w = (int32_t)cl;
    reinterpret_cast<int4*>(idx)[c] = row;
  }
  if (c <= B) off[c] = (int32_t)(c * NC);
}

// One workgroup of 1024 threads walks the sequences in tiles of 1024 with a
// block-wide exclusive scan of the per-sequence chunk counts.
__global__ __launch_bounds__(1024) void k0_varlen(const int32_t* __restrict__ cu, int32_t* __restrict__ idx,
                                                  int32_t* __restrict__ off, int32_t* __restrict__ order, int64_t N,
                                                  int32_t C) {
  __shared__ int32_t wave_tot[16];
  __shared__ int32_t tile_base;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) tile_base = 0;
  __syncthreads();
  for (int64_t n0 = 0; n0 < N; n0 += 1024) {
    const int64_t n = n0 + tid;
    int32_t s = 0, len = 0, cnt = 0;
    if (n < N) {
      s = cu[n];
      len = cu[n + 1] - s;
      cnt = (len + C - 1) / C;
    }
    // inclusive scan inside the wave
    int32_t x = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wave_tot[wv] = x;
    __syncthreads();
    int32_t before = 0;
    for (int i = 0; i < wv; ++i) before += wave_tot[i];
    const int32_t base = tile_base;
    const int32_t first = base + before + x - cnt;
    if (n < N) {
      off[n] = first;
      for (int32_t cl = 0; cl < cnt; ++cl) {
        int4 row;
        row.x = (int32_t)n;
        row.y = s + cl * C;
        row.z = (len - cl * C) < C ? (len - cl * C) : C;
        row.w = cl;
        reinterpret_cast<int4*>(idx)[first + cl] = row;
      }
    }
    __syncthreads();
    if (tid == 1023) tile_base = first + cnt;
    __syncthreads();
  }
  if (tid == 0) off[N] = tile_base;
  // sequences by decreasing chunk count (ties by index): rank of sequence n
  // = the number of sequences that come before it
  if (order != nullptr && N <= kMaxOrdered) {
    __shared__ int32_t cnts[kMaxOrdered];
    if (tid < N) cnts[tid] = (cu[tid + 1] - cu[tid] + C - 1) / C;
    __syncthreads();
    if (tid < N) {
      const int32_t mine = cnts[tid];
      int32_t rank = 0;
      for (int m = 0; m < (int)N; ++m) {
        const int32_t other = cnts[m];
        rank += (other > mine || (other == mine && m < tid)) ? 1 : 0;
      }
      order[rank] = tid;
    }
  }
}

hipError_t launch_chunk_table(const Args& a, hipStream_t s) {
  if (a.cu == nullptr) {
    const int64_t NC = (a.T + a.C - 1) / a.C;
    const int64_t work = (a.B * NC > a.B + 1) ? a.B * NC : a.B + 1;
    const int64_t blocks = (work + 255) / 256;
    hipLaunchKernelGGL(k0_dense, dim3((unsigned)blocks), dim3(256), 0, s, a.chunk_idx, a.chunk_off, a.B, a.T,
                       a.C);
  } else {
    hipLaunchKernelGGL(k0_varlen, dim3(1), dim3(1024), 0, s, a.cu, a.chunk_idx, a.chunk_off, a.seq_order, a.N,
                       a.C);
  }
  return hipGetLastError();
}

}  // namespace gdr
