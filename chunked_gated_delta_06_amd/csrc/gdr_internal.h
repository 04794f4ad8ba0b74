// Internal host/kernel interface of the gdr library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdr.h"

namespace gdr {

// Everything a forward stage needs: the problem and plain device pointers.
struct FwdArgs {
  int64_t B, T, H, HV, K, V, N, NTmax;
  int32_t C, per_channel, l2norm, dtype;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* cu;
  const float* h0;
  int32_t* chunk_idx;
  int32_t* chunk_off;
  void* Tm;
  void* w;
  void* u;
  void* h;
  void* v_new;
  float* kscale;
  void* o;
  float* ht;
};

int64_t nt_max(const gdr_problem& p);

hipError_t launch_chunk_table(const FwdArgs& a, hipStream_t s);
hipError_t launch_kkt_solve(const FwdArgs& a, hipStream_t s);
hipError_t launch_wy(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_h(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_o(const FwdArgs& a, hipStream_t s);

}  // namespace gdr
