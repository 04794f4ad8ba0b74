// Internal host/kernel interface of the gdr library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdr.h"

namespace gdr {

// Per-chunk token factors written by K1 (scalar gate), one row of
// kscale_pitch(C) floats per chunk and value head:
//   [0, C)         exp(G_L - G_t) / |k_t|   (0 past L)
//   [C, C + 4)     exp(G_L), 0, 0, 0
//   [C + 4, 2C + 4)   G_t, the chunk-local gate cumsum   (0 past L)
//   [2C + 4, 3C + 4)  1 / |k_t| (1 without the in-kernel norm; 0 past L)
constexpr int64_t kscale_pitch(int64_t C) { return 3 * C + 4; }

// Everything a stage needs: the problem and plain device pointers (forward
// stages leave the backward fields NULL).
struct Args {
  int64_t B, T, H, HV, K, V, N, NTmax;
  int32_t C, per_channel, l2norm, dtype;
  // dense batch only: the first stage derives every chunk from B, T and C and
  // writes the chunk table itself (no separate table launch)
  int32_t table_from_dims;
  // simple GLA (no delta correction): the fused K1 + K2 stage produces
  // Tm = I, w = 0 and u = v, so the scan and output stages compute
  // S_t = exp(g_t) S_{t-1} + k_t v_t^T
  int32_t gla;
  // beta holds logits: the kernels use sigmoid(beta) (see beta_value)
  int32_t beta_logits;
  // u is fp32 (written by the separate WY stage) rather than the input dtype
  // (written by the fused K1 + K2 stage); the state scans read it accordingly
  int32_t u_f32;
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
  // varlen batches of at most kMaxOrdered sequences: the sequences by
  // decreasing chunk count, written by the chunk-table stage and read by the
  // state scans' workgroup mapping (NULL: natural order)
  int32_t* seq_order;
  void* Tm;
  void* w;
  void* u;
  void* h;
  void* v_new;
  float* kscale;
  void* o;
  float* ht;
  // backward
  const void* d_o;
  const float* dht;
  void* de_local;
  float* qscale;
  void* dh;
  float* dh0;
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  // backward with a per-channel gate: the chunk's gated operand rows for the
  // reverse scan and B3, kt = exp(G_L - G_t) k^_t and qg = scale exp(G_t) q^_t
  // ([NT][HV][C][K], input dtype), and the decay dl = exp(G_L) ([NT][HV][K])
  void* kt;
  void* qg;
  float* dl;
  // forward with a per-channel gate and the fused scan + output: the chunk's
  // intra attention aqk[r][t] = scale sum_d q^_rd k^_td exp(G_rd - G_td) for
  // t <= r (fp32 [NT][HV][C][C], zero above the diagonal and past L) and its
  // gated queries scale exp(G_t) q^_t (qgs [NT][HV][kQgsTiles][C][K]: one
  // tile in the input dtype, or a hi tile and a lo tile), both written by the
  // fused per-channel K1 + K2
  float* aqk;
  void* qgs;
};

// Tiles of the gated queries of the per-channel fused forward: 1 (rounded once
// to the input dtype; the output's inter term then carries the same rounding
// as its bf16 state h) or 2 (a bf16 hi + lo pair).
constexpr int kQgsTiles = 1;

int64_t nt_max(const gdr_problem& p);
constexpr int64_t kMaxOrdered = 1024;

hipError_t launch_chunk_table(const Args& a, hipStream_t s);
hipError_t launch_kkt_solve(const Args& a, hipStream_t s);
hipError_t launch_wy(const Args& a, hipStream_t s);
// K1 + K2 fused (scalar gate): w, u and kscale, no Tm; with a.u_f32 set (kept
// states) also Tm, and u in fp32 as the separate WY stage writes it
hipError_t launch_kkt_wy(const Args& a, hipStream_t s);
// K1 + K2 fused, per-channel gate (bf16, chunk 32, K <= 128): w, u (fp32),
// kt, dl, Tm when a.Tm is set, aqk and qgs when both are set
bool kkt_wy_pc_supported(const Args& a);
hipError_t launch_kkt_wy_pc(const Args& a, hipStream_t s);
hipError_t launch_fwd_h(const Args& a, hipStream_t s);
// whether launch_fwd_h takes h = v_new = NULL (then writes neither) and, with
// them, u = NULL for u = 0: the scalar-gate warp-specialised scan
bool fwd_h_states_optional(const Args& a);
// fused state scan + output (no h / v_new); fwd_h_o_supported says whether the
// shape has an instantiation (scalar gate, staged tiles fit in LDS)
bool fwd_h_o_supported(const Args& a);
bool fwd_h_o_preferred(const Args& a);   // the full forward's choice
hipError_t launch_fwd_h_o(const Args& a, hipStream_t s);
// the fused scan + output of a kept-states forward (scalar gate): u in fp32 from
// the kept-states fused K1 + K2, h and v_new written as the separate scan does
bool fwd_h_o_keep_supported(const Args& a);
hipError_t launch_fwd_h_o_keep(const Args& a, hipStream_t s);
hipError_t launch_fwd_o(const Args& a, hipStream_t s);
// per-channel gate: the fused scan + output on the gated keys / decay and the
// aqk / qgs tiles (bf16, chunk 32, K <= 128), also storing h and v_new when
// both are set; *_preferred is the full forward's choice
bool fwd_h_o_pc_supported(const Args& a);
bool fwd_h_o_pc_preferred(const Args& a);
hipError_t launch_fwd_h_o_pc(const Args& a, hipStream_t s);
// token-by-token forward (no chunk table, no workspace)
hipError_t launch_recurrent(const Args& a, hipStream_t s);
hipError_t launch_bwd_intra(const Args& a, hipStream_t s);
// segment hand-off: fills and the merge S_in[r + 1] = M[r] S_in[r] + S_ext[r]
hipError_t launch_identity(int64_t count, int64_t K, float* out, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
// zero padding of head dims: M matrices R x C inside Rp x Cp, 2- or 4-byte words
hipError_t launch_pad(const void* src, void* dst, int64_t M, int64_t R, int64_t C, int64_t Rp, int64_t Cp,
                      int esize, hipStream_t s);
hipError_t launch_unpad(const void* src, void* dst, int64_t M, int64_t R, int64_t C, int64_t Rp, int64_t Cp,
                        int esize, hipStream_t s);
hipError_t launch_merge(int64_t R, int64_t HV, int64_t K, int64_t V, const float* M, const float* Sext,
                        const float* h0, float* Sin, hipStream_t s);
hipError_t launch_bwd_dh(const Args& a, hipStream_t s);
hipError_t launch_bwd_dqkvg(const Args& a, hipStream_t s);
// per-channel gate (chunk 32): every gradient but dh / dh0 (reads kt from the
// intra-chunk stage)
hipError_t launch_bwd_dqkvg_pc(const Args& a, hipStream_t s);

// Shapes the backward kernels take (LDS limits of the fused kernel and of the
// reverse scan; a per-channel gate at chunk 32).
bool bwd_shape_ok(const gdr_problem& p);
bool bwd_scan_fits(int dtype, int C, int K);
// per-channel gate: the warp-specialised scan on the WY stage's gated keys fits
bool fwd_pc_scan_fits(int dtype, int C, int K);
bool bwd_scan_pc_fits(int dtype, int K);   // per-channel reverse scan at chunk 32
bool bwd_fused_fits(int dtype, int C, int K);
bool bwd_pc_fits(int dtype, int K);        // per-channel B3 at chunk 32

}  // namespace gdr
