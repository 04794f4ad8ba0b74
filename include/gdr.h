/*
 * gdr.h -- C ABI of the chunked gated delta-rule operator on AMD MI355X (gfx950).
 *
 * The operator (pages: "FLA operator-kernel correctness testing and coverage
 * matrix", section 2 and section 3; "flash-linear-attention KCP precision-failure
 * root-cause manual", section "h and dh cross-rank semantics"):
 *
 *   for every sequence n, value head j (q/k head h = j / (HV / H)), token t:
 *     S' = D_t S            D_t = diag(exp(g[t, j]))  (scalar or per-channel gate)
 *     e  = beta[t, j] * (v[t, j] - S'^T k^[t, h])
 *     S  = S' + k^[t, h] e^T                                  (S is K x V)
 *     o[t, j] = scale * S^T q^[t, h]
 *   starting from h0[n, j] (or zeros) and ending in ht[n, j], where q^, k^ are
 *   q, k divided by sqrt(sum(x^2) + 1e-6) when use_qk_l2norm is set.  It is
 *   evaluated chunk by chunk (chunk_size 32 or 64) through the WY form
 *   S^r = P^r S^0 + H^r of the coverage-matrix page (section 2).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are device memory owned by the caller; the library
 *     never allocates, frees or synchronises.  Every call is asynchronous on
 *     `stream` (a hipStream_t; NULL = the null stream).
 *   - Tensors are dense and row-major with the shapes given below; every
 *     pointer must be 16-byte aligned.
 *   - "dtype" tensors (q, k, v, o and the intermediates) are bf16 when
 *     problem->dtype == GDR_BF16 and float32 when GDR_FP32; g, beta, h0, ht
 *     are always float32.
 *   - Arguments are checked on the host before any launch; a failed check
 *     returns an error code and writes nothing.  A launch failure returns
 *     GDR_ERR_HIP.  Device faults surface at the caller's next synchronisation.
 *   - cu_seqlens contents (cu[0] = 0, non-decreasing, cu[N] = T) are a
 *     precondition; gdr_validate_cu_seqlens checks a host copy.
 *   - Every output element is written (outputs may hold garbage on entry).
 *   - Calls that share a workspace or an output must not overlap in time.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDR_OK = 0,
  GDR_ERR_NULL_ARG = 1,    /* a required pointer is NULL */
  GDR_ERR_CHUNK_SIZE = 2,  /* "chunk_size must be either 32 or 64" */
  GDR_ERR_SHAPE = 3,       /* a dim < 1 (T < 0), HV % H != 0, K or V above 256 (or, for a single
                              stage, the token-by-token, segmented and simple GLA paths, not in
                              {32,64,128,256}), B*T >= 2^31, or fp32 + per-channel gate + K > 128
                              + chunk 64 */
  GDR_ERR_VARLEN = 4,      /* cu_seqlens with B != 1, N < 1, or N != B for a dense batch */
  GDR_ERR_DTYPE = 5,       /* dtype not GDR_BF16 / GDR_FP32 */
  GDR_ERR_ALIGNMENT = 6,   /* a pointer not 16-byte aligned */
  GDR_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than *_workspace_bytes */
  GDR_ERR_HIP = 8,         /* a kernel launch failed */
  GDR_ERR_CU_SEQLENS = 9,  /* gdr_validate_cu_seqlens: bad table */
  GDR_ERR_UNSUPPORTED = 10, /* backward: K above 128, or a saved-state backward that
                              would have to switch to chunk 32 (per-channel gate, or fp32
                              with K = 128, at chunk 64; see gdr_chunk_bwd); the backward
                              stage entry points: a per-channel gate; gdr_fwd_h_o: a shape
                              without the fused stage
                              (see gdr_fwd_h_o_supported); gdr_simple_gla_fwd: a per-channel
                              gate */
  GDR_ERR_SCRATCH_LIMIT = 11 /* gdr_chunk_fwd_noalloc: the problem needs more than
                                GDR_NOALLOC_SCRATCH_BYTES of scratch */
} gdr_status;

typedef enum { GDR_BF16 = 0, GDR_FP32 = 1 } gdr_dtype;

/* Problem description.  Dense batch: cu_seqlens = NULL, N = B, every row is one
 * sequence of T tokens.  Varlen batch: B = 1, T = total tokens, N = number of
 * sequences, sequence n spans tokens [cu_seqlens[n], cu_seqlens[n+1]). */
typedef struct {
  int64_t B, T, H, HV, K, V, N;
  int32_t chunk_size;        /* 32 | 64 */
  int32_t gate_per_channel;  /* 0: g is [B,T,HV]; 1: g is [B,T,HV,K] */
  int32_t use_qk_l2norm;     /* 1: normalise q, k rows in the kernels */
  int32_t dtype;             /* gdr_dtype */
  float scale;               /* output scale */
  int32_t keep_states;       /* gdr_chunk_fwd: 1 = leave Tm, h, v_new and an fp32 u in the
                                workspace (fused stages that also store them where the
                                shape has them, else the separate K1..K4 stages); 0 = use
                                the fused stages where gdr_chunk_fwd_fused reports them
                                (Tm, h and v_new are then not written).
                                gdr_chunk_bwd: 1 = take those intermediates
                                from its workspace instead of recomputing them (see
                                gdr_chunk_bwd) */
  int32_t beta_logits;       /* 1: beta holds logits and every kernel uses sigmoid(beta) (the
                                beta-mode axis of the coverage-matrix page, section 3); the
                                backward's dbeta is then the gradient with respect to the
                                logits.  0: beta is used as given */
} gdr_problem;

/* Offsets (bytes from the workspace base) of the forward intermediates that
 * gdr_chunk_fwd keeps in its workspace; NT_max = B * ceil(T / C) for a dense
 * batch and floor(T / C) + N for a varlen batch.  When the forward takes the
 * fused stages (keep_states = 0 and gdr_chunk_fwd_fused(p) != 0), the layout is
 * the compact one those stages use: Tm, h and v_new get no bytes (their
 * offsets equal the next region's) and u is in `dtype`; with a per-channel
 * gate (kind 2) the kt, dl, aqk and qgs regions below get bytes.  The
 * kept-states layout of a per-channel chunk-32 bf16 problem with K <= 128
 * keeps aqk and qgs too (its forward runs the same fused stages).  Regions a
 * layout does not use have no bytes.
 *   chunk_idx  int32 [NT_max][4]   (sequence, first token (flattened), length, chunk-in-sequence)
 *   chunk_off  int32 [N + 1]       first chunk of each sequence; chunk_off[N] = NT
 *   seq_order  int32 [N]           varlen batches of at most 1024 sequences: the sequences
 *                                  by decreasing chunk count (ties by index), the order in
 *                                  which the state scans start them; unused otherwise
 *   Tm         dtype [NT_max][HV][C][C]   (I + A)^-1 of each chunk, row-major
 *   w          dtype [NT_max][HV][C][K]   WY keys, token-major
 *   u          f32   [NT_max][HV][V][C]   WY values, transposed per chunk, as gdr_fwd_wy
 *                                         writes them (fp32 for every dtype); in the
 *                                         fused forwards' layouts (kinds 1 and 2) in `dtype`
 *   h          dtype [NT_max][HV][V][K]   state entering each chunk, transposed (h^T)
 *   v_new      dtype [NT_max][HV][V][C]   corrected values e, transposed per chunk
 *   kscale     f32   [NT_max][HV][3C + 4] scalar gate only, per chunk token factors:
 *                                         exp(G_L - G_t) / |k_t| per row t, then exp(G_L)
 *                                         and 3 zeros, then G_t (chunk-local gate cumsum),
 *                                         then 1 / |k_t| (1 without the in-kernel norm);
 *                                         0 past L
 *   kt         dtype [NT_max][HV][C][K]   per-channel gate, written by the full forward's
 *                                         WY stage for its state scan: exp(G_L - G_t) k^_t
 *                                         per row t (zero past L); no bytes otherwise
 *   dl         f32   [NT_max][HV][K]      per-channel gate: exp(G_L) per feature
 *   aqk        f32   [NT_max][HV][C][C]   per-channel fused forward only (fused K1 + K2):
 *                                         the chunk's intra attention, row r, column t:
 *                                         scale sum_d q^_rd k^_td exp(G_rd - G_td) for
 *                                         t <= r (the Q K^T o M term of the chunk form's
 *                                         output, coverage-matrix page, section 2), zero
 *                                         above the diagonal and in rows past L
 *   qgs        dtype [NT_max][HV][C][K] per-channel fused forward only (fused K1 + K2):
 *                                         the gated queries scale exp(G_t) q^_t, the
 *                                         output's inter-term operand
 * Rows past the end of a partial chunk hold zeros. */
typedef struct {
  int64_t nt_max;
  size_t chunk_idx, chunk_off, seq_order, Tm, w, u, h, v_new, kscale, kt, dl, aqk, qgs, total;
} gdr_fwd_layout;

/* ABI version of this header (bumped on incompatible changes). */
int gdr_abi_version(void);

/* Stage timing, for measurement: gdr_stage_timing(1) turns it on (and clears
 * what was recorded), 0 turns it off.  While on, every gdr_chunk_fwd,
 * gdr_chunk_fwd_noalloc and gdr_chunk_bwd call on this host thread records a
 * HIP event on its stream before its first launch and after each stage (events
 * created on first use and kept; at most 8192 per recording).  gdr_stage_times
 * waits for the last recorded event and writes, in launch order, up to
 * max_stages (stage name, milliseconds) pairs of every call since timing was
 * turned on: names are static strings ("chunk_table", "kkt_solve", "wy",
 * "kkt_wy", "fwd_h", "fwd_o", "fwd_h_o", "bwd_intra", "bwd_dh", "bwd_dqkvg",
 * "pad", "unpad").  It returns the count (0 when off or nothing was recorded,
 * -1 on a HIP error).  Calls timed back to back keep the stream busy, so each
 * interval is the stage's own time on the GPU. */
gdr_status gdr_stage_timing(int enable);
int gdr_stage_times(const char** names, float* ms, int max_stages);

/* Human-readable name of a status code (static string). */
const char* gdr_status_string(gdr_status s);

/* Host-side check of a problem description (no device access). */
gdr_status gdr_check_problem(const gdr_problem* p);

/* Check a host copy of cu_seqlens ([N+1] int32): cu[0] = 0, non-decreasing,
 * cu[N] = T.  Returns GDR_OK or GDR_ERR_CU_SEQLENS (GDR_ERR_NULL_ARG if NULL).
 * The varlen offsets are the coverage-matrix page's cu_seqlens axis (section
 * 3); the KCP manual's chunk-boundary section ("why per-chunk comparison lies
 * under varlen KCP") is why a bad table must be refused before any chunk is
 * formed.  The kernels trust cu_seqlens, so a caller that cannot vouch for it
 * checks a host copy here (the Python binding does by default). */
gdr_status gdr_validate_cu_seqlens(const int32_t* cu_host, int64_t N, int64_t T);

/* Workspace needed by gdr_chunk_fwd (bytes), and where each intermediate sits.
 * Library plumbing, not an operation of the pages: it holds the intermediates
 * of the chunk form's stages (the coverage-matrix page, section 2; the KCP
 * manual's debug-script stage order) between launches, since the library never
 * allocates.  The size is written through `bytes` so that an invalid problem
 * returns its status instead of a size. */
gdr_status gdr_fwd_workspace_bytes(const gdr_problem* p, size_t* bytes);
gdr_status gdr_fwd_workspace_layout(const gdr_problem* p, gdr_fwd_layout* layout);

/* Head dims: the stages are instantiated for K, V in {32, 64, 128, 256}.
 * gdr_chunk_fwd and gdr_chunk_bwd also take any K, V in 1..256 (the coverage-
 * matrix page's non-power-of-two D, section 3): they copy q, k, v (a
 * per-channel g, h0, d_o, dht) into zero-padded tensors of the next
 * instantiated size inside the workspace, run the padded problem and copy o, ht
 * (dq, dk, dv, dh0) back.  Zero features add only exact zeros to every norm and
 * contraction.  The workspace sizes include the padded copies, and the
 * intermediates of gdr_fwd_layout / gdr_bwd_layout then have the padded dims. */

/* Full forward: K0 chunk table -> K1 kkt + triangular inverse -> K2 WY w/u ->
 * K3 state scan -> K4 output, all on `stream`.  With p->keep_states == 0:
 *  - scalar gate, a shape that gdr_fwd_h_o_supported accepts: K1 and K2 run as
 *    the one fused stage gdr_fwd_kkt_wy and K3 and K4 as the one fused stage
 *    gdr_fwd_h_o, and the Tm, h and v_new regions are left untouched;
 *    gdr_chunk_fwd_fused(p) returns 1 exactly then;
 *  - per-channel gate, bf16, chunk 32, K <= 128: K1 and K2 run as one fused
 *    stage that also writes kt, dl, aqk and qgs (layout above), and K3 and K4
 *    as one fused scan + output stage that reads them, so Tm, h and v_new are
 *    not written; gdr_chunk_fwd_fused(p) returns 2 exactly then (0 otherwise).
 * With keep_states == 1 the same fused stages run where the shape has them,
 * writing Tm, an fp32 u, h and v_new as well (the scalar gate's kept-states
 * fused K1 + K2; the scan + output storing its staged h and e), else the
 * separate stages.
 *   q, k  dtype [B,T,H,K]      v  dtype [B,T,HV,V]
 *   g     f32 [B,T,HV] (or [B,T,HV,K] when gate_per_channel)   beta f32 [B,T,HV]
 *   cu_seqlens  int32 [N+1] device, or NULL for a dense batch
 *   h0    f32 [N,HV,K,V] or NULL (zeros)
 *   o     dtype [B,T,HV,V] (output)
 *   ht    f32 [N,HV,K,V] (output) or NULL (final state not wanted)
 *   workspace  >= gdr_fwd_workspace_bytes bytes of device memory (contents on
 *              entry are irrelevant; on return they hold the intermediates
 *              listed in gdr_fwd_layout). */
gdr_status gdr_chunk_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const int32_t* cu_seqlens,
                         const float* h0, void* o, float* ht, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Full forward that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same operator, arguments (minus the
 * workspace), kernels and results as gdr_chunk_fwd; the intermediates live in
 * a fixed scratch array of GDR_NOALLOC_SCRATCH_BYTES per device, part of the
 * library's code object (allocated when the library is loaded on a device and
 * held until the process ends).  With the scalar-gate fused stages
 * (gdr_chunk_fwd_fused(p) == 1) the scratch holds the chunk tables, w, u and kscale (about 524 bytes per
 * token and value head for bf16 with K = V = 128 at chunk 64), so such a
 * problem fits up to about 500 k (token, value head) pairs (4 x 4096 tokens x
 * 16 heads take half); a larger problem returns GDR_ERR_SCRATCH_LIMIT before
 * any launch.  Nothing in the scratch has to start at zero.  Every call on a
 * device shares that device's scratch: calls that overlap in time on one
 * device (other streams, other host threads) race and must be serialised by
 * the caller.  `stream` must belong to the current device.  The only HIP call
 * besides the launches is one hipGetSymbolAddress on the first call on each
 * device. */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
gdr_status gdr_chunk_fwd_noalloc(const gdr_problem* p, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const int32_t* cu_seqlens,
                                 const float* h0, void* o, float* ht, void* stream);

/* ---- the forward's stages, callable one by one (same layouts as above) ---- */

/* K0: chunk table.  Chunks restart at every sequence start and the last chunk of
 * a sequence may be partial (KCP page, section "why per-chunk comparison lies
 * under varlen KCP").  Writes chunk_idx [NT_max][4] and chunk_off [N+1]; table
 * rows past NT are left untouched. */
gdr_status gdr_chunk_table(const gdr_problem* p, const int32_t* cu_seqlens, int32_t* chunk_idx,
                           int32_t* chunk_off, void* stream);

/* K1: per chunk and value head, G = chunk-local cumsum of g,
 * A[r][j] = beta_r * sum_d k^_rd k^_jd exp(G_rd - G_jd) for j < r, and
 * Tm = (I + A)^-1 (unit lower triangular; upper triangle and rows >= L are 0).
 * With a scalar gate it also writes kscale (layout above; required then,
 * ignored and may be NULL for a per-channel gate). */
gdr_status gdr_fwd_kkt_solve(const gdr_problem* p, const void* k, const float* g,
                             const float* beta, const int32_t* chunk_idx,
                             const int32_t* chunk_off, void* Tm, float* kscale, void* stream);

/* K2: WY recompute, w = Tm (beta exp(G) k^), u = Tm (beta v) per chunk and value head
 * (coverage-matrix page, section 2: P^r = I - sum k^i w^i^T).  w is written in
 * `dtype`, u in fp32 (layout above): the scan's e = u - w S is small next to u,
 * and a bf16 u would carry its rounding into e, h and every gradient. */
gdr_status gdr_fwd_wy(const gdr_problem* p, const void* k, const void* v, const float* g,
                      const float* beta, const int32_t* chunk_idx, const int32_t* chunk_off,
                      const void* Tm, void* w, void* u, void* stream);

/* K1 + K2 fused (scalar gate): the results of gdr_fwd_kkt_solve and gdr_fwd_wy
 * (w, u and kscale, same layouts, but u in `dtype`: it feeds gdr_fwd_h_o) in one
 * pass per chunk and value head, with
 * (I + A)^-1 kept on chip and not written.  gdr_chunk_fwd runs it in place of
 * the two stages whenever it runs the fused scan + output stage.  Returns
 * GDR_ERR_UNSUPPORTED for a per-channel gate. */
gdr_status gdr_fwd_kkt_wy(const gdr_problem* p, const void* k, const void* v, const float* g,
                          const float* beta, const int32_t* chunk_idx, const int32_t* chunk_off,
                          void* w, void* u, float* kscale, void* stream);

/* K3: state scan.  For each sequence, value head and chunk in order: h = S (the
 * state entering the chunk, as on the KCP page, section "h and dh cross-rank
 * semantics"), e = u - w S -> v_new, then
 * S <- diag(exp(G_L)) S + sum_j (exp(G_L - G_j) k^_j) e_j^T.  S starts at h0 (or 0)
 * and is written to ht after the last chunk (if ht != NULL).  A scalar gate is
 * read through K1's kscale (g may then be NULL); a per-channel gate through g.
 * u is fp32, as gdr_fwd_wy writes it. */
gdr_status gdr_fwd_h(const gdr_problem* p, const void* k, const void* w, const void* u,
                     const float* g, const float* kscale, const int32_t* chunk_idx,
                     const int32_t* chunk_off, const float* h0, void* h, void* v_new, float* ht,
                     void* stream);

/* K4: output, o_r = scale * [ (exp(G_r) q^_r)^T h + sum_{j<=r} (q^_r . exp(G_r - G_j) k^_j) e_j ]. */
gdr_status gdr_fwd_o(const gdr_problem* p, const void* q, const void* k, const void* v_new,
                     const void* h, const float* g, const int32_t* chunk_idx,
                     const int32_t* chunk_off, void* o, void* stream);

/* K3 + K4 fused (scalar gate): the state scan of gdr_fwd_h and the output of
 * gdr_fwd_o in one pass, o computed from each chunk's h and e while they are
 * on chip, so neither is written (same operator as the two stages: the chunk
 * form of the coverage-matrix page, section 2, with h as on the KCP page,
 * section "h and dh cross-rank semantics").  g (scalar gate [B,T,HV]) and
 * K1's kscale are both required; h0 / ht as gdr_fwd_h; u in `dtype`, as
 * gdr_fwd_kkt_wy writes it.  Returns
 * GDR_ERR_UNSUPPORTED for a per-channel gate or a shape without an
 * instantiation; gdr_fwd_h_o_supported tells in advance (1 = supported). */
int gdr_fwd_h_o_supported(const gdr_problem* p);
int gdr_chunk_fwd_fused(const gdr_problem* p);
gdr_status gdr_fwd_h_o(const gdr_problem* p, const void* q, const void* k, const void* w,
                       const void* u, const float* g, const float* kscale,
                       const int32_t* chunk_idx, const int32_t* chunk_off, const float* h0,
                       void* o, float* ht, void* stream);

/* Token-by-token ("fused recurrent") forward of the same operator: the
 * recurrence at the top of this header applied one token at a time with the
 * state in registers, the per-token form that the chunk form of the
 * coverage-matrix page (section 2) reorganises; that page's coverage matrix
 * (section 3) tests such a fused_recurrent entry point beside the chunked one.
 * It needs no chunk table and no workspace, which suits decoding (T of one or a
 * few tokens per sequence, the state handed over through h0 / ht) and short
 * sequences.  Same problem description, layouts and pointer rules as
 * gdr_chunk_fwd; chunk_size and keep_states are not read, and the chunked
 * path's int32 token limit (B*T < 2^31) does not apply.
 *   q, k  dtype [B,T,H,K]      v  dtype [B,T,HV,V]
 *   g     f32 [B,T,HV] (or [B,T,HV,K] when gate_per_channel)   beta f32 [B,T,HV]
 *   cu_seqlens  int32 [N+1] device, or NULL for a dense batch
 *   h0    f32 [N,HV,K,V] or NULL (zeros)
 *   o     dtype [B,T,HV,V] (output)
 *   ht    f32 [N,HV,K,V] (output) or NULL
 * State and arithmetic are fp32; o is rounded to the input dtype.  Errors as
 * gdr_chunk_fwd (never GDR_ERR_CHUNK_SIZE or GDR_ERR_WORKSPACE). */
gdr_status gdr_fused_recurrent_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                                   const float* g, const float* beta, const int32_t* cu_seqlens,
                                   const float* h0, void* o, float* ht, void* stream);

/* Simple GLA forward: the same chunked pipeline without the delta correction,
 *   S_t = exp(g_t) S_{t-1} + k^_t v_t^T,   o_t = scale * S_t^T q^_t,
 * the variant the coverage-matrix page lists beside the delta rule (section 2,
 * simple-gla) that shares the state-scan and output stages (chunk_fwd_h,
 * chunk_fwd_o in fla/ops/common on the contributor guide's layout page).  The
 * fused K1 + K2 stage produces Tm = I, w = 0 and u = v, then the fused scan +
 * output stage (or K3 and K4 where it has no instantiation) runs unchanged.
 * Scalar gate only (GDR_ERR_UNSUPPORTED for a per-channel gate); no beta.
 * Arguments, layouts and the workspace (gdr_fwd_workspace_bytes) as
 * gdr_chunk_fwd; keep_states is not read. */
gdr_status gdr_simple_gla_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                              const float* g, const int32_t* cu_seqlens, const float* h0, void* o,
                              float* ht, void* workspace, size_t workspace_bytes, void* stream);

/* Segment hand-off on one device: the context-parallel forward of the KCP
 * page ("flash-linear-attention KCP precision-failure root-cause manual",
 * sections on the pre-process and merge kernels and "h and dh cross-rank
 * semantics") with every segment in the same launches instead of on its own
 * rank.  The problem is a varlen batch (B = 1) whose N sequences are the
 * consecutive segments of ONE sequence of T tokens, cu_seqlens (required) their
 * bounds.  Per segment r, with the chunk scan of gdr_fwd_h:
 *   S_ext[r]  = the segment's end state from a zero state,
 *   M[r]      = its transition, the product of the per-token maps
 *               D_t (I - beta_t k^_t k^_t^T) over its tokens (the same scan
 *               started from the K x K identity with no values),
 * then the merge S_in[0] = h0, S_in[r + 1] = M[r] S_in[r] + S_ext[r] (fp32, in
 * segment order), and a re-run of every segment from S_in[r] that writes o.
 * The result is that of gdr_chunk_fwd on the whole sequence (B = 1, dense) up
 * to rounding.
 *   q, k, v, g, beta   as gdr_chunk_fwd with B = 1
 *   h0          f32 [1,HV,K,V] or NULL (zeros): the sequence's initial state
 *   o           dtype [1,T,HV,V] (output)
 *   ht          f32 [1,HV,K,V] or NULL: the final state (the last segment's re-run)
 *   seg_states  f32 [N+1,HV,K,V] or NULL: S_in, the state entering each segment,
 *               and S_in[N] = the merged final state
 *   transitions f32 [N,HV,K,K] or NULL: M
 *   workspace   >= gdr_segmented_workspace_bytes bytes; gdr_segmented_workspace_layout
 *               gives the offsets (the forward intermediates of the segment batch
 *               first, as gdr_fwd_layout, then the scratch of the transition scan).
 * Errors as gdr_chunk_fwd; cu_seqlens NULL returns GDR_ERR_NULL_ARG. */
typedef struct {
  gdr_fwd_layout fwd;
  size_t u_zero, h_tr, v_tr, eye, s_ext, trans, s_in, total;
} gdr_seg_layout;

gdr_status gdr_segmented_workspace_bytes(const gdr_problem* p, size_t* bytes);
gdr_status gdr_segmented_workspace_layout(const gdr_problem* p, gdr_seg_layout* layout);
gdr_status gdr_chunk_fwd_segmented(const gdr_problem* p, const void* q, const void* k, const void* v,
                                   const float* g, const float* beta, const int32_t* cu_seqlens,
                                   const float* h0, void* o, float* ht, float* seg_states,
                                   float* transitions, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* ------------------------------------------------------------------ backward
 *
 * Gradients of L = sum(o * d_o) + sum(ht * dht) with respect to q, k, v, g,
 * beta and h0, for the same operator as gdr_chunk_fwd (scalar or per-channel gate).  dq, dk
 * are gradients with respect to q, k as passed (through the in-kernel L2 norm
 * when use_qk_l2norm is set), summed over the value heads of each GVA group;
 * dg is the gradient with respect to the per-token log gate g (not its cumsum), per
 * channel ([B,T,HV,K]) for a per-channel gate.
 *
 * Backward workspace: the forward intermediates at the offsets of `fwd`
 * (recomputed by the backward, so a forward workspace is not needed), plus
 *   de_local  dtype [NT_max][HV][V][C]  scale * P^T dO per chunk, transposed, with
 *                                       P[r][t] = q^_r . k^_t exp(G_r - G_t), t <= r
 *   qscale    f32   [NT_max][HV][C]     scale * exp(G_r) / |q_r| (0 past L)
 *   kt, qg    dtype [NT_max][HV][C][K]  per-channel gate only: exp(G_L - G_t) k^_t and
 *                                       scale exp(G_t) q^_t per chunk (zero past L)
 *   dl        f32   [NT_max][HV][K]     per-channel gate only: exp(G_L) per chunk
 *   dh        f32   [NT_max][HV][V][K]  gradient of the state leaving each chunk,
 *                                       transposed (dh^T) */
typedef struct {
  gdr_fwd_layout fwd;
  int64_t chunk_size;   /* the chunk size the backward runs at (32 where it switches, see
                           gdr_chunk_bwd); the per-chunk layouts above use it */
  size_t de_local, qscale, dh, kt, qg, dl, total;
} gdr_bwd_layout;

/* Workspace needed by gdr_chunk_bwd (bytes), and where each intermediate sits;
 * plumbing like gdr_fwd_workspace_bytes.  Its leading part is the keep-states
 * forward's layout, so a saved-state backward can read what that forward left. */
gdr_status gdr_bwd_workspace_bytes(const gdr_problem* p, size_t* bytes);
gdr_status gdr_bwd_workspace_layout(const gdr_problem* p, gdr_bwd_layout* layout);

/* Full backward: recompute K0-K3 (chunk table, T and kscale, w / u, h and
 * v_new), then B1 de_local -> B2 reverse state-gradient scan -> B3 fused
 * gradients, all on `stream`.  The pages' backward likewise recomputes the
 * forward state scan before its own stages ("flash-linear-attention KCP
 * precision-failure root-cause manual", sections "pitfall 2" and "debug script
 * layout"); the state gradient follows the hand-off of section "h and dh
 * cross-rank semantics" (dht in, dh0 out).
 *   q, k, v, g, beta, cu_seqlens, h0   as gdr_chunk_fwd (h0 may be NULL = zeros)
 *   d_o   dtype [B,T,HV,V]            gradient of o
 *   dht   f32 [N,HV,K,V] or NULL       gradient of ht (NULL = zeros)
 *   dq, dk  dtype [B,T,H,K]   dv dtype [B,T,HV,V]   dg f32 like g   dbeta f32 [B,T,HV]
 *   dh0   f32 [N,HV,K,V] or NULL       gradient of h0 (not wanted if NULL)
 *   workspace  >= gdr_bwd_workspace_bytes bytes (contents on entry irrelevant).
 * Supported: K up to 128 (padded to 32, 64 or 128), any V up to 256, scalar or
 * per-channel gate.  A per-channel gate, and fp32 with K = 128, at chunk_size 64
 * run the backward at chunk 32 (the chunk form is exact at any chunk size; the
 * workspace size follows); with keep_states that switch is impossible and it
 * returns GDR_ERR_UNSUPPORTED.  Other problems return GDR_ERR_UNSUPPORTED before any
 * launch.
 * Saved forward states: with p->keep_states = 1 the recompute is skipped and
 * the forward intermediates are taken from the workspace as they stand, which
 * requires that gdr_chunk_fwd ran with keep_states = 1, the same problem and
 * inputs, and this same workspace (its leading gdr_fwd_layout part) before this
 * call, with nothing written to that part in between.  The gradients are then
 * bitwise those of the recomputing call (the same kernels produced the
 * intermediates). */
gdr_status gdr_chunk_bwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const int32_t* cu_seqlens,
                         const float* h0, const void* d_o, const float* dht, void* dq, void* dk,
                         void* dv, float* dg, float* dbeta, float* dh0, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ---- the backward's stages (after K0-K3 of the forward, same layouts; scalar
 * gate only: with a per-channel gate they return GDR_ERR_UNSUPPORTED) ---- */

/* B1: de_local = scale P^T dO and qscale for every chunk and value head
 * (differentiating o through the intra-chunk term of the chunk form on the
 * coverage-matrix page, section 2). */
gdr_status gdr_bwd_intra(const gdr_problem* p, const void* q, const void* k, const float* g,
                         const void* d_o, const int32_t* chunk_idx, const int32_t* chunk_off,
                         void* de_local, float* qscale, void* stream);

/* B2: reverse state-gradient scan.  For each sequence and value head, dS starts
 * at dht (or 0); for the chunks from last to first: dh = dS,
 * dE = de_local + diag(kscale) K dS, dS <- exp(G_L) dS + Q^T diag(qscale) dO - W^T dE;
 * finally dh0 = dS (if dh0 != NULL).  kscale is K1's; dh is written in fp32
 * (workspace layout above). */
gdr_status gdr_bwd_dh(const gdr_problem* p, const void* q, const void* k, const void* w,
                      const void* d_o, const void* de_local, const float* qscale,
                      const float* kscale, const int32_t* chunk_idx, const int32_t* chunk_off,
                      const float* dht, void* dh, float* dh0, void* stream);

/* B3: per chunk and q/k head, every remaining gradient: dq, dk (group sums and
 * L2-norm backward included), dv, dbeta and dg, from q, k, v, g, beta, d_o, Tm
 * (K1), h and v_new (K3) and dh (B2, fp32). */
gdr_status gdr_bwd_dqkvg(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const void* d_o, const void* Tm,
                         const void* h, const void* v_new, const void* dh,
                         const int32_t* chunk_idx, const int32_t* chunk_off, void* dq, void* dk,
                         void* dv, float* dg, float* dbeta, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
