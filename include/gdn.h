/*
 * gdn.h -- C ABI of the MI355X (gfx950) chunked gated-delta-rule forward pass.
 *
 * The operation (Gated DeltaNet, and Kimi Delta Attention with a per-channel
 * gate) is the recurrence, per sequence and head, with the state S kept as a
 * K x V matrix:
 *
 *     S_t = Decay_t(S_{t-1});  S_t += beta_t k_t (v_t - S_t^T k_t)^T;
 *     o_t = scale * S_t^T q_t
 *
 * with Decay_t(S) = exp(g_t) S for GDN (g natural-log, one scalar per token
 * and head) and Decay_t(S)[d,:] = 2^(g_t[d]) S[d,:] for KDA (g in log2 units,
 * one value per token, head and key channel). q/k may be L2-normalised in
 * the kernel (x / sqrt(sum x^2 + 1e-6)) and beta may be passed as logits
 * (sigmoid in the kernel). Sources, by page title and function:
 *   - the eager chunk algorithm, the L2-norm helper and the K x V state
 *     orientation: hyper-parallel "Diff Coverage" page, gate build
 *     2026-09-10 (torch_chunk_gated_delta_rule, _l2norm,
 *     _prepare_gdn_chunks_for_summary, _run_prepared_gdn_chunks);
 *   - the native fused-forward flags (q/k L2-norm, sigmoid(beta), layout,
 *     cu_seqlens) and the contract checks: "Diff Coverage" page, gate build
 *     2026-11-06 (_load_ops, _packed_offsets, the Ascend C GDN adapter);
 *   - the prepare / chunk_fwd_h / finalize stage split, the host chunk table,
 *     packed B=1 rule and chunk size 64: the coverage page of
 *     kimi_delta_attention_ascendc.py (_packed_metadata, ascendc_chunk_kda,
 *     _AscendCKDAStages.forward).
 *
 * Contract shared by every entry point
 * ------------------------------------
 *   Sizes: K == V == 128, chunk size 64 (GDN_ERR_UNSUPPORTED otherwise).
 *   B >= 1, T >= 1, 1 <= H <= 65535, B*T < 2^30, scale finite and > 0.
 *   q, k   bf16 [B,T,H,K], v bf16 [B,T,H,V], beta bf16 [B,T,H], o bf16
 *          [B,T,H,V]: contiguous, token-major; device pointers.
 *   g      fp32 device pointer, [B,T,H] (GDN) or [B,T,H,K] (KDA).
 *   Packed input: cu_seqlens != NULL is a HOST int32 array of num_seqs+1
 *          offsets, strictly increasing from 0 to T (so no empty document);
 *          B must be 1. The library copies it before returning, so the caller
 *          may free it at once. Documents need not be multiples of 64: the
 *          last chunk of each document is partial. Chunks never span
 *          documents. Dense input: cu_seqlens == NULL and num_seqs == B.
 *   States: initial_state fp32 [N,H,K,V] device pointer or NULL (= zeros);
 *          final_state fp32 [N,H,K,V], written when non-NULL and flags has
 *          GDN_OUTPUT_FINAL_STATE. N = num_seqs.
 *   Ownership: the caller allocates every buffer. The library reads the
 *          inputs, writes only the outputs and the workspace, and keeps no
 *          pointer after it returns.
 *   Stream: `stream` is a hipStream_t (NULL = the null stream). All work is
 *          enqueued on it; nothing is synchronised. The device is the one
 *          current on the calling thread.
 *   Workspace: device memory of at least the size the matching
 *          *_workspace_bytes call returns. NULL means the library allocates
 *          it stream-ordered (hipMallocAsync) and frees it on the same stream.
 *   Errors: a non-zero status means nothing was launched and nothing was
 *          written (except for GDN_ERR_HIP raised by a launch, after which the
 *          outputs are undefined). gdn_last_error() gives the message of the
 *          calling thread's last failure.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_OK 0
#define GDN_ERR_INVALID_ARGUMENT 1 /* shape, pointer, offsets, scale, flags */
#define GDN_ERR_UNSUPPORTED 2      /* K/V != 128, device not gfx950 */
#define GDN_ERR_HIP 3              /* HIP runtime or launch failure */

#define GDN_L2NORM_QK 1u          /* normalise q and k rows in the kernel */
#define GDN_BETA_SIGMOID 2u       /* beta holds logits: beta = 1/(1+exp(-x)) */
#define GDN_OUTPUT_FINAL_STATE 4u /* write final_state */

#define GDN_CHUNK 64
#define GDN_HEAD_DIM 128
#define GDN_VEC_ROWS 8 /* per-chunk vectors in the prepare output, see below */

/* Message of the calling thread's last failed call ("" if none). */
const char* gdn_last_error(void);

/* Number of 64-token chunks over all sequences: sum over documents of
 * ceil(len/64) (dense: B * ceil(T/64)). Returns a status; *num_chunks is set
 * on success. Follows the chunk table of _packed_metadata on the coverage
 * page of kimi_delta_attention_ascendc.py. */
int gdn_num_chunks(int32_t B, int32_t T, int32_t num_seqs, const int32_t* cu_seqlens, int64_t* num_chunks);

/* Workspace bytes for gdn_chunk_fwd / kda_chunk_fwd (0 on invalid arguments;
 * gdn_last_error() then says why). */
size_t gdn_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                     int32_t num_seqs, const int32_t* cu_seqlens, uint32_t flags);
size_t kda_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                     int32_t num_seqs, const int32_t* cu_seqlens, uint32_t flags);

/* Whole forward pass, GDN (scalar natural-log gate g [B,T,H]). Computes o
 * and, with GDN_OUTPUT_FINAL_STATE, final_state, exactly as the recurrence
 * above (the chunked algorithm of torch_chunk_gated_delta_rule on the
 * 2026-09-10 "Diff Coverage" page is the method). */
int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                  int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, float scale, uint32_t flags,
                  void* o, float* final_state, void* workspace, size_t workspace_bytes, void* stream);

/* Whole forward pass, GDN, for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and results as gdn_chunk_fwd with dense input, but the
 * intermediates (the per-chunk T, output matrix and row vectors) go to a
 * fixed device array of GDN_NOALLOC_SCRATCH_BYTES inside the library instead
 * of a workspace, and the call allocates nothing (no hipMalloc, hipFree,
 * pinned host memory or events). The caller still passes every input and
 * output. Limits and behaviour:
 *   - dense input only: cu_seqlens must be NULL (GDN_ERR_UNSUPPORTED
 *     otherwise) and num_seqs == B;
 *   - the intermediates must fit: gdn_chunk_fwd_workspace_bytes() of the
 *     same problem <= GDN_NOALLOC_SCRATCH_BYTES (B=4, T=4096, H=16 fits);
 *     larger problems get GDN_ERR_INVALID_ARGUMENT and nothing is
 *     launched;
 *   - the array is per device and shared by every call on that device: two
 *     calls that overlap in time on one device (other streams or threads)
 *     race on it and their results are undefined. Each call overwrites every
 *     scratch byte it reads before reading it, so nothing needs clearing
 *     between calls;
 *   - the device address of the array is resolved on the first call on each
 *     device and kept; the array lives until the process ends;
 *   - per-kernel timing (gdn_timing_enable) does not apply to this entry.
 * Every other argument, and the error behaviour, as gdn_chunk_fwd. */
#define GDN_NOALLOC_SCRATCH_BYTES (128u << 20)
int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g, const void* beta,
                          const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                          int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, float scale, uint32_t flags,
                          void* o, float* final_state, void* stream);

/* Whole forward pass, KDA (per-key-channel log2 gate g [B,T,H,K]; the
 * chunk-local cumulative log2 decay slot gk of the KDA prepare stage on the
 * kimi_delta_attention_ascendc.py coverage page). Same arguments otherwise. */
int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                  int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, float scale, uint32_t flags,
                  void* o, float* final_state, void* workspace, size_t workspace_bytes, void* stream);

/* Whole forward pass with the gate formed in the kernel (use_gate_in_kernel
 * of the native forward contract on the 2026-11-06 "Diff Coverage" page; the
 * A_log / dt_bias gate parameters of _prepare_kda on the
 * kimi_delta_attention_ascendc.py coverage page). The pages name the inputs
 * but print no formula; the one taken is the gate of the GDN and KDA layers:
 *   GDN: g[b,t,h]   = -exp(A_log[h]) * softplus(g_raw[b,t,h] + dt_bias[h])
 *        (natural log), g_raw fp32 [B,T,H], A_log fp32 [H], dt_bias fp32 [H];
 *   KDA: g[b,t,h,d] = -exp(A_log[h]) * softplus(g_raw[b,t,h,d] + dt_bias[h,d])
 *        / ln 2 (log2), g_raw fp32 [B,T,H,K], A_log fp32 [H], dt_bias fp32
 *        [H,K]; g_raw and dt_bias 16-byte aligned;
 * softplus(y) = log(1 + e^y), evaluated in fp32. A_log and dt_bias are
 * device pointers and must be non-NULL (GDN_ERR_INVALID_ARGUMENT). The
 * result equals gdn_chunk_fwd / kda_chunk_fwd given that g; every other
 * argument, the workspace size and the error behaviour are theirs. The
 * lower-bounded "safe gate" variant is not provided (no formula is given). */
int gdn_chunk_fwd_gated(const void* q, const void* k, const void* v, const float* g_raw, const float* A_log,
                        const float* dt_bias, const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                        int32_t V, float scale, uint32_t flags, void* o, float* final_state, void* workspace,
                        size_t workspace_bytes, void* stream);
int kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const float* g_raw, const float* A_log,
                        const float* dt_bias, const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                        int32_t V, float scale, uint32_t flags, void* o, float* final_state, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Per-kernel timing of gdn_chunk_fwd / kda_chunk_fwd, for benchmarks. While
 * enabled (per calling thread), every whole-pass call records three HIP
 * events on its stream: before the prepare kernel, between the prepare and
 * the state/output kernel, and after it. gdn_timing_read() waits for the
 * recorded events, returns the summed milliseconds of each kernel and the
 * number of calls, and clears the record. Events are created by the library
 * and reused; they are never destroyed before the process ends. */
int gdn_timing_enable(int32_t enable);
int gdn_timing_read(double* prepare_ms, double* state_ms, int64_t* calls);

/* The same for gdn_chunk_bwd: while timing is enabled, every backward call
 * records six events on its stream (before the prepare kernel, after it,
 * after the forward state pass, after each of the three backward kernels).
 * gdn_bwd_timing_read() waits for them and returns, in ms[0..4], the summed
 * milliseconds of prepare, forward state pass, reverse state pass, state
 * products and per-chunk gradients, and the number of calls; it clears the
 * record. */
int gdn_bwd_timing_read(double* ms, int64_t* calls);

/*
 * Stage entry points (the prepare / chunk_fwd_h / finalize split of
 * _AscendCKDAStages.forward on the kimi_delta_attention_ascendc.py coverage
 * page). The whole-pass entries above run the same prepare kernel followed by
 * a kernel that fuses chunk_fwd_h and finalize; these entries expose the
 * chunk-form intermediates for parity checks. NT is gdn_num_chunks(); chunk
 * c is global (documents in order, chunks in order inside a document).
 * Every intermediate is head-major with 64 rows per chunk; rows of a partial
 * chunk past the end of its document are zero.
 *
 *   tmat [H,NT,64,128] bf16 T = (I + strictLower(diag(beta) Kn Kn^T * Gamma))^-1,
 *                          the forward-substitution result plus identity
 *                          (GDN: Gamma[i,j] = exp(G_i - G_j); KDA: per channel
 *                          inside the sum), Kn the normalised keys. Row i
 *                          holds hi[64] then lo[64] with hi = bf16(T_ij) and
 *                          lo = bf16(T_ij - hi), both with permuted columns:
 *                          column 32s + 16h + 4g + e (s, h in {0,1},
 *                          g, e in 0..3) is stored at position
 *                          32s + 8g + 4h + e.
 *   aqk  [H,NT,64,64] bf16 scale * (Qn Kn^T * Gamma), lower triangle with the
 *                          diagonal, zero above; columns permuted as tmat's.
 *   vec  [H,NT,8,64]  fp32 per-row vectors of the chunk, row r:
 *                          0 beta (after the sigmoid when flagged)
 *                          1 GDN: beta*rk*exp(G)      KDA: beta*rk
 *                          2 GDN: rk*exp(G_last - G)  KDA: rk
 *                          3 GDN: scale*rq*exp(G)     KDA: scale*rq
 *                          4 GDN: G (natural log)     KDA: 0
 *                          5 rq   6 rk   (1/sqrt(sum x^2 + 1e-6), or 1)
 *                          7 entry 0: GDN exp(G_last), KDA 0; others 0
 *                          with G the chunk-local cumulative sum of g.
 *   gk   [H,NT,64,128] fp32 (KDA only, else NULL) chunk-local cumulative
 *                          log2 gate per key channel.
 *   h    [H,NT,128,128] fp32 state entering each chunk (K x V).
 *   v_new [H,NT,64,128] fp32 U - W S for each chunk.
 */
int gdn_stage_prepare(int32_t kda, const void* q, const void* k, const float* g, const void* beta,
                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                      int32_t K, int32_t V, float scale, uint32_t flags,
                      void* tmat, void* aqk, float* vec, float* gk, void* stream);

int gdn_stage_fwd_h(int32_t kda, const void* k, const void* v, const void* tmat, const float* vec,
                    const float* gk, const float* initial_state, const int32_t* cu_seqlens,
                    int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                    uint32_t flags, float* h, float* v_new, float* final_state, void* stream);

int gdn_stage_finalize(int32_t kda, const void* q, const void* aqk, const float* vec, const float* gk,
                       const float* h, const float* v_new, const int32_t* cu_seqlens, int32_t num_seqs,
                       int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, void* o, void* stream);

/*
 * Backward pass, GDN scalar gate (the three stages bwd_prepare_saved,
 * bwd_state_saved and bwd_finish_saved of _GDNStateP2PTritonFunction.backward
 * on the hyper-parallel "Diff Coverage" page of 2026-09-10; as the native
 * backward of the 2026-11-06 gate build, the gate gradient is the one of the
 * raw per-token gate). For the forward of gdn_chunk_fwd with the same
 * arguments, the gradients of
 *   L = <d_o, o> + <d_final_state, final_state>
 * with respect to the raw inputs:
 *   d_o            [B,T,H,V] bf16, the output cotangent (required);
 *   d_final_state  [N,H,K,V] fp32 or NULL (zero);
 *   dq, dk         [B,T,H,K] fp32 w.r.t. q, k as passed (through the
 *                  in-kernel L2-norm when GDN_L2NORM_QK is set);
 *   dv             [B,T,H,V] fp32;
 *   dg             [B,T,H]   fp32 w.r.t. the raw gate g (natural log);
 *   dbeta          [B,T,H]   fp32 w.r.t. beta as passed (through the sigmoid
 *                  when GDN_BETA_SIGMOID is set);
 *   d_initial_state [N,H,K,V] fp32 or NULL (not written); the gradient
 *                  w.r.t. initial_state (NULL initial_state meaning zero).
 * All other arguments as gdn_chunk_fwd (GDN_OUTPUT_FINAL_STATE is ignored).
 * Outputs are device arrays owned by the caller; dq, dk, dv and d_o 16-byte
 * aligned. The call recomputes the forward intermediates (prepare kernel,
 * then the state pass storing the state entering every chunk and v_new),
 * then runs the reverse state pass and the per-chunk gradient kernels, all
 * on `stream`. workspace: as gdn_chunk_fwd, sized by
 * gdn_chunk_bwd_workspace_bytes (0 on a contract error; the forward's
 * plus NT*H*288 KiB and a few KiB for the gated variant's per-head sums).
 * Errors as gdn_chunk_fwd; nothing is launched on
 * error.
 */
size_t gdn_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                     const int32_t* cu_seqlens, uint32_t flags);
int gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                  int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, float scale, uint32_t flags,
                  const void* d_o, const float* d_final_state, float* dq, float* dk, float* dv, float* dg,
                  float* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream);

/* Backward of gdn_chunk_fwd_gated (the gate -exp(A_log[h]) softplus(g_raw +
 * dt_bias[h]) formed in the kernel): the arguments of gdn_chunk_bwd with
 * g_raw, A_log and dt_bias as gdn_chunk_fwd_gated takes them, and
 *   dg_raw   [B,T,H] fp32, the gradient w.r.t. g_raw
 *            (= -exp(A_log) sigmoid(g_raw + dt_bias) times the gate's);
 *   dA_log   [H] fp32, sum over tokens of (gradient w.r.t. the gate) * gate;
 *   ddt_bias [H] fp32, sum over tokens of dg_raw;
 * all device pointers, required (GDN_ERR_INVALID_ARGUMENT if NULL). The
 * per-head sums are taken in a fixed order (bitwise reproducible). Same
 * workspace size as gdn_chunk_bwd; errors and stream behaviour as there. The
 * pages print no gate formula: the one taken is that of gdn_chunk_fwd_gated. */
int gdn_chunk_bwd_gated(const void* q, const void* k, const void* v, const float* g_raw, const float* A_log,
                        const float* dt_bias, const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                        int32_t V, float scale, uint32_t flags, const void* d_o, const float* d_final_state,
                        float* dq, float* dk, float* dv, float* dg_raw, float* dA_log, float* ddt_bias,
                        float* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Affine state summary (_compute_gdn_state_summary_from_prepared and
 * _apply_gdn_state_summary on the 2026-09-10 "Diff Coverage" page): for every
 * sequence n and head h, the final state is affine in the initial one,
 *   S_final = M S_initial + S,
 * with M [K,K] the product over the chunks, in order, of the chunk
 * transitions decay*I - (k * decay_to_end)^T W (KDA: diag(2^G_last) and the
 * per-channel key decay), and S [K,V] the final state from a zero initial
 * state. Segments of one long sequence can then be processed independently
 * and chained by the apply step (the single-GPU half of sequence-parallel
 * processing).
 *
 * gdn_state_summary / kda_state_summary: inputs as gdn_chunk_fwd /
 *   kda_chunk_fwd (q may be NULL: no output is formed, so q and the scale
 *   are not used). flags: GDN_L2NORM_QK and GDN_BETA_SIGMOID as there;
 *   GDN_OUTPUT_FINAL_STATE is ignored. Outputs (device, fp32, caller-owned):
 *     transition [N,H,K,K]  M, row-major (M[i][j] multiplies S_initial[j][:]);
 *     state_ext  [N,H,K,V]  S.
 *   Runs the prepare kernel, then the state-only pass twice (from a zero
 *   state with v, and from the identity with v taken as zero). workspace as
 *   for gdn_chunk_fwd, sized by gdn_state_summary_workspace_bytes (0 on a
 *   contract error). Errors as gdn_chunk_fwd; nothing is launched on error.
 *
 * gdn_state_summary_apply: state_out = transition @ state_in + state_ext for
 *   N*H (sequence, head) pairs, fp32 (device arrays, 16-byte aligned,
 *   caller-owned; state_in NULL means zero; state_out may be state_ext but
 *   not transition or state_in). K = V = 128.
 */
int gdn_state_summary(const void* q, const void* k, const void* v, const float* g, const void* beta,
                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                      int32_t V, uint32_t flags, float* transition, float* state_ext, void* workspace,
                      size_t workspace_bytes, void* stream);
int kda_state_summary(const void* q, const void* k, const void* v, const float* g, const void* beta,
                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                      int32_t V, uint32_t flags, float* transition, float* state_ext, void* workspace,
                      size_t workspace_bytes, void* stream);
/* The summary with the gate formed in the kernel: kda selects the gate kind
 * (0: GDN, 1: KDA); g_raw, A_log and dt_bias as gdn_chunk_fwd_gated /
 * kda_chunk_fwd_gated take them; everything else as the summaries above. */
int gdn_state_summary_gated(int32_t kda, const void* q, const void* k, const void* v, const float* g_raw,
                            const float* A_log, const float* dt_bias, const void* beta, const int32_t* cu_seqlens,
                            int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                            uint32_t flags, float* transition, float* state_ext, void* workspace,
                            size_t workspace_bytes, void* stream);
size_t gdn_state_summary_workspace_bytes(int32_t kda, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                         int32_t num_seqs, const int32_t* cu_seqlens);
int gdn_state_summary_apply(const float* transition, const float* state_ext, const float* state_in,
                            float* state_out, int32_t N, int32_t H, int32_t K, int32_t V, void* stream);

/*
 * Backward pass, KDA (per-key-channel log2 gate): the arguments and outputs
 * of gdn_chunk_bwd for the forward of kda_chunk_fwd, with g [B,T,H,K] and
 *   dg [B,T,H,K] fp32, the gradient w.r.t. the raw log2 gate;
 * g, d_o, dq, dk, dv and dg 16-byte aligned. The call recomputes the forward
 * intermediates (the KDA prepare kernel writing the cumulative gate; the
 * state pass storing the state entering every chunk and v_new), runs the
 * reverse state pass below, the products with the saved states, and the
 * per-chunk gradients (the terms of the intra-chunk matrices with their
 * per-channel decays, the gate's reverse cumulative sum, the L2-norm and
 * sigmoid derivatives). Workspace sized by kda_chunk_bwd_workspace_bytes.
 * The pages print no backward formula; the steps are the derivatives of the
 * forward's chunk form, in the order of bwd_prepare_saved, bwd_state_saved
 * and bwd_finish_saved on the 2026-09-10 "Diff Coverage" page.
 */
size_t kda_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                     const int32_t* cu_seqlens, uint32_t flags);
int kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                  int32_t H, int32_t K, int32_t V, float scale, uint32_t flags, const void* d_o,
                  const float* d_final_state, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                  float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream);

/* Backward of kda_chunk_fwd_gated (the per-channel gate
 * -exp(A_log[h]) softplus(g_raw + dt_bias[h,d]) / ln 2 formed in the
 * kernel): the arguments of kda_chunk_bwd with g_raw [B,T,H,K], A_log [H] and
 * dt_bias [H,K] as kda_chunk_fwd_gated takes them, and
 *   dg_raw   [B,T,H,K] fp32, the gradient w.r.t. g_raw
 *            (= -exp(A_log) sigmoid(g_raw + dt_bias) / ln 2 times the gate's);
 *   dA_log   [H] fp32, sum over tokens and channels of (gradient w.r.t. the
 *            gate) * gate;
 *   ddt_bias [H,K] fp32, sum over tokens of dg_raw;
 * all device pointers, required (GDN_ERR_INVALID_ARGUMENT if NULL), dt_bias
 * 16-byte aligned. The sums are taken in a fixed order (bitwise
 * reproducible). Same workspace size as kda_chunk_bwd; errors and stream
 * behaviour as there. The pages print no gate formula: the one taken is that
 * of kda_chunk_fwd_gated. */
int kda_chunk_bwd_gated(const void* q, const void* k, const void* v, const float* g_raw, const float* A_log,
                        const float* dt_bias, const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                        int32_t V, float scale, uint32_t flags, const void* d_o, const float* d_final_state,
                        float* dq, float* dk, float* dv, float* dg_raw, float* dA_log, float* ddt_bias,
                        float* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * KDA backward, reverse state pass (the stage of the backward that carries the
 * state gradient across chunks; bwd_state_saved of the backward on the
 * 2026-09-10 "Diff Coverage" page, with the per-channel decays of the KDA
 * stages). For the forward of kda_chunk_fwd with the same q, k, g, beta,
 * scale, flags and cu_seqlens, and the loss <d_o, o> + <d_final_state,
 * final_state>, it writes per chunk, from the last to the first:
 *   dh_next [H,NT,K,V] fp32  the gradient w.r.t. the state leaving the chunk;
 *   dv_new  [H,NT,64,V] fp32 the gradient w.r.t. the chunk's
 *                            v_new = U - W S (rows past a document's end 0;
 *                            16-byte aligned);
 *   d_initial_state [N,H,K,V] fp32 or NULL  the gradient w.r.t. the initial
 *                            state.
 * NT = gdn_num_chunks(...), chunks numbered as the forward's chunk table
 * (head-major: element [h, c]). The gradient is linear in d_o and
 * d_final_state and does not depend on v or the initial state, which are not
 * arguments. d_o bf16 [B,T,H,V] (required); d_final_state fp32 [N,H,K,V] or
 * NULL (zero). Workspace sized by kda_bwd_state_pass_workspace_bytes; other
 * arguments, errors and stream behaviour as kda_chunk_fwd. It is the second
 * stage of kda_chunk_bwd, exposed for stage checks.
 */
size_t kda_bwd_state_pass_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, int32_t num_seqs,
                                          const int32_t* cu_seqlens, uint32_t flags);
int kda_bwd_state_pass(const void* q, const void* k, const float* g, const void* beta, const int32_t* cu_seqlens,
                       int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, float scale,
                       uint32_t flags, const void* d_o, const float* d_final_state, float* dh_next, float* dv_new,
                       float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal depthwise Conv1d + SiLU (the ShortConv forming q, k, v from the
 * projections; _causal_conv1d_with_cp_halo on the 2026-09-10 "Diff Coverage"
 * page): per channel c and token t,
 *   y[t,c] = act(bias[c] + sum_{j<W} weight[c,j] * x[t - (W-1-j)*dilation, c]),
 * act = SiLU (z / (1 + e^-z)) if silu != 0, else identity; rows before the
 * start of a sequence come from the halo, else zero.
 *   x     [B,T,D] bf16, token-major, 16-byte aligned; D a multiple of 8.
 *   weight [D,W] fp32 (a depthwise Conv1d's [D,1,W] weight), W in 1..8.
 *   bias  [D] fp32 or NULL.
 *   halo  bf16 or NULL: [B,(W-1)*dilation,D] rows preceding each sequence
 *         (dense), or [1,(W-1)*dilation,D] preceding the first document
 *         (packed); the preceding rank's last rows in a sequence split.
 *   cu_seqlens host int32 [num_seqs+1] or NULL, as gdn_chunk_fwd (B = 1):
 *         every document is its own sequence.
 *   y     [B,T,D] bf16 output (round to nearest even), must not alias x.
 * fp32 accumulation. workspace: gdn_short_conv_workspace_bytes (the device
 * copy of the offsets; 0 for dense input), or NULL for a stream-ordered
 * allocation. Errors as gdn_chunk_fwd (D not a multiple of 8 or W outside
 * 1..8: GDN_ERR_UNSUPPORTED); nothing is launched on error. Asynchronous on
 * `stream`; buffers are caller-owned.
 */
size_t gdn_short_conv_workspace_bytes(int32_t num_seqs, const int32_t* cu_seqlens);
int gdn_short_conv(const void* x, const float* weight, const float* bias, const void* halo,
                   const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t D, int32_t W,
                   int32_t dilation, int32_t silu, void* y, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
