/* gdn.h — C ABI of the Gated DeltaNet (GDN) token mixer for AMD Instinct MI355X (gfx950).
 *
 * What is computed (the mixer of one GDN layer; sources are web pages on Qwen3.8-Flash-Next):
 *   1. short causal depthwise conv of width 4 on the raw q, k and v channels, then SiLU
 *      ("Qwen3.8-Flash-Next：架构、效率与技术谱系" §02 configuration table, GDN row; paper
 *      reading "On the Design of Qwen3.8-Next Architecture … 精读" §四 4.1);
 *   2. L2 normalisation of q and k per head (paper summary "Qwen3.8-Flash-Next", Method);
 *   3. the gated delta rule per value head h, QK head g = floor(h * HK / HV), state S [d_k][d_v]
 *      (analysis notes §03 update equations):
 *          S~ = alpha_t S;  e = v_t - S~^T k_t;  S = S~ + beta_t k_t e^T;  y_t = scale * S^T q_t
 *   4. zero-centred RMSNorm over the d_v channels of each head, multiplier (1 + w)
 *      (analysis notes §03, changes made to GDN), then
 *   5. a sigmoid output gate, elementwise (paper summary, Method: normalised, then gated).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library allocates no memory,
 *     keeps no state between calls (beyond, per device, the kernels' raised LDS limits and the
 *     static scratch of gdn_prefill_static) and never synchronises: work is enqueued on the
 *     caller's stream (`hip_stream`, a hipStream_t; NULL = the default stream) and the call
 *     returns after the enqueue. Device faults surface at the caller's next synchronisation.
 *   - Arguments are validated on the host first. On failure the call returns a status, enqueues
 *     nothing, leaves every output untouched and records a message for gdn_last_error().
 *     A failing kernel launch returns GDN_E_HIP.
 *   - Tensor pointers must be 16-byte aligned, except alpha, beta and cu_seqlens (4-byte). Row
 *     strides are in elements and must keep every row 16-byte aligned (a multiple of 8 for bf16,
 *     of 4 for fp32).
 *   - "io" tensors (q, k, v, gate, out, conv state) have the dtype cfg->io_dtype; alpha, beta,
 *     conv weights, norm gains and recurrent states are always fp32.
 *   - Channel order of the conv (weights and conv state): all q channels [HK][d_k], then all k
 *     channels [HK][d_k], then all v channels [HV][d_v]; C_tot = 2*HK*d_k + HV*d_v.
 *   - Conv tap j (0..3) multiplies the input 3-j tokens before the current one (tap 3 = current).
 *     The conv state holds the 3 most recent raw inputs per channel, oldest first.
 *   - Functions are reentrant; concurrent calls need distinct workspaces. Prefill results are
 *     bitwise reproducible for a fixed configuration and device (no atomics).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_E_NULL = 1,        /* a required pointer is NULL                                   */
  GDN_E_SHAPE = 2,       /* head counts, dims, lengths or cu_seqlens are inconsistent    */
  GDN_E_DTYPE = 3,       /* unknown io dtype                                             */
  GDN_E_ALIGN = 4,       /* pointer or stride breaks the 16-byte rule                    */
  GDN_E_WORKSPACE = 5,   /* workspace NULL or smaller than gdn_prefill_workspace()      */
  GDN_E_UNSUPPORTED = 6, /* valid but not implemented (e.g. conv width != 4, d > 128)    */
  GDN_E_HIP = 7,         /* a HIP runtime call or kernel launch failed                   */
  GDN_E_VALUE = 8        /* a scalar parameter is out of range (eps < 0, flags)          */
} gdn_status;

typedef enum gdn_dtype { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* Stage switches (cfg->flags). GDN_CONV covers the conv and its SiLU. With NORM and GATE off the
 * output is the raw readout y. GDN_ALL is the layer as the pages describe it. */
enum { GDN_CONV = 1u, GDN_L2QK = 2u, GDN_NORM = 4u, GDN_GATE = 8u, GDN_ALL = 15u };

typedef struct gdn_cfg {
  int32_t n_qk_heads;       /* HK: 16 at the model shape                                      */
  int32_t n_v_heads;        /* HV: 48 at the model shape; HV % HK == 0                        */
  int32_t d_k;              /* key/query head dim: 128 at the model shape; 16, 32, 64 or 128 */
  int32_t d_v;              /* value head dim: 128 at the model shape; 16, 32, 64 or 128     */
  int32_t conv_width;       /* must be 4                                                      */
  int32_t io_dtype;         /* gdn_dtype                                                      */
  uint32_t flags;           /* GDN_* stage switches                                           */
  float scale;              /* readout scale on y (1.0)                                       */
  float l2_eps;             /* q/k L2: a / sqrt(sum a^2 + l2_eps) (1e-6)                      */
  float norm_eps;           /* RMSNorm: y / sqrt(mean y^2 + norm_eps) (1e-6)                  */
  int32_t norm_head_stride; /* 0: one gain vector w[d_v] for all heads; d_v: w[HV][d_v]      */
} gdn_cfg;

/* Fills *cfg with the model-shape defaults: HK=16, HV=48, d_k=d_v=128, width 4, bf16,
 * GDN_ALL, scale 1, eps 1e-6, shared gain. */
void gdn_cfg_default(gdn_cfg* cfg);

/* Bytes of device workspace gdn_prefill needs for this configuration, for any packing of
 * `total_tokens` tokens into `n_seqs` sequences. Pure host computation. */
gdn_status gdn_prefill_workspace(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens,
                                 size_t* bytes);

/* Packed (variable-length) prefill of `n_seqs` independent sequences, `total_tokens` tokens in
 * all. Sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1]).
 *
 *   cu_seqlens        device int32 [n_seqs+1], cu[0] = 0, cu[n_seqs] = total_tokens,
 *                     non-decreasing. Out-of-range device values are clamped, never read
 *                     out of bounds, but give meaningless results.
 *   cu_seqlens_host   optional host copy of the same array; when given it is validated
 *                     (GDN_E_SHAPE on violation). May be NULL.
 *   q, k              io [T][HK][d_k], token row stride ld_q / ld_k elements (>= HK*d_k).
 *   v                 io [T][HV][d_v], token row stride ld_v (>= HV*d_v).
 *   alpha, beta       fp32 [T][HV]: per-token decay in (0, 1] and write strength in [0, 1].
 *   gate              io [T][HV][d_v] sigmoid-gate logits; required iff GDN_GATE.
 *   conv_w            fp32 [C_tot][4]; required iff GDN_CONV.
 *   norm_w            fp32 [d_v] (norm_head_stride 0) or [HV][d_v]; required iff GDN_NORM.
 *   state_in          fp32 [n_seqs][HV][d_k][d_v] initial states; NULL = zeros.
 *   state_out         fp32 [n_seqs][HV][d_k][d_v] final states; NULL = not written.
 *                     May alias state_in.
 *   conv_in           io [n_seqs][3][C_tot] raw inputs before each sequence; NULL = zeros.
 *   conv_out          io [n_seqs][3][C_tot] the last 3 raw inputs of each sequence (from conv_in
 *                     when a sequence is shorter than 3); NULL = not written. May alias conv_in.
 *   out               io [T][HV][d_v] mixer output (raw y when NORM and GATE are off).
 *   workspace         device scratch of at least gdn_prefill_workspace() bytes, 256-byte
 *                     aligned; its contents on entry do not matter.
 * The bf16 path at d_k = d_v = 128 runs the chunked (64-token) WY form on bf16 MFMA with an
 * fp32 state; every other configuration (and every fp32-io call) runs a token-sequential fp32
 * recurrence, which keeps fp32 accuracy.
 * total_tokens must stay below 2^31 and small enough that every kernel grid fits in 2^32
 * work-items (about 22M tokens at 48 value heads); beyond that both calls return
 * GDN_E_UNSUPPORTED and the batch must be split. */
gdn_status gdn_prefill(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens,
                       const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                       const void* q, const void* k, const void* v,
                       int64_t ld_q, int64_t ld_k, int64_t ld_v,
                       const float* alpha, const float* beta, const void* gate,
                       const float* conv_w, const float* norm_w,
                       const float* state_in, float* state_out,
                       const void* conv_in, void* conv_out,
                       void* out, void* workspace, size_t workspace_bytes, void* hip_stream);

/* One decode step for `batch` independent sequences, one new token each: the prefill above with
 * every sequence of length 1, its state and conv cache updated in place.
 *   q, k        io [B][HK][d_k], row stride ld_q / ld_k;  v io [B][HV][d_v], row stride ld_v.
 *   alpha, beta fp32 [B][HV];  gate io [B][HV][d_v] (iff GDN_GATE).
 *   conv_w, norm_w as for gdn_prefill.
 *   conv_state  io [B][3][C_tot]: read as the history, then shifted to end with this token.
 *               Required iff GDN_CONV.
 *   state       fp32 [B][HV][d_k][d_v], updated in place.
 *   out         io [B][HV][d_v].
 * Any supported head dims and io dtype; HV / HK <= 64. */
gdn_status gdn_decode_step(const gdn_cfg* cfg, int32_t batch,
                           const void* q, const void* k, const void* v,
                           int64_t ld_q, int64_t ld_k, int64_t ld_v,
                           const float* alpha, const float* beta, const void* gate,
                           const float* conv_w, const float* norm_w,
                           void* conv_state, float* state, void* out, void* hip_stream);

/* Speculative (multi-token) decoding, as used with the multi-token-prediction (MTP) drafts of the
 * pages' four-step speculative decoding (paper summary "Qwen3.8-Flash-Next", results; analysis
 * notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" §01 MTP row, §04 results table): each sequence
 * brings a draft of K tokens, the layer runs all of them in one call (gdn_verify), and once the
 * caller knows how many were accepted, gdn_commit advances the cache by that prefix.
 *
 * gdn_verify is the prefill of each draft (a sequence of K tokens) from the sequence's cached state
 * and conv cache, which it only reads. It also fills `log` with what gdn_commit needs: per draft
 * token, the normalised key of each QK head, the error e = v - alpha S^T k of each value head
 * (fp32), alpha, beta and the raw conv inputs -- about (HK + HV) KB per token instead of a 64 KB
 * state checkpoint per value head. gdn_commit then applies the first n_accept[b] of those rank-1
 * updates, S <- alpha S + beta k e^T, in order: the cache that many decode steps would leave, up
 * to fp32 rounding. Supported for d_k = d_v = 128, HV/HK <= 4, 1 <= n_tok <= 8, either io dtype;
 * other shapes return GDN_E_UNSUPPORTED.
 *
 * gdn_verify_log_bytes: bytes of the log for (cfg, batch, n_tok). Pure host computation.
 *
 * gdn_verify arguments (B = batch, K = n_tok; the drafts of sequence b are token rows b*K .. b*K+K-1):
 *   q, k        io [B*K][HK][d_k], row stride ld_q / ld_k;  v io [B*K][HV][d_v], row stride ld_v.
 *   alpha, beta fp32 [B*K][HV];  gate io [B*K][HV][d_v] (iff GDN_GATE).
 *   conv_w, norm_w as for gdn_prefill.
 *   conv_state  io [B][3][C_tot], read only (iff GDN_CONV).
 *   state       fp32 [B][HV][d_k][d_v], read only.
 *   out         io [B*K][HV][d_v]: the layer output of every draft token.
 *   log         device buffer of at least gdn_verify_log_bytes() bytes, 256-byte aligned, owned by
 *               the caller; overwritten. It must stay unchanged until the matching gdn_commit.
 *
 * gdn_commit arguments (same cfg, batch and n_tok as the verify that filled `log`):
 *   n_accept    device int32 [B]: accepted drafts per sequence; values outside [0, K] are clamped.
 *               Sequences with 0 are left untouched.
 *   conv_state  io [B][3][C_tot], advanced in place to end with the last accepted token (iff
 *               GDN_CONV).
 *   state       fp32 [B][HV][d_k][d_v], advanced in place.
 * A commit with every n_accept = K leaves the cache a K-token decode would; calling gdn_commit
 * twice on one log applies the prefix twice. */
gdn_status gdn_verify_log_bytes(const gdn_cfg* cfg, int32_t batch, int32_t n_tok, size_t* bytes);
gdn_status gdn_verify(const gdn_cfg* cfg, int32_t batch, int32_t n_tok,
                      const void* q, const void* k, const void* v,
                      int64_t ld_q, int64_t ld_k, int64_t ld_v,
                      const float* alpha, const float* beta, const void* gate,
                      const float* conv_w, const float* norm_w,
                      const void* conv_state, const float* state, void* out,
                      void* log, size_t log_bytes, void* hip_stream);
gdn_status gdn_commit(const gdn_cfg* cfg, int32_t batch, int32_t n_tok, const int32_t* n_accept,
                      const void* log, size_t log_bytes, void* conv_state, float* state, void* hip_stream);

/* Projections around the mixer (bf16 io). The normalised residual stream goes through learned
 * projections before the short conv, with a data-dependent decay gate and a write gate (paper
 * reading "Qwen3.8-Flash-Next", 方法); the GDN input is one fused matrix of independent operators and
 * the gates have per-head vector parameters (analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系"
 * §07 optimizer table). The pages give no gate formula; the one implemented is
 *     alpha = exp(-exp(a_log[h]) * softplus(a + dt_bias[h])),  beta = sigmoid(b),  [a | b] = x W_ab^T.
 * Weights use the linear-layer layout [out features][in features], row-major, bf16.
 *
 * gdn_proj_workspace: bytes of device workspace both calls need: 0 (the arguments are kept so callers
 * need not change; `workspace` may be NULL).
 *
 * gdn_in_proj (T tokens, hidden width H, H % 32 == 0):
 *   x        bf16 [T][H], row stride ld_x (>= H, a multiple of 8): the normalised residual stream.
 *   w_qkv    bf16 [C_tot][H]: output channels in the conv's order (q heads, k heads, v heads).
 *   w_z      bf16 [HV*d_v][H]: gate logits.   w_ab  bf16 [2*HV][H]: a (rows 0..HV-1), then b.
 *   a_log, dt_bias  fp32 [HV].
 *   qkv      bf16 [T][C_tot] out: pass q, k, v to gdn_prefill as views of it (row stride C_tot).
 *   z        bf16 [T][HV][d_v] out: the gate logits gdn_prefill takes.
 *   alpha, beta  fp32 [T][HV] out (gate pre-activations accumulated in fp32).
 * gdn_out_proj: y bf16 [T][H] = o W_out^T with o bf16 [T][HV*d_v] (the mixer output) and
 *   w_out bf16 [H][HV*d_v].
 * Both calls are one hand-written bf16 MFMA GEMM kernel (fp32 accumulate): the input projection runs
 * over the stacked weights [w_qkv | w_z | w_ab] in one launch, writes q | k | v and z in bf16 and
 * applies the gate formula to the fp32 pre-activations [a | b] in its epilogue. They allocate nothing
 * and keep no state. hidden must be a multiple of 32; returns GDN_E_UNSUPPORTED for fp32 io. */
gdn_status gdn_proj_workspace(size_t* bytes);
gdn_status gdn_in_proj(const gdn_cfg* cfg, int32_t hidden, int64_t T, const void* x, int64_t ld_x,
                       const void* w_qkv, const void* w_z, const void* w_ab, const float* a_log,
                       const float* dt_bias, void* qkv, void* z, float* alpha, float* beta,
                       void* workspace, size_t workspace_bytes, void* hip_stream);
gdn_status gdn_out_proj(const gdn_cfg* cfg, int32_t hidden, int64_t T, const void* o, const void* w_out,
                        void* y, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Backward of the recurrence (step 3 above) for training: reverse-mode derivatives of
 *     S~ = alpha_t S;  e = v_t - S~^T k_t;  S = S~ + beta_t k_t e^T;  y_t = scale * S^T q_t
 * (analysis notes §03 update equations) for packed sequences, given dL/dy and dL/dS_final. Inputs are
 * the recurrence's own: q and k after the conv, SiLU and L2 (the backward of those steps and of the
 * output norm and gate is not part of this call). fp32 io (cfg->io_dtype = GDN_F32), d_k = d_v = 128,
 * any HV multiple of HK; cfg->scale is used, cfg->flags are ignored.
 *
 *   cu_seqlens      device int32 [n_seqs+1], as for gdn_prefill.
 *   q, k            fp32 [T][HK][128];  v fp32 [T][HV][128];  alpha, beta fp32 [T][HV].
 *   state_in        fp32 [n_seqs][HV][128][128] initial states; NULL = zeros.
 *   dy              fp32 [T][HV][128]: dL/dy.
 *   dstate_out      fp32 [n_seqs][HV][128][128]: dL/dS_final; NULL = zeros.
 *   dq, dk          fp32 [T][HK][128] out: summed over the value heads that read each QK head.
 *   dv              fp32 [T][HV][128] out;  dalpha, dbeta fp32 [T][HV] out.
 *   dstate_in       fp32 [n_seqs][HV][128][128] out (dL/dS_0), or NULL.
 *   workspace       gdn_recurrence_backward_workspace() bytes, 256-byte aligned, about 16 KB per token
 *                   and value head: the chunks' factors (T = (I + A)^-1, U, Wk, ...), every chunk-start
 *                   state and the products of the reverse pass; split long batches to bound it.
 * Chunked form, 64-token chunks: a forward pass over each chain's chunks recomputes the chunk factors
 * and keeps the chunk-start states, a reverse pass over the chunks carries dL/dS, and everything else
 * is chunk-parallel fp32 MFMA products; the two sequential passes split each (sequence, value head)
 * chain into 4 workgroups of 32 value columns (the columns of the state evolve independently). */
gdn_status gdn_recurrence_backward_workspace(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens,
                                             size_t* bytes);
gdn_status gdn_recurrence_backward(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens,
                                   const int32_t* cu_seqlens, const float* q, const float* k, const float* v,
                                   const float* alpha, const float* beta, const float* state_in, const float* dy,
                                   const float* dstate_out, float* dq, float* dk, float* dv, float* dalpha,
                                   float* dbeta, float* dstate_in, void* workspace, size_t workspace_bytes,
                                   void* hip_stream);

/* Backward of the whole mixer (every step on: conv + SiLU, L2, recurrence, RMSNorm, gate), for
 * training: given dL/dout and dL/dS_final, the derivatives for every input of gdn_prefill. fp32 io,
 * d_k = d_v = 128, cfg->flags = GDN_ALL, one shared norm gain (norm_head_stride 0).
 *   q, k, v, alpha, beta, gate, conv_w, norm_w, state_in (NULL = zeros), conv_in (NULL = zeros): as for
 *                   gdn_prefill, rows contiguous ([T][HK][128], [T][HV][128]).
 *   dout            fp32 [T][HV][128]: dL/dout.   dstate_out: fp32 [N][HV][128][128] or NULL (zeros).
 *   dq, dk          fp32 [T][HK][128] out (raw inputs; a QK head collects every value head reading it);
 *   dv, dgate       fp32 [T][HV][128] out;  dalpha, dbeta fp32 [T][HV] out;
 *   dconv_w         fp32 [C_tot][4] out;  dnorm_w fp32 [128] out;
 *   dstate_in       fp32 [N][HV][128][128] out or NULL;  dconv_in fp32 [N][3][C_tot] out or NULL.
 *   workspace       gdn_backward_workspace() bytes, 256-byte aligned (about 20 KB per token and value
 *                   head: the recurrence backward's chunk factors and states, and the mixer's fp32
 *                   intermediates).
 * Every output is reproducible for a fixed configuration (sums over tokens run in a fixed order). */
gdn_status gdn_backward_workspace(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens, size_t* bytes);
gdn_status gdn_backward(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens, const int32_t* cu_seqlens,
                        const float* q, const float* k, const float* v, const float* alpha, const float* beta,
                        const float* gate, const float* conv_w, const float* norm_w, const float* state_in,
                        const float* conv_in, const float* dout, const float* dstate_out, float* dq, float* dk,
                        float* dv, float* dalpha, float* dbeta, float* dgate, float* dconv_w, float* dnorm_w,
                        float* dstate_in, float* dconv_in, void* workspace, size_t workspace_bytes,
                        void* hip_stream);

/* Allocation-free prefill, for callers that cannot allocate device memory or hand over a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments
 * and results as gdn_prefill without `workspace`/`workspace_bytes`: its scratch is a static device
 * array of GDN_STATIC_WORKSPACE_BYTES inside the library, one per GPU, which the loader places when
 * the library's code first runs on that GPU and which stays until the process ends. The call allocates
 * nothing and calls no allocating routine; the first call on a device looks up that device's copy of
 * the array (hipGetSymbolAddress), later calls reuse the address.
 *   - Returns GDN_E_WORKSPACE, enqueueing nothing, when gdn_prefill_workspace() for the problem
 *     exceeds GDN_STATIC_WORKSPACE_BYTES (at the model shape, bf16: about 1,500 tokens per call).
 *   - Uses the scratch of the calling thread's current device; `hip_stream` must belong to it.
 *   - Every call on one GPU shares that GPU's array and leaves its contents behind (the kernels need
 *     none of it on entry). Calls that overlap on one GPU race: calls on different streams, or from
 *     several threads, must be serialised by the caller. */
#define GDN_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)
gdn_status gdn_prefill_static(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens,
                              const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                              const void* q, const void* k, const void* v,
                              int64_t ld_q, int64_t ld_k, int64_t ld_v,
                              const float* alpha, const float* beta, const void* gate,
                              const float* conv_w, const float* norm_w,
                              const float* state_in, float* state_out,
                              const void* conv_in, void* conv_out, void* out, void* hip_stream);

/* Stage timing for profilers (host-side, per calling thread). After this call, every gdn_prefill
 * on this thread records events[i] on its stream before stage i and events[GDN_N_STAGES] after the
 * last stage, for the stages
 *   0 chunk table, 1 conv + SiLU + L2, 2 WY transform (or the token-sequential recurrence),
 *   3 state propagation, 4 output + RMSNorm + gate, 5 conv-cache tail (on the chunked path the
 *   output stage writes the conv tail too);
 * stages a path does not run get back-to-back events. `events` holds GDN_N_STAGES + 1 hipEvent_t
 * handles created by the caller and must stay valid while set; NULL switches recording off.
 * Returns GDN_E_SHAPE if n_events != GDN_N_STAGES + 1. */
#define GDN_N_STAGES 6
gdn_status gdn_set_stage_events(void* const* events, int32_t n_events);

/* Static description of a status code. */
const char* gdn_status_string(gdn_status status);

/* Message of the last failing call on this thread ("" if none). Valid until the next call. */
const char* gdn_last_error(void);

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
