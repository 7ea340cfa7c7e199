/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) core.
 *
 * What the library computes.  For every sequence and head, with raw per-token
 * projections q, k (dk channels per head), v (dv channels per head), a
 * per-channel decay input alpha and a per-head write-strength input b:
 *
 *   1. each q, k, v channel passes a depthwise causal conv1d of kernel 4,
 *      padding 3, no bias, then SiLU;  q and k are L2-normalised per head
 *      (AliceAI-Foundation-80B-A3B page, section 二);
 *   2. g = max(-exp(A_log[h]) * softplus(alpha + dt_bias[h]), lower_bound)
 *      (same page, section 二, gate formula; the -5.0 lower bound is the safe
 *      gate of the Ling-3.0-flash-VL page, section "KDA 层的安全门");
 *      beta = sigmoid(b) (AliceAI page, section 二: beta is not doubled);
 *   3. per token, with the dk x dv state S (rows = key channels):
 *        S <- Diag(exp(g)) S;  delta = beta (v - k^T S);  S <- S + k delta^T;
 *        o = q^T S   (the read uses the updated state)
 *      (AliceAI page, section 二, the delta-rule loop; state shape
 *      (batch, v_heads, k_dim, v_dim)).
 *
 * Prefill and decode share the state interface: a prefill's final state and
 * conv history are a decode step's input (AliceAI page, section 五).  The
 * conv history of a sequence is its last 3 raw (pre-conv) inputs per channel
 * (AliceAI page, section 四: kernel-1 = 3 history elements), stored oldest
 * first with channels ordered q | k | v:  Ctot = H * (2*dk + dv).
 *
 * Entry points: kda_prefill (B equal-length sequences) and kda_varlen_prefill
 * (packed sequences), each in the chunked form or, for gates below -5.4, the
 * token recurrence; kda_decode_step (one token per sequence, in place);
 * kda_decode_multi (K tokens per sequence through state / conv-history pools,
 * with commit counts for speculative decoding); kda_decode_step_gated and
 * kda_decode_multi_gated (the same with the output epilogue fused);
 * kda_output_gate (the layer's o_norm x sigmoid output epilogue); plus the
 * workspace queries, the version and status strings.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, contiguous, row-major in the
 *    layout given, 16-byte aligned.  The caller owns every buffer; the library
 *    allocates no device memory and keeps no mutable global state, so calls on
 *    different streams are independent.  The one exception is
 *    kda_varlen_prefill_noalloc, whose fixed per-GPU scratch array is shared
 *    by all its calls on that GPU (see there).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and is asynchronous: the library never synchronises and never reads
 *    device data on the host.
 *  - Host-side validation runs before any launch.  On failure the call
 *    returns a nonzero kda_status_t, launches nothing and leaves every output
 *    untouched.  A launch failure returns KDA_ERR_HIP.  Faults inside kernels
 *    surface at the caller's next synchronisation.
 *  - NaN/Inf inputs propagate; they are not trapped.
 *  - B == 0 or N == 0 is a valid no-op returning KDA_OK.  A sequence of
 *    length 0 passes its initial state and conv history through unchanged.
 *  - Supported geometry: dk == dv, dk in {16, 32, 64, 128}; chunk_size 64.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1,    /* null required pointer, negative size, bad cu_seqlens length */
    KDA_ERR_UNSUPPORTED = 2,         /* geometry / dtype / flag combination not built */
    KDA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the size query's answer */
    KDA_ERR_HIP = 4                  /* a HIP launch reported an error */
} kda_status_t;

typedef enum kda_dtype {
    KDA_BF16 = 0,
    KDA_FP32 = 1
} kda_dtype_t;

/* Test hooks; 0 for the method as described. */
#define KDA_FLAG_SKIP_CONV   (1u << 0) /* q, k, v are already conv + SiLU outputs           */
#define KDA_FLAG_SKIP_L2NORM (1u << 1) /* q, k are used without L2 normalisation           */
#define KDA_FLAG_RAW_GATE    (1u << 2) /* alpha holds g itself (no softplus, no clamp)      */
#define KDA_FLAG_RAW_BETA    (1u << 3) /* b holds beta itself (no sigmoid)                  */
#define KDA_FLAG_BETA_X2     (1u << 4) /* beta = 2 sigmoid(b): negative eigenvalues allowed */

/* Stages of a call, for the optional per-stage timing hook below. */
typedef enum kda_stage {
    KDA_STAGE_CHUNK_TABLE = 0,  /* packed-batch chunk table (device cu_seqlens scan)          */
    KDA_STAGE_CHUNK_PREP = 1,   /* preprocess + intra-chunk solve, parallel over chunks
                                   (recurrent form: the per-token preprocess)                 */
    KDA_STAGE_CHUNK_SCAN = 2,   /* inter-chunk state propagation + chunk output, sequential
                                   (recurrent form: the token-by-token state scan)            */
    KDA_STAGE_CONV_STATE = 3,   /* conv history out                                           */
    KDA_STAGE_DECODE = 4,       /* the decode step kernel (also kda_decode_multi)             */
    KDA_STAGE_OUTPUT_GATE = 5,  /* the o_norm + sigmoid output-gate epilogue                  */
    KDA_STAGE_BACKWARD = 6,     /* the backward pass's kernels (after its chunk table)        */
    KDA_NUM_STAGES = 7
} kda_stage_t;

typedef struct kda_config {
    int32_t num_heads;        /* H                                                      */
    int32_t head_k_dim;       /* dk                                                     */
    int32_t head_v_dim;       /* dv (must equal dk)                                     */
    int32_t io_dtype;         /* kda_dtype_t of q, k, v, alpha, b, conv weights, conv history */
    int32_t out_dtype;        /* kda_dtype_t of o                                       */
    float scale;              /* multiplies the normalised q; 1.0 as on the pages       */
    float gate_lower_bound;   /* -5.0 (safe gate); any value, -INFINITY disabling the
                                 clamp.  It also picks the prefill's form: >= -5.4 the
                                 chunked form; below, the token-by-token recurrence
                                 (exact for any gate, ~2.3x slower; its workspace holds
                                 (4*dk + 4) fp32 per head and token).  With
                                 KDA_FLAG_RAW_GATE the bound is not applied to g but
                                 still picks the form: the chunked one needs every
                                 g >= -5.4                                            */
    float l2norm_eps;         /* q / sqrt(|q|^2 + eps); 1e-6                            */
    int32_t chunk_size;       /* 64                                                     */
    uint32_t flags;           /* KDA_FLAG_* test hooks, normally 0                      */
    const float *A_log;       /* [H] fp32, device                                       */
    const float *dt_bias;     /* [H*dk] fp32, device                                    */
    const void *conv_w_q;     /* [H*dk][4] io_dtype, device; tap 3 multiplies the current token */
    const void *conv_w_k;     /* [H*dk][4]                                              */
    const void *conv_w_v;     /* [H*dv][4]                                              */
    /* Optional timing hook, NULL for none: an array of 2*KDA_NUM_STAGES
     * hipEvent_t handles owned by the caller.  Entries 2*s and 2*s+1 (when
     * non-NULL) are recorded on the call's stream right before and right
     * after the launches of stage s. */
    void **stage_events;
} kda_config_t;

/* Library version, major*10000 + minor*100 + patch. */
int32_t kda_version(void);

/* Human-readable name of a status code (static storage). */
const char *kda_status_string(kda_status_t status);

/*
 * Workspace size in bytes for kda_prefill over B sequences of T tokens.
 * Returns 0 for an invalid or unsupported configuration.
 */
size_t kda_prefill_workspace_bytes(const kda_config_t *cfg, int32_t B, int32_t T);

/*
 * Chunked prefill of B equal-length sequences of T tokens.
 *   q, k           [B][T][H*dk]  io_dtype, raw projections (pre-conv)
 *   v              [B][T][H*dv]  io_dtype
 *   alpha          [B][T][H][dk] io_dtype, decay input
 *   b              [B][T][H]     io_dtype, pre-sigmoid write strength
 *   initial_state  [B][H][dk][dv] fp32, or NULL for zeros
 *   conv_state_in  [B][3][Ctot] io_dtype, oldest first, or NULL for zeros
 *   o              [B][T][H][dv] out_dtype (required)
 *   final_state    [B][H][dk][dv] fp32, or NULL; may alias initial_state
 *   conv_state_out [B][3][Ctot] io_dtype, or NULL; may alias conv_state_in
 *   workspace      device scratch of kda_prefill_workspace_bytes() for one pass
 *                  over the whole batch.  A smaller workspace runs the chunked
 *                  form (gate lower bound >= -5.4) in slabs: windows of the
 *                  longest multiple of 64 positions of every sequence whose
 *                  kda_prefill_slab_workspace_bytes() fits, one after the
 *                  other, with the state carried between them.  The results
 *                  are bit-identical to one pass.  KDA_ERR_WORKSPACE_TOO_SMALL
 *                  when not even a 64-token slab fits, or for the recurrent
 *                  form (bound below -5.4).  The per-stage timing events
 *                  (stage_events) are not recorded in slabs.
 * No other aliasing is allowed.
 */
kda_status_t kda_prefill(const kda_config_t *cfg, int32_t B, int32_t T,
                         const void *q, const void *k, const void *v,
                         const void *alpha, const void *b,
                         const float *initial_state, const void *conv_state_in,
                         void *o, float *final_state, void *conv_state_out,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace size in bytes for kda_varlen_prefill over N packed sequences
 * holding total_T tokens.  Returns 0 for an invalid configuration.
 */
size_t kda_varlen_workspace_bytes(const kda_config_t *cfg, int32_t N, int32_t total_T);

/*
 * Workspace size in bytes for the chunked prefill (kda_prefill with B = N, or
 * kda_varlen_prefill) run in slabs of slab_tokens positions per sequence
 * (rounded up to a multiple of 64): the chunk table and records of one slab
 * plus a carried state of [N][H][dk][dv] fp32.  It depends on neither T nor
 * total_T, which bounds the workspace of long prefills (4 x 32768 tokens at
 * H = 32, d = 128: 9.0 GiB in one pass, 2.3 GiB in slabs of 8192).  Returns 0
 * for an invalid configuration, N < 1, slab_tokens < 1 or a gate lower bound
 * below -5.4 (the recurrent form, which has no slabs).
 */
size_t kda_prefill_slab_workspace_bytes(const kda_config_t *cfg, int32_t N, int32_t slab_tokens);

/*
 * Chunked prefill of N sequences packed back to back (varlen).
 *   cu_seqlens     [N+1] int32, DEVICE; cu[0] = 0, cu[N] = total_T,
 *                  nondecreasing (zero-length sequences allowed).  The
 *                  library does not read it on the host; a malformed array
 *                  is undefined behaviour.
 *   q, k           [total_T][H*dk];  v [total_T][H*dv]
 *   alpha          [total_T][H][dk]; b [total_T][H]
 *   initial_state  [N][H][dk][dv] fp32 or NULL;  conv_state_in [N][3][Ctot] or NULL
 *   o              [total_T][H][dv]
 *   final_state    [N][H][dk][dv] or NULL;  conv_state_out [N][3][Ctot] or NULL
 * State and conv history restart at each sequence; chunks never straddle two
 * sequences.  Aliasing rules, and slabs for a smaller workspace, as for
 * kda_prefill (a slab is a window of positions of every sequence; the host
 * does not know the longest sequence, so it runs ceil(total_T / slab) of
 * them, the later ones empty for short sequences).
 */
kda_status_t kda_varlen_prefill(const kda_config_t *cfg, int32_t N, int32_t total_T,
                                const int32_t *cu_seqlens,
                                const void *q, const void *k, const void *v,
                                const void *alpha, const void *b,
                                const float *initial_state, const void *conv_state_in,
                                void *o, float *final_state, void *conv_state_out,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_varlen_prefill without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  The workspace is a fixed array of
 * KDA_NOALLOC_SCRATCH_BYTES in the library's device memory, one per GPU,
 * held from the first call on that GPU until the process ends; the call
 * allocates nothing.  Arguments, layouts and results as for
 * kda_varlen_prefill.
 *   - A batch whose workspace (kda_varlen_workspace_bytes) exceeds
 *     KDA_NOALLOC_SCRATCH_BYTES runs in slabs (as kda_varlen_prefill does
 *     with a small workspace); it is refused with KDA_ERR_WORKSPACE_TOO_SMALL,
 *     before any device call, when not even one slab of 64 tokens fits
 *     (kda_prefill_slab_workspace_bytes(cfg, N, 64) above the scratch: at
 *     H = 32, dk = dv = 128, bf16, 6.5 MB per sequence, a chunk's records for
 *     every head and the carried state, so N up to 39) or for the recurrent
 *     form.  One pass fits up to ~1800 (64-token chunk,
 *     head) pairs, e.g. 3 x 1024 tokens x 32 heads.
 *   - Every call on one GPU uses that GPU's single array: calls that overlap
 *     in time on one GPU (different streams, different threads) race and
 *     must be serialised by the caller.  Nothing from a previous call needs
 *     clearing: each call writes the scratch bytes it reads.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (256u << 20)

kda_status_t kda_varlen_prefill_noalloc(const kda_config_t *cfg, int32_t N, int32_t total_T,
                                        const int32_t *cu_seqlens,
                                        const void *q, const void *k, const void *v,
                                        const void *alpha, const void *b,
                                        const float *initial_state, const void *conv_state_in,
                                        void *o, float *final_state, void *conv_state_out,
                                        void *stream);

/*
 * Backward pass of kda_varlen_prefill: the gradient of a loss through o and
 * the final state with respect to every input and parameter (the models on
 * the Ling pages are trained natively with KDA layers; the pages give only
 * the forward, AliceAI page, section 二, whose reverse-mode derivative this
 * computes).  The forward is recomputed inside; nothing from a forward call
 * is needed.  Inputs are those of kda_varlen_prefill (same layouts, dtypes
 * and cu_seqlens rules) plus
 *   d_o            [total_T][H][dv] out_dtype: dLoss/do
 *   d_final_state  [N][H][dk][dv] fp32: dLoss/dfinal_state, or NULL (zero)
 * Outputs, all fp32 (every element written):
 *   dq, dk         [total_T][H*dk]   gradients of the raw (pre-conv) q, k
 *   dv             [total_T][H*dv]
 *   dalpha         [total_T][H][dk]  (0 where the safe gate clamped g)
 *   db             [total_T][H]
 *   d_initial_state [N][H][dk][dv], or NULL if not wanted
 *   d_conv_state_in [N][3][Ctot] gradient of the incoming conv history
 *                  (zeros when it was NULL), or NULL if not wanted
 *   dw_q, dw_k     [H*dk][4], dw_v [H*dv][4], ddt_bias [H*dk], dA_log [H]:
 *                  summed over all sequences of the batch
 * Supported: the chunked form's gates (gate_lower_bound >= -5.4) and
 * flags 0 or KDA_FLAG_BETA_X2; anything else is KDA_ERR_UNSUPPORTED.  The
 * workspace (kda_varlen_backward_workspace_bytes) holds per 16-token block
 * and head about 2 dk dv + 6 * 16 dk floats (~170 KB at dk = dv = 128).
 * Timing stages: KDA_STAGE_CHUNK_TABLE, then KDA_STAGE_BACKWARD.
 */
size_t kda_varlen_backward_workspace_bytes(const kda_config_t *cfg, int32_t N, int32_t total_T);

kda_status_t kda_varlen_backward(const kda_config_t *cfg, int32_t N, int32_t total_T,
                                 const int32_t *cu_seqlens,
                                 const void *q, const void *k, const void *v,
                                 const void *alpha, const void *b,
                                 const float *initial_state, const void *conv_state_in,
                                 const void *d_o, const float *d_final_state,
                                 float *dq, float *dk, float *dv, float *dalpha, float *db,
                                 float *d_initial_state, float *d_conv_state_in,
                                 float *dw_q, float *dw_k, float *dw_v, float *ddt_bias, float *dA_log,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step: one new token for each of N independent sequences
 * (the fused recurrent form; AliceAI page, section 五).
 *   q, k           [N][H*dk] io_dtype;  v [N][H*dv]
 *   alpha          [N][H][dk];          b [N][H]
 *   state          [N][H][dk][dv] fp32, read and updated in place (required)
 *   conv_state     [N][3][Ctot] io_dtype, read and shifted in place (required)
 *   o              [N][H][dv] out_dtype
 * Needs no workspace.
 */
kda_status_t kda_decode_step(const kda_config_t *cfg, int32_t N,
                             const void *q, const void *k, const void *v,
                             const void *alpha, const void *b,
                             float *state, void *conv_state, void *o, void *stream);

/*
 * Serving decode: K tokens for each of N sequences whose state and conv
 * history live in caller-owned pools (AliceAI page, section 五: the
 * recurrent state and the conv states are what decode carries; section 六:
 * speculative decoding with MTP drafts one extra token per forward, whose
 * outputs a verify pass needs before the accepted tokens are kept).
 *   slots          [N] int32, device: the pool row of each sequence; a
 *                  negative slot skips the sequence (its outputs are not
 *                  written).  NULL: sequence n uses row n.  Slots of one call
 *                  must be distinct.
 *   q, k           [N][K][H*dk]  io_dtype     v [N][K][H*dv]
 *   alpha          [N][K][H][dk] io_dtype     b [N][K][H]
 *   state_pool     [P][H][dk][dv] fp32, device (P > every slot)
 *   conv_pool      [P][3][Ctot] io_dtype, raw-input history, oldest first
 *   o              [N][K][H][dv] out_dtype: the outputs of all K tokens,
 *                  each reading the state updated by the tokens before it
 *   n_commit       [N] int32, device: keep the updates of the first
 *                  n_commit[n] tokens (clamped to 0..K): the pools receive
 *                  the state and conv history after them.  0 leaves the
 *                  pools untouched (a verify pass); NULL keeps all K.
 * The state is read once and written at most once per call, so K tokens cost
 * about the HBM traffic of one decode step.  A rejected draft is rolled back
 * by committing fewer tokens, e.g. a verify call with n_commit = 0 and then a
 * call over the accepted tokens only.  K in 1..64.  Needs no workspace.
 */
kda_status_t kda_decode_multi(const kda_config_t *cfg, int32_t N, int32_t K, const int32_t *slots,
                              const void *q, const void *k, const void *v,
                              const void *alpha, const void *b,
                              float *state_pool, void *conv_pool, void *o,
                              const int32_t *n_commit, void *stream);

/*
 * kda_decode_step and kda_decode_multi with the layer's output epilogue
 * (kda_output_gate below) fused into the step: each (sequence, head)
 * workgroup holds the whole row of dv outputs, so the row is normalised and
 * gated before it is stored and o never goes to memory
 * (AliceAI page, section 三: KDA's output goes through o_norm and a sigmoid
 * gate).  Arguments as for the plain calls, plus:
 *   gate           the output-gate projection before the sigmoid, io_dtype,
 *                  laid out like o: [N][H][dv] (step), [N][K][H][dv] (multi)
 *   o_norm_weight  [dv] fp32, one weight per channel shared by the heads
 *   eps            o_norm epsilon, >= 0 (NaN or negative, or a NULL gate or
 *                  weight: KDA_ERR_INVALID_ARGUMENT)
 *   y              out_dtype, in place of o: y = o / sqrt(mean(o^2) + eps)
 *                  * o_norm_weight * sigmoid(gate), per (token, head) row
 * The state and conv history are updated exactly as by the plain calls.
 */
kda_status_t kda_decode_step_gated(const kda_config_t *cfg, int32_t N,
                                   const void *q, const void *k, const void *v,
                                   const void *alpha, const void *b,
                                   float *state, void *conv_state,
                                   const void *gate, const float *o_norm_weight, float eps,
                                   void *y, void *stream);

kda_status_t kda_decode_multi_gated(const kda_config_t *cfg, int32_t N, int32_t K, const int32_t *slots,
                                    const void *q, const void *k, const void *v,
                                    const void *alpha, const void *b,
                                    float *state_pool, void *conv_pool,
                                    const void *gate, const float *o_norm_weight, float eps,
                                    void *y, const int32_t *n_commit, void *stream);

/*
 * The layer's output epilogue on n_tokens x H rows of dv outputs (AliceAI
 * page, section 三: KDA's output goes through o_norm and a sigmoid gate;
 * section 二: output_gate is one of the per-token control inputs):
 *   y[t][h][j] = o[t][h][j] / sqrt(mean_j' o[t][h][j']^2 + eps)
 *                * o_norm_weight[j] * sigmoid(gate[t][h][j])
 * The pages give neither the norm's epsilon nor its weight's shape: o_norm
 * is read as an RMS norm over one head's dv outputs with one weight per
 * channel shared by the heads (eps 1e-6 in the reference setting).
 *   o              [n_tokens][H][dv] out_dtype, as written by the calls above
 *   gate           [n_tokens][H][dv] io_dtype, the output-gate projection
 *                  before the sigmoid
 *   o_norm_weight  [dv] fp32
 *   eps            >= 0 (NaN or negative: KDA_ERR_INVALID_ARGUMENT)
 *   y              [n_tokens][H][dv] out_dtype; may alias o (in place)
 * Only num_heads, head_v_dim, io_dtype, out_dtype and stage_events of cfg
 * are used.  Needs no workspace.  n_tokens == 0 is a no-op.
 */
kda_status_t kda_output_gate(const kda_config_t *cfg, int64_t n_tokens,
                             const void *o, const void *gate,
                             const float *o_norm_weight, float eps,
                             void *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
