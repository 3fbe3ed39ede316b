/*
 * gqla.h - C ABI of libgqla, MI355X (gfx950) GQLA decode attention.
 *
 * Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
 * Decoding" (gist.science explainer page), technical summary section 2
 * (Methodology: Architecture, Path selection) and section 1 (Problem).
 *
 * GQLA keeps, per cached token t, one latent row c_t (width r_kv) and one
 * shared rotary key k_R,t (width d_r), and g group-indexed up-projections
 * W_UK[j], W_UV[j] (each d_h x r_kv).  Query head i (of h_q) belongs to group
 * j(i) = i / (h_q / g).  Its key for token t is [W_UK[j] c_t | k_R,t] and its
 * value W_UV[j] c_t.  Two algebraically equal decode paths read this:
 *   - MQA-absorb (section 2, memory-friendly path): W_UK is folded into the
 *     query and W_UV applied after attention; every head attends to the
 *     shared latent rows [c_t | k_R,t] (gqla_decode_absorb);
 *   - GQA (section 2, compute-friendly path): the latent is expanded once into
 *     g groups of K/V (gqla_expand_groups), and decode runs ordinary grouped
 *     attention over the expanded rows (gqla_decode_gqa).
 * Each step reads the whole cached history (section 1).  With s_q query
 * tokens per step (multi-token prediction, section 2 Path selection) the s_q
 * new tokens are the last s_q cached rows of the sequence and query s sees
 * rows t <= L_b - s_q + s.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers, owned by the caller, in the
 *     dtype of shape->dtype (bf16 or fp32; one dtype per call), row-major.
 *     ctx_lens is a device int32[batch].  The library allocates nothing.  Its
 *     state: a per-device cache of the compute-unit count; per thread, the last
 *     error message and the optional timing events of gqla_set_kernel_events;
 *     and the static device scratch of gqla_decode_gqa_noalloc (one copy per
 *     device, with its address looked up once per device).
 *   - q_rope and the k_R columns of the cache hold keys/queries with the
 *     rotary embedding already applied.
 *   - Operand range (bf16 storage): some products run on fp16 copies of the bf16
 *     inputs: the value columns V_j of the GQA and sparse decodes, their queries and
 *     key columns (k_R included) too in the kernels that some shapes select, and the
 *     latent rows c_t in the absorb decode's weighted sum u.  Values whose
 *     magnitude lies in fp16's normal range [2^-14, 65504] are converted exactly;
 *     smaller magnitudes keep fp16's subnormal spacing 2^-24 (an absolute error of at
 *     most 2^-24 per element); magnitudes above 65504 are outside the supported range
 *     (they saturate).  The absorb decode's scores, W_UK and W_UV, and the group
 *     expansion use the bf16 values as given.
 *   - stream is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work on it and never synchronise; results are ready when the stream is.
 *   - Arguments are validated on the host before any launch; a failed check
 *     returns a non-zero status and enqueues nothing.  gqla_last_error()
 *     then names the offending argument.  Launch failures map to GQLA_ERR_HIP.
 *   - ctx_lens contents are not read on the host.  Kernels clamp L_b to
 *     [0, max_ctx]; a query that sees no row returns o = 0, lse = -inf.
 *   - Thread safety: calls are reentrant; concurrent calls must use distinct
 *     workspaces (gqla_decode_gqa_noalloc: see its note on overlapping calls).
 */
#ifndef GQLA_H
#define GQLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqla_status {
    GQLA_OK = 0,
    GQLA_ERR_INVALID_ARG = 1,   /* null pointer, bad size/stride/alignment, h_q % g != 0, ... */
    GQLA_ERR_UNSUPPORTED = 2,   /* valid but not built: dims or group layout without a kernel */
    GQLA_ERR_WORKSPACE = 3,     /* workspace null or smaller than gqla_workspace_size() */
    GQLA_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} gqla_status;

typedef enum gqla_dtype { GQLA_BF16 = 0, GQLA_F32 = 1 } gqla_dtype;
typedef enum gqla_path { GQLA_PATH_ABSORB = 0, GQLA_PATH_GQA = 1, GQLA_PATH_SPARSE = 2 } gqla_path;

/* Model and step shape (section 2, Architecture): h_q query heads, g groups,
 * latent width r_kv, rotary key width d_r, per-group head width d_h, s_q query
 * tokens per step (1..4), softmax scale applied to q.k, storage dtype.
 * Kernels built: bf16 with r_kv=512, d_r=64, d_h=128 (MFMA path); fp32 with
 * r_kv <= 1024, d_r <= 256, d_h <= 256 (vector path). */
typedef struct gqla_shape {
    int32_t h_q, g, r_kv, d_r, d_h, s_q;
    float scale;
    int32_t dtype;              /* gqla_dtype */
} gqla_shape;

/* Bytes of device workspace a decode call needs (split-K partials, and for the
 * bf16 absorb path one absorbed-query record per query row and a copy of W_UV,
 * g * d_h * r_kv elements, rewritten by every call in the order its kernel reads it).  num_splits: 0 = automatic, else an upper
 * bound on context chunks per sequence.  For GQLA_PATH_SPARSE the max_ctx argument
 * is the index-list length topk (the chunks split the list).  Returns GQLA_OK and
 * writes *bytes. */
gqla_status gqla_workspace_size(const gqla_shape* shape, int32_t path, int32_t batch,
                                int32_t max_ctx, int32_t num_splits, size_t* bytes);

/* Number of context chunks per sequence and chunk length (tokens) that a decode
 * call with these arguments uses.  Host-only; for planning and tests. */
gqla_status gqla_plan_splits(const gqla_shape* shape, int32_t path, int32_t batch,
                             int32_t max_ctx, int32_t num_splits,
                             int32_t* n_split, int32_t* chunk);

/* Split-K planning from context lengths the caller holds on the host (a serving
 * scheduler usually does), for when the automatic rule, which sees only max_ctx,
 * leaves compute units idle or runs a second, mostly empty round of chunks: few long
 * ragged sequences, for instance.  The pages do not describe the split-K partition
 * (it is this library's way of spreading one sequence's context over compute units);
 * this call only chooses how finely the decode calls cut it.
 *   host_ctx_lens [batch] host memory, read only (values clamped to [0, max_ctx]).
 * Writes *num_splits, the value to pass as num_splits to gqla_workspace_size and the
 * decode call of the same shape, path, batch and max_ctx, and the *n_split and
 * *chunk that call then uses.  bf16 absorb and GQA paths: when the automatic plan
 * needs fewer than four rounds of workgroups on the device, the automatic plan and the
 * plans whose grid is exactly 1-4 rounds are compared by the estimate
 * rounds x (chunk + a fixed per-workgroup overhead), and a plan with more chunks wins
 * only when it is estimated 10 % faster; otherwise, and for other paths and dtypes, the
 * automatic plan (*num_splits = 0).  Host-only, O(batch).  Errors:
 * GQLA_ERR_INVALID_ARG on null pointers or invalid shape or sizes. */
gqla_status gqla_plan_splits_lens(const gqla_shape* shape, int32_t path, int32_t batch,
                                  int32_t max_ctx, const int32_t* host_ctx_lens,
                                  int32_t* num_splits, int32_t* n_split, int32_t* chunk);

/* Expand latent rows once into g groups of K and V (section 2, GQA path: the
 * latent is expanded into g K/V groups so decode need not re-expand it each step).
 *   latent      [batch][latent_bstride] elements; sequence b's row t starts at
 *               latent + b*latent_bstride + t*(r_kv+d_r) and is [c_t | k_R,t].
 *   w_uk, w_uv  [g][d_h][r_kv].
 *   group_cache [batch][group_bstride]; row t of sequence b (width 2 g d_h + d_r)
 *               is written as [W_UK[0]c_t .. W_UK[g-1]c_t | W_UV[0]c_t .. W_UV[g-1]c_t | k_R,t],
 *               for row_begin <= t < L_b only (other rows are not touched).
 *   Products accumulate in fp32 and are rounded once (RNE) to the dtype.
 *   Strides are in elements, multiples of 8, and at least max_ctx * row width. */
gqla_status gqla_expand_groups(const gqla_shape* shape, int32_t batch, int32_t max_ctx,
                               const void* latent, int64_t latent_bstride,
                               const void* w_uk, const void* w_uv,
                               const int32_t* ctx_lens, int32_t row_begin,
                               void* group_cache, int64_t group_bstride, void* stream);

/* MQA-absorb decode (section 2, memory-friendly path: the MLA form with group-indexed
 * up-projections): q~ = W_UK[j]^T q_nope per head, scores
 * s_t = scale [q~ | q_rope].[c_t | k_R,t], u = softmax-weighted sum of c_t,
 * o = W_UV[j] u.  The absorbed query is carried as a bf16 pair (about 16 significant
 * bits) against the latent rows as stored, so the result keeps the bf16 tolerance
 * however peaked the softmax is.
 *   q_nope [batch][s_q][h_q][d_h], q_rope [batch][s_q][h_q][d_r]
 *   w_uk, w_uv [g][d_h][r_kv]; latent as in gqla_expand_groups
 *   out [batch][s_q][h_q][d_h] (dtype); lse (nullable) fp32 [batch][s_q][h_q],
 *   natural-log log-sum-exp of the scaled scores.
 * Context is split into chunks (split-K); per-chunk partials in the workspace
 * are merged by their log-sum-exp. */
gqla_status gqla_decode_absorb(const gqla_shape* shape, int32_t batch, int32_t max_ctx,
                               const void* q_nope, const void* q_rope,
                               const void* w_uk, const void* w_uv,
                               const void* latent, int64_t latent_bstride,
                               const int32_t* ctx_lens, void* out, float* lse,
                               void* workspace, size_t workspace_bytes,
                               int32_t num_splits, void* stream);

/* GQA decode over expanded rows (section 2, compute-friendly path): head i of
 * group j scores [q_nope | q_rope].[K_j,t | k_R,t] and averages V_j,t.
 *   group_cache as written by gqla_expand_groups; other arguments as in
 *   gqla_decode_absorb. */
gqla_status gqla_decode_gqa(const gqla_shape* shape, int32_t batch, int32_t max_ctx,
                            const void* q_nope, const void* q_rope,
                            const void* group_cache, int64_t group_bstride,
                            const int32_t* ctx_lens, void* out, float* lse,
                            void* workspace, size_t workspace_bytes,
                            int32_t num_splits, void* stream);

/* Largest scratch, in bytes, that gqla_decode_gqa_noalloc may use (64 MiB). */
#define GQLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* gqla_decode_gqa for callers that cannot allocate device memory or pass a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same kernels, same split plan and bit-identical results as gqla_decode_gqa with the
 * same arguments, but the split-K partials live in a static device array of
 * GQLA_NOALLOC_SCRATCH_BYTES compiled into the library instead of a caller workspace.
 *   - The call allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   - It runs on the current device.  Each device the library runs on holds its own
 *     copy of the array until the process ends; the first call on a device looks up
 *     that copy's address (hipGetSymbolAddress) with the device current.
 *   - All calls on one device share its array, which keeps the last call's contents.
 *     Calls ordered on one stream are safe; calls that overlap on one device (two
 *     streams, or two threads without ordering between them) race, and their results
 *     are undefined.  Nothing in the array needs clearing: every partial the split-K
 *     merge reads is written earlier by the same call.
 *   - Errors: those of gqla_decode_gqa, and GQLA_ERR_WORKSPACE when the call needs more
 *     than GQLA_NOALLOC_SCRATCH_BYTES (gqla_workspace_size with GQLA_PATH_GQA and the
 *     same arguments gives the need); such a call enqueues nothing.  Fewer sequences
 *     per call or a smaller num_splits lower the need. */
gqla_status gqla_decode_gqa_noalloc(const gqla_shape* shape, int32_t batch, int32_t max_ctx,
                                    const void* q_nope, const void* q_rope,
                                    const void* group_cache, int64_t group_bstride,
                                    const int32_t* ctx_lens, void* out, float* lse,
                                    int32_t num_splits, void* stream);

/* Sparse GQLA decode (section 2, Sparse GQLA: fine-grained sparse attention keeps the
 * GQA path, since a group's h_q/g = 16 heads fill one 16-row matrix tile).  Query
 * token s of every head of group j attends only to the rows listed in
 * indices[b][s][j][0..topk) of the expanded cache; entries outside [0, L_b) or past
 * the token's causal window t <= L_b - s_q + s are skipped (-1 pads a short list), and
 * a row listed twice counts twice.  With no usable entry o = 0 and lse = -inf.
 *   indices  device int32 [batch][s_q][g][topk]; topk >= 0
 *   workspace: gqla_workspace_size(shape, GQLA_PATH_SPARSE, batch, topk, num_splits)
 *   other arguments as in gqla_decode_gqa.  Any g dividing h_q is accepted. */
gqla_status gqla_decode_gqa_sparse(const gqla_shape* shape, int32_t batch, int32_t max_ctx,
                                   const void* q_nope, const void* q_rope,
                                   const void* group_cache, int64_t group_bstride,
                                   const int32_t* ctx_lens, const int32_t* indices, int32_t topk,
                                   void* out, float* lse, void* workspace, size_t workspace_bytes,
                                   int32_t num_splits, void* stream);

/* Decode-step append (the step that feeds both decode paths; section 2,
 * Architecture: one latent row and one shared rotary key per token, a rotary query
 * part per head).  For every sequence b and new token s < s_q, at position
 * t = L_b - s_q + s (L_b = ctx_lens[b] clamped to [0, max_ctx], the new tokens
 * included; tokens with t < 0 are skipped):
 *   latent[b][t]        = [c_new[b][s] | RoPE_t(kr_new[b][s])]
 *   q_rope_out[b][s][h] = RoPE_t(q_rope_raw[b][s][h])          (when q_rope_raw != NULL)
 *   group_cache[b][t]   = the expansion of latent[b][t] as in gqla_expand_groups
 *                                                                (when group_cache != NULL)
 * RoPE pairs component k < d_r/2 with k + d_r/2 and turns the pair by the angle
 * t * rope_theta^(-2k/d_r) (x' = x cos - y sin, y' = x sin + y cos).  Angles and
 * rotated values are computed in fp64 and rounded once to fp32, then for bf16 to bf16
 * (round to nearest even); the expansion accumulates in fp32 (RNE to the dtype).
 *   c_new       [batch][s_q][r_kv]        new latent rows
 *   kr_new      [batch][s_q][d_r]         new rotary keys before rotation
 *   q_rope_raw  [batch][s_q][h_q][d_r]    rotary query parts before rotation, or NULL
 *   q_rope_out  same shape; NULL exactly when q_rope_raw is NULL (may not alias it)
 *   latent, latent_bstride                as in gqla_expand_groups (rows written)
 *   w_uk, w_uv  [g][d_h][r_kv], required when group_cache is not NULL
 *   rope_theta  rotary base, finite and > 0 (10000 in the workloads); d_r must be even.
 * Only the rows and entries listed are written. */
gqla_status gqla_append_rows(const gqla_shape* shape, int32_t batch, int32_t max_ctx,
                             const void* c_new, const void* kr_new,
                             const void* q_rope_raw, void* q_rope_out, float rope_theta,
                             const int32_t* ctx_lens,
                             void* latent, int64_t latent_bstride,
                             const void* w_uk, const void* w_uv,
                             void* group_cache, int64_t group_bstride, void* stream);

/* Roofline path selection (section 2, Path selection: the runtime picks the decode
 * path per device without retraining; section 1 gives the two devices' ridges).
 * For path in {absorb, GQA} and s_q in 1..shape->s_q (the most query tokens the model
 * proposes per step), a decode step over contexts summing to total_ctx takes
 * max(bytes / peak_bytes_per_s, flops / peak_flops) with, per cached token,
 *   absorb: bytes e (r_kv + d_r),     flops 2 s_q h_q (2 r_kv + d_r)
 *   GQA:    bytes e (2 g d_h + d_r),  flops 2 s_q h_q (2 d_h + d_r)
 * (e = 2 for bf16, 4 for fp32) and yields batch * s_q query tokens.  The choice is the
 * configuration with the most query tokens per second; on a tie the smaller s_q, then
 * the absorb path.  Host-only arithmetic: any device's peaks may be given (for this
 * one, gqla_measure_peaks measures them).  g is a property of the weights and is taken
 * from the shape. */
typedef struct gqla_path_choice {
    int32_t path;               /* gqla_path */
    int32_t s_q;                /* query tokens per step */
    int32_t compute_bound;      /* 1: the flops term sets the step time */
    int32_t reserved;           /* 0 */
    double tokens_per_s;        /* roofline query tokens per second */
} gqla_path_choice;

gqla_status gqla_select_path(const gqla_shape* shape, int32_t batch, int64_t total_ctx,
                             double peak_flops, double peak_bytes_per_s,
                             gqla_path_choice* choice);

/* Measure this device's achievable HBM read bandwidth (one streaming pass over the
 * scratch buffer, best of three after a warm-up pass) and dense bf16 MFMA rate (four
 * independent 16x16x32 chains per wave, 32 waves per compute unit), for
 * gqla_select_path.  scratch: device buffer of at least 64 MiB, 16-byte aligned, owned
 * by the caller; its contents are overwritten.  A buffer well above the last-level
 * cache (1 GiB or more on MI355X) measures HBM rather than cache.  Unlike the other
 * calls this one waits for its kernels: it returns when both measurements are done. */
gqla_status gqla_measure_peaks(void* scratch, size_t scratch_bytes, double* bytes_per_s,
                               double* flops_per_s, void* stream);

/* Timing hook for measurement tools.  When both are non-NULL, every later decode
 * call on this thread records `before` (a hipEvent_t) on its stream right before
 * launching its main attention kernel and `after` right after it, so that
 * hipEventElapsedTime(before, after) is that kernel's duration.  The absorb
 * prologue and the split-K combine fall outside the pair.  NULL, NULL turns it
 * off.  The events are the caller's; the library only records them. */
gqla_status gqla_set_kernel_events(void* before, void* after);

/* Static description of a status code. */
const char* gqla_status_string(gqla_status status);

/* Message of the last failed call on this thread ("" if none). */
const char* gqla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GQLA_H */
