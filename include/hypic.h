/*
 * hypic.h -- C ABI of libhypic: linear-attention state composition for
 * position-independent caching, on AMD MI355X (gfx950).
 *
 * Sources (the HYPIC pages):
 *   [news]   HYPIC news article, news.aibase.com/tw/news/29683
 *   [readme] HYPIC project README ("PIC modes", "Key techniques")
 *   [arxiv]  abstract of arXiv 2607.01299
 *
 * Conventions used by every call
 *   - A chain is one (layer, value-head) recurrence.  Its state S is d_k x d_v,
 *     a transition T is d_k x d_k and acts from the left: composing segment C1
 *     and then C2 gives S(C1.C2) = T(C2) S(C1) + S(C2) ([news], paragraph on
 *     linear layers and the cached transition operator).
 *   - Dense kind, the gated delta rule (Yang, Kautz & Hatamizadeh, ICLR 2025):
 *       S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *     the write not decayed at its own step; DeltaNet is log_alpha == 0.
 *     Diagonal kind (GLA):  S_t = diag(alpha_t) S_{t-1} + k_t v_t^T.
 *     Scalar kind (RetNet gamma, Mamba2): S_t = alpha_t S_{t-1} + k_t v_t^T.
 *     These are the decaying families [news] names in the same paragraph.
 *   - Per-token output o_t = S_t^T q_t, with S_t the state after token t.
 *     No 1/sqrt(d) scale is applied: the caller pre-scales q.
 *   - T is returned as T_hat * 2^T_exp: T_hat float32 with one int32 exponent
 *     per (segment, chain), because the product of hundreds of decaying
 *     transitions leaves float32's range.  The pair is not unique; only the
 *     represented value is meaningful.
 *   - Grouped-query attention: value head h reads key/query head
 *     floor(h * h_k / h_v).  log_alpha and beta are per value head.
 *   - All tensors are dense, C-contiguous, caller-owned DEVICE memory unless
 *     marked "host".  Layouts are given per field.  The library never
 *     allocates device memory and keeps no pointer after a call returns.
 *   - Every call validates all arguments on the host BEFORE any HIP call.  On
 *     failure nothing is enqueued, the call returns a status != HYPIC_OK and
 *     hypic_last_error() (thread-local) describes the problem.  A launch
 *     failure returns HYPIC_ERR_DEVICE.  Device faults surface at the caller's
 *     next synchronisation.  Every call enqueues its work on `stream` (NULL =
 *     the null stream) and host arrays may be freed when the call returns.
 *     The host segment table (cu_seqlens / cu_seam) of at most 160 segments
 *     travels inside the kernel arguments: such a call copies nothing, needs no
 *     workspace and returns without waiting for the device.  A larger table is
 *     uploaded into the call's workspace by a copy from pageable host memory,
 *     which blocks the calling thread until the runtime has staged it.
 *   - NaN/Inf inputs propagate; they are not checked.
 *   - f16 operand range (the dense kind under HYPIC_PREC_F16, which AUTO picks
 *     for bf16 inputs, and the diagonal/scalar build with bf16 inputs): v, S
 *     and the chunk intermediates enter the matrix cores as f16, so |v| and |S|
 *     must stay below 2^15 (the largest f16 is 65504) and values below 2^-14
 *     lose relative precision (f16 subnormals; zero below 2^-25).  k is
 *     expected L2-normalised (|k| <= 1).  T is renormalised by powers of two and
 *     has no range limit.  S and o are linear in v, so a caller with v outside
 *     this range scales v by a power of two and S and o back.
 *   - Supported shapes: d_k == d_v in {64, 128}; chunk == 64; conv width 4.
 *     Anything else returns HYPIC_ERR_UNSUPPORTED.
 *   - Outputs are bitwise reproducible run to run and independent of the
 *     schedule (no atomics in any reduction).
 */
#ifndef HYPIC_H
#define HYPIC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYPIC_VERSION 1

typedef struct ihipStream_t* hypic_stream_t; /* a hipStream_t */

typedef enum {
    HYPIC_OK = 0,
    HYPIC_ERR_INVALID_ARGUMENT = 1,
    HYPIC_ERR_UNSUPPORTED = 2,
    HYPIC_ERR_WORKSPACE_TOO_SMALL = 3,
    HYPIC_ERR_DEVICE = 4
} hypic_status;

/* element type of q/k/v (inputs) and of o / conv outputs */
typedef enum { HYPIC_F32 = 0, HYPIC_BF16 = 1 } hypic_dtype;

typedef enum {
    HYPIC_DENSE_DELTA = 0, /* A_t = alpha_t (I - beta_t k_t k_t^T)  (GDN, DeltaNet) */
    HYPIC_DIAG = 1,        /* A_t = diag(alpha_t)                   (GLA)          */
    HYPIC_SCALAR = 2,      /* A_t = alpha_t I                       (RetNet, Mamba2) */
    HYPIC_KDA = 3          /* A_t = diag(alpha_t) (I - beta_t k_t k_t^T), alpha_t per
                              channel (KDA); T is a dense d_k x d_k matrix, so KDA
                              elements compose exactly like HYPIC_DENSE_DELTA ones     */
} hypic_kind;

/* Order in which (segment, chain) build tasks are handed to the compute units.
 * Segment parallelism with longest-processing-time-first balancing is the
 * [news] paragraph on segment parallelism; here the workers are the GPU's
 * compute units instead of serving instances. */
typedef enum {
    HYPIC_SCHED_NATURAL = 0, /* segment-major task order, hardware dispatch          */
    HYPIC_SCHED_LPT = 1,     /* longest segments first, hardware dispatch (greedy list
                                scheduling = LPT)                                     */
    HYPIC_SCHED_RR = 2       /* persistent workgroups, task i -> slot i mod n_slots   */
} hypic_schedule;

/* Operand precision of the dense kind's matrix-core products (the segment build
 * and seams longer than 16 tokens; shorter seams always run in float32 vector
 * arithmetic).  Accumulation is always float32.  Per-segment relative errors,
 * bf16 inputs, d = 128: F16 about 8e-4 (T) and 3e-4 (S) at 1,024 tokens, T growing
 * like the square root of the chunk count; AUTO switches the T columns of segments
 * longer than 2,048 tokens to hi/lo X and Vn operands (T about 1.1e-3 at 8k tokens).
 *   AUTO: F16 for bf16 inputs; F32 for float32 inputs at d = 64.  There is no
 *         float32-operand plan at d = 128, so float32 inputs at d = 128 return
 *         HYPIC_ERR_UNSUPPORTED under AUTO; ask for F16 explicitly to accept f16
 *         operands (relative error about 1e-3 instead of about 1e-6). */
typedef enum {
    HYPIC_PREC_AUTO = 0,
    HYPIC_PREC_F32 = 1, /* float32 operands (fp32 matrix cores), for fp32 inputs   */
    HYPIC_PREC_F16 = 2, /* f16 operands, power-of-two renormalised T columns        */
    /* Segment build only (a seam takes it as F16).  S as under F16; T from a separate
     * transition-only pass with hi/lo-split f16 operands (about 22-bit) on every
     * product that touches it.  Per-segment T error about 1e-5 instead of about
     * 1e-3, so that the product of many cached transitions (hypic_compose's T_total)
     * stays within 2e-3; costs a second pass over k.  Keys are still rounded to f16
     * once, which is exact for bf16 keys of magnitude >= 2^-14. */
    HYPIC_PREC_F16_PRECISE_T = 3
} hypic_precision;

typedef enum {
    HYPIC_COMPOSE_AUTO = 0,     /* FOLD or SCAN (and its block) by a cost model     */
    HYPIC_COMPOSE_FOLD = 1,     /* sequential S <- T_i S + S_i per chain            */
    HYPIC_COMPOSE_SCAN = 2,     /* blocked reduce, scan of block aggregates, re-fold */
    HYPIC_COMPOSE_NAIVE_ADD = 3 /* S <- S + S_i: the "addition" PIC mode of [readme],
                                   exact only without decay ([news])               */
} hypic_compose_mode;

typedef enum { HYPIC_ACT_NONE = 0, HYPIC_ACT_SILU = 1 } hypic_activation;

/* ------------------------------------------------------------------------------------
 * hypic_segment_build -- per-segment transition T_C and zero-start end state S(C|0).
 *
 * [news], linear-layer paragraph: both depend only on the segment's own
 * tokens, so they are computed once when the segment is first prefilled and
 * cached.  T_C is the ordered product of the segment's per-token transitions;
 * S(C|0) is the state after the segment from S = 0.  The dense kind uses the
 * chunked WY/UT form of the gated delta rule with T carried as extra state
 * columns; the diagonal and scalar kinds use their closed forms; KDA runs its
 * token recurrence in float32 vector arithmetic, one thread per column of [T | S]
 * (whatever precision is asked for; no qk_l2norm, no outputs, no RR schedule).
 *
 * Segment s covers tokens [cu_seqlens[s] + skip_head, cu_seqlens[s+1]) of the
 * packed token axis (skip_head >= 0 leaves the seam window out of the cache
 * entry; a segment no longer than skip_head is empty: T = I, S = 0).
 *
 * Layouts (B = n_batch, typically layers; N = n_tokens):
 *   k           [B, N, h_k, d_k]   in_dtype
 *   v           [B, N, h_v, d_v]   in_dtype
 *   log_alpha   float32, <= 0: DENSE/SCALAR [B, N, h_v]; DIAG/KDA [B, N, h_v, d_k]
 *   beta        float32 [B, N, h_v] (DENSE and KDA; must be NULL otherwise)
 *   T_hat       float32 (NULL = skip T, plain state pass):
 *                 DENSE/KDA [n_seg, B, h_v, d_k, d_k]; DIAG [n_seg, B, h_v, d_k];
 *                 SCALAR [n_seg, B, h_v]
 *   T_exp       int32 [n_seg, B, h_v] (required iff T_hat)
 *   S           float32 [n_seg, B, h_v, d_k, d_v]
 * Outputs are segment-major so that they serve directly as the element store
 * of hypic_compose (slot = segment, chain = b * h_v + h).
 * Workspace: hypic_segment_build_workspace_bytes() bytes of device memory,
 * 256-byte aligned, untouched until the call's work on `stream` has finished;
 * 0 (workspace may be NULL) for at most 160 segments.
 * ---------------------------------------------------------------------------------- */
typedef struct {
    hypic_kind kind;
    hypic_dtype in_dtype;
    int32_t n_batch;
    int64_t n_tokens;
    int32_t h_k, h_v, d_k, d_v;
    int32_t chunk;              /* must be 64 */
    int32_t n_seg;
    const int64_t* cu_seqlens;  /* host [n_seg + 1], cu[0] = 0, non-decreasing, cu[n_seg] <= N */
    int32_t skip_head;          /* >= 0 */
    int32_t qk_l2norm;          /* 1: k (and q, with outputs) scaled to unit L2 norm per token
                                   and head on load */
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    float* T_hat;
    int32_t* T_exp;
    float* S;
    hypic_schedule schedule;
    hypic_precision precision;
    void* workspace;
    size_t workspace_bytes;
    /* Output-fused build (dense kind): with o != NULL every covered token t of a
     * segment also gets o_t = S_t^T q_t, S_t the segment's zero-start state after
     * token t -- the segment's own prefill outputs, with T and S(C|0) as side
     * outputs.  q [B, N, h_k, d_k] in_dtype; o [B, N, h_v, d_v] out_dtype (tokens
     * outside the covered ranges are not written).  With 16-bit inputs under the
     * f16 plans it runs on the segment-build engine: with T_hat, a transition-only
     * pass (f16 operands; hi/lo under HYPIC_PREC_F16_PRECISE_T or for segments longer
     * than 2,048 tokens) followed by the state pass with outputs.  Float32 inputs or
     * operands run the general chunk engine (one workgroup per (segment, chain)). */
    const void* q;
    void* o;
    hypic_dtype out_dtype;
} hypic_build_desc;

hypic_status hypic_segment_build(const hypic_build_desc* desc, hypic_stream_t stream);
size_t hypic_segment_build_workspace_bytes(const hypic_build_desc* desc);

/* ------------------------------------------------------------------------------------
 * hypic_compose -- constant-time composition of cached segments.
 *
 * [news], linear-layer paragraph: on reuse the running state is left-
 * multiplied by the cached T_C and the cached S(C|0) added, in request order:
 *   S <- T_{slot[i]} S + S_{slot[i]},  i = 0 .. n_elem-1,  starting from S0.
 * FOLD runs this sequentially per chain; SCAN uses the associative operator
 * (T2,S2) o (T1,S1) = (T2 T1, T2 S1 + S2) with identity (I, 0) in a blocked
 * reduce / scan / re-fold.  NAIVE_ADD is the straw-man S <- S + S_i.  AUTO picks FOLD
 * or SCAN, and SCAN's block size, from a cost model of element steps on the device's
 * compute units.
 *
 * Dense arithmetic: each product T_i X takes f16 hi/lo splits of both operands (about
 * 22-bit operands, fp32 accumulation) after scaling X by exact powers of two: per
 * column where only the state is carried (FOLD, and SCAN's fold of the block
 * aggregates and its re-fold, when T_total is NULL; each chain's columns are then
 * spread over several workgroups when that is faster), per 32-column block otherwise.
 * T_hat entries must lie within the f16 range (the builds emit them normalised to a
 * maximum below 2).
 *
 * Layouts (C = n_chain):
 *   slot        device int32 [n_elem], values in [0, n_slot); NULL = identity
 *               (then n_slot >= n_elem)
 *   T_hat       float32 element store: DENSE/KDA [n_slot, C, d_k, d_k];
 *               DIAG [n_slot, C, d_k]; SCALAR [n_slot, C]  (unused by NAIVE_ADD)
 *   T_exp       int32 [n_slot, C]
 *   S           float32 [n_slot, C, d_k, d_v]
 *   S0          float32 [C, d_k, d_v] or NULL (zero)
 *   S_final     float32 [C, d_k, d_v]
 *   S_prefix    float32 [n_elem, C, d_k, d_v] or NULL: the state ENTERING element i
 *   T_total     float32 like one element of T_hat, or NULL; T_total_exp int32 [C]
 * SCAN needs hypic_compose_workspace_bytes() of device workspace; FOLD and
 * NAIVE_ADD need none.
 * ---------------------------------------------------------------------------------- */
typedef struct {
    hypic_kind kind;
    int32_t n_chain;
    int32_t d_k, d_v;
    int32_t n_elem;
    int32_t n_slot;
    const int32_t* slot;
    const float* T_hat;
    const int32_t* T_exp;
    const float* S;
    const float* S0;
    float* S_final;
    float* S_prefix;
    float* T_total;
    int32_t* T_total_exp;
    hypic_compose_mode mode;
    int32_t scan_block;         /* elements per block for SCAN; 0 = automatic */
    void* workspace;
    size_t workspace_bytes;
} hypic_compose_desc;

hypic_status hypic_compose(const hypic_compose_desc* desc, hypic_stream_t stream);
size_t hypic_compose_workspace_bytes(const hypic_compose_desc* desc);

/* ------------------------------------------------------------------------------------
 * hypic_compose_noalloc -- hypic_compose for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.
 *
 * Same arguments, semantics and outputs as hypic_compose, except that
 * desc->workspace / workspace_bytes are ignored: the scratch SCAN needs (block
 * aggregates and block-entry states) lives in a fixed array of
 * HYPIC_NOALLOC_SCRATCH_BYTES per device, which the library holds from the moment it
 * is loaded on that device until the process ends.  A SCAN needing more (see
 * hypic_compose_workspace_bytes) returns HYPIC_ERR_UNSUPPORTED; FOLD and NAIVE_ADD
 * need none.  The call allocates nothing (no hipMalloc, no allocating library
 * routine); its first call on a device looks up the array's device address.  Every
 * call on one device shares that array and the array keeps the previous call's
 * contents (SCAN writes all of it before reading it): calls that may overlap on one
 * device -- different streams without ordering, or concurrent host threads on the
 * same stream order -- race and give wrong results.
 * ---------------------------------------------------------------------------------- */
#define HYPIC_NOALLOC_SCRATCH_BYTES (32u << 20)
hypic_status hypic_compose_noalloc(const hypic_compose_desc* desc, hypic_stream_t stream);

/* ------------------------------------------------------------------------------------
 * hypic_compose_seam -- the warm hit path in one pass: seam window and composition
 * fused, the running state kept on chip (dense kind).
 *
 * [news], seam-window paragraph: on reuse the first w tokens of each segment are
 * recomputed under the full prefix, advancing the running state and emitting their
 * outputs; [news], linear-layer paragraph: the cached rest of the segment is composed
 * by S <- T_C S + S(C|0).  For request positions i = 0 .. n_elem-1 in order, per chain:
 *   S <- the gated delta rule over seam i's tokens from S, emitting o_t = S_t^T q_t;
 *   S <- 2^T_exp[slot[i]] T_hat[slot[i]] S + S[slot[i]],
 * from S0 (NULL = 0); writes S_final and, if asked, the state entering each request
 * position before its seam (S_prefix).  Neither the seam's own (T, S) nor the prefix
 * states need to go through memory, unlike hypic_seam_advance + hypic_compose.
 * Layouts (C = n_chain = n_batch * h_v, chain = b * h_v + h):
 *   slot, T_hat, T_exp, S, S0, S_final, S_prefix as in hypic_compose (dense kind)
 *   seam tokens packed over request positions: position i owns tokens
 *   [cu_seam[i], cu_seam[i+1]) (host int64 [n_elem + 1]), at most
 *   HYPIC_COMPOSE_SEAM_MAX_W of them; q, k [B, N, h_k, d_k] and v [B, N, h_v, d_v]
 *   in_dtype (q, k L2-normalised per token on load when qk_l2norm); log_alpha, beta
 *   float32 [B, N, h_v]; o [B, N, h_v, d_v] out_dtype or NULL.
 * Workspace: hypic_compose_seam_workspace_bytes() (0 for at most 160 positions).
 * ---------------------------------------------------------------------------------- */
#define HYPIC_COMPOSE_SEAM_MAX_W 8
typedef struct {
    int32_t n_batch;
    int32_t h_k, h_v, d_k, d_v;
    int32_t n_elem;
    int32_t n_slot;
    const int32_t* slot;
    const float* T_hat;
    const int32_t* T_exp;
    const float* S;
    const float* S0;
    float* S_final;
    float* S_prefix;
    hypic_dtype in_dtype;
    hypic_dtype out_dtype;
    int64_t n_tokens;
    const int64_t* cu_seam;     /* host [n_elem + 1] */
    int32_t qk_l2norm;
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    void* o;
    void* workspace;
    size_t workspace_bytes;
} hypic_seam_compose_desc;

hypic_status hypic_compose_seam(const hypic_seam_compose_desc* desc, hypic_stream_t stream);
size_t hypic_compose_seam_workspace_bytes(const hypic_seam_compose_desc* desc);

/* ------------------------------------------------------------------------------------
 * hypic_seam_advance -- seam tokens through the running state (dense kind).
 *
 * [news], seam-window paragraph: the first w tokens of a reused segment are
 * not cached; on reuse they are recomputed under the full prefix, so the
 * linear layers compute the seam's own T and S on the fly, advance the
 * running state, and hand each seam token's output to the layers above.
 * [readme], "PIC modes": the window width is a runtime knob, default 8.
 *
 * Seam s covers tokens [cu_seam[s], cu_seam[s+1]) of the packed seam axis
 * (any length; w <= 64 runs as a single chunk).  Needs
 * hypic_seam_advance_workspace_bytes() of device workspace (0 for at most 160
 * seams).
 * Layouts (B = n_batch, N = n_tokens = packed seam tokens):
 *   q, k        [B, N, h_k, d_k]  in_dtype;   v [B, N, h_v, d_v] in_dtype
 *   log_alpha, beta  float32 [B, N, h_v]
 *   S_in        float32, seam s at S_in + s * state_stride: [B, h_v, d_k, d_v];
 *               NULL = zero.  state_stride 0 means B*h_v*d_k*d_v.
 *   o           [B, N, h_v, d_v] out_dtype, or NULL
 *   S_out       float32, same addressing as S_in (may alias S_in), or NULL
 *   T_hat       float32 [n_seam, B, h_v, d_k, d_k] or NULL; T_exp int32 [n_seam, B, h_v]
 *   S_seam      float32 [n_seam, B, h_v, d_k, d_v] or NULL: the seam's zero-start state
 * ---------------------------------------------------------------------------------- */
typedef struct {
    hypic_dtype in_dtype;
    hypic_dtype out_dtype;
    int32_t n_batch;
    int64_t n_tokens;
    int32_t h_k, h_v, d_k, d_v;
    int32_t n_seam;
    const int64_t* cu_seam;     /* host [n_seam + 1] */
    int32_t qk_l2norm;          /* 1: q and k scaled to unit L2 norm per token and head */
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const float* S_in;
    int64_t state_stride;       /* floats between consecutive seams in S_in / S_out */
    void* o;
    float* S_out;
    float* T_hat;
    int32_t* T_exp;
    float* S_seam;
    hypic_precision precision;
    void* workspace;
    size_t workspace_bytes;
} hypic_seam_desc;

hypic_status hypic_seam_advance(const hypic_seam_desc* desc, hypic_stream_t stream);
size_t hypic_seam_advance_workspace_bytes(const hypic_seam_desc* desc);

/* ------------------------------------------------------------------------------------
 * hypic_conv_warmup -- depthwise causal convolution with the state carried
 * across a segment boundary ([news], linear-layer paragraph: conv-state
 * warm-up aligns variants that run a causal conv before the recurrence).
 *
 *   y_t[c] = act( bias[c] + sum_{j=0}^{W-1} weight[c, j] * xx_{t+j}[c] )
 * where xx is the segment's W-1 carried inputs followed by its x rows, so
 * tap W-1 multiplies the current token (PyTorch Conv1d cross-correlation with
 * left padding W-1).  state_out receives the segment's last W-1 rows of xx.
 * Layouts (B = n_batch, N = n_tokens, C = channels, W = width = 4):
 *   x          [B, N, C] in_dtype
 *   state_in   [n_state, B, W-1, C] in_dtype, or NULL (zero state)
 *   state_index device int32 [n_seg]: row of state_in for segment s, -1 = zero;
 *               NULL = identity (segment s uses state_in[s], n_state >= n_seg)
 *   weight     float32 [B, C, W] (each batch entry, e.g. each layer, has its own
 *              taps);  bias float32 [B, C] or NULL
 *   y          [B, N, C] out_dtype
 *   state_out  [n_seg, B, W-1, C] in_dtype, or NULL
 * channels must be a multiple of 8.  Needs hypic_conv_warmup_workspace_bytes()
 * of device workspace (0 for at most 160 segments).
 * ---------------------------------------------------------------------------------- */
typedef struct {
    hypic_dtype in_dtype;
    hypic_dtype out_dtype;
    int32_t n_batch;
    int64_t n_tokens;
    int32_t channels;
    int32_t width;
    int32_t n_seg;
    const int64_t* cu_seqlens;  /* host [n_seg + 1] */
    const void* x;
    const void* state_in;
    int32_t n_state;
    const int32_t* state_index;
    const float* weight;
    const float* bias;
    hypic_activation activation;
    void* y;
    void* state_out;
    void* workspace;
    size_t workspace_bytes;
} hypic_conv_desc;

hypic_status hypic_conv_warmup(const hypic_conv_desc* desc, hypic_stream_t stream);
size_t hypic_conv_warmup_workspace_bytes(const hypic_conv_desc* desc);

/* ------------------------------------------------------------------------------------
 * hypic_state_rerotate -- RoPE state re-rotation of cached elements reused at a new
 * absolute offset.
 *
 * [news], linear-layer paragraph: variants that rotate q and k by absolute position
 * (RoPE) need the cached state re-rotated; [readme], "PIC modes": transition_rope
 * corrects the positions of segments reused somewhere else.  A segment cached with keys
 * rotated at positions p + t and reused at p + delta + t has keys R k with
 * R = R(delta): on each rotated channel pair (a, b) with frequency
 * theta_i = rope_base^(-2i / rotary_dim), (x_a, x_b) -> (x_a cos - x_b sin,
 * x_a sin + x_b cos) of the angle delta * theta_i; channels >= rotary_dim unchanged.
 * Its per-token transitions become R A_t R^T and its writes R k v^T, so
 *   S' = R S,   T' = R T R^T (DENSE; T_exp unchanged),   T' = T (SCALAR).
 * Per-channel (DIAG, KDA) gates do not commute with R: HYPIC_ERR_UNSUPPORTED.
 * Layouts (C = n_chain), float32, out may alias in (in-place update):
 *   S_in, S_out          [n_elem, C, d_k, d_v]
 *   T_hat_in, T_hat_out  [n_elem, C, d_k, d_k] (DENSE; NULL for SCALAR)
 *   delta                host int64 [n_elem]: new offset minus the cached offset
 * Pairs: interleaved = 1 pairs channels (2i, 2i+1); 0 pairs (i, i + rotary_dim/2).
 * rotary_dim even, 2 <= rotary_dim <= d_k; rope_base > 0.  No workspace; the shifts
 * travel in the kernel arguments (up to 160 elements per launch, more in batches).
 * ---------------------------------------------------------------------------------- */
typedef struct {
    hypic_kind kind;
    int32_t n_elem;
    int32_t n_chain;
    int32_t d_k, d_v;
    int32_t rotary_dim;
    int32_t interleaved;
    double rope_base;
    const int64_t* delta;
    const float* T_hat_in;
    float* T_hat_out;
    const float* S_in;
    float* S_out;
} hypic_rerotate_desc;

hypic_status hypic_state_rerotate(const hypic_rerotate_desc* desc, hypic_stream_t stream);

/* ------------------------------------------------------------------------------------
 * hypic_plan_schedule -- host-only planner behind HYPIC_SCHED_* (no GPU use).
 *
 * Assigns n tasks of integer weight (chunks) to `groups` workers.  LPT: tasks in
 * order of decreasing weight (ties: lower index first), each to the least-loaded
 * worker (ties: lower worker), Graham's longest-processing-time rule.  RR: task
 * i to worker i mod groups.  Writes order[n] (LPT processing order; identity
 * for RR), assign[n] and *makespan (max worker load).  Either output array may
 * be NULL.  Returns HYPIC_ERR_INVALID_ARGUMENT on negative weights, n < 0 or
 * groups < 1.
 * ---------------------------------------------------------------------------------- */
hypic_status hypic_plan_schedule(const int64_t* weights, int32_t n, int32_t groups,
                                 hypic_schedule schedule, int32_t* order, int32_t* assign,
                                 int64_t* makespan);

/* ------------------------------------------------------------------------------------
 * hypic_seam_widths -- the seam window width of each segment from the seam-width knob
 * ([readme], "PIC modes": the knob is independent of the compose mode, default 8;
 * [news], seam-window paragraph: the first w tokens of a reused segment are recomputed).
 *
 * Host-only integer arithmetic, no GPU use.  For each of the n segments of length
 * seg_lens[i] (host int64, >= 0) writes w[i] (host int32):
 *   sink == 0         -> 0 (the whole cached segment is reused, no seam);
 *   0 < sink <= 1     -> ceil(sink * len), a fraction of the segment;
 *   sink > 1          -> floor(sink), an absolute token count;
 * always capped at len.  The widths feed cu_seam of hypic_seam_advance and skip_head
 * of hypic_segment_build.  Returns HYPIC_ERR_INVALID_ARGUMENT for n < 0, NULL arrays
 * with n > 0, a negative length, or a negative or non-finite sink.
 * ---------------------------------------------------------------------------------- */
#define HYPIC_SEAM_SINK_DEFAULT 8.0
hypic_status hypic_seam_widths(const int64_t* seg_lens, int32_t n, double sink, int32_t* w);

/* ------------------------------------------------------------------------------------
 * hypic_device_status -- device-side invariant check.
 *
 * Synchronises the current device, then reads and clears its sticky status words.  The
 * waves of the dense build and of the dense compose hand work to each other through
 * bounded waits on LDS counters; a wait that runs out (a hand-off that never came) lets
 * the kernel finish and sets the word.  Returns HYPIC_OK, or HYPIC_ERR_DEVICE (with a message) when any launch since
 * the previous call set it: the outputs of those launches are unreliable.
 * ---------------------------------------------------------------------------------- */
hypic_status hypic_device_status(void);

const char* hypic_last_error(void);
int hypic_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HYPIC_H */
