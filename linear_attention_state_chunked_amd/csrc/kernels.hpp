// Internal launcher interface between the C-ABI host layer and the HIP kernels.
// Not part of the public API (include/hypic.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hypic {

// Per-segment table of one launch: first covered token and covered length of every
// segment and, when a processing order is given (LPT), the order of the segments.  Up to
// kInlineSegs segments travel inside the kernel arguments, so nothing is copied before the
// launch; a larger table lives in device memory (the call's workspace).
constexpr int kInlineSegs = 160;
struct SegTable {
    int n;                      // segments
    int inl;                    // 1: the arrays below hold the table, else the pointers
    int has_order;              // 1: segments are processed in order[] (LPT), else natural
    const long long* start_p;   // device [n]
    const int* len_p;           // device [n]
    const int* order_p;         // device [n]
    long long start[kInlineSegs];
    int len[kInlineSegs];
    int order[kInlineSegs];
};
__device__ __forceinline__ long long seg_start(const SegTable& t, int s) { return t.inl ? t.start[s] : t.start_p[s]; }
__device__ __forceinline__ int seg_len(const SegTable& t, int s) { return t.inl ? t.len[s] : t.len_p[s]; }
// Task at position it of the processing order.  The per_seg tasks of one segment (its
// batch rows and heads) are contiguous, and an order permutes whole segments.
__device__ __forceinline__ int task_at(const SegTable& t, int it, int per_seg) {
    if (!t.has_order) return it;
    const int j = it / per_seg;
    const int s = t.inl ? t.order[j] : t.order_p[j];
    return s * per_seg + (it - j * per_seg);
}

// Sticky per-device status word: a bounded wait inside a kernel that gave up sets a bit
// (an ordinary vector atomic), so a broken hand-off is reported instead of passing as
// silently wrong data.  take_device_status() reads and clears it (synchronous).
constexpr unsigned kStatusWaitExpired = 1u;
hipError_t take_device_status(unsigned* out);    // the dense build's word
hipError_t take_compose_status(unsigned* out);   // the compose kernels' word

// One dense (gated delta rule) chunk-engine launch.  Each task is one
// (segment, batch, value head) chain; it runs the segment's tokens chunk by chunk
// from X = [I | S_in] and emits T_hat/T_exp (if T_hat), the end state and, with q,
// the per-token outputs.
struct EngineArgs {
    int n_batch;
    long long n_tokens;
    int h_k, h_v;
    int n_seg;
    int qk_l2norm;
    int in_bf16;
    int out_bf16;
    int n_tasks;
    int persistent;              // 1: grid-stride over tasks (static round robin)
    const void* k;
    const void* v;
    const void* q;               // null: no outputs
    const float* log_alpha;
    const float* beta;
    const float* S_in;           // null: zero
    long long in_stride;         // floats between segments' state blocks in S_in
    float* S_out;                // may be null
    long long out_stride;
    float* T_hat;                // null: T columns skipped
    int* T_exp;
    void* o;
    int precise_T;               // 0: single f16 operands; 1: T columns with hi/lo X and Vn (with S);
                                 // 3: transition-only pass, single f16 operands;
                                 // 2: transition-only pass, hi/lo Tg, W', X, Vn (no S columns)
    // stream mode (persistent grid, equal segments, 16-bit inputs): segment s covers tokens
    // [stream_start0 + s * stream_stride, ... + stream_len); each workgroup streams the chunks
    // of its tasks it, it + grid, ... (natural order)
    int stream;
    long long stream_start0, stream_stride;
    int stream_len;
    SegTable seg;                // covered range [start, start + len) of every segment
};

// kind: 0 diagonal (GLA, per-channel log_alpha), 1 scalar
struct DiagArgs {
    int n_batch;
    long long n_tokens;
    int h_k, h_v;
    int n_seg;
    int scalar;
    int in_bf16;
    int qk_l2norm;
    int n_tasks;
    const void* k;
    const void* v;
    const float* log_alpha;
    float* T_hat;
    int* T_exp;
    float* S;
    SegTable seg;
};

// Per-channel gated delta rule (KDA) build: one workgroup per (segment, batch, value head),
// one thread per column of X = [T | S] (T columns only when T_hat is set).
struct KdaArgs {
    int n_batch;
    long long n_tokens;
    int h_k, h_v;
    int in_bf16;
    int n_tasks;
    const void* k;
    const void* v;
    const float* log_alpha;   // [B, N, h_v, d]
    const float* beta;        // [B, N, h_v]
    float* T_hat;
    int* T_exp;
    float* S;
    SegTable seg;
};
hipError_t launch_kda_build(const KdaArgs& a, int d, hipStream_t s);

// One fold launch: grid (chain, block).  Block `blk` folds elements
// [blk*per_block, min(n_elem, (blk+1)*per_block)) in order, from the state
// init_S[blk] (or zero) and transition I.
struct FoldArgs {
    int kind;                 // 0 dense, 1 diag, 2 scalar
    int n_chain;
    int n_elem;
    int per_block;
    int n_block;
    const int* slot;          // element -> slot, or null
    const float* T_hat;       // element store [n_slot, n_chain, ...]
    const int* T_exp;
    const float* S;
    const float* init_S;      // [n_block, n_chain, dk, dv] or null
    float* out_S;             // [n_block, n_chain, dk, dv] or null
    float* out_T;             // [n_block, n_chain, ...] or null
    int* out_e;               // [n_block, n_chain] or null
    float* prefix;            // [n_elem, n_chain, dk, dv] or null
    int naive;                // 1: S <- S + S_i
    // Fused seam (dense kind, one block per chain): before element el's product the running
    // state goes through the seam tokens [start, start + len) of entry el of `seam_tab`
    // (packed seam axis, at most kFusedSeamMax tokens), emitting o_t = S_t^T q_t.
    int seam;
    int n_batch, h_k, h_v;    // chain = b * h_v + h
    long long n_tokens;       // packed seam tokens
    int in_bf16, out_bf16, qk_l2norm;
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    void* o;                  // [B, n_tokens, h_v, dv]
    SegTable seam_tab;
};
constexpr int kFusedSeamMax = 8;

// One short-seam launch (every seam <= 16 tokens): one workgroup per (seam, batch,
// value head); computes whichever of o, S_out, T_hat/T_exp, S_seam are non-null.
struct SeamArgs {
    int n_batch;
    long long n_tokens;
    int h_k, h_v;
    int qk_l2norm;
    int in_bf16, out_bf16;
    int n_tasks;
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const float* S_in;           // null: zero
    long long in_stride;         // floats between seams' state blocks
    float* S_out;
    long long out_stride;
    void* o;
    float* T_hat;
    int* T_exp;
    float* S_seam;
    SegTable seg;                // seam s: tokens [start, start + len)
};

struct ConvArgs {
    int n_batch;
    long long n_tokens;
    int channels;
    int n_seg;
    int in_bf16, out_bf16;
    int silu;
    const void* x;
    const void* state_in;
    int n_state;
    const int* state_index;
    const float* weight;
    const float* bias;
    void* y;
    void* state_out;
    SegTable seg;
};

hipError_t launch_dense_engine(const EngineArgs& a, int d, int prec_f32, int grid, hipStream_t s);
// warp-specialised segment build (X = [I | 0] start, no outputs); T columns iff a.T_hat
hipError_t launch_gdn_build(const EngineArgs& a, int d, int prec_f32, int grid, hipStream_t s);
hipError_t launch_diag_build(const DiagArgs& a, int d, hipStream_t s);
hipError_t launch_fold(const FoldArgs& a, int d, int with_T, hipStream_t s);
// dense kind, running state only: the columns of each chain split over d/16 workgroups
hipError_t launch_fold_split(const FoldArgs& a, int d, hipStream_t s);
// Device address of this device's fixed compose scratch (kNoAllocScratchBytes), looked up
// once per device with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_conv(const ConvArgs& a, long long total_tokens, hipStream_t s);
// seams of at most kSeamShort tokens
constexpr int kSeamShort = 16;
// w_max: the longest seam (<= kSeamShort); seams of at most 8 tokens use a lighter instance
hipError_t launch_seam(const SeamArgs& a, int d, int w_max, hipStream_t s);

// RoPE state re-rotation of up to kRotInline elements per launch (the position shifts
// travel in the kernel arguments): S_out = R S_in and, with dense, T_out = R T_in R^T,
// R = R(delta[e]); elements elem0 + e of [n_elem, n_chain, d, d] arrays; may run in place.
constexpr int kRotInline = 160;
struct RotArgs {
    int n_chain;
    int rotary_dim;
    int interleaved;   // 1: pairs (2i, 2i+1); 0: pairs (i, i + rotary_dim/2)
    int dense;         // 1: rotate T too (rows and columns); 0: scalar T, untouched
    int elem0;
    double log2_base;
    const float* T_in;
    float* T_out;
    const float* S_in;
    float* S_out;
    long long delta[kRotInline];
};
hipError_t launch_rerotate(const RotArgs& r, int d, int n_elem, hipStream_t s);

// resident workgroups per CU for the dense engine (for persistent grids)
int dense_engine_max_lds(int d, int prec_f32, int with_q);

}  // namespace hypic
