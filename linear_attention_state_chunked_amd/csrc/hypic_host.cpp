// libhypic C ABI: argument validation, workspace layout, schedule planning, launches.
//
// Every entry point validates all of its arguments on the host before touching the
// HIP runtime; on failure it enqueues nothing and returns a status with a message in
// the thread-local hypic_last_error().
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "../../include/hypic.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

hypic_status fail(hypic_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

hypic_status ok() {
    g_err.clear();
    return HYPIC_OK;
}

hypic_status device_fail(const char* what, hipError_t e) {
    return fail(HYPIC_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
constexpr int32_t kPreciseTTokens = 2048;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validate a host offset table: cu[0] = 0, non-decreasing, cu[n] <= limit.
hypic_status check_offsets(const int64_t* cu, int32_t n, int64_t limit, const char* name) {
    if (n < 0) return fail(HYPIC_ERR_INVALID_ARGUMENT, "%s: negative segment count %d", name, n);
    if (!cu) return fail(HYPIC_ERR_INVALID_ARGUMENT, "%s is NULL", name);
    if (cu[0] != 0) return fail(HYPIC_ERR_INVALID_ARGUMENT, "%s[0] = %lld, must be 0", name, (long long)cu[0]);
    for (int32_t i = 0; i < n; ++i)
        if (cu[i + 1] < cu[i])
            return fail(HYPIC_ERR_INVALID_ARGUMENT, "%s is decreasing at %d (%lld > %lld)", name, i,
                        (long long)cu[i], (long long)cu[i + 1]);
    if (cu[n] > limit)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "%s[%d] = %lld exceeds n_tokens = %lld", name, n, (long long)cu[n],
                    (long long)limit);
    return HYPIC_OK;
}

// Segment table of a launch.  Up to hypic::kInlineSegs segments it travels inside the
// kernel arguments: no copy, no workspace, and the call is asynchronous.  A larger table
// (starts int64, lengths int32, segment order int32) is uploaded to the workspace.
struct SegTableLayout {
    size_t off_start = 0, off_len = 0, off_order = 0, bytes = 0;
};

SegTableLayout seg_table_layout(int32_t n_seg) {
    SegTableLayout t;
    if (n_seg <= hypic::kInlineSegs) return t;
    t.off_start = 0;
    t.off_len = align_up(sizeof(int64_t) * n_seg);
    t.off_order = t.off_len + align_up(sizeof(int32_t) * n_seg);
    t.bytes = t.off_order + align_up(sizeof(int32_t) * n_seg);
    return t;
}

// Fill `t` for segments (start, len) processed in `order` (empty = natural order).  A table
// too large for the kernel arguments goes to the workspace in one transfer from pageable
// host memory: the runtime stages it before returning, so the host arrays may die afterwards.
hipError_t fill_seg_table(hypic::SegTable& t, const SegTableLayout& L, void* ws, const std::vector<int64_t>& start,
                          const std::vector<int32_t>& len, const std::vector<int32_t>& order, hipStream_t s) {
    const int32_t n = (int32_t)start.size();
    t.n = n;
    t.has_order = order.empty() ? 0 : 1;
    if (n <= hypic::kInlineSegs) {
        t.inl = 1;
        for (int32_t i = 0; i < n; ++i) {
            t.start[i] = start[i];
            t.len[i] = len[i];
            t.order[i] = order.empty() ? i : order[i];
        }
        return hipSuccess;
    }
    t.inl = 0;
    std::vector<unsigned char> img(L.bytes, 0);
    memcpy(img.data() + L.off_start, start.data(), start.size() * sizeof(int64_t));
    memcpy(img.data() + L.off_len, len.data(), len.size() * sizeof(int32_t));
    if (!order.empty()) memcpy(img.data() + L.off_order, order.data(), order.size() * sizeof(int32_t));
    unsigned char* w = static_cast<unsigned char*>(ws);
    t.start_p = reinterpret_cast<const long long*>(w + L.off_start);
    t.len_p = reinterpret_cast<const int*>(w + L.off_len);
    t.order_p = reinterpret_cast<const int*>(w + L.off_order);
    return hipMemcpyAsync(ws, img.data(), L.bytes, hipMemcpyHostToDevice, s);
}

// The workspace a call needs for its segment table: present when L.bytes > 0, aligned.
hypic_status check_workspace(const char* who, size_t need, void* ws, size_t have) {
    if (need == 0) return HYPIC_OK;
    if (!ws || have < need)
        return fail(HYPIC_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    ws ? have : (size_t)0);
    if (reinterpret_cast<uintptr_t>(ws) % kAlign)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "%s: workspace must be 256-byte aligned", who);
    return HYPIC_OK;
}

bool supported_d(int d) { return d == 64 || d == 128; }

// kinds whose transition is a dense d_k x d_k matrix (composed alike)
bool dense_T(hypic_kind k) { return k == HYPIC_DENSE_DELTA || k == HYPIC_KDA; }

int64_t build_tasks(const hypic_build_desc* d) { return (int64_t)d->n_seg * d->n_batch * d->h_v; }

hypic_status validate_build(const hypic_build_desc* d) {
    if (!d) return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: desc is NULL");
    if (d->kind < HYPIC_DENSE_DELTA || d->kind > HYPIC_KDA)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: unknown kind %d", (int)d->kind);
    if (d->in_dtype != HYPIC_F32 && d->in_dtype != HYPIC_BF16)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: unknown in_dtype %d", (int)d->in_dtype);
    if (d->n_batch < 1 || d->n_tokens < 0 || d->h_k < 1 || d->h_v < 1)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: bad geometry n_batch=%d n_tokens=%lld h_k=%d h_v=%d",
                    d->n_batch, (long long)d->n_tokens, d->h_k, d->h_v);
    if (d->h_v % d->h_k != 0)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: h_v=%d is not a multiple of h_k=%d", d->h_v, d->h_k);
    if (d->d_k != d->d_v || !supported_d(d->d_k))
        return fail(HYPIC_ERR_UNSUPPORTED, "build: d_k=%d d_v=%d (supported: d_k == d_v in {64, 128})", d->d_k, d->d_v);
    if (d->chunk != 64) return fail(HYPIC_ERR_UNSUPPORTED, "build: chunk=%d (supported: 64)", d->chunk);
    if (d->skip_head < 0) return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: skip_head=%d < 0", d->skip_head);
    if (d->qk_l2norm != 0 && d->qk_l2norm != 1)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: qk_l2norm=%d must be 0 or 1", d->qk_l2norm);
    if (d->qk_l2norm && d->kind != HYPIC_DENSE_DELTA)
        return fail(HYPIC_ERR_UNSUPPORTED, "build: qk_l2norm is supported for the dense kind only");
    const bool has_beta = d->kind == HYPIC_DENSE_DELTA || d->kind == HYPIC_KDA;
    hypic_status st = check_offsets(d->cu_seqlens, d->n_seg, d->n_tokens, "build: cu_seqlens");
    if (st != HYPIC_OK) return st;
    for (int32_t i = 0; i < d->n_seg; ++i)
        if (d->cu_seqlens[i + 1] - d->cu_seqlens[i] > (int64_t)1 << 30)
            return fail(HYPIC_ERR_UNSUPPORTED, "build: segment %d longer than 2^30 tokens", i);
    if (build_tasks(d) > INT32_MAX) return fail(HYPIC_ERR_UNSUPPORTED, "build: too many (segment, chain) tasks");
    if (d->n_seg > 0 && d->n_tokens > 0) {
        if (!d->k || !d->v || !d->log_alpha)
            return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: k, v and log_alpha are required");
        if (!aligned16(d->k) || !aligned16(d->v))
            return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: k and v must be 16-byte aligned");
    }
    if (has_beta) {
        if (d->n_seg > 0 && d->n_tokens > 0 && !d->beta)
            return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: beta is required for the dense and KDA kinds");
    } else if (d->beta) {
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: beta must be NULL for the diagonal and scalar kinds");
    }
    if (d->n_seg > 0 && !d->S) return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: S is NULL");
    if (d->o) {
        if (d->kind != HYPIC_DENSE_DELTA)
            return fail(HYPIC_ERR_UNSUPPORTED, "build: per-token outputs are implemented for the dense kind only");

        if (!d->q) return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: o requested without q");
        if (!aligned16(d->q)) return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: q must be 16-byte aligned");
        if (d->out_dtype != HYPIC_F32 && d->out_dtype != HYPIC_BF16)
            return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: unknown out_dtype %d", (int)d->out_dtype);
        if (d->precision == HYPIC_PREC_F16_PRECISE_T && d->in_dtype != HYPIC_BF16)
            return fail(HYPIC_ERR_UNSUPPORTED, "build: the output-fused build's precise-T plan needs 16-bit inputs");
    }
    if ((d->T_hat == nullptr) != (d->T_exp == nullptr))
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: T_hat and T_exp must be both set or both NULL");
    if (d->schedule < HYPIC_SCHED_NATURAL || d->schedule > HYPIC_SCHED_RR)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: unknown schedule %d", (int)d->schedule);
    if (d->precision < HYPIC_PREC_AUTO || d->precision > HYPIC_PREC_F16_PRECISE_T)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: unknown precision %d", (int)d->precision);
    if (d->precision == HYPIC_PREC_F16_PRECISE_T && d->kind != HYPIC_DENSE_DELTA)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "build: F16_PRECISE_T applies to the dense kind only");
    if (d->kind == HYPIC_DENSE_DELTA) {
        if (d->precision == HYPIC_PREC_F32 && d->d_k != 64)
            return fail(HYPIC_ERR_UNSUPPORTED, "build: the F32 operand plan supports d = 64 only");
        if (d->precision == HYPIC_PREC_AUTO && d->in_dtype == HYPIC_F32 && d->d_k != 64)
            return fail(HYPIC_ERR_UNSUPPORTED,
                        "build: float32 inputs at d = %d have no float32-operand plan; request "
                        "HYPIC_PREC_F16 explicitly to accept f16 operands (about 1e-3 relative error)", d->d_k);
    }
    return HYPIC_OK;
}

bool build_prec_f32(const hypic_build_desc* d) {
    return d->precision == HYPIC_PREC_F32 ||
           (d->precision == HYPIC_PREC_AUTO && d->in_dtype == HYPIC_F32 && d->d_k == 64);
}

// compute units of the current device, queried once per device
int device_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const bool cacheable = dev >= 0 && dev < 64;
    if (cacheable && (n = cached[dev].load(std::memory_order_relaxed)) > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (cacheable && n > 0) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// LPT order of segments: longest first, ties by index.  The tasks of one segment (its
// batch rows and heads) stay together; the kernels expand a segment position to its tasks.
std::vector<int32_t> lpt_segment_order(const std::vector<int32_t>& len) {
    std::vector<int32_t> segs(len.size());
    std::iota(segs.begin(), segs.end(), 0);
    std::stable_sort(segs.begin(), segs.end(), [&](int32_t a, int32_t b) { return len[a] > len[b]; });
    return segs;
}

}  // namespace

// The public functions take C linkage from their declarations in hypic.h.

const char* hypic_last_error(void) { return g_err.c_str(); }
int hypic_version(void) { return HYPIC_VERSION; }

hypic_status hypic_device_status(void) {
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return device_fail("device status: synchronize", e);
    unsigned flags = 0, cflags = 0;
    e = hypic::take_device_status(&flags);
    if (e != hipSuccess) return device_fail("device status: read", e);
    e = hypic::take_compose_status(&cflags);
    if (e != hipSuccess) return device_fail("device status: read", e);
    if ((flags | cflags) & hypic::kStatusWaitExpired)
        return fail(HYPIC_ERR_DEVICE,
                    "device status: a bounded wait inside the %s gave up (a hand-off between the waves of a "
                    "workgroup never came); outputs since the last status call are unreliable",
                    (flags & hypic::kStatusWaitExpired) ? "dense build" : "compose");
    flags |= cflags;
    if (flags) return fail(HYPIC_ERR_DEVICE, "device status: flags 0x%x", flags);
    return ok();
}

hypic_status hypic_seam_widths(const int64_t* seg_lens, int32_t n, double sink, int32_t* w) {
    if (n < 0) return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam widths: n = %d < 0", n);
    if (n > 0 && (!seg_lens || !w)) return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam widths: NULL array");
    if (!(sink >= 0.0) || sink > 1e18) return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam widths: sink %g out of range", sink);
    for (int32_t i = 0; i < n; ++i)
        if (seg_lens[i] < 0) return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam widths: segment %d has negative length", i);
    for (int32_t i = 0; i < n; ++i) {
        const int64_t len = seg_lens[i];
        int64_t x;
        if (sink == 0.0) {
            x = 0;  // reuse the whole segment: no seam
        } else if (sink <= 1.0) {
            // a fraction of the segment: ceil(sink * len), computed exactly for the small
            // lengths involved (len < 2^53)
            const double f = sink * (double)len;
            x = (int64_t)f;
            if ((double)x < f) ++x;
        } else {
            x = (int64_t)sink;  // an absolute token count (the integer part)
        }
        w[i] = (int32_t)std::min<int64_t>(x, std::min<int64_t>(len, INT32_MAX));
    }
    return ok();
}

hypic_status hypic_plan_schedule(const int64_t* weights, int32_t n, int32_t groups, hypic_schedule schedule,
                                 int32_t* order, int32_t* assign, int64_t* makespan) {
    if (n < 0) return fail(HYPIC_ERR_INVALID_ARGUMENT, "plan: n = %d < 0", n);
    if (groups < 1) return fail(HYPIC_ERR_INVALID_ARGUMENT, "plan: groups = %d < 1", groups);
    if (n > 0 && !weights) return fail(HYPIC_ERR_INVALID_ARGUMENT, "plan: weights is NULL");
    for (int32_t i = 0; i < n; ++i)
        if (weights[i] < 0) return fail(HYPIC_ERR_INVALID_ARGUMENT, "plan: weight %d is negative", i);
    if (schedule != HYPIC_SCHED_LPT && schedule != HYPIC_SCHED_RR && schedule != HYPIC_SCHED_NATURAL)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "plan: unknown schedule %d", (int)schedule);
    std::vector<int32_t> ord(n);
    std::iota(ord.begin(), ord.end(), 0);
    std::vector<int64_t> load(groups, 0);
    std::vector<int32_t> asg(n, 0);
    if (schedule == HYPIC_SCHED_LPT) {
        std::stable_sort(ord.begin(), ord.end(), [&](int32_t a, int32_t b) { return weights[a] > weights[b]; });
        for (int32_t i : ord) {
            int32_t g = 0;
            for (int32_t j = 1; j < groups; ++j)
                if (load[j] < load[g]) g = j;
            asg[i] = g;
            load[g] += weights[i];
        }
    } else {
        for (int32_t i = 0; i < n; ++i) {
            asg[i] = i % groups;
            load[i % groups] += weights[i];
        }
    }
    if (order) std::copy(ord.begin(), ord.end(), order);
    if (assign) std::copy(asg.begin(), asg.end(), assign);
    if (makespan) *makespan = n ? *std::max_element(load.begin(), load.end()) : 0;
    return ok();
}

// ------------------------------------------------------------------------------------------
// segment build

size_t hypic_segment_build_workspace_bytes(const hypic_build_desc* d) {
    if (!d || d->n_seg < 0) return 0;
    return seg_table_layout(d->n_seg).bytes;
}

hypic_status hypic_segment_build(const hypic_build_desc* d, hypic_stream_t stream) {
    hypic_status st = validate_build(d);
    if (st != HYPIC_OK) return st;
    const int64_t n_tasks = build_tasks(d);
    if (n_tasks == 0) return ok();
    const SegTableLayout L = seg_table_layout(d->n_seg);
    st = check_workspace("build", L.bytes, d->workspace, d->workspace_bytes);
    if (st != HYPIC_OK) return st;

    std::vector<int64_t> start(d->n_seg);
    std::vector<int32_t> len(d->n_seg);
    for (int32_t i = 0; i < d->n_seg; ++i) {
        start[i] = d->cu_seqlens[i] + d->skip_head;
        len[i] = (int32_t)std::max<int64_t>(0, d->cu_seqlens[i + 1] - start[i]);
    }
    std::vector<int32_t> order;
    if (d->schedule == HYPIC_SCHED_LPT) order = lpt_segment_order(len);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hypic::SegTable tab{};
    hipError_t e = fill_seg_table(tab, L, d->workspace, start, len, order, s);
    if (e != hipSuccess) return device_fail("build: segment table upload", e);

    if (d->kind == HYPIC_DENSE_DELTA && d->o && (d->in_dtype != HYPIC_BF16 || build_prec_f32(d))) {
        // output-fused build with float32 inputs or operands: the general chunk engine from a
        // zero state, with q
        hypic::EngineArgs a{};
        a.n_batch = d->n_batch;
        a.n_tokens = d->n_tokens;
        a.h_k = d->h_k;
        a.h_v = d->h_v;
        a.n_seg = d->n_seg;
        a.qk_l2norm = d->qk_l2norm;
        a.in_bf16 = d->in_dtype == HYPIC_BF16;
        a.out_bf16 = d->out_dtype == HYPIC_BF16;
        a.seg = tab;
        a.n_tasks = (int)n_tasks;
        a.k = d->k;
        a.v = d->v;
        a.q = d->q;
        a.o = d->o;
        a.log_alpha = d->log_alpha;
        a.beta = d->beta;
        a.S_out = d->S;
        a.out_stride = (long long)d->n_batch * d->h_v * d->d_k * d->d_v;
        a.T_hat = d->T_hat;
        a.T_exp = d->T_exp;
        e = hypic::launch_dense_engine(a, d->d_k, build_prec_f32(d) ? 1 : 0, (int)n_tasks, s);
        if (e != hipSuccess) return device_fail("build: output-fused build launch", e);
    } else if (d->kind == HYPIC_DENSE_DELTA) {
        hypic::EngineArgs a{};
        a.n_batch = d->n_batch;
        a.n_tokens = d->n_tokens;
        a.h_k = d->h_k;
        a.h_v = d->h_v;
        a.n_seg = d->n_seg;
        a.qk_l2norm = d->qk_l2norm;
        a.in_bf16 = d->in_dtype == HYPIC_BF16;
        a.seg = tab;
        a.n_tasks = (int)n_tasks;
        a.k = d->k;
        a.v = d->v;
        a.log_alpha = d->log_alpha;
        a.beta = d->beta;
        a.S_out = d->S;
        a.out_stride = (long long)d->n_batch * d->h_v * d->d_k * d->d_v;
        a.T_hat = d->T_hat;
        a.T_exp = d->T_exp;
        // f16 operand rounding errors of the T columns add up over a segment's chunks
        // (relative error ~ 2.4e-4 * sqrt(chunks) for bf16 inputs): past 2048 tokens the
        // T columns switch to hi/lo operands so long segments stay well inside 2e-3
        a.precise_T = *std::max_element(len.begin(), len.end()) > kPreciseTTokens ? 1 : 0;
        int grid = (int)n_tasks;
        // Equal, evenly spaced segments of at least two chunks with 16-bit inputs: every schedule
        // gives the same task order (LPT sorts equal lengths stably), so one persistent workgroup
        // per compute unit streams the chunks of its tasks and overlaps each task's start-up with
        // the previous task's last chunk
        bool uniform = d->in_dtype == HYPIC_BF16 && !build_prec_f32(d) && len[0] > 64;
        const int64_t stride = d->n_seg > 1 ? start[1] - start[0] : 0;
        for (int32_t i = 0; uniform && i < d->n_seg; ++i)
            uniform = len[i] == len[0] && start[i] == start[0] + i * stride;
        if (uniform || d->schedule == HYPIC_SCHED_RR) {
            const int cus = device_cu_count();
            if (cus <= 0) return fail(HYPIC_ERR_DEVICE, "build: cannot query the device's compute units");
            a.persistent = 1;
            grid = (int)std::min<int64_t>(n_tasks, cus);
        }
        // the stream needs the grid to be a multiple of the heads per segment (a workgroup's
        // tasks then share batch row and head) and at least four chunks per task
        if (uniform && (len[0] <= 192 || grid % (d->n_batch * d->h_v) != 0)) {
            uniform = false;
            if (d->schedule != HYPIC_SCHED_RR) {
                a.persistent = 0;
                grid = (int)n_tasks;
            }
        }
        if (uniform) {
            a.stream = 1;
            a.stream_start0 = start[0];
            a.stream_stride = stride;
            a.stream_len = len[0];
        }
        const bool with_o = d->o != nullptr;   // 16-bit inputs here (the others took the general engine)
        if (with_o) {
            a.q = d->q;
            a.o = d->o;
            a.out_bf16 = d->out_dtype == HYPIC_BF16;
        }
        if (d->T_hat && (with_o || d->precision == HYPIC_PREC_F16_PRECISE_T)) {
            // T from a transition-only pass: hi/lo operands under the precise plan (and, with
            // outputs, for the long segments AUTO gives hi/lo T operands), else single f16 operands;
            // then the state pass (with outputs, if asked)
            hypic::EngineArgs t = a;
            t.precise_T = (d->precision == HYPIC_PREC_F16_PRECISE_T || a.precise_T == 1) ? 2 : 3;
            t.S_out = nullptr;
            t.q = nullptr;
            t.o = nullptr;
            e = hypic::launch_gdn_build(t, d->d_k, 0, grid, s);
            if (e != hipSuccess) return device_fail("build: transition pass launch", e);
            a.T_hat = nullptr;
            a.T_exp = nullptr;
            a.precise_T = 0;
        }
        e = hypic::launch_gdn_build(a, d->d_k, build_prec_f32(d) ? 1 : 0, grid, s);
        if (e != hipSuccess) return device_fail("build: dense build launch", e);
    } else if (d->kind == HYPIC_KDA) {
        if (d->schedule == HYPIC_SCHED_RR)
            return fail(HYPIC_ERR_UNSUPPORTED, "build: RR schedule is implemented for the dense kind only");
        hypic::KdaArgs a{};
        a.n_batch = d->n_batch;
        a.n_tokens = d->n_tokens;
        a.h_k = d->h_k;
        a.h_v = d->h_v;
        a.in_bf16 = d->in_dtype == HYPIC_BF16;
        a.n_tasks = (int)n_tasks;
        a.k = d->k;
        a.v = d->v;
        a.log_alpha = d->log_alpha;
        a.beta = d->beta;
        a.T_hat = d->T_hat;
        a.T_exp = d->T_exp;
        a.S = d->S;
        a.seg = tab;
        e = hypic::launch_kda_build(a, d->d_k, s);
        if (e != hipSuccess) return device_fail("build: KDA build launch", e);
    } else {
        hypic::DiagArgs a{};
        a.n_batch = d->n_batch;
        a.n_tokens = d->n_tokens;
        a.h_k = d->h_k;
        a.h_v = d->h_v;
        a.n_seg = d->n_seg;
        a.scalar = d->kind == HYPIC_SCALAR;
        a.in_bf16 = d->in_dtype == HYPIC_BF16;
        a.seg = tab;
        a.n_tasks = (int)n_tasks;
        a.k = d->k;
        a.v = d->v;
        a.log_alpha = d->log_alpha;
        a.T_hat = d->T_hat;
        a.T_exp = d->T_exp;
        a.S = d->S;
        if (d->schedule == HYPIC_SCHED_RR)
            return fail(HYPIC_ERR_UNSUPPORTED, "build: RR schedule is implemented for the dense kind only");
        e = hypic::launch_diag_build(a, d->d_k, s);
        if (e != hipSuccess) return device_fail("build: diagonal build launch", e);
    }
    return ok();
}

// ------------------------------------------------------------------------------------------
// compose

namespace {

// Dense compose cost model in element steps of fold_dense_kernel, one workgroup per compute
// unit: FOLD runs one workgroup per chain (two with the composed T) for n steps; SCAN's
// block reduce runs two per (chain, block) for B steps, the scan of the aggregates one (two)
// per chain for n/B steps, and the optional re-fold one per (chain, block) for B steps.  A
// fold of the running state alone can instead run column-split (d/16 workgroups per chain),
// whose step takes kSplitStepPct percent of a fold_dense_kernel step.
// `cus` is the device's compute unit count, looked up once per call by the caller.
int planner_cus() {
    const int n = device_cu_count();
    return n > 0 ? n : 256;
}

int64_t dense_rounds(int64_t wgs, int cus) { return (wgs + cus - 1) / cus; }

// 1.8 us against 3.5 us per element for 32 chains of d = 128 (the 64k-token layer's compose as FOLD)
constexpr int64_t kSplitStepPct = 50;

// a fold of the running state alone over `wgs` (chain, block) pairs: column-split or not
bool split_fold_better(int64_t wgs, int d, int cus) {
    return dense_rounds(wgs * (d / 16), cus) * kSplitStepPct < dense_rounds(wgs, cus) * 100;
}

// cost in percent of a fold_dense_kernel step of `steps` steps over `wgs` (chain, block) pairs
int64_t state_fold_cost(int64_t wgs, int64_t steps, int d, int cus) {
    return std::min(dense_rounds(wgs * (d / 16), cus) * kSplitStepPct, dense_rounds(wgs, cus) * 100) * steps;
}

int64_t dense_fold_cost(const hypic_compose_desc* d, int cus) {
    if (d->T_total) return dense_rounds((int64_t)d->n_chain * 2, cus) * d->n_elem * 100;
    return state_fold_cost(d->n_chain, d->n_elem, d->d_k, cus);
}

int64_t dense_scan_cost(const hypic_compose_desc* d, int64_t b, int cus) {
    const int64_t C = d->n_chain, nb = (d->n_elem + b - 1) / b;
    int64_t cost = dense_rounds(2 * C * nb, cus) * b * 100;
    cost += d->T_total ? dense_rounds(2 * C, cus) * nb * 100 : state_fold_cost(C, nb, d->d_k, cus);
    if (d->S_prefix) cost += state_fold_cost(C * nb, b, d->d_k, cus);
    return cost;
}

int scan_block_size(const hypic_compose_desc* d, int cus) {
    if (d->scan_block > 0) return d->scan_block;
    const int64_t n = d->n_elem;
    if (!dense_T(d->kind)) {
        int b = 1;
        while ((int64_t)b * b < n) ++b;  // ~sqrt(n): balances the two sequential phases
        return std::max(b, 2);
    }
    int best = 2;
    int64_t best_cost = dense_scan_cost(d, 2, cus);
    for (int64_t b = 3; b <= n; ++b) {
        const int64_t c = dense_scan_cost(d, b, cus);
        if (c < best_cost) {
            best_cost = c;
            best = (int)b;
        }
    }
    return best;
}

hypic_compose_mode resolve_mode(const hypic_compose_desc* d, int cus) {
    if (d->mode != HYPIC_COMPOSE_AUTO) return d->mode;
    if (dense_T(d->kind))
        return (d->n_elem >= 4 && dense_scan_cost(d, scan_block_size(d, cus), cus) < dense_fold_cost(d, cus))
                   ? HYPIC_COMPOSE_SCAN
                   : HYPIC_COMPOSE_FOLD;
    // few chains cannot fill the GPU with one block per chain: use the blocked scan
    return (d->n_elem >= 16 && (int64_t)d->n_chain * 4 < 1024) ? HYPIC_COMPOSE_SCAN : HYPIC_COMPOSE_FOLD;
}

struct ScanLayout {
    size_t aggT = 0, aggE = 0, aggS = 0, pre = 0, bytes = 0;
};

ScanLayout scan_layout(const hypic_compose_desc* d, int nblk) {
    const int64_t C = d->n_chain, D = d->d_k;
    const int64_t tlen = dense_T(d->kind) ? D * D : (d->kind == HYPIC_DIAG ? D : 1);
    ScanLayout L;
    L.aggT = 0;
    L.aggE = L.aggT + align_up(sizeof(float) * nblk * C * tlen);
    L.aggS = L.aggE + align_up(sizeof(int32_t) * nblk * C);
    L.pre = L.aggS + align_up(sizeof(float) * nblk * C * D * D);
    L.bytes = L.pre + (d->S_prefix ? align_up(sizeof(float) * nblk * C * D * D) : 0);
    return L;
}

hypic_status validate_compose(const hypic_compose_desc* d) {
    if (!d) return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: desc is NULL");
    if (d->kind < HYPIC_DENSE_DELTA || d->kind > HYPIC_KDA)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: unknown kind %d", (int)d->kind);
    if (d->mode < HYPIC_COMPOSE_AUTO || d->mode > HYPIC_COMPOSE_NAIVE_ADD)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: unknown mode %d", (int)d->mode);
    if (d->n_chain < 1 || d->n_elem < 0 || d->n_slot < 0)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: bad n_chain=%d n_elem=%d n_slot=%d", d->n_chain, d->n_elem,
                    d->n_slot);
    if (d->d_k != d->d_v || !supported_d(d->d_k))
        return fail(HYPIC_ERR_UNSUPPORTED, "compose: d_k=%d d_v=%d (supported: d_k == d_v in {64, 128})", d->d_k,
                    d->d_v);
    if (!d->slot && d->n_slot < d->n_elem)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: slot is NULL but n_slot=%d < n_elem=%d", d->n_slot,
                    d->n_elem);
    if (!d->S_final) return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: S_final is NULL");
    if (d->n_elem > 0 && !d->S) return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: S is NULL");
    const hypic_compose_mode m = resolve_mode(d, planner_cus());
    if (m != HYPIC_COMPOSE_NAIVE_ADD && d->n_elem > 0 && (!d->T_hat || !d->T_exp))
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: T_hat and T_exp are required");
    if ((d->T_total == nullptr) != (d->T_total_exp == nullptr))
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: T_total and T_total_exp must be both set or both NULL");
    if (m == HYPIC_COMPOSE_NAIVE_ADD && d->T_total)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: NAIVE_ADD has no transition; T_total must be NULL");
    if (d->T_hat && !aligned16(d->T_hat))
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: T_hat must be 16-byte aligned");
    if (d->scan_block < 0) return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: scan_block < 0");
    if ((int64_t)d->n_chain * d->n_elem > INT32_MAX || d->n_chain > 65535 * 1024)
        return fail(HYPIC_ERR_UNSUPPORTED, "compose: too many chains x elements");
    return HYPIC_OK;
}

}  // namespace

size_t hypic_compose_workspace_bytes(const hypic_compose_desc* d) {
    if (!d || d->n_elem <= 0 || d->n_chain <= 0) return 0;
    const int cus = planner_cus();
    if (resolve_mode(d, cus) != HYPIC_COMPOSE_SCAN) return 0;
    const int B = scan_block_size(d, cus);
    return scan_layout(d, (d->n_elem + B - 1) / B).bytes;
}

namespace {

// The composition behind both compose entry points; `ws` / `ws_bytes` is the scratch the
// SCAN mode uses (the caller's workspace, or the fixed per-device array).
hypic_status compose_impl(const hypic_compose_desc* d, hypic_stream_t stream, void* ws_ptr, size_t ws_bytes,
                          bool fixed_scratch) {
    hypic_status st = validate_compose(d);
    if (st != HYPIC_OK) return st;
    const int cus = planner_cus();
    const hypic_compose_mode m = resolve_mode(d, cus);
    const int kind = dense_T(d->kind) ? 0 : (d->kind == HYPIC_DIAG ? 1 : 2);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int D = d->d_k;
    const bool wantT = d->T_total != nullptr;
    int nblk = 1, B = d->n_elem;
    ScanLayout L;
    if (m == HYPIC_COMPOSE_SCAN && d->n_elem > 0) {
        B = scan_block_size(d, cus);
        nblk = (d->n_elem + B - 1) / B;
        L = scan_layout(d, nblk);
        if (fixed_scratch) {
            if (L.bytes > hypic::kNoAllocScratchBytes)
                return fail(HYPIC_ERR_UNSUPPORTED,
                            "compose_noalloc: this SCAN needs %zu bytes of scratch, the fixed per-device array "
                            "holds %zu (use hypic_compose with a workspace, or FOLD)",
                            L.bytes, hypic::kNoAllocScratchBytes);
            hipError_t e = hypic::noalloc_scratch(&ws_ptr);
            if (e != hipSuccess) return device_fail("compose_noalloc: scratch address", e);
            ws_bytes = hypic::kNoAllocScratchBytes;
        }
        if (!ws_ptr || ws_bytes < L.bytes)
            return fail(HYPIC_ERR_WORKSPACE_TOO_SMALL, "compose: workspace of %zu bytes needed, %zu given", L.bytes,
                        ws_ptr ? ws_bytes : (size_t)0);
        if (reinterpret_cast<uintptr_t>(ws_ptr) % kAlign)
            return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: workspace must be 256-byte aligned");
    }
    hipError_t e;
    if (m != HYPIC_COMPOSE_SCAN || d->n_elem == 0) {
        hypic::FoldArgs a{};
        a.kind = kind;
        a.n_chain = d->n_chain;
        a.n_elem = d->n_elem;
        a.per_block = std::max(1, d->n_elem);
        a.n_block = 1;
        a.slot = d->slot;
        a.T_hat = d->T_hat;
        a.T_exp = d->T_exp;
        a.S = d->S;
        a.init_S = d->S0;
        a.out_S = d->S_final;
        a.out_T = d->T_total;
        a.out_e = d->T_total_exp;
        a.prefix = d->S_prefix;
        a.naive = m == HYPIC_COMPOSE_NAIVE_ADD;
        if (kind == 0 && !a.naive && !wantT && d->n_elem > 0 && split_fold_better(d->n_chain, D, cus))
            e = hypic::launch_fold_split(a, D, s);
        else
            e = hypic::launch_fold(a, D, wantT ? 1 : 0, s);
        if (e != hipSuccess) return device_fail("compose: fold launch", e);
        return ok();
    }
    unsigned char* ws = static_cast<unsigned char*>(ws_ptr);
    float* aggT = reinterpret_cast<float*>(ws + L.aggT);
    int* aggE = reinterpret_cast<int*>(ws + L.aggE);
    float* aggS = reinterpret_cast<float*>(ws + L.aggS);
    float* pre = d->S_prefix ? reinterpret_cast<float*>(ws + L.pre) : nullptr;
    // 1) block aggregates (T_b, S_b) from (I, 0)
    hypic::FoldArgs a{};
    a.kind = kind;
    a.n_chain = d->n_chain;
    a.n_elem = d->n_elem;
    a.per_block = B;
    a.n_block = nblk;
    a.slot = d->slot;
    a.T_hat = d->T_hat;
    a.T_exp = d->T_exp;
    a.S = d->S;
    a.out_S = aggS;
    a.out_T = aggT;
    a.out_e = aggE;
    e = hypic::launch_fold(a, D, 1, s);
    if (e != hipSuccess) return device_fail("compose: scan reduce launch", e);
    // 2) fold over the block aggregates from S0: final state, block-entry states
    hypic::FoldArgs b{};
    b.kind = kind;
    b.n_chain = d->n_chain;
    b.n_elem = nblk;
    b.per_block = nblk;
    b.n_block = 1;
    b.T_hat = aggT;
    b.T_exp = aggE;
    b.S = aggS;
    b.init_S = d->S0;
    b.out_S = d->S_final;
    b.out_T = d->T_total;
    b.out_e = d->T_total_exp;
    b.prefix = pre;
    if (kind == 0 && !wantT && split_fold_better(d->n_chain, D, cus))
        e = hypic::launch_fold_split(b, D, s);
    else
        e = hypic::launch_fold(b, D, wantT ? 1 : 0, s);
    if (e != hipSuccess) return device_fail("compose: scan of block aggregates launch", e);
    // 3) re-fold each block from its entry state, writing the per-element states
    if (d->S_prefix) {
        hypic::FoldArgs c{};
        c.kind = kind;
        c.n_chain = d->n_chain;
        c.n_elem = d->n_elem;
        c.per_block = B;
        c.n_block = nblk;
        c.slot = d->slot;
        c.T_hat = d->T_hat;
        c.T_exp = d->T_exp;
        c.S = d->S;
        c.init_S = pre;
        c.prefix = d->S_prefix;
        if (kind == 0 && split_fold_better((int64_t)d->n_chain * nblk, D, cus))
            e = hypic::launch_fold_split(c, D, s);
        else
            e = hypic::launch_fold(c, D, 0, s);
        if (e != hipSuccess) return device_fail("compose: scan re-fold launch", e);
    }
    return ok();
}

}  // namespace

hypic_status hypic_compose(const hypic_compose_desc* d, hypic_stream_t stream) {
    if (!d) return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose: desc is NULL");
    return compose_impl(d, stream, d->workspace, d->workspace_bytes, false);
}

hypic_status hypic_compose_noalloc(const hypic_compose_desc* d, hypic_stream_t stream) {
    if (!d) return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose_noalloc: desc is NULL");
    return compose_impl(d, stream, nullptr, 0, true);
}

// ------------------------------------------------------------------------------------------
// fused seam + compose (warm hit path)

namespace {

hypic_status validate_compose_seam(const hypic_seam_compose_desc* d) {
    if (!d) return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose_seam: desc is NULL");
    if (d->n_batch < 1 || d->h_k < 1 || d->h_v < 1 || d->h_v % d->h_k || d->n_elem < 0 || d->n_slot < 0 ||
        d->n_tokens < 0)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose_seam: bad geometry");
    if (d->d_k != d->d_v || !supported_d(d->d_k))
        return fail(HYPIC_ERR_UNSUPPORTED, "compose_seam: d_k=%d d_v=%d (supported: d_k == d_v in {64, 128})",
                    d->d_k, d->d_v);
    if ((int64_t)d->n_batch * d->h_v > 65535 * 1024)
        return fail(HYPIC_ERR_UNSUPPORTED, "compose_seam: too many chains");
    if ((d->in_dtype != HYPIC_F32 && d->in_dtype != HYPIC_BF16) ||
        (d->out_dtype != HYPIC_F32 && d->out_dtype != HYPIC_BF16))
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose_seam: unknown dtype");
    if (d->qk_l2norm != 0 && d->qk_l2norm != 1)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose_seam: qk_l2norm must be 0 or 1");
    if (!d->S_final) return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose_seam: S_final is NULL");
    if (!d->slot && d->n_slot < d->n_elem)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose_seam: slot is NULL but n_slot=%d < n_elem=%d", d->n_slot,
                    d->n_elem);
    hypic_status st = check_offsets(d->cu_seam, d->n_elem, d->n_tokens, "compose_seam: cu_seam");
    if (st != HYPIC_OK) return st;
    int64_t w_max = 0;
    for (int32_t i = 0; i < d->n_elem; ++i) w_max = std::max<int64_t>(w_max, d->cu_seam[i + 1] - d->cu_seam[i]);
    if (w_max > hypic::kFusedSeamMax)
        return fail(HYPIC_ERR_UNSUPPORTED, "compose_seam: a seam of %lld tokens (at most %d fused; use "
                    "hypic_seam_advance and hypic_compose)", (long long)w_max, hypic::kFusedSeamMax);
    if (d->n_elem > 0 && (!d->S || !d->T_hat || !d->T_exp))
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose_seam: T_hat, T_exp and S are required");
    if (d->T_hat && !aligned16(d->T_hat))
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose_seam: T_hat must be 16-byte aligned");
    if (w_max > 0 && (!d->q || !d->k || !d->v || !d->log_alpha || !d->beta))
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "compose_seam: q, k, v, log_alpha and beta are required");
    return HYPIC_OK;
}

}  // namespace

size_t hypic_compose_seam_workspace_bytes(const hypic_seam_compose_desc* d) {
    if (!d || d->n_elem < 0) return 0;
    return seg_table_layout(d->n_elem).bytes;
}

hypic_status hypic_compose_seam(const hypic_seam_compose_desc* d, hypic_stream_t stream) {
    hypic_status st = validate_compose_seam(d);
    if (st != HYPIC_OK) return st;
    const SegTableLayout L = seg_table_layout(d->n_elem);
    st = check_workspace("compose_seam", L.bytes, d->workspace, d->workspace_bytes);
    if (st != HYPIC_OK) return st;
    std::vector<int64_t> start(d->n_elem);
    std::vector<int32_t> len(d->n_elem);
    for (int32_t i = 0; i < d->n_elem; ++i) {
        start[i] = d->cu_seam[i];
        len[i] = (int32_t)(d->cu_seam[i + 1] - d->cu_seam[i]);
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hypic::FoldArgs a{};
    hipError_t e = fill_seg_table(a.seam_tab, L, d->workspace, start, len, {}, s);
    if (e != hipSuccess) return device_fail("compose_seam: table upload", e);
    a.kind = 0;
    a.n_chain = d->n_batch * d->h_v;
    a.n_elem = d->n_elem;
    a.per_block = std::max(1, d->n_elem);
    a.n_block = 1;
    a.slot = d->slot;
    a.T_hat = d->T_hat;
    a.T_exp = d->T_exp;
    a.S = d->S;
    a.init_S = d->S0;
    a.out_S = d->S_final;
    a.prefix = d->S_prefix;
    a.seam = 1;
    a.n_batch = d->n_batch;
    a.h_k = d->h_k;
    a.h_v = d->h_v;
    a.n_tokens = d->n_tokens;
    a.in_bf16 = d->in_dtype == HYPIC_BF16;
    a.out_bf16 = d->out_dtype == HYPIC_BF16;
    a.qk_l2norm = d->qk_l2norm;
    a.q = d->q;
    a.k = d->k;
    a.v = d->v;
    a.log_alpha = d->log_alpha;
    a.beta = d->beta;
    a.o = d->o;
    e = hypic::launch_fold(a, d->d_k, 0, s);
    if (e != hipSuccess) return device_fail("compose_seam: launch", e);
    return ok();
}

// ------------------------------------------------------------------------------------------
// seam advance

namespace {

hypic_status validate_seam(const hypic_seam_desc* d) {
    if (!d) return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam: desc is NULL");
    if (d->in_dtype != HYPIC_F32 && d->in_dtype != HYPIC_BF16)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam: unknown in_dtype %d", (int)d->in_dtype);
    if (d->out_dtype != HYPIC_F32 && d->out_dtype != HYPIC_BF16)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam: unknown out_dtype %d", (int)d->out_dtype);
    if (d->n_batch < 1 || d->n_tokens < 0 || d->h_k < 1 || d->h_v < 1 || d->h_v % d->h_k)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam: bad geometry");
    if (d->d_k != d->d_v || !supported_d(d->d_k))
        return fail(HYPIC_ERR_UNSUPPORTED, "seam: d_k=%d d_v=%d (supported: d_k == d_v in {64, 128})", d->d_k, d->d_v);
    if (d->qk_l2norm != 0 && d->qk_l2norm != 1) return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam: qk_l2norm must be 0/1");
    hypic_status st = check_offsets(d->cu_seam, d->n_seam, d->n_tokens, "seam: cu_seam");
    if (st != HYPIC_OK) return st;
    if ((int64_t)d->n_seam * d->n_batch * d->h_v > INT32_MAX) return fail(HYPIC_ERR_UNSUPPORTED, "seam: too many tasks");
    if (d->n_tokens > 0 && d->n_seam > 0) {
        if (!d->k || !d->v || !d->log_alpha || !d->beta)
            return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam: k, v, log_alpha and beta are required");
        if (!aligned16(d->k) || !aligned16(d->v) || (d->q && !aligned16(d->q)))
            return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam: q, k and v must be 16-byte aligned");
    }
    if (d->o && !d->q) return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam: o requested without q");
    if ((d->T_hat == nullptr) != (d->T_exp == nullptr))
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam: T_hat and T_exp must be both set or both NULL");
    const int64_t dense = (int64_t)d->n_batch * d->h_v * d->d_k * d->d_v;
    if (d->state_stride != 0 && d->state_stride < dense)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam: state_stride %lld overlaps seams (minimum %lld)",
                    (long long)d->state_stride, (long long)dense);
    if (d->precision < HYPIC_PREC_AUTO || d->precision > HYPIC_PREC_F16_PRECISE_T)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "seam: unknown precision");
    // seams of at most kSeamShort tokens run in float32 vector arithmetic at any d; longer
    // ones run the chunk engine, whose float32-operand plan covers d = 64 only
    int64_t w_max = 0;
    for (int32_t i = 0; i < d->n_seam; ++i) w_max = std::max<int64_t>(w_max, d->cu_seam[i + 1] - d->cu_seam[i]);
    if (w_max > hypic::kSeamShort && d->d_k != 64) {
        if (d->precision == HYPIC_PREC_F32)
            return fail(HYPIC_ERR_UNSUPPORTED, "seam: the F32 operand plan supports d = 64 only (seams > %d tokens)",
                        hypic::kSeamShort);
        if (d->precision == HYPIC_PREC_AUTO && d->in_dtype == HYPIC_F32)
            return fail(HYPIC_ERR_UNSUPPORTED,
                        "seam: float32 inputs at d = %d with seams longer than %d tokens have no float32-operand "
                        "plan; request HYPIC_PREC_F16 explicitly to accept f16 operands", d->d_k, hypic::kSeamShort);
    }
    return HYPIC_OK;
}

}  // namespace

size_t hypic_seam_advance_workspace_bytes(const hypic_seam_desc* d) {
    if (!d || d->n_seam < 0) return 0;
    return seg_table_layout(d->n_seam).bytes;
}

hypic_status hypic_seam_advance(const hypic_seam_desc* d, hypic_stream_t stream) {
    hypic_status st = validate_seam(d);
    if (st != HYPIC_OK) return st;
    const int64_t n_tasks = (int64_t)d->n_seam * d->n_batch * d->h_v;
    if (n_tasks == 0) return ok();
    const SegTableLayout L = seg_table_layout(d->n_seam);
    st = check_workspace("seam", L.bytes, d->workspace, d->workspace_bytes);
    if (st != HYPIC_OK) return st;
    std::vector<int64_t> start(d->n_seam);
    std::vector<int32_t> len(d->n_seam);
    for (int32_t i = 0; i < d->n_seam; ++i) {
        start[i] = d->cu_seam[i];
        len[i] = (int32_t)(d->cu_seam[i + 1] - d->cu_seam[i]);
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hypic::SegTable tab{};
    hipError_t e = fill_seg_table(tab, L, d->workspace, start, len, {}, s);
    if (e != hipSuccess) return device_fail("seam: table upload", e);
    const int64_t dense = (int64_t)d->n_batch * d->h_v * d->d_k * d->d_v;
    const bool f32 = d->precision == HYPIC_PREC_F32 ||
                     (d->precision == HYPIC_PREC_AUTO && d->in_dtype == HYPIC_F32 && d->d_k == 64);
    const int w_max = *std::max_element(len.begin(), len.end());
    if (w_max <= hypic::kSeamShort && d->d_k == d->d_v) {
        // short seams: closed rank-w form, fp32 arithmetic, every output in one launch
        hypic::SeamArgs q{};
        q.n_batch = d->n_batch;
        q.n_tokens = d->n_tokens;
        q.h_k = d->h_k;
        q.h_v = d->h_v;
        q.qk_l2norm = d->qk_l2norm;
        q.in_bf16 = d->in_dtype == HYPIC_BF16;
        q.out_bf16 = d->out_dtype == HYPIC_BF16;
        q.seg = tab;
        q.n_tasks = (int)n_tasks;
        q.q = d->q;
        q.k = d->k;
        q.v = d->v;
        q.log_alpha = d->log_alpha;
        q.beta = d->beta;
        q.S_in = d->S_in;
        q.in_stride = d->state_stride ? d->state_stride : dense;
        q.S_out = d->S_out;
        q.out_stride = d->state_stride ? d->state_stride : dense;
        q.o = d->o;
        q.T_hat = d->T_hat;
        q.T_exp = d->T_exp;
        q.S_seam = d->S_seam;
        e = hypic::launch_seam(q, d->d_k, w_max, s);
        if (e != hipSuccess) return device_fail("seam: short-seam launch", e);
        return ok();
    }
    hypic::EngineArgs a{};
    a.n_batch = d->n_batch;
    a.n_tokens = d->n_tokens;
    a.h_k = d->h_k;
    a.h_v = d->h_v;
    a.n_seg = d->n_seam;
    a.qk_l2norm = d->qk_l2norm;
    a.in_bf16 = d->in_dtype == HYPIC_BF16;
    a.out_bf16 = d->out_dtype == HYPIC_BF16;
    a.seg = tab;
    a.n_tasks = (int)n_tasks;
    a.k = d->k;
    a.v = d->v;
    a.log_alpha = d->log_alpha;
    a.beta = d->beta;
    if (d->o || d->S_out || d->T_hat) {
        hypic::EngineArgs r = a;
        r.q = d->o ? d->q : nullptr;
        r.o = d->o;
        r.S_in = d->S_in;
        r.in_stride = d->state_stride ? d->state_stride : dense;
        r.S_out = d->S_out;
        r.out_stride = d->state_stride ? d->state_stride : dense;
        r.T_hat = d->T_hat;
        r.T_exp = d->T_exp;
        e = hypic::launch_dense_engine(r, d->d_k, f32 ? 1 : 0, (int)n_tasks, s);
        if (e != hipSuccess) return device_fail("seam: engine launch", e);
    }
    if (d->S_seam) {
        // the seam's own zero-start state (its transition comes from the run above)
        hypic::EngineArgs r = a;
        r.S_out = d->S_seam;
        r.out_stride = dense;
        e = hypic::launch_dense_engine(r, d->d_k, f32 ? 1 : 0, (int)n_tasks, s);
        if (e != hipSuccess) return device_fail("seam: zero-start engine launch", e);
    }
    return ok();
}

// ------------------------------------------------------------------------------------------
// RoPE state re-rotation

hypic_status hypic_state_rerotate(const hypic_rerotate_desc* d, hypic_stream_t stream) {
    if (!d) return fail(HYPIC_ERR_INVALID_ARGUMENT, "rerotate: desc is NULL");
    if (d->kind == HYPIC_DIAG || d->kind == HYPIC_KDA)
        return fail(HYPIC_ERR_UNSUPPORTED,
                    "rerotate: per-channel gates do not commute with the RoPE rotation (only the dense and "
                    "scalar kinds re-rotate exactly)");
    if (d->kind != HYPIC_DENSE_DELTA && d->kind != HYPIC_SCALAR)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "rerotate: unknown kind %d", (int)d->kind);
    if (d->n_elem < 0 || d->n_chain < 1)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "rerotate: bad n_elem=%d n_chain=%d", d->n_elem, d->n_chain);
    if (d->d_k != d->d_v || !supported_d(d->d_k))
        return fail(HYPIC_ERR_UNSUPPORTED, "rerotate: d_k=%d d_v=%d (supported: d_k == d_v in {64, 128})", d->d_k,
                    d->d_v);
    if (d->rotary_dim < 2 || d->rotary_dim > d->d_k || d->rotary_dim % 2)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "rerotate: rotary_dim=%d must be even and in [2, d_k]", d->rotary_dim);
    if (d->interleaved != 0 && d->interleaved != 1)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "rerotate: interleaved must be 0 or 1");
    if (!(d->rope_base > 0.0) || d->rope_base > 1e30)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "rerotate: rope_base %g must be positive and finite", d->rope_base);
    if ((int64_t)d->n_chain > INT32_MAX / 2) return fail(HYPIC_ERR_UNSUPPORTED, "rerotate: too many chains");
    if (d->n_elem == 0) return ok();
    if (!d->delta) return fail(HYPIC_ERR_INVALID_ARGUMENT, "rerotate: delta is NULL");
    if (!d->S_in || !d->S_out) return fail(HYPIC_ERR_INVALID_ARGUMENT, "rerotate: S_in and S_out are required");
    const bool dense = d->kind == HYPIC_DENSE_DELTA;
    if (dense && (!d->T_hat_in || !d->T_hat_out))
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "rerotate: the dense kind needs T_hat_in and T_hat_out");
    hypic::RotArgs r{};
    r.n_chain = d->n_chain;
    r.rotary_dim = d->rotary_dim;
    r.interleaved = d->interleaved;
    r.dense = dense ? 1 : 0;
    r.log2_base = std::log2(d->rope_base);
    r.T_in = dense ? d->T_hat_in : nullptr;
    r.T_out = dense ? d->T_hat_out : nullptr;
    r.S_in = d->S_in;
    r.S_out = d->S_out;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int32_t e0 = 0; e0 < d->n_elem; e0 += hypic::kRotInline) {
        const int n = std::min<int32_t>(hypic::kRotInline, d->n_elem - e0);
        r.elem0 = e0;
        for (int i = 0; i < n; ++i) r.delta[i] = d->delta[e0 + i];
        hipError_t e = hypic::launch_rerotate(r, d->d_k, n, s);
        if (e != hipSuccess) return device_fail("rerotate: launch", e);
    }
    return ok();
}

// ------------------------------------------------------------------------------------------
// conv warm-up

namespace {

hypic_status validate_conv(const hypic_conv_desc* d) {
    if (!d) return fail(HYPIC_ERR_INVALID_ARGUMENT, "conv: desc is NULL");
    if ((d->in_dtype != HYPIC_F32 && d->in_dtype != HYPIC_BF16) ||
        (d->out_dtype != HYPIC_F32 && d->out_dtype != HYPIC_BF16))
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "conv: unknown dtype");
    if (d->width != 4) return fail(HYPIC_ERR_UNSUPPORTED, "conv: width=%d (supported: 4)", d->width);
    if (d->n_batch < 1 || d->n_tokens < 0 || d->channels < 1)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "conv: bad geometry");
    if (d->channels % 8) return fail(HYPIC_ERR_UNSUPPORTED, "conv: channels=%d is not a multiple of 8", d->channels);
    if (d->activation != HYPIC_ACT_NONE && d->activation != HYPIC_ACT_SILU)
        return fail(HYPIC_ERR_INVALID_ARGUMENT, "conv: unknown activation");
    hypic_status st = check_offsets(d->cu_seqlens, d->n_seg, d->n_tokens, "conv: cu_seqlens");
    if (st != HYPIC_OK) return st;
    if (d->n_seg > 65535 || d->n_batch > 65535) return fail(HYPIC_ERR_UNSUPPORTED, "conv: too many segments/batches");
    if (d->n_seg > 0) {
        if (!d->weight) return fail(HYPIC_ERR_INVALID_ARGUMENT, "conv: weight is NULL");
        if (d->n_tokens > 0 && (!d->x || !d->y)) return fail(HYPIC_ERR_INVALID_ARGUMENT, "conv: x and y are required");
        if ((d->x && !aligned16(d->x)) || (d->y && !aligned16(d->y)) || (d->state_in && !aligned16(d->state_in)) ||
            (d->state_out && !aligned16(d->state_out)))
            return fail(HYPIC_ERR_INVALID_ARGUMENT, "conv: x, y and states must be 16-byte aligned");
        if (d->state_in && !d->state_index && d->n_state < d->n_seg)
            return fail(HYPIC_ERR_INVALID_ARGUMENT, "conv: state_index is NULL but n_state=%d < n_seg=%d", d->n_state,
                        d->n_seg);
    }
    return HYPIC_OK;
}

}  // namespace

size_t hypic_conv_warmup_workspace_bytes(const hypic_conv_desc* d) {
    if (!d || d->n_seg < 0) return 0;
    return seg_table_layout(d->n_seg).bytes;
}

hypic_status hypic_conv_warmup(const hypic_conv_desc* d, hypic_stream_t stream) {
    hypic_status st = validate_conv(d);
    if (st != HYPIC_OK) return st;
    if (d->n_seg == 0) return ok();
    const SegTableLayout L = seg_table_layout(d->n_seg);
    st = check_workspace("conv", L.bytes, d->workspace, d->workspace_bytes);
    if (st != HYPIC_OK) return st;
    std::vector<int64_t> start(d->n_seg);
    std::vector<int32_t> len(d->n_seg);
    int64_t span = 3;
    for (int32_t i = 0; i < d->n_seg; ++i) {
        start[i] = d->cu_seqlens[i];
        len[i] = (int32_t)(d->cu_seqlens[i + 1] - d->cu_seqlens[i]);
        span = std::max<int64_t>(span, len[i]);
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hypic::SegTable tab{};
    hipError_t e = fill_seg_table(tab, L, d->workspace, start, len, {}, s);
    if (e != hipSuccess) return device_fail("conv: table upload", e);
    hypic::ConvArgs a{};
    a.n_batch = d->n_batch;
    a.n_tokens = d->n_tokens;
    a.channels = d->channels;
    a.n_seg = d->n_seg;
    a.in_bf16 = d->in_dtype == HYPIC_BF16;
    a.out_bf16 = d->out_dtype == HYPIC_BF16;
    a.silu = d->activation == HYPIC_ACT_SILU;
    a.seg = tab;
    a.x = d->x;
    a.state_in = d->state_in;
    a.n_state = d->n_state;
    a.state_index = d->state_index;
    a.weight = d->weight;
    a.bias = d->bias;
    a.y = d->y;
    a.state_out = d->state_out;
    e = hypic::launch_conv(a, span, s);
    if (e != hipSuccess) return device_fail("conv: launch", e);
    return ok();
}
