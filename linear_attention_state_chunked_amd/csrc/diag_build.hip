// Diagonal (GLA) and scalar (RetNet, Mamba2) segment build.
//
// With A_t = diag(alpha_t) the segment's transition and zero-start state have closed
// forms (decaying families of the HYPIC news article's linear-layer paragraph):
//   T = diag(exp(G_n)),   S(C|0) = sum_t diag(exp(G_n - G_t)) k_t v_t^T,
// with G_t = sum_{j<=t} log alpha_j per channel (one value for the scalar kind).
// S is one dense contraction over the segment's tokens: K~^T V with
// K~[t][c] = k_t[c] exp(G_n[c] - G_t[c]).  Chunks are visited from the end of the
// segment backwards so the decay exponent is a running suffix sum; K~ and V are
// staged in LDS (f16, contraction axis in accumulator order) and contracted on the
// matrix cores, the d x d state staying in accumulators.  One workgroup runs a segment's
// chunks in sequence, so its loads are issued two chunks ahead into alternating register
// sets: every chunk then waits on no HBM round trip of its own.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace hypic {

template <int D, class Op>
__global__ __launch_bounds__(512) void diag_build_kernel(DiagArgs a) {
    using E = typename Op::elem;
    // 16-bit inputs feed the f16 matrix cores, 32-bit inputs the f32 ones
    constexpr bool BF = std::is_same<Op, OpF16>::value;
    using KRaw = typename std::conditional<BF, uint16_t, float>::type;
    constexpr int PAD = 16 / (int)sizeof(E);
    constexpr int RS = 64 + PAD;
    constexpr int NT = 512;
    constexpr int KS = Op::KS, KH = Op::KH;
    constexpr int TILES = (D / 32) * (D / 32);
    constexpr int TPW = (TILES + 7) / 8;      // tiles per wave
    constexpr int NP = NT / D;                // token parts per chunk
    constexpr int TP = kChunk / NP;           // tokens per part
    // values: thread (cg, tg) stages channels [CPT*cg, CPT*cg + CPT) of tokens [4*tg, 4*tg + 4)
    constexpr int CPT = D / 32;
    constexpr int VWORDS = CPT * (int)sizeof(KRaw) / 4;  // 32-bit words per token and thread
    static_assert(32 * (kChunk / 4) == NT && (VWORDS == 1 || VWORDS == 2 || VWORDS == 4), "value staging map");
    using VVec = typename std::conditional<VWORDS == 1, uint32_t,
                 typename std::conditional<VWORDS == 2, uint2, uint4>::type>::type;
    static_assert(TP % 4 == 0 && (RS * sizeof(E)) % 16 == 0, "packed key writes stay aligned");
    __shared__ __align__(16) E sKd[D * RS];   // K~^T: [c][t]
    __shared__ __align__(16) E sVt[D * RS];   // V^T : [d][t]
    __shared__ float sR[D];                   // suffix sum per channel over the whole segment
    __shared__ float sPart[NT];               // per-part decay sums
    __shared__ float sMax;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const long long N = a.n_tokens;

    const int per_seg = a.n_batch * a.h_v;
    const int task = task_at(a.seg, blockIdx.x, per_seg);
    const int seg = task / per_seg;
    const int rem = task - seg * per_seg;
    const int b = rem / a.h_v, h = rem - (rem / a.h_v) * a.h_v;
    const int hk = (h * a.h_k) / a.h_v;
    const long long start = seg_start(a.seg, seg);
    const int len = seg_len(a.seg, seg);
    const long long chain = (long long)seg * a.n_batch * a.h_v + (long long)b * a.h_v + h;
    // thread (c, p): channel c of the decayed keys over token part p of a chunk
    // p is uniform over a wave (D >= 64): per-token offsets and bounds stay in scalar registers
    const int c = tid % D, p = __builtin_amdgcn_readfirstlane(tid / D);
    static_assert(D % kWave == 0, "token parts cover whole waves");
    const int cg = tid % 32, tg = tid / 32;

    floatx16 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = zero16();

    // One chunk's inputs as loaded, undecoded, so that the loads stay in flight until the
    // chunk is consumed two chunks later.  Rows past the segment's end are clamped to its
    // last token (in bounds) and zeroed at consumption.
    struct Regs {
        KRaw k[TP];
        float la[TP];
        VVec v[4];
    };
    // per-token strides (elements) of keys, gates and values; 32-bit offsets within a chunk
    const int ks = a.h_k * D, ls = a.scalar ? a.h_v : a.h_v * D, vs = a.h_v * D;
    const int lc = a.scalar ? 0 : c;
    auto load = [&](Regs& r, int ci) {
        const int c0 = ci * kChunk;
        const int last = min(kChunk, len - c0) - 1;
        const long long row0 = b * N + start + c0;  // first token row of the chunk (uniform)
        const KRaw* kb = reinterpret_cast<const KRaw*>(a.k) + (row0 * a.h_k + hk) * D;
        const float* lb = a.log_alpha + (a.scalar ? row0 * a.h_v + h : (row0 * a.h_v + h) * D);
        const KRaw* vb = reinterpret_cast<const KRaw*>(a.v) + (row0 * a.h_v + h) * D;
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const int t = min(p * TP + u, last);
            r.k[u] = kb[t * ks + c];
            r.la[u] = lb[t * ls + lc];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r.v[j] = *reinterpret_cast<const VVec*>(vb + min(4 * tg + j, last) * vs + CPT * cg);
    };
    float rR = 0.f;  // running suffix sum of the channel's log decays (same in every part)
    // Chunk ci < 0 is an all-zero step (adds exact zeros).  Every step issues its loads, so
    // the wait before a register set's use never covers the set loaded after it.
    auto step = [&](Regs& r, int ci) {
        const int valid = ci >= 0 ? min(kChunk, len - ci * kChunk) : 0;
        float kv[TP], la[TP];
        float tot = 0.f;
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const bool ok = p * TP + u < valid;
            kv[u] = ok ? (BF ? bf16_to_f32(r.k[u]) : (float)r.k[u]) : 0.f;
            la[u] = ok ? r.la[u] : 0.f;
            tot += la[u];
        }
        sPart[p * D + c] = tot;
        // values, transposed: each channel's four tokens are adjacent in the accumulator order
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            E x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = reinterpret_cast<const uint32_t*>(&r.v[j])[BF ? e >> 1 : e];
                const float f = BF ? (e & 1 ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16))
                                   : __uint_as_float(w);
                x[j] = Op::cvt(4 * tg + j < valid ? f : 0.f);
            }
            E* dst = sVt + (CPT * cg + e) * RS + acc_pos(4 * tg);
            if constexpr (BF) {
                *reinterpret_cast<halfx4*>(dst) = halfx4{x[0], x[1], x[2], x[3]};
            } else {
                *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
            }
        }
        __syncthreads();
        // decayed keys: suffix sums of the later parts come through LDS
        float run = rR;
        for (int q = p + 1; q < NP; ++q) run += sPart[q * D + c];
        E kd[TP];
#pragma unroll
        for (int u = TP - 1; u >= 0; --u) {
            // f16 operands: the hardware exp2 (about 1 ulp of fp32) is far below their rounding
            const float dec = BF ? __builtin_amdgcn_exp2f(run * 1.4426950408889634f) : expf(run);
            kd[u] = Op::cvt(kv[u] * dec);
            run += la[u];
        }
        // four consecutive tokens sit at four adjacent positions of the accumulator order
        // (rows 8- or 16-byte aligned): one write each
#pragma unroll
        for (int m = 0; m < TP / 4; ++m) {
            E* dst = sKd + c * RS + acc_pos(p * TP + 4 * m);
            if constexpr (BF) {
                halfx4 w = {kd[4 * m], kd[4 * m + 1], kd[4 * m + 2], kd[4 * m + 3]};
                *reinterpret_cast<halfx4*>(dst) = w;
            } else {
                *reinterpret_cast<float4*>(dst) = make_float4(kd[4 * m], kd[4 * m + 1], kd[4 * m + 2], kd[4 * m + 3]);
            }
        }
        float rn = rR;
        for (int q = 0; q < NP; ++q) rn += sPart[q * D + c];
        rR = rn;
        load(r, max(ci - 2, 0));
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tile = wave * TPW + i;
            if (tile >= TILES) break;
            const int tr = tile / (D / 32), tc = tile % (D / 32);
#pragma unroll
            for (int kk = 0; kk < kChunk / KS; ++kk) {
                const auto fa = Op::load(sKd + (32 * tr + l32) * RS + KS * kk + KH * half);
                const auto fb = Op::load(sVt + (32 * tc + l32) * RS + KS * kk + KH * half);
                acc[i] = Op::mma(fa, fb, acc[i]);
            }
        }
        __syncthreads();
    };

    // Chunks are visited from the end of the segment backwards, two register sets in turn.
    const int nchunk = (len + kChunk - 1) / kChunk;
    if (nchunk > 0) {
        Regs ra, rb;
        load(ra, nchunk - 1);
        // keep the first set's loads ahead of the second's, as in the loop, so that waiting
        // for one set never waits for the other
        __builtin_amdgcn_sched_barrier(0);
        load(rb, max(nchunk - 2, 0));
        for (int ci = nchunk - 1; ci >= 0; ci -= 2) {
            step(ra, ci);
            step(rb, ci - 1);
        }
    }
    if (p == 0) sR[c] = rR;
    __syncthreads();

    float* dS = a.S + chain * D * D;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int tile = wave * TPW + i;
        if (tile >= TILES) break;
        const int tr = tile / (D / 32), tc = tile % (D / 32);
#pragma unroll
        for (int j = 0; j < 16; ++j) dS[(32 * tr + acc_row(half, j)) * D + 32 * tc + l32] = acc[i][j];
    }
    if (a.T_hat) {
        // T = exp(G_n) per channel, written as T_hat * 2^e with max T_hat in (0.5, 1]
        if (wave == 0) {
            float m = -INFINITY;
            for (int c = lane; c < (a.scalar ? 1 : D); c += 64) m = fmaxf(m, sR[c]);
            m = wave_max(m);
            if (lane == 0) sMax = m;
        }
        __syncthreads();
        const float l2e = 1.4426950408889634f;
        const int e = (int)ceilf(sMax * l2e);
        if (a.scalar) {
            if (tid == 0) a.T_hat[chain] = exp2f(sR[0] * l2e - (float)e);
        } else if (tid < D) {
            a.T_hat[chain * D + tid] = exp2f(sR[tid] * l2e - (float)e);
        }
        if (tid == 0) a.T_exp[chain] = e;
    }
}

hipError_t launch_diag_build(const DiagArgs& a, int d, hipStream_t s) {
    const int grid = a.n_tasks;
    if (d == 128) {
        if (a.in_bf16) hipLaunchKernelGGL((diag_build_kernel<128, OpF16>), dim3(grid), dim3(512), 0, s, a);
        else hipLaunchKernelGGL((diag_build_kernel<128, OpF32>), dim3(grid), dim3(512), 0, s, a);
    } else if (d == 64) {
        if (a.in_bf16) hipLaunchKernelGGL((diag_build_kernel<64, OpF16>), dim3(grid), dim3(512), 0, s, a);
        else hipLaunchKernelGGL((diag_build_kernel<64, OpF32>), dim3(grid), dim3(512), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hypic
