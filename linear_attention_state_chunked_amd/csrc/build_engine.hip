// Segment build of the dense kind (gated delta rule): T_C and S(C|0), warp-specialised.
//
// Per chunk of 64 tokens (chunked WY/UT form of the gated delta rule, see
// dense_engine.hip for the identities) the work splits into
//   * the carry  X = [T | S] <- Gamma X + K^T diag(Gamma/gamma) ([0 | U] - W' X),
//     the only sequential part (8.4 of 11.1 MFLOP per chunk and value head at d = 128);
//   * the chunk preparation: staging K and V, gate prefix, gram K K^T, the UT solve
//     Tg = (I + L)^-1 diag(beta), and W' = Tg diag(gamma) K, U = Tg V, none of which
//     depends on X.
// Carry waves (one per 32 columns of X, accumulators resident for the whole segment)
// run the carry of chunk c while four preparation waves stage chunk c+1, form its gram
// and solve it; both hand over through double-buffered LDS tiles.  Per chunk there are
// two workgroup barriers; the preparation waves order their own stages with a bounded
// LDS-counter barrier that the carry waves never wait on.
//
// The 64x64 unit lower-triangular solve is blocked: four 16x16 diagonal inverses by
// forward substitution (fp32), two 32x32 merges Inv = D - D N D (D block diagonal,
// N strictly block lower) and one 64x64 merge of the same form, the merges on the
// matrix cores with hi/lo-split f16 operands (about 22-bit operand precision).
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace hypic {

// ---------------------------------------------------------------------------------------
// precise products from fp32 data: f16 hi/lo split (three products) or plain fp32

template <class Op>
struct PF;
template <>
struct PF<OpF16> {
    halfx8 hi, lo;
};
template <>
struct PF<OpF32> {
    float v;
};

__device__ __forceinline__ PF<OpF16> pf_split8(const float (&x)[8]) {
    PF<OpF16> r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const _Float16 h = (_Float16)x[i];
        r.hi[i] = h;
        r.lo[i] = (_Float16)(x[i] - (float)h);
    }
    return r;
}

template <class Op>
__device__ __forceinline__ PF<Op> pf_lds(const float* p);
template <>
__device__ __forceinline__ PF<OpF16> pf_lds<OpF16>(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    return pf_split8(x);
}
template <>
__device__ __forceinline__ PF<OpF32> pf_lds<OpF32>(const float* p) {
    return {*p};
}

template <class Op>
__device__ __forceinline__ PF<Op> pf_acc(const floatx16& a, int st);
template <>
__device__ __forceinline__ PF<OpF16> pf_acc<OpF16>(const floatx16& a, int st) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = a[8 * st + i];
    return pf_split8(x);
}
template <>
__device__ __forceinline__ PF<OpF32> pf_acc<OpF32>(const floatx16& a, int st) {
    return {a[st]};
}

template <class Op>
__device__ __forceinline__ PF<Op> pf_zero();
template <>
__device__ __forceinline__ PF<OpF16> pf_zero<OpF16>() {
    PF<OpF16> r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.hi[i] = r.lo[i] = (_Float16)0.f;
    return r;
}
template <>
__device__ __forceinline__ PF<OpF32> pf_zero<OpF32>() {
    return {0.f};
}

__device__ __forceinline__ floatx16 pmma(const PF<OpF16>& a, const PF<OpF16>& b, floatx16 c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.lo, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.hi, b.lo, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a.hi, b.hi, c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 pmma(const PF<OpF32>& a, const PF<OpF32>& b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a.v, b.v, c, 0, 0, 0);
}

// raw 8-element input groups held in registers between prefetch and staging
template <bool BF16>
struct Raw8;
template <>
struct Raw8<true> {
    uint4 w;
    __device__ void load(const void* base, long long idx) {
        w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    }
    __device__ void zero() { w = make_uint4(0, 0, 0, 0); }
    __device__ void get(float (&x)[8]) const {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(ws[i] << 16);
            x[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
        }
    }
};
template <>
struct Raw8<false> {
    float4 a, b;
    __device__ void load(const void* base, long long idx) {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
        a = p[0];
        b = p[1];
    }
    __device__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ void get(float (&x)[8]) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};

// ---------------------------------------------------------------------------------------
// LDS layout (bytes)

template <int D, class Op>
struct BuildLayout {
    using E = typename Op::elem;
    static constexpr bool F32 = sizeof(E) == 4;
    static constexpr int PAD = F32 ? 1 : 8;          // f16 fragments are 16-byte loads
    static constexpr int RS_D = D + PAD;             // [token][d] rows
    static constexpr int RS_T = 64 + PAD;            // [d][token] and [token][token] rows
    static constexpr int LS = F32 ? 65 : 68;         // fp32 [64][LS]: L
    static constexpr int IS = F32 ? 33 : 36;         // fp32 32-wide blocks of the solve
    static constexpr int NB = D / 32;
    static constexpr int NST = 32 / Op::KS;
    static constexpr int sz_Wf = 2 * NB * 64 * 16 * (int)sizeof(E);
    static constexpr int sz_Kt = D * RS_T * (int)sizeof(E);
    static constexpr int sz_Sc = 80 * 4;
    static constexpr int sz_Kr = 64 * RS_D * (int)sizeof(E);
    static constexpr int sz_Inv = 192 * IS * 4;      // DT[64], DA[64], I1T[32], I2A[32] rows
    static constexpr int Wf0 = 0;                    // -W'^T tiles, fragment order (x2)
    static constexpr int Kt0 = Wf0 + 2 * sz_Wf;      // K^T, tokens in accumulator order (x2)
    static constexpr int Sc0 = Kt0 + 2 * sz_Kt;      // Gamma/gamma_i [64], Gamma (x2)
    static constexpr int Vt = Sc0 + 2 * sz_Sc;       // V^T staging
    static constexpr int KrInv = Vt + sz_Kt;         // K rows (gram), then the solve's blocks
    static constexpr int Lm = KrInv + (sz_Kr > sz_Inv ? sz_Kr : sz_Inv);
    static constexpr int TgA = Lm + 64 * LS * 4;     // Tg, [m][t acc order]
    static constexpr int TgG = TgA + 64 * RS_T * (int)sizeof(E);   // Tg diag(gamma)
    static constexpr int Gv = TgG + 64 * RS_T * (int)sizeof(E);    // G, gamma, beta
    static constexpr int Misc = Gv + 3 * 64 * 4;     // counter, per-wave exponents
    static constexpr int total = Misc + 32 * 4;
};

// bounded LDS-counter barrier among the preparation waves only
__device__ __forceinline__ void prep_barrier(int* cnt, int target, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    int spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1 << 22)) break;  // never hang: a broken invariant gives wrong data, not a hang
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int D, class Op, bool WITH_T, bool IN_BF16, bool PERSIST>
__global__ __launch_bounds__(((WITH_T ? 2 : 1) * D / 32 + 4) * 64) void gdn_build_kernel(EngineArgs a) {
    using E = typename Op::elem;
    using LY = BuildLayout<D, Op>;
    constexpr int NB = D / 32;
    constexpr int NC = (WITH_T ? 2 : 1) * NB;   // carry waves
    constexpr int NP = 4;                       // preparation waves
    constexpr int NT = (NC + NP) * 64;
    constexpr int KS = Op::KS, KH = Op::KH, NST = 32 / KS;
    constexpr int RS_D = LY::RS_D, RS_T = LY::RS_T, LS = LY::LS, IS = LY::IS;
    constexpr int G8 = D / 8;
    constexpr int NLD = 64 * G8 / (NP * 64);    // 8-element groups per prep thread per tensor

    __shared__ __align__(16) unsigned char smem[LY::total];
    int* sCnt = reinterpret_cast<int*>(smem + LY::Misc);
    int* sEw = sCnt + 4;

    const int tid = threadIdx.x;
    const int lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_c = wave < NC;
    const bool t_wave = WITH_T && wave < NB;
    const int col0 = ((WITH_T && !t_wave) ? wave - NB : wave) * 32;
    const long long N = a.n_tokens;

    {   // one-time init: Tg's upper-right 32x32 block is never written and must be zero
        E* tga = reinterpret_cast<E*>(smem + LY::TgA);
        E* tgg = reinterpret_cast<E*>(smem + LY::TgG);
        for (int i = tid; i < 64 * RS_T; i += NT) {
            tga[i] = Op::cvt(0.f);
            tgg[i] = Op::cvt(0.f);
        }
        if (tid == 0) sCnt[0] = 0;
    }
    int pb_target = 0;

    // Each role (T-column carry, S-column carry, preparation) runs its own copy of the task
    // and chunk loops with the same barrier sequence, so each is register-allocated on
    // its own instead of through one merged control-flow graph.
    auto run = [&](auto role) {
        constexpr int R = decltype(role)::value;  // 0: T carry, 1: S carry, 2: preparation
        for (int it = blockIdx.x; it < a.n_tasks; it += PERSIST ? (int)gridDim.x : a.n_tasks) {
            const int task = a.order ? a.order[it] : it;
            const int per_seg = a.n_batch * a.h_v;
            const int seg = task / per_seg;
            const int rem = task - seg * per_seg;
            const int b = rem / a.h_v;
            const int h = rem - b * a.h_v;
            const int hk = (h * a.h_k) / a.h_v;
            const long long start = a.seg_start[seg];
            const int len = a.seg_len[seg];
            const int nc = (len + 63) / 64;
            const long long chain_off = (long long)b * a.h_v + h;
            __syncthreads();
            if constexpr (R != 2) {
                constexpr bool TR = R == 0;
                    // =============================== carry waves ===============================
                    // identity columns of X for the T waves; the opaque zero keeps the compiler from
                    // hoisting these 64 task-invariant values out of the task loop into registers
                    int tz = 0;
                    asm volatile("" : "+v"(tz));
                    const int diag = col0 + l32 + tz - 4 * half;
                    floatx16 X[NB];
        #pragma unroll
                    for (int xb = 0; xb < NB; ++xb)
        #pragma unroll
                        for (int j = 0; j < 16; ++j)
                            X[xb][j] = (TR && 32 * xb + 8 * (j >> 2) + (j & 3) == diag) ? 1.f : 0.f;
                    floatx16 Un[2];
                    Un[0] = Un[1] = zero16();
                    int ew = 0;
                    for (int c = -1; c < nc; ++c) {
                        // opaque zeros: per-ln LDS offsets are recomputed every chunk instead of
                        // being hoisted out of the loop into long-lived registers
                        int lz = 0, lzv = 0;
                        asm volatile("" : "+s"(lz));
                        asm volatile("" : "+v"(lzv));
                        unsigned char* sm = smem + lz;
                        const int ln = lane + lzv, hf = ln >> 5, lq = ln & 31;
                        const int p = c & 1, pn = (c + 1) & 1;
                        if (c >= 0) {
                            const E* Wf = reinterpret_cast<const E*>(sm + LY::Wf0 + p * LY::sz_Wf);
                            const E* Kt = reinterpret_cast<const E*>(sm + LY::Kt0 + p * LY::sz_Kt);
                            const float* Sc = reinterpret_cast<const float*>(sm + LY::Sc0 + p * LY::sz_Sc);
                            floatx16 Vn[2];
        #pragma unroll
                            for (int mt = 0; mt < 2; ++mt) {
                                Vn[mt] = TR ? zero16() : Un[mt];
        #pragma unroll
                                for (int kb = 0; kb < NB; ++kb)
        #pragma unroll
                                    for (int st = 0; st < NST; ++st) {
                                        const auto fa = Op::load(Wf + (((mt * NB + kb) * NST + st) * 64 + ln) * KH);
                                        Vn[mt] = Op::mma(fa, Op::from_acc(X[kb], st), Vn[mt]);
                                    }
        #pragma unroll
                                for (int j = 0; j < 16; ++j) Vn[mt][j] *= Sc[32 * mt + acc_row(hf, j)];
                            }
                            const float Gamma = Sc[64];
        #pragma unroll
                            for (int xb = 0; xb < NB; ++xb) {
        #pragma unroll
                                for (int j = 0; j < 16; ++j) X[xb][j] *= Gamma;
        #pragma unroll
                                for (int mt = 0; mt < 2; ++mt)
        #pragma unroll
                                    for (int st = 0; st < NST; ++st) {
                                        const auto fa = Op::load(Kt + (32 * xb + lq) * RS_T + 32 * mt + 16 * hf + KH * st);
                                        X[xb] = Op::mma(fa, Op::from_acc(Vn[mt], st), X[xb]);
                                    }
                            }
                            if (TR) {
                                float m = 0.f;
        #pragma unroll
                                for (int xb = 0; xb < NB; ++xb)
        #pragma unroll
                                    for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(X[xb][j]));
                                const int e = exp2_of(wave_max(m));
                                if (e != 0) {
        #pragma unroll
                                    for (int xb = 0; xb < NB; ++xb)
        #pragma unroll
                                        for (int j = 0; j < 16; ++j) X[xb][j] = ldexpf(X[xb][j], -e);
                                    ew += e;
                                }
                            }
                        }
                        __syncthreads();  // preparation of chunk c+1 is complete
                        if (c + 1 < nc) {
                            const E* Ktn = reinterpret_cast<const E*>(sm + LY::Kt0 + pn * LY::sz_Kt);
                            const E* TgA = reinterpret_cast<const E*>(sm + LY::TgA);
                            const E* TgG = reinterpret_cast<const E*>(sm + LY::TgG);
                            const E* Vt = reinterpret_cast<const E*>(sm + LY::Vt);
                            E* Wfn = reinterpret_cast<E*>(sm + LY::Wf0 + pn * LY::sz_Wf);
                            // -W'^T tiles (d rows, token columns): their accumulators are exactly
                            // the operand fragments of W' X in the carry, stored in that order
                            if (TR || !WITH_T) {
                                const int dt = WITH_T ? wave : wave;
        #pragma unroll
                                for (int mt = 0; mt < 2; ++mt) {
                                    floatx16 acc = zero16();
        #pragma unroll
                                    for (int kk = 0; kk < 64 / KS; ++kk) {
                                        const auto fa = Op::load(Ktn + (32 * dt + lq) * RS_T + KS * kk + KH * hf);
                                        const auto fb = Op::load(TgG + (32 * mt + lq) * RS_T + KS * kk + KH * hf);
                                        acc = Op::mma(fa, fb, acc);
                                    }
        #pragma unroll
                                    for (int st = 0; st < NST; ++st) {
                                        E* dst = Wfn + (((mt * NB + dt) * NST + st) * 64 + ln) * KH;
        #pragma unroll
                                        for (int i = 0; i < KH; ++i) dst[i] = Op::cvt(-acc[KH * st + i]);
                                    }
                                }
                            }
                            if (!TR) {
        #pragma unroll
                                for (int mt = 0; mt < 2; ++mt) {
                                    floatx16 acc = zero16();
        #pragma unroll
                                    for (int kk = 0; kk < 64 / KS; ++kk) {
                                        const auto fa = Op::load(TgA + (32 * mt + lq) * RS_T + KS * kk + KH * hf);
                                        const auto fb = Op::load(Vt + (col0 + lq) * RS_T + KS * kk + KH * hf);
                                        acc = Op::mma(fa, fb, acc);
                                    }
                                    Un[mt] = acc;
                                }
                            }
                        }
                        __syncthreads();  // W'(c+1) written; staging buffers free
                    }
                    // epilogue: align the T waves' exponents, write T_hat / T_exp / S
                    if (TR && lane == 0) sEw[wave] = ew;
                    __syncthreads();
                    if (TR) {
                        int emax = sEw[0];
        #pragma unroll
                        for (int w = 1; w < NB; ++w) emax = max(emax, sEw[w]);
                        float* dst = a.T_hat + ((long long)seg * a.n_batch * a.h_v + chain_off) * D * D + col0 +
                                     (4 * half) * D + l32;
        #pragma unroll
                        for (int xb = 0; xb < NB; ++xb)
        #pragma unroll
                            for (int j = 0; j < 16; ++j)
                                dst[(32 * xb + 8 * (j >> 2) + (j & 3)) * D] = ldexpf(X[xb][j], ew - emax);
                        if (wave == 0 && lane == 0) a.T_exp[(long long)seg * a.n_batch * a.h_v + chain_off] = emax;
                    } else {
                        float* dst = a.S_out + seg * a.out_stride + chain_off * D * D + col0 + (4 * half) * D + l32;
        #pragma unroll
                        for (int xb = 0; xb < NB; ++xb)
        #pragma unroll
                            for (int j = 0; j < 16; ++j) dst[(32 * xb + 8 * (j >> 2) + (j & 3)) * D] = X[xb][j];
                    }
            } else {
                // ============================ preparation waves ============================
                const int pw = wave - NC;
                const int ptid = tid - NC * 64;
                Raw8<IN_BF16> pk[NLD], pv[NLD];
                float pla = 0.f, pbt = 0.f;
                auto prefetch = [&](int cc, int ln, int pt) {
                    const long long tok0 = start + 64LL * cc;
                    const int valid = min(64, len - 64 * cc);
    #pragma unroll
                    for (int r = 0; r < NLD; ++r) {
                        const int i = pt + NP * 64 * r;
                        const int t = i / G8, d0 = 8 * (i % G8);
                        if (t < valid) {
                            pk[r].load(a.k, ((b * N + tok0 + t) * a.h_k + hk) * D + d0);
                            pv[r].load(a.v, ((b * N + tok0 + t) * a.h_v + h) * D + d0);
                        } else {
                            pk[r].zero();
                            pv[r].zero();
                        }
                    }
                    if (pw == 0) {
                        const bool ok = ln < valid;
                        const long long gi = (b * N + tok0 + ln) * a.h_v + h;
                        pla = ok ? a.log_alpha[gi] : 0.f;
                        pbt = ok ? a.beta[gi] : 0.f;
                    }
                };
                auto pbar = [&]() {
                    pb_target += NP;
                    prep_barrier(sCnt, pb_target, lane);
                };
                if (nc > 0) prefetch(0, lane, ptid);
                for (int c = -1; c < nc; ++c) {
                    int lz = 0, lzv = 0;
                    asm volatile("" : "+s"(lz));
                    asm volatile("" : "+v"(lzv));
                    unsigned char* sm = smem + lz;
                    const int ln = lane + lzv, hf = ln >> 5, lq = ln & 31, pt = ptid + lzv;
                    const int pn = (c + 1) & 1;
                    if (c + 1 < nc) {
                        E* Kr = reinterpret_cast<E*>(sm + LY::KrInv);
                        E* Ktn = reinterpret_cast<E*>(sm + LY::Kt0 + pn * LY::sz_Kt);
                        E* Vt = reinterpret_cast<E*>(sm + LY::Vt);
                        float* Scn = reinterpret_cast<float*>(sm + LY::Sc0 + pn * LY::sz_Sc);
                        float* L = reinterpret_cast<float*>(sm + LY::Lm);
                        float* sG = reinterpret_cast<float*>(sm + LY::Gv);
                        float* sGam = sG + 64;
                        float* sBeta = sG + 128;
                        E* TgA = reinterpret_cast<E*>(sm + LY::TgA);
                        E* TgG = reinterpret_cast<E*>(sm + LY::TgG);
                        float* DT = reinterpret_cast<float*>(sm + LY::KrInv);
                        float* DA = DT + 64 * IS;
                        float* I1T = DT + 128 * IS;
                        float* I2A = DT + 160 * IS;

                        // ---- stage chunk c+1 from the prefetch registers
    #pragma unroll
                        for (int r = 0; r < NLD; ++r) {
                            const int i = pt + NP * 64 * r;
                            const int t = i / G8, d0 = 8 * (i % G8);
                            float x[8];
                            pk[r].get(x);
                            if (a.qk_l2norm) {
                                float ss = 0.f;
    #pragma unroll
                                for (int u = 0; u < 8; ++u) ss += x[u] * x[u];
    #pragma unroll
                                for (int o = 1; o < G8; o <<= 1) ss += __shfl_xor(ss, o, 64);
                                const float sc = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
    #pragma unroll
                                for (int u = 0; u < 8; ++u) x[u] *= sc;
                            }
    #pragma unroll
                            for (int u = 0; u < 8; ++u) {
                                const E e = Op::cvt(x[u]);
                                Kr[t * RS_D + acc_pos(d0 + u)] = e;
                                Ktn[(d0 + u) * RS_T + acc_pos(t)] = e;
                            }
                            pv[r].get(x);
    #pragma unroll
                            for (int u = 0; u < 8; ++u) Vt[(d0 + u) * RS_T + acc_pos(t)] = Op::cvt(x[u]);
                        }
                        if (pw == 0) {
                            const float G = wave_inclusive_scan(pla, ln);
                            const float Glast = __shfl(G, 63, 64);
                            sG[ln] = G;
                            sGam[ln] = expf(G);
                            sBeta[ln] = pbt;
                            Scn[ln] = expf(Glast - G);
                            if (ln == 0) Scn[64] = expf(Glast);
                        }
                        if (c + 2 < nc) prefetch(c + 2, ln, pt);
                        pbar();

                        // ---- gram K K^T -> L (three lower 32x32 tiles)
                        if (pw < 3) {
                            const int ti = pw == 0 ? 0 : 1, tj = pw == 2 ? 1 : 0;
                            floatx16 acc = zero16();
    #pragma unroll
                            for (int kk = 0; kk < D / KS; ++kk) {
                                const auto fa = Op::load(Kr + (32 * ti + lq) * RS_D + KS * kk + KH * hf);
                                const auto fb = Op::load(Kr + (32 * tj + lq) * RS_D + KS * kk + KH * hf);
                                acc = Op::mma(fa, fb, acc);
                            }
                            const int jc = 32 * tj + lq;
                            const float Gj = sG[jc];
    #pragma unroll
                            for (int j = 0; j < 16; ++j) {
                                const int i = 32 * ti + acc_row(hf, j);
                                L[i * LS + jc] = (i > jc) ? sBeta[i] * expf(sG[i] - Gj) * acc[j] : 0.f;
                            }
                        }
                        pbar();

                        // ---- solve 1: inverse of diagonal 16x16 block pw (forward substitution)
                        {
                            const int bb = pw, q = bb >> 1, o = 16 * (bb & 1), cc = ln & 15;
                            if (ln < 16) {
                                float xr[16];
    #pragma unroll
                                for (int i = 0; i < 16; ++i) xr[i] = (i == cc) ? 1.f : 0.f;
    #pragma unroll
                                for (int m = 0; m < 16; ++m) {
                                    const float xm = xr[m];
    #pragma unroll
                                    for (int i = m + 1; i < 16; ++i) xr[i] -= L[(16 * bb + i) * LS + 16 * bb + m] * xm;
                                }
    #pragma unroll
                                for (int i = 0; i < 16; ++i) {
                                    DT[(32 * q + o + cc) * IS + o + i] = xr[i];
                                    DA[(32 * q + o + i) * IS + acc_pos(o + cc)] = xr[i];
                                    DT[(32 * q + o + cc) * IS + (16 - o) + i] = 0.f;
                                    DA[(32 * q + o + i) * IS + acc_pos((16 - o) + cc)] = 0.f;
                                }
                            }
                        }
                        pbar();

                        // ---- solve 2: 32x32 merges  Inv' = D' - D' N D'
                        if (pw < 2) {
                            const int q = pw;
                            floatx16 P = zero16();
    #pragma unroll
                            for (int st = 0; st < NST; ++st) {
                                const int k0 = KS * st + KH * hf;
                                const auto fa = (lq >= 16 && k0 < 16) ? pf_lds<Op>(L + (32 * q + lq) * LS + 32 * q + k0)
                                                                       : pf_zero<Op>();
                                const auto fb = pf_lds<Op>(DT + (32 * q + lq) * IS + k0);
                                P = pmma(fa, fb, P);
                            }
                            floatx16 R = zero16();
    #pragma unroll
                            for (int st = 0; st < NST; ++st) {
                                const auto fa = pf_lds<Op>(DA + (32 * q + lq) * IS + 16 * hf + KH * st);
                                R = pmma(fa, pf_acc<Op>(P, st), R);
                            }
                            const int t = 32 * q + lq;
                            const float bt = sBeta[t], gbt = bt * sGam[t];
    #pragma unroll
                            for (int j = 0; j < 16; ++j) {
                                const int i = acc_row(hf, j);
                                const float inv = DT[(32 * q + lq) * IS + i] - R[j];
                                const int m = 32 * q + i;
                                TgA[m * RS_T + acc_pos(t)] = Op::cvt(inv * bt);
                                TgG[m * RS_T + acc_pos(t)] = Op::cvt(inv * gbt);
                                if (q == 0) I1T[lq * IS + i] = inv;
                                else I2A[i * IS + acc_pos(lq)] = inv;
                            }
                        }
                        pbar();

                        // ---- solve 3: 64x64 merge, lower-left block  -Inv'_1 L'_21 Inv'_0
                        if (pw == 0) {
                            floatx16 P = zero16();
    #pragma unroll
                            for (int st = 0; st < NST; ++st) {
                                const int k0 = KS * st + KH * hf;
                                P = pmma(pf_lds<Op>(L + (32 + lq) * LS + k0), pf_lds<Op>(I1T + lq * IS + k0), P);
                            }
                            floatx16 R = zero16();
    #pragma unroll
                            for (int st = 0; st < NST; ++st)
                                R = pmma(pf_lds<Op>(I2A + lq * IS + 16 * hf + KH * st), pf_acc<Op>(P, st), R);
                            const float bt = sBeta[lq], gbt = bt * sGam[lq];
    #pragma unroll
                            for (int j = 0; j < 16; ++j) {
                                const int m = 32 + acc_row(hf, j);
                                TgA[m * RS_T + acc_pos(lq)] = Op::cvt(-R[j] * bt);
                                TgG[m * RS_T + acc_pos(lq)] = Op::cvt(-R[j] * gbt);
                            }
                        }
                    }
                    __syncthreads();  // chunk c+1 prepared
                    __syncthreads();  // W'(c+1) written by the carry waves
                }
                __syncthreads();  // epilogue exponent exchange
            }
        }
    };
    if (is_c) {
        if (WITH_T && t_wave) run(std::integral_constant<int, 0>{});
        else run(std::integral_constant<int, 1>{});
    } else {
        run(std::integral_constant<int, 2>{});
    }
}

template <int D, class Op, bool WITH_T, bool IN_BF16>
static hipError_t launch_build_v(const EngineArgs& a, int grid, hipStream_t s) {
    constexpr int nt = ((WITH_T ? 2 : 1) * D / 32 + 4) * 64;
    if (a.persistent)
        hipLaunchKernelGGL((gdn_build_kernel<D, Op, WITH_T, IN_BF16, true>), dim3(grid), dim3(nt), 0, s, a);
    else
        hipLaunchKernelGGL((gdn_build_kernel<D, Op, WITH_T, IN_BF16, false>), dim3(grid), dim3(nt), 0, s, a);
    return hipGetLastError();
}

template <int D, class Op, bool IN_BF16>
static hipError_t launch_build_t(const EngineArgs& a, int grid, hipStream_t s) {
    return a.T_hat ? launch_build_v<D, Op, true, IN_BF16>(a, grid, s) : launch_build_v<D, Op, false, IN_BF16>(a, grid, s);
}

hipError_t launch_gdn_build(const EngineArgs& a, int d, int prec_f32, int grid, hipStream_t s) {
    const bool bf = a.in_bf16 != 0;
    if (d == 128 && !prec_f32) return bf ? launch_build_t<128, OpF16, true>(a, grid, s) : launch_build_t<128, OpF16, false>(a, grid, s);
    if (d == 64 && !prec_f32) return bf ? launch_build_t<64, OpF16, true>(a, grid, s) : launch_build_t<64, OpF16, false>(a, grid, s);
    if (d == 64 && prec_f32 && !bf) return launch_build_t<64, OpF32, false>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace hypic
