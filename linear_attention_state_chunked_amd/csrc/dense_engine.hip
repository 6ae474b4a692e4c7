// Dense (gated delta rule) chunk engine: segment build and seam advance.
//
// For each chain the engine carries X = [T | S] (d x 2d) through the segment 64 tokens
// at a time with the chunked WY/UT form of the gated delta rule, T being the
// ordered product of the per-token transitions (the cached transition operator of
// the HYPIC news article's linear-layer paragraph) and S the state.  Per chunk
// (local tokens i = 0..63, masked tokens have k = v = q = 0, beta = 0, log alpha = 0):
//
//   G_i = sum_{j<=i} log alpha_j,  gamma_i = exp(G_i),  Gamma = gamma_63
//   L   = strictly-lower(diag(beta) (exp(G_i - G_j)) o K K^T)
//   Tg  = (I + L)^-1 diag(beta)                  (UT transform, blocked solve)
//   U   = Tg V,   W' = Tg diag(gamma) K
//   Vn  = ([0 | U] - W' X) scaled by rows by Gamma / gamma_i
//   X  <- Gamma X + K^T Vn
//   with q: o = diag(gamma) Q S + M (U - W' S),  M = lower(exp(G_i - G_j) o Q K^T)
//
// Work split (d = 128: 8 waves): wave w owns 32 columns of X, waves [0, d/32) the T
// columns and the rest the S columns; columns evolve independently, so waves only
// share the per-chunk K, W', U tiles in LDS.  X stays in matrix-core accumulators for
// the whole segment and is fed back as the B operand in place (see device_common.hpp).
// T columns are renormalised by an exact power of two after every chunk (one exponent
// per wave, aligned at the end) so long decaying segments never underflow.
#include "device_common.hpp"
#include "kernels.hpp"

namespace hypic {

template <int D, class Op, bool WITH_Q>
struct EngineLayout {
    using E = typename Op::elem;
    static constexpr int PAD = 16 / (int)sizeof(E);
    static constexpr int RS_D = D + PAD;    // [token][d] rows
    static constexpr int RS_T = 64 + PAD;   // [d][token] and [token][token] rows
    static constexpr int LS = 68;           // float [64][LS] for L and its inverse
    static constexpr int sz_rowD = 64 * RS_D * (int)sizeof(E);
    static constexpr int sz_dT = D * RS_T * (int)sizeof(E);
    static constexpr int sz_tT = 64 * RS_T * (int)sizeof(E);
    static constexpr int sz_L = 64 * LS * 4;
    static_assert(sz_L >= sz_rowD || true, "");
    static constexpr int Kr = 0;                         // K rows, d in acc order
    static constexpr int Kt = Kr + sz_rowD;              // K^T, tokens in acc order
    static constexpr int Vt = Kt + sz_dT;                // V^T
    static constexpr int Qq = Vt + sz_dT;                // Q rows (WITH_Q)
    static constexpr int TgA = Qq + (WITH_Q ? sz_rowD : 0);
    static constexpr int TgG = TgA + sz_tT;
    static constexpr int Lm = TgG + sz_tT;               // L, later -W' rows
    static constexpr int sz_LW = (sz_L > sz_rowD ? sz_L : sz_rowD);
    static constexpr int Inv = Lm + sz_LW;               // (I+L)^-1, later M
    static constexpr int sz_IM = (sz_L > sz_tT ? sz_L : sz_tT);
    static constexpr int P = Inv + sz_IM;                // 3 x 16 x 17 floats
    static constexpr int Vec = P + 3 * 16 * 17 * 4;      // G, gamma, beta, Gamma/gamma
    static constexpr int Misc = Vec + 4 * 64 * 4;        // Gamma, per-wave exponents
    static constexpr int total = Misc + 32 * 4;
};

// Row-major load / store of one 32x32 accumulator tile (row stride LD floats) from a
// per-lane base pointer, so that every element address is base + constant.
template <int LD>
__device__ __forceinline__ void store_tile(float* p, const floatx16& x, int half, int l32) {
    float* q = p + (4 * half) * LD + l32;
#pragma unroll
    for (int j = 0; j < 16; ++j) q[(8 * (j >> 2) + (j & 3)) * LD] = x[j];
}
template <int LD>
__device__ __forceinline__ void load_tile(const float* p, floatx16& x, int half, int l32) {
    const float* q = p + (4 * half) * LD + l32;
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = q[(8 * (j >> 2) + (j & 3)) * LD];
}

template <int D, class Op, bool WITH_Q, bool PERSIST>
__global__ __launch_bounds__(D * 4) void dense_engine_kernel(EngineArgs a) {
    using E = typename Op::elem;
    using LY = EngineLayout<D, Op, WITH_Q>;
    constexpr int NW = D / 16;       // waves: 2d columns / 32
    constexpr int NT = NW * 64;
    constexpr int NB = D / 32;       // 32-row blocks of d
    constexpr int KS = Op::KS, KH = Op::KH;
    constexpr int NST = 32 / KS;     // operand steps per 32-block
    constexpr int RS_D = LY::RS_D, RS_T = LY::RS_T, LS = LY::LS;
    constexpr int G8 = D / 8;        // 8-element groups per row

    __shared__ __align__(16) unsigned char smem_raw[LY::total];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const bool t_wave = wave < NW / 2;
    const int col0 = (t_wave ? wave : wave - NW / 2) * 32;
    const bool do_T = a.T_hat != nullptr;
    const bool in_bf16 = a.in_bf16 != 0;
    const long long N = a.n_tokens;

    // one task per workgroup, or a grid-stride loop over tasks (static round robin)
    for (int it = blockIdx.x; it < a.n_tasks; it += PERSIST ? (int)gridDim.x : a.n_tasks) {
        const int per_seg = a.n_batch * a.h_v;
        const int task = task_at(a.seg, it, per_seg);
        const int seg = task / per_seg;
        const int rem = task - seg * per_seg;
        const int b = rem / a.h_v;
        const int h = rem - b * a.h_v;
        const int hk = (h * a.h_k) / a.h_v;
        const long long start = seg_start(a.seg, seg);
        const int len = seg_len(a.seg, seg);
        const long long chain_off = (long long)b * a.h_v + h;

        // ---- X = [I | S_in]
        floatx16 X[NB];
        if (t_wave) {
#pragma unroll
            for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    X[xb][j] = (32 * xb + acc_row(half, j) == col0 + l32) ? 1.f : 0.f;
        } else if (a.S_in) {
            const float* src = a.S_in + seg * a.in_stride + chain_off * D * D + col0;
#pragma unroll
            for (int xb = 0; xb < NB; ++xb) load_tile<D>(src + 32 * xb * D, X[xb], half, l32);
        } else {
#pragma unroll
            for (int xb = 0; xb < NB; ++xb) X[xb] = zero16();
        }
        int ew = 0;

        for (int c0 = 0; c0 < len; c0 += kChunk) {
            const int valid = min(kChunk, len - c0);
            const long long tok0 = start + c0;
            // LDS views from an opaque zero offset: stops the compiler from hoisting every
            // per-lane LDS address out of the chunk loop into long-lived registers.
            int lz = 0;
            asm volatile("" : "+s"(lz));
            unsigned char* smem = smem_raw + lz;
            E* sKr = reinterpret_cast<E*>(smem + LY::Kr);
            E* sKt = reinterpret_cast<E*>(smem + LY::Kt);
            E* sVt = reinterpret_cast<E*>(smem + LY::Vt);
            E* sQq = reinterpret_cast<E*>(smem + LY::Qq);
            E* sTgA = reinterpret_cast<E*>(smem + LY::TgA);
            E* sTgG = reinterpret_cast<E*>(smem + LY::TgG);
            float* sL = reinterpret_cast<float*>(smem + LY::Lm);
            E* sWq = reinterpret_cast<E*>(smem + LY::Lm);
            float* sInv = reinterpret_cast<float*>(smem + LY::Inv);
            E* sMq = reinterpret_cast<E*>(smem + LY::Inv);
            float* sP = reinterpret_cast<float*>(smem + LY::P);
            float* sG = reinterpret_cast<float*>(smem + LY::Vec);
            float* sGam = sG + 64;
            float* sBeta = sG + 128;
            float* sSc = sG + 192;
            float* sMisc = reinterpret_cast<float*>(smem + LY::Misc);

            // ---------------- phase 1: stage the chunk in LDS, gate prefix
            for (int i = tid; i < 64 * G8; i += NT) {
                const int t = i / G8, d0 = 8 * (i - (i / G8) * G8);
                const bool ok = t < valid;
                float x[8];
                // keys
                if (ok) load8(a.k, ((b * N + tok0 + t) * a.h_k + hk) * D + d0, in_bf16, x);
                else {
#pragma unroll
                    for (int u = 0; u < 8; ++u) x[u] = 0.f;
                }
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
                    sKr[t * RS_D + acc_pos(d0 + u)] = e;
                    sKt[(d0 + u) * RS_T + acc_pos(t)] = e;
                }
                // values
                if (ok) load8(a.v, ((b * N + tok0 + t) * a.h_v + h) * D + d0, in_bf16, x);
                else {
#pragma unroll
                    for (int u = 0; u < 8; ++u) x[u] = 0.f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) sVt[(d0 + u) * RS_T + acc_pos(t)] = Op::cvt(x[u]);
                if (WITH_Q) {
                    if (ok) load8(a.q, ((b * N + tok0 + t) * a.h_k + hk) * D + d0, in_bf16, x);
                    else {
#pragma unroll
                        for (int u = 0; u < 8; ++u) x[u] = 0.f;
                    }
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
                    for (int u = 0; u < 8; ++u) sQq[t * RS_D + acc_pos(d0 + u)] = Op::cvt(x[u]);
                }
            }
            if (wave == 0) {
                const bool ok = lane < valid;
                const long long gi = (b * N + tok0 + lane) * a.h_v + h;
                const float la = ok ? a.log_alpha[gi] : 0.f;
                const float bt = ok ? a.beta[gi] : 0.f;
                const float G = wave_inclusive_scan(la, lane);
                const float Glast = __shfl(G, 63, 64);
                sG[lane] = G;
                sGam[lane] = expf(G);
                sBeta[lane] = bt;
                sSc[lane] = expf(Glast - G);
                if (lane == 0) sMisc[0] = expf(Glast);
            }
            __syncthreads();

            // ---------------- phase 2: gram K K^T -> L (lower 32x32 tiles)
            if (wave < 3) {
                const int ti = wave == 0 ? 0 : 1, tj = wave == 2 ? 1 : 0;
                floatx16 acc = zero16();
#pragma unroll 4
                for (int kk = 0; kk < D / KS; ++kk) {
                    const auto fa = Op::load(sKr + (32 * ti + l32) * RS_D + KS * kk + KH * half);
                    const auto fb = Op::load(sKr + (32 * tj + l32) * RS_D + KS * kk + KH * half);
                    acc = Op::mma(fa, fb, acc);
                }
                const int jc = 32 * tj + l32;
                const float Gj = sG[jc];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int i = 32 * ti + acc_row(half, j);
                    sL[i * LS + jc] = (i > jc) ? sBeta[i] * expf(sG[i] - Gj) * acc[j] : 0.f;
                }
            }
            __syncthreads();

            // ---------------- phase 3: Tg = (I + L)^-1 diag(beta), blocked by 16
            if (wave == 0) {
                const int bb = lane >> 4, c = lane & 15;
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float s = (i == c) ? 1.f : 0.f;
#pragma unroll
                    for (int m = 0; m < i; ++m) s -= sL[(16 * bb + i) * LS + 16 * bb + m] * x[m];
                    x[i] = s;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) sInv[(16 * bb + i) * LS + 16 * bb + c] = x[i];
            }
            __syncthreads();
            for (int lev = 1; lev < 4; ++lev) {
                const int nblk = 4 - lev;
                for (int e = tid; e < nblk * 256; e += NT) {
                    const int J = e >> 8, I = J + lev, r = (e >> 4) & 15, cc = e & 15;
                    float s = 0.f;
                    for (int K = J; K < I; ++K)
#pragma unroll
                        for (int m = 0; m < 16; ++m)
                            s += sL[(16 * I + r) * LS + 16 * K + m] * sInv[(16 * K + m) * LS + 16 * J + cc];
                    sP[(J * 16 + r) * 17 + cc] = s;
                }
                __syncthreads();
                for (int e = tid; e < nblk * 256; e += NT) {
                    const int J = e >> 8, I = J + lev, r = (e >> 4) & 15, cc = e & 15;
                    float s = 0.f;
#pragma unroll
                    for (int m = 0; m < 16; ++m) s += sInv[(16 * I + r) * LS + 16 * I + m] * sP[(J * 16 + m) * 17 + cc];
                    sInv[(16 * I + r) * LS + 16 * J + cc] = -s;
                }
                __syncthreads();
            }
            for (int e = tid; e < 64 * 64; e += NT) {
                const int m = e >> 6, t = e & 63;
                const float v = (t <= m) ? sInv[m * LS + t] * sBeta[t] : 0.f;
                sTgA[m * RS_T + acc_pos(t)] = Op::cvt(v);
                sTgG[m * RS_T + acc_pos(t)] = Op::cvt(v * sGam[t]);
            }
            __syncthreads();

            // ---------------- phase 4: W' (LDS, negated), U (S waves, registers), M
            {
                const int mt = wave / NB, dt = wave % NB;
                floatx16 acc = zero16();
#pragma unroll
                for (int kk = 0; kk < 64 / KS; ++kk) {
                    const auto fa = Op::load(sTgG + (32 * mt + l32) * RS_T + KS * kk + KH * half);
                    const auto fb = Op::load(sKt + (32 * dt + l32) * RS_T + KS * kk + KH * half);
                    acc = Op::mma(fa, fb, acc);
                }
                const int dcol = acc_pos(32 * dt + l32);
#pragma unroll
                for (int j = 0; j < 16; ++j) sWq[(32 * mt + acc_row(half, j)) * RS_D + dcol] = Op::cvt(-acc[j]);
            }
            floatx16 Un[2];
            if (!t_wave) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    floatx16 acc = zero16();
#pragma unroll
                    for (int kk = 0; kk < 64 / KS; ++kk) {
                        const auto fa = Op::load(sTgA + (32 * mt + l32) * RS_T + KS * kk + KH * half);
                        const auto fb = Op::load(sVt + (col0 + l32) * RS_T + KS * kk + KH * half);
                        acc = Op::mma(fa, fb, acc);
                    }
                    Un[mt] = acc;
                }
            }
            if (WITH_Q && t_wave) {
                for (int job = wave; job < 3; job += NW / 2) {
                    const int ti = job == 0 ? 0 : 1, tj = job == 2 ? 1 : 0;
                    floatx16 acc = zero16();
#pragma unroll 4
                    for (int kk = 0; kk < D / KS; ++kk) {
                        const auto fa = Op::load(sQq + (32 * ti + l32) * RS_D + KS * kk + KH * half);
                        const auto fb = Op::load(sKr + (32 * tj + l32) * RS_D + KS * kk + KH * half);
                        acc = Op::mma(fa, fb, acc);
                    }
                    const int jc = 32 * tj + l32;
                    const float Gj = sG[jc];
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int i = 32 * ti + acc_row(half, j);
                        sMq[i * RS_T + acc_pos(jc)] = Op::cvt((i >= jc) ? expf(sG[i] - Gj) * acc[j] : 0.f);
                    }
                }
            }
            __syncthreads();

            // ---------------- phase 5: carry (and outputs)
            if (!t_wave || do_T) {
                floatx16 Vn[2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    Vn[mt] = t_wave ? zero16() : Un[mt];
#pragma unroll
                    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                        for (int st = 0; st < NST; ++st) {
                            const auto fa = Op::load(sWq + (32 * mt + l32) * RS_D + 32 * kb + 16 * half + KH * st);
                            Vn[mt] = Op::mma(fa, Op::from_acc(X[kb], st), Vn[mt]);
                        }
                }
                if (WITH_Q && !t_wave && a.o) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        floatx16 O = zero16();
#pragma unroll
                        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                            for (int st = 0; st < NST; ++st) {
                                const auto fa = Op::load(sQq + (32 * mt + l32) * RS_D + 32 * kb + 16 * half + KH * st);
                                O = Op::mma(fa, Op::from_acc(X[kb], st), O);
                            }
#pragma unroll
                        for (int j = 0; j < 16; ++j) O[j] *= sGam[32 * mt + acc_row(half, j)];
#pragma unroll
                        for (int mj = 0; mj <= mt; ++mj)
#pragma unroll
                            for (int st = 0; st < NST; ++st) {
                                const auto fa = Op::load(sMq + (32 * mt + l32) * RS_T + 32 * mj + 16 * half + KH * st);
                                O = Op::mma(fa, Op::from_acc(Vn[mj], st), O);
                            }
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int t = 32 * mt + acc_row(half, j);
                            if (t < valid) {
                                const long long oi = ((b * N + tok0 + t) * a.h_v + h) * D + col0 + l32;
                                if (a.out_bf16) reinterpret_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(O[j]);
                                else reinterpret_cast<float*>(a.o)[oi] = O[j];
                            }
                        }
                    }
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) Vn[mt][j] *= sSc[32 * mt + acc_row(half, j)];
                const float Gamma = sMisc[0];
#pragma unroll
                for (int xb = 0; xb < NB; ++xb) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) X[xb][j] *= Gamma;
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int st = 0; st < NST; ++st) {
                            const auto fa = Op::load(sKt + (32 * xb + l32) * RS_T + 32 * mt + 16 * half + KH * st);
                            X[xb] = Op::mma(fa, Op::from_acc(Vn[mt], st), X[xb]);
                        }
                }
                if (t_wave) {
                    float m = 0.f;
#pragma unroll
                    for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                        for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(X[xb][j]));
                    m = wave_max(m);
                    const int e = exp2_of(m);
                    if (e != 0) {
#pragma unroll
                        for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                            for (int j = 0; j < 16; ++j) X[xb][j] = ldexpf(X[xb][j], -e);
                        ew += e;
                    }
                }
            }
            __syncthreads();
        }

        // ---- epilogue: align the T waves' exponents, write T_hat / T_exp / S
        int* sEw = reinterpret_cast<int*>(smem_raw + LY::Misc) + 1;
        if (t_wave && do_T && lane == 0) sEw[wave] = ew;
        __syncthreads();
        if (t_wave && do_T) {
            int emax = sEw[0];
            for (int w = 1; w < NW / 2; ++w) emax = max(emax, sEw[w]);
            float* dst = a.T_hat + ((long long)seg * a.n_batch * a.h_v + chain_off) * D * D + col0;
#pragma unroll
            for (int xb = 0; xb < NB; ++xb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) X[xb][j] = ldexpf(X[xb][j], ew - emax);
                store_tile<D>(dst + 32 * xb * D, X[xb], half, l32);
            }
            if (tid == 0) a.T_exp[(long long)seg * a.n_batch * a.h_v + chain_off] = emax;
        }
        if (!t_wave && a.S_out) {
            float* dst = a.S_out + seg * a.out_stride + chain_off * D * D + col0;
#pragma unroll
            for (int xb = 0; xb < NB; ++xb) store_tile<D>(dst + 32 * xb * D, X[xb], half, l32);
        }
        __syncthreads();
    }
}

template <int D, class Op, bool WITH_Q>
static hipError_t launch_one(const EngineArgs& a, int grid, hipStream_t s) {
    if (a.persistent)
        hipLaunchKernelGGL((dense_engine_kernel<D, Op, WITH_Q, true>), dim3(grid), dim3(D * 4), 0, s, a);
    else
        hipLaunchKernelGGL((dense_engine_kernel<D, Op, WITH_Q, false>), dim3(grid), dim3(D * 4), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_dense_engine(const EngineArgs& a, int d, int prec_f32, int grid, hipStream_t s) {
    const bool q = a.q != nullptr;
    if (d == 128 && !prec_f32) return q ? launch_one<128, OpF16, true>(a, grid, s) : launch_one<128, OpF16, false>(a, grid, s);
    if (d == 64 && !prec_f32) return q ? launch_one<64, OpF16, true>(a, grid, s) : launch_one<64, OpF16, false>(a, grid, s);
    if (d == 64 && prec_f32) return q ? launch_one<64, OpF32, true>(a, grid, s) : launch_one<64, OpF32, false>(a, grid, s);
    return hipErrorInvalidValue;
}

int dense_engine_max_lds(int d, int prec_f32, int with_q) {
    if (d == 128 && !prec_f32) return with_q ? EngineLayout<128, OpF16, true>::total : EngineLayout<128, OpF16, false>::total;
    if (d == 64 && !prec_f32) return with_q ? EngineLayout<64, OpF16, true>::total : EngineLayout<64, OpF16, false>::total;
    if (d == 64 && prec_f32) return with_q ? EngineLayout<64, OpF32, true>::total : EngineLayout<64, OpF32, false>::total;
    return -1;
}

}  // namespace hypic
