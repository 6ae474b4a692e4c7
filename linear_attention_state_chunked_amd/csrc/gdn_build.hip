// Segment build of the dense kind (gated delta rule): T_C and S(C|0) per (segment, chain).
//
// Chunked WY/UT form (local tokens i = 0..63 of a 64-token chunk; masked tail tokens
// have k = v = 0, beta = 0, log alpha = 0):
//   G_i = sum_{j<=i} log alpha_j, gamma_i = exp(G_i), Gamma = gamma_63
//   L   = strictly-lower(diag(beta) exp(G_i - G_j) o K K^T),   Tg = (I + L)^-1 diag(beta)
//   U   = Tg V,   W' = Tg diag(gamma) K
//   X = [T | S] <- Gamma X + K^T diag(Gamma/gamma) ([0 | U] - W' X),   X_0 = [I | 0]
// T is the ordered product of the per-token transitions (the cached transition
// operator of the HYPIC news article's linear-layer paragraph), S the zero-start state.
//
// Warp specialisation.  Carry waves own 32 columns of X each (T columns, then S
// columns), keep them in matrix-core accumulators for the whole segment and run the
// carry of chunk c; four preparation waves meanwhile stage chunk c+1, form its gram and
// solve it.  Carry waves then turn the solve into W' (stored as ready-made operand
// fragments) and U (kept in registers) for chunk c+1.  Two workgroup barriers per chunk;
// the preparation waves order their own stages with a bounded LDS-counter barrier.
//
// Layout rules.  Every matrix in LDS is a natural row-major f16 tile written with
// 8- or 16-byte stores.  Row fragments are plain 16-byte reads; column fragments
// (contraction over tokens, e.g. K^T or V) come from the gfx950 transposing read
// ds_read_b64_tr_b16, which hands each lane of a 16-lane group one column of a 4x16
// block.  Products whose result must be stored are computed transposed, so that each
// lane's accumulator column is a run of a row of the result.
//
// The 64x64 unit lower-triangular solve: 16x16 diagonal inverses by substitution in
// fp32, then Inv = D - D N D merges (D block diagonal, N strictly block lower) for the
// two 32x32 halves and for the whole, on the matrix cores with hi/lo-split f16
// operands (about 22-bit operands, fp32 accumulation).
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace hypic {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// Four rows r0..r0+3 of 16 consecutive columns c0..c0+15 of a row-major f16 LDS matrix,
// transposed: lane i of each 16-lane group receives column c0 + i.  Every lane passes
// the r0 / c0 of its own group.
__device__ __forceinline__ halfx4 tr4(const _Float16* M, int rs, int r0, int c0, int lane) {
    const int s = lane & 15;
    const _Float16* p = M + (r0 + (s >> 2)) * rs + c0 + 4 * (s & 3);
    const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)p);
    return __builtin_bit_cast(halfx4, v);
}
__device__ __forceinline__ halfx8 cat8(halfx4 a, halfx4 b) {
    halfx8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}
__device__ __forceinline__ halfx8 ld8(const _Float16* p) { return *reinterpret_cast<const halfx8*>(p); }

// column fragment of a 32-column block for contraction rows in accumulator order:
// lane (column cb + l32, half h) gets rows rb + acc_row(h, 8 st + e), e = 0..7
__device__ __forceinline__ halfx8 colfrag_acc(const _Float16* M, int rs, int rb, int cb, int st, int lane) {
    const int h = lane >> 5, c0 = cb + 16 * ((lane >> 4) & 1);
    const int r0 = rb + 16 * st + 4 * h;
    return cat8(tr4(M, rs, r0, c0, lane), tr4(M, rs, r0 + 8, c0, lane));
}
// same for natural contraction order: rows rb + 16 kk + 8 h + e
__device__ __forceinline__ halfx8 colfrag_nat(const _Float16* M, int rs, int rb, int cb, int kk, int lane) {
    const int h = lane >> 5, c0 = cb + 16 * ((lane >> 4) & 1);
    const int r0 = rb + 16 * kk + 8 * h;
    return cat8(tr4(M, rs, r0, c0, lane), tr4(M, rs, r0 + 4, c0, lane));
}

// Inclusive prefix sum over the 64 lanes with DPP row shifts and row broadcasts (no
// LDS round trips): rows of 16 lanes first, then carried across rows.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, BANK_MASK, false));
}
__device__ __forceinline__ float wave_scan_dpp(float v) {
    float r = v + dpp_mov<0x111, 0xf, 0xf>(v);   // row_shr:1
    r += dpp_mov<0x112, 0xf, 0xf>(v);            // row_shr:2
    r += dpp_mov<0x113, 0xf, 0xf>(v);            // row_shr:3
    r += dpp_mov<0x114, 0xf, 0xe>(r);            // row_shr:4, lanes 4..15 of each row
    r += dpp_mov<0x118, 0xf, 0xc>(r);            // row_shr:8, lanes 8..15 of each row
    r += dpp_mov<0x142, 0xa, 0xf>(r);            // row_bcast:15 into rows 1 and 3
    r += dpp_mov<0x143, 0xc, 0xf>(r);            // row_bcast:31 into rows 2 and 3
    return r;
}

// e^x through the hardware base-2 exponential (arguments here are small and <= 0)
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

struct HL {
    halfx8 hi, lo;
};
__device__ __forceinline__ floatx16 mma3(const HL& a, const HL& b, floatx16 c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.lo, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.hi, b.lo, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a.hi, b.hi, c, 0, 0, 0);
}
// hi/lo split of fp32 values into f16 pairs: hi = f16(v), lo = f16(v - hi).  v - hi is
// exact in fp32, so lo is one fused v_fma_mix step (-1 * hi + v, rounded once) per value
// instead of an f16 -> f32 conversion, a subtraction and a second conversion.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ unsigned int pk_f16(float a, float b) {
    return __builtin_bit_cast(unsigned int, f16x2{(_Float16)a, (_Float16)b});
}
__device__ __forceinline__ unsigned int lo_pair(unsigned int hi, float a, float b) {
    unsigned int r;
    asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %1, -1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(r)
        : "v"(hi), "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ HL split_acc(const floatx16& a, int st) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = pk_f16(a[8 * st + 2 * i], a[8 * st + 2 * i + 1]);
        l[i] = lo_pair(h[i], a[8 * st + 2 * i], a[8 * st + 2 * i + 1]);
    }
    return HL{__builtin_bit_cast(halfx8, h), __builtin_bit_cast(halfx8, l)};
}
__device__ __forceinline__ void split4(const float* v, halfx4& hi, halfx4& lo) {
    const unsigned int h0 = pk_f16(v[0], v[1]), h1 = pk_f16(v[2], v[3]);
    hi = __builtin_bit_cast(halfx4, u32x2{h0, h1});
    lo = __builtin_bit_cast(halfx4, u32x2{lo_pair(h0, v[0], v[1]), lo_pair(h1, v[2], v[3])});
}
__device__ __forceinline__ void st4h(_Float16* p, halfx4 v) { *reinterpret_cast<halfx4*>(p) = v; }

// Four entries y of a row of (I + L)^-1 at token columns t0..t0+3 -> the f16 entries of
// Tg = (I + L)^-1 diag(beta) and of Tg diag(gamma) (hi and lo parts)
__device__ __forceinline__ void tg4(const float* y, const float* sBeta, const float* sBG, int t0, halfx4& ta,
                                    halfx4& tg, halfx4& tl) {
    const float4 b4 = *reinterpret_cast<const float4*>(sBeta + t0);
    const float4 g4 = *reinterpret_cast<const float4*>(sBG + t0);
    const float g[4] = {y[0] * g4.x, y[1] * g4.y, y[2] * g4.z, y[3] * g4.w};
    ta = __builtin_bit_cast(halfx4, u32x2{pk_f16(y[0] * b4.x, y[1] * b4.y), pk_f16(y[2] * b4.z, y[3] * b4.w)});
    const unsigned int h0 = pk_f16(g[0], g[1]), h1 = pk_f16(g[2], g[3]);
    tg = __builtin_bit_cast(halfx4, u32x2{h0, h1});
    tl = __builtin_bit_cast(halfx4, u32x2{lo_pair(h0, g[0], g[1]), lo_pair(h1, g[2], g[3])});
}

template <bool BF16>
struct Raw8;
template <>
struct Raw8<true> {
    uint4 w;
    __device__ void load(const void* base, long long idx) {
        w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    }
    __device__ void loadp(const unsigned char* p) { w = *reinterpret_cast<const uint4*>(p); }
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
    __device__ void loadp(const unsigned char* p) {
        a = reinterpret_cast<const float4*>(p)[0];
        b = reinterpret_cast<const float4*>(p)[1];
    }
    __device__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ void get(float (&x)[8]) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};

// ---------------------------------------------------------------------------------------
// LDS layout (bytes); f16 tiles unless noted

template <int D>
struct GLayout {
    static constexpr int NB = D / 32;
    static constexpr int RK = D + 8;                   // K, V rows
    static constexpr int RT = 64 + 8;                  // 64-wide rows: L^T, Tg
    static constexpr int RV = 32 + 8;                  // 32-wide rows: D', Inv'
    static constexpr int sz_K = 64 * RK * 2;
    static constexpr int sz_Wf = 2 * NB * 2 * 64 * 8 * 2;
    static constexpr int sz_Sc = 80 * 4;
    static constexpr int sz_T64 = 64 * RT * 2;
    static constexpr int sz_V32 = 64 * RV * 2;
    static constexpr int Kn = 0;                       // K rows (x2)
    static constexpr int Wf = Kn + 2 * sz_K;           // -W'^T operand fragments (x2)
    static constexpr int Sc = Wf + 2 * sz_Wf;          // Gamma/gamma_i, Gamma (fp32, x2)
    static constexpr int Vn = Sc + 2 * sz_Sc;          // V rows
    static constexpr int Ld = Vn + sz_K;               // fp32 diagonal 16x16 blocks of L, [4][16][20]
    static constexpr int LTh = Ld + 4 * 16 * 20 * 4;   // L^T hi / lo
    static constexpr int LTl = LTh + sz_T64;
    static constexpr int DVh = LTl + sz_T64;           // D' (block-diagonal 16x16 inverses per half) hi / lo
    static constexpr int DVl = DVh + sz_V32;
    static constexpr int IVh = DVl + sz_V32;           // Inv' (32x32 inverses of the halves) hi / lo
    static constexpr int IVl = IVh + sz_V32;
    static constexpr int TgA = IVl + sz_V32;           // Tg
    static constexpr int TgG = TgA + sz_T64;           // Tg diag(gamma)
    static constexpr int TgGl = TgG + sz_T64;          // its low part (precise-T plan)
    static constexpr int Gv = TgGl + sz_T64;           // G log2 e, beta, beta gamma (fp32)
    static constexpr int Misc = Gv + 3 * 64 * 4;       // counter, exponents
    static constexpr int total = Misc + 32 * 4;
    // regions that must start at zero and are only partly written
    static constexpr int zero_begin = LTh, zero_end = Gv;
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

// Chunk-local UT transform on four cooperating waves (pw = 0..3): from the staged K rows
// (f16, row stride D + 8) and the gate prefix, the gram K K^T, L = strictly-lower(
// beta_i e^{G_i - G_j} K K^T) and Tg = (I + L)^-1 diag(beta).  Tg leaves through
// out(row, col0, Tg[row][col0..+3], (Tg diag(gamma))[row][col0..+3] hi, lo) as f16; only
// the lower 16x16 blocks are written.  pbar() orders the four waves between the stages.
template <int D, bool PT, class Bar, class Out>
__device__ __forceinline__ void ut_solve(const _Float16* Kn1, const float* sGl, const float* sBeta, const float* sBG,
                                         float* Ld, _Float16* LTh, _Float16* LTl, _Float16* DVh, _Float16* DVl,
                                         _Float16* IVh, _Float16* IVl, int pw, int ln, Bar&& pbar, Out&& out) {
    constexpr int RK = D + 8, RT = 64 + 8, RV = 32 + 8;
    const int hf = ln >> 5, lq = ln & 31;
    // ---- gram K K^T (three lower 32x32 tiles) -> L^T rows (hi/lo) and
    //      the fp32 diagonal 16x16 blocks of L
    if (pw < 3) {
        const int ti = pw == 0 ? 0 : 1, tj = pw == 2 ? 1 : 0;
        floatx16 acc = zero16();
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const halfx8 fa = ld8(Kn1 + (32 * ti + lq) * RK + 16 * kk + 8 * hf);
            const halfx8 fb = ld8(Kn1 + (32 * tj + lq) * RK + 16 * kk + 8 * hf);
            acc = OpF16::mma(fa, fb, acc);
        }
        // lane column j; its registers hold rows i = 32 ti + 8 q + 4 h + 0..3
        const int j = 32 * tj + lq;
        // e^{G_i - G_j} = 2^{G_i log2 e - G_j log2 e}
        const float Gj = sGl[j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i0 = 32 * ti + 8 * q + 4 * hf;
            const float4 g4 = *reinterpret_cast<const float4*>(sGl + i0);
            const float4 b4 = *reinterpret_cast<const float4*>(sBeta + i0);
            const float gi[4] = {g4.x, g4.y, g4.z, g4.w};
            const float bi[4] = {b4.x, b4.y, b4.z, b4.w};
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = (i0 + u > j) ? bi[u] * __builtin_amdgcn_exp2f(gi[u] - Gj) * acc[4 * q + u] : 0.f;
            halfx4 vh, vl;
            split4(v, vh, vl);
            st4h(LTh + j * RT + i0, vh);
            st4h(LTl + j * RT + i0, vl);
            if (ti == tj && ((i0 >> 4) == (j >> 4))) {
                // L_bb[i][m] with m = j: column j of the diagonal block
                float* ld = Ld + (i0 >> 4) * (16 * 20) + (j & 15);
#pragma unroll
                for (int u = 0; u < 4; ++u) ld[((i0 + u) & 15) * 20] = v[u];
            }
        }
    }
    pbar(ln);

    // ---- solve, halves q = 0, 1 (one wave each): rows of the 16x16
    //      diagonal inverses, then Inv' = D' - D' N D'
    if (pw < 2) {
        const int q = pw;
        {   // lanes 0..31: row cr of the diagonal inverse D_bb, bb = 2q + (ln >> 4)
            const int bb = 2 * q + ((ln >> 4) & 1), cr = ln & 15, o = 16 * (bb & 1);
            if (ln < 32) {
                float y[16];
#pragma unroll
                for (int m = 0; m < 16; ++m) y[m] = (m == cr) ? 1.f : 0.f;
                const float* Lb = Ld + bb * (16 * 20);
                // rows of L_bb, loaded three steps ahead of their use
                float4 rw[16][4];
#pragma unroll
                for (int i = 15; i >= 13; --i)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        if (4 * q4 < i) rw[i][q4] = reinterpret_cast<const float4*>(Lb + i * 20)[q4];
#pragma unroll
                for (int i = 15; i >= 1; --i) {
                    if (i - 3 >= 1) {
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4)
                            if (4 * q4 < i - 3)
                                rw[i - 3][q4] = reinterpret_cast<const float4*>(Lb + (i - 3) * 20)[q4];
                    }
                    const float yi = y[i];
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        if (4 * q4 >= i) break;
                        const float l4[4] = {rw[i][q4].x, rw[i][q4].y, rw[i][q4].z, rw[i][q4].w};
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (4 * q4 + u < i) y[4 * q4 + u] -= yi * l4[u];
                    }
                }
                // y = row cr of D_bb: D' and Inv' rows (hi/lo), Tg rows
                const int rloc = o + cr;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    halfx4 vh, vl;
                    split4(y + 4 * q4, vh, vl);
                    st4h(DVh + (32 * q + rloc) * RV + o + 4 * q4, vh);
                    st4h(DVl + (32 * q + rloc) * RV + o + 4 * q4, vl);
                    st4h(IVh + (32 * q + rloc) * RV + o + 4 * q4, vh);
                    st4h(IVl + (32 * q + rloc) * RV + o + 4 * q4, vl);
                    const int t0 = 16 * bb + 4 * q4;
                    halfx4 ta, tg, tl;
                    tg4(y + 4 * q4, sBeta, sBG, t0, ta, tg, tl);
                    out(16 * bb + cr, t0, ta, tg, tl);
                }
            }
        }
        // Q = N^T D'^T: only contraction k = 16..31 and rows r < 16 of N^T are nonzero
        HL fa, fb;
        if (lq < 16) {
            fa.hi = ld8(LTh + (32 * q + lq) * RT + 32 * q + 16 + 8 * hf);
            fa.lo = ld8(LTl + (32 * q + lq) * RT + 32 * q + 16 + 8 * hf);
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) fa.hi[u] = fa.lo[u] = (_Float16)0.f;
        }
        fb.hi = ld8(DVh + (32 * q + lq) * RV + 16 + 8 * hf);
        fb.lo = ld8(DVl + (32 * q + lq) * RV + 16 + 8 * hf);
        const floatx16 Qt = mma3(fa, fb, zero16());
        // R^T = D'^T Q: Q has rows k < 16 only, i.e. contraction step 0 in
        // accumulator order
        HL da;
        da.hi = colfrag_acc(DVh + 32 * q * RV, RV, 0, 0, 0, ln);
        da.lo = colfrag_acc(DVl + 32 * q * RV, RV, 0, 0, 0, ln);
        const floatx16 Rt = mma3(da, split_acc(Qt, 0), zero16());
        // lane column m holds R[m][t], t = acc_row(h, j); nonzero for m >= 16, t < 16
        if (lq >= 16) {
            const int m = 32 * q + lq;
#pragma unroll
            for (int q4 = 0; q4 < 2; ++q4) {
                const int tl = 8 * q4 + 4 * hf;   // rows acc_row(h, 4 q4 + 0..3)
                float v[4] = {-Rt[4 * q4], -Rt[4 * q4 + 1], -Rt[4 * q4 + 2], -Rt[4 * q4 + 3]};
                halfx4 vh, vl;
                split4(v, vh, vl);
                st4h(IVh + m * RV + tl, vh);
                st4h(IVl + m * RV + tl, vl);
                const int t0 = 32 * q + tl;
                halfx4 ta, tg, tgl;
                tg4(v, sBeta, sBG, t0, ta, tg, tgl);
                out(m, t0, ta, tg, tgl);
            }
        }
    }
    pbar(ln);

    // ---- solve, lower-left 32x32 block: -Inv'_1 L'_10 Inv'_0, computed as
    //      its transpose Inv'_0^T (L'_10^T Inv'_1^T)
    if (pw == 0) {
        floatx16 Q2 = zero16();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            HL fa, fb;
            fa.hi = ld8(LTh + lq * RT + 32 + 16 * kk + 8 * hf);
            fa.lo = ld8(LTl + lq * RT + 32 + 16 * kk + 8 * hf);
            fb.hi = ld8(IVh + (32 + lq) * RV + 16 * kk + 8 * hf);
            fb.lo = ld8(IVl + (32 + lq) * RV + 16 * kk + 8 * hf);
            Q2 = mma3(fa, fb, Q2);
        }
        floatx16 R2 = zero16();
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            HL da;
            da.hi = colfrag_acc(IVh, RV, 0, 0, st, ln);
            da.lo = colfrag_acc(IVl, RV, 0, 0, st, ln);
            R2 = mma3(da, split_acc(Q2, st), R2);
        }
        const int m = 32 + lq;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int t0 = 8 * q4 + 4 * hf;
            const float v[4] = {-R2[4 * q4], -R2[4 * q4 + 1], -R2[4 * q4 + 2], -R2[4 * q4 + 3]};
            halfx4 ta, tg, tl;
            tg4(v, sBeta, sBG, t0, ta, tg, tl);
            out(m, t0, ta, tg, tl);
        }
    }
}

template <int D, bool WITH_T, bool IN_BF16, bool PERSIST, bool PT>
__global__ __launch_bounds__(((WITH_T ? 2 : 1) * D / 32 + 4) * 64) void gdn_build_kernel(EngineArgs a) {
    using LY = GLayout<D>;
    using E = _Float16;
    constexpr int NB = D / 32;
    constexpr int NC = (WITH_T ? 2 : 1) * NB;   // carry waves
    constexpr int NP = 4;                       // preparation waves
    constexpr int NT = (NC + NP) * 64;
    constexpr int RK = LY::RK, RT = LY::RT, RV = LY::RV;
    constexpr int G8 = D / 8;
    constexpr int NLD = 64 * G8 / (NP * 64);    // 8-element groups per prep thread per tensor

    __shared__ __align__(16) unsigned char smem[LY::total];
    int* sCnt = reinterpret_cast<int*>(smem + LY::Misc);
    int* sEw = sCnt + 4;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_c = wave < NC;
    const bool t_wave = WITH_T && wave < NB;
    const long long N = a.n_tokens;

    for (int i = LY::zero_begin / 16 + tid; i < LY::zero_end / 16; i += NT)
        reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
    if (tid == 0) sCnt[0] = 0;
    int pb_target = 0;

    // Each role (T-column carry, S-column carry, preparation) runs its own copy of the task
    // and chunk loops with the same barrier sequence, so each is register-allocated on its
    // own instead of through one merged control-flow graph.
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
                // =========================== carry waves ===========================
                constexpr bool TR = R == 0;
                const int col0 = ((WITH_T && !TR) ? wave - NB : wave) * 32;
                // identity columns of X for the T waves; the opaque zero keeps these 64
                // task-invariant values from being hoisted into long-lived registers
                int tz = 0;
                asm volatile("" : "+v"(tz));
                const int diag = col0 + (lane & 31) + tz - 4 * (lane >> 5);
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
                    // opaque zeros: per-lane LDS offsets are recomputed every chunk instead of
                    // being hoisted out of the loop into long-lived registers
                    int lz = 0, lzv = 0;
                    asm volatile("" : "+s"(lz));
                    asm volatile("" : "+v"(lzv));
                    unsigned char* sm = smem + lz;
                    const int ln = lane + lzv, hf = ln >> 5, lq = ln & 31;
                    const int p = c & 1, pn = (c + 1) & 1;
                    if (c >= 0) {
                        const E* Wf = reinterpret_cast<const E*>(sm + LY::Wf + p * LY::sz_Wf);
                        const E* Kn = reinterpret_cast<const E*>(sm + LY::Kn + p * LY::sz_K);
                        const float* Sc = reinterpret_cast<const float*>(sm + LY::Sc + p * LY::sz_Sc);
                        floatx16 Vn[2];
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt) {
                            Vn[mt] = TR ? zero16() : Un[mt];
#pragma unroll
                            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                                for (int st = 0; st < 2; ++st) {
                                    const halfx8 fa = ld8(Wf + (((mt * NB + kb) * 2 + st) * 64 + ln) * 8);
                                    if (PT && TR) {
                                        const HL xb = split_acc(X[kb], st);
                                        Vn[mt] = OpF16::mma(fa, xb.lo, Vn[mt]);
                                        Vn[mt] = OpF16::mma(fa, xb.hi, Vn[mt]);
                                    } else {
                                        Vn[mt] = OpF16::mma(fa, OpF16::from_acc(X[kb], st), Vn[mt]);
                                    }
                                }
                            const float4* s4 = reinterpret_cast<const float4*>(Sc + 32 * mt + 4 * hf);
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const float4 sv = s4[2 * q];   // rows 8q + 4h + 0..3
                                Vn[mt][4 * q + 0] *= sv.x;
                                Vn[mt][4 * q + 1] *= sv.y;
                                Vn[mt][4 * q + 2] *= sv.z;
                                Vn[mt][4 * q + 3] *= sv.w;
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        const float Gamma = Sc[64];
#pragma unroll
                        for (int xb = 0; xb < NB; ++xb) {
#pragma unroll
                            for (int j = 0; j < 16; ++j) X[xb][j] *= Gamma;
#pragma unroll
                            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                                for (int st = 0; st < 2; ++st) {
                                    const halfx8 fa = colfrag_acc(Kn, RK, 32 * mt, 32 * xb, st, ln);
                                    if (PT && TR) {
                                        const HL vb = split_acc(Vn[mt], st);
                                        X[xb] = OpF16::mma(fa, vb.lo, X[xb]);
                                        X[xb] = OpF16::mma(fa, vb.hi, X[xb]);
                                    } else {
                                        X[xb] = OpF16::mma(fa, OpF16::from_acc(Vn[mt], st), X[xb]);
                                    }
                                }
                        }
                        if (TR) {
                            float m = 0.f;
#pragma unroll
                            for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                                for (int j = 0; j < 16; j += 2) m = fmaxf(m, fmaxf(fabsf(X[xb][j]), fabsf(X[xb][j + 1])));
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
                        const E* Kn1 = reinterpret_cast<const E*>(sm + LY::Kn + pn * LY::sz_K);
                        const E* TgA = reinterpret_cast<const E*>(sm + LY::TgA);
                        const E* TgG = reinterpret_cast<const E*>(sm + LY::TgG);
                        const E* TgGl = reinterpret_cast<const E*>(sm + LY::TgGl);
                        const E* Vn1 = reinterpret_cast<const E*>(sm + LY::Vn);
                        E* Wf1 = reinterpret_cast<E*>(sm + LY::Wf + pn * LY::sz_Wf);
                        // -W'^T tiles (d rows, token columns): their accumulators are the operand
                        // fragments of W' X in the carry, stored in that order
                        if (TR || !WITH_T) {
                            const int dt = wave;
#pragma unroll
                            for (int mt = 0; mt < 2; ++mt) {
                                floatx16 acc = zero16();
#pragma unroll
                                for (int kk = 0; kk < 4; ++kk) {
                                    const halfx8 fa = colfrag_nat(Kn1, RK, 0, 32 * dt, kk, ln);
                                    const halfx8 fb = ld8(TgG + (32 * mt + lq) * RT + 16 * kk + 8 * hf);
                                    if (PT) {
                                        const halfx8 fl = ld8(TgGl + (32 * mt + lq) * RT + 16 * kk + 8 * hf);
                                        acc = OpF16::mma(fa, fl, acc);
                                    }
                                    acc = OpF16::mma(fa, fb, acc);
                                }
#pragma unroll
                                for (int st = 0; st < 2; ++st) {
                                    halfx8 w;
#pragma unroll
                                    for (int i = 0; i < 8; ++i) w[i] = (_Float16)(-acc[8 * st + i]);
                                    *reinterpret_cast<halfx8*>(Wf1 + (((mt * NB + dt) * 2 + st) * 64 + ln) * 8) = w;
                                }
                            }
                        }
                        if (!TR) {
                            // both token halves per V fragment: one fragment live at a time
                            Un[0] = Un[1] = zero16();
#pragma unroll
                            for (int kk = 0; kk < 4; ++kk) {
                                const halfx8 fb = colfrag_nat(Vn1, RK, 0, col0, kk, ln);
#pragma unroll
                                for (int mt = 0; mt < 2; ++mt)
                                    Un[mt] = OpF16::mma(ld8(TgA + (32 * mt + lq) * RT + 16 * kk + 8 * hf), fb, Un[mt]);
                            }
                        }
                    }
                    __syncthreads();  // W'(c+1) written; staging buffers free
                }
                // epilogue: align the T waves' exponents, write T_hat / T_exp / S
                if (TR && lane == 0) sEw[wave] = ew;
                __syncthreads();
                const int half = lane >> 5, l32 = lane & 31;
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
                // ======================== preparation waves ========================
                const int pw = wave - NC;
                const int ptid = tid - NC * 64;
                Raw8<IN_BF16> pk[NLD], pv[NLD];
                float pla = 0.f, pbt = 0.f;
                // uniform 64-bit bases per task and chunk, 32-bit per-lane byte offsets
                constexpr int ESZ = IN_BF16 ? 2 : 4;
                const long long row0 = (long long)b * N + start;
                const unsigned char* kb0 =
                    reinterpret_cast<const unsigned char*>(a.k) + (row0 * a.h_k + hk) * (D * ESZ);
                const unsigned char* vb0 =
                    reinterpret_cast<const unsigned char*>(a.v) + (row0 * a.h_v + h) * (D * ESZ);
                const float* la0 = a.log_alpha + row0 * a.h_v + h;
                const float* bt0 = a.beta + row0 * a.h_v + h;
                const unsigned kstride = (unsigned)a.h_k * (D * ESZ), vstride = (unsigned)a.h_v * (D * ESZ);
                auto prefetch = [&](int cc, int ln, int pt) {
                    const int valid = min(64, len - 64 * cc);
                    const unsigned char* kc = kb0 + (long long)(64 * cc) * kstride;
                    const unsigned char* vc = vb0 + (long long)(64 * cc) * vstride;
                    const int t0 = pt / G8;
                    const unsigned d0b = 8 * ESZ * (pt % G8);
#pragma unroll
                    for (int r = 0; r < NLD; ++r) {
                        const int t = t0 + (NP * 64 / G8) * r;
                        if (t < valid) {
                            pk[r].loadp(kc + (t * kstride + d0b));
                            pv[r].loadp(vc + (t * vstride + d0b));
                        } else {
                            pk[r].zero();
                            pv[r].zero();
                        }
                    }
                    if (pw == 0) {
                        const bool ok = ln < valid;
                        const unsigned go = (unsigned)ln * a.h_v;
                        pla = ok ? (la0 + (long long)(64 * cc) * a.h_v)[go] : 0.f;
                        pbt = ok ? (bt0 + (long long)(64 * cc) * a.h_v)[go] : 0.f;
                    }
                };
                auto pbar = [&](int ln) {
                    pb_target += NP;
                    prep_barrier(sCnt, pb_target, ln);
                };
                // the preparation waves are the critical path of every chunk: let their few
                // instructions issue ahead of the carry waves' (matrix-core bound) stream
                __builtin_amdgcn_s_setprio(2);
                if (nc > 0) prefetch(0, lane, ptid);
                for (int c = -1; c < nc; ++c) {
                    int lz = 0, lzv = 0;
                    asm volatile("" : "+s"(lz));
                    asm volatile("" : "+v"(lzv));
                    unsigned char* sm = smem + lz;
                    const int ln = lane + lzv, hf = ln >> 5, lq = ln & 31, pt = ptid + lzv;
                    const int pn = (c + 1) & 1;
                    if (c + 1 < nc) {
                        E* Kn1 = reinterpret_cast<E*>(sm + LY::Kn + pn * LY::sz_K);
                        E* Vn = reinterpret_cast<E*>(sm + LY::Vn);
                        float* Scn = reinterpret_cast<float*>(sm + LY::Sc + pn * LY::sz_Sc);
                        float* Ld = reinterpret_cast<float*>(sm + LY::Ld);
                        E* LTh = reinterpret_cast<E*>(sm + LY::LTh);
                        E* LTl = reinterpret_cast<E*>(sm + LY::LTl);
                        E* DVh = reinterpret_cast<E*>(sm + LY::DVh);
                        E* DVl = reinterpret_cast<E*>(sm + LY::DVl);
                        E* IVh = reinterpret_cast<E*>(sm + LY::IVh);
                        E* IVl = reinterpret_cast<E*>(sm + LY::IVl);
                        E* TgA = reinterpret_cast<E*>(sm + LY::TgA);
                        E* TgG = reinterpret_cast<E*>(sm + LY::TgG);
                        E* TgGl = reinterpret_cast<E*>(sm + LY::TgGl);
                        float* sGl = reinterpret_cast<float*>(sm + LY::Gv);
                        float* sBeta = sGl + 64;
                        float* sBG = sGl + 128;

                        // ---- stage chunk c+1: K and V rows, gate prefix
                        const int st0 = (unsigned)pt / G8, sd0 = 8 * ((unsigned)pt % G8);
#pragma unroll
                        for (int r = 0; r < NLD; ++r) {
                            const int t = st0 + (NP * 64 / G8) * r, d0 = sd0;
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
                            const u32x4 hk8 = {pk_f16(x[0], x[1]), pk_f16(x[2], x[3]), pk_f16(x[4], x[5]),
                                               pk_f16(x[6], x[7])};
                            pv[r].get(x);
                            const u32x4 hv8 = {pk_f16(x[0], x[1]), pk_f16(x[2], x[3]), pk_f16(x[4], x[5]),
                                               pk_f16(x[6], x[7])};
                            *reinterpret_cast<u32x4*>(Kn1 + t * RK + d0) = hk8;
                            *reinterpret_cast<u32x4*>(Vn + t * RK + d0) = hv8;
                        }
                        if (pw == 0) {
                            const float G = wave_scan_dpp(pla);
                            const float Glast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), 63));
                            const float Gl = G * 1.4426950408889634f;
                            sGl[ln] = Gl;
                            sBeta[ln] = pbt;
                            sBG[ln] = pbt * __builtin_amdgcn_exp2f(Gl);
                            Scn[ln] = fexp(Glast - G);
                            if (ln == 0) Scn[64] = fexp(Glast);
                        }
                        if (c + 2 < nc) prefetch(c + 2, ln, pt);
                        pbar(ln);

                        ut_solve<D, PT>(Kn1, sGl, sBeta, sBG, Ld, LTh, LTl, DVh, DVl, IVh, IVl, pw, ln, pbar,
                                        [&](int row, int t0, halfx4 ta, halfx4 tg, halfx4 tl) {
                                            st4h(TgA + row * RT + t0, ta);
                                            st4h(TgG + row * RT + t0, tg);
                                            if (PT) st4h(TgGl + row * RT + t0, tl);
                                        });
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

template <int D, bool WITH_T, bool IN_BF16, bool PT>
static hipError_t launch_v(const EngineArgs& a, int grid, hipStream_t s) {
    constexpr int nt = ((WITH_T ? 2 : 1) * D / 32 + 4) * 64;
    if (a.persistent)
        hipLaunchKernelGGL((gdn_build_kernel<D, WITH_T, IN_BF16, true, PT>), dim3(grid), dim3(nt), 0, s, a);
    else
        hipLaunchKernelGGL((gdn_build_kernel<D, WITH_T, IN_BF16, false, PT>), dim3(grid), dim3(nt), 0, s, a);
    return hipGetLastError();
}

template <int D, bool IN_BF16>
static hipError_t launch_t(const EngineArgs& a, int grid, hipStream_t s) {
    if (!a.T_hat) return launch_v<D, false, IN_BF16, false>(a, grid, s);
    return a.precise_T ? launch_v<D, true, IN_BF16, true>(a, grid, s) : launch_v<D, true, IN_BF16, false>(a, grid, s);
}

hipError_t launch_gdn_build(const EngineArgs& a, int d, int prec_f32, int grid, hipStream_t s) {
    if (prec_f32) return launch_dense_engine(a, d, 1, grid, s);  // fp32 operands: the general engine
    const bool bf = a.in_bf16 != 0;
    if (d == 128) return bf ? launch_t<128, true>(a, grid, s) : launch_t<128, false>(a, grid, s);
    if (d == 64) return bf ? launch_t<64, true>(a, grid, s) : launch_t<64, false>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace hypic
