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
// carry of chunk c; four preparation waves meanwhile solve chunk c+1 (gram, UT
// transform) and stage K and gates of chunk c+2 under the gram products.  After the one
// workgroup barrier per chunk the carry waves turn the solve into W' (T waves; stored as
// ready-made operand fragments) and U (S waves; kept in their accumulators for the next
// carry) while the preparation waves go on with chunk c+2; with 16-bit inputs the S waves
// (and, in the fast plan, the T waves before the barrier) stage V.  K and the gamma vectors
// are triple-buffered, V and the gate vectors doubled.  Bounded LDS counters order the
// rest: the preparation waves' own barrier, the carry waves' W' hand-off and the reuse of
// the Tg buffers (one arrival per carry wave and chunk).
//
// Task mapping.  One workgroup per (segment, batch row, value head) task, the two value
// heads of a key head on workgroups of the same XCD.  With equal segments the grid is one
// persistent workgroup per compute unit and each runs its tasks as one stream of chunks
// (the loop counter counts chunks over the stream), so a task's first chunk is prepared
// under the previous task's last carry.
//
// Layout rules.  Every K / V tile in LDS is a natural row-major f16 tile written with
// 16-byte stores.  Row fragments are plain 16-byte reads; column fragments (contraction
// over tokens, e.g. K^T or V) come from the gfx950 transposing read ds_read_b64_tr_b16,
// which hands each lane of a 16-lane group one column of a 4x16 block.  Products whose
// result must be stored are computed transposed, so that each lane's accumulator column
// is a run of a row of the result.  Tg is stored token-column-major for the same reason.
//
// The 64x64 unit lower-triangular solve works on 16x16 blocks, one token block per
// preparation wave: the diagonal inverses as the product (I+N)(I+N^2)(I+N^4)(I+N^8),
// one exchange of the diagonal inverses and the blocks of L among the four waves, then
// each wave forms its share of the off-diagonal blocks of (I + L)^-1 without further
// hand-offs; all products on the matrix cores with hi/lo-split f16 operands (about
// 22-bit operands, fp32 accumulation).  Only small 16x16 tiles pass between the waves.
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
// exact in fp32, so lo can be a fused f16-source fma (-1 * hi + v, rounded once), which
// the compiler emits as v_fma_mix instead of a conversion, a subtraction and a second
// conversion.  (Written in C, not inline assembly: the results feed matrix-core operands,
// and only compiler-visible instructions get the required VALU -> MFMA wait states.)
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ unsigned int pk_f16(float a, float b) {
    return __builtin_bit_cast(unsigned int, f16x2{(_Float16)a, (_Float16)b});
}
__device__ __forceinline__ unsigned int lo_pair(unsigned int hi, float a, float b) {
    // -1 held in a register, so that the compiler selects its fused f16-source fma
    float m1 = -1.f;
    asm("" : "+v"(m1));
    const f16x2 h = __builtin_bit_cast(f16x2, hi);
    return __builtin_bit_cast(unsigned int, f16x2{(_Float16)__builtin_fmaf((float)h[0], m1, a),
                                                  (_Float16)__builtin_fmaf((float)h[1], m1, b)});
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

constexpr int kXS = 16 + 4;         // row stride (f16) of a column-major 16x16 exchange tile
constexpr int kXT = 2 * 16 * kXS;   // one exchange slot (f16 elements): hi tile, then lo tile

// WO: the output variant (state columns and per-token outputs, no T columns): one V buffer,
// no low Tg buffer, two M tiles and one Q tile
template <int D, bool WO = false>
struct GLayout {
    static constexpr int NB = D / 32;
    // K, V rows.  gfx950's LDS serves 32 lanes per pass from 128 four-byte banks (fitted
    // to probe timings of these access patterns).  A transposing column read puts 4 rows x
    // 16 dwords in one pass, the 16-byte row-fragment reads and stores of the gram and the
    // staging 16 rows x 2 x 4 dwords; a row stride of 72 dwords (D = 128) or 56 (D = 64)
    // keeps both conflict-free (D + 8 gave two-way conflicts on the column reads).
    static constexpr int RK = D == 128 ? D + 16 : D + 48;
    static constexpr int RT = 64 + 8;                  // 64-wide rows of the Tg tiles
    static constexpr int sz_K = 64 * RK * 2;
    static constexpr int sz_Wf = 2 * NB * 2 * 64 * 8 * 2;
    static constexpr int sz_Sc = 80 * 4;
    static constexpr int sz_T64 = 64 * RT * 2;
    static constexpr int Kn = 0;                       // K rows (x3: carry, formation / solve, staging)
    static constexpr int Wf = Kn + 3 * sz_K;           // -W'^T operand fragments
    static constexpr int Sc = Wf + sz_Wf;              // Gamma/gamma_i, Gamma (fp32, x3)
    static constexpr int Vn = Sc + 3 * sz_Sc;          // V rows (x2; x1 with outputs)
    static constexpr int XB = Vn + (WO ? 1 : 2) * sz_K;  // twelve 16x16 exchange slots (hi, lo)
    static constexpr int TgA = XB + 12 * kXT * 2;      // Tg, token-column-major
    static constexpr int TgG = TgA + sz_T64;           // Tg diag(gamma)
    static constexpr int TgGl = TgG + sz_T64;          // its low part (precise-T plan)
    static constexpr int Mo = TgGl + (WO ? 0 : sz_T64);  // M = lower(e^{G_i - G_j} q_i.k_j), row-major (x2)
    static constexpr int Gv = Mo + (WO ? 2 * sz_T64 : 0);  // G log2 e, beta, beta gamma (fp32, x2)
    static constexpr int Misc = Gv + 2 * 3 * 64 * 4;   // counters, exponents
    static constexpr int Qn = Misc + 32 * 4;           // diag(gamma) Q rows (outputs)
    static constexpr int total = Qn + (WO ? sz_K : 0);
    // regions that must start at zero and are only partly written
    static constexpr int zero_begin = TgA, zero_end = Gv;
};

// Sticky status word of this device (see take_device_status).
__device__ unsigned int g_device_status;

// A bounded wait ran out: the hand-off it waited for never came.  The wave goes on, so the
// kernel still ends, and the status word records that this launch's outputs are unreliable.
__device__ __forceinline__ void wait_expired() {
    __hip_atomic_fetch_or(&g_device_status, kStatusWaitExpired, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kSpinLimit = 1 << 18;

// bounded LDS-counter barrier among a subset of waves (one arrival per wave); the polls do
// not sleep: a poll is one broadcast LDS read, and a sleep would add its wake-up delay to
// every hand-off on the critical path
__device__ __forceinline__ void prep_barrier(int* cnt, int target, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    int spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        if (++spins > kSpinLimit) {
            wait_expired();
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// one arrival per wave on an LDS counter, after the wave's earlier LDS accesses
__device__ __forceinline__ void count_arrival(int* cnt, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// bounded wait until an LDS counter reaches target (the counting side releases)
__device__ __forceinline__ void wait_count(int* cnt, int target) {
    int spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        if (++spins > kSpinLimit) {
            wait_expired();
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ---------------------------------------------------------------------------------------
// 16x16 matrix-core tiles (v_mfma_f32_16x16x16f16, v_mfma_f32_16x16x32_f16).  Accumulator
// layout: lane l holds column l & 15 and, in register i, row 4 (l >> 4) + i.  That is also
// the B-operand layout of the 16x16x16 product (contraction index in place of the row), so a
// result feeds the next product's B operand as it is; as an A operand a matrix X is supplied
// by the accumulator-layout registers of its transpose.  Tiles exchanged through LDS are
// stored column-major (each lane writes its four rows as one 8-byte run): a plain 8-byte read
// returns the B operand, a transposing read the A operand.

struct HL4 {
    halfx4 hi, lo;
};
__device__ __forceinline__ HL4 split4v(floatx4 v) {
    const unsigned int h0 = pk_f16(v[0], v[1]), h1 = pk_f16(v[2], v[3]);
    return HL4{__builtin_bit_cast(halfx4, u32x2{h0, h1}),
               __builtin_bit_cast(halfx4, u32x2{lo_pair(h0, v[0], v[1]), lo_pair(h1, v[2], v[3])})};
}
__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }
// c + a b with hi/lo-split operands (about 22-bit operands; the lo * lo term is dropped)
__device__ __forceinline__ floatx4 mm16(const HL4& a, const HL4& b, floatx4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x16f16(a.lo, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16f16(a.hi, b.lo, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a.hi, b.hi, c, 0, 0, 0);
}
__device__ __forceinline__ void st_cm(_Float16* t, floatx4 v, int lane) {
    const HL4 x = split4v(v);
    const int o = (lane & 15) * kXS + 4 * (lane >> 4);
    st4h(t + o, x.hi);
    st4h(t + 16 * kXS + o, x.lo);
}
__device__ __forceinline__ HL4 ld_b(const _Float16* t, int lane) {
    const int o = (lane & 15) * kXS + 4 * (lane >> 4);
    return HL4{*reinterpret_cast<const halfx4*>(t + o), *reinterpret_cast<const halfx4*>(t + 16 * kXS + o)};
}
__device__ __forceinline__ HL4 ld_a(const _Float16* t, int lane) {
    const int r0 = 4 * (lane >> 4);
    return HL4{tr4(t, kXS, r0, 0, lane), tr4(t + 16 * kXS, kXS, r0, 0, lane)};
}

// Block (b, a) of Tg = (I + L)^-1 diag(beta) and of Tg diag(gamma) (hi, lo) from block (b, a)
// of (I + L)^-1 in accumulator layout, into the token-column-major Tg tiles (row stride 72);
// bc, bgc: beta and beta gamma of this lane's column token 16 a + (lane & 15).
__device__ __forceinline__ void st_tg(_Float16* TgAT, _Float16* TgGT, _Float16* TgGlT, bool pt, floatx4 v, int b,
                                      int a, int lane, float bc, float bgc, const float* rr) {
    const int tc = 16 * a + (lane & 15);
    const int o = tc * (64 + 8) + 16 * b + 4 * (lane >> 4);
    floatx4 vr = v;
    if (rr) {
        // row factors Gamma / gamma_i of the lane's four row tokens
        const float4 r = *reinterpret_cast<const float4*>(rr + 16 * b + 4 * (lane >> 4));
        vr = v * floatx4{r.x, r.y, r.z, r.w};
    }
    st4h(TgAT + o, __builtin_bit_cast(halfx4, u32x2{pk_f16(vr[0] * bc, vr[1] * bc), pk_f16(vr[2] * bc, vr[3] * bc)}));
    const floatx4 gv = vr * bgc;
    const HL4 x = split4v(gv);
    st4h(TgGT + o, x.hi);
    if (pt) st4h(TgGlT + o, x.lo);
}

// (I - N)^-1 = (I + N)(I + N^2)(I + N^4)(I + N^8) for a strictly lower 16x16 N (N^16 = 0).
// The factors are polynomials in N and commute, so each step multiplies by a power of N
// from the left, with that power's transpose as the A operand.  In: N and N^T in
// accumulator layout; returns the inverse in accumulator layout.
__device__ __forceinline__ floatx4 inv16(floatx4 n, floatx4 nt, int lane) {
    floatx4 id;
#pragma unroll
    for (int i = 0; i < 4; ++i) id[i] = (4 * (lane >> 4) + i == (lane & 15)) ? 1.f : 0.f;
    const HL4 N = split4v(n), NT = split4v(nt);
    const floatx4 p2 = mm16(NT, N, zero4()), p2t = mm16(N, NT, zero4());      // N^2, (N^T)^2
    const HL4 P2 = split4v(p2), P2T = split4v(p2t);
    floatx4 r = mm16(NT, P2, id + n + p2);                                    // (I + N)(I + N^2)
    const floatx4 p4 = mm16(P2T, P2, zero4()), p4t = mm16(P2, P2T, zero4());  // N^4, (N^T)^4
    const HL4 P4 = split4v(p4), P4T = split4v(p4t);
    r = mm16(P4T, split4v(r), r);                                             // (I + N^4) ...
    const HL4 P8T = split4v(mm16(P4, P4T, zero4()));                          // (N^T)^8
    return mm16(P8T, split4v(r), r);                                          // (I + N^8) ...
}

// The off-diagonal gram blocks of wave pw: rows block rb[i], columns block cb[i].
__device__ __forceinline__ void gram_blocks_of(int pw, int& n_off, int (&rb)[2], int (&cb)[2]) {
    n_off = (pw == 0 || pw == 2) ? 2 : 1;
    rb[0] = rb[1] = 3;
    cb[0] = 0;
    cb[1] = 1;
    if (pw == 1) { rb[0] = 1; cb[0] = 0; }
    if (pw == 2) { rb[0] = 2; cb[0] = 0; rb[1] = 2; cb[1] = 1; }
    if (pw == 3) { rb[0] = 3; cb[0] = 2; }
}

// Gram blocks of wave pw from the staged K rows of a chunk: the diagonal block (pw, pw) and the
// off-diagonal blocks G_{rb[i], cb[i]} = K_rb K_cb^T in accumulator layout (rows: tokens of the
// later block rb, columns: block cb).  Each K block is read once.
template <int D>
__device__ __forceinline__ void gram_blocks(const _Float16* Kn1, int pw, int ln, floatx4& gd, floatx4 (&gt)[2]) {
    constexpr int KS = D / 32, RK = GLayout<D>::RK;
    const int g = ln >> 4, cl = ln & 15;
    auto krow = [&](int blk, int ks) { return ld8(Kn1 + (16 * blk + cl) * RK + 32 * ks + 8 * g); };
    auto mma32 = [](halfx8 x, halfx8 y, floatx4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, c, 0, 0, 0); };
    int n_off, rb[2], cb[2];
    gram_blocks_of(pw, n_off, rb, cb);
    halfx8 ka[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = krow(pw, ks);
    gd = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) gd = mma32(ka[ks], ka[ks], gd);
    gt[0] = gt[1] = zero4();
    {
        // the row block of the off-diagonal products is this wave's own (ka) except for wave 0
        // (block 3, with block 0 = ka as the first column block): each block is read once
        halfx8 kr[KS], kc[KS];
        if (pw == 0) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kr[ks] = krow(3, ks);
                kc[ks] = ka[ks];
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kr[ks] = ka[ks];
                kc[ks] = krow(cb[0], ks);
            }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) gt[0] = mma32(kr[ks], kc[ks], gt[0]);
        if (n_off > 1) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) gt[1] = mma32(kr[ks], krow(cb[1], ks), gt[1]);
        }
    }
}

// Chunk-local UT transform, wave pw of four owning token block pw: from the gram blocks of
// gram_blocks (gd, gt) and the gate vectors (G log2 e, beta, beta gamma),
// L = strictly-lower(beta_i e^{G_i - G_j} K K^T) and Tg = (I + L)^-1 diag(beta), written as
// its ten lower 16x16 blocks.  With D_b = (I + L_bb)^-1 and Inv the blocks of (I + L)^-1:
//   Inv_10 = -D_1 L_10 D_0,  Inv_32 = -D_3 L_32 D_2
//   Q_b0 = L_b0 D_0 + L_b1 Inv_10,  Q_b1 = L_b1 D_1                     (b = 2, 3)
//   Inv_2a = -D_2 Q_2a,  Inv_3a = -(Inv_32 Q_2a + D_3 Q_3a)
// Phase 1, all four waves in parallel: the diagonal gram block (pw, pw) and D_pw, and the
// off-diagonal blocks of L (0: L_30, L_31; 1: L_10; 2: L_20, L_21; 3: L_32).  Every D_b and
// L_ba goes to an exchange slot; side() (staging of later chunks) runs first, tg_wait()
// holds the first Tg write until the previous Tg has been consumed.  One barrier (pbar) among
// the four waves, then phase 2 without further hand-offs: wave 1 forms Inv_10, wave 2 block
// row 2, wave 0 Inv_32 and Inv_31, wave 3 Inv_30; each recomputes the small shared factors
// it needs (Inv_10, Inv_32, Q) instead of waiting for another wave's.
template <int D, class Bar, class Wait, class Side>
__device__ __forceinline__ void ut_blocks(const floatx4& gd, const floatx4 (&gt)[2], const float* sGl,
                                          const float* sBeta, const float* sBG, _Float16* XB, _Float16* TgAT,
                                          _Float16* TgGT, _Float16* TgGlT, bool pt, const float* rr, int pw, int ln,
                                          Bar&& pbar, Wait&& tg_wait, Side&& side) {
    const int g = ln >> 4, cl = ln & 15;
    auto slot = [&](int i) { return XB + i * kXT; };
    // exchange slots: D_b in slot b; L_10, L_20, L_21, L_30, L_31, L_32 in slots 4..9; slots 10
    // and 11 are private to waves 0 and 3 (Inv_32 turned into an A operand)
    auto lslot = [](int rb, int cb) { return rb == 1 ? 4 : rb == 2 ? 5 + cb : rb == 3 ? (cb < 2 ? 7 + cb : 9) : -1; };
    int n_off, rb[2], cb[2];
    gram_blocks_of(pw, n_off, rb, cb);
    // independent work (staging of a later chunk) first
    side();
    // beta and beta gamma of this lane's column token in each block
    float bcol[4], bgcol[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        bcol[a] = sBeta[16 * a + cl];
        bgcol[a] = sBG[16 * a + cl];
    }
    // ---- gate factors: L_{rb, cb}[r][c] = beta_r e^{G_r - G_c} G[r][c] (r later than c);
    //      N = -L_{pw,pw} and N^T for the diagonal block
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (i < n_off) {
            const float Gc = sGl[16 * cb[i] + cl];
            const float4 gr = *reinterpret_cast<const float4*>(sGl + 16 * rb[i] + 4 * g);
            const float4 br = *reinterpret_cast<const float4*>(sBeta + 16 * rb[i] + 4 * g);
            const float grs[4] = {gr.x, gr.y, gr.z, gr.w}, brs[4] = {br.x, br.y, br.z, br.w};
            floatx4 l;
#pragma unroll
            for (int u = 0; u < 4; ++u) l[u] = brs[u] * __builtin_amdgcn_exp2f(grs[u] - Gc) * gt[i][u];
            st_cm(slot(lslot(rb[i], cb[i])), l, ln);
        }
    }
    floatx4 n, nt;
    {
        const int tc = 16 * pw + cl;
        const float Gc = sGl[tc], Bc = sBeta[tc];
        const float4 gw = *reinterpret_cast<const float4*>(sGl + 16 * pw + 4 * g);
        const float4 bw = *reinterpret_cast<const float4*>(sBeta + 16 * pw + 4 * g);
        const float gws[4] = {gw.x, gw.y, gw.z, gw.w}, bws[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 4 * g + u;
            n[u] = r > cl ? -bws[u] * __builtin_amdgcn_exp2f(gws[u] - Gc) * gd[u] : 0.f;
            nt[u] = cl > r ? -Bc * __builtin_amdgcn_exp2f(Gc - gws[u]) * gd[u] : 0.f;
        }
    }
    // ---- diagonal block inverse D_pw
    const floatx4 Dm = inv16(n, nt, ln);
    st_cm(slot(pw), Dm, ln);
    tg_wait();
    st_tg(TgAT, TgGT, TgGlT, pt, Dm, pw, pw, ln, bcol[pw], bgcol[pw], rr);
    pbar(ln);
    // ---- phase 2.  A transposing read (ld_a) of a slot gives that tile as an A operand, a
    //      plain read (ld_b) as a B operand; an accumulator tile is a B operand as it is.
    if (pw == 0) {
        // Inv_32 and Inv_31 = -(Inv_32 Q_21 + D_3 Q_31)
        const HL4 D1b = ld_b(slot(1), ln), D2b = ld_b(slot(2), ln), D3a = ld_a(slot(3), ln);
        const HL4 L21a = ld_a(slot(6), ln), L31a = ld_a(slot(8), ln), L32a = ld_a(slot(9), ln);
        const floatx4 inv32 = -mm16(D3a, split4v(mm16(L32a, D2b, zero4())), zero4());
        st_cm(slot(10), inv32, ln);
        st_tg(TgAT, TgGT, TgGlT, pt, inv32, 3, 2, ln, bcol[2], bgcol[2], rr);
        const floatx4 q21 = mm16(L21a, D1b, zero4()), q31 = mm16(L31a, D1b, zero4());
        const floatx4 r1 = mm16(ld_a(slot(10), ln), split4v(q21), mm16(D3a, split4v(q31), zero4()));
        st_tg(TgAT, TgGT, TgGlT, pt, -r1, 3, 1, ln, bcol[1], bgcol[1], rr);
        return;
    }
    const HL4 D0b = ld_b(slot(0), ln), D1a = ld_a(slot(1), ln), L10a = ld_a(slot(4), ln);
    // Inv_10 = -D_1 (L_10 D_0)
    const floatx4 inv10 = -mm16(D1a, split4v(mm16(L10a, D0b, zero4())), zero4());
    if (pw == 1) {
        st_tg(TgAT, TgGT, TgGlT, pt, inv10, 1, 0, ln, bcol[0], bgcol[0], rr);
        return;
    }
    const HL4 L20a = ld_a(slot(5), ln), L21a = ld_a(slot(6), ln);
    const HL4 I10 = split4v(inv10);
    // Q_20 = L_20 D_0 + L_21 Inv_10
    const floatx4 q20 = mm16(L21a, I10, mm16(L20a, D0b, zero4()));
    if (pw == 2) {
        const HL4 D1b = ld_b(slot(1), ln), D2a = ld_a(slot(2), ln);
        const floatx4 q21 = mm16(L21a, D1b, zero4());
        st_tg(TgAT, TgGT, TgGlT, pt, -mm16(D2a, split4v(q21), zero4()), 2, 1, ln, bcol[1], bgcol[1], rr);
        st_tg(TgAT, TgGT, TgGlT, pt, -mm16(D2a, split4v(q20), zero4()), 2, 0, ln, bcol[0], bgcol[0], rr);
        return;
    }
    // wave 3: Inv_30 = -(Inv_32 Q_20 + D_3 Q_30), Q_30 = L_30 D_0 + L_31 Inv_10
    const HL4 D2b = ld_b(slot(2), ln), D3a = ld_a(slot(3), ln), L30a = ld_a(slot(7), ln),
              L31a = ld_a(slot(8), ln), L32a = ld_a(slot(9), ln);
    const floatx4 inv32 = -mm16(D3a, split4v(mm16(L32a, D2b, zero4())), zero4());
    st_cm(slot(11), inv32, ln);
    const floatx4 q30 = mm16(L31a, I10, mm16(L30a, D0b, zero4()));
    const floatx4 r0 = mm16(ld_a(slot(11), ln), split4v(q20), mm16(D3a, split4v(q30), zero4()));
    st_tg(TgAT, TgGT, TgGlT, pt, -r0, 3, 0, ln, bcol[0], bgcol[0], rr);
}

// Carry waves of a variant: D/32 per column kind present (T columns, S columns).
template <int D, bool WITH_T, bool WITH_S>
constexpr int gdn_carry_waves() {
    return ((WITH_T ? 1 : 0) + (WITH_S ? 1 : 0)) * (D / 32);
}

// WITH_T / WITH_S: the T columns and the S columns of X are carried (at least one of them).
// PT: hi/lo operands for the T columns.  Without S columns and with PT (the transition-only pass
// of the precise plan) W' itself is kept as a hi/lo pair too, in the otherwise unused V buffers.
// WO: per-token outputs o = S_t^T q_t from the segment's zero start (S columns only):
//   O = diag(gamma) Q S0 + M (U - W' S0),   M = lower(e^{G_i - G_j} q_i^T k_j) (diagonal included),
// S0 the state entering the chunk.  The S waves add diag(gamma) Q S0 to their W'X products (the
// same X operands) and M (U - W' S0) after them; the preparation waves form M of the next chunk
// after its solve, Q rows in registers against the staged K rows.
template <int D, bool WITH_T, bool WITH_S, bool IN_BF16, bool PERSIST, bool PT, bool STREAM, bool WO>
__global__ __launch_bounds__((gdn_carry_waves<D, WITH_T, WITH_S>() + 4) * 64) void gdn_build_kernel(EngineArgs a) {
    using LY = GLayout<D, WO>;
    using E = _Float16;
    constexpr int NB = D / 32;
    constexpr int NC = gdn_carry_waves<D, WITH_T, WITH_S>();   // carry waves
    static_assert(WITH_T || WITH_S, "a pass carries T columns, S columns or both");
    static_assert(!WO || (WITH_S && !WITH_T && IN_BF16 && !PT), "outputs: S columns only, 16-bit inputs, fast plan");
    constexpr int NP = 4;                       // preparation waves
    constexpr bool CV = IN_BF16 && WITH_S;      // V rows staged by carry waves
    constexpr bool PV = !IN_BF16 && WITH_S;     // ... or by the preparation waves (fp32 inputs)
    constexpr bool VS = CV;                     // ... by the S waves, after forming U
    constexpr bool VT = CV && WITH_T && !PT;    // ... and, in the fast plan, half of them by the T waves
    constexpr bool WLO = PT && !WITH_S;         // W' as hi/lo fragments (low half where V would be)
                                                //     in their idle tail before the barrier
    constexpr int NT = (NC + NP) * 64;
    // the row factors Gamma / gamma_i of Vn are folded into the Tg tiles (so into U and W') in the
    // fast plan.  The output variant keeps U - W' S0 unscaled for its outputs, and the precise plan
    // keeps the hi/lo Tg values unscaled (their low halves would sink further into the f16
    // subnormals): both scale Vn themselves, in fp32
    constexpr bool FOLD_R = !WO && !PT;
    constexpr int RK = LY::RK, RT = LY::RT;

    __shared__ __align__(16) unsigned char smem[LY::total];
    int* sCnt = reinterpret_cast<int*>(smem + LY::Misc);
    int* sEw = sCnt + 8;

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
        // STREAM: one pass runs all of this workgroup's tasks (it, it + G, it + 2G, ...; equal
        // segments) as one stream of chunks, so the preparation of a task's first chunk overlaps
        // the last carry of the previous one; c then counts chunks over the whole stream
        for (int it0 = blockIdx.x; it0 < a.n_tasks; it0 += (PERSIST && !STREAM) ? (int)gridDim.x : a.n_tasks) {
            // Within every full group of 16 task positions, positions w and w + 8 run tasks 2p and
            // 2p + 1 (p = w mod 8): the dispatcher deals workgroups to the 8 XCDs in turn, so the two
            // value heads of a key head (consecutive tasks) share an XCD and its L2, and the second
            // reads of their K rows hit there.  A bijection on the task positions (a partial last
            // group keeps its order); in the stream each group must lie inside the grid.
            const int pair_bound = STREAM ? (int)gridDim.x : a.n_tasks;
            const int it = (it0 | 15) < pair_bound ? (it0 & ~15) | (2 * (it0 & 7) + ((it0 >> 3) & 1)) : it0;
            const int per_seg = a.n_batch * a.h_v;
            const int task = STREAM ? it : task_at(a.seg, it, per_seg);
            const int seg = task / per_seg;
            const int rem = task - seg * per_seg;
            const int b = rem / a.h_v;
            const int h = rem - b * a.h_v;
            const int hk = (h * a.h_k) / a.h_v;
            const long long start = STREAM ? a.stream_start0 + seg * a.stream_stride : seg_start(a.seg, seg);
            const int len = STREAM ? a.stream_len : seg_len(a.seg, seg);
            const int ncT = (len + 63) / 64;                 // chunks per task
            const int ntw = STREAM ? (a.n_tasks - it + (int)gridDim.x - 1) / (int)gridDim.x : 1;
            const int nc = ncT * ntw;                        // chunks in this pass
            const long long chain_off = (long long)b * a.h_v + h;
            // task k of this pass is task it + k G: the same batch row and head, segment
            // seg + k dseg (the grid is a multiple of the heads per segment), so its token rows
            // start k dseg stream_stride rows further on
            const int dseg = STREAM ? (int)gridDim.x / per_seg : 0;
            auto rows_of = [&](int k) { return (long long)(k * dseg) * a.stream_stride; };
            if (tid == 0) sCnt[1] = sCnt[2] = sCnt[3] = sCnt[4] = 0;
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
                auto reset_x = [&] {
                    // a fresh opaque zero per call: the identity pattern is not loop-invariant
                    // to the compiler, so it is not kept in 64 registers across the chunk loop
                    int rz = 0;
                    asm volatile("" : "+v"(rz));
                    const int dg = diag + rz;
#pragma unroll
                    for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                        for (int j = 0; j < 16; ++j)
                            X[xb][j] = (TR && 32 * xb + 8 * (j >> 2) + (j & 3) == dg) ? 1.f : 0.f;
                };
                reset_x();
                int ew = 0;
                // T columns: rescale by an exact power of two once max |X_T| leaves [2^-4, 2) (the
                // hi/lo operands of the precise plan: [1/4, 2)), back into [0.5, 1), so the f16
                // operands of X_T and of its Vn stay clear of the f16 subnormals (a window reaching
                // down to 2^-8 raised the segment T error from 7.7e-4 to 1.2e-3).  A chunk decaying
                // T by about 2^-4 rescales every other chunk.  The NaN-propagating maximum maps to
                // gfx950's three-input maximum with |.| source modifiers (fmaxf would first
                // canonicalise every input: twice the instructions)
                auto renorm = [&] {
                    // max |X_T| of this lane as a tree of three-input maxima (22 + 8 + 3 + 1 for
                    // NB = 4): the first level takes |.| as source modifiers
                    constexpr int NX = 16 * NB, N1 = (NX + 2) / 3, N2 = (N1 + 2) / 3;
                    auto mx3 = [](float a, float b, float c) {
                        return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
                    };
                    auto xa = [&](int i) { return i < NX ? __builtin_fabsf(X[i >> 4][i & 15]) : 0.f; };
                    float m1[N1], m2[N2];
#pragma unroll
                    for (int i = 0; i < N1; ++i) m1[i] = mx3(xa(3 * i), xa(3 * i + 1), xa(3 * i + 2));
#pragma unroll
                    for (int i = 0; i < N2; ++i)
                        m2[i] = mx3(m1[3 * i], 3 * i + 1 < N1 ? m1[3 * i + 1] : 0.f, 3 * i + 2 < N1 ? m1[3 * i + 2] : 0.f);
                    float m = 0.f;
#pragma unroll
                    for (int i = 0; i < N2; i += 2) m = mx3(m, m2[i], i + 1 < N2 ? m2[i + 1] : 0.f);
                    const int e0 = exp2_of(wave_max(m));   // m in [2^(e0-1), 2^e0)
                    const int e = (e0 < (PT ? -1 : -3) || e0 > 1) ? e0 : 0;
                    if (e != 0) {
#pragma unroll
                        for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                            for (int j = 0; j < 16; ++j) X[xb][j] = ldexpf(X[xb][j], -e);
                        ew += e;
                    }
                };
                // S waves enter chunk c holding U(c) = Tg(c) V(c) in Vn (formed after the previous
                // workgroup barrier); the T waves start from zero
                floatx16 Vn[2];
                Vn[0] = Vn[1] = zero16();
                // With 16-bit inputs the S waves (and in the fast plan also the T waves) stage the
                // V rows: staging wave sw of NVW owns rows RPW sw .. RPW sw + RPW - 1, NQ 16-byte
                // pieces per lane (a row's pieces on consecutive lanes), loaded well before they
                // are stored.
                constexpr int NVW = VT ? 2 * NB : NB, RPW = 64 / NVW, CPR = D / 8, NQ = RPW * CPR / 64;
                constexpr int ESZ = IN_BF16 ? 2 : 4;
                Raw8<IN_BF16> cv[NQ];
                const int sw = (VT || !(WITH_T && !TR)) ? wave : wave - NB;
                const unsigned vstride = (unsigned)a.h_v * (D * ESZ);
                const unsigned char* vb0 =
                    reinterpret_cast<const unsigned char*>(a.v) + (((long long)b * N + start) * a.h_v + h) * (D * ESZ);
                auto cv_prefetch = [&](int cc, int ln) {
                    const unsigned char* vb = vb0;
                    if constexpr (STREAM) {
                        const int k = cc / ncT;
                        cc -= k * ncT;
                        vb += rows_of(k) * vstride;
                    }
                    const int valid = min(64, len - 64 * cc);
                    const unsigned char* base = vb + (long long)(64 * cc) * vstride;
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const int t = RPW * sw + (64 * q + ln) / CPR, ch = (64 * q + ln) % CPR;
                        if (t < valid)
                            cv[q].loadp(base + (t * vstride + ch * 8 * ESZ));
                        else
                            cv[q].zero();
                    }
                };
                auto cv_stage = [&](int cc, unsigned char* sm, int ln) {
                    E* dst = reinterpret_cast<E*>(sm + LY::Vn + (WO ? 0 : (cc & 1)) * LY::sz_K);
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const int t = RPW * sw + (64 * q + ln) / CPR, ch = (64 * q + ln) % CPR;
                        float x[8];
                        cv[q].get(x);
                        *reinterpret_cast<u32x4*>(dst + t * RK + 8 * ch) =
                            u32x4{pk_f16(x[0], x[1]), pk_f16(x[2], x[3]), pk_f16(x[4], x[5]), pk_f16(x[6], x[7])};
                    }
                };
                // WO: the S waves stage the rows of diag(gamma) Q of the next chunk (S wave sw: token
                // blocks sw, sw + NB, ...; the preparation waves' lane layout), loaded a period ahead
                // together with the chunk's log alpha, whose prefix gives gamma
                constexpr int KSQ = D / 32, NBQ = 4 / NB;
                Raw8<IN_BF16> cq[WO ? NBQ * KSQ : 1];
                float cla = 0.f;
                const unsigned qstride = (unsigned)a.h_k * (D * ESZ);
                const unsigned char* qb0 =
                    reinterpret_cast<const unsigned char*>(a.q) + (((long long)b * N + start) * a.h_k + hk) * (D * ESZ);
                const float* qla0 = a.log_alpha + ((long long)b * N + start) * a.h_v + h;
                auto cq_prefetch = [&](int cc, int ln) {
                    const unsigned char* qb = qb0;
                    const float* la = qla0;
                    if constexpr (STREAM) {
                        const int k = cc / ncT;
                        cc -= k * ncT;
                        qb += rows_of(k) * qstride;
                        la += rows_of(k) * a.h_v;
                    }
                    const int valid = min(64, len - 64 * cc);
                    const unsigned char* base = qb + (long long)(64 * cc) * qstride;
                    const unsigned d0b = 8 * ESZ * (ln >> 4);
#pragma unroll
                    for (int bl = 0; bl < NBQ; ++bl) {
                        const int t = 16 * (sw + NB * bl) + (ln & 15);
#pragma unroll
                        for (int ks = 0; ks < KSQ; ++ks) {
                            if (t < valid)
                                cq[bl * KSQ + ks].loadp(base + (t * qstride + d0b + 32 * ESZ * ks));
                            else
                                cq[bl * KSQ + ks].zero();
                        }
                    }
                    cla = ln < valid ? (la + (long long)(64 * cc) * a.h_v)[(unsigned)ln * a.h_v] : 0.f;
                };
                auto cq_stage = [&](unsigned char* sm, int ln) {
                    E* tile = reinterpret_cast<E*>(sm + LY::Qn);
                    const float gam = fexp(wave_scan_dpp(cla));    // gamma of token ln
#pragma unroll
                    for (int bl = 0; bl < NBQ; ++bl) {
                        const int t = 16 * (sw + NB * bl) + (ln & 15);
                        float sc = __shfl(gam, t, 64);
                        if (a.qk_l2norm) {
                            float ss = 0.f;
#pragma unroll
                            for (int ks = 0; ks < KSQ; ++ks) {
                                float x[8];
                                cq[bl * KSQ + ks].get(x);
#pragma unroll
                                for (int u = 0; u < 8; ++u) ss += x[u] * x[u];
                            }
                            ss += __shfl_xor(ss, 16, 64);
                            ss += __shfl_xor(ss, 32, 64);
                            sc = ss > 0.f ? sc / sqrtf(ss) : 0.f;
                        }
                        E* row = tile + t * RK + 8 * (ln >> 4);
#pragma unroll
                        for (int ks = 0; ks < KSQ; ++ks) {
                            float x[8];
                            cq[bl * KSQ + ks].get(x);
                            *reinterpret_cast<u32x4*>(row + 32 * ks) =
                                u32x4{pk_f16(x[0] * sc, x[1] * sc), pk_f16(x[2] * sc, x[3] * sc),
                                      pk_f16(x[4] * sc, x[5] * sc), pk_f16(x[6] * sc, x[7] * sc)};
                        }
                    }
                };
                // write a finished chain: the T waves align their slices to the largest of the
                // exponents in ex (one per T wave)
                auto write_out = [&](int segw, long long chw, const int* ex) {
                    const int half = lane >> 5, l32 = lane & 31;
                    if (TR) {
                        int emax = ex[0];
#pragma unroll
                        for (int w = 1; w < NB; ++w) emax = max(emax, ex[w]);
                        float* dst = a.T_hat + ((long long)segw * a.n_batch * a.h_v + chw) * D * D + col0 +
                                     (4 * half) * D + l32;
#pragma unroll
                        for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                            for (int j = 0; j < 16; ++j)
                                dst[(32 * xb + 8 * (j >> 2) + (j & 3)) * D] = ldexpf(X[xb][j], ew - emax);
                        if (wave == 0 && lane == 0) a.T_exp[(long long)segw * a.n_batch * a.h_v + chw] = emax;
                    } else {
                        float* dst = a.S_out + segw * a.out_stride + chw * D * D + col0 + (4 * half) * D + l32;
#pragma unroll
                        for (int xb = 0; xb < NB; ++xb)
#pragma unroll
                            for (int j = 0; j < 16; ++j) dst[(32 * xb + 8 * (j >> 2) + (j & 3)) * D] = X[xb][j];
                    }
                };
                if constexpr ((VS && !TR) || (VT && TR)) {
                    if (nc > 0) cv_prefetch(0, lane);
                }
                if constexpr (WO) {
                    if (nc > 0) cq_prefetch(0, lane);
                }
                for (int c = -1; c < nc; ++c) {
                    // opaque zeros: per-lane LDS offsets are recomputed every chunk instead of
                    // being hoisted out of the loop into long-lived registers
                    int lz = 0, lzv = 0;
                    asm volatile("" : "+s"(lz));
                    asm volatile("" : "+v"(lzv));
                    unsigned char* sm = smem + lz;
                    const int ln = lane + lzv, hf = ln >> 5;
                    const int p = c & 1, p3 = (c + 3) % 3, pn3 = (c + 4) % 3;
                    if (c >= 0) {
                        const E* Wf = reinterpret_cast<const E*>(sm + LY::Wf);
                        const E* Kn = reinterpret_cast<const E*>(sm + LY::Kn + p3 * LY::sz_K);
                        const float* Sc = reinterpret_cast<const float*>(sm + LY::Sc + p3 * LY::sz_Sc);
                        if (TR) Vn[0] = Vn[1] = zero16();
                        // Vn rows scaled by Gamma / gamma_i; X <- Gamma X before its update
                        auto scale_vn = [&] {
#pragma unroll
                            for (int mt = 0; mt < 2; ++mt) {
                                const float4* s4 = reinterpret_cast<const float4*>(Sc + 32 * mt + 4 * hf);
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    const float4 sv = s4[2 * q];   // rows 8q + 4h + 0..3
                                    Vn[mt][4 * q + 0] *= sv.x;
                                    Vn[mt][4 * q + 1] *= sv.y;
                                    Vn[mt][4 * q + 2] *= sv.z;
                                    Vn[mt][4 * q + 3] *= sv.w;
                                }
                            }
                        };
                        const float Gamma = Sc[64];
                        auto wfrag = [&](int mt, int kb, int st) {
                            return ld8(Wf + (((mt * NB + kb) * 2 + st) * 64 + ln) * 8);
                        };
                        const E* Wl = reinterpret_cast<const E*>(sm + LY::Vn);
                        auto wfrag_lo = [&](int mt, int kb, int st) {
                            return ld8(Wl + (((mt * NB + kb) * 2 + st) * 64 + ln) * 8);
                        };
                        if constexpr (PT && TR) {
                            // hi/lo X and Vn operands (the precise-T plan): plain loops, which
                            // keep this variant within its registers
#pragma unroll
                            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                                for (int st = 0; st < 2; ++st) {
                                    const HL xb = split_acc(X[kb], st);
#pragma unroll
                                    for (int mt = 0; mt < 2; ++mt) {
                                        const halfx8 fa = wfrag(mt, kb, st);
                                        if constexpr (WLO) Vn[mt] = OpF16::mma(wfrag_lo(mt, kb, st), xb.hi, Vn[mt]);
                                        Vn[mt] = OpF16::mma(fa, xb.lo, Vn[mt]);
                                        Vn[mt] = OpF16::mma(fa, xb.hi, Vn[mt]);
                                    }
                                    __builtin_amdgcn_sched_barrier(0);
                                }
                            if constexpr (!FOLD_R) scale_vn();
#pragma unroll
                            for (int xb = 0; xb < NB; ++xb) {
#pragma unroll
                                for (int j = 0; j < 16; ++j) X[xb][j] *= Gamma;
#pragma unroll
                                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                                    for (int st = 0; st < 2; ++st) {
                                        const halfx8 fa = colfrag_acc(Kn, RK, 32 * mt, 32 * xb, st, ln);
                                        const HL vb = split_acc(Vn[mt], st);
                                        X[xb] = OpF16::mma(fa, vb.lo, X[xb]);
                                        X[xb] = OpF16::mma(fa, vb.hi, X[xb]);
                                    }
                            }
                        } else {
                            // -W' X in steps (kb, st), each X fragment converted once for both
                            // token halves; the W' fragments are read two steps ahead (a ring of
                            // three) so that LDS latency hides behind earlier products
                            constexpr int NSW = 2 * NB;
                            halfx8 fw[3][2];
                            auto wload = [&](int i, halfx8 (&dst)[2]) {
#pragma unroll
                                for (int mt = 0; mt < 2; ++mt) dst[mt] = wfrag(mt, i >> 1, i & 1);
                            };
                            // WO: rows of diag(gamma) Q and of M as A operands in accumulator order
                            // (two 8-byte runs per lane)
                            const E* Qt = reinterpret_cast<const E*>(sm + LY::Qn);
                            auto rowfrag = [&](const E* r) {
                                return cat8(*reinterpret_cast<const halfx4*>(r), *reinterpret_cast<const halfx4*>(r + 8));
                            };
                            auto qfrag = [&](int mt, int i) {
                                return rowfrag(Qt + (32 * mt + (ln & 31)) * RK + 16 * i + 4 * hf);
                            };
                            floatx16 Oq[WO ? 2 : 1];
                            if constexpr (WO) Oq[0] = Oq[1] = zero16();
                            wload(0, fw[0]);
                            wload(1, fw[1]);
#pragma unroll
                            for (int i = 0; i < NSW; ++i) {
                                if (i + 2 < NSW) wload(i + 2, fw[(i + 2) % 3]);
                                halfx8 fq[2];
                                if constexpr (WO) {
#pragma unroll
                                    for (int mt = 0; mt < 2; ++mt) fq[mt] = qfrag(mt, i);
                                }
                                const halfx8 xf = OpF16::from_acc(X[i >> 1], i & 1);
#pragma unroll
                                for (int mt = 0; mt < 2; ++mt) Vn[mt] = OpF16::mma(fw[i % 3][mt], xf, Vn[mt]);
                                if constexpr (WO) {
                                    // diag(gamma) Q S0 on the same X operand
#pragma unroll
                                    for (int mt = 0; mt < 2; ++mt) Oq[mt] = OpF16::mma(fq[mt], xf, Oq[mt]);
                                }
                                __builtin_amdgcn_sched_barrier(0);
                            }
                            if constexpr (WO) {
                                // O += M (U - W' S0): Vn before its Gamma / gamma scaling, lower blocks of M
                                const E* Mt = reinterpret_cast<const E*>(sm + LY::Mo + p * LY::sz_T64);
#pragma unroll
                                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                                    for (int mj = 0; mj <= mt; ++mj)
#pragma unroll
                                        for (int st = 0; st < 2; ++st) {
                                            const halfx8 fm = rowfrag(Mt + (32 * mt + (ln & 31)) * RT + 32 * mj + 16 * st + 4 * hf);
                                            Oq[mt] = OpF16::mma(fm, OpF16::from_acc(Vn[mj], st), Oq[mt]);
                                        }
                                // store the chunk's outputs: lane (column col0 + l32, half hf), token rows
                                // 32 mt + acc_row(hf, j)
                                int cc = c;
                                long long row = (long long)b * N + start;
                                if constexpr (STREAM) {
                                    const int k = cc / ncT;
                                    cc -= k * ncT;
                                    row += rows_of(k);
                                }
                                const int valid = min(64, len - 64 * cc);
                                row += 64 * cc;
                                // a wave-uniform base and 32-bit per-store offsets; the full-chunk and
                                // dtype branches are uniform
                                auto store_o = [&](auto bf, auto full) {
                                    constexpr bool BF = decltype(bf)::value;
                                    constexpr unsigned ES = BF ? 2 : 4;
                                    unsigned char* ob = reinterpret_cast<unsigned char*>(a.o) + ((row * a.h_v + h) * D + col0) * ES;
                                    const unsigned rs = (unsigned)a.h_v * D * ES;    // bytes between token rows
                                    const unsigned lo = (unsigned)(ln & 31) * ES + (unsigned)(4 * hf) * rs;
#pragma unroll
                                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                                        for (int j = 0; j < 16; ++j) {
                                            const int tc = 32 * mt + 8 * (j >> 2) + (j & 3);   // token minus 4 hf
                                            if (decltype(full)::value || tc + 4 * hf < valid) {
                                                unsigned char* dst = ob + (lo + (unsigned)tc * rs);
                                                if constexpr (BF)   // round to nearest even (v_cvt_pk_bf16_f32)
                                                    *reinterpret_cast<__bf16*>(dst) = (__bf16)Oq[mt][j];
                                                else
                                                    *reinterpret_cast<float*>(dst) = Oq[mt][j];
                                            }
                                        }
                                };
                                if (a.out_bf16) {
                                    if (valid == 64) store_o(std::true_type{}, std::true_type{});
                                    else store_o(std::true_type{}, std::false_type{});
                                } else {
                                    if (valid == 64) store_o(std::false_type{}, std::true_type{});
                                    else store_o(std::false_type{}, std::false_type{});
                                }
                            }
                            if constexpr (!FOLD_R) scale_vn();
                            // X <- Gamma X + K^T Vn in steps (mt, st, xb): consecutive products on
                            // different X blocks, each Vn operand converted once for its NB steps,
                            // the K column fragments read two steps ahead
                            constexpr int NSX = 4 * NB;
                            auto kload = [&](int i) {
                                const int ms = i / NB;
                                return colfrag_acc(Kn, RK, 32 * (ms >> 1), 32 * (i % NB), ms & 1, ln);
                            };
                            halfx8 fk[3], vb;
                            fk[0] = kload(0);
                            fk[1] = kload(1);
#pragma unroll
                            for (int i = 0; i < NSX; ++i) {
                                if (i + 2 < NSX) fk[(i + 2) % 3] = kload(i + 2);
                                const int xb = i % NB, ms = i / NB;
                                if (ms == 0) {
#pragma unroll
                                    for (int j = 0; j < 16; ++j) X[xb][j] *= Gamma;
                                }
                                if (xb == 0) vb = OpF16::from_acc(Vn[ms >> 1], ms & 1);
                                X[xb] = OpF16::mma(fk[i % 3], vb, X[xb]);
                                __builtin_amdgcn_sched_barrier(0);
                            }
                        }
                        if (TR) renorm();
                    }
                    if constexpr (VS && !TR) {
                        // V of chunk 0 for U(0) after the first barrier; later chunks are
                        // staged after each U formation, off the barrier's critical path
                        if (c < 0 && nc > 0) {
                            cv_stage(0, sm, ln);
                            if (nc > 1) cv_prefetch(1, ln);
                        }
                    }
                    if constexpr (VT && TR) {
                        // V of chunk c+1 for U(c+1) after the barrier (its buffer held V(c-1),
                        // read by U(c-1) before the barrier before last); the T waves reach the
                        // barrier early, the S waves late.  The loads of chunk c+2 are issued
                        // after the W' formation below.
                        if (c + 1 < nc) cv_stage(c + 1, sm, ln);
                    }
                    // STREAM: the last chunk of a task ends here; exponent slots alternate by task
                    const bool task_end = STREAM && c >= 0 && (c + 1) % ncT == 0;
                    if (task_end && TR && lane == 0) sEw[4 * ((c / ncT) & 1) + wave] = ew;
                    // the K fragments of W'(c+1) are read before the barrier, off the post-barrier
                    // burst of LDS reads: K(c+1) was staged before the previous barrier (K(0) only
                    // after this one)
                    halfx8 fa_next[4];
                    auto load_fa = [&] {
                        const E* Kn1p = reinterpret_cast<const E*>(sm + LY::Kn + pn3 * LY::sz_K);
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) fa_next[kk] = colfrag_nat(Kn1p, RK, 0, 32 * wave, kk, ln);
                    };
                    constexpr bool FA = !PT;
                    if constexpr (FA) {
                        if ((TR || !WITH_T) && c >= 0 && c + 1 < nc) load_fa();
                    }
                    __syncthreads();  // preparation of chunk c+1 is complete
                    if constexpr (FA) {
                        if ((TR || !WITH_T) && c < 0 && nc > 0) load_fa();
                    }
                    if (task_end) {
                        const int k = c / ncT;
                        write_out(seg + k * dseg, chain_off, sEw + 4 * (k & 1));
                        reset_x();
                        ew = 0;
                    }
                    // From here the preparation waves go on to chunk c+2.  Its staging
                    // buffers are the other halves of the double buffers; its Tg waits for
                    // the formation counter below.  W' has one buffer: every read of W'(c)
                    // happened before the barrier above.
                    if (c + 1 < nc) {
                        const E* Kn1 = reinterpret_cast<const E*>(sm + LY::Kn + pn3 * LY::sz_K);
                        const E* TgG = reinterpret_cast<const E*>(sm + LY::TgG);
                        const E* TgGl = reinterpret_cast<const E*>(sm + LY::TgGl);
                        E* Wf1 = reinterpret_cast<E*>(sm + LY::Wf);
                        // -W'^T tiles (d rows, token columns): their accumulators are the operand
                        // fragments of W' X in the carry, stored in that order
                        if (TR || !WITH_T) {
                            const int dt = wave;
                            auto store_w = [&](int mt, const floatx16& acc) {
#pragma unroll
                                for (int st = 0; st < 2; ++st) {
                                    const int o = (((mt * NB + dt) * 2 + st) * 64 + ln) * 8;
                                    if constexpr (WLO) {
                                        floatx16 neg;
#pragma unroll
                                        for (int i = 0; i < 16; ++i) neg[i] = -acc[i];
                                        const HL w = split_acc(neg, st);
                                        *reinterpret_cast<halfx8*>(Wf1 + o) = w.hi;
                                        *reinterpret_cast<halfx8*>(reinterpret_cast<E*>(sm + LY::Vn) + o) = w.lo;
                                    } else {
                                        halfx8 w;
#pragma unroll
                                        for (int i = 0; i < 8; ++i) w[i] = (_Float16)(-acc[8 * st + i]);
                                        *reinterpret_cast<halfx8*>(Wf1 + o) = w;
                                    }
                                }
                            };
                            if constexpr (PT) {
#pragma unroll
                                for (int mt = 0; mt < 2; ++mt) {
                                    floatx16 acc = zero16();
#pragma unroll
                                    for (int kk = 0; kk < 2 + 2 * mt; ++kk) {   // Tg lower triangular
                                        const halfx8 fa = colfrag_nat(Kn1, RK, 0, 32 * dt, kk, ln);
                                        acc = OpF16::mma(fa, colfrag_nat(TgGl, RT, 0, 32 * mt, kk, ln), acc);
                                        acc = OpF16::mma(fa, colfrag_nat(TgG, RT, 0, 32 * mt, kk, ln), acc);
                                    }
                                    store_w(mt, acc);
                                }
                            } else {
                                // the fragments of the first half in flight before the products; Tg is
                                // lower triangular, so the first 32 tokens take keys 0..31 only
                                halfx8 fb[2];
                                const halfx8* fa = fa_next;
#pragma unroll
                                for (int kk = 0; kk < 2; ++kk) fb[kk] = colfrag_nat(TgG, RT, 0, 0, kk, ln);
#pragma unroll
                                for (int mt = 0; mt < 2; ++mt) {
                                    floatx16 acc = zero16();
#pragma unroll
                                    for (int kk = 0; kk < 2 + 2 * mt; ++kk)
                                        acc = OpF16::mma(fa[kk], mt == 0 ? fb[kk] : colfrag_nat(TgG, RT, 0, 32, kk, ln), acc);
                                    store_w(mt, acc);
                                }
                            }
                        }
                        // W'(c+1) formed (its Tg reads done): the forming waves count it on the
                        // W' hand-off counter and, with T, on the Tg-reuse counter
                        if (TR || !WITH_T) count_arrival(sCnt + 1, ln);
                        if (WITH_T && TR && ln == 0)
                            __hip_atomic_fetch_add(sCnt + 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                        if constexpr (VT && TR) {
                            if (c + 2 < nc) cv_prefetch(c + 2, ln);
                        }
                        if (!TR) {
                            // U(c+1) = Tg V for this wave's columns, both token halves per V fragment,
                            // formed beside W'(c+1) and carried into the next chunk in Vn
                            const E* TgA = reinterpret_cast<const E*>(sm + LY::TgA);
                            const E* Vc = reinterpret_cast<const E*>(sm + LY::Vn + (WO ? 0 : (p ^ 1)) * LY::sz_K);
                            Vn[0] = Vn[1] = zero16();
#pragma unroll
                            for (int kk = 0; kk < 4; ++kk) {
                                const halfx8 fb = colfrag_nat(Vc, RK, 0, col0, kk, ln);
#pragma unroll
                                for (int mt = 0; mt < 2; ++mt) {
                                    // Tg lower triangular: tokens 0..31 take values 0..31 only
                                    if (mt == 0 && kk >= 2) continue;
                                    Vn[mt] = OpF16::mma(colfrag_nat(TgA, RT, 0, 32 * mt, kk, ln), fb, Vn[mt]);
                                }
                            }
                            if constexpr (WO) {
                                // Q of chunk c+1 into the one Q tile (its last reader, the Q S0 products
                                // of chunk c, ran before the barrier); every S wave waits for this
                                // counter (below) before its next carry
                                cq_stage(sm, ln);
                                if (c + 2 < nc) cq_prefetch(c + 2, ln);
                            }
                            // Tg(c+1) consumed: the preparation of chunk c+2 may overwrite it
                            count_arrival(sCnt + 2, ln);
                            if constexpr (VS) {
                                // V of chunk c+2 into the buffer that held V(c) (read by U(c), formed
                                // before the previous barrier), then the loads of c+3.  With outputs
                                // there is one V buffer: first every S wave's U(c+1) has read it (and
                                // staged its rows of Q(c+1))
                                if constexpr (WO) wait_count(sCnt + 2, NC * (c + 2));
                                if (c + 2 < nc) {
                                    cv_stage(c + 2, sm, ln);
                                    if (c + 3 < nc) cv_prefetch(c + 3, ln);
                                }
                            }
                        }
                        // every carry wave waits for the whole of W'(c+1)
                        wait_count(sCnt + 1, NB * (c + 2));
                    }
                }
                // epilogue: align the T waves' exponents, write T_hat / T_exp / S
                if constexpr (!STREAM) {
                    if (TR && lane == 0) sEw[wave] = ew;
                    __syncthreads();
                    write_out(seg, chain_off, sEw);
                }
            } else {
                // ======================== preparation waves ========================
                // Wave pw owns token block pw (rows 16 pw .. 16 pw + 15) of every chunk in the
                // solve.  While the gram products of chunk c+1 are in flight, each wave stages the
                // K rows of its block of chunk c+2 and wave 1 its gate vectors.  With fp32 inputs
                // each wave also stages the V rows of its block of chunk c+1 after the solve (with
                // 16-bit inputs the S carry waves do that).
                const int pw = wave - NC;
                constexpr int KS = D / 32;  // 32-wide contraction steps over d
                Raw8<IN_BF16> pk[KS], pv[KS];
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
                // lane (row 16 blk + (ln & 15), d = 32 ks + 8 (ln >> 4) .. + 7)
                auto load_rows = [&](Raw8<IN_BF16>* dst, const unsigned char* base, unsigned stride, int blk, int valid,
                                     int ln) {
                    const int t = 16 * blk + (ln & 15);
                    const unsigned d0b = 8 * ESZ * (ln >> 4);
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        if (t < valid)
                            dst[ks].loadp(base + (t * stride + d0b + 32 * ESZ * ks));
                        else
                            dst[ks].zero();
                    }
                };
                // scaled: rows multiplied by sc (the key L2 normalisation)
                auto store_rows = [&](const Raw8<IN_BF16>* src, E* dst, int blk, float sc, int ln, auto scaled) {
                    E* row = dst + (16 * blk + (ln & 15)) * RK + 8 * (ln >> 4);
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        float x[8];
                        src[ks].get(x);
                        if constexpr (!decltype(scaled)::value) {
                            *reinterpret_cast<u32x4*>(row + 32 * ks) =
                                u32x4{pk_f16(x[0], x[1]), pk_f16(x[2], x[3]), pk_f16(x[4], x[5]), pk_f16(x[6], x[7])};
                            continue;
                        }
                        *reinterpret_cast<u32x4*>(row + 32 * ks) =
                            u32x4{pk_f16(x[0] * sc, x[1] * sc), pk_f16(x[2] * sc, x[3] * sc),
                                  pk_f16(x[4] * sc, x[5] * sc), pk_f16(x[6] * sc, x[7] * sc)};
                    }
                };
                // K rows of block pw and (wave 1, which has the least gram work) the gates of chunk cc
                constexpr int GW = 1;
                auto prefetch_kg = [&](int cc, int ln) {
                    const unsigned char* kb = kb0;
                    const float *la = la0, *bt = bt0;
                    if constexpr (STREAM) {
                        const int k = cc / ncT;
                        cc -= k * ncT;
                        const long long dr = rows_of(k);
                        kb += dr * kstride;
                        la += dr * a.h_v;
                        bt += dr * a.h_v;
                    }
                    const int valid = min(64, len - 64 * cc);
                    load_rows(pk, kb + (long long)(64 * cc) * kstride, kstride, pw, valid, ln);
                    if (pw == GW) {
                        const bool ok = ln < valid;
                        const unsigned go = (unsigned)ln * a.h_v;
                        pla = ok ? (la + (long long)(64 * cc) * a.h_v)[go] : 0.f;
                        pbt = ok ? (bt + (long long)(64 * cc) * a.h_v)[go] : 0.f;
                    }
                };
                auto prefetch_v = [&](int cc, int ln) {
                    const int valid = min(64, len - 64 * cc);
                    load_rows(pv, vb0 + (long long)(64 * cc) * vstride, vstride, pw, valid, ln);
                };
                // WO: the Q rows of block pw of a chunk, held in registers for its M block row
                Raw8<IN_BF16> pq[WO ? KS : 1];
                const unsigned char* qb0 =
                    reinterpret_cast<const unsigned char*>(a.q) + (row0 * a.h_k + hk) * (D * ESZ);
                auto prefetch_q = [&](int cc, int ln) {
                    const unsigned char* qb = qb0;
                    if constexpr (STREAM) {
                        const int k = cc / ncT;
                        cc -= k * ncT;
                        qb += rows_of(k) * kstride;
                    }
                    const int valid = min(64, len - 64 * cc);
                    load_rows(pq, qb + (long long)(64 * cc) * kstride, kstride, pw, valid, ln);
                };
                // M of chunk cc, block row pw: M_ij = e^{G_i - G_j} q_i.k_j for the keys j <= i of
                // blocks 0..pw, from the K rows staged for the solve; computed transposed (key rows
                // as the A operand) so that each lane stores four consecutive j of one row i
                auto form_m = [&](int cc, unsigned char* sm, int ln) {
                    const E* Kc = reinterpret_cast<const E*>(sm + LY::Kn + (cc % 3) * LY::sz_K);
                    const float* sGl = reinterpret_cast<const float*>(sm + LY::Gv + (cc & 1) * (3 * 64 * 4));
                    E* Mt = reinterpret_cast<E*>(sm + LY::Mo + (cc & 1) * LY::sz_T64);
                    const int cl = ln & 15, g = ln >> 4;
                    float qs = 1.f;
                    if (a.qk_l2norm) {
                        float ss = 0.f;
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            float x[8];
                            pq[ks].get(x);
#pragma unroll
                            for (int u = 0; u < 8; ++u) ss += x[u] * x[u];
                        }
                        ss += __shfl_xor(ss, 16, 64);
                        ss += __shfl_xor(ss, 32, 64);
                        qs = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
                    }
                    halfx8 qb[KS];
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        float x[8];
                        pq[ks].get(x);
#pragma unroll
                        for (int u = 0; u < 8; ++u) qb[ks][u] = (_Float16)(x[u] * qs);
                    }
                    const int i = 16 * pw + cl;
                    const float Gi = sGl[i];
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) {
                        if (cb > pw) break;
                        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks)
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                ld8(Kc + (16 * cb + cl) * RK + 32 * ks + 8 * g), qb[ks], acc, 0, 0, 0);
                        const float4 gj = *reinterpret_cast<const float4*>(sGl + 16 * cb + 4 * g);
                        const float gjs[4] = {gj.x, gj.y, gj.z, gj.w};
                        float m[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int j = 16 * cb + 4 * g + u;
                            m[u] = j <= i ? __builtin_amdgcn_exp2f(Gi - gjs[u]) * acc[u] : 0.f;
                        }
                        *reinterpret_cast<u32x2*>(Mt + i * RT + 16 * cb + 4 * g) =
                            u32x2{pk_f16(m[0], m[1]), pk_f16(m[2], m[3])};
                    }
                };
                auto stage_kg = [&](int cc, unsigned char* sm, int ln) {
                    float sc = 1.f;
                    if (a.qk_l2norm) {
                        float ss = 0.f;
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            float x[8];
                            pk[ks].get(x);
#pragma unroll
                            for (int u = 0; u < 8; ++u) ss += x[u] * x[u];
                        }
                        ss += __shfl_xor(ss, 16, 64);
                        ss += __shfl_xor(ss, 32, 64);
                        sc = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
                    }
                    E* kt = reinterpret_cast<E*>(sm + LY::Kn + (cc % 3) * LY::sz_K);
                    if (a.qk_l2norm)
                        store_rows(pk, kt, pw, sc, ln, std::true_type{});
                    else
                        store_rows(pk, kt, pw, sc, ln, std::false_type{});
                    if (pw == GW) {
                        float* sGl = reinterpret_cast<float*>(sm + LY::Gv + (cc & 1) * (3 * 64 * 4));
                        float* Scc = reinterpret_cast<float*>(sm + LY::Sc + (cc % 3) * LY::sz_Sc);
                        const float G = wave_scan_dpp(pla);
                        const float Glast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), 63));
                        const float Gl = G * 1.4426950408889634f;
                        sGl[ln] = Gl;
                        sGl[64 + ln] = pbt;
                        sGl[128 + ln] = pbt * __builtin_amdgcn_exp2f(Gl);
                        Scc[ln] = fexp(Glast - G);
                        if (ln == 0) Scc[64] = fexp(Glast);
                    }
                };
                auto stage_v = [&](int cc, unsigned char* sm, int ln) {
                    store_rows(pv, reinterpret_cast<E*>(sm + LY::Vn + (cc & 1) * LY::sz_K), pw, 1.f, ln, std::false_type{});
                };
                auto pbar = [&](int ln) {
                    pb_target += NP;
                    prep_barrier(sCnt, pb_target, ln);
                };
                // the preparation waves are the critical path of every chunk: let their few
                // instructions issue ahead of the carry waves' (matrix-core bound) stream
                __builtin_amdgcn_s_setprio(3);
                // gram of the next chunk to solve, formed before the workgroup barrier that precedes
                // its solve (its K rows are staged, and visible to all four waves, one barrier earlier)
                floatx4 gd, gt[2];
                if (nc > 0) {
                    prefetch_kg(0, lane);
                    if constexpr (PV) prefetch_v(0, lane);
                    if constexpr (WO) prefetch_q(0, lane);
                    stage_kg(0, smem, lane);
                    if (nc > 1) prefetch_kg(1, lane);
                    pbar(lane);
                    gram_blocks<D>(reinterpret_cast<const E*>(smem + LY::Kn), pw, lane, gd, gt);
                }
                for (int c = -1; c < nc; ++c) {
                    int lz = 0, lzv = 0;
                    asm volatile("" : "+s"(lz));
                    asm volatile("" : "+v"(lzv));
                    unsigned char* sm = smem + lz;
                    const int ln = lane + lzv;
                    if (c + 1 < nc) {
                        E* XB = reinterpret_cast<E*>(sm + LY::XB);
                        E* TgAT = reinterpret_cast<E*>(sm + LY::TgA);
                        E* TgGT = reinterpret_cast<E*>(sm + LY::TgG);
                        E* TgGlT = reinterpret_cast<E*>(sm + LY::TgGl);
                        const float* sGl = reinterpret_cast<const float*>(sm + LY::Gv + ((c + 1) & 1) * (3 * 64 * 4));
                        // solve chunk c+1 (K and gates staged before the last workgroup barrier);
                        // meanwhile stage K and gates of chunk c+2 (buffers last read before it)
                        ut_blocks<D>(gd, gt, sGl, sGl + 64, sGl + 128, XB, TgAT, TgGT, TgGlT, PT,
                                     FOLD_R ? reinterpret_cast<const float*>(sm + LY::Sc + ((c + 1) % 3) * LY::sz_Sc) : nullptr,
                                     pw, ln, pbar,
                                     [&] {
                                         // Tg(c+1) overwrites Tg(c): wait until the carry waves
                                         // formed W'(c) and U(c)
                                         wait_count(sCnt + 2, NC * (c + 1));
                                     },
                                     [&] {
                                         if (c + 2 < nc) {
                                             stage_kg(c + 2, sm, ln);
                                             if (c + 3 < nc) prefetch_kg(c + 3, ln);
                                         }
                                     });
                        // V of chunk c+1 (its buffer was last read by U(c-1), a period ago)
                        if constexpr (PV) {
                            stage_v(c + 1, sm, ln);
                            if (c + 2 < nc) prefetch_v(c + 2, ln);
                        }
                        // M of chunk c+1 (its buffer held M(c-1), read by the carry of c-1), then the
                        // Q rows of chunk c+2
                        if constexpr (WO) {
                            form_m(c + 1, sm, ln);
                            if (c + 2 < nc) prefetch_q(c + 2, ln);
                        }
                    }
                    // gram of chunk c+2: its K rows were staged before this chunk's prep barrier
                    if (c + 2 < nc) {
                        const E* Kn2 = reinterpret_cast<const E*>(sm + LY::Kn + ((c + 2) % 3) * LY::sz_K);
                        gram_blocks<D>(Kn2, pw, ln, gd, gt);
                    }
                    __syncthreads();  // chunk c+1 prepared
                }
                if constexpr (!STREAM) __syncthreads();  // epilogue exponent exchange
            }
        }
    };
    if (is_c) {
        if constexpr (WITH_T) {
            if (t_wave) run(std::integral_constant<int, 0>{});
        }
        if constexpr (WITH_S) {
            if (!t_wave) run(std::integral_constant<int, 1>{});
        }
    } else {
        run(std::integral_constant<int, 2>{});
    }
}

template <int D, bool WITH_T, bool WITH_S, bool IN_BF16, bool PT, bool WO = false>
static hipError_t launch_v(const EngineArgs& a, int grid, hipStream_t s) {
    constexpr int nt = (gdn_carry_waves<D, WITH_T, WITH_S>() + 4) * 64;
    if (a.stream) {
        // one stream of chunks per persistent workgroup (equal segments, 16-bit inputs)
        if constexpr (!IN_BF16) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gdn_build_kernel<D, WITH_T, WITH_S, IN_BF16, true, PT, IN_BF16, WO>), dim3(grid), dim3(nt), 0,
                           s, a);
    } else if (a.persistent) {
        hipLaunchKernelGGL((gdn_build_kernel<D, WITH_T, WITH_S, IN_BF16, true, PT, false, WO>), dim3(grid), dim3(nt), 0, s,
                           a);
    } else {
        hipLaunchKernelGGL((gdn_build_kernel<D, WITH_T, WITH_S, IN_BF16, false, PT, false, WO>), dim3(grid), dim3(nt), 0, s,
                           a);
    }
    return hipGetLastError();
}

template <int D, bool IN_BF16>
static hipError_t launch_t(const EngineArgs& a, int grid, hipStream_t s) {
    if (a.q) {
        // the state pass with per-token outputs (16-bit inputs; T comes from a separate pass)
        if constexpr (!IN_BF16) return hipErrorInvalidValue;
        else if (a.T_hat) return hipErrorInvalidValue;
        else return launch_v<D, false, true, IN_BF16, false, true>(a, grid, s);
    }
    if (!a.T_hat) return launch_v<D, false, true, IN_BF16, false>(a, grid, s);             // state only
    if (a.precise_T == 2) return launch_v<D, true, false, IN_BF16, true>(a, grid, s);       // transition only, hi/lo
    if (a.precise_T == 3) return launch_v<D, true, false, IN_BF16, false>(a, grid, s);      // transition only, f16
    if (a.precise_T == 1) return launch_v<D, true, true, IN_BF16, true>(a, grid, s);        // hi/lo X, Vn for T
    return launch_v<D, true, true, IN_BF16, false>(a, grid, s);
}

hipError_t take_device_status(unsigned* out) {
    unsigned v = 0;
    const unsigned z = 0;
    hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_device_status), sizeof v, 0, hipMemcpyDeviceToHost);
    if (e == hipSuccess && v) e = hipMemcpyToSymbol(HIP_SYMBOL(g_device_status), &z, sizeof z, 0, hipMemcpyHostToDevice);
    *out = v;
    return e;
}

hipError_t launch_gdn_build(const EngineArgs& a, int d, int prec_f32, int grid, hipStream_t s) {
    if (prec_f32) return launch_dense_engine(a, d, 1, grid, s);  // fp32 operands: the general engine
    const bool bf = a.in_bf16 != 0;
    if (d == 128) return bf ? launch_t<128, true>(a, grid, s) : launch_t<128, false>(a, grid, s);
    if (d == 64) return bf ? launch_t<64, true>(a, grid, s) : launch_t<64, false>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace hypic
