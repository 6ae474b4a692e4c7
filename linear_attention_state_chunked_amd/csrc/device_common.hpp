// Device helpers shared by the libhypic kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hypic {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kChunk = 64;

// ---------------------------------------------------------------------------------------
// 32x32 matrix-core tiles.
//
// Accumulator layout of a 32x32 tile (v_mfma_f32_32x32x*): lane l holds column l%32 and,
// in register j (0..15), row acc_row(l/32, j) = 8*(j/4) + 4*(l/32) + (j%4).
// Operands: lane l supplies row (A) / column (B) l%32 and KH consecutive contraction
// indices starting at KH*(l/32) within each KS-wide contraction step.
//
// An accumulator tile is fed back as the B operand of the next product without any
// lane exchange: register j of lane half h then stands for contraction row
// acc_row(h, j).  The A operand of that product must therefore be stored with its
// contraction axis permuted, inside every 32-block, by acc_pos(r) = position of row r,
// so that the 16 rows held by a lane half are contiguous: acc_pos(acc_row(h, j)) = 16h + j.
// All LDS operand tiles in this library use that "accumulator order" on their
// contraction axis.
__device__ __forceinline__ int acc_row(int half, int j) { return 8 * (j >> 2) + 4 * half + (j & 3); }
__host__ __device__ constexpr int acc_pos(int r) {
    return (r & ~31) | (16 * ((r >> 2) & 1) + 4 * ((r >> 3) & 3) + (r & 3));
}

struct OpF16 {
    using elem = _Float16;
    using frag = halfx8;
    static constexpr int KS = 16;  // contraction per instruction
    static constexpr int KH = 8;   // contraction values per lane
    __device__ static __forceinline__ floatx16 mma(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ frag load(const elem* p) { return *reinterpret_cast<const frag*>(p); }
    // registers [KH*st, KH*st+KH) of an accumulator tile as an operand
    __device__ static __forceinline__ frag from_acc(const floatx16& a, int st) {
        frag r;
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = (_Float16)a[8 * st + i];
        return r;
    }
    __device__ static __forceinline__ elem cvt(float x) { return (_Float16)x; }
};

struct OpF32 {
    using elem = float;
    using frag = float;
    static constexpr int KS = 2;
    static constexpr int KH = 1;
    __device__ static __forceinline__ floatx16 mma(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ frag load(const elem* p) { return *p; }
    __device__ static __forceinline__ frag from_acc(const floatx16& a, int st) { return a[st]; }
    __device__ static __forceinline__ elem cvt(float x) { return x; }
};

__device__ __forceinline__ floatx16 zero16() {
    floatx16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// ---------------------------------------------------------------------------------------
// scalar conversions

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float32 -> bf16 bits, round to nearest even (gfx950's v_cvt_pk_bf16_f32; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// load 8 consecutive input elements (bf16 or f32) as floats; p must be 16-byte aligned
// for bf16 and 32-byte aligned for f32.
__device__ __forceinline__ void load8(const void* base, long long idx, bool bf16, float (&x)[8]) {
    if (bf16) {
        const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(ws[i] << 16);
            x[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
        const float4 a = p[0], b = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

// ---------------------------------------------------------------------------------------
// wave reductions (64 lanes)

// Maximum over the 64 lanes with no LDS traffic: DPP lane permutations reduce each row of
// 16 lanes (quad_perm [1,0,3,2], quad_perm [2,3,0,1], half-row mirror, row mirror), then
// the four row maxima are read out with readlane.  A shuffle-based reduction issues six
// ds_bpermute round trips, which queue behind the matrix-core kernels' fragment reads.
template <int CTRL>
__device__ __forceinline__ float dpp_perm(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_perm<0xb1>(v));    // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_perm<0x4e>(v));    // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_perm<0x141>(v));   // row_half_mirror
    v = fmaxf(v, dpp_perm<0x140>(v));   // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
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

// Sum over aligned groups of G adjacent lanes (G = 4, 8 or 16, within one DPP row); every lane
// of a group gets its group's sum.  All 64 lanes must be active.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G == 4 || G == 8 || G == 16, "group of 4, 8 or 16 lanes");
    v += dpp_perm<0xb1>(v);                        // quad_perm [1,0,3,2]
    v += dpp_perm<0x4e>(v);                        // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v += dpp_perm<0x141>(v);  // row_half_mirror
    if constexpr (G >= 16) v += dpp_perm<0x140>(v); // row_mirror
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_inclusive_scan(float v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

// exponent e with m = f * 2^e, f in [0.5, 1); 0 for m == 0
__device__ __forceinline__ int exp2_of(float m) {
    int e = 0;
    if (m > 0.f) (void)frexpf(m, &e);
    return e;
}

}  // namespace hypic
