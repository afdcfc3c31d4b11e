// Device-side helpers shared by the gfx950 kernels of the MoE layer:
// vector types for the MFMA builtins, bf16 and OCP e4m3 conversions, and
// 64-lane wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// binary32 -> bf16 bits, round to nearest even; a NaN keeps its sign and
// top payload bits and is made quiet ((u >> 16) | 0x40).  gfx950's
// v_cvt_pk_bf16_f32 computes exactly this for every binary32 input in the
// kernels' default mode (nearest-even rounding, denormals kept), two values
// per instruction.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_hw{lo, hi}, bf16x2_hw));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// binary32 -> OCP FP8 E4M3FN byte: round to nearest even, saturate to +-448
// (the format has no infinity; S.1111.111 is NaN).  Normal range: keep the
// top 3 mantissa bits with RNE on the 20 dropped bits; a mantissa carry moves
// into the exponent field by plain addition.  Below 2^-6 the codes are the
// multiples of 2^-9, so the code is rint(|v| * 512).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    float af = __uint_as_float(a);
    if (!(af < 464.0f)) return sign | 0x7eu;
    if (af < 0.015625f) return sign | (uint32_t)__builtin_rintf(af * 512.0f);
    uint32_t e = (a >> 23) - 120u;  // biased e4m3 exponent, 1..15
    uint32_t keep = (a >> 20) & 7u, rem = a & 0xfffffu;
    keep += (rem > 0x80000u) | ((rem == 0x80000u) & keep);
    uint32_t code = (e << 3) + keep;
    return sign | (code > 0x7eu ? 0x7eu : code);
}

// Four values already in the e4m3 range (|v| <= 448, as a tile's values
// divided by its scale are) -> four OCP e4m3 codes in one word (byte i from
// the i-th value), by the hardware conversion: round to nearest even, the
// same codes as f32_to_e4m3 on that range (checked exhaustively over ties,
// subnormals and the top of the range on gfx950).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Scale of one e4m3 tile (1x128 activations, 128x128 weight blocks): the
// smallest power of two at or above amax / 448 (fp32 division), 1 for an
// all-zero tile.  A power of two: dividing by it is exact, and its exponent
// field is the E8M0 scale the block-scaled MFMA takes.
__device__ __forceinline__ float e4m3_tile_scale(float amax) {
    if (!(amax > 0.f)) return 1.0f;
    uint32_t b = __float_as_uint(amax / 448.0f);
    if (b & 0x7fffffu) b = (b & 0xff800000u) + 0x800000u;
    return __uint_as_float(b);
}

// The E8M0 byte of a tile scale from e4m3_tile_scale: its biased exponent
// field (OCP MX E8M0: byte e stands for 2^(e-127); the scales here are
// 2^-126 .. 2^127, bytes 1 .. 254).
__device__ __forceinline__ uint32_t e8m0_of(float pow2) { return (__float_as_uint(pow2) >> 23) & 0xffu; }

// Totally ordered key of a float (larger float -> larger unsigned key).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// v from lane (lane permuted by the DPP control CTRL), 64-bit.  A lane whose
// source is out of range keeps its own value (old = v).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
    const uint32_t plo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xf, 0xf, false);
    const uint32_t phi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xf, 0xf, false);
    return ((uint64_t)phi << 32) | plo;
}

// Maximum over the 64 lanes of a full wave (every lane active), returned
// wave-uniform: DPP within each 16-lane row (quad swaps xor 1 and xor 2, then
// the half-row and row mirrors), then the four row maxima read from lanes
// 0, 16, 32, 48.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint64_t o;
    o = dpp_u64<0xB1>(v);   // quad_perm [1,0,3,2]
    v = o > v ? o : v;
    o = dpp_u64<0x4E>(v);   // quad_perm [2,3,0,1]
    v = o > v ? o : v;
    o = dpp_u64<0x141>(v);  // row_half_mirror: lane i <-> 7 - i within 8
    v = o > v ? o : v;
    o = dpp_u64<0x140>(v);  // row_mirror: lane i <-> 15 - i within 16
    v = o > v ? o : v;
    uint64_t m = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r);
        const uint64_t x = ((uint64_t)hi << 32) | lo;
        m = x > m ? x : m;
    }
    return m;
}

__device__ __forceinline__ float wave_max_f32(float v, int width) {
    for (int s = width / 2; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, kWave));
    return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) {
        int o = __shfl_up(v, s, kWave);
        if (lane >= s) v += o;
    }
    return v;
}

}  // namespace moe
