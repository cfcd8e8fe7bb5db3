// kvq_device.hpp -- layout arithmetic and device helpers shared by the gfx950 kernels of libkvq.
//
// Storage format: see include/kv_quant.h. Everything here is product code; the CPU oracle has
// its own, independent implementation of the same format.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Typeless views of device memory: the pools, rings, workspaces and LDS buffers are raw bytes
// read and written as words of several widths (and the kernels reuse LDS for more than one
// purpose), so every access through a reinterpreted pointer uses a may_alias type and no
// type-based alias assumption can reorder two accesses to the same bytes.
typedef uint4 __attribute__((may_alias)) ma_uint4;
typedef uint2 __attribute__((may_alias)) ma_uint2;
typedef uint32_t __attribute__((may_alias)) ma_u32;
typedef uint16_t __attribute__((may_alias)) ma_u16;
typedef uint32_t __attribute__((ext_vector_type(4), may_alias)) ma_u32x4;
typedef float __attribute__((ext_vector_type(4), may_alias)) ma_f32x4;

constexpr int kPage = 16;
constexpr int kMaxGroup = 16;   // query heads per KV head handled by one MFMA tile

// byte layout of one (block, KV head) section for b-bit codes. The asymmetric format puts a
// zero point before each group's scale: K zero points (D fp16) then K scales, V zero points
// (P fp16) then V scales.
struct Section {
    uint32_t code_bytes;   // P*D*b/8
    uint32_t kzero_off;    // K zero points (D fp16; asymmetric format only)
    uint32_t kscale_off;   // K scales (D fp16)
    uint32_t vcode_off;    // V codes
    uint32_t vzero_off;    // V zero points (P fp16; asymmetric format only)
    uint32_t vscale_off;   // V scales (P fp16)
    uint32_t bytes;        // whole section
};

// (b = 16, the FP16 tier: K values then V values, no scales, in either format)
__host__ __device__ inline Section section_layout(int D, int bits, bool asym = false) {
    Section s;
    const uint32_t scales = bits == 16 ? 0u : 1u;
    const uint32_t per = (asym ? 2u : 1u) * scales;      // fp16 parameters per group
    s.code_bytes = (uint32_t)(kPage * D * bits / 8);
    s.kzero_off = s.code_bytes;
    s.kscale_off = s.code_bytes + (per - scales) * 2u * D;
    s.vcode_off = s.code_bytes + per * 2u * D;
    s.vzero_off = 2u * s.code_bytes + per * 2u * D;
    s.vscale_off = s.vzero_off + (per - scales) * 2u * kPage;
    s.bytes = 2u * s.code_bytes + per * (2u * D + 2u * kPage);
    return s;
}

__host__ __device__ inline int bits_of_tier(int tier) { return 2 << tier; }  // 0..3 -> 2,4,8,16
constexpr int kFp16Tier = 3;

// bit position of code k (0 .. 32/b-1) inside its 32-bit word: even codes fill the low half,
// odd codes the high half, each half low-first. A word thus unpacks into consecutive fp16 pairs
// (x0,x1), (x2,x3), ... with one shift and one mask per pair.
__host__ __device__ inline int field_bit(int k, int bits) { return 16 * (k & 1) + bits * (k >> 1); }

// ---------------------------------------------------------------- quantizer (binary32)
__device__ inline uint16_t f16_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }
__device__ inline float f16_val(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// smallest fp16 >= x for finite x >= 0 (round to nearest, then one step up if below)
__device__ inline uint16_t f32_to_f16_up(float x) {
    _Float16 h = (_Float16)x;
    uint16_t b = f16_bits(h);
    if ((float)h < x) b = (uint16_t)(b + 1);
    return b;
}

// scale of a group with absolute maximum `absmax` (0 for an all-zero group)
__device__ inline uint16_t group_scale(float absmax, int bits) {
    if (absmax == 0.0f) return 0;
    const float qmax = (float)((1 << (bits - 1)) - 1);
    return f32_to_f16_up(__fdiv_rn(absmax, qmax));
}

// code of x under scale s (s > 0), round half to even
__device__ inline int quant_code(float x, float s, int bits) {
    const float qmax = (float)((1 << (bits - 1)) - 1);
    float q = rintf(__fdiv_rn(x, s));
    q = fminf(fmaxf(q, -qmax), qmax);
    return (int)q;
}

// ---------------------------------------------------------------- asymmetric quantizer
// EchoKV, "Show the math": KIVI-style asymmetric groups. Zero point m = the group minimum (an
// fp16 value, +0 for a zero minimum), scale s = the least fp16 >= (max - m) / (2^b - 1) (0 for
// a constant group), code u = round-half-even((x - m) / s) in [0, 2^b - 1]; every decision in
// binary64, where the difference of two fp16 values and the quotients are exact enough that no
// rounding crosses a boundary.

// smallest fp16 >= x for finite x > 0 given in binary64: a nearby fp16 value, then one step
// toward x's side (the double-to-single-to-half rounding lands at most one step away)
__device__ inline uint16_t f64_to_f16_up(double x) {
    uint16_t b = f16_bits((_Float16)(float)x);
    if ((double)f16_val(b) < x)
        b = (uint16_t)(b + 1);
    else if (b > 0 && (double)f16_val((uint16_t)(b - 1)) >= x)
        b = (uint16_t)(b - 1);
    return b;
}

__device__ inline uint16_t asym_zero(float mn) { return mn == 0.f ? (uint16_t)0 : f16_bits((_Float16)mn); }

__device__ inline uint16_t asym_scale(float mn, float mx, int bits) {
    const double range = (double)mx - (double)mn;        // exact for fp16 inputs
    return range > 0.0 ? f64_to_f16_up(range / (double)((1 << bits) - 1)) : (uint16_t)0;
}

// code of x in a group with zero point m and scale s (s == 0: the constant group, code 0)
__device__ inline uint32_t asym_code(float x, float m, float s, int bits) {
    if (s == 0.f) return 0u;
    const double q = rint(((double)x - (double)m) / (double)s);
    return (uint32_t)fmin(fmax(q, 0.0), (double)((1 << bits) - 1));
}

// Max / sum over all 64 lanes of a wave, every lane active: within each row of 16 lanes by DPP
// (quad swaps, then rotations by 4 and 8), then across the four rows from one lane of each
// (readlane), with no LDS round trip. Every lane gets the same value, summed in one fixed order.
template <int CTRL>
__device__ __forceinline__ float row_dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_of(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, row_dpp<0xB1>(x));      // quad_perm [1,0,3,2]
    x = fmaxf(x, row_dpp<0x4E>(x));      // quad_perm [2,3,0,1]
    x = fmaxf(x, row_dpp<0x124>(x));     // row_ror:4
    x = fmaxf(x, row_dpp<0x128>(x));     // row_ror:8
    return fmaxf(fmaxf(lane_of(x, 0), lane_of(x, 16)), fmaxf(lane_of(x, 32), lane_of(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += row_dpp<0xB1>(x);
    x += row_dpp<0x4E>(x);
    x += row_dpp<0x124>(x);
    x += row_dpp<0x128>(x);
    return (lane_of(x, 0) + lane_of(x, 16)) + (lane_of(x, 32) + lane_of(x, 48));
}

}  // namespace kvq
