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

// byte layout of one (block, KV head) section for b-bit codes
struct Section {
    uint32_t code_bytes;   // P*D*b/8
    uint32_t kscale_off;   // K scales (D fp16)
    uint32_t vcode_off;    // V codes
    uint32_t vscale_off;   // V scales (P fp16)
    uint32_t bytes;        // whole section
};

// (b = 16, the FP16 tier: K values then V values, no scales)
__host__ __device__ inline Section section_layout(int D, int bits) {
    Section s;
    const uint32_t scales = bits == 16 ? 0u : 1u;
    s.code_bytes = (uint32_t)(kPage * D * bits / 8);
    s.kscale_off = s.code_bytes;
    s.vcode_off = s.code_bytes + scales * 2u * D;
    s.vscale_off = 2u * s.code_bytes + scales * 2u * D;
    s.bytes = 2u * s.code_bytes + scales * (2u * D + 2u * kPage);
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
