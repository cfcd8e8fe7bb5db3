// kv_attn.hip -- fused dequantize + grouped-query split-K decode attention (gfx950).
//
// EchoKV, "What happens to old blocks...": paged attention reads every block at the width it
// was stored with, so one layer's cache may mix INT2 / INT4 / INT8 pages. Behavior-Guided
// KV-Cache Quantization, "Storage savings": GQA head mapping (query head h reads KV head
// h / group). KV-Kaizen summary, "Background": decoding reads the entire cache per token, so
// the kernel is built to stream the packed pages at HBM rate.
//
// Work decomposition. A workgroup of 8 waves owns one (sequence, KV head, split) -- a run of
// `pps` pages; each wave takes a contiguous chunk of the split and walks it in page pairs, two
// pairs in flight. A chunk whose pages share one width (the common case) runs a loop compiled
// for that width; otherwise each page carries its own. Per page pair a wave computes, on MFMA
// (v_mfma_f32_16x16x32_f16):
//   S^T[t][h] = sum_c Kcode[t][c] * q'[h][c],  q' = q * Kscale(page, c)     (16 tokens a page)
//   o^T[c][h] += sum_t Vcode[t][c] * p'[h][t], p' = p * Vscale(t)          (32 tokens a pair)
// K and V codes become exact fp16 integers (masks, then v_perm_b32 or v_and_or_b32 with the
// exponent of 1024, then one exact packed add or fused multiply-add). Normal numbers on purpose:
// fp16 subnormal MFMA operands lose precision once their products mix with larger ones (measured
// on gfx950: about 2^-12.5 of the sum of magnitudes, against 2^-22 for normal operands). The K
// scales fold into q: exactly for INT2 (code * scale is exact when |code| <= 1), otherwise as two
// fp16 parts hi + lo of q * scale so the products stay exact to ~2^-22; the weights p * Vscale
// enter as two fp16 parts hi + lo of their fp32 product, so no term carries more than ~2^-22 of
// rounding and nothing cancels. Computing S and o transposed puts head h in lane h%16 of both
// products, so the softmax output is the PV operand in place and the rescale by
// exp(m_old - m_new) is lane-local. Query heads beyond the group are zero MFMA rows.
// Waves merge in LDS; splits merge through the workspace: the last workgroup of a (sequence,
// KV head) to finish -- found with an atomic ticket -- combines the partials in split order, so
// results do not depend on scheduling. Split s and group g map to blockIdx s * groups + g, which
// keeps all splits of a group on one XCD when groups % 8 == 0.
//
// The asymmetric format (ASYM; EchoKV, "Future work": per-token KIVI storage) adds a zero point
// m beside every scale: a logit over m + u*s is the zero-point part sum_c q_c m_c -- four more
// MFMAs per page with the zero points in every row of the A operand against q itself, exact in
// fp32 -- plus the code part on the unsigned codes u; the value side adds sum_t p_t m_t, one
// number per head, to every channel of the head after the loop.
#include "kvq_device.hpp"
#include "kvq_launch.hpp"
#include "kvq_write_dev.hpp"

#include <mutex>

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// read-only tables indexed by wave-uniform values: the constant address space lets the compiler
// use scalar loads, so block-table lookups never wait on the vector-memory counter
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

constexpr int kWaves = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSplits = 256;

// The split-ticket counters of different (sequence, KV head) groups sit 256 bytes apart: packed
// into one line, the tickets of all groups -- taken within a microsecond of each other at the
// end of a launch -- queue on that one line and the last returns microseconds later.
#ifndef KVQ_CTR_STRIDE
#define KVQ_CTR_STRIDE 64
#endif
constexpr int kCounterStride = KVQ_CTR_STRIDE;   // uint32 words per counter

struct AttnArgs {
    PoolPtrs pools;
    const uint32_t* bt;
    const int32_t* ctx_len;
    const uint16_t* q;
    float* out;
    uint32_t* counters;   // [groups][kCounterStride]: one counter per group, each in its own line
    float* ws_ml;         // [groups][group][splits][2] (max, sum) in log2 units
    float* ws_o;          // [groups][splits][group][D]
    int max_pages;
    int H;                // KV heads
    int Hq;
    int grp;              // query heads per KV head
    int groups;           // batch * H
    int splits;
    int pps;              // pages per split
    float scale_log2;     // softmax_scale * log2(e)
    // fused decode step only: the write of n_new tokens at pos, done before the attention
    const int32_t* pos;
    int n_new;
    WriteArgs wr;
};

// raw bytes of one page, as this lane needs them
struct PageRaw {
    uint32_t k[8];   // this lane's K code chunk (token lane%16, channels of lane group)
    uint32_t v[8];   // this lane's V code chunk (token quad lane/16, channels of lane%16)
    uint32_t ks;     // two K scales (channels 2*lane, 2*lane+1)
    uint32_t vs[2];  // four V scales (tokens 4*(lane/16) .. +3)
    uint32_t kz;     // asymmetric format: the two K zero points of the same channels
    uint32_t vz[2];  // asymmetric format: the four V zero points of the same tokens
    int bits;        // 0 = no page
    int ntok;        // valid tokens in the page
};

// what the width-independent page loads need, as plain values (the kernel argument block is
// never addressed, so it stays in scalar registers)
struct PageSrc {
    const uint8_t* base0;
    const uint8_t* base1;
    const uint8_t* base2;
    const uint8_t* base3;     // FP16 tier
    const uint32_t* bt_row;   // this sequence's block-table row
    int H;
};

// pool base of a tier by arithmetic rather than a select chain, which the compiler would
// otherwise turn into a lookup table in scratch memory
__device__ __forceinline__ const uint8_t* tier_base(const PageSrc& a, int tier) {
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(a.base0);
    return reinterpret_cast<const uint8_t*>(
        b0 + (uintptr_t)(tier == 1) * (reinterpret_cast<uintptr_t>(a.base1) - b0) +
        (uintptr_t)(tier == 2) * (reinterpret_cast<uintptr_t>(a.base2) - b0) +
        (uintptr_t)(tier == 3) * (reinterpret_cast<uintptr_t>(a.base3) - b0));
}

// Loads of one page for this lane, width read from its handle. The instruction sequence is the
// same for every tier (two 16-byte K loads, two 16-byte V loads, one scale dword, one scale pair):
// the second 16 bytes are only needed by INT8, so INT2/INT4 re-read their first 16 bytes (same
// cache lines, all inside the section). A fixed count lets the compiler wait for exactly one
// page's loads while the next pairs' loads stay in flight. `page` must be a valid page index
// even when `present` is false. An FP16 page (bits 16) is read later, by its own path: here its
// lane loads use INT2 offsets, which stay inside its (larger) section, and are not used.
template <int D, bool ASYM = false>
__device__ __forceinline__ void load_page(const PageSrc& a, int kv, int page, bool present,
                                          int ctx, int lane, PageRaw& r) {
    const uint32_t handle = ((const_u32_ptr)a.bt_row)[page];
    const int tier = (int)(handle >> 30);
    const uint32_t idx = handle & 0x3fffffffu;
    const int bits = bits_of_tier(tier);
    r.bits = present ? bits : 0;
    r.ntok = present ? min(kPage, ctx - page * kPage) : 0;
    const bool f16 = tier == kFp16Tier;
    constexpr uint32_t kpar = (ASYM ? 4 : 2) * D, vpar = (ASYM ? 4 : 2) * kPage;   // group parameters
    const uint32_t sec_bytes = f16 ? 4u * kPage * D : kPage * D * bits / 4 + kpar + vpar;
    const uint8_t* sec = tier_base(a, tier) + ((size_t)idx * a.H + kv) * sec_bytes;
    const int lb = f16 ? 2 : bits;                  // the layout the lane offsets follow
    const uint32_t code_bytes = kPage * D * lb / 8;
    const int t = lane & 15, G = lane >> 4;
    const int ch = D * lb / 32;                     // bytes of one lane chunk
    const uint8_t* kp = sec + t * (D * lb / 8) + G * ch;
    const uint8_t* vp = sec + code_bytes + kpar + (G * D + t * (D / 16)) * lb / 2;
    const int second = lb == 8 ? 16 : 0;
    const uint4 k0 = *reinterpret_cast<const ma_uint4*>(kp);
    const uint4 k1 = *reinterpret_cast<const ma_uint4*>(kp + second);
    const uint4 v0 = *reinterpret_cast<const ma_uint4*>(vp);
    const uint4 v1 = *reinterpret_cast<const ma_uint4*>(vp + second);
    r.ks = *reinterpret_cast<const ma_u32*>(sec + code_bytes + (kpar - 2 * D) + 4 * (lane & (D / 2 - 1)));
    const uint2 vs = *reinterpret_cast<const ma_uint2*>(sec + 2 * code_bytes + kpar + (vpar - 2 * kPage) + 8 * G);
    if constexpr (ASYM) {
        r.kz = *reinterpret_cast<const ma_u32*>(sec + code_bytes + 4 * (lane & (D / 2 - 1)));
        const uint2 vz = *reinterpret_cast<const ma_uint2*>(sec + 2 * code_bytes + kpar + 8 * G);
        r.vz[0] = vz.x; r.vz[1] = vz.y;
    }
    r.k[0] = k0.x; r.k[1] = k0.y; r.k[2] = k0.z; r.k[3] = k0.w;
    r.k[4] = k1.x; r.k[5] = k1.y; r.k[6] = k1.z; r.k[7] = k1.w;
    r.v[0] = v0.x; r.v[1] = v0.y; r.v[2] = v0.z; r.v[3] = v0.w;
    r.v[4] = v1.x; r.v[5] = v1.y; r.v[6] = v1.z; r.v[7] = v1.w;
    r.vs[0] = vs.x; r.vs[1] = vs.y;
}

// page pair `pair` of the split [pbeg, pend); pairs past the end reload the last pair (their
// data is never used) so that every iteration issues the same loads
template <int D, bool ASYM>
__device__ __forceinline__ void load_pair(const PageSrc& a, int kv, int pbeg, int pend,
                                          int pair, int npairs, int ctx, int lane, PageRaw& x,
                                          PageRaw& y) {
    const int pc = min(pair, npairs - 1);
    const int pa = pbeg + 2 * pc;
    const bool has_b = pa + 1 < pend;
    load_page<D, ASYM>(a, kv, pa, true, ctx, lane, x);
    load_page<D, ASYM>(a, kv, has_b ? pa + 1 : pa, has_b, ctx, lane, y);
}

// Loads of one page whose width is known at compile time: exactly the bytes this lane needs
// (K and V chunks of D*b/32 bytes each, one K-scale dword, one V-scale pair).
template <int D, int BITS, bool ASYM = false>
__device__ __forceinline__ void load_page_t(const uint8_t* base, uint32_t idx, int H, int kv,
                                            bool present, int ntok, int lane, PageRaw& r) {
    constexpr uint32_t kpar = (ASYM ? 4 : 2) * D, vpar = (ASYM ? 4 : 2) * kPage;   // group parameters
    constexpr uint32_t code_bytes = kPage * D * BITS / 8;
    constexpr uint32_t sec_bytes = 2 * code_bytes + kpar + vpar;
    constexpr int ch = D * BITS / 32;              // bytes of one lane chunk: 4, 8, 16 or 32
    const uint8_t* sec = base + ((size_t)idx * H + kv) * sec_bytes;
    const int t = lane & 15, G = lane >> 4;
    const uint8_t* kp = sec + t * (D * BITS / 8) + G * ch;
    const uint8_t* vp = sec + code_bytes + kpar + (G * D + t * (D / 16)) * BITS / 2;
    if constexpr (ch == 4) {
        r.k[0] = *reinterpret_cast<const ma_u32*>(kp);
        r.v[0] = *reinterpret_cast<const ma_u32*>(vp);
    } else if constexpr (ch == 8) {
        const uint2 k0 = *reinterpret_cast<const ma_uint2*>(kp);
        const uint2 v0 = *reinterpret_cast<const ma_uint2*>(vp);
        r.k[0] = k0.x; r.k[1] = k0.y;
        r.v[0] = v0.x; r.v[1] = v0.y;
    } else {
#pragma unroll
        for (int h = 0; h < ch / 16; ++h) {
            const uint4 k0 = *reinterpret_cast<const ma_uint4*>(kp + 16 * h);
            const uint4 v0 = *reinterpret_cast<const ma_uint4*>(vp + 16 * h);
            r.k[4 * h] = k0.x; r.k[4 * h + 1] = k0.y; r.k[4 * h + 2] = k0.z; r.k[4 * h + 3] = k0.w;
            r.v[4 * h] = v0.x; r.v[4 * h + 1] = v0.y; r.v[4 * h + 2] = v0.z; r.v[4 * h + 3] = v0.w;
        }
    }
    r.ks = *reinterpret_cast<const ma_u32*>(sec + code_bytes + (kpar - 2 * D) + 4 * (lane & (D / 2 - 1)));
    const uint2 vs = *reinterpret_cast<const ma_uint2*>(sec + 2 * code_bytes + kpar + (vpar - 2 * kPage) + 8 * G);
    r.vs[0] = vs.x; r.vs[1] = vs.y;
    if constexpr (ASYM) {
        r.kz = *reinterpret_cast<const ma_u32*>(sec + code_bytes + 4 * (lane & (D / 2 - 1)));
        const uint2 vz = *reinterpret_cast<const ma_uint2*>(sec + 2 * code_bytes + kpar + 8 * G);
        r.vz[0] = vz.x; r.vz[1] = vz.y;
    }
    r.bits = present ? BITS : 0;
    r.ntok = ntok;
}

__device__ __forceinline__ uint32_t hsub(uint32_t u, float bias) {
    const half2v b = {(_Float16)bias, (_Float16)bias};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, u) - b);
}

// K chunk (D*b/32 bytes) -> D/8 dwords of fp16 pairs holding the signed codes, in code order.
// Bytes of a masked word are spread into fp16 pairs 0x64uu (= 1024 + u) by v_perm_b32, then the
// offset 1024 + 2^(b-1) is subtracted exactly (ASYM: 1024, leaving the unsigned code u).
template <int D, bool ASYM = false>
__device__ __forceinline__ void unpack_k(const uint32_t* w, int bits, uint32_t* out) {
    const uint32_t hi = 0x64646464u;
    if (bits == 2) {
#pragma unroll
        for (int i = 0; i < D / 64; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {   // codes 2j, 2j+1 (bytes 0, 2) and 2j+8, 2j+9 (1, 3)
                const uint32_t m = (w[i] >> (2 * j)) & 0x03030303u;
                out[i * 8 + j] = hsub(__builtin_amdgcn_perm(hi, m, 0x04020400u), ASYM ? 1024.0f : 1026.0f);
                out[i * 8 + 4 + j] = hsub(__builtin_amdgcn_perm(hi, m, 0x04030401u), ASYM ? 1024.0f : 1026.0f);
            }
    } else if (bits == 4) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {   // codes 2j, 2j+1 (bytes 0, 2) and 2j+4, 2j+5 (1, 3)
                const uint32_t m = (w[i] >> (4 * j)) & 0x0F0F0F0Fu;
                out[i * 4 + j] = hsub(__builtin_amdgcn_perm(hi, m, 0x04020400u), ASYM ? 1024.0f : 1032.0f);
                out[i * 4 + 2 + j] = hsub(__builtin_amdgcn_perm(hi, m, 0x04030401u), ASYM ? 1024.0f : 1032.0f);
            }
    } else {
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
            out[2 * i] = hsub(__builtin_amdgcn_perm(hi, w[i], 0x04020400u), ASYM ? 1024.0f : 1152.0f);
            out[2 * i + 1] = hsub(__builtin_amdgcn_perm(hi, w[i], 0x04030401u), ASYM ? 1024.0f : 1152.0f);
        }
    }
}

__device__ __forceinline__ half8 make_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    uint4 u = {a, b, c, d};
    return __builtin_bit_cast(half8, u);
}

// max / sum over the four lanes of a head (lanes h, h+16, h+32, h+48)
__device__ __forceinline__ float rows_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float rows_sum(float x) {
    x += __shfl_xor(x, 16, 64);
    return x + __shfl_xor(x, 32, 64);
}

template <int D>
struct WaveState {
    float4v o[D / 16];   // o^T tile per channel chunk: lane (h, G) element r -> channel G*D/4 + r*D/16 + k
    float m;             // running max (log2 units) of head lane%16
    float l;             // this lane's share of the running sum of p
    float z;             // asymmetric format: this lane's share of the sum of p * (V zero point)
};

// the D/4 K parameters (scales or zero points) of this lane's channel quarter, staged in LDS
// one dword a lane (lane i: channels 2i, 2i+1)
template <int D>
__device__ __forceinline__ void read_quarter(const uint32_t* lds, int G, uint32_t* out) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        const uint4 v = *reinterpret_cast<const ma_uint4*>(lds + G * (D / 8) + 4 * i);
        out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
    }
}

// asymmetric format: the zero-point part of the logits, sum_c z_c q_c for every token row of the
// tile (the zero points stand in every row of the A operand; fp16 times fp16 is exact in fp32)
template <int D>
__device__ __forceinline__ float4v zero_point_logits(const uint32_t* kz, const uint32_t* qf) {
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            make_half8(kz[4 * i], kz[4 * i + 1], kz[4 * i + 2], kz[4 * i + 3]),
            make_half8(qf[4 * i], qf[4 * i + 1], qf[4 * i + 2], qf[4 * i + 3]), acc, 0, 0, 0);
    return acc;
}

// asymmetric format: p_i * (V zero point of token 4G+i) summed over this lane's four tokens
__device__ __forceinline__ float zero_point_mass(const float* p, uint32_t vz0, uint32_t vz1, int ntok, int G) {
    const half2v z01 = __builtin_bit_cast(half2v, vz0);
    const half2v z23 = __builtin_bit_cast(half2v, vz1);
    const float z[4] = {(float)z01[0], (float)z01[1], (float)z23[0], (float)z23[1]};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (4 * G + i < ntok) acc += p[i] * z[i];
    return acc;
}

// QK for one page: S^T for tokens 4G..4G+3 of head lane%16, in log2 units, masked. ASYM: the
// logit of an element m + u*s is the zero-point part plus the code part.
template <int D, bool ASYM = false>
__device__ __forceinline__ float4v page_logits(const PageRaw& r, int bits, const uint32_t* qf,
                                               uint32_t* lds_ks, int lane, float scale_log2) {
    const int G = lane >> 4;
    // stage the page's K scales through LDS: each lane needs the D/4 scales of its lane group
    // (one wave writes and reads its own slot; LDS serves a wave's requests in order, and the
    // wave barrier keeps the compiler from hoisting the reads above the write)
    lds_ks[lane] = r.ks;
    if constexpr (ASYM) lds_ks[128 + lane] = r.kz;
    __builtin_amdgcn_wave_barrier();
    uint32_t ks[D / 8];
    read_quarter<D>(lds_ks, G, ks);
    uint32_t kf[D / 8];
    unpack_k<D, ASYM>(r.k, bits, kf);
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (ASYM) {
        uint32_t kz[D / 8];
        read_quarter<D>(lds_ks + 128, G, kz);
        acc = zero_point_logits<D>(kz, qf);
    }
    if (!ASYM && bits == 2) {
        // INT2 codes are -1, 0, 1: code * scale is exact in fp16, so the scales fold into the
        // keys and every MFMA product is exact
#pragma unroll
        for (int i = 0; i < D / 8; ++i)
            kf[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, kf[i]) *
                                                     __builtin_bit_cast(half2v, ks[i]));
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                make_half8(kf[4 * i], kf[4 * i + 1], kf[4 * i + 2], kf[4 * i + 3]),
                make_half8(qf[4 * i], qf[4 * i + 1], qf[4 * i + 2], qf[4 * i + 3]), acc, 0, 0, 0);
    } else {
        // q * scale as two fp16 parts, hi = round(q * s) and the residual lo = q * s - hi
        // (one fused multiply-add, exact while lo is representable): a single rounded fp16
        // product would perturb the logits by ~2^-11 of |q . K|
        uint32_t qh[D / 8], ql[D / 8];
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            const half2v q2 = __builtin_bit_cast(half2v, qf[i]);
            const half2v s2 = __builtin_bit_cast(half2v, ks[i]);
            const half2v hi = q2 * s2;
            qh[i] = __builtin_bit_cast(uint32_t, hi);
            ql[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q2, s2, -hi));
        }
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const half8 kk = make_half8(kf[4 * i], kf[4 * i + 1], kf[4 * i + 2], kf[4 * i + 3]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                kk, make_half8(qh[4 * i], qh[4 * i + 1], qh[4 * i + 2], qh[4 * i + 3]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                kk, make_half8(ql[4 * i], ql[4 * i + 1], ql[4 * i + 2], ql[4 * i + 3]), acc, 0, 0, 0);
        }
    }
    float4v lg = acc * scale_log2;
    if (r.ntok < kPage) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * G + i >= r.ntok) lg[i] = -INFINITY;
    }
    return lg;
}

// softmax weights of one page times the V scales: the fp32 product p * s split into fp16 parts
// hi = round(p * s) and lo = round(p * s - hi), as pairs for this lane's four tokens; masked
// tokens get exactly 0 (their scale slot may hold anything)
__device__ __forceinline__ void page_weights(uint32_t vs0, uint32_t vs1, int ntok, const float* p,
                                             int G, uint32_t* wh, uint32_t* wl) {
    const half2v s01 = __builtin_bit_cast(half2v, vs0);
    const half2v s23 = __builtin_bit_cast(half2v, vs1);
    float ps[4] = {p[0] * (float)s01[0], p[1] * (float)s01[1], p[2] * (float)s23[0], p[3] * (float)s23[1]};
    if (ntok < kPage) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * G + i >= ntok) ps[i] = 0.f;
    }
    const half2v h01 = {(_Float16)ps[0], (_Float16)ps[1]};
    const half2v h23 = {(_Float16)ps[2], (_Float16)ps[3]};
    const half2v l01 = {(_Float16)(ps[0] - (float)h01[0]), (_Float16)(ps[1] - (float)h01[1])};
    const half2v l23 = {(_Float16)(ps[2] - (float)h23[0]), (_Float16)(ps[3] - (float)h23[1])};
    wh[0] = __builtin_bit_cast(uint32_t, h01);
    wh[1] = __builtin_bit_cast(uint32_t, h23);
    wl[0] = __builtin_bit_cast(uint32_t, l01);
    wl[1] = __builtin_bit_cast(uint32_t, l23);
}

// One page pair: QK, online softmax and PV. BITS is the width of both pages when the caller
// knows it at compile time, 0 when each page carries its own; page B may be absent (bits 0).
template <int D, int BITS, bool ASYM = false>
__device__ __forceinline__ void process_pair(const PageRaw& A, const PageRaw& B, const uint32_t* qf,
                                             uint32_t* lds_ks, int lane, float scale_log2,
                                             WaveState<D>& st) {
    const int G = lane >> 4;
    const int bits_a = BITS ? BITS : A.bits;
    const int bits_b = BITS ? BITS : B.bits;
    const float4v la = page_logits<D, ASYM>(A, bits_a, qf, lds_ks, lane, scale_log2);
    float4v lb = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (B.bits) lb = page_logits<D, ASYM>(B, bits_b, qf, lds_ks + 64, lane, scale_log2);

    // online softmax over the pair's 32 tokens, per head (lanes h, h+16, h+32, h+48)
    float mx = fmaxf(fmaxf(fmaxf(la[0], la[1]), fmaxf(la[2], la[3])),
                     fmaxf(fmaxf(lb[0], lb[1]), fmaxf(lb[2], lb[3])));
    mx = rows_max(mx);
    const float m_new = fmaxf(st.m, mx);            // finite: page A holds >= 1 valid token
    if (__builtin_amdgcn_ballot_w64(m_new != st.m)) {
        const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);   // 0 on the first pair
        st.l *= alpha;
        if constexpr (ASYM) st.z *= alpha;
#pragma unroll
        for (int k = 0; k < D / 16; ++k) st.o[k] *= alpha;
        st.m = m_new;
    }
    float pa[4], pb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pa[i] = __builtin_amdgcn_exp2f(la[i] - m_new);
        pb[i] = __builtin_amdgcn_exp2f(lb[i] - m_new);
    }
    st.l += ((pa[0] + pa[1]) + (pa[2] + pa[3])) + ((pb[0] + pb[1]) + (pb[2] + pb[3]));
    if constexpr (ASYM) {
        st.z += zero_point_mass(pa, A.vz[0], A.vz[1], A.ntok, G);
        if (B.bits) st.z += zero_point_mass(pb, B.vz[0], B.vz[1], B.ntok, G);
    }

    uint32_t wh[4], wl[4];
    page_weights(A.vs[0], A.vs[1], A.ntok, pa, G, wh, wl);
    if (B.bits) {
        page_weights(B.vs[0], B.vs[1], B.ntok, pb, G, wh + 2, wl + 2);
    } else {
        wh[2] = wh[3] = wl[2] = wl[3] = 0u;
    }
    const half8 ph = make_half8(wh[0], wh[1], wh[2], wh[3]);
    const half8 pl = make_half8(wl[0], wl[1], wl[2], wl[3]);

    uint32_t va[D / 8], vb[D / 8];
    unpack_k<D, ASYM>(A.v, bits_a, va);
    if (B.bits) {
        unpack_k<D, ASYM>(B.v, bits_b, vb);
    } else {
#pragma unroll
        for (int i = 0; i < D / 8; ++i) vb[i] = 0u;
    }
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
        const half8 vv = make_half8(va[2 * k], va[2 * k + 1], vb[2 * k], vb[2 * k + 1]);
        st.o[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vv, ph, st.o[k], 0, 0, 0);
        st.o[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vv, pl, st.o[k], 0, 0, 0);
    }
}

// Page pair q of a wave's chunk [cb, cb + npg) whose handles sit in `hv` (lane i: page cb + i),
// all of width BITS. Pairs past the end reload the last pair (their data is never used).
// The same pair for groups of at most 8 query heads. The 16 head columns of the MFMA tiles hold
// both pages: lanes with h = lane % 16 < 8 carry page A for head h, lanes h >= 8 page B for head
// h - 8. The scaled query q * Kscale is then computed once for both pages (each lane with its
// own page's scales), each lane keeps four logits and four weights instead of eight, and the PV
// product accumulates page B's share in columns 8..15, folded into 0..7 at the end.
template <int D, int BITS, bool ASYM = false>
__device__ __forceinline__ void process_pair_half(const PageRaw& A, const PageRaw& B,
                                                  const uint32_t* qf, uint32_t* lds_ks, int lane,
                                                  float scale_log2, WaveState<D>& st) {
    const int G = lane >> 4;
    const bool side = (lane & 8) != 0;
    const int bits_a = BITS ? BITS : A.bits;
    const int bits_b = BITS ? BITS : B.bits;
    const bool has_b = B.bits != 0;
    const int ntok = side ? B.ntok : A.ntok;
    lds_ks[lane] = A.ks;
    lds_ks[64 + lane] = B.ks;
    if constexpr (ASYM) {
        lds_ks[128 + lane] = A.kz;
        lds_ks[192 + lane] = B.kz;
    }
    __builtin_amdgcn_wave_barrier();
    float4v acc;
    if (!ASYM && bits_a == 2 && bits_b == 2) {
        // INT2: the scales fold exactly into each page's keys, q is used as is
        uint32_t ksa[D / 8], ksb[D / 8];
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const uint4 va = *reinterpret_cast<const ma_uint4*>(lds_ks + G * (D / 8) + 4 * i);
            const uint4 vb = *reinterpret_cast<const ma_uint4*>(lds_ks + 64 + G * (D / 8) + 4 * i);
            ksa[4 * i] = va.x; ksa[4 * i + 1] = va.y; ksa[4 * i + 2] = va.z; ksa[4 * i + 3] = va.w;
            ksb[4 * i] = vb.x; ksb[4 * i + 1] = vb.y; ksb[4 * i + 2] = vb.z; ksb[4 * i + 3] = vb.w;
        }
        uint32_t kfa[D / 8], kfb[D / 8];
        unpack_k<D>(A.k, 2, kfa);
        unpack_k<D>(B.k, 2, kfb);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            kfa[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, kfa[i]) *
                                                      __builtin_bit_cast(half2v, ksa[i]));
            kfb[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, kfb[i]) *
                                                      __builtin_bit_cast(half2v, ksb[i]));
        }
        float4v acca = {0.f, 0.f, 0.f, 0.f}, accb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const half8 qq = make_half8(qf[4 * i], qf[4 * i + 1], qf[4 * i + 2], qf[4 * i + 3]);
            acca = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                make_half8(kfa[4 * i], kfa[4 * i + 1], kfa[4 * i + 2], kfa[4 * i + 3]), qq, acca, 0, 0, 0);
            if (has_b)
                accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    make_half8(kfb[4 * i], kfb[4 * i + 1], kfb[4 * i + 2], kfb[4 * i + 3]), qq, accb, 0, 0, 0);
        }
        acc = side ? accb : acca;
    } else {
        // q * Kscale of this lane's page as fp16 hi + lo; the two pages' keys against it
        uint32_t ks[D / 8];
        const uint32_t* src = lds_ks + (side ? 64 : 0) + G * (D / 8);
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const uint4 v = *reinterpret_cast<const ma_uint4*>(src + 4 * i);
            ks[4 * i] = v.x; ks[4 * i + 1] = v.y; ks[4 * i + 2] = v.z; ks[4 * i + 3] = v.w;
        }
        uint32_t qh[D / 8], ql[D / 8];
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            const half2v q2 = __builtin_bit_cast(half2v, qf[i]);
            const half2v s2 = __builtin_bit_cast(half2v, ks[i]);
            const half2v hi = q2 * s2;
            qh[i] = __builtin_bit_cast(uint32_t, hi);
            ql[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q2, s2, -hi));
        }
        uint32_t kfa[D / 8], kfb[D / 8];
        unpack_k<D, ASYM>(A.k, bits_a, kfa);
        if (has_b) unpack_k<D, ASYM>(B.k, bits_b, kfb);
        float4v acca = {0.f, 0.f, 0.f, 0.f}, accb = {0.f, 0.f, 0.f, 0.f};
        if constexpr (ASYM) {                     // the zero-point parts, page by page
            uint32_t kz[D / 8];
            read_quarter<D>(lds_ks + 128, G, kz);
            acca = zero_point_logits<D>(kz, qf);
            if (has_b) {
                read_quarter<D>(lds_ks + 192, G, kz);
                accb = zero_point_logits<D>(kz, qf);
            }
        }
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const half8 hq = make_half8(qh[4 * i], qh[4 * i + 1], qh[4 * i + 2], qh[4 * i + 3]);
            const half8 lq = make_half8(ql[4 * i], ql[4 * i + 1], ql[4 * i + 2], ql[4 * i + 3]);
            const half8 ka = make_half8(kfa[4 * i], kfa[4 * i + 1], kfa[4 * i + 2], kfa[4 * i + 3]);
            acca = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, hq, acca, 0, 0, 0);
            acca = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, lq, acca, 0, 0, 0);
            if (has_b) {
                const half8 kb = make_half8(kfb[4 * i], kfb[4 * i + 1], kfb[4 * i + 2], kfb[4 * i + 3]);
                accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, hq, accb, 0, 0, 0);
                accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, lq, accb, 0, 0, 0);
            }
        }
        acc = side ? accb : acca;
    }
    float4v lg = acc * scale_log2;
    if (ntok < kPage) {                                  // includes an absent page B (ntok 0)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * G + i >= ntok) lg[i] = -INFINITY;
    }

    // online softmax over the pair's 32 tokens: a head's lanes are h, h+8 and the four rows
    float mx = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
    mx = rows_max(mx);
    const float m_new = fmaxf(st.m, mx);            // finite: page A holds >= 1 valid token
    if (__builtin_amdgcn_ballot_w64(m_new != st.m)) {
        const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);   // 0 on the first pair
        st.l *= alpha;
        if constexpr (ASYM) st.z *= alpha;
#pragma unroll
        for (int k = 0; k < D / 16; ++k) st.o[k] *= alpha;
        st.m = m_new;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(lg[i] - m_new);
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
    if constexpr (ASYM)
        st.z += zero_point_mass(p, side ? B.vz[0] : A.vz[0], side ? B.vz[1] : A.vz[1], ntok, G);

    uint32_t wh[2], wl[2];
    page_weights(side ? B.vs[0] : A.vs[0], side ? B.vs[1] : A.vs[1], ntok, p, G, wh, wl);
    const uint32_t z = 0u;
    const half8 ph = make_half8(side ? z : wh[0], side ? z : wh[1], side ? wh[0] : z, side ? wh[1] : z);
    const half8 pl = make_half8(side ? z : wl[0], side ? z : wl[1], side ? wl[0] : z, side ? wl[1] : z);

    uint32_t va[D / 8], vb[D / 8];
    unpack_k<D, ASYM>(A.v, bits_a, va);
    if (has_b) {
        unpack_k<D, ASYM>(B.v, bits_b, vb);
    } else {
#pragma unroll
        for (int i = 0; i < D / 8; ++i) vb[i] = 0u;
    }
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
        const half8 vv = make_half8(va[2 * k], va[2 * k + 1], vb[2 * k], vb[2 * k + 1]);
        st.o[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vv, ph, st.o[k], 0, 0, 0);
        st.o[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vv, pl, st.o[k], 0, 0, 0);
    }
}

// one pair through the layout the kernel was instantiated for
template <int D, int BITS, bool HALF, bool ASYM = false>
__device__ __forceinline__ void run_pair(const PageRaw& A, const PageRaw& B, const uint32_t* qf,
                                         uint32_t* lds_ks, int lane, float scale_log2,
                                         WaveState<D>& st) {
    if constexpr (HALF)
        process_pair_half<D, BITS, ASYM>(A, B, qf, lds_ks, lane, scale_log2, st);
    else
        process_pair<D, BITS, ASYM>(A, B, qf, lds_ks, lane, scale_log2, st);
}


// ---------------------------------------------------------------- FP16 tier
// One FP16 page as this lane needs it: K of token lane%16 for channels [G*D/4, +D/4) (the order
// of the query fragment) and V of token quad G for channels [(lane%16)*D/16, +D/16), four tokens
// a channel -- the operand layouts of the INT paths, with fp16 values in place of codes.
template <int D>
struct PageF16 {
    uint32_t k[D / 8];
    uint32_t v[D / 8];
};

template <int D>
__device__ __forceinline__ void load_page_f16(const uint8_t* sec, int lane, PageF16<D>& r) {
    const int t = lane & 15, G = lane >> 4;
    const ma_uint4* kp = reinterpret_cast<const ma_uint4*>(sec + t * 2 * D + G * (D / 2));
    const ma_uint4* vp = reinterpret_cast<const ma_uint4*>(sec + 2 * kPage * D + (G * D + t * (D / 16)) * 8);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        const uint4 kk = kp[i], vv = vp[i];
        r.k[4 * i] = kk.x; r.k[4 * i + 1] = kk.y; r.k[4 * i + 2] = kk.z; r.k[4 * i + 3] = kk.w;
        r.v[4 * i] = vv.x; r.v[4 * i + 1] = vv.y; r.v[4 * i + 2] = vv.z; r.v[4 * i + 3] = vv.w;
    }
}

// A pair of FP16 pages (B may be absent): the same QK, online softmax and PV as the INT pairs,
// with the keys and values used as they are (each MFMA product of two fp16 values is exact in
// fp32) and the softmax weights split into fp16 hi + lo.
template <int D, bool HALF>
__device__ __forceinline__ void process_pair_f16(const PageF16<D>& A, const PageF16<D>& B,
                                                 bool has_b, int ntok_a, int ntok_b,
                                                 const uint32_t* qf, int lane, float scale_log2,
                                                 WaveState<D>& st) {
    const int G = lane >> 4;
    float4v acca = {0.f, 0.f, 0.f, 0.f}, accb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        const half8 qq = make_half8(qf[4 * i], qf[4 * i + 1], qf[4 * i + 2], qf[4 * i + 3]);
        acca = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            make_half8(A.k[4 * i], A.k[4 * i + 1], A.k[4 * i + 2], A.k[4 * i + 3]), qq, acca, 0, 0, 0);
        if (has_b)
            accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                make_half8(B.k[4 * i], B.k[4 * i + 1], B.k[4 * i + 2], B.k[4 * i + 3]), qq, accb, 0, 0, 0);
    }
    const uint32_t one = 0x3C003C00u;                   // unit "V scales": weights are p itself
    uint32_t wh[4], wl[4];
    if constexpr (HALF) {
        const bool side = (lane & 8) != 0;
        const int ntok = side ? (has_b ? ntok_b : 0) : ntok_a;
        float4v lg = (side ? accb : acca) * scale_log2;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * G + i >= ntok) lg[i] = -INFINITY;
        float mx = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
        mx = rows_max(mx);
        const float m_new = fmaxf(st.m, mx);            // finite: page A holds >= 1 valid token
        if (__builtin_amdgcn_ballot_w64(m_new != st.m)) {
            const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
            st.l *= alpha;
#pragma unroll
            for (int k = 0; k < D / 16; ++k) st.o[k] *= alpha;
            st.m = m_new;
        }
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(lg[i] - m_new);
        st.l += (p[0] + p[1]) + (p[2] + p[3]);
        uint32_t h2[2], l2[2];
        page_weights(one, one, ntok, p, G, h2, l2);
        const uint32_t z = 0u;
        wh[0] = side ? z : h2[0]; wh[1] = side ? z : h2[1]; wh[2] = side ? h2[0] : z; wh[3] = side ? h2[1] : z;
        wl[0] = side ? z : l2[0]; wl[1] = side ? z : l2[1]; wl[2] = side ? l2[0] : z; wl[3] = side ? l2[1] : z;
    } else {
        float4v la = acca * scale_log2;
        float4v lb = accb * scale_log2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (4 * G + i >= ntok_a) la[i] = -INFINITY;
            if (!has_b || 4 * G + i >= ntok_b) lb[i] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(la[0], la[1]), fmaxf(la[2], la[3])),
                         fmaxf(fmaxf(lb[0], lb[1]), fmaxf(lb[2], lb[3])));
        mx = rows_max(mx);
        const float m_new = fmaxf(st.m, mx);
        if (__builtin_amdgcn_ballot_w64(m_new != st.m)) {
            const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
            st.l *= alpha;
#pragma unroll
            for (int k = 0; k < D / 16; ++k) st.o[k] *= alpha;
            st.m = m_new;
        }
        float pa[4], pb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pa[i] = __builtin_amdgcn_exp2f(la[i] - m_new);
            pb[i] = __builtin_amdgcn_exp2f(lb[i] - m_new);
        }
        st.l += ((pa[0] + pa[1]) + (pa[2] + pa[3])) + ((pb[0] + pb[1]) + (pb[2] + pb[3]));
        page_weights(one, one, ntok_a, pa, G, wh, wl);
        page_weights(one, one, has_b ? ntok_b : 0, pb, G, wh + 2, wl + 2);
    }
    const half8 ph = make_half8(wh[0], wh[1], wh[2], wh[3]);
    const half8 pl = make_half8(wl[0], wl[1], wl[2], wl[3]);
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
        const uint32_t vb0 = has_b ? B.v[2 * k] : 0u, vb1 = has_b ? B.v[2 * k + 1] : 0u;
        const half8 vv = make_half8(A.v[2 * k], A.v[2 * k + 1], vb0, vb1);
        st.o[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vv, ph, st.o[k], 0, 0, 0);
        st.o[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vv, pl, st.o[k], 0, 0, 0);
    }
}

// A wave's chunk of FP16 pages, handles in `hv` (lane i: page cb + i). Pairs are loaded and
// used in turn.
template <int D, bool HALF>
__device__ __forceinline__ void wave_chunk_f16(const uint8_t* base, uint32_t hv, int H, int kv,
                                               int cb, int npg, int ctx, int lane,
                                               const uint32_t* qf, float scale_log2,
                                               WaveState<D>& st) {
    constexpr uint32_t sec_bytes = 4u * kPage * D;
    const int nq = (npg + 1) / 2;
    for (int q = 0; q < nq; ++q) {
        const int pa = 2 * q;
        const bool has_b = pa + 1 < npg;
        const uint32_t ia = (uint32_t)__builtin_amdgcn_readlane((int)hv, pa) & 0x3fffffffu;
        const uint32_t ib =
            (uint32_t)__builtin_amdgcn_readlane((int)hv, has_b ? pa + 1 : pa) & 0x3fffffffu;
        PageF16<D> A, B;
        load_page_f16<D>(base + ((size_t)ia * H + kv) * sec_bytes, lane, A);
        load_page_f16<D>(base + ((size_t)ib * H + kv) * sec_bytes, lane, B);
        const int page = cb + pa;
        process_pair_f16<D, HALF>(A, B, has_b, min(kPage, ctx - page * kPage),
                                         has_b ? min(kPage, ctx - (page + 1) * kPage) : 0, qf,
                                         lane, scale_log2, st);
    }
}

// one pair of the general loop: pairs with an FP16 page go page by page, each FP16 page read
// here from its section (its PageRaw holds only its width and token count)
template <int D, bool HALF, bool ASYM>
__device__ __forceinline__ void run_pair_any(const PageSrc& src, int kv, int page, const PageRaw& A,
                                             const PageRaw& B, const uint32_t* qf,
                                             uint32_t* lds_ks, int lane, float scale_log2,
                                             WaveState<D>& st) {
    if (A.bits != 16 && B.bits != 16) {
        run_pair<D, 0, HALF, ASYM>(A, B, qf, lds_ks, lane, scale_log2, st);
        return;
    }
    PageRaw none = A;
    none.bits = 0;
    none.ntok = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const PageRaw& X = j == 0 ? A : B;
        if (X.bits == 16) {
            const uint32_t handle = ((const_u32_ptr)src.bt_row)[page + j];
            const uint8_t* sec = src.base3 + ((size_t)(handle & 0x3fffffffu) * src.H + kv) * (4u * kPage * D);
            PageF16<D> F;
            load_page_f16<D>(sec, lane, F);
            process_pair_f16<D, HALF>(F, F, false, X.ntok, 0, qf, lane, scale_log2, st);
        } else if (X.bits) {
            run_pair<D, 0, HALF, ASYM>(X, none, qf, lds_ks, lane, scale_log2, st);
        }
    }
}

template <int D, int BITS, bool ASYM>
__device__ __forceinline__ void load_pair_t(const uint8_t* base, uint32_t hv, int H, int kv, int cb,
                                            int npg, int q, int nq, int ctx, int lane, PageRaw& x,
                                            PageRaw& y) {
    const int pa = 2 * min(q, nq - 1);
    const bool has_b = pa + 1 < npg;
    const uint32_t ia = (uint32_t)__builtin_amdgcn_readlane((int)hv, pa) & 0x3fffffffu;
    const uint32_t ib = (uint32_t)__builtin_amdgcn_readlane((int)hv, has_b ? pa + 1 : pa) & 0x3fffffffu;
    const int page = cb + pa;
    load_page_t<D, BITS, ASYM>(base, ia, H, kv, true, min(kPage, ctx - page * kPage), lane, x);
    load_page_t<D, BITS, ASYM>(base, ib, H, kv, has_b, has_b ? min(kPage, ctx - (page + 1) * kPage) : 0,
                               lane, y);
}

// A wave's chunk of pages, all of one width, with DEPTH page pairs in flight: while pair q is
// processed, pairs q+1 .. q+DEPTH-1 are loading. The rotation over the DEPTH buffers is unrolled,
// so every buffer index is a constant. No per-page branching and no block-table reads in the loop.
template <int D, int BITS, int DEPTH, bool HALF, bool ASYM = false>
__device__ __forceinline__ void wave_chunk_uniform(const uint8_t* base, uint32_t hv, int H, int kv,
                                                   int cb, int npg, int ctx, int lane,
                                                   const uint32_t* qf, uint32_t* ks_slot,
                                                   float scale_log2, WaveState<D>& st) {
    const int nq = (npg + 1) / 2;
    PageRaw buf[DEPTH][2];
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
        load_pair_t<D, BITS, ASYM>(base, hv, H, kv, cb, npg, d, nq, ctx, lane, buf[d][0], buf[d][1]);
    // whole rotations in a loop with one exit and unconditional loads (see wave_chunk_fast),
    // then the last nq % DEPTH pairs, already loaded
    const int nfull = nq / DEPTH;
    for (int r = 0; r < nfull * DEPTH; r += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int nxt = (d + DEPTH - 1) % DEPTH;
            load_pair_t<D, BITS, ASYM>(base, hv, H, kv, cb, npg, r + d + DEPTH - 1, nq, ctx, lane,
                                       buf[nxt][0], buf[nxt][1]);
            run_pair<D, BITS, HALF, ASYM>(buf[d][0], buf[d][1], qf, ks_slot, lane, scale_log2, st);
        }
    }
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
        if (d < nq - nfull * DEPTH)
            run_pair<D, BITS, HALF, ASYM>(buf[d][0], buf[d][1], qf, ks_slot, lane, scale_log2, st);
}

// The same for a chunk whose pages may differ in width: handles from the block table, the
// width-independent loads of load_page and per-page width branches.
template <int D, bool HALF, bool ASYM = false>
__device__ __forceinline__ void wave_chunk_mixed(const PageSrc& src, int kv, int cb, int npg,
                                                 int ctx, int lane, const uint32_t* qf,
                                                 uint32_t* ks_slot, float scale_log2,
                                                 WaveState<D>& st) {
    const int nq = (npg + 1) / 2;
    PageRaw a0, a1, b0, b1;
    load_pair<D, ASYM>(src, kv, cb, cb + npg, 0, nq, ctx, lane, a0, a1);
    // two pairs per trip, one exit, unconditional loads (see wave_chunk_fast); an odd last
    // pair is already in a0, a1
    for (int q = 0; q + 1 < nq; q += 2) {
        load_pair<D, ASYM>(src, kv, cb, cb + npg, q + 1, nq, ctx, lane, b0, b1);
        run_pair_any<D, HALF, ASYM>(src, kv, cb + 2 * q, a0, a1, qf, ks_slot, lane, scale_log2, st);
        load_pair<D, ASYM>(src, kv, cb, cb + npg, q + 2, nq, ctx, lane, a0, a1);
        run_pair_any<D, HALF, ASYM>(src, kv, cb + 2 * (q + 1), b0, b1, qf, ks_slot, lane, scale_log2, st);
    }
    if (nq & 1)
        run_pair_any<D, HALF, ASYM>(src, kv, cb + 2 * (nq - 1), a0, a1, qf, ks_slot, lane, scale_log2, st);
}

// ---------------------------------------------------------------- uniform-width fast path
// A wave's chunk of pages of one width, for groups of at most 8 query heads, a page pair per
// round. The loads of the next DEPTH-1 pairs are in flight while a pair is computed; inside a
// round the QK products come first, then the update of the running maxima, then the PV
// products. As in process_pair_half, lanes with h = lane % 16 < 8 own page A of a pair for head h,
// lanes h >= 8 page B for head h - 8. The PV product instead puts the two fp16 parts of the
// weights in the two column halves -- columns 0..7 the high parts of heads 0..7 over both
// pages' tokens, columns 8..15 the low parts -- so one MFMA per channel chunk covers a pair;
// the halves fold at the end exactly as the page halves of process_pair_half do.
//
// The running maximum is lazy: the reference m is raised only when a logit exceeds it, and then
// to kLazy (log2 units) above the largest logit seen, so every weight is at most 1 and the
// accumulators are rescaled only when a logit exceeds m -- in practice about once per chunk.
constexpr float kLazy = 3.0f;
#ifndef KVQ_DEPTH2
#define KVQ_DEPTH2 2
#endif
#ifndef KVQ_DEPTH4
#define KVQ_DEPTH4 2
#endif
#ifndef KVQ_DEPTH8
#define KVQ_DEPTH8 2
#endif
constexpr int kDepth2 = KVQ_DEPTH2;     // page pairs in flight per wave, by width
constexpr int kDepth4 = KVQ_DEPTH4;
constexpr int kDepth8 = KVQ_DEPTH8;

template <int D, int BITS>
struct FastPair {
    static constexpr int KW = D * BITS / 128;    // dwords of this lane's K chunk and V chunk
    uint32_t ka[KW], kb[KW], va[KW], vb[KW];
    uint32_t ksa, ksb;                           // K-scale dwords (channels 2*lane, 2*lane+1)
    u32x2 vsa, vsb;                              // V scales, quad G of pages A and B
    uint32_t kza, kzb;                           // asymmetric format: K zero points, as ksa, ksb
    u32x2 vza, vzb;                              // asymmetric format: V zero points, as vsa, vsb
    int ntok_a, ntok_b;                          // valid tokens; 0 for an absent page
};

template <int KW>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t* w) {
    if constexpr (KW == 1) {
        w[0] = *reinterpret_cast<const ma_u32*>(p);
    } else if constexpr (KW == 2) {
        const uint2 x = *reinterpret_cast<const ma_uint2*>(p);
        w[0] = x.x; w[1] = x.y;
    } else {
#pragma unroll
        for (int h = 0; h < KW / 4; ++h) {
            const uint4 x = *reinterpret_cast<const ma_uint4*>(p + 16 * h);
            w[4 * h] = x.x; w[4 * h + 1] = x.y; w[4 * h + 2] = x.z; w[4 * h + 3] = x.w;
        }
    }
}

// this lane's byte offsets inside a section
struct LaneOffsets {
    uint32_t k, v, ks, vs, kz, vz;
};

template <int D, int BITS, bool ASYM>
__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
    constexpr uint32_t kpar = (ASYM ? 4 : 2) * D, vpar = (ASYM ? 4 : 2) * kPage;   // group parameters
    constexpr uint32_t code_bytes = kPage * D * BITS / 8;
    const int t = lane & 15, G = lane >> 4;
    LaneOffsets o;
    o.k = t * (D * BITS / 8) + G * (D * BITS / 32);
    o.v = code_bytes + kpar + (G * D + t * (D / 16)) * BITS / 2;
    o.kz = code_bytes + 4 * (lane & (D / 2 - 1));
    o.ks = o.kz + (kpar - 2 * D);
    o.vz = 2 * code_bytes + kpar + 8 * G;
    o.vs = o.vz + (vpar - 2 * kPage);
    return o;
}

template <int KW>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* w) {
    if constexpr (KW == 1) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    } else if constexpr (KW == 2) {
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        w[0] = x[0]; w[1] = x[1];
    } else {
#pragma unroll
        for (int h = 0; h < KW / 4; ++h) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * h, 0, 0);
            w[4 * h] = x[0]; w[4 * h + 1] = x[1]; w[4 * h + 2] = x[2]; w[4 * h + 3] = x[3];
        }
    }
}

// pair q of a chunk whose handles sit in hv (lane i: page cb + i); pairs past the end reload
// the last pair and carry no tokens. Each page section is read through a buffer resource
// built in scalar registers, so the lane offsets stay fixed VGPR offsets and no per-load
// address arithmetic runs on the vector unit.
template <int D, int BITS, bool ASYM>
__device__ __forceinline__ void load_pair_fast(const uint8_t* base, uint32_t hv, int H, int kv,
                                               int cb, int npg, int q, int nq, int ctx,
                                               const LaneOffsets& lo, bool side,
                                               FastPair<D, BITS>& P) {
    constexpr uint32_t sec_bytes = 2 * (kPage * D * BITS / 8) + (ASYM ? 2 : 1) * (2 * D + 2 * kPage);
    constexpr int KW = FastPair<D, BITS>::KW;
    const bool real = q < nq;
    const int pa = 2 * min(q, nq - 1);
    const bool has_b = pa + 1 < npg;
    const uint32_t ia = (uint32_t)__builtin_amdgcn_readlane((int)hv, pa) & 0x3fffffffu;
    const uint32_t ib = (uint32_t)__builtin_amdgcn_readlane((int)hv, has_b ? pa + 1 : pa) & 0x3fffffffu;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(base + ((size_t)ia * H + kv) * sec_bytes), (short)0, (int)sec_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(base + ((size_t)ib * H + kv) * sec_bytes), (short)0, (int)sec_bytes, 0x00020000);
    load_words<KW>(ra, lo.k, P.ka);
    load_words<KW>(rb, lo.k, P.kb);
    load_words<KW>(ra, lo.v, P.va);
    load_words<KW>(rb, lo.v, P.vb);
    P.ksa = __builtin_amdgcn_raw_buffer_load_b32(ra, lo.ks, 0, 0);
    P.ksb = __builtin_amdgcn_raw_buffer_load_b32(rb, lo.ks, 0, 0);
    // the V scales of both pages (one cache line each); the round picks its side's
    P.vsa = __builtin_amdgcn_raw_buffer_load_b64(ra, lo.vs, 0, 0);
    P.vsb = __builtin_amdgcn_raw_buffer_load_b64(rb, lo.vs, 0, 0);
    if constexpr (ASYM) {
        P.kza = __builtin_amdgcn_raw_buffer_load_b32(ra, lo.kz, 0, 0);
        P.kzb = __builtin_amdgcn_raw_buffer_load_b32(rb, lo.kz, 0, 0);
        P.vza = __builtin_amdgcn_raw_buffer_load_b64(ra, lo.vz, 0, 0);
        P.vzb = __builtin_amdgcn_raw_buffer_load_b64(rb, lo.vz, 0, 0);
    }
    const int page = cb + pa;
    P.ntok_a = real ? min(kPage, ctx - page * kPage) : 0;
    P.ntok_b = real && has_b ? min(kPage, ctx - (page + 1) * kPage) : 0;
}

__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t bits) {
    return (w & mask) | bits;
}

__device__ __forceinline__ uint32_t hfma(uint32_t x, float mul, float add) {
    const half2v m = {(_Float16)mul, (_Float16)mul};
    const half2v c = {(_Float16)add, (_Float16)add};
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2v, x), m, c));
}

// K chunk -> D/8 dwords of signed fp16 code pairs in code order. A field f of a 16-bit half
// sitting at bit 2^k inside the low ten bits is turned into the fp16 value 1024 + 2^k * f by one
// AND-OR with the exponent bits of 1024; one exact fused multiply-add, x * 2^-k - (1024 * 2^-k
// + 2^(b-1)), then gives the signed code. Fields above bit 9 are shifted down by 8 first.
// ASYM: the offset removed is 1024 * 2^-k alone, leaving the unsigned code u.
template <int D, int BITS, bool ASYM = false>
__device__ __forceinline__ void unpack_k_fast(const uint32_t* w, uint32_t* out) {
    constexpr float o = ASYM ? 0.0f : (float)(1 << (BITS - 1));   // the code offset 2^(b-1)
    // the exponent bits of 1024 in a VGPR: gfx9 VOP3 instructions take no literals, so with a
    // register operand the AND-OR is one v_and_or_b32 (mask from an SGPR) instead of two ops
    uint32_t E;
    asm("v_mov_b32 %0, 0x64006400" : "=v"(E));
    if constexpr (BITS == 2) {
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const uint32_t s = w[i] >> 8;
            out[8 * i + 0] = hsub(and_or(w[i], 0x00030003u, E), 1024.0f + o);
            out[8 * i + 1] = hfma(and_or(w[i], 0x000C000Cu, E), 0.25f, -256.0f - o);
            out[8 * i + 2] = hfma(and_or(w[i], 0x00300030u, E), 0.0625f, -64.0f - o);
            out[8 * i + 3] = hfma(and_or(w[i], 0x00C000C0u, E), 0.015625f, -16.0f - o);
            out[8 * i + 4] = hfma(and_or(w[i], 0x03000300u, E), 0.00390625f, -4.0f - o);
            out[8 * i + 5] = hfma(and_or(s, 0x000C000Cu, E), 0.25f, -256.0f - o);
            out[8 * i + 6] = hfma(and_or(s, 0x00300030u, E), 0.0625f, -64.0f - o);
            out[8 * i + 7] = hfma(and_or(s, 0x00C000C0u, E), 0.015625f, -16.0f - o);
        }
    } else if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const uint32_t s = w[i] >> 8;
            out[4 * i + 0] = hsub(and_or(w[i], 0x000F000Fu, E), 1024.0f + o);
            out[4 * i + 1] = hfma(and_or(w[i], 0x00F000F0u, E), 0.0625f, -64.0f - o);
            out[4 * i + 2] = hsub(and_or(s, 0x000F000Fu, E), 1024.0f + o);
            out[4 * i + 3] = hfma(and_or(s, 0x00F000F0u, E), 0.0625f, -64.0f - o);
        }
    } else {
        unpack_k<D, ASYM>(w, 8, out);
    }
}

__device__ __forceinline__ uint32_t dpp_ror8(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, false);
}

// The K scales of a round's pages staged in LDS: slot t holds a page's D/2 scale dwords, the
// D/8 dwords of channel quarter G at t*kKsSlot + G*kKsQuarter. The padding puts the four
// quarters and the two slots of a pair in different banks, so the quarter reads of a wave (all
// lanes of a quarter read the same words) do not conflict.
template <int D> constexpr int kKsQuarter = D / 8 + 4;
template <int D> constexpr int kKsSlot = 4 * kKsQuarter<D>;     // = 16 (mod 32) for D = 64, 128
template <int D>
__device__ __forceinline__ void stage_kscale(uint32_t* ks_lds, int slot, int lane, uint32_t v) {
    const int d = lane & (D / 2 - 1);                            // the lane's scale dword
    ks_lds[slot * kKsSlot<D> + (d / (D / 8)) * kKsQuarter<D> + d % (D / 8)] = v;
}
template <int D>
__device__ __forceinline__ void read_kscales(const uint32_t* ks_lds, int slot, int G, uint32_t* ks) {
    const uint32_t* src = static_cast<const uint32_t*>(
        __builtin_assume_aligned(ks_lds + slot * kKsSlot<D> + G * kKsQuarter<D>, 16));
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        const u32x4 v = *reinterpret_cast<const ma_u32x4*>(src + 4 * i);
        ks[4 * i] = v[0]; ks[4 * i + 1] = v[1]; ks[4 * i + 2] = v[2]; ks[4 * i + 3] = v[3];
    }
}

// S^T of one pair for this lane's side (tokens 4G..4G+3 of its page, head h % 8), log2 units
// SINGLE: page B is absent (a chunk's odd last page): its keys are neither decoded nor multiplied
// ASYM: the zero-point parts of both pages first (their zero points staged in slots 2, 3)
template <int D, int BITS, bool SINGLE = false, bool ASYM = false>
__device__ __forceinline__ float4v pair_logits(const FastPair<D, BITS>& P, const uint32_t* qf,
                                               const uint32_t* ks_lds, int lane, bool side,
                                               float scale_log2) {
    const int G = lane >> 4;
    float4v acca = {0.f, 0.f, 0.f, 0.f}, accb = {0.f, 0.f, 0.f, 0.f};
    if constexpr (ASYM) {
        uint32_t kz[D / 8];
        read_kscales<D>(ks_lds, 2, G, kz);
        acca = zero_point_logits<D>(kz, qf);
        if constexpr (!SINGLE) {
            read_kscales<D>(ks_lds, 3, G, kz);
            accb = zero_point_logits<D>(kz, qf);
        }
    }
    uint32_t kfa[D / 8], kfb[D / 8];
    unpack_k_fast<D, BITS, ASYM>(P.ka, kfa);
    if constexpr (!SINGLE) unpack_k_fast<D, BITS, ASYM>(P.kb, kfb);
    if constexpr (BITS == 2 && !ASYM) {
        // codes -1, 0, 1: code * scale is exact in fp16, so the scales fold into the keys
        uint32_t ksa[D / 8], ksb[D / 8];
        read_kscales<D>(ks_lds, 0, G, ksa);
        read_kscales<D>(ks_lds, 1, G, ksb);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            kfa[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, kfa[i]) * __builtin_bit_cast(half2v, ksa[i]));
            if constexpr (!SINGLE)
                kfb[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, kfb[i]) * __builtin_bit_cast(half2v, ksb[i]));
        }
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const half8 qq = make_half8(qf[4 * i], qf[4 * i + 1], qf[4 * i + 2], qf[4 * i + 3]);
            acca = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                make_half8(kfa[4 * i], kfa[4 * i + 1], kfa[4 * i + 2], kfa[4 * i + 3]), qq, acca, 0, 0, 0);
            if constexpr (!SINGLE)
                accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    make_half8(kfb[4 * i], kfb[4 * i + 1], kfb[4 * i + 2], kfb[4 * i + 3]), qq, accb, 0, 0, 0);
        }
    } else {
        // q * Kscale of this lane's side page as fp16 hi + lo, against both pages' keys
        uint32_t ks[D / 8];
        read_kscales<D>(ks_lds, side ? 1 : 0, G, ks);
        uint32_t qh[D / 8], ql[D / 8];
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            const half2v q2 = __builtin_bit_cast(half2v, qf[i]);
            const half2v s2 = __builtin_bit_cast(half2v, ks[i]);
            const half2v hi = q2 * s2;
            qh[i] = __builtin_bit_cast(uint32_t, hi);
            ql[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q2, s2, -hi));
        }
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const half8 hq = make_half8(qh[4 * i], qh[4 * i + 1], qh[4 * i + 2], qh[4 * i + 3]);
            const half8 lq = make_half8(ql[4 * i], ql[4 * i + 1], ql[4 * i + 2], ql[4 * i + 3]);
            const half8 ka = make_half8(kfa[4 * i], kfa[4 * i + 1], kfa[4 * i + 2], kfa[4 * i + 3]);
            acca = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, hq, acca, 0, 0, 0);
            acca = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, lq, acca, 0, 0, 0);
            if constexpr (!SINGLE) {
                const half8 kb = make_half8(kfb[4 * i], kfb[4 * i + 1], kfb[4 * i + 2], kfb[4 * i + 3]);
                accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, hq, accb, 0, 0, 0);
                accb = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, lq, accb, 0, 0, 0);
            }
        }
    }
    return (side ? accb : acca) * scale_log2;
}

// weights p * Vscale of this lane's four tokens as fp16 hi + lo, exchanged with the partner
// lane (h xor 8) into the PV operand: columns 0..7 hi parts, columns 8..15 lo parts, k slots
// 0..3 page A's tokens 4G..4G+3, slots 4..7 page B's
__device__ __forceinline__ half8 pair_weights(const float* p, uint32_t vs0, uint32_t vs1, bool side,
                                              bool partial, int ntok, int G) {
    const half2v s01 = __builtin_bit_cast(half2v, vs0);
    const half2v s23 = __builtin_bit_cast(half2v, vs1);
    float w[4] = {p[0] * (float)s01[0], p[1] * (float)s01[1], p[2] * (float)s23[0], p[3] * (float)s23[1]};
    if (partial) {                       // masked slots may hold any bits as their scale
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * G + i >= ntok) w[i] = 0.f;
    }
    // hi = w rounded toward zero to fp16 (two per instruction); lo = w - hi, exact in fp32 and
    // then rounded to fp16, one mixed-precision fused multiply-add each
    const half2v h01 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(w[0], w[1]));
    const half2v h23 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(w[2], w[3]));
    half2v l01, l23;
    l01[0] = (_Float16)__builtin_fmaf((float)h01[0], -1.0f, w[0]);
    l01[1] = (_Float16)__builtin_fmaf((float)h01[1], -1.0f, w[1]);
    l23[0] = (_Float16)__builtin_fmaf((float)h23[0], -1.0f, w[2]);
    l23[1] = (_Float16)__builtin_fmaf((float)h23[1], -1.0f, w[3]);
    const uint32_t H0 = __builtin_bit_cast(uint32_t, h01), H1 = __builtin_bit_cast(uint32_t, h23);
    const uint32_t L0 = __builtin_bit_cast(uint32_t, l01), L1 = __builtin_bit_cast(uint32_t, l23);
    const uint32_t r0 = dpp_ror8(side ? H0 : L0), r1 = dpp_ror8(side ? H1 : L1);
    return make_half8(side ? r0 : H0, side ? r1 : H1, side ? L0 : r0, side ? L1 : r1);
}

// max of two logits (finite or -inf) as one median-of-three against +inf held in a register
// (the compiler turns a median against a literal +inf back into a max that first quiets NaNs)
__device__ __forceinline__ float max2(float a, float b, float pinf) {
    return __builtin_amdgcn_fmed3f(a, b, pinf);
}

// one page pair: QK, the running maxima, then PV (SINGLE: page B is absent)
template <int D, int BITS, bool SINGLE = false, bool ASYM = false>
__device__ __forceinline__ void round_fast(const FastPair<D, BITS>& P, const uint32_t* qf,
                                           uint32_t* ks_lds, int lane, int bp16, int bp32, float pinf,
                                           float scale_log2, WaveState<D>& st) {
    const int G = lane >> 4;
    const bool side = (lane & 8) != 0;
    const bool partial = P.ntok_a < kPage || P.ntok_b < kPage;   // uniform: a partial or absent page
    const int ntok = side ? P.ntok_b : P.ntok_a;
    // stage the K scales of the pair's pages (a wave's LDS requests complete in order; the wave
    // barriers keep the compiler from moving LDS accesses across them)
    __builtin_amdgcn_wave_barrier();
    stage_kscale<D>(ks_lds, 0, lane, P.ksa);
    stage_kscale<D>(ks_lds, 1, lane, P.ksb);
    if constexpr (ASYM) {
        stage_kscale<D>(ks_lds, 2, lane, P.kza);
        stage_kscale<D>(ks_lds, 3, lane, P.kzb);
    }
    __builtin_amdgcn_wave_barrier();
    float4v lg = pair_logits<D, BITS, SINGLE, ASYM>(P, qf, ks_lds, lane, side, scale_log2);
    if (partial) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * G + i >= ntok) lg[i] = -INFINITY;
    }
    // The reference m of a head is the same in all eight of its lanes, so a logit above it
    // shows in its own lane: the per-head maximum (both page sides by DPP, the four lane rows
    // by two LDS permutes whose addresses stay fixed for the chunk) is formed only in a round
    // that raises some m -- the first, and then rarely.
    float mx = max2(max2(lg[0], lg[1], pinf), max2(lg[2], lg[3], pinf), pinf);
    if (__builtin_amdgcn_ballot_w64(mx > st.m)) {            // finite: the round holds a token
        mx = max2(mx, __builtin_bit_cast(float, dpp_ror8(__builtin_bit_cast(uint32_t, mx))), pinf);
        mx = max2(mx, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(bp16, __builtin_bit_cast(int, mx))), pinf);
        mx = max2(mx, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(bp32, __builtin_bit_cast(int, mx))), pinf);
        const float m_new = fmaxf(st.m, mx + kLazy);
        const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);   // 0 on the first round
        st.l *= alpha;
        if constexpr (ASYM) st.z *= alpha;
#pragma unroll
        for (int k = 0; k < D / 16; ++k) st.o[k] *= alpha;
        st.m = m_new;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(lg[i] - st.m);
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
    if constexpr (ASYM) {
        const u32x2 vza = P.vza, vzb = P.vzb;
        st.z += zero_point_mass(p, side ? vzb[0] : vza[0], side ? vzb[1] : vza[1], ntok, G);
    }
    const u32x2 vsa = P.vsa, vsb = P.vsb;          // values, so the selects stay in registers
    const uint32_t vs0 = side ? vsb[0] : vsa[0], vs1 = side ? vsb[1] : vsa[1];
    const half8 wop = pair_weights(p, vs0, vs1, side, partial, ntok, G);
    // V codes as exact fp16 integers, decoded like the K codes (the two word layouts put codes
    // in the same positions)
    uint32_t va[D / 8], vb[D / 8];
    unpack_k_fast<D, BITS, ASYM>(P.va, va);
    if constexpr (SINGLE) {
#pragma unroll
        for (int i = 0; i < D / 8; ++i) vb[i] = 0u;
    } else {
        unpack_k_fast<D, BITS, ASYM>(P.vb, vb);
    }
#pragma unroll
    for (int k = 0; k < D / 16; ++k)
        st.o[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            make_half8(va[2 * k], va[2 * k + 1], vb[2 * k], vb[2 * k + 1]), wop, st.o[k], 0, 0, 0);
}

template <int D, int BITS, int DEPTH, bool ASYM = false>
__device__ __forceinline__ void wave_chunk_fast(const uint8_t* base, uint32_t hv, int H, int kv,
                                                int cb, int npg, int ctx, int lane,
                                                const uint32_t* qf, uint32_t* ks_lds,
                                                float scale_log2, WaveState<D>& st) {
    const int nq = (npg + 1) / 2;
    const bool side = (lane & 8) != 0;
    const LaneOffsets lo = lane_offsets<D, BITS, ASYM>(lane);
    const int bp16 = (lane ^ 16) << 2, bp32 = (lane ^ 32) << 2;   // row-exchange addresses
    float pinf;
    asm("v_mov_b32 %0, 0x7f800000" : "=v"(pinf));
    // DEPTH buffers in rotation: pair q is computed while pairs q+1 .. q+DEPTH-1 load; the
    // rotation is unrolled so every buffer index is a constant. The loop runs whole rotations
    // and has one exit, and every round in it issues its loads, also past the end of the chunk
    // (they re-read the last pair, which the caches still hold). A load under a branch, or a
    // second exit, gives the compiler a path into the loop head on which other loads are
    // pending, and its wait counts there then make each round wait for the next pairs too.
    FastPair<D, BITS> b[DEPTH];
#pragma unroll
    for (int j = 0; j < DEPTH - 1; ++j)
        load_pair_fast<D, BITS, ASYM>(base, hv, H, kv, cb, npg, j, nq, ctx, lo, side, b[j]);
    // The scheduling barriers keep each round's instructions between its loads and the next
    // round's: the scheduler would otherwise start decoding the pair just requested inside
    // this round, and the waits for that data would stall the round.
    const int nfull = nq / DEPTH;
    for (int r = 0; r < nfull * DEPTH; r += DEPTH) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
            load_pair_fast<D, BITS, ASYM>(base, hv, H, kv, cb, npg, r + i + DEPTH - 1, nq, ctx, lo, side,
                                    b[(i + DEPTH - 1) % DEPTH]);
            __builtin_amdgcn_sched_barrier(0);
            round_fast<D, BITS, false, ASYM>(b[i], qf, ks_lds, lane, bp16, bp32, pinf, scale_log2, st);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the last nq % DEPTH pairs: the rotation has already loaded them into b[0 ..]; the last
    // of a chunk with an odd page count holds one page only and skips the absent page's work
#pragma unroll
    for (int i = 0; i < DEPTH - 1; ++i) {
        if (i < nq - nfull * DEPTH) {
            if ((npg & 1) && i == nq - nfull * DEPTH - 1)
                round_fast<D, BITS, true, ASYM>(b[i], qf, ks_lds, lane, bp16, bp32, pinf, scale_log2, st);
            else
                round_fast<D, BITS, false, ASYM>(b[i], qf, ks_lds, lane, bp16, bp32, pinf, scale_log2, st);
        }
    }
}

// HALF: the group has at most 8 query heads (see process_pair_half). ASYM: the asymmetric
// storage format. FUSED: the kernel first
// writes the step's new tokens (at most 64 per sequence, so at most five pages): the workgroup
// whose split holds a touched page quantizes it (256 threads a page, two pages at a time) and,
// for the first page, updates the ring, then makes its writes visible to its own loads and
// attends over pos + n_new tokens. No other workgroup reads those pages, so one launch does both steps.
template <int D, bool HALF, bool FUSED, bool ASYM>
// The block table, the lengths (ctx_len, or pos for the fused step), q and the shape integers
// that address them come first as plain arguments: the build preloads the first twelve
// kernel-argument dwords into SGPRs at wave launch, so the first loads need not wait for the
// argument segment.
__global__ __launch_bounds__(kWaves * 64) void decode_attn_kernel(const uint32_t* __restrict__ bt,
                                                                  const int32_t* __restrict__ lens,
                                                                  const uint16_t* __restrict__ qv,
                                                                  int groups, int H, int max_pages,
                                                                  int pps, int Hq, int grp,
                                                                  AttnArgs a) {
    // the K scales of a pair's pages (ASYM: then their zero points), staged per wave
    __shared__ __attribute__((aligned(16))) uint32_t lds_ks[kWaves][ASYM ? 4 : 2][64];
    // the K scales (ASYM: then the zero points) of the uniform-width loop's page pairs, staged
    // per wave (stage_kscale)
    __shared__ __attribute__((aligned(16))) uint32_t lds_ksr[kWaves][(ASYM ? 4 : 2) * kKsSlot<D>];
    // per-wave partials, one padded row per head: channel c of head h sits at h*kORow + c +
    // 4*(c/32), so the float4 writes of a wave's 64 lanes (16 heads x 4 channel quarters) spread
    // over all LDS banks instead of landing on the same four
    constexpr int kORow = D + (D / 32) * 4 + 4;
    __shared__ __attribute__((aligned(16))) float lds_o[kWaves][kMaxGroup * kORow];
    __shared__ float lds_m[kWaves][kMaxGroup];
    __shared__ float lds_l[kWaves][kMaxGroup];
    __shared__ int lds_last;

    const int split = blockIdx.x / groups, group = blockIdx.x % groups;
    const int s = group / H, kv = group % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps page math scalar
    // The handles of this wave's chunk are requested before the context length arrives, on the
    // guess that the split is full (every split but a sequence's last); the guess is checked
    // once the length is known and the last split re-reads its own.
    const int pbeg = split * pps;
    const int cb_full = pbeg + (wave * pps) / kWaves;
    const int npg_full = pbeg + ((wave + 1) * pps) / kWaves - cb_full;
    const uint32_t* bt_row = bt + (size_t)s * max_pages;
    uint32_t hv_full = 0;
    if (npg_full > 0 && npg_full <= 64)
        hv_full = bt_row[min(cb_full + min(lane, npg_full - 1), max_pages - 1)];
    // q fragment: lane (h, G) holds q[h][G*D/4 .. +D/4) as fp16 pairs (zero for h >= grp)
    const int h = lane & 15, G = lane >> 4;
    const int hq = HALF ? (h & 7) : h;                 // the query head of this lane's column
    uint32_t qf[D / 8];
    {
        const ma_u32* qp = reinterpret_cast<const ma_u32*>(
            qv + ((size_t)s * Hq + kv * grp + min(hq, grp - 1)) * D + G * (D / 4));
#pragma unroll
        for (int i = 0; i < D / 8; ++i) qf[i] = hq < grp ? qp[i] : 0u;
    }

    const int ctx = ((const_i32_ptr)lens)[s] + (FUSED ? a.n_new : 0);
    const int npages = (ctx + kPage - 1) / kPage;
    const int nsplit = (npages + a.pps - 1) / a.pps;

    if (split >= nsplit) {
        if (split == 0 && ctx <= 0)            // no keys: the rows are zero
            for (int i = tid; i < grp * D; i += kWaves * 64)
                a.out[((size_t)s * a.Hq + kv * grp) * D + i] = 0.f;
        return;
    }
    const int pend = min(pbeg + a.pps, npages);

    if constexpr (FUSED) {
        __shared__ float chan_max[2][ASYM ? 8 : 4][D];
        const int p0 = ctx - a.n_new;
        const int first_page = p0 / kPage, last_page = (ctx - 1) / kPage;
        // the touched pages this split holds, two at a time (256 threads a page)
        const int lo_page = max(first_page, pbeg), hi_page = min(last_page, pend - 1);
        if (a.n_new > 0 && lo_page <= hi_page) {         // uniform over the workgroup
            const int half = tid >> 8;                   // threads 0..255: even page, 256..511: odd
            for (int pg = lo_page; pg <= hi_page; pg += 2) {
                write_page<D, ASYM>(a.wr, s, kv, p0, pg + half - first_page, tid & 255,
                                    pg + half <= hi_page, chan_max[half]);
                __syncthreads();                         // chan_max is reused; ring reads done
            }
            if (lo_page == first_page)                   // the first page's split: the ring
                write_ring<D>(a.wr, s, kv, p0, tid, kWaves * 64);
            // the writes complete before any wave of this workgroup reads the pages: only this
            // workgroup reads them in this launch, and stores from this compute unit are seen
            // by its own later loads (workgroup scope), so no cache invalidation is needed (an
            // agent-scope acquire here invalidated the L2 and cost 1-5 us per workgroup)
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    WaveState<D> st;
    st.m = -INFINITY;
    st.l = 0.f;
    st.z = 0.f;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) st.o[k] = float4v{0.f, 0.f, 0.f, 0.f};

    uint32_t* ks_slot = &lds_ks[wave][0][0];
    // Each wave takes a contiguous chunk of the split (sizes differ by at most one page) and
    // walks it in page pairs. A chunk of at most 64 pages has its handles read once into
    // registers (lane i: page cb + i); when they all share one width -- the common case, since
    // a layer changes width at most at a tier switch -- the chunk runs a loop specialized for
    // that width.
    const int n = pend - pbeg;
    const int cb = pbeg + (wave * n) / kWaves;
    const int npg = pbeg + ((wave + 1) * n) / kWaves - cb;
    if (npg > 0) {
        bool uniform = false;
        uint32_t hv = 0;
        int tier0 = 0;
        if (npg <= 64) {
            hv = pend - pbeg == a.pps ? hv_full : bt_row[cb + min(lane, npg - 1)];
            tier0 = (int)((uint32_t)__builtin_amdgcn_readfirstlane((int)hv) >> 30);
            uniform = __builtin_amdgcn_ballot_w64((int)(hv >> 30) != tier0) == 0;
        }
        uint32_t* ks_round = &lds_ksr[wave][0];
        if (HALF && uniform && tier0 == 0)
            wave_chunk_fast<D, 2, kDepth2, ASYM>(a.pools.base[0], hv, a.H, kv, cb, npg, ctx, lane, qf,
                                           ks_round, a.scale_log2, st);
        else if (HALF && uniform && tier0 == 1)
            wave_chunk_fast<D, 4, kDepth4, ASYM>(a.pools.base[1], hv, a.H, kv, cb, npg, ctx, lane, qf,
                                           ks_round, a.scale_log2, st);
        else if (HALF && uniform && tier0 == 2)
            wave_chunk_fast<D, 8, kDepth8, ASYM>(a.pools.base[2], hv, a.H, kv, cb, npg, ctx, lane, qf,
                                           ks_round, a.scale_log2, st);
        else if (uniform && tier0 == 0)
            wave_chunk_uniform<D, 2, 2, HALF, ASYM>(a.pools.base[0], hv, a.H, kv, cb, npg, ctx, lane, qf, ks_slot,
                                     a.scale_log2, st);
        else if (uniform && tier0 == 1)
            wave_chunk_uniform<D, 4, 2, HALF, ASYM>(a.pools.base[1], hv, a.H, kv, cb, npg, ctx, lane, qf, ks_slot,
                                     a.scale_log2, st);
        else if (uniform && tier0 == 2)
            wave_chunk_uniform<D, 8, 2, HALF, ASYM>(a.pools.base[2], hv, a.H, kv, cb, npg, ctx, lane, qf, ks_slot,
                                     a.scale_log2, st);
        else if (uniform && tier0 == kFp16Tier)
            wave_chunk_f16<D, HALF>(a.pools.base[3], hv, a.H, kv, cb, npg, ctx, lane, qf,
                                    a.scale_log2, st);
        else {
            const PageSrc src = {a.pools.base[0], a.pools.base[1], a.pools.base[2],
                                 a.pools.base[3], bt_row, a.H};
            wave_chunk_mixed<D, HALF, ASYM>(src, kv, cb, npg, ctx, lane, qf, ks_slot, a.scale_log2, st);
        }
    }

    // ---- this wave's partial -> LDS
    float lsum = st.l;
    if constexpr (HALF) {                              // fold columns 8..15 into 0..7
        lsum += __builtin_bit_cast(float, dpp_ror8(__builtin_bit_cast(uint32_t, lsum)));
#pragma unroll
        for (int k = 0; k < D / 16; ++k)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // through a scalar: a bit cast applied to a vector element itself reads the
                // vector's first element with this compiler
                const float x = st.o[k][r];
                st.o[k][r] = x + __builtin_bit_cast(float, dpp_ror8(__builtin_bit_cast(uint32_t, x)));
            }
    }
    lsum = rows_sum(lsum);
    if constexpr (ASYM) {
        // the zero-point part of the values, sum_t p_t m_t, is the same for every channel of a
        // head: folded and summed like l, then added to the head's accumulators
        float zsum = st.z;
        if constexpr (HALF) zsum += __builtin_bit_cast(float, dpp_ror8(__builtin_bit_cast(uint32_t, zsum)));
        zsum = rows_sum(zsum);
#pragma unroll
        for (int k = 0; k < D / 16; ++k) st.o[k] += zsum;
    }
    if (h < grp) {
        if (G == 0) {
            lds_m[wave][h] = st.m;
            lds_l[wave][h] = lsum;
        }
        // element r of o[k] is channel G*D/4 + r*D/16 + k: for each r the D/16 channels are
        // consecutive, written as float4s
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int k4 = 0; k4 < D / 64; ++k4)
                *reinterpret_cast<ma_f32x4*>(&lds_o[wave][h * kORow + G * (D / 4) + r * (D / 16) + 4 * k4 +
                                                         4 * ((G * (D / 4) + r * (D / 16)) / 32)]) =
                    float4v{st.o[4 * k4][r], st.o[4 * k4 + 1][r], st.o[4 * k4 + 2][r], st.o[4 * k4 + 3][r]};
    }
    __syncthreads();

    // ---- merge the waves (fixed order) into this split's partial: one float4 of one head per
    // thread. Partials travel through device-coherent (sc1) stores and loads, which bypass the
    // per-XCD L2s, so no cache write-back or invalidate is needed.
    constexpr int kSc1 = 16;                              // cache-policy bit: device coherent
    const bool single = nsplit == 1;
    const int nslot = grp * D / 4;
    const __amdgpu_buffer_rsrc_t o_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        a.ws_o + (size_t)group * a.splits * grp * D, (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t ml_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        a.ws_ml + (size_t)group * a.splits * grp * 2, (short)0, 0x7fffffff, 0x00020000);
    for (int sl = tid; sl < nslot; sl += kWaves * 64) {
        const int hh = sl / (D / 4), c4 = sl - hh * (D / 4);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_m[w][hh]);
        float L = 0.f;
        float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = lds_m[w][hh];
            const float e = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            acc += e * *reinterpret_cast<const ma_f32x4*>(&lds_o[w][hh * kORow + 4 * c4 + 4 * (c4 / 8)]);
            L += e * lds_l[w][hh];
        }
        if (single) {
            const float inv = L > 0.f ? 1.f / L : 0.f;
            *reinterpret_cast<ma_f32x4*>(a.out + ((size_t)s * a.Hq + kv * grp + hh) * D + 4 * c4) = acc * inv;
        } else {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), o_rsrc,
                                                   (int)((split * grp + hh) * D + 4 * c4) * 4, 0, kSc1);
            if (c4 == 0)
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, float2v{M, L}), ml_rsrc,
                                                      (hh * a.splits + split) * 8, 0, kSc1);
        }
    }
    if (single) return;

    // ---- the last split of this (sequence, KV head) to finish merges all partials in order.
    // Every thread waits until its partial stores have completed before the workgroup takes
    // its ticket; the winner reads the partials with coherent loads issued after the ticket.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        lds_last = __hip_atomic_fetch_add(&a.counters[group * kCounterStride], 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(nsplit - 1);
    __syncthreads();
    if (!lds_last) return;

    // One wave per head. The wave first requests the head's (max, sum) pairs (lane k: splits
    // k, k+64, ...; contiguous per head) and then its first kBatch partials per lane -- lane
    // (c4, part) sums four channels over a contiguous run of the splits -- so both arrive in one
    // memory round trip. The split weights e_k = 2^(m_k - M) are formed once, at the lane that
    // holds the pair, and pass to the other lanes through the wave's own LDS row; the parts
    // combine by lane exchanges. No workgroup barrier is taken. Loads past a lane's run
    // re-read its last split and get weight zero.
    constexpr int kBatch = 16;
    constexpr int kParts = 256 / D;                      // lanes per output slot
    float* e_row = &lds_o[wave][0];                      // kMaxSplits weights of this wave's head
    const int c4 = lane % (D / 4), part = lane / (D / 4);
    const int per_part = (nsplit + kParts - 1) / kParts;
    const int k0 = min(nsplit, part * per_part), k1 = min(nsplit, k0 + per_part);
    const uint32_t stride = (uint32_t)(grp * D * 4);     // bytes from one split's partial to the next
    for (int h2 = wave; h2 < grp; h2 += kWaves) {
        float2v ml[kMaxSplits / 64];
#pragma unroll
        for (int r = 0; r < kMaxSplits / 64; ++r)
            if (64 * r < nsplit)                         // uniform
                ml[r] = __builtin_bit_cast(float2v, __builtin_amdgcn_raw_buffer_load_b64(
                    ml_rsrc, (uint32_t)((h2 * a.splits + min(64 * r + lane, nsplit - 1)) * 8), 0, kSc1));
        // the offsets in VGPRs: as scalars, the offsets of a batch would each take a register
        // (a part without splits reads split nsplit-1, in range, and gives it weight zero)
        uint32_t off = (uint32_t)((min(k0, nsplit - 1) * grp + h2) * D * 4 + c4 * 16);
        uint32_t last = k1 > k0 ? off + (uint32_t)(k1 - 1 - k0) * stride : off;
        asm("" : "+v"(off), "+v"(last));
        float4v buf[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            buf[i] = __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(
                o_rsrc, min(off + (uint32_t)i * stride, last), 0, kSc1));
        float M = -INFINITY;
#pragma unroll
        for (int r = 0; r < kMaxSplits / 64; ++r)
            if (64 * r < nsplit) M = fmaxf(M, ml[r][0]);
        M = wave_max(M);
        float L = 0.f;
#pragma unroll
        for (int r = 0; r < kMaxSplits / 64; ++r)
            if (64 * r < nsplit) {
                const int k = 64 * r + lane;
                const float e = k >= nsplit || ml[r][0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[r][0] - M);
                L += e * ml[r][1];
                if (k < nsplit) e_row[k] = e;
            }
        L = wave_sum(L);
        __builtin_amdgcn_wave_barrier();                 // the wave's LDS accesses stay in order
        float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (k0 + i < k1) acc += e_row[k0 + i] * buf[i];
        for (int kb = k0 + kBatch; kb < k1; kb += kBatch) {            // long split lists only
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                buf[i] = __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(
                    o_rsrc, min(off + (uint32_t)(kb - k0 + i) * stride, last), 0, kSc1));
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                if (kb + i < k1) acc += e_row[kb + i] * buf[i];
        }
        __builtin_amdgcn_wave_barrier();                 // e_row is rewritten for the next head
#pragma unroll
        for (int w = 64 / kParts; w < 64; w *= 2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = acc[r];
                acc[r] = x + __shfl_xor(x, w, 64);
            }
        if (part == 0) {
            const float inv = L > 0.f ? 1.f / L : 0.f;
            *reinterpret_cast<ma_f32x4*>(a.out + ((size_t)s * a.Hq + kv * grp + h2) * D + c4 * 4) = acc * inv;
        }
    }
    if (tid == 0)
        __hip_atomic_store(&a.counters[group * kCounterStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// Workspace layout: the ticket counters of every (sequence slot, KV head) of the geometry --
// sized by max_seqs, not by the call's batch, so every call on one geometry finds its counters
// at the same place, left at zero by the call before -- then the per-split (max, sum) pairs
// and partial outputs of this call, which each call writes before it reads them.
static size_t counter_region_bytes(const kv_geometry& g) {
    return (size_t)g.max_seqs * g.num_kv_heads * kCounterStride * 4 + 256;
}

size_t decode_workspace_bytes(const kv_geometry& g, int batch, int splits) {
    const size_t groups = (size_t)batch * g.num_kv_heads;
    const size_t grp = (size_t)(g.num_q_heads / g.num_kv_heads);
    size_t bytes = counter_region_bytes(g);
    bytes += ((groups * splits * grp * 2 * sizeof(float) + 255) / 256) * 256;
    bytes += groups * splits * grp * g.head_dim * sizeof(float);
    return bytes;
}

namespace {

AttnArgs attn_args(const kv_geometry& g, PoolPtrs pools, const uint32_t* bt, int batch, int splits,
                   int pages_per_split, const uint16_t* q, float softmax_scale, float* out,
                   void* workspace) {
    AttnArgs a = {};
    a.pools = pools;
    a.bt = bt;
    a.q = q;
    a.out = out;
    a.max_pages = g.max_pages_per_seq;
    a.H = g.num_kv_heads;
    a.Hq = g.num_q_heads;
    a.grp = g.num_q_heads / g.num_kv_heads;
    a.groups = batch * g.num_kv_heads;
    a.splits = splits;
    a.pps = pages_per_split;
    a.scale_log2 = softmax_scale * kLog2e;
    const size_t groups = (size_t)a.groups;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    a.counters = reinterpret_cast<uint32_t*>(ws);
    size_t off = counter_region_bytes(g);
    a.ws_ml = reinterpret_cast<float*>(ws + off);
    off += ((groups * splits * a.grp * 2 * sizeof(float) + 255) / 256) * 256;
    a.ws_o = reinterpret_cast<float*>(ws + off);
    return a;
}

template <int D, bool HALF, bool FUSED, bool ASYM>
void launch_one(const AttnArgs& a, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((decode_attn_kernel<D, HALF, FUSED, ASYM>), grid, dim3(kWaves * 64), 0, stream,
                       a.bt, FUSED ? a.pos : a.ctx_len, a.q, a.groups, a.H, a.max_pages, a.pps, a.Hq,
                       a.grp, a);
}

template <int D, bool FUSED, bool ASYM>
void launch_d(const AttnArgs& a, dim3 grid, hipStream_t stream) {
    if (a.grp <= 8) launch_one<D, true, FUSED, ASYM>(a, grid, stream);
    else launch_one<D, false, FUSED, ASYM>(a, grid, stream);
}

template <bool FUSED>
hipError_t launch(const kv_geometry& g, const AttnArgs& a, int splits, hipStream_t stream) {
    const dim3 grid((unsigned)(splits * a.groups));
    const bool asym = g.asymmetric != 0;
    if (g.head_dim == 128) {
        if (asym) launch_d<128, FUSED, true>(a, grid, stream);
        else launch_d<128, FUSED, false>(a, grid, stream);
    } else {
        if (asym) launch_d<64, FUSED, true>(a, grid, stream);
        else launch_d<64, FUSED, false>(a, grid, stream);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_attn(const kv_geometry& g, PoolPtrs pools, const uint32_t* bt,
                              const int32_t* ctx_len, int batch, int splits, int pages_per_split,
                              const uint16_t* q, float softmax_scale, float* out,
                              void* workspace, hipStream_t stream) {
    AttnArgs a = attn_args(g, pools, bt, batch, splits, pages_per_split, q, softmax_scale, out,
                           workspace);
    a.ctx_len = ctx_len;
    return launch<false>(g, a, splits, stream);
}

namespace {

void set_write_args(AttnArgs& a, const kv_geometry& g, PoolPtrs pools, const uint32_t* bt,
                    const int32_t* pos, int n_new, const uint16_t* k_new, const uint16_t* v_new,
                    uint16_t* ring) {
    a.pos = pos;
    a.n_new = n_new;
    a.wr.pools = pools;
    a.wr.bt = bt;
    a.wr.pos = pos;
    a.wr.k_new = k_new;
    a.wr.v_new = v_new;
    a.wr.ring = ring;
    a.wr.max_pages = g.max_pages_per_seq;
    a.wr.n_new = n_new;
    a.wr.H = g.num_kv_heads;
    a.wr.R = g.ring_size;
}

}  // namespace

hipError_t launch_decode_step(const kv_geometry& g, PoolPtrs pools, const uint32_t* bt,
                              const int32_t* pos, int batch, int n_new, const uint16_t* k_new,
                              const uint16_t* v_new, uint16_t* ring, int splits,
                              int pages_per_split, const uint16_t* q, float softmax_scale,
                              float* out, void* workspace, hipStream_t stream) {
    AttnArgs a = attn_args(g, pools, bt, batch, splits, pages_per_split, q, softmax_scale, out,
                           workspace);
    set_write_args(a, g, pools, bt, pos, n_new, k_new, v_new, ring);
    return launch<true>(g, a, splits, stream);
}

// ---------------------------------------------------------------- the fixed device scratch
// For callers that cannot allocate device memory (code under graph capture, tight serving
// loops): the fused step's workspace -- ticket counters, split maxima and sums, split partial
// outputs -- lives in one file-scope device array of kStaticScratchBytes, one copy per GPU,
// held until the process ends. The counters sit at a fixed place (one 256-byte line for each
// of kStaticMaxGroups (sequence, KV head) groups, whatever the geometry), so the zeros one call
// leaves there serve the next call of any geometry; the partials follow and are written before
// they are read. Calls that overlap on one GPU share the array and race.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
static_assert((size_t)kStaticMaxGroups * kCounterStride * 4 == kStaticCounterBytes,
              "one counter line per group");

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices];     // device address of `scratch` on each GPU
bool g_scratch_cleared[kMaxDevices];

__global__ void clear_words(uint32_t* p, uint32_t n) {
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        p[i] = 0u;
}

// The scratch array's address on the current device, looked up once per device with that
// device current (the array's name is a host-side stand-in, never a device address). The first
// call on a device also clears the counters with a fill kernel on the caller's stream: device
// arrays without an initializer start at zero when the code object is loaded, and the clear
// keeps that true even if this first call is captured into a graph rather than run.
hipError_t static_scratch(hipStream_t stream, uint8_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
    }
    if (!g_scratch_cleared[dev]) {
        hipLaunchKernelGGL(clear_words, dim3(256), dim3(256), 0, stream,
                           reinterpret_cast<uint32_t*>(g_scratch_ptr[dev]),
                           (uint32_t)(kStaticCounterBytes / 4));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch_cleared[dev] = true;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

size_t static_scratch_partial_bytes(const kv_geometry& g, int batch, int splits) {
    const size_t groups = (size_t)batch * g.num_kv_heads;
    const size_t grp = (size_t)(g.num_q_heads / g.num_kv_heads);
    return ((groups * splits * grp * 2 * sizeof(float) + 255) / 256) * 256 +
           groups * splits * grp * g.head_dim * sizeof(float);
}

hipError_t launch_decode_step_static(const kv_geometry& g, PoolPtrs pools, const uint32_t* bt,
                                     const int32_t* pos, int batch, int n_new,
                                     const uint16_t* k_new, const uint16_t* v_new, uint16_t* ring,
                                     int splits, int pages_per_split, const uint16_t* q,
                                     float softmax_scale, float* out, hipStream_t stream) {
    uint8_t* ws = nullptr;
    const hipError_t e = static_scratch(stream, &ws);
    if (e != hipSuccess) return e;
    AttnArgs a = attn_args(g, pools, bt, batch, splits, pages_per_split, q, softmax_scale, out, ws);
    const size_t groups = (size_t)a.groups;
    a.counters = reinterpret_cast<uint32_t*>(ws);
    a.ws_ml = reinterpret_cast<float*>(ws + kStaticCounterBytes);
    a.ws_o = reinterpret_cast<float*>(
        ws + kStaticCounterBytes +
        ((groups * splits * a.grp * 2 * sizeof(float) + 255) / 256) * 256);
    set_write_args(a, g, pools, bt, pos, n_new, k_new, v_new, ring);
    return launch<true>(g, a, splits, stream);
}

}  // namespace kvq
