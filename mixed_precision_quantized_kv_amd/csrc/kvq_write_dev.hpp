// kvq_write_dev.hpp -- quantize-on-write of one page by 256 threads, shared by the write kernel
// and the fused decode-step kernel.
//
// EchoKV, "How EchoKV works": the step's key enters the per-layer FP16 ring before it is
// quantized into the paged cache. Behavior-Guided KV-Cache Quantization, "K/V Role-Aware
// Low-Bit Quantization": keys get one scale per channel (over the page's tokens), values one
// scale per token (over its channels); "Online inference": pack and store. Pages of the FP16
// tier (a layer before the canary first fires) take the new keys and values as they are.
//
// Thread (t, g) = (tid / 16, tid % 16) owns token slot t of the page and channels
// [g*D/16, (g+1)*D/16): every input element is fetched by exactly one 8- or 16-byte load,
// issued up front, so the threads wait on memory once. Channel maxima over the page's tokens
// reduce across the four token lanes of a wave (shuffles) and the four waves (LDS); token maxima
// over D reduce across the 16 lanes of a token (shuffles). Codes are packed in registers; words
// shared by several threads are OR-reduced with shuffles.
//
// The asymmetric format (ASYM) keeps the groups and gives each a zero point and a scale from its
// minimum and maximum (EchoKV, "Show the math": KIVI-style asymmetric groups; "Future work":
// per-token KIVI storage in the paged cache); the channel reduction then carries both extremes.
#pragma once

#include "kvq_device.hpp"

namespace kvq {

struct WriteArgs {
    PoolPtrs pools;
    const uint32_t* bt;
    const int32_t* pos;
    const uint16_t* k_new;
    const uint16_t* v_new;
    uint16_t* ring;
    int max_pages;
    int n_new;
    int H;
    int R;
};

// CPT consecutive fp16 values (CPT = 4 or 8, 8- or 16-byte aligned) as floats
template <int CPT>
__device__ __forceinline__ void load_f16(const uint16_t* p, float* out) {
    if constexpr (CPT == 8) {
        const uint4 v = *reinterpret_cast<const ma_uint4*>(p);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = f16_val((uint16_t)(w[i] & 0xffffu));
            out[2 * i + 1] = f16_val((uint16_t)(w[i] >> 16));
        }
    } else {
        const uint2 v = *reinterpret_cast<const ma_uint2*>(p);
        const uint32_t w[2] = {v.x, v.y};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            out[2 * i] = f16_val((uint16_t)(w[i] & 0xffffu));
            out[2 * i + 1] = f16_val((uint16_t)(w[i] >> 16));
        }
    }
}

// CPT (4 or 8) fp16 bit patterns to 8- or 16-byte aligned memory
template <int CPT>
__device__ __forceinline__ void store_f16s(ma_u16* dst, const uint16_t* v) {
    if constexpr (CPT == 8) {
        uint4 w;
        w.x = v[0] | ((uint32_t)v[1] << 16); w.y = v[2] | ((uint32_t)v[3] << 16);
        w.z = v[4] | ((uint32_t)v[5] << 16); w.w = v[6] | ((uint32_t)v[7] << 16);
        *reinterpret_cast<ma_uint4*>(dst) = w;
    } else {
        uint2 w;
        w.x = v[0] | ((uint32_t)v[1] << 16); w.y = v[2] | ((uint32_t)v[3] << 16);
        *reinterpret_cast<ma_uint2*>(dst) = w;
    }
}

// pool base of a tier, by arithmetic (a select chain would become a lookup table in scratch)
__device__ __forceinline__ uint8_t* pool_base(const PoolPtrs& pools, int tier) {
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(pools.base[0]);
    return reinterpret_cast<uint8_t*>(
        b0 + (uintptr_t)(tier == 1) * (reinterpret_cast<uintptr_t>(pools.base[1]) - b0) +
        (uintptr_t)(tier == 2) * (reinterpret_cast<uintptr_t>(pools.base[2]) - b0) +
        (uintptr_t)(tier == 3) * (reinterpret_cast<uintptr_t>(pools.base[3]) - b0));
}

// Write page p0/P + j of sequence s, KV head kv, for the call's new tokens [p0, p0 + n_new):
// the page's K scales and the codes of all its present tokens from their FP16 originals (ring
// for positions < p0, k_new after), the new tokens' V codes and scales. `tid` is 0..255 within
// the 256 threads doing this page; `active` false (or a page past the call) writes nothing.
// Every thread of the workgroup must call this (it holds one workgroup barrier). chan_red holds
// 4 rows of D floats (the four waves' channel maxima), 8 for ASYM (then the minima follow).
template <int D, bool ASYM = false>
__device__ __forceinline__ void write_page(const WriteArgs& a, int s, int kv, int p0, int j, int tid,
                                           bool active, float (*chan_red)[D]) {
    constexpr int P = kPage;
    constexpr int CPT = D / 16;                 // channels per thread
    const int t = tid >> 4, g = tid & 15, c0 = g * CPT;
    const int wave = tid >> 6;
    const int end = p0 + a.n_new;
    const int page = p0 / P + j;
    const int lo = page * P;
    active = active && lo < end;                // uniform over the 256 threads
    const int nk = min(lo + P, end) - lo;       // present tokens after the write
    const int told = max(0, p0 - lo);           // tokens cached before this call
    const int p = lo + t;
    const bool present = active && t < nk;
    const bool is_new = present && t >= told;

    // ---- gather first (it depends only on pos): this thread's keys (ring for positions < pos,
    // input after) and new values; the block-table lookup and old V words follow
    float kf[CPT], vf[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) kf[i] = vf[i] = 0.f;
    uint16_t* ring_s = a.ring + (size_t)s * a.R * a.H * D;
    if (present) {
        const uint16_t* src = p < p0
            ? ring_s + ((size_t)(p % a.R) * a.H + kv) * D + c0
            : a.k_new + (((size_t)s * a.n_new + (p - p0)) * a.H + kv) * D + c0;
        load_f16<CPT>(src, kf);
    }
    if (is_new)
        load_f16<CPT>(a.v_new + (((size_t)s * a.n_new + (p - p0)) * a.H + kv) * D + c0, vf);

    uint32_t handle = 0;
    if (active) handle = a.bt[(size_t)s * a.max_pages + page];
    const int tier = (int)(handle >> 30);
    const int bits = bits_of_tier(tier);
    const bool fp16 = tier == kFp16Tier;
    const Section L = section_layout(D, bits, ASYM);
    uint8_t* sec = pool_base(a.pools, tier) + ((size_t)(handle & 0x3fffffffu) * a.H + kv) * L.bytes;
    const uint32_t qoff = ASYM ? 0u : 1u << (bits - 1);   // the field of the zero code
    const uint32_t fmask = (1u << bits) - 1u;

    // ---- V code words this lane will store. V codes are grouped by token quads: code index
    // ((t/4)*D + c)*4 + t%4, 32/b codes per word, so a word holds cw = 8/b channels of one quad.
    // The quad of token t is handled by the four lanes t%4 = 0..3 of one wave; lane r stores the
    // words w of its channel group with w % 4 == r. A quad seen for the first time is written
    // whole (its empty slots get the zero code); a quad that already holds tokens is read,
    // merged with the new fields and written back (its other fields are kept).
    const int cw = fp16 ? 1 : 8 / bits;         // channels per V word (FP16: unused)
    const int nwv = CPT / cw;                   // V words per (quad, channel group): 1..8
    const int quad = t >> 2, r = t & 3;
    const bool quad_old = 4 * quad < told;      // the quad holds tokens cached before the call
    const bool quad_new = 4 * quad + 3 >= told && 4 * quad < nk;
    const bool quad_store = active && (quad_new || !quad_old);   // entirely-old quads: untouched
    ma_u32* vwords = reinterpret_cast<ma_u32*>(sec + L.vcode_off);
    const int wbase = ((quad * D + c0) * 4) / (32 / bits);  // first V word of this (quad, group)
    uint32_t vold[2] = {0u, 0u};                // at most 8 words / 4 lanes
    if (quad_store && quad_old && !fp16) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int w = r + 4 * i;
            if (w < nwv) vold[i] = vwords[wbase + w];
        }
    }

    // ---- K: channel maxima of |x| over the present tokens (empty slots hold zeros); ASYM: the
    // channel maxima and minima of x over the present tokens
    float m[CPT], mn[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        float x = ASYM ? (present ? kf[i] : -INFINITY) : fabsf(kf[i]);
        x = fmaxf(x, __shfl_xor(x, 16, 64));
        m[i] = fmaxf(x, __shfl_xor(x, 32, 64));
        if constexpr (ASYM) {
            float y = present ? kf[i] : INFINITY;
            y = fminf(y, __shfl_xor(y, 16, 64));
            mn[i] = fminf(y, __shfl_xor(y, 32, 64));
        }
    }
    if ((tid & 63) < 16) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            chan_red[wave][c0 + i] = m[i];
            if constexpr (ASYM) chan_red[4 + wave][c0 + i] = mn[i];
        }
    }
    __syncthreads();
    if (!active) return;
    if (fp16) {
        // FP16 tier: the new tokens' keys and values as they are, zeros in the empty slots; the
        // slots of tokens cached before the call are not touched
        if (t >= told) {
            uint16_t kb[CPT], vb[CPT];
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                kb[i] = present ? f16_bits((_Float16)kf[i]) : (uint16_t)0;
                vb[i] = is_new ? f16_bits((_Float16)vf[i]) : (uint16_t)0;
            }
            ma_u16* krow = reinterpret_cast<ma_u16*>(sec) + (size_t)t * D + c0;
#pragma unroll
            for (int i = 0; i < CPT; i += 2)
                reinterpret_cast<ma_u32*>(krow)[i / 2] = kb[i] | ((uint32_t)kb[i + 1] << 16);
            ma_u16* vvals = reinterpret_cast<ma_u16*>(sec + L.vcode_off);
#pragma unroll
            for (int i = 0; i < CPT; ++i) vvals[((size_t)(quad * D + c0 + i)) * 4 + r] = vb[i];
        }
        return;
    }
    uint16_t ks[CPT], kz[CPT];
    uint32_t ku[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const float amax = fmaxf(fmaxf(chan_red[0][c0 + i], chan_red[1][c0 + i]),
                                 fmaxf(chan_red[2][c0 + i], chan_red[3][c0 + i]));
        if constexpr (ASYM) {
            const float amin = fminf(fminf(chan_red[4][c0 + i], chan_red[5][c0 + i]),
                                     fminf(chan_red[6][c0 + i], chan_red[7][c0 + i]));
            kz[i] = asym_zero(amin);
            ks[i] = asym_scale(amin, amax, bits);
            ku[i] = present ? asym_code(kf[i], f16_val(kz[i]), f16_val(ks[i]), bits) : 0u;
        } else {
            kz[i] = 0;
            ks[i] = group_scale(amax, bits);
            ku[i] = (present && ks[i]) ? (uint32_t)(quant_code(kf[i], f16_val(ks[i]), bits) + (int)qoff)
                                       : qoff;
        }
    }

    // ---- K codes: row t holds D codes, 32/b per word; this thread's CPT codes fill CPT*b bits
    {
        ma_u32* row = reinterpret_cast<ma_u32*>(sec + (size_t)t * (D * bits / 8));
        const int per_word = 32 / bits;
        if (CPT * bits >= 32) {                 // whole words: INT4/INT8 (D=128), INT8 (D=64)
            const int nw = CPT * bits / 32;
            for (int w = 0; w < nw; ++w) {
                uint32_t word = 0;
#pragma unroll
                for (int i = 0; i < CPT; ++i)
                    if (i / per_word == w) word |= ku[i] << field_bit(i % per_word, bits);
                row[c0 / per_word + w] = word;
            }
        } else {                                // 2 or 4 neighbouring threads share a word
            const int share = 32 / (CPT * bits);
            const int k0 = (g % share) * CPT;
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < CPT; ++i) word |= ku[i] << field_bit(k0 + i, bits);
            word |= __shfl_xor(word, 1, 64);
            if (share == 4) word |= __shfl_xor(word, 2, 64);
            if (g % share == 0) row[c0 / per_word] = word;
        }
    }
    // K scales, and ASYM zero points (slot row 0 writes them)
    if (t == 0) {
        store_f16s<CPT>(reinterpret_cast<ma_u16*>(sec + L.kscale_off) + c0, ks);
        if constexpr (ASYM) store_f16s<CPT>(reinterpret_cast<ma_u16*>(sec + L.kzero_off) + c0, kz);
    }

    // ---- V: one scale (ASYM: and zero point) per new token over its D channels (the token's
    // 16 lanes)
    float vm = ASYM ? -INFINITY : 0.f, vn = INFINITY;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        vm = fmaxf(vm, ASYM ? vf[i] : fabsf(vf[i]));
        vn = fminf(vn, vf[i]);
    }
#pragma unroll
    for (int msk = 1; msk < 16; msk <<= 1) {
        vm = fmaxf(vm, __shfl_xor(vm, msk, 64));
        if constexpr (ASYM) vn = fminf(vn, __shfl_xor(vn, msk, 64));
    }
    const uint16_t vs = !is_new ? (uint16_t)0 : ASYM ? asym_scale(vn, vm, bits) : group_scale(vm, bits);
    const uint16_t vz = ASYM && is_new ? asym_zero(vn) : (uint16_t)0;
    const float vsf = f16_val(vs), vzf = f16_val(vz);
    // this token's fields (new tokens: their codes; empty slots: the zero code) and the mask of
    // fields the call writes
    uint32_t part[8], mask[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) part[w] = mask[w] = 0u;
    if (t >= told) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            uint32_t u;
            if constexpr (ASYM)
                u = is_new ? asym_code(vf[i], vzf, vsf, bits) : 0u;
            else
                u = (is_new && vs) ? (uint32_t)(quant_code(vf[i], vsf, bits) + (int)qoff) : qoff;
            const int w = i / cw;
            const int fb = field_bit((i % cw) * 4 + r, bits);
            part[w] |= u << fb;
            mask[w] |= fmask << fb;
        }
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        if (w < nwv) {
            part[w] |= __shfl_xor(part[w], 16, 64);
            part[w] |= __shfl_xor(part[w], 32, 64);
            mask[w] |= __shfl_xor(mask[w], 16, 64);
            mask[w] |= __shfl_xor(mask[w], 32, 64);
        }
    }
    if (quad_store) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int w = r + 4 * i;
            if (w < nwv) {
                uint32_t pw = 0u, mw = 0u;
#pragma unroll
                for (int x = 0; x < 8; ++x)
                    if (x == w) { pw = part[x]; mw = mask[x]; }
                vwords[wbase + w] = quad_old ? ((vold[i] & ~mw) | pw) : pw;
            }
        }
    }
    // V scales (ASYM: and zero points): new tokens get theirs, empty slots zero; earlier tokens
    // keep theirs
    if (g == 0 && t >= told) {
        reinterpret_cast<ma_u16*>(sec + L.vscale_off)[t] = vs;
        if constexpr (ASYM) reinterpret_cast<ma_u16*>(sec + L.vzero_off)[t] = vz;
    }
}

// The ring update for sequence s, KV head kv: the newest min(n_new, R) keys into their slots.
// Called by the threads that gathered the call's first page (the only reader of the ring),
// after a barrier that follows their gather.
template <int D>
__device__ __forceinline__ void write_ring(const WriteArgs& a, int s, int kv, int p0, int tid,
                                           int nthreads) {
    constexpr int CPT = D / 16;
    uint16_t* ring_s = a.ring + (size_t)s * a.R * a.H * D;
    const int end = p0 + a.n_new;
    const int first = max(p0, end - a.R);
    const int chunks = (end - first) * 16;
    for (int i = tid; i < chunks; i += nthreads) {
        const int pp = first + i / 16, cc = (i % 16) * CPT;
        const uint16_t* src = a.k_new + (((size_t)s * a.n_new + (pp - p0)) * a.H + kv) * D + cc;
        uint16_t* dst = ring_s + ((size_t)(pp % a.R) * a.H + kv) * D + cc;
        if constexpr (CPT == 8)
            *reinterpret_cast<ma_uint4*>(dst) = *reinterpret_cast<const ma_uint4*>(src);
        else
            *reinterpret_cast<ma_uint2*>(dst) = *reinterpret_cast<const ma_uint2*>(src);
    }
}

}  // namespace kvq
