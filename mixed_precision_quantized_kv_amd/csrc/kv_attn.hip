// kv_attn.hip -- fused dequantize + grouped-query split-K decode attention (gfx950).
//
// EchoKV, "What happens to old blocks...": paged attention reads every block at the width it
// was stored with, so one layer's cache may mix INT2 / INT4 / INT8 pages. Behavior-Guided
// KV-Cache Quantization, "Storage savings": GQA head mapping (query head h reads KV head
// h / group). KV-Kaizen summary, "Background": decoding reads the entire cache per token, so
// the kernel is built to stream the packed pages at HBM rate.
//
// Work decomposition. A workgroup of NW waves owns one (sequence, KV head, split) -- a run of
// `pps` pages; its waves take page pairs round-robin. Per page pair a wave computes, on MFMA:
//   S^T[t][h] = sum_c Kcode[t][c] * q'[h][c],   q' = q * Kscale(page)   (16x16x32 f16, 16 tokens)
//   o^T[c][h] += sum_t Vcode[t][c] * p'[h][t],   p' = p * Vscale(t)     (16x16x32 f16, 32 tokens)
// Codes are exact small integers in fp16 (built with a shift, a mask and one packed add), the
// per-channel K scales are folded into q once per page, the per-token V scales into the softmax
// weights. Computing S and o transposed puts head h in lane h%16 of both products, so the
// softmax output is the PV operand in place and the rescale by exp(m_old - m_new) is lane-local.
// Query heads beyond the group (MFMA rows >= group) are zero padding.
// Waves merge in LDS; splits merge through a workspace: the last workgroup of a (sequence, KV
// head) to finish -- found with an atomic ticket -- combines the partials in split order, so
// results do not depend on scheduling. Split index s and group index g map to blockIdx
// s * groups + g, which keeps all splits of a group on one XCD when groups % 8 == 0.
#include "kvq_device.hpp"
#include "kvq_launch.hpp"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSplits = 256;

struct AttnArgs {
    PoolPtrs pools;
    const uint32_t* bt;
    const int32_t* ctx_len;
    const uint16_t* q;
    float* out;
    uint32_t* counters;   // [groups]
    float2* ws_ml;        // [groups][splits][group] (max, sum) in log2 units
    float* ws_o;          // [groups][splits][group][D]
    int max_pages;
    int H;                // KV heads
    int Hq;
    int grp;              // query heads per KV head
    int groups;           // batch * H
    int splits;
    int pps;              // pages per split
    float scale_log2;     // softmax_scale * log2(e)
};

// raw bytes of one page, as this lane needs them
struct PageRaw {
    uint32_t k[8];   // this lane's K code chunk (token lane%16, channels of lane group)
    uint32_t v[8];   // this lane's V code chunk (token quad lane/16, channels of lane%16)
    uint32_t ks;     // two K scales (channels 2*lane, 2*lane+1)
    uint32_t vs[2];  // four V scales (tokens 4*(lane/16) .. +3)
    int bits;        // 0 = no page
    int ntok;        // valid tokens in the page
};

template <int NBYTES>
__device__ inline void load_chunk(const uint8_t* p, uint32_t* dst) {
    if constexpr (NBYTES == 4) {
        dst[0] = *reinterpret_cast<const uint32_t*>(p);
    } else if constexpr (NBYTES == 8) {
        uint2 a = *reinterpret_cast<const uint2*>(p);
        dst[0] = a.x; dst[1] = a.y;
    } else if constexpr (NBYTES == 16) {
        uint4 a = *reinterpret_cast<const uint4*>(p);
        dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
    } else {
        static_assert(NBYTES == 32, "chunk size");
        uint4 a = *reinterpret_cast<const uint4*>(p);
        uint4 b = *reinterpret_cast<const uint4*>(p + 16);
        dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
        dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
    }
}

template <int D, int BITS>
__device__ inline void load_page_bits(const uint8_t* sec, int lane, PageRaw& r) {
    constexpr Section L = {(uint32_t)(kPage * D * BITS / 8), (uint32_t)(kPage * D * BITS / 8),
                           (uint32_t)(kPage * D * BITS / 8 + 2 * D),
                           (uint32_t)(2 * kPage * D * BITS / 8 + 2 * D),
                           (uint32_t)(2 * kPage * D * BITS / 8 + 2 * D + 2 * kPage)};
    constexpr int CH = D * BITS / 32;               // bytes of one lane chunk
    const int t = lane & 15, G = lane >> 4;
    load_chunk<CH>(sec + t * (D * BITS / 8) + G * CH, r.k);
    load_chunk<CH>(sec + L.vcode_off + (G * D + t * (D / 16)) * BITS / 2, r.v);
    r.ks = lane < D / 2 ? *reinterpret_cast<const uint32_t*>(sec + L.kscale_off + 4 * lane) : 0u;
    uint2 vs = *reinterpret_cast<const uint2*>(sec + L.vscale_off + 8 * G);
    r.vs[0] = vs.x; r.vs[1] = vs.y;
}

template <int D>
__device__ inline void load_page(const AttnArgs& a, int s, int kv, int page, int ctx, int lane,
                                 PageRaw& r) {
    const uint32_t handle = a.bt[(size_t)s * a.max_pages + page];
    const int tier = (int)(handle >> 30);
    const uint32_t idx = handle & 0x3fffffffu;
    r.bits = bits_of_tier(tier);
    r.ntok = min(kPage, ctx - page * kPage);
    const uint32_t sb = section_layout(D, r.bits).bytes;
    const uint8_t* sec = a.pools.base[tier] + ((size_t)idx * a.H + kv) * sb;
    if (tier == 0) load_page_bits<D, 2>(sec, lane, r);
    else if (tier == 1) load_page_bits<D, 4>(sec, lane, r);
    else load_page_bits<D, 8>(sec, lane, r);
}

// one packed word of codes -> consecutive fp16 pairs holding the signed codes
__device__ inline uint32_t hadd_bias(uint32_t u, float bias) {
    half2v x = __builtin_bit_cast(half2v, u);
    half2v b = {(_Float16)bias, (_Float16)bias};
    return __builtin_bit_cast(uint32_t, x + b);
}

// unpack a lane chunk (D*BITS/32 bytes) into D/8 dwords of fp16 pairs, in code order
template <int D>
__device__ inline void unpack_chunk(const uint32_t* w, int bits, uint32_t* out) {
    if (bits == 2) {
#pragma unroll
        for (int i = 0; i < D / 64; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                out[i * 8 + j] = hadd_bias(((w[i] >> (2 * j)) & 0x00030003u) | 0x64006400u, -1026.0f);
    } else if (bits == 4) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                out[i * 4 + j] = hadd_bias(((w[i] >> (4 * j)) & 0x000F000Fu) | 0x64006400u, -1032.0f);
    } else {
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
            out[2 * i] = hadd_bias(__builtin_amdgcn_perm(0x64646464u, w[i], 0x04020400u), -1152.0f);
            out[2 * i + 1] = hadd_bias(__builtin_amdgcn_perm(0x64646464u, w[i], 0x04030401u), -1152.0f);
        }
    }
}

__device__ inline half8 make_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    uint4 u = {a, b, c, d};
    return __builtin_bit_cast(half8, u);
}

template <int D>
struct WaveState {
    float4v o[D / 16];   // o^T tile per channel chunk: lane (h, G) element r -> channel G*D/4 + r*D/16 + k
    float m;             // running max (log2 units) of head lane%16
    float l;             // this lane's share of the running sum
};

// QK for one page: returns S^T for tokens 4G..4G+3 of head lane%16 (log2 units, masked)
template <int D>
__device__ inline float4v page_logits(const PageRaw& r, const uint32_t* qf, uint32_t* lds_ks,
                                      int lane, float scale_log2) {
    const int G = lane >> 4;
    // stage the page's K scales through LDS: each lane needs the D/4 scales of its lane group
    lds_ks[lane] = r.ks;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t ks[D / 8];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        uint4 v = *reinterpret_cast<const uint4*>(lds_ks + G * (D / 8) + 4 * i);
        ks[4 * i] = v.x; ks[4 * i + 1] = v.y; ks[4 * i + 2] = v.z; ks[4 * i + 3] = v.w;
    }
    uint32_t kf[D / 8];
    unpack_chunk<D>(r.k, r.bits, kf);
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    if (r.bits == 2) {
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
    float4v lg;
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[i] = (4 * G + i < r.ntok) ? acc[i] * scale_log2 : -INFINITY;
    return lg;
}

template <int D>
__device__ inline void process_pair(const PageRaw& A, const PageRaw& B, const uint32_t* qf,
                                    uint32_t* lds_ks, int lane, float scale_log2, WaveState<D>& st) {
    const int G = lane >> 4;
    float4v la = page_logits<D>(A, qf, lds_ks, lane, scale_log2);
    float4v lb = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (B.bits) lb = page_logits<D>(B, qf, lds_ks + 64, lane, scale_log2);

    // online softmax over the pair's 32 tokens, per head (lanes h, h+16, h+32, h+48)
    float mx = fmaxf(fmaxf(fmaxf(la[0], la[1]), fmaxf(la[2], la[3])),
                     fmaxf(fmaxf(lb[0], lb[1]), fmaxf(lb[2], lb[3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(st.m, mx);            // finite: page A holds >= 1 valid token
    const float alpha = exp2f(st.m - m_new);        // 0 on the first pair (m = -inf)
    st.m = m_new;
    float pa[4], pb[4], sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pa[i] = exp2f(la[i] - m_new);
        pb[i] = exp2f(lb[i] - m_new);
        sum += pa[i] + pb[i];
    }
    st.l = st.l * alpha + sum;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) st.o[k] *= alpha;

    // p' = p * V scale of the token; masked tokens get exactly 0 (their scale may be anything)
    auto vscale = [](const PageRaw& r, int i) {
        const uint32_t w = r.vs[i >> 1];
        return f16_val((uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu)));
    };
    float wa[4], wb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        wa[i] = (4 * G + i < A.ntok) ? pa[i] * vscale(A, i) : 0.f;
        wb[i] = (B.bits && 4 * G + i < B.ntok) ? pb[i] * vscale(B, i) : 0.f;
    }
    const half8 pf = {(_Float16)wa[0], (_Float16)wa[1], (_Float16)wa[2], (_Float16)wa[3],
                      (_Float16)wb[0], (_Float16)wb[1], (_Float16)wb[2], (_Float16)wb[3]};

    uint32_t va[D / 8], vb[D / 8];
    unpack_chunk<D>(A.v, A.bits, va);
    if (B.bits) {
        unpack_chunk<D>(B.v, B.bits, vb);
    } else {
#pragma unroll
        for (int i = 0; i < D / 8; ++i) vb[i] = 0u;
    }
#pragma unroll
    for (int k = 0; k < D / 16; ++k)
        st.o[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            make_half8(va[2 * k], va[2 * k + 1], vb[2 * k], vb[2 * k + 1]), pf, st.o[k], 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void decode_attn_kernel(AttnArgs a) {
    __shared__ uint32_t lds_ks[kWaves][2][64];
    __shared__ float lds_o[kWaves][kMaxGroup][D];
    __shared__ float lds_m[kWaves][kMaxGroup];
    __shared__ float lds_l[kWaves][kMaxGroup];
    __shared__ float lds_w[kMaxSplits][kMaxGroup];   // split weights in the final merge
    __shared__ float lds_L[kMaxGroup];
    __shared__ int lds_last;

    const int split = blockIdx.x / a.groups, group = blockIdx.x % a.groups;
    const int s = group / a.H, kv = group % a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = a.grp;
    const int ctx = a.ctx_len[s];
    const int npages = (ctx + kPage - 1) / kPage;
    const int nsplit = (npages + a.pps - 1) / a.pps;

    if (split >= nsplit) {
        if (split == 0 && ctx <= 0)            // no keys: the rows are zero
            for (int i = tid; i < grp * D; i += kWaves * 64)
                a.out[((size_t)s * a.Hq + kv * grp) * D + i] = 0.f;
        return;
    }
    const int pbeg = split * a.pps;
    const int pend = min(pbeg + a.pps, npages);
    const int npairs = (pend - pbeg + 1) / 2;

    // q fragment: lane (h, G) holds q[h][G*D/4 .. +D/4) as fp16 pairs (zero for h >= grp)
    const int h = lane & 15, G = lane >> 4;
    uint32_t qf[D / 8];
    {
        const uint32_t* qp = reinterpret_cast<const uint32_t*>(
            a.q + ((size_t)s * a.Hq + kv * grp + min(h, grp - 1)) * D + G * (D / 4));
#pragma unroll
        for (int i = 0; i < D / 8; ++i) qf[i] = h < grp ? qp[i] : 0u;
    }

    WaveState<D> st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) st.o[k] = float4v{0.f, 0.f, 0.f, 0.f};

    uint32_t* ks_slot = &lds_ks[wave][0][0];
    PageRaw bufA0, bufA1, bufB0, bufB1;
    auto load_pair = [&](int pair, PageRaw& x, PageRaw& y) {
        const int pa = pbeg + 2 * pair;
        load_page<D>(a, s, kv, pa, ctx, lane, x);
        if (pa + 1 < pend) load_page<D>(a, s, kv, pa + 1, ctx, lane, y);
        else y.bits = 0, y.ntok = 0;
    };
    int pair = wave;
    if (pair < npairs) load_pair(pair, bufA0, bufA1);
    while (pair < npairs) {
        int next = pair + kWaves;
        if (next < npairs) load_pair(next, bufB0, bufB1);
        process_pair<D>(bufA0, bufA1, qf, ks_slot, lane, a.scale_log2, st);
        pair = next;
        if (pair >= npairs) break;
        next = pair + kWaves;
        if (next < npairs) load_pair(next, bufA0, bufA1);
        process_pair<D>(bufB0, bufB1, qf, ks_slot, lane, a.scale_log2, st);
        pair = next;
    }

    // ---- this wave's partial -> LDS
    float lsum = st.l;
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (h < grp) {
        if (G == 0) {
            lds_m[wave][h] = st.m;
            lds_l[wave][h] = lsum;
        }
#pragma unroll
        for (int k = 0; k < D / 16; ++k)
#pragma unroll
            for (int r = 0; r < 4; ++r) lds_o[wave][h][G * (D / 4) + r * (D / 16) + k] = st.o[k][r];
    }
    __syncthreads();

    // ---- merge the waves (fixed order) into this split's partial
    const bool single = nsplit == 1;
    const size_t part = (size_t)group * a.splits + split;
    for (int i = tid; i < grp * D; i += kWaves * 64) {
        const int hh = i / D, c = i - hh * D;
        float M = -INFINITY;
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_m[w][hh]);
        float acc = 0.f, L = 0.f;
        for (int w = 0; w < kWaves; ++w) {
            const float mw = lds_m[w][hh];
            const float e = mw == -INFINITY ? 0.f : exp2f(mw - M);
            acc += e * lds_o[w][hh][c];
            L += e * lds_l[w][hh];
        }
        if (single) {
            a.out[((size_t)s * a.Hq + kv * grp + hh) * D + c] = L > 0.f ? acc / L : 0.f;
        } else {
            a.ws_o[part * grp * D + i] = acc;
            if (c == 0) a.ws_ml[part * grp + hh] = make_float2(M, L);
        }
    }
    if (single) return;

    // ---- the last split of this (sequence, KV head) to finish merges all partials in order
    __threadfence();
    __syncthreads();
    if (tid == 0) lds_last = atomicAdd(&a.counters[group], 1u) == (unsigned)(nsplit - 1);
    __syncthreads();
    if (!lds_last) return;
    __threadfence();
    const float2* ml = a.ws_ml + (size_t)group * a.splits * grp;
    if (tid < grp) {
        float M = -INFINITY;
        for (int k = 0; k < nsplit; ++k) M = fmaxf(M, ml[k * grp + tid].x);
        float L = 0.f;
        for (int k = 0; k < nsplit; ++k) {
            const float2 v = ml[k * grp + tid];
            const float e = v.x == -INFINITY ? 0.f : exp2f(v.x - M);
            lds_w[k][tid] = e;
            L += e * v.y;
        }
        lds_L[tid] = L;
    }
    __syncthreads();
    const float* po = a.ws_o + (size_t)group * a.splits * grp * D;
    for (int i = tid; i < grp * D; i += kWaves * 64) {
        const int hh = i / D;
        float acc = 0.f;
        for (int k = 0; k < nsplit; ++k) acc += lds_w[k][hh] * po[(size_t)k * grp * D + i];
        const float L = lds_L[hh];
        a.out[((size_t)s * a.Hq + kv * grp) * D + i] = L > 0.f ? acc / L : 0.f;
    }
    if (tid == 0) a.counters[group] = 0u;   // ready for the next call
}

}  // namespace

size_t decode_workspace_bytes(const kv_geometry& g, int batch, int splits) {
    const size_t groups = (size_t)batch * g.num_kv_heads;
    const size_t grp = (size_t)(g.num_q_heads / g.num_kv_heads);
    size_t bytes = 256;                                           // counters, padded
    bytes += ((groups * 4 + 255) / 256) * 256;
    bytes += ((groups * splits * grp * sizeof(float2) + 255) / 256) * 256;
    bytes += groups * splits * grp * g.head_dim * sizeof(float);
    return bytes;
}

hipError_t launch_decode_attn(const kv_geometry& g, PoolPtrs pools, const uint32_t* bt,
                              const int32_t* ctx_len, int batch, int splits, int pages_per_split,
                              const uint16_t* q, float softmax_scale, float* out,
                              void* workspace, hipStream_t stream) {
    AttnArgs a;
    a.pools = pools;
    a.bt = bt;
    a.ctx_len = ctx_len;
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
    size_t off = ((groups * 4 + 255) / 256) * 256 + 256;
    a.ws_ml = reinterpret_cast<float2*>(ws + off);
    off += ((groups * splits * a.grp * sizeof(float2) + 255) / 256) * 256;
    a.ws_o = reinterpret_cast<float*>(ws + off);
    dim3 grid((unsigned)(splits * a.groups));
    if (g.head_dim == 128)
        hipLaunchKernelGGL(decode_attn_kernel<128>, grid, dim3(kWaves * 64), 0, stream, a);
    else
        hipLaunchKernelGGL(decode_attn_kernel<64>, grid, dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq
