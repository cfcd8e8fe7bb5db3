// kv_canary.hip -- the KL canary over the FP16 key ring (gfx950).
//
// EchoKV, "Show the math": for each layer and each candidate width b in {2, 4, 8},
//   delta_b = KL( softmax(Q K_ref^T) || softmax(Q quant_b(K_ref)^T) ),
// summed over keys and averaged over the queries. K_ref is the per-layer FP16 ring of the
// newest keys ("The absolute canary"); "Do we store the whole cache in FP16?": only the ring
// is kept at full precision, and the canary measures it against short-lived quantized copies
// of its own keys at each candidate width.
// quant_b is the cache's own quantizer (one scale per page and channel), so complete pages in
// the ring get exactly the codes the cache stores.
//
// One workgroup per (sequence, KV head, width). The ring keys and the group's queries go to
// LDS once (16-byte loads); the workgroup takes the reference logits, then turns the keys in
// place into its width's temporary copy (one scale per (page group, channel), then one code per
// element) and takes the copy's logits with one wave
// per query head and one lane per key -- the keys sit in LDS rows padded to D + 1 floats, so the
// 64 lanes of a wave read 64 different banks while the query element is a broadcast. One wave
// per head then takes the log-sum-exp form of the divergence. Rows are stored with
// device-coherent stores; the last workgroup to take the ticket averages every row, in row order,
// from device-coherent loads (no cache flushes).
//
// EchoKV describes its canary quantizer as asymmetric per group, in the manner of KIVI; the ASYM
// instance builds the copies that way, over the same groups: zero point = the group minimum m, scale
// s = RU16((max - m) / (2^b - 1)), code = round-half-even((x - m) / s) in [0, 2^b - 1], value
// m + code * s. These decisions are taken in binary64, where they are exact for fp16 inputs.
// kv_canary_kl and kv_canary_kl_layers build the copies with the cache's own quantizer: the
// symmetric one, or the asymmetric one for a geometry in the asymmetric storage format.
#include "kvq_device.hpp"
#include "kvq_launch.hpp"

#include <mutex>

namespace kvq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 512;   // eight waves: one query head each for groups of up to 8
constexpr int kWavesC = kThreads / 64;
constexpr int kMaxRing = 128;   // largest ring the geometry check accepts
constexpr int kCtrStride = 64;  // uint32 words between the widths' counters (256 bytes)
constexpr int kRowBatch = 16;   // row loads a lane has in flight in the final average
constexpr uint32_t kNowhere = 0xffffff00u;   // a buffer offset past every range: reads zero

struct CanaryLayer {
    const uint16_t* ring;   // [batch][R][H][D]
    const uint16_t* q;      // [batch][Hq][D]
};

// NL: room for that many layers in the argument block (1 for a single layer's call, the
// multi-layer limit for a whole firing); layer l is blockIdx.z
template <int NL>
struct CanaryArgs {
    const int32_t* seq_len;
    float* kl_out;        // [L][3]
    float* kl_rows;       // optional, [L][batch][Hq][3]
    float* ws_rows;       // [L][batch][Hq][3]
    uint32_t* counter;    // [L][3][kCtrStride]: one ticket counter per (layer, width), each in its own line
    int H, Hq, grp, R, batch;
    float scale;
    CanaryLayer layer[NL];
};

// logits of every query head of the group against n keys held in LDS rows of stride D + 1
template <int D>
__device__ __forceinline__ void group_logits(const float* qs, const float* keys, int grp, int n,
                                             int R, float scale, int wave, int lane, float* out) {
    for (int hh = wave; hh < grp; hh += kWavesC) {
        const float* qrow = qs + hh * D;
        for (int k = lane; k < n; k += 64) {
            const float* krow = keys + k * (D + 1);
            float acc = 0.f;
#pragma unroll 16
            for (int c = 0; c < D; ++c) acc = fmaf(qrow[c], krow[c], acc);
            out[hh * R + k] = scale * acc;
        }
    }
}

template <int D, bool ASYM, int NL>
__global__ __launch_bounds__(kThreads) void canary_kernel(CanaryArgs<NL> a) {
    extern __shared__ float smem[];
    const int R = a.R;
    float* kref = smem;                          // [R][D + 1]; later the copy, in place
    float* qs = kref + R * (D + 1);              // [grp][D]
    float* sc = qs + kMaxGroup * D;              // [R / P + 1][D] scales of the copy
    float* zp = sc + (R / kPage + 1) * D;        // [R / P + 1][D] zero points (ASYM only)
    float* lref = zp + (ASYM ? (R / kPage + 1) * D : 0);   // [grp][R]
    float* lb = lref + kMaxGroup * R;            // [grp][R]
    __shared__ int last;

    const int ti = blockIdx.y;                   // width 2, 4, 8
    const int bits = 2 << ti;
    const int layer = NL == 1 ? 0 : (int)blockIdx.z;
    const uint16_t* ring = a.layer[layer].ring;
    const uint16_t* qv = a.layer[layer].q;
    const size_t row0 = (size_t)layer * a.batch * a.Hq;   // this layer's first row
    const int s = blockIdx.x / a.H, kv = blockIdx.x % a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = a.grp;

    // ---- every ring slot of this (sequence, KV head), 8 fp16 a load, requested together and
    // before the length is known (a slot's key index follows from the length afterwards), so
    // the keys arrive after one memory round trip; slots past the ring read zero
    constexpr int kChunks = D / 8;                              // 16-byte chunks per key
    constexpr int kLoads = kMaxRing * kChunks / kThreads;       // per thread
    const __amdgpu_buffer_rsrc_t ring_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(ring + (size_t)s * R * a.H * D), (short)0, R * a.H * D * 2, 0x00020000);
    u32x4 kbuf[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int i = tid + j * kThreads, slot = i / kChunks, c8 = (i % kChunks) * 8;
        kbuf[j] = __builtin_amdgcn_raw_buffer_load_b128(
            ring_rsrc, slot < R ? (uint32_t)(((slot * a.H + kv) * D + c8) * 2) : kNowhere, 0, 0);
    }
    const int N = max(a.seq_len[s], 0);
    const int n = min(N, R);
    const int first = N - n;
    // key index k = (slot - first) mod R holds position first + k
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int i = tid + j * kThreads, slot = i / kChunks, c8 = (i % kChunks) * 8;
        const int k = slot < R ? (slot - first % R + R) % R : R;
        if (k < n) {
            float* dst = kref + k * (D + 1) + c8;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dst[2 * e] = f16_val((uint16_t)(kbuf[j][e] & 0xffffu));
                dst[2 * e + 1] = f16_val((uint16_t)(kbuf[j][e] >> 16));
            }
        }
    }
    for (int i = tid; i < grp * (D / 8); i += kThreads) {
        const uint4 v = *reinterpret_cast<const ma_uint4*>(qv + ((size_t)s * a.Hq + kv * grp) * D + 8 * i);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            qs[8 * i + 2 * j] = f16_val((uint16_t)(w[j] & 0xffffu));
            qs[8 * i + 2 * j + 1] = f16_val((uint16_t)(w[j] >> 16));
        }
    }
    __syncthreads();

    // ---- the copy's scales: one per (page group, channel) over its ring-resident keys
    const int pfirst = first / kPage;
    const int npg = n > 0 ? (N - 1) / kPage - pfirst + 1 : 0;
    for (int i = tid; i < npg * D; i += kThreads) {
        const int pg = i / D, c = i - pg * D;
        const int k0 = max(first, (pfirst + pg) * kPage) - first;
        const int k1 = min(N, (pfirst + pg + 1) * kPage) - first;
        if constexpr (ASYM) {
            float mn = kref[k0 * (D + 1) + c], mx = mn;
            for (int k = k0 + 1; k < k1; ++k) {
                mn = fminf(mn, kref[k * (D + 1) + c]);
                mx = fmaxf(mx, kref[k * (D + 1) + c]);
            }
            sc[pg * D + c] = f16_val(asym_scale(mn, mx, bits));
            zp[pg * D + c] = mn;
        } else {
            float amax = 0.f;
            for (int k = k0; k < k1; ++k) amax = fmaxf(amax, fabsf(kref[k * (D + 1) + c]));
            sc[pg * D + c] = f16_val(group_scale(amax, bits));
        }
    }
    // reference logits meanwhile (they only read the keys and queries)
    group_logits<D>(qs, kref, grp, n, R, a.scale, wave, lane, lref);
    __syncthreads();
    // ---- the copy itself, in place of the keys: code * scale, one element a thread and step
    for (int i = tid; i < n * D; i += kThreads) {
        const int k = i / D, c = i - k * D;
        const int gi = ((first + k) / kPage - pfirst) * D + c;
        const float sf = sc[gi];
        const float x = kref[k * (D + 1) + c];
        if constexpr (ASYM) {
            const double m = (double)zp[gi];
            double q = sf != 0.f ? rint(((double)x - m) / (double)sf) : 0.0;
            q = fmin(fmax(q, 0.0), (double)((1 << bits) - 1));
            kref[k * (D + 1) + c] = (float)(m + q * (double)sf);
        } else {
            kref[k * (D + 1) + c] = sf != 0.f ? (float)quant_code(x, sf, bits) * sf : 0.f;
        }
    }
    __syncthreads();
    group_logits<D>(qs, kref, grp, n, R, a.scale, wave, lane, lb);
    __syncthreads();

    // ---- KL(P_ref || P_b) = sum_k P_k (l_k - m_k) - LSE(l) + LSE(m), one wave per head
    for (int hh = wave; hh < grp; hh += kWavesC) {
        float ml = -INFINITY, mm = -INFINITY;
        for (int k = lane; k < n; k += 64) {
            ml = fmaxf(ml, lref[hh * R + k]);
            mm = fmaxf(mm, lb[hh * R + k]);
        }
        ml = wave_max(ml);
        mm = wave_max(mm);
        float sl = 0.f, sm = 0.f;
        for (int k = lane; k < n; k += 64) {
            sl += expf(lref[hh * R + k] - ml);
            sm += expf(lb[hh * R + k] - mm);
        }
        sl = wave_sum(sl);
        sm = wave_sum(sm);
        const float lse_l = ml + logf(sl), lse_m = mm + logf(sm);
        float acc = 0.f;
        for (int k = lane; k < n; k += 64)
            acc += expf(lref[hh * R + k] - lse_l) * (lref[hh * R + k] - lb[hh * R + k]);
        acc = wave_sum(acc);
        const float kl = n > 0 ? fmaxf(acc - lse_l + lse_m, 0.f) : 0.f;
        if (lane == 0) {
            const size_t row = (row0 + (size_t)s * a.Hq + kv * grp + hh) * 3 + ti;
            __hip_atomic_store(a.ws_rows + row, kl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (a.kl_rows) a.kl_rows[row] = kl;
        }
    }

    // ---- the last workgroup of this width averages the width's rows, in row order (each lane
    // sums rows lane, lane + 64, ... in turn; then a fixed tree). Its coherent stores complete
    // before the ticket; the winner reads the rows with coherent loads issued after it, a batch
    // of kRowBatch per lane at a time. Each width has its own counter, on its own line.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    uint32_t* counter = a.counter + (layer * 3 + ti) * kCtrStride;
    if (tid == 0)
        last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               gridDim.x - 1;
    __syncthreads();
    if (!last) return;
    constexpr int kSc1 = 16;                                    // device-coherent load
    const __amdgpu_buffer_rsrc_t rows_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.ws_rows + row0 * 3, (short)0, 0x7fffffff, 0x00020000);
    if (wave == 0) {
        const int rows = a.batch * a.Hq;
        float acc = 0.f;
        for (int r0 = 0; r0 < rows; r0 += 64 * kRowBatch) {
            float v[kRowBatch];
#pragma unroll
            for (int j = 0; j < kRowBatch; ++j) {
                const int r = r0 + 64 * j + lane;
                v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                     rows_rsrc, r < rows ? (uint32_t)((r * 3 + ti) * 4) : kNowhere, 0, kSc1));
            }
#pragma unroll
            for (int j = 0; j < kRowBatch; ++j) acc += v[j];
        }
        acc = wave_sum(acc);
        if (lane == 0) a.kl_out[layer * 3 + ti] = acc / (float)rows;
    }
    if (tid == 0)
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// Workspace: the ticket counters of `counter_layers` layers (three lines each), then the rows of
// the call. The counters stay at the same place whatever the call's batch and layer count, so a
// workspace left at zero by one call is ready for the next.
size_t canary_workspace_bytes(const kv_geometry& g, int counter_layers, int num_layers, int batch) {
    return (size_t)counter_layers * 3 * kCtrStride * 4 +
           (size_t)num_layers * batch * g.num_q_heads * 3 * sizeof(float);
}

namespace {

size_t canary_lds_bytes(int R, int D, bool asym) {
    return sizeof(float) * ((size_t)R * (D + 1) + kMaxGroup * D +
                            (asym ? 2 : 1) * ((size_t)R / kPage + 1) * D +
                            2 * kMaxGroup * (size_t)R);
}

template <int D, bool ASYM, int NL>
hipError_t launch_one(const CanaryArgs<NL>& a, dim3 grid, size_t lds, hipStream_t stream) {
    // the LDS footprint exceeds the 64 KiB default for rings of 64 keys at D = 128: raise the
    // limit to the largest footprint any supported ring needs, once per process and kernel (so
    // that launches stay plain stream work, e.g. under graph capture)
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&canary_kernel<D, ASYM, NL>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)canary_lds_bytes(kMaxRing, D, ASYM));
    });
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((canary_kernel<D, ASYM, NL>), grid, dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

template <int NL>
void fill_common(CanaryArgs<NL>& a, const kv_geometry& g, const int32_t* seq_len, int counter_layers,
                 int batch, float softmax_scale, float* kl_out, float* kl_rows, void* workspace) {
    a.seq_len = seq_len;
    a.kl_out = kl_out;
    a.kl_rows = kl_rows;
    a.counter = static_cast<uint32_t*>(workspace);
    a.ws_rows = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                         (size_t)counter_layers * 3 * kCtrStride * 4);
    a.H = g.num_kv_heads;
    a.Hq = g.num_q_heads;
    a.grp = g.num_q_heads / g.num_kv_heads;
    a.R = g.ring_size;
    a.batch = batch;
    a.scale = softmax_scale;
}

}  // namespace

hipError_t launch_canary(const kv_geometry& g, const uint16_t* ring, const int32_t* seq_len,
                         int batch, const uint16_t* q, float softmax_scale, bool asymmetric,
                         float* kl_out, float* kl_rows, void* workspace, hipStream_t stream) {
    CanaryArgs<1> a;
    fill_common(a, g, seq_len, 1, batch, softmax_scale, kl_out, kl_rows, workspace);
    a.layer[0] = CanaryLayer{ring, q};
    const int D = g.head_dim;
    const size_t lds = canary_lds_bytes(a.R, D, asymmetric);
    dim3 grid((unsigned)(batch * g.num_kv_heads), 3u);
    if (D == 128)
        return asymmetric ? launch_one<128, true>(a, grid, lds, stream)
                          : launch_one<128, false>(a, grid, lds, stream);
    return asymmetric ? launch_one<64, true>(a, grid, lds, stream)
                      : launch_one<64, false>(a, grid, lds, stream);
}

hipError_t launch_canary_layers(const kv_geometry& g, int num_layers,
                                const uint16_t* const* rings, const int32_t* seq_len, int batch,
                                const uint16_t* const* q, float softmax_scale, float* kl_out,
                                float* kl_rows, void* workspace, hipStream_t stream) {
    CanaryArgs<kMaxCanaryLayers> a;
    fill_common(a, g, seq_len, canary_counter_layers(g), batch, softmax_scale, kl_out, kl_rows,
                workspace);
    for (int l = 0; l < kMaxCanaryLayers; ++l)
        a.layer[l] = l < num_layers ? CanaryLayer{rings[l], q[l]} : CanaryLayer{nullptr, nullptr};
    const int D = g.head_dim;
    const bool asym = g.asymmetric != 0;          // the cache's own quantizer
    const size_t lds = canary_lds_bytes(a.R, D, asym);
    dim3 grid((unsigned)(batch * g.num_kv_heads), 3u, (unsigned)num_layers);
    if (D == 128) return asym ? launch_one<128, true>(a, grid, lds, stream)
                              : launch_one<128, false>(a, grid, lds, stream);
    return asym ? launch_one<64, true>(a, grid, lds, stream) : launch_one<64, false>(a, grid, lds, stream);
}

}  // namespace kvq
