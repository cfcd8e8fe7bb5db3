// kv_write.hip -- quantize-on-write for one layer (gfx950).
//
// EchoKV, "How EchoKV works": the step's key enters the per-layer FP16 ring before it is
// quantized into the paged cache. Behavior-Guided KV-Cache Quantization, "K/V Role-Aware
// Low-Bit Quantization": keys get one scale per channel (over the page's tokens), values one
// scale per token (over its channels); "Online inference": pack and store.
//
// One workgroup per (page touched, KV head, sequence). The workgroup of the first page touched
// is the only reader of the ring (the page's earlier keys live there), so it also performs the
// ring update after a barrier: no other workgroup reads the slots it overwrites.
#include "kvq_device.hpp"
#include "kvq_launch.hpp"

namespace kvq {
namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void quant_write_kernel(
    PoolPtrs pools, const uint32_t* __restrict__ bt, int max_pages, const int32_t* __restrict__ pos,
    int n_new, int H, int R, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ ring) {
    constexpr int P = kPage;
    __shared__ float keys[P][D];          // the page's present keys
    __shared__ float vals[P][D];          // the new value vectors of this page
    __shared__ int8_t kq[P][D];           // K codes
    __shared__ int8_t vq[P][D];           // V codes of new tokens
    __shared__ uint16_t kscale[D];
    __shared__ uint16_t vscale[P];        // final V scale of every slot
    __shared__ uint32_t vold[P * D * 8 / 32];   // old V code words (only the first page)

    const int j = blockIdx.x, kv = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x;
    const int p0 = pos[s];
    const int end = p0 + n_new;
    const int page = p0 / P + j;
    const int lo = page * P;
    if (lo >= end) return;
    const int hi = min(lo + P, end);
    const int nk = hi - lo;                       // present tokens in the page after the write
    const int told = max(0, p0 - lo);             // tokens cached before this call

    const uint32_t handle = bt[(size_t)s * max_pages + page];
    const int tier = (int)(handle >> 30);
    const int bits = bits_of_tier(tier);
    const Section L = section_layout(D, bits);
    uint8_t* sec = pools.base[tier] + (size_t)(handle & 0x3fffffffu) * H * L.bytes +
                   (size_t)kv * L.bytes;
    const int qoff = 1 << (bits - 1);

    // ---- gather: earlier keys of the page from the ring, new keys and values from the input
    uint16_t* ring_s = ring + (size_t)s * R * H * D;
    for (int i = tid; i < nk * D; i += kThreads) {
        const int t = i / D, c = i - t * D, p = lo + t;
        uint16_t h = p < p0 ? ring_s[((size_t)(p % R) * H + kv) * D + c]
                            : k_new[(((size_t)s * n_new + (p - p0)) * H + kv) * D + c];
        keys[t][c] = f16_val(h);
        if (p >= p0)
            vals[t][c] = f16_val(v_new[(((size_t)s * n_new + (p - p0)) * H + kv) * D + c]);
    }
    const int vwords = (int)(L.code_bytes / 4);
    if (told > 0) {
        const uint32_t* vw = reinterpret_cast<const uint32_t*>(sec + L.vcode_off);
        for (int w = tid; w < vwords; w += kThreads) vold[w] = vw[w];
        if (tid < P)
            vscale[tid] = tid < told ? reinterpret_cast<const uint16_t*>(sec + L.vscale_off)[tid] : 0;
    } else if (tid < P) {
        vscale[tid] = 0;
    }
    __syncthreads();

    // ---- K: one scale per channel over the present tokens, zero code for empty slots
    for (int c = tid; c < D; c += kThreads) {
        float a = 0.0f;
        for (int t = 0; t < nk; ++t) a = fmaxf(a, fabsf(keys[t][c]));
        const uint16_t sb = group_scale(a, bits);
        kscale[c] = sb;
        const float sf = f16_val(sb);
        for (int t = 0; t < P; ++t) kq[t][c] = (int8_t)((t < nk && sb) ? quant_code(keys[t][c], sf, bits) : 0);
    }
    // ---- V: one scale per new token over its D channels (a wave per token)
    const int wave = tid / 64, lane = tid % 64;
    for (int t = told + wave; t < nk; t += kThreads / 64) {
        float a = 0.0f;
        for (int c = lane; c < D; c += 64) a = fmaxf(a, fabsf(vals[t][c]));
        a = wave_max(a);
        const uint16_t sb = group_scale(a, bits);
        const float sf = f16_val(sb);
        for (int c = lane; c < D; c += 64) vq[t][c] = (int8_t)(sb ? quant_code(vals[t][c], sf, bits) : 0);
        if (lane == 0) vscale[t] = sb;
    }
    __syncthreads();

    // ---- pack and store the whole section
    const int per_word = 32 / bits;
    const uint32_t fmask = (1u << bits) - 1u;
    uint32_t* kw = reinterpret_cast<uint32_t*>(sec);
    for (int w = tid; w < vwords; w += kThreads) {
        uint32_t word = 0;
        for (int k = 0; k < per_word; ++k) {
            const int i = w * per_word + k;
            const int t = i / D, c = i - t * D;
            word |= (uint32_t)(kq[t][c] + qoff) << field_bit(k, bits);
        }
        kw[w] = word;
    }
    uint32_t* ksw = reinterpret_cast<uint32_t*>(sec + L.kscale_off);
    for (int w = tid; w < D / 2; w += kThreads)
        ksw[w] = (uint32_t)kscale[2 * w] | ((uint32_t)kscale[2 * w + 1] << 16);
    uint32_t* vw = reinterpret_cast<uint32_t*>(sec + L.vcode_off);
    for (int w = tid; w < vwords; w += kThreads) {
        uint32_t word = 0;
        for (int k = 0; k < per_word; ++k) {
            const int i = w * per_word + k;
            const int quad = i / (4 * D), c = (i / 4) % D, t = 4 * quad + (i & 3);
            const int fb = field_bit(k, bits);
            uint32_t u;
            if (t < told) u = (vold[w] >> fb) & fmask;
            else if (t < nk) u = (uint32_t)(vq[t][c] + qoff);
            else u = (uint32_t)qoff;
            word |= u << fb;
        }
        vw[w] = word;
    }
    uint32_t* vsw = reinterpret_cast<uint32_t*>(sec + L.vscale_off);
    for (int w = tid; w < P / 2; w += kThreads) {
        const uint16_t a = 2 * w < nk ? vscale[2 * w] : 0;
        const uint16_t b = 2 * w + 1 < nk ? vscale[2 * w + 1] : 0;
        vsw[w] = (uint32_t)a | ((uint32_t)b << 16);
    }

    // ---- ring: the newest min(n_new, R) keys of this KV head (first page's workgroup only;
    // its ring reads above completed before the barrier)
    if (j == 0) {
        const int first = max(p0, end - R);
        for (int i = tid; i < (end - first) * D; i += kThreads) {
            const int p = first + i / D, c = i % D;
            ring_s[((size_t)(p % R) * H + kv) * D + c] =
                k_new[(((size_t)s * n_new + (p - p0)) * H + kv) * D + c];
        }
    }
}

}  // namespace

hipError_t launch_quant_write(const kv_geometry& g, PoolPtrs pools, const uint32_t* bt,
                              const int32_t* pos, int batch, int n_new, const uint16_t* k_new,
                              const uint16_t* v_new, uint16_t* ring, hipStream_t stream) {
    // pages touched per sequence: at most ceil(n_new / P) + 1 (the first may be partial)
    dim3 grid((unsigned)((n_new + kPage - 1) / kPage + 1), (unsigned)g.num_kv_heads, (unsigned)batch);
    if (g.head_dim == 128)
        hipLaunchKernelGGL(quant_write_kernel<128>, grid, dim3(kThreads), 0, stream, pools, bt,
                           g.max_pages_per_seq, pos, n_new, g.num_kv_heads, g.ring_size, k_new,
                           v_new, ring);
    else
        hipLaunchKernelGGL(quant_write_kernel<64>, grid, dim3(kThreads), 0, stream, pools, bt,
                           g.max_pages_per_seq, pos, n_new, g.num_kv_heads, g.ring_size, k_new,
                           v_new, ring);
    return hipGetLastError();
}

}  // namespace kvq
