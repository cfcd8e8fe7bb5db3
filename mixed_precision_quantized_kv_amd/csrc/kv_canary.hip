// kv_canary.hip -- the KL canary over the FP16 key ring (gfx950).
//
// EchoKV, "Show the math": for each layer and each candidate width b in {2, 4, 8},
//   delta_b = KL( softmax(Q K_ref^T) || softmax(Q quant_b(K_ref)^T) ),
// summed over keys and averaged over the queries. K_ref is the per-layer FP16 ring of the
// newest keys ("The absolute canary"); "Do we store the whole cache in FP16?": the canary
// compares the ring against a temporary INT2/INT4/INT8 copy of those same keys.
// quant_b is the cache's own quantizer (one scale per page and channel), so complete pages in
// the ring get exactly the codes the cache stores.
//
// One workgroup per (sequence, KV head): ring keys -> LDS, temporary copies built in LDS, one
// thread per (head, key) dot product, one wave per head for the log-sum-exp reductions. The
// mean over all rows is taken by the last workgroup to finish (atomic ticket), in row order.
#include "kvq_device.hpp"
#include "kvq_launch.hpp"

namespace kvq {
namespace {

constexpr int kThreads = 256;

struct CanaryArgs {
    const uint16_t* ring;
    const int32_t* seq_len;
    const uint16_t* q;
    float* kl_out;
    float* kl_rows;       // optional
    float* ws_rows;       // [batch][Hq][3]
    uint32_t* counter;
    int H, Hq, grp, R, batch;
    float scale;
};

// dot product of a query row and a key row held in LDS (fixed order)
template <int D>
__device__ inline float row_dot(const float* qrow, const float* krow) {
    float acc = 0.f;
#pragma unroll 8
    for (int c = 0; c < D; ++c) acc = fmaf(qrow[c], krow[c], acc);
    return acc;
}

template <int D>
__global__ __launch_bounds__(kThreads) void canary_kernel(CanaryArgs a) {
    extern __shared__ float smem[];
    const int R = a.R;
    float* kref = smem;                      // [R][D]
    float* kb = kref + R * D;                // [R][D] temporary copy
    float* qh = kb + R * D;                  // [grp][D]
    float* lref = qh + kMaxGroup * D;        // [grp][R]
    float* lb = lref + kMaxGroup * R;        // [grp][R]
    __shared__ int last;

    const int s = blockIdx.x / a.H, kv = blockIdx.x % a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = a.grp;
    const int N = max(a.seq_len[s], 0);
    const int n = min(N, R);
    const int first = N - n;

    for (int i = tid; i < n * D; i += kThreads) {
        const int k = i / D, c = i - k * D;
        kref[i] = f16_val(a.ring[(((size_t)s * R + (first + k) % R) * a.H + kv) * D + c]);
    }
    for (int i = tid; i < grp * D; i += kThreads)
        qh[i] = f16_val(a.q[((size_t)s * a.Hq + kv * grp) * D + i]);
    __syncthreads();
    for (int i = tid; i < grp * n; i += kThreads) {
        const int hh = i / n, k = i - hh * n;
        lref[hh * R + k] = a.scale * row_dot<D>(qh + hh * D, kref + k * D);
    }

    const int pfirst = first / kPage;
    const int npg = n > 0 ? (N - 1) / kPage - pfirst + 1 : 0;
    for (int ti = 0; ti < 3; ++ti) {
        const int bits = 2 << ti;
        // temporary b-bit copy: one scale per (page group, channel) over its ring-resident keys
        for (int i = tid; i < npg * D; i += kThreads) {
            const int pg = i / D, c = i - pg * D;
            const int k0 = max(first, (pfirst + pg) * kPage) - first;
            const int k1 = min(N, (pfirst + pg + 1) * kPage) - first;
            float amax = 0.f;
            for (int k = k0; k < k1; ++k) amax = fmaxf(amax, fabsf(kref[k * D + c]));
            const uint16_t sb = group_scale(amax, bits);
            const float sf = f16_val(sb);
            for (int k = k0; k < k1; ++k)
                kb[k * D + c] = sb ? (float)quant_code(kref[k * D + c], sf, bits) * sf : 0.f;
        }
        __syncthreads();
        for (int i = tid; i < grp * n; i += kThreads) {
            const int hh = i / n, k = i - hh * n;
            lb[hh * R + k] = a.scale * row_dot<D>(qh + hh * D, kb + k * D);
        }
        __syncthreads();
        // KL(P_ref || P_b) = sum_k P_k (l_k - m_k) - LSE(l) + LSE(m), one wave per head
        for (int hh = wave; hh < grp; hh += kThreads / 64) {
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
                const size_t row = ((size_t)s * a.Hq + kv * grp + hh) * 3 + ti;
                a.ws_rows[row] = kl;
                if (a.kl_rows) a.kl_rows[row] = kl;
            }
        }
        __syncthreads();
    }

    // the last workgroup averages all rows, in row order
    __threadfence();
    __syncthreads();
    if (tid == 0) last = atomicAdd(a.counter, 1u) == (unsigned)(gridDim.x - 1);
    __syncthreads();
    if (!last) return;
    __threadfence();
    if (wave < 3) {
        const int rows = a.batch * a.Hq;
        float acc = 0.f;
        for (int r = lane; r < rows; r += 64) acc += a.ws_rows[(size_t)r * 3 + wave];
        acc = wave_sum(acc);
        if (lane == 0) a.kl_out[wave] = acc / (float)rows;
    }
    if (tid == 0) *a.counter = 0u;
}

}  // namespace

size_t canary_workspace_bytes(const kv_geometry& g, int batch) {
    return 256 + (size_t)batch * g.num_q_heads * 3 * sizeof(float);
}

hipError_t launch_canary(const kv_geometry& g, const uint16_t* ring, const int32_t* seq_len,
                         int batch, const uint16_t* q, float softmax_scale, float* kl_out,
                         float* kl_rows, void* workspace, hipStream_t stream) {
    CanaryArgs a;
    a.ring = ring;
    a.seq_len = seq_len;
    a.q = q;
    a.kl_out = kl_out;
    a.kl_rows = kl_rows;
    a.counter = static_cast<uint32_t*>(workspace);
    a.ws_rows = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + 256);
    a.H = g.num_kv_heads;
    a.Hq = g.num_q_heads;
    a.grp = g.num_q_heads / g.num_kv_heads;
    a.R = g.ring_size;
    a.batch = batch;
    a.scale = softmax_scale;
    const int D = g.head_dim;
    const size_t lds = sizeof(float) * (2 * (size_t)a.R * D + kMaxGroup * D + 2 * kMaxGroup * (size_t)a.R);
    dim3 grid((unsigned)(batch * g.num_kv_heads));
    // the LDS footprint exceeds the 64 KiB default for rings of 64 keys at D = 128
    const void* fn = D == 128 ? reinterpret_cast<const void*>(&canary_kernel<128>)
                              : reinterpret_cast<const void*>(&canary_kernel<64>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (D == 128)
        hipLaunchKernelGGL(canary_kernel<128>, grid, dim3(kThreads), lds, stream, a);
    else
        hipLaunchKernelGGL(canary_kernel<64>, grid, dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace kvq
