// kv_write.hip -- quantize-on-write for one layer (gfx950).
//
// EchoKV, "How EchoKV works": the step's key enters the per-layer FP16 ring before it is
// quantized into the paged cache. Behavior-Guided KV-Cache Quantization, "K/V Role-Aware
// Low-Bit Quantization": keys get one scale per channel (over the page's tokens), values one
// scale per token (over its channels); "Online inference": pack and store.
//
// One 256-thread workgroup per (page touched, KV head, sequence). Thread (t, g) = (tid / 16,
// tid % 16) owns token slot t of the page and channels [g*D/16, (g+1)*D/16): every input element
// is fetched by exactly one 8- or 16-byte load, issued up front, so the workgroup waits on
// memory once. Channel maxima over the
// page's tokens reduce across the four token lanes of a wave (shuffles) and the four waves
// (LDS); token maxima over D reduce across the 16 lanes of a token (shuffles). Codes are packed
// in registers; words shared by several threads are OR-reduced with shuffles. A geometry with the
// asymmetric format gives each group a zero point and a scale from its minimum and maximum.
//
// The workgroup of the first page touched is the only reader of the ring (the page's earlier
// keys live there), so it also performs the ring update, after a barrier.
#include "kvq_device.hpp"
#include "kvq_launch.hpp"
#include "kvq_write_dev.hpp"

namespace kvq {
namespace {

constexpr int kThreads = 256;

template <int D, bool ASYM>
__global__ __launch_bounds__(kThreads) void quant_write_kernel(WriteArgs a) {
    __shared__ float chan_red[ASYM ? 8 : 4][D];   // per-wave channel maxima of |K| (ASYM: of K, then minima)
    const int j = blockIdx.x, kv = blockIdx.y, s = blockIdx.z;
    const int p0 = a.pos[s];
    write_page<D, ASYM>(a, s, kv, p0, j, threadIdx.x, true, chan_red);
    if (j == 0 && p0 / kPage * kPage < p0 + a.n_new) {   // the first page's workgroup
        __syncthreads();                                  // its ring reads are done
        write_ring<D>(a, s, kv, p0, threadIdx.x, kThreads);
    }
}

}  // namespace

hipError_t launch_quant_write(const kv_geometry& g, PoolPtrs pools, const uint32_t* bt,
                              const int32_t* pos, int batch, int n_new, const uint16_t* k_new,
                              const uint16_t* v_new, uint16_t* ring, hipStream_t stream) {
    WriteArgs a;
    a.pools = pools;
    a.bt = bt;
    a.pos = pos;
    a.k_new = k_new;
    a.v_new = v_new;
    a.ring = ring;
    a.max_pages = g.max_pages_per_seq;
    a.n_new = n_new;
    a.H = g.num_kv_heads;
    a.R = g.ring_size;
    // pages touched per sequence: at most ceil(n_new / P) + 1 (the first may be partial)
    dim3 grid((unsigned)((n_new + kPage - 1) / kPage + 1), (unsigned)g.num_kv_heads, (unsigned)batch);
    const bool asym = g.asymmetric != 0;
    if (g.head_dim == 128) {
        if (asym) hipLaunchKernelGGL((quant_write_kernel<128, true>), grid, dim3(kThreads), 0, stream, a);
        else hipLaunchKernelGGL((quant_write_kernel<128, false>), grid, dim3(kThreads), 0, stream, a);
    } else {
        if (asym) hipLaunchKernelGGL((quant_write_kernel<64, true>), grid, dim3(kThreads), 0, stream, a);
        else hipLaunchKernelGGL((quant_write_kernel<64, false>), grid, dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace kvq
