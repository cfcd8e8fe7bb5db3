// kvq_launch.hpp -- internal launch entry points (called by the C ABI in kv_api.cpp after all
// arguments have been validated on the host).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv_quant.h"

namespace kvq {

struct PoolPtrs {
    uint8_t* base[KV_NUM_TIERS];   // INT2, INT4, INT8, FP16
};

hipError_t launch_quant_write(const kv_geometry& g, PoolPtrs pools, const uint32_t* bt,
                              const int32_t* pos, int batch, int n_new, const uint16_t* k_new,
                              const uint16_t* v_new, uint16_t* ring, hipStream_t stream);

// split-K decode attention; splits = ceil(max_pages / pages_per_split)
hipError_t launch_decode_attn(const kv_geometry& g, PoolPtrs pools, const uint32_t* bt,
                              const int32_t* ctx_len, int batch, int splits, int pages_per_split,
                              const uint16_t* q, float softmax_scale, float* out,
                              void* workspace, hipStream_t stream);

// write of n_new <= 64 tokens per sequence (at most five pages) fused into the decode attention
// over pos + n_new
hipError_t launch_decode_step(const kv_geometry& g, PoolPtrs pools, const uint32_t* bt,
                              const int32_t* pos, int batch, int n_new, const uint16_t* k_new,
                              const uint16_t* v_new, uint16_t* ring, int splits,
                              int pages_per_split, const uint16_t* q, float softmax_scale,
                              float* out, void* workspace, hipStream_t stream);

// workspace layout of the decode attention (bytes)
size_t decode_workspace_bytes(const kv_geometry& g, int batch, int splits);

// the fused step with its workspace in a fixed file-scope device array (one per GPU): ticket
// counters for kStaticMaxGroups (sequence, KV head) groups first, then the split partials
constexpr int kStaticMaxGroups = 4096;
constexpr size_t kStaticCounterBytes = (size_t)kStaticMaxGroups * 256;      // 1 MiB
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;                    // 16 MiB
size_t static_scratch_partial_bytes(const kv_geometry& g, int batch, int splits);
hipError_t launch_decode_step_static(const kv_geometry& g, PoolPtrs pools, const uint32_t* bt,
                                     const int32_t* pos, int batch, int n_new,
                                     const uint16_t* k_new, const uint16_t* v_new, uint16_t* ring,
                                     int splits, int pages_per_split, const uint16_t* q,
                                     float softmax_scale, float* out, hipStream_t stream);

// asymmetric: build the temporary copies with the min / max (zero point) quantizer
hipError_t launch_canary(const kv_geometry& g, const uint16_t* ring, const int32_t* seq_len,
                         int batch, const uint16_t* q, float softmax_scale, bool asymmetric,
                         float* kl_out, float* kl_rows, void* workspace, hipStream_t stream);
// every layer's canary in one grid: rings[l], q[l] (host arrays of device pointers, copied
// into the launch), l < num_layers <= kMaxCanaryLayers
constexpr int kMaxCanaryLayers = KV_CANARY_MAX_LAYERS;
hipError_t launch_canary_layers(const kv_geometry& g, int num_layers,
                                const uint16_t* const* rings, const int32_t* seq_len, int batch,
                                const uint16_t* const* q, float softmax_scale, float* kl_out,
                                float* kl_rows, void* workspace, hipStream_t stream);
size_t canary_workspace_bytes(const kv_geometry& g, int counter_layers, int num_layers, int batch);
// the multi-layer call keeps a ticket line per (layer, width) for every layer it may be given
inline int canary_counter_layers(const kv_geometry& g) {
    return g.num_layers < kMaxCanaryLayers ? g.num_layers : kMaxCanaryLayers;
}

}  // namespace kvq
