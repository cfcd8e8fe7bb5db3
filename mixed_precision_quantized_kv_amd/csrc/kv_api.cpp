// kv_api.cpp -- the C ABI of libkvq (include/kv_quant.h): argument validation, byte sizes,
// the host block allocator, and dispatch to the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "kv_quant.h"
#include "kvq_device.hpp"
#include "kvq_host.hpp"
#include "kvq_launch.hpp"

namespace kvq {

thread_local char g_last_error[512] = "";

kv_status fail(kv_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

kv_status ok() {
    g_last_error[0] = '\0';
    return KV_OK;
}

const char* last_error() { return g_last_error; }

}  // namespace kvq

namespace {

int tier_of_bits(int bits);

}  // namespace

bool kvq::alloc_accepts_bits(int bits) { return tier_of_bits(bits) >= 0; }

namespace {

using kvq::fail;
using kvq::ok;

kv_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(KV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int tier_of_bits(int bits) {
    return bits == 2 ? 0 : bits == 4 ? 1 : bits == 8 ? 2 : bits == 16 ? 3 : -1;
}

constexpr int kTiers = KV_NUM_TIERS;

kv_status check_geometry(const kv_geometry* g) {
    if (!g) return fail(KV_EINVAL, "geometry is NULL");
    if (g->num_layers < 1 || g->num_q_heads < 1 || g->num_kv_heads < 1 || g->max_seqs < 1 ||
        g->max_pages_per_seq < 1)
        return fail(KV_EINVAL, "geometry counts must be positive");
    if (g->num_q_heads % g->num_kv_heads != 0)
        return fail(KV_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    g->num_q_heads, g->num_kv_heads);
    if (g->page_size != kvq::kPage) return fail(KV_EUNSUPPORTED, "page_size must be 16");
    if (g->ring_size < g->page_size || g->ring_size > 128 || g->ring_size % g->page_size != 0)
        return fail(KV_EINVAL, "ring_size %d must be a multiple of page_size in [16, 128]",
                    g->ring_size);
    if (g->head_dim != 64 && g->head_dim != 128)
        return fail(KV_EUNSUPPORTED, "head_dim %d: only 64 and 128 are built", g->head_dim);
    if (g->num_q_heads / g->num_kv_heads > kvq::kMaxGroup)
        return fail(KV_EUNSUPPORTED, "GQA group %d exceeds 16", g->num_q_heads / g->num_kv_heads);
    if ((int64_t)g->max_pages_per_seq * g->page_size > (int64_t)1 << 30)
        return fail(KV_EINVAL, "max_pages_per_seq too large");
    if (g->asymmetric != 0 && g->asymmetric != 1)
        return fail(KV_EINVAL, "asymmetric must be 0 or 1, not %d", g->asymmetric);
    return ok();
}

kv_status check_pools(const kv_geometry* g, const kv_layer_pools* p) {
    if (!p) return fail(KV_EINVAL, "pools is NULL");
    for (int t = 0; t < kTiers; ++t) {
        if (p->capacity[t] > 0x3fffffffu) return fail(KV_EINVAL, "pool %d capacity too large", t);
        if (p->capacity[t] > 0 && !p->base[t]) return fail(KV_EINVAL, "pool %d base is NULL", t);
        if (reinterpret_cast<uintptr_t>(p->base[t]) % 16 != 0)
            return fail(KV_EINVAL, "pool %d base is not 16-byte aligned", t);
    }
    (void)g;
    return ok();
}

kvq::PoolPtrs pool_ptrs(const kv_layer_pools* p) {
    kvq::PoolPtrs r;
    for (int t = 0; t < kTiers; ++t) r.base[t] = static_cast<uint8_t*>(p->base[t]);
    return r;
}

// splitmix64: seeded shuffles of each pool's free list
uint64_t splitmix64(uint64_t& x) {
    uint64_t z = (x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

constexpr int64_t kMaxPagesPerSplit = 512;      // 8 waves x 64 pages

int auto_pages_per_split(const kv_geometry& g, int batch, int max_pages) {
    // one workgroup per CU (the kernel holds one 8-wave workgroup per CU): split each
    // (sequence, KV head) so that the grid has about 256 workgroups, pages in pairs, at most
    // 256 splits
    const int64_t groups = (int64_t)batch * g.num_kv_heads;
    int64_t splits = std::max<int64_t>(1, (256 + groups - 1) / groups);
    int64_t pps = (max_pages + splits - 1) / splits;
    pps = std::max<int64_t>(pps, 2);
    // a wave keeps the handles of at most 64 pages in registers (the width-specialised loop)
    pps = std::min<int64_t>(pps, kMaxPagesPerSplit);
    pps = std::max<int64_t>(pps, (max_pages + 255) / 256);
    pps += pps & 1;
    return (int)pps;
}

// The fused step: the workgroup of a sequence's last split also writes the step's tokens
// before it attends (four memory round trips per two pages, about 6 us: the loop time of 30 to
// 50 pages), so the plan keeps the split count and moves pages out of the last split: pps grows
// until the last split is kWriteReservePages per round of writes (at most half a split) shorter
// than the others.
constexpr int64_t kWriteReservePages = 40;       // per round of two pages written
constexpr int kMaxFusedNew = 64;                  // new tokens per sequence in one fused step

int step_pages_per_split(int64_t max_pages, int pps, int n_new, int page_size) {
    const int64_t splits = (max_pages + pps - 1) / pps;
    if (splits < 2 || n_new <= 0) return pps;
    const int64_t touched = (n_new + page_size - 1) / page_size + 1;   // at most
    const int64_t reserve = std::min<int64_t>(kWriteReservePages * ((touched + 1) / 2), pps / 2);
    int64_t p = (max_pages + reserve + splits - 1) / splits;
    p += p & 1;
    p = std::min<int64_t>(p, kMaxPagesPerSplit);
    if (p <= pps || (max_pages + p - 1) / p != splits) return pps;   // keep the grid
    return (int)p;
}

}  // namespace

struct kv_alloc {
    kv_geometry g;
    std::vector<int> bits;                       // current tier of each layer
    std::vector<uint32_t> capacity;              // [L][kTiers]
    std::vector<std::vector<uint32_t>> free;     // [L*kTiers]: free block indices, next at back
    std::vector<std::vector<uint32_t>> owned;    // [L*max_seqs]: the handles handed out, by page
    std::vector<int32_t> len;                    // tokens per sequence
};

extern "C" {

int kv_abi_version(void) { return KV_ABI_VERSION; }

const char* kv_strerror(kv_status s) {
    switch (s) {
        case KV_OK: return "ok";
        case KV_EINVAL: return "invalid argument";
        case KV_ENOBLOCKS: return "pool exhausted";
        case KV_EUNSUPPORTED: return "unsupported configuration";
        case KV_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* kv_last_error(void) { return kvq::last_error(); }

kv_status kv_validate(const kv_geometry* g) { return check_geometry(g); }

uint32_t kv_handle(int bits, uint32_t index) {
    const int t = tier_of_bits(bits);
    if (t < 0 || index > 0x3fffffffu) return KV_NO_BLOCK;
    return ((uint32_t)t << 30) | index;
}

size_t kv_block_bytes(const kv_geometry* g, int bits) {
    if (check_geometry(g) != KV_OK || tier_of_bits(bits) < 0) return 0;
    return (size_t)g->num_kv_heads * kvq::section_layout(g->head_dim, bits, g->asymmetric != 0).bytes;
}

size_t kv_ring_bytes(const kv_geometry* g) {
    if (check_geometry(g) != KV_OK) return 0;
    return (size_t)g->max_seqs * g->ring_size * g->num_kv_heads * g->head_dim * 2;
}

double kv_cache_bytes_per_token(const kv_geometry* g, const int* bits) {
    if (check_geometry(g) != KV_OK || !bits) return -1.0;
    double total = 0.0;
    for (int l = 0; l < g->num_layers; ++l) {
        if (tier_of_bits(bits[l]) >= 0)
            total += (double)kv_block_bytes(g, bits[l]) / g->page_size;
        else
            return -1.0;
    }
    return total;
}

// ---------------------------------------------------------------- allocator
kv_status kv_alloc_create(const kv_geometry* g, const uint32_t* capacity, const int* bits,
                          uint64_t shuffle_seed, kv_alloc** out) {
    kv_status st = check_geometry(g);
    if (st != KV_OK) return st;
    if (!capacity || !bits || !out) return fail(KV_EINVAL, "NULL argument");
    for (int l = 0; l < g->num_layers; ++l) {
        if (tier_of_bits(bits[l]) < 0) return fail(KV_EINVAL, "layer %d bits %d", l, bits[l]);
        for (int t = 0; t < kTiers; ++t)
            if (capacity[l * kTiers + t] > 0x3fffffffu) return fail(KV_EINVAL, "capacity too large");
    }
    kv_alloc* a = new (std::nothrow) kv_alloc;
    if (!a) return fail(KV_EINVAL, "out of host memory");
    try {
        a->g = *g;
        a->bits.assign(bits, bits + g->num_layers);
        a->capacity.assign(capacity, capacity + kTiers * g->num_layers);
        a->free.resize(kTiers * (size_t)g->num_layers);
        uint64_t x = shuffle_seed;
        for (size_t i = 0; i < a->free.size(); ++i) {
            std::vector<uint32_t>& f = a->free[i];
            f.resize(a->capacity[i]);
            for (uint32_t j = 0; j < a->capacity[i]; ++j) f[j] = j;
            for (size_t j = f.size(); j > 1; --j) std::swap(f[j - 1], f[splitmix64(x) % j]);
            std::reverse(f.begin(), f.end());     // handed out from the back
        }
        a->owned.resize((size_t)g->num_layers * g->max_seqs);
        a->len.assign(g->max_seqs, 0);
    } catch (const std::bad_alloc&) {
        delete a;
        return fail(KV_EINVAL, "out of host memory for the pools' free lists");
    }
    *out = a;
    return ok();
}

kv_status kv_alloc_set_layer_bits(kv_alloc* a, int layer, int bits) {
    if (!a) return fail(KV_EINVAL, "allocator is NULL");
    if (layer < 0 || layer >= a->g.num_layers) return fail(KV_EINVAL, "layer %d", layer);
    if (tier_of_bits(bits) < 0) return fail(KV_EINVAL, "bits %d", bits);
    a->bits[layer] = bits;
    return ok();
}

kv_status kv_alloc_extend(kv_alloc* a, int seq, int32_t new_len, uint32_t* bt) {
    if (!a || !bt) return fail(KV_EINVAL, "NULL argument");
    const kv_geometry& g = a->g;
    if (seq < 0 || seq >= g.max_seqs) return fail(KV_EINVAL, "seq %d", seq);
    const int32_t old_len = a->len[seq];
    if (new_len < old_len) return fail(KV_EINVAL, "new_len %d below current %d", new_len, old_len);
    const int64_t old_pages = (old_len + g.page_size - 1) / g.page_size;
    const int64_t new_pages = ((int64_t)new_len + g.page_size - 1) / g.page_size;
    if (new_pages > g.max_pages_per_seq)
        return fail(KV_EINVAL, "%lld pages exceed max_pages_per_seq", (long long)new_pages);
    const int64_t need = new_pages - old_pages;
    for (int l = 0; l < g.num_layers; ++l) {
        const std::vector<uint32_t>& f = a->free[(size_t)l * kTiers + tier_of_bits(a->bits[l])];
        if ((int64_t)f.size() < need)
            return fail(KV_ENOBLOCKS, "layer %d: %lld free %d-bit blocks, %lld needed", l,
                        (long long)f.size(), a->bits[l], (long long)need);
    }
    try {              // room for the new handles in every layer's record before anything moves
        for (int l = 0; l < g.num_layers; ++l)
            a->owned[(size_t)l * g.max_seqs + seq].reserve((size_t)new_pages);
    } catch (const std::bad_alloc&) {
        return fail(KV_EINVAL, "out of host memory");
    }
    for (int l = 0; l < g.num_layers; ++l) {
        const int t = tier_of_bits(a->bits[l]);
        std::vector<uint32_t>& f = a->free[(size_t)l * kTiers + t];
        std::vector<uint32_t>& mine = a->owned[(size_t)l * g.max_seqs + seq];
        uint32_t* row = bt + ((size_t)l * g.max_seqs + seq) * g.max_pages_per_seq;
        for (int64_t p = old_pages; p < new_pages; ++p) {
            row[p] = ((uint32_t)t << 30) | f.back();
            mine.push_back(row[p]);
            f.pop_back();
        }
    }
    a->len[seq] = new_len;
    return ok();
}

kv_status kv_alloc_free_seq(kv_alloc* a, int seq, uint32_t* bt) {
    if (!a || !bt) return fail(KV_EINVAL, "NULL argument");
    const kv_geometry& g = a->g;
    if (seq < 0 || seq >= g.max_seqs) return fail(KV_EINVAL, "seq %d", seq);
    // the blocks come back from the allocator's own record, whatever the table now holds, so
    // an edited table cannot return a block twice; a pool's free list never outgrows the
    // storage it was created with, so the returns allocate nothing
    for (int l = 0; l < g.num_layers; ++l) {
        std::vector<uint32_t>& mine = a->owned[(size_t)l * g.max_seqs + seq];
        for (const uint32_t h : mine)
            a->free[(size_t)l * kTiers + (h >> 30)].push_back(h & 0x3fffffffu);
        mine.clear();
        uint32_t* row = bt + ((size_t)l * g.max_seqs + seq) * g.max_pages_per_seq;
        for (int64_t p = 0; p < g.max_pages_per_seq; ++p) row[p] = KV_NO_BLOCK;
    }
    a->len[seq] = 0;
    return ok();
}

int32_t kv_alloc_seq_len(const kv_alloc* a, int seq) {
    if (!a || seq < 0 || seq >= a->g.max_seqs) return -1;
    return a->len[seq];
}

int64_t kv_alloc_free_blocks(const kv_alloc* a, int layer, int bits) {
    if (!a || layer < 0 || layer >= a->g.num_layers || tier_of_bits(bits) < 0) return -1;
    return (int64_t)a->free[(size_t)layer * kTiers + tier_of_bits(bits)].size();
}

int kv_alloc_layer_bits(const kv_alloc* a, int layer) {
    if (!a || layer < 0 || layer >= a->g.num_layers) return 0;
    return a->bits[layer];
}

void kv_alloc_destroy(kv_alloc* a) { delete a; }

kv_status kv_check_block_table(const kv_alloc* a, const uint32_t* bt) {
    if (!a || !bt) return fail(KV_EINVAL, "NULL argument");
    const kv_geometry& g = a->g;
    for (int l = 0; l < g.num_layers; ++l) {
        for (int s = 0; s < g.max_seqs; ++s) {
            const uint32_t* row = bt + ((size_t)l * g.max_seqs + s) * g.max_pages_per_seq;
            const std::vector<uint32_t>& mine = a->owned[(size_t)l * g.max_seqs + s];
            for (int64_t p = 0; p < g.max_pages_per_seq; ++p) {
                const uint32_t h = row[p];
                if (p >= (int64_t)mine.size()) {
                    if (h != KV_NO_BLOCK)
                        return fail(KV_EINVAL, "layer %d seq %d page %lld: stale handle", l, s,
                                    (long long)p);
                    continue;
                }
                if (h != mine[p])
                    return fail(KV_EINVAL,
                                "layer %d seq %d page %lld: handle 0x%08x, but block 0x%08x was "
                                "handed out for it", l, s, (long long)p, h, mine[p]);
            }
        }
    }
    return ok();
}

// ---------------------------------------------------------------- kernels
kv_status kv_quant_write(const kv_geometry* g, const kv_layer_pools* pools, const uint32_t* bt,
                         const int32_t* pos, int batch, int n_new, const uint16_t* k_new,
                         const uint16_t* v_new, uint16_t* ring, void* stream) {
    kv_status st = check_geometry(g);
    if (st != KV_OK) return st;
    if ((st = check_pools(g, pools)) != KV_OK) return st;
    if (batch < 0 || batch > g->max_seqs) return fail(KV_EINVAL, "batch %d", batch);
    if (n_new < 0 || (int64_t)n_new > (int64_t)g->max_pages_per_seq * g->page_size)
        return fail(KV_EINVAL, "n_new %d", n_new);
    if (batch == 0 || n_new == 0) return ok();
    if (!bt || !pos || !k_new || !v_new || !ring) return fail(KV_EINVAL, "NULL device pointer");
    if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16 ||
        reinterpret_cast<uintptr_t>(ring) % 16)
        return fail(KV_EINVAL, "k_new, v_new and ring must be 16-byte aligned");
    return hip_status(kvq::launch_quant_write(*g, pool_ptrs(pools), bt, pos, batch, n_new, k_new,
                                              v_new, ring, static_cast<hipStream_t>(stream)),
                      "kv_quant_write");
}

int kv_decode_pages_per_split(const kv_geometry* g, int batch, int max_ctx_len) {
    if (check_geometry(g) != KV_OK || batch < 1 || max_ctx_len < 0) return 0;
    const int max_pages = std::max(1, (max_ctx_len + g->page_size - 1) / g->page_size);
    return auto_pages_per_split(*g, batch, max_pages);
}

int kv_decode_pages_per_split_for(const kv_geometry* g, int batch, const int32_t* ctx_len_host) {
    if (check_geometry(g) != KV_OK || batch < 1 || batch > g->max_seqs || !ctx_len_host) return 0;
    int64_t total = 0, longest = 0;
    for (int s = 0; s < batch; ++s) {
        if (ctx_len_host[s] < 0 || (int64_t)ctx_len_host[s] > (int64_t)g->max_pages_per_seq * g->page_size)
            return 0;
        const int64_t pages = (ctx_len_host[s] + g->page_size - 1) / g->page_size;
        total += pages;
        longest = std::max(longest, pages);
    }
    const int uniform = auto_pages_per_split(*g, batch, (int)std::max<int64_t>(1, longest));
    if (10 * total >= 9 * longest * batch) return uniform;
    // ragged: about 1.8 workgroups' worth of pages per compute unit over the whole batch (the
    // sequences' shorter last splits make the workgroup count ~2.3 per CU). Measured on 64
    // log-uniform lengths in [1K, 32K]: 1.8 -> 122.6 us per launch, 2.0 -> 128.8 us, 1.6 -> 125.7
    // us; smaller splits add per-workgroup round trips, larger ones leave compute units idle at
    // the end.
    int64_t pps = (total * g->num_kv_heads + 459) / 460;
    pps = std::min<int64_t>(std::max<int64_t>(pps, 2), uniform);
    pps = std::max<int64_t>(pps, (longest + 255) / 256);
    pps += pps & 1;
    return (int)pps;
}

int kv_decode_step_pages_per_split_for(const kv_geometry* g, int batch, const int32_t* pos_host,
                                       int n_new) {
    if (check_geometry(g) != KV_OK || batch < 1 || batch > g->max_seqs || !pos_host ||
        n_new < 0 || n_new > kMaxFusedNew)
        return 0;
    std::vector<int32_t> ctx;
    try {
        ctx.resize(batch);
    } catch (const std::bad_alloc&) {
        return 0;
    }
    int64_t longest = 0, shortest = INT64_MAX;
    for (int s = 0; s < batch; ++s) {
        if (pos_host[s] < 0) return 0;
        const int64_t c = (int64_t)pos_host[s] + n_new;
        if (c > (int64_t)g->max_pages_per_seq * g->page_size) return 0;
        ctx[s] = (int32_t)c;
        longest = std::max(longest, c);
        shortest = std::min(shortest, c);
    }
    const int pps = kv_decode_pages_per_split_for(g, batch, ctx.data());
    if (pps == 0 || n_new == 0) return pps;
    // the reserve suits a batch whose sequences end in the same split
    const int64_t last_pages = (longest + g->page_size - 1) / g->page_size;
    const int64_t first_pages = (shortest + g->page_size - 1) / g->page_size;
    if ((last_pages - 1) / pps != (first_pages - 1) / pps) return pps;
    return step_pages_per_split(last_pages, pps, n_new, g->page_size);
}

// step_new > 0: the plan of a fused step writing step_new tokens, when the caller leaves the
// plan to the library
static kv_status decode_plan(const kv_geometry* g, int batch, int max_ctx_len, int pps_in,
                             int* pps, int* splits, int step_new = 0) {
    if (batch < 1 || batch > g->max_seqs) return fail(KV_EINVAL, "batch %d", batch);
    if (max_ctx_len < 0 || (int64_t)max_ctx_len > (int64_t)g->max_pages_per_seq * g->page_size)
        return fail(KV_EINVAL, "max_ctx_len %d", max_ctx_len);
    const int max_pages = std::max(1, (max_ctx_len + g->page_size - 1) / g->page_size);
    int p = pps_in ? pps_in : auto_pages_per_split(*g, batch, max_pages);
    if (!pps_in && step_new > 0) p = step_pages_per_split(max_pages, p, step_new, g->page_size);
    if (p < 2 || p % 2 != 0) return fail(KV_EINVAL, "pages_per_split %d: an even number >= 2", p);
    const int s = (max_pages + p - 1) / p;
    if (s > 256) return fail(KV_EINVAL, "pages_per_split %d gives %d splits (max 256)", p, s);
    *pps = p;
    *splits = s;
    return ok();
}

size_t kv_decode_workspace_bytes(const kv_geometry* g, int batch, int max_ctx_len,
                                 int pages_per_split) {
    if (check_geometry(g) != KV_OK) return 0;
    int pps, splits;
    if (decode_plan(g, batch, max_ctx_len, pages_per_split, &pps, &splits) != KV_OK) return 0;
    return kvq::decode_workspace_bytes(*g, batch, splits);
}

kv_status kv_decode_attn(const kv_geometry* g, const kv_layer_pools* pools, const uint32_t* bt,
                         const int32_t* ctx_len, int batch, int max_ctx_len, const uint16_t* q,
                         float softmax_scale, float* out, void* workspace,
                         size_t workspace_bytes, int pages_per_split, void* stream) {
    kv_status st = check_geometry(g);
    if (st != KV_OK) return st;
    if ((st = check_pools(g, pools)) != KV_OK) return st;
    int pps, splits;
    if ((st = decode_plan(g, batch, max_ctx_len, pages_per_split, &pps, &splits)) != KV_OK)
        return st;
    if (!bt || !ctx_len || !q || !out || !workspace) return fail(KV_EINVAL, "NULL device pointer");
    if (reinterpret_cast<uintptr_t>(q) % 4 || reinterpret_cast<uintptr_t>(out) % 16 ||
        reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(KV_EINVAL, "q must be 4-byte, out 16-byte and workspace 256-byte aligned");
    const size_t need = kvq::decode_workspace_bytes(*g, batch, splits);
    if (workspace_bytes < need)
        return fail(KV_EINVAL, "workspace %zu bytes, %zu needed", workspace_bytes, need);
    if (!std::isfinite(softmax_scale))
        return fail(KV_EINVAL, "softmax_scale %g is not finite", (double)softmax_scale);
    return hip_status(kvq::launch_decode_attn(*g, pool_ptrs(pools), bt, ctx_len, batch, splits, pps,
                                              q, softmax_scale, out, workspace,
                                              static_cast<hipStream_t>(stream)),
                      "kv_decode_attn");
}

kv_status kv_decode_step(const kv_geometry* g, const kv_layer_pools* pools, const uint32_t* bt,
                         const int32_t* pos, int batch, int n_new, const uint16_t* k_new,
                         const uint16_t* v_new, uint16_t* ring, int max_ctx_len, const uint16_t* q,
                         float softmax_scale, float* out, void* workspace,
                         size_t workspace_bytes, int pages_per_split, void* stream) {
    kv_status st = check_geometry(g);
    if (st != KV_OK) return st;
    if ((st = check_pools(g, pools)) != KV_OK) return st;
    if (n_new < 0 || n_new > kMaxFusedNew)
        return fail(KV_EINVAL, "n_new %d: the fused step writes 0..%d tokens", n_new, kMaxFusedNew);
    int pps, splits;
    if ((st = decode_plan(g, batch, max_ctx_len, pages_per_split, &pps, &splits, n_new)) != KV_OK)
        return st;
    if (!bt || !pos || !q || !out || !workspace) return fail(KV_EINVAL, "NULL device pointer");
    if (n_new > 0 && (!k_new || !v_new || !ring)) return fail(KV_EINVAL, "NULL device pointer");
    if (reinterpret_cast<uintptr_t>(q) % 4 || reinterpret_cast<uintptr_t>(out) % 16 ||
        reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(KV_EINVAL, "q must be 4-byte, out 16-byte and workspace 256-byte aligned");
    if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16 ||
        reinterpret_cast<uintptr_t>(ring) % 16)
        return fail(KV_EINVAL, "k_new, v_new and ring must be 16-byte aligned");
    const size_t need = kvq::decode_workspace_bytes(*g, batch, splits);
    if (workspace_bytes < need)
        return fail(KV_EINVAL, "workspace %zu bytes, %zu needed", workspace_bytes, need);
    if (!std::isfinite(softmax_scale))
        return fail(KV_EINVAL, "softmax_scale %g is not finite", (double)softmax_scale);
    return hip_status(kvq::launch_decode_step(*g, pool_ptrs(pools), bt, pos, batch, n_new, k_new,
                                              v_new, ring, splits, pps, q, softmax_scale, out,
                                              workspace, static_cast<hipStream_t>(stream)),
                      "kv_decode_step");
}

kv_status kv_decode_step_noalloc(const kv_geometry* g, const kv_layer_pools* pools,
                                 const uint32_t* bt, const int32_t* pos, int batch, int n_new,
                                 const uint16_t* k_new, const uint16_t* v_new, uint16_t* ring,
                                 int max_ctx_len, const uint16_t* q, float softmax_scale,
                                 float* out, int pages_per_split, void* stream) {
    kv_status st = check_geometry(g);
    if (st != KV_OK) return st;
    if ((st = check_pools(g, pools)) != KV_OK) return st;
    if (n_new < 0 || n_new > kMaxFusedNew)
        return fail(KV_EINVAL, "n_new %d: the fused step writes 0..%d tokens", n_new, kMaxFusedNew);
    int pps, splits;
    if ((st = decode_plan(g, batch, max_ctx_len, pages_per_split, &pps, &splits, n_new)) != KV_OK)
        return st;
    if (!bt || !pos || !q || !out) return fail(KV_EINVAL, "NULL device pointer");
    if (n_new > 0 && (!k_new || !v_new || !ring)) return fail(KV_EINVAL, "NULL device pointer");
    if (reinterpret_cast<uintptr_t>(q) % 4 || reinterpret_cast<uintptr_t>(out) % 16)
        return fail(KV_EINVAL, "q must be 4-byte and out 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16 ||
        reinterpret_cast<uintptr_t>(ring) % 16)
        return fail(KV_EINVAL, "k_new, v_new and ring must be 16-byte aligned");
    if ((int64_t)batch * g->num_kv_heads > kvq::kStaticMaxGroups)
        return fail(KV_EINVAL,
                    "batch %d x %d KV heads: the static scratch holds counters for %d groups",
                    batch, g->num_kv_heads, kvq::kStaticMaxGroups);
    const size_t need = kvq::static_scratch_partial_bytes(*g, batch, splits);
    const size_t room = kvq::kStaticScratchBytes - kvq::kStaticCounterBytes;
    if (need > room)
        return fail(KV_EINVAL,
                    "the split partials need %zu bytes (%d splits); the static scratch holds %zu",
                    need, splits, room);
    if (!std::isfinite(softmax_scale))
        return fail(KV_EINVAL, "softmax_scale %g is not finite", (double)softmax_scale);
    return hip_status(kvq::launch_decode_step_static(*g, pool_ptrs(pools), bt, pos, batch, n_new,
                                                     k_new, v_new, ring, splits, pps, q,
                                                     softmax_scale, out,
                                                     static_cast<hipStream_t>(stream)),
                      "kv_decode_step_noalloc");
}

size_t kv_canary_workspace_bytes(const kv_geometry* g, int batch) {
    if (check_geometry(g) != KV_OK || batch < 1) return 0;
    return kvq::canary_workspace_bytes(*g, 1, 1, batch);
}

size_t kv_canary_layers_workspace_bytes(const kv_geometry* g, int num_layers, int batch) {
    if (check_geometry(g) != KV_OK || batch < 1 || num_layers < 1 ||
        num_layers > std::min(g->num_layers, KV_CANARY_MAX_LAYERS))
        return 0;
    return kvq::canary_workspace_bytes(*g, kvq::canary_counter_layers(*g), num_layers, batch);
}

static kv_status canary(const kv_geometry* g, const uint16_t* ring, const int32_t* seq_len,
                        int batch, const uint16_t* q, float softmax_scale, bool asymmetric,
                        float* kl_out, float* kl_rows, void* workspace, size_t workspace_bytes,
                        void* stream, const char* name) {
    kv_status st = check_geometry(g);
    if (st != KV_OK) return st;
    if (batch < 1 || batch > g->max_seqs) return fail(KV_EINVAL, "batch %d", batch);
    if (!ring || !seq_len || !q || !kl_out || !workspace)
        return fail(KV_EINVAL, "NULL device pointer");
    if (reinterpret_cast<uintptr_t>(ring) % 16 || reinterpret_cast<uintptr_t>(q) % 16)
        return fail(KV_EINVAL, "ring and q must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(KV_EINVAL, "workspace must be 256-byte aligned");
    const size_t need = kvq::canary_workspace_bytes(*g, 1, 1, batch);
    if (workspace_bytes < need)
        return fail(KV_EINVAL, "workspace %zu bytes, %zu needed", workspace_bytes, need);
    if (!std::isfinite(softmax_scale))
        return fail(KV_EINVAL, "softmax_scale %g is not finite", (double)softmax_scale);
    return hip_status(kvq::launch_canary(*g, ring, seq_len, batch, q, softmax_scale, asymmetric,
                                         kl_out, kl_rows, workspace,
                                         static_cast<hipStream_t>(stream)),
                      name);
}

kv_status kv_canary_kl(const kv_geometry* g, const uint16_t* ring, const int32_t* seq_len,
                       int batch, const uint16_t* q, float softmax_scale, float* kl_out,
                       float* kl_rows, void* workspace, size_t workspace_bytes, void* stream) {
    // the cache's own quantizer: the asymmetric copies for a geometry in the asymmetric format
    return canary(g, ring, seq_len, batch, q, softmax_scale, g && g->asymmetric == 1, kl_out,
                  kl_rows, workspace, workspace_bytes, stream, "kv_canary_kl");
}

kv_status kv_canary_kl_layers(const kv_geometry* g, int num_layers, const uint16_t* const* rings,
                              const int32_t* seq_len, int batch, const uint16_t* const* q,
                              float softmax_scale, float* kl_out, float* kl_rows, void* workspace,
                              size_t workspace_bytes, void* stream) {
    kv_status st = check_geometry(g);
    if (st != KV_OK) return st;
    if (num_layers < 1 || num_layers > std::min(g->num_layers, KV_CANARY_MAX_LAYERS))
        return fail(KV_EINVAL, "num_layers %d: 1 .. min(geometry layers %d, %d)", num_layers,
                    g->num_layers, KV_CANARY_MAX_LAYERS);
    if (batch < 1 || batch > g->max_seqs) return fail(KV_EINVAL, "batch %d", batch);
    if (!rings || !q) return fail(KV_EINVAL, "NULL host pointer array");
    if (!seq_len || !kl_out || !workspace) return fail(KV_EINVAL, "NULL device pointer");
    for (int l = 0; l < num_layers; ++l) {
        if (!rings[l] || !q[l]) return fail(KV_EINVAL, "layer %d: NULL device pointer", l);
        if (reinterpret_cast<uintptr_t>(rings[l]) % 16 || reinterpret_cast<uintptr_t>(q[l]) % 16)
            return fail(KV_EINVAL, "layer %d: ring and q must be 16-byte aligned", l);
    }
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(KV_EINVAL, "workspace must be 256-byte aligned");
    const size_t need =
        kvq::canary_workspace_bytes(*g, kvq::canary_counter_layers(*g), num_layers, batch);
    if (workspace_bytes < need)
        return fail(KV_EINVAL, "workspace %zu bytes, %zu needed", workspace_bytes, need);
    if (!std::isfinite(softmax_scale))
        return fail(KV_EINVAL, "softmax_scale %g is not finite", (double)softmax_scale);
    return hip_status(kvq::launch_canary_layers(*g, num_layers, rings, seq_len, batch, q,
                                                softmax_scale, kl_out, kl_rows, workspace,
                                                static_cast<hipStream_t>(stream)),
                      "kv_canary_kl_layers");
}

kv_status kv_canary_kl_asym(const kv_geometry* g, const uint16_t* ring, const int32_t* seq_len,
                            int batch, const uint16_t* q, float softmax_scale, float* kl_out,
                            float* kl_rows, void* workspace, size_t workspace_bytes,
                            void* stream) {
    return canary(g, ring, seq_len, batch, q, softmax_scale, true, kl_out, kl_rows, workspace,
                  workspace_bytes, stream, "kv_canary_kl_asym");
}

}  // extern "C"
