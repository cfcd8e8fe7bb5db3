/* A plain C99 client of kv_quant.h: the header compiles with -std=c99 -pedantic, links against
 * libkvq, and the host-only calls (sizes, handles, validation, allocator, controller, argument
 * checks of the device calls) behave as the header states. No device memory is touched.
 * Prints one line per failed check and exits with the number of failures. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "kv_quant.h"

static int failures = 0;

#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            printf("FAIL line %d: %s [%s]\n", __LINE__, #cond, kv_last_error()); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static kv_geometry geometry(void) {
    kv_geometry g;
    memset(&g, 0, sizeof g);
    g.num_layers = 2;
    g.num_q_heads = 8;
    g.num_kv_heads = 2;
    g.head_dim = 64;
    g.page_size = 16;
    g.ring_size = 64;
    g.max_seqs = 2;
    g.max_pages_per_seq = 8;
    g.asymmetric = 0;
    return g;
}

/* the header's section size: P*D*b/4 + 2*D + 2*P bytes (symmetric), 4*P*D (fp16) */
static size_t section_bytes(const kv_geometry* g, int bits) {
    size_t P = (size_t)g->page_size, D = (size_t)g->head_dim;
    if (bits == 16) return 4 * P * D;
    return P * D * (size_t)bits / 4 + (g->asymmetric ? 4 : 2) * (D + P);
}

static void sizes_and_handles(void) {
    kv_geometry g = geometry();
    int b;
    const int widths[4] = {2, 4, 8, 16};
    CHECK(kv_abi_version() == KV_ABI_VERSION);
    CHECK(kv_validate(&g) == KV_OK);
    for (b = 0; b < 4; ++b)
        CHECK(kv_block_bytes(&g, widths[b]) == (size_t)g.num_kv_heads * section_bytes(&g, widths[b]));
    CHECK(kv_block_bytes(&g, 3) == 0);
    CHECK(kv_ring_bytes(&g) == (size_t)g.max_seqs * 64 * 2 * 64 * 2);
    g.asymmetric = 1;
    CHECK(kv_validate(&g) == KV_OK);
    CHECK(kv_block_bytes(&g, 4) == (size_t)g.num_kv_heads * section_bytes(&g, 4));
    CHECK(kv_block_bytes(&g, 16) == (size_t)g.num_kv_heads * section_bytes(&g, 16));
    CHECK(kv_handle(2, 5) == 5u);
    CHECK(kv_handle(4, 7) == ((1u << 30) | 7u));
    CHECK(kv_handle(8, 0) == (2u << 30));
    CHECK(kv_handle(16, 9) == ((3u << 30) | 9u));
    CHECK(kv_handle(3, 0) == KV_NO_BLOCK);
    CHECK(kv_handle(2, 1u << 30) == KV_NO_BLOCK);
    CHECK(kv_strerror(KV_OK) != NULL && kv_strerror(KV_EHIP) != NULL);
}

static void validation(void) {
    kv_geometry g = geometry();
    g.head_dim = 96;
    CHECK(kv_validate(&g) == KV_EUNSUPPORTED);
    CHECK(strlen(kv_last_error()) > 0);
    g = geometry();
    g.num_q_heads = 9;
    CHECK(kv_validate(&g) == KV_EINVAL);
    g = geometry();
    g.ring_size = 24;
    CHECK(kv_validate(&g) == KV_EINVAL);
    CHECK(kv_validate(NULL) == KV_EINVAL);
}

/* a two-layer cache: 16 blocks per (layer, tier) */
static void allocator(void) {
    kv_geometry g = geometry();
    uint32_t capacity[2 * KV_NUM_TIERS];
    int bits[2] = {4, 8};
    uint32_t bt[2 * 2 * 8];
    uint32_t before[2 * 2 * 8];
    kv_alloc* a = NULL;
    int i, p;
    for (i = 0; i < 2 * KV_NUM_TIERS; ++i) capacity[i] = 16;
    for (i = 0; i < 2 * 2 * 8; ++i) bt[i] = KV_NO_BLOCK;
    CHECK(kv_alloc_create(&g, capacity, bits, 7, &a) == KV_OK && a != NULL);
    if (a == NULL) return;
    CHECK(kv_alloc_extend(a, 0, 40, bt) == KV_OK);           /* 3 pages in every layer */
    CHECK(kv_alloc_seq_len(a, 0) == 40);
    CHECK(kv_alloc_free_blocks(a, 0, 4) == 13 && kv_alloc_free_blocks(a, 1, 8) == 13);
    CHECK(kv_alloc_free_blocks(a, 0, 2) == 16);
    for (p = 0; p < 3; ++p) {
        CHECK(bt[p] >> 30 == 1u);                             /* layer 0, seq 0: INT4 */
        CHECK(bt[2 * 8 + p] >> 30 == 2u);                     /* layer 1, seq 0: INT8 */
    }
    CHECK(bt[3] == KV_NO_BLOCK && bt[8] == KV_NO_BLOCK);
    CHECK(kv_check_block_table(a, bt) == KV_OK);
    /* forward-only: layer 1's later pages come from INT2, its first three stay INT8 */
    CHECK(kv_alloc_set_layer_bits(a, 1, 2) == KV_OK && kv_alloc_layer_bits(a, 1) == 2);
    CHECK(kv_alloc_extend(a, 0, 60, bt) == KV_OK);
    CHECK(bt[2 * 8 + 2] >> 30 == 2u && bt[2 * 8 + 3] >> 30 == 0u);
    CHECK(kv_alloc_free_blocks(a, 1, 2) == 15);
    /* more pages than a block-table row holds: rejected, nothing changes */
    memcpy(before, bt, sizeof bt);
    CHECK(kv_alloc_extend(a, 1, 16 * 8 + 1, bt) == KV_EINVAL);
    CHECK(memcmp(before, bt, sizeof bt) == 0);
    CHECK(kv_alloc_seq_len(a, 1) == 0);
    /* a table naming one block twice is caught */
    CHECK(kv_alloc_extend(a, 1, 1, bt) == KV_OK);
    CHECK(kv_check_block_table(a, bt) == KV_OK);
    memcpy(before, bt, sizeof bt);
    before[8] = before[0];                                    /* seq 1 page 0 := seq 0 page 0 */
    CHECK(kv_check_block_table(a, before) != KV_OK);
    memcpy(before, bt, sizeof bt);
    before[9] = before[8];                                    /* a page past seq 1's length */
    CHECK(kv_check_block_table(a, before) != KV_OK);
    CHECK(kv_alloc_free_seq(a, 1, bt) == KV_OK);
    CHECK(kv_alloc_free_seq(a, 0, bt) == KV_OK);
    CHECK(kv_alloc_free_blocks(a, 0, 4) == 16 && kv_alloc_free_blocks(a, 1, 8) == 16);
    CHECK(kv_alloc_free_blocks(a, 1, 2) == 16);
    for (i = 0; i < 2 * 2 * 8; ++i) CHECK(bt[i] == KV_NO_BLOCK);
    CHECK(kv_alloc_seq_len(a, 5) == -1 && kv_alloc_layer_bits(a, 9) == 0);
    kv_alloc_destroy(a);
}

/* too many pages for the pools: KV_ENOBLOCKS, allocator and table unchanged */
static void allocator_full(void) {
    kv_geometry g = geometry();
    uint32_t capacity[2 * KV_NUM_TIERS] = {4, 4, 4, 4, 4, 4, 4, 4};
    int bits[2] = {2, 2};
    uint32_t bt[2 * 2 * 8];
    uint32_t before[2 * 2 * 8];
    kv_alloc* a = NULL;
    int i;
    for (i = 0; i < 2 * 2 * 8; ++i) bt[i] = KV_NO_BLOCK;
    CHECK(kv_alloc_create(&g, capacity, bits, 1, &a) == KV_OK);
    if (a == NULL) return;
    CHECK(kv_alloc_extend(a, 0, 64, bt) == KV_OK);           /* the 4 blocks of each INT2 pool */
    memcpy(before, bt, sizeof bt);
    CHECK(kv_alloc_extend(a, 1, 1, bt) == KV_ENOBLOCKS);
    CHECK(memcmp(before, bt, sizeof bt) == 0 && kv_alloc_seq_len(a, 1) == 0);
    CHECK(kv_alloc_free_blocks(a, 0, 2) == 0 && kv_alloc_free_blocks(a, 0, 4) == 4);
    kv_alloc_destroy(a);
}

/* the budget tau0 * sqrt(L / L0), and the least width under it */
static void controller(void) {
    kv_controller* c = NULL;
    int init[2] = {16, 16};
    int bits[2] = {0, 0};
    double ema[6];
    int64_t firings = -1;
    /* layer 0: every width under the budget -> INT2; layer 1: only INT8 under it -> INT8 */
    float kl[6] = {0.01f, 0.005f, 0.001f, 0.5f, 0.3f, 0.01f};
    CHECK(kv_controller_tau(0.022, 4096.0, 16384.0) == 0.044);
    CHECK(isnan(kv_controller_tau(0.022, 4096.0, 0.0)));
    CHECK(kv_controller_create(2, init, 0.1, 0.022, 4096.0, &c) == KV_OK && c != NULL);
    if (c == NULL) return;
    CHECK(kv_controller_state(c, ema, bits, &firings) == KV_OK);
    CHECK(bits[0] == 16 && bits[1] == 16 && firings == 0 && isnan(ema[0]));
    CHECK(kv_controller_observe(c, kl, 4096.0, bits) == KV_OK);
    CHECK(bits[0] == 2 && bits[1] == 8);
    CHECK(kv_controller_state(c, ema, NULL, &firings) == KV_OK);
    CHECK(firings == 1 && ema[0] == (double)0.01f && ema[5] == (double)0.01f);
    CHECK(kv_controller_set_frozen(c, 1) == KV_OK);
    kl[0] = 1.0f;
    CHECK(kv_controller_observe(c, kl, 4096.0, bits) == KV_OK);
    CHECK(kv_controller_state(c, ema, bits, &firings) == KV_OK);
    CHECK(firings == 1 && ema[0] == (double)0.01f && bits[0] == 2);
    kl[0] = -1.0f;
    CHECK(kv_controller_observe(c, kl, 4096.0, bits) == KV_EINVAL);
    kv_controller_destroy(c);
}

/* the device calls reject bad arguments on the host, before anything is launched */
static void device_call_arguments(void) {
    kv_geometry g = geometry();
    kv_layer_pools pools;
    memset(&pools, 0, sizeof pools);
    CHECK(kv_decode_attn(&g, &pools, NULL, NULL, 0, 0, NULL, 0.125f, NULL, NULL, 0, 0, NULL)
          == KV_EINVAL);
    CHECK(strstr(kv_last_error(), "batch 0") != NULL);
    CHECK(kv_quant_write(&g, &pools, NULL, NULL, 0, 0, NULL, NULL, NULL, NULL) == KV_OK);
    CHECK(kv_canary_kl(&g, NULL, NULL, 0, NULL, 0.125f, NULL, NULL, NULL, 0, NULL) == KV_EINVAL);
    CHECK(kv_decode_workspace_bytes(&g, 2, 128, 2) > 0);
    CHECK(kv_decode_pages_per_split(&g, 2, 128) >= 2);
    CHECK(kv_decode_pages_per_split(&g, 2, 128) % 2 == 0);
    g.head_dim = 96;
    CHECK(kv_decode_workspace_bytes(&g, 2, 128, 2) == 0);
}

int main(void) {
    sizes_and_handles();
    validation();
    allocator();
    allocator_full();
    controller();
    device_call_arguments();
    printf("%d failures\n", failures);
    return failures;
}
