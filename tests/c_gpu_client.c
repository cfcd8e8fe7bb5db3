/* A C program that drives the whole path through libkvq with no Python in between: the block
 * allocator routes the pages of three ragged sequences through FP16, INT8, INT4 and INT2 pools
 * of one layer; kv_quant_write prefills each sequence in chunks, kv_decode_step writes three new
 * tokens per sequence and attends, kv_decode_attn attends again at another split plan and
 * kv_canary_kl fires the canary. Device memory comes from hipMalloc; the results are compared
 * with the oracle (libkvq_oracle) on the same inputs: pool bytes and the ring bit for bit,
 * attention rows within 2e-3 of the oracle (relative to the row's largest value), canary KL
 * within 1e-4. Prints one line per failed check and exits with the number of failures.
 * Arguments: "asym" stores the cache in the asymmetric format (zero point + scale per group);
 * "noalloc" takes the step through kv_decode_step_noalloc (no workspace argument). */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kv_quant.h"
#include "kvq_oracle.h"

#define HQ 16
#define HKV 4
#define D 128
#define P 16
#define R 64
#define SEQS 3
#define MAXP 24
#define NEW 3
#define TMAX (MAXP * P)

static int failures = 0;

#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            printf("FAIL line %d: ", __LINE__);            \
            printf(__VA_ARGS__);                           \
            printf("\n");                                  \
            ++failures;                                    \
        }                                                  \
    } while (0)

#define HIP_OK(call)                                                        \
    do {                                                                    \
        hipError_t e_ = (call);                                             \
        if (e_ != hipSuccess) {                                             \
            printf("HIP error %d at line %d: %s\n", (int)e_, __LINE__, #call); \
            exit(100);                                                      \
        }                                                                   \
    } while (0)

#define KV_OK_(call)                                                        \
    do {                                                                    \
        kv_status s_ = (call);                                              \
        if (s_ != KV_OK) {                                                  \
            printf("kv error %d at line %d: %s [%s]\n", (int)s_, __LINE__, #call, kv_last_error()); \
            exit(101);                                                      \
        }                                                                   \
    } while (0)

/* seeded inputs: splitmix64 draws turned into fp16 bit patterns with a random sign, a
 * magnitude between 2^-5 and 2^2 and a random mantissa, one value in 64 exactly zero */
static uint64_t rng_state = 20261202u;
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static uint16_t draw_f16(void) {
    const uint64_t r = next_u64();
    if ((r & 63) == 0) return 0;
    const uint16_t sign = (uint16_t)((r >> 6) & 1) << 15;
    const uint16_t expo = (uint16_t)(10 + (r >> 7) % 8);        /* biased: 2^-5 .. 2^2 */
    const uint16_t mant = (uint16_t)((r >> 16) & 0x3ff);
    return (uint16_t)(sign | (expo << 10) | mant);
}

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    HIP_OK(hipMalloc(&p, bytes ? bytes : 16));
    HIP_OK(hipMemset(p, 0, bytes ? bytes : 16));
    return p;
}

int main(int argc, char** argv) {
    const int prefill[SEQS] = {200, 17, 330};
    const int widths_in_order[4] = {16, 8, 4, 2};
    /* each sequence's length after each width's turn: its pages come from that width's pool */
    const int32_t grow[4][SEQS] = {{40, 5, 64}, {90, 10, 150}, {150, 17, 250}, {203, 20, 333}};
    kv_geometry g;
    orc_geom og;
    kv_alloc* alloc = NULL;
    uint32_t capacity[KV_NUM_TIERS];
    int layer_bits[1] = {16};
    uint32_t bt[SEQS * MAXP];
    uint16_t *K, *V, *q;
    uint8_t* opools[4];
    uint16_t* oring;
    double *oout, okl[3], orows[SEQS * HQ * 3];
    kv_layer_pools pools;
    int t, s, i, w;
    const float scale = 1.0f / sqrtf((float)D);
    int asym = 0, noalloc = 0;

    for (i = 1; i < argc; ++i) {
        if (strcmp(argv[i], "asym") == 0) asym = 1;
        else if (strcmp(argv[i], "noalloc") == 0) noalloc = 1;
        else {
            printf("unknown argument %s\n", argv[i]);
            return 102;
        }
    }
    printf("format %s, step %s\n", asym ? "asymmetric" : "symmetric",
           noalloc ? "kv_decode_step_noalloc" : "kv_decode_step");

    memset(&g, 0, sizeof g);
    g.num_layers = 1;
    g.num_q_heads = HQ;
    g.num_kv_heads = HKV;
    g.head_dim = D;
    g.page_size = P;
    g.ring_size = R;
    g.max_seqs = SEQS;
    g.max_pages_per_seq = MAXP;
    g.asymmetric = asym;
    memset(&og, 0, sizeof og);
    og.num_q_heads = HQ;
    og.num_kv_heads = HKV;
    og.head_dim = D;
    og.page_size = P;
    og.ring_size = R;
    og.asymmetric = asym;

    /* the block table: every tier gets pages, in the order FP16 -> INT8 -> INT4 -> INT2 */
    for (t = 0; t < KV_NUM_TIERS; ++t) capacity[t] = SEQS * MAXP;
    for (i = 0; i < SEQS * MAXP; ++i) bt[i] = KV_NO_BLOCK;
    KV_OK_(kv_alloc_create(&g, capacity, layer_bits, 99, &alloc));
    for (w = 0; w < 4; ++w) {
        KV_OK_(kv_alloc_set_layer_bits(alloc, 0, widths_in_order[w]));
        for (s = 0; s < SEQS; ++s) KV_OK_(kv_alloc_extend(alloc, s, grow[w][s], bt));
    }
    KV_OK_(kv_check_block_table(alloc, bt));

    /* inputs: keys and values of every position, the step's queries */
    K = malloc(sizeof(uint16_t) * SEQS * TMAX * HKV * D);
    V = malloc(sizeof(uint16_t) * SEQS * TMAX * HKV * D);
    q = malloc(sizeof(uint16_t) * SEQS * HQ * D);
    for (i = 0; i < SEQS * TMAX * HKV * D; ++i) K[i] = draw_f16();
    for (i = 0; i < SEQS * TMAX * HKV * D; ++i) V[i] = draw_f16();
    for (i = 0; i < SEQS * HQ * D; ++i) q[i] = draw_f16();

    /* device side */
    {
        const int bits_of_tier[4] = {2, 4, 8, 16};
        uint32_t* bt_d = dev_alloc(sizeof bt);
        int32_t* pos_d = dev_alloc(sizeof(int32_t) * SEQS);
        int32_t* ctx_d = dev_alloc(sizeof(int32_t) * SEQS);
        uint16_t* ring_d = dev_alloc(kv_ring_bytes(&g));
        uint16_t* kin_d = dev_alloc(sizeof(uint16_t) * SEQS * TMAX * HKV * D);
        uint16_t* vin_d = dev_alloc(sizeof(uint16_t) * SEQS * TMAX * HKV * D);
        uint16_t* q_d = dev_alloc(sizeof(uint16_t) * SEQS * HQ * D);
        float* out_d = dev_alloc(sizeof(float) * SEQS * HQ * D);
        float* out2_d = dev_alloc(sizeof(float) * SEQS * HQ * D);
        float* kl_d = dev_alloc(sizeof(float) * 3);
        float* rows_d = dev_alloc(sizeof(float) * SEQS * HQ * 3);
        int32_t pos[SEQS], ctx[SEQS];
        int max_ctx = 0;
        size_t ws_bytes, ws2_bytes, cws_bytes;
        void *ws_d, *ws2_d, *cws_d;
        float* out = malloc(sizeof(float) * SEQS * HQ * D);
        float* out2 = malloc(sizeof(float) * SEQS * HQ * D);
        float kl[3], rows[SEQS * HQ * 3];
        uint8_t* got_pool;
        uint16_t* got_ring;

        for (t = 0; t < 4; ++t) {
            pools.base[t] = dev_alloc(capacity[t] * kv_block_bytes(&g, bits_of_tier[t]));
            pools.capacity[t] = capacity[t];
        }
        HIP_OK(hipMemcpy(bt_d, bt, sizeof bt, hipMemcpyHostToDevice));
        /* per sequence, position-major copies of its tokens: [TMAX][HKV][D] each */
        HIP_OK(hipMemcpy(kin_d, K, sizeof(uint16_t) * SEQS * TMAX * HKV * D, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(vin_d, V, sizeof(uint16_t) * SEQS * TMAX * HKV * D, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(q_d, q, sizeof(uint16_t) * SEQS * HQ * D, hipMemcpyHostToDevice));

        /* prefill: each sequence in two chunks, through its own rows of bt, pos and ring */
        for (s = 0; s < SEQS; ++s) {
            const int cut = prefill[s] / 3;
            const int bounds[3] = {0, cut, prefill[s]};
            int c;
            for (c = 0; c < 2; ++c) {
                const int32_t p0 = bounds[c];
                const int n = bounds[c + 1] - bounds[c];
                const size_t tok = ((size_t)s * TMAX + p0) * HKV * D;
                HIP_OK(hipMemcpy(pos_d + s, &p0, sizeof p0, hipMemcpyHostToDevice));
                KV_OK_(kv_quant_write(&g, &pools, bt_d + s * MAXP, pos_d + s, 1, n, kin_d + tok,
                                      vin_d + tok, ring_d + (size_t)s * R * HKV * D, NULL));
                HIP_OK(hipDeviceSynchronize());
            }
        }
        /* the step: NEW tokens per sequence, written and attended in one launch; the step's
           keys and values are packed [SEQS][NEW][HKV][D] */
        {
            uint16_t* knew = malloc(sizeof(uint16_t) * SEQS * NEW * HKV * D);
            uint16_t* vnew = malloc(sizeof(uint16_t) * SEQS * NEW * HKV * D);
            uint16_t* knew_d = dev_alloc(sizeof(uint16_t) * SEQS * NEW * HKV * D);
            uint16_t* vnew_d = dev_alloc(sizeof(uint16_t) * SEQS * NEW * HKV * D);
            for (s = 0; s < SEQS; ++s) {
                memcpy(knew + (size_t)s * NEW * HKV * D, K + ((size_t)s * TMAX + prefill[s]) * HKV * D,
                       sizeof(uint16_t) * NEW * HKV * D);
                memcpy(vnew + (size_t)s * NEW * HKV * D, V + ((size_t)s * TMAX + prefill[s]) * HKV * D,
                       sizeof(uint16_t) * NEW * HKV * D);
                pos[s] = prefill[s];
                ctx[s] = prefill[s] + NEW;
                if (ctx[s] > max_ctx) max_ctx = ctx[s];
            }
            HIP_OK(hipMemcpy(knew_d, knew, sizeof(uint16_t) * SEQS * NEW * HKV * D, hipMemcpyHostToDevice));
            HIP_OK(hipMemcpy(vnew_d, vnew, sizeof(uint16_t) * SEQS * NEW * HKV * D, hipMemcpyHostToDevice));
            HIP_OK(hipMemcpy(pos_d, pos, sizeof pos, hipMemcpyHostToDevice));
            HIP_OK(hipMemcpy(ctx_d, ctx, sizeof ctx, hipMemcpyHostToDevice));
            ws_bytes = kv_decode_workspace_bytes(&g, SEQS, max_ctx, 0);
            CHECK(ws_bytes > 0, "workspace size");
            ws_d = dev_alloc(ws_bytes);
            if (noalloc)
                KV_OK_(kv_decode_step_noalloc(&g, &pools, bt_d, pos_d, SEQS, NEW, knew_d, vnew_d,
                                              ring_d, max_ctx, q_d, scale, out_d, 0, NULL));
            else
                KV_OK_(kv_decode_step(&g, &pools, bt_d, pos_d, SEQS, NEW, knew_d, vnew_d, ring_d,
                                      max_ctx, q_d, scale, out_d, ws_d, ws_bytes, 0, NULL));
            HIP_OK(hipDeviceSynchronize());
            HIP_OK(hipFree(knew_d));
            HIP_OK(hipFree(vnew_d));
            free(knew);
            free(vnew);
        }
        /* attention again, two pages per split; and the canary over the rings */
        ws2_bytes = kv_decode_workspace_bytes(&g, SEQS, max_ctx, 2);
        ws2_d = dev_alloc(ws2_bytes);
        KV_OK_(kv_decode_attn(&g, &pools, bt_d, ctx_d, SEQS, max_ctx, q_d, scale, out2_d, ws2_d,
                              ws2_bytes, 2, NULL));
        cws_bytes = kv_canary_workspace_bytes(&g, SEQS);
        cws_d = dev_alloc(cws_bytes);
        KV_OK_(kv_canary_kl(&g, ring_d, ctx_d, SEQS, q_d, scale, kl_d, rows_d, cws_d, cws_bytes,
                            NULL));
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(out, out_d, sizeof(float) * SEQS * HQ * D, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(out2, out2_d, sizeof(float) * SEQS * HQ * D, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(kl, kl_d, sizeof kl, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(rows, rows_d, sizeof rows, hipMemcpyDeviceToHost));

        /* the oracle on the same inputs, the same chunks and the same block table */
        oring = calloc((size_t)SEQS * R * HKV * D, sizeof(uint16_t));
        for (t = 0; t < 4; ++t)
            opools[t] = calloc(capacity[t] * orc_block_bytes(&og, bits_of_tier[t]), 1);
        for (s = 0; s < SEQS; ++s) {
            const int cut = prefill[s] / 3;
            const int bounds[4] = {0, cut, prefill[s], prefill[s] + NEW};
            int c;
            for (c = 0; c < 3; ++c) {
                const int32_t p0 = bounds[c];
                const size_t tok = ((size_t)s * TMAX + p0) * HKV * D;
                CHECK(orc_quant_write(&og, opools, bt + s * MAXP, MAXP, &p0, 1, bounds[c + 1] - p0,
                                      K + tok, V + tok, oring + (size_t)s * R * HKV * D) == 0,
                      "oracle write");
            }
        }
        oout = malloc(sizeof(double) * SEQS * HQ * D);
        CHECK(orc_decode_attn(&og, opools, bt, MAXP, ctx, SEQS, q, scale, oout) == 0, "oracle attention");
        orc_canary_kl(&og, oring, ctx, SEQS, q, scale, okl, orows);

        /* bytes: every pool and the ring, bit for bit */
        for (t = 0; t < 4; ++t) {
            const size_t nb = capacity[t] * kv_block_bytes(&g, bits_of_tier[t]);
            got_pool = malloc(nb);
            HIP_OK(hipMemcpy(got_pool, pools.base[t], nb, hipMemcpyDeviceToHost));
            CHECK(nb == capacity[t] * orc_block_bytes(&og, bits_of_tier[t]), "pool %d size", t);
            CHECK(memcmp(got_pool, opools[t], nb) == 0, "pool of %d-bit blocks differs", bits_of_tier[t]);
            free(got_pool);
        }
        got_ring = malloc(kv_ring_bytes(&g));
        HIP_OK(hipMemcpy(got_ring, ring_d, kv_ring_bytes(&g), hipMemcpyDeviceToHost));
        CHECK(memcmp(got_ring, oring, kv_ring_bytes(&g)) == 0, "ring differs");
        free(got_ring);

        /* attention rows (both launches) and the canary */
        {
            double worst = 0.0, worst2 = 0.0;
            for (i = 0; i < SEQS * HQ; ++i) {
                double ref_max = 0.0, err = 0.0, err2 = 0.0;
                int c;
                for (c = 0; c < D; ++c) {
                    const double r = oout[(size_t)i * D + c];
                    if (fabs(r) > ref_max) ref_max = fabs(r);
                    if (fabs(out[(size_t)i * D + c] - r) > err) err = fabs(out[(size_t)i * D + c] - r);
                    if (fabs(out2[(size_t)i * D + c] - r) > err2) err2 = fabs(out2[(size_t)i * D + c] - r);
                }
                if (ref_max > 0) {
                    err /= ref_max;
                    err2 /= ref_max;
                }
                if (err > worst) worst = err;
                if (err2 > worst2) worst2 = err2;
            }
            printf("attention: max row err %.3e (fused step), %.3e (attention, 2 pages per split)\n",
                   worst, worst2);
            CHECK(worst <= 2e-3, "fused step rows off by %.3e", worst);
            CHECK(worst2 <= 2e-3, "attention rows off by %.3e", worst2);
        }
        {
            double worst = 0.0;
            for (i = 0; i < 3; ++i)
                if (fabs(kl[i] - okl[i]) > worst) worst = fabs(kl[i] - okl[i]);
            for (i = 0; i < SEQS * HQ * 3; ++i)
                if (fabs(rows[i] - orows[i]) > worst) worst = fabs(rows[i] - orows[i]);
            printf("canary: kl %.6f %.6f %.6f (oracle %.6f %.6f %.6f), max err %.3e\n", kl[0],
                   kl[1], kl[2], okl[0], okl[1], okl[2], worst);
            CHECK(worst <= 1e-4, "canary off by %.3e", worst);
            CHECK(okl[0] >= okl[1] && okl[1] >= okl[2], "wider copies should not diverge more");
        }

        for (t = 0; t < 4; ++t) {
            HIP_OK(hipFree(pools.base[t]));
            free(opools[t]);
        }
        HIP_OK(hipFree(bt_d));
        HIP_OK(hipFree(pos_d));
        HIP_OK(hipFree(ctx_d));
        HIP_OK(hipFree(ring_d));
        HIP_OK(hipFree(kin_d));
        HIP_OK(hipFree(vin_d));
        HIP_OK(hipFree(q_d));
        HIP_OK(hipFree(out_d));
        HIP_OK(hipFree(out2_d));
        HIP_OK(hipFree(kl_d));
        HIP_OK(hipFree(rows_d));
        HIP_OK(hipFree(ws_d));
        HIP_OK(hipFree(ws2_d));
        HIP_OK(hipFree(cws_d));
        free(out);
        free(out2);
        free(oout);
        free(oring);
    }
    kv_alloc_destroy(alloc);
    free(K);
    free(V);
    free(q);
    printf("%d failures\n", failures);
    return failures;
}
