/*
 * kvq_oracle.h -- plain CPU oracle for per-layer mixed-precision quantized KV-cache decode.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library includes, links or calls this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg load it. It shares no code,
 * header, table or constant with the GPU library.
 *
 * What it computes (sources are the three web pages studied for this project):
 *   - EchoKV (jaizunt.github.io/echokv.html), "How EchoKV works": every decode step the key is
 *     first goes to the layer's FP16 ring (its 64 newest keys), and only then is it quantized
 *     into the paged cache; "What happens to old blocks...": a block keeps the bit-width it was admitted with and
 *     paged attention reads each block at its stored width; "Show the math": the canary
 *     KL(softmax(Q K^T) || softmax(Q quant_b(K)^T)), summed over keys, averaged over queries,
 *     one number per (layer, b) for b in {2,4,8}.
 *   - Behavior-Guided KV-Cache Quantization, "K/V Role-Aware Low-Bit Quantization": keys are
 *     quantized per channel, values per token; symmetric integer codes; "Storage savings":
 *     packed low-bit storage, GQA head mapping.
 *   - KV-Kaizen summary, "Three Non-Eviction Compression Axes" (symmetric uniform quantization)
 *     and "Action Space and Cost Model" (C0 = L * 2 * n_kv * d_h * 16 bits per token).
 *
 * Everything real-valued is computed in double. The one place where floating point decides an
 * integer (a quantizer's scale and codes) is computed in IEEE binary32, the precision the GPU
 * kernels take the same decision in; tests pin that binary32 decision to exact rational
 * arithmetic over the whole fp16 domain.
 *
 * Storage format (the pages fix none; this is the library's format, described in words so a
 * reader can check the code against it):
 *   tier index 0,1,2 <-> b = 2,4,8 bits;  qmax_b = 2^(b-1) - 1;  code q in [-qmax_b, qmax_b].
 *   block handle = (tier << 30) | block_index;  0xFFFFFFFF = no block.
 *   A block holds one page (P tokens) of one layer for all KV heads: H_kv sections of
 *   S_b = P*D*b/4 + 2*D + 2*P bytes, KV head h at byte h*S_b.  Block j of a tier pool is at
 *   byte j*H_kv*S_b.  A section is, in order:
 *     K codes  (P*D*b/8 bytes): code sequence index of (token t, channel c) = t*D + c
 *     K scales (D fp16):        one per channel, over the page's tokens
 *     V codes  (P*D*b/8 bytes): code sequence index of (t, c) = ((t/4)*D + c)*4 + t%4
 *     V scales (P fp16):        one per token, over its D channels
 *   A code sequence is stored as 32-bit little-endian words of 32/b codes; code k of a word
 *   (k = i mod 32/b) is the unsigned field u = q + 2^(b-1) at bit 16*(k%2) + b*(k/2).
 *   Token slots of a page that hold no token yet carry the zero code and a zero scale.
 *   tier 3 <-> b = 16, plain FP16 (EchoKV, "How EchoKV works": a layer's initial state before
 *   the canary first fires): a section is 4*P*D bytes, the keys at index t*D + c then the values
 *   at index ((t/4)*D + c)*4 + t%4, fp16 each, no scales; empty slots are +0.
 * Asymmetric format (geometry flag `asymmetric`; EchoKV, "Future work": the paged cache itself
 *   held at INT2/4/8 in KIVI's asymmetric form): the same groups (K per page and channel, V per
 *   token) with the asymmetric quantizer below; a section is S_b = P*D*b/4 + 4*D + 4*P bytes:
 *     K codes, K zero points (D fp16), K scales (D fp16), V codes, V zero points (P fp16),
 *     V scales (P fp16);
 *   the field of a code is the code u in [0, 2^b - 1] itself, and an element is z + u * s.
 *   Empty token slots carry u = 0 and a zero scale and zero point.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int num_q_heads;   /* H_q */
    int num_kv_heads;  /* H_kv; H_q % H_kv == 0 */
    int head_dim;      /* D */
    int page_size;     /* P */
    int ring_size;     /* R, a multiple of P */
    int asymmetric;    /* 0: symmetric codes; 1: the asymmetric format (zero point + scale) */
} orc_geom;

/* ---- fp16 ---- */
double   orc_f16_to_f64(uint16_t h);          /* exact, subnormals included */
uint16_t orc_f64_to_f16_rne(double x);        /* round to nearest, ties to even */
uint16_t orc_f64_to_f16_ru(double x);         /* smallest fp16 >= x (x >= 0) */

/* ---- quantizer over one group of n fp16 values (elements x[i*stride]) ---- */
void orc_quantize_group(const uint16_t* x, int n, ptrdiff_t stride, int bits,
                        uint16_t* scale_out, int* codes_out);

/* ---- asymmetric (KIVI-style) quantizer over one group: zero point = the group minimum m (its
 * fp16 bits, +0 for a zero minimum), scale s = RU16((max - m) / (2^b - 1)) (0 for a constant
 * group), codes round-half-even((x - m) / s) in [0, 2^b - 1]; value m + code * s ---- */
void orc_quantize_group_asym(const uint16_t* x, int n, ptrdiff_t stride, int bits,
                             uint16_t* scale_out, uint16_t* zero_out, int* codes_out);

/* ---- packing of a code sequence ---- */
void orc_pack(const int* q, int n, int bits, uint8_t* out);   /* n a multiple of 32/bits */
void orc_unpack(const uint8_t* in, int n, int bits, int* q);

/* ---- layout ---- */
int    orc_bits_of_tier(int tier);
size_t orc_section_bytes(const orc_geom* g, int bits);
size_t orc_block_bytes(const orc_geom* g, int bits);
/* decode one K or V code / scale of a section (test helpers) */
int    orc_k_code(const orc_geom* g, const uint8_t* sec, int bits, int t, int c);
int    orc_v_code(const orc_geom* g, const uint8_t* sec, int bits, int t, int c);
double orc_k_scale(const orc_geom* g, const uint8_t* sec, int bits, int c);
double orc_v_scale(const orc_geom* g, const uint8_t* sec, int bits, int t);
double orc_k_zero(const orc_geom* g, const uint8_t* sec, int bits, int c);   /* 0 if symmetric */
double orc_v_zero(const orc_geom* g, const uint8_t* sec, int bits, int t);   /* 0 if symmetric */

/* ---- quantize-on-write: one layer, `batch` sequences, n_new tokens each ----
 * pools[tier]: host copies of the four tier pools (INT2, INT4, INT8, FP16); bt: [batch][max_pages] handles;
 * pos[s]: tokens already cached; k_new, v_new: [batch][n_new][H_kv][D] fp16 bits;
 * ring: [batch][R][H_kv][D] fp16 bits, updated in place.  Returns 0, or -1 on a bad handle. */
int orc_quant_write(const orc_geom* g, uint8_t* const pools[4], const uint32_t* bt, int max_pages,
                    const int32_t* pos, int batch, int n_new,
                    const uint16_t* k_new, const uint16_t* v_new, uint16_t* ring);

/* ---- dequantized cache of one (sequence, kv head): K, V as [n][D] doubles (for the
 * asymmetric format, zero point + code * scale) ---- */
int orc_dequant_kv(const orc_geom* g, uint8_t* const pools[4], const uint32_t* bt_row, int n,
                   int kv, double* K, double* V);

/* ---- decode attention: out [batch][H_q][D] in double ---- */
int orc_decode_attn(const orc_geom* g, uint8_t* const pools[4], const uint32_t* bt, int max_pages,
                    const int32_t* ctx_len, int batch, const uint16_t* q, float softmax_scale,
                    double* out);
/* one output row (sequence s, query head h); bt_row = that sequence's block table */
int orc_decode_attn_row(const orc_geom* g, uint8_t* const pools[4], const uint32_t* bt_row,
                        int ctx_len, const uint16_t* q_row, int h, float softmax_scale, double* out);

/* ---- canary: kl3[b] = mean over batch*H_q rows of KL(P_ref || P_b), b = 2,4,8;
 * rows (optional) [batch][H_q][3]. ring [batch][R][H_kv][D]; q [batch][H_q][D]. The copies are
 * built with the cache's own quantizer (asymmetric when g->asymmetric). */
void orc_canary_kl(const orc_geom* g, const uint16_t* ring, const int32_t* seq_len, int batch,
                   const uint16_t* q, float softmax_scale, double* kl3, double* rows);
/* the same with the temporary copies built by the asymmetric quantizer when asymmetric != 0
 * (EchoKV describes its canary quantizer as asymmetric per group, after KIVI); same groups */
void orc_canary_kl_mode(const orc_geom* g, const uint16_t* ring, const int32_t* seq_len, int batch,
                        const uint16_t* q, float softmax_scale, int asymmetric, double* kl3,
                        double* rows);
/* KL of two logit vectors, in the log-sum-exp form used by the canary (test helper) */
double orc_kl_logits(const double* l, const double* m, int n);

/* ---- accounting ---- */
/* bytes of cache per token over all layers; bits[l] in {2,4,8}, or 16 for a plain fp16 cache */
double orc_cache_bytes_per_token(const orc_geom* g, int num_layers, const int* bits);
/* FP16 reference ring bytes over all layers */
double orc_ring_bytes(const orc_geom* g, int num_layers);

int orc_num_threads(void);
void orc_set_num_threads(int n);   /* threads of the parallel loops; results do not depend on it */

#ifdef __cplusplus
}
#endif
#endif
