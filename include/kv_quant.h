/*
 * kv_quant.h -- C ABI of libkvq: single-token decode over a paged KV cache stored as packed
 * symmetric INT2 / INT4 / INT8 codes (or plain FP16) with a bit-width chosen per layer, for AMD
 * MI355X (gfx950).
 *
 * The operations follow three web pages on mixed-precision KV-cache quantization:
 *   [EchoKV]  "EchoKV: watching a language model decide its own precision"
 *   [RoleKV]  "Behavior-Guided KV-Cache Quantization"
 *   [Kaizen]  "KV-Kaizen: Learning Context-Adaptive Cache Compression Choices" (summary)
 *
 * Conventions for every call:
 *   - Plain C99 types only. fp16 values travel as uint16_t bit patterns.
 *   - "dev" pointers are HIP device memory owned by the caller; the library never allocates,
 *     frees or retains device memory. "host" pointers are ordinary host memory.
 *   - Kernel calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL = the null
 *     stream). The caller synchronizes before reading results on the host.
 *   - Every argument is checked on the host before anything is launched; on error the call
 *     returns a nonzero kv_status, launches nothing and changes nothing. kv_last_error() then
 *     holds a one-line description (thread-local). Contents of device buffers (block handles,
 *     lengths) are not checked on the hot path: out-of-range contents give undefined results.
 *   - Inputs are finite fp16 values; a product |q_c| * max|K_c| / qmax beyond the fp16 range is
 *     outside the supported domain.
 *
 * Storage format (the pages fix none of it; it is this library's):
 *   tier 0, 1, 2  <->  b = 2, 4, 8 bits;  qmax_b = 2^(b-1) - 1;  codes q in [-qmax_b, qmax_b].
 *   block handle = (tier << 30) | block_index;  KV_NO_BLOCK = 0xFFFFFFFF.
 *   One block = one page of P tokens of one layer, all KV heads: H_kv sections of
 *   S_b = P*D*b/4 + 2*D + 2*P bytes (head h at h*S_b); block j of a tier pool is at j*H_kv*S_b.
 *   A section holds, in order:
 *     K codes  P*D*b/8 bytes, code sequence index of (token t, channel c) = t*D + c
 *     K scales D fp16, one per channel over the page's tokens      ([RoleKV] keys per channel)
 *     V codes  P*D*b/8 bytes, code sequence index of (t, c) = ((t/4)*D + c)*4 + t%4
 *     V scales P fp16, one per token over its D channels           ([RoleKV] values per token)
 *   A code sequence is stored as little-endian 32-bit words of 32/b codes; code k of a word is
 *   the unsigned field q + 2^(b-1) at bit 16*(k%2) + b*(k/2). Token slots of a page that hold
 *   no token carry the zero code and a zero scale.
 *   tier 3 <-> b = 16, plain FP16 ([EchoKV] "How EchoKV works": a layer starts at FP16 before
 *   the canary first fires): S_16 = 4*P*D bytes, K values [P][D] (index t*D + c) then V values
 *   at index ((t/4)*D + c)*4 + t%4, no scales; token slots that hold no token are +0.
 *   Quantizer over a group with absolute maximum a: scale s = smallest fp16 >= a/qmax_b
 *   (0 if a == 0), code = round-half-even(x/s); both decided in IEEE binary32, which equals the
 *   exact rational result for fp16 inputs ([Kaizen] "symmetric uniform quantization").
 * Asymmetric format (kv_geometry.asymmetric = 1; [EchoKV] "Future work": the paged cache
 *   itself held at INT2/4/8 in KIVI's form, with the KIVI-style quantizer of "Show the math"):
 *   the same groups; a section of S_b = P*D*b/4 + 4*D + 4*P bytes holds K codes, K zero points
 *   (D fp16), K scales (D fp16), V codes, V zero points (P fp16), V scales (P fp16). A group
 *   with minimum m and maximum M gets the zero point m (+0 for a zero minimum), the scale
 *   s = smallest fp16 >= (M - m)/(2^b - 1) (0 if M == m) and codes u = round-half-even((x - m)/s)
 *   in [0, 2^b - 1], decided in IEEE binary64 (exact for fp16 inputs); the field of a code is u
 *   itself and an element is m + u*s. Empty token slots carry u = 0, zero point 0, scale 0.
 *   The FP16 tier and the block handles are the same in both formats.
 */
#ifndef KV_QUANT_H
#define KV_QUANT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KV_ABI_VERSION 3
#define KV_NUM_TIERS 4          /* INT2, INT4, INT8, FP16 */
#define KV_NO_BLOCK 0xFFFFFFFFu

typedef enum {
    KV_OK = 0,
    KV_EINVAL = 1,        /* an argument is out of range or a pointer is NULL */
    KV_ENOBLOCKS = 2,     /* a tier pool has too few free blocks (allocator unchanged) */
    KV_EUNSUPPORTED = 3,  /* valid but not built: head_dim not 64/128, GQA group > 16, ... */
    KV_EHIP = 4           /* the HIP runtime reported an error; see kv_last_error() */
} kv_status;

typedef struct {
    int32_t num_layers;
    int32_t num_q_heads;        /* H_q; a multiple of num_kv_heads, group H_q/H_kv <= 16 */
    int32_t num_kv_heads;       /* H_kv */
    int32_t head_dim;           /* D: 64 or 128 */
    int32_t page_size;          /* P: 16 */
    int32_t ring_size;          /* R: FP16 key ring per sequence, a multiple of P, P..128 */
    int32_t max_seqs;           /* rows of a block table / ring */
    int32_t max_pages_per_seq;  /* columns of a block table */
    int32_t asymmetric;         /* 0: symmetric codes (the format above); 1: the asymmetric
                                   format below, for every INT tier of every layer */
} kv_geometry;

/* the tier pools of one layer: base[t] holds capacity[t] blocks of kv_block_bytes(g, b_t),
   b = 2, 4, 8, 16 for t = 0..3; each base is 16-byte aligned device memory (or NULL with
   capacity 0) */
typedef struct {
    void* base[KV_NUM_TIERS];
    uint32_t capacity[KV_NUM_TIERS];
} kv_layer_pools;

/* ---------------------------------------------------------------- version, errors, sizes */
int         kv_abi_version(void);
const char* kv_strerror(kv_status status);
const char* kv_last_error(void);                    /* thread-local; "" when none */
kv_status   kv_validate(const kv_geometry* g);
uint32_t    kv_handle(int bits, uint32_t index);     /* bits 2,4,8,16; KV_NO_BLOCK if invalid */
size_t      kv_block_bytes(const kv_geometry* g, int bits);  /* one block, all KV heads; 0 if invalid */
size_t      kv_ring_bytes(const kv_geometry* g);    /* one layer's ring: max_seqs*R*H_kv*D*2 */
/* bytes of cache per token over all layers, bits_per_layer[l] in {2,4,8} or 16 (plain fp16);
   [Kaizen] "Action Space and Cost Model": C0 = L*2*n_kv*d_h*16 bits for the fp16 cache */
double      kv_cache_bytes_per_token(const kv_geometry* g, const int* bits_per_layer);

/* ---------------------------------------------------------------- tier / block-table setup
 * Host-side block allocator ([EchoKV] "How EchoKV works": the tier vector routes future blocks
 * to the right pool; "What happens to old blocks...": already-allocated blocks keep their
 * admit-time width). One pool per (layer, tier); each hands out its blocks in a seeded random
 * order (shuffled physical block tables). Not thread-safe; the library owns the object.
 * The allocator and the controller below hold host memory only; a call that finds none left
 * returns KV_EINVAL and changes nothing.
 * Block tables are host arrays bt_host[L][max_seqs][max_pages_per_seq] of handles; the caller
 * copies the rows it needs to the device (one [max_seqs][max_pages_per_seq] table per layer). */
typedef struct kv_alloc kv_alloc;

/* capacity[l*KV_NUM_TIERS + t] blocks in pool (l, t); bits[l] in {2,4,8,16} is layer l's current
   width (the tier its new blocks come from) */
kv_status kv_alloc_create(const kv_geometry* g, const uint32_t* capacity, const int* bits,
                          uint64_t shuffle_seed, kv_alloc** out);
/* forward-only: later pages of the layer come from the new tier's pool; existing blocks,
   including the page being filled, keep their tier */
kv_status kv_alloc_set_layer_bits(kv_alloc* a, int layer, int bits);
/* grow sequence `seq` to new_len tokens in every layer (all-or-nothing: KV_ENOBLOCKS leaves
   the allocator and bt_host untouched); writes the new handles into bt_host */
kv_status kv_alloc_extend(kv_alloc* a, int seq, int32_t new_len, uint32_t* bt_host);
/* return every block of `seq` to its pool and reset its bt_host rows to KV_NO_BLOCK; the
   allocator keeps its own record of the handles it handed out and returns those, whatever
   bt_host holds */
kv_status kv_alloc_free_seq(kv_alloc* a, int seq, uint32_t* bt_host);
int32_t   kv_alloc_seq_len(const kv_alloc* a, int seq);              /* -1 if seq invalid */
int64_t   kv_alloc_free_blocks(const kv_alloc* a, int layer, int bits); /* -1 if invalid */
int       kv_alloc_layer_bits(const kv_alloc* a, int layer);          /* 0 if invalid */
void      kv_alloc_destroy(kv_alloc* a);
/* CPU check of a host block table against the allocator: every page below the sequence
   length holds the handle the allocator handed out for it (so no block appears twice), every
   other entry is KV_NO_BLOCK */
kv_status kv_check_block_table(const kv_alloc* a, const uint32_t* bt_host);

/* ---------------------------------------------------------------- controller (host)
 * [EchoKV] "Show the math - what the canary actually computes": every canary firing gives one
 * KL reading per (layer, width b in {2,4,8}); each goes into its own exponential moving average
 * EMA <- (1 - alpha) EMA + alpha * reading (alpha = 0.1 on the page), and each layer's width
 * becomes the least b whose EMA is below tau(L) = tau0 * sqrt(L / L0) (tau0 = 0.022 at
 * L0 = 4096, "The tau(L) scaling"; L is the context length), chosen again at every firing
 * ("Bidirectional adjustment"). "Measurement protocol - warmup, freeze, measure": a frozen
 * controller ignores readings. Readings of the silent points: a pair's first reading starts its
 * EMA; no width under the budget gives INT8; before its first firing a layer keeps its initial
 * width. EMAs are binary64, each update two IEEE products and one sum (no contraction).
 * A host object owned by the library; not thread-safe. */
typedef struct kv_controller kv_controller;

/* budget tau0 * sqrt(context_len / l0); NaN unless all three are > 0 */
double    kv_controller_tau(double tau0, double l0, double context_len);
/* initial_bits[num_layers] in {2,4,8,16}; alpha in (0,1]; tau0, l0 > 0 and finite */
kv_status kv_controller_create(int num_layers, const int* initial_bits, double alpha, double tau0,
                               double l0, kv_controller** out);
/* one firing: kl_host[num_layers][3] = the readings of widths 2, 4, 8 (finite, >= 0; e.g. the
   kl_out of kv_canary_kl for each layer, copied to the host); context_len > 0 sets the budget
   (for a batch, the mean length of its sequences: the readings are means over its rows).
   Writes the widths to bits_out[num_layers] when it is not NULL. A rejected call changes
   nothing. */
kv_status kv_controller_observe(kv_controller* c, const float* kl_host, double context_len,
                                int* bits_out);
kv_status kv_controller_set_frozen(kv_controller* c, int frozen);
/* any output may be NULL: ema[num_layers][3] (NaN before a pair's first reading),
   bits[num_layers], firings (readings taken while not frozen) */
kv_status kv_controller_state(const kv_controller* c, double* ema, int* bits, int64_t* firings);
/* route later blocks of every layer to its current width (kv_alloc_set_layer_bits for each
   layer); all-or-nothing: KV_EINVAL if the layer counts differ, KV_EUNSUPPORTED if a width has
   no pool */
kv_status kv_controller_apply(const kv_controller* c, kv_alloc* a);
void      kv_controller_destroy(kv_controller* c);

/* ---------------------------------------------------------------- quantize-on-write
 * [EchoKV] "How EchoKV works": each step's key is written into the layer's FP16 ring before it
 * is quantized into the paged cache. [RoleKV] "K/V Role-Aware Low-Bit Quantization": keys per
 * channel, values per token; "Online inference": write quantized KV = pack and store.
 *
 * One layer, `batch` sequences (rows 0..batch-1 of bt, pos, ring), n_new tokens each:
 *   bt     dev uint32 [max_seqs][max_pages_per_seq]  handles; every page touched must be allocated
 *   pos    dev int32  [batch]      tokens already cached in each sequence
 *   k_new, v_new  dev fp16 [batch][n_new][H_kv][D] (16-byte aligned)
 *   ring   dev fp16 [max_seqs][R][H_kv][D] (16-byte aligned), in/out: position p lives in slot p % R
 * For every page touched, the K scales and codes of all its present tokens are recomputed from
 * their FP16 originals (ring for positions < pos, k_new after), so writing token by token gives
 * the same bytes as writing at once. Each new value vector gets its own scale; codes of earlier
 * tokens are kept. Afterwards the ring holds the new keys. batch is 0 .. max_seqs; batch == 0
 * or n_new == 0 is a no-op. A geometry with asymmetric = 1 writes the asymmetric format (a zero
 * point and a scale per group). */
kv_status kv_quant_write(const kv_geometry* g, const kv_layer_pools* pools, const uint32_t* bt,
                         const int32_t* pos, int batch, int n_new, const uint16_t* k_new,
                         const uint16_t* v_new, uint16_t* ring, void* stream);

/* ---------------------------------------------------------------- decode attention
 * [EchoKV] "What happens to old blocks...": paged attention reads each block at its stored
 * width, so one layer may mix widths. [RoleKV] "Storage savings": GQA head mapping; query head
 * h reads KV head h / (H_q/H_kv).
 *   out[s][h][:] = sum_t w_t V^_t / sum_t w_t,  w_t = exp(l_t - max l),
 *   l_t = softmax_scale * sum_c q[s][h][c] K^_t[c],  t in [0, ctx_len[s]),
 *   K^_t[c] = code * K scale of (page of t, c),  V^_t[c] = code * V scale of t
 *   (asymmetric format: zero point + code * scale, with the same groups).
 *   batch    1 .. max_seqs (rows 0..batch-1 of bt and ctx_len); 0 is KV_EINVAL
*   ctx_len  dev int32 [batch], each in [0, max_ctx_len]; a zero length gives a zero row
 *   q        dev fp16 [batch][H_q][D] (4-byte aligned);  out  dev fp32 [batch][H_q][D] (16-byte aligned)
 *   max_ctx_len    host upper bound on ctx_len, sizes the launch (<= max_pages_per_seq * P)
 *   softmax_scale  finite, of either sign (0 gives the mean of V^ over the context); a NaN or
 *                  infinite scale is KV_EINVAL
 *   pages_per_split  pages one workgroup reads (even, >= 2); 0 = chosen by the library
 *   workspace  dev, >= kv_decode_workspace_bytes(...) bytes, zero-filled before its first use;
 *              the call leaves it ready for the next call on the same geometry, whatever that
 *              call's batch and lengths (its own size requirement still applies); zero it again
 *              before using it with another geometry. One workspace per in-flight call.
 * The split-K partials are merged in a fixed order, so results are bitwise reproducible. */
size_t    kv_decode_workspace_bytes(const kv_geometry* g, int batch, int max_ctx_len,
                                    int pages_per_split);
/* The library's split plan when only the longest length is known: about one workgroup per
 * compute unit for a batch of equal lengths, at most 512 pages per split. Returns 0 on invalid
 * arguments. */
int       kv_decode_pages_per_split(const kv_geometry* g, int batch, int max_ctx_len);
/* The split plan for known lengths (host int32 [batch], each >= 0; not retained): the plan of
 * kv_decode_pages_per_split for the longest length when the lengths are nearly equal (mean at
 * least 0.9 of the maximum); otherwise splits sized so that the batch's pages make about 1.8
 * workgroups' worth per compute unit, which the hardware scheduler then balances. Returns 0 on
 * invalid arguments. */
int       kv_decode_pages_per_split_for(const kv_geometry* g, int batch, const int32_t* ctx_len_host);
kv_status kv_decode_attn(const kv_geometry* g, const kv_layer_pools* pools, const uint32_t* bt,
                         const int32_t* ctx_len, int batch, int max_ctx_len, const uint16_t* q,
                         float softmax_scale, float* out, void* workspace,
                         size_t workspace_bytes, int pages_per_split, void* stream);

/* ---------------------------------------------------------------- fused decode step
 * [EchoKV] "How EchoKV works": each step appends the new key to the ring, quantizes, then
 * attends. The write of kv_quant_write and the attention of kv_decode_attn in one launch (one per layer
 * and step): for each sequence s, n_new tokens are written at positions pos[s] .. pos[s]+n_new-1
 * exactly as kv_quant_write writes them (same bytes, same ring), and the attention then runs
 * over ctx_len = pos[s] + n_new tokens exactly as kv_decode_attn runs it (same outputs). The
 * workgroup whose split holds a touched page writes it before it reads it; no other workgroup
 * reads that page.
 *   n_new            0 .. 64 (at most five pages per sequence); 0 = attention over pos
 *   pos, k_new, v_new, ring   as for kv_quant_write (k_new, v_new, ring 16-byte aligned)
 *   max_ctx_len      host upper bound on pos[s] + n_new
 *   q, softmax_scale, out, workspace, workspace_bytes, pages_per_split   as for kv_decode_attn
 *                    (the workspace is sized by kv_decode_workspace_bytes(g, batch, max_ctx_len,
 *                    pages_per_split))
 * Errors: as for the two calls it joins; n_new outside 0..64 is KV_EINVAL. */
kv_status kv_decode_step(const kv_geometry* g, const kv_layer_pools* pools, const uint32_t* bt,
                         const int32_t* pos, int batch, int n_new, const uint16_t* k_new,
                         const uint16_t* v_new, uint16_t* ring, int max_ctx_len, const uint16_t* q,
                         float softmax_scale, float* out, void* workspace,
                         size_t workspace_bytes, int pages_per_split, void* stream);
/* kv_decode_step for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same write and attention, same
 * bytes, ring and outputs, with the workspace taken from a fixed device array inside the
 * library (16 MiB per GPU, held until the process ends) instead of an argument. The call
 * allocates nothing. Limits: batch * H_kv <= 4096, and the split partials
 * (batch*H_kv*splits*(H_q/H_kv)*(D+2)*4 bytes, about) within 15 MiB -- larger calls return
 * KV_EINVAL with the sizes in kv_last_error(). Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (two streams, two threads) race and must not be issued. The
 * first call on a device also launches a small kernel that clears the array's counters.
 * Arguments and other errors as for kv_decode_step, without workspace and workspace_bytes. */
kv_status kv_decode_step_noalloc(const kv_geometry* g, const kv_layer_pools* pools,
                                 const uint32_t* bt, const int32_t* pos, int batch, int n_new,
                                 const uint16_t* k_new, const uint16_t* v_new, uint16_t* ring,
                                 int max_ctx_len, const uint16_t* q, float softmax_scale,
                                 float* out, int pages_per_split, void* stream);
/* The split plan for a fused step whose positions are known on the host (pos_host int32
 * [batch], each >= 0; not retained; n_new as for kv_decode_step): the plan of
 * kv_decode_pages_per_split_for for the lengths pos + n_new, then -- when n_new > 0 and every
 * sequence ends in the same split -- with the same split count but longer splits, so that the
 * last split, whose workgroup also writes the step's tokens (two pages at a time, each round
 * about the loop time of 30 to 50 pages), is 40 pages per round (at most half a split) shorter
 * than the others. kv_decode_step with pages_per_split = 0 plans the same way from max_ctx_len.
 * Size the workspace with the pages_per_split the call will pass:
 * kv_decode_workspace_bytes(g, batch, max_ctx_len, pps) for this plan's pps, or with 0 for
 * pages_per_split = 0 (for a ragged batch this plan can have more splits than the plan of 0).
 * Returns 0 on invalid arguments. */
int       kv_decode_step_pages_per_split_for(const kv_geometry* g, int batch, const int32_t* pos_host,
                                             int n_new);

/* ---------------------------------------------------------------- canary
 * [EchoKV] "Show the math": delta_b = KL(softmax(Q K_ref^T) || softmax(Q quant_b(K_ref)^T)),
 * summed over keys, averaged over queries; one number per b in {2, 4, 8}. K_ref is the ring:
 * for each sequence the n = min(seq_len[s], R) newest keys (positions seq_len-n .. seq_len-1).
 * quant_b is the cache's own quantizer, grouped by each key's page (one scale per page and
 * channel): the symmetric one, or the asymmetric one (as kv_canary_kl_asym) for a geometry with
 * asymmetric = 1; the copies are temporary. Rows use the softmax_scale of attention (finite;
 * otherwise KV_EINVAL).
 *   batch    1 .. max_seqs (a mean over no rows is undefined); 0 is KV_EINVAL
 *   ring     dev fp16 [max_seqs][R][H_kv][D] (16-byte aligned);  seq_len dev int32 [batch], >= 0
 *   q        dev fp16 [batch][H_q][D] (16-byte aligned)
 *   kl_out   dev fp32 [3]: mean over batch*H_q rows for b = 2, 4, 8
 *   kl_rows  dev fp32 [batch][H_q][3] or NULL
 *   workspace dev, >= kv_canary_workspace_bytes(g, batch), zero-filled before its first use;
 *             the call leaves it ready for the next call, whatever that call's batch */
size_t    kv_canary_workspace_bytes(const kv_geometry* g, int batch);
kv_status kv_canary_kl(const kv_geometry* g, const uint16_t* ring, const int32_t* seq_len,
                       int batch, const uint16_t* q, float softmax_scale, float* kl_out,
                       float* kl_rows, void* workspace, size_t workspace_bytes, void* stream);
/* One firing for every layer in one launch ([EchoKV] "Show the math": a firing yields one
 * number per (layer, width), 3L numbers; at the page's rate of one firing per 64 steps the whole
 * pipeline is meant to cost a small fraction of a step, so it runs as one grid of
 * batch*H_kv*3*num_layers workgroups instead of num_layers launches). Layer l's readings are
 * exactly those kv_canary_kl gives for rings[l] and q[l]; all layers share seq_len (every layer
 * holds the same tokens).
 *   num_layers  1 .. min(g->num_layers, KV_CANARY_MAX_LAYERS)
 *   rings, q    HOST arrays [num_layers] of device pointers (each 16-byte aligned), read during
 *               the call and not retained: rings[l] as the ring of kv_canary_kl, q[l] [batch][H_q][D]
 *   kl_out      dev fp32 [num_layers][3];  kl_rows  dev fp32 [num_layers][batch][H_q][3] or NULL
 *   workspace   dev, >= kv_canary_layers_workspace_bytes(g, num_layers, batch) bytes, zero-filled
 *               before its first use; left ready for the next kv_canary_kl_layers call on the
 *               same geometry, whatever its batch and layer count (its ticket counters, one
 *               256-byte line per (layer, width) for min(g->num_layers, KV_CANARY_MAX_LAYERS)
 *               layers, come first and do not move)
 * Errors as for kv_canary_kl; a NULL or misaligned pointer of any layer is KV_EINVAL. */
#define KV_CANARY_MAX_LAYERS 128
size_t    kv_canary_layers_workspace_bytes(const kv_geometry* g, int num_layers, int batch);
kv_status kv_canary_kl_layers(const kv_geometry* g, int num_layers, const uint16_t* const* rings,
                              const int32_t* seq_len, int batch, const uint16_t* const* q,
                              float softmax_scale, float* kl_out, float* kl_rows, void* workspace,
                              size_t workspace_bytes, void* stream);
/* The same divergence with the temporary copies built by the asymmetric quantizer ([EchoKV]
 * "Show the math" describes its canary quantizer as asymmetric per group, in the manner of KIVI),
 * over the same groups (each ring key's page, one group per channel): zero point m = the group
 * minimum, scale s = RU16((max - m) / (2^b - 1)) (0 for a constant group), code =
 * round-half-even((x - m) / s) in [0, 2^b - 1], value m + code * s; decided in binary64, which
 * is exact for fp16 keys. Arguments, workspace and errors as for kv_canary_kl. */
kv_status kv_canary_kl_asym(const kv_geometry* g, const uint16_t* ring, const int32_t* seq_len,
                            int batch, const uint16_t* q, float softmax_scale, float* kl_out,
                            float* kl_rows, void* workspace, size_t workspace_bytes,
                            void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KV_QUANT_H */
