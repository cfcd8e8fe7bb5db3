/*
 * kvq_oracle.c -- plain, slow CPU oracle (test infrastructure; see kvq_oracle.h for what it
 * computes, the storage format, and the pages each function follows).
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fopenmp -fPIC -shared (no fast-math).
 * Only the outermost independent loops carry an OpenMP pragma; the arithmetic is left plain.
 */
#include "kvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------------ */
/* fp16 (IEEE binary16): 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits.              */

double orc_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = m ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

uint16_t orc_f64_to_f16_rne(double x) {
    if (isnan(x)) return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: count of 2^-24 units, rounded half to even (rint is exact here) */
        double units = rint(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)units);     /* units == 1024 is the smallest normal */
    }
    int E;
    frexp(a, &E);                                      /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                                     /* a in [2^e, 2^(e+1)) */
    double mant = rint(ldexp(a, 10 - e));              /* in [1024, 2048] */
    if (mant == 2048.0) { mant = 1024.0; e += 1; }
    int biased = e + 15;
    if (biased >= 31) return (uint16_t)(sign | 0x7c00); /* overflow to infinity */
    return (uint16_t)(sign | (biased << 10) | ((int)mant - 1024));
}

uint16_t orc_f64_to_f16_ru(double x) {
    /* smallest fp16 value >= x, for x >= 0: nearest, then one step up if it fell below x */
    uint16_t h = orc_f64_to_f16_rne(x);
    if (orc_f16_to_f64(h) < x) h = (uint16_t)(h + 1);   /* positive patterns are ordered */
    return h;
}

/* ------------------------------------------------------------------------------------------ */
/* Symmetric uniform quantizer Q_b over one group (per-channel K group, per-token V group).     */
/* Scale s = RU16(absmax / qmax), codes q = round-half-even(x / s), both decided in binary32.   */

void orc_quantize_group(const uint16_t* x, int n, ptrdiff_t stride, int bits,
                        uint16_t* scale_out, int* codes_out) {
    const int qmax = (1 << (bits - 1)) - 1;
    float absmax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float v = fabsf((float)orc_f16_to_f64(x[i * stride]));
        if (v > absmax) absmax = v;
    }
    if (absmax == 0.0f) {
        *scale_out = 0;
        for (int i = 0; i < n; ++i) codes_out[i] = 0;
        return;
    }
    float ratio = absmax / (float)qmax;                    /* binary32 division */
    uint16_t s = orc_f64_to_f16_ru((double)ratio);
    float sf = (float)orc_f16_to_f64(s);
    for (int i = 0; i < n; ++i) {
        float xf = (float)orc_f16_to_f64(x[i * stride]);
        float qf = rintf(xf / sf);                         /* binary32 division, ties to even */
        if (qf > (float)qmax) qf = (float)qmax;
        if (qf < (float)-qmax) qf = (float)-qmax;
        codes_out[i] = (int)qf;
    }
    *scale_out = s;
}

/* ------------------------------------------------------------------------------------------ */
/* Asymmetric (KIVI-style) quantizer over one group: zero point = the group minimum m, scale    */
/* s = RU16((max - m) / (2^b - 1)), codes q = round-half-even((x - m) / s) in [0, 2^b - 1],     */
/* value m + q * s.  Every step is exact in double: the difference of two fp16 values, the      */
/* quotient's rounding up to fp16 and the code's rounding are decided on values no double       */
/* rounding can move across a boundary (pinned against exact rational arithmetic).              */

void orc_quantize_group_asym(const uint16_t* x, int n, ptrdiff_t stride, int bits,
                             uint16_t* scale_out, uint16_t* zero_out, int* codes_out) {
    const int top = (1 << bits) - 1;
    double mn = 0.0, mx = 0.0;
    uint16_t mn_bits = 0;
    for (int i = 0; i < n; ++i) {
        const double v = orc_f16_to_f64(x[i * stride]);
        if (i == 0 || v < mn) { mn = v; mn_bits = x[i * stride]; }
        if (i == 0 || v > mx) mx = v;
    }
    if (n > 0 && mn == 0.0) mn_bits = 0;               /* -0 and +0 are the same zero point */
    *zero_out = mn_bits;
    const double range = mx - mn;                      /* exact: two fp16 values */
    if (range == 0.0) {
        *scale_out = 0;
        for (int i = 0; i < n; ++i) codes_out[i] = 0;
        return;
    }
    const uint16_t s = orc_f64_to_f16_ru(range / (double)top);
    const double sd = orc_f16_to_f64(s);
    for (int i = 0; i < n; ++i) {
        double q = rint((orc_f16_to_f64(x[i * stride]) - mn) / sd);
        if (q > (double)top) q = (double)top;
        if (q < 0.0) q = 0.0;
        codes_out[i] = (int)q;
    }
    *scale_out = s;
}

/* ------------------------------------------------------------------------------------------ */
/* Packing: 32/b codes per little-endian 32-bit word, code k at bit 16*(k%2) + b*(k/2).        */

static int field_bit(int k, int bits) { return 16 * (k % 2) + bits * (k / 2); }

/* fields u[i] (already unsigned) into words */
static void pack_fields(const int* u, int n, int bits, uint8_t* out) {
    const int per_word = 32 / bits;
    for (int w = 0; w < n / per_word; ++w) {
        uint32_t word = 0;
        for (int k = 0; k < per_word; ++k)
            word |= (uint32_t)u[w * per_word + k] << field_bit(k, bits);
        out[4 * w + 0] = (uint8_t)(word & 0xff);
        out[4 * w + 1] = (uint8_t)((word >> 8) & 0xff);
        out[4 * w + 2] = (uint8_t)((word >> 16) & 0xff);
        out[4 * w + 3] = (uint8_t)((word >> 24) & 0xff);
    }
}

/* symmetric codes q in [-qmax, qmax] are stored as the fields q + 2^(b-1) */
void orc_pack(const int* q, int n, int bits, uint8_t* out) {
    int* u = malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < n; ++i) u[i] = q[i] + (1 << (bits - 1));
    pack_fields(u, n, bits, out);
    free(u);
}

static int field_of(const uint8_t* in, int i, int bits) {
    const int per_word = 32 / bits;
    const int w = i / per_word, k = i % per_word;
    uint32_t word = (uint32_t)in[4 * w] | ((uint32_t)in[4 * w + 1] << 8) |
                    ((uint32_t)in[4 * w + 2] << 16) | ((uint32_t)in[4 * w + 3] << 24);
    return (int)((word >> field_bit(k, bits)) & ((1u << bits) - 1u));
}

static int unpack_one(const uint8_t* in, int i, int bits) {
    return field_of(in, i, bits) - (1 << (bits - 1));
}

void orc_unpack(const uint8_t* in, int n, int bits, int* q) {
    for (int i = 0; i < n; ++i) q[i] = unpack_one(in, i, bits);
}

/* ------------------------------------------------------------------------------------------ */
/* Layout                                                                                       */

int orc_bits_of_tier(int tier) {
    return tier == 0 ? 2 : tier == 1 ? 4 : tier == 2 ? 8 : tier == 3 ? 16 : 0;
}

static size_t code_bytes(const orc_geom* g, int bits) {
    return (size_t)g->page_size * g->head_dim * bits / 8;
}
/* bytes of the per-channel K parameters and of the per-token V parameters of a section: a
   scale each, and for the asymmetric format a zero point each before the scales */
static size_t kparam_bytes(const orc_geom* g) { return (g->asymmetric ? 4u : 2u) * (size_t)g->head_dim; }
static size_t vparam_bytes(const orc_geom* g) { return (g->asymmetric ? 4u : 2u) * (size_t)g->page_size; }
size_t orc_section_bytes(const orc_geom* g, int bits) {
    if (bits == 16) return 2 * code_bytes(g, bits);       /* FP16 keys and values, no scales */
    return 2 * code_bytes(g, bits) + kparam_bytes(g) + vparam_bytes(g);
}
size_t orc_block_bytes(const orc_geom* g, int bits) {
    return (size_t)g->num_kv_heads * orc_section_bytes(g, bits);
}
static size_t off_kzero(const orc_geom* g, int bits) { return code_bytes(g, bits); }  /* asymmetric */
static size_t off_kscale(const orc_geom* g, int bits) {
    return code_bytes(g, bits) + (g->asymmetric ? 2 * (size_t)g->head_dim : 0);
}
static size_t off_vcodes(const orc_geom* g, int bits) {
    if (bits == 16) return code_bytes(g, bits);
    return code_bytes(g, bits) + kparam_bytes(g);
}
static size_t off_vzero(const orc_geom* g, int bits) {                               /* asymmetric */
    return 2 * code_bytes(g, bits) + kparam_bytes(g);
}
static size_t off_vscale(const orc_geom* g, int bits) {
    return 2 * code_bytes(g, bits) + kparam_bytes(g) + (g->asymmetric ? 2 * (size_t)g->page_size : 0);
}
static int k_index(const orc_geom* g, int t, int c) { return t * g->head_dim + c; }
static int v_index(const orc_geom* g, int t, int c) { return ((t / 4) * g->head_dim + c) * 4 + t % 4; }

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xff); p[1] = (uint8_t)(v >> 8); }

/* the code of an element: q for the symmetric format, the field u itself for the asymmetric */
int orc_k_code(const orc_geom* g, const uint8_t* sec, int bits, int t, int c) {
    return g->asymmetric ? field_of(sec, k_index(g, t, c), bits) : unpack_one(sec, k_index(g, t, c), bits);
}
int orc_v_code(const orc_geom* g, const uint8_t* sec, int bits, int t, int c) {
    const uint8_t* v = sec + off_vcodes(g, bits);
    return g->asymmetric ? field_of(v, v_index(g, t, c), bits) : unpack_one(v, v_index(g, t, c), bits);
}
double orc_k_zero(const orc_geom* g, const uint8_t* sec, int bits, int c) {
    return g->asymmetric ? orc_f16_to_f64(rd16(sec + off_kzero(g, bits) + 2 * (size_t)c)) : 0.0;
}
double orc_v_zero(const orc_geom* g, const uint8_t* sec, int bits, int t) {
    return g->asymmetric ? orc_f16_to_f64(rd16(sec + off_vzero(g, bits) + 2 * (size_t)t)) : 0.0;
}
double orc_k_scale(const orc_geom* g, const uint8_t* sec, int bits, int c) {
    return orc_f16_to_f64(rd16(sec + off_kscale(g, bits) + 2 * (size_t)c));
}
double orc_v_scale(const orc_geom* g, const uint8_t* sec, int bits, int t) {
    return orc_f16_to_f64(rd16(sec + off_vscale(g, bits) + 2 * (size_t)t));
}

/* the section of (handle, kv head), or NULL for an invalid handle */
static uint8_t* section_of(const orc_geom* g, uint8_t* const pools[4], uint32_t handle, int kv,
                           int* bits_out) {
    if (handle == 0xffffffffu) return NULL;
    int tier = (int)(handle >> 30);
    uint32_t index = handle & 0x3fffffffu;
    int bits = orc_bits_of_tier(tier);
    if (bits == 0) return NULL;
    *bits_out = bits;
    return pools[tier] + (size_t)index * orc_block_bytes(g, bits) +
           (size_t)kv * orc_section_bytes(g, bits);
}

/* ------------------------------------------------------------------------------------------ */
/* Quantize-on-write.                                                                           */
/* The open page's keys are re-quantized from their FP16 originals on every write: positions    */
/* already cached come from the ring as it was before this call (the ring holds the last R >= P  */
/* keys), new positions come from k_new.  Each new value vector is quantized over its D         */
/* channels into its token slot.  Then the new keys enter the ring.                             */

int orc_quant_write(const orc_geom* g, uint8_t* const pools[4], const uint32_t* bt, int max_pages,
                    const int32_t* pos, int batch, int n_new,
                    const uint16_t* k_new, const uint16_t* v_new, uint16_t* ring) {
    const int P = g->page_size, D = g->head_dim, H = g->num_kv_heads, R = g->ring_size;
    if (n_new <= 0) return 0;
    int status = 0;
    uint16_t* keys = malloc(sizeof(uint16_t) * (size_t)P * D);   /* one page of one kv head */
    int* kq = malloc(sizeof(int) * (size_t)P * D);
    int* vq = malloc(sizeof(int) * (size_t)P * D);
    uint16_t* vs = malloc(sizeof(uint16_t) * (size_t)P);
    uint16_t* vz = malloc(sizeof(uint16_t) * (size_t)P);
    int* codes = malloc(sizeof(int) * (size_t)(P > D ? P : D));
    const int asym = g->asymmetric != 0;
    for (int s = 0; s < batch && status == 0; ++s) {
        const int p0 = pos[s], end = p0 + n_new;
        const uint16_t* kn = k_new + (size_t)s * n_new * H * D;
        const uint16_t* vn = v_new + (size_t)s * n_new * H * D;
        uint16_t* rg = ring + (size_t)s * R * H * D;
        for (int page = p0 / P; page <= (end - 1) / P; ++page) {
            const int lo = page * P, hi = (lo + P < end) ? lo + P : end;
            if (page >= max_pages) { status = -1; break; }
            for (int kv = 0; kv < H; ++kv) {
                int bits = 0;
                uint8_t* sec = section_of(g, pools, bt[(size_t)s * max_pages + page], kv, &bits);
                if (!sec) { status = -1; break; }
                if (bits == 16) {
                    /* FP16 tier: new tokens' keys and values stored as they are, empty slots +0,
                       tokens cached before untouched */
                    for (int t = 0; t < P; ++t) {
                        const int p = lo + t;
                        if (p < p0) continue;
                        for (int c = 0; c < D; ++c) {
                            const uint16_t kb = p < hi ? kn[((size_t)(p - p0) * H + kv) * D + c] : 0;
                            const uint16_t vb = p < hi ? vn[((size_t)(p - p0) * H + kv) * D + c] : 0;
                            wr16(sec + 2 * (size_t)k_index(g, t, c), kb);
                            wr16(sec + off_vcodes(g, bits) + 2 * (size_t)v_index(g, t, c), vb);
                        }
                    }
                    continue;
                }
                /* gather the page's present keys [lo, hi) */
                for (int p = lo; p < hi; ++p)
                    for (int c = 0; c < D; ++c)
                        keys[(p - lo) * D + c] =
                            p < p0 ? rg[((size_t)(p % R) * H + kv) * D + c]
                                   : kn[((size_t)(p - p0) * H + kv) * D + c];
                /* K: one scale (and, asymmetric, one zero point) per channel over the present
                   tokens; the zero code elsewhere */
                for (int i = 0; i < P * D; ++i) kq[i] = 0;
                for (int c = 0; c < D; ++c) {
                    uint16_t sc, zp;
                    if (asym) {
                        orc_quantize_group_asym(keys + c, hi - lo, D, bits, &sc, &zp, codes);
                        wr16(sec + off_kzero(g, bits) + 2 * (size_t)c, zp);
                    } else {
                        orc_quantize_group(keys + c, hi - lo, D, bits, &sc, codes);
                    }
                    for (int t = 0; t < hi - lo; ++t) kq[k_index(g, t, c)] = codes[t];
                    wr16(sec + off_kscale(g, bits) + 2 * (size_t)c, sc);
                }
                if (asym) pack_fields(kq, P * D, bits, sec);
                else orc_pack(kq, P * D, bits, sec);
                /* V: tokens cached before keep their codes (and scale, zero point), new tokens
                   are quantized, empty slots get the zero code, scale 0 and zero point 0 */
                for (int t = 0; t < P; ++t) {
                    const int p = lo + t;
                    vz[t] = 0;
                    if (p < p0) {
                        for (int c = 0; c < D; ++c)
                            vq[v_index(g, t, c)] = orc_v_code(g, sec, bits, t, c);
                        vs[t] = rd16(sec + off_vscale(g, bits) + 2 * (size_t)t);
                        if (asym) vz[t] = rd16(sec + off_vzero(g, bits) + 2 * (size_t)t);
                    } else if (p < hi) {
                        const uint16_t* x = vn + ((size_t)(p - p0) * H + kv) * D;
                        if (asym) orc_quantize_group_asym(x, D, 1, bits, &vs[t], &vz[t], codes);
                        else orc_quantize_group(x, D, 1, bits, &vs[t], codes);
                        for (int c = 0; c < D; ++c) vq[v_index(g, t, c)] = codes[c];
                    } else {
                        for (int c = 0; c < D; ++c) vq[v_index(g, t, c)] = 0;
                        vs[t] = 0;
                    }
                }
                if (asym) pack_fields(vq, P * D, bits, sec + off_vcodes(g, bits));
                else orc_pack(vq, P * D, bits, sec + off_vcodes(g, bits));
                for (int t = 0; t < P; ++t) {
                    wr16(sec + off_vscale(g, bits) + 2 * (size_t)t, vs[t]);
                    if (asym) wr16(sec + off_vzero(g, bits) + 2 * (size_t)t, vz[t]);
                }
            }
            if (status) break;
        }
        /* ring: positions in increasing order, so only the last R survive */
        for (int p = p0; p < end && status == 0; ++p)
            memcpy(rg + (size_t)(p % R) * H * D, kn + (size_t)(p - p0) * H * D,
                   sizeof(uint16_t) * (size_t)H * D);
    }
    free(keys); free(kq); free(vq); free(vs); free(vz); free(codes);
    return status;
}

/* ------------------------------------------------------------------------------------------ */
/* Dequantized cache: K^_t[c] = code * s_K(page(t), c),  V^_t[c] = code * s_V(t); for the       */
/* asymmetric format K^_t[c] = z_K(page(t), c) + u * s_K(page(t), c), V^_t[c] = z_V(t) + u * s_V(t). */
/* Exact doubles.                                                                               */

int orc_dequant_kv(const orc_geom* g, uint8_t* const pools[4], const uint32_t* bt_row, int n,
                   int kv, double* K, double* V) {
    const int P = g->page_size, D = g->head_dim;
    for (int t = 0; t < n; ++t) {
        int bits = 0;
        const uint8_t* sec = section_of(g, pools, bt_row[t / P], kv, &bits);
        if (!sec) return -1;
        const int slot = t % P;
        if (bits == 16) {                                /* FP16 tier: the values themselves */
            for (int c = 0; c < D; ++c) {
                K[(size_t)t * D + c] = orc_f16_to_f64(rd16(sec + 2 * (size_t)k_index(g, slot, c)));
                V[(size_t)t * D + c] =
                    orc_f16_to_f64(rd16(sec + off_vcodes(g, bits) + 2 * (size_t)v_index(g, slot, c)));
            }
            continue;
        }
        const double sv = orc_v_scale(g, sec, bits, slot), zv = orc_v_zero(g, sec, bits, slot);
        for (int c = 0; c < D; ++c) {
            K[(size_t)t * D + c] = orc_k_zero(g, sec, bits, c) +
                                   orc_k_code(g, sec, bits, slot, c) * orc_k_scale(g, sec, bits, c);
            V[(size_t)t * D + c] = zv + orc_v_code(g, sec, bits, slot, c) * sv;
        }
    }
    return 0;
}

/* softmax attention of one query row over n dequantized keys/values, in double */
static void attend(const double* qd, const double* K, const double* V, int n, int D,
                   double scale, double* logit, double* out) {
    for (int c = 0; c < D; ++c) out[c] = 0.0;
    if (n <= 0) return;                              /* no keys: the row is zero */
    double mx = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int c = 0; c < D; ++c) dot += qd[c] * K[(size_t)t * D + c];
        logit[t] = scale * dot;
        if (logit[t] > mx) mx = logit[t];
    }
    double sum = 0.0;
    for (int t = 0; t < n; ++t) {
        double w = exp(logit[t] - mx);
        sum += w;
        for (int c = 0; c < D; ++c) out[c] += w * V[(size_t)t * D + c];
    }
    for (int c = 0; c < D; ++c) out[c] /= sum;
}

int orc_decode_attn_row(const orc_geom* g, uint8_t* const pools[4], const uint32_t* bt_row,
                        int ctx_len, const uint16_t* q_row, int h, float softmax_scale,
                        double* out) {
    const int D = g->head_dim, grp = g->num_q_heads / g->num_kv_heads;
    const int n = ctx_len > 0 ? ctx_len : 0;
    double* K = malloc(sizeof(double) * ((size_t)n * D + 1));
    double* V = malloc(sizeof(double) * ((size_t)n * D + 1));
    double* logit = malloc(sizeof(double) * ((size_t)n + 1));
    double qd[256];
    int rc = orc_dequant_kv(g, pools, bt_row, n, h / grp, K, V);
    if (rc == 0) {
        for (int c = 0; c < D; ++c) qd[c] = orc_f16_to_f64(q_row[c]);
        attend(qd, K, V, n, D, (double)softmax_scale, logit, out);
    }
    free(K); free(V); free(logit);
    return rc;
}

int orc_decode_attn(const orc_geom* g, uint8_t* const pools[4], const uint32_t* bt, int max_pages,
                    const int32_t* ctx_len, int batch, const uint16_t* q, float softmax_scale,
                    double* out) {
    const int D = g->head_dim, Hq = g->num_q_heads, H = g->num_kv_heads, grp = Hq / H;
    int status = 0;
    /* one independent item per (sequence, kv head): dequantize its cache once, then attend
       with each of the grp query heads that share it (kv = h / grp) */
#pragma omp parallel for schedule(dynamic) reduction(| : status)
    for (int item = 0; item < batch * H; ++item) {
        const int s = item / H, kv = item % H;
        const int n = ctx_len[s] > 0 ? ctx_len[s] : 0;
        double* K = malloc(sizeof(double) * ((size_t)n * D + 1));
        double* V = malloc(sizeof(double) * ((size_t)n * D + 1));
        double* logit = malloc(sizeof(double) * ((size_t)n + 1));
        double qd[256];
        if (orc_dequant_kv(g, pools, bt + (size_t)s * max_pages, n, kv, K, V) != 0) {
            status |= 1;
        } else {
            for (int h = kv * grp; h < (kv + 1) * grp; ++h) {
                for (int c = 0; c < D; ++c) qd[c] = orc_f16_to_f64(q[((size_t)s * Hq + h) * D + c]);
                attend(qd, K, V, n, D, (double)softmax_scale, logit, out + ((size_t)s * Hq + h) * D);
            }
        }
        free(K); free(V); free(logit);
    }
    return status ? -1 : 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Canary.  KL(P || Q) with P = softmax(l), Q = softmax(m):                                     */
/*   sum_p P_p (log P_p - log Q_p) = sum_p P_p (l_p - m_p) - LSE(l) + LSE(m).                    */

static double lse(const double* v, int n) {
    double mx = -INFINITY;
    for (int i = 0; i < n; ++i) if (v[i] > mx) mx = v[i];
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += exp(v[i] - mx);
    return mx + log(s);
}

double orc_kl_logits(const double* l, const double* m, int n) {
    if (n <= 0) return 0.0;
    const double L = lse(l, n), M = lse(m, n);
    double acc = 0.0;
    for (int i = 0; i < n; ++i) acc += exp(l[i] - L) * (l[i] - m[i]);
    double kl = acc - L + M;
    return kl > 0.0 ? kl : 0.0;          /* it can only dip below zero by rounding */
}

void orc_canary_kl(const orc_geom* g, const uint16_t* ring, const int32_t* seq_len, int batch,
                   const uint16_t* q, float softmax_scale, double* kl3, double* rows) {
    /* the cache's own quantizer: asymmetric copies for a geometry in the asymmetric format */
    orc_canary_kl_mode(g, ring, seq_len, batch, q, softmax_scale, g->asymmetric != 0, kl3, rows);
}

void orc_canary_kl_mode(const orc_geom* g, const uint16_t* ring, const int32_t* seq_len, int batch,
                        const uint16_t* q, float softmax_scale, int asymmetric, double* kl3,
                        double* rows) {
    const int P = g->page_size, D = g->head_dim, H = g->num_kv_heads, R = g->ring_size;
    const int Hq = g->num_q_heads, grp = Hq / H;
    const int tiers[3] = {2, 4, 8};
    double total[3] = {0.0, 0.0, 0.0};
    for (int s = 0; s < batch; ++s) {
        const int N = seq_len[s] > 0 ? seq_len[s] : 0;
        const int n = N < R ? N : R;
        const int first = N - n;                       /* ring positions [first, N) */
        const uint16_t* rg = ring + (size_t)s * R * H * D;
        for (int kv = 0; kv < H; ++kv) {
            /* the FP16 reference keys K_ref, and their temporary b-bit copies */
            double* Kref = malloc(sizeof(double) * ((size_t)n * D + 1));
            double* Kb = malloc(sizeof(double) * (3 * (size_t)n * D + 1));
            uint16_t* grpbuf = malloc(sizeof(uint16_t) * (size_t)P);
            int* codes = malloc(sizeof(int) * (size_t)P);
            for (int i = 0; i < n; ++i)
                for (int c = 0; c < D; ++c)
                    Kref[(size_t)i * D + c] =
                        orc_f16_to_f64(rg[((size_t)((first + i) % R) * H + kv) * D + c]);
            for (int ti = 0; ti < 3; ++ti) {
                /* group the ring positions by their logical page; one scale per channel */
                int i = 0;
                while (i < n) {
                    const int page = (first + i) / P;
                    int j = i;
                    while (j < n && (first + j) / P == page) ++j;
                    for (int c = 0; c < D; ++c) {
                        uint16_t sc, zp;
                        for (int k = i; k < j; ++k)
                            grpbuf[k - i] = rg[((size_t)((first + k) % R) * H + kv) * D + c];
                        if (asymmetric) {
                            orc_quantize_group_asym(grpbuf, j - i, 1, tiers[ti], &sc, &zp, codes);
                            for (int k = i; k < j; ++k)
                                Kb[((size_t)ti * n + k) * D + c] =
                                    orc_f16_to_f64(zp) + codes[k - i] * orc_f16_to_f64(sc);
                        } else {
                            orc_quantize_group(grpbuf, j - i, 1, tiers[ti], &sc, codes);
                            for (int k = i; k < j; ++k)
                                Kb[((size_t)ti * n + k) * D + c] = codes[k - i] * orc_f16_to_f64(sc);
                        }
                    }
                    i = j;
                }
            }
            double* l = malloc(sizeof(double) * ((size_t)n + 1));
            double* m = malloc(sizeof(double) * ((size_t)n + 1));
            for (int h = kv * grp; h < (kv + 1) * grp; ++h) {
                const uint16_t* qh = q + ((size_t)s * Hq + h) * D;
                for (int i = 0; i < n; ++i) {
                    double dot = 0.0;
                    for (int c = 0; c < D; ++c) dot += orc_f16_to_f64(qh[c]) * Kref[(size_t)i * D + c];
                    l[i] = (double)softmax_scale * dot;
                }
                for (int ti = 0; ti < 3; ++ti) {
                    for (int i = 0; i < n; ++i) {
                        double dot = 0.0;
                        for (int c = 0; c < D; ++c)
                            dot += orc_f16_to_f64(qh[c]) * Kb[((size_t)ti * n + i) * D + c];
                        m[i] = (double)softmax_scale * dot;
                    }
                    const double kl = orc_kl_logits(l, m, n);
                    total[ti] += kl;
                    if (rows) rows[((size_t)s * Hq + h) * 3 + ti] = kl;
                }
            }
            free(l); free(m); free(Kref); free(Kb); free(grpbuf); free(codes);
        }
    }
    for (int ti = 0; ti < 3; ++ti)
        kl3[ti] = batch > 0 ? total[ti] / ((double)batch * Hq) : 0.0;
}

/* ------------------------------------------------------------------------------------------ */
/* Accounting                                                                                   */

double orc_cache_bytes_per_token(const orc_geom* g, int num_layers, const int* bits) {
    double total = 0.0;
    for (int l = 0; l < num_layers; ++l) {
        if (bits[l] == 16)
            total += 2.0 * g->num_kv_heads * g->head_dim * 2.0;    /* K and V, 2 bytes each */
        else
            total += (double)orc_block_bytes(g, bits[l]) / g->page_size;
    }
    return total;
}

double orc_ring_bytes(const orc_geom* g, int num_layers) {
    return (double)num_layers * g->ring_size * g->num_kv_heads * g->head_dim * 2.0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* threads of the parallel attention loop (a timing knob of the CPU baseline; no effect on results) */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
