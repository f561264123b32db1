/*
 * CPU oracle for the low-bit MLA cache and its decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, independent
 * reference that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or constant with the GPU library; the two agree only
 * because both follow the same written definition.
 *
 * What it computes (sources: the three QuantMLA pages):
 *  - MLA keeps, per token, one content latent that serves as both key and
 *    value, and one small decoupled RoPE key that carries position
 *    ("QuantMLA: INT4 (and INT2) for both halves of the MLA cache", TL;DR and
 *    flowchart).  Content-path error reaches the output through both the
 *    query-key match and the value aggregation ("Key findings", error model),
 *    so the cached latent is the value as well as the key: absorbed-weight
 *    MLA decode.
 *  - The content path is stored at 4 or 2 bits, the RoPE path at 4 bits
 *    (same page, flowchart and "Key findings", bits; "Hugging Face Releases
 *    QuantMLA", Engineering Trade-offs and Performance; the C4R4 name comes
 *    from "QuantMLA's INT4/INT2 KV-cache quantization reports 5x ...",
 *    section "What the low-bit cache changes").
 *  - The attention kernel unpacks and dequantizes inside attention (wiki
 *    note, flowchart and "Key findings", systems), so decode output is
 *    attention over the dequantized cache.
 *
 * The pages fix no quantizer details.  The readings used here (asymmetric
 * min/max per token and channel group, fp16 scale and zero, zero = fp16 of
 * the group minimum, codes from the stored fp16 values with IEEE fp32
 * subtract/divide and round-half-to-even, clamp to [0, 2^b-1], canonical
 * dequantized value = bf16_rne(fma(code, S, Z))) are listed with their
 * reasons in the design notes.  Attention is computed in fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 * Parity pins for every function here live in the CPU test suite.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Number formats (IEEE 754 binary32 -> binary16 / bfloat16, RNE)     */
/* ------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

float oracle_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* Round a finite binary32 to bfloat16, ties to even.  bfloat16 keeps the
 * top 16 bits of binary32, so rounding drops the low 16 bits. */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u = f32_to_bits(f);
    uint32_t keep = u >> 16, rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

float oracle_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    if (e == 0) {                      /* zero or subnormal: m * 2^-24 */
        float v = (float)m * 0x1p-24f; /* exact: m < 2^10 */
        return sign ? -v : v;
    }
    if (e == 31) return bits_to_f32(sign | 0x7F800000u | (m << 13));
    return bits_to_f32(sign | ((e - 15 + 127) << 23) | (m << 13));
}

/* Round a binary32 to binary16, ties to even.  Returns 0 and sets *out on
 * success; returns -1 for NaN, infinity, or a value that rounds beyond the
 * binary16 range (|x| >= 65520). */
int oracle_f32_to_f16(float f, uint16_t *out) {
    uint32_t u = f32_to_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    int32_t e = (int32_t)((u >> 23) & 0xFFu);
    uint32_t man = u & 0x7FFFFFu;
    if (e == 0xFF) return -1;
    if (e == 0) { *out = sign; return 0; } /* binary32 zero/subnormal < 2^-126: rounds to 0 */
    uint32_t full = man | 0x800000u;       /* value = full * 2^(e-150) */
    int32_t e16 = e - 127 + 15;
    if (e16 >= 1) {
        /* normal range: keep 10 fraction bits, drop 13 */
        uint32_t q = full >> 13, rest = full & 0x1FFFu;
        if (rest > 0x1000u || (rest == 0x1000u && (q & 1u))) q += 1u;
        /* q in [2^10, 2^11]; carry moves into the exponent */
        uint32_t bits = ((uint32_t)e16 << 10) + (q - 0x400u);
        if (bits >= 0x7C00u) return -1;
        *out = (uint16_t)(sign | bits);
        return 0;
    }
    /* subnormal result: units of 2^-24; value/2^-24 = full * 2^(e-126) */
    int32_t shift = 126 - e; /* >= 14 */
    if (shift > 25) { *out = sign; return 0; }
    uint64_t f64 = full;
    uint64_t q = f64 >> shift, rest = f64 & ((1ull << shift) - 1ull), half = 1ull << (shift - 1);
    if (rest > half || (rest == half && (q & 1ull))) q += 1ull;
    *out = (uint16_t)(sign | (uint16_t)q); /* q == 0x400 encodes the smallest normal */
    return 0;
}

/* ------------------------------------------------------------------ */
/* Quantizer: one group of one path of one token                      */
/* ------------------------------------------------------------------ */

/* Asymmetric b-bit quantization of G values (reading: min/max range, fp16
 * scale S = fp16((max-min)/qmax), fp16 zero Z = fp16(min), codes computed
 * from the stored S and Z).  Returns 0, or -1 when S or Z do not fit fp16 or
 * an input is not finite. */
int oracle_quant_group(const float *x, int G, int bits,
                       uint8_t *codes, uint16_t *s16, uint16_t *z16) {
    const int qmax = (1 << bits) - 1;
    float mn = x[0], mx = x[0];
    for (int i = 0; i < G; ++i) {
        if (!isfinite(x[i])) return -1;
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    mn = mn + 0.0f; /* a minimum or maximum of -0 becomes +0 */
    mx = mx + 0.0f;
    float range = mx - mn;
    float s32 = range / (float)qmax;
    if (oracle_f32_to_f16(s32, s16) != 0) return -1;
    if (oracle_f32_to_f16(mn, z16) != 0) return -1;
    float S = oracle_f16_to_f32(*s16), Z = oracle_f16_to_f32(*z16);
    for (int i = 0; i < G; ++i) {
        if (S == 0.0f) { codes[i] = 0; continue; }
        float t = (x[i] - Z) / S;
        float r = rintf(t); /* default rounding mode: nearest, ties to even */
        if (r < 0.0f) r = 0.0f;
        if (r > (float)qmax) r = (float)qmax;
        codes[i] = (uint8_t)r;
    }
    return 0;
}

/* Canonical dequantized value: one fused multiply-add in binary32, then
 * bfloat16 with ties to even.  Returned widened to float (exact). */
float oracle_dequant_value(int code, uint16_t s16, uint16_t z16) {
    float v = fmaf((float)code, oracle_f16_to_f32(s16), oracle_f16_to_f32(z16));
    return oracle_bf16_to_f32(oracle_f32_to_bf16(v));
}

/* ------------------------------------------------------------------ */
/* Physical page layout                                               */
/* ------------------------------------------------------------------ */
/* A page holds page_size tokens.  Quantized formats (bits 2 or 4):
 *   region A  content codes : [chunk][token][16 bytes]; chunk j holds
 *             channels [j*E, (j+1)*E) with E = 128/c_bits elements;
 *             element e of a chunk sits in byte e*b/8 at bit (e*b)%8.
 *   region B  content scale/zero : [group][token][S16, Z16] (little endian)
 *   region C  RoPE codes    : as region A with d_r and r_bits
 *   region D  RoPE scale/zero : as region B
 * The 16-bit format stores bf16 rows [token][d_c + d_r]. */

typedef struct {
    int c_bits, c_group, r_bits, r_group, d_c, d_r, page;
} ofmt;

static ofmt make_fmt(const int32_t *f) {
    ofmt m = {f[0], f[1], f[2], f[3], f[4], f[5], f[6]};
    return m;
}

static int fmt_valid(ofmt f) {
    if (f.page <= 0 || f.d_c <= 0 || f.d_r <= 0) return 0;
    if (f.c_bits == 16 && f.r_bits == 16) return 1;
    if (!(f.c_bits == 2 || f.c_bits == 4 || f.c_bits == 8)) return 0;
    if (!(f.r_bits == 2 || f.r_bits == 4 || f.r_bits == 8)) return 0;
    if (f.c_group <= 0 || f.r_group <= 0) return 0;
    if (f.d_c % f.c_group || f.d_r % f.r_group) return 0;
    if ((f.d_c * f.c_bits) % 128 || (f.d_r * f.r_bits) % 128) return 0;
    return 1;
}

static int64_t region_a(ofmt f) { return (int64_t)f.d_c * f.c_bits / 128 * f.page * 16; }
static int64_t region_b(ofmt f) { return (int64_t)(f.d_c / f.c_group) * f.page * 4; }
static int64_t region_c(ofmt f) { return (int64_t)f.d_r * f.r_bits / 128 * f.page * 16; }
static int64_t region_d(ofmt f) { return (int64_t)(f.d_r / f.r_group) * f.page * 4; }

int64_t oracle_page_bytes(const int32_t *fmt) {
    ofmt f = make_fmt(fmt);
    if (!fmt_valid(f)) return -1;
    if (f.c_bits == 16) return (int64_t)f.page * (f.d_c + f.d_r) * 2;
    return region_a(f) + region_b(f) + region_c(f) + region_d(f);
}

/* Write one path (codes region at `codes_off`, scale/zero region at
 * `sz_off`) of one token into a page. */
static int put_path(uint8_t *page, ofmt f, int64_t codes_off, int64_t sz_off,
                    const float *x, int d, int bits, int group, int tok) {
    uint8_t codes[256];
    const int per_chunk = 128 / bits;
    for (int g = 0; g < d / group; ++g) {
        uint16_t s16, z16;
        if (group > 256) return -1;
        if (oracle_quant_group(x + g * group, group, bits, codes, &s16, &z16)) return -1;
        uint8_t *sz = page + sz_off + ((int64_t)g * f.page + tok) * 4;
        sz[0] = (uint8_t)(s16 & 0xFF); sz[1] = (uint8_t)(s16 >> 8);
        sz[2] = (uint8_t)(z16 & 0xFF); sz[3] = (uint8_t)(z16 >> 8);
        for (int i = 0; i < group; ++i) {
            int ch = g * group + i;
            int chunk = ch / per_chunk, e = ch % per_chunk;
            uint8_t *cb = page + codes_off + ((int64_t)chunk * f.page + tok) * 16;
            int byte = (e * bits) / 8, sh = (e * bits) % 8;
            uint8_t mask = (uint8_t)(((1 << bits) - 1) << sh);
            cb[byte] = (uint8_t)((cb[byte] & ~mask) | ((codes[i] << sh) & mask));
        }
    }
    return 0;
}

/* Quantize n_new tokens (bf16 bit patterns) and write each into the slot
 * slot_mapping[n] = page * page_size + offset; negative slots are skipped.
 * Returns 0, -1 for a bad format, -2 for a slot beyond num_pages, -3 for a
 * group whose scale or zero does not fit fp16. */
int oracle_quant_append(const int32_t *fmt, const uint16_t *latent, const uint16_t *rope,
                        const int32_t *slot_mapping, int32_t n_new,
                        uint8_t *cache, int64_t num_pages) {
    ofmt f = make_fmt(fmt);
    if (!fmt_valid(f)) return -1;
    int64_t pb = oracle_page_bytes(fmt);
    float xc[4096], xr[4096];
    if (f.d_c > 4096 || f.d_r > 4096) return -1;
    for (int32_t n = 0; n < n_new; ++n) {
        int32_t slot = slot_mapping[n];
        if (slot < 0) continue;
        int64_t pg = slot / f.page;
        int tok = slot % f.page;
        if (pg >= num_pages) return -2;
        uint8_t *page = cache + pg * pb;
        if (f.c_bits == 16) {
            uint8_t *row = page + (int64_t)tok * (f.d_c + f.d_r) * 2;
            memcpy(row, latent + (int64_t)n * f.d_c, (size_t)f.d_c * 2);
            memcpy(row + (size_t)f.d_c * 2, rope + (int64_t)n * f.d_r, (size_t)f.d_r * 2);
            continue;
        }
        for (int i = 0; i < f.d_c; ++i) xc[i] = oracle_bf16_to_f32(latent[(int64_t)n * f.d_c + i]);
        for (int i = 0; i < f.d_r; ++i) xr[i] = oracle_bf16_to_f32(rope[(int64_t)n * f.d_r + i]);
        int64_t a = 0, b = region_a(f), c = b + region_b(f), d = c + region_c(f);
        if (put_path(page, f, a, b, xc, f.d_c, f.c_bits, f.c_group, tok)) return -3;
        if (put_path(page, f, c, d, xr, f.d_r, f.r_bits, f.r_group, tok)) return -3;
    }
    return 0;
}

/* Read back the codes, scales and zeros of one path of one token. */
static void get_path(const uint8_t *page, ofmt f, int64_t codes_off, int64_t sz_off,
                     int d, int bits, int group, int tok, float *out) {
    const int per_chunk = 128 / bits;
    for (int ch = 0; ch < d; ++ch) {
        int g = ch / group;
        const uint8_t *sz = page + sz_off + ((int64_t)g * f.page + tok) * 4;
        uint16_t s16 = (uint16_t)(sz[0] | (sz[1] << 8));
        uint16_t z16 = (uint16_t)(sz[2] | (sz[3] << 8));
        int chunk = ch / per_chunk, e = ch % per_chunk;
        const uint8_t *cb = page + codes_off + ((int64_t)chunk * f.page + tok) * 16;
        int code = (cb[(e * bits) / 8] >> ((e * bits) % 8)) & ((1 << bits) - 1);
        out[ch] = oracle_dequant_value(code, s16, z16);
    }
}

/* Canonical dequantized row (d_c + d_r floats) of token `tok` in page `pg`. */
static void dequant_token(const uint8_t *cache, ofmt f, int64_t pb, int64_t pg, int tok, float *out) {
    const uint8_t *page = cache + pg * pb;
    if (f.c_bits == 16) {
        const uint8_t *row = page + (int64_t)tok * (f.d_c + f.d_r) * 2;
        for (int i = 0; i < f.d_c + f.d_r; ++i)
            out[i] = oracle_bf16_to_f32((uint16_t)(row[2 * i] | (row[2 * i + 1] << 8)));
        return;
    }
    int64_t a = 0, b = region_a(f), c = b + region_b(f), d = c + region_c(f);
    get_path(page, f, a, b, f.d_c, f.c_bits, f.c_group, tok, out);
    get_path(page, f, c, d, f.d_r, f.r_bits, f.r_group, tok, out + f.d_c);
}

/* Dequantized keys of every sequence: out[b][t][d_c + d_r] for t < max_len
 * (rows at t >= seq_lens[b] are set to 0).  Returns 0 or -1. */
int oracle_dequant_cache(const int32_t *fmt, const uint8_t *cache, int64_t num_pages,
                         const int32_t *block_table, const int32_t *seq_lens,
                         int32_t batch, int32_t max_pages, int32_t max_len, float *out) {
    ofmt f = make_fmt(fmt);
    if (!fmt_valid(f)) return -1;
    int64_t pb = oracle_page_bytes(fmt);
    int D = f.d_c + f.d_r;
    for (int32_t b = 0; b < batch; ++b) {
        for (int32_t t = 0; t < max_len; ++t) {
            float *row = out + ((int64_t)b * max_len + t) * D;
            if (t >= seq_lens[b]) { memset(row, 0, sizeof(float) * D); continue; }
            int64_t pg = block_table[(int64_t)b * max_pages + t / f.page];
            if (pg < 0 || pg >= num_pages) return -1;
            dequant_token(cache, f, pb, pg, t % f.page, row);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Decode attention (fp64)                                            */
/* ------------------------------------------------------------------ */

/* For each sequence b and head h, over the tokens t in [t_begin, t_end)
 * clipped to [0, seq_lens[b]):
 *   l_t   = scale * <q[b,h,:], khat[t,:]>          (all d_c + d_r channels)
 *   m     = max_t l_t,  p_t = exp(l_t - m),  Zs = sum_t p_t
 *   out   = sum_t (p_t / Zs) * khat[t, :d_c]       (the latent is the value)
 *   lse   = m + log(Zs)
 * An empty range gives out = 0 and lse = -inf.  q holds bf16 bit patterns
 * [batch][heads][d_c + d_r].  `weights`, if not NULL, receives p_t / Zs at
 * [b][h][t] for t < max_len.  `nthreads` <= 0 uses the OpenMP default. */
int oracle_decode_range(const int32_t *fmt, const uint16_t *q, const uint8_t *cache, int64_t num_pages,
                        const int32_t *block_table, const int32_t *seq_lens,
                        int32_t batch, int32_t heads, int32_t max_pages, float softmax_scale,
                        int32_t t_begin, int32_t t_end,
                        double *out, double *lse, double *weights, int32_t max_len, int nthreads) {
    ofmt f = make_fmt(fmt);
    if (!fmt_valid(f)) return -1;
    const int D = f.d_c + f.d_r;
    const double scale = (double)softmax_scale;
    int64_t pb = oracle_page_bytes(fmt);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    for (int32_t b = 0; b < batch; ++b) {
        int32_t L = seq_lens[b];
        int32_t t0 = t_begin < 0 ? 0 : t_begin;
        int32_t t1 = t_end < L ? t_end : L;
        int32_t n = t1 > t0 ? t1 - t0 : 0;
        /* step 1: the dequantized keys of this sequence's tokens */
        float *K = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1) * D);
        if (!K) return -4;
        int bad = 0;
        for (int32_t i = 0; i < n; ++i) {
            int32_t t = t0 + i;
            int64_t pg = block_table[(int64_t)b * max_pages + t / f.page];
            if (pg < 0 || pg >= num_pages) { bad = 1; break; }
            dequant_token(cache, f, pb, pg, t % f.page, K + (size_t)i * D);
        }
        if (bad) { free(K); return -2; }
        /* step 2: attention for every head */
#pragma omp parallel for schedule(static)
        for (int32_t h = 0; h < heads; ++h) {
            const uint16_t *qh = q + ((int64_t)b * heads + h) * D;
            double *o = out + ((int64_t)b * heads + h) * f.d_c;
            double *w = weights ? weights + ((int64_t)b * heads + h) * max_len : NULL;
            double qd[4096];
            for (int i = 0; i < D; ++i) qd[i] = (double)oracle_bf16_to_f32(qh[i]);
            for (int c = 0; c < f.d_c; ++c) o[c] = 0.0;
            if (w) for (int32_t t = 0; t < max_len; ++t) w[t] = 0.0;
            if (n == 0) { lse[(int64_t)b * heads + h] = -INFINITY; continue; }
            double *l = (double *)malloc(sizeof(double) * (size_t)n);
            double m = -INFINITY;
            for (int32_t i = 0; i < n; ++i) {
                const float *k = K + (size_t)i * D;
                double s = 0.0;
                for (int c = 0; c < D; ++c) s += qd[c] * (double)k[c];
                l[i] = scale * s;
                if (l[i] > m) m = l[i];
            }
            double Zs = 0.0;
            for (int32_t i = 0; i < n; ++i) { l[i] = exp(l[i] - m); Zs += l[i]; }
            for (int32_t i = 0; i < n; ++i) {
                double p = l[i] / Zs;
                const float *k = K + (size_t)i * D;
                for (int c = 0; c < f.d_c; ++c) o[c] += p * (double)k[c];
                if (w && t0 + i < max_len) w[t0 + i] = p;
            }
            lse[(int64_t)b * heads + h] = m + log(Zs);
            free(l);
        }
        free(K);
    }
    return 0;
}

/* Merge S partial results of the same (b, h) rows: partial s covers a
 * disjoint token range and holds its normalized output o_s and log-sum-exp
 * lse_s.  out = sum_s w_s o_s / sum_s w_s with w_s = exp(lse_s - M),
 * M = max_s lse_s; lse = M + log(sum_s w_s).  Rows whose partials are all
 * empty (lse = -inf) give out = 0 and lse = -inf.
 * Layouts: o_parts[s][rows][d], lse_parts[s][rows], out[rows][d]. */
void oracle_combine(int32_t S, int64_t rows, int32_t d, const double *o_parts,
                    const double *lse_parts, double *out, double *lse) {
    for (int64_t r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int32_t s = 0; s < S; ++s) if (lse_parts[(int64_t)s * rows + r] > M) M = lse_parts[(int64_t)s * rows + r];
        for (int32_t c = 0; c < d; ++c) out[r * d + c] = 0.0;
        if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
        double W = 0.0;
        for (int32_t s = 0; s < S; ++s) {
            double ls = lse_parts[(int64_t)s * rows + r];
            if (ls == -INFINITY) continue;
            double w = exp(ls - M);
            W += w;
            const double *o = o_parts + ((int64_t)s * rows + r) * d;
            for (int32_t c = 0; c < d; ++c) out[r * d + c] += w * o[c];
        }
        for (int32_t c = 0; c < d; ++c) out[r * d + c] /= W;
        lse[r] = M + log(W);
    }
}
