/*
 * mla_oracle.c -- CPU oracle for MLA flash attention over the latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no source with the HIP path.
 *
 * What it computes is the plain definition the flash method must reproduce
 * exactly up to rounding order: softmax attention of every query head over one
 * latent key/value head, in fp64, with the full score row and the full weight row
 * materialised.  Sources, all from the pages:
 *   - flash attention keeps a running max and running sum and, after each key
 *     block, corrects what it accumulated so far with the new max; the result is
 *     the ordinary softmax-weighted sum ("Vulkan backend fused Flash Attention:
 *     DeepSeek MLA local inference", sections 2.1 and 2.2);
 *   - the MLA cache row is kv_lora_rank (512) + n_embd_head_qk_rope (64) = 576
 *     wide; with flash attention the cache is K-only and V is derived from that
 *     same row, shared by every head ("ik_llama.cpp -mla flag deep-dive",
 *     sections "what MLA is" and "the four -mla levels"); V is taken as the first
 *     512 columns of the row;
 *   - the mask is f16 and additive; a cell whose mask is -inf is not kept
 *     ("baguaai Flash Attention tag page", f16 FA mask digest; "llama.cpp Vulkan
 *     backend adds sparse Flash Attention for quantized K/V", commit text);
 *   - `-ctk q8_0` stores the cache as Q8_0 blocks: an f16 scale d then 32 int8
 *     codes, value = code * d ("ik_llama.cpp -mla flag deep-dive", recommended
 *     DeepSeek command combinations);
 *   - the sparse index list is the ascending list of kept cells of a mask row
 *     (sparse FA commit text above).
 * Readings where the pages are silent: the mask is added after scaling; a causal
 * chunk of n_tok queries ending at cache position n_kv-1 lets token t see keys
 * j <= n_kv - n_tok + t; a row with no kept key outputs zeros.
 *
 * Parity pins live in tests/test_oracle_pins.py (exhaustive conversions, mpmath
 * brute force, torch float64 SDPA, closed forms and invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F16 1
#define OR_BF16 2
#define OR_Q8_0 3
#define OR_F16_NEG_INF 0xFC00u

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 = the upper half of IEEE-754 binary32: 1 sign, 8 exponent (bias 127),
 * 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* f/2^7 * 2^-126 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);     /* (1 + f/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

/* One Q8_0 row of dk values (dk/32 blocks of 34 bytes). */
void oracle_q8_0_row_to_f64(const uint8_t *row, int dk, double *out) {
    for (int b = 0; b < dk / 32; ++b) {
        const uint8_t *blk = row + 34 * b;
        double d = oracle_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
        for (int i = 0; i < 32; ++i)
            out[32 * b + i] = (double)(int8_t)blk[2 + i] * d;
    }
}

/* Elementwise decode of n values of type f16 / bf16 (src = uint16 bits), or of
 * n/32 Q8_0 blocks (src = bytes). */
int oracle_decode(const void *src, int type, int64_t n, double *dst) {
    if (type == OR_F16 || type == OR_BF16) {
        const uint16_t *s = (const uint16_t *)src;
        for (int64_t i = 0; i < n; ++i)
            dst[i] = type == OR_F16 ? oracle_f16_to_f64(s[i]) : oracle_bf16_to_f64(s[i]);
        return 0;
    }
    if (type == OR_Q8_0) {
        if (n % 32) return -1;
        oracle_q8_0_row_to_f64((const uint8_t *)src, (int)n, dst);
        return 0;
    }
    return -1;
}

static void decode_row(const uint8_t *p, int type, int dk, double *out) {
    if (type == OR_Q8_0) {
        oracle_q8_0_row_to_f64(p, dk, out);
        return;
    }
    const uint16_t *s = (const uint16_t *)p;
    for (int d = 0; d < dk; ++d)
        out[d] = type == OR_F16 ? oracle_f16_to_f64(s[d]) : oracle_bf16_to_f64(s[d]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * out[i][d] (d < dv) for each selected row i = (s, t, h), flat id (s*n_tok + t)*n_head + h.
 *
 *   q    : bits [n_seq][n_tok][n_head][dk], f16 or bf16
 *   kv   : row j of sequence s starts at kv + s*kv_seq_stride + j*kv_row_stride
 *          (bytes; kv_seq_stride 0 = all sequences share one cache)
 *   kv_len : valid cells per sequence (clamped to [0, n_kv]), or NULL = n_kv for all
 *   causal : token t of sequence s sees cells j <= L_s - n_tok + t (L_s its valid length)
 *   mask : f16 bits, element (s, t, j) at s*mask_seq_stride + t*mask_tok_stride + j,
 *          or NULL; -inf (bits 0xFC00) drops the cell, any other value is an additive
 *          bias on the scaled score
 *   alibi : per-head slope, or NULL; with it the bias of a kept cell is slope * mask
 *          value (a dropped cell stays dropped)
 *   sinks : per-head sink logit, or NULL; it joins the softmax normaliser as one more
 *          term exp(sink - m) that carries no value
 *   softcap : 0 = off; else the scaled score x becomes softcap * tanh(x / softcap),
 *          before the bias is added
 *   rows : flat row ids to evaluate (NULL = all n_seq*n_tok*n_head, in order)
 *   row_max / row_sum : optional, per row the max m over kept scores and the sink, and
 *          the normaliser sum of exp(score - m) (+ exp(sink - m)); m = -inf and sum 0
 *          for a row with neither kept cell nor sink
 * Returns the number of rows with no kept cell, or a negative value on bad input.
 */
static int64_t attention_core(const uint16_t *q, int q_type, const double *q64, const uint8_t *kv,
                              int kv_type, int64_t kv_row_stride, int64_t kv_seq_stride, int n_seq,
                              int n_tok, int n_head, int64_t n_kv, int dk, int dv,
                              const int32_t *kv_len, int causal, const uint16_t *mask,
                              int64_t mask_tok_stride, int64_t mask_seq_stride,
                              const double *alibi, const double *sinks, double softcap,
                              double scale, const int64_t *rows, int64_t n_rows, double *out,
                              double *row_max, double *row_sum);

int64_t oracle_mla_attention_ext(const uint16_t *q, int q_type, const uint8_t *kv, int kv_type,
                                 int64_t kv_row_stride, int64_t kv_seq_stride, int n_seq,
                                 int n_tok, int n_head, int64_t n_kv, int dk, int dv,
                                 const int32_t *kv_len, int causal, const uint16_t *mask,
                                 int64_t mask_tok_stride, int64_t mask_seq_stride,
                                 const double *alibi, const double *sinks, double softcap,
                                 double scale, const int64_t *rows, int64_t n_rows, double *out,
                                 double *row_max, double *row_sum) {
    if (!q || (q_type != OR_F16 && q_type != OR_BF16)) return -1;
    return attention_core(q, q_type, NULL, kv, kv_type, kv_row_stride, kv_seq_stride, n_seq, n_tok,
                          n_head, n_kv, dk, dv, kv_len, causal, mask, mask_tok_stride, mask_seq_stride,
                          alibi, sinks, softcap, scale, rows, n_rows, out, row_max, row_sum);
}

/* The same with the queries given in fp64, q64[n_seq][n_tok][n_head][dk] (used where the
 * query is itself computed, e.g. absorbed from per-head dims; no rounding to 16 bits). */
int64_t oracle_mla_attention_q64(const double *q64, const uint8_t *kv, int kv_type,
                                 int64_t kv_row_stride, int64_t kv_seq_stride, int n_seq,
                                 int n_tok, int n_head, int64_t n_kv, int dk, int dv,
                                 const int32_t *kv_len, int causal, const uint16_t *mask,
                                 int64_t mask_tok_stride, int64_t mask_seq_stride, double scale,
                                 const int64_t *rows, int64_t n_rows, double *out) {
    if (!q64) return -1;
    return attention_core(NULL, 0, q64, kv, kv_type, kv_row_stride, kv_seq_stride, n_seq, n_tok,
                          n_head, n_kv, dk, dv, kv_len, causal, mask, mask_tok_stride, mask_seq_stride,
                          NULL, NULL, 0.0, scale, rows, n_rows, out, NULL, NULL);
}

static int64_t attention_core(const uint16_t *q, int q_type, const double *q64, const uint8_t *kv,
                              int kv_type, int64_t kv_row_stride, int64_t kv_seq_stride, int n_seq,
                              int n_tok, int n_head, int64_t n_kv, int dk, int dv,
                              const int32_t *kv_len, int causal, const uint16_t *mask,
                              int64_t mask_tok_stride, int64_t mask_seq_stride,
                              const double *alibi, const double *sinks, double softcap,
                              double scale, const int64_t *rows, int64_t n_rows, double *out,
                              double *row_max, double *row_sum) {
    if (!kv || !out || n_seq < 1 || n_tok < 1 || n_head < 1 || n_kv < 1 || dk < 1 ||
        dv < 1 || dv > dk || softcap < 0.0)
        return -1;
    if (kv_type == OR_Q8_0 && dk % 32) return -1;
    int64_t total = (int64_t)n_seq * n_tok * n_head;
    if (!rows) n_rows = total;
    int64_t n_empty = 0;

    for (int s = 0; s < n_seq; ++s) {
        int wanted = 0;
        for (int64_t i = 0; i < n_rows && !wanted; ++i) {
            int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= total) return -2;
            wanted = (r / ((int64_t)n_tok * n_head)) == s;
        }
        if (!wanted) continue;
        int64_t len = n_kv;
        if (kv_len) len = kv_len[s] < 0 ? 0 : (kv_len[s] > n_kv ? n_kv : kv_len[s]);

        /* The sequence's valid cells, decoded once to fp64. */
        double *K = (double *)malloc((size_t)(len > 0 ? len : 1) * dk * sizeof(double));
        if (!K) return -3;
        const uint8_t *kv_s = kv + (int64_t)s * kv_seq_stride;
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < len; ++j)
            decode_row(kv_s + j * kv_row_stride, kv_type, dk, K + j * dk);

#pragma omp parallel for schedule(dynamic, 1) reduction(+ : n_empty)
        for (int64_t i = 0; i < n_rows; ++i) {
            int64_t r = rows ? rows[i] : i;
            if (r / ((int64_t)n_tok * n_head) != s) continue;
            int t = (int)((r / n_head) % n_tok);
            int h = (int)(r % n_head);
            double *qv = (double *)malloc((size_t)dk * sizeof(double));
            double *score = (double *)malloc((size_t)(len > 0 ? len : 1) * sizeof(double));
            double *p = (double *)malloc((size_t)(len > 0 ? len : 1) * sizeof(double));
            double *o = out + i * dv;
            if (q64)
                memcpy(qv, q64 + r * dk, (size_t)dk * sizeof(double));
            else
                decode_row((const uint8_t *)(q + r * dk), q_type, dk, qv);

            /* score_j = cap(scale * q.k_j) + bias_j, or -inf for a cell that is not kept */
            double m = -INFINITY;
            int kept = 0;
            for (int64_t j = 0; j < len; ++j) {
                double bias = 0.0;
                if (mask) {
                    uint16_t mb = mask[(int64_t)s * mask_seq_stride + (int64_t)t * mask_tok_stride + j];
                    bias = oracle_f16_to_f64(mb);
                    if (alibi && bias != -INFINITY) bias = alibi[h] * bias;
                }
                if (causal && j > len - n_tok + t) bias = -INFINITY;
                if (bias == -INFINITY) {
                    score[j] = -INFINITY;
                    continue;
                }
                double dot = 0.0;
                for (int d = 0; d < dk; ++d) dot += qv[d] * K[j * dk + d];
                double x = scale * dot;
                if (softcap > 0.0) x = softcap * tanh(x / softcap);
                score[j] = x + bias;
                kept = 1;
                if (score[j] > m) m = score[j];
            }
            const double sink = sinks ? sinks[h] : -INFINITY;
            if (sink > m) m = sink;

            for (int d = 0; d < dv; ++d) o[d] = 0.0;
            if (!kept) n_empty += 1;
            if (m == -INFINITY) {
                /* neither a kept cell nor a sink: output zeros */
                if (row_max) row_max[i] = -INFINITY;
                if (row_sum) row_sum[i] = 0.0;
            } else {
                /* softmax weights, materialised in full; the sink adds to the normaliser */
                double l = sink == -INFINITY ? 0.0 : exp(sink - m);
                for (int64_t j = 0; j < len; ++j) {
                    p[j] = score[j] == -INFINITY ? 0.0 : exp(score[j] - m);
                    l += p[j];
                }
                for (int64_t j = 0; j < len; ++j) p[j] /= l;
                /* weighted sum of V = the first dv columns of each row */
                for (int64_t j = 0; j < len; ++j) {
                    if (p[j] == 0.0) continue;
                    const double *v = K + j * dk;
                    for (int d = 0; d < dv; ++d) o[d] += p[j] * v[d];
                }
                if (row_max) row_max[i] = m;
                if (row_sum) row_sum[i] = l;
            }
            free(qv);
            free(score);
            free(p);
        }
        free(K);
    }
    return n_empty;
}

/* The plain call: every sequence holds n_kv cells; no ALiBi, sinks or softcap. */
int64_t oracle_mla_attention(const uint16_t *q, int q_type, const uint8_t *kv, int kv_type,
                             int64_t kv_row_stride, int64_t kv_seq_stride, int n_seq,
                             int n_tok, int n_head, int64_t n_kv, int dk, int dv, int causal,
                             const uint16_t *mask, int64_t mask_tok_stride,
                             int64_t mask_seq_stride, double scale, const int64_t *rows,
                             int64_t n_rows, double *out, double *row_max, double *row_sum) {
    return oracle_mla_attention_ext(q, q_type, kv, kv_type, kv_row_stride, kv_seq_stride, n_seq, n_tok,
                                    n_head, n_kv, dk, dv, NULL, causal, mask, mask_tok_stride,
                                    mask_seq_stride, NULL, NULL, 0.0, scale, rows, n_rows, out,
                                    row_max, row_sum);
}

/*
 * Per-head attention with separate K and V (the non-absorbed MLA prefill shape, e.g.
 * dk = 192 = 128 + 64 RoPE, dv = 128), out[i][d] for each selected row i = t*n_head + h:
 *
 *   q    : bits [n_tok][n_head][dk], f16 or bf16
 *   k    : bits, key j of head h at k + j*k_row_stride + h*dk (elements), f16 or bf16
 *   v    : bits, value j of head h at v + j*v_row_stride + h*dv (elements), same type as k
 *   causal : token t sees keys j <= n_kv - n_tok + t
 *   mask : f16 bits [n_tok][mask_row_stride] or NULL (-inf drops a key, else added)
 * score_j = scale * q.k_j + mask_j, softmax over kept keys, out = sum_j p_j v_j
 * (zeros for a row with no kept key).  Returns the number of such rows, or < 0 on bad input.
 */
int64_t oracle_mha_attention(const uint16_t *q, int q_type, const uint16_t *k, const uint16_t *v,
                             int kv_type, int64_t k_row_stride, int64_t v_row_stride, int n_tok,
                             int n_head, int64_t n_kv, int dk, int dv, int causal,
                             const uint16_t *mask, int64_t mask_row_stride, double scale,
                             const int64_t *rows, int64_t n_rows, double *out) {
    if (!q || !k || !v || !out || n_tok < 1 || n_head < 1 || n_kv < 1 || dk < 1 || dv < 1) return -1;
    if ((q_type != OR_F16 && q_type != OR_BF16) || (kv_type != OR_F16 && kv_type != OR_BF16)) return -1;
    const int64_t total = (int64_t)n_tok * n_head;
    if (!rows) n_rows = total;
    int64_t n_empty = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : n_empty)
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t r = rows ? rows[i] : i;
        double *o = out + i * dv;
        for (int d = 0; d < dv; ++d) o[d] = 0.0;
        if (r < 0 || r >= total) continue;
        const int t = (int)(r / n_head), h = (int)(r % n_head);
        double *qv = (double *)malloc((size_t)dk * sizeof(double));
        double *kv_ = (double *)malloc((size_t)dk * sizeof(double));
        double *vv = (double *)malloc((size_t)dv * sizeof(double));
        double *score = (double *)malloc((size_t)n_kv * sizeof(double));
        decode_row((const uint8_t *)(q + r * dk), q_type, dk, qv);
        double m = -INFINITY;
        for (int64_t j = 0; j < n_kv; ++j) {
            double bias = mask ? oracle_f16_to_f64(mask[(int64_t)t * mask_row_stride + j]) : 0.0;
            if (causal && j > n_kv - n_tok + t) bias = -INFINITY;
            if (bias == -INFINITY) {
                score[j] = -INFINITY;
                continue;
            }
            decode_row((const uint8_t *)(k + j * k_row_stride + (int64_t)h * dk), kv_type, dk, kv_);
            double dot = 0.0;
            for (int d = 0; d < dk; ++d) dot += qv[d] * kv_[d];
            score[j] = scale * dot + bias;
            if (score[j] > m) m = score[j];
        }
        if (m == -INFINITY) {
            n_empty += 1;
        } else {
            double l = 0.0;
            for (int64_t j = 0; j < n_kv; ++j) {
                score[j] = score[j] == -INFINITY ? 0.0 : exp(score[j] - m);
                l += score[j];
            }
            for (int64_t j = 0; j < n_kv; ++j) {
                if (score[j] == 0.0) continue;
                decode_row((const uint8_t *)(v + j * v_row_stride + (int64_t)h * dv), kv_type, dv, vv);
                const double p = score[j] / l;
                for (int d = 0; d < dv; ++d) o[d] += p * vv[d];
            }
        }
        free(qv);
        free(kv_);
        free(vv);
        free(score);
    }
    return n_empty;
}

/* Sparse-mask index compaction: for each mask row, the ascending list of cells
 * whose f16 mask is not -inf (bits != 0xFC00), and its length. */
void oracle_mask_compact(const uint16_t *mask, int64_t mask_row_stride, int n_rows, int64_t n_kv,
                         int32_t *idx, int64_t idx_row_stride, int32_t *count) {
    for (int r = 0; r < n_rows; ++r) {
        int32_t c = 0;
        const uint16_t *m = mask + (int64_t)r * mask_row_stride;
        for (int64_t j = 0; j < n_kv; ++j)
            if (m[j] != OR_F16_NEG_INF) idx[(int64_t)r * idx_row_stride + c++] = (int32_t)j;
        count[r] = c;
    }
}
