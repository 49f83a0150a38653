/*
 * CPU oracle for paged MLA decode -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 reference of what the decode path computes.  Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may call it; the
 * product library never does.  It shares no source with the GPU library.
 *
 * Sources (page titles as published):
 *  [FlashMLA] "为什么 FlashMLA 的解码内核能跑到 660 TFLOPS——内核里的 5 个关键设计"
 *      - "设计 2" (FP8 KV cache): 656-byte token = 512 e4m3 NoPE codes quantised per
 *        1x128 tile with four fp32 scales, then 64 bf16 RoPE values; dequantise
 *        to bf16 before any product.  The writer side (quantise, append by
 *        block table) follows the same layout.
 *      - "上手示例" (usage): sparse semantics -- gather rows by index, scores
 *        P = (Q K^T) * sm_scale, lse = log2 of the sum of 2^P, weights
 *        2^(P - lse), output = weights times the gathered rows.
 *  [Modular] "Modular Platform 设计文档全景导读"
 *      - section 四 (PagedAttention): token index -> (page, slot) by divmod
 *        with the page size, then the block table gives the physical page.
 *      - section 六 / 七 (online softmax): running max / sum with a correction
 *        factor; partial results over disjoint key sets merge exactly.
 *      - section 九 (MLA): absorbed MLA is MQA with Q [heads, 576],
 *        one K head of 576 values, and V = the first 512 values of K.
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes): base-2 exponent and log throughout (natural base on request);
 * causal alignment is bottom-right (query i of s_q sees t <= L - s_q + i);
 * sparse index values < 0 or >= L are skipped, duplicates count twice; an
 * empty visible set gives lse = -inf and a zero output; dequantised value =
 * bf16_rne(float(decode(code)) * scale) with the product taken in float32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_D_QK 576
#define ORACLE_D_V 512
#define ORACLE_D_NOPE 512
#define ORACLE_ROW_BF16 1152
#define ORACLE_ROW_FP8 656

/* bf16 bit pattern -> value (exact: bf16 is the top half of an fp32). */
static float bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16 with round-to-nearest, ties to even (NaN stays a quiet NaN). */
uint16_t oracle_bf16_round(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7fffu + keep_lsb;
    return (uint16_t)(u >> 16);
}

/* OCP e4m3fn: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; exponent 15 with mantissa 7 is NaN; exponent 0 is subnormal
 * with value 2^-6 * m / 8. */
double oracle_e4m3_value(uint8_t c) {
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Nearest e4m3fn code to v (ties to the code with an even mantissa LSB),
 * saturated to +-448, sign from v's sign bit: a brute-force search over
 * the 127 finite magnitudes, every one exact in double, so each distance
 * is exact.  (FlashMLA page, "设计 2": codes are e4m3; the rounding rule is
 * this library's reading: round to nearest even, as IEEE conversions do.) */
uint8_t oracle_e4m3_encode(float v) {
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7e;
    int best = 0;
    double best_d = a;
    for (int c = 1; c <= 0x7e; ++c) {
        const double d = fabs(oracle_e4m3_value((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) != 0)) {
            best = c;
            best_d = d;
        }
    }
    return sign | (uint8_t)best;
}

/* One bf16 latent row (576 values) -> the 656-byte FP8 layout (FlashMLA
 * page, "设计 2"): per 1x128 tile k of the 512 NoPE values, amax = max |x|,
 * scale = amax / 448 as one float division (round to nearest even), code =
 * e4m3(x / scale) with the quotient also one float division; amax = 0 gives
 * scale 0 and all codes 0.  Bytes [0, 512) codes, [512, 528) the four
 * scales (little endian), [528, 656) the 64 RoPE values copied as bf16. */
void oracle_quantize_row_fp8(const uint16_t* x576, uint8_t* out656) {
    for (int k = 0; k < 4; ++k) {
        float amax = 0.0f;
        for (int d = 128 * k; d < 128 * (k + 1); ++d) {
            const float x = fabsf(bf16_value(x576[d]));
            if (x > amax) amax = x;
        }
        const float scale = amax / 448.0f;
        for (int d = 128 * k; d < 128 * (k + 1); ++d)
            out656[d] = amax == 0.0f ? 0 : oracle_e4m3_encode(bf16_value(x576[d]) / scale);
        memcpy(out656 + ORACLE_D_NOPE + 4 * k, &scale, 4);
    }
    memcpy(out656 + ORACLE_D_NOPE + 16, x576 + ORACLE_D_NOPE, 128);
}

/* Append n_new tokens per sequence to a paged FP8 cache: token j of
 * sequence b (bf16 row kv_new[b][j]) goes to logical position
 * t = start_pos[b] + j, i.e. slot t mod page_size of page
 * block_table[b][t div page_size] (Modular page, section 四: divmod of the
 * token index by the page size, then the block table).  Tokens whose page
 * index or page entry is out of range are skipped; nothing else is
 * written. */
void oracle_kv_append_fp8(int batch, int n_new, int page_size, int num_pages, int max_pages,
                          const uint16_t* kv_new, const int32_t* start_pos,
                          const int32_t* block_table, uint8_t* kv_pool) {
    for (int b = 0; b < batch; ++b)
        for (int j = 0; j < n_new; ++j) {
            const long t = (long)start_pos[b] + j;
            if (t < 0 || t / page_size >= max_pages) continue;
            const int page = block_table[(long)b * max_pages + t / page_size];
            if (page < 0 || page >= num_pages) continue;
            uint8_t* row = kv_pool + ((long)page * page_size + t % page_size) * ORACLE_ROW_FP8;
            oracle_quantize_row_fp8(kv_new + ((long)b * n_new + j) * ORACLE_D_QK, row);
        }
}

/* One cached latent row -> 576 values (bf16-exact, stored as float). */
void oracle_decode_row(const uint8_t* row, int kv_format, float* out576) {
    if (kv_format == 0) {
        const uint16_t* h = (const uint16_t*)row;
        for (int d = 0; d < ORACLE_D_QK; ++d) out576[d] = bf16_value(h[d]);
        return;
    }
    float scale[4];
    memcpy(scale, row + ORACLE_D_NOPE, 16);
    for (int d = 0; d < ORACLE_D_NOPE; ++d) {
        float v = (float)oracle_e4m3_value(row[d]); /* exact in float */
        float prod = v * scale[d / 128];           /* one fp32 rounding */
        out576[d] = bf16_value(oracle_bf16_round(prod));
    }
    const uint8_t* rope = row + ORACLE_D_NOPE + 16;
    for (int d = 0; d < 64; ++d) {
        uint16_t h;
        memcpy(&h, rope + 2 * d, 2);
        out576[ORACLE_D_NOPE + d] = bf16_value(h);
    }
}

/* Softmax over one list of scores, in base 2 or base e: returns lse and
 * writes normalised weights.  Empty list: lse = -inf. */
static double softmax_weights(const double* p, int n, int natural, double* w) {
    if (n == 0) return -INFINITY;
    double m = -INFINITY;
    for (int t = 0; t < n; ++t)
        if (p[t] > m) m = p[t];
    double sum = 0.0;
    for (int t = 0; t < n; ++t) sum += natural ? exp(p[t] - m) : exp2(p[t] - m);
    double lse = natural ? m + log(sum) : m + log2(sum);
    for (int t = 0; t < n; ++t) w[t] = natural ? exp(p[t] - lse) : exp2(p[t] - lse);
    return lse;
}

/* Attention of one query row (576 values) over rows K[0..n): out = w @ K[:, :512]. */
static double attend(const double* q, const float* K, int n, double scale,
                     int natural, double* p, double* w, double* out512) {
    for (int t = 0; t < n; ++t) {
        const float* k = K + (size_t)t * ORACLE_D_QK;
        double acc = 0.0;
        for (int d = 0; d < ORACLE_D_QK; ++d) acc += q[d] * (double)k[d];
        p[t] = acc * scale;
    }
    double lse = softmax_weights(p, n, natural, w);
    for (int j = 0; j < ORACLE_D_V; ++j) out512[j] = 0.0;
    for (int t = 0; t < n; ++t) {
        const float* k = K + (size_t)t * ORACLE_D_QK;
        for (int j = 0; j < ORACLE_D_V; ++j) out512[j] += w[t] * (double)k[j];
    }
    return lse;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Paged MLA decode.
 *   q            bf16 bits [batch, s_q, h_q, 576]
 *   kv           pool bytes [num_pages, page_size, row_bytes]
 *   block_table  int32 [batch, max_pages]
 *   seqlens      int32 [batch]
 *   indices      int32 [batch, s_q, topk] when topk > 0, else unused
 *   n_splits     1: plain definition.  >1: cut each visible list into that
 *                many contiguous chunks, attend over each, and merge the
 *                chunk results with the log-sum-exp identity.
 *   unit_mask    NULL, or uint8 [batch * s_q]: only (b, i) with a nonzero
 *                entry are computed; the others are left untouched.
 *   out          fp64 [batch, s_q, h_q, 512];  lse fp64 [batch, s_q, h_q]
 * Returns 0, or a negative value on a malformed argument.
 */
int oracle_mla_decode(int batch, int s_q, int h_q, int page_size, int num_pages,
                      int max_pages, int kv_format, int topk, int is_causal,
                      int natural, float softmax_scale, const uint16_t* q,
                      const uint8_t* kv, const int32_t* block_table,
                      const int32_t* seqlens, const int32_t* indices,
                      int n_splits, const uint8_t* unit_mask, double* out,
                      double* lse) {
    if (batch < 0 || s_q < 1 || h_q < 1 || page_size < 1 || n_splits < 1) return -1;
    if (topk > 0 && indices == NULL) return -2;
    const size_t row_bytes = kv_format == 0 ? ORACLE_ROW_BF16 : ORACLE_ROW_FP8;
    const double scale = (double)softmax_scale;
    int status = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < batch * s_q; ++u) {
        if (unit_mask && !unit_mask[u]) continue;
        const int b = u / s_q, i = u % s_q;
        const int L = seqlens[b];
        /* visible key list */
        int cap = topk > 0 ? topk : (L > 0 ? L : 0);
        int* vis = (int*)malloc(sizeof(int) * (size_t)(cap > 0 ? cap : 1));
        int n = 0;
        if (topk > 0) {
            for (int k = 0; k < topk; ++k) {
                int t = indices[((size_t)b * s_q + i) * topk + k];
                if (t >= 0 && t < L) vis[n++] = t;
            }
        } else {
            int last = is_causal ? L - s_q + i : L - 1; /* inclusive */
            for (int t = 0; t < L && t <= last; ++t) vis[n++] = t;
        }
        /* gather + decode rows through the block table */
        float* K = (float*)malloc(sizeof(float) * ORACLE_D_QK * (size_t)(n > 0 ? n : 1));
        int bad = 0;
        for (int v = 0; v < n; ++v) {
            int t = vis[v];
            int lp = t / page_size, slot = t % page_size;
            if (lp >= max_pages) { bad = 1; break; }
            int page = block_table[(size_t)b * max_pages + lp];
            if (page < 0 || page >= num_pages) { bad = 1; break; }
            const uint8_t* row = kv + ((size_t)page * page_size + slot) * row_bytes;
            oracle_decode_row(row, kv_format, K + (size_t)v * ORACLE_D_QK);
        }
        double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double* w = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double qd[ORACLE_D_QK];
        double part[ORACLE_D_V];
        double* part_o = (double*)malloc(sizeof(double) * ORACLE_D_V * (size_t)n_splits);
        double* part_l = (double*)malloc(sizeof(double) * (size_t)n_splits);
        for (int h = 0; h < h_q && !bad; ++h) {
            const size_t row = ((size_t)b * s_q + i) * h_q + h;
            for (int d = 0; d < ORACLE_D_QK; ++d) qd[d] = bf16_value(q[row * ORACLE_D_QK + d]);
            double* o = out + row * ORACLE_D_V;
            if (n_splits == 1) {
                lse[row] = attend(qd, K, n, scale, natural, p, w, o);
                continue;
            }
            /* split path: contiguous chunks of the visible list, then merge */
            for (int c = 0; c < n_splits; ++c) {
                int lo = (int)((long long)n * c / n_splits);
                int hi = (int)((long long)n * (c + 1) / n_splits);
                part_l[c] = attend(qd, K + (size_t)lo * ORACLE_D_QK, hi - lo, scale,
                                   natural, p, w, part);
                memcpy(part_o + (size_t)c * ORACLE_D_V, part, sizeof(part));
            }
            double M = -INFINITY;
            for (int c = 0; c < n_splits; ++c)
                if (part_l[c] > M) M = part_l[c];
            for (int j = 0; j < ORACLE_D_V; ++j) o[j] = 0.0;
            if (M == -INFINITY) { lse[row] = -INFINITY; continue; }
            double tot = 0.0;
            for (int c = 0; c < n_splits; ++c)
                tot += natural ? exp(part_l[c] - M) : exp2(part_l[c] - M);
            double L2 = natural ? M + log(tot) : M + log2(tot);
            for (int c = 0; c < n_splits; ++c) {
                double wc = natural ? exp(part_l[c] - L2) : exp2(part_l[c] - L2);
                for (int j = 0; j < ORACLE_D_V; ++j) o[j] += wc * part_o[(size_t)c * ORACLE_D_V + j];
            }
            lse[row] = L2;
        }
        if (bad) {
#pragma omp atomic write
            status = -3;
        }
        free(part_o); free(part_l); free(p); free(w); free(K); free(vis);
    }
    return status;
}
