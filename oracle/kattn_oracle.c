/*
 * kattn_oracle.c -- FP64 CPU oracle for packed variable-length attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's cpu_baseline leg load this library.  The GPU library never links,
 * includes or calls it, and this file shares no code, header, table or
 * constant with the GPU path.
 *
 * It is the plain definition of what the hot path computes, written out with
 * no blocking, fusion or reordering:
 *
 *   for every query row i of sequence s (rows cu[s] .. cu[s+1]-1, position
 *   i - cu[s]) and every q head h (kv head g = h / (H/G)):
 *     q' = RoPE(q_i, pos_i), k'_j = RoPE(k_j, pos_j)      (FP64, half-split pairs)
 *     S_ij = scale * <q', k'_j>                             for every j of s
 *     M_ij = 0 if visible(i, j) else -inf                   (materialised)
 *     P_i  = softmax_j(S_ij + M_ij)                         (two passes: max, then exp/sum)
 *     O_i  = sum_j P_ij v_j, rounded once to FP32.
 *
 * Sources (the pages are docs.rs source listings):
 *   - kime-cpu 0.0.17 `src/kime_cpu/plan.rs`: packed rows indexed by `cu`,
 *     position = row - cu[seq[row]] (`CpuBackend::run`, `Ctx::step` Rope and
 *     Attention arms); the qkv row holds q heads, then k heads, then v heads.
 *   - kime-cuda 0.0.3 `src/plan.rs`: `rope_tables` (how the cos/sin tables
 *     are rounded), the i32 window with -1 meaning none (`lower`, Attention).
 *   - ffai-argus 0.7.3 `src/text.rs`: module docs (skipping a masked column is
 *     the same as a -inf mask; 1/8 scale), `CausalSoftmax` (row max, exp,
 *     sum, masked tail zero), `KvAppend` (cache layout (heads, cap, 64) and
 *     in-place append at the position), the GQA fold in `block` (q heads
 *     [0,1,2] read kv head 0, ...), `rope` (candle's non-interleaved rope).
 *
 * Readings where the pages leave a step open are listed per function.
 *
 * Status: 0 on success, -1 on a bad argument (the oracle checks its inputs
 * and never reads out of range).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define HD 64          /* head width: the pages only lower heads of 64 */
#define HALF (HD / 2)  /* rotated pairs per head */

/*
 * cos/sin tables [len][32] for one RoPE base.  Reading R5 of the CUDA backend
 * page's `rope_tables` (which that page says matches the CPU backend):
 *   - the inverse frequency of pair i is the f32 reciprocal of theta^(i/32),
 *     the power evaluated in double and rounded to f32 (i/32 is exact in
 *     binary, so the exponent carries no rounding);
 *   - the angle at position p is p times that inverse frequency, formed in
 *     f32 (p itself is exact in f32);
 *   - the table entries are the cosine and sine of that f32 angle, evaluated
 *     in double and rounded to f32.
 */
static float inverse_frequency(double theta, int i) {
    const float power = (float)pow(theta, (double)i / HALF);
    return 1.0f / power;
}

int oracle_rope_tables(double theta, int32_t len, float* cos_out, float* sin_out) {
    if (len < 0 || !(theta > 0.0) || (len > 0 && (!cos_out || !sin_out))) return -1;
    for (int i = 0; i < HALF; ++i) {
        const float freq = inverse_frequency(theta, i);
        for (int32_t p = 0; p < len; ++p) {
            const float angle = (float)p * freq;
            cos_out[(int64_t)p * HALF + i] = (float)cos((double)angle);
            sin_out[(int64_t)p * HALF + i] = (float)sin((double)angle);
        }
    }
    return 0;
}

/*
 * RoPE of one 64-wide head in FP64 from the given f32 tables at position p.
 * Reading: half-split ("rotate-half") pairs (x[i], x[i+32]), i < 32, the
 * convention of candle's non-interleaved `rope` that the argus tower calls.
 *   y[i]    = x[i] cos - x[i+32] sin
 *   y[i+32] = x[i+32] cos + x[i] sin
 * With tables == NULL the head is copied unrotated (inputs already rotated).
 */
static void rope_head(const float* x, const float* cos_t, const float* sin_t, int32_t p,
                      double* y) {
    if (!cos_t) {
        for (int d = 0; d < HD; ++d) y[d] = (double)x[d];
        return;
    }
    const float* c = cos_t + (int64_t)p * HALF;
    const float* s = sin_t + (int64_t)p * HALF;
    for (int i = 0; i < HALF; ++i) {
        double a = (double)x[i], b = (double)x[i + HALF];
        double cc = (double)c[i], ss = (double)s[i];
        y[i] = a * cc - b * ss;
        y[i + HALF] = b * cc + a * ss;
    }
}

/*
 * The rotated rows the RoPE step leaves behind, rounded once to f32:
 * out[r][h*64 + d] = f32(RoPE(x[r][h*64 ..], pos[r])[d]) for r < T, h < heads.
 * The step rotates q heads and k heads only; v is never touched
 * (kime-cpu plan.rs, `Ctx::step` Rope arm: the first two thirds of the row).
 */
int oracle_rope_apply(float* out, int64_t out_stride, const float* x, int64_t x_stride,
                      int32_t T, int32_t heads, const int32_t* pos, const float* cos_t,
                      const float* sin_t, int32_t table_len) {
    if (T < 0 || heads < 1 || !out || !x || !pos || !cos_t || !sin_t) return -1;
    if (out_stride < (int64_t)heads * HD || x_stride < (int64_t)heads * HD) return -1;
    for (int32_t r = 0; r < T; ++r)
        if (pos[r] < 0 || pos[r] >= table_len) return -1;
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < T; ++r) {
        double y[HD];
        for (int32_t h = 0; h < heads; ++h) {
            rope_head(x + (int64_t)r * x_stride + (int64_t)h * HD, cos_t, sin_t, pos[r], y);
            for (int d = 0; d < HD; ++d)
                out[(int64_t)r * out_stride + (int64_t)h * HD + d] = (float)y[d];
        }
    }
    return 0;
}

/* visible(i, j) for positions inside one sequence.
 * Reading of the window: `window = w` is the full width of a bidirectional
 * local layer, so key j is visible from query i when |i - j| <= floor(w/2);
 * w < 0 means no window (the CUDA page's -1).  Causal keeps j <= i. */
static int visible(int32_t i, int32_t j, int32_t window, int32_t causal) {
    if (causal && j > i) return 0;
    if (window >= 0) {
        int32_t d = i > j ? i - j : j - i;
        if (d > window / 2) return 0;
    }
    return 1;
}

static int check_cu(const int32_t* cu, int32_t S, int32_t T) {
    if (!cu || S < 0 || T < 0) return -1;
    if (cu[0] != 0 || cu[S] != T) return -1;
    for (int32_t s = 0; s < S; ++s)
        if (cu[s + 1] < cu[s]) return -1;
    return 0;
}

/*
 * Varlen attention over a packed batch.
 *
 * q: (T, H*64) row stride q_stride; k, v: (T, G*64) strides k_stride, v_stride.
 * cu: [S+1] cumulative offsets.  cos_t/sin_t: the oracle's own tables
 * (oracle_rope_tables) or NULL for inputs that are already rotated.
 * rows == NULL: every row r < T, written to out + r*out_stride.
 * rows != NULL: the listed rows, row t of the list written to out + t*out_stride.
 * mask_mode 0: materialise M_ij = -inf and add it (the definition).
 * mask_mode 1: leave masked columns out of the max, the sum and P.V (the
 *              skip the argus text.rs module docs argue is bit-identical).
 * threads <= 0: the OpenMP default.
 * The RoPE step comes first, as in the pages' plan (a Rope step, then the
 * Attention step): every key row is rotated once, in FP64, at its position
 * inside its sequence, and the scores read those rotated keys.  Queries are
 * rotated as their rows are visited.
 */
static int varlen_attention(void* out, int out_f64, int64_t out_stride, const float* q,
                            int64_t q_stride, const float* k, int64_t k_stride, const float* v,
                            int64_t v_stride, const int32_t* cu, int32_t S, int32_t T, int32_t H,
                            int32_t G, int32_t window, int32_t causal, double scale,
                            const float* cos_t, const float* sin_t, int32_t table_len,
                            const int32_t* rows, int32_t nrows, int32_t mask_mode,
                            int32_t threads) {
    if (check_cu(cu, S, T) != 0) return -1;
    if (!out || !q || !k || !v || H < 1 || G < 1 || H % G != 0) return -1;
    if (q_stride < (int64_t)H * HD || k_stride < (int64_t)G * HD || v_stride < (int64_t)G * HD)
        return -1;
    if (out_stride < (int64_t)H * HD) return -1;
    if ((cos_t == NULL) != (sin_t == NULL)) return -1;
    int32_t max_len = 0;
    for (int32_t s = 0; s < S; ++s)
        if (cu[s + 1] - cu[s] > max_len) max_len = cu[s + 1] - cu[s];
    if (cos_t && table_len < max_len) return -1;
    int32_t n_out = rows ? nrows : T;
    if (n_out < 0) return -1;
    if (rows)
        for (int32_t t = 0; t < nrows; ++t)
            if (rows[t] < 0 || rows[t] >= T) return -1;
    const int32_t R = H / G; /* q heads per kv head */
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
    /* the RoPE step on the keys: krot[(r*G + g)*64 + d] = RoPE(k row r, head g, pos r - cu[s]) */
    double* krot = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * (size_t)G * HD);
    if (!krot) return -1;
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < T; ++r) {
        int32_t a = 0, b = S - 1; /* the last sequence s with cu[s] <= r (empty ones skipped) */
        while (a < b) {
            int32_t mid = (a + b + 1) / 2;
            if (cu[mid] <= r) a = mid; else b = mid - 1;
        }
        for (int32_t g = 0; g < G; ++g)
            rope_head(k + (int64_t)r * k_stride + (int64_t)g * HD, cos_t, sin_t, r - cu[a],
                      krot + ((int64_t)r * G + g) * HD);
    }
    int bad = 0;
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
        double* e = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
        if (!z || !e) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int32_t t = 0; t < n_out; ++t) {
                int32_t r = rows ? rows[t] : t;
                int32_t s = 0; /* the sequence holding row r */
                while (!(cu[s] <= r && r < cu[s + 1])) ++s;
                int32_t lo = cu[s], n = cu[s + 1] - cu[s], i = r - lo;
                for (int32_t h = 0; h < H; ++h) {
                    int32_t g = h / R;
                    double qr[HD];
                    rope_head(q + (int64_t)r * q_stride + (int64_t)h * HD, cos_t, sin_t, i, qr);
                    /* scores and the additive mask over every key of the sequence */
                    for (int32_t j = 0; j < n; ++j) {
                        int vis = visible(i, j, window, causal);
                        if (mask_mode == 1 && !vis) continue;
                        const double* kr = krot + ((int64_t)(lo + j) * G + g) * HD;
                        double dot = 0.0;
                        for (int d = 0; d < HD; ++d) dot += qr[d] * kr[d];
                        double sij = scale * dot;
                        double mij = vis ? 0.0 : -INFINITY;
                        z[j] = sij + mij;
                    }
                    /* pass 1: row max (the diagonal is always visible, so it is finite) */
                    double m = -INFINITY;
                    for (int32_t j = 0; j < n; ++j) {
                        if (mask_mode == 1 && !visible(i, j, window, causal)) continue;
                        if (z[j] > m) m = z[j];
                    }
                    /* pass 2: exponentials and their sum */
                    double l = 0.0;
                    for (int32_t j = 0; j < n; ++j) {
                        if (mask_mode == 1 && !visible(i, j, window, causal)) continue;
                        e[j] = exp(z[j] - m);
                        l += e[j];
                    }
                    /* P = e / l, O = P V */
                    double o[HD];
                    for (int d = 0; d < HD; ++d) o[d] = 0.0;
                    for (int32_t j = 0; j < n; ++j) {
                        if (mask_mode == 1 && !visible(i, j, window, causal)) continue;
                        double p = e[j] / l;
                        const float* vj = v + (int64_t)(lo + j) * v_stride + (int64_t)g * HD;
                        for (int d = 0; d < HD; ++d) o[d] += p * (double)vj[d];
                    }
                    if (out_f64) {
                        double* orow = (double*)out + (int64_t)t * out_stride + (int64_t)h * HD;
                        for (int d = 0; d < HD; ++d) orow[d] = o[d];
                    } else {
                        float* orow = (float*)out + (int64_t)t * out_stride + (int64_t)h * HD;
                        for (int d = 0; d < HD; ++d) orow[d] = (float)o[d];
                    }
                }
            }
        }
        free(z);
        free(e);
    }
    free(krot);
    return bad ? -1 : 0;
}

int oracle_varlen_attention(float* out, int64_t out_stride, const float* q, int64_t q_stride,
                            const float* k, int64_t k_stride, const float* v, int64_t v_stride,
                            const int32_t* cu, int32_t S, int32_t T, int32_t H, int32_t G,
                            int32_t window, int32_t causal, double scale, const float* cos_t,
                            const float* sin_t, int32_t table_len, const int32_t* rows,
                            int32_t nrows, int32_t mask_mode, int32_t threads) {
    return varlen_attention(out, 0, out_stride, q, q_stride, k, k_stride, v, v_stride, cu, S, T,
                            H, G, window, causal, scale, cos_t, sin_t, table_len, rows, nrows,
                            mask_mode, threads);
}

/*
 * The same, with the FP64 result left unrounded (for outputs of another
 * precision, which are then rounded once from FP64).
 */
int oracle_varlen_attention64(double* out, int64_t out_stride, const float* q, int64_t q_stride,
                              const float* k, int64_t k_stride, const float* v, int64_t v_stride,
                              const int32_t* cu, int32_t S, int32_t T, int32_t H, int32_t G,
                              int32_t window, int32_t causal, double scale, const float* cos_t,
                              const float* sin_t, int32_t table_len, const int32_t* rows,
                              int32_t nrows, int32_t mask_mode, int32_t threads) {
    return varlen_attention(out, 1, out_stride, q, q_stride, k, k_stride, v, v_stride, cu, S, T,
                            H, G, window, causal, scale, cos_t, sin_t, table_len, rows, nrows,
                            mask_mode, threads);
}

/*
 * One decode step against preallocated per-sequence caches
 * (ffai-argus text.rs: `KvAppend`, the KV-cache part of `block`, and
 * `CausalSoftmax` with q_len 1 and offset L-1).
 *
 * q_new: [B][H*64], k_new, v_new: [B][G*64]; caches [B][G][cap][64] (the
 * page's (kv_heads, cap, 64) layout stacked over the batch).  used[b] = L_b
 * counts the new token.  For each b, with p = L_b - 1:
 *   1. the new k is rotated at p (f64, rounded to f32) and written with the
 *      new v into cache row p of every kv head (other rows untouched);
 *   2. the new q is rotated at p and kept in f64;
 *   3. every cached row 0..L_b-1 (f32 values as stored) is scored, with no
 *      mask: a decode row is the last causal row, so it sees the whole cache;
 *   4. two-pass softmax and P.V in f64, one rounding to f32.
 * With cos_t == NULL the new q and k are taken as already rotated.
 * The caches passed in are modified (the caller hands the oracle copies).
 */
int oracle_decode(float* out, const float* q_new, const float* k_new, const float* v_new,
                  float* k_cache, float* v_cache, int32_t cap, const int32_t* used, int32_t B,
                  int32_t H, int32_t G, double scale, const float* cos_t, const float* sin_t,
                  int32_t table_len, int32_t threads) {
    if (!out || !q_new || !k_new || !v_new || !k_cache || !v_cache || !used) return -1;
    if (B < 0 || H < 1 || G < 1 || H % G != 0 || cap < 1) return -1;
    if ((cos_t == NULL) != (sin_t == NULL)) return -1;
    for (int32_t b = 0; b < B; ++b) {
        if (used[b] < 1 || used[b] > cap) return -1;
        if (cos_t && used[b] > table_len) return -1;
    }
    const int32_t R = H / G;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
    /* step 1: append */
    for (int32_t b = 0; b < B; ++b) {
        int32_t p = used[b] - 1;
        for (int32_t g = 0; g < G; ++g) {
            double kr[HD];
            rope_head(k_new + ((int64_t)b * G + g) * HD, cos_t, sin_t, p, kr);
            float* krow = k_cache + (((int64_t)b * G + g) * cap + p) * HD;
            float* vrow = v_cache + (((int64_t)b * G + g) * cap + p) * HD;
            const float* vn = v_new + ((int64_t)b * G + g) * HD;
            for (int d = 0; d < HD; ++d) {
                krow[d] = (float)kr[d];
                vrow[d] = vn[d];
            }
        }
    }
    int bad = 0;
#pragma omp parallel
    {
        int32_t maxl = 1;
        for (int32_t b = 0; b < B; ++b)
            if (used[b] > maxl) maxl = used[b];
        double* z = (double*)malloc(sizeof(double) * (size_t)maxl);
        if (!z) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
                int32_t b = (int32_t)(bh / H), h = (int32_t)(bh % H), g = h / R;
                int32_t L = used[b], p = L - 1;
                double qr[HD];
                rope_head(q_new + ((int64_t)b * H + h) * HD, cos_t, sin_t, p, qr);
                const float* kb = k_cache + ((int64_t)b * G + g) * cap * HD;
                const float* vb = v_cache + ((int64_t)b * G + g) * cap * HD;
                double m = -INFINITY;
                for (int32_t j = 0; j < L; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < HD; ++d) dot += qr[d] * (double)kb[(int64_t)j * HD + d];
                    z[j] = scale * dot;
                    if (z[j] > m) m = z[j];
                }
                double l = 0.0;
                for (int32_t j = 0; j < L; ++j) {
                    z[j] = exp(z[j] - m);
                    l += z[j];
                }
                double o[HD];
                for (int d = 0; d < HD; ++d) o[d] = 0.0;
                for (int32_t j = 0; j < L; ++j) {
                    double pj = z[j] / l;
                    for (int d = 0; d < HD; ++d) o[d] += pj * (double)vb[(int64_t)j * HD + d];
                }
                float* orow = out + ((int64_t)b * H + h) * HD;
                for (int d = 0; d < HD; ++d) orow[d] = (float)o[d];
            }
        }
        free(z);
    }
    return bad ? -1 : 0;
}

/*
 * Chunked prefill that continues from a KV cache (ffai-argus text.rs:
 * `KvAppend` at the cache's fill point, then `CausalSoftmax` with q_len > 1
 * and an offset, whose causal limit for query i is key offset + i).
 *
 * Sequence b of the batch brings n_b = cu[b+1] - cu[b] new rows (packed rows
 * cu[b] .. cu[b+1]-1 of q, k_new, v_new) and already holds off_b = offset[b]
 * rows in its caches [B][G][cap][64].  Reading taken: the new rows sit at
 * positions off_b + i (RoPE and cache row), which is where the page's
 * append puts them.  For each b:
 *   1. k_new row i is rotated at off_b + i (f64, rounded to f32) and written
 *      with v_new row i into cache row off_b + i of every kv head;
 *   2. q row i is rotated at off_b + i and kept in f64;
 *   3. it is scored against the stored f32 cache rows 0 .. off_b + i (rows
 *      past the causal limit are masked out, which is the same as -inf);
 *   4. two-pass softmax and P.V in f64, one rounding to f32, into out row
 *      cu[b] + i.
 * With n_b = 1 this is exactly one decode step with L = off_b + 1, and the
 * arithmetic is done in the same order as oracle_decode.
 * Requires 0 <= off_b and off_b + n_b <= cap (and <= table_len when rotating).
 * The caches passed in are modified (the caller hands the oracle copies).
 */
int oracle_prefill_cached(float* out, int64_t out_stride, const float* q, int64_t q_stride,
                          const float* k_new, int64_t k_stride, const float* v_new,
                          int64_t v_stride, const int32_t* cu, const int32_t* offset, int32_t B,
                          int32_t T, float* k_cache, float* v_cache, int32_t cap, int32_t H,
                          int32_t G, double scale, const float* cos_t, const float* sin_t,
                          int32_t table_len, int32_t threads) {
    if (check_cu(cu, B, T) != 0) return -1;
    if (!out || !q || !k_new || !v_new || !k_cache || !v_cache || !offset) return -1;
    if (H < 1 || G < 1 || H % G != 0 || cap < 1) return -1;
    if (q_stride < (int64_t)H * HD || k_stride < (int64_t)G * HD || v_stride < (int64_t)G * HD ||
        out_stride < (int64_t)H * HD)
        return -1;
    if ((cos_t == NULL) != (sin_t == NULL)) return -1;
    int32_t max_ctx = 1;
    for (int32_t b = 0; b < B; ++b) {
        int32_t n = cu[b + 1] - cu[b];
        if (offset[b] < 0 || (int64_t)offset[b] + n > cap) return -1;
        if (cos_t && (int64_t)offset[b] + n > table_len) return -1;
        if (offset[b] + n > max_ctx) max_ctx = offset[b] + n;
    }
    const int32_t R = H / G;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
    /* step 1: append the chunk */
    for (int32_t b = 0; b < B; ++b) {
        for (int32_t i = 0; i < cu[b + 1] - cu[b]; ++i) {
            int32_t r = cu[b] + i, p = offset[b] + i;
            for (int32_t g = 0; g < G; ++g) {
                double kr[HD];
                rope_head(k_new + (int64_t)r * k_stride + (int64_t)g * HD, cos_t, sin_t, p, kr);
                float* krow = k_cache + (((int64_t)b * G + g) * cap + p) * HD;
                float* vrow = v_cache + (((int64_t)b * G + g) * cap + p) * HD;
                const float* vn = v_new + (int64_t)r * v_stride + (int64_t)g * HD;
                for (int d = 0; d < HD; ++d) {
                    krow[d] = (float)kr[d];
                    vrow[d] = vn[d];
                }
            }
        }
    }
    int bad = 0;
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)max_ctx);
        if (!z) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t rh = 0; rh < (int64_t)T * H; ++rh) {
                int32_t r = (int32_t)(rh / H), h = (int32_t)(rh % H), g = h / R;
                int32_t b = 0; /* the sequence holding row r */
                while (!(cu[b] <= r && r < cu[b + 1])) ++b;
                int32_t p = offset[b] + (r - cu[b]); /* this query's position */
                int32_t L = p + 1;                   /* keys 0 .. p are visible */
                double qr[HD];
                rope_head(q + (int64_t)r * q_stride + (int64_t)h * HD, cos_t, sin_t, p, qr);
                const float* kb = k_cache + ((int64_t)b * G + g) * cap * HD;
                const float* vb = v_cache + ((int64_t)b * G + g) * cap * HD;
                double m = -INFINITY;
                for (int32_t j = 0; j < L; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < HD; ++d) dot += qr[d] * (double)kb[(int64_t)j * HD + d];
                    z[j] = scale * dot;
                    if (z[j] > m) m = z[j];
                }
                double l = 0.0;
                for (int32_t j = 0; j < L; ++j) {
                    z[j] = exp(z[j] - m);
                    l += z[j];
                }
                double o[HD];
                for (int d = 0; d < HD; ++d) o[d] = 0.0;
                for (int32_t j = 0; j < L; ++j) {
                    double pj = z[j] / l;
                    for (int d = 0; d < HD; ++d) o[d] += pj * (double)vb[(int64_t)j * HD + d];
                }
                float* orow = out + (int64_t)r * out_stride + (int64_t)h * HD;
                for (int d = 0; d < HD; ++d) orow[d] = (float)o[d];
            }
        }
        free(z);
    }
    return bad ? -1 : 0;
}
