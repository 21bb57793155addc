/*
 * oracle.c -- plain, slow CPU reference of the Muse Glimmer attention core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library: every step below is written from the pages' definitions.
 *
 * Sources (the four pages bundled with the task; cited by title and section):
 *   [Ch9]  "Chapter 9 - The Muse Glimmer architecture"
 *   [Ch14] "Chapter 14 - QK-norm and RoPE - rotating only the layers that rotate"
 *   [News] "How Muse Glimmer Fits an Agent on Your Device"
 *
 * Arithmetic: every intermediate is an IEEE double.  The only roundings to a
 * narrower type are the ones the method itself fixes:
 *   - the RoPE frequency table is a table of f32 values ([Ch14] 14.4.1), and
 *     the angle pos*theta_i is an f32 product ([Ch14] 14.5 kernel listing);
 *   - the KV cache stores K-hat and V in the storage dtype (f32 or bf16),
 *     rounded to nearest, ties to even.
 * Softmax is the plain definition (max-shifted for range, which is exact).
 * No tiling, no online softmax, no split-K.
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_D 128     /* head_dim, [Ch9] 9.2: key_length 128           */
#define OR_H 32      /* query heads, [Ch9] 9.6                         */
#define OR_G 2       /* KV heads, [Ch9] 9.6                            */
#define OR_HPG 16    /* query heads per KV head, [Ch9] Figure 9.3      */

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_SLIDING_ROPE = 0, OR_FULL_NOPE = 1 };
enum { OR_ANGLE_F32 = 0, OR_ANGLE_EXACT = 1 };

/* Layer parameters.  Plain doubles: the caller passes the exact value of the
 * f32 parameters the library receives. */
typedef struct {
    int32_t kind;        /* OR_SLIDING_ROPE or OR_FULL_NOPE                     */
    int32_t window;      /* sliding: keys with p - j < window are visible       */
    double  rope_theta;  /* RoPE base (sliding only)                            */
    double  rms_eps;     /* QK-norm epsilon                                     */
    double  q_gain;      /* constant QK-norm weight for Q ([Ch14] 14.3)         */
    double  k_gain;      /* constant QK-norm weight for K                       */
    double  scale;       /* softmax scale, 1/sqrt(128) ([Ch9] 9.5)              */
    int32_t store_dtype; /* dtype of the KV cache (and of all inputs)           */
    int32_t angle_mode;  /* OR_ANGLE_F32 (the method) or OR_ANGLE_EXACT (pins)  */
} oracle_layer;

/* ---------------------------------------------------------------- scalars */

/* Layer kind: full (NoPE) iff l % 4 == 3 ([Ch9] 9.4 listing, Figure 9.4). */
int oracle_layer_kind(int layer) { return (layer % 4 == 3) ? OR_FULL_NOPE : OR_SLIDING_ROPE; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the following calls use (n >= 1; for timing the oracle on one core). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Value of a bf16 bit pattern (bf16 is the top half of an IEEE f32). */
static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value (ties to even), returned as a
 * double.  bf16 = 1 sign, 8 exponent, 7 stored mantissa bits: 8 significant
 * bits for normal numbers, a fixed quantum of 2^-133 below 2^-126.  The
 * rounding is done once, directly from the double. */
double oracle_round_bf16(double x) {
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    double ax = fabs(x);
    double r;
    if (ax < ldexp(1.0, -126)) {
        r = ldexp(nearbyint(ldexp(x, 133)), -133);          /* subnormal range */
    } else {
        int e;
        double m = frexp(x, &e);                             /* x = m * 2^e, |m| in [0.5, 1) */
        r = ldexp(nearbyint(ldexp(m, 8)), e - 8);            /* 8 significant bits */
    }
    /* largest finite bf16 is (2 - 2^-7) * 2^127; beyond its rounding midpoint -> inf */
    if (fabs(r) > ldexp(255.0, 120)) r = copysign(INFINITY, x);
    return r;
}

/* Round to the storage dtype (f32 via C's correctly rounded conversion). */
double oracle_round_store(double x, int dtype) {
    return dtype == OR_BF16 ? oracle_round_bf16(x) : (double)(float)x;
}

/* Element i of an f32 or bf16 array, as a double (exact). */
static double load_elem(const void* p, int64_t i, int dtype) {
    if (dtype == OR_BF16) return bf16_bits_to_double(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

/* ------------------------------------------------------------ A1 QK-norm */

/* Per-head RMSNorm with a constant weight ([Ch9] 9.5 formula; [Ch14] 14.3):
 *   y = x / sqrt(mean(x^2) + eps) * gain. */
void oracle_rms_norm(const double* x, int n, double eps, double gain, double* y) {
    double ss = 0.0;
    for (int d = 0; d < n; ++d) ss += x[d] * x[d];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int d = 0; d < n; ++d) y[d] = x[d] * r * gain;
}

/* ------------------------------------------------------------- A2 RoPE */

/* Frequency table theta_i = base^(-2i/n), i < n/2, as f32 values
 * ([Ch14] 14.4.1: one table per engine, built in f32).  Evaluated in double
 * and rounded once to f32. */
void oracle_rope_theta_table(double base, int n, float* out) {
    for (int i = 0; i < n / 2; ++i) out[i] = (float)pow(base, -(2.0 * i) / (double)n);
}

/* Rotate the adjacent (GPT-J / "NORM") pairs (x[2i], x[2i+1]) of an n-vector
 * by angle a_i = pos * theta_i ([Ch14] 14.1 formula, 14.4.2, Figure 14.2):
 *   x0' = x0 cos a - x1 sin a,   x1' = x0 sin a + x1 cos a.
 * OR_ANGLE_F32: theta_i is the f32 table value and a_i the f32 product
 *   (an integer below 2^24 times an f32 is exact in a double, so rounding
 *   that product once to f32 is the f32 multiply of [Ch14] 14.5).
 * OR_ANGLE_EXACT: theta_i and a_i in double (used only by invariant pins). */
void oracle_rope(const double* x, int n, int64_t pos, double base, int angle_mode, double* y) {
    for (int i = 0; i < n / 2; ++i) {
        double a;
        if (angle_mode == OR_ANGLE_EXACT) {
            a = (double)pos * pow(base, -(2.0 * i) / (double)n);
        } else {
            float th = (float)pow(base, -(2.0 * i) / (double)n);
            a = (double)(float)((double)pos * (double)th);
        }
        double c = cos(a), s = sin(a);
        double x0 = x[2 * i], x1 = x[2 * i + 1];
        y[2 * i] = x0 * c - x1 * s;
        y[2 * i + 1] = x0 * s + x1 * c;
    }
}

/* Norm then (sliding layers only) RoPE of one head vector held in the
 * storage dtype: the per-head transform applied to Q and K before attention
 * ([Ch14] 14.1 steps 1-3; NoPE on full layers, [Ch9] 9.7). */
static void norm_rope_head(const oracle_layer* L, const void* src, int64_t off, int dtype,
                           double gain, int64_t pos, double* y) {
    double x[OR_D], t[OR_D];
    for (int d = 0; d < OR_D; ++d) x[d] = load_elem(src, off + d, dtype);
    oracle_rms_norm(x, OR_D, L->rms_eps, gain, t);
    if (L->kind == OR_SLIDING_ROPE)
        oracle_rope(t, OR_D, pos, L->rope_theta, L->angle_mode, y);
    else
        memcpy(y, t, sizeof t);
}

/* ------------------------------------------------------- A9 sigmoid gate */

/* sigma(g) = 1 / (1 + e^-g) ([Ch9] 9.8 listing). */
double oracle_sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }

/* ------------------------------------------------- A3 + A4..A9, one layer */

/*
 * One attention layer over a batch of sequences, evaluated for a chosen list
 * of (sequence, new-token) rows.
 *
 *   seq_len[s]       rows already in sequence s's cache (its prefix length L_s)
 *   k_new, v_new     [S][N][2][128] raw K and V of the N new tokens
 *   cache_k/v        [S][capacity][2][128] prefix rows (rows j < L_s are read)
 *   rows             n_rows pairs (s, t), t < N; the new token t of sequence s
 *                    sits at position p = L_s + t
 *   q_rows           [n_rows][32][128] raw Q of those rows
 *   gate_rows        [n_rows][4096]   gate of those rows
 *   out              [n_rows][4096]   gated attention output (double)
 *   k_store, v_store [S][N][2][128]   the rows this layer appends to the
 *                    cache, as stored (double holding storage-dtype values);
 *                    may be NULL
 * All arrays other than out/k_store/v_store are in L->store_dtype.
 *
 * Steps, for every new token (s, t) at p = L_s + t:
 *  1. K-hat = QK-norm(K) with k_gain, then RoPE at p on sliding layers; the
 *     cache row p receives round_store(K-hat) and V unchanged ([Ch14] 14.7:
 *     rotate before the store; V is never rotated).  All N new rows are
 *     appended before any attention: the chunk is causal within itself.
 *  2. Q-hat = QK-norm(Q) with q_gain, then RoPE at p on sliding layers.
 *  3. Visible keys j: j <= p, and on sliding layers p - j < window
 *     ([Ch9] 9.7); full layers see every j <= p.
 *  4. Query head h reads KV head g = h / 16 ([Ch9] Figure 9.3).
 *     score_j = (Q-hat_h . Kcache_j) * scale ([Ch9] 9.5).
 *  5. w_j = softmax(score)_j;  o_h = sum_j w_j Vcache_j.
 *  6. out[h*128 + d] = o_h[d] * sigma(gate[h*128 + d]) ([Ch9] 9.8).
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_attn_rows(const oracle_layer* L, int n_seq, int n_new, const int32_t* seq_len,
                     const void* k_new, const void* v_new,
                     const void* cache_k, const void* cache_v, int64_t capacity,
                     int n_rows, const int32_t* row_s, const int32_t* row_t,
                     const void* q_rows, const void* gate_rows,
                     double* out, double* k_store, double* v_store) {
    if (!L || n_seq < 0 || n_new < 0 || n_rows < 0) return -1;
    if (L->kind == OR_SLIDING_ROPE && L->window < 1) return -1;
    const int dt = L->store_dtype;
    const int64_t kv_row = (int64_t)OR_G * OR_D;         /* elements per token in K or V */

    /* step 1: the appended rows, as stored */
    int64_t n_app = (int64_t)n_seq * n_new * kv_row;
    double* kst = (double*)malloc(sizeof(double) * (n_app > 0 ? n_app : 1));
    double* vst = (double*)malloc(sizeof(double) * (n_app > 0 ? n_app : 1));
    if (!kst || !vst) { free(kst); free(vst); return -1; }
    int64_t max_vis = 1;
    for (int s = 0; s < n_seq; ++s) {
        if (seq_len[s] < 0 || (int64_t)seq_len[s] + n_new > capacity) { free(kst); free(vst); return -1; }
        int64_t v = (int64_t)seq_len[s] + n_new;
        if (v > max_vis) max_vis = v;
    }
#pragma omp parallel for schedule(static)
    for (int64_t st = 0; st < (int64_t)n_seq * n_new; ++st) {
        int s = (int)(st / (n_new > 0 ? n_new : 1));
        int t = (int)(st % (n_new > 0 ? n_new : 1));
        int64_t p = (int64_t)seq_len[s] + t;
        for (int g = 0; g < OR_G; ++g) {
            int64_t off = st * kv_row + (int64_t)g * OR_D;
            double kh[OR_D];
            norm_rope_head(L, k_new, off, dt, L->k_gain, p, kh);
            for (int d = 0; d < OR_D; ++d) {
                kst[off + d] = oracle_round_store(kh[d], dt);
                vst[off + d] = load_elem(v_new, off + d, dt);
            }
        }
    }

    /* steps 2-6, one (row, head) at a time */
    int bad = 0;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)max_vis);
        if (!w) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t rh = 0; rh < (int64_t)n_rows * OR_H; ++rh) {
            if (!w) continue;
            int r = (int)(rh / OR_H), h = (int)(rh % OR_H);
            int s = row_s[r], t = row_t[r];
            if (s < 0 || s >= n_seq || t < 0 || t >= n_new) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int64_t Ls = seq_len[s];
            int64_t p = Ls + t;
            int g = h / OR_HPG;
            double qh[OR_D];
            norm_rope_head(L, q_rows, ((int64_t)r * OR_H + h) * OR_D, dt, L->q_gain, p, qh);

            int64_t lo = 0;
            if (L->kind == OR_SLIDING_ROPE) { lo = p - L->window + 1; if (lo < 0) lo = 0; }

            double m = -INFINITY;
            for (int64_t j = lo; j <= p; ++j) {
                double dot = 0.0;
                if (j < Ls) {
                    int64_t off = (((int64_t)s * capacity + j) * OR_G + g) * OR_D;
                    for (int d = 0; d < OR_D; ++d) dot += qh[d] * load_elem(cache_k, off + d, dt);
                } else {
                    int64_t off = (((int64_t)s * n_new + (j - Ls)) * OR_G + g) * OR_D;
                    for (int d = 0; d < OR_D; ++d) dot += qh[d] * kst[off + d];
                }
                double sc = dot * L->scale;
                w[j - lo] = sc;
                if (sc > m) m = sc;
            }
            double den = 0.0, o[OR_D];
            for (int d = 0; d < OR_D; ++d) o[d] = 0.0;
            for (int64_t j = lo; j <= p; ++j) {
                double e = exp(w[j - lo] - m);
                den += e;
                if (j < Ls) {
                    int64_t off = (((int64_t)s * capacity + j) * OR_G + g) * OR_D;
                    for (int d = 0; d < OR_D; ++d) o[d] += e * load_elem(cache_v, off + d, dt);
                } else {
                    int64_t off = (((int64_t)s * n_new + (j - Ls)) * OR_G + g) * OR_D;
                    for (int d = 0; d < OR_D; ++d) o[d] += e * vst[off + d];
                }
            }
            for (int d = 0; d < OR_D; ++d) {
                int64_t c = (int64_t)h * OR_D + d;
                double gv = load_elem(gate_rows, (int64_t)r * OR_H * OR_D + c, dt);
                out[(int64_t)r * OR_H * OR_D + c] = (o[d] / den) * oracle_sigmoid(gv);
            }
        }
        free(w);
    }
    if (k_store) memcpy(k_store, kst, sizeof(double) * (size_t)n_app);
    if (v_store) memcpy(v_store, vst, sizeof(double) * (size_t)n_app);
    free(kst);
    free(vst);
    return bad ? -1 : 0;
}

/* ------------------------------- next step: o_proj and the post-attention norm */

/*
 * The attention block's tail ([Ch9] 9.8 and 9.9, Figure 9.1): the gated
 * attention output goes through o_proj [4096 -> 6656], the post-attention
 * RMSNorm (its own epsilon, 1e-8 in the model) scales the projection, and
 * the result joins the residual stream:
 *
 *   proj[n] = sum_k attn[k] * W[n][k]              (W is [n_out][k_in])
 *   y[n]    = proj[n] / sqrt(mean_n(proj^2) + eps) * gamma[n] + residual[n]
 *
 * gamma is the norm's effective gain: [News] ("Sandwich norms control what
 * each branch writes") stores it as an offset from one; the caller passes
 * the gain itself.  attn, W and residual are bf16 bit patterns; gamma is f32.
 * Rows (tokens) are independent, so a chosen list of rows is evaluated.
 * Everything is double; nothing is rounded.  proj_out may be NULL.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_out_proj(int64_t n_rows_total, int k_in, int n_out, const uint16_t* attn, const uint16_t* w,
                    const float* gamma, const uint16_t* residual, double eps,
                    int64_t n_rows, const int64_t* rows, double* y_out, double* proj_out) {
    if (k_in <= 0 || n_out <= 0 || n_rows < 0 || !attn || !w || !gamma || !residual || !rows || !y_out)
        return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= n_rows_total) return -1;
    double* wd = (double*)malloc(sizeof(double) * (size_t)n_out * (size_t)k_in);
    if (!wd) return -1;
    for (int64_t i = 0; i < (int64_t)n_out * k_in; ++i) wd[i] = bf16_bits_to_double(w[i]);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t t = rows[r];
        double* x = (double*)malloc(sizeof(double) * (size_t)k_in);
        double* p = (double*)malloc(sizeof(double) * (size_t)n_out);
        if (!x || !p) {
            free(x);
            free(p);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        for (int k = 0; k < k_in; ++k) x[k] = bf16_bits_to_double(attn[t * k_in + k]);
        double ss = 0.0;
        for (int n = 0; n < n_out; ++n) {
            const double* wr = wd + (int64_t)n * k_in;
            double acc = 0.0;
            for (int k = 0; k < k_in; ++k) acc += x[k] * wr[k];
            p[n] = acc;
            ss += acc * acc;
        }
        const double inv = 1.0 / sqrt(ss / (double)n_out + eps);
        for (int n = 0; n < n_out; ++n) {
            y_out[r * n_out + n] = p[n] * inv * (double)gamma[n] + bf16_bits_to_double(residual[t * n_out + n]);
            if (proj_out) proj_out[r * n_out + n] = p[n];
        }
        free(x);
        free(p);
    }
    free(wd);
    return bad ? -1 : 0;
}
