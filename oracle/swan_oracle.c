/*
 * swan_oracle.c -- plain, slow, float64 CPU oracle of the SWAN hybrid-cache
 * decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * HIP library; each side is written from the pages on its own.
 *
 * Sources (the pages a reader of this file has):
 *   [SWAN]  "SWAN: Sparse Winnowed Attention for Reduced Inference Memory via
 *           Decompression-Free KV-Cache Compression" (arXiv 2511.18936).
 *   [PAGE3] "Reuse, Evict, or Limit Earlier Context" (int8ai LLM foundations).
 *
 * Arithmetic is IEEE double throughout.  The only places a value is rounded
 * to binary16 are where the method stores it in the cache: the rotated key and
 * the value when they enter the dense buffer ([SWAN] hybrid-cache paragraphs;
 * values are stored as float16 per its memory-savings paragraphs).  Stored values are kept as doubles that are
 * exactly representable in binary16, so widening them back is exact.  With
 * 8-bit sparse values (memory-savings paragraphs) the values a pruned row keeps are rounded
 * once more, to E4M3, when they enter the sparse cache.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - RoPE pairs coordinate i with i + d/2 ("rotate half"), angle pos*theta_i,
 *     theta_i = base^(-2i/d), positions 0-based.  The pages only name RoPE.
 *   - Step order: project, append the new token to the dense buffer, evict the
 *     oldest buffered token (prune it into the sparse cache), then attend over
 *     the sparse cache plus the whole buffer, new token included.
 *   - Magnitude top-k uses the total order (|x| descending, index ascending);
 *     kept entries are written with ascending indices.
 *   - Softmax scale is 1/sqrt(d_h) with the full head dimension.
 *   - R = 0 (no dense buffer): the new token is pruned straight into the
 *     sparse cache before attention.
 *
 * Parity pins (tests, not this file): binary16 rounding against numpy; RoPE
 * against closed forms; projection + sparse decode with k = d_h, R = 0 and no
 * rounding against textbook attention after un-rotation (Lemmas 1 and 2);
 * sparse k = d_h against dense; densified brute force on tiny inputs; top-k
 * against a brute-force sort; the ring slot trace of [PAGE3] section 3.2.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* binary16 storage rounding                                                */
/* ------------------------------------------------------------------------ */

/* Round a double to the nearest binary16 value, ties to even (IEEE 754
 * roundTiesToEven), returned as a double.  binary16 has 10 fraction bits,
 * normal exponents -14..15 and subnormal spacing 2^-24; magnitudes that round
 * past the largest finite value 65504 become infinity.  Used where the
 * memory-savings paragraphs of [SWAN] store values as float16. */
double so_round_f16(double x)
{
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    double ax = fabs(x);
    int e;
    frexp(ax, &e);            /* ax = m * 2^e with m in [0.5, 1) */
    int ex = e - 1;           /* floor(log2(ax)) */
    if (ex < -14)
        ex = -14;             /* subnormal range: fixed spacing 2^-24 */
    double ulp = ldexp(1.0, ex - 10);
    double r = nearbyint(ax / ulp) * ulp; /* exact scaling; default mode is ties-to-even */
    if (r >= 65536.0)
        r = INFINITY;
    return copysign(r, x);
}

/* Elementwise so_round_f16 over an array (y may alias x). */
void so_round_f16_array(long n, const double *x, double *y)
{
    for (long i = 0; i < n; ++i)
        y[i] = so_round_f16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* 8-bit float sparse values ([SWAN] memory-savings paragraphs: the values */
/* kept in a
/* sparse vector may be stored as 8-bit floats, 2k + 2 bytes a vector)    */
/* ------------------------------------------------------------------------ */

/* Round a double to the nearest E4M3 value, ties to even.  The pages name
 * no 8-bit format and no scale; the reading here is the OCP E4M3 encoding
 * (4 exponent bits with bias 7, 3 fraction bits, normal exponents -6..8,
 * subnormal spacing 2^-9, largest finite value 448, no infinities) applied
 * with no scale, saturating: magnitudes that round past 448 become 448.
 * NaN stays NaN. */
double so_round_e4m3(double x)
{
    if (isnan(x) || x == 0.0)
        return x;
    if (isinf(x))
        return copysign(448.0, x);
    double ax = fabs(x);
    int e;
    frexp(ax, &e);            /* ax = m * 2^e with m in [0.5, 1) */
    int ex = e - 1;           /* floor(log2(ax)) */
    if (ex < -6)
        ex = -6;              /* subnormal range: fixed spacing 2^-9 */
    double ulp = ldexp(1.0, ex - 3);
    double r = nearbyint(ax / ulp) * ulp;
    if (r > 448.0)
        r = 448.0;
    return copysign(r, x);
}

void so_round_e4m3_array(long n, const double *x, double *y)
{
    for (long i = 0; i < n; ++i)
        y[i] = so_round_e4m3(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Runtime projection: q -> RoPE(q) -> RoPE(q) P_QK                        */
/* ([SWAN] projection-absorption paragraphs)                                */
/* ------------------------------------------------------------------------ */

/* Rotary position embedding (Su et al., as cited in the [SWAN] projection-absorption paragraphs):
 * each pair (x_i, x_{i+d/2}) is rotated by the angle pos * base^(-2i/d). */
void so_rope(int d, const double *x, double pos, double base, double *y)
{
    int half = d / 2;
    for (int i = 0; i < half; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)d);
        double a = pos * theta;
        double c = cos(a), s = sin(a);
        y[i] = x[i] * c - x[i + half] * s;
        y[i + half] = x[i + half] * c + x[i] * s;
    }
}

/* Row-vector product y = x P with P stored row-major [d][d] (P[c][j]). */
void so_rowvec_mat(int d, const double *x, const double *P, double *y)
{
    for (int j = 0; j < d; ++j) {
        double s = 0.0;
        for (int c = 0; c < d; ++c)
            s += x[c] * P[(size_t)c * d + j];
        y[j] = s;
    }
}

/* x_hat = RoPE(x, pos) P  ([SWAN] projection-absorption paragraphs: the projection follows RoPE). */
void so_project(int d, const double *x, double pos, double base, const double *P, double *y)
{
    double tmp[512];
    so_rope(d, x, pos, base, tmp);
    so_rowvec_mat(d, tmp, P, y);
}

/* ------------------------------------------------------------------------ */
/* Magnitude top-k pruning  ([SWAN] pruning paragraph)                      */
/* ------------------------------------------------------------------------ */

typedef struct { double mag; int idx; } so_key;

/* total order: larger |x| first; equal |x| -> lower index first */
static int so_key_cmp(const void *a, const void *b)
{
    const so_key *u = (const so_key *)a, *v = (const so_key *)b;
    if (u->mag > v->mag) return -1;
    if (u->mag < v->mag) return 1;
    return (u->idx > v->idx) - (u->idx < v->idx);
}

/* Keep the k coordinates of x with the largest absolute value (ties to the
 * lower index) and write them as (index, value) pairs in ascending index
 * order.  Values are copied unchanged. */
void so_prune(int d, int k, const double *x, uint8_t *idx, double *val)
{
    so_key keys[512];
    unsigned char keep[512];
    for (int c = 0; c < d; ++c) {
        keys[c].mag = fabs(x[c]);
        keys[c].idx = c;
        keep[c] = 0;
    }
    qsort(keys, (size_t)d, sizeof(so_key), so_key_cmp);
    for (int r = 0; r < k; ++r)
        keep[keys[r].idx] = 1;
    int w = 0;
    for (int c = 0; c < d; ++c)
        if (keep[c]) {
            idx[w] = (uint8_t)c;
            val[w] = x[c];
            ++w;
        }
}

/* ------------------------------------------------------------------------ */
/* Hybrid attention of one (sequence, kv-head) unit                          */
/* ([SWAN] hybrid-cache paragraphs and Appendix A.2 steps 2-4; the decode  */
/* formula of its background on autoregressive generation)                  */
/* ------------------------------------------------------------------------ */

/* For each of the g query heads sharing this kv-head:
 *   score of sparse token t = (sum_i q[kidx_t,i] * kval_t,i) / sqrt(d)
 *   score of dense token t  = (q . kd_t) / sqrt(d)
 *   a = softmax over all n + nd scores together
 *   out = sum_t a_t v_t, sparse v_t scattered to its stored indices.
 * Sparse key rows hold exactly k entries each (row t at t*k), value rows kv
 * entries (row t at t*kv; kv = k unless keys and values keep different
 * counts, the key/value ablation of [SWAN] Appendix A.5, Table 2).  scratch
 * must hold n + nd doubles.  out is in the rotated value basis. */
void so_attend(int d, int g, const double *qhat,
               long n, int k, const uint8_t *kidx, const double *kval,
               int kv, const uint8_t *vidx, const double *vval,
               long nd, const double *kd, const double *vd,
               double *out, double *scratch)
{
    double scale = 1.0 / sqrt((double)d);
    long L = n + nd;
    for (int h = 0; h < g; ++h) {
        const double *q = qhat + (size_t)h * d;
        double *o = out + (size_t)h * d;
        double m = -INFINITY;
        for (long t = 0; t < n; ++t) {
            double s = 0.0;
            for (int i = 0; i < k; ++i)
                s += q[kidx[(size_t)t * k + i]] * kval[(size_t)t * k + i];
            scratch[t] = s * scale;
        }
        for (long t = 0; t < nd; ++t) {
            double s = 0.0;
            for (int c = 0; c < d; ++c)
                s += q[c] * kd[(size_t)t * d + c];
            scratch[n + t] = s * scale;
        }
        for (long t = 0; t < L; ++t)
            if (scratch[t] > m) m = scratch[t];
        double sum = 0.0;
        for (long t = 0; t < L; ++t) {
            scratch[t] = exp(scratch[t] - m);
            sum += scratch[t];
        }
        for (int c = 0; c < d; ++c)
            o[c] = 0.0;
        for (long t = 0; t < n; ++t) {
            double a = scratch[t] / sum;
            for (int i = 0; i < kv; ++i)
                o[vidx[(size_t)t * kv + i]] += a * vval[(size_t)t * kv + i];
        }
        for (long t = 0; t < nd; ++t) {
            double a = scratch[n + t] / sum;
            for (int c = 0; c < d; ++c)
                o[c] += a * vd[(size_t)t * d + c];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Batched state operations.  Logical layout, all row-major:                 */
/*   kidx, kval  uint8, double [B][H][ncap][k]   key rows, row t = token t  */
/*   vidx, vval  uint8, double [B][H][ncap][kv]  value rows (kv = k unless    */
/*               keys and values keep different counts)                      */
/*   ringk,ringv double [B][H][R][d]        dense buffer, slot = pos mod R   */
/* ([PAGE3] section 3.2: circular buffer, slot = t mod W)                    */
/* ------------------------------------------------------------------------ */

static size_t unit_off(int b, int h, int H, size_t per) { return ((size_t)b * H + h) * per; }

/* Move one token's stored (rounded) key/value into the cache at position
 * pos, evicting and pruning the token that leaves the buffer ([SWAN]
 * hybrid-cache paragraphs: the oldest buffered vectors are evicted, pruned
 * and appended to the sparse cache). */
/* Prune x into a sparse row and store its kept values in the sparse value
 * format: binary16 as they are (vfmt 0) or rounded to E4M3 (vfmt 1). */
static void so_prune_store(int d, int k, int vfmt, const double *x, uint8_t *idx, double *val)
{
    so_prune(d, k, x, idx, val);
    if (vfmt == 1)
        for (int i = 0; i < k; ++i)
            val[i] = so_round_e4m3(val[i]);
}

static void so_append_unit(int d, int R, int k, int kv, long ncap, long pos,
                           const double *khat, const double *vhat,
                           uint8_t *kidx, double *kval, uint8_t *vidx, double *vval,
                           double *ringk, double *ringv, int vfmt, int *err)
{
    if (pos < 0) return; /* inactive sequence (a library convention, not the pages'): nothing appended */
    if (R == 0) {
        if (pos >= ncap) { *err = 1; return; }
        so_prune_store(d, k, vfmt, khat, kidx + (size_t)pos * k, kval + (size_t)pos * k);
        so_prune_store(d, kv, vfmt, vhat, vidx + (size_t)pos * kv, vval + (size_t)pos * kv);
        return;
    }
    long slot = pos % R;
    if (pos >= R) {
        long row = pos - R;  /* the evicted token's position = its sparse row */
        if (row >= ncap) { *err = 1; return; }
        so_prune_store(d, k, vfmt, ringk + (size_t)slot * d, kidx + (size_t)row * k, kval + (size_t)row * k);
        so_prune_store(d, kv, vfmt, ringv + (size_t)slot * d, vidx + (size_t)row * kv, vval + (size_t)row * kv);
    }
    memcpy(ringk + (size_t)slot * d, khat, sizeof(double) * d);
    memcpy(ringv + (size_t)slot * d, vhat, sizeof(double) * d);
}

/* Build the hybrid cache of every unit from a prefilled history of T[b]
 * tokens at positions 0..T[b]-1: raw keys Kraw [B][H][Tmax][d] get RoPE at
 * their own position and P_QK, keys and values are rounded to binary16, and
 * the tokens are appended in order.  Returns nonzero if a sequence needs
 * more than ncap sparse rows. */
int so_prefill(int B, int H, int d, int R, int k, int kv, long ncap, long Tmax, const long *T,
               const double *Kraw, const double *Vraw, const double *P, double base,
               uint8_t *kidx, double *kval, uint8_t *vidx, double *vval,
               double *ringk, double *ringv, int nthreads, int vfmt)
{
    int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nthreads) reduction(| : err)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            double kh[512], vh[512];
            const double *Ph = P + (size_t)h * d * d;
            for (long t = 0; t < T[b]; ++t) {
                const double *kr = Kraw + unit_off(b, h, H, (size_t)Tmax * d) + (size_t)t * d;
                const double *vr = Vraw + unit_off(b, h, H, (size_t)Tmax * d) + (size_t)t * d;
                so_project(d, kr, (double)t, base, Ph, kh);
                for (int c = 0; c < d; ++c) {
                    kh[c] = so_round_f16(kh[c]);
                    vh[c] = so_round_f16(vr[c]);
                }
                so_append_unit(d, R, k, kv, ncap, t, kh, vh,
                               kidx + unit_off(b, h, H, (size_t)ncap * k), kval + unit_off(b, h, H, (size_t)ncap * k),
                               vidx + unit_off(b, h, H, (size_t)ncap * kv), vval + unit_off(b, h, H, (size_t)ncap * kv),
                               ringk + unit_off(b, h, H, (size_t)R * d), ringv + unit_off(b, h, H, (size_t)R * d),
                               vfmt, &err);
            }
        }
    return err;
}

/* Projection only: qhat [B][N][d] and khat [B][H][d] in double, unrounded. */
void so_project_batch(int B, int N, int H, int d, const double *q, const double *kraw,
                      const long *pos, const double *P, double base, double *qhat, double *khat)
{
    int g = N / H;
    for (int b = 0; b < B; ++b) {
        for (int j = 0; j < N; ++j)
            so_project(d, q + ((size_t)b * N + j) * d, (double)pos[b], base,
                       P + (size_t)(j / g) * d * d, qhat + ((size_t)b * N + j) * d);
        for (int h = 0; h < H; ++h)
            so_project(d, kraw + ((size_t)b * H + h) * d, (double)pos[b], base,
                       P + (size_t)h * d * d, khat + ((size_t)b * H + h) * d);
    }
}

/* Append only: round khat/vhat [B][H][d] to binary16 and append at pos[b]. */
int so_append_batch(int B, int H, int d, int R, int k, int kv, long ncap, const long *pos,
                    const double *khat, const double *vhat,
                    uint8_t *kidx, double *kval, uint8_t *vidx, double *vval,
                    double *ringk, double *ringv, int vfmt)
{
    int err = 0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            double kh[512], vh[512];
            for (int c = 0; c < d; ++c) {
                kh[c] = so_round_f16(khat[((size_t)b * H + h) * d + c]);
                vh[c] = so_round_f16(vhat[((size_t)b * H + h) * d + c]);
            }
            so_append_unit(d, R, k, kv, ncap, pos[b], kh, vh,
                           kidx + unit_off(b, h, H, (size_t)ncap * k), kval + unit_off(b, h, H, (size_t)ncap * k),
                           vidx + unit_off(b, h, H, (size_t)ncap * kv), vval + unit_off(b, h, H, (size_t)ncap * kv),
                           ringk + unit_off(b, h, H, (size_t)R * d), ringv + unit_off(b, h, H, (size_t)R * d), vfmt,
                           &err);
        }
    return err;
}

/* Attention only, for every unit, with the cache state as it stands after
 * the token at pos[b] was appended: n = max(0, pos+1-R) sparse rows and
 * min(pos+1, R) buffered tokens.  qhat [B][N][d] -> out [B][N][d]. */
void so_decode_batch(int B, int N, int H, int d, int R, int k, int kv, long ncap, const long *pos,
                     const double *qhat,
                     const uint8_t *kidx, const double *kval, const uint8_t *vidx, const double *vval,
                     const double *ringk, const double *ringv, double *out, int nthreads)
{
    int g = N / H;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nthreads)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            long ctx = pos[b] + 1; /* <= 0: inactive sequence, nothing attended, output zero */
            long n = ctx > R ? ctx - R : 0;
            long nd = ctx <= 0 ? 0 : (ctx < R ? ctx : R);
            if (n > ncap) n = ncap;
            double *scratch = (double *)malloc(sizeof(double) * (size_t)(n + nd + 1));
            so_attend(d, g, qhat + ((size_t)b * N + (size_t)h * g) * d,
                      n, k,
                      kidx + unit_off(b, h, H, (size_t)ncap * k), kval + unit_off(b, h, H, (size_t)ncap * k),
                      kv,
                      vidx + unit_off(b, h, H, (size_t)ncap * kv), vval + unit_off(b, h, H, (size_t)ncap * kv),
                      nd, ringk + unit_off(b, h, H, (size_t)R * d), ringv + unit_off(b, h, H, (size_t)R * d),
                      out + ((size_t)b * N + (size_t)h * g) * d, scratch);
            free(scratch);
        }
}

/* One whole decode step ([SWAN] hybrid-cache paragraphs, in their order): project the new
 * query and key, append the rounded key and value (evicting and pruning the
 * oldest buffered token), then attend.  Outputs qhat (double, unrounded),
 * khat (binary16-rounded) and out.  Returns nonzero on sparse overflow. */
int so_step(int B, int N, int H, int d, int R, int k, int kv, long ncap, const long *pos,
            const double *q, const double *kraw, const double *vnew, const double *P, double base,
            uint8_t *kidx, double *kval, uint8_t *vidx, double *vval, double *ringk, double *ringv,
            double *qhat, double *khat, double *out, int nthreads, int vfmt)
{
    so_project_batch(B, N, H, d, q, kraw, pos, P, base, qhat, khat);
    int err = so_append_batch(B, H, d, R, k, kv, ncap, pos, khat, vnew, kidx, kval, vidx, vval, ringk, ringv, vfmt);
    for (size_t i = 0; i < (size_t)B * H * d; ++i)
        khat[i] = so_round_f16(khat[i]);
    so_decode_batch(B, N, H, d, R, k, kv, ncap, pos, qhat, kidx, kval, vidx, vval, ringk, ringv, out, nthreads);
    return err;
}
