/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the
 * batch-invariant linear layer and the batch-invariant MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source, header, table or helper with
 * the HIP library.
 *
 * Arithmetic: every product and sum is carried in IEEE binary64 and each
 * storage point is rounded exactly once, round-to-nearest-even.  Inputs of
 * type fp32 or bf16 convert to binary64 exactly, and a product of two such
 * values is exact in binary64 (at most 24+24 significant bits).  Sums run in
 * ascending index order.  Built with -ffp-contract=off so no multiply-add is
 * fused behind the reader's back.
 *
 * Sources (the three pages on batch-invariant inference):
 *  - "[BI][DSv4] Batch-invariant GateLinear router with fp32 persistent
 *    matmul", section "What": the router computes Y = X W^T + b in fp32 and
 *    must never round through bf16; section "Tests": correctness against an
 *    fp32 linear at atol 2e-3 / rtol 1e-4.
 *  - "Batch-invariance generation with vLLM fused-MoE backend", section
 *    "What's included": gated SwiGLU with routing probabilities applied at
 *    the activation (fp32 math, one final bf16 rounding), fp32-accumulate
 *    expert GEMMs, and a top-k reduction with unit weights summed in fp64;
 *    review summary: gate|up half-split and a fixed slot-order reduction.
 *  - "[BI][DSv4] Pin sparse-MLA decode and prefill scheduling", commit notes
 *    of the deterministic per-row top-k: the larger score comes first, equal
 *    scores are taken in column order, and a negative zero counts as a
 *    positive one; for the indexer's top-k every fp32 bit pattern gets a
 *    monotone int32 rank, a lane outside the row's window never outranks one
 *    inside it, and the chosen columns are returned sorted, counted from the
 *    window start, with -1 filling the unused slots.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- rounding */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a binary64 value to bf16 (8 significant bits, exponent range of
 * binary32) with round-to-nearest, ties-to-even, in ONE step -- no detour
 * through binary32, which would round twice.  The value is scaled by a power
 * of two so that one bf16 ulp becomes 1.0, rounded to an integer with rint()
 * (ties-to-even in the default rounding mode), and scaled back. */
static uint16_t f64_to_bf16(double v)
{
    if (isnan(v))
        return 0x7fc0;
    if (v == 0.0 || isinf(v)) {
        float f = (float)v;
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        return (uint16_t)(u >> 16);
    }
    int e;
    frexp(fabs(v), &e);               /* |v| = m * 2^e, m in [0.5, 1) */
    int ulp_exp = e - 8;              /* 8 significant bits */
    if (ulp_exp < -133)               /* bf16 subnormal spacing is 2^-133 */
        ulp_exp = -133;
    double q = rint(ldexp(fabs(v), -ulp_exp));
    double r = ldexp(q, ulp_exp);     /* exact, or 2^128 on overflow */
    float f = (r >= 0x1p128) ? INFINITY : (float)r;
    if (v < 0)
        f = -f;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* binary64 -> binary32 is a C conversion: IEEE round-to-nearest-even. */
static float f64_to_f32(double v) { return (float)v; }

int oracle_f64_to_bf16(const double* in, uint16_t* out, long n)
{
    if (n < 0 || (n > 0 && (!in || !out)))
        return -1;
    for (long i = 0; i < n; ++i)
        out[i] = f64_to_bf16(in[i]);
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ linear */

/* Y[m,n] = RN_f32( sum_{k ascending} x[m,k] * w[n,k]  +  b[n] ).
 *
 * GateLinear page, section "What": the router is a plain linear layer,
 * Y = X W^T + b, computed in fp32.  w is the nn.Linear weight, [N,K]
 * row-major, which is the memory behind the weight.t() [K,N] view the
 * matmul receives.  b may be NULL (no bias term at all).  If y64 is not
 * NULL it receives the binary64 value before the final rounding. */
int oracle_linear_f32(const float* x, const float* w, const float* b,
                      float* y, double* y64, long M, long N, long K)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (M == 0 || N == 0)
        return 0;
    if (!x || !w || !y)
        return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (long m = 0; m < M; ++m) {
        for (long n = 0; n < N; ++n) {
            double s = 0.0;
            for (long k = 0; k < K; ++k)
                s += (double)x[m * K + k] * (double)w[n * K + k];
            if (b)
                s += (double)b[n];
            y[m * N + n] = f64_to_f32(s);
            if (y64)
                y64[m * N + n] = s;
        }
    }
    return 0;
}

/* Same definition with bf16 operands: bf16 x bf16 products are exact in
 * binary64.  The single storage rounding goes to bf16 (y_bf16) and/or to
 * fp32 (y_f32); either pointer may be NULL but not both. */
int oracle_linear_bf16(const uint16_t* x, const uint16_t* w, const float* b,
                       uint16_t* y_bf16, float* y_f32, double* y64,
                       long M, long N, long K)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (M == 0 || N == 0)
        return 0;
    if (!x || !w || (!y_bf16 && !y_f32))
        return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (long m = 0; m < M; ++m) {
        for (long n = 0; n < N; ++n) {
            double s = 0.0;
            for (long k = 0; k < K; ++k)
                s += bf16_to_f64(x[m * K + k]) * bf16_to_f64(w[n * K + k]);
            if (b)
                s += (double)b[n];
            if (y_bf16)
                y_bf16[m * N + n] = f64_to_bf16(s);
            if (y_f32)
                y_f32[m * N + n] = f64_to_f32(s);
            if (y64)
                y64[m * N + n] = s;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------- top-k */

/* Top-k of one row of fp32 scores: slot j holds the j-th largest value;
 * equal values are taken in ascending index order; -0.0 and +0.0 compare
 * equal (C's == already does).  Selection by repeated maximum: obviously
 * correct, O(k*E).  NaN is outside the definition and is rejected. */
static int topk_row(const float* v, long E, long k, int32_t* ids)
{
    for (long e = 0; e < E; ++e)
        if (isnan(v[e]))
            return -1;
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    if (!taken)
        return -1;
    for (long j = 0; j < k; ++j) {
        long best = -1;
        for (long e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || v[e] > v[best])   /* strict: earlier index wins ties */
                best = e;
        }
        taken[best] = 1;
        ids[j] = (int32_t)best;
    }
    free(taken);
    return 0;
}

int oracle_topk(const float* scores, int32_t* ids, long M, long E, long k)
{
    if (M < 0 || E <= 0 || k <= 0 || k > E)
        return -1;
    if (M == 0)
        return 0;
    if (!scores || !ids)
        return -1;
    int bad = 0;
    for (long m = 0; m < M; ++m)
        if (topk_row(scores + m * E, E, k, ids + m * k))
            bad = 1;
    return bad ? -1 : 0;
}

/* ------------------------------------------------------- indexer top-k rows */

/* The ranking key of an fp32 score (Sparse-MLA page, deterministic top-k
 * commit notes): -0.0 is first replaced by +0.0, then the bit pattern b is
 * read as a signed 32-bit integer and, when the sign bit is set, its 31 low
 * bits are inverted.  Larger key = larger score for every non-NaN value; the
 * key also orders every NaN pattern (positive NaNs above +inf, negative NaNs
 * below -inf, 0xffffffff lowest at INT32_MIN). */
static int32_t topk_key(float v)
{
    uint32_t b;
    memcpy(&b, &v, 4);
    if (b == 0x80000000u)
        b = 0;
    int32_t k;
    memcpy(&k, &b, 4);
    if (k < 0)
        k = (int32_t)(b ^ 0x7fffffffu);
    return k;
}

typedef struct {
    int valid;
    int32_t key;
    long col;
} topk_lane;

/* Rank order: in-window lanes first, then larger key, then lower column. */
static int topk_lane_cmp(const void* pa, const void* pb)
{
    const topk_lane* a = (const topk_lane*)pa;
    const topk_lane* b = (const topk_lane*)pb;
    if (a->valid != b->valid)
        return a->valid ? -1 : 1;
    if (a->key != b->key)
        return a->key > b->key ? -1 : 1;
    return a->col < b->col ? -1 : (a->col > b->col ? 1 : 0);
}

static long clamp_long(long v, long lo, long hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* Per-row top-k of an indexer score matrix.  Row r considers columns
 * [0, cols); its window is [rs, re) with rs = clamp(row_start[r], 0, cols)
 * and re = clamp(row_end[r], 0, cols) (0 and cols when the arrays are NULL).
 * The first min(topk, re - rs) lanes of the rank order are selected and
 * written to out[r, 0..] in ascending column order as row-local indices
 * (column - rs); the remaining slots of the row hold -1. */
int oracle_topk_rows(const float* scores, long ld, long rows, long cols,
                     const int64_t* row_start, const int64_t* row_end, long topk,
                     int32_t* out, long ld_out)
{
    if (rows < 0 || cols < 0 || topk <= 0 || ld < cols || ld_out < topk)
        return -1;
    if (rows == 0)
        return 0;
    if (!scores || !out)
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (long r = 0; r < rows; ++r) {
        const long rs = row_start ? clamp_long((long)row_start[r], 0, cols) : 0;
        const long re = row_end ? clamp_long((long)row_end[r], 0, cols) : cols;
        topk_lane* lanes = (topk_lane*)malloc(sizeof(topk_lane) * (size_t)(cols > 0 ? cols : 1));
        unsigned char* sel = (unsigned char*)calloc((size_t)(cols > 0 ? cols : 1), 1);
        if (!lanes || !sel) {
            bad = 1;
            free(lanes);
            free(sel);
            continue;
        }
        for (long c = 0; c < cols; ++c) {
            lanes[c].valid = (c >= rs && c < re);
            lanes[c].key = topk_key(scores[r * ld + c]);
            lanes[c].col = c;
        }
        qsort(lanes, (size_t)cols, sizeof(topk_lane), topk_lane_cmp);
        const long nvalid = re > rs ? re - rs : 0;
        const long take = topk < nvalid ? topk : nvalid;
        for (long j = 0; j < take; ++j)
            sel[lanes[j].col] = 1;
        long o = 0;
        for (long c = 0; c < cols; ++c)
            if (sel[c])
                out[r * ld_out + o++] = (int32_t)(c - rs);
        for (; o < topk; ++o)
            out[r * ld_out + o] = -1;
        free(lanes);
        free(sel);
    }
    return bad ? -1 : 0;
}

/* --------------------------------------------------------------------- MoE */

/* One token through the batch-invariant MoE layer (fused-MoE page):
 *
 *  1. router logits  l[e]  = RN_f32( sum_h x[h] * wr[e,h] + br[e] )
 *     (the fp32 router is the batch-invariant linear above, fed the bf16
 *     activations widened to fp32; its fp32 output is a storage point and
 *     the expert choice is taken on it)
 *  2. ids = top-k of l (descending, ties to the lower expert index), or the
 *     caller's ids_in when given
 *  3. p[j] = exp(l[id_j] - max l) / sum_{e ascending} exp(l[e] - max l),
 *     the full-softmax probability of the chosen expert, not renormalised
 *  4. per slot j (expert e = ids[j]):  h[c] = RN_bf16( sum_h x[h]*w1[e,c,h] )
 *     gated (SwiGLU): c in [0, 2I), the first I rows of w1[e] are the gate,
 *     the next I the up projection (gate|up half-split);
 *     squared-ReLU: c in [0, I)
 *  5. a[i] = RN_bf16( act_i * q ), q = p[j] when the probability is applied
 *     at the activation, else 1, computed in binary64 with one rounding:
 *     SwiGLU act_i = (g*s) * u, g = h[i], u = h[I+i], s = 1 / (1 + exp(-g));
 *     squared-ReLU act_i = max(h[i], 0)^2
 *  6. y_j[c] = sum_{i ascending} a[i] * w2[e,c,i]
 *  7. combine in slot order j = 0..topk-1, with w_j = p[j] when the weights
 *     are applied here, else 1:
 *     acc_fp64:  out[c] = RN_f32( sum_j w_j * y_j[c] ) in binary64
 *     fp32:      the slot partials are fp32 storage points and the sum is
 *                fp32: acc = +0; acc = RN_f32(acc + t_j) with
 *                t_j = RN_f32(RN_f32(p[j]) * RN_f32(y_j[c])) when weighted,
 *                t_j = RN_f32(y_j[c]) otherwise
 * The options (fused-MoE page: the gated activation with the probability at
 * the activation and an unweighted fp64 combine; the squared-ReLU activation
 * and the (apply_weights, acc_fp64) matrix of the top-k sum, whose (false,
 * false) point must apply no weights) are independent switches here.
 */
/* Step 5 for one (token, slot) pair: a[i] = RN_bf16(act_i(h) * q) in
 * binary64, q = p when the probability is applied at the activation, else 1.
 * h holds the bf16 storage point of step 4 widened to binary64; act 1 is
 * SwiGLU on the gate|up halves, act 2 squared-ReLU. */
static void moe_activation_row(const double* h, long I, int act, double q, uint16_t* a)
{
    for (long i = 0; i < I; ++i) {
        double v;
        if (act == 1) {
            double g = h[i], u = h[I + i];
            double sg = 1.0 / (1.0 + exp(-g));
            v = (g * sg) * u;
        } else {
            double r = h[i] > 0.0 ? h[i] : 0.0;
            v = r * r;
        }
        a[i] = f64_to_bf16(v * q);
    }
}

/* Step 7 for one output element of one token: the slot-order sum of the
 * slot values s[j] (binary64 y_j), weighted by p[j] when apply_weights. */
static float moe_combine_elem(const double* s, const double* p, long topk, long stride, int apply_weights,
                              int acc_fp64)
{
    double acc = 0.0;
    float acc32 = 0.0f;
    for (long j = 0; j < topk; ++j) {
        const double v = s[j * stride];
        if (acc_fp64) {
            acc += apply_weights ? p[j] * v : v;
        } else {
            const double part = (double)f64_to_f32(v);
            const double t = apply_weights ? (double)f64_to_f32((double)f64_to_f32(p[j]) * part) : part;
            acc32 = f64_to_f32((double)acc32 + t);
        }
    }
    return acc_fp64 ? f64_to_f32(acc) : acc32;
}

/* Step 5 alone, for P pairs: h [P, rows1] bf16 (rows1 = 2I for SwiGLU, I for
 * squared-ReLU), p [P] binary64, a [P, I] bf16 out. */
int oracle_moe_activation(const uint16_t* h, const double* p, long P, long I, int act, int probs_at_act,
                          uint16_t* a)
{
    if (P < 0 || I <= 0 || (act != 1 && act != 2) || (P > 0 && (!h || !p || !a)))
        return -1;
    const long rows1 = act == 1 ? 2 * I : I;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (long r = 0; r < P; ++r) {
        double* hv = (double*)malloc(sizeof(double) * (size_t)rows1);
        if (!hv) {
            bad = 1;
            continue;
        }
        for (long c = 0; c < rows1; ++c)
            hv[c] = bf16_to_f64(h[r * rows1 + c]);
        moe_activation_row(hv, I, act, probs_at_act ? p[r] : 1.0, a + r * I);
        free(hv);
    }
    return bad ? -1 : 0;
}

/* Step 7 alone: part [M, topk, H] binary64 slot values, p [M, topk]
 * binary64, y [M, H] fp32 out. */
int oracle_moe_combine(const double* part, const double* p, long M, long topk, long H, int apply_weights,
                       int acc_fp64, float* y)
{
    if (M < 0 || topk <= 0 || H <= 0 || (M > 0 && (!part || !p || !y)))
        return -1;
#pragma omp parallel for schedule(static)
    for (long m = 0; m < M; ++m)
        for (long c = 0; c < H; ++c)
            y[m * H + c] = moe_combine_elem(part + m * topk * H + c, p + m * topk, topk, H, apply_weights,
                                            acc_fp64);
    return 0;
}

/* The same layer, also returning its storage points per (token, slot) pair
 * m * topk + j (each output may be NULL):
 *   h_out     [M, topk, rows1] bf16 bit patterns of step 4
 *   a_out     [M, topk, I]     bf16 bit patterns of step 5
 *   part_out  [M, topk, H]     binary64 y_j of step 6 (before any weight)   */
int oracle_moe_stages(const uint16_t* x, const float* wr, const float* br,
                      const uint16_t* w1, const uint16_t* w2,
                      long M, long H, long E, long I, long topk,
                      int act, int probs_at_act, int apply_weights, int acc_fp64,
                      const int32_t* ids_in, float* logits_out, int32_t* ids_out,
                      double* probs_out, float* y,
                      uint16_t* h_out, uint16_t* a_out, double* part_out)
{
    if (M < 0 || H <= 0 || E <= 0 || I <= 0 || topk <= 0 || topk > E)
        return -1;
    if (act != 1 && act != 2)
        return -1;
    if (M == 0)
        return 0;
    if (!x || !wr || !w1 || !w2 || !ids_out || !probs_out || !y)
        return -1;
    const long rows1 = act == 1 ? 2 * I : I;     /* rows of one expert's first weight */
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long m = 0; m < M; ++m) {
        const uint16_t* xm = x + m * H;
        float* l = (float*)malloc(sizeof(float) * (size_t)E);
        double* h = (double*)malloc(sizeof(double) * (size_t)rows1);
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
        uint16_t* ab = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
        double* ys = (double*)malloc(sizeof(double) * (size_t)(topk * H));
        int32_t* ids = ids_out + m * topk;
        if (!l || !h || !a || !ab || !ys) {
            bad = 1;
            goto done;
        }
        /* 1. router logits, stored as fp32 */
        for (long e = 0; e < E; ++e) {
            double s = 0.0;
            for (long k = 0; k < H; ++k)
                s += bf16_to_f64(xm[k]) * (double)wr[e * H + k];
            if (br)
                s += (double)br[e];
            l[e] = f64_to_f32(s);
        }
        if (logits_out)
            memcpy(logits_out + m * E, l, sizeof(float) * (size_t)E);
        /* 2. expert choice */
        if (ids_in) {
            for (long j = 0; j < topk; ++j) {
                if (ids_in[m * topk + j] < 0 || ids_in[m * topk + j] >= E)
                    bad = 1;
                ids[j] = ids_in[m * topk + j];
            }
            if (bad)
                goto done;
        } else if (topk_row(l, E, topk, ids)) {
            bad = 1;
            goto done;
        }
        /* 3. softmax probabilities of the chosen experts */
        double mx = l[0];
        for (long e = 1; e < E; ++e)
            if (l[e] > mx)
                mx = l[e];
        double den = 0.0;
        for (long e = 0; e < E; ++e)
            den += exp((double)l[e] - mx);
        for (long j = 0; j < topk; ++j) {
            double p = exp((double)l[ids[j]] - mx) / den;
            probs_out[m * topk + j] = p;
            long e = ids[j];
            /* 4. first projection, bf16 storage point */
            const uint16_t* w1e = w1 + e * rows1 * H;
            for (long c = 0; c < rows1; ++c) {
                double s = 0.0;
                for (long k = 0; k < H; ++k)
                    s += bf16_to_f64(xm[k]) * bf16_to_f64(w1e[c * H + k]);
                const uint16_t hb = f64_to_bf16(s);
                h[c] = bf16_to_f64(hb);
                if (h_out)
                    h_out[(m * topk + j) * rows1 + c] = hb;
            }
            /* 5. activation (probability applied here or not), bf16 storage point */
            moe_activation_row(h, I, act, probs_at_act ? p : 1.0, ab);
            for (long i = 0; i < I; ++i)
                a[i] = bf16_to_f64(ab[i]);
            if (a_out)
                memcpy(a_out + (m * topk + j) * I, ab, sizeof(uint16_t) * (size_t)I);
            /* 6. down projection of the slot */
            const uint16_t* w2e = w2 + e * H * I;
            for (long c = 0; c < H; ++c) {
                double s = 0.0;
                for (long i = 0; i < I; ++i)
                    s += a[i] * bf16_to_f64(w2e[c * I + i]);
                ys[j * H + c] = s;
            }
        }
        if (part_out)
            memcpy(part_out + m * topk * H, ys, sizeof(double) * (size_t)(topk * H));
        /* 7. combine over slots in slot order */
        for (long c = 0; c < H; ++c)
            y[m * H + c] = moe_combine_elem(ys + c, probs_out + m * topk, topk, H, apply_weights, acc_fp64);
    done:
        free(l);
        free(h);
        free(a);
        free(ab);
        free(ys);
    }
    return bad ? -1 : 0;
}

int oracle_moe_ex(const uint16_t* x, const float* wr, const float* br,
                  const uint16_t* w1, const uint16_t* w2,
                  long M, long H, long E, long I, long topk,
                  int act, int probs_at_act, int apply_weights, int acc_fp64,
                  const int32_t* ids_in, float* logits_out, int32_t* ids_out,
                  double* probs_out, float* y)
{
    return oracle_moe_stages(x, wr, br, w1, w2, M, H, E, I, topk, act, probs_at_act, apply_weights, acc_fp64,
                             ids_in, logits_out, ids_out, probs_out, y, NULL, NULL, NULL);
}

/* The gated layer with the probability at the activation and an unweighted
 * binary64 combine (the fused-MoE page's shipped configuration). */
int oracle_moe(const uint16_t* x, const float* wr, const float* br,
               const uint16_t* w13, const uint16_t* w2,
               long M, long H, long E, long I, long topk,
               const int32_t* ids_in, float* logits_out, int32_t* ids_out,
               double* probs_out, float* y)
{
    return oracle_moe_ex(x, wr, br, w13, w2, M, H, E, I, topk, 1, 1, 0, 1, ids_in, logits_out, ids_out,
                         probs_out, y);
}
