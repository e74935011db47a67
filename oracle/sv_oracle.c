/*
 * CPU oracle for the compensated-tree float32 sum and the shifted/centred
 * float32 variance.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the CPU-baseline leg of the benchmark may call it; the product path never
 * does.  It shares no code, header or constant with the HIP library.
 *
 * Sources (cited by page title and section):
 *   [VAR]  S. Pennacchio, "Variance in float32 with a first-element shift, a
 *          local centring and a compensated tree sum" (Oct 2026): §1 (the
 *          naive and the two-term reference formulae), §2 steps 1-4 (the
 *          kernel), §3 (results tables).
 *   [ORD]  "Reduction order and compensation solve related but different
 *          problems": sequential vs pairwise order, the Kahan recurrence.
 *   [KAHAN] "Kahan's Summation Formula" (blog post): the sequential naive and
 *          Kahan loops over 10^6 copies of 0.001f.
 *   TwoSum itself is the published error-free transformation that [VAR] §2
 *   step 3 cites (Ogita-Rump-Oishi 2005 Alg. 3.1, Shewchuk 1997 Thm 7); the
 *   pages name it but do not print it.
 *
 * Arithmetic contract: IEEE binary32, round to nearest even, every operation
 * rounded on its own (no FMA contraction, no reassociation, no flush of
 * subnormals).  Build with -O2 -ffp-contract=off -fno-fast-math on x86-64
 * (SSE scalar float, so no excess precision).
 *
 * Readings of the pages that the pages leave open are marked READING and are
 * listed in the design notes of the repository.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(__FAST_MATH__)
#error "the oracle must not be built with fast-math"
#endif
#if defined(__FLT_EVAL_METHOD__) && __FLT_EVAL_METHOD__ != 0
#error "float expressions must be evaluated in float (FLT_EVAL_METHOD 0)"
#endif

/* ------------------------------------------------------------------ */
/* TwoSum: s = fl(a+b) and the exact rounding error e, s + e == a + b. */
/* ------------------------------------------------------------------ */
static inline float two_sum(float a, float b, float *err) {
    float s = a + b;
    float bv = s - a;          /* the part of s that came from b   */
    float av = s - bv;         /* the part of s that came from a   */
    float ea = a - av;
    float eb = b - bv;
    *err = ea + eb;
    return s;
}

float orc_two_sum(float a, float b, float *err) { return two_sum(a, b, err); }

/* Smallest power of two >= n (n >= 1). */
static int64_t pow2_ceil(int64_t n) {
    int64_t p = 1;
    while (p < n) p <<= 1;
    return p;
}

/*
 * READING (tree topology, [VAR] §2 step 3): the n values are padded with
 * +0 to P = 2^ceil(log2 n) (or to the caller's larger power of two) and each
 * level adds adjacent pairs (2k, 2k+1).  Node k of level l thus covers
 * elements [k*2^l, (k+1)*2^l).
 *
 * Compensated tree: level by level, s'_k = fl(s_2k + s_2k+1) with TwoSum
 * error e_k, and the error array carries c'_k = fl(fl(c_2k + c_2k+1) + e_k).
 * The result is fl(s_0 + c_0).
 * READING (non-finite root): if s_0 is Inf or NaN the result is s_0, so that
 * Inf and NaN inputs give what a plain sum gives.
 *
 * x is read with a stride of `stride` floats.  `pad_to` = 0 means P; a larger
 * power of two pads further (used to check that extra zero padding leaves
 * the bits unchanged).  Returns NaN for an invalid pad_to.
 */
float orc_tree_sum_f32(const float *x, int64_t n, int64_t stride, int64_t pad_to) {
    if (n <= 0) return 0.0f;
    int64_t P = pow2_ceil(n);
    if (pad_to != 0) {
        if (pad_to < P || (pad_to & (pad_to - 1)) != 0) return NAN;
        P = pad_to;
    }
    float *s = (float *)malloc((size_t)P * sizeof(float));
    float *c = (float *)malloc((size_t)P * sizeof(float));
    if (!s || !c) { free(s); free(c); return NAN; }
    for (int64_t i = 0; i < P; ++i) {
        s[i] = (i < n) ? x[i * stride] : 0.0f;
        c[i] = 0.0f;
    }
    for (int64_t len = P; len > 1; len >>= 1) {
        for (int64_t k = 0; k < len / 2; ++k) {
            float e;
            float sk = two_sum(s[2 * k], s[2 * k + 1], &e);
            float ck = (c[2 * k] + c[2 * k + 1]) + e;
            s[k] = sk;
            c[k] = ck;
        }
    }
    float root_s = s[0], root_c = c[0];
    free(s);
    free(c);
    if (!isfinite(root_s)) return root_s;
    return root_s + root_c;
}

/*
 * Double-word carries: the same topology and the same node, followed by a
 * renormalisation of the pair with TwoSum, (s, c) <- TwoSum(s', c') with
 * s' = fl(s_2k + s_2k+1) and c' = fl(fl(c_2k + c_2k+1) + e_k).  The pair
 * then stays a normalised double-word (|c| <= ulp(s)/2), so the carry is
 * rounded relative to ulp(s) at every node instead of growing unchecked.
 * READING ([ORD] points to wider or expansion-based accumulators for
 * stronger guarantees; this is the double-word form of the method's own
 * node): leaves are nodes of two values with zero carries, the result is
 * fl(s_0 + c_0) with the same root guard as the compensated tree, and a
 * node whose sum is Inf or NaN is not renormalised (fl(Inf + NaN) would turn
 * an Inf into NaN), so Inf and NaN behave as in the compensated tree.
 */
float orc_tree_sum_dw_f32(const float *x, int64_t n, int64_t stride, int64_t pad_to) {
    if (n <= 0) return 0.0f;
    int64_t P = pow2_ceil(n);
    if (pad_to != 0) {
        if (pad_to < P || (pad_to & (pad_to - 1)) != 0) return NAN;
        P = pad_to;
    }
    float *s = (float *)malloc((size_t)P * sizeof(float));
    float *c = (float *)malloc((size_t)P * sizeof(float));
    if (!s || !c) { free(s); free(c); return NAN; }
    for (int64_t i = 0; i < P; ++i) {
        s[i] = (i < n) ? x[i * stride] : 0.0f;
        c[i] = 0.0f;
    }
    for (int64_t len = P; len > 1; len >>= 1) {
        for (int64_t k = 0; k < len / 2; ++k) {
            float e, r;
            float sk = two_sum(s[2 * k], s[2 * k + 1], &e);
            float ck = (c[2 * k] + c[2 * k + 1]) + e;
            if (isfinite(sk)) {
                s[k] = two_sum(sk, ck, &r);
                c[k] = r;
            } else {           /* keep Inf (or NaN) in s: the root guard returns it */
                s[k] = sk;
                c[k] = ck;
            }
        }
    }
    float root_s = s[0], root_c = c[0];
    free(s);
    free(c);
    if (!isfinite(root_s)) return root_s;
    return root_s + root_c;
}

/*
 * The root node (s_0, c_0) of the compensated tree over x padded to pad_to
 * (a power of two >= n; n may be 0).  An aligned subtree of a larger tree,
 * so that a sum can be cut into 2^k pieces computed separately and their
 * nodes combined with the same rule: the bits equal the whole tree's.
 * Returns 0, or -1 for a bad pad_to.
 */
int orc_tree_node_f32(const float *x, int64_t n, int64_t pad_to, float *s_out, float *c_out) {
    if (n < 0 || pad_to < 1 || (pad_to & (pad_to - 1)) != 0 || pad_to < n) return -1;
    float *s = (float *)malloc((size_t)pad_to * sizeof(float));
    float *c = (float *)malloc((size_t)pad_to * sizeof(float));
    if (!s || !c) { free(s); free(c); return -1; }
    for (int64_t i = 0; i < pad_to; ++i) {
        s[i] = (i < n) ? x[i] : 0.0f;
        c[i] = 0.0f;
    }
    for (int64_t len = pad_to; len > 1; len >>= 1) {
        for (int64_t k = 0; k < len / 2; ++k) {
            float e;
            float sk = two_sum(s[2 * k], s[2 * k + 1], &e);
            float ck = (c[2 * k] + c[2 * k + 1]) + e;
            s[k] = sk;
            c[k] = ck;
        }
    }
    *s_out = s[0];
    *c_out = c[0];
    free(s);
    free(c);
    return 0;
}

/* Same topology without the error array: the plain pairwise tree.
 * READING (the root of a plain tree, [VAR] §2 step 3: "the result is the
 * final sum plus the final carry"): a plain tree's carry is zero, so its
 * value is fl(s_0 + 0).  That differs from s_0 only when s_0 is -0 (every
 * value -0), and it makes the result independent of how far the values are
 * padded with +0, as for the compensated tree, whose carries are never -0. */
float orc_tree_plain_f32(const float *x, int64_t n, int64_t stride, int64_t pad_to) {
    if (n <= 0) return 0.0f;
    int64_t P = pow2_ceil(n);
    if (pad_to != 0) {
        if (pad_to < P || (pad_to & (pad_to - 1)) != 0) return NAN;
        P = pad_to;
    }
    float *s = (float *)malloc((size_t)P * sizeof(float));
    if (!s) return NAN;
    for (int64_t i = 0; i < P; ++i) s[i] = (i < n) ? x[i * stride] : 0.0f;
    for (int64_t len = P; len > 1; len >>= 1)
        for (int64_t k = 0; k < len / 2; ++k) s[k] = s[2 * k] + s[2 * k + 1];
    float r = s[0] + 0.0f;
    free(s);
    return r;
}

/* ------------------------------------------------------------------ */
/* Sequential sums ([KAHAN], [ORD]): comparators, not on the hot path.  */
/* ------------------------------------------------------------------ */
float orc_seq_naive_f32(const float *x, int64_t n) {
    float sum = 0.0f;
    for (int64_t i = 0; i < n; ++i) sum = sum + x[i];
    return sum;
}

/* Kahan's compensated summation (W. Kahan, "Further remarks on reducing
 * truncation errors", CACM 8(1), 1965; stated as Algorithm 4.2 in Higham,
 * "Accuracy and Stability of Numerical Algorithms", 2nd ed., section 4.3).
 * c holds the low-order part that the last addition to s dropped, with its
 * sign reversed; it is taken off the next term before that term is added.
 * Starting from s = c = 0, the first pass leaves s = x[0] and c = 0.  The
 * [KAHAN] page prints what this recurrence gives on 10^6 copies of 0.001f
 * (1000.00006), which pins it. */
float orc_seq_kahan_f32(const float *x, int64_t n) {
    float s = 0.0f, c = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float y = x[i] - c;        /* the term, corrected by the lost part */
        float t = s + y;           /* the new sum, rounded                 */
        c = (t - s) - y;           /* what the rounding of t dropped       */
        s = t;
    }
    return s;
}

/* Neumaier's variant ([ORD]): the branch on magnitudes picks which operand's
 * low part was lost; the accumulated correction is added at the end. */
float orc_seq_neumaier_f32(const float *x, int64_t n) {
    float sum = 0.0f, corr = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float t = sum + x[i];
        if (fabsf(sum) >= fabsf(x[i]))
            corr = corr + ((sum - t) + x[i]);
        else
            corr = corr + ((x[i] - t) + sum);
        sum = t;
    }
    return sum + corr;
}

/* ------------------------------------------------------------------ */
/* Variance of one slice                                                */
/* ------------------------------------------------------------------ */

/* READING (max(., 0), [VAR] §1 and §2 step 4): NaN propagates (a NaN input
 * to the max returns NaN), any other value <= 0 gives +0. */
static inline float max0_nan(float v) {
    if (v != v) return v;
    return (v > 0.0f) ? v : 0.0f;
}

/* READING (ddof rescale, [VAR] §2 step 4): applied after the max as
 * v * fl(fl(n) / fl(max(n - ddof, 0))); nothing is done when ddof == 0. */
static inline float ddof_scale(float v, int64_t n, int64_t ddof) {
    if (ddof == 0) return v;
    int64_t den = n - ddof;
    if (den < 0) den = 0;
    float f = (float)n / (float)den;
    return v * f;
}

/* Gather one slice (n elements at `stride`) into a contiguous buffer. */
static void gather(const float *x, int64_t n, int64_t stride, float *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = x[i * stride];
}

/*
 * The kernel of [VAR] §2, one slice.
 *   step 1  x0 = x[0]; y_i = fl(x_i - x0)
 *   step 2  m = fl(Sy / fl(n)); d_i = fl(y_i - m)
 *           READING: Sy is the plain pairwise tree of y (comp_sy == 0, the
 *           method): step 2 writes a plain sum(y), and step 3 describes the
 *           compensated tree for the sums of the residuals only.  comp_sy != 0
 *           is the other reading, every sum of the slice on the compensated
 *           tree.
 *   step 3  S1 = Tree(d), S2 = Tree(q) with q_i = fl(d_i * d_i)
 *   step 4  v = max(fl(fl(S2/n) - fl(b*b)), 0) with b = fl(S1/n), then the
 *           ddof rescale; mean = fl(x0 + m).
 * READING (empty slice): n == 0 gives var = mean = NaN.
 */
static void var_kernel_slice(const float *x, int64_t n, int64_t stride, int64_t ddof,
                             int comp_sy, float *buf, float *var, float *mean) {
    if (n <= 0) {
        *var = NAN;
        *mean = NAN;
        return;
    }
    gather(x, n, stride, buf);
    float x0 = buf[0];
    for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] - x0;               /* y */
    float sy = comp_sy ? orc_tree_sum_f32(buf, n, 1, 0) : orc_tree_plain_f32(buf, n, 1, 0);
    float fn = (float)n;
    float m = sy / fn;
    for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] - m;                /* d */
    float s1 = orc_tree_sum_f32(buf, n, 1, 0);
    for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] * buf[i];           /* q */
    float s2 = orc_tree_sum_f32(buf, n, 1, 0);
    float a = s2 / fn;
    float b = s1 / fn;
    float bb = b * b;
    float v = max0_nan(a - bb);
    *var = ddof_scale(v, n, ddof);
    *mean = x0 + m;
}

/*
 * Ablation variants of [VAR] §4, one step of the kernel changed at a time.
 * Flags:
 *   shift    y = x - x0 (else y = x and mean = m)
 *   sum_kind how the sums of the residuals (S1 and S2, the sums that the
 *            kernel takes on the compensated tree) are formed: 0 plain tree,
 *            1 compensated tree, 2 sequential Kahan scan, 3 compensated tree
 *            with double-word carries
 *   twoterm  v = max(S2/n - (S1/n)^2, 0) (else v = max(S2/n, 0))
 * READING: the local mean keeps the kernel's plain tree of y in every row
 * (no row of the table names the centring's sum as the step it changes).
 * READING: "no two-term" is v = max(S2/n, 0); the Kahan-scan row of the
 * table ("shift + centring, Kahan sequential scan") has no two-term step,
 * like the other rows whose label does not add one.
 */
static float slice_sum(const float *v, int64_t n, int sum_kind) {
    if (sum_kind == 0) return orc_tree_plain_f32(v, n, 1, 0);
    if (sum_kind == 1) return orc_tree_sum_f32(v, n, 1, 0);
    if (sum_kind == 3) return orc_tree_sum_dw_f32(v, n, 1, 0);
    return orc_seq_kahan_f32(v, n);
}

static void var_variant_slice(const float *x, int64_t n, int64_t stride, int64_t ddof, int shift, int sum_kind,
                              int twoterm, float *buf, float *var, float *mean) {
    if (n <= 0) {
        *var = NAN;
        *mean = NAN;
        return;
    }
    gather(x, n, stride, buf);
    float x0 = buf[0];
    if (shift)
        for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] - x0;             /* y */
    float fn = (float)n;
    float m = orc_tree_plain_f32(buf, n, 1, 0) / fn;
    for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] - m;                  /* d */
    float s1 = twoterm ? slice_sum(buf, n, sum_kind) : 0.0f;
    for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] * buf[i];             /* q */
    float s2 = slice_sum(buf, n, sum_kind);
    float a = s2 / fn;
    float v;
    if (twoterm) {
        float b = s1 / fn;
        float bb = b * b;
        v = max0_nan(a - bb);
    } else {
        v = max0_nan(a);
    }
    *var = ddof_scale(v, n, ddof);
    *mean = shift ? x0 + m : m;
}

/*
 * READING (mean in the naive and reference formulae, [VAR] §1): mean(u) is
 * the plain pairwise tree of u multiplied by the rounded reciprocal fl(1/n).
 * The identical-values table of [VAR] §3 fixes this choice (a correctly
 * rounded division would give 0 for the naive formula in every row).
 */
static float mean_recip(const float *u, int64_t n) {
    float inv = 1.0f / (float)n;
    return orc_tree_plain_f32(u, n, 1, 0) * inv;
}

/* The two-term reference formula of [VAR] §1: m = mean(x), d = x - m,
 * v = max(mean(d^2) - mean(d)^2, 0), then the ddof rescale. */
static void var_reference_slice(const float *x, int64_t n, int64_t stride, int64_t ddof,
                                float *buf, float *buf2, float *var, float *mean) {
    if (n <= 0) {
        *var = NAN;
        *mean = NAN;
        return;
    }
    gather(x, n, stride, buf);
    float m = mean_recip(buf, n);
    for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] - m;
    for (int64_t i = 0; i < n; ++i) buf2[i] = buf[i] * buf[i];
    float md = mean_recip(buf, n);
    float mq = mean_recip(buf2, n);
    float v = max0_nan(mq - md * md);
    *var = ddof_scale(v, n, ddof);
    *mean = m;
}

/* The naive formula of [VAR] §1: mean((x - mean(x))^2), then the ddof rescale. */
static void var_naive_slice(const float *x, int64_t n, int64_t stride, int64_t ddof,
                            float *buf, float *var, float *mean) {
    if (n <= 0) {
        *var = NAN;
        *mean = NAN;
        return;
    }
    gather(x, n, stride, buf);
    float m = mean_recip(buf, n);
    for (int64_t i = 0; i < n; ++i) {
        float d = buf[i] - m;
        buf[i] = d * d;
    }
    *var = ddof_scale(mean_recip(buf, n), n, ddof);
    *mean = m;
}

/*
 * Batched entry points over a row-major [rows, cols] array.
 *   axis 1: rows slices of length cols (contiguous)
 *   axis 0: cols slices of length rows (stride cols)
 * method: 0 the kernel (plain Sy tree), 1 the kernel with a compensated Sy
 * tree, 2 two-term reference, 3 naive, and the [VAR] §4 ablation rows:
 *   4 shift + centring, plain tree, no two-term
 *   5 shift + centring + two-term, plain tree
 *   6 no shift, two-term, compensated tree
 *   7 shift + centring, compensated tree, no two-term
 *   8 shift + centring, sequential Kahan scan, no two-term
 *   9 the kernel with double-word carries in its compensated trees
 * mean may be NULL.  Returns 0, or -1 on bad arguments.
 */
int orc_variance_f32(const float *x, int64_t rows, int64_t cols, int axis, int64_t ddof,
                     int method, float *var, float *mean) {
    if (rows < 0 || cols < 0 || ddof < 0 || (axis != 0 && axis != 1) || method < 0 || method > 9)
        return -1;
    int64_t nslices = axis == 1 ? rows : cols;
    int64_t n = axis == 1 ? cols : rows;
    int64_t stride = axis == 1 ? 1 : cols;
    int64_t sstride = axis == 1 ? cols : 1;
    float *buf = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    float *buf2 = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (!buf || !buf2) { free(buf); free(buf2); return -2; }
    for (int64_t s = 0; s < nslices; ++s) {
        const float *xs = x + s * sstride;
        float v, mu;
        switch (method) {
        case 0: var_kernel_slice(xs, n, stride, ddof, 0, buf, &v, &mu); break;
        case 1: var_kernel_slice(xs, n, stride, ddof, 1, buf, &v, &mu); break;
        case 2: var_reference_slice(xs, n, stride, ddof, buf, buf2, &v, &mu); break;
        case 3: var_naive_slice(xs, n, stride, ddof, buf, &v, &mu); break;
        case 4: var_variant_slice(xs, n, stride, ddof, 1, 0, 0, buf, &v, &mu); break;
        case 5: var_variant_slice(xs, n, stride, ddof, 1, 0, 1, buf, &v, &mu); break;
        case 6: var_variant_slice(xs, n, stride, ddof, 0, 1, 1, buf, &v, &mu); break;
        case 7: var_variant_slice(xs, n, stride, ddof, 1, 1, 0, buf, &v, &mu); break;
        case 8: var_variant_slice(xs, n, stride, ddof, 1, 2, 0, buf, &v, &mu); break;
        default: var_variant_slice(xs, n, stride, ddof, 1, 3, 1, buf, &v, &mu); break;
        }
        var[s] = v;
        if (mean) mean[s] = mu;
    }
    free(buf);
    free(buf2);
    return 0;
}

/* ------------------------------------------------------------------ */
/* The method in binary64 (the float64 path; [VAR] §5 lists float64 as  */
/* not measured on the page).  The same steps, topology and readings as */
/* the float32 functions above, every operation in double.             */
/* ------------------------------------------------------------------ */
static inline double two_sum_d(double a, double b, double *err) {
    double s = a + b;
    double bv = s - a;
    double av = s - bv;
    *err = (a - av) + (b - bv);
    return s;
}

double orc_two_sum_f64(double a, double b, double *err) { return two_sum_d(a, b, err); }

/* Compensated tree in double: same padding, pairing, carry and root guard. */
double orc_tree_sum_f64(const double *x, int64_t n, int64_t stride, int64_t pad_to) {
    if (n <= 0) return 0.0;
    int64_t P = pow2_ceil(n);
    if (pad_to != 0) {
        if (pad_to < P || (pad_to & (pad_to - 1)) != 0) return NAN;
        P = pad_to;
    }
    double *s = (double *)malloc((size_t)P * sizeof(double));
    double *c = (double *)malloc((size_t)P * sizeof(double));
    if (!s || !c) { free(s); free(c); return NAN; }
    for (int64_t i = 0; i < P; ++i) {
        s[i] = (i < n) ? x[i * stride] : 0.0;
        c[i] = 0.0;
    }
    for (int64_t len = P; len > 1; len >>= 1) {
        for (int64_t k = 0; k < len / 2; ++k) {
            double e;
            double sk = two_sum_d(s[2 * k], s[2 * k + 1], &e);
            double ck = (c[2 * k] + c[2 * k + 1]) + e;
            s[k] = sk;
            c[k] = ck;
        }
    }
    double root_s = s[0], root_c = c[0];
    free(s);
    free(c);
    if (!isfinite(root_s)) return root_s;
    return root_s + root_c;
}

static double tree_plain_d(const double *x, int64_t n) {
    if (n <= 0) return 0.0;
    int64_t P = pow2_ceil(n);
    double *s = (double *)malloc((size_t)P * sizeof(double));
    if (!s) return NAN;
    for (int64_t i = 0; i < P; ++i) s[i] = (i < n) ? x[i] : 0.0;
    for (int64_t len = P; len > 1; len >>= 1)
        for (int64_t k = 0; k < len / 2; ++k) s[k] = s[2 * k] + s[2 * k + 1];
    double r = s[0] + 0.0;  /* the root rule of the float32 plain tree */
    free(s);
    return r;
}

static inline double max0_nan_d(double v) {
    if (v != v) return v;
    return (v > 0.0) ? v : 0.0;
}

static inline double ddof_scale_d(double v, int64_t n, int64_t ddof) {
    if (ddof == 0) return v;
    int64_t den = n - ddof;
    if (den < 0) den = 0;
    double f = (double)n / (double)den;
    return v * f;
}

/* The kernel of [VAR] §2 on one slice, in double, with the same reading
 * of step 2 as in float32: Sy is the plain tree (comp_sy == 0) or, in the
 * other reading, the compensated tree. */
static void var_kernel_slice_d(const double *x, int64_t n, int64_t stride, int64_t ddof, int comp_sy,
                               double *buf, double *var, double *mean) {
    if (n <= 0) {
        *var = NAN;
        *mean = NAN;
        return;
    }
    for (int64_t i = 0; i < n; ++i) buf[i] = x[i * stride];
    double x0 = buf[0];
    for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] - x0;
    double fn = (double)n;
    double sy = comp_sy ? orc_tree_sum_f64(buf, n, 1, 0) : tree_plain_d(buf, n);
    double m = sy / fn;
    for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] - m;
    double s1 = orc_tree_sum_f64(buf, n, 1, 0);
    for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] * buf[i];
    double s2 = orc_tree_sum_f64(buf, n, 1, 0);
    double a = s2 / fn;
    double b = s1 / fn;
    double bb = b * b;
    *var = ddof_scale_d(max0_nan_d(a - bb), n, ddof);
    *mean = x0 + m;
}

/* The two-term reference formula of [VAR] §1 in double (means as the plain
 * tree times fl(1/n), as in float32). */
static void var_reference_slice_d(const double *x, int64_t n, int64_t stride, int64_t ddof, double *buf,
                                  double *buf2, double *var, double *mean) {
    if (n <= 0) {
        *var = NAN;
        *mean = NAN;
        return;
    }
    for (int64_t i = 0; i < n; ++i) buf[i] = x[i * stride];
    double inv = 1.0 / (double)n;
    double m = tree_plain_d(buf, n) * inv;
    for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] - m;
    for (int64_t i = 0; i < n; ++i) buf2[i] = buf[i] * buf[i];
    double md = tree_plain_d(buf, n) * inv;
    double mq = tree_plain_d(buf2, n) * inv;
    *var = ddof_scale_d(max0_nan_d(mq - md * md), n, ddof);
    *mean = m;
}

/* Variance of a row-major double [rows, cols] array; method 0 the kernel,
 * 1 the kernel with a compensated Sy tree, 2 the two-term reference.
 * Returns 0, or -1 on bad arguments. */
int orc_variance_f64(const double *x, int64_t rows, int64_t cols, int axis, int64_t ddof, int method,
                     double *var, double *mean) {
    if (rows < 0 || cols < 0 || ddof < 0 || (axis != 0 && axis != 1) || method < 0 || method > 2) return -1;
    int64_t nslices = axis == 1 ? rows : cols;
    int64_t n = axis == 1 ? cols : rows;
    int64_t stride = axis == 1 ? 1 : cols;
    int64_t sstride = axis == 1 ? cols : 1;
    double *buf = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double *buf2 = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!buf || !buf2) { free(buf); free(buf2); return -2; }
    for (int64_t s = 0; s < nslices; ++s) {
        double v, mu;
        if (method != 2) var_kernel_slice_d(x + s * sstride, n, stride, ddof, method, buf, &v, &mu);
        else var_reference_slice_d(x + s * sstride, n, stride, ddof, buf, buf2, &v, &mu);
        var[s] = v;
        if (mean) mean[s] = mu;
    }
    free(buf);
    free(buf2);
    return 0;
}
