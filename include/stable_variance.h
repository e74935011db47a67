/*
 * stable_variance.h - C ABI of libstable_variance.so (MI355X / gfx950).
 *
 * Accurate float32 reductions by a compensated pairwise tree:
 *
 *   sv_tree_sum_f32   the sum of n float32 values by a binary tree of TwoSum
 *                     additions whose exact rounding errors are carried up a
 *                     second array (Pennacchio, "Variance in float32 with a
 *                     first-element shift, a local centring and a compensated
 *                     tree sum", §2 step 3).
 *   sv_variance_f32   the variance and the mean of each slice of a row-major
 *                     [rows, cols] array along an axis (same page, §2 steps
 *                     1-4): shift by the slice's first element, local
 *                     centring by the plain tree of the shifted values,
 *                     compensated trees of d and d^2, two-term correction
 *                     and ddof rescale.
 *
 * Arithmetic: IEEE binary32, round to nearest even, every operation rounded
 * on its own (no FMA contraction, no reassociation, subnormals kept).
 *
 * Tree topology (fixed, independent of launch geometry, stream and run):
 * the n values are padded with +0 to a power of two and each level adds
 * adjacent pairs, so node k of level l covers elements [k*2^l, (k+1)*2^l).
 * A node combines (s_l, c_l) and (s_r, c_r) into s = fl(s_l + s_r) with the
 * TwoSum error e, and c = fl(fl(c_l + c_r) + e).  A tree's value is
 * fl(s + c) at the root, or s when s is Inf or NaN.  Results are therefore
 * bit-identical from run to run and equal to the CPU oracle's.
 *
 * Conventions for every entry point:
 *   - Device pointers only (memory from hipMalloc / torch on the current HIP
 *     device); the caller owns every buffer.  Host pointers are not accepted.
 *   - The call validates its arguments on the host first.  On any error it
 *     returns a nonzero status, launches nothing and leaves the outputs
 *     untouched; sv_last_error_message() then describes the error.
 *   - The call is asynchronous: it enqueues work on `stream` (a hipStream_t;
 *     NULL is the default stream) and returns.  Outputs are valid once the
 *     stream has been synchronised.  Inputs must stay valid until then.
 *   - Calls never throw and never allocate device memory.  They make no
 *     memset or copy calls and no host synchronisation, and every counter
 *     they use is reset by the kernels, so a sequence of calls can be
 *     captured once in a HIP graph and replayed.
 *   - Calls that share a workspace must be ordered (same stream); two
 *     concurrent calls need two workspaces.
 */
#ifndef STABLE_VARIANCE_H
#define STABLE_VARIANCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 1

typedef int sv_status;
#define SV_OK 0
#define SV_ERR_INVALID_ARGUMENT 1 /* bad size, axis, ddof or null pointer        */
#define SV_ERR_WORKSPACE 2        /* workspace missing, too small or misaligned  */
#define SV_ERR_NO_DEVICE 3        /* no usable HIP device                        */
#define SV_ERR_HIP 4              /* a HIP runtime call or a launch failed       */
#define SV_ERR_UNSUPPORTED 5      /* shape outside what the library supports     */

/* Version of this ABI (SV_ABI_VERSION of the header the library was built with). */
int sv_abi_version(void);

/* Static, human-readable name of a status code. */
const char *sv_status_string(sv_status status);

/* Description of the last error raised on the calling thread ("" if none).
 * The pointer stays valid until the next call on the same thread. */
const char *sv_last_error_message(void);

/* Bytes of ticket counters at the start of a tree-sum workspace. */
#define SV_TREE_SUM_COUNTER_BYTES 33024

/*
 * Bytes of workspace sv_tree_sum_f32 needs for n values (0 for n <= 0,
 * (size_t)-1 for an unsupported n).  The workspace must be 256-byte aligned.
 * Its first SV_TREE_SUM_COUNTER_BYTES bytes hold ticket counters that must
 * be ZERO before the first use; every call leaves them zero again, so the
 * workspace can be reused by later calls in stream order.  The rest is
 * scratch (partial nodes) and needs no initialisation.
 */
size_t sv_tree_sum_f32_workspace_size(int64_t n);

/*
 * out[0] = compensated tree sum of x[0 .. n).
 *   x          device pointer to n float32 values (any alignment; n > 0)
 *   n          number of values, 0 <= n <= 2^36 (n == 0 writes +0)
 *   out        device pointer to one float32
 *   workspace  device buffer of sv_tree_sum_f32_workspace_size(n) bytes
 *              whose counter bytes are zero (see above); may be NULL when
 *              that size is 0
 *   stream     hipStream_t or NULL
 * Source: Pennacchio, "Variance in float32 ...", §2 step 3 (the tree of
 * TwoSum additions with the errors carried up a second array).
 */
sv_status sv_tree_sum_f32(const float *x, int64_t n, float *out, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * The same tree with double-word carries: after every node the pair (s, c)
 * is renormalised with TwoSum, so that |c| <= ulp(s)/2 and each carry
 * addition is rounded relative to the node's own value.  Per node the added
 * error is at most about 3 u^2 (|s_l| + |s_r|) (u = 2^-24) instead of growing
 * with the depth, which matters when large partial sums cancel: on the 10^8
 * cancelling-pairs workload the plain carry ends 3.9e-7 from the exact sum,
 * this one at the correctly rounded value.  Arguments, workspace (the same
 * size and counter rules as sv_tree_sum_f32), errors and asynchrony as for
 * sv_tree_sum_f32.
 * Source: "Reduction order and compensation solve related but different
 * problems" (wider or expansion-based accumulators for stronger
 * guarantees), applied to the method's own node.
 */
sv_status sv_tree_sum_dw_f32(const float *x, int64_t n, float *out, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * sv_tree_sum_f32 for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same result, arguments (without the workspace),
 * errors and asynchrony as sv_tree_sum_f32, and n <= 2^36 (a larger n gives
 * SV_ERR_UNSUPPORTED).  It allocates nothing: the workspace is a
 * SV_TREE_SUM_NOALLOC_SCRATCH_BYTES-byte array inside the library, one per
 * GPU, held until the process ends.  Its first call on a device looks the
 * array up (with that device current) and clears its ticket counters on
 * `stream` with a small kernel; every call leaves them zero again.  All calls
 * on one GPU share that array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give wrong results, so order them, e.g.
 * on one stream.
 */
#define SV_TREE_SUM_NOALLOC_SCRATCH_BYTES 99584
sv_status sv_tree_sum_f32_noalloc(const float *x, int64_t n, float *out, void *stream);

/*
 * Bytes of workspace sv_variance_f32 needs.
 *   axis 1: 0 when every row fits one workgroup (n <= 16384 values), else 24
 *           bytes per 16384-value chunk of every row plus 4 bytes per row
 *           (long rows are reduced in chunks, reading the input twice; with
 *           256 or more rows of up to 65536 values each row takes one
 *           workgroup instead and the workspace is not used, but the size
 *           stays the chunked path's, independent of the tuning knobs).
 *   axis 0: whenever rows and cols are both nonzero: three arrays of 8
 *           bytes per 64-row chunk per column and 4 bytes per column, each
 *           rounded up to 256 bytes.  Columns of up to 4096 rows are reduced
 *           in one launch that reads the input once (whole columns per
 *           workgroup); longer columns in row chunks, reading the input
 *           twice.  The size does not depend on the tuning knobs.
 * (size_t)-1 for an unsupported shape (an axis-1 row of more than 8192
 * chunks, a bad axis, rows * cols > 2^36).  The workspace must be 256-byte
 * aligned; it is scratch (no initialisation, nothing kept between calls), so
 * calls that share one must be ordered on one stream.
 */
size_t sv_variance_f32_workspace_size(int64_t rows, int64_t cols, int axis);

/*
 * Variance (and mean) of each slice of the row-major [rows, cols] float32
 * array x, along `axis`:
 *   axis 1 or -1  rows slices, each the cols contiguous values of a row;
 *                 var_out/mean_out have rows entries
 *   axis 0 or -2  cols slices, each the rows values of a column (stride
 *                 cols); var_out/mean_out have cols entries
 * For each slice x[0..n) (Pennacchio, "Variance in float32 ...", §2):
 *   step 1  y_i = fl(x_i - x_0)
 *   step 2  m = fl(Plain(y) / fl(n)),  d_i = fl(y_i - m), where Plain is
 *           the same adjacent-pair tree without the error array (step 2
 *           writes a plain sum; step 3 introduces the compensated tree for
 *           the sums of the residuals)
 *   step 3  S1 = Tree(d),  S2 = Tree(fl(d_i * d_i))
 *   step 4  var = max(fl(fl(S2/n) - fl(b*b)), 0) with b = fl(S1/n), where a
 *           NaN stays NaN and any other value <= 0 gives +0; if ddof != 0
 *           var = fl(var * fl(fl(n) / fl(max(n - ddof, 0))));
 *           mean = fl(x_0 + m).
 * An empty slice (n == 0) gives var = mean = NaN.
 *   ddof       >= 0
 *   mean_out   may be NULL (the mean is then not written)
 *   workspace  device buffer of sv_variance_f32_workspace_size(...) bytes;
 *              may be NULL when that size is 0
 * rows and cols must be >= 0 with rows * cols <= 2^36 (256 GiB of float32,
 * about the most one 288 GB GPU holds: every launch then stays within HIP's
 * 2^32 - 1 work-items per grid); an axis-1 row may hold at most 8192 chunks
 * (134,217,728 values).
 */
sv_status sv_variance_f32(const float *x, int64_t rows, int64_t cols, int axis, int64_t ddof,
                          float *var_out, float *mean_out, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Complex64 variance (Pennacchio, "Variance in float32 ...", §2: a complex
 * input is split into its real and imaginary parts and the two variances
 * are added, which is E|z - mean(z)|^2).
 *   z          device pointer to a row-major [rows, cols] complex64 array
 *              (interleaved re, im float32 pairs), 8-byte aligned
 *   axis       as for sv_variance_f32
 *   var_out    float32, one per slice: fl(var(re) + var(im)), each part
 *              computed exactly as sv_variance_f32 computes it
 *   mean_out   complex64 (interleaved), one per slice, or NULL:
 *              (mean(re), mean(im))
 *   workspace  sv_variance_c64_workspace_size(rows, cols, axis) bytes,
 *              256-byte aligned, no initialisation; NULL allowed when that
 *              size is 0.  Axis 1 rows of up to 32768 values are read once
 *              and need none; longer rows (up to 8192 chunks of 8192
 *              values) are read twice in chunks, the parts split in
 *              registers (8 bytes per row and 24 per chunk per part); rows
 *              beyond that stage the split parts (8 bytes per input value);
 *              axis 0 reads the interleaved array as float32 [rows, 2 * cols]
 *              columns
 * Errors and asynchrony as for sv_variance_f32.
 */
size_t sv_variance_c64_workspace_size(int64_t rows, int64_t cols, int axis);
sv_status sv_variance_c64(const float *z, int64_t rows, int64_t cols, int axis, int64_t ddof, float *var_out,
                          float *mean_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The variants of the method page's ablation (Pennacchio, "Variance in
 * float32 ...", §4: one step changed at a time) and the two formulae of its
 * §1, for accuracy and speed comparisons.  `variant`:
 *   0  the method (same result as sv_variance_f32)
 *   1  the method with the compensated tree for the local mean too,
 *      m = fl(Tree(y) / fl(n)) (the other reading of §2 step 2)
 *   2  two-term reference formula: m = mean(x), d = x - m,
 *      var = max(mean(d^2) - mean(d)^2, 0); mean() = plain tree * fl(1/n);
 *      no shift (the returned mean is m)
 *   3  naive formula: var = mean((x - mean(x))^2), means as in 2
 *   4  shift + centring, plain trees, no two-term: var = max(S2/n, 0)
 *   5  shift + centring + two-term, plain trees
 *   6  no shift, two-term, compensated trees (the returned mean is m)
 *   7  shift + centring, compensated trees, no two-term
 *   8  shift + centring, sequential Kahan scan, no two-term: m from the plain
 *      tree of y as in the method, then S2 = Kahan's compensated recurrence
 *      over q_i = (y_i - m)^2 in index order (s = c = 0; for each q:
 *      t = s + (q - c), c = (t - s) - (q - c), s = t), var = max(S2/n, 0)
 *      and the ddof rescale.  A serial chain per slice (a lane per slice),
 *      so it runs far below the other variants' speed, as on the page
 * "Plain tree" is the same adjacent-pair topology without the error array.
 * Every variant but 1 takes the plain tree for the local mean, as the method
 * does; "plain" and "compensated" name the trees of d and d^2.
 * Shapes: axis 1 with n <= 16384, axis 0 with n <= 1024; variant 8 any
 * axis with n <= 4194304 (else SV_ERR_UNSUPPORTED; longer slices of
 * variants 0-7 take sv_variance_variant_ws_f32).  No workspace; otherwise
 * as sv_variance_f32.
 */
sv_status sv_variance_variant_f32(const float *x, int64_t rows, int64_t cols, int axis, int64_t ddof, int variant,
                                  float *var_out, float *mean_out, void *stream);

/*
 * The same variants with a caller-provided device workspace, for slices
 * longer than one workgroup holds (same page, §4; the slice computation of
 * §2 with one step changed).  Rows of more than 16384 values are reduced in
 * chunks of 16384 (aligned nodes of the slice's tree, so the same bits as
 * one workgroup would give); columns of more than 1024 rows are first
 * transposed into the workspace (a copy: the same values in the same order,
 * hence the same trees), then reduced as rows.  Slices of up to 8192 chunks
 * (2^27 values); rows * cols <= 2^36.
 * workspace: device memory, 256-byte aligned, at least
 * sv_variance_variant_f32_workspace_size(rows, cols, axis, variant) bytes
 * (0 for the shapes sv_variance_variant_f32 takes, and then it may be NULL);
 * scratch, contents on entry ignored; SV_ERR_WORKSPACE when it is missing,
 * short or misaligned.  The size function returns (size_t)-1 for an
 * invalid argument or a shape beyond these limits.  Everything else as
 * sv_variance_variant_f32.
 */
size_t sv_variance_variant_f32_workspace_size(int64_t rows, int64_t cols, int axis, int variant);
sv_status sv_variance_variant_ws_f32(const float *x, int64_t rows, int64_t cols, int axis, int64_t ddof,
                                     int variant, float *var_out, float *mean_out, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * The method in binary64 (the float64 path): the compensated tree sum and
 * the variance of Pennacchio, "Variance in float32 ...", §2 steps 1-4, with
 * every operation in double (§5 of that page lists float64 as not
 * measured).  Same topology, carries, root guard, max, ddof and empty-slice
 * readings as the float32 entry points.
 *
 * sv_tree_sum_f64: x n device doubles (8-byte aligned), 0 <= n <= 2^35;
 *   out one device double; workspace of sv_tree_sum_f64_workspace_size(n)
 *   bytes, 256-byte aligned, whose first SV_TREE_SUM_COUNTER_BYTES bytes are
 *   ticket counters with the same rules as for sv_tree_sum_f32.
 * sv_variance_f64: x row-major [rows, cols] device doubles (8-byte aligned),
 *   rows * cols <= 2^35 (256 GiB of float64; every launch then stays
 *   within HIP's 2^32 - 1 work-items per grid); var_out (and mean_out if
 *   not NULL) one double per slice; workspace of sv_variance_f64_workspace_size(rows, cols, axis)
 *   bytes, 256-byte aligned scratch, NULL allowed when that size is 0.
 * sv_variance_f64_workspace_size: 0 when every slice fits one workgroup
 *   (axis 1: n <= 16384; axis 0: n <= 1024).  Longer slices are reduced in
 *   chunks (8192 values of a row; 128 rows of a column, or a multiple of 128
 *   for narrow matrices), reading the input twice: three arrays of 16 bytes
 *   per 128-value chunk per slice and 8 bytes per slice, each rounded up to
 *   256 bytes.  (size_t)-1 for an unsupported
 *   shape (a bad axis, rows * cols > 2^35, an axis-1 row of more than 8192
 *   chunks, i.e. 67,108,864 values).
 * Errors and asynchrony as for the float32 entry points.
 */
size_t sv_tree_sum_f64_workspace_size(int64_t n);
sv_status sv_tree_sum_f64(const double *x, int64_t n, double *out, void *workspace, size_t workspace_bytes,
                          void *stream);
size_t sv_variance_f64_workspace_size(int64_t rows, int64_t cols, int axis);
sv_status sv_variance_f64(const double *x, int64_t rows, int64_t cols, int axis, int64_t ddof, double *var_out,
                          double *mean_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Ahrens-Demmel-Nguyen binned reproducible sum of float32 values, as the
 * "SyclReproSum" README describes it ("How It Works", "Accumulator capacity",
 * "Template Parameters"): every value is deposited into `fold` (K) primary
 * values on a fixed global grid of 13-bit exponent bins, plus K carry
 * counts; primaries renormalise into carries every 512 deposits; partial
 * accumulators merge exactly; the total is converted to float through a
 * running double value.  The result has the same bits for any order of the
 * values, any launch geometry and any run.
 *
 * Readings where the page is silent (the CPU oracle takes the same ones):
 *   - bins b = 0..21 hold the weights 2^(13b - 146) .. 2^(13b - 134); the
 *     folds are bins top, top-1, .., top-K+1, where top is the smallest bin
 *     with |x| < 2^(13 top - 134) for every finite x, and at least K-1;
 *   - each fold rounds what reaches it to its unit, to nearest with ties
 *     away from zero (the sticky bit), and passes the exact rest on; the
 *     rounding of the last fold is the only loss (at most
 *     N * 2^(-13(K-1)) * max|x| in total, the page's dominant error term);
 *   - the result is float(y), y the running double sum of the exact fold
 *     values from the coarsest fold; an empty sum or a sum of zeros is +0;
 *   - any NaN, or +Inf together with -Inf, gives 0x7fc00000; otherwise a
 *     single-signed Inf gives that Inf (both from the page); a finite total
 *     beyond the float range gives +-Inf.
 *
 * x: n device floats (any alignment; 16-byte alignment takes vector loads).
 * fold: 2 .. SV_ADN_MAX_FOLD = 21, every fold count the page allows for
 *   float (outside 2..21 SV_ERR_INVALID_ARGUMENT).  From 21 folds, and from
 *   any index in the two coarsest bins, the deposits take the kernel's
 *   general path (slower, same bits).
 * n: 0 .. SV_ADN_MAX_COUNT (the page's capacity for float; above it
 *   SV_ERR_UNSUPPORTED before anything else is touched).
 * out: one device float.
 * workspace: device memory of sv_adn_sum_f32_workspace_size(n) bytes (0 for
 *   n == 0), 256-byte aligned; its first SV_ADN_SUM_COUNTER_BYTES bytes are
 *   ticket counters that must be zero before the first use and that every
 *   call leaves zero; calls sharing a workspace must be ordered on one
 *   stream.  Errors and asynchrony as for sv_tree_sum_f32.
 */
#define SV_ADN_MAX_FOLD 21
#define SV_ADN_MAX_COUNT 4294966784LL
#define SV_ADN_SUM_COUNTER_BYTES 33024
size_t sv_adn_sum_f32_workspace_size(int64_t n);
sv_status sv_adn_sum_f32(const float *x, int64_t n, int fold, float *out, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * Measurement aid, not part of the method: reads x[0 .. n) once from HBM with
 * plain non-temporal 16-byte loads (x 16-byte aligned, n <= 2^36) and does no
 * arithmetic of the method, so its duration is the practical read ceiling
 * the reduction kernels are compared with.  out (one float) is never written
 * for finite data.  Asynchronous on `stream` like the entry points above.
 */
sv_status sv_probe_read_bandwidth(const float *x, int64_t n, float *out, void *stream);

/*
 * Launch-geometry tuning for tests and benchmarks.  A knob only changes how
 * the work is mapped onto the GPU, never a result bit.  Keys (defaults are
 * the fastest settings measured on MI355X):
 *   "sum_load_path"  tree sum: 0 = coalesced 16-byte loads transposed through
 *                    LDS into lane-contiguous order (default), 1 = each lane
 *                    loads its own contiguous values
 *   "sum_nt"         tree sum: 1 = non-temporal loads (default), 0 = ordinary
 *   "sum_e"          values per lane in a tree-sum chunk: 16 or 32 (default)
 *   "sum_depth"      tree-sum chunks in flight per wave: 2 (default) or 4
 *   "sum_blocks"     target number of tree-sum workgroups, 1..8192 (default
 *                    8192); each wave then streams a power-of-two run of chunks
 *   "var_load_path"  row variance: as sum_load_path (default 1), or 2 =
 *                    coalesced loads transposed through LDS in four stages of
 *                    16 lanes each (a quarter of the LDS of path 0)
 *   "var_nt"         row variance: as sum_nt (default 0)
 *   "var_full_rows"  rows that fill their power-of-two tile exactly and
 *                    start 16-byte aligned: 1 (default) = the kernel without
 *                    masks or clamped loads, 0 = the general row kernel
 *   "var_split"      rows of 1025..16384 values: waves per 4096 values of
 *                    the row's power-of-two tile, 1, 2, 4 or 8 (64, 32, 16
 *                    or 8 values per lane; a 2048-value tile takes at most 32
 *                    values per lane, a 16384-value tile at most 16 waves), or
 *                    0 (default): four waves per row for tiles of up to 4096
 *                    values, eight above
 *   "var_lds_pad"    unused dynamic LDS bytes per row workgroup, 0..65536
 *                    (default 0): a cap on resident waves, for measurements
 *   "var_short_rows" rows of at most 512 values: 1 (default) = several rows
 *                    per wave (a group of lanes per row), 0 = one workgroup
 *                    per row
 *   "var_long_rows"  axis 1, rows of 16385..65536 floats (16385..32768
 *                    doubles) when there are at least 256 rows: 1 (default)
 *                    = one workgroup of 16 waves per row, the row read once
 *                    (the workspace is then not used); 0 = the chunked path
 *   "var_cols_short" axis 0, columns of at most 15 rows with a 16-byte
 *                    aligned base and a width divisible by 4: 1 (default) =
 *                    four columns per lane, every tree in-lane; 0 = a lane
 *                    per column
 *   "var_cols_one"   axis 0, columns of 65 to var_cols_single_max rows:
 *                    one launch of G row groups per wave with 2 = four
 *                    columns per lane (one 16-byte load per row for a 16-byte
 *                    aligned base and a width divisible by 4, else four
 *                    4-byte loads; widths below 4 take one), 3 = one column
 *                    per lane, 1 (default) = four for 513 rows or more,
 *                    8192 columns or more and 16-byte loads, else one;
 *                    0 = 64 columns per workgroup, a lane per column, not one launch per tile
 *   "var_cols_single_max"  axis 0: columns of up to this many rows are
 *                    held by one workgroup and read once (0..1024, default
 *                    1024); longer columns are reduced in row chunks
 *   "var_cols_waves" axis 0, chunked: waves per workgroup, 4, 8 or 16
 *                    (chunks of 16 rows per wave times the row groups per
 *                    wave), or 0 (default): 16, or 8 for matrices of at
 *                    most 32 columns with 16-byte loads (8 of other widths)
 *                    and where a grid of 16-wave workgroups, one per CU at
 *                    a time, would leave its last round mostly empty
 *   "var_cols_once"  axis 0, columns of 1025..4096 rows: 1 (default) = 16
 *                    whole columns per workgroup of up to 16 waves, one
 *                    column per lane, the input read once, when that grid
 *                    fills at least three quarters of the chip's last round
 *                    of workgroups, else the row-chunk launches; 0 = always
 *                    the row-chunk launches; 2 = always the one-read launch.
 *                    The same setting picks the float64 launch of columns of
 *                    1025..4096 rows (at least two columns): eight or four
 *                    whole columns per workgroup of 8 waves, read once (under
 *                    1, only columns of at least 1280 or 2560 rows, 5/8 of
 *                    their 2048- or 4096-row tile, and when that grid fills
 *                    three quarters of its last round of one workgroup per
 *                    CU); columns of exactly 2048 or 4096 rows with a 16-byte
 *                    aligned base and an even width take sixteen or eight
 *                    whole columns per workgroup of 16 waves instead when
 *                    that grid fills the chip by the same rule (under 2,
 *                    always)
 *   "sum_xcd"        tree sum: 1 = renumber the workgroups so that each of the
 *                    eight dies (XCDs) streams one contiguous region; 0 =
 *                    dispatch order, consecutive regions spread over the dies
 *                    (default, faster on MI355X)
 *   "var_xcd"        row variance: as sum_xcd, over rows (default 0)
 *   "var_cols_pairs" axis 0, two columns of more than 4096 rows: 1 (default)
 *                    = one row of pairs in chunks (wide loads), 0 = the
 *                    column chunks; float32 and float64
 *   "adn_e"         values per lane in an ADN-sum chunk: 16 (default) or 32
 *                    (32 only with three folds; other counts use 16)
 *   "adn_blocks"     target number of ADN-sum workgroups, 1..8192 (default 512)
 *   "launch_items"   work-items per launch before a grid is cut into
 *                    batches (each batch one launch with a first-workgroup
 *                    offset): 1024 .. 2^32 - 1 (default 2^32 - 1, HIP's
 *                    limit; lower values run the batched launches on small
 *                    inputs, for tests)
 *   "reset"          any value: restore every default
 * Returns SV_ERR_INVALID_ARGUMENT for an unknown key or value.  The settings
 * belong to the calling host thread: they steer that thread's later calls
 * only, and every other thread keeps its own (a new thread starts from the
 * defaults).
 */
sv_status sv_set_tuning(const char *key, int64_t value);

#ifdef __cplusplus
}
#endif

#endif /* STABLE_VARIANCE_H */
