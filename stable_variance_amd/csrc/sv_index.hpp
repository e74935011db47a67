// Index arithmetic and launch geometry of the library's kernels, as constexpr
// functions: the kernels compute their global load indices with them and the
// launchers their grids, and a host-only test evaluates the same functions
// over whole planned launches (every workgroup, lane and load) to check that
// each index lies inside the data and each launch within the dispatch
// limits.  Plain C++17, no device code: constexpr functions are callable from
// kernels as they are.  Indices count elements (floats, or doubles in the
// float64 path) from the start of the array a kernel reads.
#pragma once

#include <stdint.h>

namespace svx {

// ---------------------------------------------------------------- limits and geometry constants

constexpr int64_t SUM_MAX_N = 1LL << 36;        // tree sum: values per call
constexpr int SUM_W = 4;                        // tree sum: waves per workgroup
constexpr int SUM_MAX_BLOCKS = 8192;            // tree sum: workgroups of one launch
constexpr int SUM_MAX_LOG2_GROUP = 16;          // tree sum: chunks per wave <= 2^16
constexpr int64_t VAR_MAX_ELEMS = 1LL << 36;    // variance: rows * cols per call
constexpr int64_t SEG_MAX_N = 512;              // rows that share waves
constexpr int64_t ROWS_MAX_N = 16384;           // rows of one tile, any number of rows
constexpr int64_t ROWS_ONE_MAX_N = 65536;       // rows of one workgroup when there are enough rows
constexpr int64_t ROWS_ONE_MIN_ROWS = 256;
constexpr int64_t LS_ROW_CHUNK = 64LL * 64 * 4; // long rows: 16384-value chunks (4 waves x 64 lanes x 64)
constexpr int LS_TOP_PER_THREAD = 32;           // long rows: chunk nodes per thread of the top tree
constexpr int LS_MAX_CHUNKS = 256 * LS_TOP_PER_THREAD;
constexpr int CC_E = 16;                        // axis 0: rows per lane in a chunk
constexpr int CC_MIN_W = 4;                     // axis 0: the workspace is sized for the shortest chunk
constexpr int CC_GROUP = 32;                    // axis 0: chunk nodes per column k_cols_dq reduces for m itself
constexpr int TOP_BIG_LEVELS = 16;              // axis 0: 64 * 64 * 2^15 chunk nodes per column
constexpr int64_t COLS_MAX_R = 1024;            // axis 0: single-tile column kernels
constexpr int64_t COLS_ONE_LONG_MAX_R = 4096;   // axis 0: columns read once
constexpr int64_t C64_FUSED_MAX_N = 32768;      // complex rows reduced in one pass
constexpr int KS_T = 64;                        // Kahan scan: values per chunk
constexpr int KS_LEVELS = 16;                   // Kahan scan: 2^16 chunks

// ---------------------------------------------------------------- clamps

// A clamped load of w consecutive elements: e when the group starts inside
// [0, lim), else the last whole group lim - w.  With lim a positive multiple
// of w every group is wholly inside or wholly past the data.  (I: int for
// indices inside one tile, which keeps them in 32-bit registers; int64_t
// for indices into a whole array.)
template <class I>
constexpr I clamp_group(I e, I lim, int w) { return e < lim ? e : lim - w; }

// An index clamped to the last of count (count >= 1).
template <class I>
constexpr I clamp_last(I i, I count) { return i < count ? i : count - 1; }

// ---------------------------------------------------------------- row tiles

// Data values of a tile of `tile` values whose data run has len values left.
constexpr int tile_lim(int64_t len, int tile) { return len <= 0 ? 0 : (len >= tile ? tile : (int)len); }

// Index in a tile of 64*E values of load k of `lane`: per-lane ranges (lane
// owns [lane*E, lane*E + E)) or coalesced (16-byte load k covers the 256
// values [256k, 256k + 256), 4-byte load k the 64 values [64k, 64k + 64)).
// vec: 16-byte loads, k < E/4; else 4-byte loads, k < E.
constexpr int tile_index(bool per_lane, bool vec, int E, int lane, int k) {
  return per_lane ? lane * E + (vec ? 4 * k : k) : (vec ? 256 * k + 4 * lane : 64 * k + lane);
}

// Elements readable from the tile at `base` of row `row` to the end of the
// last row of the launch: rows [row, nrows) of stride ld, the last n long.
constexpr int64_t rows_avail(int64_t nrows, int64_t row, int64_t ld, int64_t n, int64_t base) {
  return (nrows - 1 - row) * ld + (n - base);
}

// The range of virtual lane 2 (L mod 32) + L / 32 held by lane L (the order
// in which the d and d^2 trees share their cross-lane levels).
constexpr int vlane_pair32(int lane) { return 2 * (lane & 31) + (lane >> 5); }

// Workgroup b of nb runs on die b mod 8; the renumbering that gives each die
// one contiguous run of logical indices (die x takes the x-th run, the first
// nb mod 8 runs one longer).  A bijection of [0, nb).
constexpr int xcd_contiguous(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, die = b & 7, i = b >> 3;
  return (die < r ? die * (q + 1) : r * (q + 1) + (die - r) * q) + i;
}

// Short rows sharing waves: the row of `lane` in wave w of workgroup b, S
// lanes per row, 64/S rows per wave, four waves per workgroup.
constexpr int64_t seg_row(int64_t b, int w, int lane, int S) { return (b * 4 + w) * (64 / S) + lane / S; }

// ---------------------------------------------------------------- column tiles

// First of the V adjacent columns a lane loads: c0, or the last V columns
// when c0 lies past the matrix (C >= V).
constexpr int64_t cols_first(int64_t c0, int64_t C, int V) { return c0 < C ? c0 : C - V; }

// Column block of workgroup b of nb when blocks of nc < 32 four-byte words
// (columns of float32, or half as many of float64) share a 128-byte line
// with the next P - 1 blocks (P = 32 / nc): within each full group of 8P
// workgroups, the P that run on one die (b mod 8) take P adjacent blocks.
// A bijection of [0, nb).
template <class I>
constexpr I line_on_one_die(I b, I nb, int nc) {
  if (nc >= 32) return b;
  const I P = 32 / nc, grp = b / (8 * P), r = b % (8 * P);
  return (grp + 1) * (8 * P) <= nb ? grp * (8 * P) + P * (r % 8) + r / 8 : b;
}

// ---------------------------------------------------------------- launch plans

// Work-items of one launch: at most 2^32 - 1.
constexpr int64_t MAX_LAUNCH_ITEMS = 0xffffffffLL;

// The tree sum: chunks of 64*e values, SUM_W-wave workgroups, each wave
// streaming 2^log2_g consecutive chunks; log2_g is the smallest value that
// keeps the workgroup count at or below target_blocks (clamped to
// [1, max_blocks]), capped at max_log2_g.
struct SumPlan {
  int e;
  int log2_g;
  int64_t blocks;
};
constexpr SumPlan plan_sum(int64_t n, int e, int64_t target_blocks, int sum_w, int64_t max_blocks, int max_log2_g) {
  const int64_t chunk = 64LL * e;
  const int64_t chunks = (n + chunk - 1) / chunk;
  const int64_t waves = (chunks + sum_w - 1) / sum_w;
  if (target_blocks > max_blocks) target_blocks = max_blocks;
  if (target_blocks < 1) target_blocks = 1;
  int g = 0;
  while (g < max_log2_g && ((waves + (1LL << g) - 1) >> g) > target_blocks) ++g;
  return {e, g, (waves + (1LL << g) - 1) >> g};
}

// Waves per 4096 values of a row of 1025..16384 values when var_split is 0:
// four waves per row for tiles of up to 4096 values and eight above.
constexpr int auto_split(int64_t n) {
  int64_t tile = 2048;
  while (tile < n) tile *= 2;
  const int64_t w = tile <= 4096 ? 4 : 8;
  return (int)(64 * 64 * w / tile);
}

// Axis 1, one workgroup per row (rows of 257..65536 values not on the
// short-row path): E values per lane, W waves.  split: var_split (0 auto).
struct RowsPlan {
  int E, W;
};
constexpr RowsPlan rows_plan(int64_t n, int split) {
  if (n <= 256) return {4, 1};
  if (n <= 1024) return {16, 1};
  const int s = split != 0 ? split : auto_split(n);
  if (n <= 2048) return s <= 2 ? RowsPlan{32, 1} : s == 4 ? RowsPlan{16, 2} : RowsPlan{8, 4};
  if (n <= 4096)
    return s == 1 ? RowsPlan{64, 1} : s == 2 ? RowsPlan{32, 2} : s == 4 ? RowsPlan{16, 4} : RowsPlan{8, 8};
  if (n <= 8192)
    return s == 1 ? RowsPlan{64, 2} : s == 2 ? RowsPlan{32, 4} : s == 4 ? RowsPlan{16, 8} : RowsPlan{8, 16};
  if (n <= 16384) return s == 1 ? RowsPlan{64, 4} : s == 2 ? RowsPlan{32, 8} : RowsPlan{16, 16};
  if (n <= 32768) return {32, 16};
  return {64, 16};
}

// Waves a row of n values reaches in a plan of W waves of 64*E values.
constexpr int rows_waves(int64_t n, int E, int W) {
  const int64_t reach = (n + 64 * E - 1) / (64 * E);
  return reach < W ? (int)reach : W;
}

// The ablation variants' rows (up to 16384 values, one workgroup per row).
constexpr RowsPlan variant_rows_plan(int64_t n) {
  if (n <= 256) return {4, 1};
  if (n <= 1024) return {16, 1};
  if (n <= 4096) return {32, 2};
  return {64, 4};
}

// Short rows (n <= 512): E values per lane and S lanes per row, S*E the
// row's power-of-two tile.
struct SegPlan {
  int E, S;
};
constexpr SegPlan seg_plan(int64_t n) {
  if (n <= 4) return {4, 1};
  if (n <= 8) return {8, 1};
  if (n <= 16) return {16, 1};
  if (n <= 32) return {16, 2};
  if (n <= 64) return {16, 4};
  if (n <= 128) return {16, 8};
  if (n <= 256) return {16, 16};
  return {16, 32};
}

// Load width of the short-row kernel: 4 floats for 16-byte aligned rows of
// a multiple of 4 values, 2 for 8-byte aligned rows of an even count, else 1.
constexpr int seg_vw(uint64_t addr, int64_t ld) {
  return (addr % 16 == 0 && ld % 4 == 0) ? 4 : (addr % 8 == 0 && ld % 2 == 0) ? 2 : 1;
}

// Complex rows of up to 32768 values in one pass: E values per lane, W waves.
constexpr RowsPlan c64_rows_plan(int64_t n) {
  if (n <= 256) return {4, 1};
  if (n <= 1024) return {16, 1};
  if (n <= 2048) return {16, 2};
  if (n <= 4096) return {16, 4};
  if (n <= 8192) return {16, 8};
  if (n <= 16384) return {16, 16};
  return {32, 16};
}

// Axis 0, lane per column (k_var_cols): E rows per lane, W waves, 64 columns
// per workgroup.
constexpr RowsPlan cols_lane_plan(int64_t R) {
  if (R <= 4) return {4, 1};
  if (R <= 16) return {16, 1};
  if (R <= 64) return {64, 1};
  if (R <= 128) return {64, 2};
  if (R <= 256) return {64, 4};
  if (R <= 512) return {64, 8};
  return {64, 16};
}

// Axis 0, columns of fewer than 16 rows: E rows per lane (the power of two
// at or above R, at least 2), four columns per lane.
constexpr int cols_short_e(int64_t R) { return R <= 2 ? 2 : R <= 4 ? 4 : R <= 8 ? 8 : 16; }

// Axis 0, 65..1024 rows in one launch (k_cols_one): G row groups per wave,
// W waves, 16 rows per lane, V adjacent columns per lane; 16*G*W is the power
// of two at or above R and V*64/G columns per workgroup.
struct ColsOnePlan {
  int G, W;
  int64_t blocks;
};
// Four columns per lane: of the (G, W) pairs that hold exactly that many
// rows (G in 1, 4, 16; W up to 8), the smallest G that still gives 512
// workgroups, else the largest.
constexpr ColsOnePlan cols_one4_plan(int64_t R, int64_t C) {
  int64_t cap = 16;
  while (cap < R) cap *= 2;
  const int gw = (int)(cap / 16);
  int g = gw >= 16 ? gw / 8 : 1;
  if (g == 2 || g == 8) g *= 2;
  while (g < 16 && g * 4 <= gw && (C + 4 * 64 / g - 1) / (4 * 64 / g) < 512) g *= 4;
  return {g, gw / g, (C + 4 * 64 / g - 1) / (4 * 64 / g)};
}
// Four columns per lane, columns that fill at most 5/8 of the plan's tile of
// 16*G*W rows: every wave masked (one code path), only the waves row R reaches.
constexpr bool cols_one4_masked(int64_t R, const ColsOnePlan &p) { return 8 * R <= 5 * 16LL * p.G * p.W; }
// One column per lane: G in 1, 4 (row segments of at least 16 lanes), W up
// to 16; G = 1 when that gives 512 workgroups.
constexpr ColsOnePlan cols_one1_plan(int64_t R, int64_t C) {
  int64_t cap = 16;
  while (cap < R) cap *= 2;
  const int gw = (int)(cap / 16);
  const int g = (gw > 16 || (C + 63) / 64 < 512) && gw >= 8 ? 4 : 1;
  return {g, gw / g, (C + 64 / g - 1) / (64 / g)};
}

// Axis 0, 1025..4096 rows read once: sixteen columns per workgroup, E rows
// per lane (32 up to 2048 rows, else 64), four row groups per wave, the waves
// the column's rows reach; mode 1 when every wave is full, else 2.
struct ColsLongPlan {
  int E, waves, mode;
  int64_t blocks;
};
constexpr ColsLongPlan cols_long_plan(int64_t R, int64_t C) {
  const int e = R <= 2048 ? 32 : 64;
  return {e, (int)((R + 4 * e - 1) / (4 * e)), (R == 2048 || R == 4096) ? 1 : 2, (C + 15) / 16};
}

// A grid of `blocks` workgroups, one per CU at a time on `cus` CUs, fills
// at least three quarters of its last round (false without a CU count).
constexpr bool one_round_fill(int64_t blocks, int64_t cus) {
  if (cus <= 0) return false;
  const int64_t rounds = (blocks + cus - 1) / cus;
  return 4 * blocks >= 3 * rounds * cus;
}

// Axis 0 in row chunks: G row groups per wave (lanes stay on columns: G = 1
// for at least 64 groups of V columns, 4 for 9..63, 8 for 5..8, 16 for 3..4,
// 32 for two, 64 for one, so that at most 64/G groups of lanes hold more
// than half the matrix's columns), chunks of 16*W*G rows, V*64/G columns per
// block.
struct ColsChunkPlan {
  int G;
  int64_t nch, ncb;
};
constexpr ColsChunkPlan cols_chunk_plan(int V, int W, int64_t R, int64_t C) {
  const int64_t groups = (C + V - 1) / V;
  const int g = groups >= 64 ? 1 : groups > 8 ? 4 : groups > 4 ? 8 : groups > 2 ? 16 : groups > 1 ? 32 : 64;
  const int64_t ch = 16LL * W * g;
  const int nc = V * (64 / g);
  return {g, (R + ch - 1) / ch, (C + nc - 1) / nc};
}
// Waves per chunk workgroup when var_cols_waves is 0 (auto): 16, or 8 for
// narrow matrices (8 or more row groups per wave) and where the grid of
// 16-wave workgroups (one per CU at a time) leaves its last round mostly
// empty; 16 without a CU count.
constexpr int cols_chunk_waves(int V, int64_t R, int64_t C, int64_t cus) {
  const ColsChunkPlan p = cols_chunk_plan(V, 16, R, C);
  if (cus <= 0) return 16;
  return (p.G >= 8 || !one_round_fill(p.nch * p.ncb, cus)) ? 8 : 16;
}

// ---------------------------------------------------------------- float32 variance routes

// The launch path of a float32 variance of a [rows, cols] matrix (n > 0
// values per slice), given the launch knobs and, for columns of 1025..4096
// rows, whether the one-read grid fills the chip (one_read_fills).
enum class Route {
  LONG_ROWS_CHUNKED,  // axis 1, rows longer than one tile: chunk launches
  ROWS_SEG,           // axis 1, short rows sharing waves
  ROWS_TILE,          // axis 1, one workgroup per row (rows_plan)
  COLS_PAIRS,         // axis 0, two columns of more than 4096 rows: one row of pairs in chunks
  COLS_ONE_READ,      // axis 0, 1025..4096 rows read once (cols_long_plan)
  COLS_CHUNKED,       // axis 0, row chunks (cols_chunk_plan)
  COLS_SHORT,         // axis 0, fewer than 16 rows, four columns per lane
  COLS_ONE4,          // axis 0, 65..1024 rows, four columns per lane (cols_one4_plan)
  COLS_ONE1,          // axis 0, 65..1024 rows, one column per lane (cols_one1_plan)
  COLS_LANE,          // axis 0, a lane per column (cols_lane_plan)
};
struct RouteKnobs {
  int var_long_rows, var_cols_once, var_cols_single_max, var_short_rows, var_cols_short, var_cols_one,
      var_cols_pairs;
};
// Columns that are candidates for the one-read launch.
constexpr bool cols_one_read_candidate(bool ax1, int64_t n, const RouteKnobs &k) {
  return !ax1 && n > COLS_MAX_R && n <= COLS_ONE_LONG_MAX_R && k.var_cols_once != 0 &&
         k.var_cols_single_max == COLS_MAX_R;
}
// vec16: the matrix starts 16-byte aligned and cols is a multiple of 4.
constexpr Route f32_route(int64_t rows, int64_t cols, bool ax1, bool vec16, const RouteKnobs &k,
                          bool one_read_fills) {
  const int64_t n = ax1 ? cols : rows;
  if (ax1 && n > ROWS_MAX_N && !(k.var_long_rows && n <= ROWS_ONE_MAX_N && rows >= ROWS_ONE_MIN_ROWS))
    return Route::LONG_ROWS_CHUNKED;
  if (!ax1 && cols == 2 && n > COLS_ONE_LONG_MAX_R && k.var_cols_pairs &&
      (n + LS_ROW_CHUNK / 2 - 1) / (LS_ROW_CHUNK / 2) <= LS_MAX_CHUNKS)
    return Route::COLS_PAIRS;
  if (cols_one_read_candidate(ax1, n, k) && (k.var_cols_once == 2 || one_read_fills)) return Route::COLS_ONE_READ;
  if (!ax1 && n > k.var_cols_single_max) return Route::COLS_CHUNKED;
  if (ax1) return n <= SEG_MAX_N && k.var_short_rows ? Route::ROWS_SEG : Route::ROWS_TILE;
  if (n < 16 && k.var_cols_short && vec16) return Route::COLS_SHORT;
  if (k.var_cols_one && n > 64) {
    // four columns per lane for long columns (513..1024 rows) of wide
    // matrices that take 16-byte loads, else one (four 4-byte loads per row
    // measured slower than one column per lane)
    const bool four =
        cols >= 4 && (k.var_cols_one == 2 || (k.var_cols_one == 1 && n > 512 && cols >= 8192 && vec16));
    return four ? Route::COLS_ONE4 : Route::COLS_ONE1;
  }
  return Route::COLS_LANE;
}

// ---------------------------------------------------------------- float64 path

constexpr int64_t S64_MAX_N = 1LL << 35;         // float64 tree sum: values per call
constexpr int S64_W = 4;                         // float64 tree sum: waves per workgroup
constexpr int S64_EF = 32;                       // floats per lane per chunk (16 doubles)
constexpr int S64_MAX_BLOCKS = 8192;
constexpr int S64_MAX_LOG2_G = 16;
constexpr int64_t V64_MAX_ELEMS = 1LL << 35;     // float64 variance: rows * cols per call (256 GiB)
constexpr int64_t V64_ROWS_MAX_N = 16384;        // one workgroup per row
constexpr int64_t V64_ROWS_ONE_MAX_N = 32768;    // ... with at least V64_ROWS_ONE_MIN_ROWS rows
constexpr int64_t V64_ROWS_ONE_MIN_ROWS = 256;
constexpr int64_t V64_COLS_MAX_R = 1024;         // whole columns in one workgroup
constexpr int64_t V64_COLS_ONE_MAX_R = 4096;     // ... or up to this many, read once, when the grid fills
constexpr int L64_E = 16;                        // doubles per lane (long slices)
constexpr int L64_W = 8;                         // waves per workgroup (long slices)
constexpr int64_t L64_ROW_CHUNK = 64LL * L64_E * L64_W;  // 8192 doubles
constexpr int L64_TOP_MAX_K = 32;
constexpr int64_t L64_MAX_CHUNKS = 256LL * L64_TOP_MAX_K;
constexpr int64_t C64_CHUNK = (int64_t)L64_E * L64_W;   // 128 rows
constexpr int C64_GROUP = 32;
constexpr int TOP_BIG_LEVELS_D = 16;

enum class Route64 {
  LONG_ROWS_CHUNKED,  // axis 1, rows longer than one workgroup holds
  ROWS_SEG,           // axis 1, up to 512 values, rows sharing waves (seg_plan)
  ROWS_TILE,          // axis 1, one workgroup per row (rows64_plan)
  COLS_PAIRS,         // axis 0, two columns of more than 4096 rows: one row of pairs in chunks
  COLS_CHUNKED,       // axis 0, more than 1024 rows (cols_chunk64_plan)
  COLS_ONE,           // axis 0, 65..1024 rows, or 1025..4096 read once (cols_one64_plan)
  COLS_SHORT,         // axis 0, fewer than 16 rows, two columns per lane
  COLS_LANE,          // axis 0, a lane per column (cols_lane64_plan)
};
// Columns that are candidates for the one-read launch of 1025..4096 rows
// (var_cols_once: the float32 knob, 0 never, 1 when the grid fills, 2 always).
// Under knob 1 the column also fills at least 5/8 of its tile (2048 or 4096
// rows): a tile half padding ([1025, 16384]: 72 against 62 us for the row
// chunks) holds a CU for half the data.
constexpr bool cols_one_read64_candidate(bool ax1, int64_t rows, int64_t cols, int var_cols_once) {
  const int64_t tile = rows > 2048 ? 4096 : 2048;
  return !ax1 && rows > V64_COLS_MAX_R && rows <= V64_COLS_ONE_MAX_R && cols >= 2 && var_cols_once != 0 &&
         (var_cols_once == 2 || 8 * rows >= 5 * tile);
}
// vec16: the matrix starts 16-byte aligned and cols is even.  one_read: the
// one-read launch is chosen for a candidate (above).  pairs: the float32 knob
// var_cols_pairs.  long_rows: the float32 knob var_long_rows (0: rows of
// 16385..32768 values take the chunks whatever the row count).
constexpr Route64 f64_route(int64_t rows, int64_t cols, bool ax1, bool vec16, bool one_read = false,
                            bool pairs = true, bool long_rows = true) {
  const int64_t n = ax1 ? cols : rows;
  if (ax1) {
    if (n <= 512) return Route64::ROWS_SEG;
    if (n <= V64_ROWS_MAX_N || (long_rows && n <= V64_ROWS_ONE_MAX_N && rows >= V64_ROWS_ONE_MIN_ROWS))
      return Route64::ROWS_TILE;
    return Route64::LONG_ROWS_CHUNKED;
  }
  if (cols == 2 && n > V64_COLS_ONE_MAX_R && pairs &&
      (n + L64_ROW_CHUNK / 2 - 1) / (L64_ROW_CHUNK / 2) <= L64_MAX_CHUNKS)
    return Route64::COLS_PAIRS;
  if (n > V64_COLS_MAX_R) return (one_read && n <= V64_COLS_ONE_MAX_R && cols >= 2) ? Route64::COLS_ONE
                                                                                    : Route64::COLS_CHUNKED;
  if (n > 64) return Route64::COLS_ONE;
  if (n < 16 && vec16) return Route64::COLS_SHORT;
  return Route64::COLS_LANE;
}
// Axis-1 rows of 513..32768 doubles: 16 doubles per lane and the waves of the
// power-of-two tile, 32 per lane and 16 waves above 16384.
constexpr RowsPlan rows64_plan(int64_t n) {
  if (n <= 1024) return {16, 1};
  if (n <= 2048) return {16, 2};
  if (n <= 4096) return {16, 4};
  if (n <= 8192) return {16, 8};
  if (n <= V64_ROWS_MAX_N) return {16, 16};
  return {32, 16};
}
// Axis 0, 65..4096 rows in one launch: V adjacent columns per lane (two above
// 512 rows, one below or for a single column), G row groups, W waves of 16
// rows per lane (above 1024 rows: at least two columns, 8 waves, and 32 row
// groups above 2048), `blocks` workgroups of V*64/G columns.  wide: columns
// of exactly 2048 or 4096 rows with 16-byte loads take 16 waves instead, and
// 8 or 16 row groups (sixteen or eight columns per workgroup).
struct ColsOne64Plan {
  int V, G, W;
  int64_t blocks;
};
constexpr bool cols_one64_wide_ok(int64_t R, bool vec16) { return vec16 && (R == 2048 || R == 4096); }
constexpr ColsOne64Plan cols_one64_plan(int64_t R, int64_t C, bool vec16, bool wide = false) {
  if (wide && cols_one64_wide_ok(R, vec16))
    return R == 4096 ? ColsOne64Plan{2, 16, 16, (C + 7) / 8} : ColsOne64Plan{2, 8, 16, (C + 15) / 16};
  if (R > 2048) return {2, 32, 8, (C + 3) / 4};
  if (R > V64_COLS_MAX_R) return {2, 16, 8, (C + 7) / 8};
  if (R > 512) return (vec16 || C >= 2) ? ColsOne64Plan{2, 16, 4, (C + 7) / 8} : ColsOne64Plan{1, 16, 4, (C + 3) / 4};
  int64_t cap = L64_E;
  while (cap < R) cap *= 2;
  const int gw = (int)(cap / L64_E);
  const int g = (gw > 16 || (C + 63) / 64 < 512) ? 4 : 1;
  return {1, g, gw / g, (C + 64 / g - 1) / (64 / g)};
}
// Axis 0, a lane per column (up to 64 rows).
constexpr RowsPlan cols_lane64_plan(int64_t R) {
  if (R <= 4) return {4, 1};
  if (R <= 16) return {16, 1};
  return {16, 4};
}
// Axis 0 in chunks of 128*G rows of a block of V*64/G columns: G = 1 for at
// least 64 column groups of V, 4 for 9..63, 8 for 5..8, 16 for 3..4, 32 for
// 2, 64 for one.
constexpr ColsChunkPlan cols_chunk64_plan(int V, int64_t R, int64_t C) {
  const int64_t groups = (C + V - 1) / V;
  const int g = groups >= 64 ? 1 : groups > 8 ? 4 : groups > 4 ? 8 : groups > 2 ? 16 : groups > 1 ? 32 : 64;
  const int64_t ch = C64_CHUNK * g;
  const int nc = V * (64 / g);
  return {g, (R + ch - 1) / ch, (C + nc - 1) / nc};
}

// ---------------------------------------------------------------- ADN sum

constexpr int ADN_REC = 44;              // 32-bit words per accumulator record (2K + 2 <= 44)
constexpr int ADN_WAVES = 4;             // waves per workgroup
constexpr int ADN_MAX_BLOCKS = 8192;
constexpr int ADN_GROUP = 64;            // workgroups per first-level ticket
constexpr int ADN_COUNTER_STRIDE = 64;   // counters 256 bytes apart (32-bit words)
// The counter header (the top counter, then one per group of ADN_GROUP
// workgroups), then ADN_MAX_BLOCKS workgroup records and one record per group.
constexpr int64_t ADN_WS_HEADER = 256 * (1 + ADN_MAX_BLOCKS / ADN_GROUP);

// The ADN sum's launch over n values: chunks of 64*e values, g consecutive
// chunks per wave, `blocks` workgroups of ADN_WAVES waves, at most
// target_blocks (<= ADN_MAX_BLOCKS).
struct AdnPlan {
  int64_t chunks, g, blocks;
};
constexpr AdnPlan adn_plan(int64_t n, int e, int64_t target_blocks) {
  const int64_t chunks = (n + 64LL * e - 1) / (64LL * e);
  const int64_t waves_target = ADN_WAVES * target_blocks;
  const int64_t g = (chunks + waves_target - 1) / waves_target;
  const int64_t waves = (chunks + g - 1) / g;
  return {chunks, g, (waves + ADN_WAVES - 1) / ADN_WAVES};
}
// Value t (0..3) of group j of a lane's E values in the chunk at `base`:
// 16-byte loads (vec) give lane l the values 4(l + 64j) .. 4(l + 64j) + 3,
// single loads the values l + 64(4j + t).
constexpr int64_t adn_index(int64_t base, int lane, int j, int t, bool vec) {
  return vec ? base + 4 * (lane + 64 * j) + t : base + lane + 64 * (4 * j + t);
}

}  // namespace svx
