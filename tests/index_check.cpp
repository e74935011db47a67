// Host-only check of the float32 library's global load indices and launch
// plans.  The launch geometry (svx::f32_route and the *_plan functions) and
// the index arithmetic of every load (svx::clamp_*, tile_index, rows_avail,
// seg_row, cols_first, line_on_one_die, ...) are the functions the kernels
// and launchers call; this program walks each planned launch the way the
// kernel walks its data (workgroups, waves, lanes, loads) and checks that
// every element a load touches lies inside the array, and that every launch
// stays within the dispatch limits (at most 2^32 - 1 work-items, 2^31 - 1
// workgroups).  Large grids are sampled: their first and last workgroups
// and an even spread between.
//
// Build: g++ -std=c++17 -O2 index_check.cpp -o index_check; run: ./index_check
// (prints one line per failure, at most 40, and a summary; exit 1 on any).
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <set>
#include <string>
#include <vector>

#include "../include/stable_variance.h"
#include "../stable_variance_amd/csrc/sv_index.hpp"

using namespace svx;

namespace {

int64_t g_checks = 0, g_launches = 0, g_fail = 0;
std::set<std::string> g_seen;  // one line per (path, shape, kind of failure)

struct Where {
  const char *path;
  int64_t rows, cols;
  int64_t total;  // elements of the array the loads read
};

void report(const Where &c, const char *what, int64_t a, int64_t b, int64_t block, int lane) {
  ++g_fail;
  char key[160];
  snprintf(key, sizeof key, "%s %lld %lld %s", c.path, (long long)c.rows, (long long)c.cols, what);
  if (g_seen.insert(key).second && g_seen.size() <= 40)
    printf("FAIL %s [%lld, %lld] %s: %lld %lld (workgroup %lld lane %d)\n", c.path, (long long)c.rows,
           (long long)c.cols, what, (long long)a, (long long)b, (long long)block, lane);
}

// A load of w elements at idx.
inline void load(const Where &c, int64_t idx, int w, int64_t block, int lane) {
  ++g_checks;
  if (idx < 0 || idx + w > c.total) report(c, "load index, width", idx, w, block, lane);
}

// HIP's dispatch limits: a grid dimension of at most 2^32 - 1 work-items
// and 2^31 - 1 workgroups (stated here, not taken from the header).
void launch(const Where &c, int64_t blocks, int64_t threads) {
  ++g_launches;
  if (blocks < 1 || blocks > 0x7fffffffLL || blocks * threads > 0xffffffffLL)
    report(c, "launch blocks, threads", blocks, threads, -1, -1);
}

// Workgroups of a grid of nb to walk: all of a small grid, else the first
// and last 12 and 8 spread between.
std::vector<int64_t> visit(int64_t nb) {
  std::vector<int64_t> v;
  if (nb <= 32) {
    for (int64_t b = 0; b < nb; ++b) v.push_back(b);
    return v;
  }
  for (int64_t b = 0; b < 12; ++b) v.push_back(b);
  for (int64_t b = nb - 12; b < nb; ++b) v.push_back(b);
  for (int64_t i = 1; i <= 8; ++i) v.push_back(12 + (nb - 24) * i / 9);
  std::sort(v.begin(), v.end());
  v.erase(std::unique(v.begin(), v.end()), v.end());
  return v;
}

// ------------------------------------------------------------------ tiles

// The loads of load_tile<E, VEC, LOADP> for one lane (`lane` is the lane
// argument the kernel passes), as offsets from the tile's start.
template <class F>
void tile_loads(int E, bool vec, int loadp, int64_t len, int64_t avail, int lane, F &&f) {
  const int TILE = 64 * E, J = E / 4;
  const bool full = len >= TILE;
  const int lim = tile_lim(len, TILE);
  if (lim == 0) return;
  if (loadp == 2 && full && vec) {
    for (int k = 0; k < J; ++k) f(tile_index(false, true, E, lane, k), 4);
    return;
  }
  if (loadp == 1 || loadp == 2) {
    if (full || avail >= TILE) {
      for (int j = 0; j < J; ++j) {
        if (vec) f(tile_index(true, true, E, lane, j), 4);
        else
          for (int t = 0; t < 4; ++t) f(tile_index(true, false, E, lane, 4 * j + t), 1);
      }
    } else if (vec) {
      for (int j = 0; j < J; ++j) f(clamp_group(tile_index(true, true, E, lane, j), lim, 4), 4);
    } else {
      for (int i = 0; i < E; ++i) f(clamp_group(tile_index(true, false, E, lane, i), lim, 1), 1);
    }
  } else {
    if (vec && !full) {
      for (int k = 0; k < J; ++k) f(clamp_group(tile_index(false, true, E, lane, k), lim, 4), 4);
    } else if (full && vec) {
      for (int k = 0; k < J; ++k) f(tile_index(false, true, E, lane, k), 4);
    } else {
      for (int k = 0; k < E; ++k) {
        const int e = tile_index(false, false, E, lane, k);
        f(full ? e : clamp_group(e, lim, 1), 1);
      }
    }
  }
}

// k_var_rows (and its ablation variants): one launch over rows [r0, r0+nr).
void rows_launch(const Where &c, int64_t r0, int64_t nr, int64_t n, int64_t ld, int E, int W, bool vec, int loadp) {
  const int waves = rows_waves(n, E, W);
  launch(c, nr, 64 * waves);
  for (int64_t b : visit(nr)) {
    const int64_t row = b;  // also every permutation of the rows (xcd_contiguous)
    const int64_t p = (r0 + row) * ld;
    for (int w = 0; w < waves; ++w) {
      const int64_t base = (int64_t)w * 64 * E;
      for (int lane = 0; lane < 64; ++lane) {
        tile_loads(E, vec, loadp, n - base, rows_avail(nr, row, ld, n, base), vlane_pair32(lane),
                   [&](int64_t i, int wd) { load(c, p + base + i, wd, b, lane); });
        load(c, p, 1, b, lane);  // x0
      }
    }
  }
}

// k_var_rows_full: rows of exactly 64*E*W values.
void rows_full_launch(const Where &c, int64_t r0, int64_t nr, int64_t ld, int E, int W) {
  launch(c, nr, 64 * W);
  for (int64_t b : visit(nr)) {
    const int64_t p = (r0 + b) * ld;
    for (int w = 0; w < W; ++w)
      for (int lane = 0; lane < 64; ++lane) {
        for (int j = 0; j < E / 4; ++j) load(c, p + (int64_t)w * 64 * E + vlane_pair32(lane) * E + 4 * j, 4, b, lane);
        load(c, p, 1, b, lane);
      }
  }
}

// Rows in batches of at most g_items work-items (svh::in_batches; 2^32 - 1
// by default, lowered by the launch_items knob).
int64_t g_items = MAX_LAUNCH_ITEMS;
template <class F>
void batches(int64_t total, int64_t per_block, int64_t threads, F &&f) {
  const int64_t batch = (g_items / threads) * per_block;
  for (int64_t s0 = 0; s0 < total; s0 += batch) f(s0, std::min(batch, total - s0));
}

// The load path the row launchers pick for a plan (E, W) and var_load_path
// (0 coalesced + LDS transpose, 1 per lane, 2 coalesced + staged transpose):
// (E, W) of launch_rows_ew, the two 16-wave plans (per lane), or the rest
// (launch_rows_split).
int rows_loadp(int E, int W, bool vec, int vlp) {
  const bool ew = (E == 4 && W == 1) || (E == 16 && W == 1) || (E == 64 && W == 1) || (E == 64 && W == 4);
  if (ew) {
    if (E % 16 == 0 && vlp == 2) return vec ? 2 : 1;
    return vlp != 0 ? 1 : 0;
  }
  if (W == 16 && (E == 32 || E == 64)) return 1;
  if (!vec) return 1;
  if (vlp == 0) return 0;
  return vlp == 2 && E % 16 == 0 ? 2 : 1;
}

void rows_tile(const Where &c, int64_t rows, int64_t n, bool vec, int split, int vlp, bool full_rows) {
  const RowsPlan p = rows_plan(n, split);
  const int loadp = rows_loadp(p.E, p.W, vec, vlp);
  const bool full_kernel = vec && loadp == 1 && full_rows && n == 64LL * p.E * p.W;
  const int waves = full_kernel ? p.W : rows_waves(n, p.E, p.W);
  batches(rows, 1, 64 * waves, [&](int64_t r0, int64_t nr) {
    if (full_kernel) rows_full_launch(c, r0, nr, n, p.E, p.W);
    else rows_launch(c, r0, nr, n, n, p.E, p.W, vec, loadp);
  });
}

// k_var_rows_seg (cplx = 1) and k_var_rows_c64_seg (cplx = 2: complex values
// of two floats, loads of vw complex values).
void rows_seg(const Where &c, int64_t rows, int64_t n, int vw, int cplx) {
  const SegPlan sp = seg_plan(n);
  const int rpb = 4 * (64 / sp.S);
  batches(rows, rpb, 256, [&](int64_t r0, int64_t nr) {
    const int64_t nb = (nr + rpb - 1) / rpb;
    launch(c, nb, 256);
    const bool full = n == (int64_t)sp.S * sp.E;
    for (int64_t b : visit(nb))
      for (int w = 0; w < 4; ++w)
        for (int lane = 0; lane < 64; ++lane) {
          const int64_t row = seg_row(b, w, lane, sp.S);
          const int64_t p = cplx * (r0 + clamp_last(row, nr)) * n;
          const int64_t e0 = (int64_t)(lane % sp.S) * sp.E;
          for (int j = 0; j < sp.E / vw; ++j) {
            const int64_t e = e0 + (int64_t)vw * j;
            load(c, p + cplx * (full ? e : clamp_group(e, n, vw)), cplx * vw, b, lane);
          }
          load(c, p, cplx, b, lane);  // x0
        }
  });
}

// k_var_rows_c64: rows of n complex values, load_tile over 2*E floats.
void rows_c64(const Where &c, int64_t rows, int64_t n, bool vec) {
  const RowsPlan p = c64_rows_plan(n);
  const int waves = rows_waves(n, p.E, p.W);  // only the waves the row reaches
  batches(rows, 1, 64 * waves, [&](int64_t r0, int64_t nr) {
    launch(c, nr, 64 * waves);
    for (int64_t b : visit(nr)) {
      const int64_t pr = 2 * (r0 + b) * n;
      for (int w = 0; w < waves; ++w) {
        const int64_t base = (int64_t)w * 64 * p.E;
        for (int lane = 0; lane < 64; ++lane) {
          tile_loads(2 * p.E, vec, 1, 2 * (n - base), 2 * rows_avail(nr, b, n, n, base), lane,
                     [&](int64_t i, int wd) { load(c, pr + 2 * base + i, wd, b, lane); });
          load(c, pr, 2, b, lane);
        }
      }
    }
  });
}

// k_long_rows (both passes) and k_long_top.
void long_rows(const Where &c, int64_t rows, int64_t n, bool vec) {
  const int64_t nch = (n + LS_ROW_CHUNK - 1) / LS_ROW_CHUNK;
  const int64_t nb = rows * nch;
  launch(c, nb, 256);
  launch(c, rows, 256);
  for (int64_t b : visit(nb)) {
    const int64_t r = b / nch, ch = b % nch;
    for (int w = 0; w < 4; ++w) {
      const int64_t base = ch * LS_ROW_CHUNK + (int64_t)w * 64 * 64;
      for (int lane = 0; lane < 64; ++lane) {
        tile_loads(64, vec, 1, n - base, rows_avail(nb / nch, r, n, n, base), lane,
                   [&](int64_t i, int wd) { load(c, r * n + base + i, wd, b, lane); });
        load(c, r * n, 1, b, lane);
      }
    }
  }
  for (int64_t sl : visit(rows)) load(c, sl * n, 1, sl, 0);  // finalize's x0
}

// k_long_rows<PASS, VEC, 2> and k_long_top<PASS, K, 2>: rows of n pairs (two
// interleaved slices per row, row stride ld floats).
void long_pairs(const Where &c, int64_t rows, int64_t n, int64_t ld, bool vec) {
  const int64_t chunk = LS_ROW_CHUNK / 2, nch = (n + chunk - 1) / chunk;
  const int64_t nb = rows * nch;
  launch(c, nb, 256);
  launch(c, 2 * rows, 256);
  for (int64_t b : visit(nb)) {
    const int64_t r = b / nch, ch = b % nch;
    for (int w = 0; w < 4; ++w) {
      const int64_t base = ch * chunk + (int64_t)w * 64 * 32;
      for (int lane = 0; lane < 64; ++lane) {
        tile_loads(64, vec, 1, 2 * (n - base), 2 * rows_avail(nb / nch, r, ld / 2, n, base), lane,
                   [&](int64_t i, int wd) { load(c, r * ld + 2 * base + i, wd, b, lane); });
        load(c, r * ld, 2, b, lane);  // x0 of both slices
      }
    }
  }
  for (int64_t sl : visit(2 * rows)) load(c, (sl / 2) * ld + sl % 2, 1, sl, 0);  // finalize's x0
}

// ------------------------------------------------------------------ axis 0

// The V adjacent columns x rows of load_cols_tile<V, E, VEC16> and the x0
// loads of the column kernels (clamped: k_cols_one; not: k_cols_y, k_cols_dq).
void cols_tile(const Where &c, int64_t R, int64_t C, int64_t c0, int64_t r0, bool full, int V, int E, bool vec16,
               int64_t b, int lane) {
  const int64_t cc = cols_first(c0, C, V);
  for (int i = 0; i < E; ++i) {
    const int64_t r = full ? r0 + i : clamp_last(r0 + i, R);
    if (V > 1 && vec16) load(c, r * C + cc, V, b, lane);  // 16 bytes: four floats or two doubles
    else
      for (int k = 0; k < V; ++k) load(c, r * C + clamp_last(cc + k, C), 1, b, lane);
  }
}

// k_cols_one<V, W, G, VEC16, E, MODE> over `waves` waves.
// words: 4-byte words per element (the die pairing counts a block's width in
// words: 1 for float32, 2 for float64).
void cols_one(const Where &c, int64_t R, int64_t C, int V, int W, int G, bool vec16, int E, int mode, int64_t blocks,
              int waves, int words = 1) {
  batches(blocks, 1, 64 * waves, [&](int64_t, int64_t cnt) { launch(c, cnt, 64 * waves); });
  const int nc = V * (64 / G);
  if ((C + nc - 1) / nc != blocks) report(c, "column blocks", blocks, nc, -1, -1);
  for (int64_t b : visit(blocks)) {
    const int64_t cb = line_on_one_die<int>((int)b, (int)((C + nc - 1) / nc), words * nc);
    if (cb < 0 || cb >= blocks) report(c, "column block", cb, blocks, b, -1);
    for (int w = 0; w < waves; ++w)
      for (int lane = 0; lane < 64; ++lane) {
        const int q = lane / G, g = lane % G;
        const int64_t c0 = cb * nc + (int64_t)q * V;
        const int64_t rw = (int64_t)w * E * G, r0 = rw + (int64_t)g * E;
        const bool full = mode == 1 || r0 + E <= R;
        if (mode != 0 || rw < R) cols_tile(c, R, C, c0, r0, full, V, E, vec16, b, lane);
        const int64_t cc = cols_first(c0, C, V);
        for (int k = 0; k < V; ++k) load(c, clamp_last(cc + k, C), 1, b, lane);
      }
  }
  (void)W;
}

// k_cols_y and k_cols_dq (the chunked path; the workspace reads are clamped
// to the nch chunk nodes the workspace holds).
void cols_chunked(const Where &c, int64_t R, int64_t C, int V, int W, const ColsChunkPlan &p, int64_t ws_chunks,
                  int group) {
  const int nc = V * (64 / p.G);
  const int64_t nb = p.ncb * p.nch;
  batches(nb, 1, 64 * W, [&](int64_t, int64_t cnt) {
    launch(c, cnt, 64 * W);  // k_cols_y
    launch(c, cnt, 64 * W);  // k_cols_dq
  });
  // the top trees: 64/S columns per wave (S lanes per column) for at most
  // CC_GROUP chunks, else a wave per column
  const int pw = p.nch <= 4 ? 16 : p.nch <= 8 ? 8 : p.nch <= 16 ? 4 : p.nch <= group ? 2 : 1;
  batches((C + 4 * pw - 1) / (4 * pw), 1, 256, [&](int64_t, int64_t cnt) { launch(c, cnt, 256); });
  if (p.nch > ws_chunks) report(c, "chunks beyond the workspace", p.nch, ws_chunks, -1, -1);
  for (int64_t b : visit(nb)) {
    const int64_t cb = b / p.nch, j = b % p.nch;
    for (int w = 0; w < W; ++w)
      for (int lane = 0; lane < 64; ++lane) {
        const int q = lane / p.G, g = lane % p.G;
        const int64_t c0 = cb * nc + (int64_t)q * V;
        const int64_t rw = j * ((int64_t)CC_E * p.G * W) + (int64_t)w * (CC_E * p.G), r0 = rw + (int64_t)g * CC_E;
        cols_tile(c, R, C, c0, r0, r0 + CC_E <= R, V, CC_E, V > 1, b, lane);
        const int64_t cc = cols_first(c0, C, V);
        for (int k = 0; k < V; ++k) load(c, cc + k, 1, b, lane);
      }
  }
}

// k_var_cols: a lane per column.
void cols_lane(const Where &c, int64_t R, int64_t C, const RowsPlan &p) {
  const int64_t nb = (C + 63) / 64;
  batches(nb, 1, 64 * p.W, [&](int64_t, int64_t cnt) { launch(c, cnt, 64 * p.W); });
  for (int64_t b : visit(nb))
    for (int w = 0; w < p.W; ++w)
      for (int lane = 0; lane < 64; ++lane) {
        const int64_t col = b * 64 + lane, r0 = (int64_t)w * p.E;
        const bool full = r0 + p.E <= R, allcols = b * 64 + 64 <= C;
        for (int i = 0; i < p.E; ++i) {
          if (full && allcols) load(c, (r0 + i) * C + col, 1, b, lane);
          else load(c, clamp_last(r0 + i, R) * C + clamp_last(col, C), 1, b, lane);
        }
        load(c, clamp_last(col, C), 1, b, lane);
      }
}

// k_cols_short(_d): V columns per lane (four floats or two doubles, 16
// bytes), R < 16 rows.
void cols_short(const Where &c, int64_t R, int64_t C, int V) {
  const int E = cols_short_e(R);
  const int64_t nb = (C / V + 255) / 256;
  batches(nb, 1, 256, [&](int64_t, int64_t cnt) { launch(c, cnt, 256); });
  for (int64_t b : visit(nb))
    for (int t = 0; t < 256; ++t) {
      const int64_t c0 = (b * 256 + t) * V;
      if (c0 >= C) continue;
      for (int i = 0; i < E; ++i) load(c, clamp_last<int64_t>(i, R) * C + c0, V, b, t);
    }
}

// ------------------------------------------------------------------ routes

struct Knobs {
  RouteKnobs r;
  int split, loadp, full_rows;
  int cols_waves;
};

// off: the matrix's address modulo 16 bytes (0, 8 or 4).
void variance_f32(int64_t rows, int64_t cols, int axis, int off, const Knobs &k, bool fills) {
  const bool ax1 = axis == 1;
  const int64_t n = ax1 ? cols : rows;
  if (rows == 0 || cols == 0) return;
  const bool vec16 = off == 0 && cols % 4 == 0;
  const Route route = f32_route(rows, cols, ax1, vec16, k.r, fills);
  char name[64];
  snprintf(name, sizeof name, "f32 axis %d route %d", axis, (int)route);
  const Where c{name, rows, cols, rows * cols};
  switch (route) {
    case Route::LONG_ROWS_CHUNKED: long_rows(c, rows, n, vec16); break;
    case Route::ROWS_SEG: rows_seg(c, rows, n, seg_vw(off, cols), 1); break;
    case Route::ROWS_TILE: rows_tile(c, rows, n, vec16, k.split, k.loadp, k.full_rows); break;
    case Route::COLS_PAIRS: long_pairs(c, 1, rows, 2 * rows, off == 0 && rows % 2 == 0); break;
    case Route::COLS_ONE_READ: {
      const ColsLongPlan p = cols_long_plan(rows, cols);
      cols_one(c, rows, cols, 1, 16, 4, false, p.E, p.mode, p.blocks, p.waves);
      break;
    }
    case Route::COLS_CHUNKED: {
      const int V = vec16 ? 4 : 1;
      // cols_waves 0: the automatic choice on 256 CUs
      const int cw = k.cols_waves ? k.cols_waves : cols_chunk_waves(V, rows, cols, 256);
      cols_chunked(c, rows, cols, V, cw, cols_chunk_plan(V, cw, rows, cols),
                   (rows + CC_E * CC_MIN_W - 1) / (CC_E * CC_MIN_W), CC_GROUP);
      break;
    }
    case Route::COLS_SHORT: cols_short(c, rows, cols, 4); break;
    case Route::COLS_ONE4: {
      // mode 2 over the waves row R reaches (clamped loads in every wave)
      // for columns that fill at most 5/8 of the tile, else mode 0
      const ColsOnePlan p = cols_one4_plan(rows, cols);
      const bool sparse = cols_one4_masked(rows, p);
      const int reached = (int)((rows + (int64_t)CC_E * p.G - 1) / ((int64_t)CC_E * p.G));
      cols_one(c, rows, cols, 4, p.W, p.G, vec16, CC_E, sparse ? 2 : 0, p.blocks, sparse ? reached : p.W);
      break;
    }
    case Route::COLS_ONE1: {
      const ColsOnePlan p = cols_one1_plan(rows, cols);
      cols_one(c, rows, cols, 1, p.W, p.G, false, CC_E, 0, p.blocks, p.W);
      break;
    }
    case Route::COLS_LANE: cols_lane(c, rows, cols, cols_lane_plan(rows)); break;
  }
}

void variance_c64(int64_t rows, int64_t cols, int off, int short_rows) {
  if (rows == 0 || cols == 0) return;
  const Where c{"c64 axis 1", rows, cols, 2 * rows * cols};
  const bool vec = off == 0 && cols % 2 == 0;
  if (cols > C64_FUSED_MAX_N) {
    if ((cols + LS_ROW_CHUNK / 2 - 1) / (LS_ROW_CHUNK / 2) <= LS_MAX_CHUNKS) long_pairs(c, rows, cols, 2 * cols, vec);
    return;
  }
  if (cols <= SEG_MAX_N && short_rows) rows_seg(c, rows, cols, vec ? 2 : 1, 2);
  else rows_c64(c, rows, cols, vec);
}

// Rows of more than 16384 values take the long-row chunks; columns of more
// than 1024 rows are transposed (k_transpose: 32 x 32 tiles, 256 threads)
// into a 256-byte aligned workspace and reduced as rows.
void variant_f32(int64_t rows, int64_t cols, int axis, int off) {
  const Where c{"variant", rows, cols, rows * cols};
  if (axis == 1 && cols > ROWS_MAX_N) {
    long_rows(c, rows, cols, off == 0 && cols % 4 == 0);
    return;
  }
  if (axis == 0 && rows > COLS_MAX_R) {
    const int64_t tc = (cols + 31) / 32, tiles = ((rows + 31) / 32) * tc;
    batches(tiles, 1, 256, [&](int64_t b0, int64_t nb) {
      launch(c, nb, 256);
      for (int64_t b : visit(nb))
        for (int t = 0; t < 256; ++t)
          for (int k = 0; k < 32; k += 8) {
            const int64_t r = ((b0 + b) / tc) * 32 + (t >> 5) + k, col = ((b0 + b) % tc) * 32 + (t & 31);
            if (r < rows && col < cols) load(c, r * cols + col, 1, b, t);
          }
    });
    variant_f32(cols, rows, 1, 0);
    return;
  }
  if (axis == 1) {
    const RowsPlan p = variant_rows_plan(cols);
    const bool vec = off == 0 && cols % 4 == 0;
    batches(rows, 1, 64 * p.W, [&](int64_t r0, int64_t nr) { rows_launch(c, r0, nr, cols, cols, p.E, p.W, vec, 1); });
  } else {
    cols_lane(c, rows, cols, cols_lane_plan(rows));
  }
}

// k_long_rows_d<PASS, VEC, 2> and k_long_top_d<PASS, K, 2>: one row of n
// pairs of doubles (c in doubles, cf the same array in floats).
void long_pairs_d(const Where &c, const Where &cf, int64_t n, bool vec) {
  const int64_t chunk = L64_ROW_CHUNK / 2, nch = (n + chunk - 1) / chunk;
  launch(c, nch, 64 * L64_W);
  launch(c, 2, 256);
  for (int64_t b : visit(nch))
    for (int w = 0; w < L64_W; ++w) {
      const int64_t base = b * chunk + (int64_t)w * 64 * (L64_E / 2);
      for (int lane = 0; lane < 64; ++lane) {
        tile_loads(2 * L64_E, vec, 1, 4 * (n - base), 4 * rows_avail(1, 0, n, n, base), lane,
                   [&](int64_t i, int wd) { load(cf, 4 * base + i, wd, b, lane); });
        load(c, 0, 2, b, lane);  // x0 of both slices
      }
    }
  for (int64_t sl = 0; sl < 2; ++sl) load(c, sl, 1, sl, 0);  // finalize's x0
}

// The float64 variance (indices in doubles; the row tiles load floats, two
// per double).  off: the matrix's address modulo 16 bytes (0 or 8).
void variance_f64_route(int64_t rows, int64_t cols, int axis, int off, bool one_read, bool pairs,
                        bool long_rows = true, bool wide = false) {
  const bool ax1 = axis == 1;
  const int64_t n = ax1 ? cols : rows;
  if (rows == 0 || cols == 0) return;
  const bool vec = off == 0 && cols % 2 == 0;
  const Route64 route = f64_route(rows, cols, ax1, vec, one_read, pairs, long_rows);
  char name[64];
  snprintf(name, sizeof name, "f64 axis %d route %d", axis, (int)route);
  const Where c{name, rows, cols, rows * cols};
  const Where cf{name, rows, cols, 2 * rows * cols};  // the same array in floats
  switch (route) {
    case Route64::ROWS_SEG: rows_seg(c, rows, n, vec ? 2 : 1, 1); break;
    case Route64::ROWS_TILE: {
      const RowsPlan p = rows64_plan(n);
      const int waves = rows_waves(n, p.E, p.W);  // only the waves the row reaches
      batches(rows, 1, 64 * waves, [&](int64_t r0, int64_t nr) {
        launch(c, nr, 64 * waves);
        for (int64_t b : visit(nr)) {
          const int64_t pr = (r0 + b) * cols;
          for (int w = 0; w < waves; ++w) {
            const int64_t base = (int64_t)w * 64 * p.E;
            for (int lane = 0; lane < 64; ++lane) {
              tile_loads(2 * p.E, vec, 1, 2 * (n - base), 2 * rows_avail(nr, b, cols, n, base), vlane_pair32(lane),
                         [&](int64_t i, int wd) { load(cf, 2 * (pr + base) + i, wd, b, lane); });
              load(c, pr, 1, b, lane);
            }
          }
        }
      });
      break;
    }
    case Route64::LONG_ROWS_CHUNKED: {
      const int64_t nch = (n + L64_ROW_CHUNK - 1) / L64_ROW_CHUNK, nb = rows * nch;
      launch(c, nb, 64 * L64_W);
      launch(c, rows, 256);
      for (int64_t b : visit(nb)) {
        const int64_t r = b / nch, ch = b % nch;
        for (int w = 0; w < L64_W; ++w) {
          const int64_t base = ch * L64_ROW_CHUNK + (int64_t)w * 64 * L64_E;
          for (int lane = 0; lane < 64; ++lane) {
            tile_loads(2 * L64_E, vec, 1, 2 * (n - base), 2 * rows_avail(nb / nch, r, cols, n, base), lane,
                       [&](int64_t i, int wd) { load(cf, 2 * (r * cols + base) + i, wd, b, lane); });
            load(c, r * cols, 1, b, lane);
          }
        }
      }
      break;
    }
    case Route64::COLS_PAIRS: long_pairs_d(c, cf, rows, vec); break;
    case Route64::COLS_CHUNKED: {
      const int V = vec ? 2 : 1;
      cols_chunked(c, rows, cols, V, L64_W, cols_chunk64_plan(V, rows, cols), (rows + C64_CHUNK - 1) / C64_CHUNK,
                   C64_GROUP);
      break;
    }
    case Route64::COLS_ONE: {
      const ColsOne64Plan p = cols_one64_plan(rows, cols, vec, wide);
      cols_one(c, rows, cols, p.V, p.W, p.G, vec, L64_E, 0, p.blocks, p.W, 2);
      break;
    }
    case Route64::COLS_SHORT: cols_short(c, rows, cols, 2); break;
    case Route64::COLS_LANE: cols_lane(c, rows, cols, cols_lane64_plan(rows)); break;
  }
}

// Both launch choices of a candidate for the one-read columns (and the wide
// tile where it applies), of two columns (pairs or column chunks) and of
// rows of 16385..32768 doubles with 256 or more rows (one workgroup per row
// or chunks).
void variance_f64(int64_t rows, int64_t cols, int axis, int off) {
  variance_f64_route(rows, cols, axis, off, false, true);
  if (cols_one_read64_candidate(axis == 1, rows, cols, 2)) {
    variance_f64_route(rows, cols, axis, off, true, true);
    if (cols_one64_wide_ok(rows, off == 0 && cols % 2 == 0))
      variance_f64_route(rows, cols, axis, off, true, true, true, true);
  }
  if (axis == 0 && cols == 2) variance_f64_route(rows, cols, axis, off, false, false);
  if (axis == 1 && cols > V64_ROWS_MAX_N && cols <= V64_ROWS_ONE_MAX_N && rows >= V64_ROWS_ONE_MIN_ROWS)
    variance_f64_route(rows, cols, axis, off, false, true, false);
}

// k_var_kahan: a lane per slice, chunks of 64 values.
void kahan(int64_t rows, int64_t cols, int axis, int off) {
  const bool ax1 = axis == 1;
  const int64_t nsl = ax1 ? rows : cols, n = ax1 ? cols : rows, ld = cols;
  const bool vec = ax1 && off == 0 && cols % 4 == 0;
  const Where c{"kahan", rows, cols, rows * cols};
  const int64_t nb = (nsl + 63) / 64, nch = (n + KS_T - 1) / KS_T;
  launch(c, nb, 64);
  for (int64_t b : visit(nb)) {
    const int64_t s0 = b * 64;
    for (int lane = 0; lane < 64; ++lane) {
      const int64_t slc = clamp_last(s0 + lane, nsl);
      load(c, ax1 ? slc * ld : slc, 1, b, lane);
      for (int64_t ch0 = 0; ch0 < nch + 2; ++ch0) {
        const int64_t ch = clamp_last(ch0, nch);
        if (ax1) {
          for (int j = 0; j < 16; ++j) {
            const int64_t row = clamp_last(s0 + 4 * j + (lane >> 4), nsl);
            const int64_t col = ch * KS_T + 4 * (lane & 15);
            if (vec && col + 3 < n) load(c, row * ld + col, 4, b, lane);
            else
              for (int t = 0; t < 4; ++t) load(c, row * ld + clamp_last(col + t, n), 1, b, lane);
          }
        } else {
          for (int kk = 0; kk < KS_T; ++kk) load(c, clamp_last(ch * KS_T + kk, n) * ld + slc, 1, b, lane);
        }
        if (nch > 8 && ch0 == 2) ch0 = nch - 3;  // long slices: the first and last chunks
      }
    }
  }
}

// ------------------------------------------------------------------ tree sum

void tree_sum(int64_t n, int e, int64_t target, bool vec, int loadp, bool xcd) {
  if (n == 0) return;
  const SumPlan p = plan_sum(n, e, target, SUM_W, SUM_MAX_BLOCKS, SUM_MAX_LOG2_GROUP);
  const Where c{"tree sum", 1, n, n};
  launch(c, p.blocks, 64 * SUM_W);
  if (p.blocks > SUM_MAX_BLOCKS) report(c, "blocks above the workspace", p.blocks, SUM_MAX_BLOCKS, -1, -1);
  const int64_t size = 64LL * e, G = 1LL << p.log2_g;
  for (int64_t b : visit(p.blocks)) {
    const int64_t bid = xcd ? xcd_contiguous((int)b, (int)p.blocks) : b;
    for (int w = 0; w < SUM_W; ++w) {
      const int64_t c0 = (bid * SUM_W + w) * G;
      const bool run_full = (c0 + G) * size <= n;
      for (int64_t j = 0; j < G; ++j) {
        if (G > 8 && j == 4) j = G - 4;  // long runs: the first and last chunks
        const int64_t ch = c0 + j, len = n - ch * size;
        const int lim = tile_lim(len, (int)size);
        for (int lane = 0; lane < 64; ++lane) {
          if (run_full || lim == size) {
            if (vec)
              for (int k = 0; k < e / 4; ++k) load(c, ch * size + tile_index(loadp == 1, true, e, lane, k), 4, b, lane);
            else
              for (int i = 0; i < e; ++i) {
                const int idx = loadp == 1 ? tile_index(true, false, e, lane, i) : tile_index(false, false, e, lane, i);
                load(c, ch * size + idx, 1, b, lane);
              }
          } else if (lim > 0) {
            for (int i = 0; i < e; ++i) {
              const int raw = loadp == 1 ? tile_index(true, false, e, lane, i)
                              : vec      ? tile_index(false, true, e, lane, i / 4) + (i % 4)
                                         : tile_index(false, false, e, lane, i);
              load(c, ch * size + clamp_group(raw, lim, 1), 1, b, lane);
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ ADN sum

// k_adn_sum<K, E, VEC>: wave w of workgroup b streams chunks [c0, c1) of
// 64*e values (a whole chunk with e/4 16-byte loads or e single loads per
// lane, the ragged last one value by value below n); then the workgroup's
// record, its group's counter and record, and the top counter, all inside
// the workspace the size function gives (in 32-bit words).
void adn_sum(int64_t n, int e, int64_t target, bool vec) {
  if (n == 0) return;
  const AdnPlan p = adn_plan(n, e, target);
  const Where c{"adn sum", 1, n, n};
  launch(c, p.blocks, 64 * ADN_WAVES);
  if (p.blocks > target || p.blocks > ADN_MAX_BLOCKS) report(c, "blocks above the target", p.blocks, target, -1, -1);
  const int64_t ngroups = (p.blocks + ADN_GROUP - 1) / ADN_GROUP;
  if (ngroups > 128) report(c, "group records beyond two per lane", ngroups, 128, -1, -1);
  const int64_t header_words = ADN_WS_HEADER / 4, rec_words = (int64_t)ADN_MAX_BLOCKS * ADN_REC;
  const Where ws{"adn workspace", 1, header_words + rec_words + (ADN_MAX_BLOCKS / ADN_GROUP) * ADN_REC,
                 header_words + rec_words + (ADN_MAX_BLOCKS / ADN_GROUP) * ADN_REC};
  const int64_t size = 64LL * e;
  for (int64_t b : visit(p.blocks)) {
    const int64_t grp = b / ADN_GROUP;
    load(ws, header_words + b * ADN_REC, ADN_REC, b, 0);                        // the workgroup's record
    load(ws, (int64_t)ADN_COUNTER_STRIDE * (1 + grp), 1, b, 0);                 // its group's counter
    if (ADN_COUNTER_STRIDE * (1 + grp) >= header_words) report(ws, "group counter past the header", grp, 0, b, 0);
    load(ws, header_words + rec_words + grp * ADN_REC, ADN_REC, b, 0);          // its group's record
    for (int lane = 0; lane < 64; ++lane) {
      const int64_t idx = grp * ADN_GROUP + lane;  // the group's last workgroup reads these records
      if (idx < p.blocks) load(ws, header_words + idx * ADN_REC, ADN_REC, b, lane);
      for (int k = 0; k < 2; ++k)
        if (2 * lane + k < ngroups) load(ws, header_words + rec_words + (2 * lane + k) * ADN_REC, ADN_REC, b, lane);
    }
    for (int w = 0; w < ADN_WAVES; ++w) {
      const int64_t c0 = (b * ADN_WAVES + w) * p.g, c1 = std::min(c0 + p.g, p.chunks);
      for (int64_t ch = c0; ch < c1; ++ch) {
        if (c1 - c0 > 8 && ch == c0 + 4) ch = c1 - 4;  // long runs: the first and last chunks
        const int64_t base = ch * size;
        const bool whole = base + size <= n;
        for (int lane = 0; lane < 64; ++lane)
          for (int j = 0; j < e / 4; ++j) {
            if (whole && vec) {
              load(c, adn_index(base, lane, j, 0, true), 4, b, lane);
              continue;
            }
            for (int t = 0; t < 4; ++t) {
              const int64_t i = adn_index(base, lane, j, t, vec);
              if (whole || i < n) load(c, i, 1, b, lane);
            }
          }
      }
    }
  }
  load(ws, 0, 1, -1, 0);  // the top counter
}

}  // namespace

// The route the dispatchers take for shapes whose choice was decided by
// measurement (the launch geometry, never the result bits, depends on it).
void route_expectations() {
  const RouteKnobs k{1, 1, 1024, 1, 1, 1, 1};
  struct F32 {
    int64_t R, C;
    bool ax1, vec16, fills;
    Route want;
    const char *why;
  };
  const F32 f32[] = {
      {4096, 4096, true, true, false, Route::ROWS_TILE, "the headline rows"},
      {300, 50000, true, true, false, Route::ROWS_TILE, "long rows, 256+ of them: one workgroup each"},
      {100, 200000, true, true, false, Route::LONG_ROWS_CHUNKED, "rows above 65536 values"},
      {200, 20000, true, true, false, Route::LONG_ROWS_CHUNKED, "long rows, fewer than 256"},
      {100, 300, true, true, false, Route::ROWS_SEG, "short rows share waves"},
      {4096, 4096, false, true, true, Route::COLS_ONE_READ, "4096-row columns, the grid fills"},
      {3000, 4100, false, true, false, Route::COLS_CHUNKED, "the one-read grid would leave the chip idle"},
      {8000000, 2, false, true, false, Route::COLS_PAIRS, "two long columns: one row of pairs"},
      {1000, 20000, false, true, false, Route::COLS_ONE4, "16-byte loads, long columns of a wide matrix"},
      {1000, 20001, false, false, false, Route::COLS_ONE1, "odd width: one column per lane"},
      {300, 700, false, true, false, Route::COLS_ONE1, "short columns: one column per lane"},
      {10, 100000, false, true, false, Route::COLS_SHORT, "at most 15 rows"},
      {40, 1000, false, true, false, Route::COLS_LANE, "16..64 rows: a lane per column"},
  };
  for (const F32 &e : f32) {
    const Route got = f32_route(e.R, e.C, e.ax1, e.vec16, k, e.fills);
    if (got != e.want) {
      printf("FAIL route f32 [%lld, %lld] axis %d: %d, want %d (%s)\n", (long long)e.R, (long long)e.C, e.ax1 ? 1 : 0,
             (int)got, (int)e.want, e.why);
      ++g_fail;
    }
  }
  struct F64 {
    int64_t R, C;
    bool ax1, vec16, candidate;
    Route64 want;
    const char *why;
  };
  const F64 f64[] = {
      {4096, 4096, true, true, false, Route64::ROWS_TILE, "rows of up to 16384 doubles"},
      {300, 50000, true, true, false, Route64::LONG_ROWS_CHUNKED, "rows above 32768 doubles"},
      {4096, 4096, false, true, true, Route64::COLS_ONE, "4096-row columns read once (when the grid fills)"},
      {1025, 16384, false, true, false, Route64::COLS_CHUNKED, "1025 rows: the tile half padding"},
      {2560, 5000, false, true, true, Route64::COLS_ONE, "5/8 of a 4096-row tile"},
      {8000000, 2, false, true, false, Route64::COLS_PAIRS, "two long columns: one row of pairs"},
      {1000, 3001, false, false, false, Route64::COLS_ONE, "65..1024 rows: one launch"},
      {10, 100000, false, true, false, Route64::COLS_SHORT, "at most 15 rows"},
  };
  for (const F64 &e : f64) {
    const bool cand = cols_one_read64_candidate(e.ax1, e.R, e.C, 1);
    if (cand != e.candidate) {
      printf("FAIL one-read candidate f64 [%lld, %lld]: %d, want %d (%s)\n", (long long)e.R, (long long)e.C, cand,
             e.candidate, e.why);
      ++g_fail;
    }
    const Route64 got = f64_route(e.R, e.C, e.ax1, e.vec16, cand, true);
    if (got != e.want) {
      printf("FAIL route f64 [%lld, %lld] axis %d: %d, want %d (%s)\n", (long long)e.R, (long long)e.C, e.ax1 ? 1 : 0,
             (int)got, (int)e.want, e.why);
      ++g_fail;
    }
  }
  // float64 columns of 1025..4096 rows on 256 CUs: the one read when its
  // grid fills, and the wide 16-wave tile when its own grid does
  struct Fill64 {
    int64_t R, C;
    bool one_read, wide;
    const char *why;
  };
  const Fill64 fill64[] = {
      {4096, 4096, true, true, "two full rounds of 16-wave tiles"},
      {4096, 3000, true, false, "375 wide tiles: the second round half empty"},
      {4096, 1024, true, false, "128 wide tiles: half the CUs"},
      {2048, 8192, true, true, "512 tiles of sixteen columns"},
      {2048, 2002, true, false, "126 wide tiles"},
      {3000, 4100, true, false, "not a whole tile: no wide tile"},
      {4096, 2050, false, false, "513 and 257 tiles: the last round nearly empty"},
  };
  // float32 column chunks under var_cols_waves 0 on 256 CUs (16-byte loads)
  struct Waves {
    int64_t R, C;
    int want;
    const char *why;
  };
  const Waves waves[] = {
      {16384, 1024, 16, "256 workgroups of 16 waves: one full round"},
      {65536, 256, 16, "256 workgroups: one full round"},
      {20001, 1000, 8, "316 workgroups: the second round nearly empty"},
      {4097, 4097, 8, "289 workgroups"},
      {8000000, 8, 8, "two column groups: 32 row groups per wave"},
      {3200000, 20, 8, "five column groups: 8 row groups per wave"},
  };
  for (const Waves &e : waves) {
    const int got = cols_chunk_waves(4, e.R, e.C, 256);
    if (got != e.want) {
      printf("FAIL chunk waves [%lld, %lld]: %d, want %d (%s)\n", (long long)e.R, (long long)e.C, got, e.want, e.why);
      ++g_fail;
    }
  }
  for (const Fill64 &e : fill64) {
    const bool wide = cols_one64_wide_ok(e.R, true) && one_round_fill(cols_one64_plan(e.R, e.C, true, true).blocks, 256);
    const bool one = one_round_fill(cols_one64_plan(e.R, e.C, true).blocks, 256) || wide;
    if (one != e.one_read || wide != e.wide) {
      printf("FAIL fill f64 [%lld, %lld]: one read %d wide %d, want %d %d (%s)\n", (long long)e.R, (long long)e.C, one,
             wide, e.one_read, e.wide, e.why);
      ++g_fail;
    }
  }
}

int main() {
  route_expectations();
  // shapes: boundaries of every plan, ragged tails, odd widths
  const int64_t sizes[] = {1,    2,    3,    4,    5,    7,    8,    15,   16,   17,   31,   33,   63,    64,
                           65,   100,  127,  128,  129,  255,  256,  257,  300,  511,  512,  513,  777,   1000,
                           1023, 1024, 1025, 1500, 2047, 2048, 2049, 3000, 4095, 4096, 4097, 6000, 8191,  8192,
                           8193, 12345, 16383, 16384, 16385, 20000, 32768, 32769, 65535, 65536, 65537, 100003};
  const RouteKnobs dflt{1, 1, 1024, 1, 1, 1, 1};
  std::vector<Knobs> knobs;
  knobs.push_back({dflt, 0, 1, 1, 0});
  for (int split : {1, 2, 4, 8}) knobs.push_back({dflt, split, 1, 1, 16});
  for (int lp : {0, 2}) knobs.push_back({dflt, 0, lp, 1, 16});
  knobs.push_back({dflt, 0, 1, 0, 16});
  for (int cw : {4, 8, 16}) knobs.push_back({{1, 0, 1024, 1, 1, 1, 0}, 0, 1, 1, cw});
  knobs.push_back({{0, 1, 1024, 0, 0, 0, 1}, 0, 1, 1, 16});
  knobs.push_back({{1, 1, 1024, 1, 1, 2, 1}, 0, 1, 1, 16});
  knobs.push_back({{1, 1, 1024, 1, 1, 3, 1}, 0, 1, 1, 16});
  knobs.push_back({{1, 2, 1024, 1, 1, 1, 1}, 0, 1, 1, 16});
  knobs.push_back({{1, 1, 512, 1, 1, 1, 1}, 0, 1, 1, 16});
  knobs.push_back({{1, 1, 0, 1, 1, 1, 1}, 0, 1, 1, 16});

  // every shape in the default knobs, the knob variants on a subset
  const int64_t some[] = {1, 3, 16, 17, 64, 65, 257, 513, 1000, 1025, 2048, 3000, 4096, 4097, 16385, 65537};
  auto in_some = [&](int64_t v) { return std::find(std::begin(some), std::end(some), v) != std::end(some); };
  // The address offset (mod 16 bytes) only decides the load width: 16-byte
  // loads need 0, the short rows' 8-byte loads 8; 4 stands for the rest.
  for (int64_t R : sizes)
    for (int64_t C : sizes) {
      if (R * C > (1LL << 24)) continue;
      for (int axis : {0, 1}) {
        const int64_t n = axis == 1 ? C : R;
        if (axis == 1 && n > ROWS_MAX_N && (n + LS_ROW_CHUNK - 1) / LS_ROW_CHUNK > LS_MAX_CHUNKS) continue;
        const bool cand = cols_one_read_candidate(axis == 1, n, dflt);
        const bool seg = axis == 1 && n <= SEG_MAX_N;
        const size_t nk = in_some(R) && in_some(C) ? knobs.size() : 1;
        for (int off : {0, 8, 4}) {
          if (off == 8 && !seg) continue;
          for (size_t i = 0; i < nk; ++i)
            for (bool fills : {true, false})
              if (fills || cand || i > 0) variance_f32(R, C, axis, off, knobs[i], fills);
          if (off == 8 || (axis == 0 && off != 0)) continue;
          if (n <= LS_MAX_CHUNKS * LS_ROW_CHUNK) variant_f32(R, C, axis, off);
          if (n <= ((int64_t)KS_T << KS_LEVELS)) kahan(R, C, axis, off);
        }
      }
      for (int off : {0, 4})
        for (int sr : {0, 1}) variance_c64(R, C, off, sr);
      for (int axis : {0, 1}) {
        const int64_t n = axis == 1 ? C : R;
        if (axis == 1 && n > V64_ROWS_ONE_MAX_N && (n + L64_ROW_CHUNK - 1) / L64_ROW_CHUNK > L64_MAX_CHUNKS) continue;
        for (int off : {0, 8}) variance_f64(R, C, axis, off);
      }
    }
  for (int64_t n : {1LL, 5LL, 2047LL, 2048LL, 2049LL, 100000000LL, 100000003LL})
    for (int e : {16, 32})
      for (int64_t target : {1LL, 64LL, 8192LL})
        for (bool vec : {true, false})
          for (int lp : {0, 1})
            for (bool xcd : {false, true}) tree_sum(n, e, target, vec, lp, xcd);

  // the batched launches at the smallest launch_items knob (1024 work-items)
  g_items = 1024;
  for (int64_t R : {(int64_t)3, (int64_t)70, (int64_t)700, (int64_t)1500, (int64_t)2049, (int64_t)5000})
    for (int64_t C : {(int64_t)3, (int64_t)33, (int64_t)300, (int64_t)1030, (int64_t)17000})
      for (int axis : {0, 1}) {
        for (int off : {0, 8, 4})
          for (bool fills : {true, false}) variance_f32(R, C, axis, off, knobs[0], fills);
        variant_f32(R, C, axis, 0);
        for (int off : {0, 8}) variance_f64(R, C, axis, off);
        for (int off : {0, 4}) variance_c64(R, C, off, 1);
      }
  g_items = MAX_LAUNCH_ITEMS;

  // launch limits at the largest accepted shapes (no loads walked beyond the
  // sampled workgroups)
  for (int64_t C : sizes) {
    const int64_t R = VAR_MAX_ELEMS / C;
    if (R > 0x7fffffffLL && C > 0) continue;  // more slices than a grid holds: refused
    for (int axis : {0, 1}) {
      const int64_t n = axis == 1 ? C : R, nsl = axis == 1 ? R : C;
      if (nsl > 0x7fffffffLL) continue;
      if (axis == 1 && n > ROWS_MAX_N && (n + LS_ROW_CHUNK - 1) / LS_ROW_CHUNK > LS_MAX_CHUNKS) continue;
      if (axis == 0 && (n + 63) / 64 > ((int64_t)64 * 64 << (TOP_BIG_LEVELS - 1))) continue;
      for (const Knobs &k : knobs)
        for (bool fills : {true, false}) variance_f32(R, C, axis, 0, k, fills);
    }
  }
  for (int64_t R : sizes) {
    const int64_t C = VAR_MAX_ELEMS / R;
    for (int axis : {0, 1}) {
      const int64_t n = axis == 1 ? C : R, nsl = axis == 1 ? R : C;
      if (nsl > 0x7fffffffLL) continue;
      if (axis == 1 && n > ROWS_MAX_N && (n + LS_ROW_CHUNK - 1) / LS_ROW_CHUNK > LS_MAX_CHUNKS) continue;
      for (const Knobs &k : knobs)
        for (bool fills : {true, false}) variance_f32(R, C, axis, 0, k, fills);
    }
  }
  for (int e : {16, 32}) tree_sum(SUM_MAX_N, e, 8192, true, 0, false);
  for (int64_t C : sizes) {
    for (int64_t R : {V64_MAX_ELEMS / C, C > 0 ? V64_MAX_ELEMS / C : 0}) {
      for (int axis : {0, 1}) {
        const int64_t n = axis == 1 ? C : R, nsl = axis == 1 ? R : C;
        if (nsl > 0x7fffffffLL || R == 0) continue;
        if (axis == 1 && n > V64_ROWS_ONE_MAX_N && (n + L64_ROW_CHUNK - 1) / L64_ROW_CHUNK > L64_MAX_CHUNKS) continue;
        if (axis == 0 && (n + C64_CHUNK - 1) / C64_CHUNK > ((int64_t)64 * 64 << (TOP_BIG_LEVELS_D - 1))) continue;
        variance_f64(R, C, axis, 0);
        variance_f64(C, R, axis, 0);
      }
    }
  }
  // the ADN sum: the default and extreme workgroup targets, both load forms,
  // sizes around a chunk and up to the accumulator's capacity
  for (int64_t n : {(int64_t)1, (int64_t)1023, (int64_t)1024, (int64_t)1025, (int64_t)2049, (int64_t)100000000,
                    (int64_t)100000003, (int64_t)SV_ADN_MAX_COUNT})
    for (int e : {16, 32})
      for (int64_t target : {(int64_t)1, (int64_t)7, (int64_t)512, (int64_t)ADN_MAX_BLOCKS})
        for (bool vec : {true, false}) adn_sum(n, e, target, vec);

  // the float64 sum: chunks of 1024 doubles, i.e. the float chunks of 2048
  // of Chunk<32> over the same bytes (the same plan, in floats)
  for (int64_t n : {(int64_t)1, (int64_t)1023, (int64_t)1025, (int64_t)50000000, S64_MAX_N}) {
    const SumPlan pd = plan_sum(n, S64_EF / 2, S64_MAX_BLOCKS, S64_W, S64_MAX_BLOCKS, S64_MAX_LOG2_G);
    const SumPlan pf = plan_sum(2 * n, S64_EF, S64_MAX_BLOCKS, SUM_W, SUM_MAX_BLOCKS, SUM_MAX_LOG2_GROUP);
    if (pd.blocks != pf.blocks || pd.log2_g != pf.log2_g) printf("FAIL f64 sum plan %lld\n", (long long)n), ++g_fail;
    for (bool vec : {true, false}) tree_sum(2 * n, S64_EF, S64_MAX_BLOCKS, vec, 0, false);
  }

  printf("%lld loads and %lld launches checked, %lld failures\n", (long long)g_checks, (long long)g_launches,
         (long long)g_fail);
  return g_fail ? 1 : 0;
}
