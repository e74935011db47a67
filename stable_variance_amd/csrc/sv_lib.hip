// libstable_variance: compensated-tree float32 sum and variance on gfx950.
//
// Method: Pennacchio, "Variance in float32 with a first-element shift, a
// local centring and a compensated tree sum", §2 steps 1-4.  The C ABI is
// declared (and its contract stated) in include/stable_variance.h.
//
// Kernels
//   k_tree_sum   one workgroup per group of 2^g tiles of 64*E*W values; tile
//                nodes are combined in tree order, each group node is written
//                to the workspace, and the last workgroup to finish (a ticket
//                counter) combines the group nodes in tree order.
//   k_var_rows   axis 1: one workgroup per row; the W waves own consecutive
//                64*E ranges of the row, each lane E consecutive values (lane
//                L holds the range of virtual lane 2 (L mod 32) + L / 32, so
//                that the d and d^2 trees share their cross-lane levels).  The
//                row stays in registers between the two passes (y, then d and
//                d^2), so HBM is read once.
//   k_var_cols   axis 0: lanes own columns (coalesced across a row), waves own
//                consecutive blocks of E rows, so every tree level before the
//                cross-wave ones is in-lane.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "../../include/stable_variance.h"
#include "sv_device.hpp"
#include "sv_host.hpp"

using sv::Node;

// ------------------------------------------------------------------ shared host helpers

namespace svh {

thread_local char g_err[512];

sv_status fail(sv_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

sv_status ok() {
  g_err[0] = 0;
  return SV_OK;
}

sv_status check_device() {
  int cnt = 0;
  const hipError_t e = hipGetDeviceCount(&cnt);
  if (e != hipSuccess || cnt <= 0) return fail(SV_ERR_NO_DEVICE, "no HIP device available (%s)", hipGetErrorString(e));
  return SV_OK;
}

sv_status check_launch(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SV_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

const char *last_error() { return g_err; }

}  // namespace svh

using svh::check_device;
using svh::check_launch;
using svh::fail;
using svh::ok;
using svh::aligned16;

namespace {

// ------------------------------------------------------------------ device helpers

// Combine the wave nodes of the W waves of a workgroup (wave w covers the
// w-th consecutive range).  Every thread returns the workgroup's node.
template <int W, int KIND>
__device__ __forceinline__ Node block_tree(Node n, Node *slots, int w, int lane) {
  if constexpr (W == 1) {
    return n;
  } else {
    if (lane == 0) slots[w] = n;
    __syncthreads();
    Node nd[W];
#pragma unroll
    for (int i = 0; i < W; ++i) nd[i] = slots[i];
    __syncthreads();
    return sv::node_tree<0, W, W, KIND>(nd);
  }
}

// Variants of the slice computation (the ablation rows of the method page's
// §4, numbered as the C ABI's `variant`).  V_KERNEL is the method.
enum Variant {
  V_KERNEL = 0,           // shift + centring + two-term; plain tree of y, compensated trees of d and d^2
  V_COMP_Y = 1,           // the same with a compensated tree of y (the other reading of step 2)
  V_REFERENCE = 2,        // two-term formula: means as plain tree * fl(1/n), no shift
  V_NAIVE = 3,            // mean((x - mean(x))^2), means as plain tree * fl(1/n)
  V_SHIFT_PLAIN_NO2T = 4,
  V_SHIFT_PLAIN_2T = 5,
  V_NOSHIFT_COMP_2T = 6,
  V_SHIFT_COMP_NO2T = 7,
  V_SHIFT_KAHAN_NO2T = 8,  // shift + centring, Kahan sequential scan, no two-term (k_var_kahan)
};
template <int V>
struct VariantFlags {
  static constexpr bool shift = V == V_KERNEL || V == V_COMP_Y || V == V_SHIFT_PLAIN_NO2T || V == V_SHIFT_PLAIN_2T ||
                                V == V_SHIFT_COMP_NO2T;
  static constexpr bool comp = V == V_KERNEL || V == V_COMP_Y || V == V_NOSHIFT_COMP_2T || V == V_SHIFT_COMP_NO2T;
  static constexpr bool comp_y = V == V_COMP_Y;  // every other row keeps the kernel's plain tree of y
  static constexpr bool twoterm = V == V_KERNEL || V == V_COMP_Y || V == V_REFERENCE || V == V_SHIFT_PLAIN_2T ||
                                  V == V_NOSHIFT_COMP_2T;
  static constexpr bool recip = V == V_REFERENCE || V == V_NAIVE;
  static constexpr int ykind = comp_y ? sv::NODE_TWOSUM : sv::NODE_PLAIN;
  static constexpr int yleaf = comp_y ? sv::LEAF_FAST : sv::LEAF_PLAIN;
};

// The value of a slice sum: the compensated tree's root, or the plain tree's
// (the s part of the same nodes, formed as in a plain pairwise tree, and its
// root rule fl(s + 0)).
template <bool COMP>
__device__ __forceinline__ float tree_value(Node n) {
  return COMP ? sv::root_value(n) : sv::root_value_k<sv::NODE_PLAIN>(n);
}

// m from the slice sum of y: a division by fl(n), or the product with
// fl(1/n) for the formulae whose means are tree * fl(1/n).
template <int V>
__device__ __forceinline__ float local_mean(Node ny, int64_t n) {
  using F = VariantFlags<V>;
  const float sy = sv::root_value_k<F::ykind>(ny);
  const float fn = (float)n;
  if constexpr (F::recip) {
    const float inv = 1.0f / fn;
    return sy * inv;
  } else {
    return sy / fn;
  }
}

__device__ __forceinline__ float max0_nan(float v) { return (v != v) ? v : ((v > 0.0f) ? v : 0.0f); }

__device__ __forceinline__ float ddof_rescale(float v, int64_t n, int64_t ddof) {
  if (ddof == 0) return v;
  int64_t den = n - ddof;
  if (den < 0) den = 0;
  const float f = (float)n / (float)den;
  return v * f;
}

// Step 4 of a variant (see finalize for the method itself).
template <int V>
__device__ __forceinline__ void finalize_v(Node nd, Node nq, float x0, float m, int64_t n, int64_t ddof,
                                           float *var_out, float *mean_out) {
  using F = VariantFlags<V>;
  const float fn = (float)n;
  const float s1 = tree_value<F::comp>(nd);
  const float s2 = tree_value<F::comp>(nq);
  float v;
  if constexpr (F::recip) {
    const float inv = 1.0f / fn;
    const float a = s2 * inv;
    if constexpr (F::twoterm) {
      const float b = s1 * inv;
      const float bb = b * b;
      v = max0_nan(a - bb);
    } else {
      v = a;
    }
  } else {
    const float a = s2 / fn;
    if constexpr (F::twoterm) {
      const float b = s1 / fn;
      const float bb = b * b;
      v = max0_nan(a - bb);
    } else {
      v = max0_nan(a);
    }
  }
  *var_out = ddof_rescale(v, n, ddof);
  if (mean_out) *mean_out = F::shift ? x0 + m : m;
}

// Step 4 of the method: two-term correction, NaN-propagating max with 0,
// ddof rescale, and the mean x0 + m.
__device__ __forceinline__ void finalize(Node nd, Node nq, float x0, float m, int64_t n, int64_t ddof,
                                         float *var_out, float *mean_out) {
  const float fn = (float)n;
  const float s1 = sv::root_value(nd);
  const float s2 = sv::root_value(nq);
  const float a = s2 / fn;
  const float b = s1 / fn;
  const float bb = b * b;
  float v = a - bb;
  v = (v != v) ? v : ((v > 0.0f) ? v : 0.0f);
  if (ddof != 0) {
    int64_t den = n - ddof;
    if (den < 0) den = 0;
    const float f = fn / (float)den;
    v = v * f;
  }
  *var_out = v;
  if (mean_out) *mean_out = x0 + m;
}

// Per-call constants of step 2 and step 4, formed on the host.  When fl(n)
// is a power of two, x / fl(n) and x * rn with rn = 1 / fl(n) (exact) are the
// same rounding of the same real number, so the kernels multiply; dfac is
// the ddof factor fl(fl(n) / fl(max(n - ddof, 0))), a correctly rounded
// division on the host as it would be on the device.
struct StepConsts {
  float fn;    // fl(n)
  float rn;    // 1 / fl(n) when fl(n) is a power of two, else 0 (divide)
  float dfac;  // the ddof factor (unused when ddof == 0)
  int ddof_on; // ddof != 0
};

__device__ __forceinline__ float div_n(float a, const StepConsts &k) { return k.rn != 0.0f ? a * k.rn : a / k.fn; }

// Step 4 from the roots of the d and d^2 trees: the two-term correction,
// the NaN-propagating max with 0, the ddof rescale and the mean x0 + m.
__device__ __forceinline__ void finalize_k(Node nd, Node nq, float x0, float m, const StepConsts &k, float *var_out,
                                           float *mean_out) {
  const float a = div_n(sv::root_value(nq), k);
  const float b = div_n(sv::root_value(nd), k);
  const float bb = b * b;
  float v = a - bb;
  v = (v != v) ? v : ((v > 0.0f) ? v : 0.0f);
  if (k.ddof_on) v = v * k.dfac;
  *var_out = v;
  if (mean_out) *mean_out = x0 + m;
}


__device__ __forceinline__ void store_node_agent(Node *dst, Node v) {
  sv::store_u32_agent(reinterpret_cast<unsigned *>(&dst->s), __builtin_bit_cast(unsigned, v.s));
  sv::store_u32_agent(reinterpret_cast<unsigned *>(&dst->c), __builtin_bit_cast(unsigned, v.c));
}

using sv::wait_vmem_stores;

__device__ __forceinline__ Node load_node_agent(const Node *src) {
  const unsigned s = sv::load_u32_agent(reinterpret_cast<const unsigned *>(&src->s));
  const unsigned c = sv::load_u32_agent(reinterpret_cast<const unsigned *>(&src->c));
  return {__builtin_bit_cast(float, s), __builtin_bit_cast(float, c)};
}

// ------------------------------------------------------------------ tree sum

using svx::SUM_W;                // waves per workgroup
using svx::SUM_MAX_BLOCKS;       // workgroups of one tree-sum launch
using svx::SUM_MAX_LOG2_GROUP;   // chunks per wave <= 2^16
constexpr int SUM_GROUP = 64;                       // workgroups per first-level ticket
static_assert(SV_TREE_SUM_COUNTER_BYTES == 256 * (1 + SUM_MAX_BLOCKS / SUM_GROUP), "header constant");
constexpr int SUM_COUNTER_STRIDE = 64;              // counters 256 bytes apart
// counters: the top one, then one per group of SUM_GROUP workgroups
constexpr size_t SUM_WS_HEADER = 256 * (1 + SUM_MAX_BLOCKS / SUM_GROUP);

// Each wave streams its own run of G = 2^log2_g consecutive chunks of 64*E
// values (chunks beyond n are zero nodes), reducing chunk j while the loads
// of chunk j+1 are in flight, and combines the chunk nodes in tree order
// with a binary-counter stack.  The W wave nodes of a workgroup are
// consecutive, so their tree is the workgroup's group node; it goes to the
// workspace and the last workgroup to take a ticket reduces the group nodes.
#ifndef SV_SUM_MINW
#define SV_SUM_MINW 1
#endif
template <int E, int W, bool VEC, int LOADP, bool NT, int D, int KIND = sv::NODE_TWOSUM>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(SV_SUM_MINW, 8))) void k_tree_sum(const float *__restrict__ x, int64_t n, int log2_g,
                                                     Node *__restrict__ part, unsigned *__restrict__ counter,
                                                     float *__restrict__ out, int xcd) {
  using C = sv::Chunk<E, VEC, LOADP, NT>;
  constexpr int LPW = (LOADP == 0) ? sv::lds_floats_per_wave<E>() : 1;
  __shared__ float lds[W * LPW];
  __shared__ Node wstack[W][SUM_MAX_LOG2_GROUP + 1];
  __shared__ Node slots[W];
  __shared__ unsigned is_last;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int64_t G = 1LL << log2_g;
  const int nb = (int)gridDim.x;
  const int bid = xcd ? sv::xcd_contiguous((int)blockIdx.x, nb) : (int)blockIdx.x;  // logical workgroup
  const int64_t c0 = ((int64_t)bid * W + w) * G;  // first chunk of this wave
  float *const my_lds = lds + w * LPW;
  Node *const st = wstack[w];
  int sp = 0;  // meaningful in lane 0

  auto reduce_chunk = [&](const float (&raw)[E], int64_t j) {
    float v[E];
    C::finish(raw, my_lds, lane, v);
    Node nd = sv::lane_tree<KIND == sv::NODE_DW ? sv::LEAF_DW : sv::LEAF_CANON, 0, E, E>(v);
    nd = sv::wave_tree<KIND>(nd);
    if (lane == 0) {
      for (int64_t k = j; k & 1; k >>= 1) nd = sv::combine_k<KIND>(st[--sp], nd);
      st[sp++] = nd;
    }
  };
  auto chunk_ptr = [&](int64_t c) { return x + c * C::SIZE; };
  auto chunk_len = [&](int64_t c) { return n - c * C::SIZE; };

  // Ring of D register buffers: chunk j is reduced while chunks j+1 .. j+D-1
  // are loading.  G is a power of two; runs shorter than D use a smaller ring.
  auto stream = [&](auto depth) {
    constexpr int DD = decltype(depth)::value;
    float r[DD][E];
#pragma unroll
    for (int u = 0; u < DD - 1; ++u) C::issue(chunk_ptr(c0 + u), chunk_len(c0 + u), lane, r[u]);
    for (int64_t j = 0; j < G; j += DD) {
#pragma unroll
      for (int u = 0; u < DD; ++u) {
        const int64_t ahead = j + u + DD - 1;
        if (ahead < G) C::issue(chunk_ptr(c0 + ahead), chunk_len(c0 + ahead), lane, r[(u + DD - 1) % DD]);
        reduce_chunk(r[u], j + u);
      }
    }
  };
  // The same ring for a run whose chunks all lie inside the data (every
  // wave but the last): the loads are issued without any branch around them
  // (the steady loop, then a last block with no issue), so the compiler
  // waits only for the chunk being reduced.  A load behind a branch makes it
  // wait for every outstanding load, the prefetched chunks included.
  auto stream_full = [&](auto depth) {
    constexpr int DD = decltype(depth)::value;
    float r[DD][E];
    if (G == DD) {  // the whole run in flight at once
#pragma unroll
      for (int u = 0; u < DD; ++u) C::issue_full(chunk_ptr(c0 + u), lane, r[u]);
#pragma unroll
      for (int u = 0; u < DD; ++u) reduce_chunk(r[u], u);
      return;
    }
#pragma unroll
    for (int u = 0; u < DD - 1; ++u) C::issue_full(chunk_ptr(c0 + u), lane, r[u]);
    int64_t j = 0;
    for (; j + DD < G; j += DD) {
#pragma unroll
      for (int u = 0; u < DD; ++u) {
        C::issue_full(chunk_ptr(c0 + j + u + DD - 1), lane, r[(u + DD - 1) % DD]);
        reduce_chunk(r[u], j + u);
      }
    }
#pragma unroll
    for (int u = 0; u < DD; ++u) {
      if (u == 0) C::issue_full(chunk_ptr(c0 + j + DD - 1), lane, r[DD - 1]);  // the run's last chunk
      reduce_chunk(r[u], j + u);
    }
  };
  const bool run_full = (c0 + G) * C::SIZE <= n;  // wave-uniform
  if (run_full) {
    if (G >= D) stream_full(std::integral_constant<int, D>{});
    else if (G >= 2) stream_full(std::integral_constant<int, 2>{});
    else stream_full(std::integral_constant<int, 1>{});
  } else {
    if (G >= D) stream(std::integral_constant<int, D>{});
    else if (G >= 2) stream(std::integral_constant<int, 2>{});
    else stream(std::integral_constant<int, 1>{});
  }
  if (lane == 0) slots[w] = st[0];
  __syncthreads();

  // Two-level ticket.  Workgroups are grouped by SUM_GROUP consecutive
  // indices; each publishes its node and takes a ticket on its group's
  // counter; the last of a group reduces the group's nodes (an aligned run,
  // so a node of the same tree) and takes a ticket on the top counter; the
  // last group reduces the group nodes and writes the result.  Separate
  // counters keep the same-address atomics to SUM_GROUP per counter instead
  // of one per workgroup on a single address.
  //
  // Nodes are written with device-coherent (agent scope) stores and read
  // with device-coherent loads, so no cache writeback or invalidation is
  // needed; waiting for the stores' completion (vmcnt 0) before the ticket
  // increment orders the two.  An agent-scope release fence would instead
  // write back the whole L2 of the XCD for every workgroup.
  const int grp = bid / SUM_GROUP;
  const int ngroups = (nb + SUM_GROUP - 1) / SUM_GROUP;
  const int in_group = (grp == ngroups - 1) ? nb - grp * SUM_GROUP : SUM_GROUP;
  unsigned *const top_counter = counter;
  unsigned *const grp_counter = counter + SUM_COUNTER_STRIDE * (1 + grp);
  Node *const grp_nodes = part + SUM_MAX_BLOCKS;
  if (threadIdx.x == 0) {
    Node nd[W];
#pragma unroll
    for (int i = 0; i < W; ++i) nd[i] = slots[i];
    store_node_agent(part + bid, sv::node_tree<0, W, W, KIND>(nd));
    wait_vmem_stores();
    const unsigned ticket = __hip_atomic_fetch_add(grp_counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (ticket == (unsigned)in_group - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!is_last || w != 0) return;

  // Last workgroup of its group (wave 0): tree over the group's SUM_GROUP
  // block nodes (one per lane, zero past the grid).
  {
    const int idx = grp * SUM_GROUP + lane;
    Node g = (idx < nb) ? load_node_agent(part + idx) : sv::zero_node();
    g = sv::wave_tree<KIND>(g);
    unsigned top_ticket = 0;
    if (lane == 0) {
      __hip_atomic_store(grp_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      store_node_agent(grp_nodes + grp, g);
      wait_vmem_stores();
      top_ticket = __hip_atomic_fetch_add(top_counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    top_ticket = __shfl(top_ticket, 0, 64);
    if (top_ticket != (unsigned)ngroups - 1) return;
  }

  // Last group: tree over the ngroups group nodes (GPL consecutive ones per
  // lane), padded with zeros to SUM_MAX_BLOCKS / SUM_GROUP.
  constexpr int GPL = SUM_MAX_BLOCKS / SUM_GROUP / 64;
  static_assert(GPL >= 1 && (GPL & (GPL - 1)) == 0, "group nodes per lane: a power of two");
  Node t[GPL];
#pragma unroll
  for (int k = 0; k < GPL; ++k) {
    const int idx = GPL * lane + k;
    t[k] = (idx < ngroups) ? load_node_agent(grp_nodes + idx) : sv::zero_node();
  }
  Node r = sv::wave_tree<KIND>(sv::node_tree<0, GPL, GPL, KIND>(t));
  if (lane == 0) {
    out[0] = sv::root_value(r);
    __hip_atomic_store(top_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------------ complex64

// Complex data as two float32 arrays (Pennacchio, "Variance in float32 ...",
// §2: the real and imaginary parts are split and their variances added).
// Row r of a [rows, cols] complex64 array (interleaved re, im) becomes rows
// 2r (re) and 2r+1 (im) of a [2*rows, cols] float32 array.
// Rows stride by gridDim.y and columns by gridDim.x * 256 (no integer
// division in the index arithmetic).
__global__ __launch_bounds__(256) void k_split_rows(const float *__restrict__ z, int64_t rows, int64_t cols,
                                                    float *__restrict__ out) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const float2 *__restrict__ zr = reinterpret_cast<const float2 *>(z) + r * cols;
    float *__restrict__ re = out + (2 * r) * cols;
    float *__restrict__ im = re + cols;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < cols; c += (int64_t)gridDim.x * 256) {
      const float2 v = zr[c];
      re[c] = v.x;
      im[c] = v.y;
    }
  }
}

// Axis 1 in one pass: a row of n complex values is read once (8 bytes per
// value), each lane holding E consecutive values, split in registers into
// its real and imaginary parts; the two float32 variances run side by side
// with the same tree topology as k_var_rows, and var = fl(var(re) +
// var(im)), mean = (mean(re), mean(im)).  W waves own consecutive 64*E
// ranges; the launch holds only the waves the row reaches (svx::rows_waves),
// the tree's other wave nodes are +0.
template <int E, int W, bool VEC>
__global__ __launch_bounds__(64 * W) void k_var_rows_c64(const float *__restrict__ z, int64_t n, int64_t ddof,
                                                         float *__restrict__ var_out, float *__restrict__ mean_out) {
  __shared__ Node slots[6][W];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = blockIdx.x;
  const float *__restrict__ p = z + 2 * row * n;
  const int64_t base = (int64_t)w * 64 * E;  // first complex value of this wave
  const bool empty = base >= n;
  float f[2 * E];
  const int64_t avail = 2 * svx::rows_avail(gridDim.x, row, n, n, base);  // floats to the launch's last row
  sv::load_tile<2 * E, VEC, 1, false>(p + 2 * base, 2 * (n - base), nullptr, f, lane, avail);
  const float x0r = p[0], x0i = p[1];
  const bool full = base + 64 * E <= n;
  const int64_t left = n - base - (int64_t)lane * E;
  const int valid = left < 0 ? 0 : (left > E ? E : (int)left);
  float re[E], im[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    re[i] = (full || i < valid) ? f[2 * i] - x0r : 0.0f;
    im[i] = (full || i < valid) ? f[2 * i + 1] - x0i : 0.0f;
  }
  Node yr = sv::zero_node(), yi = sv::zero_node();
  if (!empty) {
    yr = sv::wave_tree<sv::Y_KIND>(sv::lane_tree<sv::Y_LEAF, 0, E, E>(re));
    yi = sv::wave_tree<sv::Y_KIND>(sv::lane_tree<sv::Y_LEAF, 0, E, E>(im));
  }
  // The tree over the waves' nodes: lane l < W takes wave l's real node,
  // lane W + l its imaginary node, and the first log2(W) cross-lane levels
  // pair them in tree order (one node per lane instead of all W in every
  // lane's registers); waves not launched give zero nodes.
  const int nw = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));
  const bool launched = (lane & (W - 1)) < nw;
  if constexpr (W > 1) {
    if (lane == 0) {
      slots[0][w] = yr;
      slots[1][w] = yi;
    }
    __syncthreads();
    const Node t = sv::seg_tree<sv::Y_KIND, W>(lane < 2 * W && launched ? (&slots[0][0])[lane] : sv::zero_node());
    yr = {sv::readlane_f(t.s, 0), sv::readlane_f(t.c, 0)};
    yi = {sv::readlane_f(t.s, W), sv::readlane_f(t.c, W)};
  }
  const float mr = sv::root_value_k<sv::Y_KIND>(yr) / (float)n;
  const float mi = sv::root_value_k<sv::Y_KIND>(yi) / (float)n;
  Node dr = sv::zero_node(), qr = sv::zero_node(), di = sv::zero_node(), qi = sv::zero_node();
  if (!empty) {
    if (full) {
      sv::lane_tree_dq<false, 0, E, E>(re, mr, E, dr, qr);
      sv::lane_tree_dq<false, 0, E, E>(im, mi, E, di, qi);
    } else {
      sv::lane_tree_dq<true, 0, E, E>(re, mr, valid, dr, qr);
      sv::lane_tree_dq<true, 0, E, E>(im, mi, valid, di, qi);
    }
    dr = sv::wave_tree<sv::NODE_TWOSUM>(dr);
    qr = sv::wave_tree<sv::NODE_NN>(qr);
    di = sv::wave_tree<sv::NODE_TWOSUM>(di);
    qi = sv::wave_tree<sv::NODE_NN>(qi);
  }
  // Wave 0 alone: lanes [k*W, (k+1)*W) take the waves' nodes of tree k (d
  // and d^2 of the real part, then of the imaginary part).  The d^2 trees
  // take the TwoSum node here: on non-negative operands its error is the
  // same exact value as the Fast2Sum form's.
  if constexpr (W > 1) {
    static_assert(4 * W <= 64, "four trees of W nodes in one wave");
    if (lane == 0) {
      slots[2][w] = dr;
      slots[3][w] = qr;
      slots[4][w] = di;
      slots[5][w] = qi;
    }
    __syncthreads();
    if (w != 0) return;
    const Node t =
        sv::seg_tree<sv::NODE_TWOSUM, W>(lane < 4 * W && launched ? (&slots[2][0])[lane] : sv::zero_node());
    dr = {sv::readlane_f(t.s, 0), sv::readlane_f(t.c, 0)};
    qr = {sv::readlane_f(t.s, W), sv::readlane_f(t.c, W)};
    di = {sv::readlane_f(t.s, 2 * W), sv::readlane_f(t.c, 2 * W)};
    qi = {sv::readlane_f(t.s, 3 * W), sv::readlane_f(t.c, 3 * W)};
  }
  if (threadIdx.x == 0) {
    float vr, vi, mean_r, mean_i;
    finalize(dr, qr, x0r, mr, n, ddof, &vr, &mean_r);
    finalize(di, qi, x0i, mi, n, ddof, &vi, &mean_i);
    var_out[row] = vr + vi;
    if (mean_out) {
      mean_out[2 * row] = mean_r;
      mean_out[2 * row + 1] = mean_i;
    }
  }
}

// Short complex rows (n <= 512): 64/S rows per wave, row k on lanes
// [k*S, (k+1)*S), each lane E consecutive complex values, split in registers
// as in k_var_rows_c64; the in-lane levels and the first log2(S) cross-lane
// levels per part.  VW2 = 2 complex values per 16-byte load (16-byte aligned
// rows of an even count), else one (8 bytes); every load issued, clamped and
// masked.
template <int E, int S, int VW2>
__global__ __launch_bounds__(256) void k_var_rows_c64_seg(const float *__restrict__ z, int64_t rows, int64_t n,
                                                          StepConsts k, float *__restrict__ var_out,
                                                          float *__restrict__ mean_out) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = lane % S;
  const int64_t row = svx::seg_row(blockIdx.x, w, lane, S);
  const bool rowok = row < rows;
  const float *__restrict__ p = z + 2 * svx::clamp_last(row, rows) * n;
  const bool full = (n == (int64_t)S * E);
  const int64_t e0 = (int64_t)l * E;
  const int64_t left = n - e0;
  const int valid = left < 0 ? 0 : (left > E ? E : (int)left);
  float re[E], im[E];
  if constexpr (VW2 == 2) {
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
      const int64_t e = e0 + 2 * j;
      const float4 g = *reinterpret_cast<const float4 *>(p + 2 * (full ? e : svx::clamp_group(e, n, 2)));
      re[2 * j] = g.x; im[2 * j] = g.y; re[2 * j + 1] = g.z; im[2 * j + 1] = g.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int64_t e = e0 + i;
      const float2 g = *reinterpret_cast<const float2 *>(p + 2 * (full ? e : svx::clamp_group(e, n, 1)));
      re[i] = g.x; im[i] = g.y;
    }
  }
  const float x0r = p[0], x0i = p[1];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    re[i] = (full || i < valid) ? re[i] - x0r : 0.0f;
    im[i] = (full || i < valid) ? im[i] - x0i : 0.0f;
  }
  const Node yr = sv::seg_tree<sv::Y_KIND, S>(sv::lane_tree<sv::Y_LEAF, 0, E, E>(re));
  const Node yi = sv::seg_tree<sv::Y_KIND, S>(sv::lane_tree<sv::Y_LEAF, 0, E, E>(im));
  const float mr = div_n(sv::root_value_k<sv::Y_KIND>(yr), k);
  const float mi = div_n(sv::root_value_k<sv::Y_KIND>(yi), k);
  Node dr, qr, di, qi;
  if (full) {
    sv::lane_tree_dq<false, 0, E, E>(re, mr, E, dr, qr);
    sv::lane_tree_dq<false, 0, E, E>(im, mi, E, di, qi);
  } else {
    sv::lane_tree_dq<true, 0, E, E>(re, mr, valid, dr, qr);
    sv::lane_tree_dq<true, 0, E, E>(im, mi, valid, di, qi);
  }
  dr = sv::seg_tree<sv::NODE_TWOSUM, S>(dr);
  qr = sv::seg_tree<sv::NODE_NN, S>(qr);
  di = sv::seg_tree<sv::NODE_TWOSUM, S>(di);
  qi = sv::seg_tree<sv::NODE_NN, S>(qi);
  if (l == 0 && rowok) {
    float vr, vi, mean_r, mean_i;
    finalize_k(dr, qr, x0r, mr, k, &vr, &mean_r);
    finalize_k(di, qi, x0i, mi, k, &vi, &mean_i);
    var_out[row] = vr + vi;
    if (mean_out) {
      mean_out[2 * row] = mean_r;
      mean_out[2 * row + 1] = mean_i;
    }
  }
}

// var[j] = fl(v[2j] + v[2j+1]): the variance of the real part plus that of
// the imaginary part.
__global__ __launch_bounds__(256) void k_pair_add(const float *__restrict__ v, int64_t count, float *__restrict__ out) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < count) out[j] = v[2 * j] + v[2 * j + 1];
}

// ------------------------------------------------------------------ measurement aid

// Plain streaming read of n floats (non-temporal 16-byte loads, 4 per lane,
// one 4 KiB block per workgroup).  It computes nothing of the method: the
// loaded values are folded into a float that is stored only when it equals
// a value no finite input produces, so the loads cannot be removed.  Used to
// measure the practical HBM read ceiling next to the reduction kernels.
__global__ __launch_bounds__(256) void k_stream_read(const float *__restrict__ x, int64_t n, float *__restrict__ out) {
  const int64_t base = ((int64_t)blockIdx.x * 256 * 4 + threadIdx.x) * 4;
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t e = base + (int64_t)k * 1024;
    if (e + 4 <= n) {
      const float4 g = sv::ld4<true>(x + e);
      acc += (g.x + g.y) + (g.z + g.w);
    } else {
      for (int t = 0; t < 4; ++t)
        if (e + t < n) acc += x[e + t];
    }
  }
  if (__builtin_bit_cast(unsigned, acc) == 0x7f800001u) out[0] = acc;  // a NaN payload, never the sum of finite data
}

__global__ void k_fill(float *__restrict__ out, int64_t count, float value) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) out[i] = value;
}

// ------------------------------------------------------------------ variance, axis 1

// Axis 1, rows that fill their power-of-two tile exactly (n = 64*E*W) and
// start 16 bytes aligned: every wave is full, so there are no masks, clamped
// loads or empty waves.  Lane L holds the E consecutive values of virtual
// lane 2 (L mod 32) + L / 32 of its wave's range (the order in which the d
// and d^2 trees share their cross-lane levels); the row stays in registers
// from the y pass to the d pass, so HBM is read once.
template <int E, int W>
__global__ __launch_bounds__(64 * W) void k_var_rows_full(const float *__restrict__ x, int64_t ld, StepConsts k,
                                                          float *__restrict__ var_out, float *__restrict__ mean_out) {
  static_assert(E % 4 == 0 && W >= 1 && W <= 16, "tile of whole 16-byte groups, at most 16 waves");
  __shared__ float ys[W];
  __shared__ Node dqs[2][W];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = blockIdx.x;
  const float *__restrict__ p = x + row * ld;
  const float *__restrict__ src = p + w * (64 * E) + sv::vlane_pair32(lane) * E;
  float v[E];
#pragma unroll
  for (int j = 0; j < E / 4; ++j) {
    const float4 g = *reinterpret_cast<const float4 *>(src + 4 * j);
    v[4 * j] = g.x; v[4 * j + 1] = g.y; v[4 * j + 2] = g.z; v[4 * j + 3] = g.w;
  }
  const float x0 = p[0];

  // step 1: y = x - x0
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = v[i] - x0;

  // step 2: the plain tree of y, m = Sy / n
  float sy = sv::wave_tree_p32<sv::Y_KIND>(sv::lane_tree<sv::Y_LEAF, 0, E, E>(v)).s;
  if constexpr (W > 1) {
    if (lane == 0) ys[w] = sy;
    __syncthreads();
    Node t[W];
#pragma unroll
    for (int i = 0; i < W; ++i) t[i] = {ys[i], 0.0f};
    sy = sv::node_tree<0, W, W, sv::Y_KIND>(t).s;
  }
  const float m = div_n(sy, k);

  // step 3: Tree(d), Tree(d^2); lanes 0..31 end with the wave's d node,
  // lanes 32..63 with its d^2 node
  Node nd, nq;
  sv::lane_tree_dq<false, 0, E, E>(v, m, E, nd, nq);
  const Node ndq = sv::wave_tree_dq(nd, nq);
  nd = {sv::readlane_f(ndq.s, 0), sv::readlane_f(ndq.c, 0)};
  nq = {sv::readlane_f(ndq.s, 32), sv::readlane_f(ndq.c, 32)};
  if constexpr (W > 1) {
    if (lane == 0) {
      dqs[0][w] = nd;
      dqs[1][w] = nq;
    }
    __syncthreads();
    if (w != 0) return;
    if constexpr (W >= 4) {
      // lanes [0, W) the d nodes, [W, 2W) the d^2 nodes, and the first
      // log2(W) cross-lane levels (TwoSum nodes: on non-negative operands
      // the same exact error as the Fast2Sum form)
      const Node t = sv::seg_tree<sv::NODE_TWOSUM, W>(lane < 2 * W ? (&dqs[0][0])[lane] : sv::zero_node());
      nd = {sv::readlane_f(t.s, 0), sv::readlane_f(t.c, 0)};
      nq = {sv::readlane_f(t.s, W), sv::readlane_f(t.c, W)};
    } else {
      Node td[W], tq[W];
#pragma unroll
      for (int i = 0; i < W; ++i) {
        td[i] = dqs[0][i];
        tq[i] = dqs[1][i];
      }
      nd = sv::node_tree<0, W, W>(td);
      nq = sv::node_tree<0, W, W, sv::NODE_NN>(tq);
    }
  }

  // step 4
  if (lane == 0) finalize_k(nd, nq, x0, m, k, var_out + row, mean_out ? mean_out + row : nullptr);
}

template <int E, int W, bool VEC, int LOADP, bool NT, int V = V_KERNEL>
__global__ __launch_bounds__(64 * W) void k_var_rows(const float *__restrict__ x, int64_t n, int64_t ld, int64_t ddof,
                                                     float *__restrict__ var_out, float *__restrict__ mean_out,
                                                     int xcd) {
  using F = VariantFlags<V>;
  constexpr int LPW = (LOADP == 0) ? sv::lds_floats_per_wave<E>() : (LOADP == 2) ? sv::lds_floats_staged<E>() : 1;
  __shared__ float lds[W * LPW];
  __shared__ Node slots[3][W];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int vl = sv::vlane_pair32(lane);  // this lane holds the range of virtual lane vl
  const int64_t row = xcd ? sv::xcd_contiguous((int)blockIdx.x, (int)gridDim.x) : (int)blockIdx.x;
  const float *__restrict__ p = x + row * ld;
  const int64_t base = (int64_t)w * 64 * E;

  // A wave whose range lies wholly beyond the row holds only padding: its
  // nodes are (+0, +0), which is what its trees would compute, so it skips
  // them (the branch is wave-uniform).
  const bool empty = base >= n;
  float v[E];
  const int64_t avail = svx::rows_avail(gridDim.x, row, ld, n, base);  // to the launch's last row
  sv::load_tile<E, VEC, LOADP, NT>(p + base, n - base, lds + w * LPW, v, vl, avail);
  const float x0 = p[0];

  // step 1: shift by the first element (padding stays +0)
  const bool full = base + 64 * E <= n;
  int64_t left = n - base - (int64_t)vl * E;
  const int valid = left < 0 ? 0 : (left > E ? E : (int)left);
  if constexpr (F::shift) {
    if (full) {
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = v[i] - x0;
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = (i < valid) ? v[i] - x0 : 0.0f;
    }
  }

  // step 2: m = (the tree of y) / n: the plain tree (the compensated one in V_COMP_Y)
  Node ny = sv::zero_node();
  if (!empty) {
    ny = sv::lane_tree<F::yleaf, 0, E, E>(v);
    ny = sv::wave_tree_p32<F::ykind>(ny);
  }
  // The launch may hold fewer than W waves (the ones the row reaches); the
  // tree's other wave nodes are (+0, +0).
  // From four waves on, the tree over the wave nodes takes one node per lane
  // (lane l < W wave l's) and the first log2(W) cross-lane levels, instead
  // of all W nodes in every lane's registers.
  const int nw = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));
  if constexpr (W > 1) {
    if (lane == 0) slots[0][w] = ny;
    __syncthreads();
    if constexpr (W >= 4) {
      const Node t = sv::seg_tree<F::ykind, W>(lane < nw ? slots[0][lane] : sv::zero_node());
      ny = {sv::readlane_f(t.s, 0), sv::readlane_f(t.c, 0)};
    } else {
      Node t[W];
#pragma unroll
      for (int i = 0; i < W; ++i) t[i] = i < nw ? slots[0][i] : sv::zero_node();
      ny = sv::node_tree<0, W, W, F::ykind>(t);
    }
  }
  const float m = local_mean<V>(ny, n);

  // step 3: Tree(d), Tree(d^2): lanes 0..31 end with the wave's d node,
  // lanes 32..63 with its d^2 node
  Node nd = sv::zero_node(), nq = sv::zero_node();
  if (!empty) {
    if (full) sv::lane_tree_dq<false, 0, E, E>(v, m, E, nd, nq);
    else sv::lane_tree_dq<true, 0, E, E>(v, m, valid, nd, nq);
    const Node ndq = sv::wave_tree_dq(nd, nq);
    nd = {sv::readlane_f(ndq.s, 0), sv::readlane_f(ndq.c, 0)};
    nq = {sv::readlane_f(ndq.s, 32), sv::readlane_f(ndq.c, 32)};
  }
  if constexpr (W > 1) {
    // one LDS round for both trees (their slots are not reused: no second barrier)
    if (lane == 0) {
      slots[1][w] = nd;
      slots[2][w] = nq;
    }
    __syncthreads();
    if constexpr (W >= 4) {
      // wave 0: lanes [0, W) the d nodes, [W, 2W) the d^2 nodes; the d^2
      // tree takes the TwoSum node, whose error on non-negative operands is
      // the same exact value as the Fast2Sum form's
      if (w != 0) return;
      const int i = lane & (W - 1);
      const Node t = sv::seg_tree<sv::NODE_TWOSUM, W>(lane < 2 * W && i < nw ? (&slots[1][0])[lane] : sv::zero_node());
      nd = {sv::readlane_f(t.s, 0), sv::readlane_f(t.c, 0)};
      nq = {sv::readlane_f(t.s, W), sv::readlane_f(t.c, W)};
    } else {
      if (threadIdx.x != 0) return;
      Node td[W], tq[W];
#pragma unroll
      for (int i = 0; i < W; ++i) {
        td[i] = i < nw ? slots[1][i] : sv::zero_node();
        tq[i] = i < nw ? slots[2][i] : sv::zero_node();
      }
      nd = sv::node_tree<0, W, W>(td);
      nq = sv::node_tree<0, W, W, sv::NODE_NN>(tq);
    }
  }

  // step 4
  if (threadIdx.x == 0) {
    if constexpr (V == V_KERNEL) finalize(nd, nq, x0, m, n, ddof, var_out + row, mean_out ? mean_out + row : nullptr);
    else finalize_v<V>(nd, nq, x0, m, n, ddof, var_out + row, mean_out ? mean_out + row : nullptr);
  }
}

// Axis 1, short rows (n <= 512): a wave holds 64/S rows, row k on lanes
// [k*S, (k+1)*S), each lane E consecutive values of its row, so that no lane
// idles on a row much shorter than the wave.  The row's tree is the in-lane
// levels and then the first log2(S) cross-lane levels (S*E is a power of two
// >= n; the values past n are +0).  Four waves per workgroup, independent.
// The divisions by fl(n) and the ddof factor come from the per-call
// constants (k): multiplies by the exact reciprocal when fl(n) is a power of
// two, where a row of a few values would otherwise spend most of its
// instructions in division sequences.
template <int E, int S, int VW>
__global__ __launch_bounds__(256) void k_var_rows_seg(const float *__restrict__ x, int64_t rows, int64_t n,
                                                      int64_t ld, StepConsts k, float *__restrict__ var_out,
                                                      float *__restrict__ mean_out) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = lane % S;
  const int64_t row = svx::seg_row(blockIdx.x, w, lane, S);  // 64/S rows per wave
  const bool rowok = row < rows;
  const float *__restrict__ p = x + svx::clamp_last(row, rows) * ld;  // past the last row: read it again
  const bool full = (n == (int64_t)S * E);                           // uniform
  const int64_t e0 = (int64_t)l * E;
  const int64_t left = n - e0;
  const int valid = left < 0 ? 0 : (left > E ? E : (int)left);

  // Loads of VW floats (16 or 8 bytes, or single floats): every one issued;
  // an index past the row reads its last values (n is a multiple of VW, so
  // a group is wholly inside the row or wholly past it).
  float v[E];
  if constexpr (VW == 4) {
#pragma unroll
    for (int j = 0; j < E / 4; ++j) {
      const int64_t e = e0 + 4 * j;
      const float4 g = *reinterpret_cast<const float4 *>(p + (full ? e : svx::clamp_group(e, n, 4)));
      v[4 * j] = g.x; v[4 * j + 1] = g.y; v[4 * j + 2] = g.z; v[4 * j + 3] = g.w;
    }
  } else if constexpr (VW == 2) {
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
      const int64_t e = e0 + 2 * j;
      const float2 g = *reinterpret_cast<const float2 *>(p + (full ? e : svx::clamp_group(e, n, 2)));
      v[2 * j] = g.x; v[2 * j + 1] = g.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int64_t e = e0 + i;
      v[i] = p[full ? e : svx::clamp_group(e, n, 1)];
    }
  }
  const float x0 = p[0];
  if (full) {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = v[i] - x0;
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = (i < valid) ? v[i] - x0 : 0.0f;
  }
  Node ny = sv::seg_tree<sv::Y_KIND, S>(sv::lane_tree<sv::Y_LEAF, 0, E, E>(v));
  const float m = div_n(sv::root_value_k<sv::Y_KIND>(ny), k);
  Node nd, nq;
  if (full) sv::lane_tree_dq<false, 0, E, E>(v, m, E, nd, nq);
  else sv::lane_tree_dq<true, 0, E, E>(v, m, valid, nd, nq);
  nd = sv::seg_tree<sv::NODE_TWOSUM, S>(nd);
  nq = sv::seg_tree<sv::NODE_NN, S>(nq);
  if (l == 0 && rowok) finalize_k(nd, nq, x0, m, k, var_out + row, mean_out ? mean_out + row : nullptr);
}

// ------------------------------------------------------------------ variance, axis 0

template <int E, int W, int V = V_KERNEL>
__global__ __launch_bounds__(64 * W) void k_var_cols(const float *__restrict__ x, int64_t R, int64_t C, int64_t ddof,
                                                     float *__restrict__ var_out, float *__restrict__ mean_out,
                                                     int64_t b0) {
  using F = VariantFlags<V>;
  __shared__ Node sy[W][64];
  __shared__ Node sd[W][64];
  __shared__ Node sq[W][64];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t blk = b0 + blockIdx.x;  // launches of at most 2^32 - 1 work-items
  const int64_t col = blk * 64 + lane;
  const bool colok = col < C;
  const int64_t r0 = (int64_t)w * E;

  // Loads: for a fixed row the 64 lanes read 64 consecutive floats.  Out of
  // range rows/columns read a clamped in-range address and are replaced by 0.
  const bool full = r0 + E <= R;
  const bool allcols = blk * 64 + 64 <= C;
  const int64_t ccol = svx::clamp_last(col, C);
  float v[E];
  if (full && allcols) {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = x[(r0 + i) * C + col];
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int64_t r = r0 + i;
      const float t = x[svx::clamp_last(r, R) * C + ccol];
      v[i] = (colok && r < R) ? t : 0.0f;
    }
  }
  const float x0 = x[ccol];

  int64_t vl = R - r0;
  const int valid = vl < 0 ? 0 : (vl > E ? E : (int)vl);
  if constexpr (F::shift) {
    if (full) {
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = v[i] - x0;
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = (i < valid) ? v[i] - x0 : 0.0f;
    }
  }

  Node ny = sv::lane_tree<F::yleaf, 0, E, E>(v);
  sy[w][lane] = ny;
  __syncthreads();
  {
    Node nn[W];
#pragma unroll
    for (int i = 0; i < W; ++i) nn[i] = sy[i][lane];
    ny = sv::node_tree<0, W, W, F::ykind>(nn);
  }
  const float m = local_mean<V>(ny, R);

  Node nd, nq;
  if (full) sv::lane_tree_dq<false, 0, E, E>(v, m, E, nd, nq);
  else sv::lane_tree_dq<true, 0, E, E>(v, m, valid, nd, nq);
  sd[w][lane] = nd;
  sq[w][lane] = nq;
  __syncthreads();
  if (w == 0 && colok) {
    Node a[W], b[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      a[i] = sd[i][lane];
      b[i] = sq[i][lane];
    }
#pragma unroll
    for (int len = W; len > 1; len >>= 1)
#pragma unroll
      for (int k = 0; k < len / 2; ++k) {
        a[k] = sv::combine(a[2 * k], a[2 * k + 1]);
        b[k] = sv::combine_nn(b[2 * k], b[2 * k + 1]);
      }
    if constexpr (V == V_KERNEL) finalize(a[0], b[0], x0, m, R, ddof, var_out + col, mean_out ? mean_out + col : nullptr);
    else finalize_v<V>(a[0], b[0], x0, m, R, ddof, var_out + col, mean_out ? mean_out + col : nullptr);
  }
}

// ------------------------------------------------------------------ variance, axis 0, chunked

// Axis 0 with the column's rows cut into chunks of CH = E*W rows (aligned
// nodes of the column's tree).  A workgroup owns one chunk of a block of
// 64*V adjacent columns: lane L holds columns [V*L, V*L + V) of the block (one
// 16-byte load per row when V = 4, so a wave reads 1 KiB of each row) for the
// E consecutive rows of its wave, and wave w owns rows [w*E, (w+1)*E) of the
// chunk.  Three or four launches, ordered by the stream (each reads what the
// previous ones wrote; the workspace is scratch):
//   k_cols_y    the y-tree node of every (chunk, column)
//   m           per column m = Plain(y)/n, the tree over its chunk nodes: for
//               at most 32 chunks per column each k_cols_dq workgroup forms
//               the m of its own columns (no launch); else a wave per column
//               (k_cols_top up to 4096 chunks, k_cols_top_big beyond)
//   k_cols_dq   the tile read again (mostly from the chip's last-level cache
//               when the input fits in it): the d- and d^2-tree node of
//               every (chunk, column)
//   step 4      per column the trees over its d and d^2 chunk nodes: a group
//               of lanes (up to 32 chunks) or a wave per column (k_cols_top,
//               k_cols_top_big)

using svx::CC_E;                     // rows per lane in a chunk
using svx::CC_MIN_W;                 // the workspace is sized for the shortest chunk
using svx::CC_GROUP;                 // chunk nodes per column that k_cols_dq reduces for m itself

struct ColsWs {
  Node *ny;  // [nch][C] y-tree node of each chunk of each column
  Node *nd;  // [nch][C] d-tree nodes
  Node *nq;  // [nch][C] d^2-tree nodes
  float *m;  // [C]
};

// Loads rows [r0, r0 + E) of the V columns starting at c0 (c0 a multiple of
// V).  Columns past C read the last in-range columns instead (their results
// are never written); rows past R read row R-1 (masked to +0 afterwards).
// VEC16: one 16-byte load per row when V = 4 (base and width allow it);
// else V 4-byte loads, which read the same cache lines.
template <int V, int E, bool VEC16 = true>
__device__ __forceinline__ void load_cols_tile(const float *__restrict__ x, int64_t R, int64_t C, int64_t c0,
                                               int64_t r0, bool full, float (&v)[V][E]) {
  const int64_t cc = svx::cols_first(c0, C, V);
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int64_t r = full ? r0 + i : svx::clamp_last(r0 + i, R);
    const float *p = x + r * C + cc;
    if constexpr (V == 4 && VEC16) {
      const float4 g = *reinterpret_cast<const float4 *>(p);
      v[0][i] = g.x;
      v[1][i] = g.y;
      v[2][i] = g.z;
      v[3][i] = g.w;
    } else {
      // columns past C (a partial last group of an odd width) read the last
      // column instead; their results are never written
#pragma unroll
      for (int k = 0; k < V; ++k) v[k][i] = x[r * C + svx::clamp_last(cc + k, C)];
    }
  }
}

// Step 1 on a tile: y = x - x0, and +0 for rows past the slice.
template <int V, int E>
__device__ __forceinline__ void shift_cols_tile(float (&v)[V][E], const float (&x0)[V], bool full, int valid) {
#pragma unroll
  for (int k = 0; k < V; ++k)
#pragma unroll
    for (int i = 0; i < E; ++i) v[k][i] = (full || i < valid) ? v[k][i] - x0[k] : 0.0f;
}

// G row groups per wave: lane L = q*G + g holds the V adjacent columns of
// column group q (Q = 64/G groups, V*Q columns per block) for the E rows
// [g*E, (g+1)*E) of the wave's G*E rows; the wave's node of a column is the
// in-lane levels and then the first log2(G) cross-lane levels (lanes of one
// column group are adjacent).  G = 1 for blocks of 64*V columns; narrow
// matrices take G up to 64 so that no lane idles.  Chunks of W*G*E rows.
template <int V, int W, int G>
__global__ __launch_bounds__(64 * W) void k_cols_y(const float *__restrict__ x, int64_t R, int64_t C, int64_t nch,
                                                   ColsWs ws, int64_t b0) {
  constexpr int E = CC_E, Q = 64 / G, NC = V * Q;
  static_assert(64 * W >= NC, "one thread per column of the block");
  __shared__ Node s[W][V][Q];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane / G, g = lane % G;
  const int64_t blk = b0 + blockIdx.x;  // launches of at most 2^32 - 1 work-items
  const int64_t cb = blk / nch, j = blk % nch;
  const int64_t c0 = cb * NC + (int64_t)q * V;
  const int64_t rw = j * ((int64_t)E * G * W) + (int64_t)w * (E * G);  // the wave's first row
  const int64_t r0 = rw + (int64_t)g * E;
  const bool full = r0 + E <= R;
  const bool wave_full = rw + (int64_t)E * G <= R;  // uniform
  const int64_t left = R - r0;
  const int valid = left < 0 ? 0 : (left > E ? E : (int)left);

  float v[V][E];
  load_cols_tile<V, E>(x, R, C, c0, r0, full, v);
  float x0[V];
  const int64_t cc = svx::cols_first(c0, C, V);
#pragma unroll
  for (int k = 0; k < V; ++k) x0[k] = x[cc + k];
  shift_cols_tile<V, E>(v, x0, wave_full, valid);
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const Node nd = sv::seg_tree<sv::Y_KIND, G>(sv::lane_tree<sv::Y_LEAF, 0, E, E>(v[k]));
    if (g == 0) s[w][k][q] = nd;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < NC) {
    const int k = t / Q, qq = t % Q;  // thread t combines column V*qq + k of the block
    const int64_t col = cb * NC + (int64_t)qq * V + k;
    if (col < C) {
      Node nn[W];
#pragma unroll
      for (int i = 0; i < W; ++i) nn[i] = s[i][k][qq];
      ws.ny[j * C + col] = sv::node_tree<0, W, W, sv::Y_KIND>(nn);
    }
  }
}

// Tree of the local mean over the nch <= CC_GROUP y chunk nodes p[0],
// p[stride], ... (one group, nothing written back).
__device__ __forceinline__ Node chunk_tree_1(const Node *p, int64_t stride, int64_t nch) {
  Node sub[CC_GROUP / 8];
#pragma unroll
  for (int b = 0; b < CC_GROUP / 8; ++b) {
    Node nd[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t idx = b * 8 + k;
      const Node t = p[svx::clamp_last(idx, nch) * stride];
      nd[k] = idx < nch ? t : sv::zero_node();
    }
    sub[b] = sv::node_tree<0, 8, 8, sv::Y_KIND>(nd);
  }
  return sv::node_tree<0, CC_GROUP / 8, CC_GROUP / 8, sv::Y_KIND>(sub);
}

// The per-column trees over the chunk nodes with S lanes per column (64/S
// columns per wave, four waves per workgroup): lane l of a column's group
// takes nodes [l*K, (l+1)*K) (zero nodes past nch), the in-lane levels and
// then the first log2(S) cross-lane levels give the tree of the column's
// chunks padded to S*K nodes.  PASS 0: m; PASS 1: step 4.
template <int PASS, int K, int S>
__global__ __launch_bounds__(256) void k_cols_top(const float *__restrict__ x, int64_t R, int64_t C, int64_t nch,
                                                  int64_t ddof, ColsWs ws, float *__restrict__ var_out,
                                                  float *__restrict__ mean_out, int64_t b0) {
  constexpr int PW = 64 / S;
  const int lane = threadIdx.x & 63;
  const int64_t col0 = ((b0 + blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * PW;
  if (col0 >= C) return;  // the whole wave
  const int64_t col = col0 + lane / S;
  const int sl = lane % S;
  const bool colok = col < C;
  const int64_t cc = svx::clamp_last(col, C);
  auto tree = [&](const Node *p, auto kind) {
    constexpr int KIND = decltype(kind)::value;
    Node nd[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t idx = (int64_t)sl * K + k;
      const Node t = p[svx::clamp_last(idx, nch) * C];  // every load issued
      nd[k] = idx < nch ? t : sv::zero_node();
    }
    return sv::seg_tree<KIND, S>(sv::node_tree<0, K, K, KIND>(nd));
  };
  if constexpr (PASS == 0) {
    const Node ny = tree(ws.ny + cc, std::integral_constant<int, sv::Y_KIND>{});
    if (sl == 0 && colok) ws.m[col] = sv::root_value_k<sv::Y_KIND>(ny) / (float)R;
  } else {
    const Node nd = tree(ws.nd + cc, std::integral_constant<int, sv::NODE_TWOSUM>{});
    const Node nq = tree(ws.nq + cc, std::integral_constant<int, sv::NODE_NN>{});
    if (sl == 0 && colok)
      finalize(nd, nq, x[col], ws.m[col], R, ddof, var_out + col, mean_out ? mean_out + col : nullptr);
  }
}

// The per-column trees over more than 4096 chunk nodes, a wave per column:
// lane l reduces the run of 64*P nodes [l*64*P, (l+1)*64*P) (P = 2^log2p,
// zero nodes past nch) in batches of 64, merging the batch nodes in tree
// order with a binary counter (the loop is wave-uniform, so every stack
// index is a constant), then the wave's six levels.  PASS 0: m; PASS 1:
// step 4.
using svx::TOP_BIG_LEVELS;  // P up to 2^15: 2^27 chunks per column
template <int PASS>
__global__ __launch_bounds__(256) void k_cols_top_big(const float *__restrict__ x, int64_t R, int64_t C,
                                                      int64_t nch, int log2p, int64_t ddof, ColsWs ws,
                                                      float *__restrict__ var_out, float *__restrict__ mean_out,
                                                      int64_t b0) {
  constexpr int K = 64;
  const int lane = threadIdx.x & 63;
  const int64_t col = (b0 + blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (col >= C) return;  // the whole wave
  const int64_t P = (int64_t)1 << log2p;
  auto tree = [&](const Node *p, auto kind) {
    constexpr int KIND = decltype(kind)::value;
    Node st[TOP_BIG_LEVELS];
#pragma unroll
    for (int lv = 0; lv < TOP_BIG_LEVELS; ++lv) st[lv] = sv::zero_node();
    for (int64_t b = 0; b < P; ++b) {
      Node nd[K];
      const int64_t i0 = ((int64_t)lane * P + b) * K;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t idx = i0 + k;
        const Node t = p[svx::clamp_last(idx, nch) * C];  // every load issued
        nd[k] = idx < nch ? t : sv::zero_node();
      }
      Node carry = sv::node_tree<0, K, K, KIND>(nd);
      bool placed = false;
#pragma unroll
      for (int lv = 0; lv < TOP_BIG_LEVELS; ++lv) {
        if (!placed) {
          if ((b >> lv) & 1) {
            carry = sv::combine_k<KIND>(st[lv], carry);
          } else {
            st[lv] = carry;
            placed = true;
          }
        }
      }
    }
    Node r = sv::zero_node();
#pragma unroll
    for (int lv = 0; lv < TOP_BIG_LEVELS; ++lv)
      if (lv == log2p) r = st[lv];
    return sv::wave_tree<KIND>(r);
  };
  if constexpr (PASS == 0) {
    const Node ny = tree(ws.ny + col, std::integral_constant<int, sv::Y_KIND>{});
    if (lane == 0) ws.m[col] = sv::root_value_k<sv::Y_KIND>(ny) / (float)R;
  } else {
    const Node nd = tree(ws.nd + col, std::integral_constant<int, sv::NODE_TWOSUM>{});
    const Node nq = tree(ws.nq + col, std::integral_constant<int, sv::NODE_NN>{});
    if (lane == 0) finalize(nd, nq, x[col], ws.m[col], R, ddof, var_out + col, mean_out ? mean_out + col : nullptr);
  }
}

// MLOCAL: nch <= CC_GROUP, and every workgroup forms m for its own columns
// from their y chunk nodes (no separate launch); else m comes from
// k_cols_top or k_cols_top_big.
// Tile layout as in k_cols_y.
template <int V, int W, int G, bool MLOCAL>
__global__ __launch_bounds__(64 * W) void k_cols_dq(const float *__restrict__ x, int64_t R, int64_t C, int64_t nch,
                                                    ColsWs ws, int64_t b0) {
  constexpr int E = CC_E, Q = 64 / G, NC = V * Q;
  static_assert(64 * W >= NC, "one thread per column of the block");
  __shared__ Node sd[W][V][Q];
  __shared__ Node sq[W][V][Q];
  __shared__ float sm[V][Q];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane / G, g = lane % G;
  const int64_t blk = b0 + blockIdx.x;  // launches of at most 2^32 - 1 work-items
  const int64_t cb = blk / nch, j = blk % nch;
  const int64_t c0 = cb * NC + (int64_t)q * V;
  const int64_t rw = j * ((int64_t)E * G * W) + (int64_t)w * (E * G);
  const int64_t r0 = rw + (int64_t)g * E;
  const bool full = r0 + E <= R;
  const bool wave_full = rw + (int64_t)E * G <= R;  // uniform
  const int64_t left = R - r0;
  const int valid = left < 0 ? 0 : (left > E ? E : (int)left);

  float x0[V], m[V];
  const int64_t cc = svx::cols_first(c0, C, V);
  if constexpr (MLOCAL) {
    const int t = threadIdx.x;
    if (t < NC) {
      const int k = t / Q, qq = t % Q;  // column V*qq + k of the block, clamped like the loads
      const int64_t col = cb * NC + (int64_t)qq * V + k;
      const int64_t ccol = svx::clamp_last(col, C);
      sm[k][qq] = sv::root_value_k<sv::Y_KIND>(chunk_tree_1(ws.ny + ccol, C, nch)) / (float)R;
    }
    __syncthreads();
  }
  // the tile is loaded after m: the chunk nodes and the tile together do not
  // fit in the registers of 16 waves
  float v[V][E];
  load_cols_tile<V, E>(x, R, C, c0, r0, full, v);
#pragma unroll
  for (int k = 0; k < V; ++k) {
    x0[k] = x[cc + k];
    m[k] = MLOCAL ? sm[k][q] : ws.m[cc + k];
  }
  shift_cols_tile<V, E>(v, x0, wave_full, valid);
#pragma unroll
  for (int k = 0; k < V; ++k) {
    Node nd, nq;
    if (wave_full) sv::lane_tree_dq<false, 0, E, E>(v[k], m[k], E, nd, nq);
    else sv::lane_tree_dq<true, 0, E, E>(v[k], m[k], valid, nd, nq);
    nd = sv::seg_tree<sv::NODE_TWOSUM, G>(nd);
    nq = sv::seg_tree<sv::NODE_NN, G>(nq);
    if (g == 0) {
      sd[w][k][q] = nd;
      sq[w][k][q] = nq;
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < NC) {
    const int k = t / Q, qq = t % Q;  // thread t combines column V*qq + k of the block
    const int64_t col = cb * NC + (int64_t)qq * V + k;
    if (MLOCAL && j == 0 && col < C) ws.m[col] = sm[k][qq];  // for step 4
    if (col < C) {
      Node a[W], b[W];
#pragma unroll
      for (int i = 0; i < W; ++i) {
        a[i] = sd[i][k][qq];
        b[i] = sq[i][k][qq];
      }
      ws.nd[j * C + col] = sv::node_tree<0, W, W>(a);
      ws.nq[j * C + col] = sv::node_tree<0, W, W, sv::NODE_NN>(b);
    }
  }
}

// Whole columns in one workgroup (R <= E*G*W rows): the tile layout of
// k_cols_y with a single chunk, and y, m, d and d^2 in one launch, the tile
// kept in registers between the two passes.  Waves wholly past the last row
// load nothing (their values are the +0 padding).
// E rows per lane (16; 32 or 64 for one column per lane and columns of up
// to 2048 or 4096 rows in one workgroup of 16 waves).  MODE 0 branches per
// wave between full and ragged row ranges; MODE 1 is for R = E*G*W (no
// masks), MODE 2 masks every wave (one code path: with 64 rows per lane the
// two paths of MODE 0 would keep two copies of the shifted tile).
template <int V, int W, int G, bool VEC16, int E = CC_E, int MODE = 0>
__global__ __launch_bounds__(64 * W) void k_cols_one(const float *__restrict__ x, int64_t R, int64_t C, int64_t ddof,
                                                     float *__restrict__ var_out, float *__restrict__ mean_out,
                                                     int b0) {
  constexpr int Q = 64 / G, NC = V * Q;
  __shared__ Node sd[W][V][Q];
  __shared__ Node sq[W][V][Q];
  __shared__ float sm[V][Q];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // MODE 2 launches only the waves that reach row R; the others' nodes are
  // the zero nodes of the padding
  const int nw = MODE == 2 ? __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6)) : W;
  const int q = lane / G, g = lane % G;
  // Blocks narrower than a 128-byte cache line (NC < 32 columns) share each
  // line with the next P - 1 blocks.  The dispatcher deals workgroups round
  // robin to the eight dies, each with its own L2, so block b would run on
  // die b % 8 and P dies would fetch the same line.  Within each full group
  // of 8P workgroups, the P on one die take P adjacent blocks instead.
  // b0: the launch's first workgroup (launches of at most 2^32 - 1
  // work-items; fewer than 2^31 workgroups in all)
  const int64_t cb = svx::line_on_one_die<int>(b0 + (int)blockIdx.x, (int)((C + NC - 1) / NC), NC);
  const int64_t c0 = cb * NC + (int64_t)q * V;
  const int64_t rw = (int64_t)w * (E * G);  // the wave's first row
  const int64_t r0 = rw + (int64_t)g * E;
  const bool full = MODE == 1 || r0 + E <= R;
  const bool wave_full = MODE == 1 || (MODE == 0 && rw + (int64_t)E * G <= R);  // uniform
  const int64_t left = R - r0;
  const int valid = left < 0 ? 0 : (left > E ? E : (int)left);

  float v[V][E];
  // MODE 0 skips the loads of a wave wholly past R; MODE 2 issues them at
  // rows clamped to R - 1, so that no branch makes the first use of a
  // value wait for all of them
  if (MODE != 0 || rw < R) load_cols_tile<V, E, VEC16>(x, R, C, c0, r0, full, v);
  float x0[V];
  const int64_t cc = svx::cols_first(c0, C, V);
#pragma unroll
  for (int k = 0; k < V; ++k) x0[k] = x[svx::clamp_last(cc + k, C)];
  shift_cols_tile<V, E>(v, x0, wave_full, valid);  // +0 past the last row
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const Node nd = sv::seg_tree<sv::Y_KIND, G>(sv::lane_tree<sv::Y_LEAF, 0, E, E>(v[k]));
    if (g == 0) sd[w][k][q] = nd;
  }
  __syncthreads();
  // thread t forms m (then step 4) of columns V*tq + tk of the block, t = tk*Q + tq
  for (int t = threadIdx.x; t < NC; t += blockDim.x) {
    const int tk = t / Q, tq = t % Q;
    Node nn[W];
#pragma unroll
    for (int i = 0; i < W; ++i) nn[i] = i < nw ? sd[i][tk][tq] : sv::zero_node();
    sm[tk][tq] = sv::root_value_k<sv::Y_KIND>(sv::node_tree<0, W, W, sv::Y_KIND>(nn)) / (float)R;
  }
  __syncthreads();
  // The step-3 masks are compared afresh from an opaque copy of `valid`:
  // with E = 64 rows per lane, keeping the step-1 masks (one 64-bit scalar
  // pair per row) alive across the barrier would overflow the scalar
  // registers into vector ones and spill.
  int valid_dq = valid;
  if constexpr (MODE == 2) asm volatile("" : "+v"(valid_dq));
#pragma unroll
  for (int k = 0; k < V; ++k) {
    Node nd, nq;
    if (wave_full) sv::lane_tree_dq<false, 0, E, E>(v[k], sm[k][q], E, nd, nq);
    else sv::lane_tree_dq<true, 0, E, E>(v[k], sm[k][q], valid_dq, nd, nq);
    nd = sv::seg_tree<sv::NODE_TWOSUM, G>(nd);
    nq = sv::seg_tree<sv::NODE_NN, G>(nq);
    if (g == 0) {
      sd[w][k][q] = nd;  // the y nodes were read before the barrier
      sq[w][k][q] = nq;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < NC; t += blockDim.x) {
    const int tk = t / Q, tq = t % Q;
    const int64_t col = cb * NC + (int64_t)tq * V + tk;
    if (col < C) {
      Node a[W], b[W];
#pragma unroll
      for (int i = 0; i < W; ++i) {
        a[i] = i < nw ? sd[i][tk][tq] : sv::zero_node();
        b[i] = i < nw ? sq[i][tk][tq] : sv::zero_node();
      }
      finalize(sv::node_tree<0, W, W>(a), sv::node_tree<0, W, W, sv::NODE_NN>(b), x[col], sm[tk][tq], R, ddof,
               var_out + col, mean_out ? mean_out + col : nullptr);
    }
  }
}

// ------------------------------------------------------------------ long slices

// Rows longer than one workgroup's registers hold (axis 1, n > 16384) are
// cut into aligned chunks (a chunk is a node of the row's tree) and reduced
// in four launches: y-tree node per chunk -> per row m = Plain(y)/n -> d- and
// d^2-tree nodes per chunk -> per row top trees and step 4.  The input is
// read twice.  Workspace per row: nchunks y nodes, 2*nchunks d/d^2 nodes and
// m.

using svx::LS_TOP_PER_THREAD;  // chunk nodes per thread at the top
using svx::LS_MAX_CHUNKS;      // 8192 chunks per slice
using svx::LS_ROW_CHUNK;       // axis 1: 16384 values (4 waves x 64 lanes x 64)

struct LongWs {
  Node *ny;   // [nslices][nch]
  Node *nd;   // [nslices][nch]
  Node *nq;   // [nslices][nch]
  float *m;   // [nslices]
};

// Axis 1, pass 0 or 1 over chunk c of row r (block index = r * nch + c).
// P = 2: each row holds n pairs (2n floats) of two interleaved slices (the
// real and imaginary parts of complex values, or the two columns of a
// [n, 2] matrix), slices 2r and 2r + 1 of the launch: a lane holds E/2
// consecutive pairs (E floats, one per-lane load of 4 values at a time) and
// splits them in registers; the chunk covers LS_ROW_CHUNK / 2 pairs, and
// both slices' nodes go to the workspace.
// V: an ablation variant (its shift and tree of y; the d and d^2 trees are
// the compensated ones, whose s parts are the plain trees).
template <int PASS, bool VEC, int P = 1, int V = V_KERNEL>
__global__ __launch_bounds__(256) void k_long_rows(const float *__restrict__ x, int64_t n, int64_t ld, int64_t nch,
                                                   LongWs ws) {
  using F = VariantFlags<V>;
  constexpr int E = 64, W = 4, EP = E / P;  // EP values of each slice per lane
  constexpr int64_t CHUNK = LS_ROW_CHUNK / P;
  __shared__ Node slots[2 * P][W];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x / nch;
  const int64_t c = (int64_t)blockIdx.x % nch;
  const float *__restrict__ row = x + r * ld;
  const int64_t base = c * CHUNK + (int64_t)w * 64 * EP;  // first value of this wave, of each slice
  float f[E];
  float dummy_lds[1];
  const int64_t avail = P * svx::rows_avail(gridDim.x / nch, r, ld / P, n, base);  // floats to the launch's last row
  sv::load_tile<E, VEC, 1, false>(row + P * base, P * (n - base), dummy_lds, f, lane, avail);
  const bool full = base + 64 * EP <= n;
  const int64_t vl = n - base - (int64_t)lane * EP;
  const int valid = vl < 0 ? 0 : (vl > EP ? EP : (int)vl);
  float v[P][EP];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const float x0 = row[j];
#pragma unroll
    for (int i = 0; i < EP; ++i) v[j][i] = (full || i < valid) ? (F::shift ? f[P * i + j] - x0 : f[P * i + j]) : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int64_t out = (P * r + j) * nch + c;
    if constexpr (PASS == 0) {
      Node ny = sv::lane_tree<F::yleaf, 0, EP, EP>(v[j]);
      ny = sv::wave_tree<F::ykind>(ny);
      ny = block_tree<W, F::ykind>(ny, slots[2 * j], w, lane);
      if (threadIdx.x == 0) ws.ny[out] = ny;
    } else {
      const float m = ws.m[P * r + j];
      // the step-3 masks are compared afresh from an opaque copy of `valid`:
      // kept from step 1 (a 64-bit scalar pair per value) they spilled
      int valid_dq = valid;
      asm volatile("" : "+v"(valid_dq));
      Node nd, nq;
      if (full) sv::lane_tree_dq<false, 0, EP, EP>(v[j], m, EP, nd, nq);
      else sv::lane_tree_dq<true, 0, EP, EP>(v[j], m, valid_dq, nd, nq);
      nd = sv::wave_tree<sv::NODE_TWOSUM>(nd);
      nq = sv::wave_tree<sv::NODE_NN>(nq);
      nd = block_tree<W, sv::NODE_TWOSUM>(nd, slots[2 * j], w, lane);
      nq = block_tree<W, sv::NODE_NN>(nq, slots[2 * j + 1], w, lane);
      if (threadIdx.x == 0) {
        ws.nd[out] = nd;
        ws.nq[out] = nq;
      }
    }
  }
}

// Tree over the nch chunk nodes of one slice (one workgroup per slice), the
// chunk nodes padded with zeros to 256 * K.
template <int KIND, int K>
__device__ __forceinline__ Node top_tree(const Node *__restrict__ nodes, int64_t nch, Node *slots) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  Node nd[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t idx = (int64_t)threadIdx.x * K + k;
    const Node t = nodes[svx::clamp_last(idx, nch)];  // unconditional: the loads overlap
    nd[k] = idx < nch ? t : sv::zero_node();
  }
  Node r = sv::node_tree<0, K, K, KIND>(nd);
  r = sv::wave_tree<KIND>(r);
  return block_tree<4, KIND>(r, slots, w, lane);
}

// PASS 0: m = Plain(y) / n.  PASS 1: the top trees of d and d^2 and step 4.
// One 256-thread workgroup per slice; slice s's first value is at
// x[(s / P) * sstride + s % P] (P interleaved slices per row).  V: an
// ablation variant (its tree of y, local mean and step 4).
template <int PASS, int K, int P = 1, int V = V_KERNEL>
__global__ __launch_bounds__(256) void k_long_top(const float *__restrict__ x, int64_t n, int64_t sstride,
                                                  int64_t nch, int64_t ddof, LongWs ws, float *__restrict__ var_out,
                                                  float *__restrict__ mean_out) {
  using F = VariantFlags<V>;
  __shared__ Node slots[2][4];
  const int64_t sl = blockIdx.x;
  if constexpr (PASS == 0) {
    const Node ny = top_tree<F::ykind, K>(ws.ny + sl * nch, nch, slots[0]);
    if (threadIdx.x == 0) ws.m[sl] = local_mean<V>(ny, n);
  } else {
    const Node nd = top_tree<sv::NODE_TWOSUM, K>(ws.nd + sl * nch, nch, slots[0]);
    const Node nq = top_tree<sv::NODE_NN, K>(ws.nq + sl * nch, nch, slots[1]);
    if (threadIdx.x == 0) {
      const float x0 = x[(sl / P) * sstride + sl % P];
      float *mo = mean_out ? mean_out + sl : nullptr;
      if constexpr (V == V_KERNEL) finalize(nd, nq, x0, ws.m[sl], n, ddof, var_out + sl, mo);
      else finalize_v<V>(nd, nq, x0, ws.m[sl], n, ddof, var_out + sl, mo);
    }
  }
}

// ------------------------------------------------------------------ host side

using svx::C64_FUSED_MAX_N;  // complex rows reduced in one pass (k_var_rows_c64)

// Launch-geometry tuning (never changes a result bit).  Each host thread has
// its own settings: sv_set_tuning on one thread leaves the calls of every
// other thread alone.
struct Tuning {
  int sum_load_path = 0;      // 0: coalesced loads + LDS transpose, 1: per-lane contiguous loads
  int sum_nt = 1;             // non-temporal loads of the summed input
  int sum_e = 32;             // values per lane in a tree-sum chunk: 16 or 32
  int sum_depth = 2;          // chunks in flight per wave (register ring): 2 or 4
  int64_t sum_blocks = 8192;  // target workgroup count of the tree sum
  int var_load_path = 1;      // as sum_load_path, for the row-variance kernel
  int var_nt = 0;             // non-temporal loads in the row-variance kernel
  int var_split = 0;          // waves per 4096 values of a row of 1025..16384 values (1, 2, 4, 8; 0 auto)
  int var_lds_pad = 0;        // unused dynamic LDS bytes per row workgroup (caps resident waves)
  int var_cols_single_max = 1024;  // axis 0: rows up to which one workgroup holds a column tile (<= 1024)
  int var_cols_waves = 0;     // axis 0, chunked: waves per workgroup (4, 8, 16; 0 auto); chunks of 16 * waves rows
  int var_short_rows = 1;     // rows of <= 512 values share waves (0: one workgroup per row)
  int var_cols_one = 1;       // axis 0, 65..1024 rows: 1 auto, 2 four columns per lane, 3 one, 0 the lane kernel
  int var_long_rows = 1;      // rows of 16385..65536 values, 256+ rows: 1 one workgroup per row, 0 chunked
  int var_cols_short = 1;     // axis 0, columns of <= 15 rows: 1 four columns per lane, 0 the lane kernel
  int sum_xcd = 0;            // tree sum: each die (XCD) streams one contiguous region
  int var_xcd = 0;            // row variance: each die (XCD) takes one contiguous run of rows
  int var_full_rows = 1;      // rows that fill their tile exactly take the kernel without masks (0: the general one)
  int var_cols_once = 1;      // axis 0, 1025..4096 rows: one workgroup per 16 columns, one read, when the
                             // grid fills the chip (0: row chunks; 2: one read whatever the fill)
  int64_t launch_items = svx::MAX_LAUNCH_ITEMS;  // work-items per launch before a grid is cut into batches
  int var_cols_pairs = 1;     // axis 0, two columns of 4097+ rows: one row of pairs in chunks (0: column chunks)
};
thread_local Tuning g_tune;

}  // namespace

int64_t svh::launch_items() { return g_tune.launch_items; }
int svh::cols_once() { return g_tune.var_cols_once; }
int svh::cols_pairs() { return g_tune.var_cols_pairs; }
int svh::long_rows() { return g_tune.var_long_rows; }

namespace {

// The per-call constants of steps 2 and 4 (see StepConsts).
StepConsts step_consts(int64_t n, int64_t ddof) {
  StepConsts k;
  k.fn = (float)n;
  int ex = 0;
  k.rn = (n > 0 && frexpf(k.fn, &ex) == 0.5f) ? 1.0f / k.fn : 0.0f;
  k.ddof_on = ddof != 0;
  const int64_t den = n - ddof < 0 ? 0 : n - ddof;
  k.dfac = ddof != 0 ? k.fn / (float)den : 1.0f;
  return k;
}

using svx::SUM_MAX_N;
using svx::VAR_MAX_ELEMS;
using svx::ROWS_MAX_N;  // single-tile row kernel for any number of rows
// Rows of up to 65536 values also take one workgroup per row (16 waves) when
// there are enough rows to fill the chip; fewer rows take the chunked path.
using svx::ROWS_ONE_MAX_N;
using svx::ROWS_ONE_MIN_ROWS;
using svx::COLS_MAX_R;           // single-tile column kernel
using svx::COLS_ONE_LONG_MAX_R;  // one column per lane, 64 rows per lane, 16 waves

// Long-slice workspace: y, d and d^2 chunk nodes per slice, then m.
size_t long_ws_bytes(int64_t nslices, int64_t nch) {
  return (size_t)nslices * (size_t)nch * 3 * sizeof(Node) + (size_t)nslices * sizeof(float);
}

LongWs long_ws(void *workspace, int64_t nslices, int64_t nch) {
  char *p = reinterpret_cast<char *>(workspace);
  const size_t nodes = (size_t)nslices * (size_t)nch * sizeof(Node);
  return {reinterpret_cast<Node *>(p), reinterpret_cast<Node *>(p + nodes), reinterpret_cast<Node *>(p + 2 * nodes),
          reinterpret_cast<float *>(p + 3 * nodes)};
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Axis-0 chunked workspace: the three node arrays (room for the shortest
// chunks, CC_E * CC_MIN_W rows) and m.  Independent of the launch knobs.
struct ColsLayout {
  size_t nodes, m, total;
};

ColsLayout cols_layout(int64_t R, int64_t C) {
  const int64_t nch = (R + CC_E * CC_MIN_W - 1) / (CC_E * CC_MIN_W);
  ColsLayout L;
  L.nodes = round256((size_t)nch * (size_t)C * sizeof(Node));
  L.m = round256((size_t)C * sizeof(float));
  L.total = 3 * L.nodes + L.m;
  return L;
}

ColsWs cols_ws(void *workspace, const ColsLayout &L) {
  char *p = reinterpret_cast<char *>(workspace);
  ColsWs ws;
  ws.ny = reinterpret_cast<Node *>(p);
  p += L.nodes;
  ws.nd = reinterpret_cast<Node *>(p);
  p += L.nodes;
  ws.nq = reinterpret_cast<Node *>(p);
  p += L.nodes;
  ws.m = reinterpret_cast<float *>(p);
  return ws;
}

template <int V, int W, int G>
void launch_cols_chunked(const float *x, int64_t R, int64_t C, int64_t ddof, const ColsWs &ws, float *var,
                         float *mean, hipStream_t st) {
  const svx::ColsChunkPlan p = svx::cols_chunk_plan(V, W, R, C);  // G = p.G
  const int64_t nch = p.nch, ncb = p.ncb;
  const dim3 block(64 * W);
  // workgroup b = cb * nch + j takes chunk j of column block cb
  svh::in_batches(ncb * nch, 1, 64 * W, [&](int64_t b0, int64_t nb) {
    k_cols_y<V, W, G><<<dim3((unsigned)nb), block, 0, st>>>(x, R, C, nch, ws, b0);
  });
  auto dq = [&](auto mlocal) {
    svh::in_batches(ncb * nch, 1, 64 * W, [&](int64_t b0, int64_t nb) {
      k_cols_dq<V, W, G, decltype(mlocal)::value><<<dim3((unsigned)nb), block, 0, st>>>(x, R, C, nch, ws, b0);
    });
  };
  // the top kernels: four waves of per_wave columns each per workgroup,
  // launches of at most 2^32 - 1 work-items
  auto top = [&](int per_wave, auto &&launch) {
    svh::in_batches((C + 4 * per_wave - 1) / (4 * per_wave), 1, 256,
                    [&](int64_t b0, int64_t nb) { launch(dim3((unsigned)nb), b0); });
  };
  if (nch <= CC_GROUP) {
    dq(std::true_type{});
    // the final trees: a group of S >= nch lanes per column, one node each
#define SV_TOP(PASS, K, S, PW)                                                                           \
  top(PW, [&](dim3 g, int64_t b0) {                                                                      \
    k_cols_top<PASS, K, S><<<g, dim3(256), 0, st>>>(x, R, C, nch, ddof, ws, var, mean, b0);              \
  })
    if (nch <= 4) SV_TOP(1, 1, 4, 16);
    else if (nch <= 8) SV_TOP(1, 1, 8, 8);
    else if (nch <= 16) SV_TOP(1, 1, 16, 4);
    else SV_TOP(1, 1, 32, 2);
  } else if (nch <= 64 * 64) {
    // many chunks: a wave per column for m and for the final trees
    if (nch <= 64 * 4) {
      SV_TOP(0, 4, 64, 1);
      dq(std::false_type{});
      SV_TOP(1, 4, 64, 1);
    } else if (nch <= 64 * 16) {
      SV_TOP(0, 16, 64, 1);
      dq(std::false_type{});
      SV_TOP(1, 16, 64, 1);
    } else {
      SV_TOP(0, 64, 64, 1);
      dq(std::false_type{});
      SV_TOP(1, 64, 64, 1);
    }
  } else {
    int log2p = 0;  // runs of 64 * 2^log2p chunk nodes per lane
    while (((int64_t)64 * 64 << log2p) < nch) ++log2p;
    top(1, [&](dim3 g, int64_t b0) {
      k_cols_top_big<0><<<g, dim3(256), 0, st>>>(x, R, C, nch, log2p, ddof, ws, var, mean, b0);
    });
    dq(std::false_type{});
    top(1, [&](dim3 g, int64_t b0) {
      k_cols_top_big<1><<<g, dim3(256), 0, st>>>(x, R, C, nch, log2p, ddof, ws, var, mean, b0);
    });
  }
#undef SV_TOP
}

// Row groups per wave, so that lanes stay on columns: G = 1 (64 column
// groups of V per block) for matrices of at least 64 groups, G = 4 (16 groups
// per block) for 9 to 63, G = 8 (8 groups) for 5 to 8, G = 16 (4 groups) for
// 3 and 4, G = 32 (2 groups) for two, G = 64 for one.
template <int V, int W>
void launch_cols_g(const float *x, int64_t R, int64_t C, int64_t ddof, const ColsWs &ws, float *var, float *mean,
                   hipStream_t st) {
  switch (svx::cols_chunk_plan(V, W, R, C).G) {
    case 1: launch_cols_chunked<V, W, 1>(x, R, C, ddof, ws, var, mean, st); break;
    case 4: launch_cols_chunked<V, W, 4>(x, R, C, ddof, ws, var, mean, st); break;
    case 8: launch_cols_chunked<V, W, 8>(x, R, C, ddof, ws, var, mean, st); break;
    case 16: launch_cols_chunked<V, W, 16>(x, R, C, ddof, ws, var, mean, st); break;
    case 32: launch_cols_chunked<V, W, 32>(x, R, C, ddof, ws, var, mean, st); break;
    default: launch_cols_chunked<V, W, 64>(x, R, C, ddof, ws, var, mean, st); break;
  }
}

template <int V>
void launch_cols_v(const float *x, int64_t R, int64_t C, int64_t ddof, const ColsWs &ws, float *var, float *mean,
                   hipStream_t st) {
  int waves = g_tune.var_cols_waves;
  if (waves == 0) {  // auto: svx::cols_chunk_waves on this device's CU count
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 0;
    waves = svx::cols_chunk_waves(V, R, C, cus);
  }
  if (waves == 16) launch_cols_g<V, 16>(x, R, C, ddof, ws, var, mean, st);
  else if (waves == 8) launch_cols_g<V, 8>(x, R, C, ddof, ws, var, mean, st);
  else launch_cols_g<V, 4>(x, R, C, ddof, ws, var, mean, st);
}

// Columns of 64 < R <= 1024 rows in one launch (k_cols_one), four adjacent
// columns per lane (one 16-byte load per row when VEC16, else four 4-byte
// loads): 16*G*W
// = the power of two at or above R rows per workgroup, 4*64/G columns.  Of
// the (G, W) pairs that hold exactly that many rows (G in 1, 4, 16; W in 1,
// 2, 4, 8), the smallest G that still gives 512 workgroups, else the largest.
// A column that fills at most 5/8 of its tile takes MODE 2 (one masked
// code path: 91-106 VGPRs against 140-150, and only the waves row R reaches);
// fuller tiles keep MODE 0, whose full waves skip the masks (µs, MODE 0 /
// MODE 2: [520, 65536] 53.0 / 48.5, [513, 30000] 26.7 / 25.0, [800, 10000]
// 15.3 / 16.5, [1000, 8192] 14.5 / 15.9).
template <bool VEC16>
void launch_cols_one(const float *x, int64_t R, int64_t C, int64_t ddof, float *var, float *mean, hipStream_t st) {
  const svx::ColsOnePlan p = svx::cols_one4_plan(R, C);
  const int g = p.G, w = p.W;
  const bool sparse = svx::cols_one4_masked(R, p);
  const int reached = (int)((R + 16LL * g - 1) / (16LL * g));  // the waves row R reaches
#define SV_ONE(G_, W_)                                                                                        \
  if (!sparse)                                                                                                \
    svh::in_batches(p.blocks, 1, 64 * W_, [&](int64_t b0, int64_t nb) {                                       \
      k_cols_one<4, W_, G_, VEC16><<<dim3((unsigned)nb), dim3(64 * W_), 0, st>>>(x, R, C, ddof, var, mean, (int)b0); \
    });                                                                                                       \
  else                                                                                                        \
    svh::in_batches(p.blocks, 1, 64 * reached, [&](int64_t b0, int64_t nb) {                                  \
      k_cols_one<4, W_, G_, VEC16, CC_E, 2><<<dim3((unsigned)nb), dim3(64 * (unsigned)reached), 0, st>>>(      \
          x, R, C, ddof, var, mean, (int)b0);                                                                 \
    })
  switch (g * 16 + w) {  // R > 64: 16*G*W >= 128
    case 16 * 1 + 8: SV_ONE(1, 8); break;
    case 16 * 4 + 2: SV_ONE(4, 2); break;
    case 16 * 4 + 4: SV_ONE(4, 4); break;
    case 16 * 4 + 8: SV_ONE(4, 8); break;
    case 16 * 16 + 1: SV_ONE(16, 1); break;
    case 16 * 16 + 2: SV_ONE(16, 2); break;
    default: SV_ONE(16, 4); break;  // gw = 64
  }
#undef SV_ONE
}

// The same with one column per lane (16 values per lane: four times the
// waves of four columns per lane): G in 1, 4 (row segments of at least 16
// lanes, 64 bytes), W up to 16; G = 1 when that gives 512 workgroups.
void launch_cols_one1(const float *x, int64_t R, int64_t C, int64_t ddof, float *var, float *mean, hipStream_t st) {
  const svx::ColsOnePlan p = svx::cols_one1_plan(R, C);
  const int g = p.G, w = p.W;
#define SV_ONE(G_, W_)                                                                                   \
  svh::in_batches(p.blocks, 1, 64 * W_, [&](int64_t b0, int64_t nb) {                                    \
    k_cols_one<1, W_, G_, false><<<dim3((unsigned)nb), dim3(64 * W_), 0, st>>>(x, R, C, ddof, var, mean, (int)b0); \
  })
  switch (g * 32 + w) {  // R > 64: 16*G*W >= 128
    case 32 * 1 + 8: SV_ONE(1, 8); break;
    case 32 * 1 + 16: SV_ONE(1, 16); break;
    case 32 * 4 + 2: SV_ONE(4, 2); break;
    case 32 * 4 + 4: SV_ONE(4, 4); break;
    case 32 * 4 + 8: SV_ONE(4, 8); break;
    default: SV_ONE(4, 16); break;  // gw = 64
  }
#undef SV_ONE
}

// The top trees over nch <= LS_MAX_CHUNKS chunk nodes per slice: 256
// threads of K nodes each, K the smallest of 1, 4, 32 that holds nch (the
// zero padding beyond nch changes no bit).
template <int PASS, int P = 1, int V = V_KERNEL>
void launch_long_top(const float *x, int64_t n, int64_t sstride, int64_t nch, int64_t ddof, const LongWs &ws,
                     float *var, float *mean, dim3 grid, hipStream_t st) {
  if (nch <= 256) k_long_top<PASS, 1, P, V><<<grid, 256, 0, st>>>(x, n, sstride, nch, ddof, ws, var, mean);
  else if (nch <= 1024) k_long_top<PASS, 4, P, V><<<grid, 256, 0, st>>>(x, n, sstride, nch, ddof, ws, var, mean);
  else k_long_top<PASS, LS_TOP_PER_THREAD, P, V><<<grid, 256, 0, st>>>(x, n, sstride, nch, ddof, ws, var, mean);
}

// Rows of n pairs (two interleaved slices per row, row stride ld floats) in
// chunks: slices 2r and 2r + 1 of row r; var and mean get 2 * rows entries
// (slice order).  Workspace: long_ws of 2 * rows slices of
// ceil(n / (LS_ROW_CHUNK / 2)) chunks.
void launch_long_pairs(bool vec, const float *x, int64_t rows, int64_t n, int64_t ld, int64_t ddof, void *workspace,
                       float *var, float *mean, hipStream_t st) {
  const int64_t nch = (n + LS_ROW_CHUNK / 2 - 1) / (LS_ROW_CHUNK / 2);
  const LongWs ws = long_ws(workspace, 2 * rows, nch);
  const dim3 grid((unsigned)(rows * nch)), block(256), top((unsigned)(2 * rows));
  if (vec) k_long_rows<0, true, 2><<<grid, block, 0, st>>>(x, n, ld, nch, ws);
  else k_long_rows<0, false, 2><<<grid, block, 0, st>>>(x, n, ld, nch, ws);
  launch_long_top<0, 2>(x, n, ld, nch, ddof, ws, var, mean, top, st);
  if (vec) k_long_rows<1, true, 2><<<grid, block, 0, st>>>(x, n, ld, nch, ws);
  else k_long_rows<1, false, 2><<<grid, block, 0, st>>>(x, n, ld, nch, ws);
  launch_long_top<1, 2>(x, n, ld, nch, ddof, ws, var, mean, top, st);
}

// The tree sum's plan: chunks of 64*e values, each wave of a SUM_W-wave
// workgroup streaming 2^log2_g of them, log2_g the smallest value that keeps
// the workgroup count at or below `target_blocks`; with log2_g capped at
// SUM_MAX_LOG2_GROUP the count stays at or below SUM_MAX_BLOCKS for every
// n <= SUM_MAX_N.
using svx::SumPlan;
SumPlan plan_sum(int64_t n, int e, int64_t target_blocks) {
  return svx::plan_sum(n, e, target_blocks, SUM_W, SUM_MAX_BLOCKS, SUM_MAX_LOG2_GROUP);
}

size_t sum_workspace_bytes(int64_t n) {
  if (n <= 0) return 0;
  // counters, then one node per workgroup (room for the largest grid) and
  // one per group of SUM_GROUP workgroups
  return SUM_WS_HEADER + (size_t)(SUM_MAX_BLOCKS + SUM_MAX_BLOCKS / SUM_GROUP) * sizeof(Node);
}

template <int E, bool VEC, int LOADP, bool NT>
void launch_sum_t(const float *x, int64_t n, const SumPlan &p, Node *part, unsigned *counter, float *out,
                  hipStream_t st) {
  const dim3 grid((unsigned)p.blocks), block(64 * SUM_W);
  if (g_tune.sum_depth == 4) k_tree_sum<E, SUM_W, VEC, LOADP, NT, 4><<<grid, block, 0, st>>>(x, n, p.log2_g, part, counter, out, g_tune.sum_xcd);
  else k_tree_sum<E, SUM_W, VEC, LOADP, NT, 2><<<grid, block, 0, st>>>(x, n, p.log2_g, part, counter, out, g_tune.sum_xcd);
}

// The double-word-carry sum in the default load configuration (coalesced
// loads through LDS, non-temporal, two chunks in flight).
template <int E>
void launch_sum_dw(bool vec, const float *x, int64_t n, const SumPlan &p, Node *part, unsigned *counter, float *out,
                   hipStream_t st) {
  const dim3 grid((unsigned)p.blocks), block(64 * SUM_W);
  if (vec) k_tree_sum<E, SUM_W, true, 0, true, 2, sv::NODE_DW><<<grid, block, 0, st>>>(x, n, p.log2_g, part, counter, out, g_tune.sum_xcd);
  else k_tree_sum<E, SUM_W, false, 0, true, 2, sv::NODE_DW><<<grid, block, 0, st>>>(x, n, p.log2_g, part, counter, out, g_tune.sum_xcd);
}

template <int E>
void launch_sum_e(bool vec, const float *x, int64_t n, const SumPlan &p, Node *part, unsigned *counter, float *out,
                  hipStream_t st) {
  const int sel = (vec ? 4 : 0) + (g_tune.sum_load_path ? 2 : 0) + (g_tune.sum_nt ? 1 : 0);
  switch (sel) {
    case 0: launch_sum_t<E, false, 0, false>(x, n, p, part, counter, out, st); break;
    case 1: launch_sum_t<E, false, 0, true>(x, n, p, part, counter, out, st); break;
    case 2: launch_sum_t<E, false, 1, false>(x, n, p, part, counter, out, st); break;
    case 3: launch_sum_t<E, false, 1, true>(x, n, p, part, counter, out, st); break;
    case 4: launch_sum_t<E, true, 0, false>(x, n, p, part, counter, out, st); break;
    case 5: launch_sum_t<E, true, 0, true>(x, n, p, part, counter, out, st); break;
    case 6: launch_sum_t<E, true, 1, false>(x, n, p, part, counter, out, st); break;
    default: launch_sum_t<E, true, 1, true>(x, n, p, part, counter, out, st); break;
  }
}

template <int E, int W, bool VEC, int LOADP, bool NT>
void launch_rows_t(const float *x, int64_t rows, int64_t n, int64_t ld, int64_t ddof, float *var, float *mean,
                   hipStream_t st) {
  if constexpr (VEC && LOADP == 1 && !NT) {
    // rows that fill the tile exactly: the kernel without masks
    if (n == 64LL * E * W && g_tune.var_full_rows && !g_tune.var_lds_pad && !g_tune.var_xcd) {
      const StepConsts k = step_consts(n, ddof);
      svh::in_batches(rows, 1, 64 * W, [&](int64_t r0, int64_t nr) {
        k_var_rows_full<E, W><<<dim3((unsigned)nr), dim3(64 * W), 0, st>>>(x + r0 * ld, ld, k, var + r0,
                                                                           mean ? mean + r0 : nullptr);
      });
      return;
    }
  }
  // only the waves the row reaches (the tree pads the others with zero
  // nodes); var_lds_pad: unused dynamic LDS per workgroup, a cap on resident
  // waves
  const int waves = svx::rows_waves(n, E, W);
  svh::in_batches(rows, 1, 64 * waves, [&](int64_t r0, int64_t nr) {
    k_var_rows<E, W, VEC, LOADP, NT><<<dim3((unsigned)nr), dim3(64 * waves), (size_t)g_tune.var_lds_pad, st>>>(
        x + r0 * ld, n, ld, ddof, var + r0, mean ? mean + r0 : nullptr, g_tune.var_xcd);
  });
}

// A row shared by W waves of E values per lane; 16-byte loads follow
// var_load_path (0 coalesced + LDS transpose, 1 per lane, 2 coalesced +
// staged transpose), scalar loads are per lane.
template <int E, int W>
void launch_rows_split(bool vec, const float *x, int64_t rows, int64_t n, int64_t ld, int64_t ddof, float *var,
                       float *mean, hipStream_t st) {
  if (!vec) launch_rows_t<E, W, false, 1, false>(x, rows, n, ld, ddof, var, mean, st);
  else if (g_tune.var_load_path == 0) launch_rows_t<E, W, true, 0, false>(x, rows, n, ld, ddof, var, mean, st);
  else if (g_tune.var_load_path == 2 && E % 16 == 0) {
    if constexpr (E % 16 == 0) launch_rows_t<E, W, true, 2, false>(x, rows, n, ld, ddof, var, mean, st);
  } else {
    launch_rows_t<E, W, true, 1, false>(x, rows, n, ld, ddof, var, mean, st);
  }
}

template <int E, int W>
void launch_rows_ew(bool vec, const float *x, int64_t rows, int64_t n, int64_t ld, int64_t ddof, float *var,
                    float *mean, hipStream_t st) {
  if constexpr (E % 16 == 0) {
    if (g_tune.var_load_path == 2) {
      if (vec) launch_rows_t<E, W, true, 2, false>(x, rows, n, ld, ddof, var, mean, st);
      else launch_rows_t<E, W, false, 1, false>(x, rows, n, ld, ddof, var, mean, st);
      return;
    }
  }
  const int sel = (vec ? 4 : 0) + (g_tune.var_load_path != 0 ? 2 : 0) + (g_tune.var_nt ? 1 : 0);
  switch (sel) {
    case 0: launch_rows_t<E, W, false, 0, false>(x, rows, n, ld, ddof, var, mean, st); break;
    case 1: launch_rows_t<E, W, false, 0, true>(x, rows, n, ld, ddof, var, mean, st); break;
    case 2: launch_rows_t<E, W, false, 1, false>(x, rows, n, ld, ddof, var, mean, st); break;
    case 3: launch_rows_t<E, W, false, 1, true>(x, rows, n, ld, ddof, var, mean, st); break;
    case 4: launch_rows_t<E, W, true, 0, false>(x, rows, n, ld, ddof, var, mean, st); break;
    case 5: launch_rows_t<E, W, true, 0, true>(x, rows, n, ld, ddof, var, mean, st); break;
    case 6: launch_rows_t<E, W, true, 1, false>(x, rows, n, ld, ddof, var, mean, st); break;
    default: launch_rows_t<E, W, true, 1, true>(x, rows, n, ld, ddof, var, mean, st); break;
  }
}

using svx::SEG_MAX_N;  // rows that share waves (k_var_rows_seg)

// vw: 4 for 16-byte aligned rows of a multiple of 4 values, 2 for 8-byte
// aligned rows of an even count, else 1.
template <int E, int S>
void launch_seg_t(int vw, const float *x, int64_t rows, int64_t n, int64_t ld, int64_t ddof, float *var,
                  float *mean, hipStream_t st) {
  constexpr int RPB = 4 * (64 / S);  // rows per workgroup
  const StepConsts k = step_consts(n, ddof);
  svh::in_batches(rows, RPB, 256, [&](int64_t r0, int64_t nr) {
    const dim3 grid((unsigned)((nr + RPB - 1) / RPB)), block(256);
    const float *xr = x + r0 * ld;
    float *vr = var + r0, *mr = mean ? mean + r0 : nullptr;
    if (vw == 4) k_var_rows_seg<E, S, 4><<<grid, block, 0, st>>>(xr, nr, n, ld, k, vr, mr);
    else if (vw == 2) k_var_rows_seg<E, S, 2><<<grid, block, 0, st>>>(xr, nr, n, ld, k, vr, mr);
    else k_var_rows_seg<E, S, 1><<<grid, block, 0, st>>>(xr, nr, n, ld, k, vr, mr);
  });
}

// Short rows: E values per lane (4, 8 or 16) and S lanes per row with S*E
// the row's power-of-two tile.
void launch_rows_seg(const float *x, int64_t rows, int64_t n, int64_t ld, int64_t ddof, float *var, float *mean,
                     hipStream_t st) {
  const int vec = svx::seg_vw(reinterpret_cast<uintptr_t>(x), ld);
  const svx::SegPlan p = svx::seg_plan(n);
  switch (p.E * 100 + p.S) {
    case 401: launch_seg_t<4, 1>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 801: launch_seg_t<8, 1>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 1601: launch_seg_t<16, 1>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 1602: launch_seg_t<16, 2>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 1604: launch_seg_t<16, 4>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 1608: launch_seg_t<16, 8>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 1616: launch_seg_t<16, 16>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    default: launch_seg_t<16, 32>(vec, x, rows, n, ld, ddof, var, mean, st); break;
  }
}

// Rows of 1025..16384 values: the row's power-of-two tile (2048 .. 16384
// values) is shared by var_split waves per 4096 values, E = 64 / var_split
// values per lane (a 2048-value tile takes at most 32 values per lane, a
// 16384-value tile at most 16 waves).
// var_split 0 (auto): four waves per row for tiles of up to 4096 values and
// eight above (E = 8, 16, 16, 32 for tiles of 2048 .. 16384 values).  Small
// waves finish their loads early and leave the SIMD to the next ones, which
// hides memory latency better than fewer, larger waves with less cross-lane
// work per value: measured on MI355X over 64 MB inputs, [4096, 4096] 13.3 us
// (E 16) against 14.3 (E 32) and 13.7 (E 8); [2048, 8192] 12.3 against 13.0
// (E 32); [8192, 2048] 12.1 (E 8) against 13.3 (E 32); [1024, 16384] 13.0
// (E 32) against 14.7 (E 16).
void launch_rows_tile(bool vec, const float *x, int64_t rows, int64_t n, int64_t ld, int64_t ddof, float *var,
                      float *mean, hipStream_t st) {
  const svx::RowsPlan p = svx::rows_plan(n, g_tune.var_split);
  switch (p.E * 100 + p.W) {
    case 401: launch_rows_ew<4, 1>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 1601: launch_rows_ew<16, 1>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 3201: launch_rows_split<32, 1>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 1602: launch_rows_split<16, 2>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 804: launch_rows_split<8, 4>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 6401: launch_rows_ew<64, 1>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 3202: launch_rows_split<32, 2>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 1604: launch_rows_split<16, 4>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 808: launch_rows_split<8, 8>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 6402: launch_rows_split<64, 2>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 3204: launch_rows_split<32, 4>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 1608: launch_rows_split<16, 8>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 816: launch_rows_split<8, 16>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 6404: launch_rows_ew<64, 4>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 3208: launch_rows_split<32, 8>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 1616: launch_rows_split<16, 16>(vec, x, rows, n, ld, ddof, var, mean, st); break;
    case 3216:  // 16 waves of 32 values (per-lane loads)
      if (vec) launch_rows_t<32, 16, true, 1, false>(x, rows, n, ld, ddof, var, mean, st);
      else launch_rows_t<32, 16, false, 1, false>(x, rows, n, ld, ddof, var, mean, st);
      break;
    default:  // 16 waves of 64 values
      if (vec) launch_rows_t<64, 16, true, 1, false>(x, rows, n, ld, ddof, var, mean, st);
      else launch_rows_t<64, 16, false, 1, false>(x, rows, n, ld, ddof, var, mean, st);
      break;
  }
}

// Axis 0, short columns (R <= E rows, E <= 16, R < 16): each lane owns four adjacent
// columns (one 16-byte load per row, 16-byte aligned base and a width
// divisible by 4) and all three trees are in-lane: no cross-lane levels, no
// LDS, no barrier.  Rows past R are the +0 padding of the column's tree.
template <int E>
__global__ __launch_bounds__(256) void k_cols_short(const float *__restrict__ x, int64_t R, int64_t C, int64_t ddof,
                                                    float *__restrict__ var_out, float *__restrict__ mean_out,
                                                    int64_t b0) {
  const int64_t c0 = ((b0 + blockIdx.x) * 256 + threadIdx.x) * 4;
  if (c0 >= C) return;
  const float *__restrict__ p = x + c0;
  float v[4][E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const float4 g = *reinterpret_cast<const float4 *>(p + svx::clamp_last<int64_t>(i, R) * C);
    v[0][i] = g.x;
    v[1][i] = g.y;
    v[2][i] = g.z;
    v[3][i] = g.w;
  }
  const int valid = (int)R;  // R <= E
  float var4[4], mean4[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x0 = v[k][0];
#pragma unroll
    for (int i = 0; i < E; ++i) v[k][i] = (i < valid) ? v[k][i] - x0 : 0.0f;
    const float m = sv::root_value_k<sv::Y_KIND>(sv::lane_tree<sv::Y_LEAF, 0, E, E>(v[k])) / (float)R;
    Node nd, nq;
    sv::lane_tree_dq<true, 0, E, E>(v[k], m, valid, nd, nq);
    finalize(nd, nq, x0, m, R, ddof, &var4[k], &mean4[k]);
  }
  // one 16-byte store per output (c0 is a multiple of 4, the outputs 16-byte
  // aligned when they are; else four 4-byte stores)
  auto store4 = [&](float *out, const float (&t)[4]) {
    float *o = out + c0;
    if ((reinterpret_cast<uintptr_t>(out) & 15u) == 0) {
      *reinterpret_cast<float4 *>(o) = make_float4(t[0], t[1], t[2], t[3]);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = t[k];
    }
  };
  store4(var_out, var4);
  if (mean_out) store4(mean_out, mean4);
}

void launch_cols_short(const float *x, int64_t R, int64_t C, int64_t ddof, float *var, float *mean, hipStream_t st) {
  const int e = svx::cols_short_e(R);
  svh::in_batches((C / 4 + 255) / 256, 1, 256, [&](int64_t b0, int64_t nb) {
    const dim3 grid((unsigned)nb), block(256);
    switch (e) {
      case 2: k_cols_short<2><<<grid, block, 0, st>>>(x, R, C, ddof, var, mean, b0); break;
      case 4: k_cols_short<4><<<grid, block, 0, st>>>(x, R, C, ddof, var, mean, b0); break;
      case 8: k_cols_short<8><<<grid, block, 0, st>>>(x, R, C, ddof, var, mean, b0); break;
      default: k_cols_short<16><<<grid, block, 0, st>>>(x, R, C, ddof, var, mean, b0); break;
    }
  });
}

// Lane per column (k_var_cols): E rows per lane, W waves, 64 columns per
// workgroup.
template <int V>
void launch_cols_lane(const float *x, int64_t R, int64_t C, int64_t ddof, float *var, float *mean, hipStream_t st) {
  const svx::RowsPlan p = svx::cols_lane_plan(R);
#define SV_COLS(E, W)                                                                                    \
  svh::in_batches((C + 63) / 64, 1, 64 * W, [&](int64_t b0, int64_t nb) {                                \
    k_var_cols<E, W, V><<<dim3((unsigned)nb), dim3(64 * W), 0, st>>>(x, R, C, ddof, var, mean, b0);      \
  })
  switch (p.E * 100 + p.W) {
    case 401: SV_COLS(4, 1); break;
    case 1601: SV_COLS(16, 1); break;
    case 6401: SV_COLS(64, 1); break;
    case 6402: SV_COLS(64, 2); break;
    case 6404: SV_COLS(64, 4); break;
    case 6408: SV_COLS(64, 8); break;
    default: SV_COLS(64, 16); break;
  }
#undef SV_COLS
}

// The ablation row "shift + centring, Kahan sequential scan" of the method
// page's §4: the local mean from the plain tree of y (as in the method),
// then S2 summed by Kahan's compensated recurrence in index order, one value
// after the other, and var = max(S2 / n, 0) with the ddof rescale (no
// two-term step).  The scan is serial per slice, so a lane owns a slice and
// a wave 64 slices.  Axis 1 rows reach the lanes through LDS tiles of 64 rows
// by 64 values (loaded 1 KiB per instruction, written and read back 16 bytes
// per lane, rows 68 floats apart);
// axis 0 columns are read directly, one row of the wave's 64 columns per
// load.  Two passes over the data: the plain tree of y (64-value chunks in
// registers, the chunk nodes merged in tree order by a binary counter whose
// state is the same in every lane), then the scan.
using svx::KS_T;                         // values per chunk (tile width)
constexpr int KS_LD = KS_T + 4;          // LDS tile row stride: 16-byte aligned rows, 16 lanes per bank cycle
using svx::KS_LEVELS;                    // chunk-tree levels: 2^16 chunks
template <bool AX1, bool VEC>
__global__ __launch_bounds__(64) void k_var_kahan(const float *__restrict__ x, int64_t nsl, int64_t n, int64_t ld,
                                                  int64_t ddof, float *__restrict__ var_out,
                                                  float *__restrict__ mean_out) {
  __shared__ float4 tile4[AX1 ? KS_T * KS_LD / 4 : 1];
  float *const tile = reinterpret_cast<float *>(tile4);
  const int lane = threadIdx.x;
  const int64_t s0 = (int64_t)blockIdx.x * 64;
  const int64_t sl = s0 + lane;
  const bool real = sl < nsl;
  const int64_t slc = svx::clamp_last(sl, nsl);  // lanes past the last slice read it again
  const int64_t nch = (n + KS_T - 1) / KS_T;

  // A chunk is loaded in two steps, so that the next chunk's loads are in
  // flight while the current one is reduced: issue() fills raw registers
  // (every load issued, at indices clamped to the data), lanes() turns them
  // into this lane's values v[k] = slice[c*64 + k] (through the LDS tile on
  // axis 1).  Values past n are masked by the callers.
  auto issue = [&](int64_t c, float(&raw)[KS_T]) {
    c = svx::clamp_last(c, nch);
    if constexpr (AX1) {
      // lane L loads values 4 (L mod 16) .. +3 of the chunk in row 4j + L/16
      // of the wave's 64 rows: 16 bytes at once when the group lies inside
      // the row and rows are 16-byte aligned (VEC), else one by one
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = 4 * j + (lane >> 4);
        const int64_t row = svx::clamp_last(s0 + r, nsl);
        const int64_t col = c * KS_T + 4 * (lane & 15);
        const float *__restrict__ q = x + row * ld;
        float4 g;
        if (VEC && col + 3 < n) {
          g = *reinterpret_cast<const float4 *>(q + col);
        } else {
          g = make_float4(q[svx::clamp_last(col, n)], q[svx::clamp_last(col + 1, n)],
                          q[svx::clamp_last(col + 2, n)], q[svx::clamp_last(col + 3, n)]);
        }
        raw[4 * j] = g.x; raw[4 * j + 1] = g.y; raw[4 * j + 2] = g.z; raw[4 * j + 3] = g.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < KS_T; ++k) {
        const int64_t i = c * KS_T + k;
        raw[k] = x[svx::clamp_last(i, n) * ld + slc];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto lanes = [&](const float(&raw)[KS_T], float(&v)[KS_T]) {
    if constexpr (AX1) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        *reinterpret_cast<float4 *>(tile + (4 * j + (lane >> 4)) * KS_LD + 4 * (lane & 15)) =
            make_float4(raw[4 * j], raw[4 * j + 1], raw[4 * j + 2], raw[4 * j + 3]);
      sv::wave_lds_sync();
#pragma unroll
      for (int k = 0; k < KS_T / 4; ++k) {
        const float4 t = *reinterpret_cast<const float4 *>(tile + lane * KS_LD + 4 * k);
        v[4 * k] = t.x; v[4 * k + 1] = t.y; v[4 * k + 2] = t.z; v[4 * k + 3] = t.w;
      }
      sv::wave_lds_sync();
    } else {
#pragma unroll
      for (int k = 0; k < KS_T; ++k) v[k] = raw[k];
    }
  };
  // every chunk c < nch through `body`, two register sets alternating
  auto stream = [&](auto &&body) {
    float ra[KS_T], rb[KS_T], v[KS_T];
    issue(0, ra);
    for (int64_t c = 0; c < nch; c += 2) {
      issue(c + 1, rb);
      lanes(ra, v);
      body(c, v);
      issue(c + 2, ra);
      if (c + 1 < nch) {  // uniform
        lanes(rb, v);
        body(c + 1, v);
      }
    }
  };
  const float x0 = AX1 ? x[slc * ld] : x[slc];

  // pass 1: the plain tree of y
  float st[KS_LEVELS];
#pragma unroll
  for (int lv = 0; lv < KS_LEVELS; ++lv) st[lv] = 0.0f;
  stream([&](int64_t c, float(&v)[KS_T]) {
#pragma unroll
    for (int k = 0; k < KS_T; ++k) v[k] = (c * KS_T + k < n) ? v[k] - x0 : 0.0f;
    float carry = sv::lane_tree<sv::LEAF_PLAIN, 0, KS_T, KS_T>(v).s;
    bool placed = false;
#pragma unroll
    for (int lv = 0; lv < KS_LEVELS; ++lv) {
      if (!placed) {
        if ((c >> lv) & 1) {
          carry = st[lv] + carry;
        } else {
          st[lv] = carry;
          placed = true;
        }
      }
    }
  });
  // the pending left nodes, combined in tree order (their right siblings
  // beyond the data are zero subtrees), then the plain tree's root rule
  float sy = 0.0f;
  bool any = false;
#pragma unroll
  for (int lv = 0; lv < KS_LEVELS; ++lv) {
    if ((nch >> lv) & 1) {
      sy = any ? st[lv] + sy : st[lv];
      any = true;
    }
  }
  sy = sy + 0.0f;
  const float fn = (float)n;
  const float m = sy / fn;

  // pass 2: Kahan's recurrence over q_i = (y_i - m)^2 in index order
  float sum = 0.0f, corr = 0.0f;
  stream([&](int64_t c, float(&v)[KS_T]) {
#pragma unroll
    for (int k = 0; k < KS_T; ++k) {
      if (c * KS_T + k < n) {  // uniform
        const float d = (v[k] - x0) - m;
        const float q = d * d;
        const float yk = q - corr;
        const float t = sum + yk;
        corr = (t - sum) - yk;
        sum = t;
      }
    }
  });
  if (real) {
    const float a = sum / fn;
    float var = (a != a) ? a : ((a > 0.0f) ? a : 0.0f);
    if (ddof != 0) {
      int64_t den = n - ddof;
      if (den < 0) den = 0;
      var = var * (fn / (float)den);
    }
    var_out[sl] = var;
    if (mean_out) mean_out[sl] = x0 + m;
  }
}

// A variant over rows of more than 16384 values: the method's long-row chunk
// launches (k_long_rows, k_long_top) with the variant's shift, tree of y,
// local mean and step 4.  Workspace: long_ws of `rows` slices.
template <int V>
void launch_long_variant(bool vec, const float *x, int64_t rows, int64_t n, int64_t ld, int64_t ddof,
                         void *workspace, float *var, float *mean, hipStream_t st) {
  const int64_t nch = (n + LS_ROW_CHUNK - 1) / LS_ROW_CHUNK;
  const LongWs ws = long_ws(workspace, rows, nch);
  const dim3 grid((unsigned)(rows * nch)), block(256), top((unsigned)rows);
  if (vec) k_long_rows<0, true, 1, V><<<grid, block, 0, st>>>(x, n, ld, nch, ws);
  else k_long_rows<0, false, 1, V><<<grid, block, 0, st>>>(x, n, ld, nch, ws);
  launch_long_top<0, 1, V>(x, n, ld, nch, ddof, ws, var, mean, top, st);
  if (vec) k_long_rows<1, true, 1, V><<<grid, block, 0, st>>>(x, n, ld, nch, ws);
  else k_long_rows<1, false, 1, V><<<grid, block, 0, st>>>(x, n, ld, nch, ws);
  launch_long_top<1, 1, V>(x, n, ld, nch, ddof, ws, var, mean, top, st);
}

// xt = the transpose of x ([R, C] -> [C, R], both row-major): 32 x 32 tiles
// through LDS, coalesced on both sides; workgroup b0 + blockIdx.x takes tile
// (b / ceil(C/32), b mod ceil(C/32)).  A copy: the values keep their bits.
__global__ __launch_bounds__(256) void k_transpose(const float *__restrict__ x, int64_t R, int64_t C,
                                                   float *__restrict__ xt, int64_t b0) {
  __shared__ float t[32][33];
  const int64_t tiles_c = (C + 31) / 32;
  const int64_t b = b0 + blockIdx.x;
  const int64_t r0 = (b / tiles_c) * 32, c0 = (b % tiles_c) * 32;
  const int lx = threadIdx.x & 31, ly = threadIdx.x >> 5;  // 32 x 8 threads
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int64_t r = r0 + ly + k, c = c0 + lx;
    if (r < R && c < C) t[ly + k][lx] = x[r * C + c];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int64_t c = c0 + ly + k, r = r0 + lx;
    if (r < R && c < C) xt[c * R + r] = t[lx][ly + k];
  }
}

template <int V>
void launch_variant(bool ax1, bool vec, const float *x, int64_t rows, int64_t cols, int64_t ddof, float *var,
                    float *mean, hipStream_t st) {
  if (ax1) {
    const int64_t n = cols;
#define SV_ROWS(E, W)                                                                                   \
  svh::in_batches(rows, 1, 64 * W, [&](int64_t r0, int64_t nr) {                                        \
    const float *xr = x + r0 * cols;                                                                    \
    float *vr = var + r0, *mr = mean ? mean + r0 : nullptr;                                             \
    if (vec) k_var_rows<E, W, true, 1, false, V><<<dim3((unsigned)nr), dim3(64 * W), 0, st>>>(xr, n, cols, ddof, vr, mr, 0); \
    else k_var_rows<E, W, false, 1, false, V><<<dim3((unsigned)nr), dim3(64 * W), 0, st>>>(xr, n, cols, ddof, vr, mr, 0);   \
  })
    const svx::RowsPlan p = svx::variant_rows_plan(n);
    switch (p.E * 100 + p.W) {
      case 401: SV_ROWS(4, 1); break;
      case 1601: SV_ROWS(16, 1); break;
      case 3202: SV_ROWS(32, 2); break;
      default: SV_ROWS(64, 4); break;
    }
#undef SV_ROWS
  } else {
    launch_cols_lane<V>(x, rows, cols, ddof, var, mean, st);
  }
}

// ------------------------------------------------------------------ tree sum, no workspace argument

// The tree sum's workspace as a file-scope device array (ticket counters,
// then partial nodes: the layout of a caller's workspace).  Every GPU the
// library runs on holds its own copy until the process ends.  Host code
// never passes this name to a kernel (on the host it is only a stand-in for
// the symbol): it takes each device's address with hipGetSymbolAddress.
constexpr size_t NOALLOC_BYTES = SUM_WS_HEADER + (size_t)(SUM_MAX_BLOCKS + SUM_MAX_BLOCKS / SUM_GROUP) * sizeof(Node);
static_assert(NOALLOC_BYTES == SV_TREE_SUM_NOALLOC_SCRATCH_BYTES, "header constant");

}  // namespace

static __device__ __align__(256) unsigned char scratch[NOALLOC_BYTES];

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[NOALLOC_MAX_DEVICES];  // each device's address of `scratch`, once set up

// The current device's address of `scratch`.  On the first call on a device
// it is looked up (with that device current) and *first is set, so that the
// caller clears the counters before their first use.
sv_status scratch_address(const char *who, void **ptr, bool *first) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SV_ERR_HIP, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
    return fail(SV_ERR_UNSUPPORTED, "%s: device %d beyond the %d devices set up", who, dev, NOALLOC_MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  *first = false;
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SV_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", who, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
    *first = true;
  }
  *ptr = g_scratch_ptr[dev];
  return SV_OK;
}

}  // namespace

// ==================================================================== C ABI

extern "C" {

int sv_abi_version(void) { return SV_ABI_VERSION; }

const char *sv_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "SV_OK";
    case SV_ERR_INVALID_ARGUMENT: return "SV_ERR_INVALID_ARGUMENT";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE";
    case SV_ERR_NO_DEVICE: return "SV_ERR_NO_DEVICE";
    case SV_ERR_HIP: return "SV_ERR_HIP";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED";
    default: return "SV_ERR_UNKNOWN";
  }
}

const char *sv_last_error_message(void) { return svh::last_error(); }

size_t sv_tree_sum_f32_workspace_size(int64_t n) {
  if (n > SUM_MAX_N) return (size_t)-1;
  return sum_workspace_bytes(n);
}

static sv_status tree_sum_impl(const char *who, bool dw, const float *x, int64_t n, float *out, void *workspace,
                               size_t workspace_bytes, void *stream) {
  if (n < 0) return fail(SV_ERR_INVALID_ARGUMENT, "%s: n = %lld < 0", who, (long long)n);
  if (n > SUM_MAX_N) return fail(SV_ERR_UNSUPPORTED, "%s: n = %lld above 2^36", who, (long long)n);
  if (!out) return fail(SV_ERR_INVALID_ARGUMENT, "%s: out is NULL", who);
  if (n > 0 && !x) return fail(SV_ERR_INVALID_ARGUMENT, "%s: x is NULL with n > 0", who);
  const size_t need = sum_workspace_bytes(n);
  if (need > 0) {
    if (!workspace) return fail(SV_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", who, need);
    if (workspace_bytes < need)
      return fail(SV_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", who, workspace_bytes, need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(SV_ERR_WORKSPACE, "%s: workspace is not 256-byte aligned", who);
  }
  const sv_status dev = check_device();
  if (dev != SV_OK) return dev;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (n == 0) {
    k_fill<<<1, 64, 0, st>>>(out, 1, 0.0f);
    return check_launch(who);
  }
  unsigned *counter = reinterpret_cast<unsigned *>(workspace);
  Node *part = reinterpret_cast<Node *>(reinterpret_cast<char *>(workspace) + SUM_WS_HEADER);
  const bool vec = aligned16(x);
  const SumPlan p = plan_sum(n, g_tune.sum_e, g_tune.sum_blocks);
  if (dw) {
    if (p.e == 16) launch_sum_dw<16>(vec, x, n, p, part, counter, out, st);
    else launch_sum_dw<32>(vec, x, n, p, part, counter, out, st);
  } else {
    if (p.e == 16) launch_sum_e<16>(vec, x, n, p, part, counter, out, st);
    else launch_sum_e<32>(vec, x, n, p, part, counter, out, st);
  }
  return check_launch(who);
}

sv_status sv_tree_sum_f32(const float *x, int64_t n, float *out, void *workspace, size_t workspace_bytes,
                          void *stream) {
  return tree_sum_impl("sv_tree_sum_f32", false, x, n, out, workspace, workspace_bytes, stream);
}

sv_status sv_tree_sum_dw_f32(const float *x, int64_t n, float *out, void *workspace, size_t workspace_bytes,
                             void *stream) {
  return tree_sum_impl("sv_tree_sum_dw_f32", true, x, n, out, workspace, workspace_bytes, stream);
}

sv_status sv_tree_sum_f32_noalloc(const float *x, int64_t n, float *out, void *stream) {
  const char *who = "sv_tree_sum_f32_noalloc";
  if (n < 0) return fail(SV_ERR_INVALID_ARGUMENT, "%s: n = %lld < 0", who, (long long)n);
  if (n > SUM_MAX_N)
    return fail(SV_ERR_UNSUPPORTED, "%s: n = %lld above 2^36, the most its %zu-byte scratch array serves", who,
                (long long)n, NOALLOC_BYTES);
  if (!out) return fail(SV_ERR_INVALID_ARGUMENT, "%s: out is NULL", who);
  if (n > 0 && !x) return fail(SV_ERR_INVALID_ARGUMENT, "%s: x is NULL with n > 0", who);
  const sv_status dev = check_device();
  if (dev != SV_OK) return dev;
  void *ptr = nullptr;
  bool first = false;
  const sv_status sc = scratch_address(who, &ptr, &first);
  if (sc != SV_OK) return sc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (first) {
    // the ticket counters start at zero (a fill kernel, no memset call);
    // every sum leaves them zero again
    k_fill<<<dim3((unsigned)(SUM_WS_HEADER / 4 + 255) / 256), 256, 0, st>>>(reinterpret_cast<float *>(ptr),
                                                                          (int64_t)(SUM_WS_HEADER / 4), 0.0f);
    const sv_status rc = check_launch(who);
    if (rc != SV_OK) return rc;
  }
  return tree_sum_impl(who, false, x, n, out, ptr, NOALLOC_BYTES, stream);
}

size_t sv_variance_f32_workspace_size(int64_t rows, int64_t cols, int axis) {
  if (rows < 0 || cols < 0) return (size_t)-1;
  if (axis != 0 && axis != 1 && axis != -1 && axis != -2) return (size_t)-1;
  if (cols > 0 && rows > VAR_MAX_ELEMS / cols) return (size_t)-1;
  const bool ax1 = (axis == 1 || axis == -1);
  const int64_t n = ax1 ? cols : rows;
  const int64_t nslices = ax1 ? rows : cols;
  if (!ax1 && (n + 63) / 64 > ((int64_t)64 * 64 << (TOP_BIG_LEVELS - 1))) return (size_t)-1;
  if (!ax1) return (n == 0 || nslices == 0) ? 0 : cols_layout(n, nslices).total;
  if (n <= ROWS_MAX_N) return 0;
  const int64_t nch = (n + LS_ROW_CHUNK - 1) / LS_ROW_CHUNK;
  if (nch > LS_MAX_CHUNKS) return (size_t)-1;
  return long_ws_bytes(nslices, nch);
}

sv_status sv_variance_f32(const float *x, int64_t rows, int64_t cols, int axis, int64_t ddof, float *var_out,
                          float *mean_out, void *workspace, size_t workspace_bytes, void *stream) {
  if (rows < 0 || cols < 0)
    return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_f32: negative shape [%lld, %lld]", (long long)rows,
                (long long)cols);
  if (axis != 0 && axis != 1 && axis != -1 && axis != -2)
    return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_f32: axis %d not in {0, 1, -1, -2}", axis);
  if (ddof < 0) return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_f32: ddof = %lld < 0", (long long)ddof);
  if (cols > 0 && rows > VAR_MAX_ELEMS / cols)
    return fail(SV_ERR_UNSUPPORTED, "sv_variance_f32: rows * cols above 2^36");
  const bool ax1 = (axis == 1 || axis == -1);
  const int64_t nslices = ax1 ? rows : cols;
  const int64_t n = ax1 ? cols : rows;
  if (nslices == 0) return ok();
  if (!var_out) return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_f32: var_out is NULL");
  if (n > 0 && !x) return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_f32: x is NULL");
  if (nslices > 0x7fffffffLL)
    return fail(SV_ERR_UNSUPPORTED, "sv_variance_f32: %lld slices exceed the grid", (long long)nslices);
  const bool is_long = ax1 && n > ROWS_MAX_N;
  const int64_t nch = is_long ? (n + LS_ROW_CHUNK - 1) / LS_ROW_CHUNK : 0;
  if (is_long && nch > LS_MAX_CHUNKS)
    return fail(SV_ERR_UNSUPPORTED, "sv_variance_f32: slices of length %lld exceed %d chunks", (long long)n,
                LS_MAX_CHUNKS);
  // axis 0: the per-column trees hold up to 64 * 64 * 2^(TOP_BIG_LEVELS - 1)
  // chunk nodes; chunks are at least 64 rows
  if (!ax1 && (n + 63) / 64 > ((int64_t)64 * 64 << (TOP_BIG_LEVELS - 1)))
    return fail(SV_ERR_UNSUPPORTED, "sv_variance_f32: columns of %lld rows exceed the chunk trees", (long long)n);
  if (is_long || (!ax1 && n > 0)) {
    const size_t need = is_long ? long_ws_bytes(nslices, nch) : cols_layout(n, nslices).total;
    if (!workspace) return fail(SV_ERR_WORKSPACE, "sv_variance_f32: workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
      return fail(SV_ERR_WORKSPACE, "sv_variance_f32: workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(SV_ERR_WORKSPACE, "sv_variance_f32: workspace is not 256-byte aligned");
  }
  const sv_status dev = check_device();
  if (dev != SV_OK) return dev;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (n == 0) {
    const unsigned blocks = (unsigned)((nslices + 255) / 256);
    k_fill<<<blocks, 256, 0, st>>>(var_out, nslices, __builtin_nanf(""));
    if (mean_out) k_fill<<<blocks, 256, 0, st>>>(mean_out, nslices, __builtin_nanf(""));
    return check_launch("sv_variance_f32");
  }
  if (!ax1 && cols == 1 && rows <= (int64_t)LS_MAX_CHUNKS * LS_ROW_CHUNK) {
    // A single column [rows, 1] is one contiguous slice, as is the single row
    // [1, rows]: the same values in the same order, hence the same tree and
    // the same bits.  The row form reads it with wide loads; its workspace
    // (none, or 24 bytes per 16384-value chunk) is smaller than the column
    // form's, which the caller sized.
    return sv_variance_f32(x, 1, rows, 1, ddof, var_out, mean_out, workspace, workspace_bytes, stream);
  }
  const svx::RouteKnobs knobs{g_tune.var_long_rows,  g_tune.var_cols_once,  g_tune.var_cols_single_max,
                              g_tune.var_short_rows, g_tune.var_cols_short, g_tune.var_cols_one,
                              g_tune.var_cols_pairs};
  const bool vec16 = aligned16(x) && cols % 4 == 0;
  // Columns of 1025..4096 rows: sixteen whole columns per workgroup of up to
  // 16 waves (four row groups of E rows per wave; a shorter column launches
  // only the waves its rows reach), read once -- unless the grid would leave
  // the chip's last round of workgroups mostly empty (each workgroup holds
  // 256 KB in registers, so one or two fit a CU).  MODE 1 when every wave is
  // full (2048 or 4096 rows), else MODE 2.
  using ColsOneFn = void (*)(const float *, int64_t, int64_t, int64_t, float *, float *, int);
  ColsOneFn one_read = nullptr;
  svx::ColsLongPlan one_plan{};
  bool fills = false;
  if (svx::cols_one_read_candidate(ax1, n, knobs)) {
    one_plan = svx::cols_long_plan(n, cols);
    const bool exact = one_plan.mode == 1, big = one_plan.E == 64;
    one_read = big ? (exact ? k_cols_one<1, 16, 4, false, 64, 1> : k_cols_one<1, 16, 4, false, 64, 2>)
                   : (exact ? k_cols_one<1, 16, 4, false, 32, 1> : k_cols_one<1, 16, 4, false, 32, 2>);
    int per_cu = 0, cus = 0, dev = 0;
    if (g_tune.var_cols_once != 2 && hipGetDevice(&dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(one_read),
                                                     64 * one_plan.waves, 0) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && per_cu > 0) {
      const int64_t cap = (int64_t)per_cu * cus, rounds = (one_plan.blocks + cap - 1) / cap;
      fills = 4 * one_plan.blocks >= 3 * rounds * cap;
    }
  }
  switch (svx::f32_route(rows, cols, ax1, vec16, knobs, fills)) {
    case svx::Route::LONG_ROWS_CHUNKED: {
      const LongWs ws = long_ws(workspace, nslices, nch);
      const dim3 grid((unsigned)(rows * nch)), block(256), top((unsigned)rows);
      if (vec16) k_long_rows<0, true><<<grid, block, 0, st>>>(x, n, cols, nch, ws);
      else k_long_rows<0, false><<<grid, block, 0, st>>>(x, n, cols, nch, ws);
      launch_long_top<0>(x, n, cols, nch, ddof, ws, var_out, mean_out, top, st);
      if (vec16) k_long_rows<1, true><<<grid, block, 0, st>>>(x, n, cols, nch, ws);
      else k_long_rows<1, false><<<grid, block, 0, st>>>(x, n, cols, nch, ws);
      launch_long_top<1>(x, n, cols, nch, ddof, ws, var_out, mean_out, top, st);
      break;
    }
    case svx::Route::COLS_PAIRS:
      // two columns: the matrix is one row of `rows` pairs (two interleaved
      // slices, the same values in the same order per column), in chunks of
      // LS_ROW_CHUNK / 2 rows read with wide per-lane loads; its workspace is
      // smaller than the column chunks' that the caller sized
      launch_long_pairs(aligned16(x) && rows % 2 == 0, x, 1, rows, 2 * rows, ddof, workspace, var_out, mean_out, st);
      break;
    case svx::Route::COLS_ONE_READ:
      svh::in_batches(one_plan.blocks, 1, 64 * one_plan.waves, [&](int64_t b0, int64_t nb) {
        one_read<<<dim3((unsigned)nb), dim3(64 * (unsigned)one_plan.waves), 0, st>>>(x, rows, cols, ddof, var_out,
                                                                                  mean_out, (int)b0);
      });
      break;
    case svx::Route::COLS_CHUNKED: {
      const ColsWs ws = cols_ws(workspace, cols_layout(rows, cols));
      if (vec16) launch_cols_v<4>(x, rows, cols, ddof, ws, var_out, mean_out, st);
      else launch_cols_v<1>(x, rows, cols, ddof, ws, var_out, mean_out, st);
      break;
    }
    case svx::Route::ROWS_SEG: launch_rows_seg(x, rows, n, cols, ddof, var_out, mean_out, st); break;
    case svx::Route::ROWS_TILE: launch_rows_tile(vec16, x, rows, n, cols, ddof, var_out, mean_out, st); break;
    // columns of at most 15 rows: four columns per lane, every tree in-lane
    // (at 16 rows the lane kernel's lanes hold exactly 16: [16, 1000000] 12.7
    // against 16.7 us);
    case svx::Route::COLS_SHORT: launch_cols_short(x, rows, cols, ddof, var_out, mean_out, st); break;
    // more than 64 rows: one launch of G row groups per wave, four columns
    // per lane for long columns (513..1024 rows) of wide matrices, else one:
    // [1000, 20000] 31.0 against 37.1 us, [300, 50000] 34.1 against 24.0,
    // [512, 4096] 7.0 against 4.8
    case svx::Route::COLS_ONE4:
      if (vec16) launch_cols_one<true>(x, rows, cols, ddof, var_out, mean_out, st);
      else launch_cols_one<false>(x, rows, cols, ddof, var_out, mean_out, st);
      break;
    case svx::Route::COLS_ONE1: launch_cols_one1(x, rows, cols, ddof, var_out, mean_out, st); break;
    // otherwise the lane-per-column kernel, whose lanes hold exactly 4, 16
    // or 64 rows (faster than G row groups there: [4, 1000000] 6.5 against
    // 16 us)
    case svx::Route::COLS_LANE: launch_cols_lane<V_KERNEL>(x, rows, cols, ddof, var_out, mean_out, st); break;
  }
  return check_launch("sv_variance_f32");
}

size_t sv_variance_variant_f32_workspace_size(int64_t rows, int64_t cols, int axis, int variant) {
  if (rows < 0 || cols < 0 || (axis != 0 && axis != 1 && axis != -1 && axis != -2)) return (size_t)-1;
  if (variant < V_KERNEL || variant > V_SHIFT_KAHAN_NO2T) return (size_t)-1;
  if (cols > 0 && rows > VAR_MAX_ELEMS / cols) return (size_t)-1;
  const bool ax1 = (axis == 1 || axis == -1);
  const int64_t n = ax1 ? cols : rows, nsl = ax1 ? rows : cols;
  if (variant == V_SHIFT_KAHAN_NO2T) return n > ((int64_t)KS_T << KS_LEVELS) ? (size_t)-1 : 0;
  if (n == 0 || nsl == 0 || (ax1 ? n <= ROWS_MAX_N : n <= COLS_MAX_R)) return 0;
  const int64_t nch = (n + LS_ROW_CHUNK - 1) / LS_ROW_CHUNK;
  if (n > ROWS_MAX_N && nch > LS_MAX_CHUNKS) return (size_t)-1;
  // axis 0: the transposed matrix, then (columns of more than 16384 rows)
  // the chunk nodes of its rows
  size_t b = ax1 ? 0 : round256((size_t)rows * (size_t)cols * sizeof(float));
  if (n > ROWS_MAX_N) b += long_ws_bytes(nsl, nch);
  return b;
}

}  // extern "C"

namespace {

sv_status variant_f32(const char *who, const float *x, int64_t rows, int64_t cols, int axis, int64_t ddof,
                      int variant, float *var_out, float *mean_out, void *workspace, size_t workspace_bytes,
                      bool has_ws, void *stream) {
  if (rows < 0 || cols < 0)
    return fail(SV_ERR_INVALID_ARGUMENT, "%s: negative shape [%lld, %lld]", who, (long long)rows, (long long)cols);
  if (axis != 0 && axis != 1 && axis != -1 && axis != -2)
    return fail(SV_ERR_INVALID_ARGUMENT, "%s: axis %d not in {0, 1, -1, -2}", who, axis);
  if (ddof < 0) return fail(SV_ERR_INVALID_ARGUMENT, "%s: ddof = %lld < 0", who, (long long)ddof);
  if (variant != V_KERNEL && variant != V_COMP_Y && variant != V_REFERENCE && variant != V_NAIVE &&
      variant != V_SHIFT_PLAIN_NO2T && variant != V_SHIFT_PLAIN_2T && variant != V_NOSHIFT_COMP_2T &&
      variant != V_SHIFT_COMP_NO2T && variant != V_SHIFT_KAHAN_NO2T)
    return fail(SV_ERR_INVALID_ARGUMENT, "%s: unknown variant %d", who, variant);
  const bool ax1 = (axis == 1 || axis == -1);
  const int64_t nslices = ax1 ? rows : cols;
  const int64_t n = ax1 ? cols : rows;
  if (cols > 0 && rows > VAR_MAX_ELEMS / cols) return fail(SV_ERR_UNSUPPORTED, "%s: rows * cols above 2^36", who);
  if (nslices == 0) return ok();
  if (!var_out) return fail(SV_ERR_INVALID_ARGUMENT, "%s: var_out is NULL", who);
  if (n > 0 && !x) return fail(SV_ERR_INVALID_ARGUMENT, "%s: x is NULL", who);
  // the tree variants take one workgroup per slice (rows of up to 16384
  // values, columns of up to 1024) or, with a workspace, the long-slice
  // launches; the Kahan scan takes a lane per slice and slices of up to 2^16
  // chunks of 64 values
  const bool kahan = variant == V_SHIFT_KAHAN_NO2T;
  const bool single = ax1 ? n <= ROWS_MAX_N : n <= COLS_MAX_R;
  const int64_t nch = (n + LS_ROW_CHUNK - 1) / LS_ROW_CHUNK;
  if (nslices > 0x7fffffffLL || (kahan ? n > ((int64_t)KS_T << KS_LEVELS)
                                       : (!single && (!has_ws || (n > ROWS_MAX_N && nch > LS_MAX_CHUNKS)))))
    return fail(SV_ERR_UNSUPPORTED, "%s: shape [%lld, %lld] along axis %d not supported%s", who, (long long)rows,
                (long long)cols, axis,
                (!kahan && !single && !has_ws) ? " (longer slices: sv_variance_variant_ws_f32)" : "");
  const size_t need = kahan || single ? 0 : sv_variance_variant_f32_workspace_size(rows, cols, axis, variant);
  if (need > 0) {
    if (!workspace) return fail(SV_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", who, need);
    if (workspace_bytes < need)
      return fail(SV_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", who, workspace_bytes, need);
    if (!svh::aligned256(workspace)) return fail(SV_ERR_WORKSPACE, "%s: workspace is not 256-byte aligned", who);
  }
  const sv_status dev = check_device();
  if (dev != SV_OK) return dev;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (n == 0) {
    const unsigned blocks = (unsigned)((nslices + 255) / 256);
    k_fill<<<blocks, 256, 0, st>>>(var_out, nslices, __builtin_nanf(""));
    if (mean_out) k_fill<<<blocks, 256, 0, st>>>(mean_out, nslices, __builtin_nanf(""));
    return check_launch(who);
  }
  const bool vec = aligned16(x) && (cols % 4 == 0);
  if (variant == V_SHIFT_KAHAN_NO2T) {
    const dim3 grid((unsigned)((nslices + 63) / 64)), block(64);
    if (!ax1) k_var_kahan<false, false><<<grid, block, 0, st>>>(x, nslices, n, cols, ddof, var_out, mean_out);
    else if (vec) k_var_kahan<true, true><<<grid, block, 0, st>>>(x, nslices, n, cols, ddof, var_out, mean_out);
    else k_var_kahan<true, false><<<grid, block, 0, st>>>(x, nslices, n, cols, ddof, var_out, mean_out);
    return check_launch(who);
  }
  // Slices longer than one workgroup: columns are transposed into the
  // workspace first (the same values in the same order, so the same trees),
  // then rows of more than 16384 values take the chunk launches.
  const float *xs = x;
  int64_t srows = rows, scols = cols;
  bool svec = vec, sax1 = ax1;
  char *wp = reinterpret_cast<char *>(workspace);
  if (!single && !ax1) {
    float *xt = reinterpret_cast<float *>(wp);
    const int64_t tiles = ((rows + 31) / 32) * ((cols + 31) / 32);
    svh::in_batches(tiles, 1, 256, [&](int64_t b0, int64_t nb) {
      k_transpose<<<dim3((unsigned)nb), dim3(256), 0, st>>>(x, rows, cols, xt, b0);
    });
    wp += round256((size_t)rows * (size_t)cols * sizeof(float));
    xs = xt;
    srows = cols;
    scols = rows;
    svec = scols % 4 == 0;  // the workspace is 256-byte aligned
    sax1 = true;
  }
#define SV_VARIANT(V_)                                                                                           do {                                                                                                             if (sax1 && scols > ROWS_MAX_N)                                                                                   launch_long_variant<V_>(svec, xs, srows, scols, scols, ddof, wp, var_out, mean_out, st);                     else                                                                                                             launch_variant<V_>(sax1, svec, xs, srows, scols, ddof, var_out, mean_out, st);                             } while (0)
  switch (variant) {
    case V_KERNEL: SV_VARIANT(V_KERNEL); break;
    case V_COMP_Y: SV_VARIANT(V_COMP_Y); break;
    case V_REFERENCE: SV_VARIANT(V_REFERENCE); break;
    case V_NAIVE: SV_VARIANT(V_NAIVE); break;
    case V_SHIFT_PLAIN_NO2T: SV_VARIANT(V_SHIFT_PLAIN_NO2T); break;
    case V_SHIFT_PLAIN_2T: SV_VARIANT(V_SHIFT_PLAIN_2T); break;
    case V_NOSHIFT_COMP_2T: SV_VARIANT(V_NOSHIFT_COMP_2T); break;
    default: SV_VARIANT(V_SHIFT_COMP_NO2T); break;
  }
#undef SV_VARIANT
  return check_launch(who);
}

}  // namespace

extern "C" {

sv_status sv_variance_variant_f32(const float *x, int64_t rows, int64_t cols, int axis, int64_t ddof, int variant,
                                  float *var_out, float *mean_out, void *stream) {
  return variant_f32("sv_variance_variant_f32", x, rows, cols, axis, ddof, variant, var_out, mean_out, nullptr, 0,
                     false, stream);
}

sv_status sv_variance_variant_ws_f32(const float *x, int64_t rows, int64_t cols, int axis, int64_t ddof,
                                     int variant, float *var_out, float *mean_out, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  return variant_f32("sv_variance_variant_ws_f32", x, rows, cols, axis, ddof, variant, var_out, mean_out, workspace,
                     workspace_bytes, true, stream);
}


size_t sv_variance_c64_workspace_size(int64_t rows, int64_t cols, int axis) {
  if (rows < 0 || cols < 0) return (size_t)-1;
  if (axis != 0 && axis != 1 && axis != -1 && axis != -2) return (size_t)-1;
  if (cols > 0 && rows > VAR_MAX_ELEMS / 2 / cols) return (size_t)-1;
  const bool ax1 = (axis == 1 || axis == -1);
  const int64_t nslices = ax1 ? rows : cols;
  if (ax1 && cols <= C64_FUSED_MAX_N) return 0;  // one pass, no staging
  const int64_t pair_chunks = (cols + LS_ROW_CHUNK / 2 - 1) / (LS_ROW_CHUNK / 2);
  if (ax1 && pair_chunks <= LS_MAX_CHUNKS)  // per-part variances, then the pair chunks' nodes
    return round256((size_t)2 * rows * sizeof(float)) + long_ws_bytes(2 * rows, pair_chunks);
  const size_t inner = ax1 ? sv_variance_f32_workspace_size(2 * rows, cols, 1)
                           : sv_variance_f32_workspace_size(rows, 2 * cols, 0);
  if (inner == (size_t)-1) return (size_t)-1;
  size_t b = round256((size_t)2 * nslices * sizeof(float));  // per-component variances
  if (ax1) b += round256((size_t)2 * rows * cols * sizeof(float));  // split rows
  return b + inner;
}

sv_status sv_variance_c64(const float *z, int64_t rows, int64_t cols, int axis, int64_t ddof, float *var_out,
                          float *mean_out, void *workspace, size_t workspace_bytes, void *stream) {
  if (rows < 0 || cols < 0)
    return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_c64: negative shape [%lld, %lld]", (long long)rows,
                (long long)cols);
  if (axis != 0 && axis != 1 && axis != -1 && axis != -2)
    return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_c64: axis %d not in {0, 1, -1, -2}", axis);
  if (ddof < 0) return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_c64: ddof = %lld < 0", (long long)ddof);
  const bool ax1 = (axis == 1 || axis == -1);
  const int64_t nslices = ax1 ? rows : cols;
  const size_t need = sv_variance_c64_workspace_size(rows, cols, axis);
  if (need == (size_t)-1) return fail(SV_ERR_UNSUPPORTED, "sv_variance_c64: shape [%lld, %lld] not supported",
                                      (long long)rows, (long long)cols);
  if (nslices == 0) return ok();
  if (nslices > 0x7fffffffLL)
    return fail(SV_ERR_UNSUPPORTED, "sv_variance_c64: %lld slices exceed the grid", (long long)nslices);
  if (!var_out) return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_c64: var_out is NULL");
  if (rows * cols > 0 && !z) return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_c64: z is NULL");
  if (reinterpret_cast<uintptr_t>(z) & 7u) return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_c64: z is not 8-byte aligned");
  if (need > 0) {
    if (!workspace) return fail(SV_ERR_WORKSPACE, "sv_variance_c64: workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
      return fail(SV_ERR_WORKSPACE, "sv_variance_c64: workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(SV_ERR_WORKSPACE, "sv_variance_c64: workspace is not 256-byte aligned");
  }
  const sv_status dev = check_device();
  if (dev != SV_OK) return dev;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (ax1 && cols <= C64_FUSED_MAX_N) {
    if (cols == 0) {  // empty rows: var and both mean parts are NaN
      k_fill<<<dim3((unsigned)((rows + 255) / 256)), 256, 0, st>>>(var_out, rows, __builtin_nanf(""));
      if (mean_out) k_fill<<<dim3((unsigned)((2 * rows + 255) / 256)), 256, 0, st>>>(mean_out, 2 * rows, __builtin_nanf(""));
      return check_launch("sv_variance_c64");
    }
    // rows start 16-byte aligned when z is and cols is even
    const bool vec = aligned16(z) && (cols % 2 == 0);
#define SV_ROWS_C64(E, W)                                                                                 \
  svh::in_batches(rows, 1, 64 * svx::rows_waves(cols, E, W), [&](int64_t r0, int64_t nr) {             \
    const float *zr = z + 2 * r0 * cols;                                                                \
    float *mr = mean_out ? mean_out + 2 * r0 : nullptr;                                                 \
    const dim3 block(64 * svx::rows_waves(cols, E, W));  /* only the waves the row reaches */          \
    if (vec) k_var_rows_c64<E, W, true><<<dim3((unsigned)nr), block, 0, st>>>(zr, cols, ddof, var_out + r0, mr); \
    else k_var_rows_c64<E, W, false><<<dim3((unsigned)nr), block, 0, st>>>(zr, cols, ddof, var_out + r0, mr);   \
  })
    if (cols <= SEG_MAX_N && g_tune.var_short_rows) {
      const int vw2 = vec ? 2 : 1;
      const StepConsts sk = step_consts(cols, ddof);
#define SV_SEG_C64(E, S)                                                                                \
  svh::in_batches(rows, 4 * (64 / S), 256, [&](int64_t r0, int64_t nr) {                                \
    const dim3 sgrid((unsigned)((nr + 4 * (64 / S) - 1) / (4 * (64 / S))));                             \
    const float *zr = z + 2 * r0 * cols;                                                                \
    float *vr = var_out + r0, *mr = mean_out ? mean_out + 2 * r0 : nullptr;                             \
    if (vw2 == 2) k_var_rows_c64_seg<E, S, 2><<<sgrid, dim3(256), 0, st>>>(zr, nr, cols, sk, vr, mr);   \
    else k_var_rows_c64_seg<E, S, 1><<<sgrid, dim3(256), 0, st>>>(zr, nr, cols, sk, vr, mr);           \
  })
      const svx::SegPlan sp = svx::seg_plan(cols);
      switch (sp.E * 100 + sp.S) {
        case 401: SV_SEG_C64(4, 1); break;
        case 801: SV_SEG_C64(8, 1); break;
        case 1601: SV_SEG_C64(16, 1); break;
        case 1602: SV_SEG_C64(16, 2); break;
        case 1604: SV_SEG_C64(16, 4); break;
        case 1608: SV_SEG_C64(16, 8); break;
        case 1616: SV_SEG_C64(16, 16); break;
        default: SV_SEG_C64(16, 32); break;
      }
#undef SV_SEG_C64
    } else {
      const svx::RowsPlan rp = svx::c64_rows_plan(cols);
      switch (rp.E * 100 + rp.W) {
        case 401: SV_ROWS_C64(4, 1); break;
        case 1601: SV_ROWS_C64(16, 1); break;
        case 1602: SV_ROWS_C64(16, 2); break;
        case 1604: SV_ROWS_C64(16, 4); break;
        case 1608: SV_ROWS_C64(16, 8); break;
        case 1616: SV_ROWS_C64(16, 16); break;
        default: SV_ROWS_C64(32, 16); break;
      }
    }
#undef SV_ROWS_C64
    return check_launch("sv_variance_c64");
  }
  char *wp = reinterpret_cast<char *>(workspace);
  float *vparts = reinterpret_cast<float *>(wp);
  wp += round256((size_t)2 * nslices * sizeof(float));
  sv_status rc;
  const int64_t pair_chunks = (cols + LS_ROW_CHUNK / 2 - 1) / (LS_ROW_CHUNK / 2);
  if (ax1 && pair_chunks <= LS_MAX_CHUNKS) {
    // Rows of more than 32768 values: chunks of LS_ROW_CHUNK / 2 complex
    // values read once, the parts split in registers (two interleaved
    // slices per row, the same values in the same order as the split rows),
    // then the pair add.
    launch_long_pairs(aligned16(z) && cols % 2 == 0, z, rows, cols, 2 * cols, ddof, wp, vparts, mean_out, st);
    rc = check_launch("sv_variance_c64");
  } else if (ax1) {
    // rows of more than 8192 chunks of pairs: the parts staged as float rows
    float *split = reinterpret_cast<float *>(wp);
    wp += round256((size_t)2 * rows * cols * sizeof(float));
    const size_t inner = sv_variance_f32_workspace_size(2 * rows, cols, 1);
    if (rows * cols > 0) {
      const int64_t bx = (cols + 255) / 256 < 65536 ? (cols + 255) / 256 : 65536;
      const int64_t by_max = 65535 / bx > 1 ? 65535 / bx : 1;
      const int64_t by = rows < by_max ? rows : by_max;
      k_split_rows<<<dim3((unsigned)bx, (unsigned)by), dim3(256), 0, st>>>(z, rows, cols, split);
      rc = check_launch("sv_variance_c64");
      if (rc != SV_OK) return rc;
    }
    rc = sv_variance_f32(split, 2 * rows, cols, 1, ddof, vparts, mean_out, inner ? wp : nullptr, inner, stream);
  } else {
    const size_t inner = sv_variance_f32_workspace_size(rows, 2 * cols, 0);
    rc = sv_variance_f32(z, rows, 2 * cols, 0, ddof, vparts, mean_out, inner ? wp : nullptr, inner, stream);
  }
  if (rc != SV_OK) return rc;
  k_pair_add<<<dim3((unsigned)((nslices + 255) / 256)), dim3(256), 0, st>>>(vparts, nslices, var_out);
  return check_launch("sv_variance_c64");
}

sv_status sv_probe_read_bandwidth(const float *x, int64_t n, float *out, void *stream) {
  if (n < 0) return fail(SV_ERR_INVALID_ARGUMENT, "sv_probe_read_bandwidth: n = %lld < 0", (long long)n);
  if (n > 0 && (!x || !out)) return fail(SV_ERR_INVALID_ARGUMENT, "sv_probe_read_bandwidth: NULL pointer");
  if (n > SUM_MAX_N) return fail(SV_ERR_UNSUPPORTED, "sv_probe_read_bandwidth: n above 2^36");
  if (!aligned16(x)) return fail(SV_ERR_INVALID_ARGUMENT, "sv_probe_read_bandwidth: x must be 16-byte aligned");
  if (n == 0) return ok();
  const sv_status dev = check_device();
  if (dev != SV_OK) return dev;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t blocks = (n + 4095) / 4096;
  k_stream_read<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(x, n, out);
  return check_launch("sv_probe_read_bandwidth");
}

sv_status sv_set_tuning(const char *key, int64_t value) {
  if (!key) return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: key is NULL");
  auto flag = [&](int *dst) {
    if (value != 0 && value != 1) return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: %s must be 0 or 1", key);
    *dst = (int)value;
    return ok();
  };
  if (strcmp(key, "sum_load_path") == 0) return flag(&g_tune.sum_load_path);
  if (strcmp(key, "sum_nt") == 0) return flag(&g_tune.sum_nt);
  if (strcmp(key, "var_load_path") == 0) {
    if (value < 0 || value > 2) return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: var_load_path must be 0, 1 or 2");
    g_tune.var_load_path = (int)value;
    return ok();
  }
  if (strcmp(key, "var_nt") == 0) return flag(&g_tune.var_nt);
  if (strcmp(key, "var_cols_single_max") == 0) {
    if (value < 0 || value > COLS_MAX_R)
      return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: var_cols_single_max must be in [0, %lld]",
                  (long long)COLS_MAX_R);
    g_tune.var_cols_single_max = (int)value;
    return ok();
  }
  if (strcmp(key, "var_cols_waves") == 0) {
    if (value != 0 && value != 4 && value != 8 && value != 16)
      return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: var_cols_waves must be 0, 4, 8 or 16");
    g_tune.var_cols_waves = (int)value;
    return ok();
  }
  if (strcmp(key, "var_short_rows") == 0) return flag(&g_tune.var_short_rows);
  if (strcmp(key, "var_long_rows") == 0) return flag(&g_tune.var_long_rows);
  if (strcmp(key, "var_cols_short") == 0) return flag(&g_tune.var_cols_short);
  if (strcmp(key, "var_cols_one") == 0) {
    if (value < 0 || value > 3)
      return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: var_cols_one must be 0, 1, 2 or 3");
    g_tune.var_cols_one = (int)value;
    return ok();
  }
  if (strcmp(key, "sum_xcd") == 0) return flag(&g_tune.sum_xcd);
  if (strcmp(key, "var_full_rows") == 0) return flag(&g_tune.var_full_rows);
  if (strcmp(key, "var_cols_once") == 0) {
    if (value < 0 || value > 2)
      return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: var_cols_once must be 0, 1 or 2");
    g_tune.var_cols_once = (int)value;
    return ok();
  }
  if (strcmp(key, "var_xcd") == 0) return flag(&g_tune.var_xcd);
  if (strcmp(key, "var_cols_pairs") == 0) return flag(&g_tune.var_cols_pairs);
  if (strcmp(key, "var_lds_pad") == 0) {
    if (value < 0 || value > 65536) return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: var_lds_pad must be in [0, 65536]");
    g_tune.var_lds_pad = (int)value;
    return ok();
  }
  if (strcmp(key, "var_split") == 0) {
    if (value != 0 && value != 1 && value != 2 && value != 4 && value != 8)
      return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: var_split must be 0, 1, 2, 4 or 8");
    g_tune.var_split = (int)value;
    return ok();
  }
  if (strcmp(key, "sum_e") == 0) {
    if (value != 16 && value != 32) return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: sum_e must be 16 or 32");
    g_tune.sum_e = (int)value;
    return ok();
  }
  if (strcmp(key, "sum_depth") == 0) {
    if (value != 2 && value != 4) return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: sum_depth must be 2 or 4");
    g_tune.sum_depth = (int)value;
    return ok();
  }
  if (strcmp(key, "sum_blocks") == 0) {
    if (value < 1 || value > SUM_MAX_BLOCKS)
      return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: sum_blocks must be in [1, %d]", SUM_MAX_BLOCKS);
    g_tune.sum_blocks = value;
    return ok();
  }
  if (strcmp(key, "launch_items") == 0) {
    if (value < 1024 || value > svx::MAX_LAUNCH_ITEMS)
      return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: launch_items must be in [1024, 2^32 - 1]");
    g_tune.launch_items = value;
    return ok();
  }
  bool handled = false;
  const sv_status adn = svh::adn_set_tuning(key, value, &handled);
  if (strcmp(key, "reset") == 0) {
    g_tune = Tuning{};
    return ok();
  }
  if (handled) return adn;
  return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: unknown key '%s'", key);
}

}  // extern "C"
