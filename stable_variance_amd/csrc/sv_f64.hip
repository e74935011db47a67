// The method in binary64 on gfx950: the compensated tree sum and the stable
// variance with every operation in double.
//
// Method: Pennacchio, "Variance in float32 with a first-element shift, a
// local centring and a compensated tree sum", §2 steps 1-4, carried out in
// double (§5 of that page lists float64 as not measured).  Same tree
// topology, carries, root guard, max and ddof readings as the float32 path.
//
// The loads reuse the float32 tiles: a run of 2^k doubles is a run of
// 2^(k+1) floats, and a lane that holds 2E consecutive floats holds E
// consecutive doubles (low word first).  Cross-lane moves of a double are two
// 32-bit moves (DPP or permlane swap).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/stable_variance.h"
#include "sv_device.hpp"
#include "sv_host.hpp"

using svh::check_device;
using svh::check_launch;
using svh::fail;
using svh::ok;

namespace {

// ------------------------------------------------------------------ nodes

struct NodeD {
  double s, c;
};

__device__ __forceinline__ NodeD combine_d(NodeD l, NodeD r) {
  const double s = l.s + r.s;
  const double bv = s - l.s;
  const double av = s - bv;
  const double e = (l.s - av) + (r.s - bv);
  return {s, (l.c + r.c) + e};
}

// Leaves: the sum keeps the carry as 0 + e (the oracle's (0 + 0) + e); the
// variance trees keep e (only a zero's sign differs, which no output sees).
__device__ __forceinline__ NodeD leaf_canon_d(double a, double b) {
  const double s = a + b;
  const double bv = s - a;
  const double av = s - bv;
  return {s, 0.0 + ((a - av) + (b - bv))};
}

__device__ __forceinline__ NodeD leaf_fast_d(double a, double b) {
  const double s = a + b;
  const double bv = s - a;
  const double av = s - bv;
  return {s, (a - av) + (b - bv)};
}

// Non-negative operands (the d^2 tree): Fast2Sum after a max/min gives the
// same exact error as TwoSum.
__device__ __forceinline__ NodeD combine_nn_d(NodeD l, NodeD r) {
  const double s = l.s + r.s;
  const double hi = __builtin_fmax(l.s, r.s);
  const double lo = __builtin_fmin(l.s, r.s);
  return {s, (l.c + r.c) + (lo - (s - hi))};
}

__device__ __forceinline__ NodeD leaf_nn_d(double a, double b) {
  const double s = a + b;
  const double hi = __builtin_fmax(a, b);
  const double lo = __builtin_fmin(a, b);
  return {s, lo - (s - hi)};
}

__device__ __forceinline__ double root_value_d(NodeD n) { return __builtin_isfinite(n.s) ? n.s + n.c : n.s; }

// Node kinds of the double trees: 0 (false) TwoSum, 1 (true) the
// non-negative node, KD_PLAIN the plain pairwise node fl(l.s + r.s) with no
// carry, the tree of the local mean (method page §2 step 2).
constexpr int KD_PLAIN = 2;

template <int NN>
__device__ __forceinline__ NodeD comb_d(NodeD l, NodeD r) {
  if constexpr (NN == KD_PLAIN) return {l.s + r.s, 0.0};
  else if constexpr (NN) return combine_nn_d(l, r);
  else return combine_d(l, r);
}

// The value at the root of a tree of kind K (a plain tree: fl(s + 0)).
template <int K>
__device__ __forceinline__ double root_value_kd(NodeD n) {
  if constexpr (K == KD_PLAIN) return n.s + 0.0;  // fl(s + 0): an all -0 sum gives +0
  else return root_value_d(n);
}

enum { LEAF_CANON_D = 0, LEAF_FAST_D = 1, LEAF_NN_D = 2, LEAF_PLAIN_D = 3 };

template <int LEAF, int OFF, int N, int E>
__device__ __forceinline__ NodeD lane_tree_d(const double (&v)[E]) {
  if constexpr (N == 2) {
    if constexpr (LEAF == LEAF_CANON_D) return leaf_canon_d(v[OFF], v[OFF + 1]);
    else if constexpr (LEAF == LEAF_FAST_D) return leaf_fast_d(v[OFF], v[OFF + 1]);
    else if constexpr (LEAF == LEAF_PLAIN_D) return {v[OFF] + v[OFF + 1], 0.0};
    else return leaf_nn_d(v[OFF], v[OFF + 1]);
  } else {
    const NodeD l = lane_tree_d<LEAF, OFF, N / 2, E>(v);
    const NodeD r = lane_tree_d<LEAF, OFF + N / 2, N / 2, E>(v);
    return comb_d<LEAF == LEAF_PLAIN_D ? KD_PLAIN : (LEAF == LEAF_NN_D ? 1 : 0)>(l, r);
  }
}

template <int OFF, int N, int K, int NN>
__device__ __forceinline__ NodeD node_tree_d(const NodeD (&nd)[K]) {
  if constexpr (N == 1) return nd[OFF];
  else return comb_d<NN>(node_tree_d<OFF, N / 2, K, NN>(nd), node_tree_d<OFF + N / 2, N / 2, K, NN>(nd));
}

// d = y - m and q = d * d, then their trees, leaf pair by leaf pair; entries
// at or past `valid` are +0 (padding), not fl(0 - m).
template <bool MASK, int OFF, int N, int E>
__device__ __forceinline__ void lane_tree_dq_d(const double (&y)[E], double m, int valid, NodeD &nd, NodeD &nq) {
  if constexpr (N == 2) {
    double d0 = y[OFF] - m;
    double d1 = y[OFF + 1] - m;
    if constexpr (MASK) {
      d0 = (OFF < valid) ? d0 : 0.0;
      d1 = (OFF + 1 < valid) ? d1 : 0.0;
    }
    nd = leaf_fast_d(d0, d1);
    nq = leaf_nn_d(d0 * d0, d1 * d1);
  } else {
    NodeD ld, lq, rd, rq;
    lane_tree_dq_d<MASK, OFF, N / 2, E>(y, m, valid, ld, lq);
    lane_tree_dq_d<MASK, OFF + N / 2, N / 2, E>(y, m, valid, rd, rq);
    nd = combine_d(ld, rd);
    nq = combine_nn_d(lq, rq);
  }
}

// ------------------------------------------------------------------ cross-lane

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, 0xF, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

template <int CTRL, int NN = 0>
__device__ __forceinline__ NodeD dpp_node_d(NodeD n) {
  if constexpr (NN == KD_PLAIN) return {dpp_d<CTRL>(n.s), 0.0};  // a plain tree's carries are +0
  else return {dpp_d<CTRL>(n.s), dpp_d<CTRL>(n.c)};
}

// A lane's double and its partner's (lane ^ XOR): both words of each copy go
// through the same permlane swap (the float helper), so the two results hold
// the two doubles, in some order; the node is symmetric.
template <int XOR>
__device__ __forceinline__ void swap_d(double v, double &a, double &b) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  float la, lb, ha, hb;
  sv::swap_halves<XOR>(__builtin_bit_cast(float, (unsigned)u), la, lb);
  sv::swap_halves<XOR>(__builtin_bit_cast(float, (unsigned)(u >> 32)), ha, hb);
  a = __builtin_bit_cast(double, ((unsigned long long)__builtin_bit_cast(unsigned, ha) << 32) |
                                     __builtin_bit_cast(unsigned, la));
  b = __builtin_bit_cast(double, ((unsigned long long)__builtin_bit_cast(unsigned, hb) << 32) |
                                     __builtin_bit_cast(unsigned, lb));
}

template <int XOR, int NN>
__device__ __forceinline__ NodeD swap_level_d(NodeD n) {
  NodeD a, b;
  swap_d<XOR>(n.s, a.s, b.s);
  if constexpr (NN == KD_PLAIN) {
    a.c = 0.0;
    b.c = 0.0;
  } else {
    swap_d<XOR>(n.c, a.c, b.c);
  }
  return comb_d<NN>(a, b);
}

// The six cross-lane levels (lane k holds range k); every lane ends with the
// wave's node.  The mirrors reach the sibling because the lower lanes agree.
template <int NN>
__device__ __forceinline__ NodeD wave_tree_d(NodeD n) {
  n = comb_d<NN>(n, dpp_node_d<sv::DPP_QUAD_XOR1, NN>(n));
  n = comb_d<NN>(n, dpp_node_d<sv::DPP_QUAD_XOR2, NN>(n));
  n = comb_d<NN>(n, dpp_node_d<sv::DPP_ROW_HALF_MIRROR, NN>(n));
  n = comb_d<NN>(n, dpp_node_d<sv::DPP_ROW_MIRROR, NN>(n));
  n = swap_level_d<16, NN>(n);
  return swap_level_d<32, NN>(n);
}

// The permuted lane order of the float32 row kernels: lane L holds the range
// of virtual lane 2 (L mod 32) + L / 32 (svx::vlane_pair32), so the first
// cross-lane level pairs L and L ^ 32, then xor 1, xor 2, the two mirrors
// and xor 16.  Every lane ends with the wave's node.
template <int NN>
__device__ __forceinline__ NodeD wave_tree_p32_d(NodeD n) {
  n = swap_level_d<32, NN>(n);
  n = comb_d<NN>(n, dpp_node_d<sv::DPP_QUAD_XOR1, NN>(n));
  n = comb_d<NN>(n, dpp_node_d<sv::DPP_QUAD_XOR2, NN>(n));
  n = comb_d<NN>(n, dpp_node_d<sv::DPP_ROW_HALF_MIRROR, NN>(n));
  n = comb_d<NN>(n, dpp_node_d<sv::DPP_ROW_MIRROR, NN>(n));
  return swap_level_d<16, NN>(n);
}

// The words of two doubles through one v_permlane32_swap each (the float
// helper): lanes 0..31 end with x of their own lane and of lane + 32, lanes
// 32..63 with y of lane - 32 and of their own.
__device__ __forceinline__ void swap32_two_d(double x, double y, double &a, double &b) {
  const unsigned long long ux = __builtin_bit_cast(unsigned long long, x);
  const unsigned long long uy = __builtin_bit_cast(unsigned long long, y);
  float al, bl, ah, bh;
  sv::swap32_two(__builtin_bit_cast(float, (unsigned)ux), __builtin_bit_cast(float, (unsigned)uy), al, bl);
  sv::swap32_two(__builtin_bit_cast(float, (unsigned)(ux >> 32)), __builtin_bit_cast(float, (unsigned)(uy >> 32)), ah,
                 bh);
  a = __builtin_bit_cast(double, ((unsigned long long)__builtin_bit_cast(unsigned, ah) << 32) |
                                     __builtin_bit_cast(unsigned, al));
  b = __builtin_bit_cast(double, ((unsigned long long)__builtin_bit_cast(unsigned, bh) << 32) |
                                     __builtin_bit_cast(unsigned, bl));
}

// The d and d^2 trees of a wave together, in the permuted lane order: one
// swap gives lanes 0..31 the pairs of the d tree and lanes 32..63 those of
// the d^2 tree, and the other five levels run once for both.  Lanes 0..31
// return the wave's d node, lanes 32..63 its d^2 node.  The d^2 levels take
// the TwoSum node: on non-negative operands its error is the same exact
// value, with the same sign of zero, as the Fast2Sum form's.
__device__ __forceinline__ NodeD wave_tree_dq_d(NodeD nd, NodeD nq) {
  NodeD a, b;
  swap32_two_d(nd.s, nq.s, a.s, b.s);
  swap32_two_d(nd.c, nq.c, a.c, b.c);
  NodeD n = comb_d<0>(a, b);
  n = comb_d<0>(n, dpp_node_d<sv::DPP_QUAD_XOR1, 0>(n));
  n = comb_d<0>(n, dpp_node_d<sv::DPP_QUAD_XOR2, 0>(n));
  n = comb_d<0>(n, dpp_node_d<sv::DPP_ROW_HALF_MIRROR, 0>(n));
  n = comb_d<0>(n, dpp_node_d<sv::DPP_ROW_MIRROR, 0>(n));
  return swap_level_d<16, 0>(n);
}

// The first log2(S) of those levels: every lane ends with the node of its
// aligned group of S lanes.
template <int NN, int S>
__device__ __forceinline__ NodeD seg_tree_d(NodeD n) {
  if constexpr (S >= 2) n = comb_d<NN>(n, dpp_node_d<sv::DPP_QUAD_XOR1, NN>(n));
  if constexpr (S >= 4) n = comb_d<NN>(n, dpp_node_d<sv::DPP_QUAD_XOR2, NN>(n));
  if constexpr (S >= 8) n = comb_d<NN>(n, dpp_node_d<sv::DPP_ROW_HALF_MIRROR, NN>(n));
  if constexpr (S >= 16) n = comb_d<NN>(n, dpp_node_d<sv::DPP_ROW_MIRROR, NN>(n));
  if constexpr (S >= 32) n = swap_level_d<16, NN>(n);
  if constexpr (S >= 64) n = swap_level_d<32, NN>(n);
  return n;
}

// Lane l's double, as a wave-uniform value (both words read from lane l).
__device__ __forceinline__ double readlane_d(double v, int l) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), l);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// E doubles from 2E floats held lane-contiguously (low word first).  Built
// with the hi/lo intrinsic: the 64-bit shift-and-or form left, at 32 doubles
// per lane, one private-memory slot per double (float stores, double loads).
template <int E>
__device__ __forceinline__ void floats_to_doubles(const float (&f)[2 * E], double (&d)[E]) {
#pragma unroll
  for (int i = 0; i < E; ++i)
    d[i] = __hiloint2double(__builtin_bit_cast(int, f[2 * i + 1]), __builtin_bit_cast(int, f[2 * i]));
}

__device__ __forceinline__ void store_node_d(NodeD *dst, NodeD v) {
  unsigned *w = reinterpret_cast<unsigned *>(dst);
  const unsigned long long s = __builtin_bit_cast(unsigned long long, v.s);
  const unsigned long long c = __builtin_bit_cast(unsigned long long, v.c);
  sv::store_u32_agent(w, (unsigned)s);
  sv::store_u32_agent(w + 1, (unsigned)(s >> 32));
  sv::store_u32_agent(w + 2, (unsigned)c);
  sv::store_u32_agent(w + 3, (unsigned)(c >> 32));
}

__device__ __forceinline__ NodeD load_node_d(const NodeD *src) {
  const unsigned *w = reinterpret_cast<const unsigned *>(src);
  const unsigned long long s = ((unsigned long long)sv::load_u32_agent(w + 1) << 32) | sv::load_u32_agent(w);
  const unsigned long long c = ((unsigned long long)sv::load_u32_agent(w + 3) << 32) | sv::load_u32_agent(w + 2);
  return {__builtin_bit_cast(double, s), __builtin_bit_cast(double, c)};
}

// ------------------------------------------------------------------ tree sum

using svx::S64_W;                        // waves per workgroup
using svx::S64_EF;                       // floats per lane per chunk (16 doubles)
constexpr int S64_E = S64_EF / 2;
constexpr int S64_CHUNK = 64 * S64_E;    // doubles per chunk
using svx::S64_MAX_BLOCKS;
constexpr int S64_GROUP = 64;
constexpr int S64_COUNTER_STRIDE = 64;
using svx::S64_MAX_LOG2_G;
constexpr size_t S64_WS_HEADER = 256 * (1 + S64_MAX_BLOCKS / S64_GROUP);
using svx::S64_MAX_N;
static_assert(S64_WS_HEADER == SV_TREE_SUM_COUNTER_BYTES, "same counter layout as the float32 sum");

// Each wave reduces a power-of-two run of chunks of 1024 doubles in tree
// order (the next chunk loading meanwhile), keeps chunk nodes on a
// binary-counter stack, and the workgroup's waves form its node; the
// two-level ticket of the float32 sum combines the workgroups.
template <bool VEC>
__global__ __launch_bounds__(64 * S64_W) void k_tree_sum_f64(const double *__restrict__ x, int64_t n, int log2_g,
                                                             NodeD *__restrict__ part,
                                                             unsigned *__restrict__ counter,
                                                             double *__restrict__ out) {
  using C = sv::Chunk<S64_EF, VEC, 0, true>;
  constexpr int LPW = sv::lds_floats_per_wave<S64_EF>();
  __shared__ float lds[S64_W * LPW];
  __shared__ NodeD wstack[S64_W][S64_MAX_LOG2_G + 1];
  __shared__ NodeD slots[S64_W];
  __shared__ unsigned is_last;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t G = 1LL << log2_g;
  const int64_t c0 = ((int64_t)blockIdx.x * S64_W + w) * G;
  const float *__restrict__ xf = reinterpret_cast<const float *>(x);
  const int64_t nf = 2 * n;
  float *const my_lds = lds + w * LPW;
  NodeD *const st = wstack[w];
  int sp = 0;

  auto reduce = [&](const float (&raw)[S64_EF], int64_t j) {
    float vf[S64_EF];
    C::finish(raw, my_lds, lane, vf);
    double v[S64_E];
    floats_to_doubles<S64_E>(vf, v);
    NodeD nd = lane_tree_d<LEAF_CANON_D, 0, S64_E, S64_E>(v);
    nd = wave_tree_d<false>(nd);
    if (lane == 0) {
      for (int64_t k = j; k & 1; k >>= 1) nd = combine_d(st[--sp], nd);
      st[sp++] = nd;
    }
  };
  auto issue = [&](int64_t c, float (&raw)[S64_EF]) {
    C::issue(xf + c * C::SIZE, nf - c * C::SIZE, lane, raw);
  };
  {
    // every load block below is unconditional, so the wait counts stay exact
    float ra[S64_EF], rb[S64_EF];
    int64_t j = 0;
    issue(c0, ra);
    while (j + 2 < G) {
      issue(c0 + j + 1, rb);
      reduce(ra, j);
      issue(c0 + j + 2, ra);
      reduce(rb, j + 1);
      j += 2;
    }
    if (j + 1 < G) {
      issue(c0 + j + 1, rb);
      reduce(ra, j);
      reduce(rb, j + 1);
    } else {
      reduce(ra, j);
    }
  }
  if (lane == 0) slots[w] = st[0];
  __syncthreads();

  const int nb = (int)gridDim.x;
  const int grp = (int)blockIdx.x / S64_GROUP;
  const int ngroups = (nb + S64_GROUP - 1) / S64_GROUP;
  const int in_group = (grp == ngroups - 1) ? nb - grp * S64_GROUP : S64_GROUP;
  unsigned *const top_counter = counter;
  unsigned *const grp_counter = counter + S64_COUNTER_STRIDE * (1 + grp);
  NodeD *const grp_nodes = part + S64_MAX_BLOCKS;
  if (threadIdx.x == 0) {
    NodeD nd[S64_W];
#pragma unroll
    for (int i = 0; i < S64_W; ++i) nd[i] = slots[i];
    store_node_d(part + blockIdx.x, node_tree_d<0, S64_W, S64_W, false>(nd));
    sv::wait_vmem_stores();
    const unsigned ticket = __hip_atomic_fetch_add(grp_counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (ticket == (unsigned)in_group - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!is_last || w != 0) return;
  {
    const int idx = grp * S64_GROUP + lane;
    NodeD g = (idx < nb) ? load_node_d(part + idx) : NodeD{0.0, 0.0};
    g = wave_tree_d<false>(g);
    unsigned top_ticket = 0;
    if (lane == 0) {
      __hip_atomic_store(grp_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      store_node_d(grp_nodes + grp, g);
      sv::wait_vmem_stores();
      top_ticket = __hip_atomic_fetch_add(top_counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    top_ticket = __builtin_amdgcn_readfirstlane(top_ticket);
    if (top_ticket != (unsigned)ngroups - 1) return;
  }
  constexpr int GPL = S64_MAX_BLOCKS / S64_GROUP / 64;
  NodeD t[GPL];
#pragma unroll
  for (int k = 0; k < GPL; ++k) {
    const int idx = GPL * lane + k;
    t[k] = (idx < ngroups) ? load_node_d(grp_nodes + idx) : NodeD{0.0, 0.0};
  }
  const NodeD r = wave_tree_d<false>(node_tree_d<0, GPL, GPL, false>(t));
  if (lane == 0) {
    out[0] = root_value_d(r);
    __hip_atomic_store(top_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ void k_zero_d(double *out) { out[0] = 0.0; }

// ------------------------------------------------------------------ variance

__device__ __forceinline__ double max0_nan_d(double v) { return (v != v) ? v : ((v > 0.0) ? v : 0.0); }

__device__ __forceinline__ void finalize_d(NodeD nd, NodeD nq, double x0, double m, int64_t n, int64_t ddof,
                                           double *var_out, double *mean_out) {
  const double fn = (double)n;
  const double a = root_value_d(nq) / fn;
  const double b = root_value_d(nd) / fn;
  double v = max0_nan_d(a - b * b);
  if (ddof != 0) {
    int64_t den = n - ddof;
    if (den < 0) den = 0;
    v = v * (fn / (double)den);
  }
  *var_out = v;
  if (mean_out) *mean_out = x0 + m;
}

// Per-call constants of the divisions by fl(n) and the ddof factor, formed
// on the host: when fl(n) is a power of two, x / fl(n) and x * rn with
// rn = 1 / fl(n) (exact) are the same rounding of the same real number.
struct StepConstsD {
  double fn;    // fl(n)
  double rn;    // 1 / fl(n) when fl(n) is a power of two, else 0 (divide)
  double dfac;  // fl(n) / fl(max(n - ddof, 0)), correctly rounded (unused when ddof == 0)
  int ddof_on;
};

StepConstsD step_consts_d(int64_t n, int64_t ddof) {
  StepConstsD k;
  k.fn = (double)n;
  int ex = 0;
  k.rn = (n > 0 && frexp(k.fn, &ex) == 0.5) ? 1.0 / k.fn : 0.0;
  k.ddof_on = ddof != 0;
  const int64_t den = n - ddof < 0 ? 0 : n - ddof;
  k.dfac = ddof != 0 ? k.fn / (double)den : 1.0;
  return k;
}

__device__ __forceinline__ double div_n_d(double a, const StepConstsD &k) { return k.rn != 0.0 ? a * k.rn : a / k.fn; }

// finalize_d with the per-call constants (the same results).
__device__ __forceinline__ void finalize_dk(NodeD nd, NodeD nq, double x0, double m, const StepConstsD &k,
                                            double *var_out, double *mean_out) {
  const double a = div_n_d(root_value_d(nq), k);
  const double b = div_n_d(root_value_d(nd), k);
  double v = max0_nan_d(a - b * b);
  if (k.ddof_on) v = v * k.dfac;
  *var_out = v;
  if (mean_out) *mean_out = x0 + m;
}

// Axis 1: one workgroup per row, W waves own consecutive 64*E ranges, each
// lane E consecutive doubles (lane L those of virtual lane
// svx::vlane_pair32(L), the order in which the d and d^2 trees share their
// cross-lane levels); the row stays in registers between passes.
// The launch holds only the waves the row reaches (svx::rows_waves); the
// tree's other wave nodes are (+0, +0).  At 32 doubles per lane every wave
// takes the masked code path (one path instead of two: 93-95 VGPRs instead
// of 118) and the kernel asks for five waves per SIMD, so two workgroups of
// up to ten waves (rows of up to 20480 doubles) share a CU.
template <int E, int W, bool VEC>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(E == 32 ? 5 : 1, 8))) void k_var_rows_f64(const double *__restrict__ x, int64_t n, int64_t ld,
                                                         int64_t ddof, double *__restrict__ var_out,
                                                         double *__restrict__ mean_out) {
  __shared__ NodeD slots[3][W];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = blockIdx.x;
  const double *__restrict__ p = x + row * ld;
  const int64_t base = (int64_t)w * 64 * E;
  // a wave wholly past the row holds only padding: its nodes are (+0, +0),
  // what its trees would compute, so it skips them (wave-uniform)
  const bool empty = base >= n;
  const int vl = svx::vlane_pair32(lane);  // this lane holds the range of virtual lane vl

  float vf[2 * E];
  const int64_t avail = 2 * svx::rows_avail(gridDim.x, row, ld, n, base);  // floats to the launch's last row
  sv::load_tile<2 * E, VEC, 1, false>(reinterpret_cast<const float *>(p + base), 2 * (n - base), nullptr, vf, vl,
                                      avail);
  double v[E];
  floats_to_doubles<E>(vf, v);
  const double x0 = p[0];

  const bool full = base + 64 * E <= n;
  const int64_t left = n - base - (int64_t)vl * E;
  const int valid = left < 0 ? 0 : (left > E ? E : (int)left);
  if (full && E != 32) {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = v[i] - x0;
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = (i < valid) ? v[i] - x0 : 0.0;
  }

  NodeD ny = {0.0, 0.0};
  if (!empty) ny = wave_tree_p32_d<KD_PLAIN>(lane_tree_d<LEAF_PLAIN_D, 0, E, E>(v));
  const int nw = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));  // the waves launched
  // From four waves on, the tree over the wave nodes takes one node per lane
  // (lane l < W wave l's) and the first log2(W) cross-lane levels.
  if constexpr (W > 1) {
    if (lane == 0) slots[0][w] = ny;
    __syncthreads();
    if constexpr (W >= 4) {
      const NodeD t = seg_tree_d<KD_PLAIN, W>(lane < nw ? slots[0][lane] : NodeD{0.0, 0.0});
      ny = {readlane_d(t.s, 0), readlane_d(t.c, 0)};
    } else {
      NodeD t[W];
#pragma unroll
      for (int i = 0; i < W; ++i) t[i] = i < nw ? slots[0][i] : NodeD{0.0, 0.0};
      ny = node_tree_d<0, W, W, KD_PLAIN>(t);
    }
  }
  const double m = root_value_kd<KD_PLAIN>(ny) / (double)n;

  NodeD nd = {0.0, 0.0}, nq = {0.0, 0.0};
  if (!empty) {
    if (full && E != 32) lane_tree_dq_d<false, 0, E, E>(v, m, E, nd, nq);
    else lane_tree_dq_d<true, 0, E, E>(v, m, valid, nd, nq);
    const NodeD ndq = wave_tree_dq_d(nd, nq);  // lanes 0..31: d, 32..63: d^2
    nd = {readlane_d(ndq.s, 0), readlane_d(ndq.c, 0)};
    nq = {readlane_d(ndq.s, 32), readlane_d(ndq.c, 32)};
  }
  if constexpr (W > 1) {
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
      const NodeD t =
          seg_tree_d<false, W>(lane < 2 * W && (lane & (W - 1)) < nw ? (&slots[1][0])[lane] : NodeD{0.0, 0.0});
      nd = {readlane_d(t.s, 0), readlane_d(t.c, 0)};
      nq = {readlane_d(t.s, W), readlane_d(t.c, W)};
    } else {
      if (threadIdx.x != 0) return;
      NodeD td[W], tq[W];
#pragma unroll
      for (int i = 0; i < W; ++i) {
        td[i] = i < nw ? slots[1][i] : NodeD{0.0, 0.0};
        tq[i] = i < nw ? slots[2][i] : NodeD{0.0, 0.0};
      }
      nd = node_tree_d<0, W, W, false>(td);
      nq = node_tree_d<0, W, W, true>(tq);
    }
  }
  if (threadIdx.x == 0) finalize_d(nd, nq, x0, m, n, ddof, var_out + row, mean_out ? mean_out + row : nullptr);
}

// Axis 1, short rows (n <= 512): a wave holds 64/S rows, row k on lanes
// [k*S, (k+1)*S), each lane E consecutive doubles; the in-lane levels, then
// the first log2(S) cross-lane levels (S*E a power of two >= n, values past
// n are +0).  VW = 2: 16-byte loads of two doubles (16-byte aligned rows of
// an even count), else single doubles; every load issued, clamped, masked.
template <int E, int S, int VW>
__global__ __launch_bounds__(256) void k_var_rows_seg_d(const double *__restrict__ x, int64_t rows, int64_t n,
                                                        int64_t ld, StepConstsD k, double *__restrict__ var_out,
                                                        double *__restrict__ mean_out) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = lane % S;
  const int64_t row = svx::seg_row(blockIdx.x, w, lane, S);  // 64/S rows per wave
  const bool rowok = row < rows;
  const double *__restrict__ p = x + svx::clamp_last(row, rows) * ld;
  const bool full = (n == (int64_t)S * E);
  const int64_t e0 = (int64_t)l * E;
  const int64_t left = n - e0;
  const int valid = left < 0 ? 0 : (left > E ? E : (int)left);
  double v[E];
  if constexpr (VW == 2) {
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
      const int64_t e = e0 + 2 * j;
      const double2 g = *reinterpret_cast<const double2 *>(p + (full ? e : svx::clamp_group(e, n, 2)));
      v[2 * j] = g.x;
      v[2 * j + 1] = g.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int64_t e = e0 + i;
      v[i] = p[full ? e : svx::clamp_group(e, n, 1)];
    }
  }
  const double x0 = p[0];
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = (full || i < valid) ? v[i] - x0 : 0.0;
  const NodeD ny = seg_tree_d<KD_PLAIN, S>(lane_tree_d<LEAF_PLAIN_D, 0, E, E>(v));
  const double m = div_n_d(root_value_kd<KD_PLAIN>(ny), k);
  NodeD nd, nq;
  if (full) lane_tree_dq_d<false, 0, E, E>(v, m, E, nd, nq);
  else lane_tree_dq_d<true, 0, E, E>(v, m, valid, nd, nq);
  nd = seg_tree_d<false, S>(nd);
  nq = seg_tree_d<true, S>(nq);
  if (l == 0 && rowok) finalize_dk(nd, nq, x0, m, k, var_out + row, mean_out ? mean_out + row : nullptr);
}

// Axis 0: lanes own columns (a row of 64 consecutive doubles per load), the
// W waves own consecutive blocks of E rows; levels below the cross-wave ones
// are in-lane.
template <int E, int W>
__global__ __launch_bounds__(64 * W) void k_var_cols_f64(const double *__restrict__ x, int64_t R, int64_t C,
                                                         int64_t ddof, double *__restrict__ var_out,
                                                         double *__restrict__ mean_out, int64_t b0) {
  __shared__ NodeD sy[W][64];
  __shared__ NodeD sd[W][64];
  __shared__ NodeD sq[W][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t col = (b0 + blockIdx.x) * 64 + lane;  // b0: launches of at most 2^32 - 1 work-items
  const bool colok = col < C;
  const int64_t r0 = (int64_t)w * E;
  const bool full = r0 + E <= R;
  const int64_t ccol = svx::clamp_last(col, C);
  double v[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int64_t r = r0 + i;
    const double t = x[svx::clamp_last(r, R) * C + ccol];
    v[i] = (colok && r < R) ? t : 0.0;
  }
  const double x0 = x[ccol];
  const int64_t left = R - r0;
  const int valid = left < 0 ? 0 : (left > E ? E : (int)left);
  if (full) {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = v[i] - x0;
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = (i < valid) ? v[i] - x0 : 0.0;
  }
  NodeD ny = lane_tree_d<LEAF_PLAIN_D, 0, E, E>(v);
  sy[w][lane] = ny;
  __syncthreads();
  {
    NodeD nn[W];
#pragma unroll
    for (int i = 0; i < W; ++i) nn[i] = sy[i][lane];
    ny = node_tree_d<0, W, W, KD_PLAIN>(nn);
  }
  const double m = root_value_kd<KD_PLAIN>(ny) / (double)R;
  NodeD nd, nq;
  if (full) lane_tree_dq_d<false, 0, E, E>(v, m, E, nd, nq);
  else lane_tree_dq_d<true, 0, E, E>(v, m, valid, nd, nq);
  sd[w][lane] = nd;
  sq[w][lane] = nq;
  __syncthreads();
  if (w == 0 && colok) {
    NodeD a[W], b[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      a[i] = sd[i][lane];
      b[i] = sq[i][lane];
    }
    finalize_d(node_tree_d<0, W, W, false>(a), node_tree_d<0, W, W, true>(b), x0, m, R, ddof, var_out + col,
               mean_out ? mean_out + col : nullptr);
  }
}

// ------------------------------------------------------------------ long slices

// Slices longer than one workgroup holds, cut into aligned chunks (nodes of
// the slice's tree), as in the float32 path:
//   axis 1, rows of more than 16384 values: chunks of 8192 values (8 waves
//     of 64 lanes of 16 doubles); a y node per chunk, a per-row top tree
//     giving m, d and d^2 nodes per chunk, per-row top trees and step 4.
//   axis 0, columns of more than 1024 values: chunks of 128*G rows of a
//     block of V*64/G columns (lane L = q*G + g holds the V adjacent columns
//     of group q, one 16-byte load per row when V = 2, for 16 rows; G = 1
//     for wide matrices, up to 64 for narrow ones); a y node per (chunk,
//     column), m per column, d and d^2 nodes per (chunk, column), per-column
//     trees (a wave per column when there are many chunks) and step 4.
// The input is read twice; the workspace is scratch.

using svx::L64_E;           // doubles per lane
using svx::L64_W;           // waves per workgroup (up to 256 VGPRs: no spills)
using svx::L64_ROW_CHUNK;   // 8192 doubles
using svx::L64_TOP_MAX_K;   // chunk nodes per thread of a top tree
using svx::L64_MAX_CHUNKS;
using svx::C64_CHUNK;       // 128 rows
using svx::C64_GROUP;       // chunk nodes per column that k_cols_dq_d reduces for m itself

struct SliceWsD {
  NodeD *ny;  // y-tree node of every chunk of every slice
  NodeD *nd;  // d-tree nodes
  NodeD *nq;  // d^2-tree nodes
  double *m;  // per slice
};

// The W wave nodes of a workgroup (every lane of wave w holds node w) ->
// the workgroup's node, valid in thread 0 (and every thread after the
// barrier reads of `slots`).
template <int W, int NN>
__device__ __forceinline__ NodeD block_tree_d(NodeD n, NodeD *slots, int w, int lane) {
  if (lane == 0) slots[w] = n;
  __syncthreads();
  NodeD t[W];
#pragma unroll
  for (int i = 0; i < W; ++i) t[i] = slots[i];
  __syncthreads();
  return node_tree_d<0, W, W, NN>(t);
}

// P interleaved slices per row (P = 2: a matrix of two columns read as one
// row of pairs): each slice's chunks hold 8192 / P values, EP = 16 / P per
// lane, taken apart from the lane's 16 loaded doubles; slice j of row r is
// slice P*r + j.
template <int PASS, bool VEC, int P = 1>
__global__ __launch_bounds__(64 * L64_W) void k_long_rows_d(const double *__restrict__ x, int64_t n, int64_t ld,
                                                            int64_t nch, SliceWsD ws) {
  constexpr int E = L64_E, W = L64_W, EP = E / P;
  constexpr int64_t CHUNK = L64_ROW_CHUNK / P;
  __shared__ NodeD slots[2 * P][W];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r = (int64_t)blockIdx.x / nch;
  const int64_t c = (int64_t)blockIdx.x % nch;
  const double *__restrict__ row = x + r * ld;
  const int64_t base = c * CHUNK + (int64_t)w * 64 * EP;  // first value of this wave, of each slice
  const bool empty = base >= n;  // wave-uniform: only padding, nodes (+0, +0)
  float vf[2 * E];
  // floats to the launch's last row
  const int64_t avail = 2 * P * svx::rows_avail(gridDim.x / nch, r, ld / P, n, base);
  sv::load_tile<2 * E, VEC, 1, false>(reinterpret_cast<const float *>(row + P * base), 2 * P * (n - base), nullptr,
                                      vf, lane, avail);
  double f[E];
  floats_to_doubles<E>(vf, f);
  const bool full = base + 64 * EP <= n;
  const int64_t left = n - base - (int64_t)lane * EP;
  const int valid = left < 0 ? 0 : (left > EP ? EP : (int)left);
  double v[P][EP];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const double x0 = row[j];
#pragma unroll
    for (int i = 0; i < EP; ++i) v[j][i] = (full || i < valid) ? f[P * i + j] - x0 : 0.0;
  }
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int64_t out = (P * r + j) * nch + c;
    if constexpr (PASS == 0) {
      NodeD ny = {0.0, 0.0};
      if (!empty) ny = wave_tree_d<KD_PLAIN>(lane_tree_d<LEAF_PLAIN_D, 0, EP, EP>(v[j]));
      ny = block_tree_d<W, KD_PLAIN>(ny, slots[2 * j], w, lane);
      if (threadIdx.x == 0) ws.ny[out] = ny;
    } else {
      const double m = ws.m[P * r + j];
      NodeD nd = {0.0, 0.0}, nq = {0.0, 0.0};
      if (!empty) {
        if (full) lane_tree_dq_d<false, 0, EP, EP>(v[j], m, EP, nd, nq);
        else lane_tree_dq_d<true, 0, EP, EP>(v[j], m, valid, nd, nq);
        nd = wave_tree_d<false>(nd);
        nq = wave_tree_d<true>(nq);
      }
      nd = block_tree_d<W, false>(nd, slots[2 * j], w, lane);
      nq = block_tree_d<W, true>(nq, slots[2 * j + 1], w, lane);
      if (threadIdx.x == 0) {
        ws.nd[out] = nd;
        ws.nq[out] = nq;
      }
    }
  }
}

// Tree over the nch chunk nodes of one row (256 threads of K nodes each,
// padded with zero nodes to 256 * K: the padding changes no bit).
template <int NN, int K>
__device__ __forceinline__ NodeD top_tree_d(const NodeD *__restrict__ nodes, int64_t nch, NodeD *slots) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  NodeD nd[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t idx = (int64_t)threadIdx.x * K + k;
    const NodeD t = nodes[svx::clamp_last(idx, nch)];  // unconditional: the loads overlap
    nd[k] = idx < nch ? t : NodeD{0.0, 0.0};
  }
  NodeD r = wave_tree_d<NN>(node_tree_d<0, K, K, NN>(nd));
  return block_tree_d<4, NN>(r, slots, w, lane);
}

// One workgroup per slice; slice s's first value is at
// x[(s / P) * ld + s % P] (P interleaved slices per row).
template <int PASS, int K, int P = 1>
__global__ __launch_bounds__(256) void k_long_top_d(const double *__restrict__ x, int64_t n, int64_t ld,
                                                    int64_t nch, int64_t ddof, SliceWsD ws,
                                                    double *__restrict__ var_out, double *__restrict__ mean_out) {
  __shared__ NodeD slots[2][4];
  const int64_t r = blockIdx.x;
  if constexpr (PASS == 0) {
    const NodeD ny = top_tree_d<KD_PLAIN, K>(ws.ny + r * nch, nch, slots[0]);
    if (threadIdx.x == 0) ws.m[r] = root_value_kd<KD_PLAIN>(ny) / (double)n;
  } else {
    const NodeD nd = top_tree_d<false, K>(ws.nd + r * nch, nch, slots[0]);
    const NodeD nq = top_tree_d<true, K>(ws.nq + r * nch, nch, slots[1]);
    if (threadIdx.x == 0)
      finalize_d(nd, nq, x[(r / P) * ld + r % P], ws.m[r], n, ddof, var_out + r, mean_out ? mean_out + r : nullptr);
  }
}

// Axis 0: rows [r0, r0 + E) of the V columns starting at c0 (a multiple of
// V); columns past C read the last in-range ones (never written), rows past
// R read row R-1 (masked to +0 afterwards).
// VEC16: one 16-byte load per row when V = 2 (base and width allow it);
// else V 8-byte loads, which read the same cache lines.
template <int V, int E, bool VEC16 = true>
__device__ __forceinline__ void load_cols_tile_d(const double *__restrict__ x, int64_t R, int64_t C, int64_t c0,
                                                 int64_t r0, bool full, double (&v)[V][E]) {
  const int64_t cc = svx::cols_first(c0, C, V);
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int64_t r = full ? r0 + i : svx::clamp_last(r0 + i, R);
    const double *p = x + r * C + cc;
    if constexpr (V == 2 && VEC16) {
      const double2 g = *reinterpret_cast<const double2 *>(p);
      v[0][i] = g.x;
      v[1][i] = g.y;
    } else {
      // columns past C (a partial last pair of an odd width) read the last
      // column instead; their results are never written
#pragma unroll
      for (int k = 0; k < V; ++k) v[k][i] = x[r * C + svx::clamp_last(cc + k, C)];
    }
  }
}

template <int V, int E>
__device__ __forceinline__ void shift_cols_tile_d(double (&v)[V][E], const double (&x0)[V], bool full, int valid) {
#pragma unroll
  for (int k = 0; k < V; ++k)
#pragma unroll
    for (int i = 0; i < E; ++i) v[k][i] = (full || i < valid) ? v[k][i] - x0[k] : 0.0;
}

// Tree of the local mean over the nch <= C64_GROUP y chunk nodes p[0],
// p[stride], ..., padded with zero nodes to C64_GROUP (the padding changes no
// bit).
__device__ __forceinline__ NodeD chunk_tree_1_d(const NodeD *p, int64_t stride, int64_t nch) {
  NodeD sub[C64_GROUP / 8];
#pragma unroll
  for (int b = 0; b < C64_GROUP / 8; ++b) {
    NodeD nd[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t idx = b * 8 + k;
      const NodeD t = p[svx::clamp_last(idx, nch) * stride];
      nd[k] = idx < nch ? t : NodeD{0.0, 0.0};
    }
    sub[b] = node_tree_d<0, 8, 8, KD_PLAIN>(nd);
  }
  return node_tree_d<0, C64_GROUP / 8, C64_GROUP / 8, KD_PLAIN>(sub);
}

// G row groups per wave: lane L = q*G + g holds the V adjacent columns of
// column group q (Q = 64/G groups, V*Q columns per block) for the E rows
// [g*E, (g+1)*E) of the wave's G*E rows; the wave's node of a column is the
// in-lane levels and then the first log2(G) cross-lane levels (the lanes of
// a column group are adjacent).  G = 1 for blocks of 64*V columns; narrow
// matrices take larger G so that lanes stay on columns.  Chunks of W*G*E
// rows.
template <int V, int G>
__global__ __launch_bounds__(64 * L64_W) void k_cols_y_d(const double *__restrict__ x, int64_t R, int64_t C,
                                                         int64_t nch, SliceWsD ws, int64_t b0) {
  constexpr int E = L64_E, W = L64_W, Q = 64 / G, NC = V * Q;
  __shared__ NodeD s[W][V][Q];
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
  double v[V][E];
  load_cols_tile_d<V, E>(x, R, C, c0, r0, full, v);
  double x0[V];
  const int64_t cc = svx::cols_first(c0, C, V);
#pragma unroll
  for (int k = 0; k < V; ++k) x0[k] = x[cc + k];
  shift_cols_tile_d<V, E>(v, x0, wave_full, valid);
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const NodeD nd = seg_tree_d<KD_PLAIN, G>(lane_tree_d<LEAF_PLAIN_D, 0, E, E>(v[k]));
    if (g == 0) s[w][k][q] = nd;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < NC) {
    const int k = t / Q, qq = t % Q;  // thread t combines column V*qq + k of the block
    const int64_t col = cb * NC + (int64_t)qq * V + k;
    if (col < C) {
      NodeD nn[W];
#pragma unroll
      for (int i = 0; i < W; ++i) nn[i] = s[i][k][qq];
      ws.ny[j * C + col] = node_tree_d<0, W, W, KD_PLAIN>(nn);
    }
  }
}

// The per-column trees over the chunk nodes with S lanes per column (64/S
// columns per wave, four waves per workgroup): lane l of a column's group
// takes nodes [l*K, (l+1)*K) (zero nodes past nch), the in-lane levels and
// then the first log2(S) cross-lane levels give the tree of the column's
// chunks padded to S*K nodes.  PASS 0: m; PASS 1: step 4.
template <int PASS, int K, int S>
__global__ __launch_bounds__(256) void k_cols_top_d(const double *__restrict__ x, int64_t R, int64_t C, int64_t nch,
                                                    int64_t ddof, SliceWsD ws, double *__restrict__ var_out,
                                                    double *__restrict__ mean_out, int64_t b0) {
  constexpr int PW = 64 / S;
  const int lane = threadIdx.x & 63;
  const int64_t col0 = ((b0 + blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * PW;
  if (col0 >= C) return;  // the whole wave
  const int64_t col = col0 + lane / S;
  const int sl = lane % S;
  const bool colok = col < C;
  const int64_t cc = svx::clamp_last(col, C);
  auto tree = [&](const NodeD *p, auto nn) {
    constexpr int NN = decltype(nn)::value;
    NodeD nd[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t idx = (int64_t)sl * K + k;
      const NodeD t = p[svx::clamp_last(idx, nch) * C];  // every load issued
      nd[k] = idx < nch ? t : NodeD{0.0, 0.0};
    }
    return seg_tree_d<NN, S>(node_tree_d<0, K, K, NN>(nd));
  };
  if constexpr (PASS == 0) {
    const NodeD ny = tree(ws.ny + cc, std::integral_constant<int, KD_PLAIN>{});
    if (sl == 0 && colok) ws.m[col] = root_value_kd<KD_PLAIN>(ny) / (double)R;
  } else {
    const NodeD nd = tree(ws.nd + cc, std::false_type{});
    const NodeD nq = tree(ws.nq + cc, std::true_type{});
    if (sl == 0 && colok)
      finalize_d(nd, nq, x[col], ws.m[col], R, ddof, var_out + col, mean_out ? mean_out + col : nullptr);
  }
}

// The per-column trees over more than 4096 chunk nodes, a wave per column:
// lane l reduces the run of 64*P nodes [l*64*P, (l+1)*64*P) (P = 2^log2p,
// zero nodes past nch) in batches of 64, merging the batch nodes in tree
// order with a binary counter (wave-uniform loop, constant stack indices),
// then the wave's six levels.  PASS 0: m; PASS 1: step 4.
using svx::TOP_BIG_LEVELS_D;  // P up to 2^15
template <int PASS>
__global__ __launch_bounds__(256) void k_cols_top_big_d(const double *__restrict__ x, int64_t R, int64_t C,
                                                        int64_t nch, int log2p, int64_t ddof, SliceWsD ws,
                                                        double *__restrict__ var_out, double *__restrict__ mean_out,
                                                        int64_t b0) {
  constexpr int K = 64;
  const int lane = threadIdx.x & 63;
  const int64_t col = (b0 + blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (col >= C) return;  // the whole wave
  const int64_t P = (int64_t)1 << log2p;
  auto tree = [&](const NodeD *p, auto nn) {
    constexpr int NN = decltype(nn)::value;
    NodeD st[TOP_BIG_LEVELS_D];
#pragma unroll
    for (int lv = 0; lv < TOP_BIG_LEVELS_D; ++lv) st[lv] = NodeD{0.0, 0.0};
    for (int64_t b = 0; b < P; ++b) {
      NodeD nd[K];
      const int64_t i0 = ((int64_t)lane * P + b) * K;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t idx = i0 + k;
        const NodeD t = p[svx::clamp_last(idx, nch) * C];  // every load issued
        nd[k] = idx < nch ? t : NodeD{0.0, 0.0};
      }
      NodeD carry = node_tree_d<0, K, K, NN>(nd);
      bool placed = false;
#pragma unroll
      for (int lv = 0; lv < TOP_BIG_LEVELS_D; ++lv) {
        if (!placed) {
          if ((b >> lv) & 1) {
            carry = comb_d<NN>(st[lv], carry);
          } else {
            st[lv] = carry;
            placed = true;
          }
        }
      }
    }
    NodeD r = {0.0, 0.0};
#pragma unroll
    for (int lv = 0; lv < TOP_BIG_LEVELS_D; ++lv)
      if (lv == log2p) r = st[lv];
    return wave_tree_d<NN>(r);
  };
  if constexpr (PASS == 0) {
    const NodeD ny = tree(ws.ny + col, std::integral_constant<int, KD_PLAIN>{});
    if (lane == 0) ws.m[col] = root_value_kd<KD_PLAIN>(ny) / (double)R;
  } else {
    const NodeD nd = tree(ws.nd + col, std::false_type{});
    const NodeD nq = tree(ws.nq + col, std::true_type{});
    if (lane == 0) finalize_d(nd, nq, x[col], ws.m[col], R, ddof, var_out + col, mean_out ? mean_out + col : nullptr);
  }
}

// MLOCAL: nch <= C64_GROUP, and every workgroup forms m for its own columns
// (no separate launch); else m comes from k_cols_top_d or k_cols_top_big_d.
// Tile layout as in k_cols_y_d.
template <int V, int G, bool MLOCAL>
__global__ __launch_bounds__(64 * L64_W) void k_cols_dq_d(const double *__restrict__ x, int64_t R, int64_t C,
                                                          int64_t nch, SliceWsD ws, int64_t b0) {
  constexpr int E = L64_E, W = L64_W, Q = 64 / G, NC = V * Q;
  __shared__ NodeD sd[W][V][Q];
  __shared__ NodeD sq[W][V][Q];
  __shared__ double sm[V][Q];
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
  const int64_t cc = svx::cols_first(c0, C, V);
  if constexpr (MLOCAL) {
    const int t = threadIdx.x;
    if (t < NC) {
      const int k = t / Q, qq = t % Q;  // column V*qq + k of the block, clamped like the loads
      const int64_t col = cb * NC + (int64_t)qq * V + k;
      const int64_t ccol = svx::clamp_last(col, C);
      sm[k][qq] = root_value_kd<KD_PLAIN>(chunk_tree_1_d(ws.ny + ccol, C, nch)) / (double)R;
    }
    __syncthreads();
  }
  double v[V][E];  // loaded after m, which holds fewer registers at once
  load_cols_tile_d<V, E>(x, R, C, c0, r0, full, v);
  double x0[V], m[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    x0[k] = x[cc + k];
    m[k] = MLOCAL ? sm[k][q] : ws.m[cc + k];
  }
  shift_cols_tile_d<V, E>(v, x0, wave_full, valid);
#pragma unroll
  for (int k = 0; k < V; ++k) {
    NodeD nd, nq;
    if (wave_full) lane_tree_dq_d<false, 0, E, E>(v[k], m[k], E, nd, nq);
    else lane_tree_dq_d<true, 0, E, E>(v[k], m[k], valid, nd, nq);
    nd = seg_tree_d<false, G>(nd);
    nq = seg_tree_d<true, G>(nq);
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
      NodeD a[W], b[W];
#pragma unroll
      for (int i = 0; i < W; ++i) {
        a[i] = sd[i][k][qq];
        b[i] = sq[i][k][qq];
      }
      ws.nd[j * C + col] = node_tree_d<0, W, W, false>(a);
      ws.nq[j * C + col] = node_tree_d<0, W, W, true>(b);
    }
  }
}

// Whole columns in one workgroup (R <= 16*G*W rows): the tile layout of
// k_cols_y_d with a single chunk, and y, m, d and d^2 in one launch, the tile
// kept in registers between the two passes.  Waves wholly past the last row
// load nothing (their values are the +0 padding).  MODE 0 branches per wave
// between the full and the masked code paths; MODE 1 is for R = 16*G*W (no
// lane holds padding: no masks); MODE 2 masks every wave (one code path).
// Both paths together took the 8-wave tile of 32 doubles per lane to 164
// VGPRs and one workgroup per CU; one path takes 102-116, and two.
template <int V, int W, int G, bool VEC16 = true, int MODE = 0>
__global__ __launch_bounds__(64 * W) void k_cols_one_d(const double *__restrict__ x, int64_t R, int64_t C,
                                                       int64_t ddof, double *__restrict__ var_out,
                                                       double *__restrict__ mean_out, int b0) {
  constexpr int E = L64_E, Q = 64 / G, NC = V * Q;
  __shared__ NodeD sd[W][V][Q];
  __shared__ NodeD sq[W][V][Q];
  __shared__ double sm[V][Q];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane / G, g = lane % G;
  // b0: launches of at most 2^32 - 1 work-items.  Blocks of fewer than 16
  // doubles share a 128-byte line with the next block: the blocks of one
  // line run on one die (svx::line_on_one_die, in 4-byte units).
  const int64_t cb = svx::line_on_one_die<int>(b0 + (int)blockIdx.x, (int)((C + NC - 1) / NC), 2 * NC);
  const int64_t c0 = cb * NC + (int64_t)q * V;
  const int64_t rw = (int64_t)w * (E * G);  // the wave's first row
  const int64_t r0 = rw + (int64_t)g * E;
  const bool full = MODE == 1 || r0 + E <= R;
  const bool wave_full = MODE == 1 || (MODE == 0 && rw + (int64_t)E * G <= R);  // uniform
  const int64_t left = R - r0;
  const int valid = left < 0 ? 0 : (left > E ? E : (int)left);
  double v[V][E];
  if (rw < R) load_cols_tile_d<V, E, VEC16>(x, R, C, c0, r0, full, v);
  double x0[V];
  const int64_t cc = svx::cols_first(c0, C, V);
#pragma unroll
  for (int k = 0; k < V; ++k) x0[k] = x[svx::clamp_last(cc + k, C)];
  shift_cols_tile_d<V, E>(v, x0, wave_full, valid);  // +0 past the last row
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const NodeD nd = seg_tree_d<KD_PLAIN, G>(lane_tree_d<LEAF_PLAIN_D, 0, E, E>(v[k]));
    if (g == 0) sd[w][k][q] = nd;
  }
  __syncthreads();
  // thread t forms m (then step 4) of column V*tq + tk of the block, t = tk*Q + tq
  for (int t = threadIdx.x; t < NC; t += 64 * W) {
    const int tk = t / Q, tq = t % Q;
    NodeD nn[W];
#pragma unroll
    for (int i = 0; i < W; ++i) nn[i] = sd[i][tk][tq];
    sm[tk][tq] = root_value_kd<KD_PLAIN>(node_tree_d<0, W, W, KD_PLAIN>(nn)) / (double)R;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < V; ++k) {
    NodeD nd, nq;
    if (wave_full) lane_tree_dq_d<false, 0, E, E>(v[k], sm[k][q], E, nd, nq);
    else lane_tree_dq_d<true, 0, E, E>(v[k], sm[k][q], valid, nd, nq);
    nd = seg_tree_d<false, G>(nd);
    nq = seg_tree_d<true, G>(nq);
    if (g == 0) {
      sd[w][k][q] = nd;  // the y nodes were read before the barrier
      sq[w][k][q] = nq;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < NC; t += 64 * W) {
    const int tk = t / Q, tq = t % Q;
    const int64_t col = cb * NC + (int64_t)tq * V + tk;
    if (col < C) {
      NodeD a[W], b[W];
#pragma unroll
      for (int i = 0; i < W; ++i) {
        a[i] = sd[i][tk][tq];
        b[i] = sq[i][tk][tq];
      }
      finalize_d(node_tree_d<0, W, W, false>(a), node_tree_d<0, W, W, true>(b), x[col], sm[tk][tq], R, ddof,
                 var_out + col, mean_out ? mean_out + col : nullptr);
    }
  }
}

// Axis 0, short columns (R <= E rows, E <= 16, R < 16): each lane owns two
// adjacent columns (one 16-byte load per row, 16-byte aligned base and an
// even width) and all three trees are in-lane: no cross-lane levels, no
// LDS, no barrier.  Rows past R are the +0 padding of the column's tree.
template <int E>
__global__ __launch_bounds__(256) void k_cols_short_d(const double *__restrict__ x, int64_t R, int64_t C,
                                                      int64_t ddof, double *__restrict__ var_out,
                                                      double *__restrict__ mean_out, int64_t b0) {
  const int64_t c0 = ((b0 + blockIdx.x) * 256 + threadIdx.x) * 2;
  if (c0 >= C) return;
  const double *__restrict__ p = x + c0;
  double v[2][E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const double2 g = *reinterpret_cast<const double2 *>(p + svx::clamp_last<int64_t>(i, R) * C);
    v[0][i] = g.x;
    v[1][i] = g.y;
  }
  const int valid = (int)R;  // R <= E
  double var2[2], mean2[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const double x0 = v[k][0];
#pragma unroll
    for (int i = 0; i < E; ++i) v[k][i] = (i < valid) ? v[k][i] - x0 : 0.0;
    const double m = root_value_kd<KD_PLAIN>(lane_tree_d<LEAF_PLAIN_D, 0, E, E>(v[k])) / (double)R;
    NodeD nd, nq;
    lane_tree_dq_d<true, 0, E, E>(v[k], m, valid, nd, nq);
    finalize_d(nd, nq, x0, m, R, ddof, &var2[k], &mean2[k]);
  }
  auto store2 = [&](double *out, const double (&t)[2]) {
    double *o = out + c0;
    if ((reinterpret_cast<uintptr_t>(out) & 15u) == 0) {
      *reinterpret_cast<double2 *>(o) = make_double2(t[0], t[1]);
    } else {
      o[0] = t[0];
      o[1] = t[1];
    }
  };
  store2(var_out, var2);
  if (mean_out) store2(mean_out, mean2);
}

__global__ void k_fill_nan_d(double *__restrict__ a, double *__restrict__ b, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) {
    a[i] = __builtin_nan("");
    if (b) b[i] = __builtin_nan("");
  }
}

using svx::V64_ROWS_MAX_N;  // one workgroup per row
// Rows of up to 32768 values take one workgroup of 32 values per lane when
// there are enough rows to fill the chip (fewer take the chunked path, which
// spreads a row over several workgroups); the workspace is sized for the
// chunked path either way.
using svx::V64_ROWS_ONE_MAX_N;
using svx::V64_ROWS_ONE_MIN_ROWS;
using svx::V64_COLS_MAX_R;  // whole columns in one workgroup
using svx::V64_MAX_ELEMS;   // 2^35 doubles: every launch within 2^32 - 1 work-items

size_t round256_d(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace of the long-slice paths: three node arrays of nodes_per_array
// nodes and one double per slice, each part 256-byte aligned.
size_t slice_ws_bytes(int64_t nodes_per_array, int64_t nslices) {
  return 3 * round256_d((size_t)nodes_per_array * sizeof(NodeD)) + round256_d((size_t)nslices * sizeof(double));
}

SliceWsD slice_ws(void *workspace, int64_t nodes_per_array) {
  char *p = reinterpret_cast<char *>(workspace);
  const size_t a = round256_d((size_t)nodes_per_array * sizeof(NodeD));
  return {reinterpret_cast<NodeD *>(p), reinterpret_cast<NodeD *>(p + a), reinterpret_cast<NodeD *>(p + 2 * a),
          reinterpret_cast<double *>(p + 3 * a)};
}

// Workspace bytes (0: single-workgroup slices; -1: unsupported).
size_t var64_ws(int64_t rows, int64_t cols, bool ax1) {
  const int64_t n = ax1 ? cols : rows, nslices = ax1 ? rows : cols;
  if (n == 0 || nslices == 0) return 0;
  if (ax1) {
    if (n <= V64_ROWS_MAX_N) return 0;
    const int64_t nch = (n + L64_ROW_CHUNK - 1) / L64_ROW_CHUNK;
    if (nch > L64_MAX_CHUNKS) return (size_t)-1;
    return slice_ws_bytes(rows * nch, rows);
  }
  if (n <= V64_COLS_MAX_R) return 0;
  return slice_ws_bytes(((n + C64_CHUNK - 1) / C64_CHUNK) * cols, cols);
}

template <int PASS, int P = 1>
void launch_long_top_d(const double *x, int64_t n, int64_t ld, int64_t nch, int64_t ddof, const SliceWsD &ws,
                       double *var, double *mean, dim3 grid, hipStream_t st) {
  if (nch <= 256) k_long_top_d<PASS, 1, P><<<grid, 256, 0, st>>>(x, n, ld, nch, ddof, ws, var, mean);
  else if (nch <= 1024) k_long_top_d<PASS, 4, P><<<grid, 256, 0, st>>>(x, n, ld, nch, ddof, ws, var, mean);
  else k_long_top_d<PASS, L64_TOP_MAX_K, P><<<grid, 256, 0, st>>>(x, n, ld, nch, ddof, ws, var, mean);
}

// A matrix of two columns along axis 0 as one row of n pairs: the chunk
// launches of k_long_rows_d over both interleaved slices at once (16-byte
// loads of whole rows), chunks of 4096 rows.  The workspace holds the node
// arrays of 2 * nch chunk nodes.
void launch_long_pairs_d(bool vec, const double *x, int64_t n, int64_t ddof, void *workspace, double *var,
                         double *mean, hipStream_t st) {
  const int64_t nch = (n + L64_ROW_CHUNK / 2 - 1) / (L64_ROW_CHUNK / 2);
  const SliceWsD ws = slice_ws(workspace, 2 * nch);
  const dim3 grid((unsigned)nch), block(64 * L64_W), top(2);
  if (vec) k_long_rows_d<0, true, 2><<<grid, block, 0, st>>>(x, n, 2 * n, nch, ws);
  else k_long_rows_d<0, false, 2><<<grid, block, 0, st>>>(x, n, 2 * n, nch, ws);
  launch_long_top_d<0, 2>(x, n, 2 * n, nch, ddof, ws, var, mean, top, st);
  if (vec) k_long_rows_d<1, true, 2><<<grid, block, 0, st>>>(x, n, 2 * n, nch, ws);
  else k_long_rows_d<1, false, 2><<<grid, block, 0, st>>>(x, n, 2 * n, nch, ws);
  launch_long_top_d<1, 2>(x, n, 2 * n, nch, ddof, ws, var, mean, top, st);
}

template <int V, int G>
void launch_cols_d(const double *x, int64_t R, int64_t C, int64_t ddof, const SliceWsD &ws, double *var,
                   double *mean, hipStream_t st) {
  const svx::ColsChunkPlan p = svx::cols_chunk64_plan(V, R, C);  // G = p.G
  const int64_t nch = p.nch, ncb = p.ncb;
  const dim3 block(64 * L64_W);
  // workgroup b = cb * nch + j takes chunk j of column block cb; launches of
  // at most 2^32 - 1 work-items
  svh::in_batches(ncb * nch, 1, 64 * L64_W, [&](int64_t b0, int64_t nb) {
    k_cols_y_d<V, G><<<dim3((unsigned)nb), block, 0, st>>>(x, R, C, nch, ws, b0);
  });
  auto dq = [&](auto mlocal) {
    svh::in_batches(ncb * nch, 1, 64 * L64_W, [&](int64_t b0, int64_t nb) {
      k_cols_dq_d<V, G, decltype(mlocal)::value><<<dim3((unsigned)nb), block, 0, st>>>(x, R, C, nch, ws, b0);
    });
  };
  // the top kernels: four waves of per_wave columns each per workgroup
  auto top = [&](int per_wave, auto &&launch) {
    svh::in_batches((C + 4 * per_wave - 1) / (4 * per_wave), 1, 256,
                    [&](int64_t b0, int64_t nb) { launch(dim3((unsigned)nb), b0); });
  };
#define SV_TOP64(PASS, K, S, PW)                                                                          \
  top(PW, [&](dim3 g, int64_t b0) {                                                                      \
    k_cols_top_d<PASS, K, S><<<g, dim3(256), 0, st>>>(x, R, C, nch, ddof, ws, var, mean, b0);            \
  })
  if (nch <= C64_GROUP) {
    dq(std::true_type{});
    // the final trees: a group of S >= nch lanes per column, one node each
    if (nch <= 4) SV_TOP64(1, 1, 4, 16);
    else if (nch <= 8) SV_TOP64(1, 1, 8, 8);
    else if (nch <= 16) SV_TOP64(1, 1, 16, 4);
    else SV_TOP64(1, 1, 32, 2);
  } else if (nch <= 64 * 64) {
    // many chunks: a wave per column for m and for the final trees
    if (nch <= 64 * 4) {
      SV_TOP64(0, 4, 64, 1);
      dq(std::false_type{});
      SV_TOP64(1, 4, 64, 1);
    } else if (nch <= 64 * 16) {
      SV_TOP64(0, 16, 64, 1);
      dq(std::false_type{});
      SV_TOP64(1, 16, 64, 1);
    } else {
      SV_TOP64(0, 64, 64, 1);
      dq(std::false_type{});
      SV_TOP64(1, 64, 64, 1);
    }
  } else {
    int log2p = 0;  // runs of 64 * 2^log2p chunk nodes per lane
    while (((int64_t)64 * 64 << log2p) < nch) ++log2p;
    top(1, [&](dim3 g, int64_t b0) {
      k_cols_top_big_d<0><<<g, dim3(256), 0, st>>>(x, R, C, nch, log2p, ddof, ws, var, mean, b0);
    });
    dq(std::false_type{});
    top(1, [&](dim3 g, int64_t b0) {
      k_cols_top_big_d<1><<<g, dim3(256), 0, st>>>(x, R, C, nch, log2p, ddof, ws, var, mean, b0);
    });
  }
#undef SV_TOP64
}

// Row groups per wave, so that lanes stay on columns (svx::cols_chunk64_plan):
// with `groups` column groups of V, G = 1 for at least 64 groups, 4 for 9 to
// 63 (16 groups per block), 8 for 5 to 8, 16 for 3 and 4, 32 for 2 and 64
// for one.
template <int V>
void launch_cols_gd(const double *x, int64_t R, int64_t C, int64_t ddof, const SliceWsD &ws, double *var,
                    double *mean, hipStream_t st) {
  switch (svx::cols_chunk64_plan(V, R, C).G) {
    case 1: launch_cols_d<V, 1>(x, R, C, ddof, ws, var, mean, st); break;
    case 4: launch_cols_d<V, 4>(x, R, C, ddof, ws, var, mean, st); break;
    case 8: launch_cols_d<V, 8>(x, R, C, ddof, ws, var, mean, st); break;
    case 16: launch_cols_d<V, 16>(x, R, C, ddof, ws, var, mean, st); break;
    case 32: launch_cols_d<V, 32>(x, R, C, ddof, ws, var, mean, st); break;
    default: launch_cols_d<V, 64>(x, R, C, ddof, ws, var, mean, st); break;
  }
}

// Columns of 64 < R <= 4096 rows in one launch (k_cols_one_d), 16*G*W = the
// power of two at or above R rows per workgroup:
//   R <= 512: one column per lane (16 doubles per lane), G 1 or 4 (row
//     segments of at least 16 lanes, 128 bytes), W up to 16, G = 1 when that
//     still gives 512 workgroups;
//   R > 512: two adjacent columns per lane (one 16-byte load per row for an
//     aligned base and an even width, else two 8-byte loads; one column for
//     a single column); G = 16, W = 4;
//   R > 1024 (at least two columns): as above with W = 8 (512 work-items
//     holding 32 doubles each), and G = 32 above 2048 rows (four columns
//     per workgroup).  At 16 waves the 128 registers a lane may then use
//     hold too little for the masked kernel: the tile spills.  At exactly
//     2048 or 4096 rows the mask-free instance runs instead, and with
//     `wide` (16-byte loads, a grid that fills the chip) 16 waves with G = 8
//     or 16: sixteen or eight columns, 128- or 64-byte row segments.
// Measured (us, one column per lane against two): [100, 140000] 26.5 / 39.6,
// [512, 4096] 8.0 / 10.9; [1000, 20000] 65.2 / 52.5, [1000, 1000] 13.0 / 6.9.
void launch_cols_one_d(const double *x, int64_t R, int64_t C, int64_t ddof, bool vec, bool wide, double *var,
                       double *mean, hipStream_t st) {
  const svx::ColsOne64Plan p = svx::cols_one64_plan(R, C, vec, wide);
#define SV_ONE64(V_, W_, G_, ...)                                                                         \
  svh::in_batches(p.blocks, 1, 64 * W_, [&](int64_t b0, int64_t nb) {                                    \
    k_cols_one_d<V_, W_, G_, ##__VA_ARGS__><<<dim3((unsigned)nb), dim3(64 * W_), 0, st>>>(x, R, C, ddof, var, \
                                                                                         mean, (int)b0);  \
  })
  if (p.W == 16 && p.V == 2) {  // the wide tiles (exactly 2048 or 4096 rows, 16-byte loads)
    if (p.G == 16) SV_ONE64(2, 16, 16, true, 1);
    else SV_ONE64(2, 16, 8, true, 1);
  } else if (p.V == 2 && p.G == 32) {
    if (R == 4096) {
      if (vec) SV_ONE64(2, 8, 32, true, 1);
      else SV_ONE64(2, 8, 32, false, 1);
    } else if (vec) SV_ONE64(2, 8, 32, true, 2);
    else SV_ONE64(2, 8, 32, false, 2);
  } else if (p.V == 2 && p.W == 8) {
    if (R == 2048) {
      if (vec) SV_ONE64(2, 8, 16, true, 1);
      else SV_ONE64(2, 8, 16, false, 1);
    } else if (vec) SV_ONE64(2, 8, 16, true, 2);
    else SV_ONE64(2, 8, 16, false, 2);
  } else if (p.V == 2) {
    if (vec) SV_ONE64(2, 4, 16);
    else SV_ONE64(2, 4, 16, false);  // two 8-byte loads
  } else if (p.G == 16) {
    SV_ONE64(1, 4, 16);  // a single column of 513..1024 rows
  } else {
    switch (p.G * 32 + p.W) {  // 64 < R <= 512: 128 <= 16*G*W <= 512
      case 32 * 1 + 8: SV_ONE64(1, 8, 1); break;
      case 32 * 1 + 16: SV_ONE64(1, 16, 1); break;
      case 32 * 4 + 2: SV_ONE64(1, 2, 4); break;
      case 32 * 4 + 4: SV_ONE64(1, 4, 4); break;
      default: SV_ONE64(1, 8, 4); break;  // gw = 32
    }
  }
#undef SV_ONE64
}

}  // namespace

extern "C" {

size_t sv_tree_sum_f64_workspace_size(int64_t n) {
  if (n < 0 || n > S64_MAX_N) return (size_t)-1;
  if (n == 0) return 0;
  return S64_WS_HEADER + (size_t)(S64_MAX_BLOCKS + S64_MAX_BLOCKS / S64_GROUP) * sizeof(NodeD);
}

sv_status sv_tree_sum_f64(const double *x, int64_t n, double *out, void *workspace, size_t workspace_bytes,
                          void *stream) {
  if (n < 0) return fail(SV_ERR_INVALID_ARGUMENT, "sv_tree_sum_f64: n = %lld < 0", (long long)n);
  if (n > S64_MAX_N) return fail(SV_ERR_UNSUPPORTED, "sv_tree_sum_f64: n = %lld above 2^35", (long long)n);
  if (!out) return fail(SV_ERR_INVALID_ARGUMENT, "sv_tree_sum_f64: out is NULL");
  if (n > 0 && !x) return fail(SV_ERR_INVALID_ARGUMENT, "sv_tree_sum_f64: x is NULL with n > 0");
  if (reinterpret_cast<uintptr_t>(x) & 7u) return fail(SV_ERR_INVALID_ARGUMENT, "sv_tree_sum_f64: x is not 8-byte aligned");
  const size_t need = sv_tree_sum_f64_workspace_size(n);
  if (n > 0) {
    if (!workspace) return fail(SV_ERR_WORKSPACE, "sv_tree_sum_f64: workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
      return fail(SV_ERR_WORKSPACE, "sv_tree_sum_f64: workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (!svh::aligned256(workspace)) return fail(SV_ERR_WORKSPACE, "sv_tree_sum_f64: workspace is not 256-byte aligned");
  }
  const sv_status dev = check_device();
  if (dev != SV_OK) return dev;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (n == 0) {
    k_zero_d<<<1, 1, 0, st>>>(out);
    return check_launch("sv_tree_sum_f64");
  }
  // chunks of 64 * 16 doubles, each wave streaming 2^g of them, g the
  // smallest value that keeps the workgroup count at or below S64_MAX_BLOCKS
  const svx::SumPlan plan = svx::plan_sum(n, S64_EF / 2, S64_MAX_BLOCKS, S64_W, S64_MAX_BLOCKS, S64_MAX_LOG2_G);
  const int g = plan.log2_g;
  const int64_t blocks = plan.blocks;
  unsigned *counter = reinterpret_cast<unsigned *>(workspace);
  NodeD *part = reinterpret_cast<NodeD *>(reinterpret_cast<char *>(workspace) + S64_WS_HEADER);
  const dim3 grid((unsigned)blocks), block(64 * S64_W);
  if (svh::aligned16(x)) k_tree_sum_f64<true><<<grid, block, 0, st>>>(x, n, g, part, counter, out);
  else k_tree_sum_f64<false><<<grid, block, 0, st>>>(x, n, g, part, counter, out);
  return check_launch("sv_tree_sum_f64");
}

size_t sv_variance_f64_workspace_size(int64_t rows, int64_t cols, int axis) {
  if (rows < 0 || cols < 0) return (size_t)-1;
  if (axis != 0 && axis != 1 && axis != -1 && axis != -2) return (size_t)-1;
  if (cols > 0 && rows > V64_MAX_ELEMS / cols) return (size_t)-1;
  const bool ax1 = (axis == 1 || axis == -1);
  if (!ax1 && (rows + C64_CHUNK - 1) / C64_CHUNK > ((int64_t)64 * 64 << (TOP_BIG_LEVELS_D - 1))) return (size_t)-1;
  return var64_ws(rows, cols, ax1);
}

sv_status sv_variance_f64(const double *x, int64_t rows, int64_t cols, int axis, int64_t ddof, double *var_out,
                          double *mean_out, void *workspace, size_t workspace_bytes, void *stream) {
  if (rows < 0 || cols < 0)
    return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_f64: negative shape [%lld, %lld]", (long long)rows,
                (long long)cols);
  if (axis != 0 && axis != 1 && axis != -1 && axis != -2)
    return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_f64: axis %d not in {0, 1, -1, -2}", axis);
  if (ddof < 0) return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_f64: ddof = %lld < 0", (long long)ddof);
  const bool ax1 = (axis == 1 || axis == -1);
  const int64_t nslices = ax1 ? rows : cols;
  const int64_t n = ax1 ? cols : rows;
  if (cols > 0 && rows > V64_MAX_ELEMS / cols)
    return fail(SV_ERR_UNSUPPORTED, "sv_variance_f64: rows * cols above 2^35");
  if (nslices == 0) return ok();
  if (!var_out) return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_f64: var_out is NULL");
  if (n > 0 && !x) return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_f64: x is NULL");
  if (reinterpret_cast<uintptr_t>(x) & 7u) return fail(SV_ERR_INVALID_ARGUMENT, "sv_variance_f64: x is not 8-byte aligned");
  if (nslices > 0x7fffffffLL)
    return fail(SV_ERR_UNSUPPORTED, "sv_variance_f64: %lld slices exceed the grid", (long long)nslices);
  // axis 0: the per-column trees hold up to 64 * 64 * 2^(TOP_BIG_LEVELS_D - 1)
  // chunk nodes; chunks are at least 128 rows
  if (!ax1 && (n + C64_CHUNK - 1) / C64_CHUNK > ((int64_t)64 * 64 << (TOP_BIG_LEVELS_D - 1)))
    return fail(SV_ERR_UNSUPPORTED, "sv_variance_f64: columns of %lld rows exceed the chunk trees", (long long)n);
  const size_t need = var64_ws(rows, cols, ax1);
  if (need == (size_t)-1)
    return fail(SV_ERR_UNSUPPORTED, "sv_variance_f64: rows of %lld values exceed %lld chunks", (long long)n,
                (long long)L64_MAX_CHUNKS);
  if (need > 0) {
    if (!workspace) return fail(SV_ERR_WORKSPACE, "sv_variance_f64: workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
      return fail(SV_ERR_WORKSPACE, "sv_variance_f64: workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (!svh::aligned256(workspace)) return fail(SV_ERR_WORKSPACE, "sv_variance_f64: workspace is not 256-byte aligned");
  }
  const sv_status dev = check_device();
  if (dev != SV_OK) return dev;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (n == 0) {
    k_fill_nan_d<<<dim3((unsigned)((nslices + 255) / 256)), dim3(256), 0, st>>>(var_out, mean_out, nslices);
    return check_launch("sv_variance_f64");
  }
  if (!ax1 && cols == 1 && rows <= L64_MAX_CHUNKS * L64_ROW_CHUNK) {
    // A single column is one contiguous slice, as is the single row
    // [1, rows]: the same values in the same order, hence the same tree and
    // bits; the row form reads it with wide loads and needs less workspace
    // than the column form, which the caller sized.
    return sv_variance_f64(x, 1, rows, 1, ddof, var_out, mean_out, workspace, workspace_bytes, stream);
  }
  const bool vec = svh::aligned16(x) && (cols % 2 == 0);
  // Columns of 1025..4096 rows: read once by workgroups of eight or four
  // whole columns (32 doubles per lane) unless that grid leaves the chip's
  // last round mostly empty, a round being one workgroup per CU.  Columns of
  // exactly 2048 or 4096 rows with 16-byte loads take the wide 16-wave tile
  // when its own grid fills the chip by the same rule.  var_cols_once 2
  // takes the one read, and the wide tile where it applies, whatever the fill.
  bool one_read = false, wide = false;
  if (svx::cols_one_read64_candidate(ax1, rows, cols, svh::cols_once())) {
    const bool forced = svh::cols_once() == 2;
    int cus = 0, dev = 0;
    if (!forced && (hipGetDevice(&dev) != hipSuccess ||
                    hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess))
      cus = 0;
    const svx::ColsOne64Plan p = svx::cols_one64_plan(rows, cols, vec);
    one_read = forced || svx::one_round_fill(p.blocks, cus);
    if (svx::cols_one64_wide_ok(rows, vec)) {
      wide = forced || svx::one_round_fill(svx::cols_one64_plan(rows, cols, vec, true).blocks, cus);
      one_read = one_read || wide;
    }
  }
  switch (svx::f64_route(rows, cols, ax1, vec, one_read, svh::cols_pairs(), svh::long_rows() != 0)) {
    case svx::Route64::ROWS_SEG: {
      // rows of up to 512 doubles sharing waves: 16-byte loads of two
      // doubles for aligned rows of an even count, else single doubles
      const StepConstsD sk = step_consts_d(n, ddof);
#define SV_SEG64(E, S)                                                                                  \
  svh::in_batches(rows, 4 * (64 / S), 256, [&](int64_t r0, int64_t nr) {                                \
    const dim3 sgrid((unsigned)((nr + 4 * (64 / S) - 1) / (4 * (64 / S))));                             \
    const double *xr = x + r0 * cols;                                                                   \
    double *vr = var_out + r0, *mr = mean_out ? mean_out + r0 : nullptr;                                \
    if (vec) k_var_rows_seg_d<E, S, 2><<<sgrid, dim3(256), 0, st>>>(xr, nr, n, cols, sk, vr, mr);       \
    else k_var_rows_seg_d<E, S, 1><<<sgrid, dim3(256), 0, st>>>(xr, nr, n, cols, sk, vr, mr);           \
  })
      const svx::SegPlan sp = svx::seg_plan(n);
      switch (sp.E * 100 + sp.S) {
        case 401: SV_SEG64(4, 1); break;
        case 801: SV_SEG64(8, 1); break;
        case 1601: SV_SEG64(16, 1); break;
        case 1602: SV_SEG64(16, 2); break;
        case 1604: SV_SEG64(16, 4); break;
        case 1608: SV_SEG64(16, 8); break;
        case 1616: SV_SEG64(16, 16); break;
        default: SV_SEG64(16, 32); break;
      }
#undef SV_SEG64
      break;
    }
    case svx::Route64::ROWS_TILE: {
#define SV_ROWS64(E, W)                                                                                      \
  svh::in_batches(rows, 1, 64 * svx::rows_waves(n, E, W), [&](int64_t r0, int64_t nr) {                     \
    const double *xr = x + r0 * cols;                                                                        \
    double *mr = mean_out ? mean_out + r0 : nullptr;                                                         \
    const dim3 block(64 * svx::rows_waves(n, E, W));  /* only the waves the row reaches */                  \
    if (vec) k_var_rows_f64<E, W, true><<<dim3((unsigned)nr), block, 0, st>>>(xr, n, cols, ddof, var_out + r0, mr); \
    else k_var_rows_f64<E, W, false><<<dim3((unsigned)nr), block, 0, st>>>(xr, n, cols, ddof, var_out + r0, mr);   \
  })
      const svx::RowsPlan rp = svx::rows64_plan(n);
      switch (rp.E * 100 + rp.W) {
        case 1601: SV_ROWS64(16, 1); break;
        case 1602: SV_ROWS64(16, 2); break;
        case 1604: SV_ROWS64(16, 4); break;
        case 1608: SV_ROWS64(16, 8); break;
        case 1616: SV_ROWS64(16, 16); break;
        default: SV_ROWS64(32, 16); break;
      }
#undef SV_ROWS64
      break;
    }
    case svx::Route64::LONG_ROWS_CHUNKED: {
      const int64_t nch = (n + L64_ROW_CHUNK - 1) / L64_ROW_CHUNK;
      const SliceWsD ws = slice_ws(workspace, rows * nch);
      const dim3 lgrid((unsigned)(rows * nch)), lblock(64 * L64_W), grid((unsigned)rows);
      if (vec) k_long_rows_d<0, true><<<lgrid, lblock, 0, st>>>(x, n, cols, nch, ws);
      else k_long_rows_d<0, false><<<lgrid, lblock, 0, st>>>(x, n, cols, nch, ws);
      launch_long_top_d<0>(x, n, cols, nch, ddof, ws, var_out, mean_out, grid, st);
      if (vec) k_long_rows_d<1, true><<<lgrid, lblock, 0, st>>>(x, n, cols, nch, ws);
      else k_long_rows_d<1, false><<<lgrid, lblock, 0, st>>>(x, n, cols, nch, ws);
      launch_long_top_d<1>(x, n, cols, nch, ddof, ws, var_out, mean_out, grid, st);
      break;
    }
    case svx::Route64::COLS_CHUNKED: {
      const SliceWsD ws = slice_ws(workspace, ((n + C64_CHUNK - 1) / C64_CHUNK) * cols);
      if (vec) launch_cols_gd<2>(x, rows, cols, ddof, ws, var_out, mean_out, st);
      else launch_cols_gd<1>(x, rows, cols, ddof, ws, var_out, mean_out, st);
      break;
    }
    case svx::Route64::COLS_ONE: launch_cols_one_d(x, rows, cols, ddof, vec, wide, var_out, mean_out, st); break;
    case svx::Route64::COLS_PAIRS: launch_long_pairs_d(vec, x, rows, ddof, workspace, var_out, mean_out, st); break;
    case svx::Route64::COLS_SHORT: {
      const int e = svx::cols_short_e(n);
      svh::in_batches((cols / 2 + 255) / 256, 1, 256, [&](int64_t b0, int64_t nb) {
        const dim3 grid((unsigned)nb), block(256);
        switch (e) {
          case 2: k_cols_short_d<2><<<grid, block, 0, st>>>(x, rows, cols, ddof, var_out, mean_out, b0); break;
          case 4: k_cols_short_d<4><<<grid, block, 0, st>>>(x, rows, cols, ddof, var_out, mean_out, b0); break;
          case 8: k_cols_short_d<8><<<grid, block, 0, st>>>(x, rows, cols, ddof, var_out, mean_out, b0); break;
          default: k_cols_short_d<16><<<grid, block, 0, st>>>(x, rows, cols, ddof, var_out, mean_out, b0); break;
        }
      });
      break;
    }
    case svx::Route64::COLS_LANE: {
      const svx::RowsPlan lp = svx::cols_lane64_plan(n);
#define SV_COLS64(E, W)                                                                                  \
  svh::in_batches((cols + 63) / 64, 1, 64 * W, [&](int64_t b0, int64_t nb) {                             \
    k_var_cols_f64<E, W><<<dim3((unsigned)nb), dim3(64 * W), 0, st>>>(x, rows, cols, ddof, var_out, mean_out, b0); \
  })
      switch (lp.E * 100 + lp.W) {
        case 401: SV_COLS64(4, 1); break;
        case 1601: SV_COLS64(16, 1); break;
        default: SV_COLS64(16, 4); break;
      }
#undef SV_COLS64
      break;
    }
  }
  return check_launch("sv_variance_f64");
}

}  // extern "C"
