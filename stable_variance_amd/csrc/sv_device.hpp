// Device building blocks of the compensated pairwise tree on gfx950 (CDNA4).
//
// Method: Pennacchio, "Variance in float32 with a first-element shift, a
// local centring and a compensated tree sum", §2 step 3: a binary tree whose
// levels add pairs of partial sums with TwoSum, the exact errors carried up a
// second array, the result being the final sum plus the final carry.
//
// Topology (fixed): values padded with +0 to a power of two, adjacent pairs
// at each level, so a node covers a power-of-two aligned range.  On the GPU a
// lane owns E consecutive values (in-lane levels), the 64 lanes of a wave own
// 64 consecutive lane ranges (6 cross-lane levels) and the waves of a
// workgroup own consecutive wave ranges (LDS levels).  Larger power-of-two
// tiles than the data needs only add +0 padding, which leaves the result bits
// unchanged (TwoSum(a, +0) = (a, +0) up to the sign of a zero, and the carry
// of a compensated tree is never -0).
//
// Node order.  TwoSum's error is the unique exact value a + b - fl(a + b), so
// a node combined as (left, right) or (right, left) has the same bits on a
// finite sum; the cross-lane levels use that freedom.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_index.hpp"

#if defined(__FAST_MATH__)
#error "stable_variance must be built without fast-math (TwoSum needs exact IEEE rounding)"
#endif
#if defined(__FINITE_MATH_ONLY__) && __FINITE_MATH_ONLY__
#error "stable_variance must be built without finite-math-only"
#endif

namespace sv {

struct Node {
  float s;  // partial sum
  float c;  // carried rounding errors
};

// ---------------------------------------------------------------- launch order

// The eight dies (XCDs) of the chip take a grid's workgroups round robin in
// dispatch order: workgroup b runs on die b mod 8.  xcd_contiguous renumbers
// the grid so that each die's workgroups get one contiguous run of logical
// indices (die x takes the x-th run, the first nb mod 8 runs one longer), so
// a die streams one region of the buffer.  A bijection of [0, nb): results
// depend only on logical indices, so the renumbering changes no bit.
using svx::xcd_contiguous;

// ---------------------------------------------------------------- nodes

// TwoSum of the two partial sums, the error added to the sum of the carries.
__device__ __forceinline__ Node combine(Node l, Node r) {
  const float s = l.s + r.s;
  const float bv = s - l.s;
  const float av = s - bv;
  const float e = (l.s - av) + (r.s - bv);
  return {s, (l.c + r.c) + e};
}

// A level-1 node from two raw values.  The carry is fl(fl(0 + 0) + e), i.e.
// e with a -0 turned into +0 (needed for the exact sign of an all -0 sum).
__device__ __forceinline__ Node leaf_canon(float a, float b) {
  const float s = a + b;
  const float bv = s - a;
  const float av = s - bv;
  const float e = (a - av) + (b - bv);
  return {s, 0.0f + e};
}

// Level-1 node whose carry keeps e as is.  Only the sign of a zero carry can
// differ from leaf_canon, which the variance outputs never see (S1 enters
// squared, and the sum of y or of d^2 is never -0).
__device__ __forceinline__ Node leaf_fast(float a, float b) {
  const float s = a + b;
  const float bv = s - a;
  const float av = s - bv;
  return {s, (a - av) + (b - bv)};
}

// Nodes of non-negative values (the tree of d^2): every partial sum is >= 0,
// so the larger operand is known after one max/min, and Fast2Sum (Dekker)
// gives the same exact error as TwoSum in 3 operations instead of 4.  The
// sum itself is formed from the operands directly, so a NaN still
// propagates through s; a non-finite s makes the root return s anyway.
__device__ __forceinline__ Node combine_nn(Node l, Node r) {
  const float s = l.s + r.s;
  const float hi = __builtin_fmaxf(l.s, r.s);
  const float lo = __builtin_fminf(l.s, r.s);
  const float e = lo - (s - hi);
  return {s, (l.c + r.c) + e};
}

__device__ __forceinline__ Node leaf_nn(float a, float b) {
  const float s = a + b;
  const float hi = __builtin_fmaxf(a, b);
  const float lo = __builtin_fminf(a, b);
  return {s, lo - (s - hi)};
}

// Double-word node: the compensated node, then the pair renormalised with
// TwoSum, (s, c) <- TwoSum(s, c), so that |c| <= ulp(s)/2 after every node.
// The renormalisation of a pair that TwoSum produced returns it unchanged,
// so zero padding still leaves the bits alone; TwoSum is symmetric in its
// operands, so the node is too.  A pair whose sum is Inf or NaN stays as it
// is (Inf + NaN would turn an Inf into NaN; the root guard returns s).
__device__ __forceinline__ Node renorm_dw(Node n) {
  const float s = n.s + n.c;
  const float bv = s - n.s;
  const float av = s - bv;
  const float c = (n.s - av) + (n.c - bv);
  const bool fin = __builtin_isfinite(n.s);
  return {fin ? s : n.s, fin ? c : n.c};
}

__device__ __forceinline__ Node combine_dw(Node l, Node r) { return renorm_dw(combine(l, r)); }

__device__ __forceinline__ Node leaf_dw(float a, float b) { return renorm_dw(leaf_canon(a, b)); }

// Plain pairwise node: fl(l.s + r.s) and no carry (c stays +0).  Its s part
// is the same sum as the compensated node's s, so a plain tree is the s half
// of a compensated tree of the same topology.
__device__ __forceinline__ Node combine_plain(Node l, Node r) { return {l.s + r.s, 0.0f}; }

// Node kinds of the cross-lane and node-array trees.
enum NodeKind { NODE_TWOSUM = 0, NODE_NN = 1, NODE_DW = 2, NODE_PLAIN = 3 };

template <int KIND>
__device__ __forceinline__ Node combine_k(Node l, Node r) {
  if constexpr (KIND == NODE_NN) return combine_nn(l, r);
  else if constexpr (KIND == NODE_DW) return combine_dw(l, r);
  else if constexpr (KIND == NODE_PLAIN) return combine_plain(l, r);
  else return combine(l, r);
}

// Value of a tree at its root: fl(s + c), or s when s is Inf or NaN.
__device__ __forceinline__ float root_value(Node n) {
  return __builtin_isfinite(n.s) ? n.s + n.c : n.s;
}

// Value at the root of a tree of the given kind.  A plain tree's carry is
// zero, so its value is fl(s + 0): s itself, except that an all -0 sum gives
// +0, whatever the +0 padding beyond the data (the compensated tree's
// carries are never -0, so fl(s + c) has the same property).
template <int KIND>
__device__ __forceinline__ float root_value_k(Node n) {
  if constexpr (KIND == NODE_PLAIN) return n.s + 0.0f;
  else return root_value(n);
}

__device__ __forceinline__ Node zero_node() { return {0.0f, 0.0f}; }

// ---------------------------------------------------------------- in-lane trees

enum LeafKind { LEAF_CANON = 0, LEAF_FAST = 1, LEAF_NN = 2, LEAF_DW = 3, LEAF_PLAIN = 4 };

// The tree of the local mean, m = sum(y) / n (method page §2 step 2): the
// plain pairwise tree, the s half of the compensated tree's topology.  The
// sums of d and d^2 (step 3) take the compensated tree.
constexpr int Y_KIND = NODE_PLAIN;
constexpr int Y_LEAF = LEAF_PLAIN;

// Subtrees of at least this many values are scheduled one after the other
// (a scheduling barrier between siblings): the compiler then interleaves
// only within a subtree, which keeps about log2(E) partial nodes live instead
// of a whole tree level.
#ifndef SV_SCHED_BLOCK
#define SV_SCHED_BLOCK 16
#endif
constexpr int SCHED_BLOCK = SV_SCHED_BLOCK;

// Compensated tree over v[OFF .. OFF+N) (N a power of two >= 2).
template <int LEAF, int OFF, int N, int E>
__device__ __forceinline__ Node lane_tree(const float (&v)[E]) {
  static_assert(N >= 2 && (N & (N - 1)) == 0, "power of two");
  if constexpr (N == 2) {
    if constexpr (LEAF == LEAF_CANON) return leaf_canon(v[OFF], v[OFF + 1]);
    else if constexpr (LEAF == LEAF_FAST) return leaf_fast(v[OFF], v[OFF + 1]);
    else if constexpr (LEAF == LEAF_DW) return leaf_dw(v[OFF], v[OFF + 1]);
    else if constexpr (LEAF == LEAF_PLAIN) return {v[OFF] + v[OFF + 1], 0.0f};
    else return leaf_nn(v[OFF], v[OFF + 1]);
  } else {
    const Node l = lane_tree<LEAF, OFF, N / 2, E>(v);
    if constexpr (N / 2 >= SCHED_BLOCK && LEAF != LEAF_PLAIN) __builtin_amdgcn_sched_barrier(0);
    const Node r = lane_tree<LEAF, OFF + N / 2, N / 2, E>(v);
    if constexpr (N / 2 >= SCHED_BLOCK && LEAF != LEAF_PLAIN) __builtin_amdgcn_sched_barrier(0);
    if constexpr (LEAF == LEAF_NN) return combine_nn(l, r);
    else if constexpr (LEAF == LEAF_DW) return combine_dw(l, r);
    else if constexpr (LEAF == LEAF_PLAIN) return combine_plain(l, r);
    else return combine(l, r);
  }
}

// Tree over an array of nodes nd[OFF .. OFF+N).
template <int OFF, int N, int K, int KIND = NODE_TWOSUM>
__device__ __forceinline__ Node node_tree(const Node (&nd)[K]) {
  if constexpr (N == 1) {
    return nd[OFF];
  } else {
    return combine_k<KIND>(node_tree<OFF, N / 2, K, KIND>(nd), node_tree<OFF + N / 2, N / 2, K, KIND>(nd));
  }
}

// The two trees of the second pass, d_i = fl(y_i - m) and q_i = fl(d_i*d_i),
// built leaf pair by leaf pair so that only log2(E) partial nodes stay live.
// MASK: element OFF+i of this lane is beyond the slice when OFF+i >= valid;
// its d and q are then +0 (the padding of the tree), not fl(0 - m).
template <bool MASK, int OFF, int N, int E>
__device__ __forceinline__ void lane_tree_dq(const float (&y)[E], float m, int valid, Node &nd, Node &nq) {
  if constexpr (N == 2) {
    float d0 = y[OFF] - m;
    float d1 = y[OFF + 1] - m;
    if constexpr (MASK) {
      d0 = (OFF < valid) ? d0 : 0.0f;
      d1 = (OFF + 1 < valid) ? d1 : 0.0f;
    }
    const float q0 = d0 * d0;
    const float q1 = d1 * d1;
    nd = leaf_fast(d0, d1);
    nq = leaf_nn(q0, q1);
  } else {
    Node ld, lq, rd, rq;
    lane_tree_dq<MASK, OFF, N / 2, E>(y, m, valid, ld, lq);
    if constexpr (N / 2 >= SCHED_BLOCK) __builtin_amdgcn_sched_barrier(0);
    lane_tree_dq<MASK, OFF + N / 2, N / 2, E>(y, m, valid, rd, rq);
    if constexpr (N / 2 >= SCHED_BLOCK) __builtin_amdgcn_sched_barrier(0);
    nd = combine(ld, rd);
    nq = combine_nn(lq, rq);
  }
}

// ---------------------------------------------------------------- cross-lane levels

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// DPP controls (gfx9 family)
constexpr int DPP_QUAD_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <- lane 7-i within 8
constexpr int DPP_ROW_MIRROR = 0x140;       // lane i <- lane 15-i within 16

// The neighbour's node; a plain tree moves only its sums (its carries are
// +0 everywhere).
template <int CTRL, int KIND = NODE_TWOSUM>
__device__ __forceinline__ Node dpp_node(Node n) {
  if constexpr (KIND == NODE_PLAIN) return {dpp<CTRL>(n.s), 0.0f};
  else return {dpp<CTRL>(n.s), dpp<CTRL>(n.c)};
}

// Cross-row exchanges of gfx950 (one VALU instruction per register, no LDS):
// v_permlane16_swap on two copies of x leaves, in every lane L, x[L] and
// x[L ^ 16] in the two registers (one in each); v_permlane32_swap likewise
// for x[L ^ 32].  Which register holds the lane's own value does not matter:
// the node combine is symmetric bit for bit.  Written as inline assembly
// because the compiler builtin's second result has been miscompiled (read as
// a copy of the first) once the results feed arithmetic.  The wait states
// around the instruction cover the VALU-write-then-permlane hazards.
struct NodePair { Node a, b; };

template <int XOR>
__device__ __forceinline__ void swap_halves(float v, float &a, float &b) {
  static_assert(XOR == 16 || XOR == 32, "lane distance 16 or 32");
  unsigned x = __builtin_bit_cast(unsigned, v), y = x;
  if constexpr (XOR == 16)
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  else
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  a = __builtin_bit_cast(float, x);
  b = __builtin_bit_cast(float, y);
}

template <int XOR, int KIND = NODE_TWOSUM>
__device__ __forceinline__ NodePair swap_node(Node n) {
  NodePair p;
  swap_halves<XOR>(n.s, p.a.s, p.b.s);
  if constexpr (KIND == NODE_PLAIN) {
    p.a.c = 0.0f;
    p.b.c = 0.0f;
  } else {
    swap_halves<XOR>(n.c, p.a.c, p.b.c);
  }
  return p;
}

// The six cross-lane levels: lane k's node covers lane range k; afterwards
// every lane holds the wave's node.  Level 1 pairs lanes (2k, 2k+1), level 2
// pairs of pairs, and so on.  The mirror permutations reach the right sibling
// because all lanes of the previous group already hold the same node.
template <int KIND>
__device__ __forceinline__ Node wave_tree(Node n) {
  auto comb = [](Node a, Node b) { return combine_k<KIND>(a, b); };
  n = comb(n, dpp_node<DPP_QUAD_XOR1, KIND>(n));
  n = comb(n, dpp_node<DPP_QUAD_XOR2, KIND>(n));
  n = comb(n, dpp_node<DPP_ROW_HALF_MIRROR, KIND>(n));
  n = comb(n, dpp_node<DPP_ROW_MIRROR, KIND>(n));
  NodePair p = swap_node<16, KIND>(n);
  n = comb(p.a, p.b);
  p = swap_node<32, KIND>(n);
  return comb(p.a, p.b);
}

// The first log2(S) of those levels: afterwards every lane holds the node of
// its aligned group of S lanes (S = 1, 2, 4, ..., 64).
template <int KIND, int S>
__device__ __forceinline__ Node seg_tree(Node n) {
  static_assert(S >= 1 && S <= 64 && (S & (S - 1)) == 0, "segment of a power-of-two lanes");
  auto comb = [](Node a, Node b) { return combine_k<KIND>(a, b); };
  if constexpr (S >= 2) n = comb(n, dpp_node<DPP_QUAD_XOR1, KIND>(n));
  if constexpr (S >= 4) n = comb(n, dpp_node<DPP_QUAD_XOR2, KIND>(n));
  if constexpr (S >= 8) n = comb(n, dpp_node<DPP_ROW_HALF_MIRROR, KIND>(n));
  if constexpr (S >= 16) n = comb(n, dpp_node<DPP_ROW_MIRROR, KIND>(n));
  if constexpr (S >= 32) {
    const NodePair p = swap_node<16, KIND>(n);
    n = comb(p.a, p.b);
  }
  if constexpr (S >= 64) {
    const NodePair p = swap_node<32, KIND>(n);
    n = comb(p.a, p.b);
  }
  return n;
}

// ---------------------------------------------------------------- permuted lane order

// Lane L holding the range of virtual lane v(L) = 2 (L mod 32) + L / 32: the
// tree's first cross-lane level then pairs lanes L and L ^ 32, virtual bits
// 1..5 are lane bits 0..4, and the level order below follows.
using svx::vlane_pair32;

// Lane l's value of v, as a wave-uniform (scalar) value.
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// v_permlane32_swap on two registers: afterwards lanes 0..31 hold x of their
// own lane and of lane + 32, lanes 32..63 y of lane - 32 and of their own.
__device__ __forceinline__ void swap32_two(float x, float y, float &a, float &b) {
  unsigned u = __builtin_bit_cast(unsigned, x), t = __builtin_bit_cast(unsigned, y);
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(u), "+v"(t));
  a = __builtin_bit_cast(float, u);
  b = __builtin_bit_cast(float, t);
}

// The six cross-lane levels in the permuted order (lane xor 32 first, then
// xor 1, 2, the two mirrors, xor 16); every lane ends with the wave's node.
template <int KIND>
__device__ __forceinline__ Node wave_tree_p32(Node n) {
  auto comb = [](Node a, Node b) { return combine_k<KIND>(a, b); };
  NodePair p = swap_node<32, KIND>(n);
  n = comb(p.a, p.b);
  n = comb(n, dpp_node<DPP_QUAD_XOR1, KIND>(n));
  n = comb(n, dpp_node<DPP_QUAD_XOR2, KIND>(n));
  n = comb(n, dpp_node<DPP_ROW_HALF_MIRROR, KIND>(n));
  n = comb(n, dpp_node<DPP_ROW_MIRROR, KIND>(n));
  p = swap_node<16, KIND>(n);
  return comb(p.a, p.b);
}

// The d and d^2 trees of a wave together, in the permuted order: one swap of
// the two registers gives lanes 0..31 the pairs of the d tree and lanes
// 32..63 those of the d^2 tree, and the remaining five levels run once for
// both.  Lanes 0..31 return the wave's d node, lanes 32..63 its d^2 node.
// The d^2 levels use the TwoSum node: on non-negative operands its error is
// the same exact value, with the same sign of zero, as the Fast2Sum form.
__device__ __forceinline__ Node wave_tree_dq(Node nd, Node nq) {
  Node a, b;
  swap32_two(nd.s, nq.s, a.s, b.s);
  swap32_two(nd.c, nq.c, a.c, b.c);
  Node n = combine(a, b);
  n = combine(n, dpp_node<DPP_QUAD_XOR1>(n));
  n = combine(n, dpp_node<DPP_QUAD_XOR2>(n));
  n = combine(n, dpp_node<DPP_ROW_HALF_MIRROR>(n));
  n = combine(n, dpp_node<DPP_ROW_MIRROR>(n));
  const NodePair p = swap_node<16>(n);
  return combine(p.a, p.b);
}

// ---------------------------------------------------------------- device-coherent words

// Relaxed agent-scope (device-coherent) 32-bit store and load: they bypass
// the non-coherent caches, so a value published by one workgroup is seen by
// another without a cache writeback or invalidation.
__device__ __forceinline__ void store_u32_agent(unsigned *dst, unsigned v) {
  __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned load_u32_agent(const unsigned *src) {
  return __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt vmcnt(0): every vector memory operation of this wave, including
// the device-coherent stores above, has completed.
__device__ __forceinline__ void wait_vmem_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------- loads

// Wave-scope ordering of LDS traffic between the lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Number of floats of LDS one wave needs to transpose a 64*E tile: each
// reader lane's E values are padded by 4 floats so that neither the
// coalesced 16-byte writes nor the lane-contiguous 16-byte reads of 16
// consecutive lanes share a bank.
template <int E>
constexpr int lds_floats_per_wave() { return 64 * (E + 4); }

// LDS floats for the staged transpose (LOADP 2): one quarter of the lanes'
// ranges at a time, each padded by 4 floats.
template <int E>
constexpr int lds_floats_staged() { return 16 * (E + 4); }

// Values p[lane*E + i], i < E, of a 64*E tile starting at p; in a ragged
// tile, elements at or beyond `len` read as 0 (len may be <= 0, see below).
//
// LOADP 0: coalesced loads (each instruction covers 64 consecutive 16-byte
//          chunks, or 64 consecutive floats when !VEC), transposed through
//          this wave's LDS region into lane-contiguous order.
// LOADP 1: each lane loads its own E contiguous values directly.
// VEC: 16-byte loads; p must be 16-byte aligned and len, when below the
// tile, a multiple of 4.
// A wave whose tile lies entirely inside the data takes a branch-free path;
// a ragged tile (the slice's last) loads at addresses clamped to [0, len)
// (whole 16-byte groups when VEC, single floats otherwise); a tile entirely
// beyond the data loads nothing and leaves v unwritten (every caller masks
// the values past the slice, so zero-filling it would only cost one move per
// value on every wave).
typedef float sv_v4f __attribute__((ext_vector_type(4)));

// 16-byte and 4-byte loads; NT marks them non-temporal (streamed data that
// is read once and should not displace other lines in the caches).
template <bool NT>
__device__ __forceinline__ float4 ld4(const float *p) {
  if constexpr (NT) {
    const sv_v4f v = __builtin_nontemporal_load(reinterpret_cast<const sv_v4f *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const float4 *>(p);
  }
}

template <bool NT>
__device__ __forceinline__ float ld1(const float *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// avail: floats readable from p (the rest of the matrix, at least len).  A
// ragged tile with a whole tile readable (every row but the last few) loads
// as a full one, one base address with immediate offsets, and masks the
// values past len; otherwise each load's index is clamped to the data.
template <int E, bool VEC, int LOADP, bool NT = false>
__device__ __forceinline__ void load_tile(const float *__restrict__ p, int64_t len, float *__restrict__ lds,
                                          float (&v)[E], int lane, int64_t avail = 0) {
  static_assert(E >= 4 && (E & (E - 1)) == 0, "E must be a power of two >= 4");
  constexpr int J = E / 4;
  constexpr int STR = E + 4;
  constexpr int TILE = 64 * E;
  const bool full = len >= TILE;  // wave-uniform
  // ragged: number of valid values in [0, TILE]
  const int lim = svx::tile_lim(len, TILE);
  if (lim == 0) return;  // the whole tile lies beyond the data: no load, v left as is
  if constexpr (LOADP == 2) {
    // Staged transpose: coalesced 16-byte loads (instruction k covers values
    // [256k, 256k + 256)), then four stages through a quarter-size LDS region:
    // stage s holds the ranges of lanes 16s..16s+15, which read them back.
    static_assert(E % 16 == 0, "staged transpose needs E multiple of 16");
    constexpr int KS = J / 4;  // load instructions per stage
    if (full && VEC) {
      float4 g[J];
#pragma unroll
      for (int k = 0; k < J; ++k) g[k] = ld4<NT>(p + svx::tile_index(false, true, E, lane, k));
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          const int e = 256 * (st * KS + j) + 4 * lane;  // value index in the tile
          const int r = e / E - 16 * st;                 // reader lane within the stage
          *reinterpret_cast<float4 *>(lds + r * STR + (e % E)) = g[st * KS + j];
        }
        wave_lds_sync();
        if (lane / 16 == st) {
#pragma unroll
          for (int j = 0; j < J; ++j) {
            const float4 t = *reinterpret_cast<const float4 *>(lds + (lane - 16 * st) * STR + 4 * j);
            v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
          }
        }
        wave_lds_sync();
      }
      return;
    }
    // other cases: per-lane loads as LOADP 1
  }
  if constexpr (LOADP == 1 || LOADP == 2) {
    const int e0 = lane * E;
    if (full || avail >= TILE) {  // wave-uniform
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if constexpr (VEC) {
          const float4 g = ld4<NT>(p + svx::tile_index(true, true, E, lane, j));
          v[4 * j] = g.x; v[4 * j + 1] = g.y; v[4 * j + 2] = g.z; v[4 * j + 3] = g.w;
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) v[4 * j + t] = ld1<NT>(p + svx::tile_index(true, false, E, lane, 4 * j + t));
        }
      }
      if (!full) {
#pragma unroll
        for (int i = 0; i < E; ++i) v[i] = (e0 + i < lim) ? v[i] : 0.0f;
      }
    } else if constexpr (VEC) {
      // lim is a multiple of 4 (16-byte aligned rows of a multiple of 4
      // values), so each 16-byte group is wholly inside or wholly beyond the
      // data: clamped 16-byte loads, every one issued
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int e = svx::tile_index(true, true, E, lane, j);
        const float4 g = ld4<NT>(p + svx::clamp_group(e, lim, 4));
        const bool in = e < lim;
        v[4 * j] = in ? g.x : 0.0f; v[4 * j + 1] = in ? g.y : 0.0f;
        v[4 * j + 2] = in ? g.z : 0.0f; v[4 * j + 3] = in ? g.w : 0.0f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int e = svx::tile_index(true, false, E, lane, i);
        const float g = p[svx::clamp_group(e, lim, 1)];
        v[i] = (e < lim) ? g : 0.0f;
      }
    }
  } else {
    if (VEC && !full) {
      // as above: whole 16-byte groups, clamped, then the same transpose
      float4 g[J];
#pragma unroll
      for (int k = 0; k < J; ++k) {
        const int e = svx::tile_index(false, true, E, lane, k);
        const float4 t = ld4<NT>(p + svx::clamp_group(e, lim, 4));
        const bool in = e < lim;
        g[k] = make_float4(in ? t.x : 0.0f, in ? t.y : 0.0f, in ? t.z : 0.0f, in ? t.w : 0.0f);
      }
#pragma unroll
      for (int k = 0; k < J; ++k) {
        const int e = 256 * k + 4 * lane;
        *reinterpret_cast<float4 *>(lds + (e / E) * STR + (e % E)) = g[k];
      }
    } else if (full && VEC) {
      float4 g[J];
#pragma unroll
      for (int k = 0; k < J; ++k) g[k] = ld4<NT>(p + svx::tile_index(false, true, E, lane, k));
#pragma unroll
      for (int k = 0; k < J; ++k) {
        const int e = 256 * k + 4 * lane;
        *reinterpret_cast<float4 *>(lds + (e / E) * STR + (e % E)) = g[k];
      }
    } else {
      float g[E];
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const int e = svx::tile_index(false, false, E, lane, k);
        if (full) {
          g[k] = ld1<NT>(p + e);
        } else {
          const float t = p[svx::clamp_group(e, lim, 1)];
          g[k] = (e < lim) ? t : 0.0f;
        }
      }
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const int e = 64 * k + lane;
        lds[(e / E) * STR + (e % E)] = g[k];
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float4 t = *reinterpret_cast<const float4 *>(lds + lane * STR + 4 * j);
      v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
    }
    wave_lds_sync();
  }
}

// ---------------------------------------------------------------- streamed chunks

// A chunk is the 64*E consecutive values one wave reduces in one step.  Its
// load is split in two so that the next chunk's loads can be in flight while
// the current one is reduced:
//   issue()   starts the loads into `raw` (no wait),
//   finish()  turns `raw` into lane-contiguous values v[i] = chunk[lane*E+i]
//             (through this wave's LDS region when LOADP == 0).
// Raw layouts: LOADP 0 and VEC: raw[4k+t] = chunk[256k + 4*lane + t];
//              LOADP 0, !VEC:   raw[k]    = chunk[64k + lane];
//              LOADP 1:         raw[i]    = chunk[lane*E + i].
// Values at or beyond `len` are 0; a chunk entirely beyond the data issues no
// load; a ragged one loads at addresses clamped to [0, len).
template <int E, bool VEC, int LOADP, bool NT>
struct Chunk {
  static_assert(E >= 4 && (E & (E - 1)) == 0, "E must be a power of two >= 4");
  static constexpr int J = E / 4;
  static constexpr int STR = E + 4;
  static constexpr int SIZE = 64 * E;

  __device__ static __forceinline__ int raw_index(int i, int lane) {
    if constexpr (LOADP == 1) return svx::tile_index(true, false, E, lane, i);
    else if constexpr (VEC) return svx::tile_index(false, true, E, lane, i / 4) + (i % 4);
    else return svx::tile_index(false, false, E, lane, i);
  }

  // Loads of a chunk that lies wholly inside the data: no branch.
  __device__ static __forceinline__ void issue_full(const float *__restrict__ p, int lane, float (&raw)[E]) {
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < J; ++k) {
        const int e = svx::tile_index(LOADP == 1, true, E, lane, k);
        const float4 g = ld4<NT>(p + e);
        raw[4 * k] = g.x; raw[4 * k + 1] = g.y; raw[4 * k + 2] = g.z; raw[4 * k + 3] = g.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) raw[i] = ld1<NT>(p + raw_index(i, lane));
    }
  }

  __device__ static __forceinline__ void issue(const float *__restrict__ p, int64_t len, int lane, float (&raw)[E]) {
    const int lim = svx::tile_lim(len, SIZE);
    if (lim == SIZE) {
      if constexpr (VEC) {
#pragma unroll
        for (int k = 0; k < J; ++k) {
          const int e = svx::tile_index(LOADP == 1, true, E, lane, k);
          const float4 g = ld4<NT>(p + e);
          raw[4 * k] = g.x; raw[4 * k + 1] = g.y; raw[4 * k + 2] = g.z; raw[4 * k + 3] = g.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) raw[i] = ld1<NT>(p + raw_index(i, lane));
      }
    } else if (lim == 0) {
#pragma unroll
      for (int i = 0; i < E; ++i) raw[i] = 0.0f;
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int e = raw_index(i, lane);
        const float t = p[svx::clamp_group(e, lim, 1)];
        raw[i] = (e < lim) ? t : 0.0f;
      }
    }
  }

  __device__ static __forceinline__ void finish(const float (&raw)[E], float *__restrict__ lds, int lane,
                                                float (&v)[E]) {
    if constexpr (LOADP == 1) {
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = raw[i];
    } else {
      if constexpr (VEC) {
#pragma unroll
        for (int k = 0; k < J; ++k) {
          const int e = 256 * k + 4 * lane;
          *reinterpret_cast<float4 *>(lds + (e / E) * STR + (e % E)) =
              make_float4(raw[4 * k], raw[4 * k + 1], raw[4 * k + 2], raw[4 * k + 3]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int e = 64 * i + lane;
          lds[(e / E) * STR + (e % E)] = raw[i];
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const float4 t = *reinterpret_cast<const float4 *>(lds + lane * STR + 4 * j);
        v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
      }
      wave_lds_sync();
    }
  }
};

}  // namespace sv
