// Kernels of the ADN binned reproducible float32 sum (included by the
// translation units that instantiate them: the fold counts are spread over
// several units so that they compile in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/stable_variance.h"
#include "sv_device.hpp"
#include "sv_index.hpp"

namespace {

constexpr int ADN_W = 13;                   // bin width ("Template Parameters", float)
constexpr int ADN_GRID0 = -146;             // log2 of bin 0's unit
constexpr int ADN_SCALE_FROM = 20;          // bins whose primary 1.5*2^q overflows a float ...
constexpr int ADN_SCALE_SHIFT = 40;         // ... are stored scaled by 2^-40
constexpr int ADN_RENORM = 512;             // 2^(24 - 13 - 2) deposits between renormalisations
using svx::ADN_REC;             // 32-bit words per accumulator record
using svx::ADN_WAVES;           // waves per workgroup
using svx::ADN_MAX_BLOCKS;
using svx::ADN_GROUP;           // workgroups per first-level ticket
using svx::ADN_COUNTER_STRIDE;  // counters 256 bytes apart
constexpr size_t ADN_WS_HEADER = (size_t)svx::ADN_WS_HEADER;
static_assert(ADN_WS_HEADER == SV_ADN_SUM_COUNTER_BYTES, "header constant");
static_assert(2 * SV_ADN_MAX_FOLD + 2 <= ADN_REC, "record size");
static_assert(ADN_MAX_BLOCKS / ADN_GROUP == 128, "two group records per lane");

constexpr uint32_t FLAG_NAN = 1u, FLAG_PINF = 2u, FLAG_NINF = 4u;

// ------------------------------------------------------------------ bins

__device__ __forceinline__ int scale_exp(int b) { return b >= ADN_SCALE_FROM ? -ADN_SCALE_SHIFT : 0; }

// Binade q of bin b's primary (ulp(1.5 * 2^q) = the bin's unit), scaled.
__device__ __forceinline__ int primary_exp(int b) { return ADN_GRID0 + ADN_W * b + 23 + scale_exp(b); }

__device__ __forceinline__ float base_of(int b) {  // 1.5 * 2^q: the empty primary
  return __builtin_bit_cast(float, ((unsigned)(primary_exp(b) + 127) << 23) | 0x400000u);
}

__device__ __forceinline__ float quarter_of(int b) {  // 2^(q-2): one carry
  return __builtin_bit_cast(float, (unsigned)(primary_exp(b) - 2 + 127) << 23);
}

// The value with its lowest significand bit set: added to a primary, it
// rounds to the bin's unit to nearest with ties away from zero, whatever the
// primary's current value.
__device__ __forceinline__ float sticky(float v) {
  return __builtin_bit_cast(float, __builtin_bit_cast(unsigned, v) | 1u);
}

// Smallest bin b with a < 2^(13b - 134), for finite a > 0.
__device__ __forceinline__ int bin_of(float a) {
  const int e = __builtin_amdgcn_frexp_expf(a);  // a = f * 2^e, f in [0.5, 1)
  const int t = (e - 1) + 135;
  return t <= 0 ? 0 : (t + 12) / 13;
}

__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

template <int CTRL>
__device__ __forceinline__ unsigned dpp_u(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Wave-wide maximum (every lane returns it).
__device__ __forceinline__ float wave_max(float m) {
  m = fmaxf(m, sv::dpp<sv::DPP_QUAD_XOR1>(m));
  m = fmaxf(m, sv::dpp<sv::DPP_QUAD_XOR2>(m));
  m = fmaxf(m, sv::dpp<sv::DPP_ROW_HALF_MIRROR>(m));
  m = fmaxf(m, sv::dpp<sv::DPP_ROW_MIRROR>(m));
  float a, b;
  sv::swap_halves<16>(m, a, b);
  m = fmaxf(a, b);
  sv::swap_halves<32>(m, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ int wave_max_i(int m) {
  m = max(m, (int)dpp_u<sv::DPP_QUAD_XOR1>((unsigned)m));
  m = max(m, (int)dpp_u<sv::DPP_QUAD_XOR2>((unsigned)m));
  m = max(m, (int)dpp_u<sv::DPP_ROW_HALF_MIRROR>((unsigned)m));
  m = max(m, (int)dpp_u<sv::DPP_ROW_MIRROR>((unsigned)m));
  float a, b;
  sv::swap_halves<16>(__builtin_bit_cast(float, m), a, b);
  m = max(__builtin_bit_cast(int, a), __builtin_bit_cast(int, b));
  sv::swap_halves<32>(__builtin_bit_cast(float, m), a, b);
  return max(__builtin_bit_cast(int, a), __builtin_bit_cast(int, b));
}

// ------------------------------------------------------------------ accumulator

// K primaries (fold k holds bin top - k), K carry counts (float integers),
// the index and the Inf/NaN flags.
template <int K>
struct Acc {
  float p[K];
  float c[K];
  int top;
  unsigned flags;
};

template <int K>
__device__ __forceinline__ void acc_init(Acc<K> &a) {
  a.top = K - 1;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    a.p[k] = base_of(K - 1 - k);
    a.c[k] = 0.0f;
  }
  a.flags = 0;
}

// Raise the index to t >= top: folds move to finer positions, the finest
// ones drop out (their bins lie below the K kept under the new top), new
// coarse folds start empty.
template <int K>
__device__ __forceinline__ void acc_raise(Acc<K> &a, int t) {
  if (t - a.top >= K) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      a.p[k] = base_of(t - k);
      a.c[k] = 0.0f;
    }
    a.top = t;
    return;
  }
  while (a.top < t) {
#pragma unroll
    for (int k = K - 1; k > 0; --k) {
      a.p[k] = a.p[k - 1];
      a.c[k] = a.c[k - 1];
    }
    a.top += 1;
    a.p[0] = base_of(a.top);
    a.c[0] = 0.0f;
  }
}

// Keep every primary in [1.25, 1.75) * 2^q by moving one quarter into the
// carry count (the drift since the last call is below a quarter).
template <int K>
__device__ __forceinline__ void acc_renorm(Acc<K> &a) {
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int b = a.top - k;
    const float B = base_of(b), u = quarter_of(b);
    // step = -1, 0 or +1 quarters (exact float arithmetic on small integers)
    const float step = (a.p[k] >= B + u ? 1.0f : 0.0f) - (a.p[k] < B - u ? 1.0f : 0.0f);
    a.p[k] = a.p[k] - step * u;
    a.c[k] = a.c[k] + step;
  }
}

// Deposit when no fold is a scaled bin (index below 20): per fold, round the
// remainder into the primary, take back the exact rest.
template <int K>
__device__ __forceinline__ void deposit_fast(Acc<K> &a, float r) {
#pragma unroll
  for (int k = 0; k < K - 1; ++k) {
    const float s = a.p[k] + sticky(r);
    const float d = a.p[k] - s;  // minus the part this fold took (exact)
    a.p[k] = s;
    r = r + d;                   // exact remainder
  }
  a.p[K - 1] = a.p[K - 1] + sticky(r);
}

// Any index: a fold of bin 20 or 21 works on the remainder scaled by 2^-40.
// If it takes nothing, the remainder passes on unchanged (the scaled copy
// may have lost bits); if it takes a part, the remainder was large and both
// the scaling and the subtraction are exact.
template <int K>
__device__ __forceinline__ void deposit_general(Acc<K> &a, float r) {
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const bool sc = (a.top - k) >= ADN_SCALE_FROM;
    const float rs = sc ? r * 0x1p-40f : r;
    if (k < K - 1) {
      const float s = a.p[k] + sticky(rs);
      const float d = a.p[k] - s;
      a.p[k] = s;
      if (!sc) r = r + d;
      else if (d != 0.0f) r = (rs + d) * 0x1p40f;
    } else {
      a.p[k] = a.p[k] + sticky(rs);
    }
  }
}

// a += other, both renormalised and with the same index: primaries add
// their offsets from the base exactly (the sum stays in [1, 2) * 2^q).
template <int K>
__device__ __forceinline__ void acc_add_same(Acc<K> &a, const float (&op)[K], const float (&oc)[K], unsigned of) {
#pragma unroll
  for (int k = 0; k < K; ++k) {
    a.p[k] = a.p[k] + (op[k] - base_of(a.top - k));
    a.c[k] = a.c[k] + oc[k];
  }
  a.flags |= of;
  acc_renorm(a);
}

// a += b for any two accumulators (one lane).
template <int K>
__device__ __forceinline__ void acc_merge(Acc<K> &a, Acc<K> b) {
  const int t = max(a.top, b.top);
  acc_raise(a, t);
  acc_raise(b, t);
  acc_renorm(a);
  acc_renorm(b);
  acc_add_same(a, b.p, b.c, b.flags);
}

template <int K, int CTRL>
__device__ __forceinline__ void merge_level_dpp(Acc<K> &a) {
  float op[K], oc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    op[k] = sv::dpp<CTRL>(a.p[k]);
    oc[k] = sv::dpp<CTRL>(a.c[k]);
  }
  acc_add_same(a, op, oc, dpp_u<CTRL>(a.flags));
}

template <int K, int XOR>
__device__ __forceinline__ void merge_level_swap(Acc<K> &a) {
  float pa[K], pb[K], ca[K], cb[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    sv::swap_halves<XOR>(a.p[k], pa[k], pb[k]);
    sv::swap_halves<XOR>(a.c[k], ca[k], cb[k]);
  }
  float fa, fb;
  sv::swap_halves<XOR>(__builtin_bit_cast(float, a.flags), fa, fb);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    a.p[k] = pa[k];
    a.c[k] = ca[k];
  }
  a.flags = __builtin_bit_cast(unsigned, fa);
  acc_add_same(a, pb, cb, __builtin_bit_cast(unsigned, fb));
}

// Merge the 64 lane accumulators (same index, renormalised); every lane
// returns the wave's accumulator.  The merge is exact and symmetric, so the
// mirror permutations reach an equal partner once the lower lanes agree.
template <int K>
__device__ __forceinline__ void wave_merge(Acc<K> &a) {
  merge_level_dpp<K, sv::DPP_QUAD_XOR1>(a);
  merge_level_dpp<K, sv::DPP_QUAD_XOR2>(a);
  merge_level_dpp<K, sv::DPP_ROW_HALF_MIRROR>(a);
  merge_level_dpp<K, sv::DPP_ROW_MIRROR>(a);
  merge_level_swap<K, 16>(a);
  merge_level_swap<K, 32>(a);
}

// Lanes with different indices: raise all to the wave's largest first.
template <int K>
__device__ __forceinline__ void wave_merge_any(Acc<K> &a) {
  acc_raise(a, wave_max_i(a.top));
  acc_renorm(a);
  wave_merge(a);
}

// Result ("How It Works"): NaN, or +Inf with -Inf, gives 0x7fc00000; a
// single-signed Inf stays; otherwise each fold's exact value (offset of the
// primary plus carries times the quarter, exact in double) goes into a
// running double sum from the coarsest fold, rounded once to float.
template <int K>
__device__ __forceinline__ float acc_convert(const Acc<K> &a) {
  if ((a.flags & FLAG_NAN) || (a.flags & (FLAG_PINF | FLAG_NINF)) == (FLAG_PINF | FLAG_NINF))
    return __builtin_bit_cast(float, 0x7FC00000u);
  if (a.flags & FLAG_PINF) return __builtin_bit_cast(float, 0x7F800000u);
  if (a.flags & FLAG_NINF) return __builtin_bit_cast(float, 0xFF800000u);
  double y = 0.0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int b = a.top - k;
    const double v = (double)(a.p[k] - base_of(b)) + (double)a.c[k] * (double)quarter_of(b);
    y = y + ldexp(v, -scale_exp(b));
  }
  return (float)y;
}

template <int K>
__device__ __forceinline__ void rec_store_agent(unsigned *dst, const Acc<K> &a) {
#pragma unroll
  for (int k = 0; k < K; ++k) {
    sv::store_u32_agent(dst + k, __builtin_bit_cast(unsigned, a.p[k]));
    sv::store_u32_agent(dst + K + k, __builtin_bit_cast(unsigned, a.c[k]));
  }
  sv::store_u32_agent(dst + 2 * K, (unsigned)a.top);
  sv::store_u32_agent(dst + 2 * K + 1, a.flags);
}

template <int K>
__device__ __forceinline__ Acc<K> rec_load_agent(const unsigned *src) {
  Acc<K> a;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    a.p[k] = __builtin_bit_cast(float, sv::load_u32_agent(src + k));
    a.c[k] = __builtin_bit_cast(float, sv::load_u32_agent(src + K + k));
  }
  a.top = (int)sv::load_u32_agent(src + 2 * K);
  a.flags = sv::load_u32_agent(src + 2 * K + 1);
  return a;
}

// ------------------------------------------------------------------ kernel

// Values [base, base + 64E) of x (zeros past n): lane l holds, for j < E/4,
// the 16 bytes at base + 4*(l + 64 j) (VEC) or the floats base + l + 64 i.
template <int E, bool VEC>
__device__ __forceinline__ void adn_load(const float *__restrict__ x, int64_t n, int64_t base, int lane,
                                         float (&v)[E]) {
  if (base + 64 * E <= n) {  // wave-uniform: the whole chunk is inside, no per-lane checks
#pragma unroll
    for (int j = 0; j < (VEC ? E / 4 : 0); ++j) {
      const float4 g = sv::ld4<true>(x + svx::adn_index(base, lane, j, 0, true));
      v[4 * j] = g.x;
      v[4 * j + 1] = g.y;
      v[4 * j + 2] = g.z;
      v[4 * j + 3] = g.w;
    }
#pragma unroll
    for (int i = 0; i < (VEC ? 0 : E); ++i) v[i] = sv::ld1<true>(x + svx::adn_index(base, lane, i / 4, i % 4, false));
    return;
  }
  // the last, ragged chunk: element by element, zeros past n
#pragma unroll
  for (int j = 0; j < E / 4; ++j) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t i = svx::adn_index(base, lane, j, t, VEC);
      v[4 * j + t] = i < n ? x[i] : 0.0f;
    }
  }
}

// One chunk into the lane's accumulator; the index stays uniform across the
// wave.  `since` counts deposits since the last renormalisation.
template <int K, int E>
__device__ __forceinline__ void adn_chunk(Acc<K> &a, float (&v)[E], int &since) {
  if (since + E > ADN_RENORM) {
    acc_renorm(a);
    since = 0;
  }
  since += E;
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) m = fmaxf(m, fabsf(v[i]));
  m = uniform_f(wave_max(m));
  const bool finite = m < __builtin_inff();  // false for Inf and for a NaN the max kept
  if (finite && m > 0.0f) {
    const int nb = uniform_i(bin_of(m));
    if (nb > a.top) acc_raise(a, nb);
  }
  if (finite && a.top < ADN_SCALE_FROM) {
    float keep[K];
#pragma unroll
    for (int k = 0; k < K; ++k) keep[k] = a.p[k];
#pragma unroll
    for (int i = 0; i < E; ++i) deposit_fast(a, v[i]);
    // a NaN the max ignored turns the first primary into NaN: redo the chunk
    if (__builtin_amdgcn_ballot_w64(a.p[0] != a.p[0]) == 0) return;
#pragma unroll
    for (int k = 0; k < K; ++k) a.p[k] = keep[k];
  }
  // general path: flag and zero Inf/NaN, index from the finite values
  float mf = 0.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const float t = v[i];
    if (!(fabsf(t) < __builtin_inff())) {
      a.flags |= (t != t) ? FLAG_NAN : (t > 0.0f ? FLAG_PINF : FLAG_NINF);
      v[i] = 0.0f;
    } else {
      mf = fmaxf(mf, fabsf(t));
    }
  }
  mf = uniform_f(wave_max(mf));
  if (mf > 0.0f) {
    const int nb = uniform_i(bin_of(mf));
    if (nb > a.top) acc_raise(a, nb);
  }
#pragma unroll
  for (int i = 0; i < E; ++i) deposit_general(a, v[i]);
}

template <int K>
__device__ __forceinline__ void lds_store(unsigned *dst, const Acc<K> &a) {
#pragma unroll
  for (int k = 0; k < K; ++k) {
    dst[k] = __builtin_bit_cast(unsigned, a.p[k]);
    dst[K + k] = __builtin_bit_cast(unsigned, a.c[k]);
  }
  dst[2 * K] = (unsigned)a.top;
  dst[2 * K + 1] = a.flags;
}

template <int K>
__device__ __forceinline__ Acc<K> lds_load(const unsigned *src) {
  Acc<K> a;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    a.p[k] = __builtin_bit_cast(float, src[k]);
    a.c[k] = __builtin_bit_cast(float, src[K + k]);
  }
  a.top = (int)src[2 * K];
  a.flags = src[2 * K + 1];
  return a;
}

template <int K, int E, bool VEC>
__global__ __launch_bounds__(64 * ADN_WAVES) void k_adn_sum(const float *__restrict__ x, int64_t n, int64_t chunks,
                                                            int64_t g, unsigned *__restrict__ recs,
                                                            unsigned *__restrict__ counter, float *__restrict__ out) {
  __shared__ unsigned srec[ADN_WAVES][ADN_REC];
  __shared__ unsigned is_last;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop control
  const int64_t c0 = ((int64_t)blockIdx.x * ADN_WAVES + w) * g;
  const int64_t c1 = min(c0 + g, chunks);

  Acc<K> a;
  acc_init(a);
  int since = 0;
  if (c0 < c1) {
    // Two register buffers: the next chunk loads while one is deposited.
    // Every block below issues its loads unconditionally, so the compiler's
    // wait counts stay exact (a conditional load would force a full wait).
    float ra[E], rb[E];
    int64_t c = c0;
    adn_load<E, VEC>(x, n, c * 64 * E, lane, ra);
    while (c + 2 < c1) {  // chunks c, c+1, c+2 exist
      adn_load<E, VEC>(x, n, (c + 1) * 64 * E, lane, rb);
      adn_chunk<K, E>(a, ra, since);
      adn_load<E, VEC>(x, n, (c + 2) * 64 * E, lane, ra);
      adn_chunk<K, E>(a, rb, since);
      c += 2;
    }
    if (c + 1 < c1) {  // two chunks left
      adn_load<E, VEC>(x, n, (c + 1) * 64 * E, lane, rb);
      adn_chunk<K, E>(a, ra, since);
      adn_chunk<K, E>(a, rb, since);
    } else {
      adn_chunk<K, E>(a, ra, since);
    }
  }
  acc_renorm(a);
  wave_merge(a);
  if (lane == 0) lds_store(srec[w], a);
  __syncthreads();

  // workgroup record, then the two-level ticket of the tree sum
  const int nb = (int)gridDim.x;
  const int grp = (int)blockIdx.x / ADN_GROUP;
  const int ngroups = (nb + ADN_GROUP - 1) / ADN_GROUP;
  const int in_group = (grp == ngroups - 1) ? nb - grp * ADN_GROUP : ADN_GROUP;
  unsigned *const top_counter = counter;
  unsigned *const grp_counter = counter + ADN_COUNTER_STRIDE * (1 + grp);
  unsigned *const grp_recs = recs + (size_t)ADN_MAX_BLOCKS * ADN_REC;
  if (threadIdx.x == 0) {
    Acc<K> t = lds_load<K>(srec[0]);
#pragma unroll
    for (int i = 1; i < ADN_WAVES; ++i) acc_merge(t, lds_load<K>(srec[i]));
    rec_store_agent(recs + (size_t)blockIdx.x * ADN_REC, t);
    sv::wait_vmem_stores();
    const unsigned ticket = __hip_atomic_fetch_add(grp_counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (ticket == (unsigned)in_group - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!is_last || w != 0) return;

  // last workgroup of its group (wave 0): one record per lane
  {
    const int idx = grp * ADN_GROUP + lane;
    Acc<K> t;
    if (idx < nb) t = rec_load_agent<K>(recs + (size_t)idx * ADN_REC);
    else acc_init(t);
    wave_merge_any(t);
    unsigned top_ticket = 0;
    if (lane == 0) {
      __hip_atomic_store(grp_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      rec_store_agent(grp_recs + (size_t)grp * ADN_REC, t);
      sv::wait_vmem_stores();
      top_ticket = __hip_atomic_fetch_add(top_counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    top_ticket = __builtin_amdgcn_readfirstlane(top_ticket);
    if (top_ticket != (unsigned)ngroups - 1) return;
  }

  // last group: up to 128 group records, two per lane
  Acc<K> t;
  acc_init(t);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = 2 * lane + k;
    if (idx < ngroups) acc_merge(t, rec_load_agent<K>(grp_recs + (size_t)idx * ADN_REC));
  }
  wave_merge_any(t);
  if (lane == 0) {
    out[0] = acc_convert(t);
    __hip_atomic_store(top_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}


// ------------------------------------------------------------------ host

template <int K, int E>
void launch_k(bool vec, dim3 grid, const float *x, int64_t n, int64_t chunks, int64_t g, unsigned *recs,
              unsigned *counter, float *out, hipStream_t st) {
  if (vec)
    k_adn_sum<K, E, true><<<grid, dim3(64 * ADN_WAVES), 0, st>>>(x, n, chunks, g, recs, counter, out);
  else
    k_adn_sum<K, E, false><<<grid, dim3(64 * ADN_WAVES), 0, st>>>(x, n, chunks, g, recs, counter, out);
}

}  // namespace

namespace sva {

// k_adn_sum<K, 16> for one range of fold counts, each range in its own
// translation unit; false for a fold count outside the range.
bool launch_folds_2_8(int fold, bool vec, dim3 grid, const float *x, int64_t n, int64_t chunks, int64_t g,
                      unsigned *recs, unsigned *counter, float *out, hipStream_t st);
bool launch_folds_9_14(int fold, bool vec, dim3 grid, const float *x, int64_t n, int64_t chunks, int64_t g,
                       unsigned *recs, unsigned *counter, float *out, hipStream_t st);
bool launch_folds_15_21(int fold, bool vec, dim3 grid, const float *x, int64_t n, int64_t chunks, int64_t g,
                        unsigned *recs, unsigned *counter, float *out, hipStream_t st);

}  // namespace sva

// One case of a fold-range launcher.
#define SV_ADN_FOLD(K)                                                                                  \
  case K: launch_k<K, 16>(vec, grid, x, n, chunks, g, recs, counter, out, st); return true;
