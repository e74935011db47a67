// ADN binned reproducible float32 sum on gfx950.
//
// Method: the Ahrens-Demmel-Nguyen binned format as the "SyclReproSum"
// README describes it ("How It Works", "Accumulator capacity", "Template
// Parameters"): K folds of 13-bit bins on a fixed global grid, a deposit of
// each value into the folds with a few float additions and a sticky bit,
// renormalisation of each primary into its carry count every 512 deposits,
// exact bin-by-bin merges, and a conversion through a running double value.
// The readings taken where the page is silent (anchoring of the grid, the
// index rule, storage of the two coarsest bins, the conversion order) are
// stated with sv_adn_sum_f32 in include/stable_variance.h.
//
// Because every deposit rounds on the same absolute grid, the result does
// not depend on which lane deposits which value or on the merge order; the
// kernel therefore reads the input with plain coalesced loads, lets each
// lane keep its own accumulator and merges lanes, waves and workgroups in
// whatever order is cheapest.
//
// Kernel k_adn_sum: each wave streams a run of chunks of 64*E values.  Per
// chunk the wave takes the largest magnitude (a wave-wide max), raises its
// accumulators' index if needed (uniform across the wave), and deposits.
// Chunks with Inf/NaN, or an index in the two coarsest bins, take a slower
// general path.  Lane accumulators merge across the wave with DPP and
// permlane swaps, waves through LDS, workgroups through the workspace and
// a two-level ticket (as the tree sum): the last workgroup converts.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/stable_variance.h"
#include "sv_adn_kernel.hpp"
#include "sv_host.hpp"

using svh::check_device;
using svh::check_launch;
using svh::fail;
using svh::ok;

namespace {

__global__ void k_adn_zero(float *out) { out[0] = 0.0f; }

struct AdnTuning {
  int e = 16;                  // values per lane in a chunk: 16 or 32
  int64_t blocks = 512;        // target number of workgroups (few: each merge is costly)
};
thread_local AdnTuning g_adn;  // per host thread, like the other launch knobs

}  // namespace

namespace sva {

bool launch_folds_2_8(int fold, bool vec, dim3 grid, const float *x, int64_t n, int64_t chunks, int64_t g,
                      unsigned *recs, unsigned *counter, float *out, hipStream_t st) {
  switch (fold) {
    SV_ADN_FOLD(2) SV_ADN_FOLD(3) SV_ADN_FOLD(4) SV_ADN_FOLD(5) SV_ADN_FOLD(6) SV_ADN_FOLD(7) SV_ADN_FOLD(8)
    default: return false;
  }
}

}  // namespace sva

namespace svh {

// Tuning keys of the ADN sum, reached through sv_set_tuning.
sv_status adn_set_tuning(const char *key, int64_t value, bool *handled) {
  *handled = true;
  if (strcmp(key, "reset") == 0) {
    g_adn = AdnTuning{};
    return ok();
  }
  if (strcmp(key, "adn_e") == 0) {
    if (value != 16 && value != 32) return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: adn_e must be 16 or 32");
    g_adn.e = (int)value;
    return ok();
  }
  if (strcmp(key, "adn_blocks") == 0) {
    if (value < 1 || value > ADN_MAX_BLOCKS)
      return fail(SV_ERR_INVALID_ARGUMENT, "sv_set_tuning: adn_blocks must be in [1, %d]", ADN_MAX_BLOCKS);
    g_adn.blocks = value;
    return ok();
  }
  *handled = false;
  return SV_OK;
}

}  // namespace svh

extern "C" {

size_t sv_adn_sum_f32_workspace_size(int64_t n) {
  if (n < 0 || n > SV_ADN_MAX_COUNT) return (size_t)-1;
  if (n == 0) return 0;
  return ADN_WS_HEADER + (size_t)(ADN_MAX_BLOCKS + ADN_MAX_BLOCKS / ADN_GROUP) * ADN_REC * sizeof(unsigned);
}

sv_status sv_adn_sum_f32(const float *x, int64_t n, int fold, float *out, void *workspace, size_t workspace_bytes,
                         void *stream) {
  if (n < 0) return fail(SV_ERR_INVALID_ARGUMENT, "sv_adn_sum_f32: n = %lld < 0", (long long)n);
  if (fold < 2 || fold > 21) return fail(SV_ERR_INVALID_ARGUMENT, "sv_adn_sum_f32: fold %d outside 2..21", fold);
  if (fold > SV_ADN_MAX_FOLD)
    return fail(SV_ERR_UNSUPPORTED, "sv_adn_sum_f32: fold %d above the %d this library builds", fold,
                SV_ADN_MAX_FOLD);
  if (n > SV_ADN_MAX_COUNT)
    return fail(SV_ERR_UNSUPPORTED, "sv_adn_sum_f32: %lld values exceed the accumulator capacity %lld",
                (long long)n, (long long)SV_ADN_MAX_COUNT);
  if (!out) return fail(SV_ERR_INVALID_ARGUMENT, "sv_adn_sum_f32: out is NULL");
  if (n > 0 && !x) return fail(SV_ERR_INVALID_ARGUMENT, "sv_adn_sum_f32: x is NULL");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (n == 0) {
    const sv_status dev = check_device();
    if (dev != SV_OK) return dev;
    (void)hipGetLastError();
    k_adn_zero<<<1, 1, 0, st>>>(out);
    return check_launch("sv_adn_sum_f32");
  }
  const size_t need = sv_adn_sum_f32_workspace_size(n);
  if (!workspace) return fail(SV_ERR_WORKSPACE, "sv_adn_sum_f32: workspace is NULL (%zu bytes needed)", need);
  if (workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE, "sv_adn_sum_f32: workspace has %zu bytes, %zu needed", workspace_bytes, need);
  if (!svh::aligned256(workspace)) return fail(SV_ERR_WORKSPACE, "sv_adn_sum_f32: workspace is not 256-byte aligned");
  const sv_status dev = check_device();
  if (dev != SV_OK) return dev;
  (void)hipGetLastError();

  const int e = (g_adn.e == 32 && fold == 3) ? 32 : 16;
  const svx::AdnPlan plan = svx::adn_plan(n, e, g_adn.blocks);  // blocks <= g_adn.blocks
  const int64_t chunks = plan.chunks, g = plan.g, blocks = plan.blocks;
  unsigned *counter = reinterpret_cast<unsigned *>(workspace);
  unsigned *recs = reinterpret_cast<unsigned *>(reinterpret_cast<char *>(workspace) + ADN_WS_HEADER);
  const bool vec = svh::aligned16(x);
  const dim3 grid((unsigned)blocks);
  // 32 values per lane is built for three folds only (a geometry knob: the
  // result bits do not depend on it); other fold counts use 16.
  if (e == 32 && fold == 3) launch_k<3, 32>(vec, grid, x, n, chunks, g, recs, counter, out, st);
  else if (!sva::launch_folds_2_8(fold, vec, grid, x, n, chunks, g, recs, counter, out, st) &&
           !sva::launch_folds_9_14(fold, vec, grid, x, n, chunks, g, recs, counter, out, st))
    sva::launch_folds_15_21(fold, vec, grid, x, n, chunks, g, recs, counter, out, st);
  return check_launch("sv_adn_sum_f32");
}

}  // extern "C"
