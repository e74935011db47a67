// Host helpers shared by the library's translation units: status reporting
// for the C ABI (one thread-local message per host thread) and argument
// checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/stable_variance.h"

namespace svh {

// Records a printf-style message for sv_last_error_message and returns st.
__attribute__((visibility("hidden"))) sv_status fail(sv_status st, const char *fmt, ...)
    __attribute__((format(printf, 2, 3)));
// Clears the message and returns SV_OK.
__attribute__((visibility("hidden"))) sv_status ok();
// SV_ERR_NO_DEVICE unless a HIP device is visible.
__attribute__((visibility("hidden"))) sv_status check_device();
// SV_ERR_HIP if the last launch on this host thread failed, else ok().
__attribute__((visibility("hidden"))) sv_status check_launch(const char *what);
__attribute__((visibility("hidden"))) const char *last_error();
// Tuning keys of the ADN sum ("reset" restores them); *handled is false for
// a key it does not know.
__attribute__((visibility("hidden"))) sv_status adn_set_tuning(const char *key, int64_t value, bool *handled);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The work-items one launch may hold: 2^32 - 1 (HIP's limit), or fewer when
// sv_set_tuning("launch_items") lowers it (at least 1024) so that tests run
// the batched launches on small inputs.  Per host thread.
__attribute__((visibility("hidden"))) int64_t launch_items();
// sv_set_tuning("var_cols_once") of this host thread: 0, 1 (default) or 2.
__attribute__((visibility("hidden"))) int cols_once();
// sv_set_tuning("var_cols_pairs") of this host thread: 0 or 1 (default).
__attribute__((visibility("hidden"))) int cols_pairs();
// sv_set_tuning("var_long_rows") of this host thread: 0 or 1 (default).
__attribute__((visibility("hidden"))) int long_rows();

// in_batches(total, per_block, threads, fn) calls fn(first, count) over
// [0, total) in runs of whole blocks (per_block items of `threads`
// work-items each), every run within launch_items(), so that a launcher can
// advance its pointers (or its first workgroup) by `first` items.
template <class Fn>
inline void in_batches(int64_t total, int64_t per_block, int64_t threads, Fn &&fn) {
  const int64_t batch = (launch_items() / threads) * per_block;
  for (int64_t s0 = 0; s0 < total; s0 += batch) fn(s0, total - s0 < batch ? total - s0 : batch);
}
inline bool aligned256(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

}  // namespace svh
