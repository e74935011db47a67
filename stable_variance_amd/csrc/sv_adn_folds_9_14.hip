// The ADN binned sum's kernels for 9 to 14 folds (see sv_adn.hip).
#include "sv_adn_kernel.hpp"

namespace sva {

bool launch_folds_9_14(int fold, bool vec, dim3 grid, const float *x, int64_t n, int64_t chunks, int64_t g,
                       unsigned *recs, unsigned *counter, float *out, hipStream_t st) {
  switch (fold) {
    SV_ADN_FOLD(9) SV_ADN_FOLD(10) SV_ADN_FOLD(11) SV_ADN_FOLD(12) SV_ADN_FOLD(13) SV_ADN_FOLD(14)
    default: return false;
  }
}

}  // namespace sva
