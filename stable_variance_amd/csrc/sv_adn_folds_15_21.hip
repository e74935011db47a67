// The ADN binned sum's kernels for 15 to 21 folds (see sv_adn.hip).
#include "sv_adn_kernel.hpp"

namespace sva {

bool launch_folds_15_21(int fold, bool vec, dim3 grid, const float *x, int64_t n, int64_t chunks, int64_t g,
                        unsigned *recs, unsigned *counter, float *out, hipStream_t st) {
  switch (fold) {
    SV_ADN_FOLD(15) SV_ADN_FOLD(16) SV_ADN_FOLD(17) SV_ADN_FOLD(18) SV_ADN_FOLD(19) SV_ADN_FOLD(20) SV_ADN_FOLD(21)
    default: return false;
  }
}

}  // namespace sva
