// Instantiations of the fold kernel for FoldMode::kHierAll (one translation
// unit per mode so the library builds in parallel).
#include "rr_fold_impl.h"

namespace rr {

hipError_t launch_fold_hier_all(const FoldLaunch& f, hipStream_t s) { return fold_by_kind<FoldMode::kHierAll>(f, s); }

}  // namespace rr
