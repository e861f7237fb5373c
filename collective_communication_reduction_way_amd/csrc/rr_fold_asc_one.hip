// Instantiations of the fold kernel for FoldMode::kAscOne (one translation
// unit per mode so the library builds in parallel).
#include "rr_fold_impl.h"

namespace rr {

hipError_t launch_fold_asc_one(const FoldLaunch& f, hipStream_t s) { return fold_by_kind<FoldMode::kAscOne>(f, s); }

}  // namespace rr
