// Instantiations of the fold kernel for FoldMode::kRingShard (one translation
// unit per mode so the library builds in parallel).
#include "rr_fold_impl.h"

namespace rr {

hipError_t launch_fold_ring_shard(const FoldLaunch& f, hipStream_t s) { return fold_by_kind<FoldMode::kRingShard>(f, s); }

}  // namespace rr
