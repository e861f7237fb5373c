// Instantiations of the phased fold for FoldMode::kHierAll (one translation
// unit per mode so the library builds in parallel): k_phase and, for
// launches of several rounds, the batched k_phase_batch (run-time rank loop).
#include "rr_phase_impl.h"

namespace rr {

hipError_t phase_launch_hier(const PhaseArgs& a, Kind k, rr_op_t op, unsigned grid, int unroll, bool sync,
                             bool static_p, int* occ, hipStream_t s) {
  return phase_dispatch<FoldMode::kHierAll>(a, k, op, grid, unroll, sync, static_p, occ, s);
}

hipError_t phase_launch_hier_batch(const PhaseArgs& a, Kind k, rr_op_t op, unsigned grid, int batch, int* occ,
                                   hipStream_t s) {
  return batch_dispatch<FoldMode::kHierAll>(a, k, op, grid, batch, false, occ, s);
}

hipError_t phase_timeouts_hier(unsigned long long* count) { return sync_timeouts_here(count); }

}  // namespace rr
