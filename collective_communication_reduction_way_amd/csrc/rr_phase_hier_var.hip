// Instantiations for the hierarchical variants (FoldMode::kHierRing, the
// page-literal ring all-reduce inside each group, and the two modes that
// round every group partial to the storage type): the phased fold, its
// batched rounds and the single-pass fold for unaligned buffers, all with the
// run-time rank loop.
#include "rr_phase_impl.h"

namespace rr {

hipError_t phase_launch_hier_var(const PhaseArgs& a, FoldMode m, Kind k, rr_op_t op, unsigned grid, int unroll,
                                 bool sync, int* occ, hipStream_t s) {
  switch (m) {
    case FoldMode::kHierRing: return phase_dispatch<FoldMode::kHierRing>(a, k, op, grid, unroll, sync, false, occ, s);
    case FoldMode::kHierAllWire:
      return phase_dispatch<FoldMode::kHierAllWire>(a, k, op, grid, unroll, sync, false, occ, s);
    case FoldMode::kHierRingWire:
      return phase_dispatch<FoldMode::kHierRingWire>(a, k, op, grid, unroll, sync, false, occ, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t phase_launch_hier_var_batch(const PhaseArgs& a, FoldMode m, Kind k, rr_op_t op, unsigned grid, int batch,
                                       int* occ, hipStream_t s) {
  switch (m) {
    case FoldMode::kHierRing: return batch_dispatch<FoldMode::kHierRing>(a, k, op, grid, batch, false, occ, s);
    case FoldMode::kHierAllWire: return batch_dispatch<FoldMode::kHierAllWire>(a, k, op, grid, batch, false, occ, s);
    case FoldMode::kHierRingWire:
      return batch_dispatch<FoldMode::kHierRingWire>(a, k, op, grid, batch, false, occ, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t phase_timeouts_hier_var(unsigned long long* count) { return sync_timeouts_here(count); }

hipError_t launch_fold_hier_var(const FoldLaunch& f, hipStream_t s) {
  switch (f.mode) {
    case FoldMode::kHierRing: return fold_var_dispatch<FoldMode::kHierRing>(f, s);
    case FoldMode::kHierAllWire: return fold_var_dispatch<FoldMode::kHierAllWire>(f, s);
    case FoldMode::kHierRingWire: return fold_var_dispatch<FoldMode::kHierRingWire>(f, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace rr
