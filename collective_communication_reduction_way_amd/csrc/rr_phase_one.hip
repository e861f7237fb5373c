// Instantiations of the phased fold for the folds with one output per set of
// p inputs: FoldMode::kRingShard (reduce-scatter, chunk c to rank c) and
// FoldMode::kAscOne (reduce to the root), without a barrier (k_phase) and in
// batched rounds with the barrier (k_phase_batch).
#include "rr_phase_impl.h"

namespace rr {

hipError_t phase_launch_one(const PhaseArgs& a, FoldMode m, Kind k, rr_op_t op, unsigned grid, int unroll, bool sync,
                            bool static_p, int* occ, hipStream_t s) {
  switch (m) {
    case FoldMode::kRingShard:
      return phase_dispatch<FoldMode::kRingShard>(a, k, op, grid, unroll, sync, static_p, occ, s);
    case FoldMode::kAscOne: return phase_dispatch<FoldMode::kAscOne>(a, k, op, grid, unroll, sync, static_p, occ, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t phase_launch_one_batch(const PhaseArgs& a, FoldMode m, Kind k, rr_op_t op, unsigned grid, int batch,
                                  bool static_p, int* occ, hipStream_t s) {
  switch (m) {
    case FoldMode::kRingShard: return batch_dispatch<FoldMode::kRingShard>(a, k, op, grid, batch, static_p, occ, s);
    case FoldMode::kAscOne: return batch_dispatch<FoldMode::kAscOne>(a, k, op, grid, batch, static_p, occ, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t phase_timeouts_one(unsigned long long* count) { return sync_timeouts_here(count); }

}  // namespace rr
