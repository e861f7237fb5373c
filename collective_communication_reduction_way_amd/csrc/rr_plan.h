// rr_plan.h -- host-side chunk scheduler and byte accounting (internal).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "rr.h"

namespace rr {

// One transfer of the ring: in `phase` 0 (reduce-scatter) the receiver
// accumulates, in phase 1 (all-gather) it overwrites.
struct Transfer {
  int phase;
  int step;
  int src;
  int dst;
  int chunk;
};

// The ring schedule for p ranks, in execution order (2(p-1) steps of p
// transfers each).
std::vector<Transfer> ring_schedule(int p);

// bounds[c] = floor(c*n/p), c = 0..p.
void chunk_bounds(int p, uint64_t n, uint64_t* bounds);

size_t elem_size(rr_dtype_t dt);

}  // namespace rr
