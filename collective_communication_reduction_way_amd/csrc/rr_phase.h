// rr_phase.h -- the phased streaming fold: argument block, barrier constants
// and per-mode launchers (internal to librr.so).  The schedule and the
// barrier are described in rr_phase_impl.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "rr_kernels.h"

namespace rr {

constexpr int kSyncSlots = 64;                     // barrier counter sets per device
constexpr int kSyncSubs = 8;                       // arrival counters per set
constexpr int kSyncCounters = kSyncSubs + 1;       // arrival counters, then the top counter
constexpr int kSyncStride = 16;                    // 64-bit words: one 128-byte line per counter
constexpr int kLaunchShift = 24;                   // counter = (launch tag << 24) + count
constexpr uint64_t kMaxBarrierTiles = 1ull << 23;  // a counter's arrivals (2 per round) stay below 2^24
// Launch tag of a launch captured into a graph: a graph replays its kernel
// arguments unchanged, so such a launch always carries this tag (eager
// launches use 2, 3, ...), and a reset of the slot's counters is captured
// just before it.
constexpr unsigned long long kCapturedTag = 1ull << kLaunchShift;

// Per-segment tiling is computed on the host, so that the kernel makes no
// 64-bit comparisons of uniform values: with ROCm 7.2's compiler, a 64-bit
// "x < c ? x : c" that also steers a branch was seen to select on a stale SCC
// bit (the copy of the vector compare's result into SCC was dropped), which
// turned partial tiles into full ones.  Only 32-bit compares remain below.
struct PhaseArgs {
  FoldArgs f;
  uint32_t seg_tile[RR_MAX_RANKS + 1];  // first tile of each segment; seg_tile[segments] = tiles
  uint32_t seg_last[RR_MAX_RANKS];      // groups in the segment's last tile (1 .. kBlock*U)
  uint8_t head_len[RR_MAX_RANKS];       // elements before the segment's first whole group (< V)
  uint8_t tail_len[RR_MAX_RANKS];       // elements after its last whole group (< V)
  uint32_t tiles;
  // Common case (every segment has the same length and tiling): tiles per
  // segment, groups in each segment's last tile, and the segment length in
  // elements, so that a tile's place is pure arithmetic, with no argument
  // loads that depend on the tile.  uniform_tiles = 0 otherwise.
  uint32_t uniform_tiles;
  uint32_t uniform_last;
  uint64_t seg_len;
  int32_t edges;  // 1 = some segment has a head or a tail
  uint32_t rounds;
  uint32_t slot;
  uint32_t timeout_ticks;  // bounded wait per barrier, in wall-clock ticks
  unsigned long long tag;  // launch tag << kLaunchShift
  int32_t segments;
  int32_t captured;  // 1: launched under graph capture (tag = kCapturedTag; reset first)
  // Interleaved tiles (uniform tilings only): the first strip_tiles tiles of
  // every segment form runs of `strips` tiles whose strips (kBlock groups
  // each) interleave: tile j of a run takes strips j, j + strips, ...  The
  // other tiles, and every tile when strips <= 1, are contiguous.
  uint32_t strips;
  uint32_t strip_tiles;
};

// Fill `y` for a launch with a barrier on stream s (any translation unit:
// each keeps its own counters, the slots are per stream).
hipError_t phase_sync_args(hipStream_t s, int timeout_us, SyncArgs* y);

// Groups per lane per tile of the phased fold: 8 (32 KiB per rank and tile
// for 4-byte types); 4 for the bfloat16 hierarchy, whose second set of
// partials (the running total over groups) would otherwise cost too many
// registers.  Sums can also run with U = 4 (tuning).
int phase_default_unroll(Kind k, FoldMode m);

// Launch the phased fold of one mode (rr_phase_ring.hip, rr_phase_hier.hip):
// `sync` selects the kernel with the soft barrier between the read and the
// write phase of each round, `static_p` the kernel compiled for p = 8 when p
// is 8; the heads and tails of the segments, if any,
// follow in a second, small launch on the same stream.
// With occ != NULL nothing is launched: *occ receives how many workgroups of
// the selected kernel fit on one compute unit.
hipError_t phase_launch_ring(const PhaseArgs& a, Kind k, rr_op_t op, unsigned grid, int unroll, bool sync,
                             bool static_p, int* occ, hipStream_t s);
// The ring all-reduce in batched rounds (k_phase_batch): `batch` (2 or 4)
// tiles of 4 groups per lane per workgroup and round, interleaved in runs of
// PhaseArgs::strips tiles, the soft barrier between the phases; the grid must
// be resident.
hipError_t phase_launch_ring_batch(const PhaseArgs& a, Kind k, rr_op_t op, unsigned grid, int batch, bool static_p,
                                   int* occ, hipStream_t s);
hipError_t phase_launch_hier(const PhaseArgs& a, Kind k, rr_op_t op, unsigned grid, int unroll, bool sync,
                             bool static_p, int* occ, hipStream_t s);
// The hierarchical all-reduce (kHierAll) in batched rounds, as
// phase_launch_ring_batch, with the run-time rank loop.
hipError_t phase_launch_hier_batch(const PhaseArgs& a, Kind k, rr_op_t op, unsigned grid, int batch, int* occ,
                                   hipStream_t s);
// The hierarchical variants (kHierRing, kHierAllWire, kHierRingWire), run-time
// rank loop only (rr_phase_hier_var.hip).
hipError_t phase_launch_hier_var(const PhaseArgs& a, FoldMode m, Kind k, rr_op_t op, unsigned grid, int unroll,
                                 bool sync, int* occ, hipStream_t s);
// The same in batched rounds (as phase_launch_hier_batch).
hipError_t phase_launch_hier_var_batch(const PhaseArgs& a, FoldMode m, Kind k, rr_op_t op, unsigned grid, int batch,
                                       int* occ, hipStream_t s);
// Barrier timeouts counted by each translation unit's kernels on the
// current device.
hipError_t phase_timeouts_ring(unsigned long long* count);
hipError_t phase_timeouts_hier(unsigned long long* count);
hipError_t phase_timeouts_hier_var(unsigned long long* count);
// Reduce-scatter (kRingShard) and reduce (kAscOne): one output per input
// set (rr_phase_one.hip).
hipError_t phase_launch_one(const PhaseArgs& a, FoldMode m, Kind k, rr_op_t op, unsigned grid, int unroll, bool sync,
                            bool static_p, int* occ, hipStream_t s);
// The same folds in batched rounds (k_phase_batch): `batch` (2 or 4) tiles of
// 4 groups per lane per workgroup and round, the soft barrier between the
// read and the write phase; the grid must be resident.
hipError_t phase_launch_one_batch(const PhaseArgs& a, FoldMode m, Kind k, rr_op_t op, unsigned grid, int batch,
                                  bool static_p, int* occ, hipStream_t s);
hipError_t phase_timeouts_one(unsigned long long* count);

}  // namespace rr
