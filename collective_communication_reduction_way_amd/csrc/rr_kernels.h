// rr_kernels.h -- kernel argument blocks and launchers (internal to librr.so).
//
// Every argument block is passed to its kernel by value (kernarg segment, at
// most a few KiB), so a launch needs no device-side pointer table, no copy
// and no allocation.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "rr.h"

namespace rr {

constexpr int kBlock = 256;  // threads per workgroup: 4 wavefronts of 64 lanes

// Which inputs a fold reads, in which order, and where it writes.
enum class FoldMode : int {
  // Ring all-reduce: workgroup row y = chunk c; element i of chunk c folds
  // in[(c+1)%p], in[(c+2)%p], ..., in[c]; the result goes to out[0..p-1][i].
  kRingAll = 0,
  // Ring reduce-scatter: same fold; chunk c goes to out[c][i - bound[c]].
  kRingShard = 1,
  // Ascending fold per segment: row y = segment j folds in[j*p + 0..p-1] in
  // that order into out[j][i].  (Reduce: one segment.  Staged hierarchy step
  // one: one segment per group.)
  kAscOne = 2,
  // Hierarchical: in[0..p-1] folded ascending inside groups of `group`
  // consecutive inputs, the group partials folded ascending; the result goes
  // to out[0..p-1][i].
  kHierAll = 3,
  // Hierarchical, each group's partial formed by a ring all-reduce of the
  // group: row y = group-chunk k (bounds floor(k*n/group)); inside group j
  // the fold order is members (k+1) mod G, ..., k mod G; then as kHierAll.
  kHierRing = 4,
  // kHierAll / kHierRing with every group partial rounded to the storage
  // type and widened again before the cross-group fold (the partial crosses
  // groups in the storage type).  16-bit kinds only.
  kHierAllWire = 5,
  kHierRingWire = 6,
};

constexpr bool is_hier(FoldMode m) {
  return m == FoldMode::kHierAll || m == FoldMode::kHierRing || m == FoldMode::kHierAllWire ||
         m == FoldMode::kHierRingWire;
}
constexpr bool is_hier_ring(FoldMode m) { return m == FoldMode::kHierRing || m == FoldMode::kHierRingWire; }
constexpr bool is_wire(FoldMode m) { return m == FoldMode::kHierAllWire || m == FoldMode::kHierRingWire; }
// Modes whose rows are bounded by bound[]: the ring's chunks, the group-chunks.
constexpr bool uses_bounds(FoldMode m) {
  return m == FoldMode::kRingAll || m == FoldMode::kRingShard || is_hier_ring(m);
}

enum class Kind : int { kI32 = 0, kF32 = 1, kBF16 = 2, kF16 = 3 };

constexpr bool is_half(Kind k) { return k == Kind::kBF16 || k == Kind::kF16; }

struct FoldArgs {
  const void* in[RR_MAX_RANKS];
  void* out[RR_MAX_RANKS];
  uint64_t bound[RR_MAX_RANKS + 1];  // ring modes: chunk bounds floor(c*n/p)
  uint64_t n;                         // elements per input buffer
  int32_t p;                          // inputs folded per output element
  int32_t group;                      // kHierAll: group size (divides p)
  int32_t vec;                        // 1: every buffer is 16-byte aligned
  int32_t div;                        // AVG: the divisor (the number of ranks); unused otherwise
};

struct FoldLaunch {
  FoldArgs args;
  FoldMode mode;
  Kind in_kind;
  Kind out_kind;
  rr_op_t op;
  int segments;    // grid rows: chunks (ring modes), segments (kAscOne) or 1
  int unroll;      // groups per lane per tile (1, 2 or 4); 0 = default
  int nontemporal; // 1 = nontemporal loads/stores
  int grid_cap;    // max workgroups in total (0 = one tile per workgroup)
};

// One source to many destinations: row y copies seg_bytes from src[y] to
// dst[r] + y*dst_seg_stride for every r < ndst, except r == y when bit y of
// skip_diag is set (an in-place shard that already sits in its slot).
struct FanoutArgs {
  const void* src[RR_MAX_RANKS];
  void* dst[RR_MAX_RANKS];
  uint64_t seg_bytes;
  uint64_t dst_seg_stride;
  uint64_t skip_diag;
  int32_t nseg;
  int32_t ndst;
};

// Independent transfers: row y moves len[y] elements from src[y] to dst[y]
// (copy, type conversion, or, for the ring step, dst = src (+) dst).
struct PairArgs {
  const void* src[RR_MAX_RANKS];
  void* dst[RR_MAX_RANKS];
  // Ring reduce-scatter step only: where the receiver's own value is read
  // (dst = src (+) aux); the other kinds of launch leave it unused.
  const void* aux[RR_MAX_RANKS];
  uint64_t len[RR_MAX_RANKS];
  int32_t npairs;
  int32_t vec;
  int32_t div;  // conversions: > 0 divides every value by div first (AVG's last step)
  int32_t pad;
};

// Schedule of the phased fold (rr_phase.cpp): per_cu workgroups per compute
// unit (0 = chosen by the schedule) or an explicit grid; unroll 0 = chosen by
// the schedule, 4 = the smaller tile (sums only); sync = 1 puts
// a soft barrier between the read and the write phase of every round;
// timeout_us bounds each barrier wait.
struct PhaseTuning {
  int sync;
  int per_cu;
  int grid;
  int unroll;
  int timeout_us;
  int static_p;  // 1 = the kernels compiled for p = 8 serve p = 8, 0 = the run-time loop, -1 = by mode
  int strips;    // tiles per run of interleaved tiles (PhaseArgs::strips); 1 = contiguous tiles, 0 = by mode
  int batch;     // reduce-scatter / reduce: tiles per workgroup and round of the batched kernel (2, 4);
                 // 1 = never batched, 0 = by the schedule
  int ar_batch;  // ring all-reduce of several rounds: the same for its batched kernel
};

// Bucketed all-reduce (rr_multi.hip): the tensors of a bucket are folded as
// if laid end to end, each element in the ring order of its chunk of the
// bucket.  One launch serves a batch of "pieces": a piece is a run of
// elements of one tensor inside one chunk, moved either as 16-byte groups
// (every pointer of the tensor 16-byte aligned and the run group-aligned) or
// element by element.  Tables are passed by value (under 4 KiB).
constexpr int kBucketPtrs = 192;   // pointer slots per launch: p inputs then p outputs per tensor
constexpr int kBucketPieces = 96;  // pieces per launch

// The barrier fields of one launch (rr_sync.h): the stream's counter slot,
// the launch tag (kCapturedTag under graph capture, then captured = 1), and
// the bound of one wait in wall-clock ticks.
struct SyncArgs {
  unsigned long long tag;
  uint32_t slot;
  uint32_t timeout_ticks;
  int32_t captured;
  int32_t pad;
};

struct BucketArgs {
  const void* ptr[kBucketPtrs];
  uint64_t start[kBucketPieces];       // first element of the piece in its tensor
  uint32_t units[kBucketPieces];       // 16-byte groups (vector pieces) or elements (scalar pieces)
  uint32_t tile0[kBucketPieces + 1];   // first tile of each piece; tile0[npieces] = tiles
  uint16_t base[kBucketPieces];        // slot of the piece's tensor's rank-0 input; outputs at base + p
  uint8_t rot[kBucketPieces];          // chunk c of the bucket: fold order c+1, ..., c (mod p)
  uint8_t vec[kBucketPieces];          // 1 = 16-byte groups
  int32_t npieces;
  int32_t p;
  int32_t div;  // AVG: p; unused otherwise
  uint32_t tiles;
  uint32_t rounds;  // tiles / grid, rounded up
  SyncArgs sync;    // the soft barrier between the read and write phases (multi-round launches)
  // Multi-round launches: runs of `strips` whole tiles of a vector piece
  // whose kBlock-unit strips interleave (tile j of a run takes strips j,
  // j + strips, ...); 0 or 1 = contiguous tiles.
  uint32_t strips;
};

// Units per lane and tile of the bucket kernel: a tile is kBlock*kBucketU
// units, 16-byte groups in vector pieces and single elements in scalar ones.
constexpr int kBucketU = 4;

// per_cu: workgroups per compute unit of the launch (the kernels stride over
// their work); 0 = the default.  sync: a launch of several rounds separates
// the read and the write phase of each round with the soft barrier
// (timeout_us bounds one wait); batch = 1 keeps one tile per workgroup and
// round, else such a launch takes the batched rounds.
hipError_t launch_bucket(const BucketArgs& a, Kind k, rr_op_t op, int per_cu, int sync, int batch, int timeout_us,
                         hipStream_t stream);
// Barrier timeouts of the bucket kernel on the current device.
hipError_t bucket_timeouts(unsigned long long* count);

// Tensor-parallel layouts (rr_multi.hip) on row-major [rows, cols] matrices
// with cols = p*w.  "Units" are 16-byte groups, or narrower units (4, 2, 1
// bytes) for the copy, or single elements for an unaligned fold.
struct ColsArgs {
  const void* src[RR_MAX_RANKS];
  void* dst[RR_MAX_RANKS];
  uint64_t rows;
  uint64_t wu;  // units per row of one slice (w elements)
  uint64_t du;  // units per row of the full matrix (p*w elements)
  int32_t p;
  int32_t div;  // AVG: p; unused otherwise
};

// All-gather along dim 1: dst[r][b, c*w + j] = src[c][b, j] for every r.
// xcd_dst: destinations per workgroup of the XCD layout (1, 2, 4), 0 = never,
// -1 = by the bytes written.
hipError_t launch_gather_cols(const ColsArgs& a, int unit_bytes, int nontemporal, int per_cu, int xcd_dst,
                              hipStream_t stream);
// Reduce-scatter along dim 1: dst[c][b, j] = fold over k = 1..p of
// src[(c+k) mod p][b, c*w + j] (ring order of chunk c), then the op's last
// step and the one conversion.  vec = 1: 16-byte groups, else elements.
hipError_t launch_fold_cols(const ColsArgs& a, Kind k, rr_op_t op, int vec, int per_cu, hipStream_t stream);

// The ring schedule in one persistent kernel (rr_exec.hip).  in/out: the
// ranks' inputs and outputs; work: the ranks' working buffers (float32 slots
// of a workspace for 16-bit types, else the outputs).  nslices, slot, tag and
// timeout_ticks are set by the launcher.
struct ExecArgs {
  const void* in[RR_MAX_RANKS];
  void* out[RR_MAX_RANKS];
  void* work[RR_MAX_RANKS];
  uint64_t bound[RR_MAX_RANKS + 1];  // chunk bounds floor(c*n/p)
  uint64_t timeout_ticks;            // bounded wait per flag, wall-clock ticks
  unsigned long long tag;            // launch tag << 24
  int32_t p;
  int32_t nslices;
  int32_t div;   // AVG: p
  int32_t vec;   // 1: every buffer 16-byte aligned
  uint32_t slot;
  int32_t captured;  // 1: launched under graph capture (fixed tag, flags reset first)
  int32_t xcds;      // > 0: workers of a slice are workgroups congruent mod xcds (one XCD each)
  int32_t pad;
};

// per_cu_cap > 0 limits the workers per compute unit; max_slices (1..64)
// limits the slices per chunk; timeout_us bounds each wait of a worker on a
// flag.
hipError_t launch_ring_exec(const ExecArgs& a, Kind k, rr_op_t op, int per_cu_cap, int max_slices, int timeout_us,
                            hipStream_t stream);
// Launches of the ring executor on `device` that stopped on a timed-out wait.
hipError_t ring_exec_failures(int device, unsigned long long* count);

hipError_t launch_fold(const FoldLaunch& f, hipStream_t stream);
// The phased fold serves same-kind folds on 16-byte-aligned buffers.
bool phase_supported(const FoldLaunch& f);
hipError_t launch_fold_phase(const FoldLaunch& f, const PhaseTuning& pt, hipStream_t stream);
// Number of phase barriers on `device` that ended by timeout since load.
hipError_t phase_barrier_timeouts(int device, unsigned long long* count);
hipError_t launch_fold_ring_all(const FoldLaunch& f, hipStream_t stream);
hipError_t launch_fold_ring_shard(const FoldLaunch& f, hipStream_t stream);
hipError_t launch_fold_asc_one(const FoldLaunch& f, hipStream_t stream);
hipError_t launch_fold_hier_all(const FoldLaunch& f, hipStream_t stream);
// The hierarchical variants (kHierRing, kHierAllWire, kHierRingWire), run-time p.
hipError_t launch_fold_hier_var(const FoldLaunch& f, hipStream_t stream);
// Copies move units of unit_bytes in {16, 4, 2, 1}; nontemporal != 0 uses
// nontemporal loads, and nontemporal stores for copy_pairs and for a fan-out
// of 16-byte units that writes at most 128 MiB; grid_cap 0 = the default
// workgroup count (fan-out of 16-byte units: one tile per workgroup, with
// units_per_lane units per lane, 4 unless 1, 2 or 8).
// One source segment per seg to every destination.  xcd_dst: destinations
// per workgroup of the XCD layout (1, 2 or 4), 0 = never, -1 = by the bytes
// written; xcd_window: its blocks per XCD window (0 = default) (see
// rr_copy.hip).
hipError_t launch_fanout(const FanoutArgs& a, int unit_bytes, int nontemporal, int grid_cap, int units_per_lane,
                         int xcd_dst, int xcd_window, hipStream_t stream);
// Plain copy: len[] in bytes.
hipError_t launch_copy_pairs(const PairArgs& a, int unit_bytes, int nontemporal, int grid_cap, hipStream_t stream);
// Element conversion (len[] in elements): 16-bit kinds <-> float32, or
// float32 -> float32 (src may equal dst); with a.div > 0 every value is first
// divided by a.div.
hipError_t launch_convert_pairs(const PairArgs& a, Kind from, Kind to, int grid_cap, hipStream_t stream);
// Ring reduce-scatter step on accumulator-type buffers: dst = src (+) dst.
hipError_t launch_ring_step(const PairArgs& a, Kind acc_kind, rr_op_t op, int grid_cap,
                            hipStream_t stream);

}  // namespace rr
