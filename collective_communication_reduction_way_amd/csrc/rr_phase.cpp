// rr_phase.cpp -- host side of the phased streaming fold: tiling of the
// segments into tiles, heads and tails, grid and round count, and the state
// of the soft barrier (a counter set per stream and a fresh launch tag per
// launch).  The kernels and the design are in rr_phase_impl.h.
#include <hip/hip_runtime_api.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>

#include "rr_phase.h"

namespace rr {

namespace {

constexpr int kMaxDevices = 64;

struct DeviceState {
  std::once_flag once;
  int cus = 0;
  int wall_khz = 0;
  std::atomic<unsigned long long> launches{0};
  std::mutex mu;
  std::map<hipStream_t, uint32_t> slot_of;
  std::map<uint32_t, int> occupancy;  // resident workgroups per CU, by kernel key
};

DeviceState g_dev[kMaxDevices];

hipError_t device_of(hipStream_t s, int* dev) {
  if (s != nullptr) return hipStreamGetDevice(s, dev);
  return hipGetDevice(dev);
}

uint32_t slot_for(DeviceState& d, hipStream_t s) {
  std::lock_guard<std::mutex> lock(d.mu);
  auto it = d.slot_of.find(s);
  if (it != d.slot_of.end()) return it->second;
  // a program that keeps making streams must not grow the map without bound;
  // starting the assignment afresh only makes some streams share counters,
  // which costs time, never results (the barrier orders no data)
  if (d.slot_of.size() >= 4096) d.slot_of.clear();
  const uint32_t slot = static_cast<uint32_t>(d.slot_of.size() % kSyncSlots);
  d.slot_of.emplace(s, slot);
  return slot;
}

DeviceState* state_of(hipStream_t s, hipError_t* err) {
  int dev = 0;
  *err = device_of(s, &dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  DeviceState& d = g_dev[dev];
  std::call_once(d.once, [&] {
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) d.cus = 0;
    if (hipDeviceGetAttribute(&d.wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) d.wall_khz = 0;
  });
  return &d;
}

// Slot, tag and wait bound of a barrier launch on stream s.  Eager launches
// take tags 2, 3, ...; a launch under graph capture takes kCapturedTag (its
// launcher captures a reset of the counters ahead of it).
hipError_t sync_args_on(DeviceState& d, hipStream_t s, int timeout_us, SyncArgs* y) {
  memset(y, 0, sizeof(*y));
  y->slot = slot_for(d, s);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return e;
  if (cs == hipStreamCaptureStatusActive) {
    y->captured = 1;
    y->tag = kCapturedTag;
  } else {
    const unsigned long long id = d.launches.fetch_add(1) + 2;
    y->tag = (id & ((1ull << (64 - kLaunchShift)) - 1)) << kLaunchShift;
    if (y->tag <= kCapturedTag) y->tag = 2 * kCapturedTag;
  }
  const uint64_t khz = d.wall_khz > 0 ? static_cast<uint64_t>(d.wall_khz) : 100000;
  uint64_t ticks = khz * static_cast<uint64_t>(timeout_us > 0 ? timeout_us : 1) / 1000;
  if (ticks < 1) ticks = 1;
  if (ticks > 0xFFFFFFFFull) ticks = 0xFFFFFFFFull;
  y->timeout_ticks = static_cast<uint32_t>(ticks);
  return hipSuccess;
}

// Cut every segment into 16-byte groups and the groups into tiles of `tile`
// groups; fills the per-segment tables of `a` and returns the tile count.
uint64_t tile_segments(const FoldLaunch& f, uint64_t V, uint64_t tile, PhaseArgs& a) {
  uint64_t tiles = 0;
  const bool ring = uses_bounds(f.mode);  // rows bounded by bound[] (else one row of n)
  a.edges = 0;
  for (int sg = 0; sg < f.segments; ++sg) {
    const uint64_t lo = ring ? f.args.bound[sg] : 0;
    const uint64_t hi = ring ? f.args.bound[sg + 1] : f.args.n;
    const uint64_t g_lo = (lo + V - 1) / V;
    const uint64_t g_hi = hi / V;
    const uint64_t groups = g_hi > g_lo ? g_hi - g_lo : 0;
    const uint64_t seg_tiles = (groups + tile - 1) / tile;
    a.seg_tile[sg] = static_cast<uint32_t>(tiles);
    a.seg_last[sg] = static_cast<uint32_t>(seg_tiles ? groups - (seg_tiles - 1) * tile : 0);
    // head [lo, min(g_lo*V, hi)) and tail [max(g_hi, g_lo)*V, hi): each < V
    const uint64_t head_end = g_lo * V < hi ? g_lo * V : hi;
    const uint64_t tail_beg = (g_hi > g_lo ? g_hi : g_lo) * V;
    a.head_len[sg] = static_cast<uint8_t>(head_end > lo ? head_end - lo : 0);
    a.tail_len[sg] = static_cast<uint8_t>(hi > tail_beg ? hi - tail_beg : 0);
    if (a.head_len[sg] || a.tail_len[sg]) a.edges = 1;
    tiles += seg_tiles;
  }
  if (tiles >= 0x7FFFFFFFull) return tiles;
  a.seg_tile[f.segments] = static_cast<uint32_t>(tiles);
  a.tiles = static_cast<uint32_t>(tiles);
  // uniform tiling: equal segment lengths (p | n for the ring modes) whose
  // first element starts a group, hence equal tile counts and last tiles
  a.uniform_tiles = a.seg_tile[1] - a.seg_tile[0];
  a.uniform_last = a.seg_last[0];
  a.seg_len = ring ? f.args.bound[1] - f.args.bound[0] : f.args.n;
  for (int sg = 0; sg < f.segments; ++sg) {
    const uint64_t lo = ring ? f.args.bound[sg] : 0;
    const uint64_t hi = ring ? f.args.bound[sg + 1] : f.args.n;
    if (hi - lo != a.seg_len || lo != static_cast<uint64_t>(sg) * a.seg_len || lo % V != 0 ||
        a.seg_tile[sg + 1] - a.seg_tile[sg] != a.uniform_tiles || a.seg_last[sg] != a.uniform_last)
      a.uniform_tiles = 0;
  }
  return tiles;
}

hipError_t launch_mode(const FoldLaunch& f, const PhaseArgs& a, unsigned grid, int unroll, bool sync, bool static_p,
                       int* occ, hipStream_t s) {
  switch (f.mode) {
    case FoldMode::kRingAll: return phase_launch_ring(a, f.in_kind, f.op, grid, unroll, sync, static_p, occ, s);
    case FoldMode::kHierAll: return phase_launch_hier(a, f.in_kind, f.op, grid, unroll, sync, static_p, occ, s);
    case FoldMode::kHierRing:
    case FoldMode::kHierAllWire:
    case FoldMode::kHierRingWire: return phase_launch_hier_var(a, f.mode, f.in_kind, f.op, grid, unroll, sync, occ, s);
    case FoldMode::kRingShard:
    case FoldMode::kAscOne: return phase_launch_one(a, f.mode, f.in_kind, f.op, grid, unroll, sync, static_p, occ, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

// The batched kernel (k_phase_batch) of a mode: launch, or only report its
// occupancy when occ is not NULL.
hipError_t launch_batch_mode(const FoldLaunch& f, const PhaseArgs& a, unsigned grid, int K, bool sp, int* occ,
                             hipStream_t s) {
  if (f.mode == FoldMode::kRingAll) return phase_launch_ring_batch(a, f.in_kind, f.op, grid, K, sp, occ, s);
  if (f.mode == FoldMode::kHierAll) return phase_launch_hier_batch(a, f.in_kind, f.op, grid, K, occ, s);
  if (is_hier(f.mode)) return phase_launch_hier_var_batch(a, f.mode, f.in_kind, f.op, grid, K, occ, s);
  return phase_launch_one_batch(a, f.mode, f.in_kind, f.op, grid, K, sp, occ, s);
}

// Workgroups of the batched kernel that fit on one compute unit, cached per
// device and kernel.
hipError_t batch_occupancy(DeviceState& d, const FoldLaunch& f, const PhaseArgs& a, int K, bool sp, hipStream_t s,
                           int* occ) {
  const uint32_t key = 0x80000000u | (static_cast<uint32_t>(f.mode) << 16) |
                       (static_cast<uint32_t>(f.in_kind) << 12) | (static_cast<uint32_t>(f.op) << 8) |
                       (static_cast<uint32_t>(K) << 4) | (sp ? 1u : 0u);
  {
    std::lock_guard<std::mutex> lock(d.mu);
    auto it = d.occupancy.find(key);
    if (it != d.occupancy.end()) {
      *occ = it->second;
      return hipSuccess;
    }
  }
  int o = 0;
  const hipError_t e = launch_batch_mode(f, a, 1, K, sp, &o, s);
  if (e != hipSuccess) return e;
  if (o < 1) o = 1;
  std::lock_guard<std::mutex> lock(d.mu);
  d.occupancy[key] = o;
  *occ = o;
  return hipSuccess;
}

// Launch the batched kernel on `resident` workgroups (all resident at once),
// with a barrier slot of stream s.
hipError_t launch_batched(DeviceState& d, const FoldLaunch& f, const PhaseArgs& a, uint64_t tiles, uint64_t resident,
                          int K, bool sp, const PhaseTuning& pt, hipStream_t s) {
  PhaseArgs b = a;
  b.rounds = static_cast<uint32_t>((tiles + resident * K - 1) / (resident * K));
  SyncArgs y;
  const hipError_t e = sync_args_on(d, s, pt.timeout_us, &y);
  if (e != hipSuccess) return e;
  b.slot = y.slot;
  b.tag = y.tag;
  b.timeout_ticks = y.timeout_ticks;
  b.captured = y.captured;
  return launch_batch_mode(f, b, static_cast<unsigned>(resident), K, sp, nullptr, s);
}

// Workgroups per CU of a batched launch: `asked` if > 0, else 3 or 2, each
// capped at the kernel's occupancy, whichever leaves fewer empty tile slots
// in the last round (ties: the fewer rounds).  Full rounds measured best
// (float32 48 MiB per rank, all-reduce: one round at 3 per CU 80.1-81.0%,
// two at 2 per CU with the second half empty 77-78%; reduce-scatter 80.8%
// against 78%).  0 when not even one round of K tiles per workgroup is full,
// except that a single round at least `min_fill` percent full counts too,
// with its empty slots as the waste (min_fill > 100: never).
uint64_t batch_per_cu(uint64_t tiles, uint64_t cus, int K, int occ, int asked, int min_fill) {
  uint64_t best = 0;
  uint64_t best_waste = ~0ull;
  const int options[2] = {asked > 0 ? asked : 3, asked > 0 ? asked : 2};
  for (int c : options) {
    const uint64_t pc = static_cast<uint64_t>(c < occ ? c : occ);
    const uint64_t slots = cus * pc * static_cast<uint64_t>(K);
    if (pc == 0 || (tiles < slots && tiles * 100 < slots * static_cast<uint64_t>(min_fill))) continue;
    const uint64_t waste = (tiles + slots - 1) / slots * slots - tiles;
    if (waste < best_waste) {
      best_waste = waste;
      best = pc;
    }
  }
  return best;
}

}  // namespace

int phase_default_unroll(Kind k, FoldMode m) { return (is_hier(m) && is_half(k)) ? 4 : 8; }

bool phase_supported(const FoldLaunch& f) {
  const bool mode_ok = f.mode == FoldMode::kRingAll || is_hier(f.mode) || f.mode == FoldMode::kRingShard ||
                       f.mode == FoldMode::kAscOne;
  return mode_ok && f.args.vec && f.in_kind == f.out_kind && f.segments >= 1 && f.segments <= RR_MAX_RANKS;
}

// Schedule choice (measured on MI355X; every knob can be forced through
// PhaseTuning; the tile layout, contiguous or interleaved, is chosen last,
// below):
//   ring all-reduce, one round: 8 groups per lane, 2 workgroups per CU, the
//     kernel compiled for p = 8 when p is 8 (float16: the run-time loop);
//     between one and two 8-group tiles per CU: 2, 4 or 8 groups as the
//     8-group tiles number up to 1.25, 1.5 or 2 per CU, one tile per
//     workgroup, the run-time loop (float32 with 8 groups: p = 8 compiled);
//     fewer 8-group tiles than CUs (16-bit types: exactly one per CU too): 4
//     groups per lane, then 2 and 1 while the tiles still fit one per CU;
//   ring all-reduce, several rounds: 4 groups per lane; the batched kernel
//     (below), in one partial round when the tiles do not fill one round of
//     4 tiles per workgroup; with the batches switched off, 4 workgroups per
//     CU of one tile each (shorter phases between barriers), the kernel
//     compiled for p = 8 for bfloat16, the run-time rank loop for the other
//     types;
//   hierarchical all-reduce: the run-time rank loop, 4 workgroups per CU with
//     the 16-bit tile of 4 groups per lane, else 2; with several rounds the
//     batched kernel as for the ring (bfloat16 / float32 24-128 MiB per rank
//     72.8-75.3 / 73.5-75.1% -> 76.3-81.0 / 77.5-81.8% of the HBM peak);
//   reduce-scatter and reduce: 4 groups per lane; with at least one full
//     round of 4 tiles per workgroup at 2 workgroups per CU, the batched
//     kernel behind the barrier (below), else 32 workgroups per CU (the grid
//     oversubscribes the device; workgroups start as others finish) without
//     a barrier; the kernel compiled for p = 8.
// With the barrier, the grid never exceeds what the device can keep resident
// at once (the kernel's occupancy times the compute units): workgroups that
// had to wait for a free slot would make every barrier run into its timeout.
hipError_t launch_fold_phase(const FoldLaunch& f, const PhaseTuning& pt, hipStream_t s) {
  hipError_t e = hipSuccess;
  DeviceState* dp = state_of(s, &e);
  if (!dp) return e;
  DeviceState& d = *dp;
  const uint64_t cus = d.cus > 0 ? static_cast<uint64_t>(d.cus) : 256;
  const bool ring = f.mode == FoldMode::kRingAll;
  const uint64_t V = is_half(f.in_kind) ? 8 : 4;
  // the kernels with fewer than 8 groups per lane exist for every op of the
  // ring all-reduce, reduce-scatter and reduce, and for sums elsewhere
  const bool small_ok = f.op == RR_SUM || f.op == RR_AVG || f.mode == FoldMode::kRingAll ||
                        f.mode == FoldMode::kRingShard || f.mode == FoldMode::kAscOne;
  // the kernels compiled for p = 8: default for the modes that read p inputs
  // and write one output or all of them in ring order, binary16 excepted:
  // with every rank unrolled its conversions are hoisted past 256 registers
  // (one wave per SIMD), and the run-time rank loop measured faster (8 MiB
  // per rank 71% -> 72.5% of the HBM peak, 128 MiB 55% -> 73%)
  const bool f16 = f.in_kind == Kind::kF16;
  bool static_p = pt.static_p >= 0 ? pt.static_p != 0
                                   : (!f16 && (ring || f.mode == FoldMode::kRingShard || f.mode == FoldMode::kAscOne));
  // reduce-scatter and reduce: one output per p inputs
  const bool one_out = f.mode == FoldMode::kRingShard || f.mode == FoldMode::kAscOne;
  int unroll = phase_default_unroll(f.in_kind, f.mode);
  if ((pt.unroll == 4 || (one_out && pt.unroll == 0)) && small_ok) unroll = 4;
  // 2 and 1 groups per lane: compiled for the ring all-reduce, reduce-scatter
  // and reduce without the barrier
  if ((pt.unroll == 1 || pt.unroll == 2) && small_ok && (ring || one_out)) unroll = pt.unroll;
  // one-output modes run without the barrier, so nothing ties their grid to
  // residency: 32 workgroups per CU (about one tile each) measured best
  int per_cu = pt.per_cu > 0 ? pt.per_cu : (one_out ? 32 : (unroll == 4 ? 4 : 2));

  PhaseArgs a;
  memset(&a, 0, sizeof(a));
  a.f = f.args;
  a.segments = f.segments;
  uint64_t tiles = tile_segments(f, V, static_cast<uint64_t>(kBlock) * unroll, a);
  if (tiles >= 0x7FFFFFFFull) return hipErrorInvalidValue;
  uint64_t grid = pt.grid > 0 ? static_cast<uint64_t>(pt.grid) : cus * static_cast<uint64_t>(per_cu);
  bool several = false;  // ring all-reduce of several rounds, default tiling
  // Batched rounds (below) also take the ring all-reduces of more than 13,
  // and the hierarchical ones of more than 12, strips of kBlock groups per
  // CU, which one round of their default tile would hold: one batched round
  // with the barrier against one barrier-free round, measured through this
  // library on one MI355X, p = 8 (per-rank MiB): ring float32 13 / 14 / 16
  // MiB 75.0 / 73.7 / 76.8% -> 73.5 / 74.1 / 78.1% of the HBM peak,
  // bfloat16 13 / 16 MiB 74.6 / 75.9% -> 72.7 / 77.1%, float16 16 MiB 75.6%
  // -> 77.7%; hierarchical bfloat16 12 / 13 / 16 MiB 77.7 / 65.0 / 74.8% ->
  // 71.5 / 71.5 / 76.7%, with wire rounding 16 MiB 70.9% -> 72.3%, float32
  // 16 MiB 75.9% -> 77.5%; at 10 and 12 MiB the barrier-free ring round
  // stays ahead by 3-7 points.
  const uint64_t batch_strips_per_cu = is_hier(f.mode) ? 12 : 13;
  const bool batch_early = pt.ar_batch != 1 && pt.sync;
  if (ring && pt.unroll == 0 && pt.grid == 0 && small_ok && unroll == 8 &&
      (tiles > grid || (batch_early && tiles * unroll > batch_strips_per_cu * cus))) {
    // several rounds: the smaller tile, more workgroups
    several = true;
    unroll = 4;
    if (pt.per_cu <= 0) per_cu = 4;
    if (pt.static_p < 0) static_p = f.in_kind == Kind::kBF16;
    tiles = tile_segments(f, V, static_cast<uint64_t>(kBlock) * unroll, a);
    if (tiles >= 0x7FFFFFFFull) return hipErrorInvalidValue;
    grid = cus * static_cast<uint64_t>(per_cu);
  } else if (ring && pt.unroll == 0 && pt.grid == 0 && small_ok && unroll == 8 && tiles > cus &&
             tiles < 2 * cus) {
    // one round of between one and two tiles of 8 groups per lane per CU:
    // the tile that spreads the launch most evenly, one tile per workgroup,
    // the run-time rank loop (float32 keeps p = 8 unrolled with 8 groups).
    // Measured through this library on one MI355X, p = 8, against 8 groups
    // per lane at 2 workgroups per CU (16-bit types: 4 groups, 4 per CU):
    // float32 8.5 / 9.5 / 10 MiB per rank (up to 1.25 tiles of 8 groups per
    // CU) with 2 groups 59 / 60 / 63% -> 74 / 74.5 / 75% of the HBM peak,
    // 10.5 / 11 / 11.5 MiB (up to 1.5) with 4 groups 64 / 67 / 70.5% -> 73 /
    // 72 / 75%; bfloat16 8.5 / 10 MiB 67.6 / 71.6% -> 73.4 / 73.9%, 13.5 /
    // 14 / 15 MiB (above 1.5) with 8 groups 69 / 69.4 / 69.1% -> 74.4 /
    // 73.8 / 74.5%.  Above 1.5 tiles per CU the batched round above now
    // takes the launch, unless batches are switched off.
    if (4 * tiles <= 5 * cus) {
      unroll = 2;
    } else if (2 * tiles <= 3 * cus) {
      unroll = 4;
    }
    if (pt.static_p < 0) static_p = unroll == 8 && !is_half(f.in_kind);
    if (unroll != 8) {
      tiles = tile_segments(f, V, static_cast<uint64_t>(kBlock) * unroll, a);
      if (tiles >= 0x7FFFFFFFull) return hipErrorInvalidValue;
    }
    grid = tiles;
  } else if (ring && pt.unroll == 0 && pt.grid == 0 && small_ok && unroll == 8 &&
             (tiles < cus || (is_half(f.in_kind) && tiles < 2 * cus))) {
    // one round with too few tiles of 8 groups per lane to fill the device
    // (fewer than one per CU; for 16-bit types, which also convert, fewer
    // than two): the smaller tile.  With at most one tile per CU all p = 8
    // ranks unrolled measured best, with more the run-time rank loop.
    unroll = 4;
    if (pt.per_cu <= 0) per_cu = 4;
    tiles = tile_segments(f, V, static_cast<uint64_t>(kBlock) * unroll, a);
    if (tiles >= 0x7FFFFFFFull) return hipErrorInvalidValue;
    // at most half as many tiles as CUs (small launches): 2 groups per lane,
    // then 1, as long as the tiles still fit one per CU (1 MiB fp32 per rank:
    // 29% -> 39-40% of the HBM peak; 3 MiB, where the halving would give 1.5
    // tiles per CU, stays at 4 groups)
    while (unroll > 1 && 2 * tiles <= cus) {
      unroll /= 2;
      tiles = tile_segments(f, V, static_cast<uint64_t>(kBlock) * unroll, a);
      if (tiles >= 0x7FFFFFFFull) return hipErrorInvalidValue;
    }
    if (pt.static_p < 0) static_p = tiles <= cus;
    grid = cus * static_cast<uint64_t>(per_cu);
  }
  if (several && pt.ar_batch != 1 && pt.sync && tiles <= kMaxBarrierTiles) {
    // The ring all-reduce of several rounds in batched rounds (k_phase_batch):
    // K tiles of 4 groups per lane per workgroup and round at 2 or 3
    // workgroups per CU, interleaved in runs, the write phase output by
    // output.  Measured
    // through this library on one MI355X, p = 8, against one tile per
    // workgroup and round at 4 per CU: float32 32 MiB per rank 75.5% ->
    // 80.4-81.8% of the HBM peak, 96 MiB 76% -> 78.3-78.5%, 128 MiB 76.5% ->
    // 78.2-78.6%; bfloat16 128 MiB 77% -> 78.8-79.1%.  Below one full round
    // (16-32 MiB per rank) a single partial round, same run: float32 18 / 20
    // / 24 / 27 / 30 MiB 70-71 / 72 / 75 / 74 / 74-75% -> 75-76 / 77.5 / 79 /
    // 76-77 / 78.5-79%, bfloat16 18 / 20 / 22 / 26 / 30 MiB 69-70 / 72 / 72 /
    // 75 / 74% -> 77 / 78 / 78 / 78 / 79%; and where the last round would be
    // short, one partial round at 3 per CU (float32 34 / 36 / 40 / 44 MiB
    // 76.6 / 77.6 / 75.5 / 77% -> 79.3 / 80.5 / 80 / 80.3%).  With the
    // workgroups meeting again before each later read phase (k_phase_batch):
    // float32 96 / 128 MiB 81 / 83%, bfloat16 128 MiB 83%.
    const bool sp = (pt.static_p >= 0 ? pt.static_p != 0 : !f16) && f.args.p == 8;
    const int K = pt.ar_batch == 2 || pt.ar_batch == 4 ? pt.ar_batch : 4;
    int occ = 0;
    e = batch_occupancy(d, f, a, K, sp, s, &occ);
    if (e != hipSuccess) return e;
    const uint64_t per_cu_b = batch_per_cu(tiles, cus, K, occ, pt.per_cu, 0);
    if (per_cu_b > 0) {
      // interleaved runs of 16 tiles: against 8, same runs, 64 / 96 / 128
      // MiB per rank float32 80.1 / 79.0 / 79.3% -> 80.8 / 79.3 / 79.6%,
      // bfloat16 80.3 / 79.5 / 80.4% -> 80.9 / 79.9 / 81.0% of the HBM
      // peak; runs of 32 and 64 lost 2-4 points
      const int strips = pt.strips > 0 ? pt.strips : 16;
      if (strips > 1 && a.uniform_tiles != 0) {
        const uint32_t tile = static_cast<uint32_t>(kBlock * unroll);
        const uint32_t full = a.uniform_last == tile ? a.uniform_tiles : a.uniform_tiles - 1;
        a.strips = static_cast<uint32_t>(strips);
        a.strip_tiles = full - full % a.strips;
      }
      return launch_batched(d, f, a, tiles, cus * per_cu_b, K, sp, pt, s);
    }
  }
  if (is_hier(f.mode) && pt.unroll == 0 && pt.grid == 0 && pt.ar_batch != 1 && pt.sync &&
      (tiles > grid || tiles * static_cast<uint64_t>(unroll) > batch_strips_per_cu * cus)) {
    // The hierarchical all-reduce and its variants of several rounds in
    // batched rounds: as the ring's (K tiles of 4 groups per lane per
    // workgroup and round, one partial round allowed, interleaved runs),
    // with the run-time rank loop.
    const int K = pt.ar_batch == 2 || pt.ar_batch == 4 ? pt.ar_batch : 4;
    const uint64_t tiles4 = tile_segments(f, V, static_cast<uint64_t>(kBlock) * 4, a);
    if (tiles4 >= 0x7FFFFFFFull) return hipErrorInvalidValue;
    if (tiles4 <= kMaxBarrierTiles) {
      int occ = 0;
      e = batch_occupancy(d, f, a, K, false, s, &occ);
      if (e != hipSuccess) return e;
      const uint64_t per_cu_b = batch_per_cu(tiles4, cus, K, occ, pt.per_cu, 0);
      if (per_cu_b > 0) {
        const int strips = pt.strips > 0 ? pt.strips : 8;
        if (strips > 1 && a.uniform_tiles != 0) {
          const uint32_t tile = static_cast<uint32_t>(kBlock * 4);
          const uint32_t full = a.uniform_last == tile ? a.uniform_tiles : a.uniform_tiles - 1;
          a.strips = static_cast<uint32_t>(strips);
          a.strip_tiles = full - full % a.strips;
        }
        return launch_batched(d, f, a, tiles4, cus * per_cu_b, K, false, pt, s);
      }
    }
    tiles = tile_segments(f, V, static_cast<uint64_t>(kBlock) * unroll, a);
    if (tiles >= 0x7FFFFFFFull) return hipErrorInvalidValue;
  }
  if (one_out && pt.batch != 1 && pt.unroll == 0 && pt.grid == 0 && pt.sync && unroll == 4 &&
      tiles <= kMaxBarrierTiles) {
    // Reduce-scatter and reduce with at least one full round of K tiles per
    // resident workgroup: the batched kernel (k_phase_batch), K tiles per
    // workgroup and round behind the soft barrier, so that the writes come in
    // bursts instead of trickling between the reads.  Measured through this
    // library on one MI355X, p = 8, against one tile per workgroup without a
    // barrier (two machines): float32 96 MiB per rank 75-76% -> 79-81.5% of the
    // HBM peak, bfloat16 128 MiB 75% -> 80.5-82%, 64 MiB 75% -> 80%; at
    // 16 MiB and below (less than one full round) the batches lost.
    const int K = pt.batch == 2 || pt.batch == 4 ? pt.batch : 4;
    const bool sp = static_p && f.args.p == 8;
    int occ = 0;
    e = batch_occupancy(d, f, a, K, sp, s, &occ);
    if (e != hipSuccess) return e;
    // 4 per CU measured worse for float32 (128 MiB per rank, two full rounds:
    // 77% against 80% with 2 per CU), hence at most 3
    // one partial round when at least 70% full: float32 / bfloat16 24 and
    // 28 MiB per rank (75% and 87.5% full) 77.5-78.5% -> 79.3-79.9% of the
    // HBM peak for reduce-scatter and reduce; at 50-62.5% full (16, 20 MiB)
    // the partial round lost 1-2 points
    const uint64_t per_cu_b = batch_per_cu(tiles, cus, K, occ, pt.per_cu, 70);
    if (per_cu_b > 0) return launch_batched(d, f, a, tiles, cus * per_cu_b, K, sp, pt, s);
  }
  if (one_out && pt.unroll == 0 && pt.grid == 0 && unroll == 4) {
    // reduce-scatter and reduce too small for a tile of 4 groups per lane on
    // every CU: 2, then 1, while the tiles still fit one per CU
    while (unroll > 1 && 2 * tiles <= cus) {
      unroll /= 2;
      tiles = tile_segments(f, V, static_cast<uint64_t>(kBlock) * unroll, a);
      if (tiles >= 0x7FFFFFFFull) return hipErrorInvalidValue;
    }
  }
  if (grid > tiles) grid = tiles;
  if (grid < 1) grid = 1;
  a.rounds = static_cast<uint32_t>((tiles + grid - 1) / grid);
  // Writes are 1/(p+1) of the traffic of the one-output modes: a barrier
  // between the phases of one tile per workgroup gained nothing there
  // (measured); only the batched kernel above separates them.
  const bool sync = pt.sync && !one_out && a.rounds > 1 && unroll >= 4 && tiles <= kMaxBarrierTiles;
  if (sync) {
    // occupancy of the kernel about to run, cached per device and kernel
    const uint32_t key = (static_cast<uint32_t>(f.mode) << 16) | (static_cast<uint32_t>(f.in_kind) << 12) |
                         (static_cast<uint32_t>(f.op) << 8) | (static_cast<uint32_t>(unroll) << 4) |
                         ((static_p && f.args.p == 8) ? 1u : 0u);
    int occ = 0;
    {
      std::lock_guard<std::mutex> lock(d.mu);
      auto it = d.occupancy.find(key);
      if (it != d.occupancy.end()) occ = it->second;
    }
    if (occ == 0) {
      e = launch_mode(f, a, 1, unroll, true, static_p, &occ, s);
      if (e != hipSuccess) return e;
      if (occ < 1) occ = 1;
      std::lock_guard<std::mutex> lock(d.mu);
      d.occupancy[key] = occ;
    }
    const uint64_t resident = cus * static_cast<uint64_t>(occ);
    if (grid > resident) {
      grid = resident;
      a.rounds = static_cast<uint32_t>((tiles + grid - 1) / grid);
    }
    SyncArgs y;
    e = sync_args_on(d, s, pt.timeout_us, &y);
    if (e != hipSuccess) return e;
    a.slot = y.slot;
    a.tag = y.tag;
    a.timeout_ticks = y.timeout_ticks;
    a.captured = y.captured;
  }
  // Interleaved tiles: whole runs of `strips` full tiles at the start of
  // every segment (uniform tilings only).  Measured with the bench on one
  // MI355X, each figure against the kernels without interleaving on the
  // same machine: the folds that write every rank gain when a launch has
  // several rounds (96 MiB float32 all-reduce 72.8% -> 75.6% of the HBM
  // peak with runs of 8; 128 MiB bfloat16 74.5% -> 77.1% with runs of 4).
  // One-round launches (8 MiB per rank) lost with it, and reduce-scatter
  // and reduce gained nothing.
  // Only the kernels of these modes compiled with the barrier can
  // interleave (can_interleave in rr_phase_impl.h).
  const bool interleaves = (ring || is_hier(f.mode)) && sync;
  int strips = pt.strips;
  if (strips == 0) strips = (ring && !is_half(f.in_kind)) ? 8 : 4;
  if (strips > 1 && interleaves && a.uniform_tiles != 0) {
    const uint32_t tile = static_cast<uint32_t>(kBlock * unroll);
    const uint32_t full = a.uniform_last == tile ? a.uniform_tiles : a.uniform_tiles - 1;
    a.strips = static_cast<uint32_t>(strips);
    a.strip_tiles = full - full % a.strips;
  }
  return launch_mode(f, a, static_cast<unsigned>(grid), unroll, sync, static_p, nullptr, s);
}

hipError_t phase_sync_args(hipStream_t s, int timeout_us, SyncArgs* y) {
  hipError_t e = hipSuccess;
  DeviceState* d = state_of(s, &e);
  if (!d) return e;
  return sync_args_on(*d, s, timeout_us, y);
}

hipError_t phase_barrier_timeouts(int device, unsigned long long* count) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (device != cur && (e = hipSetDevice(device)) != hipSuccess) return e;
  unsigned long long ring = 0;
  unsigned long long hier = 0;
  unsigned long long var = 0;
  unsigned long long one = 0;
  unsigned long long bucket = 0;
  e = phase_timeouts_ring(&ring);
  if (e == hipSuccess) e = phase_timeouts_hier(&hier);
  if (e == hipSuccess) e = phase_timeouts_hier_var(&var);
  if (e == hipSuccess) e = phase_timeouts_one(&one);
  if (e == hipSuccess) e = bucket_timeouts(&bucket);
  *count = ring + hier + var + one + bucket;
  if (device != cur) {
    const hipError_t e2 = hipSetDevice(cur);
    if (e == hipSuccess) e = e2;
  }
  return e;
}

}  // namespace rr
