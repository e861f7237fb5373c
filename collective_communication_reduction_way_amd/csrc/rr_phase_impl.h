// rr_phase_impl.h -- the phased streaming fold (gfx950): the fused ring
// all-reduce and the fused hierarchical all-reduce on 16-byte-aligned
// buffers.  Included once per mode (rr_phase_ring.hip, rr_phase_hier.hip);
// the host side is rr_phase.cpp.
//
// What is computed is exactly what k_fold computes (same fold orders, same
// single rounding; see rr_fold_impl.h): element i of chunk c folds
// x_{c+1}, ..., x_c, the order in which the reduce-scatter phase of page "LLM
// Parallelism 基础", section "Ring AllReduce", accumulates chunk c.  Only the
// schedule of the memory traffic differs.
//
// Schedule.  A persistent grid of G workgroups (about two per compute unit)
// walks the tiles of all chunks in rounds; a tile is kBlock*U 16-byte groups
// (32 KiB per rank for float32).  In each round a workgroup first reads its
// tile from every rank, one rank after the other with the next rank's loads
// in flight while the current one is folded, keeping the partial results in
// registers; then it writes the result to every output.  HBM serves pure read
// streams and pure write streams at a much higher rate than an interleaving of
// both, so between the read phase and the write phase of a round the
// workgroups meet at a soft grid barrier, and in batched rounds
// (k_phase_batch) the folds that write every rank meet again between a
// round's write phase and the next round's read phase: for the length of a
// phase the whole chip then reads, or writes, only.  Without the second
// barrier the workgroups that finish their stores first start the next
// round's reads while the others still write; per-workgroup wall-clock stamps
// of a 96 MiB float32 all-reduce (two batched rounds) showed each pure phase
// at about 85% of the HBM peak and that mixed stretch at about 75%, and the
// second barrier took the launch from 78% to 81% (128 MiB bfloat16, four
// rounds: 80.5% -> 83%).  In k_phase's rounds of one tile per workgroup the
// phases are short and the second barrier lost up to 2.5 points, so those
// rounds keep one.  The barrier orders nothing that the
// results depend on (every workgroup reads and writes only its own tiles), so
// it only shapes the traffic: its wait is bounded by a wall-clock timeout, and
// a workgroup that times out simply goes on.  Results are therefore the same
// whether or not the barrier ever synchronises (for instance when the
// workgroups are not all resident because other kernels share the GPU).
//
// Barrier state.  Per slot, kSyncSubs arrival counters and one top counter,
// each a 64-bit word on its own 128-byte line.  Workgroup b arrives on
// counter b % kSyncSubs (so the arrivals do not all contend for one line);
// the last arrival of a counter in a round bumps the top counter, and the
// waiters poll only the top counter.  Every counter holds
// (launch tag << kLaunchShift) + count: each launch carries a fresh, larger
// tag and claims a counter with an atomic max before counting on it, which
// discards whatever older launches left there without any reset.  Slots are
// assigned per stream, so kernels that may run concurrently use different
// counters; if two ever share one, barriers pass early or time out, and the
// results are unaffected.
//
// Interleaved tiles.  In the launches with the barrier (several rounds) the
// whole tiles of a segment are taken in runs of PhaseArgs::strips tiles
// whose strips of kBlock groups interleave: tile j of a run holds strips j,
// j + strips, j + 2*strips, ... of the run, so that neighbouring workgroups
// share one region of memory instead of each owning U contiguous strips.
// That layout is compiled only into those kernels (can_interleave below).
//
// Used for the folds that write every rank (ring and hierarchical
// all-reduce), whose traffic is half reads and half writes, and for
// reduce-scatter and reduce, which write one output per p inputs.
#pragma once

#include <hip/hip_runtime.h>

#include "rr_fold_impl.h"
#include "rr_phase.h"
#include "rr_sync.h"

namespace rr {

namespace {

// The soft barrier, on this mode's PhaseArgs (rr_sync.h).
__device__ __forceinline__ void sync_claim(const PhaseArgs& a) { sync_claim_at(a.slot, a.tag); }

__device__ __forceinline__ void soft_barrier(const PhaseArgs& a, uint32_t round) {
  soft_barrier_at(a.slot, a.tag, a.timeout_ticks, round);
}

// Loads of one rank's tile.  In a partial tile (valid < kBlock*U groups) the
// lanes past the end re-read the tile's last group instead of branching
// around the load, so that one code path serves every tile; their values are
// never stored.
//
// IL (kernels that can interleave their tiles): `gap` groups lie between the
// end of one strip of kBlock groups and the start of the next (0 for a
// contiguous tile; only whole tiles interleave).  Without IL the gap is not
// part of the code at all.
template <bool IL, class E, int V, int U>
__device__ __forceinline__ void load_tile(Raw<E, V> (&x)[U], const char* base, uint32_t valid, uint32_t gap) {
  const uint32_t lane = threadIdx.x;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t g = min(lane + u * kBlock, valid - 1);
    if constexpr (IL) g += u * gap;
    load_group<true>(x[u], reinterpret_cast<const typename E::S*>(base + g * 16u));
  }
}

// Read phase of one tile: fold the p inputs (in the mode's order) into acc.
// P > 0 (p known at compile time): the rotated source pointers are loaded
// once into scalar registers and the rank loop is unrolled, leaving the
// interleaving of loads and folds to the scheduler.  P == 0: a run-time loop
// that keeps the next rank's loads in flight while the current rank is
// folded.
template <class E, class OP, int P, int U, FoldMode M, bool IL>
__device__ __forceinline__ void read_fold(const FoldArgs& f, int seg, int p, uint64_t in_off, uint32_t valid,
                                          uint32_t gap, typename E::A (&acc)[U][16 / sizeof(typename E::S)]) {
  constexpr int V = 16 / sizeof(typename E::S);
  using A = typename E::A;
  A tot[U][V];
  if constexpr (P > 0) {
    const char* src[P];
#pragma unroll
    for (int k = 0; k < P; ++k) src[k] = static_cast<const char*>(f.in[fold_src<M>(k, seg, P, f.group)]) + in_off;
    {
      Raw<E, V> x[U];
      load_tile<IL>(x, src[0], valid, gap);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        unpack(x[u], acc[u]);
#pragma unroll
        for (int j = 0; j < V; ++j) tot[u][j] = acc[u][j];
      }
    }
#pragma unroll
    for (int k = 1; k < P; ++k) {
      Raw<E, V> x[U];
      load_tile<IL>(x, src[k], valid, gap);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        A v[V];
        unpack(x[u], v);
#pragma unroll
        for (int j = 0; j < V; ++j) fold_step<E, OP, M>(acc[u][j], tot[u][j], v[j], k, f.group);
      }
    }
  } else {
    Raw<E, V> cur[U];
    Raw<E, V> nxt[U];
    load_tile<IL>(cur, static_cast<const char*>(f.in[fold_src<M>(0, seg, p, f.group)]) + in_off, valid, gap);
    if (p > 1) load_tile<IL>(nxt, static_cast<const char*>(f.in[fold_src<M>(1, seg, p, f.group)]) + in_off, valid, gap);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      unpack(cur[u], acc[u]);
#pragma unroll
      for (int j = 0; j < V; ++j) tot[u][j] = acc[u][j];
    }
#pragma unroll 1
    for (int k = 1; k < p; ++k) {
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
      if (k + 1 < p)
        load_tile<IL>(nxt, static_cast<const char*>(f.in[fold_src<M>(k + 1, seg, p, f.group)]) + in_off, valid, gap);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        A x[V];
        unpack(cur[u], x);
#pragma unroll
        for (int j = 0; j < V; ++j) fold_step<E, OP, M>(acc[u][j], tot[u][j], x[j], k, f.group);
      }
    }
  }
  const int pp = P > 0 ? P : p;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int j = 0; j < V; ++j) acc[u][j] = fold_finish<E, OP, M>(acc[u][j], tot[u][j], pp, f.group, f.div);
}

template <bool GUARD, bool IL, class E, int V, int U>
__device__ __forceinline__ void store_tile(char* base, const Raw<E, V> (&o)[U], uint32_t valid, uint32_t gap) {
  const uint32_t lane = threadIdx.x;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t g = lane + u * kBlock;
    if constexpr (IL) {
      if (!GUARD || g < valid) store_group<true>(reinterpret_cast<typename E::S*>(base + (g + u * gap) * 16u), o[u]);
    } else {
      if (!GUARD || g < valid) store_group<true>(reinterpret_cast<typename E::S*>(base + g * 16u), o[u]);
    }
  }
}

// Store drain between the outputs of the folds that write every rank, in the
// launches without the barrier (one round): each wave waits until its stores
// to one output have left before it issues those to the next, so that the
// chip writes one output's region at a time instead of spreading its writes
// over all p buffers while other workgroups still read.  Measured through
// this library on one MI355X, p = 8: 16 MiB float32 per rank 71% -> 75.7% of
// the HBM peak, 8 MiB bfloat16 72.5% -> 74%, the 8 MiB bfloat16 hierarchy
// 75.3% -> 76.5%.  With the barrier (the write phase already separate) it
// lost 0.5-2 points, so those kernels are compiled without it.
// RR_DRAIN_STORES=0 at build time compiles it out (for comparisons).
#ifndef RR_DRAIN_STORES
#define RR_DRAIN_STORES 1
#endif
__device__ __forceinline__ void drain_stores() {
#if RR_DRAIN_STORES
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
}

// Waves per SIMD that the register allocation must leave room for (1 = no
// bound).  For the 4-byte types of the modes without running totals a bound
// of three keeps more loads in flight than the allocation the scheduler picks
// by itself (8 MiB fp32 all-reduce: 74.5% -> 75.9% of the HBM peak).  The
// hierarchical modes keep a second set of partials and spill under a bound;
// the 16-bit kinds measured no gain from one.
template <class E, FoldMode M>
constexpr int phase_waves() {
  if constexpr (sizeof(typename E::S) == 4 && (M == FoldMode::kRingAll || M == FoldMode::kRingShard ||
                                               M == FoldMode::kAscOne))
    return 3;
  return 1;
}

// Kernels that can lay their tiles out interleaved (PhaseArgs::strips): the
// folds that write every rank, with the barrier (several rounds).  The
// others are compiled without that arithmetic: in the one-round float32
// all-reduce its mere presence, with the layout switched off, cost about 3
// points of the HBM peak, and the one-round bfloat16 hierarchy lost 2.3
// points with it switched on.
template <class E, FoldMode M, bool SYNC>
constexpr bool can_interleave() {
  return writes_all(M) && SYNC;
}

// SYNC: the soft barrier between the phases of a round is compiled in.  The
// kernel without it is a separate instantiation: barrier code that is
// present but skipped still costs several percent of throughput (it
// constrains how the stores can be scheduled after the folds).
template <class E, class OP, int P, int U, FoldMode M, bool SYNC>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(phase_waves<E, M>()))) void k_phase(PhaseArgs a) {
  using S = typename E::S;
  using A = typename E::A;
  constexpr int V = 16 / sizeof(S);
  constexpr uint32_t kTile = kBlock * U;
  constexpr bool IL = can_interleave<E, M, SYNC>();
  const int p = P > 0 ? P : a.f.p;
  if constexpr (SYNC) sync_claim(a);
  for (uint32_t r = 0; r < a.rounds; ++r) {
    const uint32_t t = r * gridDim.x + blockIdx.x;
    const bool live = t < a.tiles;
    int seg = 0;
    uint32_t valid = 0;
    uint64_t off = 0;  // byte offset of the tile's first group in an input buffer
    uint64_t lo = 0;
    uint32_t gap = 0;  // groups between a tile's strips (interleaved tiles)
    A acc[U][V];
    if (live) {
      uint32_t k;
      if (a.uniform_tiles) {
        seg = static_cast<int>(t / a.uniform_tiles);
        k = t - static_cast<uint32_t>(seg) * a.uniform_tiles;
        valid = (k + 1 == a.uniform_tiles) ? a.uniform_last : kTile;
        if constexpr (uses_bounds(M)) lo = static_cast<uint64_t>(seg) * a.seg_len;
      } else {
        while (a.seg_tile[seg + 1] <= t) ++seg;
        k = t - a.seg_tile[seg];
        valid = (k + 1 == a.seg_tile[seg + 1] - a.seg_tile[seg]) ? a.seg_last[seg] : kTile;
        if constexpr (uses_bounds(M)) lo = a.f.bound[seg];
      }
      if constexpr (IL) {
        uint64_t gk = static_cast<uint64_t>(k) * kTile;  // the tile's first group in the segment
        if (a.strips > 1 && k < a.strip_tiles) {
          const uint32_t run = k / a.strips;
          const uint32_t j = k - run * a.strips;
          gk = static_cast<uint64_t>(run) * a.strips * kTile + j * kBlock;
          gap = (a.strips - 1) * kBlock;
        }
        off = ((lo + V - 1) / V + gk) * 16;
      } else {
        const uint64_t g0 = (lo + V - 1) / V + static_cast<uint64_t>(k) * kTile;
        off = g0 * 16;
      }
      read_fold<E, OP, P, U, M, IL>(a.f, seg, p, off, valid, gap, acc);
    }
    if constexpr (SYNC) soft_barrier(a, r);
    if (live) {
      Raw<E, V> o[U];
#pragma unroll
      for (int u = 0; u < U; ++u) pack(acc[u], o[u]);
      if constexpr (writes_all(M)) {
        if constexpr (P > 0) {
          // every output pointer in scalar registers before the first store
          char* dst[P];
#pragma unroll
          for (int q = 0; q < P; ++q) dst[q] = static_cast<char*>(a.f.out[q]) + off;
          if (valid == kTile) {
#pragma unroll
            for (int q = 0; q < P; ++q) {
              store_tile<false, IL>(dst[q], o, valid, gap);
              if constexpr (!SYNC) drain_stores();
            }
          } else {
#pragma unroll
            for (int q = 0; q < P; ++q) {
              store_tile<true, IL>(dst[q], o, valid, gap);
              if constexpr (!SYNC) drain_stores();
            }
          }
        } else if (valid == kTile) {
          for (int q = 0; q < p; ++q) {
            store_tile<false, IL>(static_cast<char*>(a.f.out[q]) + off, o, valid, gap);
            if constexpr (!SYNC) drain_stores();
          }
        } else {
          for (int q = 0; q < p; ++q) {
            store_tile<true, IL>(static_cast<char*>(a.f.out[q]) + off, o, valid, gap);
            if constexpr (!SYNC) drain_stores();
          }
        }
      } else {
        // reduce-scatter outputs hold only the chunk: group g sits at g*V - lo
        const uint64_t shift = (M == FoldMode::kRingShard) ? lo * sizeof(S) : 0;
        char* d = static_cast<char*>(a.f.out[seg]) + (off - shift);
        if (valid == kTile) {
          store_tile<false, IL>(d, o, valid, gap);
        } else {
          store_tile<true, IL>(d, o, valid, gap);
        }
      }
    }
  }
}


// Batched rounds: in round r, workgroup b folds tiles t = (r K + j) G + b for
// j < K, keeping the K results in registers, meets the others at the soft
// barrier, then writes the K results.  Fewer, larger rounds than k_phase,
// with more loads in flight per workgroup in the read phase.
//   Reduce-scatter and reduce (one output per p inputs): their reads alone
// stream at the read ceiling, but the writes interleaved with them, though
// only 1/(p+1) of the bytes, cost about ten points of the HBM peak (96 MiB
// float32 per rank: 86% with the writes dropped, 75% with them); batching
// separates the phases and keeps the write phase short against the barrier.
// Tiles are contiguous.
//   Ring and hierarchical all-reduce (every output): the tiles interleave in
// runs as in k_phase, and the write phase goes output by output for all K
// tiles.
// The barrier orders nothing the results depend on, as in k_phase.
template <class E, class OP, int P, int U, int K, FoldMode M>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void k_phase_batch(PhaseArgs a) {
  using S = typename E::S;
  using A = typename E::A;
  constexpr int V = 16 / sizeof(S);
  constexpr uint32_t kTile = kBlock * U;
  static_assert(M == FoldMode::kRingShard || M == FoldMode::kAscOne || writes_all(M),
                "batched rounds: reduce-scatter, reduce, the ring and the hierarchical all-reduces");
  constexpr bool IL = writes_all(M);
  // WB: the workgroups meet again between a round's write phase and the
  // next round's read phase (the folds that write every rank).
  constexpr bool WB = writes_all(M);
  const int p = P > 0 ? P : a.f.p;
  sync_claim(a);
  for (uint32_t r = 0; r < a.rounds; ++r) {
    A acc[K][U][V];
    int seg[K];
    uint32_t valid[K];
    uint32_t gap[K];
    uint64_t off[K];
    uint64_t lo[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t t = (r * K + j) * gridDim.x + blockIdx.x;
      seg[j] = 0;
      valid[j] = 0;
      gap[j] = 0;
      off[j] = 0;
      lo[j] = 0;
      if (t < a.tiles) {
        uint32_t k;
        if (a.uniform_tiles) {
          seg[j] = static_cast<int>(t / a.uniform_tiles);
          k = t - static_cast<uint32_t>(seg[j]) * a.uniform_tiles;
          valid[j] = (k + 1 == a.uniform_tiles) ? a.uniform_last : kTile;
          if constexpr (uses_bounds(M)) lo[j] = static_cast<uint64_t>(seg[j]) * a.seg_len;
        } else {
          int sg = 0;
          while (a.seg_tile[sg + 1] <= t) ++sg;
          seg[j] = sg;
          k = t - a.seg_tile[sg];
          valid[j] = (k + 1 == a.seg_tile[sg + 1] - a.seg_tile[sg]) ? a.seg_last[sg] : kTile;
          if constexpr (uses_bounds(M)) lo[j] = a.f.bound[sg];
        }
        uint64_t gk = static_cast<uint64_t>(k) * kTile;  // the tile's first group in the segment
        if constexpr (IL) {
          if (a.strips > 1 && k < a.strip_tiles) {
            const uint32_t run = k / a.strips;
            const uint32_t jj = k - run * a.strips;
            gk = static_cast<uint64_t>(run) * a.strips * kTile + jj * kBlock;
            gap[j] = (a.strips - 1) * kBlock;
          }
        }
        off[j] = ((lo[j] + V - 1) / V + gk) * 16;
        read_fold<E, OP, P, U, M, IL>(a.f, seg[j], p, off[j], valid[j], gap[j], acc[j]);
      }
    }
    soft_barrier(a, WB ? 2 * r : r);
    Raw<E, V> o[K][U];
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) pack(acc[j][u], o[j][u]);
    if constexpr (writes_all(M)) {
      for (int q = 0; q < p; ++q) {
        char* d = static_cast<char*>(a.f.out[q]);
#pragma unroll
        for (int j = 0; j < K; ++j) {
          if (valid[j] == kTile) {
            store_tile<false, IL>(d + off[j], o[j], valid[j], gap[j]);
          } else if (valid[j] != 0) {
            store_tile<true, IL>(d + off[j], o[j], valid[j], gap[j]);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        if (valid[j] == 0) continue;
        // reduce-scatter outputs hold only the chunk: group g sits at g*V - lo
        const uint64_t shift = (M == FoldMode::kRingShard) ? lo[j] * sizeof(S) : 0;
        char* d = static_cast<char*>(a.f.out[seg[j]]) + (off[j] - shift);
        if (valid[j] == kTile) {
          store_tile<false, false>(d, o[j], valid[j], 0);
        } else {
          store_tile<true, false>(d, o[j], valid[j], 0);
        }
      }
    }
    if constexpr (WB) {
      if (r + 1 < a.rounds) soft_barrier(a, 2 * r + 1);
    }
  }
}

// Heads and tails of the segments (fewer than V elements each), in the same
// fold order: one workgroup per segment, 2V lanes.  Launched only when a
// segment has any, after the phased fold on the same stream; the elements are
// disjoint from the phased fold's groups.
template <class E, class OP, FoldMode M>
__global__ __launch_bounds__(64) void k_edges(PhaseArgs a) {
  constexpr int V = 16 / sizeof(typename E::S);
  const int seg = blockIdx.x;
  const int p = a.f.p;
  uint64_t lo = 0;
  uint64_t hi = a.f.n;
  if constexpr (uses_bounds(M)) {
    lo = a.f.bound[seg];
    hi = a.f.bound[seg + 1];
  }
  const uint32_t lane = threadIdx.x;
  if (lane < V) {
    if (lane < a.head_len[seg]) fold_scalar<E, E, OP, M>(a.f, lo + lane, lo, seg, p);
  } else if (lane < 2 * V && lane - V < a.tail_len[seg]) {
    fold_scalar<E, E, OP, M>(a.f, hi - a.tail_len[seg] + (lane - V), lo, seg, p);
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch of one mode's kernels.

// Launch `kernel`, or, when occ is not NULL, only report how many of its
// workgroups fit on one compute unit at once.
template <class K>
hipError_t phase_go(K kernel, const PhaseArgs& a, unsigned grid, unsigned block, int* occ, hipStream_t s) {
  if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, reinterpret_cast<const void*>(kernel), block, 0);
  PhaseArgs copy = a;
  void* kp[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block), kp, 0, s);
}

template <class E, FoldMode M>
constexpr int phase_unroll() {
  return (is_hier(M) && sizeof(typename E::S) == 2) ? 4 : 8;
}

template <class E, class OP, int P, FoldMode M, bool SYNC>
hipError_t phase_by_u(const PhaseArgs& a, unsigned grid, int unroll, int* occ, hipStream_t s) {
  constexpr int kU = phase_unroll<E, M>();
  if (unroll == kU) return phase_go(&k_phase<E, OP, P, kU, M, SYNC>, a, grid, kBlock, occ, s);
  // the smaller tiles: for sums in every mode, for every op in the modes
  // whose schedule uses them (ring all-reduce, reduce-scatter, reduce)
  constexpr bool kSmall = __is_same(OP, OpSum) || __is_same(OP, OpAvg) || M == FoldMode::kRingAll ||
                          M == FoldMode::kRingShard || M == FoldMode::kAscOne;
  if constexpr (kSmall && kU != 4) {
    if (unroll == 4) return phase_go(&k_phase<E, OP, P, 4, M, SYNC>, a, grid, kBlock, occ, s);
    // launches too small for a tile of 4 groups per lane on every CU (ring
    // all-reduce in one round, reduce-scatter, reduce)
    if constexpr ((M == FoldMode::kRingAll || M == FoldMode::kRingShard || M == FoldMode::kAscOne) && !SYNC) {
      if (unroll == 2) return phase_go(&k_phase<E, OP, P, 2, M, false>, a, grid, kBlock, occ, s);
      if (unroll == 1) return phase_go(&k_phase<E, OP, P, 1, M, false>, a, grid, kBlock, occ, s);
    }
  }
  return hipErrorInvalidValue;
}

// p = 8 (the rank count of the workloads) is compiled with its rotated
// pointers in registers; every other p takes the run-time loop.
template <class E, class OP, FoldMode M>
hipError_t phase_by_p(const PhaseArgs& a, unsigned grid, int unroll, bool sync, bool static_p, int* occ,
                      hipStream_t s) {
  hipError_t e;
  // the hierarchical variants are compiled with the run-time loop only
  constexpr bool kStatic = M == FoldMode::kRingAll || M == FoldMode::kHierAll || M == FoldMode::kRingShard ||
                           M == FoldMode::kAscOne;
  // reduce-scatter and reduce are compiled without the barrier
  constexpr bool kSync = writes_all(M);
  if (kStatic && static_p && a.f.p == 8) {
    e = (kSync && sync) ? phase_by_u<E, OP, kStatic ? 8 : 0, M, kSync>(a, grid, unroll, occ, s)
                        : phase_by_u<E, OP, kStatic ? 8 : 0, M, false>(a, grid, unroll, occ, s);
  } else {
    e = (kSync && sync) ? phase_by_u<E, OP, 0, M, kSync>(a, grid, unroll, occ, s)
                        : phase_by_u<E, OP, 0, M, false>(a, grid, unroll, occ, s);
  }
  if (e != hipSuccess || occ || !a.edges) return e;
  return phase_go(&k_edges<E, OP, M>, a, static_cast<unsigned>(a.segments), 64, nullptr, s);
}

template <class E, FoldMode M>
hipError_t phase_by_op(const PhaseArgs& a, rr_op_t op, unsigned grid, int unroll, bool sync, bool static_p,
                       int* occ, hipStream_t s) {
  switch (op) {
    case RR_SUM: return phase_by_p<E, OpSum, M>(a, grid, unroll, sync, static_p, occ, s);
    case RR_MAX: return phase_by_p<E, OpMax, M>(a, grid, unroll, sync, static_p, occ, s);
    case RR_MIN: return phase_by_p<E, OpMin, M>(a, grid, unroll, sync, static_p, occ, s);
    case RR_AVG:
      if constexpr (__is_same(typename E::A, float)) return phase_by_p<E, OpAvg, M>(a, grid, unroll, sync, static_p,
                                                                                      occ, s);
      break;
  }
  return hipErrorInvalidValue;
}

template <FoldMode M>
hipError_t phase_dispatch(const PhaseArgs& a, Kind k, rr_op_t op, unsigned grid, int unroll, bool sync,
                          bool static_p, int* occ, hipStream_t s) {
  if (sync && occ == nullptr && a.captured) {
    // this translation unit's counters, cleared on the same stream first
    SyncArgs y{};
    y.slot = a.slot;
    y.captured = 1;
    const hipError_t e = sync_reset_if_captured(y, s);
    if (e != hipSuccess) return e;
  }
  if constexpr (!is_wire(M)) {
    if (k == Kind::kI32) return phase_by_op<EI32, M>(a, op, grid, unroll, sync, static_p, occ, s);
    if (k == Kind::kF32) return phase_by_op<EF32, M>(a, op, grid, unroll, sync, static_p, occ, s);
  }
  // (rounding a partial to a 4-byte storage type changes nothing: the wire
  // modes exist for the 16-bit kinds only)
  if (k == Kind::kBF16) return phase_by_op<EBF16, M>(a, op, grid, unroll, sync, static_p, occ, s);
  if (k == Kind::kF16) return phase_by_op<EF16, M>(a, op, grid, unroll, sync, static_p, occ, s);
  return hipErrorInvalidValue;
}

// The batched one-output kernels: K tiles of 4 groups per lane per round.
template <class E, class OP, FoldMode M>
hipError_t batch_by_p(const PhaseArgs& a, unsigned grid, int K, bool static_p, int* occ, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  bool launched = false;
  // binary16 takes the run-time rank loop only: with all p = 8 ranks
  // unrolled its conversions are hoisted past 256 registers and spill; the
  // hierarchy (two accumulators per value) too
  if constexpr (!__is_same(E, EF16) && !is_hier(M)) {
    if (static_p && a.f.p == 8) {
      e = K == 2 ? phase_go(&k_phase_batch<E, OP, 8, 4, 2, M>, a, grid, kBlock, occ, s)
                 : phase_go(&k_phase_batch<E, OP, 8, 4, 4, M>, a, grid, kBlock, occ, s);
      launched = true;
    }
  }
  if (!launched) {
    e = K == 2 ? phase_go(&k_phase_batch<E, OP, 0, 4, 2, M>, a, grid, kBlock, occ, s)
               : phase_go(&k_phase_batch<E, OP, 0, 4, 4, M>, a, grid, kBlock, occ, s);
  }
  if (e != hipSuccess || occ || !a.edges) return e;
  return phase_go(&k_edges<E, OP, M>, a, static_cast<unsigned>(a.segments), 64, nullptr, s);
}

template <class E, FoldMode M>
hipError_t batch_by_op(const PhaseArgs& a, rr_op_t op, unsigned grid, int K, bool static_p, int* occ,
                       hipStream_t s) {
  switch (op) {
    case RR_SUM: return batch_by_p<E, OpSum, M>(a, grid, K, static_p, occ, s);
    case RR_MAX: return batch_by_p<E, OpMax, M>(a, grid, K, static_p, occ, s);
    case RR_MIN: return batch_by_p<E, OpMin, M>(a, grid, K, static_p, occ, s);
    case RR_AVG:
      if constexpr (__is_same(typename E::A, float)) return batch_by_p<E, OpAvg, M>(a, grid, K, static_p, occ, s);
      break;
  }
  return hipErrorInvalidValue;
}

template <FoldMode M>
hipError_t batch_dispatch(const PhaseArgs& a, Kind k, rr_op_t op, unsigned grid, int K, bool static_p, int* occ,
                          hipStream_t s) {
  if (occ == nullptr && a.captured) {
    // this translation unit's counters, cleared on the same stream first
    SyncArgs y{};
    y.slot = a.slot;
    y.captured = 1;
    const hipError_t e = sync_reset_if_captured(y, s);
    if (e != hipSuccess) return e;
  }
  switch (k) {
    case Kind::kI32: return batch_by_op<EI32, M>(a, op, grid, K, static_p, occ, s);
    case Kind::kF32: return batch_by_op<EF32, M>(a, op, grid, K, static_p, occ, s);
    case Kind::kBF16: return batch_by_op<EBF16, M>(a, op, grid, K, static_p, occ, s);
    case Kind::kF16: return batch_by_op<EF16, M>(a, op, grid, K, static_p, occ, s);
  }
  return hipErrorInvalidValue;
}

// Single-pass fold for the hierarchical variants (unaligned buffers): the
// run-time-p kernel of rr_fold_impl.h.
template <FoldMode M>
hipError_t fold_var_dispatch(const FoldLaunch& f, hipStream_t s) {
  if (f.in_kind != f.out_kind) return hipErrorInvalidValue;
  if constexpr (!is_wire(M)) {
    if (f.in_kind == Kind::kI32) {
      switch (f.op) {
        case RR_SUM: return fold_go<EI32, EI32, OpSum, 0, 2, false, M>(f, s);
        case RR_MAX: return fold_go<EI32, EI32, OpMax, 0, 2, false, M>(f, s);
        case RR_MIN: return fold_go<EI32, EI32, OpMin, 0, 2, false, M>(f, s);
        default: return hipErrorInvalidValue;
      }
    }
    if (f.in_kind == Kind::kF32) return fold_mixed_by_op<EF32, EF32, M>(f, s);
  }
  if (f.in_kind == Kind::kBF16) return fold_mixed_by_op<EBF16, EBF16, M>(f, s);
  if (f.in_kind == Kind::kF16) return fold_mixed_by_op<EF16, EF16, M>(f, s);
  return hipErrorInvalidValue;
}

}  // namespace

}  // namespace rr
