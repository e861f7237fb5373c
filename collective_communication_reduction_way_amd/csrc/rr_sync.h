// rr_sync.h -- the soft grid barrier between the read phase and the write
// phase of a round, and between the rounds (gfx950), shared by the phased
// fold (rr_phase_impl.h) and the bucketed all-reduce (rr_multi.hip).
// Internal header.
//
// Per slot, kSyncSubs arrival counters and one top counter, each a 64-bit
// word on its own 128-byte line.  Workgroup b arrives on counter
// b % kSyncSubs (so the arrivals do not all contend for one line); the last
// arrival of a counter in a round bumps the top counter, and the waiters poll
// only the top counter.  Every counter holds (launch tag << kLaunchShift) +
// count: each launch carries a fresh, larger tag and claims a counter with an
// atomic max before counting on it, which discards whatever older launches
// left there without any reset.  A launch captured into a graph carries the
// fixed kCapturedTag instead and a reset kernel (k_sync_reset) is captured
// ahead of it.  The barrier orders nothing that results depend on, so every
// wait is bounded by a wall-clock timeout and a workgroup that times out goes
// on (and is counted).  All atomics are relaxed at device scope.
//
// The counters and the timeout count are per translation unit (and per
// device), zero when the code object loads; slots are assigned per stream by
// the host (phase_sync_args), so launches that may run concurrently count on
// different words.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_phase.h"

namespace rr {

namespace {

__device__ __align__(256) unsigned long long g_sync[kSyncSlots * kSyncCounters * kSyncStride];
__device__ unsigned long long g_sync_timeouts;

__device__ __forceinline__ unsigned long long* sync_counter(uint32_t slot, uint32_t i) {
  return g_sync + (static_cast<size_t>(slot) * kSyncCounters + i) * kSyncStride;
}

__device__ __forceinline__ unsigned long long atomic_add_relaxed(unsigned long long* p, unsigned long long v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void atomic_max_relaxed(unsigned long long* p, unsigned long long v) {
  __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Claim this workgroup's arrival counter for the launch (once, at the start).
__device__ __forceinline__ void sync_claim_at(uint32_t slot, unsigned long long tag) {
  if (threadIdx.x == 0) atomic_max_relaxed(sync_counter(slot, blockIdx.x % kSyncSubs), tag);
}

// Clear one slot's counters: captured ahead of a launch whose tag is fixed
// (graph replays), so that every replay counts from zero like an eager
// launch with a fresh tag.
__global__ __launch_bounds__(64) void k_sync_reset(uint32_t slot) {
  if (threadIdx.x < static_cast<uint32_t>(kSyncCounters))
    __hip_atomic_store(sync_counter(slot, threadIdx.x), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrive at barrier number `round` of the launch (0, 1, 2, ... in order: one
// or two per round of the kernel) and wait (bounded) until all G workgroups
// have.
__device__ __forceinline__ void soft_barrier_at(uint32_t slot, unsigned long long tag, uint32_t timeout_ticks,
                                                uint32_t round) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t G = gridDim.x;
    const uint32_t sub = blockIdx.x % kSyncSubs;
    const uint32_t nsub = G < kSyncSubs ? G : kSyncSubs;
    const uint32_t per = G / kSyncSubs + (sub < G % kSyncSubs ? 1u : 0u);  // workgroups on this counter
    unsigned long long* top = sync_counter(slot, kSyncSubs);
    const unsigned long long seen = atomic_add_relaxed(sync_counter(slot, sub), 1ull) + 1 - tag;
    if (seen == static_cast<unsigned long long>(round + 1) * per) {
      // the top counter is claimed for the launch by the first completion of
      // every sub-counter (round 0); later rounds find it claimed, and the
      // claim would only add a serial atomic to the barrier's critical path
      if (round == 0) atomic_max_relaxed(top, tag);
      atomic_add_relaxed(top, 1ull);
    }
    const unsigned long long target = tag + static_cast<unsigned long long>(round + 1) * nsub;
    const uint64_t t0 = wall_clock64();
    // Every waiting workgroup polls the one top line; a pause of 8 x 64
    // clocks between polls eases that line for the increments the waiters
    // wait for (sleep 2 / 4 / 8 / 16 / 32: 96 MiB fp32 all-reduce 76.0 /
    // 76.3 / 76.4 / 76.2 / 75.1%, 128 MiB bf16 77.7 / 77.9 / 78.0 / 77.6 /
    // 76.1%, the same machine).
    while (__hip_atomic_load(top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(8);
      if (wall_clock64() - t0 > timeout_ticks) {
        atomic_add_relaxed(&g_sync_timeouts, 1ull);
        break;
      }
    }
  }
  __syncthreads();
}

// Host: capture the reset of this unit's counters of `slot` on `s` when the
// launch that follows is being captured (SyncArgs::captured).
inline hipError_t sync_reset_if_captured(const SyncArgs& y, hipStream_t s) {
  if (!y.captured) return hipSuccess;
  uint32_t slot = y.slot;
  void* kp[] = {&slot};
  return hipLaunchKernel(reinterpret_cast<const void*>(&k_sync_reset), dim3(1), dim3(64), kp, 0, s);
}

// Host: this unit's barrier timeouts on the current device.
inline hipError_t sync_timeouts_here(unsigned long long* count) {
  return hipMemcpyFromSymbol(count, HIP_SYMBOL(g_sync_timeouts), sizeof(*count), 0, hipMemcpyDeviceToHost);
}

}  // namespace

}  // namespace rr
