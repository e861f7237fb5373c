// rr_exec.hip -- the ring schedule executed by one persistent kernel (gfx950).
//
// Page "LLM Parallelism 基础", section "Ring AllReduce": p-1 reduce-scatter
// steps in which every rank passes one chunk to the next rank, which
// accumulates it, then p-1 all-gather steps in which the next rank
// overwrites its copy.  The staged algorithm runs each step as a launch of
// its own; here one launch runs them all, the ranks advancing independently
// and handing chunks on through completion flags in device memory -- the
// structure a multi-GPU ring has, with the rank buffers playing the part of
// peer memory.
//
// Workers.  The workgroups are (slice b, rank q) pairs, slice-major.  Every
// chunk is cut into B slices; worker (b, q) performs rank q's side of every
// step for slice b of the chunk that step moves.  Workers of different
// slices never wait for each other.
//
// Steps of worker (b, q), with r = q-1 mod p the ring predecessor:
//   t = 1..p-1     reduce-scatter step s = t-1: chunk c = (r-1-s) mod p,
//                  work[q] = m (+) in[q] on slice b, the message m first (the
//                  receiver of the ring accumulates): m is r's input in step
//                  0 and work[r], the partial sum r wrote in step s-1, after
//                  that; q's own contribution is read from its input, where
//                  it still is.  The last step completes chunk q and writes
//                  it finished (AVG's division, the one rounding of 16-bit
//                  types) to q's output instead of work[q].  The working
//                  buffers are float32 for 16-bit types, else the outputs.
//   t = p..2p-2    all-gather step s = t-p: chunk c = (r-s) mod p,
//                  out[q] = out[r] on slice b.
// Step 0 of the ring (each rank's own copy) moves nothing: step 1 reads the
// inputs.  flag[q][b] = t + 1 once worker (b, q) has completed step t.  Step
// t >= 2 of (b, q) reads what (b, r) wrote in step t-1, so it waits for
// flag[r][b] >= t.  All-gather step s overwrites chunk r-s of q's output,
// which (b, q+1) read in reduce-scatter step s when the outputs are the
// working buffers (4-byte types), and in step 0 (s = 0) when q runs in
// place, so it then also waits for flag[q+1][b] >= s+2.  Every wait points
// to an earlier step, so the waits form no cycle.  p = 1 is one copy.
//
// Memory ordering.  The flags order data between workgroups that may run on
// different XCDs, each with its own L2.  The slices are laid out so that a
// slice's p workers are workgroups congruent modulo the XCD count, which the
// dispatcher places on one XCD when it deals workgroups to the XCDs in turn.
// This is checked, not assumed: at the start each worker publishes the XCD it
// runs on (tagged with the launch) and reads its slice's p entries.  When they
// all agree, the slice exchanges data inside one L2, coherent for its CUs: a
// step is published once every wave's stores are acknowledged by the L2
// (s_waitcnt 0, barrier) and the flag is raised, with no write-back, and the
// waiter takes no fence.  What remains is each CU's own L1, which the other
// CUs' stores do not update: a read must not be served by a line the CU
// cached before the data changed.  Within a launch only all-gather steps
// repeat a read of an address on a CU: with the outputs as working buffers
// (4-byte kinds), step s >= 1 reads predecessor chunks that a reduce-scatter
// step read while they held partial sums; in place, step 1 reads the chunk
// that reduce-scatter step 0 read as input.  Those copies use device-scope
// loads (sc1), served by the L2 around the L1.  A probe on MI355X settled which
// forms work: two CUs of one XCD exchanging one 4 KiB region 2000 times read
// the previous value in 99.95% of the words with plain loads, with or
// without the workgroup-scope invalidation (buffer_inv sc0, which leaves the
// L1 alone in this mode), and in none with device-scope loads or after the
// agent-scope acquire (buffer_inv sc1).  An acquire before every step
// instead costs 25% at 8 MiB per rank.  A slice whose workers are not all on
// one XCD publishes a step as follows: every wave waits until its stores are
// acknowledged by the L2 (s_waitcnt 0), the workgroup meets at a barrier, and
// thread 0 takes an agent-scope release fence -- on gfx950 an L2 write-back of the whole XCD's L2 (buffer_wbl2 sc1), which therefore
// covers every wave's stores -- before it raises the flag.  A waiter's
// thread 0 sees the flag and takes an agent-scope acquire fence, which
// invalidates the CU's L1 and the XCD's L2 for every wave (buffer_inv sc1),
// before the workgroup barrier that releases the readers.  One write-back
// and one invalidation per workgroup and step: a fence in every thread
// measured five times slower (each write-back walks the L2).
//
// Flags hold (launch tag << 24) + steps; each launch has a fresh, larger tag
// and raises flags with atomic max, so nothing needs resetting -- except
// under graph capture: a graph replays its kernel arguments unchanged, so a
// captured launch carries the fixed tag 1 (eager launches use 2, 3, ...)
// and a reset of the slot's flags and abort word is captured just before it.
// Without it, a replay would find the previous replay's flags already at
// their final values and read chunks before they are written.  The reset
// clears the placement words too.  Every wait
// is bounded by a wall-clock timeout; a worker that times out (workers not
// all resident, for instance) raises the slot's abort word, counts the
// failure and stops, and every other waiter of the launch stops as soon as
// it sees the abort word.  A failed launch leaves its outputs incomplete;
// rr_ring_exec_failures() reports it.  The host caps the grid at what the
// device keeps resident, and workgroups are dispatched in order, so a slice's
// workers start together.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>

#include "rr_device.h"
#include "rr_kernels.h"

namespace rr {

namespace {

constexpr int kExecStreamSlots = 16;  // slots [0, 16): one per stream with launches in flight
constexpr int kExecSlots = 64;        // slots [16, 64): one per launch captured into a graph
constexpr int kExecMaxWorkers = 2048;  // p * B per launch
constexpr int kExecStride = 8;         // 64-bit words: one 64-byte line per flag
constexpr int kExecShift = 24;         // flag = (tag << 24) + steps
constexpr unsigned long long kExecCapturedTag = 1ull << kExecShift;
constexpr int kExecXcds = 8;           // XCDs of an MI355X (the placement is checked at run time)

__device__ __align__(256) unsigned long long g_exec_flags[kExecSlots * kExecMaxWorkers * kExecStride];
__device__ __align__(256) unsigned long long g_exec_abort[kExecSlots * 16];
// Placement of each worker, published at the start of a launch: tag + XCC id.
__device__ __align__(256) unsigned long long g_exec_place[kExecSlots * kExecMaxWorkers];
__device__ unsigned long long g_exec_failures;

__device__ __forceinline__ unsigned long long* exec_flag(uint32_t slot, int worker) {
  return g_exec_flags + (static_cast<size_t>(slot) * kExecMaxWorkers + worker) * kExecStride;
}

// Clear the flags of workers [0, workers) of a slot and its abort word
// (ahead of a captured launch).
__global__ __launch_bounds__(kBlock) void k_exec_reset(uint32_t slot, int workers) {
  for (int w = threadIdx.x; w < workers; w += kBlock) {
    __hip_atomic_store(exec_flag(slot, w), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(g_exec_place + static_cast<size_t>(slot) * kExecMaxWorkers + w, 0ull, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x == 0) __hip_atomic_store(g_exec_abort + slot * 16, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until *f >= target, the launch's abort word is raised, or the bound
// runs out.  Thread 0 only.  Returns false when the launch must stop.
__device__ bool wait_flag(const ExecArgs& a, const unsigned long long* f, unsigned long long target) {
  unsigned long long* abort_word = g_exec_abort + a.slot * 16;
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (__hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= a.tag) return false;
    __builtin_amdgcn_s_sleep(1);
    if (wall_clock64() - t0 > a.timeout_ticks) {
      // the first worker to give up on this launch counts it
      const unsigned long long was = __hip_atomic_fetch_max(abort_word, a.tag, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
      if (was < a.tag) __hip_atomic_fetch_add(&g_exec_failures, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
  return true;
}

// The XCC (XCD) this wave runs on.
__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xFu;  // HW_REG_XCC_ID, bits 0-3
}

// Apply `f` to the elements [e0, e1) of a slice: whole U-element units where
// every buffer involved is 16-byte aligned (vec), single elements elsewhere.
template <int U, class FV, class FS>
__device__ __forceinline__ void for_slice(uint64_t e0, uint64_t e1, bool vec, FV&& fv, FS&& fs) {
  const uint32_t lane = threadIdx.x;
  uint64_t u0 = e1, u1 = e1;
  if (vec) {
    u0 = (e0 + U - 1) / U * U;
    u1 = e1 / U * U;
    if (u1 < u0) u0 = u1 = e1;
  }
  for (uint64_t i = e0 + lane; i < (vec ? u0 : e1); i += kBlock) fs(i);
  for (uint64_t g = u0 / U + lane; g < u1 / U; g += kBlock) fv(g * U);
  for (uint64_t i = u1 + lane; i < e1; i += kBlock) fs(i);
}

// Copy the elements [e0, e1) of a slice from src to dst: 16-byte words where
// both buffers are 16-byte aligned (vec), kCopyBatch words per lane and pass
// at a distance of one workgroup, all loaded before the first is stored
// (every wave access is 1 KiB of consecutive bytes); single elements
// elsewhere.  COHERENT (slices under 4 GiB): every load is device-scope
// (sc1), served by the XCD's L2 around the CU's L1.
constexpr int kCopyBatch = 8;
template <bool COHERENT, class S>
__device__ __forceinline__ void copy_slice(const S* src, S* dst, uint64_t e0, uint64_t e1, bool vec) {
  constexpr int W = 16 / static_cast<int>(sizeof(S));
  const uint32_t lane = threadIdx.x;
  uint64_t u0 = e1, u1 = e1;
  if (vec) {
    u0 = (e0 + W - 1) / W * W;
    u1 = e1 / W * W;
    if (u1 < u0) u0 = u1 = e1;
  }
  // COHERENT: a raw buffer over the slice (0x00020000: the gfx9 descriptor
  // word 3 for untyped 32-bit accesses); unused otherwise
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<S*>(src + e0), 0, static_cast<int>(static_cast<uint32_t>((e1 - e0) * sizeof(S))), 0x00020000);
  auto one = [&](uint64_t i) {
    if constexpr (COHERENT) {
      using B = std::conditional_t<sizeof(S) == 4, uint32_t, uint16_t>;
      const B v = __hip_atomic_load(reinterpret_cast<const B*>(src + i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      reinterpret_cast<B*>(dst)[i] = v;
    } else {
      dst[i] = src[i];
    }
  };
  auto word = [&](uint64_t g) -> u32x4 {
    if constexpr (COHERENT) {
      return __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>((g * W - e0) * sizeof(S)), 0, 16);
    } else {
      return reinterpret_cast<const u32x4*>(src)[g];
    }
  };
  for (uint64_t i = e0 + lane; i < (vec ? u0 : e1); i += kBlock) one(i);
  const uint64_t g1 = u1 / W;
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  for (uint64_t g0 = u0 / W + lane; g0 < g1; g0 += kCopyBatch * kBlock) {
    u32x4 x[kCopyBatch];
#pragma unroll
    for (int j = 0; j < kCopyBatch; ++j)
      if (g0 + j * kBlock < g1) x[j] = word(g0 + j * kBlock);
#pragma unroll
    for (int j = 0; j < kCopyBatch; ++j)
      if (g0 + j * kBlock < g1) d[g0 + j * kBlock] = x[j];
  }
  for (uint64_t i = u1 + lane; i < e1; i += kBlock) one(i);
}

// dst = msg (+) own on the elements [e0, e1) of a slice, the message first;
// FINISH: then the op's last step (AVG's division) before the conversion to
// dst's kind.  The kinds share one accumulator type.  8-element units,
// kFoldBatch per lane and pass at a distance of one workgroup, all loaded
// before the first is folded and stored.
constexpr int kFoldBatch = 4;
template <class EM, class EO, class ED, class OP, bool FINISH>
__device__ __forceinline__ void fold_step(const typename EM::S* msg, const typename EO::S* own, typename ED::S* dst,
                                          uint64_t e0, uint64_t e1, bool vec, int32_t div) {
  using A = typename ED::A;
  constexpr int U = 8;
  const uint32_t lane = threadIdx.x;
  uint64_t u0 = e1, u1 = e1;
  if (vec) {
    u0 = (e0 + U - 1) / U * U;
    u1 = e1 / U * U;
    if (u1 < u0) u0 = u1 = e1;
  }
  auto one = [&](uint64_t i) {
    A v = OP::apply(load_one<EM>(msg + i), load_one<EO>(own + i));
    if constexpr (FINISH) v = op_finish<OP>(v, div);
    store_one<ED>(dst + i, v);
  };
  for (uint64_t i = e0 + lane; i < (vec ? u0 : e1); i += kBlock) one(i);
  const uint64_t g1 = u1 / U;
  for (uint64_t g0 = u0 / U + lane; g0 < g1; g0 += kFoldBatch * kBlock) {
    Raw<EM, U> m[kFoldBatch];
    Raw<EO, U> l[kFoldBatch];
#pragma unroll
    for (int j = 0; j < kFoldBatch; ++j) {
      if (g0 + j * kBlock < g1) {
        load_group<false>(m[j], msg + (g0 + j * kBlock) * U);
        load_group<false>(l[j], own + (g0 + j * kBlock) * U);
      }
    }
#pragma unroll
    for (int j = 0; j < kFoldBatch; ++j) {
      if (g0 + j * kBlock < g1) {
        A vm[U], vl[U];
        unpack(m[j], vm);
        unpack(l[j], vl);
#pragma unroll
        for (int k = 0; k < U; ++k) {
          vm[k] = OP::apply(vm[k], vl[k]);
          if constexpr (FINISH) vm[k] = op_finish<OP>(vm[k], div);
        }
        Raw<ED, U> o;
        pack(vm, o);
        store_group<false>(dst + (g0 + j * kBlock) * U, o);
      }
    }
  }
  for (uint64_t i = u1 + lane; i < e1; i += kBlock) one(i);
}

// E: storage kind; EA: accumulator kind of the working buffers.
template <class E, class EA, class OP>
__global__ __launch_bounds__(kBlock) void k_ring_exec(ExecArgs a) {
  using S = typename E::S;
  using SA = typename EA::S;
  using A = typename E::A;
  const int p = a.p;
  // worker (slice b, rank q).  With a.xcds > 0 the p workers of a slice are
  // workgroups congruent mod a.xcds: one XCD each when the dispatcher deals
  // workgroups to the XCDs in turn (checked below, not assumed).
  int b, q;
  if (a.xcds > 0) {
    const int j = static_cast<int>(blockIdx.x) / a.xcds;
    const int jb = j / p;
    b = jb * a.xcds + (static_cast<int>(blockIdx.x) - j * a.xcds);
    q = j - jb * p;
  } else {
    b = blockIdx.x / p;
    q = blockIdx.x - b * p;
  }
  const int r = q == 0 ? p - 1 : q - 1;
  const int nx = q + 1 == p ? 0 : q + 1;
  const bool vec = a.vec != 0;
  constexpr bool kSeparate = !__is_same(E, EA);  // working buffers apart from the outputs
  constexpr int U = 8;  // elements per unit of a lane
  __shared__ int go;
  __shared__ int local;  // 1: every worker of the slice runs on this XCD
  auto slice_lo = [&](int c) {
    const uint64_t len = a.bound[c + 1] - a.bound[c];
    return a.bound[c] + len * static_cast<uint64_t>(b) / static_cast<uint64_t>(a.nslices);
  };
  auto slice_hi = [&](int c) {
    const uint64_t len = a.bound[c + 1] - a.bound[c];
    return a.bound[c] + len * static_cast<uint64_t>(b + 1) / static_cast<uint64_t>(a.nslices);
  };
  // Step t re-reads addresses that this worker read before in the launch
  // (the predecessor's output; its L1 lines may be stale): with the outputs
  // as working buffers, all-gather steps s >= 1 read chunks that a
  // reduce-scatter step read while they held partial sums; in place, all-
  // gather step 1 reads the chunk that step 0 read as the predecessor's
  // input.  No other read in a launch repeats an address on one CU: a
  // slice's data crosses only between the p workers of that slice, and
  // slices that share an XCD are never adjacent (no shared cache lines).
  auto reread = [&](int t) { return kSeparate ? t == p + 1 && a.in[r] == a.out[r] : t >= p + 1; };
  auto coherent_fits = [&](int t) {
    int c = r - (t - p);
    while (c < 0) c += p;
    return (slice_hi(c) - slice_lo(c)) * sizeof(S) < (1ull << 32);
  };
  SA* wq = static_cast<SA*>(a.work[q]);
  if (threadIdx.x == 0) {
    // Placement: publish this worker's XCC, wait for the slice's p workers,
    // and take the XCD-local protocol only if they all share it.  Every
    // worker of a slice reads the same p words, so all take the same one.
    bool ok = true;
    bool same = a.xcds > 0;
    if (same) {
      unsigned long long* pl = g_exec_place + static_cast<size_t>(a.slot) * kExecMaxWorkers;
      const unsigned long long mine = xcc_id();
      __hip_atomic_store(pl + b * p + q, a.tag + mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int k = 0; k < p && ok; ++k) {
        ok = wait_flag(a, pl + b * p + k, a.tag);
        if (ok && __hip_atomic_load(pl + b * p + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.tag + mine)
          same = false;
      }
    }
    go = ok ? 1 : 0;
    local = same ? 1 : 0;
  }
  __syncthreads();
  if (!go) return;
  // p = 1: the output is the input, through the op's last step
  if (p == 1) {
    const S* in = static_cast<const S*>(a.in[0]);
    S* o = static_cast<S*>(a.out[0]);
    if (static_cast<const void*>(in) != static_cast<const void*>(o) || is_avg<OP>()) {
      for_slice<U>(
          slice_lo(0), slice_hi(0), vec,
          [&](uint64_t i) {
            Raw<E, U> x;
            load_group<false>(x, in + i);
            A v[U];
            unpack(x, v);
#pragma unroll
            for (int j = 0; j < U; ++j) v[j] = op_finish<OP>(v[j], a.div);
            pack(v, x);
            store_group<false>(o + i, x);
          },
          [&](uint64_t i) { store_one<E>(o + i, op_finish<OP>(load_one<E>(in + i), a.div)); });
    }
    return;
  }
  const bool in_place_q = a.in[q] == a.out[q];
  // Step t = 1 .. 2p-2 (step 0, a copy-in, moves nothing: the first
  // reduce-scatter step reads the inputs); flag = t + 1 once step t is done.
  for (int t = 1; t <= 2 * p - 2; ++t) {
    // wait for the predecessor's step t-1 (the inputs of step 1 are ready at
    // the launch), and before an all-gather overwrite of a buffer that the
    // successor reads, for that read: with the outputs as working buffers,
    // the partial sum it read in reduce-scatter step s; else, in place, the
    // input chunk it read in step 0
    if (t > 1) {
      if (threadIdx.x == 0) {
        bool ok = wait_flag(a, exec_flag(a.slot, b * p + r), a.tag + static_cast<unsigned long long>(t));
        if (ok && t >= p && (!kSeparate || (t == p && in_place_q)))
          ok = wait_flag(a, exec_flag(a.slot, b * p + nx), a.tag + static_cast<unsigned long long>(t - p + 2));
        // XCD-local slices need no acquire except where a re-read reads
        // around the CU's L1 and cannot (a slice of 4 GiB or more)
        if (ok && (!local || (reread(t) && !coherent_fits(t)))) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        go = ok ? 1 : 0;
      }
      __syncthreads();
      if (!go) return;
    }
    if (t < p) {
      // reduce-scatter step s: message (+) own chunk, the message first.
      // q's own contribution to chunk c is read from its input, where it
      // still is (q folds chunk c in this step only); the message is r's
      // input in step 0 and the partial sum r wrote in step s - 1 after
      // that.  The last step completes chunk q and finishes it into q's
      // output (AVG's division, the one rounding of 16-bit kinds).  Only q
      // writes its working buffer and its output, and an input that is also
      // the output is overwritten by q's all-gather step 0 only after the
      // successor's step-0 read (the wait above).
      const int s = t - 1;
      int c = r - 1 - s;
      while (c < 0) c += p;
      const uint64_t lo = slice_lo(c), hi = slice_hi(c);
      const S* own = static_cast<const S*>(a.in[q]);
      const bool first = s == 0, last = s == p - 2;
      if (first && last) {
        fold_step<E, E, E, OP, true>(static_cast<const S*>(a.in[r]), own, static_cast<S*>(a.out[q]), lo, hi, vec, a.div);
      } else if (first) {
        fold_step<E, E, EA, OP, false>(static_cast<const S*>(a.in[r]), own, wq, lo, hi, vec, a.div);
      } else if (last) {
        fold_step<EA, E, E, OP, true>(static_cast<const SA*>(a.work[r]), own, static_cast<S*>(a.out[q]), lo, hi, vec,
                                      a.div);
      } else {
        fold_step<EA, E, EA, OP, false>(static_cast<const SA*>(a.work[r]), own, wq, lo, hi, vec, a.div);
      }
    } else {
      // all-gather step s: rank q overwrites its copy of chunk c
      const int s = t - p;
      int c = r - s;
      while (c < 0) c += p;
      const S* orr = static_cast<const S*>(a.out[r]);
      S* oq = static_cast<S*>(a.out[q]);
      if (local && reread(t) && coherent_fits(t)) {
        copy_slice<true>(orr, oq, slice_lo(c), slice_hi(c), vec);
      } else {
        copy_slice<false>(orr, oq, slice_lo(c), slice_hi(c), vec);
      }
    }
    // publish step t: every wave's stores acknowledged, then one release
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      // XCD-local: the stores are in the XCD's L2 (acknowledged above), which
      // every worker of the slice reads; else write the L2 back for all XCDs
      if (!local) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_fetch_max(exec_flag(a.slot, b * p + q), a.tag + static_cast<unsigned long long>(t + 1),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: per-device launch tags, a slot per stream, the resident-grid cap.

constexpr int kMaxDevices = 64;

// A slot's flags belong to one stream at a time, or to one captured launch.
// `done` is recorded after the slot's last eager launch; once it has
// completed, no launch uses the slot any more and the next eager call
// returns it to the free list.  A launch captured into a graph takes a slot
// of its own and keeps it for the rest of the process (`graph`): replays may
// come at any time, on any stream, and two captured launches -- of one graph
// or of two, even when captured on the same stream -- must never share
// flags, since two graphs may be replayed at the same time.
struct ExecSlot {
  hipStream_t owner = nullptr;
  bool used = false;
  bool pinned = false;
  bool graph = false;
  hipEvent_t done = nullptr;
};

struct ExecDevice {
  std::once_flag once;
  int cus = 0;
  int wall_khz = 0;
  unsigned long long launches = 0;
  std::mutex mu;  // slots, tags and the launches that use them
  ExecSlot slots[kExecSlots];
  std::map<uint32_t, int> occupancy;
};

ExecDevice g_exec_dev[kMaxDevices];

// Return to the free list every slot whose last launch has completed.  Eager
// calls only: querying an event is not allowed while a stream is being
// captured.  Called with d.mu held.
void exec_release_done(ExecDevice& d) {
  for (ExecSlot& x : d.slots) {
    if (x.used && !x.pinned && x.done && hipEventQuery(x.done) == hipSuccess) {
      x.used = false;
      x.owner = nullptr;
    }
  }
}

// The slot of an eager launch on stream s: the stream's own, else a free one
// (after releasing the completed ones).  A captured launch always takes a
// free slot of its own, pinned to it.  -1 when none is free.  Called with
// d.mu held.
int exec_slot_for(ExecDevice& d, hipStream_t s, bool captured) {
  if (!captured) {
    for (int i = 0; i < kExecStreamSlots; ++i)
      if (d.slots[i].used && d.slots[i].owner == s) return i;
    exec_release_done(d);
  }
  for (int i = captured ? kExecStreamSlots : 0; i < (captured ? kExecSlots : kExecStreamSlots); ++i) {
    ExecSlot& x = d.slots[i];
    if (!x.used) {
      x.used = true;
      x.graph = captured;
      x.pinned = captured;
      x.owner = captured ? nullptr : s;
      return i;
    }
  }
  return -1;
}

template <class E, class EA, class OP>
hipError_t exec_go(ExecArgs a, int budget_per_cu_cap, int max_slices, int timeout_us, hipStream_t s, ExecDevice& d,
                   uint32_t key) {
  const void* kernel = reinterpret_cast<const void*>(&k_ring_exec<E, EA, OP>);
  int occ = 0;
  {
    std::lock_guard<std::mutex> lock(d.mu);
    auto it = d.occupancy.find(key);
    if (it != d.occupancy.end()) occ = it->second;
  }
  if (occ == 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kBlock, 0);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    std::lock_guard<std::mutex> lock(d.mu);
    d.occupancy[key] = occ;
  }
  if (budget_per_cu_cap > 0 && occ > budget_per_cu_cap) occ = budget_per_cu_cap;
  const int cus = d.cus > 0 ? d.cus : 256;
  // slices: as many as stay resident together, at most max_slices, at least 1
  int slices = (cus * occ) / a.p;
  if (slices > max_slices) slices = max_slices;
  if (slices * a.p > kExecMaxWorkers) slices = kExecMaxWorkers / a.p;
  // no slice shorter than one 8-element unit per lane of the smallest chunk
  uint64_t shortest = ~0ull;
  for (int c = 0; c < a.p; ++c) shortest = std::min<uint64_t>(shortest, a.bound[c + 1] - a.bound[c]);
  const uint64_t by_size = shortest / (8ull * kBlock) + 1;
  if (static_cast<uint64_t>(slices) > by_size) slices = static_cast<int>(by_size);
  if (slices < 1) slices = 1;
  // a multiple of the XCD count: the workers of each slice then share an XCD
  // when workgroups are dealt to the XCDs in turn (checked by the kernel)
  a.xcds = 0;
  if (slices >= kExecXcds) {
    slices -= slices % kExecXcds;
    a.xcds = kExecXcds;
  }
  a.nslices = slices;
  const uint64_t khz = d.wall_khz > 0 ? static_cast<uint64_t>(d.wall_khz) : 100000;
  uint64_t ticks = khz * static_cast<uint64_t>(timeout_us) / 1000;
  if (ticks < 1) ticks = 1;
  a.timeout_ticks = ticks;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return e;
  const bool captured = cs == hipStreamCaptureStatusActive;
  // The flags order data, so launches that may run at the same time (on
  // different streams) never share a slot.  The lock covers the choice of
  // the slot, the launch and the record of its completion event, so that no
  // other thread can take the slot in between.
  std::lock_guard<std::mutex> lock(d.mu);
  const int si = exec_slot_for(d, s, captured);
  if (si < 0) return hipErrorOutOfMemory;
  ExecSlot& slot = d.slots[si];
  a.slot = static_cast<uint32_t>(si);
  if (captured) {
    a.captured = 1;
    a.tag = kExecCapturedTag;
    uint32_t sl = a.slot;
    int workers = slices * a.p;
    void* rp[] = {&sl, &workers};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&k_exec_reset), dim3(1), dim3(kBlock), rp, 0, s);
    if (e != hipSuccess) return e;
  } else {
    const unsigned long long id = ++d.launches + 1;  // 2, 3, ...: 1 belongs to captured launches
    a.tag = (id & ((1ull << (64 - kExecShift)) - 1)) << kExecShift;
    if (a.tag <= kExecCapturedTag) a.tag = 2 * kExecCapturedTag;
  }
  void* kp[] = {&a};
  e = hipLaunchKernel(kernel, dim3(static_cast<unsigned>(slices * a.p)), dim3(kBlock), kp, 0, s);
  if (e != hipSuccess || captured) return e;
  // the completion event lets the slot pass to another stream later; if it
  // cannot be recorded, the slot simply stays with this stream
  if (!slot.done && hipEventCreateWithFlags(&slot.done, hipEventDisableTiming) != hipSuccess) slot.done = nullptr;
  if (!slot.done || hipEventRecord(slot.done, s) != hipSuccess) slot.pinned = true;
  return hipSuccess;
}

template <class E, class EA>
hipError_t exec_by_op(const ExecArgs& a, rr_op_t op, int cap, int ms, int timeout_us, hipStream_t s, ExecDevice& d,
                      uint32_t key) {
  switch (op) {
    case RR_SUM: return exec_go<E, EA, OpSum>(a, cap, ms, timeout_us, s, d, key);
    case RR_MAX: return exec_go<E, EA, OpMax>(a, cap, ms, timeout_us, s, d, key);
    case RR_MIN: return exec_go<E, EA, OpMin>(a, cap, ms, timeout_us, s, d, key);
    case RR_AVG:
      if constexpr (__is_same(typename E::A, float)) return exec_go<E, EA, OpAvg>(a, cap, ms, timeout_us, s, d, key);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ring_exec(const ExecArgs& a, Kind k, rr_op_t op, int per_cu_cap, int max_slices, int timeout_us,
                            hipStream_t s) {
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ExecDevice& d = g_exec_dev[dev];
  std::call_once(d.once, [&] {
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) d.cus = 0;
    if (hipDeviceGetAttribute(&d.wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) d.wall_khz = 0;
  });
  const uint32_t key = (static_cast<uint32_t>(k) << 8) | static_cast<uint32_t>(op);
  if (max_slices < 1 || max_slices > 64) max_slices = 64;
  switch (k) {
    case Kind::kI32: return exec_by_op<EI32, EI32>(a, op, per_cu_cap, max_slices, timeout_us, s, d, key);
    case Kind::kF32: return exec_by_op<EF32, EF32>(a, op, per_cu_cap, max_slices, timeout_us, s, d, key);
    case Kind::kBF16: return exec_by_op<EBF16, EF32>(a, op, per_cu_cap, max_slices, timeout_us, s, d, key);
    case Kind::kF16: return exec_by_op<EF16, EF32>(a, op, per_cu_cap, max_slices, timeout_us, s, d, key);
  }
  return hipErrorInvalidValue;
}

hipError_t ring_exec_failures(int device, unsigned long long* count) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (device != cur && (e = hipSetDevice(device)) != hipSuccess) return e;
  e = hipMemcpyFromSymbol(count, HIP_SYMBOL(g_exec_failures), sizeof(*count), 0, hipMemcpyDeviceToHost);
  if (device != cur) {
    const hipError_t e2 = hipSetDevice(cur);
    if (e == hipSuccess) e = e2;
  }
  return e;
}

}  // namespace rr
