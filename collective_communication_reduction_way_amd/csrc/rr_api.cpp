// rr_api.cpp -- the C ABI of librr.so: argument validation, planning and
// kernel dispatch for the collective reductions over p virtual ranks.
//
// Semantics follow page "分布式训练/推理", section "通信原语：rank、world size
// 和 collective operations" (broadcast, reduce, all-gather, reduce-scatter,
// all-reduce; all_reduce = reduce_scatter + all_gather), page "LLM Parallelism
// 基础", sections "MPI Collective Operations" and "Ring AllReduce", and page
// "大模型并行的最小闭环：集合通信、TP、FSDP/ZeRO-3 到权重分片", section
// "Source Log: 2026-05-05" (hierarchical AllReduce).  Each entry point checks
// every argument before the first launch, so a rejected call writes nothing,
// then enqueues its kernels on the caller's stream and returns without
// synchronizing.
#include <hip/hip_runtime_api.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "rr.h"
#include "rr_kernels.h"
#include "rr_plan.h"

namespace {

using rr::Kind;

thread_local std::string g_last_error;

rr_status_t fail(rr_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

rr_status_t ok() {
  g_last_error.clear();
  return RR_SUCCESS;
}

rr_status_t hip_fail(hipError_t e, const char* what) {
  return fail(RR_ERROR_HIP, "%s: HIP error %d (%s)", what, static_cast<int>(e), hipGetErrorString(e));
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

// Tuning knobs (all optional): RR_UNROLL (1, 2 or 4 groups per lane on the
// tunable single-pass fold kernels), RR_NT (0 = ordinary instead of
// nontemporal loads and stores there and in the copy kernels), RR_GRID_CAP
// (maximum workgroups per single-pass launch; 0 = one tile per workgroup),
// RR_PHASE (0 = single-pass fold kernel instead of the phased one on aligned
// buffers), RR_PHASE_SYNC (0 = no barrier between the read and write phases),
// RR_PHASE_PER_CU (workgroups per compute unit of the phased fold; 0 = by the
// schedule), RR_PHASE_GRID (explicit workgroup count), RR_PHASE_U (4 = the
// smaller tile for sums, 8 = the mode's default tile everywhere, 2 or 1 =
// the smallest tiles, ring all-reduce, reduce-scatter and reduce without the
// barrier, 0 = by the schedule), RR_PHASE_STATIC (1 / 0 = the kernels compiled for
// p = 8 / the run-time rank loop; -1 = by mode),
// RR_PHASE_TIMEOUT_US (bound of one barrier wait, default 200),
// RR_PHASE_STRIPS (runs of that many tiles whose 256-group strips
// interleave, up to 64; 1 = contiguous tiles, 0 = by the schedule), RR_PHASE_BATCH
// (reduce-scatter and reduce: tiles per workgroup and round of the batched
// kernel, 2 or 4; 1 = never; 0 = by the schedule), RR_AR_BATCH (the same
// for the ring and hierarchical all-reduces of several rounds; 1 also keeps
// the bucketed all-reduce at one tile of 4 units per workgroup and round),
// RR_MULTI_PER_CU (workgroups per compute unit of the bucket and dim-1
// kernels; 0 = the default), RR_EXEC_TIMEOUT_US (bound of one wait of the persistent ring executor on a
// neighbour's flag, default 1 s), RR_EXEC_PER_CU (cap on its workgroups per
// compute unit; 0 = as many as stay resident), RR_EXEC_SLICES (slices per
// chunk, 1..64; default 64),
// RR_COPY_U (16-byte units per lane of the all-gather and broadcast fan-out:
// 1, 2, 4 or 8; default 4), RR_FANOUT_XCD (destinations per workgroup of the
// XCD-laid-out fan-out: 1, 2 or 4; 0 = never; default by the bytes written),
// RR_FANOUT_WIN (its blocks per XCD window; 0 = default),
// RR_LOG (1 = print each launch plan to stderr).  Defaults are the measured
// best on MI355X: every byte of these collectives is touched once, so
// nontemporal access (no reuse expected) keeps the caches from holding dead
// lines, and separating the read and write traffic of the fused folds in time
// raises their HBM throughput.
// Slices per chunk of the persistent ring executor (at most 64; fewer when
// the device cannot keep them resident or the chunks are short).  With the
// workers of a slice on one XCD, more slices measured faster: at 1 MiB
// chunks 226 / 145 / 102 / 100 us for 8 / 16 / 32 / 64 slices.
constexpr int kExecDefaultSlices = 64;

struct Tuning {
  int unroll;
  int nontemporal;
  int grid_cap;
  int log;
  int phase;
  rr::PhaseTuning pt;
  int multi_per_cu;
  int exec_timeout_us;
  int exec_per_cu;
  int exec_slices;
  int copy_u;
  int fanout_xcd;
  int fanout_win;
};

// The environment is read once per process, at the first call (or by
// rr_reload_tuning), into an immutable snapshot; the call path only loads the
// snapshot's pointer, so no collective call reads the environment (getenv
// races with setenv in multithreaded hosts, and costs host time on the
// latency-bound small calls).  A reload publishes a new snapshot and keeps
// the old ones alive, since a call on another thread may still be reading
// one; reloads are rare (tuning sweeps and tests), so they are never freed.
Tuning read_tuning() {
  Tuning t;
  t.unroll = env_int("RR_UNROLL", 2);
  if (t.unroll != 1 && t.unroll != 2 && t.unroll != 4) t.unroll = 2;
  t.nontemporal = env_int("RR_NT", 1) ? 1 : 0;
  t.grid_cap = env_int("RR_GRID_CAP", 0);
  if (t.grid_cap < 0) t.grid_cap = 0;
  t.log = env_int("RR_LOG", 0);
  t.phase = env_int("RR_PHASE", 1) ? 1 : 0;
  t.pt.sync = env_int("RR_PHASE_SYNC", 1) ? 1 : 0;
  t.pt.per_cu = env_int("RR_PHASE_PER_CU", 0);
  if (t.pt.per_cu < 0 || t.pt.per_cu > 64) t.pt.per_cu = 0;
  t.pt.grid = env_int("RR_PHASE_GRID", 0);
  if (t.pt.grid < 0) t.pt.grid = 0;
  t.pt.unroll = env_int("RR_PHASE_U", 0);
  if (t.pt.unroll != 1 && t.pt.unroll != 2 && t.pt.unroll != 4 && t.pt.unroll != 8) t.pt.unroll = 0;
  t.pt.timeout_us = env_int("RR_PHASE_TIMEOUT_US", 200);
  t.pt.static_p = env_int("RR_PHASE_STATIC", -1);
  t.pt.strips = env_int("RR_PHASE_STRIPS", 0);
  if (t.pt.strips < 0 || t.pt.strips > 64) t.pt.strips = 0;
  t.pt.batch = env_int("RR_PHASE_BATCH", 0);
  if (t.pt.batch != 1 && t.pt.batch != 2 && t.pt.batch != 4) t.pt.batch = 0;
  t.pt.ar_batch = env_int("RR_AR_BATCH", 0);
  if (t.pt.ar_batch != 1 && t.pt.ar_batch != 2 && t.pt.ar_batch != 4) t.pt.ar_batch = 0;
  if (t.pt.static_p > 1) t.pt.static_p = 1;
  if (t.pt.timeout_us < 1) t.pt.timeout_us = 200;
  t.multi_per_cu = env_int("RR_MULTI_PER_CU", 0);
  if (t.multi_per_cu < 0 || t.multi_per_cu > 64) t.multi_per_cu = 0;
  t.exec_timeout_us = env_int("RR_EXEC_TIMEOUT_US", 1000000);
  if (t.exec_timeout_us < 1) t.exec_timeout_us = 1;
  t.exec_per_cu = env_int("RR_EXEC_PER_CU", 0);
  if (t.exec_per_cu < 0) t.exec_per_cu = 0;
  t.exec_slices = env_int("RR_EXEC_SLICES", kExecDefaultSlices);
  t.copy_u = env_int("RR_COPY_U", 4);
  t.fanout_xcd = env_int("RR_FANOUT_XCD", -1);
  if (t.fanout_xcd != 0 && t.fanout_xcd != 1 && t.fanout_xcd != 2 && t.fanout_xcd != 4) t.fanout_xcd = -1;
  t.fanout_win = env_int("RR_FANOUT_WIN", 0);
  if (t.fanout_win < 0 || t.fanout_win > 4096) t.fanout_win = 0;
  return t;
}

std::atomic<const Tuning*> g_tuning{nullptr};
std::mutex g_tuning_mu;

void publish_tuning() {
  std::lock_guard<std::mutex> lk(g_tuning_mu);
  g_tuning.store(new Tuning(read_tuning()), std::memory_order_release);
}

const Tuning& tuning() {
  static std::once_flag once;
  std::call_once(once, [] {
    if (!g_tuning.load(std::memory_order_acquire)) publish_tuning();
  });
  return *g_tuning.load(std::memory_order_acquire);
}

constexpr uint64_t kMaxElems = 1ull << 56;


Kind kind_of(rr_dtype_t d) {
  switch (d) {
    case RR_INT32: return Kind::kI32;
    case RR_FLOAT32: return Kind::kF32;
    case RR_FLOAT16: return Kind::kF16;
    default: return Kind::kBF16;
  }
}

bool is_half_dtype(rr_dtype_t d) { return d == RR_BFLOAT16 || d == RR_FLOAT16; }

// AVG divides the folded value by the number of ranks; other ops ignore it.
int32_t divisor_for(rr_op_t op, int p) { return op == RR_AVG ? p : 0; }

Kind acc_kind_of(rr_dtype_t d) { return d == RR_INT32 ? Kind::kI32 : Kind::kF32; }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

rr_status_t check_dtype(rr_dtype_t dt) {
  if (rr::elem_size(dt) == 0) return fail(RR_ERROR_UNSUPPORTED, "unknown dtype %d", static_cast<int>(dt));
  return RR_SUCCESS;
}

rr_status_t check_op(rr_op_t op) {
  if (op != RR_SUM && op != RR_MAX && op != RR_MIN && op != RR_AVG)
    return fail(RR_ERROR_UNSUPPORTED, "unknown op %d", static_cast<int>(op));
  return RR_SUCCESS;
}

// The op must be defined for the dtype: AVG only for the float dtypes.
rr_status_t check_op_dtype(rr_op_t op, rr_dtype_t dt) {
  rr_status_t st = check_op(op);
  if (st) return st;
  if (op == RR_AVG && dt == RR_INT32) return fail(RR_ERROR_UNSUPPORTED, "AVG is defined for float dtypes only");
  return RR_SUCCESS;
}

rr_status_t check_p(int p) {
  if (p < 1 || p > RR_MAX_RANKS) return fail(RR_ERROR_INVALID_ARGUMENT, "p=%d outside [1, %d]", p, RR_MAX_RANKS);
  return RR_SUCCESS;
}

rr_status_t check_n(size_t n) {
  if (static_cast<uint64_t>(n) > kMaxElems)
    return fail(RR_ERROR_INVALID_ARGUMENT, "n=%zu exceeds the limit of 2^56 elements", n);
  return RR_SUCCESS;
}

rr_status_t check_buf(const void* ptr, size_t esz, const char* what, int r) {
  if (!ptr) return fail(RR_ERROR_INVALID_ARGUMENT, "%s[%d] is NULL", what, r);
  if (reinterpret_cast<uintptr_t>(ptr) % esz)
    return fail(RR_ERROR_INVALID_ARGUMENT, "%s[%d] is not aligned to the element size %zu", what, r, esz);
  return RR_SUCCESS;
}

// Byte range of one buffer, for the aliasing rules.
struct Range {
  uintptr_t lo;
  uintptr_t hi;  // exclusive
  int rank;
};

Range range_of(const void* ptr, uint64_t bytes, int rank) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
  return Range{lo, lo + static_cast<uintptr_t>(bytes), rank};
}

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// Outputs must be pairwise disjoint; output r may overlap input q only when
// allowed(r, q) says the pair is the entry point's exact in-place form.
template <class ALLOWED>
rr_status_t check_aliasing(const std::vector<Range>& outs, const std::vector<Range>& ins, ALLOWED allowed) {
  for (size_t i = 0; i < outs.size(); ++i)
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(outs[i], outs[j]))
        return fail(RR_ERROR_INVALID_ARGUMENT, "output buffers of ranks %d and %d overlap", outs[i].rank,
                    outs[j].rank);
  for (const Range& o : outs)
    for (const Range& in : ins)
      if (overlap(o, in) && !allowed(o, in))
        return fail(RR_ERROR_INVALID_ARGUMENT,
                    "output of rank %d overlaps input of rank %d (only the exact in-place form is allowed)",
                    o.rank, in.rank);
  return RR_SUCCESS;
}

// The same rules for many buffers, in O(m log m): outputs sorted by address
// must not overlap their neighbours; every input is checked against the
// outputs that could overlap it.
template <class ALLOWED>
rr_status_t check_aliasing_sorted(std::vector<Range> outs, const std::vector<Range>& ins, ALLOWED allowed) {
  outs.erase(std::remove_if(outs.begin(), outs.end(), [](const Range& r) { return r.lo == r.hi; }), outs.end());
  std::sort(outs.begin(), outs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < outs.size(); ++i)
    if (outs[i].lo < outs[i - 1].hi)
      return fail(RR_ERROR_INVALID_ARGUMENT, "output buffers %d and %d overlap", outs[i - 1].rank, outs[i].rank);
  for (const Range& in : ins) {
    if (in.lo == in.hi) continue;
    // first output ending after in.lo: outputs are disjoint and sorted, so their ends are sorted too
    size_t k = std::lower_bound(outs.begin(), outs.end(), in.lo, [](const Range& o, uintptr_t v) { return o.hi <= v; }) -
               outs.begin();
    for (; k < outs.size() && outs[k].lo < in.hi; ++k)
      if (!allowed(outs[k], in))
        return fail(RR_ERROR_INVALID_ARGUMENT,
                    "output buffer %d overlaps input buffer %d (only the exact in-place form is allowed)",
                    outs[k].rank, in.rank);
  }
  return RR_SUCCESS;
}

// Widest unit (16/4/2/1 bytes) dividing every address and byte count.
int copy_unit(const std::vector<uintptr_t>& addrs, const std::vector<uint64_t>& sizes) {
  uintptr_t acc = 0;
  for (uintptr_t a : addrs) acc |= a;
  for (uint64_t s : sizes) acc |= static_cast<uintptr_t>(s);
  if ((acc & 15u) == 0) return 16;
  if ((acc & 3u) == 0) return 4;
  if ((acc & 1u) == 0) return 2;
  return 1;
}

rr::FoldLaunch base_fold(const Tuning& t) {
  rr::FoldLaunch f;
  memset(&f, 0, sizeof(f));
  f.unroll = t.unroll;
  f.nontemporal = t.nontemporal;
  f.grid_cap = t.grid_cap;
  return f;
}

void log_fold(const Tuning& t, const char* what, const rr::FoldLaunch& f) {
  if (!t.log) return;
  fprintf(stderr, "[rr] %s: mode=%d p=%d group=%d n=%llu segments=%d vec=%d unroll=%d nt=%d grid_cap=%d\n", what,
          static_cast<int>(f.mode), f.args.p, f.args.group, static_cast<unsigned long long>(f.args.n), f.segments,
          f.args.vec, f.unroll, f.nontemporal, f.grid_cap);
}

rr_status_t run_fold(const Tuning& t, const char* what, const rr::FoldLaunch& f, hipStream_t s) {
  log_fold(t, what, f);
  const bool phased = t.phase && rr::phase_supported(f);
  if (t.log && phased) fprintf(stderr, "[rr] %s: phased fold\n", what);
  const hipError_t e = phased ? rr::launch_fold_phase(f, t.pt, s) : rr::launch_fold(f, s);
  if (e != hipSuccess) return hip_fail(e, what);
  return RR_SUCCESS;
}

// Common validation of a rank-array collective.
rr_status_t check_rank_arrays(const void* const* send, void* const* recv, int p, size_t esz, size_t n) {
  if (!send) return fail(RR_ERROR_INVALID_ARGUMENT, "sendbufs is NULL");
  if (!recv) return fail(RR_ERROR_INVALID_ARGUMENT, "recvbufs is NULL");
  if (n == 0) return RR_SUCCESS;
  for (int r = 0; r < p; ++r) {
    rr_status_t st = check_buf(send[r], esz, "sendbufs", r);
    if (st) return st;
    st = check_buf(recv[r], esz, "recvbufs", r);
    if (st) return st;
  }
  return RR_SUCCESS;
}

// ---------------------------------------------------------------------------
// All-reduce variants.

rr_status_t ar_ring_fused(const void* const* send, void* const* recv, int p, uint64_t n, rr_dtype_t dt, rr_op_t op,
                          const Tuning& t, hipStream_t s) {
  rr::FoldLaunch f = base_fold(t);
  f.mode = rr::FoldMode::kRingAll;
  f.in_kind = f.out_kind = kind_of(dt);
  f.op = op;
  f.segments = p;
  f.args.n = n;
  f.args.p = p;
  f.args.group = p;
  f.args.div = divisor_for(op, p);
  bool vec = true;
  for (int r = 0; r < p; ++r) {
    f.args.in[r] = send[r];
    f.args.out[r] = recv[r];
    vec = vec && aligned16(send[r]) && aligned16(recv[r]);
  }
  f.args.vec = vec ? 1 : 0;
  rr::chunk_bounds(p, n, f.args.bound);
  return run_fold(t, "all_reduce(ring, fused)", f, s);
}

// The fold mode of a hierarchical all-reduce with variant flags.  Rounding a
// partial to a 4-byte storage type is the identity, so the wire modes are
// used for the 16-bit types only.
rr::FoldMode hier_mode(rr_dtype_t dt, int flags) {
  const bool ring = flags & RR_HIER_INTRA_RING;
  const bool wire = (flags & RR_HIER_WIRE_ROUND) && is_half_dtype(dt);
  if (ring) return wire ? rr::FoldMode::kHierRingWire : rr::FoldMode::kHierRing;
  return wire ? rr::FoldMode::kHierAllWire : rr::FoldMode::kHierAll;
}

rr_status_t ar_hier_fused(const void* const* send, void* const* recv, int p, uint64_t n, rr_dtype_t dt, rr_op_t op,
                          int G, int flags, const Tuning& t, hipStream_t s) {
  rr::FoldLaunch f = base_fold(t);
  f.mode = hier_mode(dt, flags);
  f.in_kind = f.out_kind = kind_of(dt);
  f.op = op;
  f.segments = 1;
  f.args.n = n;
  f.args.p = p;
  f.args.group = G;
  f.args.div = divisor_for(op, p);
  if (rr::is_hier_ring(f.mode)) {
    // rows = the G group-chunks, bounds floor(k*n/G)
    f.segments = G;
    rr::chunk_bounds(G, n, f.args.bound);
  }
  bool vec = true;
  for (int r = 0; r < p; ++r) {
    f.args.in[r] = send[r];
    f.args.out[r] = recv[r];
    vec = vec && aligned16(send[r]) && aligned16(recv[r]);
  }
  f.args.vec = vec ? 1 : 0;
  return run_fold(t, "all_reduce(hierarchical, fused)", f, s);
}

rr_status_t launch_pairs_copy(const Tuning& t, const std::vector<const void*>& src, const std::vector<void*>& dst,
                              const std::vector<uint64_t>& bytes, const char* what, hipStream_t s) {
  for (size_t base = 0; base < src.size(); base += RR_MAX_RANKS) {
    rr::PairArgs a;
    memset(&a, 0, sizeof(a));
    std::vector<uintptr_t> addrs;
    std::vector<uint64_t> sizes;
    const size_t m = src.size() - base < RR_MAX_RANKS ? src.size() - base : RR_MAX_RANKS;
    for (size_t i = 0; i < m; ++i) {
      a.src[i] = src[base + i];
      a.dst[i] = dst[base + i];
      a.len[i] = bytes[base + i];
      addrs.push_back(reinterpret_cast<uintptr_t>(src[base + i]));
      addrs.push_back(reinterpret_cast<uintptr_t>(dst[base + i]));
      sizes.push_back(bytes[base + i]);
    }
    a.npairs = static_cast<int>(m);
    const int unit = copy_unit(addrs, sizes);
    if (t.log) fprintf(stderr, "[rr] %s: copy pairs=%d unit=%d\n", what, a.npairs, unit);
    const hipError_t e = rr::launch_copy_pairs(a, unit, t.nontemporal, t.grid_cap, s);
    if (e != hipSuccess) return hip_fail(e, what);
  }
  return RR_SUCCESS;
}

rr_status_t ar_ring_staged(const void* const* send, void* const* recv, int p, uint64_t n, rr_dtype_t dt, rr_op_t op,
                           void* ws, const Tuning& t, hipStream_t s) {
  const size_t esz = rr::elem_size(dt);
  uint64_t b[RR_MAX_RANKS + 1];
  rr::chunk_bounds(p, n, b);
  const std::vector<rr::Transfer> sched = rr::ring_schedule(p);
  const bool bf16 = is_half_dtype(dt);  // 16-bit storage: float32 partials in the workspace
  // Working buffers of the reduce-scatter phase (accumulator type).
  std::vector<char*> work(p);
  for (int r = 0; r < p; ++r)
    work[r] = bf16 ? static_cast<char*>(ws) + static_cast<uint64_t>(r) * n * 4 : static_cast<char*>(recv[r]);
  const size_t wsz = bf16 ? 4 : esz;
  rr_status_t st;
  // Load every rank's input into its working buffer.
  if (bf16) {
    rr::PairArgs a;
    memset(&a, 0, sizeof(a));
    bool vec = true;
    for (int r = 0; r < p; ++r) {
      a.src[r] = send[r];
      a.dst[r] = work[r];
      a.len[r] = n;
      vec = vec && aligned16(send[r]) && aligned16(work[r]);
    }
    a.npairs = p;
    a.vec = vec;
    const hipError_t e = rr::launch_convert_pairs(a, kind_of(dt), Kind::kF32, t.grid_cap, s);
    if (e != hipSuccess) return hip_fail(e, "all_reduce(ring, staged): widen");
  } else if (p == 1) {
    if (send[0] != recv[0]) {
      st = launch_pairs_copy(t, {send[0]}, {recv[0]}, {n * esz}, "all_reduce(ring, staged): copy", s);
      if (st) return st;
    }
  }
  // 4-byte types need no copy of the inputs into the receive buffers: in
  // reduce-scatter step s the receiver's own chunk has not been written yet
  // (it receives that chunk only in this step), so it is read from its
  // input, and the message is the sender's input in step 0 and the sender's
  // buffer (the chunk it received in step s - 1) later; every chunk of every
  // buffer is written by the reduce-scatter or the all-gather phase.
  const bool direct = !bf16;
  // Reduce-scatter: one launch per step, p transfers each.
  for (int step = 0; step < p - 1; ++step) {
    rr::PairArgs a;
    memset(&a, 0, sizeof(a));
    bool vec = true;
    int m = 0;
    for (const rr::Transfer& x : sched) {
      if (x.phase != 0 || x.step != step) continue;
      const uint64_t off = b[x.chunk] * wsz;
      if (direct) {
        a.src[m] = static_cast<const char*>(step == 0 ? send[x.src] : recv[x.src]) + off;
        a.aux[m] = static_cast<const char*>(send[x.dst]) + off;
      } else {
        a.src[m] = work[x.src] + off;
        a.aux[m] = work[x.dst] + off;
      }
      a.dst[m] = work[x.dst] + off;
      a.len[m] = b[x.chunk + 1] - b[x.chunk];
      vec = vec && aligned16(a.src[m]) && aligned16(a.dst[m]) && aligned16(a.aux[m]);
      ++m;
    }
    a.npairs = m;
    a.vec = vec;
    if (t.log) fprintf(stderr, "[rr] ring reduce-scatter step %d: %d transfers vec=%d\n", step, m, a.vec);
    const hipError_t e = rr::launch_ring_step(a, acc_kind_of(dt), op, t.grid_cap, s);
    if (e != hipSuccess) return hip_fail(e, "all_reduce(ring, staged): reduce-scatter step");
  }
  // The owner of each chunk finishes its reduced chunk: 16-bit types are
  // rounded once (AVG divides first); float32 AVG divides in place.
  if (bf16 || op == RR_AVG) {
    rr::PairArgs a;
    memset(&a, 0, sizeof(a));
    bool vec = true;
    for (int c = 0; c < p; ++c) {
      a.src[c] = work[c] + b[c] * wsz;
      a.dst[c] = static_cast<char*>(recv[c]) + b[c] * esz;
      a.len[c] = b[c + 1] - b[c];
      vec = vec && aligned16(a.src[c]) && aligned16(a.dst[c]);
    }
    a.npairs = p;
    a.vec = vec;
    a.div = divisor_for(op, p);
    const hipError_t e = rr::launch_convert_pairs(a, Kind::kF32, kind_of(dt), t.grid_cap, s);
    if (e != hipSuccess) return hip_fail(e, "all_reduce(ring, staged): finish the reduced chunks");
  }
  // All-gather: one launch per step; the receiver overwrites.
  for (int step = 0; step < p - 1; ++step) {
    std::vector<const void*> src;
    std::vector<void*> dst;
    std::vector<uint64_t> bytes;
    for (const rr::Transfer& x : sched) {
      if (x.phase != 1 || x.step != step) continue;
      const uint64_t off = b[x.chunk] * esz;
      src.push_back(static_cast<const char*>(recv[x.src]) + off);
      dst.push_back(static_cast<char*>(recv[x.dst]) + off);
      bytes.push_back((b[x.chunk + 1] - b[x.chunk]) * esz);
    }
    st = launch_pairs_copy(t, src, dst, bytes, "all_reduce(ring, staged): all-gather step", s);
    if (st) return st;
  }
  return RR_SUCCESS;
}

// The ring schedule in one persistent kernel: the staged algorithm's
// buffers (float32 workspace slots for 16-bit types, else the outputs as
// working buffers) and arithmetic, steps handed on through device flags.
rr_status_t ar_ring_exec(const void* const* send, void* const* recv, int p, uint64_t n, rr_dtype_t dt, rr_op_t op,
                         void* ws, const Tuning& t, hipStream_t s) {
  rr::ExecArgs a;
  memset(&a, 0, sizeof(a));
  const bool half = is_half_dtype(dt);
  bool vec = true;
  for (int r = 0; r < p; ++r) {
    a.in[r] = send[r];
    a.out[r] = recv[r];
    a.work[r] = half ? static_cast<char*>(ws) + static_cast<uint64_t>(r) * n * 4 : recv[r];
    vec = vec && aligned16(send[r]) && aligned16(recv[r]) && aligned16(a.work[r]);
  }
  rr::chunk_bounds(p, n, a.bound);
  a.p = p;
  a.div = divisor_for(op, p);
  a.vec = vec ? 1 : 0;
  const int slices = t.exec_slices > 0 ? t.exec_slices : kExecDefaultSlices;
  if (t.log) fprintf(stderr, "[rr] all_reduce(ring, persistent): p=%d n=%llu vec=%d\n", p, (unsigned long long)n, a.vec);
  const hipError_t e = rr::launch_ring_exec(a, kind_of(dt), op, t.exec_per_cu, slices, t.exec_timeout_us, s);
  if (e == hipErrorOutOfMemory)
    return fail(RR_ERROR_HIP,
                "all_reduce(ring, persistent): no free step-flag slot on this device (16 for streams with launches "
                "in flight, 48 for launches captured into graphs, each kept for the rest of the process)");
  if (e != hipSuccess) return hip_fail(e, "all_reduce(ring, persistent)");
  return RR_SUCCESS;
}

// Bytes between the group partials of the staged hierarchy in its
// workspace: n partial values (the accumulator type, or the storage type
// with wire rounding on a 16-bit dtype) rounded up to a multiple of 16.
uint64_t hier_part_stride(uint64_t n, rr_dtype_t dt, int flags) {
  const bool wire = (flags & RR_HIER_WIRE_ROUND) && is_half_dtype(dt);
  const uint64_t bytes = n * (wire ? rr::elem_size(dt) : 4);
  return (bytes + 15) / 16 * 16;
}

rr_status_t ar_hier_staged(const void* const* send, void* const* recv, int p, uint64_t n, rr_dtype_t dt, rr_op_t op,
                           int G, int flags, void* ws, const Tuning& t, hipStream_t s) {
  const int J = p / G;
  const size_t esz = rr::elem_size(dt);
  // With wire rounding the partials cross groups in the storage type.
  const bool wire = (flags & RR_HIER_WIRE_ROUND) && is_half_dtype(dt);
  const Kind part_kind = wire ? kind_of(dt) : acc_kind_of(dt);
  // each group's partial starts on a 16-byte boundary of the workspace, so
  // that the vector path's 16-byte accesses stay aligned for any n
  const uint64_t part_stride = hier_part_stride(n, dt, flags);
  // Steps 1-2: each group reduces into its representative's partial
  // (accumulator type, or the storage type with wire rounding, in the
  // workspace).
  rr::FoldLaunch f1 = base_fold(t);
  f1.mode = rr::FoldMode::kAscOne;
  f1.in_kind = kind_of(dt);
  f1.out_kind = part_kind;
  f1.op = op == RR_AVG ? RR_SUM : op;  // group partials; AVG divides at the end
  f1.segments = J;
  f1.args.n = n;
  f1.args.p = G;
  f1.args.group = G;
  bool vec = aligned16(ws);
  for (int r = 0; r < p; ++r) {
    f1.args.in[r] = send[r];
    vec = vec && aligned16(send[r]) && aligned16(recv[r]);
  }
  for (int j = 0; j < J; ++j) f1.args.out[j] = static_cast<char*>(ws) + static_cast<uint64_t>(j) * part_stride;
  f1.args.vec = vec ? 1 : 0;
  rr_status_t st = run_fold(t, "all_reduce(hierarchical, staged): group reduce", f1, s);
  if (st) return st;
  // Steps 3-5: the representatives' partials are combined across groups and
  // the result lands at every representative.
  rr::FoldLaunch f2 = base_fold(t);
  f2.mode = rr::FoldMode::kHierAll;
  f2.in_kind = part_kind;
  f2.out_kind = kind_of(dt);
  f2.op = op;
  f2.segments = 1;
  f2.args.n = n;
  f2.args.p = J;
  f2.args.group = J;
  f2.args.div = divisor_for(op, p);  // the mean is over all p ranks
  for (int j = 0; j < J; ++j) {
    f2.args.in[j] = f1.args.out[j];
    f2.args.out[j] = recv[j * G];
  }
  f2.args.vec = vec ? 1 : 0;
  st = run_fold(t, "all_reduce(hierarchical, staged): cross-group reduce", f2, s);
  if (st) return st;
  // Step 6: each representative broadcasts inside its group, one fan-out
  // launch per group (the representative's buffer is read once and written
  // to its G - 1 members; as G - 1 pair copies it was read G - 1 times).
  if (G > 1) {
    for (int j = 0; j < J; ++j) {
      rr::FanoutArgs a;
      memset(&a, 0, sizeof(a));
      std::vector<uintptr_t> addrs{reinterpret_cast<uintptr_t>(recv[j * G])};
      a.src[0] = recv[j * G];
      for (int i = 1; i < G; ++i) {
        a.dst[i - 1] = recv[j * G + i];
        addrs.push_back(reinterpret_cast<uintptr_t>(recv[j * G + i]));
      }
      a.seg_bytes = n * esz;
      a.dst_seg_stride = 0;
      a.nseg = 1;
      a.ndst = G - 1;
      const int unit = copy_unit(addrs, {n * esz});
      const hipError_t e = rr::launch_fanout(a, unit, t.nontemporal, t.grid_cap, t.copy_u, t.fanout_xcd, t.fanout_win, s);
      if (e != hipSuccess) return hip_fail(e, "all_reduce(hierarchical, staged): group broadcast");
    }
  }
  return RR_SUCCESS;
}

size_t workspace_bytes(rr_algo_t algo, int p, int G, uint64_t n, rr_dtype_t dt, int flags = 0) {
  switch (algo) {
    case RR_ALGO_RING_STAGED:
    case RR_ALGO_RING_PERSISTENT: return is_half_dtype(dt) ? static_cast<size_t>(p) * n * 4 : 0;
    case RR_ALGO_HIER_STAGED: return static_cast<size_t>(p / G) * hier_part_stride(n, dt, flags);
    default: return 0;
  }
}

// rr_all_reduce_ex and rr_all_reduce_hier: `flags` holds the hierarchical
// variant bits (0 for the ring algorithms).
rr_status_t all_reduce_impl(const void* const* sendbufs, void* const* recvbufs, int p, size_t n, rr_dtype_t dtype,
                            rr_op_t op, rr_algo_t algo, int group_size, int flags, void* workspace,
                            size_t ws_bytes, rr_stream_t stream) {
  rr_status_t st;
  if ((st = check_p(p)) || (st = check_dtype(dtype)) || (st = check_op_dtype(op, dtype)) || (st = check_n(n)))
    return st;
  if (algo != RR_ALGO_RING_FUSED && algo != RR_ALGO_RING_STAGED && algo != RR_ALGO_HIER_FUSED &&
      algo != RR_ALGO_HIER_STAGED && algo != RR_ALGO_RING_PERSISTENT)
    return fail(RR_ERROR_INVALID_ARGUMENT, "unknown algo %d", static_cast<int>(algo));
  const bool hier = algo == RR_ALGO_HIER_FUSED || algo == RR_ALGO_HIER_STAGED;
  if (hier && (group_size < 1 || group_size > p || p % group_size))
    return fail(RR_ERROR_INVALID_ARGUMENT, "group_size=%d must be in [1, p] and divide p=%d", group_size, p);
  const size_t esz = rr::elem_size(dtype);
  if ((st = check_rank_arrays(sendbufs, recvbufs, p, esz, n))) return st;
  const size_t need = workspace_bytes(algo, p, hier ? group_size : 1, n, dtype, flags);
  if (need > 0 && n > 0) {
    if (!workspace) return fail(RR_ERROR_INVALID_ARGUMENT, "algo %d needs %zu bytes of workspace", algo, need);
    if (ws_bytes < need)
      return fail(RR_ERROR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                  need);
    if (!aligned16(workspace)) return fail(RR_ERROR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");
  }
  if (n == 0) return ok();
  std::vector<Range> outs, ins;
  for (int r = 0; r < p; ++r) {
    outs.push_back(range_of(recvbufs[r], n * esz, r));
    ins.push_back(range_of(sendbufs[r], n * esz, r));
  }
  if (need > 0) {
    // The workspace is written: it must not touch any rank buffer.
    const Range w = range_of(workspace, need, -1);
    for (const Range& o : outs)
      if (overlap(w, o)) return fail(RR_ERROR_INVALID_ARGUMENT, "workspace overlaps the output of rank %d", o.rank);
    for (const Range& i : ins)
      if (overlap(w, i)) return fail(RR_ERROR_INVALID_ARGUMENT, "workspace overlaps the input of rank %d", i.rank);
  }
  st = check_aliasing(outs, ins, [](const Range& o, const Range& i) { return o.rank == i.rank && o.lo == i.lo; });
  if (st) return st;
  const Tuning& t = tuning();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (algo) {
    case RR_ALGO_RING_FUSED: st = ar_ring_fused(sendbufs, recvbufs, p, n, dtype, op, t, s); break;
    case RR_ALGO_RING_STAGED: st = ar_ring_staged(sendbufs, recvbufs, p, n, dtype, op, workspace, t, s); break;
    case RR_ALGO_RING_PERSISTENT: st = ar_ring_exec(sendbufs, recvbufs, p, n, dtype, op, workspace, t, s); break;
    case RR_ALGO_HIER_FUSED:
      st = ar_hier_fused(sendbufs, recvbufs, p, n, dtype, op, group_size, flags, t, s);
      break;
    case RR_ALGO_HIER_STAGED:
      st = ar_hier_staged(sendbufs, recvbufs, p, n, dtype, op, group_size, flags, workspace, t, s);
      break;
  }
  return st ? st : ok();
}

constexpr int kHierFlags = RR_HIER_INTRA_RING | RR_HIER_WIRE_ROUND | RR_HIER_STAGED;

}  // namespace

namespace rr {

// A failure message for rr_last_error() from the library's other
// translation units (rr_scratch.hip).
rr_status_t record_failure(rr_status_t st, const char* msg) { return fail(st, "%s", msg); }

}  // namespace rr

extern "C" {

rr_status_t rr_all_reduce_ex(const void* const* sendbufs, void* const* recvbufs, int p, size_t n, rr_dtype_t dtype,
                             rr_op_t op, rr_algo_t algo, int group_size, void* workspace, size_t ws_bytes,
                             rr_stream_t stream) {
  return all_reduce_impl(sendbufs, recvbufs, p, n, dtype, op, algo, group_size, 0, workspace, ws_bytes, stream);
}

rr_status_t rr_all_reduce_hier(const void* const* sendbufs, void* const* recvbufs, int p, size_t n,
                               rr_dtype_t dtype, rr_op_t op, int group_size, int flags, void* workspace,
                               size_t ws_bytes, rr_stream_t stream) {
  if (flags & ~kHierFlags) return fail(RR_ERROR_INVALID_ARGUMENT, "unknown hierarchy flags 0x%x", flags);
  if ((flags & RR_HIER_STAGED) && (flags & RR_HIER_INTRA_RING))
    return fail(RR_ERROR_UNSUPPORTED, "the staged hierarchy has no intra-group ring variant");
  const rr_algo_t algo = (flags & RR_HIER_STAGED) ? RR_ALGO_HIER_STAGED : RR_ALGO_HIER_FUSED;
  return all_reduce_impl(sendbufs, recvbufs, p, n, dtype, op, algo, group_size, flags, workspace, ws_bytes, stream);
}

size_t rr_hier_workspace_size(int p, int group_size, size_t n, rr_dtype_t dtype, int flags) {
  if (p < 1 || p > RR_MAX_RANKS || rr::elem_size(dtype) == 0 || static_cast<uint64_t>(n) > kMaxElems) return 0;
  if (group_size < 1 || group_size > p || p % group_size || (flags & ~kHierFlags)) return 0;
  if (!(flags & RR_HIER_STAGED)) return 0;
  return workspace_bytes(RR_ALGO_HIER_STAGED, p, group_size, n, dtype, flags);
}

rr_status_t rr_all_reduce(const void* const* sendbufs, void* const* recvbufs, int p, size_t n, rr_dtype_t dtype,
                          rr_op_t op, rr_stream_t stream) {
  return rr_all_reduce_ex(sendbufs, recvbufs, p, n, dtype, op, RR_ALGO_RING_FUSED, 0, nullptr, 0, stream);
}

rr_status_t rr_reduce_scatter(const void* const* sendbufs, void* const* recvbufs, int p, size_t n, rr_dtype_t dtype,
                              rr_op_t op, rr_stream_t stream) {
  rr_status_t st;
  if ((st = check_p(p)) || (st = check_dtype(dtype)) || (st = check_op_dtype(op, dtype)) || (st = check_n(n)))
    return st;
  if (n % static_cast<size_t>(p))
    return fail(RR_ERROR_INVALID_ARGUMENT, "reduce-scatter needs p | n (p=%d, n=%zu)", p, n);
  const size_t esz = rr::elem_size(dtype);
  if ((st = check_rank_arrays(sendbufs, recvbufs, p, esz, n))) return st;
  if (n == 0) return ok();
  const uint64_t L = n / p;
  std::vector<Range> outs, ins;
  for (int r = 0; r < p; ++r) {
    outs.push_back(range_of(recvbufs[r], L * esz, r));
    ins.push_back(range_of(sendbufs[r], n * esz, r));
  }
  st = check_aliasing(outs, ins, [&](const Range& o, const Range& i) {
    return o.rank == i.rank && o.lo == i.lo + static_cast<uintptr_t>(o.rank) * L * esz;
  });
  if (st) return st;
  const Tuning& t = tuning();
  rr::FoldLaunch f = base_fold(t);
  f.mode = rr::FoldMode::kRingShard;
  f.in_kind = f.out_kind = kind_of(dtype);
  f.op = op;
  f.segments = p;
  f.args.n = n;
  f.args.p = p;
  f.args.group = p;
  f.args.div = divisor_for(op, p);
  bool vec = (L * esz) % 16 == 0;
  for (int r = 0; r < p; ++r) {
    f.args.in[r] = sendbufs[r];
    f.args.out[r] = recvbufs[r];
    vec = vec && aligned16(sendbufs[r]) && aligned16(recvbufs[r]);
  }
  f.args.vec = vec ? 1 : 0;
  rr::chunk_bounds(p, n, f.args.bound);
  st = run_fold(t, "reduce_scatter", f, reinterpret_cast<hipStream_t>(stream));
  return st ? st : ok();
}

rr_status_t rr_all_gather(const void* const* sendbufs, void* const* recvbufs, int p, size_t n, rr_dtype_t dtype,
                          rr_stream_t stream) {
  rr_status_t st;
  if ((st = check_p(p)) || (st = check_dtype(dtype)) || (st = check_n(n))) return st;
  if (n % static_cast<size_t>(p))
    return fail(RR_ERROR_INVALID_ARGUMENT, "all-gather needs p | n (p=%d, n=%zu)", p, n);
  const size_t esz = rr::elem_size(dtype);
  if ((st = check_rank_arrays(sendbufs, recvbufs, p, esz, n))) return st;
  if (n == 0) return ok();
  const uint64_t L = n / p;
  std::vector<Range> outs, ins;
  for (int r = 0; r < p; ++r) {
    outs.push_back(range_of(recvbufs[r], n * esz, r));
    ins.push_back(range_of(sendbufs[r], L * esz, r));
  }
  st = check_aliasing(outs, ins, [&](const Range& o, const Range& i) {
    return o.rank == i.rank && i.lo == o.lo + static_cast<uintptr_t>(o.rank) * L * esz;
  });
  if (st) return st;
  rr::FanoutArgs a;
  memset(&a, 0, sizeof(a));
  std::vector<uintptr_t> addrs;
  for (int r = 0; r < p; ++r) {
    a.src[r] = sendbufs[r];
    a.dst[r] = recvbufs[r];
    addrs.push_back(reinterpret_cast<uintptr_t>(sendbufs[r]));
    addrs.push_back(reinterpret_cast<uintptr_t>(recvbufs[r]));
    if (static_cast<const char*>(sendbufs[r]) == static_cast<const char*>(recvbufs[r]) + L * esz * r)
      a.skip_diag |= 1ull << r;
  }
  a.seg_bytes = L * esz;
  a.dst_seg_stride = L * esz;
  a.nseg = p;
  a.ndst = p;
  const Tuning& t = tuning();
  const int unit = copy_unit(addrs, {L * esz});
  if (t.log) fprintf(stderr, "[rr] all_gather: p=%d shard_bytes=%llu unit=%d\n", p, (unsigned long long)(L * esz), unit);
  const hipError_t e = rr::launch_fanout(a, unit, t.nontemporal, t.grid_cap, t.copy_u, t.fanout_xcd,
                                       t.fanout_win, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "all_gather");
  return ok();
}

rr_status_t rr_reduce(const void* const* sendbufs, void* recvbuf, int root, int p, size_t n, rr_dtype_t dtype,
                      rr_op_t op, rr_stream_t stream) {
  rr_status_t st;
  if ((st = check_p(p)) || (st = check_dtype(dtype)) || (st = check_op_dtype(op, dtype)) || (st = check_n(n)))
    return st;
  if (root < 0 || root >= p) return fail(RR_ERROR_INVALID_ARGUMENT, "root=%d outside [0, p=%d)", root, p);
  if (!sendbufs) return fail(RR_ERROR_INVALID_ARGUMENT, "sendbufs is NULL");
  const size_t esz = rr::elem_size(dtype);
  if (n == 0) return ok();
  for (int r = 0; r < p; ++r)
    if ((st = check_buf(sendbufs[r], esz, "sendbufs", r))) return st;
  if ((st = check_buf(recvbuf, esz, "recvbuf", root))) return st;
  std::vector<Range> outs{range_of(recvbuf, n * esz, root)}, ins;
  for (int r = 0; r < p; ++r) ins.push_back(range_of(sendbufs[r], n * esz, r));
  st = check_aliasing(outs, ins, [](const Range& o, const Range& i) { return o.rank == i.rank && o.lo == i.lo; });
  if (st) return st;
  const Tuning& t = tuning();
  rr::FoldLaunch f = base_fold(t);
  f.mode = rr::FoldMode::kAscOne;
  f.in_kind = f.out_kind = kind_of(dtype);
  f.op = op;
  f.segments = 1;
  f.args.n = n;
  f.args.p = p;
  f.args.group = p;
  f.args.div = divisor_for(op, p);
  bool vec = aligned16(recvbuf);
  for (int r = 0; r < p; ++r) {
    f.args.in[r] = sendbufs[r];
    vec = vec && aligned16(sendbufs[r]);
  }
  f.args.out[0] = recvbuf;
  f.args.vec = vec ? 1 : 0;
  st = run_fold(t, "reduce", f, reinterpret_cast<hipStream_t>(stream));
  return st ? st : ok();
}

rr_status_t rr_broadcast(const void* sendbuf, void* const* recvbufs, int root, int p, size_t n, rr_dtype_t dtype,
                         rr_stream_t stream) {
  rr_status_t st;
  if ((st = check_p(p)) || (st = check_dtype(dtype)) || (st = check_n(n))) return st;
  if (root < 0 || root >= p) return fail(RR_ERROR_INVALID_ARGUMENT, "root=%d outside [0, p=%d)", root, p);
  if (!recvbufs) return fail(RR_ERROR_INVALID_ARGUMENT, "recvbufs is NULL");
  const size_t esz = rr::elem_size(dtype);
  if (n == 0) return ok();
  if ((st = check_buf(sendbuf, esz, "sendbuf", root))) return st;
  for (int r = 0; r < p; ++r)
    if ((st = check_buf(recvbufs[r], esz, "recvbufs", r))) return st;
  std::vector<Range> outs, ins{range_of(sendbuf, n * esz, root)};
  for (int r = 0; r < p; ++r) outs.push_back(range_of(recvbufs[r], n * esz, r));
  st = check_aliasing(outs, ins, [](const Range& o, const Range& i) { return o.rank == i.rank && o.lo == i.lo; });
  if (st) return st;
  rr::FanoutArgs a;
  memset(&a, 0, sizeof(a));
  std::vector<uintptr_t> addrs{reinterpret_cast<uintptr_t>(sendbuf)};
  int m = 0;
  for (int r = 0; r < p; ++r) {
    if (recvbufs[r] == sendbuf) continue;  // the root's in-place copy
    a.dst[m++] = recvbufs[r];
    addrs.push_back(reinterpret_cast<uintptr_t>(recvbufs[r]));
  }
  if (m == 0) return ok();
  a.src[0] = sendbuf;
  a.seg_bytes = n * esz;
  a.dst_seg_stride = 0;
  a.nseg = 1;
  a.ndst = m;
  const Tuning& t = tuning();
  const int unit = copy_unit(addrs, {n * esz});
  if (t.log) fprintf(stderr, "[rr] broadcast: %d copies of %llu bytes unit=%d\n", m, (unsigned long long)(n * esz), unit);
  const hipError_t e = rr::launch_fanout(a, unit, t.nontemporal, t.grid_cap, t.copy_u, t.fanout_xcd,
                                       t.fanout_win, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "broadcast");
  return ok();
}

// Scatter and gather: p independent slice copies in one launch, the root's
// own slice skipped when it is already in place.
rr_status_t rr_scatter(const void* sendbuf, void* const* recvbufs, int root, int p, size_t n, rr_dtype_t dtype,
                       rr_stream_t stream) {
  rr_status_t st;
  if ((st = check_p(p)) || (st = check_dtype(dtype)) || (st = check_n(n))) return st;
  if (root < 0 || root >= p) return fail(RR_ERROR_INVALID_ARGUMENT, "root=%d outside [0, p=%d)", root, p);
  if (n % static_cast<size_t>(p)) return fail(RR_ERROR_INVALID_ARGUMENT, "scatter needs p | n (p=%d, n=%zu)", p, n);
  if (!recvbufs) return fail(RR_ERROR_INVALID_ARGUMENT, "recvbufs is NULL");
  const size_t esz = rr::elem_size(dtype);
  if (n == 0) return ok();
  if ((st = check_buf(sendbuf, esz, "sendbuf", root))) return st;
  for (int r = 0; r < p; ++r)
    if ((st = check_buf(recvbufs[r], esz, "recvbufs", r))) return st;
  const uint64_t L = n / p;
  std::vector<Range> outs, ins{range_of(sendbuf, n * esz, root)};
  for (int r = 0; r < p; ++r) outs.push_back(range_of(recvbufs[r], L * esz, r));
  st = check_aliasing(outs, ins, [&](const Range& o, const Range& i) {
    return o.rank == root && o.lo == i.lo + static_cast<uintptr_t>(root) * L * esz;
  });
  if (st) return st;
  std::vector<const void*> src;
  std::vector<void*> dst;
  std::vector<uint64_t> bytes;
  for (int c = 0; c < p; ++c) {
    const char* from = static_cast<const char*>(sendbuf) + static_cast<uint64_t>(c) * L * esz;
    if (from == recvbufs[c]) continue;  // the root's slice, in place
    src.push_back(from);
    dst.push_back(recvbufs[c]);
    bytes.push_back(L * esz);
  }
  if (src.empty()) return ok();
  st = launch_pairs_copy(tuning(), src, dst, bytes, "scatter", reinterpret_cast<hipStream_t>(stream));
  return st ? st : ok();
}

rr_status_t rr_gather(const void* const* sendbufs, void* recvbuf, int root, int p, size_t n, rr_dtype_t dtype,
                      rr_stream_t stream) {
  rr_status_t st;
  if ((st = check_p(p)) || (st = check_dtype(dtype)) || (st = check_n(n))) return st;
  if (root < 0 || root >= p) return fail(RR_ERROR_INVALID_ARGUMENT, "root=%d outside [0, p=%d)", root, p);
  if (n % static_cast<size_t>(p)) return fail(RR_ERROR_INVALID_ARGUMENT, "gather needs p | n (p=%d, n=%zu)", p, n);
  if (!sendbufs) return fail(RR_ERROR_INVALID_ARGUMENT, "sendbufs is NULL");
  const size_t esz = rr::elem_size(dtype);
  if (n == 0) return ok();
  for (int r = 0; r < p; ++r)
    if ((st = check_buf(sendbufs[r], esz, "sendbufs", r))) return st;
  if ((st = check_buf(recvbuf, esz, "recvbuf", root))) return st;
  const uint64_t L = n / p;
  std::vector<Range> outs{range_of(recvbuf, n * esz, root)}, ins;
  for (int r = 0; r < p; ++r) ins.push_back(range_of(sendbufs[r], L * esz, r));
  st = check_aliasing(outs, ins, [&](const Range& o, const Range& i) {
    return i.rank == root && i.lo == o.lo + static_cast<uintptr_t>(root) * L * esz;
  });
  if (st) return st;
  std::vector<const void*> src;
  std::vector<void*> dst;
  std::vector<uint64_t> bytes;
  for (int c = 0; c < p; ++c) {
    char* to = static_cast<char*>(recvbuf) + static_cast<uint64_t>(c) * L * esz;
    if (sendbufs[c] == to) continue;  // the root's slice, in place
    src.push_back(sendbufs[c]);
    dst.push_back(to);
    bytes.push_back(L * esz);
  }
  if (src.empty()) return ok();
  st = launch_pairs_copy(tuning(), src, dst, bytes, "gather", reinterpret_cast<hipStream_t>(stream));
  return st ? st : ok();
}

// ---------------------------------------------------------------------------
// Bucketed all-reduce: tensor t of rank r is sendbufs[t*p + r] (counts[t]
// elements); the bucket is their concatenation and its chunk c is
// [floor(c*N/p), floor((c+1)*N/p)) of the N bucket elements.  The host cuts
// every tensor at the chunk bounds, splits each run into a 16-byte-aligned
// body and element-wise head and tail, and packs the pieces into as few
// launches as the argument tables allow.

rr_status_t rr_all_reduce_bucket(const void* const* sendbufs, void* const* recvbufs, const size_t* counts,
                                 int ntensors, int p, rr_dtype_t dtype, rr_op_t op, rr_stream_t stream) {
  rr_status_t st;
  if ((st = check_p(p)) || (st = check_dtype(dtype)) || (st = check_op_dtype(op, dtype))) return st;
  if (ntensors < 0) return fail(RR_ERROR_INVALID_ARGUMENT, "ntensors=%d is negative", ntensors);
  if (ntensors == 0) return ok();
  if (!counts) return fail(RR_ERROR_INVALID_ARGUMENT, "counts is NULL");
  if (!sendbufs) return fail(RR_ERROR_INVALID_ARGUMENT, "sendbufs is NULL");
  if (!recvbufs) return fail(RR_ERROR_INVALID_ARGUMENT, "recvbufs is NULL");
  const size_t esz = rr::elem_size(dtype);
  uint64_t total = 0;
  for (int t = 0; t < ntensors; ++t) {
    if (static_cast<uint64_t>(counts[t]) > kMaxElems || total + counts[t] > kMaxElems)
      return fail(RR_ERROR_INVALID_ARGUMENT, "the bucket exceeds the limit of 2^56 elements");
    total += counts[t];
  }
  std::vector<Range> outs, ins;
  for (int t = 0; t < ntensors; ++t) {
    if (counts[t] == 0) continue;
    for (int r = 0; r < p; ++r) {
      const int i = t * p + r;
      if ((st = check_buf(sendbufs[i], esz, "sendbufs", i)) || (st = check_buf(recvbufs[i], esz, "recvbufs", i)))
        return st;
      outs.push_back(range_of(recvbufs[i], counts[t] * esz, i));
      ins.push_back(range_of(sendbufs[i], counts[t] * esz, i));
    }
  }
  st = check_aliasing_sorted(outs, ins, [](const Range& o, const Range& i) { return o.rank == i.rank && o.lo == i.lo; });
  if (st) return st;
  if (total == 0) return ok();
  const Tuning& t = tuning();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const Kind k = kind_of(dtype);
  const uint64_t V = 16 / esz;
  // A tile is kBlock*kBucketU units: 16-byte groups in vector pieces, single
  // elements in scalar pieces.
  const uint64_t kTileUnits = static_cast<uint64_t>(rr::kBlock) * rr::kBucketU;
  const uint64_t kMaxUnits = 1ull << 30;  // keeps the kernel's tile arithmetic in 32 bits
  uint64_t b[RR_MAX_RANKS + 1];
  rr::chunk_bounds(p, total, b);

  rr::BucketArgs a;
  int batch_tensor = -1;  // tensor whose pointers the batch's last slots hold
  int nslots = 0;
  int launches = 0;
  auto reset = [&] {
    memset(&a, 0, sizeof(a));
    a.p = p;
    a.div = divisor_for(op, p);
    a.strips = static_cast<uint32_t>(t.pt.strips);  // 0: by the round count (rr_multi.hip)
    batch_tensor = -1;
    nslots = 0;
  };
  auto flush = [&]() -> rr_status_t {
    if (a.npieces == 0) return RR_SUCCESS;
    a.tile0[a.npieces] = a.tiles;
    if (t.log) fprintf(stderr, "[rr] all_reduce_bucket: launch %d, %d pieces, %u tiles\n", launches, a.npieces, a.tiles);
    const hipError_t e = rr::launch_bucket(a, k, op, t.multi_per_cu, t.pt.sync, t.pt.ar_batch, t.pt.timeout_us, s);
    if (e != hipSuccess) return hip_fail(e, "all_reduce_bucket");
    ++launches;
    reset();
    return RR_SUCCESS;
  };
  // Add a piece of `units` units of tensor `tt` starting at element `start`.
  auto add = [&](int tt, uint64_t start, uint64_t units, int chunk, bool vec) -> rr_status_t {
    while (units > 0) {
      const uint64_t u = units < kMaxUnits ? units : kMaxUnits;
      if (a.npieces == rr::kBucketPieces || (batch_tensor != tt && nslots + 2 * p > rr::kBucketPtrs)) {
        rr_status_t e = flush();
        if (e) return e;
      }
      if (batch_tensor != tt) {
        for (int r = 0; r < p; ++r) {
          a.ptr[nslots + r] = sendbufs[tt * p + r];
          a.ptr[nslots + p + r] = recvbufs[tt * p + r];
        }
        batch_tensor = tt;
        nslots += 2 * p;
      }
      const int i = a.npieces++;
      a.start[i] = start;
      a.units[i] = static_cast<uint32_t>(u);
      a.tile0[i] = a.tiles;
      a.base[i] = static_cast<uint16_t>(nslots - 2 * p);
      a.rot[i] = static_cast<uint8_t>(chunk);
      a.vec[i] = vec ? 1 : 0;
      a.tiles += static_cast<uint32_t>((u + kTileUnits - 1) / kTileUnits);
      start += vec ? u * V : u;
      units -= u;
      if (a.tiles > 0x40000000u) {
        rr_status_t e = flush();
        if (e) return e;
      }
    }
    return RR_SUCCESS;
  };
  reset();
  uint64_t o = 0;
  for (int tt = 0; tt < ntensors; ++tt) {
    const uint64_t n = counts[tt];
    if (n == 0) continue;
    bool aligned = true;
    for (int r = 0; r < p; ++r)
      aligned = aligned && aligned16(sendbufs[tt * p + r]) && aligned16(recvbufs[tt * p + r]);
    for (int c = 0; c < p; ++c) {
      const uint64_t lo = std::max(o, b[c]) - o;
      const uint64_t hi = std::min(o + n, b[c + 1]) - o;
      if (b[c + 1] <= o || b[c] >= o + n || lo >= hi) continue;
      const uint64_t g_lo = (lo + V - 1) / V;
      const uint64_t g_hi = hi / V;
      if (aligned && g_hi > g_lo) {
        if (g_lo * V > lo && (st = add(tt, lo, g_lo * V - lo, c, false))) return st;
        if ((st = add(tt, g_lo * V, g_hi - g_lo, c, true))) return st;
        if (hi > g_hi * V && (st = add(tt, g_hi * V, hi - g_hi * V, c, false))) return st;
      } else if ((st = add(tt, lo, hi - lo, c, false))) {
        return st;
      }
    }
    o += n;
  }
  st = flush();
  return st ? st : ok();
}

// ---------------------------------------------------------------------------
// Tensor-parallel layouts on row-major [rows, cols] matrices, cols = p*w.

rr_status_t check_cols_shape(int p, size_t rows, size_t cols) {
  if (cols % static_cast<size_t>(p))
    return fail(RR_ERROR_INVALID_ARGUMENT, "cols=%zu is not divisible by p=%d", cols, p);
  if (rows > 0 && cols > 0 && (static_cast<uint64_t>(rows) > kMaxElems / static_cast<uint64_t>(cols)))
    return fail(RR_ERROR_INVALID_ARGUMENT, "rows*cols exceeds the limit of 2^56 elements");
  return RR_SUCCESS;
}

rr_status_t rr_all_gather_dim1(const void* const* sendbufs, void* const* recvbufs, int p, size_t rows, size_t cols,
                               rr_dtype_t dtype, rr_stream_t stream) {
  rr_status_t st;
  if ((st = check_p(p)) || (st = check_dtype(dtype)) || (st = check_cols_shape(p, rows, cols))) return st;
  const size_t esz = rr::elem_size(dtype);
  const uint64_t n = static_cast<uint64_t>(rows) * cols;
  if ((st = check_rank_arrays(sendbufs, recvbufs, p, esz, n))) return st;
  if (n == 0) return ok();
  const uint64_t w = cols / p;
  std::vector<Range> outs, ins;
  for (int r = 0; r < p; ++r) {
    outs.push_back(range_of(recvbufs[r], n * esz, r));
    ins.push_back(range_of(sendbufs[r], rows * w * esz, r));
  }
  st = check_aliasing(outs, ins, [](const Range&, const Range&) { return false; });
  if (st) return st;
  rr::ColsArgs a;
  memset(&a, 0, sizeof(a));
  std::vector<uintptr_t> addrs;
  for (int r = 0; r < p; ++r) {
    a.src[r] = sendbufs[r];
    a.dst[r] = recvbufs[r];
    addrs.push_back(reinterpret_cast<uintptr_t>(sendbufs[r]));
    addrs.push_back(reinterpret_cast<uintptr_t>(recvbufs[r]));
  }
  const int unit = copy_unit(addrs, {w * esz});
  a.rows = rows;
  a.wu = w * esz / unit;
  a.du = cols * esz / unit;
  a.p = p;
  const Tuning& t = tuning();
  if (t.log) fprintf(stderr, "[rr] all_gather_dim1: p=%d rows=%zu cols=%zu unit=%d\n", p, rows, cols, unit);
  const hipError_t e =
      rr::launch_gather_cols(a, unit, t.nontemporal, t.multi_per_cu, t.fanout_xcd, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "all_gather_dim1");
  return ok();
}

rr_status_t rr_reduce_scatter_dim1(const void* const* sendbufs, void* const* recvbufs, int p, size_t rows,
                                   size_t cols, rr_dtype_t dtype, rr_op_t op, rr_stream_t stream) {
  rr_status_t st;
  if ((st = check_p(p)) || (st = check_dtype(dtype)) || (st = check_op_dtype(op, dtype)) ||
      (st = check_cols_shape(p, rows, cols)))
    return st;
  const size_t esz = rr::elem_size(dtype);
  const uint64_t n = static_cast<uint64_t>(rows) * cols;
  if ((st = check_rank_arrays(sendbufs, recvbufs, p, esz, n))) return st;
  if (n == 0) return ok();
  const uint64_t w = cols / p;
  std::vector<Range> outs, ins;
  for (int r = 0; r < p; ++r) {
    outs.push_back(range_of(recvbufs[r], rows * w * esz, r));
    ins.push_back(range_of(sendbufs[r], n * esz, r));
  }
  st = check_aliasing(outs, ins, [](const Range&, const Range&) { return false; });
  if (st) return st;
  rr::ColsArgs a;
  memset(&a, 0, sizeof(a));
  bool vec = (w * esz) % 16 == 0;
  for (int r = 0; r < p; ++r) {
    a.src[r] = sendbufs[r];
    a.dst[r] = recvbufs[r];
    vec = vec && aligned16(sendbufs[r]) && aligned16(recvbufs[r]);
  }
  const uint64_t unit = vec ? 16 : esz;
  a.rows = rows;
  a.wu = w * esz / unit;
  a.du = cols * esz / unit;
  a.p = p;
  a.div = divisor_for(op, p);
  const Tuning& t = tuning();
  if (t.log) fprintf(stderr, "[rr] reduce_scatter_dim1: p=%d rows=%zu cols=%zu vec=%d\n", p, rows, cols, vec ? 1 : 0);
  const hipError_t e = rr::launch_fold_cols(a, kind_of(dtype), op, vec ? 1 : 0, t.multi_per_cu,
                                            reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "reduce_scatter_dim1");
  return ok();
}

size_t rr_workspace_size(rr_algo_t algo, int p, int group_size, size_t n, rr_dtype_t dtype) {
  if (p < 1 || p > RR_MAX_RANKS || rr::elem_size(dtype) == 0 || static_cast<uint64_t>(n) > kMaxElems) return 0;
  if (algo == RR_ALGO_HIER_STAGED && (group_size < 1 || group_size > p || p % group_size)) return 0;
  return workspace_bytes(algo, p, group_size, n, dtype);
}

const char* rr_status_string(rr_status_t status) {
  switch (status) {
    case RR_SUCCESS: return "success";
    case RR_ERROR_INVALID_ARGUMENT: return "invalid argument";
    case RR_ERROR_UNSUPPORTED: return "unsupported dtype or op";
    case RR_ERROR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

rr_status_t rr_barrier_timeouts(int device, uint64_t* count) {
  if (!count) return fail(RR_ERROR_INVALID_ARGUMENT, "count is NULL");
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_fail(e, "barrier_timeouts");
  if (device < 0 || device >= ndev) return fail(RR_ERROR_INVALID_ARGUMENT, "device %d outside [0, %d)", device, ndev);
  unsigned long long c = 0;
  e = rr::phase_barrier_timeouts(device, &c);
  if (e != hipSuccess) return hip_fail(e, "barrier_timeouts");
  *count = c;
  return ok();
}

rr_status_t rr_ring_exec_failures(int device, uint64_t* count) {
  if (!count) return fail(RR_ERROR_INVALID_ARGUMENT, "count is NULL");
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_fail(e, "ring_exec_failures");
  if (device < 0 || device >= ndev) return fail(RR_ERROR_INVALID_ARGUMENT, "device %d outside [0, %d)", device, ndev);
  unsigned long long c = 0;
  e = rr::ring_exec_failures(device, &c);
  if (e != hipSuccess) return hip_fail(e, "ring_exec_failures");
  *count = c;
  return ok();
}

void rr_reload_tuning(void) {
  tuning();  // the first snapshot, if no call has taken it yet
  publish_tuning();
}

const char* rr_last_error(void) { return g_last_error.c_str(); }

const char* rr_version(void) { return "rr 0.1.0 (gfx950)"; }

}  // extern "C"
