// rr_fold_impl.h -- the p-way streaming fold kernel (gfx950) and its dispatch.
//
// One kernel template serves every reduction of the library: ring all-reduce
// (each chunk folded in the ring's reduce-scatter order, all p outputs written
// in the same pass, i.e. reduce-scatter and all-gather fused), ring
// reduce-scatter, reduce, the fused hierarchical all-reduce and the steps of
// the staged hierarchy.  The ring order comes from page "LLM Parallelism 基础",
// section "Ring AllReduce" (every rank sends to the next rank; the receiver
// accumulates), which folds chunk c as x_{c+1}, x_{c+2}, ..., x_c.
//
// Work decomposition.  Workgroup row blockIdx.y is a chunk (ring modes) or a
// segment; along x, workgroups stride over tiles of kBlock*U groups, a group
// being V elements moved with 16-byte accesses.  Each lane owns whole groups:
// it issues the loads of all p inputs for its U groups first (p*U 16-byte
// loads in flight per lane), then folds in registers in the fixed order,
// converts once and stores to every output.  The reduction across ranks thus
// happens inside each lane; no LDS, no barriers, no cross-lane traffic, so the
// float order is exactly the specified one and in-place operation is safe
// (a lane reads all inputs of an element before writing any output of it).
// Chunk heads and tails that do not fill a group, and buffers that are not
// 16-byte aligned, take a scalar path with the same order.
#pragma once

#include "rr_device.h"
#include "rr_kernels.h"

namespace rr {

template <class TI, class TO>
constexpr int group_len() {
  return 16 / static_cast<int>(sizeof(typename TI::S) < sizeof(typename TO::S) ? sizeof(typename TI::S)
                                                                               : sizeof(typename TO::S));
}

constexpr bool is_ring(FoldMode m) { return m == FoldMode::kRingAll || m == FoldMode::kRingShard; }
constexpr bool writes_all(FoldMode m) { return m == FoldMode::kRingAll || is_hier(m); }

// k-th input in the fold order of row `seg`.
template <FoldMode M>
__device__ __forceinline__ int fold_src(int k, int seg, int p, int group) {
  if constexpr (is_ring(M)) {
    const int r = seg + 1 + k;  // seg <= p-1 and k <= p-1, so r <= 2p-1
    return r >= p ? r - p : r;
  } else if constexpr (M == FoldMode::kAscOne) {
    return seg * p + k;
  } else if constexpr (is_hier_ring(M)) {
    // member i of group j, the group's ring starting after member seg
    const int j = k / group;
    const int i = seg + 1 + (k - j * group);  // seg <= group-1, so i <= 2*group-1
    return j * group + (i >= group ? i - group : i);
  } else {
    return k;
  }
}

// A finished group partial as it enters the cross-group fold: for the wire
// modes rounded to the storage type (nearest even) and widened again.
template <class E, FoldMode M, class A>
__device__ __forceinline__ A group_partial(A v) {
  if constexpr (is_wire(M) && sizeof(typename E::S) == 2) {
    return half_to_f32<E>(f32_to_half<E>(v));
  } else {
    return v;
  }
}

// Fold step k (k >= 1) of value x into the running state.  For the hierarchy,
// `acc` is the running group partial and `tot` the running fold of finished
// groups; a new group starts at every multiple of `group`.
template <class E, class OP, FoldMode M, class A>
__device__ __forceinline__ void fold_step(A& acc, A& tot, A x, int k, int group) {
  if constexpr (is_hier(M)) {
    if (k % group == 0) {
      const A g = group_partial<E, M>(acc);
      tot = (k == group) ? g : OP::apply(tot, g);
      acc = x;
    } else {
      acc = OP::apply(acc, x);
    }
  } else {
    acc = OP::apply(acc, x);
  }
}

// The folded value of an element: for the hierarchy the last group's partial
// joins the total; then the op's last step (AVG: the division by `div`).
template <class E, class OP, FoldMode M, class A>
__device__ __forceinline__ A fold_finish(A acc, A tot, int p, int group, int32_t div) {
  if constexpr (is_hier(M)) {
    const A g = group_partial<E, M>(acc);
    return op_finish<OP>((p > group) ? OP::apply(tot, g) : g, div);
  } else {
    return op_finish<OP>(acc, div);
  }
}

// Scalar path: element i of row seg.
template <class TI, class TO, class OP, FoldMode M>
__device__ __forceinline__ void fold_scalar(const FoldArgs& a, uint64_t i, uint64_t lo, int seg, int p) {
  using SI = typename TI::S;
  using SO = typename TO::S;
  using A = typename TI::A;
  A acc = load_one<TI>(static_cast<const SI*>(a.in[fold_src<M>(0, seg, p, a.group)]) + i);
  A tot = acc;
  for (int k = 1; k < p; ++k) {
    const A x = load_one<TI>(static_cast<const SI*>(a.in[fold_src<M>(k, seg, p, a.group)]) + i);
    fold_step<TI, OP, M>(acc, tot, x, k, a.group);
  }
  acc = fold_finish<TI, OP, M>(acc, tot, p, a.group, a.div);
  if constexpr (writes_all(M)) {
    for (int r = 0; r < p; ++r) store_one<TO>(static_cast<SO*>(a.out[r]) + i, acc);
  } else if constexpr (M == FoldMode::kRingShard) {
    store_one<TO>(static_cast<SO*>(a.out[seg]) + (i - lo), acc);
  } else {
    store_one<TO>(static_cast<SO*>(a.out[seg]) + i, acc);
  }
}

// Addressing of the vector path.  A tile is kBlock*U consecutive groups whose
// first group is uniform across the workgroup: every rank's tile base is
// computed once per tile, and lane t, slot u reaches the group at tile base +
// (t + u*kBlock) groups through a 32-bit offset that stays the same from tile
// to tile.  Consecutive lanes touch consecutive 16-byte words, so each
// wavefront-wide access covers whole 64-byte segments.

// Vector path, compile-time p: all p*U loads first, then the folds.
// `valid` = groups of this tile inside the row (only used when GUARD).
template <class TI, class TO, class OP, int P, int U, bool NT, FoldMode M, bool GUARD>
__device__ __forceinline__ void fold_tile(const char* const* sb, char* const* db, uint32_t valid, int group,
                                          int32_t div) {
  constexpr int V = group_len<TI, TO>();
  constexpr uint32_t GBI = V * sizeof(typename TI::S);
  constexpr uint32_t GBO = V * sizeof(typename TO::S);
  using SI = typename TI::S;
  using SO = typename TO::S;
  using A = typename TI::A;
  const uint32_t lane = threadIdx.x;
  Raw<TI, V> raw[U][P];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t off = (lane + u * kBlock) * GBI;
    if (!GUARD || lane + u * kBlock < valid) {
#pragma unroll
      for (int k = 0; k < P; ++k) load_group<NT>(raw[u][k], reinterpret_cast<const SI*>(sb[k] + off));
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (GUARD && lane + u * kBlock >= valid) continue;
    const uint32_t off = (lane + u * kBlock) * GBO;
    A acc[V];
    A tot[V];
    unpack(raw[u][0], acc);
#pragma unroll
    for (int j = 0; j < V; ++j) tot[j] = acc[j];
#pragma unroll
    for (int k = 1; k < P; ++k) {
      A x[V];
      unpack(raw[u][k], x);
#pragma unroll
      for (int j = 0; j < V; ++j) fold_step<TI, OP, M>(acc[j], tot[j], x[j], k, group);
    }
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] = fold_finish<TI, OP, M>(acc[j], tot[j], P, group, div);
    Raw<TO, V> o;
    pack(acc, o);
    constexpr int ND = writes_all(M) ? P : 1;
#pragma unroll
    for (int r = 0; r < ND; ++r) store_group<NT>(reinterpret_cast<SO*>(db[r] + off), o);
  }
}

// Vector path, run-time p: inputs are streamed one rank at a time, U groups
// per lane in flight.  `in_base(k)` / `out_base(r)` give the tile's byte base
// of the k-th input in fold order / of output r.
template <class TI, class TO, class OP, int U, bool NT, FoldMode M, bool GUARD>
__device__ __forceinline__ void fold_tile_dyn(const FoldArgs& a, int seg, int p, uint64_t in_tile_off,
                                              int64_t out_tile_off, uint32_t valid) {
  constexpr int V = group_len<TI, TO>();
  constexpr uint32_t GBI = V * sizeof(typename TI::S);
  constexpr uint32_t GBO = V * sizeof(typename TO::S);
  using SI = typename TI::S;
  using SO = typename TO::S;
  using A = typename TI::A;
  const uint32_t lane = threadIdx.x;
  A acc[U][V];
  A tot[U][V];
  {
    const char* s0 = static_cast<const char*>(a.in[fold_src<M>(0, seg, p, a.group)]) + in_tile_off;
    Raw<TI, V> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!GUARD || lane + u * kBlock < valid)
        load_group<NT>(raw[u], reinterpret_cast<const SI*>(s0 + (lane + u * kBlock) * GBI));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      unpack(raw[u], acc[u]);
#pragma unroll
      for (int j = 0; j < V; ++j) tot[u][j] = acc[u][j];
    }
  }
  for (int k = 1; k < p; ++k) {
    const char* sk = static_cast<const char*>(a.in[fold_src<M>(k, seg, p, a.group)]) + in_tile_off;
    Raw<TI, V> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!GUARD || lane + u * kBlock < valid)
        load_group<NT>(raw[u], reinterpret_cast<const SI*>(sk + (lane + u * kBlock) * GBI));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      A x[V];
      unpack(raw[u], x);
#pragma unroll
      for (int j = 0; j < V; ++j) fold_step<TI, OP, M>(acc[u][j], tot[u][j], x[j], k, a.group);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (GUARD && lane + u * kBlock >= valid) continue;
    const uint32_t off = (lane + u * kBlock) * GBO;
#pragma unroll
    for (int j = 0; j < V; ++j) acc[u][j] = fold_finish<TI, OP, M>(acc[u][j], tot[u][j], p, a.group, a.div);
    Raw<TO, V> o;
    pack(acc[u], o);
    if constexpr (writes_all(M)) {
      for (int r = 0; r < p; ++r)
        store_group<NT>(reinterpret_cast<SO*>(static_cast<char*>(a.out[r]) + out_tile_off + off), o);
    } else {
      store_group<NT>(reinterpret_cast<SO*>(static_cast<char*>(a.out[seg]) + out_tile_off + off), o);
    }
  }
}

template <class TI, class TO, class OP, int P, int U, bool NT, FoldMode M>
__global__ __launch_bounds__(kBlock) void k_fold(FoldArgs a) {
  constexpr int V = group_len<TI, TO>();
  using SI = typename TI::S;
  using SO = typename TO::S;
  const int p = (P > 0) ? P : a.p;
  const int seg = blockIdx.y;
  uint64_t lo = 0;
  uint64_t hi = a.n;
  if constexpr (uses_bounds(M)) {
    lo = a.bound[seg];
    hi = a.bound[seg + 1];
  }
  if (!a.vec) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = lo + static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < hi; i += stride)
      fold_scalar<TI, TO, OP, M>(a, i, lo, seg, p);
    return;
  }
  const uint64_t g_lo = (lo + V - 1) / V;
  uint64_t g_hi = hi / V;
  if (g_hi < g_lo) g_hi = g_lo;
  const uint64_t ngroups = g_hi - g_lo;
  constexpr uint64_t kTile = static_cast<uint64_t>(kBlock) * U;
  const uint64_t ntiles = (ngroups + kTile - 1) / kTile;
  constexpr uint64_t GBI = V * sizeof(SI);
  constexpr uint64_t GBO = V * sizeof(SO);
  // Byte offset of group g in an output: outputs of kRingShard hold only the
  // row's chunk, so their group g sits (g*V - lo) elements in.
  const int64_t out_shift = (M == FoldMode::kRingShard) ? -static_cast<int64_t>(lo * sizeof(SO)) : 0;
  if constexpr (P > 0) {
    // Rotated input pointers and output pointers, uniform across the
    // workgroup (scalar registers).
    const char* src[P];
#pragma unroll
    for (int k = 0; k < P; ++k) src[k] = static_cast<const char*>(a.in[fold_src<M>(k, seg, P, a.group)]);
    constexpr int ND = writes_all(M) ? P : 1;
    char* dst[ND];
    if constexpr (writes_all(M)) {
#pragma unroll
      for (int r = 0; r < P; ++r) dst[r] = static_cast<char*>(a.out[r]);
    } else {
      dst[0] = static_cast<char*>(a.out[seg]);
    }
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
      const uint64_t g_first = g_lo + t * kTile;
      const char* sb[P];
#pragma unroll
      for (int k = 0; k < P; ++k) sb[k] = src[k] + g_first * GBI;
      char* db[ND];
#pragma unroll
      for (int r = 0; r < ND; ++r) db[r] = dst[r] + static_cast<int64_t>(g_first * GBO) + out_shift;
      const uint64_t rem = ngroups - t * kTile;
      if (rem >= kTile) {
        fold_tile<TI, TO, OP, P, U, NT, M, false>(sb, db, 0, a.group, a.div);
      } else {
        fold_tile<TI, TO, OP, P, U, NT, M, true>(sb, db, static_cast<uint32_t>(rem), a.group, a.div);
      }
    }
  } else {
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
      const uint64_t g_first = g_lo + t * kTile;
      const uint64_t in_off = g_first * GBI;
      const int64_t out_off = static_cast<int64_t>(g_first * GBO) + out_shift;
      const uint64_t rem = ngroups - t * kTile;
      if (rem >= kTile) {
        fold_tile_dyn<TI, TO, OP, U, NT, M, false>(a, seg, p, in_off, out_off, 0);
      } else {
        fold_tile_dyn<TI, TO, OP, U, NT, M, true>(a, seg, p, in_off, out_off, static_cast<uint32_t>(rem));
      }
    }
  }
  // Head [lo, g_lo*V) and tail [g_hi*V, hi) of the row: fewer than V elements
  // each, done by the first 2V lanes of workgroup 0 of the row.
  if (blockIdx.x == 0 && threadIdx.x < 2 * V) {
    const uint64_t vb = g_lo * V;
    const uint64_t head_end = vb < hi ? vb : hi;
    const bool is_head = threadIdx.x < V;
    const uint64_t i = is_head ? lo + threadIdx.x : g_hi * V + (threadIdx.x - V);
    if (is_head ? (i < head_end) : (i < hi)) fold_scalar<TI, TO, OP, M>(a, i, lo, seg, p);
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch.

template <class TI, class TO, class OP, int P, int U, bool NT, FoldMode M>
hipError_t fold_go(const FoldLaunch& f, hipStream_t s) {
  constexpr int V = group_len<TI, TO>();
  uint64_t longest = 0;
  if constexpr (uses_bounds(M)) {
    for (int c = 0; c < f.segments; ++c) {
      const uint64_t len = f.args.bound[c + 1] - f.args.bound[c];
      if (len > longest) longest = len;
    }
  } else {
    longest = f.args.n;
  }
  uint64_t blocks_x;
  if (f.args.vec) {
    const uint64_t groups = longest / V + 1;
    blocks_x = (groups + static_cast<uint64_t>(kBlock) * U - 1) / (static_cast<uint64_t>(kBlock) * U);
  } else {
    blocks_x = (longest + kBlock - 1) / kBlock;
  }
  if (blocks_x < 1) blocks_x = 1;
  if (f.grid_cap > 0) {
    uint64_t cap_x = static_cast<uint64_t>(f.grid_cap) / static_cast<uint64_t>(f.segments);
    if (cap_x < 1) cap_x = 1;
    if (blocks_x > cap_x) blocks_x = cap_x;
  }
  if (blocks_x > 0x7FFFFFFFull) blocks_x = 0x7FFFFFFFull;
  dim3 grid(static_cast<unsigned>(blocks_x), static_cast<unsigned>(f.segments), 1);
  FoldArgs args = f.args;
  void* kp[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&k_fold<TI, TO, OP, P, U, NT, M>), grid, dim3(kBlock),
                         kp, 0, s);
}

// Variants compiled for the tunable path (sum, p in {4, 8}): U in {1, 2, 4},
// nontemporal on/off.  Everything else uses U = 2 (U = 1 for p = 16) and
// ordinary loads/stores.
template <class TI, class TO, class OP, int P, FoldMode M>
hipError_t fold_variants(const FoldLaunch& f, hipStream_t s) {
  constexpr bool kTunable = __is_same(OP, OpSum) && (P == 4 || P == 8);
  if constexpr (kTunable) {
    const int u = f.unroll;
    const bool nt = f.nontemporal != 0;
    if (u == 1) return nt ? fold_go<TI, TO, OP, P, 1, true, M>(f, s) : fold_go<TI, TO, OP, P, 1, false, M>(f, s);
    if (u == 4) return nt ? fold_go<TI, TO, OP, P, 4, true, M>(f, s) : fold_go<TI, TO, OP, P, 4, false, M>(f, s);
    return nt ? fold_go<TI, TO, OP, P, 2, true, M>(f, s) : fold_go<TI, TO, OP, P, 2, false, M>(f, s);
  } else {
    constexpr int kU = (P >= 16) ? 1 : 2;
    return fold_go<TI, TO, OP, P, kU, false, M>(f, s);
  }
}

template <class TI, class TO, class OP, FoldMode M>
hipError_t fold_by_p(const FoldLaunch& f, hipStream_t s) {
  switch (f.args.p) {
    case 2: return fold_variants<TI, TO, OP, 2, M>(f, s);
    case 4: return fold_variants<TI, TO, OP, 4, M>(f, s);
    case 8: return fold_variants<TI, TO, OP, 8, M>(f, s);
    case 16: return fold_variants<TI, TO, OP, 16, M>(f, s);
    default: return fold_go<TI, TO, OP, 0, 2, false, M>(f, s);
  }
}

template <class TI, class TO, FoldMode M>
hipError_t fold_by_op(const FoldLaunch& f, hipStream_t s) {
  switch (f.op) {
    case RR_SUM: return fold_by_p<TI, TO, OpSum, M>(f, s);
    case RR_MAX: return fold_by_p<TI, TO, OpMax, M>(f, s);
    case RR_MIN: return fold_by_p<TI, TO, OpMin, M>(f, s);
    case RR_AVG:
      if constexpr (__is_same(typename TI::A, float)) return fold_by_p<TI, TO, OpAvg, M>(f, s);
      break;
  }
  return hipErrorInvalidValue;
}

// Mixed kinds (a 16-bit kind and float32 partials) take the run-time-p kernel.
template <class TI, class TO, FoldMode M>
hipError_t fold_mixed_by_op(const FoldLaunch& f, hipStream_t s) {
  switch (f.op) {
    case RR_SUM: return fold_go<TI, TO, OpSum, 0, 2, false, M>(f, s);
    case RR_MAX: return fold_go<TI, TO, OpMax, 0, 2, false, M>(f, s);
    case RR_MIN: return fold_go<TI, TO, OpMin, 0, 2, false, M>(f, s);
    case RR_AVG: return fold_go<TI, TO, OpAvg, 0, 2, false, M>(f, s);
  }
  return hipErrorInvalidValue;
}

// Same-kind folds for every mode; the mixed 16-bit <-> f32 pairs exist for the
// staged hierarchy (kAscOne writes float32 partials, kHierAll reads them).
template <FoldMode M>
hipError_t fold_by_kind(const FoldLaunch& f, hipStream_t s) {
  if (f.in_kind == f.out_kind) {
    switch (f.in_kind) {
      case Kind::kI32: return fold_by_op<EI32, EI32, M>(f, s);
      case Kind::kF32: return fold_by_op<EF32, EF32, M>(f, s);
      case Kind::kBF16: return fold_by_op<EBF16, EBF16, M>(f, s);
      case Kind::kF16: return fold_by_op<EF16, EF16, M>(f, s);
    }
    return hipErrorInvalidValue;
  }
  if constexpr (M == FoldMode::kAscOne || M == FoldMode::kHierAll) {
    if (f.in_kind == Kind::kBF16 && f.out_kind == Kind::kF32) return fold_mixed_by_op<EBF16, EF32, M>(f, s);
    if (f.in_kind == Kind::kF32 && f.out_kind == Kind::kBF16) return fold_mixed_by_op<EF32, EBF16, M>(f, s);
    if (f.in_kind == Kind::kF16 && f.out_kind == Kind::kF32) return fold_mixed_by_op<EF16, EF32, M>(f, s);
    if (f.in_kind == Kind::kF32 && f.out_kind == Kind::kF16) return fold_mixed_by_op<EF32, EF16, M>(f, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rr
