// rr_copy.hip -- data-movement kernels (gfx950): one-to-many copies
// (all-gather, broadcast), independent transfers (the ring's all-gather steps,
// the staged hierarchy's in-group broadcast), type conversions and the ring's
// reduce-scatter step.
//
// Page "分布式训练/推理", section "通信原语": broadcast copies one rank's tensor
// to every rank; all-gather gives every rank the concatenation of all shards.
// Page "LLM Parallelism 基础", section "Ring AllReduce": in a reduce-scatter
// step the receiver accumulates the incoming chunk into its own; in an
// all-gather step it overwrites its own chunk.
//
// Each lane moves whole units (16, 4, 2 or 1 bytes, the widest that every
// address and length allows); a lane loads U units and stores them to every
// destination, so a one-to-many copy reads its source once.
#include "rr_device.h"
#include "rr_kernels.h"

namespace rr {

namespace {

template <int B>
struct UnitT;
template <>
struct UnitT<16> {
  using T = u32x4;
};
template <>
struct UnitT<4> {
  using T = uint32_t;
};
template <>
struct UnitT<2> {
  using T = uint16_t;
};
template <>
struct UnitT<1> {
  using T = uint8_t;
};

// Units per lane per tile, and the default workgroup count of a copy: the
// measured best for 16-byte streaming copies on MI355X is two units per lane
// with about 8192 workgroups striding over the tiles.
constexpr int kCopyU = 2;
constexpr int kCopyGrid = 8192;
// Fan-out launches that write at most this many bytes use nontemporal stores.
constexpr uint64_t kFanoutNtStoreBytes = 128ull << 20;

template <bool NT, class T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(p);
  } else {
    return *p;
  }
}

template <bool NT, class T>
__device__ __forceinline__ void st(T* p, T v) {
  if constexpr (NT) {
    __builtin_nontemporal_store(v, p);
  } else {
    *p = v;
  }
}

// One source to p outputs.  NT: nontemporal loads; NTS: nontemporal stores
// (chosen by the bytes a launch writes, see launch_fanout).
template <int B, bool NT, int U = kCopyU, bool NTS = false>
__global__ __launch_bounds__(kBlock) void k_fanout(FanoutArgs a) {
  using T = typename UnitT<B>::T;
  const int seg = blockIdx.y;
  const uint64_t units = a.seg_bytes / B;
  const T* src = static_cast<const T*>(a.src[seg]);
  const uint64_t dst_off = static_cast<uint64_t>(seg) * (a.dst_seg_stride / B);
  constexpr uint64_t kTile = static_cast<uint64_t>(kBlock) * U;
  for (uint64_t base = static_cast<uint64_t>(blockIdx.x) * kTile + threadIdx.x; base < units;
       base += static_cast<uint64_t>(gridDim.x) * kTile) {
    T v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t i = base + static_cast<uint64_t>(u) * kBlock;
      if (i < units) v[u] = ld<NT>(src + i);
    }
    for (int r = 0; r < a.ndst; ++r) {
      if (r == seg && ((a.skip_diag >> seg) & 1ull)) continue;
      T* dst = static_cast<T*>(a.dst[r]) + dst_off;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t i = base + static_cast<uint64_t>(u) * kBlock;
        if (i < units) st<NTS>(dst + i, v[u]);
      }
    }
  }
}

// One-to-many copy laid out for the XCDs (16-byte units).  The sources are
// cut into blocks of kBlock units (4 KiB); a workgroup copies one block to D
// destinations and exits.  Block b belongs to XCD b mod kXcds; each XCD takes
// its blocks in windows of W, and inside a window destination group by
// destination group: W consecutive workgroups of the XCD write W consecutive
// blocks to group g, the next W write the same blocks to group g + 1, and so
// on.  The dispatcher deals workgroups to the XCDs in turn, so the workgroups
// of a window run on one XCD close together: a block, read with ordinary
// (cached) loads, comes from HBM once and from that XCD's L2 for the other
// groups, and every workgroup writes one 4 KiB block per destination, the
// store pattern at which HBM takes writes fastest.  Placement only affects
// speed: a workgroup that runs elsewhere reads its block again, with the same
// result.
//
// Workgroup w: x = w mod kXcds, j = w div kXcds, window v = j div (G W),
// group g = (j mod (G W)) div W, block b = (v W + j mod W) kXcds + x, with
// G = ceil(ndst / D); blocks are numbered segment by segment.  w ranges over
// kXcds * W * G * ceil(ceil(blocks / kXcds) / W), so blocks past the last and
// destinations past ndst exit.  The uniform block arithmetic is 32-bit (the
// host launches this kernel only when the grid, hence every block index, is
// below 2^31): no 64-bit comparison of uniform values steers a branch here.
constexpr int kXcds = 8;

template <int D>
__global__ __launch_bounds__(kBlock) void k_fanout_xcd(FanoutArgs a, uint32_t blocks_per_seg, uint32_t blocks,
                                                       uint32_t W) {
  const uint32_t w = blockIdx.x;
  const uint32_t x = w % kXcds;
  const uint32_t j = w / kXcds;
  const uint32_t G = (static_cast<uint32_t>(a.ndst) + D - 1) / D;
  const uint32_t v = j / (G * W);
  const uint32_t rem = j - v * G * W;
  const uint32_t g = rem / W;
  const uint32_t b = (v * W + (rem - g * W)) * kXcds + x;
  if (b >= blocks) return;
  const int seg = static_cast<int>(b / blocks_per_seg);
  const uint64_t units = a.seg_bytes / 16;
  const uint64_t i = static_cast<uint64_t>(b - static_cast<uint32_t>(seg) * blocks_per_seg) * kBlock + threadIdx.x;
  if (i >= units) return;
  const u32x4 val = static_cast<const u32x4*>(a.src[seg])[i];
  const uint64_t dst_off = static_cast<uint64_t>(seg) * (a.dst_seg_stride / 16);
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int r = static_cast<int>(g) * D + d;
    if (r >= a.ndst) break;
    if (r == seg && ((a.skip_diag >> seg) & 1ull)) continue;
    __builtin_nontemporal_store(val, static_cast<u32x4*>(a.dst[r]) + dst_off + i);
  }
}

template <int B, bool NT>
__global__ __launch_bounds__(kBlock) void k_copy_pairs(PairArgs a) {
  using T = typename UnitT<B>::T;
  const int y = blockIdx.y;
  const uint64_t units = a.len[y] / B;
  const T* src = static_cast<const T*>(a.src[y]);
  T* dst = static_cast<T*>(a.dst[y]);
  constexpr uint64_t kTile = static_cast<uint64_t>(kBlock) * kCopyU;
  for (uint64_t base = static_cast<uint64_t>(blockIdx.x) * kTile + threadIdx.x; base < units;
       base += static_cast<uint64_t>(gridDim.x) * kTile) {
    T v[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint64_t i = base + static_cast<uint64_t>(u) * kBlock;
      if (i < units) v[u] = ld<NT>(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint64_t i = base + static_cast<uint64_t>(u) * kBlock;
      if (i < units) st<NT>(dst + i, v[u]);
    }
  }
}

// Element-wise conversion (16-bit kinds <-> f32 for the staged paths, with
// AVG's division when a.div > 0) or the ring's reduce-scatter step
// (dst = src (+) aux, message first; aux is the receiver's own value, its
// buffer or, before the receiver has written that chunk, its input).  8 elements per group on the vector
// path, scalar otherwise (and for the last partial group).
template <class EF, class ET, class OP, bool STEP>
__global__ __launch_bounds__(kBlock) void k_pairs_elem(PairArgs a) {
  constexpr int V = 8;
  using A = typename EF::A;
  const int y = blockIdx.y;
  const uint64_t n = a.len[y];
  const typename EF::S* src = static_cast<const typename EF::S*>(a.src[y]);
  typename ET::S* dst = static_cast<typename ET::S*>(a.dst[y]);
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
  const uint64_t ngroups = a.vec ? n / V : 0;
  for (uint64_t g = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; g < ngroups; g += stride) {
    Raw<EF, V> rs;
    load_group<false>(rs, src + g * V);
    A x[V];
    unpack(rs, x);
    if constexpr (STEP) {
      Raw<ET, V> rd;
      load_group<false>(rd, static_cast<const typename ET::S*>(a.aux[y]) + g * V);
      A d[V];
      unpack(rd, d);
#pragma unroll
      for (int j = 0; j < V; ++j) x[j] = OP::apply(x[j], d[j]);
    } else if constexpr (__is_same(A, float)) {
      if (a.div > 0) {
#pragma unroll
        for (int j = 0; j < V; ++j) x[j] = x[j] / static_cast<float>(a.div);
      }
    }
    Raw<ET, V> o;
    pack(x, o);
    store_group<false>(dst + g * V, o);
  }
  for (uint64_t i = ngroups * V + static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
    A x = load_one<EF>(src + i);
    if constexpr (STEP) {
      x = OP::apply(x, load_one<ET>(static_cast<const typename ET::S*>(a.aux[y]) + i));
    } else if constexpr (__is_same(A, float)) {
      if (a.div > 0) x = x / static_cast<float>(a.div);
    }
    store_one<ET>(dst + i, x);
  }
}

uint64_t blocks_for(uint64_t units, uint64_t per_block, int rows, int grid_cap) {
  uint64_t b = (units + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (grid_cap > 0) {
    uint64_t cap = static_cast<uint64_t>(grid_cap) / static_cast<uint64_t>(rows > 0 ? rows : 1);
    if (cap < 1) cap = 1;
    if (b > cap) b = cap;
  }
  if (b > 0x7FFFFFFFull) b = 0x7FFFFFFFull;
  return b;
}

template <class K, class ARGS>
hipError_t go(K kernel, const ARGS& args, uint64_t bx, int rows, hipStream_t s) {
  ARGS copy = args;
  void* kp[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(bx), rows, 1),
                         dim3(kBlock), kp, 0, s);
}

template <class EF, class ET, class OP, bool STEP>
hipError_t pairs_elem(const PairArgs& a, int grid_cap, hipStream_t s) {
  uint64_t longest = 0;
  for (int y = 0; y < a.npairs; ++y) longest = a.len[y] > longest ? a.len[y] : longest;
  const uint64_t bx = blocks_for(a.vec ? longest / 8 + 1 : longest, kBlock, a.npairs, grid_cap);
  return go(&k_pairs_elem<EF, ET, OP, STEP>, a, bx, a.npairs, s);
}

template <class E>
hipError_t ring_step_kind(const PairArgs& a, rr_op_t op, int grid_cap, hipStream_t s) {
  switch (op) {
    case RR_SUM: return pairs_elem<E, E, OpSum, true>(a, grid_cap, s);
    case RR_MAX: return pairs_elem<E, E, OpMax, true>(a, grid_cap, s);
    case RR_MIN: return pairs_elem<E, E, OpMin, true>(a, grid_cap, s);
    case RR_AVG: return pairs_elem<E, E, OpSum, true>(a, grid_cap, s);  // partial sums; the division comes last
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fanout(const FanoutArgs& a, int unit_bytes, int nontemporal, int grid_cap, int units_per_lane,
                         int xcd_dst, int xcd_window, hipStream_t s) {
  const uint64_t units = a.seg_bytes / static_cast<uint64_t>(unit_bytes);
  const bool nt = nontemporal != 0;
  if (unit_bytes == 16 && nt && grid_cap == 0 && xcd_dst != 0) {
    // The XCD layout (k_fanout_xcd), two destinations per workgroup, windows
    // of one block, for launches that write more than kFanoutNtStoreBytes
    // (128 MiB); smaller ones keep the tile kernel below, with nontemporal
    // stores.  All-gather p = 8 at 12 / 16 / 18 / 20 / 22 MiB per rank, tile
    // kernel -> XCD layout: 78.6 -> 75.1, 70.7 -> 71.4, 69.5 -> 81.2, 72.5
    // -> 78.0, 66.6 -> 84.8% of the HBM peak; broadcast 16 / 20 MiB 71.8 ->
    // 70.8, 73.8 -> 78.3%; bfloat16 all-gather 20 MiB 72.7 -> 78.9%.  Measured on MI355X against the tile
    // kernel, % of the 8 TB/s HBM peak, the launch's buffers among two
    // rotating sets: all-gather p = 8 at 24 / 32 / 64 / 96 / 128 MiB per rank
    // 66.8 -> 80.7, 66.7 -> 78.4, 66.5 -> 76.5, 68.3 -> 86.6-87.4, 65.4 ->
    // 73.6; broadcast p = 8 of 96 MiB 67.5 -> 72.6-86; p = 4, 96 MiB per rank
    // 71.4 -> 74.1; p = 16, 48 MiB per rank 63.9 -> 81.4.  At 8 and 16 MiB
    // per rank it lost (71.5 -> 55, 69 -> 67).  The layout is fast while the
    // GPU's address translations of the buffers are cached: with a 4 GiB
    // sweep of other memory between launches it falls to the tile kernel's
    // rate (66-67%), where one destination per workgroup, faster still with
    // warm translations (81-91%), falls to 46-49%; so two destinations it is.
    const uint64_t written = a.seg_bytes * static_cast<uint64_t>(a.nseg) * static_cast<uint64_t>(a.ndst);
    int D = xcd_dst;
    if (D < 0) D = written > kFanoutNtStoreBytes ? 2 : 0;
    const uint32_t W = xcd_window > 0 ? static_cast<uint32_t>(xcd_window) : 1u;
    if (D == 1 || D == 2 || D == 4) {
      const uint64_t bps = (units + kBlock - 1) / kBlock;
      const uint64_t blocks = bps * static_cast<uint64_t>(a.nseg);
      const uint64_t G = (static_cast<uint64_t>(a.ndst) + D - 1) / D;
      const uint64_t per_xcd = (blocks + kXcds - 1) / kXcds;
      const uint64_t grid = (per_xcd + W - 1) / W * W * G * kXcds;
      if (grid <= 0x7FFFFFFFull) {
        FanoutArgs copy = a;
        uint32_t bps_arg = static_cast<uint32_t>(bps);
        uint32_t blocks_arg = static_cast<uint32_t>(blocks);
        uint32_t w_arg = W;
        void* kp[] = {&copy, &bps_arg, &blocks_arg, &w_arg};
        const void* k = D == 1 ? reinterpret_cast<const void*>(&k_fanout_xcd<1>)
                               : (D == 2 ? reinterpret_cast<const void*>(&k_fanout_xcd<2>)
                                         : reinterpret_cast<const void*>(&k_fanout_xcd<4>));
        return hipLaunchKernel(k, dim3(static_cast<unsigned>(grid)), dim3(kBlock), kp, 0, s);
      }
    }
  }
  if (unit_bytes == 16) {
    // 16-byte units: `units_per_lane` (1, 2, 4 or 8) per lane, and without a
    // cap one tile per workgroup.  A grid that strides leaves some
    // workgroups one tile more than others at the end of the launch; at 96
    // MiB per rank (768 tiles of 4 units per lane per shard) one tile each
    // measured 64.0% -> 68.3% of the HBM peak for all-gather and 64.3% ->
    // 67.9% for broadcast against 8192 striding workgroups of 2 units per
    // lane; 8 MiB per rank is within noise (68.3-69.3%) for every choice.
    //
    // Stores: nontemporal while the launch writes at most kFanoutNtStoreBytes
    // (half the 256 MB Infinity Cache), plain above.  Sweep with cold
    // sources, all-gather and broadcast alike, plain -> nontemporal: 4 / 8 /
    // 16 MiB per rank (32-128 MiB written) 55.5 -> 65.0%, 67.9 -> 72.1%,
    // 66.7 -> 69.4% of the HBM peak; 24 / 32 / 48 / 64 / 96 MiB per rank
    // 68.4 -> 67.0%, 66.5 -> 65.5%, 67.6 -> 64.4%, 66.7 -> 63.5%,
    // 67.8 -> 63.5%.
    const int u = (units_per_lane == 1 || units_per_lane == 2 || units_per_lane == 8) ? units_per_lane : 4;
    const uint64_t bx = blocks_for(units, static_cast<uint64_t>(kBlock) * u, a.nseg, grid_cap);
    const uint64_t written = a.seg_bytes * static_cast<uint64_t>(a.nseg) * static_cast<uint64_t>(a.ndst);
    if (nt && written <= kFanoutNtStoreBytes) {
      switch (u) {
        case 1: return go(&k_fanout<16, true, 1, true>, a, bx, a.nseg, s);
        case 2: return go(&k_fanout<16, true, 2, true>, a, bx, a.nseg, s);
        case 8: return go(&k_fanout<16, true, 8, true>, a, bx, a.nseg, s);
        default: return go(&k_fanout<16, true, 4, true>, a, bx, a.nseg, s);
      }
    }
    switch (u) {
      case 1: return nt ? go(&k_fanout<16, true, 1>, a, bx, a.nseg, s) : go(&k_fanout<16, false, 1>, a, bx, a.nseg, s);
      case 2: return nt ? go(&k_fanout<16, true, 2>, a, bx, a.nseg, s) : go(&k_fanout<16, false, 2>, a, bx, a.nseg, s);
      case 8: return nt ? go(&k_fanout<16, true, 8>, a, bx, a.nseg, s) : go(&k_fanout<16, false, 8>, a, bx, a.nseg, s);
      default: return nt ? go(&k_fanout<16, true, 4>, a, bx, a.nseg, s) : go(&k_fanout<16, false, 4>, a, bx, a.nseg, s);
    }
  }
  const uint64_t bx =
      blocks_for(units, static_cast<uint64_t>(kBlock) * kCopyU, a.nseg, grid_cap > 0 ? grid_cap : kCopyGrid);
  switch (unit_bytes) {
    case 4: return nt ? go(&k_fanout<4, true>, a, bx, a.nseg, s) : go(&k_fanout<4, false>, a, bx, a.nseg, s);
    case 2: return nt ? go(&k_fanout<2, true>, a, bx, a.nseg, s) : go(&k_fanout<2, false>, a, bx, a.nseg, s);
    case 1: return nt ? go(&k_fanout<1, true>, a, bx, a.nseg, s) : go(&k_fanout<1, false>, a, bx, a.nseg, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_copy_pairs(const PairArgs& a, int unit_bytes, int nontemporal, int grid_cap, hipStream_t s) {
  uint64_t longest = 0;
  for (int y = 0; y < a.npairs; ++y) longest = a.len[y] > longest ? a.len[y] : longest;
  const uint64_t bx = blocks_for(longest / static_cast<uint64_t>(unit_bytes), static_cast<uint64_t>(kBlock) * kCopyU,
                                 a.npairs, grid_cap > 0 ? grid_cap : kCopyGrid);
  const bool nt = nontemporal != 0;
  switch (unit_bytes) {
    case 16: return nt ? go(&k_copy_pairs<16, true>, a, bx, a.npairs, s) : go(&k_copy_pairs<16, false>, a, bx, a.npairs, s);
    case 4: return nt ? go(&k_copy_pairs<4, true>, a, bx, a.npairs, s) : go(&k_copy_pairs<4, false>, a, bx, a.npairs, s);
    case 2: return nt ? go(&k_copy_pairs<2, true>, a, bx, a.npairs, s) : go(&k_copy_pairs<2, false>, a, bx, a.npairs, s);
    case 1: return nt ? go(&k_copy_pairs<1, true>, a, bx, a.npairs, s) : go(&k_copy_pairs<1, false>, a, bx, a.npairs, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_convert_pairs(const PairArgs& a, Kind from, Kind to, int grid_cap, hipStream_t s) {
  if (from == Kind::kBF16 && to == Kind::kF32) return pairs_elem<EBF16, EF32, OpSum, false>(a, grid_cap, s);
  if (from == Kind::kF32 && to == Kind::kBF16) return pairs_elem<EF32, EBF16, OpSum, false>(a, grid_cap, s);
  if (from == Kind::kF16 && to == Kind::kF32) return pairs_elem<EF16, EF32, OpSum, false>(a, grid_cap, s);
  if (from == Kind::kF32 && to == Kind::kF16) return pairs_elem<EF32, EF16, OpSum, false>(a, grid_cap, s);
  if (from == Kind::kF32 && to == Kind::kF32) return pairs_elem<EF32, EF32, OpSum, false>(a, grid_cap, s);
  return hipErrorInvalidValue;
}

hipError_t launch_ring_step(const PairArgs& a, Kind acc_kind, rr_op_t op, int grid_cap, hipStream_t s) {
  switch (acc_kind) {
    case Kind::kI32: return ring_step_kind<EI32>(a, op, grid_cap, s);
    case Kind::kF32: return ring_step_kind<EF32>(a, op, grid_cap, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fold(const FoldLaunch& f, hipStream_t s) {
  switch (f.mode) {
    case FoldMode::kRingAll: return launch_fold_ring_all(f, s);
    case FoldMode::kRingShard: return launch_fold_ring_shard(f, s);
    case FoldMode::kAscOne: return launch_fold_asc_one(f, s);
    case FoldMode::kHierAll: return launch_fold_hier_all(f, s);
    case FoldMode::kHierRing:
    case FoldMode::kHierAllWire:
    case FoldMode::kHierRingWire: return launch_fold_hier_var(f, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rr
