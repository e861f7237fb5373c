// rr_multi.hip -- collectives over many tensors and over strided layouts
// (gfx950): the bucketed all-reduce, and the two tensor-parallel layouts
// (all-gather along dim 1, reduce-scatter along dim 1).
//
// Bucketed all-reduce: page "分布式训练/推理", section "Ring all-reduce 的带宽账"
// (the gradients are flattened and all-reduced in one call instead of one
// call per parameter, which cuts the fixed cost per call) and page
// "分布式训练——如何把大模型分到多张卡上" (DDP synchronises gradients in buckets;
// gradient_as_bucket_view keeps each gradient as a view of its bucket).  A
// bucket is the concatenation of its tensors; the ring cuts the bucket, not
// each tensor, into p chunks, so element e of the bucket folds
// x_{c+1}, ..., x_c where c is the bucket chunk holding e.  No bucket is ever
// materialised: the host cuts every tensor at the chunk bounds into pieces
// and one launch folds up to kBucketPieces pieces of many tensors in place.
//
// Tensor-parallel layouts: page "分布式训练/推理", tensor-parallel section.
// The column-parallel outputs [B, d/p] of the p ranks are concatenated along
// dim 1 on every rank; in the scatter strategy the partial [B, D] outputs are
// summed over ranks and rank c keeps feature slice c (psum_scatter).  Slice c
// is chunk c of the ring over the feature dimension, so its fold order is
// x_{c+1}, ..., x_c, as for reduce-scatter.
//
// All three are HBM streams: every input byte is read once and every output
// byte written once; the reduction across ranks happens in each lane's
// registers.
#include <type_traits>

#include "rr_device.h"
#include "rr_kernels.h"
#include "rr_sync.h"

namespace rr {

namespace {

// Fold U units per lane over the p ranks, the k-th term (k = 0..p-1) from
// rank (rot + 1 + k) mod p.  Unit u of the lane sits off[u] bytes into every
// rank's buffer `ptr[rank]`.  A unit is a 16-byte group of V elements (VEC)
// or one element.  The next rank's loads are issued before the current
// rank's values are folded.
template <class E, class OP, int U, bool VEC>
struct RotFold {
  using S = typename E::S;
  using A = typename E::A;
  static constexpr int V = VEC ? 16 / static_cast<int>(sizeof(S)) : 1;
  using Unit = typename std::conditional<VEC, Raw<E, (VEC ? 16 / sizeof(S) : 8)>, S>::type;

  __device__ __forceinline__ static void load(Unit (&x)[U], const char* base, const uint64_t (&off)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (VEC) {
        load_group<true>(x[u], reinterpret_cast<const S*>(base + off[u]));
      } else {
        x[u] = __builtin_nontemporal_load(reinterpret_cast<const S*>(base + off[u]));
      }
    }
  }

  __device__ __forceinline__ static void widen(const Unit& x, A (&a)[V]) {
    if constexpr (VEC) {
      unpack(x, a);
    } else if constexpr (sizeof(S) == 2) {
      a[0] = half_to_f32<E>(static_cast<uint32_t>(x));
    } else {
      a[0] = x;
    }
  }

  __device__ __forceinline__ static void run(const void* const* ptr, int rot, int p, const uint64_t (&off)[U],
                                             int32_t div, A (&acc)[U][V]) {
    int r = rot + 1 >= p ? rot + 1 - p : rot + 1;
    Unit cur[U];
    Unit nxt[U];
    load(cur, static_cast<const char*>(ptr[r]), off);
    int rn = r + 1 >= p ? 0 : r + 1;
    if (p > 1) load(nxt, static_cast<const char*>(ptr[rn]), off);
#pragma unroll
    for (int u = 0; u < U; ++u) widen(cur[u], acc[u]);
#pragma unroll 1
    for (int k = 1; k < p; ++k) {
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
      rn = rn + 1 >= p ? 0 : rn + 1;
      if (k + 1 < p) load(nxt, static_cast<const char*>(ptr[rn]), off);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        A x[V];
        widen(cur[u], x);
#pragma unroll
        for (int j = 0; j < V; ++j) acc[u][j] = OP::apply(acc[u][j], x[j]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < V; ++j) acc[u][j] = op_finish<OP>(acc[u][j], div);
  }

  // Convert once and store unit u to `dst + off`.
  __device__ __forceinline__ static void store(char* dst, uint64_t off, const A (&a)[V]) {
    if constexpr (VEC) {
      Raw<E, V> o;
      pack(a, o);
      store_group<true>(reinterpret_cast<S*>(dst + off), o);
    } else {
      store_one<E>(reinterpret_cast<S*>(dst + off), a[0]);
    }
  }
};

// ---------------------------------------------------------------------------
// Bucketed all-reduce.

// Tile k of piece pc: byte offsets of the lane's units (lanes past the end
// re-read the tile's last unit; never stored) and the valid unit count.
// IL (the kernel with the barrier): the whole tiles at the start of a vector
// piece are taken in runs of a.strips tiles whose strips interleave.
template <class E, bool VEC, bool IL, int U>
__device__ __forceinline__ uint32_t bucket_offsets(const BucketArgs& a, int pc, uint32_t k, uint64_t (&off)[U]) {
  constexpr uint32_t kUnits = static_cast<uint32_t>(kBlock) * U;
  constexpr uint32_t kUnitBytes = VEC ? 16u : static_cast<uint32_t>(sizeof(typename E::S));
  const uint32_t lane = threadIdx.x;
  if constexpr (IL && VEC) {
    const uint32_t S = a.strips;
    const uint32_t whole = a.units[pc] / kUnits;
    if (S > 1 && k < whole - whole % S) {
      const uint32_t run = k / S;
      const uint32_t j = k - run * S;
      const uint64_t base =
          a.start[pc] * sizeof(typename E::S) + (static_cast<uint64_t>(run) * S * kUnits + j * kBlock) * kUnitBytes;
#pragma unroll
      for (int u = 0; u < U; ++u) off[u] = base + static_cast<uint64_t>(lane + u * S * kBlock) * kUnitBytes;
      return kUnits;
    }
  }
  const uint32_t valid = min(kUnits, a.units[pc] - k * kUnits);  // units of this tile, >= 1
  const uint64_t base = a.start[pc] * sizeof(typename E::S) + static_cast<uint64_t>(k) * kUnits * kUnitBytes;
#pragma unroll
  for (int u = 0; u < U; ++u) off[u] = base + min(lane + u * kBlock, valid - 1) * kUnitBytes;
  return valid;
}

// Write the folded tile to all p outputs of piece pc.
template <class E, class OP, bool VEC, int U>
__device__ __forceinline__ void bucket_store(const BucketArgs& a, int pc, uint32_t valid, const uint64_t (&off)[U],
                                             const typename E::A (&acc)[U][RotFold<E, OP, U, VEC>::V]) {
  using F = RotFold<E, OP, U, VEC>;
  const uint32_t lane = threadIdx.x;
  const int p = a.p;
  for (int r = 0; r < p; ++r) {
    char* d = static_cast<char*>(const_cast<void*>(a.ptr[a.base[pc] + p + r]));
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (lane + u * kBlock < valid) F::store(d, off[u], acc[u]);
  }
}

// The piece of tile t: the last piece whose first tile is <= t.
__device__ __forceinline__ int bucket_piece(const BucketArgs& a, uint32_t t) {
  int lo = 0;
  int hi = a.npieces - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.tile0[mid] <= t) {
      lo = mid;
    } else {
      hi = mid - 1;
    }
  }
  return lo;
}

// Rounds of K tiles per workgroup: tile t = (round*K + j)*gridDim.x +
// blockIdx.x, j < K.  In a round a workgroup folds its tiles from every rank
// into registers, then writes them to every output.  SYNC (several rounds,
// or one batched round): the workgroups meet at the soft barrier between
// the two phases, and with K > 1 again between a round's writes and the
// next round's reads, so that for the length of a phase the device only
// reads, or only writes (as in the phased fold's batched rounds; a 96 MiB
// bucket of 4 float32 tensors 77% -> 79% of the HBM peak, 64 MiB of 2
// tensors 70% -> 73%).  Tiles of scalar pieces (elements
// of tensors that are not 16-byte aligned) are written before the barrier.
template <class E, class OP, bool SYNC, int K, int U>
__global__ __launch_bounds__(kBlock) void k_bucket(BucketArgs a) {
  using FV = RotFold<E, OP, U, true>;
  using FS = RotFold<E, OP, U, false>;
  if constexpr (SYNC) sync_claim_at(a.sync.slot, a.sync.tag);
  for (uint32_t r = 0; r < a.rounds; ++r) {
    int pc[K];
    bool vec[K];
    uint32_t valid[K];
    uint64_t off[K][U];
    typename E::A acc[K][U][FV::V];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t t = (r * K + j) * gridDim.x + blockIdx.x;
      vec[j] = false;
      pc[j] = 0;
      valid[j] = 0;
      if (t < a.tiles) {
        pc[j] = bucket_piece(a, t);
        const uint32_t k = t - a.tile0[pc[j]];
        vec[j] = a.vec[pc[j]] != 0;
        if (vec[j]) {
          valid[j] = bucket_offsets<E, true, SYNC, U>(a, pc[j], k, off[j]);
          FV::run(a.ptr + a.base[pc[j]], a.rot[pc[j]], a.p, off[j], a.div, acc[j]);
        } else {
          typename E::A one[U][FS::V];
          const uint32_t n1 = bucket_offsets<E, false, SYNC, U>(a, pc[j], k, off[j]);
          FS::run(a.ptr + a.base[pc[j]], a.rot[pc[j]], a.p, off[j], a.div, one);
          bucket_store<E, OP, false, U>(a, pc[j], n1, off[j], one);
        }
      }
    }
    if constexpr (SYNC) soft_barrier_at(a.sync.slot, a.sync.tag, a.sync.timeout_ticks, K > 1 ? 2 * r : r);
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (vec[j]) bucket_store<E, OP, true, U>(a, pc[j], valid[j], off[j], acc[j]);
    if constexpr (SYNC && K > 1) {
      if (r + 1 < a.rounds) soft_barrier_at(a.sync.slot, a.sync.tag, a.sync.timeout_ticks, 2 * r + 1);
    }
  }
}

// ---------------------------------------------------------------------------
// Reduce-scatter along dim 1.  Row b of output c holds w elements: unit i of
// output c (i = b*wu + j) reads unit b*du + c*wu + j of every input.  IDX is
// the index type: 32-bit when rows*du < 2^32 (cheap division), else 64-bit.

template <class IDX>
__device__ __forceinline__ void row_split(IDX i, IDX w, IDX& b, IDX& j) {
  b = i / w;
  j = i - b * w;
}

template <class E, class OP, bool VEC, class IDX>
__global__ __launch_bounds__(kBlock) void k_fold_cols(ColsArgs a) {
  constexpr int U = 4;
  using F = RotFold<E, OP, U, VEC>;
  constexpr uint64_t kUnitBytes = VEC ? 16 : sizeof(typename E::S);
  const int c = blockIdx.y;
  const int p = a.p;
  const IDX wu = static_cast<IDX>(a.wu);
  const IDX du = static_cast<IDX>(a.du);
  const IDX total = static_cast<IDX>(a.rows) * wu;
  const IDX col0 = static_cast<IDX>(c) * wu;
  const IDX stride = static_cast<IDX>(gridDim.x) * kBlock * U;
  char* d = static_cast<char*>(a.dst[c]);
  for (IDX t0 = static_cast<IDX>(blockIdx.x) * kBlock * U; t0 < total; t0 += stride) {
    uint64_t in_off[U];
    uint64_t out_off[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      IDX i = t0 + threadIdx.x + static_cast<IDX>(u) * kBlock;
      ok[u] = i < total;
      if (!ok[u]) i = total - 1;  // re-read a valid unit; never stored
      IDX b, j;
      row_split(i, wu, b, j);
      in_off[u] = (static_cast<uint64_t>(b) * du + col0 + j) * kUnitBytes;
      out_off[u] = static_cast<uint64_t>(i) * kUnitBytes;
    }
    typename E::A acc[U][F::V];
    F::run(a.src, c, p, in_off, a.div, acc);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) F::store(d, out_off[u], acc[u]);
  }
}

// ---------------------------------------------------------------------------
// All-gather along dim 1, walked in output order: unit i of every output
// (row b = i / du, column unit q = i % du) comes from source c = q / wu,
// unit b*wu + (q - c*wu).  Consecutive lanes write consecutive units of all p
// outputs (long contiguous runs at the same offsets) and read runs of wu
// units from one source.

template <int B>
struct Word;
template <>
struct Word<16> {
  using T = u32x4;
};
template <>
struct Word<4> {
  using T = uint32_t;
};
template <>
struct Word<2> {
  using T = uint16_t;
};
template <>
struct Word<1> {
  using T = uint8_t;
};

template <int B, bool NT, class IDX>
__global__ __launch_bounds__(kBlock) void k_gather_cols(ColsArgs a) {
  using T = typename Word<B>::T;
  constexpr int U = 4;
  const IDX wu = static_cast<IDX>(a.wu);
  const IDX du = static_cast<IDX>(a.du);
  const IDX total = static_cast<IDX>(a.rows) * du;
  const IDX stride = static_cast<IDX>(gridDim.x) * kBlock * U;
  for (IDX t0 = static_cast<IDX>(blockIdx.x) * kBlock * U; t0 < total; t0 += stride) {
    T v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const IDX i = t0 + threadIdx.x + static_cast<IDX>(u) * kBlock;
      const IDX ic = i < total ? i : total - 1;
      IDX b, q, c, j;
      row_split(ic, du, b, q);
      row_split(q, wu, c, j);
      const T* src = static_cast<const T*>(a.src[c]) + static_cast<uint64_t>(b) * wu + j;
      if constexpr (NT) {
        v[u] = __builtin_nontemporal_load(src);
      } else {
        v[u] = *src;
      }
    }
    for (int r = 0; r < a.p; ++r) {
      T* dst = static_cast<T*>(a.dst[r]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const IDX i = t0 + threadIdx.x + static_cast<IDX>(u) * kBlock;
        if (i < total) {
          if constexpr (NT) {
            __builtin_nontemporal_store(v[u], dst + i);
          } else {
            dst[i] = v[u];
          }
        }
      }
    }
  }
}

// All-gather along dim 1 in the XCD layout of the fan-out (k_fanout_xcd in
// rr_copy.hip): the outputs are cut into blocks of kBlock 16-byte units (4
// KiB); a workgroup moves one block to D destinations and exits.  Block b
// belongs to XCD b mod 8, and the G = ceil(p / D) workgroups of a block are
// congruent modulo 8 and consecutive in that XCD's dispatch order (the
// dispatcher deals workgroups to the 8 XCDs in turn), so the block's source
// runs are read from HBM once, with ordinary cached loads, and from the XCD's
// L2 by the others.  Workgroup w: XCD x = w mod 8, j = w / 8, block
// (j / G) * 8 + x, destinations (j mod G) * D ...  Placement only decides
// speed: a workgroup that lands elsewhere reads its source again.  All
// uniform index arithmetic is 32-bit; only the per-lane unit index is wider.
template <int D, class IDX>
__global__ __launch_bounds__(kBlock) void k_gather_cols_xcd(ColsArgs a, uint32_t G, uint32_t blocks) {
  const uint32_t w = blockIdx.x;
  const uint32_t x = w % 8;
  const uint32_t j = w / 8;
  const uint32_t v = j / G;
  const uint32_t g = j - v * G;
  const uint32_t blk = v * 8 + x;
  if (blk >= blocks) return;
  const IDX wu = static_cast<IDX>(a.wu);
  const IDX du = static_cast<IDX>(a.du);
  const IDX total = static_cast<IDX>(a.rows) * du;
  const IDX i = static_cast<IDX>(blk) * kBlock + threadIdx.x;
  if (i >= total) return;
  IDX b, q, c, jj;
  row_split(i, du, b, q);
  row_split(q, wu, c, jj);
  const u32x4 val = static_cast<const u32x4*>(a.src[c])[static_cast<uint64_t>(b) * wu + jj];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int r = static_cast<int>(g) * D + d;
    if (r >= a.p) break;
    __builtin_nontemporal_store(val, static_cast<u32x4*>(a.dst[r]) + i);
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch.

constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices];

// Compute units of the stream's device (0 if unknown), read once per device.
int cus_of(hipStream_t s) {
  int dev = 0;
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return 0;
  int v = __atomic_load_n(&g_cus[dev], __ATOMIC_RELAXED);
  if (v == 0 && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    __atomic_store_n(&g_cus[dev], v, __ATOMIC_RELAXED);
  return v;
}

template <class K, class ARGS>
hipError_t launch(K kernel, const ARGS& args, dim3 grid, hipStream_t s) {
  ARGS copy = args;
  void* kp[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(kBlock), kp, 0, s);
}

// Workgroups of a streaming launch: per_cu per compute unit, never more than
// there is work.  Defaults (measured): 32 per CU for the dim-1 layouts (the
// grid oversubscribes the device, about one tile per workgroup), 4 for the
// bucket.
constexpr int kColsPerCu = 32;
constexpr int kBucketPerCu = 4;
// Tiles per workgroup and round of the batched bucket kernel.
constexpr int kBucketBatch = 4;

unsigned stream_grid(uint64_t work_units, uint64_t per_block, int rows, int per_cu, hipStream_t s) {
  const int cus = cus_of(s);
  uint64_t cap = static_cast<uint64_t>(cus > 0 ? cus : 256) * static_cast<uint64_t>(per_cu);
  cap = (cap + static_cast<uint64_t>(rows) - 1) / static_cast<uint64_t>(rows);
  uint64_t g = (work_units + per_block - 1) / per_block;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return static_cast<unsigned>(g);
}

// Workgroups of k_bucket<..., true, K, kBucketU> that one compute unit keeps
// resident, per (kind, op, K), queried once.
template <class E, class OP, int K>
int bucket_occupancy() {
  static int occ = 0;
  int v = __atomic_load_n(&occ, __ATOMIC_RELAXED);
  if (v == 0) {
    const void* kernel = reinterpret_cast<const void*>(&k_bucket<E, OP, true, K, kBucketU>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, kBlock, 0) != hipSuccess || v < 1)
      v = 1;
    __atomic_store_n(&occ, v, __ATOMIC_RELAXED);
  }
  return v;
}

template <class E, class OP>
hipError_t bucket_go(BucketArgs a, int per_cu, int sync, int batch, int timeout_us, hipStream_t s) {
  unsigned grid = stream_grid(a.tiles, 1, 1, per_cu > 0 ? per_cu : kBucketPerCu, s);
  a.rounds = (a.tiles + grid - 1) / grid;
  if (sync && a.rounds > 1) {
    hipError_t e = phase_sync_args(s, timeout_us, &a.sync);
    if (e != hipSuccess) return e;
    e = sync_reset_if_captured(a.sync, s);
    if (e != hipSuccess) return e;
    const int cus = cus_of(s);
    const uint64_t ncu = static_cast<uint64_t>(cus > 0 ? cus : 256);
    if (batch != 1) {
      // Batched rounds: kBucketBatch tiles per workgroup and round at 3 or
      // 2 workgroups per CU (capped at the occupancy), whichever leaves
      // fewer empty tile slots in the last round (ties: fewer rounds); a
      // single round may be partial.  Interleaved runs of 8 tiles.
      // Measured through this library on one MI355X, float32 p = 8, against
      // one tile per workgroup and round at 4 per CU (runs of 2 from three
      // rounds on): a GPT-2 block's 12 gradients (27 MiB per rank, AVG)
      // 68.3% -> 74.5% of the HBM peak, one 27 MiB tensor 70.2% -> 73.6%, 4
      // tensors of 24 MiB 76.8% -> 78.1%; runs of 1 / 2 / 4 / 16 tiles gave
      // 69.4 / 70.3 / 72.1 / 73.6% on the GPT-2 block.
      constexpr int K = kBucketBatch;
      const uint64_t occ = static_cast<uint64_t>(bucket_occupancy<E, OP, K>());
      uint64_t best = 0, best_waste = ~0ull;
      const uint64_t asked = per_cu > 0 ? static_cast<uint64_t>(per_cu) : 0;
      for (uint64_t c : {asked ? asked : 3ull, asked ? asked : 2ull}) {
        const uint64_t pc = c < occ ? c : occ;
        const uint64_t slots = ncu * pc * K;
        const uint64_t waste = (a.tiles + slots - 1) / slots * slots - a.tiles;
        if (waste < best_waste) {
          best_waste = waste;
          best = pc;
        }
      }
      grid = static_cast<unsigned>(ncu * best);
      a.rounds = static_cast<uint32_t>((a.tiles + static_cast<uint64_t>(grid) * K - 1) / (static_cast<uint64_t>(grid) * K));
      if (a.strips == 0) a.strips = 8;
      return launch(&k_bucket<E, OP, true, K, kBucketU>, a, dim3(grid), s);
    }
    // the barrier needs every workgroup resident at once
    const uint64_t resident = ncu * bucket_occupancy<E, OP, 1>();
    if (grid > resident) grid = static_cast<unsigned>(resident);
    a.rounds = (a.tiles + grid - 1) / grid;
    // interleaved tiles (runs of 2) from three rounds on: a 96 MiB-per-rank
    // bucket of 4 tensors (6 rounds) 71.9-73.1% -> 76.6% of the HBM peak,
    // while a GPT-2 block's 12 gradients (27 MiB, 2 rounds) lost 1-3
    // points with any run length
    if (a.strips == 0) a.strips = a.rounds >= 3 ? 2 : 1;
    return launch(&k_bucket<E, OP, true, 1, kBucketU>, a, dim3(grid), s);
  }
  // One round of between one and two tiles of twice the units per CU (the
  // ring all-reduce's rule): tiles of 8 units per lane, one per workgroup.
  if (batch != 1 && per_cu <= 0) {
    const int cus = cus_of(s);
    const uint64_t ncu = static_cast<uint64_t>(cus > 0 ? cus : 256);
    constexpr uint32_t kUnits8 = static_cast<uint32_t>(kBlock) * 8;
    uint32_t tiles8 = 0;
    for (int i = 0; i < a.npieces; ++i) tiles8 += (a.units[i] + kUnits8 - 1) / kUnits8;
    if (tiles8 > ncu && tiles8 < 2 * ncu) {
      for (int i = 0; i < a.npieces; ++i) a.tile0[i + 1] = a.tile0[i] + (a.units[i] + kUnits8 - 1) / kUnits8;
      a.tiles = tiles8;
      a.rounds = 1;
      return launch(&k_bucket<E, OP, false, 1, 8>, a, dim3(tiles8), s);
    }
  }
  return launch(&k_bucket<E, OP, false, 1, kBucketU>, a, dim3(grid), s);
}

template <class E>
hipError_t bucket_by_op(const BucketArgs& a, rr_op_t op, int per_cu, int sync, int batch, int timeout_us,
                        hipStream_t s) {
  switch (op) {
    case RR_SUM: return bucket_go<E, OpSum>(a, per_cu, sync, batch, timeout_us, s);
    case RR_MAX: return bucket_go<E, OpMax>(a, per_cu, sync, batch, timeout_us, s);
    case RR_MIN: return bucket_go<E, OpMin>(a, per_cu, sync, batch, timeout_us, s);
    case RR_AVG:
      if constexpr (__is_same(typename E::A, float)) return bucket_go<E, OpAvg>(a, per_cu, sync, batch, timeout_us, s);
      break;
  }
  return hipErrorInvalidValue;
}

// 32-bit unit indices when every index of the launch, including a loop
// counter one grid stride past the end, fits: rows*du + stride < 2^32.  The
// stride is at most (compute units) * (workgroups per CU, <= 64) * kBlock * 4
// units, below 2^28 for up to 1024 compute units: that is the margin kept.
bool small_index(const ColsArgs& a) { return a.du > 0 && a.rows < (0xFFFFFFFFull - (1ull << 28)) / a.du; }

template <class E, bool VEC, class IDX>
hipError_t fold_cols_by_op(const ColsArgs& a, rr_op_t op, int per_cu, hipStream_t s) {
  const dim3 grid(stream_grid(a.rows * a.wu, static_cast<uint64_t>(kBlock) * 4, a.p, per_cu > 0 ? per_cu : kColsPerCu, s),
                  a.p);
  switch (op) {
    case RR_SUM: return launch(&k_fold_cols<E, OpSum, VEC, IDX>, a, grid, s);
    case RR_MAX: return launch(&k_fold_cols<E, OpMax, VEC, IDX>, a, grid, s);
    case RR_MIN: return launch(&k_fold_cols<E, OpMin, VEC, IDX>, a, grid, s);
    case RR_AVG:
      if constexpr (__is_same(typename E::A, float)) return launch(&k_fold_cols<E, OpAvg, VEC, IDX>, a, grid, s);
      break;
  }
  return hipErrorInvalidValue;
}

template <class E>
hipError_t fold_cols_kind(const ColsArgs& a, rr_op_t op, int vec, int pc, hipStream_t s) {
  if (small_index(a))
    return vec ? fold_cols_by_op<E, true, uint32_t>(a, op, pc, s) : fold_cols_by_op<E, false, uint32_t>(a, op, pc, s);
  return vec ? fold_cols_by_op<E, true, uint64_t>(a, op, pc, s) : fold_cols_by_op<E, false, uint64_t>(a, op, pc, s);
}

template <int B, bool NT>
hipError_t gather_cols_go(const ColsArgs& a, int per_cu, hipStream_t s) {
  const dim3 grid(stream_grid(a.rows * a.du, static_cast<uint64_t>(kBlock) * 4, 1, per_cu > 0 ? per_cu : kColsPerCu, s));
  return small_index(a) ? launch(&k_gather_cols<B, NT, uint32_t>, a, grid, s)
                        : launch(&k_gather_cols<B, NT, uint64_t>, a, grid, s);
}

}  // namespace

hipError_t launch_bucket(const BucketArgs& a, Kind k, rr_op_t op, int per_cu, int sync, int batch, int timeout_us,
                         hipStream_t s) {
  if (a.tiles == 0) return hipSuccess;
  switch (k) {
    case Kind::kI32: return bucket_by_op<EI32>(a, op, per_cu, sync, batch, timeout_us, s);
    case Kind::kF32: return bucket_by_op<EF32>(a, op, per_cu, sync, batch, timeout_us, s);
    case Kind::kBF16: return bucket_by_op<EBF16>(a, op, per_cu, sync, batch, timeout_us, s);
    case Kind::kF16: return bucket_by_op<EF16>(a, op, per_cu, sync, batch, timeout_us, s);
  }
  return hipErrorInvalidValue;
}

hipError_t bucket_timeouts(unsigned long long* count) { return sync_timeouts_here(count); }

hipError_t launch_fold_cols(const ColsArgs& a, Kind k, rr_op_t op, int vec, int per_cu, hipStream_t s) {
  if (a.rows * a.wu == 0) return hipSuccess;
  switch (k) {
    case Kind::kI32: return fold_cols_kind<EI32>(a, op, vec, per_cu, s);
    case Kind::kF32: return fold_cols_kind<EF32>(a, op, vec, per_cu, s);
    case Kind::kBF16: return fold_cols_kind<EBF16>(a, op, vec, per_cu, s);
    case Kind::kF16: return fold_cols_kind<EF16>(a, op, vec, per_cu, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gather_cols(const ColsArgs& a, int unit_bytes, int nontemporal, int per_cu, int xcd_dst,
                              hipStream_t s) {
  if (a.rows * a.wu == 0) return hipSuccess;
  const bool nt = nontemporal != 0;
  // The XCD layout, two destinations per workgroup, for launches of 16-byte
  // units that write at least 192 MiB (as measured for this layout; the
  // plain fan-out switches above 128 MiB); xcd_dst forces the destinations
  // per workgroup (1, 2, 4) or turns it off (0).
  if (unit_bytes == 16 && nt && per_cu <= 0 && xcd_dst != 0) {
    const uint64_t units = a.rows * a.du;
    const uint64_t written = units * 16 * static_cast<uint64_t>(a.p);
    const int D = xcd_dst < 0 ? (written >= (192ull << 20) ? 2 : 0) : xcd_dst;
    const uint64_t blocks = (units + kBlock - 1) / kBlock;
    const uint64_t G = (static_cast<uint64_t>(a.p) + (D > 0 ? D : 1) - 1) / (D > 0 ? D : 1);
    const uint64_t grid = (blocks + 7) / 8 * 8 * G;
    if ((D == 1 || D == 2 || D == 4) && grid <= 0x7FFFFFFFull && blocks <= 0xFFFFFFFFull) {
      const uint32_t g32 = static_cast<uint32_t>(G);
      const uint32_t b32 = static_cast<uint32_t>(blocks);
      const bool small = units + kBlock <= 0xFFFFFFFFull;
      const dim3 gd(static_cast<unsigned>(grid));
      void* kp[3];
      ColsArgs copy = a;
      uint32_t gg = g32, bb = b32;
      kp[0] = &copy;
      kp[1] = &gg;
      kp[2] = &bb;
      const void* k = nullptr;
      if (D == 1) k = small ? reinterpret_cast<const void*>(&k_gather_cols_xcd<1, uint32_t>)
                            : reinterpret_cast<const void*>(&k_gather_cols_xcd<1, uint64_t>);
      if (D == 2) k = small ? reinterpret_cast<const void*>(&k_gather_cols_xcd<2, uint32_t>)
                            : reinterpret_cast<const void*>(&k_gather_cols_xcd<2, uint64_t>);
      if (D == 4) k = small ? reinterpret_cast<const void*>(&k_gather_cols_xcd<4, uint32_t>)
                            : reinterpret_cast<const void*>(&k_gather_cols_xcd<4, uint64_t>);
      return hipLaunchKernel(k, gd, dim3(kBlock), kp, 0, s);
    }
  }
  switch (unit_bytes) {
    case 16: return nt ? gather_cols_go<16, true>(a, per_cu, s) : gather_cols_go<16, false>(a, per_cu, s);
    case 4: return nt ? gather_cols_go<4, true>(a, per_cu, s) : gather_cols_go<4, false>(a, per_cu, s);
    case 2: return nt ? gather_cols_go<2, true>(a, per_cu, s) : gather_cols_go<2, false>(a, per_cu, s);
    case 1: return nt ? gather_cols_go<1, true>(a, per_cu, s) : gather_cols_go<1, false>(a, per_cu, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace rr
