// rr_device.h -- device numerics and 128-bit memory access for the rr kernels
// (gfx950, CDNA4).  Internal header; not part of the C ABI.
//
// Element kinds: each kind names a storage type S and the accumulator type A
// that folds run in.  bfloat16 and IEEE binary16 are stored as their 16-bit
// patterns and widened to float32 exactly; every fold of a 16-bit type runs in
// float32 and is rounded once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct EI32 {
  using S = int32_t;
  using A = int32_t;
};
struct EF32 {
  using S = float;
  using A = float;
};
struct EBF16 {
  using S = uint16_t;
  using A = float;
};
struct EF16 {
  using S = uint16_t;
  using A = float;
};

// ---------------------------------------------------------------------------
// bfloat16 <-> float32.
//
// widen: the 16 bits become the upper half of a float32 (exact).
// narrow: round to nearest, ties to even, as on the integer pattern: adding
// 0x7FFF plus the lowest kept bit and truncating rounds half-way cases to the
// even neighbour; a mantissa carry moves into the exponent, so overflow gives
// +-inf.  A NaN keeps sign and top payload and gets the quiet bit (0x0040 in
// bf16) so it cannot become an infinity.  Denormals round like any value.
// gfx950's conversion instruction (v_cvt_pk_bf16_f32, two values per
// instruction) gives exactly these bits: an exhaustive comparison over all
// 2^32 float32 inputs, in the floating-point mode the library is built with
// (denormals kept, round to nearest even), found no difference.
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two values narrowed by one instruction: lo in bits 0-15, hi in 16-31.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---------------------------------------------------------------------------
// IEEE binary16 <-> float32.
//
// widen: the hardware conversion, exact for every binary16 value (subnormals
// included: the library is built without denormal flushing).
// narrow: the hardware conversion (v_cvt_f16_f32, or v_cvt_pk_f16_f32 for two
// values), which rounds to nearest even in the default rounding mode, gives
// binary16 subnormals for results below 2^-14 and +-inf for magnitudes that
// round to 2^16 or more; a NaN keeps its sign and the top 9 payload bits and
// gets the quiet bit.  Checked against that rule, written out on the bit
// pattern, for all 2^32 float32 inputs in both forms: no difference.
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two values narrowed by one instruction: lo in bits 0-15, hi in 16-31.
__device__ __forceinline__ uint32_t f32x2_to_f16x2_bits(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// 16-bit storage pattern <-> float32, by kind.
template <class E>
__device__ __forceinline__ float half_to_f32(uint32_t h) {
  if constexpr (__is_same(E, EF16)) {
    return f16_bits_to_f32(h);
  } else {
    return __uint_as_float(h << 16);
  }
}

template <class E>
__device__ __forceinline__ uint32_t f32_to_half(float f) {
  if constexpr (__is_same(E, EF16)) {
    return f32_to_f16_bits(f);
  } else {
    return f32_to_bf16_bits(f);
  }
}

// ---------------------------------------------------------------------------
// Reduction operators.  `acc` is the running value, `v` the next term.
//   sum: int32 wraps modulo 2^32 (done in uint32 to stay defined); float32 is
//        one IEEE-754 round-to-nearest-even addition.
//   max/min: compare-and-select; only a strictly greater (smaller) v replaces
//        acc, so ties keep the running value, a NaN acc stays, a NaN v is
//        skipped.  Written as a select so that no min/max instruction (whose
//        NaN and signed-zero rules differ) is used.
struct OpSum {
  __device__ __forceinline__ static int32_t apply(int32_t acc, int32_t v) {
    return static_cast<int32_t>(static_cast<uint32_t>(acc) + static_cast<uint32_t>(v));
  }
  __device__ __forceinline__ static float apply(float acc, float v) { return acc + v; }
};
struct OpMax {
  template <class A>
  __device__ __forceinline__ static A apply(A acc, A v) {
    return (v > acc) ? v : acc;
  }
};
struct OpMin {
  template <class A>
  __device__ __forceinline__ static A apply(A acc, A v) {
    return (v < acc) ? v : acc;
  }
};
// AVG (the averaged gradient of data parallelism): folds like a sum, then the
// accumulator is divided by the number of ranks, one IEEE-754 division
// (round to nearest even; the build keeps float division correctly rounded),
// before the one conversion to the storage type.  Float kinds only.
struct OpAvg : OpSum {};

template <class OP>
constexpr bool is_avg() {
  return __is_same(OP, OpAvg);
}

// The op's last step on a folded value: AVG divides by `div`, others return
// the value unchanged.
template <class OP, class A>
__device__ __forceinline__ A op_finish(A v, int32_t div) {
  if constexpr (is_avg<OP>()) {
    return v / static_cast<float>(div);
  } else {
    return v;
  }
}
// ---------------------------------------------------------------------------
// A "group" is V consecutive elements moved with 16-byte accesses.  V is chosen
// per kernel so that the narrower of its input/output types fills exactly one
// 16-byte access (4 x 32-bit or 8 x bf16); the wider type then takes one or two.
template <class E, int V>
struct Raw {
  static constexpr int BYTES = V * static_cast<int>(sizeof(typename E::S));
  static_assert(BYTES % 16 == 0, "a group must be whole 16-byte words");
  static constexpr int NW = BYTES / 16;
  u32x4 w[NW];
};

template <bool NT, class E, int V>
__device__ __forceinline__ void load_group(Raw<E, V>& r, const typename E::S* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < Raw<E, V>::NW; ++i) {
    if constexpr (NT) {
      r.w[i] = __builtin_nontemporal_load(q + i);
    } else {
      r.w[i] = q[i];
    }
  }
}

template <bool NT, class E, int V>
__device__ __forceinline__ void store_group(typename E::S* p, const Raw<E, V>& r) {
  u32x4* q = reinterpret_cast<u32x4*>(p);
#pragma unroll
  for (int i = 0; i < Raw<E, V>::NW; ++i) {
    if constexpr (NT) {
      __builtin_nontemporal_store(r.w[i], q + i);
    } else {
      q[i] = r.w[i];
    }
  }
}

// Raw storage words -> V accumulator values.
template <class E, int V>
__device__ __forceinline__ void unpack(const Raw<E, V>& r, typename E::A* a) {
  if constexpr (sizeof(typename E::S) == 4) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const uint32_t w = r.w[j / 4][j % 4];
      if constexpr (__is_same(typename E::A, float)) {
        a[j] = __uint_as_float(w);
      } else {
        a[j] = static_cast<int32_t>(w);
      }
    }
  } else if constexpr (__is_same(E, EBF16)) {
#pragma unroll
    for (int j = 0; j < V; j += 2) {
      const uint32_t w = r.w[j / 8][(j % 8) / 2];
      a[j] = bf16_lo_to_f32(w);
      a[j + 1] = bf16_hi_to_f32(w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < V; j += 2) {
      const uint32_t w = r.w[j / 8][(j % 8) / 2];
      a[j] = f16_bits_to_f32(w & 0xFFFFu);
      a[j + 1] = f16_bits_to_f32(w >> 16);
    }
  }
}

// V accumulator values -> raw storage words of kind E (one rounding for the
// 16-bit kinds).
template <class E, int V, class A>
__device__ __forceinline__ void pack(const A* a, Raw<E, V>& r) {
  if constexpr (sizeof(typename E::S) == 4) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      if constexpr (__is_same(A, float)) {
        r.w[j / 4][j % 4] = __float_as_uint(a[j]);
      } else {
        r.w[j / 4][j % 4] = static_cast<uint32_t>(a[j]);
      }
    }
  } else if constexpr (__is_same(E, EBF16)) {
#pragma unroll
    for (int j = 0; j < V; j += 2) r.w[j / 8][(j % 8) / 2] = f32x2_to_bf16x2_bits(a[j], a[j + 1]);
  } else {
#pragma unroll
    for (int j = 0; j < V; j += 2) r.w[j / 8][(j % 8) / 2] = f32x2_to_f16x2_bits(a[j], a[j + 1]);
  }
}

// Scalar element access for heads, tails and unaligned buffers.
template <class E>
__device__ __forceinline__ typename E::A load_one(const typename E::S* p) {
  if constexpr (sizeof(typename E::S) == 2) {
    return half_to_f32<E>(static_cast<uint32_t>(*p));
  } else {
    return *p;
  }
}

template <class E, class A>
__device__ __forceinline__ void store_one(typename E::S* p, A v) {
  if constexpr (sizeof(typename E::S) == 2) {
    *p = static_cast<uint16_t>(f32_to_half<E>(v));
  } else {
    *p = v;
  }
}

}  // namespace rr
