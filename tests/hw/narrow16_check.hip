// Exhaustive check of librr's float32 -> 16-bit narrowing (rr_device.h, the
// hardware conversions) against the rounding rules it documents, written out
// here on the bit pattern.  Every one of the 2^32 float32 bit patterns goes
// through the single-value and the two-value (packed) form of each kind.
//   bfloat16: round to nearest, ties to even, by adding 0x7FFF plus the
//     lowest kept bit and truncating; a NaN keeps sign and top payload and
//     gets the quiet bit.
//   binary16: round to nearest, ties to even, at binary16 precision, with
//     binary16 subnormals below 2^-14 and +-inf from 65520 up; a NaN keeps
//     sign and top 9 payload bits and gets the quiet bit.
// Test infrastructure: built by __graft_entry__.build(), loaded by
// tests/test_gpu_narrow16.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_device.h"

namespace {

__device__ __forceinline__ uint32_t bf16_rule(uint32_t u) {
  const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x0040u;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? quiet : rounded;
}

// Round the magnitude m (a float32 pattern without its sign) to binary16
// bits, nearest even, by integer arithmetic only.
__device__ __forceinline__ uint32_t f16_magnitude(uint32_t m) {
  if (m > 0x7F800000u) return 0x7E00u | ((m >> 13) & 0x03FFu);  // NaN
  if (m >= 0x477FF000u) return 0x7C00u;                          // >= 65520 (and inf): inf
  const uint32_t e = m >> 23;                                     // biased float32 exponent
  if (e >= 113) {                                                 // normal binary16 (2^-14 and up)
    const uint32_t v = m - (112u << 23);                          // rebias to binary16 in the float32 layout
    const uint32_t lsb = (v >> 13) & 1u;
    return (v + 0x0FFFu + lsb) >> 13;                             // a carry out of the mantissa bumps the exponent
  }
  if (e < 102) return 0;                                          // below 2^-25: rounds to zero
  // subnormal binary16: value = mant * 2^(e-150) with the implicit bit; the
  // result counts units of 2^-24
  const uint32_t mant = (m & 0x007FFFFFu) | 0x00800000u;
  const uint32_t shift = 126u - e;                                // 14 .. 24
  const uint32_t q = mant >> shift;
  const uint32_t rem = mant & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1u);
  return q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
}

__device__ __forceinline__ uint32_t f16_rule(uint32_t u) { return ((u >> 16) & 0x8000u) | f16_magnitude(u & 0x7FFFFFFFu); }

__device__ void record(unsigned long long* count, uint32_t* first, uint32_t u, uint32_t got, uint32_t want,
                       uint32_t form) {
  const unsigned long long k = atomicAdd(count, 1ull);
  if (k < 16) {
    first[4 * k] = u;
    first[4 * k + 1] = got;
    first[4 * k + 2] = want;
    first[4 * k + 3] = form;
  }
}

// Thread i checks patterns i, i + T, i + 2T, ... (T threads in all); the
// packed forms pair each pattern with its bitwise complement.
// form: 0/1/2 bfloat16 single / packed low / packed high, 3/4/5 binary16.
__global__ __launch_bounds__(256) void k_check(unsigned long long* count, uint32_t* first) {
  const uint64_t step = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < (1ull << 32); i += step) {
    const uint32_t u = static_cast<uint32_t>(i);
    const uint32_t v = ~u;
    const float fu = __uint_as_float(u);
    const float fv = __uint_as_float(v);
    {
      const uint32_t want = bf16_rule(u);
      const uint32_t one = rr::f32_to_bf16_bits(fu);
      if (one != want) record(count, first, u, one, want, 0);
      const uint32_t two = rr::f32x2_to_bf16x2_bits(fu, fv);
      if ((two & 0xFFFFu) != want) record(count, first, u, two & 0xFFFFu, want, 1);
      if ((two >> 16) != bf16_rule(v)) record(count, first, v, two >> 16, bf16_rule(v), 2);
    }
    {
      const uint32_t want = f16_rule(u);
      const uint32_t one = rr::f32_to_f16_bits(fu);
      if (one != want) record(count, first, u, one, want, 3);
      const uint32_t two = rr::f32x2_to_f16x2_bits(fu, fv);
      if ((two & 0xFFFFu) != want) record(count, first, u, two & 0xFFFFu, want, 4);
      if ((two >> 16) != f16_rule(v)) record(count, first, v, two >> 16, f16_rule(v), 5);
    }
  }
}

}  // namespace

// count: one device word (zeroed by the caller); first: 64 device words.
extern "C" int narrow16_check(unsigned long long* count, uint32_t* first, hipStream_t s) {
  hipLaunchKernelGGL(k_check, dim3(2048), dim3(256), 0, s, count, first);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
