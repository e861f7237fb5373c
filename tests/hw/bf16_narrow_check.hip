// Exhaustive check of librr's float32 -> bfloat16 narrowing (rr_device.h,
// the hardware conversion) against the rounding rule it documents, written
// out here on the integer pattern: round to nearest, ties to even, by adding
// 0x7FFF plus the lowest kept bit and truncating; a NaN keeps sign and top
// payload and gets the quiet bit.  Every one of the 2^32 float32 bit
// patterns goes through the single-value and the two-value (packed) forms.
// Test infrastructure: built by __graft_entry__.build(), loaded by
// tests/test_gpu_bf16_narrow.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_device.h"

namespace {

__device__ __forceinline__ uint32_t rule_bits(uint32_t u) {
  const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x0040u;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? quiet : rounded;
}

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
// packed form pairs each pattern with its bitwise complement.
__global__ __launch_bounds__(256) void k_check(unsigned long long* count, uint32_t* first) {
  const uint64_t step = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < (1ull << 32); i += step) {
    const uint32_t u = static_cast<uint32_t>(i);
    const uint32_t want = rule_bits(u);
    const uint32_t one = rr::f32_to_bf16_bits(__uint_as_float(u));
    if (one != want) record(count, first, u, one, want, 0);
    const uint32_t v = ~u;
    const uint32_t two = rr::f32x2_to_bf16x2_bits(__uint_as_float(u), __uint_as_float(v));
    if ((two & 0xFFFFu) != want) record(count, first, u, two & 0xFFFFu, want, 1);
    if ((two >> 16) != rule_bits(v)) record(count, first, v, two >> 16, rule_bits(v), 2);
  }
}

}  // namespace

// count: one device word (zeroed by the caller); first: 64 device words.
extern "C" int bf16_narrow_check(unsigned long long* count, uint32_t* first, hipStream_t s) {
  hipLaunchKernelGGL(k_check, dim3(2048), dim3(256), 0, s, count, first);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
