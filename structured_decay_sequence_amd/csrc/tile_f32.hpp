// fp32 MFMA tile helpers (gfx950, wave64) shared by the general path and the
// query-conditioned composition.
//
// A product tile is 16x16 on v_mfma_f32_16x16x4_f32.  A 16-deep slice of K
// is taken as four such MFMAs over a permuted K: lane (i, g) (i = lane % 16,
// g = lane / 16) reads the 16-byte piece k0 + 4g .. k0 + 4g + 3 of its row of
// each operand (the A operand's row i, the B operand's column i), and product
// e pairs the e-th value of both.  The accumulator holds rows 4g .. 4g + 3 of
// column i in lane (i, g), which is also the B-operand layout of the next
// product, so a result tile feeds the next product with no lane exchange.
#pragma once

#include <hip/hip_runtime.h>

namespace lattn {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }

// acc += A B over one 16-deep K slice in the permuted-K form above.
__device__ __forceinline__ f32x4 mfma16(const f32x4& a, const f32x4& b, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  return acc;
}

}  // namespace lattn
