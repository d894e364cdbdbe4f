// One 8-bit matrix instruction in isolation, for tests of its arithmetic.
//
// Each 64-lane wave evaluates one product with
// v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 operands with both block scales
// 2^0 (E8M0 byte 127), the form the FP8 attention forward issues:
//
//   d[p][i][j] = c[p][i][j] + sum_k a[p][i][k] * b[p][j][k]
//
// a, b: [n][32][64] E4M3 bytes (row, reduction index); c, d: [n][32][32]
// fp32 row-major; all device pointers.  Lane l holds row l % 32 of a and of
// b, reduction bytes 32 (l / 32) .. 32 (l / 32) + 31; whatever order the
// hardware reduces in, byte s of lane group g of a meets byte s of lane
// group g of b, so the sum above is what the instruction computes.  The
// accumulator holds column j = l % 32 and rows 8 (r / 4) + 4 (l / 32) + r % 4
// in register r.  Returns a hipError_t (0 on success); n = 0 is a no-op.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(64) void mma_fp8_kernel(const uint8_t* __restrict__ a,
                                                     const uint8_t* __restrict__ b,
                                                     const float* __restrict__ c,
                                                     float* __restrict__ d) {
  const int p = blockIdx.x;
  const int l = threadIdx.x;
  const int row = l & 31, g = l >> 5;
  const uint32_t* ap = reinterpret_cast<const uint32_t*>(a + (size_t)p * 2048 + row * 64 + g * 32);
  const uint32_t* bp = reinterpret_cast<const uint32_t*>(b + (size_t)p * 2048 + row * 64 + g * 32);
  i32x8 av, bv;
  for (int w = 0; w < 8; ++w) {
    av[w] = (int)ap[w];
    bv[w] = (int)bp[w];
  }
  const float* cp = c + (size_t)p * 1024;
  float* dp = d + (size_t)p * 1024;
  f32x16 acc;
  for (int r = 0; r < 16; ++r) acc[r] = cp[(8 * (r >> 2) + 4 * g + (r & 3)) * 32 + row];
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
  for (int r = 0; r < 16; ++r) dp[(8 * (r >> 2) + 4 * g + (r & 3)) * 32 + row] = acc[r];
}

}  // namespace

extern "C" int mma_fp8_probe(const uint8_t* a, const uint8_t* b, const float* c, float* d,
                             int n, hipStream_t stream) {
  if (n < 0 || (n > 0 && (!a || !b || !c || !d))) return (int)hipErrorInvalidValue;
  if (n == 0) return 0;
  hipLaunchKernelGGL(mma_fp8_kernel, dim3(n), dim3(64), 0, stream, a, b, c, d);
  return (int)hipGetLastError();
}
