// A hardware probe for the tests (not part of libdsa.so): the gfx950 scaled
// fp8 matrix-core product v_mfma_scale_f32_16x16x128_f8f6f4 on given e4m3fn
// codes, in exactly the operand layout and scale form the prefill indexer's
// approximate stage uses (A = 16 rows with one E8M0 scale code per row, B =
// 16 columns with scale 1).  The tests compare its results with exact sums to
// check the error bound the prefill Top-k's exactness argument relies on.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// One wave per tile p: a [n_tiles, 16, 128] codes (row n = A row), b
// [n_tiles, 16, 128] (row n = B column), code [n_tiles, 16] E8M0 scale codes
// of A's rows, out [n_tiles, 16, 16] f32 (out[p][i][j] = A row i . B col j
// times 2^(code_i - 127)).  Lane (g, n) holds bytes [16 g, 16 g + 16) and
// [64 + 16 g, 64 + 16 g + 16) of row n of A and of column n of B.
__global__ __launch_bounds__(64) void k_fp8_mfma_probe(const uint8_t* __restrict__ a,
                                                       const uint8_t* __restrict__ b,
                                                       const int* __restrict__ code,
                                                       float* __restrict__ out) {
  const int p = blockIdx.x, lane = threadIdx.x, n = lane & 15, g = lane >> 4;
  const uint4* ar = reinterpret_cast<const uint4*>(a + (static_cast<int64_t>(p) * 16 + n) * 128);
  const uint4* br = reinterpret_cast<const uint4*>(b + (static_cast<int64_t>(p) * 16 + n) * 128);
  const uint4 alo = ar[g], ahi = ar[4 + g], blo = br[g], bhi = br[4 + g];
  const v8i A = {static_cast<int>(alo.x), static_cast<int>(alo.y), static_cast<int>(alo.z),
                 static_cast<int>(alo.w), static_cast<int>(ahi.x), static_cast<int>(ahi.y),
                 static_cast<int>(ahi.z), static_cast<int>(ahi.w)};
  const v8i B = {static_cast<int>(blo.x), static_cast<int>(blo.y), static_cast<int>(blo.z),
                 static_cast<int>(blo.w), static_cast<int>(bhi.x), static_cast<int>(bhi.y),
                 static_cast<int>(bhi.z), static_cast<int>(bhi.w)};
  const int sa = code[p * 16 + n];
  const v4f c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                 0, sa, 0, 127);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[(static_cast<int64_t>(p) * 16 + 4 * g + i) * 16 + n] = c[i];
}

extern "C" int fp8_mfma_probe(const void* a, const void* b, const void* code, void* out,
                              int n_tiles, void* stream) {
  if (!a || !b || !code || !out || n_tiles < 1) return -1;
  hipLaunchKernelGGL(k_fp8_mfma_probe, dim3(n_tiles), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(b),
                     static_cast<const int*>(code), static_cast<float*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
