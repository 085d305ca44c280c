// Offline quantization of a frozen weight to the 4-bit base the gather-GEMMs
// read (SparseLoRA article §六: SparseLoRA over a QLoRA-style quantized base).
//
// Each row is cut into blocks of 64 consecutive elements.  A block gets one
// fp32 scale s = max|w| / 7 (0 for an all-zero block) and one signed 4-bit
// code q = rint(w / s) in [-7, 7] per element (IEEE fp32 division, ties to
// even); the weight the layer then uses is q * s.  Codes: element 2j of a row
// in the low nibble of byte j, element 2j+1 in the high nibble, two's
// complement.  One thread per block: 64 elements in registers, 32 code bytes
// and one scale out.
#include "sl_common.hpp"
#include "sl_host.hpp"

#include <hip/hip_runtime.h>

namespace sl {

template <typename T>
__global__ void __launch_bounds__(256) quantize_q4_kernel(const T* __restrict__ W, long long nblocks, int cols,
                                                          unsigned char* __restrict__ codes,
                                                          float* __restrict__ scales) {
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const int nb = cols / 64;
  const long long r = b / nb;
  const int c0 = (int)(b % nb) * 64;
  const T* src = W + r * cols + c0;
  float v[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) v[j] = Elem<T>::load(src, j);
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 64; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const float s = amax / 7.0f;
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t x = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float q = s > 0.f ? rintf(v[8 * i + e] / s) : 0.f;
      q = fminf(fmaxf(q, -7.f), 7.f);
      x |= ((uint32_t)(int)q & 0xFu) << (4 * e);
    }
    w[i] = x;
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + r * (cols / 2) + c0 / 2);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  scales[b] = s;
}

}  // namespace sl

using namespace sl;

extern "C" sl_status sl_quantize_q4(sl_dtype dt, const void* W, int64_t rows, int64_t cols, void* codes,
                                    float* scales, void* stream) {
  if (!W || !codes || !scales) SL_FAIL(SL_ERR_NULL, "W, codes and scales must be non-NULL");
  if (dt != SL_BF16 && dt != SL_F32) SL_FAIL(SL_ERR_DTYPE, "dtype must be SL_F32 or SL_BF16");
  if (rows <= 0 || cols <= 0 || cols % 64 != 0)
    SL_FAIL(SL_ERR_SHAPE, "rows > 0 and cols a positive multiple of 64 (got %lld x %lld)", (long long)rows,
            (long long)cols);
  if (cols > (1LL << 30) || rows * cols >= (1LL << 40)) SL_FAIL(SL_ERR_RANGE, "weight too large");
  if (!aligned16(W) || !aligned16(codes) || !aligned16(scales))
    SL_FAIL(SL_ERR_ALIGN, "W, codes and scales must be 16-byte aligned");
  sl_status st = check_arch();
  if (st != SL_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const long long nblocks = rows * (cols / 64);
  const dim3 grid((unsigned)((nblocks + 255) / 256)), block(256);
  if (dt == SL_BF16)
    hipLaunchKernelGGL(quantize_q4_kernel<bf16>, grid, block, 0, s, reinterpret_cast<const bf16*>(W), nblocks,
                       (int)cols, reinterpret_cast<unsigned char*>(codes), scales);
  else
    hipLaunchKernelGGL(quantize_q4_kernel<float>, grid, block, 0, s, reinterpret_cast<const float*>(W), nblocks,
                       (int)cols, reinterpret_cast<unsigned char*>(codes), scales);
  SL_HIP(hipGetLastError());
  return SL_OK;
}
