// Dequantization of the stored INT4 form: x_hat[r, k] = c[r, k] * s[r, k / 128]
// in the transformed domain (the complex-domain quantization page, section
// 2.1: Q(x) = Delta * round(x / Delta); for Rotated Runtime Smooth the stored
// scale a_t * s_g already carries the smoothing factor).  This is what a
// consumer of an INT4 KV cache reads back: rotated keys against rotated
// queries (the Rotated Runtime Smooth experiments quantize the KV cache with
// sub-channel groups of 128; the OstQuant page rotates Q and K alike).
//
// One lane per 16 stored bytes (32 codes of one row); the product code * scale
// is rounded once to fp32, then to bf16 (round to nearest even) when asked.
#include "rw4_device.h"
#include "rw4_internal.h"

namespace rw4 {

// log2g: log2 of the group (6, 7 or 8); a lane's 32 codes lie in one group.
template <bool BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ q,
                                                      const float* __restrict__ s, int64_t M, int64_t K,
                                                      int log2g, void* __restrict__ out, int64_t ldo) {
  const int64_t chunks_per_row = K / 32;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= M * chunks_per_row) return;
  const int64_t row = idx / chunks_per_row;
  const int64_t k0 = (idx - row * chunks_per_row) * 32;
  const uint4 w4 = *reinterpret_cast<const uint4*>(q + row * (K / 2) + k0 / 2);
  const float sc = s[row * (K >> log2g) + (k0 >> log2g)];
  const uint32_t words[4] = {w4.x, w4.y, w4.z, w4.w};
  float v[32];
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    const uint32_t w = words[wi];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t mag = (w >> (4 * e)) & 7u;
      const uint32_t neg = (w >> (4 * ((e + 1) & 7) + 3)) & 1u;  // sign of code e: bit 3 of nibble e + 1
      const float c = neg ? -float(mag) : float(mag);
      v[wi * 8 + e] = c * sc;
    }
  }
  if constexpr (BF16) {
    uint32_t packed[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t lo = __float_as_uint(v[2 * i]), hi = __float_as_uint(v[2 * i + 1]);
      lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
      hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) & 0xFFFF0000u;
      packed[i] = lo | hi;
    }
    uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + row * ldo + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dst[i] = make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
  } else {
    float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + row * ldo + k0);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

hipError_t launch_dequantize(const uint8_t* q, const float* s, int64_t M, int64_t K, int group, void* out,
                             bool out_bf16, int64_t ldo, hipStream_t st) {
  const int log2g = group == 64 ? 6 : group == 256 ? 8 : 7;
  const int64_t lanes = M * (K / 32);
  const int64_t blocks = (lanes + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (out_bf16)
    hipLaunchKernelGGL((dequant_kernel<true>), dim3(blocks), dim3(256), 0, st, q, s, M, K, log2g, out, ldo);
  else
    hipLaunchKernelGGL((dequant_kernel<false>), dim3(blocks), dim3(256), 0, st, q, s, M, K, log2g, out, ldo);
  return hipGetLastError();
}

}  // namespace rw4
