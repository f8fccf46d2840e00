// Dequantization of the stored INT4 form: x_hat[r, k] = c[r, k] * s[r, k / g]
// in the transformed domain (the complex-domain quantization page, section
// 2.1: Q(x) = Delta * round(x / Delta); for Rotated Runtime Smooth the stored
// scale a_t * s_g already carries the smoothing factor).  This is what a
// consumer of an INT4 KV cache reads back: rotated keys against rotated
// queries (the Rotated Runtime Smooth experiments quantize the KV cache with
// sub-channel groups of 128; the OstQuant page rotates Q and K alike).
//
// One lane per stored word (8 codes): consecutive lanes read consecutive
// words and write consecutive 16-byte (bf16) or 32-byte (fp32) runs.  The
// grid's y dimension is the row (in launches of at most 65535 rows), x
// covers the row's words with blocks of 64 to 256 lanes.  The product
// code * scale is rounded once to fp32, then to bf16 (round to nearest even)
// when asked.  A word gives its 8 codes as 6-bit sign-magnitude fields
// (pair_fields: the inverse of the stored form's fold, from the word and
// its partner w ^ 3 in the same 16-byte chunk, read by this lane too).
#include "rw4_device.h"
#include "rw4_internal.h"

namespace rw4 {

template <bool BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ q,
                                                      const float* __restrict__ s, int64_t row0, int64_t K,
                                                      int log2g, void* __restrict__ out, int64_t ldo) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;  // word of the row
  if (j >= K / 8) return;
  const int64_t row = row0 + blockIdx.y;
  const uint32_t* qrow = reinterpret_cast<const uint32_t*>(q + row * (K / 2));
  const uint32_t w = qrow[j], wp = qrow[j ^ 3];  // rows hold whole 16-byte chunks (K % 64 == 0)
  const float sc = s[row * (K >> log2g) + ((j * 8) >> log2g)];
  uint32_t lo, hi;
  pair_fields<true>(w, wp, (j & 2) != 0, lo, hi);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t f = field6(lo, hi, e);
    const float mag = float(f & 7u);
    v[e] = ((f & 32u) ? -mag : mag) * sc;
  }
  if constexpr (BF16) {
    __bf16 h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = static_cast<__bf16>(v[i]);  // round to nearest even
    *reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(out) + row * ldo + j * 8) =
        *reinterpret_cast<const uint4*>(h);
  } else {
    float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + row * ldo + j * 8);
    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

hipError_t launch_dequantize(const uint8_t* q, const float* s, int64_t M, int64_t K, int group, void* out,
                             bool out_bf16, int64_t ldo, hipStream_t st) {
  const int log2g = group == 64 ? 6 : group == 256 ? 8 : 7;
  const int64_t words = K / 8;
  const int bd = words >= 256 ? 256 : int((words + 63) / 64 * 64);
  const int64_t bx = (words + bd - 1) / bd;
  if (bx > 0x7FFFFFFF) return hipErrorInvalidValue;
  constexpr int64_t kMaxRows = 65535;  // grid y limit
  for (int64_t r0 = 0; r0 < M; r0 += kMaxRows) {
    const int64_t rows = M - r0 < kMaxRows ? M - r0 : kMaxRows;
    const dim3 grid{unsigned(bx), unsigned(rows), 1u};
    if (out_bf16)
      hipLaunchKernelGGL((dequant_kernel<true>), grid, dim3(bd), 0, st, q, s, r0, K, log2g, out, ldo);
    else
      hipLaunchKernelGGL((dequant_kernel<false>), grid, dim3(bd), 0, st, q, s, r0, K, log2g, out, ldo);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Asymmetric codes (unsigned stored form, groups of 128): x_hat = s (q - z), with
// q - z an exact small integer, so the product is rounded once to fp32 (then
// to bf16 when asked).  One lane per stored word, as dequant_kernel.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void dequant_asym_kernel(const uint8_t* __restrict__ q,
                                                           const float* __restrict__ s,
                                                           const float* __restrict__ z, int64_t row0, int64_t K,
                                                           void* __restrict__ out, int64_t ldo) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= K / 8) return;
  const int64_t row = row0 + blockIdx.y;
  const uint32_t* qrow = reinterpret_cast<const uint32_t*>(q + row * (K / 2));
  const uint32_t w = qrow[j], wp = qrow[j ^ 3];
  const int64_t gi = row * (K / kGroup) + (j * 8) / kGroup;
  const float sc = s[gi], zp = z[gi];
  uint32_t lo, hi;
  pair_fields<false>(w, wp, (j & 2) != 0, lo, hi);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float(field6(lo, hi, e)) - zp) * sc;
  if constexpr (BF16) {
    __bf16 h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = static_cast<__bf16>(v[i]);
    *reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(out) + row * ldo + j * 8) =
        *reinterpret_cast<const uint4*>(h);
  } else {
    float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + row * ldo + j * 8);
    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

hipError_t launch_dequantize_asym(const uint8_t* q, const float* s, const float* z, int64_t M, int64_t K, void* out,
                                  bool out_bf16, int64_t ldo, hipStream_t st) {
  const int64_t words = K / 8;
  const int bd = words >= 256 ? 256 : int((words + 63) / 64 * 64);
  const int64_t bx = (words + bd - 1) / bd;
  if (bx > 0x7FFFFFFF) return hipErrorInvalidValue;
  constexpr int64_t kMaxRows = 65535;
  for (int64_t r0 = 0; r0 < M; r0 += kMaxRows) {
    const int64_t rows = M - r0 < kMaxRows ? M - r0 : kMaxRows;
    const dim3 grid{unsigned(bx), unsigned(rows), 1u};
    if (out_bf16)
      hipLaunchKernelGGL((dequant_asym_kernel<true>), grid, dim3(bd), 0, st, q, s, z, r0, K, out, ldo);
    else
      hipLaunchKernelGGL((dequant_asym_kernel<false>), grid, dim3(bd), 0, st, q, s, z, r0, K, out, ldo);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Code sums of packed (signed) weight rows per 128-group: the totals an
// asymmetric activation's zero point multiplies.  One lane per (row,
// group); offline, with the weight pack.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void weight_code_sums_kernel(const uint8_t* __restrict__ qw, int64_t N, int64_t G,
                                                               float* __restrict__ cw) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= N * G) return;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(qw + i * 64);  // row n = i / G, group i % G
  int sum = 0;
  for (int k = 0; k < 16; ++k) {
    uint32_t lo, hi;
    pair_fields<true>(w[k], w[k ^ 3], (k & 2) != 0, lo, hi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t f = field6(lo, hi, e);
      sum += (f & 32u) ? -int(f & 7u) : int(f & 7u);
    }
  }
  cw[i] = float(sum);
}

hipError_t launch_weight_code_sums(const uint8_t* qw, int64_t N, int64_t K, float* cw, hipStream_t st) {
  const int64_t n = N * (K / kGroup);
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(weight_code_sums_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, qw, N, K / kGroup, cw);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weights for 8-bit activation groups: every row of the packed weights with
// the groups listed in groups8 appended again (codes and scales), so that
// the INT4 GEMM over K + 128 n8 multiplies an 8-bit group's two planes by
// the same weights.  One lane per 16-byte chunk of an output row; a listed
// group outside [0, G) yields zero codes and scale.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void extend_weight_groups_kernel(const uint8_t* __restrict__ qw,
                                                                   const float* __restrict__ sw, int64_t G,
                                                                   const int32_t* __restrict__ groups8, int64_t n8,
                                                                   int64_t row0, uint8_t* __restrict__ qx,
                                                                   float* __restrict__ sx) {
  const int64_t Gx = G + n8;
  const int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;  // 16-byte chunk of the output row
  if (c >= Gx * 4) return;
  const int64_t n = row0 + blockIdx.y;
  const int64_t gx = c >> 2;
  int64_t src = gx;
  if (gx >= G) src = groups8[gx - G];
  const bool ok = src >= 0 && src < G;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (ok) v = *reinterpret_cast<const uint4*>(qw + n * (G * 64) + src * 64 + (c & 3) * 16);
  *reinterpret_cast<uint4*>(qx + n * (Gx * 64) + c * 16) = v;
  if ((c & 3) == 0) sx[n * Gx + gx] = ok ? sw[n * G + src] : 0.0f;
}

hipError_t launch_extend_weight_groups(const uint8_t* qw, const float* sw, int64_t N, int64_t K,
                                       const int32_t* groups8, int64_t n8, uint8_t* qx, float* sx, hipStream_t st) {
  const int64_t G = K / kGroup, chunks = (G + n8) * 4;
  const int64_t bx = (chunks + 255) / 256;
  if (bx > 0x7FFFFFFF) return hipErrorInvalidValue;
  constexpr int64_t kMaxRows = 65535;
  for (int64_t r0 = 0; r0 < N; r0 += kMaxRows) {
    const int64_t rows = N - r0 < kMaxRows ? N - r0 : kMaxRows;
    hipLaunchKernelGGL(extend_weight_groups_kernel, dim3(unsigned(bx), unsigned(rows)), dim3(256), 0, st, qw, sw, G,
                       groups8, n8, r0, qx, sx);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rw4
