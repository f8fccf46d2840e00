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
// when asked.
//
// Each stored word gives its even and odd codes as FP8 E4M3 bytes of value
// c * 2^-9 (w & 0x87878787, rotr(w, 4) & 0x87878787, as the GEMM reads
// them); v_cvt_pk_f32_fp8 widens two at a time exactly, and
// (c * 2^-9) * (s * 2^9) is the exact product c * s rounded once, as long
// as s * 2^9 is finite (s < 2^119).  Larger scales take the per-code path.
#include "rw4_device.h"
#include "rw4_internal.h"

namespace rw4 {

typedef float v2f __attribute__((ext_vector_type(2)));

template <bool BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ q,
                                                      const float* __restrict__ s, int64_t row0, int64_t K,
                                                      int log2g, void* __restrict__ out, int64_t ldo) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;  // word of the row
  if (j >= K / 8) return;
  const int64_t row = row0 + blockIdx.y;
  const uint32_t w = reinterpret_cast<const uint32_t*>(q + row * (K / 2))[j];
  const float sc = s[row * (K >> log2g) + ((j * 8) >> log2g)];
  float v[8];
  if (sc < 0x1p119f) {
    const float s9 = sc * 512.0f;  // exact
    const int ev = int(w & 0x87878787u);                                   // codes 0, 2, 4, 6
    const int od = int(__builtin_amdgcn_alignbit(w, w, 4) & 0x87878787u);  // codes 1, 3, 5, 7
    const v2f e0 = __builtin_amdgcn_cvt_pk_f32_fp8(ev, false), e1 = __builtin_amdgcn_cvt_pk_f32_fp8(ev, true);
    const v2f o0 = __builtin_amdgcn_cvt_pk_f32_fp8(od, false), o1 = __builtin_amdgcn_cvt_pk_f32_fp8(od, true);
    v[0] = e0[0] * s9; v[1] = o0[0] * s9; v[2] = e0[1] * s9; v[3] = o0[1] * s9;
    v[4] = e1[0] * s9; v[5] = o1[0] * s9; v[6] = e1[1] * s9; v[7] = o1[1] * s9;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t mag = (w >> (4 * e)) & 7u;
      const uint32_t neg = (w >> (4 * ((e + 1) & 7) + 3)) & 1u;  // sign of code e: bit 3 of nibble e + 1
      v[e] = (neg ? -float(mag) : float(mag)) * sc;
    }
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

}  // namespace rw4
