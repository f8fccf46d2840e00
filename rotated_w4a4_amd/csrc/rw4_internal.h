// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rw4 {

enum class TransformKind { Hadamard, Givens };

// Device-resident description of a transform.  For Givens, every (group,
// layer) has exactly 64 slots forming a perfect matching of the group's 128
// channels; lut_idx holds i | j << 8 and lut_cs holds (cos, sin) in fp32.
struct TransformDev {
  TransformKind kind;
  int64_t K;
  int64_t block;        // Hadamard block size
  int layers;           // Givens layers
  uint16_t* lut_idx;    // [G][layers][64]
  float2* lut_cs;       // [G][layers][64]
  float* alpha;         // [K] exp(beta)
  float* alpha_inv;     // [K] exp(-beta)
  uint32_t* sign_mask;  // Hadamard with random signs: [K], 0 or 0x80000000 (else null)
};

bool rowh_supported(int64_t K);

// group: the quantization group size (64, 128 or 256; which combinations
// are supported is checked by the C ABI layer before these are called).
hipError_t launch_quantize_act(const TransformDev& t, bool rrs, const void* x, bool bf16, int64_t M,
                               int64_t ldx, uint8_t* q, float* s, float* smooth, int group, hipStream_t st);

hipError_t launch_pack_weight(const TransformDev& t, const void* w, bool bf16, int64_t N, int64_t sk,
                              int64_t sn, uint8_t* q, float* s, int group, hipStream_t st);

hipError_t launch_dequantize(const uint8_t* q, const float* s, int64_t M, int64_t K, int group, void* out,
                             bool out_bf16, int64_t ldo, hipStream_t st);

hipError_t launch_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                       int64_t M, int64_t N, int64_t K, int group, void* y, bool y_bf16, int64_t ldy,
                       hipStream_t st);

}  // namespace rw4
