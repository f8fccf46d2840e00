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

// Asymmetric (s, z) activations, block-128 Hadamard, groups of 128: plain
// unsigned codes (stored form), scales and zero points (floats) [M][K / 128].
hipError_t launch_quantize_act_asym(const TransformDev& t, const void* x, bool bf16, int64_t M, int64_t ldx,
                                    uint8_t* q, float* s, float* z, hipStream_t st);
// Block-128 Hadamard activations with the groups whose slot_of_group entry
// is in [0, n8) kept at 8 bits as two INT4 planes (rows of G + n8 groups).
hipError_t launch_quantize_act_mixed(const TransformDev& t, const void* x, bool bf16, int64_t M, int64_t ldx,
                                     const int32_t* slot_of_group, int64_t n8, uint8_t* q, float* s, hipStream_t st);
// Packed weights [N][K/2] and scales with the groups of groups8 [n8] appended.
hipError_t launch_extend_weight_groups(const uint8_t* qw, const float* sw, int64_t N, int64_t K,
                                       const int32_t* groups8, int64_t n8, uint8_t* qx, float* sx, hipStream_t st);
// cw[n][g] = sum of the 128 codes of group g of packed weight row n (floats).
hipError_t launch_weight_code_sums(const uint8_t* qw, int64_t N, int64_t K, float* cw, hipStream_t st);
// y = sum_g sa sw (sum_k qa qw - za cw) with unsigned activation codes (groups of 128).
hipError_t launch_gemm_asym(const uint8_t* qa, const float* sa, const float* za, const uint8_t* qw, const float* sw,
                            const float* cw, int64_t M, int64_t N, int64_t K, void* y, bool y_bf16, int64_t ldy,
                            hipStream_t st);
// x_hat = s (q - z) from unsigned codes (groups of 128).
hipError_t launch_dequantize_asym(const uint8_t* q, const float* s, const float* z, int64_t M, int64_t K, void* out,
                                  bool out_bf16, int64_t ldo, hipStream_t st);

hipError_t launch_pack_weight(const TransformDev& t, const void* w, bool bf16, int64_t N, int64_t sk,
                              int64_t sn, uint8_t* q, float* s, int group, hipStream_t st);

hipError_t launch_rotate_act(const TransformDev& t, const void* x, bool bf16, int64_t M, int64_t ldx, void* out,
                             bool out_bf16, int64_t ldo, hipStream_t st);

// Rotated Runtime Smooth with the channel reorder (Hadamard transforms, K in
// {512, 1024, 2048, 4096}); workspace of rrs_reorder_workspace_bytes(K).
bool rrs_reorder_supported(int64_t K);
int64_t rrs_reorder_workspace_bytes(int64_t K);
hipError_t launch_quantize_act_rrs_reorder(const TransformDev& t, const void* x, bool bf16, int64_t M, int64_t ldx,
                                           uint8_t* q, float* s, int32_t* order, void* workspace, hipStream_t st);
hipError_t launch_pack_weight_per_channel(const TransformDev& t, const void* w, bool bf16, int64_t N, int64_t sk,
                                          int64_t sn, uint8_t* q, float* s, hipStream_t st);
hipError_t launch_permute_codes(const uint8_t* q, int64_t rows, int64_t K, const int32_t* order, uint8_t* out,
                                hipStream_t st);

hipError_t launch_dequantize(const uint8_t* q, const float* s, int64_t M, int64_t K, int group, void* out,
                             bool out_bf16, int64_t ldo, hipStream_t st);

// One decode step (M <= 16, block-128 Hadamard with optional signs,
// 128-wide groups) in one launch: every wave quantizes the activation
// slices it consumes, then multiplies them.
hipError_t launch_decode_fused(const void* x, bool x_bf16, int64_t ldx, const uint32_t* sign_mask, float post,
                               const uint8_t* qw, const float* sw, int64_t M, int64_t N, int64_t K, void* y,
                               bool y_bf16, int64_t ldy, hipStream_t st);

hipError_t launch_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                       int64_t M, int64_t N, int64_t K, int group, void* y, bool y_bf16, int64_t ldy,
                       hipStream_t st);

}  // namespace rw4
