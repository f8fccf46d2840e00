// C ABI of the rotated W4A4 library: argument checks, transform objects,
// dispatch to the kernel launchers.  See include/rw4.h for the contract.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/rw4.h"
#include "rw4_internal.h"

struct rw4_transform {
  rw4::TransformDev dev;
  int device;
};

namespace {

constexpr int64_t kGroup = 128;
constexpr int kSlots = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

rw4_status from_hip(hipError_t e) {
  if (e == hipSuccess) return RW4_OK;
  if (e == hipErrorOutOfMemory) return RW4_ERR_NOMEM;
  return RW4_ERR_HIP;
}

// Host tables beyond this many channels are refused (no GEMM takes K above
// 2^24 either), so the host staging vectors stay bounded.
constexpr int64_t kMaxK = int64_t(1) << 24;

// A transform with device tables must be used on the device it was created on.
bool on_home_device(const rw4_transform* t) {
  const bool tables = t->dev.lut_idx || t->dev.sign_mask;
  if (!tables) return true;
  int d = -1;
  return hipGetDevice(&d) == hipSuccess && d == t->device;
}

}  // namespace

// Scratch of rw4_quantize_act_static: the Rotated Runtime Smooth group
// maxima s_g (K / 128 floats, K <= 8192) for callers that cannot allocate.
// Each GPU holds its own copy for the life of the process; every call on a
// GPU uses that GPU's copy.
constexpr int64_t kScratchFloats = 64;
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's copy of `scratch`, looked up on the
// first call on that GPU (with it current) and kept.  The array's name is
// only a host-side stand-in: kernels get this address.
hipError_t scratch_address(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* rw4_status_str(rw4_status s) {
  switch (s) {
    case RW4_OK: return "RW4_OK";
    case RW4_ERR_ARG: return "RW4_ERR_ARG: invalid argument (null, unknown enum, misaligned, or bad table)";
    case RW4_ERR_SHAPE: return "RW4_ERR_SHAPE: invalid shape (K % 128, group does not divide K, block, layers)";
    case RW4_ERR_UNSUPPORTED: return "RW4_ERR_UNSUPPORTED: valid but unimplemented combination";
    case RW4_ERR_HIP: return "RW4_ERR_HIP: HIP runtime call or kernel launch failed";
    case RW4_ERR_NOMEM: return "RW4_ERR_NOMEM: device allocation failed";
  }
  return "RW4_ERR_UNKNOWN";
}

const char* rw4_version(void) { return "0.1.0"; }

int64_t rw4_transform_k(const rw4_transform* t) { return t ? t->dev.K : 0; }

rw4_status rw4_transform_hadamard(int64_t K, int32_t block, void* stream, rw4_transform** out) {
  (void)stream;
  if (!out) return RW4_ERR_ARG;
  *out = nullptr;
  if (K <= 0 || K % kGroup) return RW4_ERR_SHAPE;
  if (!pow2(block) || block < 128 || block > K || K % block) return RW4_ERR_SHAPE;
  if (block > 128 && !rw4::rowh_supported(K)) return RW4_ERR_UNSUPPORTED;
  auto* t = new (std::nothrow) rw4_transform();
  if (!t) return RW4_ERR_NOMEM;
  t->dev = rw4::TransformDev{rw4::TransformKind::Hadamard, K, block, 0, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (hipGetDevice(&t->device) != hipSuccess) t->device = -1;
  *out = t;
  return RW4_OK;
}

static rw4_status transform_hadamard_signed_impl(int64_t K, int32_t block, const int8_t* signs_host,
                                        void* stream, rw4_transform** out) {
  if (!out) return RW4_ERR_ARG;
  *out = nullptr;
  if (!signs_host) return RW4_ERR_ARG;
  if (K <= 0 || K % kGroup || K > kMaxK) return RW4_ERR_SHAPE;
  if (!pow2(block) || block < 128 || block > K || K % block) return RW4_ERR_SHAPE;
  if (block > 128 && !rw4::rowh_supported(K)) return RW4_ERR_UNSUPPORTED;
  std::vector<uint32_t> mask(K);
  for (int64_t k = 0; k < K; ++k) {
    if (signs_host[k] != 1 && signs_host[k] != -1) return RW4_ERR_ARG;
    mask[k] = signs_host[k] < 0 ? 0x80000000u : 0u;
  }
  auto* t = new (std::nothrow) rw4_transform();
  if (!t) return RW4_ERR_NOMEM;
  t->dev = rw4::TransformDev{rw4::TransformKind::Hadamard, K, block, 0, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (hipGetDevice(&t->device) != hipSuccess) {
    delete t;
    return RW4_ERR_HIP;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMalloc(&t->dev.sign_mask, K * sizeof(uint32_t));
  if (e == hipSuccess)
    e = hipMemcpyAsync(t->dev.sign_mask, mask.data(), K * sizeof(uint32_t), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);  // the host table dies on return
  if (e != hipSuccess) {
    rw4_transform_destroy(t);
    return from_hip(e);
  }
  *out = t;
  return RW4_OK;
}

rw4_status rw4_transform_hadamard_signed(int64_t K, int32_t block, const int8_t* signs_host,
                                        void* stream, rw4_transform** out) {
  try {  // host staging vectors: no exception may cross the C ABI
    return transform_hadamard_signed_impl(K, block, signs_host, stream, out);
  } catch (...) {
    return RW4_ERR_NOMEM;
  }
}

static rw4_status transform_givens_impl(int64_t K, int32_t layers, const uint8_t* pairs_host,
                                const float* theta_host, const float* beta_host, void* stream,
                                rw4_transform** out) {
  if (!out) return RW4_ERR_ARG;
  *out = nullptr;
  if (!pairs_host || !theta_host || !beta_host) return RW4_ERR_ARG;
  if (K <= 0 || K % kGroup || K > kMaxK) return RW4_ERR_SHAPE;
  if (layers < 1 || layers > 64) return RW4_ERR_SHAPE;
  const int64_t G = K / kGroup;
  const size_t n_slots = size_t(G) * layers * kSlots;
  std::vector<uint16_t> idx(n_slots);
  std::vector<float> cs(2 * n_slots);
  std::vector<float> alpha(K), alpha_inv(K);

  for (int64_t g = 0; g < G; ++g) {
    for (int l = 0; l < layers; ++l) {
      const size_t base = (size_t(g) * layers + l) * kSlots;
      bool used[kGroup] = {};
      int n_real = 0;
      // real pairs first, in slot order
      for (int s = 0; s < kSlots; ++s) {
        const uint8_t i = pairs_host[(base + s) * 2], j = pairs_host[(base + s) * 2 + 1];
        if (i == 0xFF && j == 0xFF) continue;
        if (i >= kGroup || j >= kGroup || i >= j || used[i] || used[j]) return RW4_ERR_ARG;
        used[i] = used[j] = true;
        const double th = double(theta_host[base + s]);
        if (!std::isfinite(th)) return RW4_ERR_ARG;
        idx[base + n_real] = uint16_t(i | (j << 8));
        cs[2 * (base + n_real)] = float(std::cos(th));
        cs[2 * (base + n_real) + 1] = float(std::sin(th));
        ++n_real;
      }
      // pad with zero-angle pairs of the unused channels: exactly the identity
      int pending = -1, s = n_real;
      for (int c = 0; c < kGroup; ++c) {
        if (used[c]) continue;
        if (pending < 0) {
          pending = c;
        } else {
          idx[base + s] = uint16_t(pending | (c << 8));
          cs[2 * (base + s)] = 1.0f;
          cs[2 * (base + s) + 1] = 0.0f;
          ++s;
          pending = -1;
        }
      }
      if (s != kSlots) return RW4_ERR_ARG;  // unreachable: 128 channels always fill 64 slots
    }
  }
  for (int64_t k = 0; k < K; ++k) {
    const double b = double(beta_host[k]);
    alpha[k] = float(std::exp(b));
    alpha_inv[k] = float(std::exp(-b));
    // a non-finite beta, or one whose scale leaves the fp32 range, has no
    // usable channel scale
    if (!std::isfinite(b) || !std::isfinite(alpha[k]) || !std::isfinite(alpha_inv[k]) || alpha[k] == 0.0f ||
        alpha_inv[k] == 0.0f)
      return RW4_ERR_ARG;
  }

  auto* t = new (std::nothrow) rw4_transform();
  if (!t) return RW4_ERR_NOMEM;
  t->dev = rw4::TransformDev{rw4::TransformKind::Givens, K, 0, layers, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (hipGetDevice(&t->device) != hipSuccess) {
    delete t;
    return RW4_ERR_HIP;
  }
  hipError_t e = hipMalloc(&t->dev.lut_idx, n_slots * sizeof(uint16_t));
  if (e == hipSuccess) e = hipMalloc(&t->dev.lut_cs, n_slots * sizeof(float2));
  if (e == hipSuccess) e = hipMalloc(&t->dev.alpha, K * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&t->dev.alpha_inv, K * sizeof(float));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (e == hipSuccess) e = hipMemcpyAsync(t->dev.lut_idx, idx.data(), n_slots * sizeof(uint16_t), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipMemcpyAsync(t->dev.lut_cs, cs.data(), n_slots * sizeof(float2), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipMemcpyAsync(t->dev.alpha, alpha.data(), K * sizeof(float), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipMemcpyAsync(t->dev.alpha_inv, alpha_inv.data(), K * sizeof(float), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);  // host staging buffers die on return
  if (e != hipSuccess) {
    rw4_transform_destroy(t);
    return from_hip(e);
  }
  *out = t;
  return RW4_OK;
}

rw4_status rw4_transform_givens(int64_t K, int32_t layers, const uint8_t* pairs_host,
                                const float* theta_host, const float* beta_host, void* stream,
                                rw4_transform** out) {
  try {  // host staging vectors: no exception may cross the C ABI
    return transform_givens_impl(K, layers, pairs_host, theta_host, beta_host, stream, out);
  } catch (...) {
    return RW4_ERR_NOMEM;
  }
}

// IEEE binary16 bits to float (exact: every half value is a float).
static float half_bits_to_float(uint16_t h) {
  const uint32_t sign = uint32_t(h >> 15) << 31;
  const uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
  uint32_t bits;
  if (e == 0x1F) {
    bits = sign | 0x7F800000u | (m << 13);  // inf / nan
  } else if (e != 0) {
    bits = sign | ((e + 112) << 23) | (m << 13);
  } else if (m == 0) {
    bits = sign;
  } else {  // subnormal half: m * 2^-24
    float f = float(m) * 0x1p-24f;
    std::memcpy(&bits, &f, 4);
    bits |= sign;
  }
  float f;
  std::memcpy(&f, &bits, 4);
  return f;
}

static rw4_status transform_givens_f16_impl(int64_t K, int32_t layers, const uint8_t* pairs_host,
                                    const uint16_t* theta_f16_host, const float* beta_host, void* stream,
                                    rw4_transform** out) {
  if (!out) return RW4_ERR_ARG;
  *out = nullptr;
  if (!theta_f16_host) return RW4_ERR_ARG;
  if (K <= 0 || K % kGroup || K > kMaxK) return RW4_ERR_SHAPE;
  if (layers < 1 || layers > 64) return RW4_ERR_SHAPE;
  const size_t n = size_t(K / kGroup) * layers * kSlots;
  std::vector<float> theta(n);
  for (size_t i = 0; i < n; ++i) {
    theta[i] = half_bits_to_float(theta_f16_host[i]);
    if (!std::isfinite(theta[i])) return RW4_ERR_ARG;
  }
  return rw4_transform_givens(K, layers, pairs_host, theta.data(), beta_host, stream, out);
}

rw4_status rw4_transform_givens_f16(int64_t K, int32_t layers, const uint8_t* pairs_host,
                                    const uint16_t* theta_f16_host, const float* beta_host, void* stream,
                                    rw4_transform** out) {
  try {  // host staging vectors: no exception may cross the C ABI
    return transform_givens_f16_impl(K, layers, pairs_host, theta_f16_host, beta_host, stream, out);
  } catch (...) {
    return RW4_ERR_NOMEM;
  }
}

rw4_status rw4_transform_destroy(rw4_transform* t) {
  if (!t) return RW4_OK;
  hipError_t e = hipSuccess;
  for (void* p : {(void*)t->dev.lut_idx, (void*)t->dev.lut_cs, (void*)t->dev.alpha, (void*)t->dev.alpha_inv,
                  (void*)t->dev.sign_mask}) {
    if (p) {
      const hipError_t f = hipFree(p);
      if (e == hipSuccess) e = f;
    }
  }
  delete t;
  return from_hip(e);
}

static bool group_known(int32_t g) { return g == 64 || g == 128 || g == 256; }

rw4_status rw4_quantize_act_g(const rw4_transform* t, rw4_act_mode mode, int32_t group, const void* x,
                              rw4_dtype x_dtype, int64_t M, int64_t ldx, uint8_t* qa, float* sa,
                              float* workspace, void* stream) {
  if (!t) return RW4_ERR_ARG;
  if (mode != RW4_ACT_GROUP128 && mode != RW4_ACT_RRS_PER_TOKEN) return RW4_ERR_ARG;
  if (x_dtype != RW4_F32 && x_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (!group_known(group)) return RW4_ERR_ARG;
  if (M < 0) return RW4_ERR_SHAPE;
  const int64_t K = t->dev.K;
  if (K % group) return RW4_ERR_SHAPE;
  const bool rrs = mode == RW4_ACT_RRS_PER_TOKEN;
  if (rrs && (t->dev.kind != rw4::TransformKind::Hadamard || !rw4::rowh_supported(K)))
    return RW4_ERR_UNSUPPORTED;
  if (group != 128 && (rrs || t->dev.kind != rw4::TransformKind::Hadamard || t->dev.block != 128))
    return RW4_ERR_UNSUPPORTED;
  if (!on_home_device(t)) return RW4_ERR_ARG;
  if (M == 0) return RW4_OK;
  if (!x || !qa || !sa) return RW4_ERR_ARG;
  if (rrs && !workspace) return RW4_ERR_ARG;
  if (ldx < K) return RW4_ERR_ARG;
  const int64_t esz = x_dtype == RW4_BF16 ? 2 : 4;
  if (!aligned16(x) || (ldx * esz) % 16 || !aligned16(qa) || !aligned16(sa)) return RW4_ERR_ARG;
  if (rrs && !aligned16(workspace)) return RW4_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_quantize_act(t->dev, rrs, x, x_dtype == RW4_BF16, M, ldx, qa, sa,
                                           workspace, group, st));
}

rw4_status rw4_quantize_act(const rw4_transform* t, rw4_act_mode mode, const void* x,
                            rw4_dtype x_dtype, int64_t M, int64_t ldx, uint8_t* qa, float* sa,
                            float* workspace, void* stream) {
  return rw4_quantize_act_g(t, mode, 128, x, x_dtype, M, ldx, qa, sa, workspace, stream);
}

rw4_status rw4_quantize_act_asym(const rw4_transform* t, const void* x, rw4_dtype x_dtype, int64_t M, int64_t ldx,
                                 uint8_t* qa, float* sa, float* za, void* stream) {
  if (!t) return RW4_ERR_ARG;
  if (x_dtype != RW4_F32 && x_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (M < 0) return RW4_ERR_SHAPE;
  if (t->dev.kind != rw4::TransformKind::Hadamard || t->dev.block != 128) return RW4_ERR_UNSUPPORTED;
  if (!on_home_device(t)) return RW4_ERR_ARG;
  if (M == 0) return RW4_OK;
  if (!x || !qa || !sa || !za) return RW4_ERR_ARG;
  const int64_t K = t->dev.K;
  if (ldx < K) return RW4_ERR_ARG;
  const int64_t esz = x_dtype == RW4_BF16 ? 2 : 4;
  if (!aligned16(x) || (ldx * esz) % 16 || !aligned16(qa) || !aligned16(sa) || !aligned16(za)) return RW4_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_quantize_act_asym(t->dev, x, x_dtype == RW4_BF16, M, ldx, qa, sa, za, st));
}

rw4_status rw4_quantize_act_mixed(const rw4_transform* t, const void* x, rw4_dtype x_dtype, int64_t M, int64_t ldx,
                                  const int32_t* slot_of_group, int64_t n8, uint8_t* qa, float* sa, void* stream) {
  if (!t) return RW4_ERR_ARG;
  if (x_dtype != RW4_F32 && x_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (M < 0 || n8 < 0) return RW4_ERR_SHAPE;
  if (t->dev.kind != rw4::TransformKind::Hadamard || t->dev.block != 128) return RW4_ERR_UNSUPPORTED;
  const int64_t K = t->dev.K;
  if (n8 > K / kGroup) return RW4_ERR_SHAPE;
  if (!on_home_device(t)) return RW4_ERR_ARG;
  if (M == 0) return RW4_OK;
  if (!x || !slot_of_group || !qa || !sa) return RW4_ERR_ARG;
  if (ldx < K) return RW4_ERR_ARG;
  const int64_t esz = x_dtype == RW4_BF16 ? 2 : 4;
  if (!aligned16(x) || (ldx * esz) % 16 || !aligned16(qa) || !aligned16(sa)) return RW4_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_quantize_act_mixed(t->dev, x, x_dtype == RW4_BF16, M, ldx, slot_of_group, n8, qa, sa,
                                                 st));
}

rw4_status rw4_extend_weight_groups(const uint8_t* qw, const float* sw, int64_t N, int64_t K, const int32_t* groups8,
                                    int64_t n8, uint8_t* qw_ext, float* sw_ext, void* stream) {
  if (N < 0 || n8 < 0 || K <= 0 || K % kGroup || K > (int64_t(1) << 24) || n8 > K / kGroup) return RW4_ERR_SHAPE;
  if (N == 0) return RW4_OK;
  if (!qw || !sw || !qw_ext || !sw_ext || (n8 > 0 && !groups8)) return RW4_ERR_ARG;
  if (!aligned16(qw) || !aligned16(qw_ext)) return RW4_ERR_ARG;
  return from_hip(rw4::launch_extend_weight_groups(qw, sw, N, K, groups8, n8, qw_ext, sw_ext,
                                                   static_cast<hipStream_t>(stream)));
}

rw4_status rw4_weight_code_sums(const uint8_t* qw, int64_t N, int64_t K, float* cw, void* stream) {
  if (N < 0 || K <= 0 || K % kGroup || K > (int64_t(1) << 24)) return RW4_ERR_SHAPE;
  if (N == 0) return RW4_OK;
  if (!qw || !cw) return RW4_ERR_ARG;
  if (!aligned16(qw) || !aligned16(cw)) return RW4_ERR_ARG;
  return from_hip(rw4::launch_weight_code_sums(qw, N, K, cw, static_cast<hipStream_t>(stream)));
}

rw4_status rw4_w4a4_gemm_asym(const uint8_t* qa, const float* sa, const float* za, const uint8_t* qw,
                              const float* sw, const float* cw, int64_t M, int64_t N, int64_t K, void* y,
                              rw4_dtype y_dtype, int64_t ldy, void* stream) {
  if (y_dtype != RW4_F32 && y_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (M < 0 || N < 0 || K <= 0 || K % kGroup || K > (int64_t(1) << 24)) return RW4_ERR_SHAPE;
  if (M == 0 || N == 0) return RW4_OK;
  if (!qa || !sa || !za || !qw || !sw || !cw || !y) return RW4_ERR_ARG;
  if (ldy < N) return RW4_ERR_ARG;
  if (!aligned16(qa) || !aligned16(qw) || !aligned16(sa) || !aligned16(sw) || !aligned16(za) || !aligned16(cw) ||
      !aligned16(y))
    return RW4_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_gemm_asym(qa, sa, za, qw, sw, cw, M, N, K, y, y_dtype == RW4_BF16, ldy, st));
}

rw4_status rw4_dequantize_asym(const uint8_t* q, const float* s, const float* z, int64_t M, int64_t K, void* out,
                               rw4_dtype out_dtype, int64_t ldo, void* stream) {
  if (out_dtype != RW4_F32 && out_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (M < 0 || K <= 0 || K % kGroup) return RW4_ERR_SHAPE;
  if (M == 0) return RW4_OK;
  if (!q || !s || !z || !out) return RW4_ERR_ARG;
  if (ldo < K) return RW4_ERR_ARG;
  const int64_t esz = out_dtype == RW4_BF16 ? 2 : 4;
  if (!aligned16(q) || !aligned16(s) || !aligned16(z) || !aligned16(out) || (ldo * esz) % 16) return RW4_ERR_ARG;
  return from_hip(rw4::launch_dequantize_asym(q, s, z, M, K, out, out_dtype == RW4_BF16, ldo,
                                              static_cast<hipStream_t>(stream)));
}

rw4_status rw4_rotate_act(const rw4_transform* t, const void* x, rw4_dtype x_dtype, int64_t M, int64_t ldx,
                          void* out, rw4_dtype out_dtype, int64_t ldo, void* stream) {
  if (!t) return RW4_ERR_ARG;
  if (x_dtype != RW4_F32 && x_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (out_dtype != RW4_F32 && out_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (M < 0) return RW4_ERR_SHAPE;
  if (!on_home_device(t)) return RW4_ERR_ARG;
  if (M == 0) return RW4_OK;
  if (!x || !out) return RW4_ERR_ARG;
  const int64_t K = t->dev.K;
  if (ldx < K || ldo < K) return RW4_ERR_ARG;
  const int64_t xe = x_dtype == RW4_BF16 ? 2 : 4, oe = out_dtype == RW4_BF16 ? 2 : 4;
  if (!aligned16(x) || (ldx * xe) % 16 || !aligned16(out) || (ldo * oe) % 16) return RW4_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_rotate_act(t->dev, x, x_dtype == RW4_BF16, M, ldx, out, out_dtype == RW4_BF16,
                                         ldo, st));
}

rw4_status rw4_quantize_act_static(const rw4_transform* t, rw4_act_mode mode, const void* x, rw4_dtype x_dtype,
                                   int64_t M, int64_t ldx, uint8_t* qa, float* sa, void* stream) {
  if (mode != RW4_ACT_RRS_PER_TOKEN)  // no scratch needed: exactly rw4_quantize_act
    return rw4_quantize_act(t, mode, x, x_dtype, M, ldx, qa, sa, nullptr, stream);
  if (!t) return RW4_ERR_ARG;
  if (t->dev.K / kGroup > kScratchFloats) return RW4_ERR_SHAPE;  // beyond the static scratch
  // the checks of rw4_quantize_act come first (a NULL workspace would fail them)
  float* ws = nullptr;
  if (M > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return from_hip(e);
  }
  return rw4_quantize_act(t, mode, x, x_dtype, M, ldx, qa, sa, ws, stream);
}

rw4_status rw4_decode_fused(const rw4_transform* t, const void* x, rw4_dtype x_dtype, int64_t M, int64_t ldx,
                            const uint8_t* qw, const float* sw, int64_t N, void* y, rw4_dtype y_dtype, int64_t ldy,
                            void* stream) {
  if (!t) return RW4_ERR_ARG;
  if (x_dtype != RW4_F32 && x_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (y_dtype != RW4_F32 && y_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (M < 0 || M > 16 || N < 0) return RW4_ERR_SHAPE;
  if (t->dev.kind != rw4::TransformKind::Hadamard || t->dev.block != 128) return RW4_ERR_UNSUPPORTED;
  const int64_t K = t->dev.K;
  if (K > (int64_t(1) << 24)) return RW4_ERR_SHAPE;
  if (!on_home_device(t)) return RW4_ERR_ARG;
  if (M == 0 || N == 0) return RW4_OK;
  if (!x || !qw || !sw || !y) return RW4_ERR_ARG;
  if (ldx < K || ldy < N) return RW4_ERR_ARG;
  const int64_t esz = x_dtype == RW4_BF16 ? 2 : 4;
  if (!aligned16(x) || (ldx * esz) % 16 || !aligned16(qw) || !aligned16(sw) || !aligned16(y)) return RW4_ERR_ARG;
  // the kernel addresses x with 32-bit buffer offsets
  if (((M - 1) * ldx + K) * esz > 0x7FFFFFFF) return RW4_ERR_SHAPE;
  const float post = (1.0f / 7.0f) / sqrtf(128.0f);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_decode_fused(x, x_dtype == RW4_BF16, ldx, t->dev.sign_mask, post, qw, sw, M, N, K, y,
                                           y_dtype == RW4_BF16, ldy, st));
}

int64_t rw4_rrs_reorder_workspace_bytes(int64_t K) {
  if (K <= 0 || K % kGroup) return 0;
  return rw4::rrs_reorder_workspace_bytes(K);
}

rw4_status rw4_quantize_act_rrs_reorder(const rw4_transform* t, const void* x, rw4_dtype x_dtype, int64_t M,
                                        int64_t ldx, uint8_t* qa, float* sa, int32_t* order, void* workspace,
                                        void* stream) {
  if (!t) return RW4_ERR_ARG;
  if (x_dtype != RW4_F32 && x_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (M < 0) return RW4_ERR_SHAPE;
  const int64_t K = t->dev.K;
  if (t->dev.kind != rw4::TransformKind::Hadamard || !rw4::rrs_reorder_supported(K)) return RW4_ERR_UNSUPPORTED;
  if (!on_home_device(t)) return RW4_ERR_ARG;
  if (M == 0) return RW4_OK;
  if (!x || !qa || !sa || !order || !workspace) return RW4_ERR_ARG;
  if (ldx < K) return RW4_ERR_ARG;
  const int64_t esz = x_dtype == RW4_BF16 ? 2 : 4;
  if (!aligned16(x) || (ldx * esz) % 16 || !aligned16(qa) || !aligned16(sa) || !aligned16(order) ||
      !aligned16(workspace))
    return RW4_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_quantize_act_rrs_reorder(t->dev, x, x_dtype == RW4_BF16, M, ldx, qa, sa, order,
                                                       workspace, st));
}

rw4_status rw4_pack_weight_per_channel(const rw4_transform* t, const void* w, rw4_dtype w_dtype, int64_t N,
                                       int64_t stride_k, int64_t stride_n, uint8_t* qw, float* sw, void* stream) {
  if (!t) return RW4_ERR_ARG;
  if (w_dtype != RW4_F32 && w_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (N < 0) return RW4_ERR_SHAPE;
  if (t->dev.kind != rw4::TransformKind::Hadamard || !rw4::rowh_supported(t->dev.K)) return RW4_ERR_UNSUPPORTED;
  if (!on_home_device(t)) return RW4_ERR_ARG;
  if (N == 0) return RW4_OK;
  if (!w || !qw || !sw) return RW4_ERR_ARG;
  if (stride_k <= 0 || stride_n <= 0) return RW4_ERR_ARG;
  const int64_t esz = w_dtype == RW4_BF16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(w) % esz) || !aligned16(qw) || !aligned16(sw)) return RW4_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_pack_weight_per_channel(t->dev, w, w_dtype == RW4_BF16, N, stride_k, stride_n, qw, sw,
                                                      st));
}

rw4_status rw4_permute_codes(const uint8_t* q, int64_t rows, int64_t K, const int32_t* order, uint8_t* out,
                             void* stream) {
  if (rows < 0 || K <= 0 || K % kGroup || K > 8192) return RW4_ERR_SHAPE;
  if (rows == 0) return RW4_OK;
  if (!q || !order || !out || q == out) return RW4_ERR_ARG;
  if (!aligned16(q) || !aligned16(order) || !aligned16(out)) return RW4_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_permute_codes(q, rows, K, order, out, st));
}

rw4_status rw4_pack_weight_g(const rw4_transform* t, int32_t group, const void* w, rw4_dtype w_dtype,
                             int64_t N, int64_t stride_k, int64_t stride_n, uint8_t* qw, float* sw,
                             void* stream) {
  if (!t) return RW4_ERR_ARG;
  if (w_dtype != RW4_F32 && w_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (!group_known(group)) return RW4_ERR_ARG;
  if (N < 0) return RW4_ERR_SHAPE;
  if (t->dev.K % group) return RW4_ERR_SHAPE;
  // groups other than 128 with the block-128 Hadamard
  if (group != 128 && (t->dev.kind != rw4::TransformKind::Hadamard || t->dev.block != 128))
    return RW4_ERR_UNSUPPORTED;
  if (!on_home_device(t)) return RW4_ERR_ARG;
  if (N == 0) return RW4_OK;
  if (!w || !qw || !sw) return RW4_ERR_ARG;
  if (stride_k <= 0 || stride_n <= 0) return RW4_ERR_ARG;
  const int64_t esz = w_dtype == RW4_BF16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(w) % esz) || !aligned16(qw) || !aligned16(sw)) return RW4_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_pack_weight(t->dev, w, w_dtype == RW4_BF16, N, stride_k, stride_n, qw,
                                          sw, group, st));
}

rw4_status rw4_pack_weight(const rw4_transform* t, const void* w, rw4_dtype w_dtype, int64_t N,
                           int64_t stride_k, int64_t stride_n, uint8_t* qw, float* sw,
                           void* stream) {
  return rw4_pack_weight_g(t, 128, w, w_dtype, N, stride_k, stride_n, qw, sw, stream);
}

rw4_status rw4_dequantize_g(const uint8_t* q, const float* s, int64_t M, int64_t K, int32_t group, void* out,
                            rw4_dtype out_dtype, int64_t ldo, void* stream) {
  if (out_dtype != RW4_F32 && out_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (!group_known(group)) return RW4_ERR_ARG;
  if (M < 0 || K <= 0 || K % group) return RW4_ERR_SHAPE;
  if (M == 0) return RW4_OK;
  if (!q || !s || !out) return RW4_ERR_ARG;
  if (ldo < K) return RW4_ERR_ARG;
  const int64_t esz = out_dtype == RW4_BF16 ? 2 : 4;
  if (!aligned16(q) || !aligned16(s) || !aligned16(out) || (ldo * esz) % 16) return RW4_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_dequantize(q, s, M, K, group, out, out_dtype == RW4_BF16, ldo, st));
}

rw4_status rw4_dequantize(const uint8_t* q, const float* s, int64_t M, int64_t K, void* out,
                          rw4_dtype out_dtype, int64_t ldo, void* stream) {
  return rw4_dequantize_g(q, s, M, K, 128, out, out_dtype, ldo, stream);
}

rw4_status rw4_w4a4_gemm_g(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           int64_t M, int64_t N, int64_t K, int32_t group, void* y, rw4_dtype y_dtype,
                           int64_t ldy, void* stream) {
  if (y_dtype != RW4_F32 && y_dtype != RW4_BF16) return RW4_ERR_ARG;
  if (!group_known(group)) return RW4_ERR_ARG;
  if (M < 0 || N < 0 || K <= 0 || K % kGroup || K % group || K > (int64_t(1) << 24)) return RW4_ERR_SHAPE;
  if (M == 0 || N == 0) return RW4_OK;
  if (!qa || !sa || !qw || !sw || !y) return RW4_ERR_ARG;
  if (ldy < N) return RW4_ERR_ARG;
  if (!aligned16(qa) || !aligned16(qw) || !aligned16(sa) || !aligned16(sw) || !aligned16(y))
    return RW4_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return from_hip(rw4::launch_gemm(qa, sa, qw, sw, M, N, K, group, y, y_dtype == RW4_BF16, ldy, st));
}

rw4_status rw4_w4a4_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                         int64_t M, int64_t N, int64_t K, void* y, rw4_dtype y_dtype, int64_t ldy,
                         void* stream) {
  return rw4_w4a4_gemm_g(qa, sa, qw, sw, M, N, K, 128, y, y_dtype, ldy, stream);
}

}  // extern "C"
