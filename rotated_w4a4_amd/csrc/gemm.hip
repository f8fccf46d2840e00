// W4A4 GEMM on the gfx950 i8 matrix cores.
//
//   Y[m, n] = sum over 128-wide groups g of sa[m, g] * sw[n, g] * acc[m, n, g]
//   acc[m, n, g] = sum over k in g of qa[m, k] * qw[n, k]     (exact int32)
//
// (the Rotated Runtime Smooth page, main equation and Figure 4 (3): the
// GEMM block equals the quantization group and the scale multiplies the
// block's partial result; the QuIP#/QTIP page, section 4.2, folds the
// rotation into the weights so the GEMM itself is a plain product.)
//
// INT4 -> int8 unpack: for a packed dword d holding codes k0..k7 (code 2b
// in the low nibble of byte b), d & 0xF0F0F0F0 gives the odd codes and
// (d << 4) & 0xF0F0F0F0 the even codes, each byte equal to 16 * code, a
// valid int8.  Both operands use the same unpack, so the int32 result is
// 256 * acc exactly (|256 acc| <= 2^21); the 2^-8 is folded into the
// activation scale.  The unpack permutes codes inside each 8-code block,
// identically for A and B, which leaves the dot product unchanged.
//
// MFMA: v_mfma_i32_16x16x64_i8.  Lane l supplies row (l % 16) of the A tile
// and row (l % 16) of the B tile (= column of B^T), 16 bytes each; lane l
// receives D[4 * (l / 16) + r][l % 16], r = 0..3.
#include "rw4_device.h"
#include "rw4_internal.h"

namespace rw4 {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t unpack_lo(uint32_t d) { return (d << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t unpack_hi(uint32_t d) { return d & 0xF0F0F0F0u; }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ void store_y(void* y, int64_t ldy, int64_t m, int64_t n, float v) {
  if constexpr (BF16) {
    reinterpret_cast<uint16_t*>(y)[m * ldy + n] = f32_to_bf16_rne(v);
  } else {
    reinterpret_cast<float*>(y)[m * ldy + n] = v;
  }
}

// ---------------------------------------------------------------------------
// Prefill kernel: BM x BN block tile, 4 waves in a 2 x 2 layout, each wave
// WM x WN = (BM/2) x (BN/2) made of 16 x 16 MFMA tiles.  Per 128-wide group:
// packed tiles are loaded to registers (one group ahead), unpacked to int8
// into LDS, then every wave runs 2 MFMAs per tile and the fp32 epilogue.
// ---------------------------------------------------------------------------
constexpr int kRowBytes = 128 + 16;  // unpacked group row + pad (bank spread)

template <int BM, int BN, bool BF16>
__global__ __launch_bounds__(256) void gemm_prefill_kernel(const uint8_t* __restrict__ qa,
                                                           const float* __restrict__ sa,
                                                           const uint8_t* __restrict__ qw,
                                                           const float* __restrict__ sw, int64_t M,
                                                           int64_t N, int64_t K, void* __restrict__ y,
                                                           int64_t ldy) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int A_CHUNKS = BM * 4 / 256;  // 16-byte packed chunks per thread
  constexpr int B_CHUNKS = BN * 4 / 256;
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint8_t As[BM * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[BN * kRowBytes];
  __shared__ float sA[BM];
  __shared__ float sB[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t G = K / kGroup;
  const int64_t rowbytes = K / 2;

  // Tile order: consecutive blocks walk down M for a fixed N-strip.
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t m0 = (blockIdx.x % tiles_m) * BM;
  const int64_t n0 = (blockIdx.x / tiles_m) * BN;

  uint4 ra[A_CHUNKS], rb[B_CHUNKS];
  float rsa = 0.0f, rsb = 0.0f;

  auto load_group = [&](int64_t g) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 2, part = c & 3;
      const int64_t m = m0 + row;
      ra[i] = (m < M) ? *reinterpret_cast<const uint4*>(qa + m * rowbytes + g * 64 + part * 16)
                      : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 2, part = c & 3;
      const int64_t n = n0 + row;
      rb[i] = (n < N) ? *reinterpret_cast<const uint4*>(qw + n * rowbytes + g * 64 + part * 16)
                      : make_uint4(0, 0, 0, 0);
    }
    if (tid < BM) rsa = (m0 + tid < M) ? sa[(m0 + tid) * G + g] * (1.0f / 256.0f) : 0.0f;
    if (tid < BN) rsb = (n0 + tid < N) ? sw[(n0 + tid) * G + g] : 0.0f;
  };

  auto store_chunk = [&](uint8_t* base, int c, uint4 p) {
    const int row = c >> 2, part = c & 3;
    uint4* dst = reinterpret_cast<uint4*>(base + row * kRowBytes + part * 32);
    dst[0] = make_uint4(unpack_lo(p.x), unpack_hi(p.x), unpack_lo(p.y), unpack_hi(p.y));
    dst[1] = make_uint4(unpack_lo(p.z), unpack_hi(p.z), unpack_lo(p.w), unpack_hi(p.w));
  };

  float acc_y[TM][TN][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc_y[i][j][r] = 0.0f;

  load_group(0);
  for (int64_t g = 0; g < G; ++g) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) store_chunk(As, tid + 256 * i, ra[i]);
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) store_chunk(Bs, tid + 256 * i, rb[i]);
    if (tid < BM) sA[tid] = rsa;
    if (tid < BN) sB[tid] = rsb;
    __syncthreads();
    if (g + 1 < G) load_group(g + 1);

    v4i fa[TM][2], fb[TN][2];
    const int frow = lane & 15, fcol = (lane >> 4) * 16;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
        fa[i][kh] = *reinterpret_cast<const v4i*>(As + (wm * WM + i * 16 + frow) * kRowBytes + kh * 64 + fcol);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
        fb[j][kh] = *reinterpret_cast<const v4i*>(Bs + (wn * WN + j * 16 + frow) * kRowBytes + kh * 64 + fcol);

    float sa_r[TM][4], sb_c[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) sa_r[i][r] = sA[wm * WM + i * 16 + (lane >> 4) * 4 + r];
#pragma unroll
    for (int j = 0; j < TN; ++j) sb_c[j] = sB[wn * WN + j * 16 + (lane & 15)];

#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        v4i acc = {0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i][0], fb[j][0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i][1], fb[j][1], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc_y[i][j][r] = fmaf(float(acc[r]), sa_r[i][r] * sb_c[j], acc_y[i][j][r]);
      }
    }
  }

  // store
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + wn * WN + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * WM + i * 16 + (lane >> 4) * 4 + r;
        if (m < M && n < N) store_y<BF16>(y, ldy, m, n, acc_y[i][j][r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small-M kernel (decode, M <= 16): one block per 16 output channels; the
// 4 waves split the groups; A and B fragments come straight from global
// memory (16 bytes per lane per group, no reuse to stage); the partial
// results are summed across waves in LDS.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void gemm_small_kernel(const uint8_t* __restrict__ qa,
                                                         const float* __restrict__ sa,
                                                         const uint8_t* __restrict__ qw,
                                                         const float* __restrict__ sw, int64_t M,
                                                         int64_t N, int64_t K, void* __restrict__ y,
                                                         int64_t ldy) {
  constexpr int NB = 8;  // groups in flight per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t G = K / kGroup;
  const int64_t rowbytes = K / 2;
  const int64_t n0 = int64_t(blockIdx.x) * 16;
  const int64_t am = lane & 15;               // A row supplied by this lane
  const int64_t bn = n0 + (lane & 15);        // B row (output channel)
  const int part = lane >> 4;
  const bool a_ok = am < M, b_ok = bn < N;

  float yv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t gb = wave; gb < G; gb += 4 * NB) {
    uint4 pa[NB], pb[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int64_t g = gb + 4 * t;
      const bool in = g < G;
      pa[t] = (in && a_ok) ? *reinterpret_cast<const uint4*>(qa + am * rowbytes + g * 64 + part * 16)
                           : make_uint4(0, 0, 0, 0);
      pb[t] = (in && b_ok) ? *reinterpret_cast<const uint4*>(qw + bn * rowbytes + g * 64 + part * 16)
                           : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int64_t g = gb + 4 * t;
      if (g >= G) break;
      const v4i a0 = {int(unpack_lo(pa[t].x)), int(unpack_hi(pa[t].x)), int(unpack_lo(pa[t].y)), int(unpack_hi(pa[t].y))};
      const v4i a1 = {int(unpack_lo(pa[t].z)), int(unpack_hi(pa[t].z)), int(unpack_lo(pa[t].w)), int(unpack_hi(pa[t].w))};
      const v4i b0 = {int(unpack_lo(pb[t].x)), int(unpack_hi(pb[t].x)), int(unpack_lo(pb[t].y)), int(unpack_hi(pb[t].y))};
      const v4i b1 = {int(unpack_lo(pb[t].z)), int(unpack_hi(pb[t].z)), int(unpack_lo(pb[t].w)), int(unpack_hi(pb[t].w))};
      v4i acc = {0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc, 0, 0, 0);
      const float swv = b_ok ? sw[bn * G + g] * (1.0f / 256.0f) : 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = (lane >> 4) * 4 + r;
        const float sav = (m < M) ? sa[m * G + g] : 0.0f;
        yv[r] = fmaf(float(acc[r]), sav * swv, yv[r]);
      }
    }
  }
  __shared__ float red[4][64][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][lane][r] = yv[r];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = red[0][lane][r] + red[1][lane][r] + red[2][lane][r] + red[3][lane][r];
      const int64_t m = (lane >> 4) * 4 + r;
      if (m < M && b_ok) store_y<BF16>(y, ldy, m, bn, v);
    }
  }
}

hipError_t launch_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                       int64_t M, int64_t N, int64_t K, void* y, bool y_bf16, int64_t ldy,
                       hipStream_t st) {
  if (M <= 16) {
    const int64_t blocks = (N + 15) / 16;
    if (y_bf16)
      hipLaunchKernelGGL((gemm_small_kernel<true>), dim3(blocks), dim3(256), 0, st, qa, sa, qw, sw, M,
                         N, K, y, ldy);
    else
      hipLaunchKernelGGL((gemm_small_kernel<false>), dim3(blocks), dim3(256), 0, st, qa, sa, qw, sw, M,
                         N, K, y, ldy);
    return hipGetLastError();
  }
  constexpr int BM = 128, BN = 128;
  const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (y_bf16)
    hipLaunchKernelGGL((gemm_prefill_kernel<BM, BN, true>), dim3(blocks), dim3(256), 0, st, qa, sa, qw,
                       sw, M, N, K, y, ldy);
  else
    hipLaunchKernelGGL((gemm_prefill_kernel<BM, BN, false>), dim3(blocks), dim3(256), 0, st, qa, sa, qw,
                       sw, M, N, K, y, ldy);
  return hipGetLastError();
}

}  // namespace rw4
