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
// Two kernels:
//   gemm_dl_kernel     M > 16: 128 x 128 block tiles, 4 waves of 64 x 64,
//                      v_mfma_i32_32x32x32_i8 (4 per group per 32 x 32 tile);
//                      the scale products sa * sw of a 32 x 32 tile come from
//                      one v_mfma_f32_32x32x16_bf16 on a 3-way bf16 split of
//                      each scale, so the VALU only converts and accumulates.
//   gemm_small_kernel  M <= 16 (decode): 16 output channels per block, the
//                      four waves split the groups, v_mfma_i32_16x16x64_i8
//                      with fragments loaded straight from global memory.
// MFMA layouts: lane l supplies row (l % T) of the A tile and row (l % T) of
// B^T (T = 32 or 16), 16 int8 values; lane l receives, for 32 x 32,
// D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32], r = 0..15, and for 16 x 16,
// D[4 (l / 16) + r][l % 16], r = 0..3.
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

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// bf16 truncations with a + b + c == x exactly (8 + 8 + 8 significant bits).
__device__ __forceinline__ void split3(float x, uint32_t& a, uint32_t& b, uint32_t& c) {
  const uint32_t xa = __float_as_uint(x) & 0xFFFF0000u;
  const float r1 = x - __uint_as_float(xa);
  const uint32_t xb = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(xb);
  a = xa >> 16;
  b = xb >> 16;
  c = __float_as_uint(r2) >> 16;
}

// ---------------------------------------------------------------------------
// Direct-to-LDS prefill kernel.  Packed INT4 tiles go from global memory
// straight into LDS (global_load_lds_dwordx4: no VGPR round trip, no VALU)
// through an S-stage ring, one 128-wide group per stage, with S - 1 groups
// in flight.  Each wave waits only for the oldest stage (vmcnt) before the
// block barrier.  LDS rows hold 64 packed bytes as four 16-byte slots, slot
// index XOR-swizzled by (row >> 2) & 3 so that 16 lanes reading 16 rows hit
// 16 distinct 4-bank groups.  Lane l of a 32 x 32 tile reads the 32 packed
// bytes [32 h, 32 h + 32) of its row (h = l / 32) and unpacks k-step ks from
// bytes 32 h + 8 ks .. + 8; A and B use the same order, so the dot product
// over the group is unchanged.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds_base, 4, 0, 0);
}
// Wait until at most n vector-memory instructions of this wave are in flight
// and all its LDS instructions are done, then a block barrier.  The asm
// barrier keeps the compiler from moving memory accesses across it without
// the memory-model fence that would wait for every in-flight DMA stage.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0x0 << 8) | ((N >> 4) << 14));
  asm volatile("s_barrier" ::: "memory");
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}
// Eight 16-byte LDS reads and four 4-byte LDS reads in one block that waits
// for all of them before returning (the results are complete on exit).  The
// data was produced by DMA that the caller has already waited for; keeping
// these reads out of the compiler's sight stops it from adding a wait for
// every DMA still in flight.
__device__ __forceinline__ void lds_read_8x16_4x4(v4u (&v)[8], uint32_t (&w)[4], const uint32_t (&a)[8],
                                                  const uint32_t (&b)[4]) {
  asm volatile(
      "ds_read_b128 %0, %12\n"
      "ds_read_b128 %1, %13\n"
      "ds_read_b128 %2, %14\n"
      "ds_read_b128 %3, %15\n"
      "ds_read_b128 %4, %16\n"
      "ds_read_b128 %5, %17\n"
      "ds_read_b128 %6, %18\n"
      "ds_read_b128 %7, %19\n"
      "ds_read_b32 %8, %20\n"
      "ds_read_b32 %9, %21\n"
      "ds_read_b32 %10, %22\n"
      "ds_read_b32 %11, %23\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
        "=&v"(v[7]), "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3])
      : "memory");
}

template <int BM, int BN>
struct alignas(16) DlStage {
  uint8_t a[BM * 64];
  uint8_t b[BN * 64];
  float sc[BM + BN + 64];  // sa rows, then sw rows, then a landing area for padding loads
};

template <int BM, int BN, int WM, int WN, int S, bool BF16>
__global__ __launch_bounds__(256) void gemm_dl_kernel(const uint8_t* __restrict__ qa,
                                                      const float* __restrict__ sa,
                                                      const uint8_t* __restrict__ qw,
                                                      const float* __restrict__ sw, int64_t M,
                                                      int64_t N, int64_t K, void* __restrict__ y,
                                                      int64_t ldy) {
  constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * WAVES_N == 4, "4 waves");
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int IA = BM / 64, IB = BN / 64;          // 1 KB DMA instructions per wave
  constexpr int SC_BLOCKS = (BM + BN) / 64;          // 64-scale blocks per stage
  constexpr int SCI = (SC_BLOCKS + 3) / 4;           // scale DMA instructions per wave
  constexpr int LPW = IA + IB + SCI;                 // vector-memory instructions per wave per stage
  static_assert(S >= 2 && S <= 4, "stages");
  static_assert((S - 2) * LPW < 64, "vmcnt");

  __shared__ DlStage<BM, BN> st0;
  __shared__ DlStage<BM, BN> st1;
  __shared__ DlStage<BM, BN> st2;
  __shared__ DlStage<BM, BN> st3;
  auto stage = [&](int i) -> DlStage<BM, BN>& {
    return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : st3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int64_t G = K / kGroup;
  const int64_t rowbytes = K / 2;
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t m0 = (blockIdx.x % tiles_m) * BM;
  const int64_t n0 = (blockIdx.x / tiles_m) * BN;

  // per-lane DMA source offsets (rows clamped into range: every wave issues
  // the same instructions; data of clamped rows is never stored)
  const int srow = lane >> 2;                                   // row within a 16-row block
  const int schunk = ((lane & 3) ^ ((lane >> 4) & 3)) * 16;     // swizzled source chunk
  int64_t a_off[IA], b_off[IB];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int64_t m = m0 + (wave * IA + i) * 16 + srow;
    a_off[i] = (m < M ? m : M - 1) * rowbytes + schunk;
  }
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    const int64_t n = n0 + (wave * IB + i) * 16 + srow;
    b_off[i] = (n < N ? n : N - 1) * rowbytes + schunk;
  }
  // scale block q of a stage: sa rows [64q, 64q + 64) for q < BM / 64, then
  // sw rows; blocks past SC_BLOCKS are padding loads (uniform instruction
  // count per wave) that land in the spare area and are never read
  const float* sc_src[SCI];
  int64_t sc_step[SCI];
  int sc_dst[SCI];
#pragma unroll
  for (int j = 0; j < SCI; ++j) {
    const int q = wave * SCI + j;
    if (q < BM / 64) {
      const int64_t m = m0 + q * 64 + lane;
      sc_src[j] = sa + (m < M ? m : M - 1) * G;
      sc_step[j] = 1;
      sc_dst[j] = q * 64;
    } else if (q < SC_BLOCKS) {
      const int64_t n = n0 + (q - BM / 64) * 64 + lane;
      sc_src[j] = sw + (n < N ? n : N - 1) * G;
      sc_step[j] = 1;
      sc_dst[j] = q * 64;
    } else {
      sc_src[j] = sa;
      sc_step[j] = 0;
      sc_dst[j] = BM + BN;
    }
  }

  auto issue = [&](DlStage<BM, BN>& stg, int64_t g) {
#pragma unroll
    for (int i = 0; i < IA; ++i) dma16(qa + a_off[i] + g * 64, stg.a + (wave * IA + i) * 1024);
#pragma unroll
    for (int i = 0; i < IB; ++i) dma16(qw + b_off[i] + g * 64, stg.b + (wave * IB + i) * 1024);
#pragma unroll
    for (int j = 0; j < SCI; ++j) dma4(sc_src[j] + sc_step[j] * g, stg.sc + sc_dst[j]);
  };

  float yacc[TM][TN][16];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) yacc[i][j][r] = 0.0f;

  const int frow = lane & 31, h = lane >> 5;
  auto compute = [&](DlStage<BM, BN>& stg) {
    // packed fragments: 8 dwords per tile row/column, plus the scales this
    // lane needs (one per tile row/column)
    static_assert(TM == 2 && TN == 2, "batched LDS read assumes a 2 x 2 tile grid per wave");
    uint32_t pa[TM][8], pb[TN][8];
    uint32_t addr[8], saddr[4];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WM + i * 32 + frow;
      const int f = (r >> 2) & 3;
      addr[2 * i] = lds_off(stg.a + r * 64 + (((2 * h) ^ f) * 16));
      addr[2 * i + 1] = lds_off(stg.a + r * 64 + (((2 * h + 1) ^ f) * 16));
      saddr[i] = lds_off(stg.sc + wm * WM + i * 32 + frow);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * WN + j * 32 + frow;
      const int f = (r >> 2) & 3;
      addr[4 + 2 * j] = lds_off(stg.b + r * 64 + (((2 * h) ^ f) * 16));
      addr[4 + 2 * j + 1] = lds_off(stg.b + r * 64 + (((2 * h + 1) ^ f) * 16));
      saddr[2 + j] = lds_off(stg.sc + BM + wn * WN + j * 32 + frow);
    }
    v4u rv[8];
    uint32_t rs[4];
    lds_read_8x16_4x4(rv, rs, addr, saddr);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pa[i][e] = rv[2 * i][e];
        pa[i][4 + e] = rv[2 * i + 1][e];
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[j][e] = rv[4 + 2 * j][e];
        pb[j][4 + e] = rv[4 + 2 * j + 1][e];
      }
    }
    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      v4i fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = v4i{int(unpack_lo(pa[i][2 * ks])), int(unpack_hi(pa[i][2 * ks])),
                    int(unpack_lo(pa[i][2 * ks + 1])), int(unpack_hi(pa[i][2 * ks + 1]))};
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = v4i{int(unpack_lo(pb[j][2 * ks])), int(unpack_hi(pb[j][2 * ks])),
                    int(unpack_lo(pb[j][2 * ks + 1])), int(unpack_hi(pb[j][2 * ks + 1]))};
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    {
      v8bf va[TM], vb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (h == 0) {
          uint32_t a1, a2, a3;
          split3(__uint_as_float(rs[i]) * (1.0f / 256.0f), a1, a2, a3);
          u = make_uint4(a1 | (a1 << 16), a2 | (a1 << 16), a2 | (a3 << 16), 0u);
        }
        va[i] = __builtin_bit_cast(v8bf, u);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (h == 0) {
          uint32_t b1, b2, b3;
          split3(__uint_as_float(rs[2 + j]), b1, b2, b3);
          u = make_uint4(b1 | (b2 << 16), b1 | (b3 << 16), b2 | (b1 << 16), 0u);
        }
        vb[j] = __builtin_bit_cast(v8bf, u);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          v16f p = {};
          p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], vb[j], p, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) yacc[i][j][r] = fmaf(float(acc[i][j][r]), p[r], yacc[i][j][r]);
        }
      }
    }
  };

  // prologue: groups 0 .. S-2 in flight.  Every iteration issues exactly one
  // stage (past the last group it reloads group G-1 into a stage that is
  // never read again), so the in-flight count is the same static number
  // everywhere and the compiler can track which stage each DMA writes.
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(stage(s), s < G ? s : G - 1);

  for (int64_t g0 = 0; g0 < G; g0 += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int64_t g = g0 + u;
      if (g >= G) break;
      // group g has landed for every wave after the barrier; stage u-1
      // (read in the previous iteration) is free for reuse
      wait_vm_barrier<(S - 2) * LPW>();
      const int64_t gn = g + S - 1;
      issue(stage((u + S - 1) % S), gn < G ? gn : G - 1);
      compute(stage(u));
    }
  }
  // drain the trailing loads: no DMA may outlive the block's LDS allocation
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));

#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + wn * WN + j * 32 + frow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * WM + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        if (m < M && n < N) store_y<BF16>(y, ldy, m, n, yacc[i][j][r]);
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

template <int BM, int BN, int WM, int WN, int S>
static hipError_t launch_dl(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                            int64_t M, int64_t N, int64_t K, void* y, bool y_bf16, int64_t ldy,
                            hipStream_t st) {
  const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (y_bf16)
    hipLaunchKernelGGL((gemm_dl_kernel<BM, BN, WM, WN, S, true>), dim3(blocks), dim3(256), 0, st,
                       qa, sa, qw, sw, M, N, K, y, ldy);
  else
    hipLaunchKernelGGL((gemm_dl_kernel<BM, BN, WM, WN, S, false>), dim3(blocks), dim3(256), 0, st,
                       qa, sa, qw, sw, M, N, K, y, ldy);
  return hipGetLastError();
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
  return launch_dl<128, 128, 64, 64, 2>(qa, sa, qw, sw, M, N, K, y, y_bf16, ldy, st);
}

}  // namespace rw4
