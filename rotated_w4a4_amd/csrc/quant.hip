// Fused transform + INT4 quantize + pack kernels (gfx950).
//
// One HBM pass over the activations: load, rotate in registers, group
// absmax, round, pack, store (the independent-rotation article on
// codearts.csdn.net, section 3.2, fuses rotate + scale + quantize in one
// kernel; the QuIP#/QTIP page on mhpn.cn, section 4.2, factors the Hadamard
// matrix into butterflies).  The same kernels, fed by a strided gather,
// pack the weights offline.
//
// Kernel families:
//   quant_h128_act  block-128 Hadamard, group-128 scales, row-major
//                   activations: 16 lanes own one (row, group), each lane
//                   8 consecutive channels; 3 butterfly stages in registers
//                   + 4 across lanes as DPP-fused multiply-adds; persistent
//                   waves that prefetch their next row.
//   quant_h128      the same transform for the offline weight pack (any
//                   strides; lane distance 4 through ds_swizzle).
//   quant_rowh      one wave per row for Hadamard blocks up to the whole row
//                   (K = 512 * E / 8): lane i holds channels 512c + 8i + e,
//                   so bits 0-2 and 9+ are register stages and bits 3-8 are
//                   lane stages.  Modes: group-128 scales, or the second
//                   pass of Rotated Runtime Smooth (divide by the group
//                   maxima, per-token scale).
//   rrs_colmax      first RRS pass: the same row transform, then the maximum
//                   of |x~| over all rows per 128-channel group
//                   (the Rotated Runtime Smooth page, main equation: s_j is
//                   a max over tokens; Figure 4 (2): one scale per block).
//   quant_givens    ParoQuant-style layers of disjoint pair rotations from
//                   a lookup table, then the alpha scale, in LDS.
#include "rw4_device.h"
#include "rw4_internal.h"

namespace rw4 {

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// quant_h128
// ---------------------------------------------------------------------------
// A block covers 16 U consecutive groups of one row: wave w of the block
// takes groups [4 (U w + u), 4 (U w + u) + 4) for u < U, 16 lanes per
// group, 8 channels per lane (one 16-byte load for bf16).  Blocks run over
// rows and their group ranges in a flat 1-D grid; the row and range come
// from the block index (uniform), so the lanes do no index division.
// GS: quantization group, 64 (lanes 0-7 / 8-15 of a group's 16), 128, or
// 256 (two adjacent groups of a quad).
template <class Src, int U, int GS>
__global__ __launch_bounds__(256) void quant_h128_kernel(Src src, int64_t G, int64_t blocks_per_row,
                                                         uint8_t* __restrict__ q, float* __restrict__ s,
                                                         float post_scale) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int seg = lane >> 4;   // which group of the quad
  const int sub = lane & 15;   // 8-channel slice of the group
  const int64_t row = int64_t(blockIdx.x) / blocks_per_row;
  const int64_t g_blk = (int64_t(blockIdx.x) - row * blocks_per_row) * (16 * U);

  float v[U][8];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t grp = g_blk + (wave * U + u) * 4 + seg;
    if (grp < G) {
      src.load8(row, grp * kGroup + sub * 8, v[u]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[u][e] = 0.0f;
    }
  }
  uint8_t* qrow = q + row * (G * 64);
  float* srow = s + row * (G * kGroup / GS);
  // lane stages in the negating form: the values of this lane end up
  // multiplied by flip = (-1)^popcount(lane & 15), undone in the encoder
  const float c1 = (lane & 1) ? -1.0f : 1.0f, c2 = (lane & 2) ? -1.0f : 1.0f;
  const float c4 = (lane & 4) ? -1.0f : 1.0f, c8 = (lane & 8) ? -1.0f : 1.0f;
  const float flip = (__builtin_popcount(lane & 15) & 1) ? -1.0f : 1.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    fwht8(v[u]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = v[u][e];
      x = butterfly_neg_x<1>(x, c1);
      x = butterfly_neg_x<2>(x, c2);
      x = butterfly_neg_x<4>(x, c4);
      x = butterfly_neg_x<8>(x, c8);
      v[u][e] = x;
    }
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[u][e]));
    m = max_x<1>(m);
    m = max_x<2>(m);
    m = max_x<4>(m);
    if constexpr (GS >= 128) m = max_x<8>(m);
    if constexpr (GS == 256) m = max_x<16>(m);
    uint32_t b[8];
    encode<8>(v[u], m, b, flip);
    const uint32_t packed = pack8_bits(b);
    const int64_t grp = g_blk + (wave * U + u) * 4 + seg;
    if (grp < G) {
      reinterpret_cast<uint32_t*>(qrow + grp * 64)[sub] = packed;
      if constexpr (GS == 64) {
        if ((sub & 7) == 0) srow[grp * 2 + (sub >> 3)] = m * post_scale;
      } else if constexpr (GS == 128) {
        if (sub == 0) srow[grp] = m * post_scale;
      } else {
        if ((lane & 31) == 0) srow[grp >> 1] = m * post_scale;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// quant_h128_act: the activation form of quant_h128 (row-major X) as a
// persistent loop.  Wave w keeps one quad of groups (quad w % Q of Q per
// row) and walks the rows w / Q, w / Q + R, ...; the load of the next row
// is issued before the current one is transformed (D rows ahead), so the
// memory system has work queued while the wave computes.  Every pass issues
// the same memory operations (rows past the end use empty buffer ranges),
// which keeps the compiler's counted waits exact across the loop.
//
// The four lane stages run along lane masks 1, 2, 7 and 8, each one DPP
// move (quad_perm, row_half_mirror, row_ror:8) fused into a v_fmac_f32:
// x += c_k * x[lane ^ m_k] with c_k = (-1)^parity(lane & t_k) for the dual
// functionals t = (5, 6, 4, 8) (parity(m_j & t_k) = [j == k]).  The product
// of these stages is the Walsh-Hadamard transform of the 16-lane index up
// to a signed permutation: lane l ends with (-1)^popcount(l) times the
// outputs of Sylvester lane f(l), where f is GF(2)-linear with f(1) = 5,
// f(2) = 6, f(4) = 7, f(8) = 8.  The sign is undone in the encoder (the
// absolute maximum is unchanged) and the packed word is stored at word f(l)
// of the group.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int h128_lane_word(int l) {
  return ((l & 1) ? 5 : 0) ^ ((l & 2) ? 6 : 0) ^ ((l & 4) ? 7 : 0) ^ (l & 8);
}
__device__ __forceinline__ float parity_sign(int x) { return (__builtin_popcount(x) & 1) ? -1.0f : 1.0f; }

// The four lane stages on 8 values (asm: the compiler does not fuse the DPP
// move into the multiply-add).  Each DPP read follows the write of its
// register by at least 2 wait states: s_nop 1 at entry, then 8 independent
// instructions between the stages of one value.
__device__ __forceinline__ void lane_stages_dpp(float (&v)[8], float c1, float c2, float c7, float c8) {
#define RW4_STAGE(CTRL, C)                                            \
  "v_fmac_f32_dpp %0, %0, " C " " CTRL " row_mask:0xf bank_mask:0xf\n" \
  "v_fmac_f32_dpp %1, %1, " C " " CTRL " row_mask:0xf bank_mask:0xf\n" \
  "v_fmac_f32_dpp %2, %2, " C " " CTRL " row_mask:0xf bank_mask:0xf\n" \
  "v_fmac_f32_dpp %3, %3, " C " " CTRL " row_mask:0xf bank_mask:0xf\n" \
  "v_fmac_f32_dpp %4, %4, " C " " CTRL " row_mask:0xf bank_mask:0xf\n" \
  "v_fmac_f32_dpp %5, %5, " C " " CTRL " row_mask:0xf bank_mask:0xf\n" \
  "v_fmac_f32_dpp %6, %6, " C " " CTRL " row_mask:0xf bank_mask:0xf\n" \
  "v_fmac_f32_dpp %7, %7, " C " " CTRL " row_mask:0xf bank_mask:0xf\n"
  asm volatile("s_nop 1\n"
               RW4_STAGE("quad_perm:[1,0,3,2]", "%8")
               RW4_STAGE("quad_perm:[2,3,0,1]", "%9")
               RW4_STAGE("row_half_mirror", "%10")
               RW4_STAGE("row_ror:8", "%11")
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
                 "+v"(v[7])
               : "v"(c1), "v"(c2), "v"(c7), "v"(c8));
#undef RW4_STAGE
}
// Maximum over the 16 lanes of a DPP row (lane masks 1, 2, 7, 8 span them).
__device__ __forceinline__ float row16_max_dpp(float m) {
  asm volatile(
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n"
      : "+v"(m));
  return m;
}

// Buffer resource over [base, base + bytes), bytes < 2^31 (checked on the
// host); raw access: a lane whose offset lies outside reads zeros and its
// store is dropped, and a resource of 0 bytes touches no memory at all.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;

// 2 x 2 transposes of a register pair and lane bit 4 (swap16) or lane bit 5
// (swap32): afterwards a holds the values of lane bit 0 of (a, b), b those
// of lane bit 1, and the lane bit indexes the old register.
__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Maximum over each 8-lane half of a DPP row (lane masks 1, 2, 7).
__device__ __forceinline__ float row8_max_dpp(float m) {
  asm volatile(
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n"
      : "+v"(m));
  return m;
}

template <bool BF16>
struct RawRow {
  v4u32 w[BF16 ? 1 : 2];
};

// GS: quantization group (64, 128 or 256 channels).  The transform block
// stays 128: a 64-group is one 8-lane half of a DPP row (lane l holds
// Sylvester lane f(l), and f keeps lane bit 3), a 256-group two adjacent
// rows (lanes l and l ^ 16).
template <bool BF16, bool SIGNED, int D, int GS>
__global__ __launch_bounds__(256) void quant_h128_act_kernel(const void* __restrict__ x, int64_t ldx,
                                                             int64_t rows, int64_t G, int64_t Q, int64_t R,
                                                             const uint32_t* __restrict__ sign_mask,
                                                             uint8_t* __restrict__ q, float* __restrict__ s,
                                                             float post_scale) {
  constexpr int ES = BF16 ? 2 : 4;  // bytes per input element
  const int lane = threadIdx.x & 63;
  // wave index, Q and R below 2^31 (checked on the host): 32-bit division
  const uint32_t w = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  if (w >= uint32_t(Q * R)) return;
  const int64_t quad = w % uint32_t(Q), r0 = w / uint32_t(Q);
  const int sub = lane & 15;
  const int64_t grp = quad * 4 + (lane >> 4);
  const int64_t K = G * kGroup;
  // byte offsets inside one row; lanes of groups past the end fall outside
  // the row's buffer range (their loads read zeros, their stores vanish)
  const uint32_t x_off = uint32_t((grp * kGroup + sub * 8) * ES);
  const uint32_t q_off = uint32_t(grp * 64 + h128_lane_word(sub) * 4);
  const int64_t GSN = G * kGroup / GS;  // scale columns per row
  uint32_t s_off;
  if constexpr (GS == 64)
    s_off = (sub & 7) == 0 ? uint32_t((grp * 2 + (sub >> 3)) * 4) : kOutOfRange;
  else if constexpr (GS == 128)
    s_off = sub == 0 ? uint32_t(grp * 4) : kOutOfRange;
  else
    s_off = (lane & 31) == 0 ? uint32_t((grp >> 1) * 4) : kOutOfRange;

  uint32_t smask[8];
  if constexpr (SIGNED) {
#pragma unroll
    for (int e = 0; e < 8; ++e) smask[e] = grp < G ? sign_mask[grp * kGroup + sub * 8 + e] : 0u;
  }
  const float c1 = parity_sign(lane & 5), c2 = parity_sign(lane & 6);
  const float c7 = parity_sign(lane & 4), c8 = parity_sign(lane & 8);
  const float flip = parity_sign(lane & 15);

  // rows at or past the end get an empty range: the prefetch past the last
  // row is issued like any other (so every path has the same memory
  // operations in flight) but reads nothing
  auto load = [&](int64_t row) {
    RawRow<BF16> raw;
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(reinterpret_cast<const uint8_t*>(x) + row * ldx * ES,
                                              row < rows ? K * ES : 0);
#pragma unroll
    for (int i = 0; i < (BF16 ? 1 : 2); ++i)
      raw.w[i] = __builtin_amdgcn_raw_buffer_load_b128(r, int(x_off + 16 * i), 0, 0);
    return raw;
  };

  // issue order fixed (slot 0 first) and kept in the loop below, so the
  // counted wait before each slot's use leaves the later loads in flight
  RawRow<BF16> raw[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    raw[d] = load(r0 + d * R);
    __builtin_amdgcn_sched_barrier(0);
  }

  for (int64_t row0 = r0; row0 < rows; row0 += D * R) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      // a row past the end (the last pass of a wave whose row count is not
      // a multiple of D) is computed on zeros and stored into empty ranges
      const int64_t row = row0 + d * R;
      const bool live = row < rows;
      float v[8];
      if constexpr (BF16) {
        const v4u32 u = raw[d].w[0];
        v[0] = bf16_lo(u[0]); v[1] = bf16_hi(u[0]);
        v[2] = bf16_lo(u[1]); v[3] = bf16_hi(u[1]);
        v[4] = bf16_lo(u[2]); v[5] = bf16_hi(u[2]);
        v[6] = bf16_lo(u[3]); v[7] = bf16_hi(u[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(raw[d].w[e >> 2][e & 3]);
      }
      if constexpr (SIGNED) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ smask[e]);
      }
      raw[d] = load(row + D * R);
      fwht8(v);
      lane_stages_dpp(v, c1, c2, c7, c8);
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
      if constexpr (GS == 64) {
        m = row8_max_dpp(m);
      } else {
        m = row16_max_dpp(m);
        if constexpr (GS == 256) {
          float t = m;
          swap16(m, t);
          m = fmaxf(m, t);
        }
      }
      // groups whose maximum is below 2^-100 are lifted by 2^64 (exact) so
      // that 7 / m stays finite; rare, so the whole wave branches around it
      float mm = m;
      if (__builtin_amdgcn_ballot_w64(m > 0.0f && m < kTinyMax) != 0) {
        if (m > 0.0f && m < kTinyMax) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= kTinyLift;
          mm = m * kTinyLift;
        }
      }
      // 7 / m as the hardware reciprocal of m / 7: a few ulp from the rounded
      // quotient, which moves v * 7 / m by ~1e-6 of a code step at most.
      // (The reciprocal flushes subnormal results, so it is taken of m / 7,
      // whose reciprocal is normal for every finite m >= 2^-100; 1 / m is
      // not, for m above 2^126.)
      const float inv = mm > 0.0f ? flip * __builtin_amdgcn_rcpf(mm * (1.0f / 7.0f)) : 0.0f;
      uint32_t b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = rne_code_bits(v[e], inv);
      const uint32_t packed = pack8_bits(b);
      const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + row * (G * 64), live ? G * 64 : 0);
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(s + row * GSN, live ? GSN * 4 : 0);
      __builtin_amdgcn_raw_buffer_store_b32(packed, rq, int(q_off), 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m * post_scale), rs, int(s_off), 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------------------
// quant_rowh / rrs_colmax: one wave per row, E = K / 64 channels per lane.
// ---------------------------------------------------------------------------
template <int E, class Src>
__device__ __forceinline__ void load_row(const Src& src, int64_t row, int lane, float v[E]) {
#pragma unroll
  for (int c = 0; c < E / 8; ++c) src.load8(row, int64_t(c) * 512 + lane * 8, &v[c * 8]);
}

// Unnormalized Walsh-Hadamard transform over blocks of 2^log2b channels.
template <int E>
__device__ __forceinline__ void fwht_row(float v[E], int lane, int log2b) {
  // bits 0..2: inside each 8-register chunk
#pragma unroll
  for (int c = 0; c < E / 8; ++c) fwht8(&v[c * 8]);
  // bits 3..8: across lanes (lane bit = index bit - 3)
  if (log2b > 3) {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = butterfly_x<1>(v[e], lane);
  }
  if (log2b > 4) {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = butterfly_x<2>(v[e], lane);
  }
  if (log2b > 5) {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = butterfly_x<4>(v[e], lane);
  }
  if (log2b > 6) {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = butterfly_x<8>(v[e], lane);
  }
  if (log2b > 7) {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = butterfly_x<16>(v[e], lane);
  }
  if (log2b > 8) {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = butterfly_x<32>(v[e], lane);
  }
  // bits 9..: across chunks, in registers
#pragma unroll
  for (int hc = 1; hc < E / 8; hc <<= 1) {
    if ((hc << 9) >= (1 << log2b)) break;
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
      if ((c & hc) == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = v[c * 8 + e], b = v[(c | hc) * 8 + e];
          v[c * 8 + e] = a + b;
          v[(c | hc) * 8 + e] = a - b;
        }
      }
    }
  }
}

// Max |v| over the 16 lanes x 8 registers of chunk c (one 128-channel group).
template <int E>
__device__ __forceinline__ float group_absmax(const float v[E], int c) {
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[c * 8 + e]));
  m = max_x<1>(m);
  m = max_x<2>(m);
  m = max_x<4>(m);
  m = max_x<8>(m);
  return m;
}

template <int E, class Src, bool RRS>
__global__ __launch_bounds__(256) void quant_rowh_kernel(Src src, int64_t M, int log2b,
                                                         uint8_t* __restrict__ q, float* __restrict__ s,
                                                         const float* __restrict__ smooth,
                                                         float post_scale) {
  constexpr int NC = E / 8;           // chunks per lane
  constexpr int64_t G = E / 2;        // K / 128
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const int sub = lane & 15;

  // RRS: reciprocal of this lane's group maxima (group of chunk c = 4c + lane/16)
  float inv_s[NC], s_g[NC];
  if constexpr (RRS) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      s_g[c] = smooth[c * 4 + (lane >> 4)];
      inv_s[c] = safe_inv(s_g[c], 1.0f);
    }
  }

  for (int64_t row = wave; row < M; row += n_waves) {
    float v[E];
    load_row<E>(src, row, lane, v);
    fwht_row<E>(v, lane, log2b);
    uint32_t* qrow = reinterpret_cast<uint32_t*>(q + row * (G * 64));
    if constexpr (!RRS) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float m = group_absmax<E>(v, c);
        uint32_t b[8];
        encode<8>(&v[c * 8], m, b);
        qrow[c * 64 + lane] = pack8_bits(b);
        if (sub == 0) s[row * G + c * 4 + (lane >> 4)] = m * post_scale;
      }
    } else {
      float m = 0.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[c * 8 + e] *= inv_s[c];
          m = fmaxf(m, fabsf(v[c * 8 + e]));
        }
      }
      m = max_x<1>(m);
      m = max_x<2>(m);
      m = max_x<4>(m);
      m = max_x<8>(m);
      m = max_x<16>(m);
      m = max_x<32>(m);
      const float a_t = m * (1.0f / 7.0f);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint32_t b[8];
        encode<8>(&v[c * 8], m, b);
        qrow[c * 64 + lane] = pack8_bits(b);
        if (sub == 0) s[row * G + c * 4 + (lane >> 4)] = a_t * (s_g[c] * post_scale);
      }
    }
  }
}

// First RRS pass.  smooth[] must be zero on entry (fill_kernel); it receives
// max over rows of the unnormalized |H x| per 128-channel group.  Values
// are non-negative, so their float bit patterns order like unsigned ints.
template <int E, class Src>
__global__ __launch_bounds__(256) void rrs_colmax_kernel(Src src, int64_t M, int log2b,
                                                         float* __restrict__ smooth) {
  constexpr int NC = E / 8;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  float gmax[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) gmax[c] = 0.0f;
  for (int64_t row = wave; row < M; row += n_waves) {
    float v[E];
    load_row<E>(src, row, lane, v);
    fwht_row<E>(v, lane, log2b);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) gmax[c] = fmaxf(gmax[c], fabsf(v[c * 8 + e]));
    }
  }
  __shared__ float red[4][E / 2];
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float m = gmax[c];
    m = max_x<1>(m);
    m = max_x<2>(m);
    m = max_x<4>(m);
    m = max_x<8>(m);
    if ((lane & 15) == 0) red[w][c * 4 + (lane >> 4)] = m;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < E / 2; g += blockDim.x) {
    const float m = fmaxf(fmaxf(red[0][g], red[1][g]), fmaxf(red[2][g], red[3][g]));
    if (m > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(smooth) + g, __float_as_uint(m));
  }
}

// ---------------------------------------------------------------------------
// Rotated Runtime Smooth with the Hadamard block equal to the whole row,
// K = 512 NC (NC >= 4 chunks of 8 channels per lane).  Lane l, chunk c,
// register e hold channel 512 c + 8 l + e after the load.  Stages:
//   bits 0-2      in registers (fwht8),
//   bits 9..      in registers, across chunks,
//   bits 3-6      lane bits 0-3 by the fused DPP stages of quant_h128_act,
//   bits 7, 8     lane bits 4, 5: v_permlane16_swap / v_permlane32_swap
//                 trade them for chunk bits 0, 1 (a 2 x 2 transpose of a
//                 register pair and a lane bit), then an in-register
//                 butterfly.
// Afterwards lane bits 0-3 hold f(l) (bits 3-6, see h128_lane_word), lane
// bits 4, 5 hold bits 9, 10, chunk bits 0, 1 hold bits 7, 8 and chunk bits
// 2.. hold bits 11..; the values of lane l carry the sign (-1)^popcount(l &
// 15).  A 128-channel group (bits 7.. fixed) is one chunk of one 16-lane
// DPP row.
// ---------------------------------------------------------------------------
template <int NC>
__device__ __forceinline__ int64_t rrs_word(int l, int c) {  // index of the 8-channel word
  return h128_lane_word(l & 15) | ((c & 3) << 4) | (((l >> 4) & 3) << 6) | (int64_t(c >> 2) << 8);
}
__device__ __forceinline__ int rrs_group(int l, int c) {  // 128-channel group
  return (c & 3) | (((l >> 4) & 3) << 2) | ((c >> 2) << 4);
}

template <int NC>
__device__ __forceinline__ void fwht_row_full(float (&v)[NC][8], float c1, float c2, float c7, float c8) {
#pragma unroll
  for (int c = 0; c < NC; ++c) fwht8(v[c]);
#pragma unroll
  for (int hc = 1; hc < NC; hc <<= 1) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c & hc) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a = v[c][e], b = v[c | hc][e];
        v[c][e] = a + b;
        v[c | hc][e] = a - b;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) lane_stages_dpp(v[c], c1, c2, c7, c8);
#pragma unroll
  for (int c = 0; c < NC; c += 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      swap16(v[c][e], v[c + 1][e]);
      const float a = v[c][e], b = v[c + 1][e];
      v[c][e] = a + b;
      v[c + 1][e] = a - b;
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c & 2) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      swap32(v[c][e], v[c + 2][e]);
      const float a = v[c][e], b = v[c + 2][e];
      v[c][e] = a + b;
      v[c + 2][e] = a - b;
    }
  }
}

template <int NC, bool BF16>
struct RawFullRow {
  v4u32 w[NC * (BF16 ? 1 : 2)];
};
template <int NC, bool BF16>
__device__ __forceinline__ RawFullRow<NC, BF16> load_full_row(const void* x, int64_t ldx, int64_t rows,
                                                              int64_t row, int lane) {
  constexpr int ES = BF16 ? 2 : 4;
  RawFullRow<NC, BF16> raw;
  const __amdgpu_buffer_rsrc_t r = buf_rsrc(reinterpret_cast<const uint8_t*>(x) + row * ldx * ES,
                                            row < rows ? int64_t(NC) * 512 * ES : 0);
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < (BF16 ? 1 : 2); ++i)
      raw.w[c * (BF16 ? 1 : 2) + i] =
          __builtin_amdgcn_raw_buffer_load_b128(r, (512 * c + 8 * lane) * ES + 16 * i, 0, 0);
  return raw;
}
template <int NC, bool BF16>
__device__ __forceinline__ void unpack_full_row(const RawFullRow<NC, BF16>& raw, float (&v)[NC][8]) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if constexpr (BF16) {
      const v4u32 u = raw.w[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[c][2 * i] = bf16_lo(u[i]);
        v[c][2 * i + 1] = bf16_hi(u[i]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[c][e] = __uint_as_float(raw.w[2 * c + (e >> 2)][e & 3]);
    }
  }
}

// First pass: per 128-channel group, the maximum of |H x| over all rows.
// smooth[] is zero on entry; waves reduce in registers, then per block in
// LDS, then one atomic maximum per group and block.
template <int NC, bool BF16>
__global__ __launch_bounds__(256) void rrs_colmax_full_kernel(const void* __restrict__ x, int64_t ldx,
                                                              int64_t rows, float* __restrict__ smooth) {
  constexpr int G = 4 * NC;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  // wave-uniform (the buffer descriptors built from it must be scalar)
  const int64_t w = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int64_t W = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const float c1 = parity_sign(lane & 5), c2 = parity_sign(lane & 6);
  const float c7 = parity_sign(lane & 4), c8 = parity_sign(lane & 8);
  float gmax[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) gmax[c] = 0.0f;
  RawFullRow<NC, BF16> raw = load_full_row<NC, BF16>(x, ldx, rows, w, lane);
  for (int64_t row = w; row < rows; row += W) {
    float v[NC][8];
    unpack_full_row<NC, BF16>(raw, v);
    raw = load_full_row<NC, BF16>(x, ldx, rows, row + W, lane);
    fwht_row_full<NC>(v, c1, c2, c7, c8);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) gmax[c] = fmaxf(gmax[c], fabsf(v[c][e]));
  }
  __shared__ float red[4][G];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float m = row16_max_dpp(gmax[c]);
    if ((lane & 15) == 0) red[wv][rrs_group(lane, c)] = m;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const float m = fmaxf(fmaxf(red[0][g], red[1][g]), fmaxf(red[2][g], red[3][g]));
    if (m > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(smooth) + g, __float_as_uint(m));
  }
}

// Second pass: z = (H x) / s_g (as a multiplication by 1 / s_g), per-token
// scale a_t = max |z| / 7, codes rne(z / a_t), stored scale a_t * s_g
// (times post_scale).
template <int NC, bool BF16>
__global__ __launch_bounds__(256) void quant_rrs_full_kernel(const void* __restrict__ x, int64_t ldx,
                                                             int64_t rows, const float* __restrict__ smooth,
                                                             uint8_t* __restrict__ q, float* __restrict__ s,
                                                             float post_scale) {
  constexpr int G = 4 * NC;
  const int lane = threadIdx.x & 63;
  // wave-uniform (the buffer descriptors built from it must be scalar)
  const int64_t w = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int64_t W = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const float c1 = parity_sign(lane & 5), c2 = parity_sign(lane & 6);
  const float c7 = parity_sign(lane & 4), c8 = parity_sign(lane & 8);
  const float flip = parity_sign(lane & 15);
  float inv_s[NC], sg[NC];
  uint32_t q_off[NC], s_off[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int g = rrs_group(lane, c);
    sg[c] = smooth[g];
    inv_s[c] = safe_inv(sg[c], 1.0f);
    q_off[c] = uint32_t(rrs_word<NC>(lane, c) * 4);
    s_off[c] = (lane & 15) == 0 ? uint32_t(g * 4) : kOutOfRange;
  }
  RawFullRow<NC, BF16> raw = load_full_row<NC, BF16>(x, ldx, rows, w, lane);
  for (int64_t row = w; row < rows; row += W) {
    float v[NC][8];
    unpack_full_row<NC, BF16>(raw, v);
    raw = load_full_row<NC, BF16>(x, ldx, rows, row + W, lane);
    fwht_row_full<NC>(v, c1, c2, c7, c8);
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[c][e] *= inv_s[c];
        m = fmaxf(m, fabsf(v[c][e]));
      }
    m = row16_max_dpp(m);
    {
      float t = m;
      swap16(m, t);
      m = fmaxf(m, t);
      t = m;
      swap32(m, t);
      m = fmaxf(m, t);
    }
    // rows whose maximum |z| is below 2^-100 are lifted by 2^64 (exact) so
    // that 7 / m stays finite (m is uniform over the wave)
    float mm = m;
    if (__builtin_amdgcn_ballot_w64(m > 0.0f && m < kTinyMax) != 0) {
      mm = m * kTinyLift;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[c][e] *= kTinyLift;
    }
    const float k = mm > 0.0f ? flip * __builtin_amdgcn_rcpf(mm * (1.0f / 7.0f)) : 0.0f;
    const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + row * (G * 64), G * 64);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(s + row * G, G * 4);
    const float a_t = m * (1.0f / 7.0f);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint32_t b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = rne_code_bits(v[c][e], k);
      __builtin_amdgcn_raw_buffer_store_b32(pack8_bits(b), rq, int(q_off[c]), 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a_t * (sg[c] * post_scale)), rs, int(s_off[c]), 0, 0);
    }
  }
}

__global__ void fill_kernel(float* p, int64_t n, float value) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

// ---------------------------------------------------------------------------
// quant_givens: one wave per (group, ROWS rows).  The lookup table holds,
// per (group, layer, slot), the pair (i | j << 8) and (cos, sin); every
// layer is a full matching of the 128 channels (padding pairs have angle 0).
// chan_scale is alpha^-1 for activations (x~ = x R D^-1) and alpha for
// weights (row n of W~^T is w_n^T R D).
// ---------------------------------------------------------------------------
template <class Src, int ROWS>
__global__ __launch_bounds__(64) void quant_givens_kernel(Src src, int64_t M, int64_t G, int L,
                                                          const uint16_t* __restrict__ lut_idx,
                                                          const float2* __restrict__ lut_cs,
                                                          const float* __restrict__ chan_scale,
                                                          uint8_t* __restrict__ q, float* __restrict__ s) {
  __shared__ float buf[ROWS][kGroup];
  const int lane = threadIdx.x;
  const int64_t grp = blockIdx.x % G;
  const int64_t row0 = (blockIdx.x / G) * ROWS;
  const int nrows = int(M - row0 < ROWS ? M - row0 : ROWS);

  const uint16_t* idx = lut_idx + grp * L * 64;
  const float2* cs = lut_cs + grp * L * 64;
  // the table entries of 8 layers are loaded together (one memory latency
  // per 8 layers instead of one per layer), then applied in order; the
  // first 8 are requested before the rows, so both latencies overlap
  constexpr int LB = 8;
  uint32_t pr[LB];
  float2 t[LB];
  auto load_tables = [&](int l0) {
#pragma unroll
    for (int k = 0; k < LB; ++k) {
      const bool in = l0 + k < L;
      pr[k] = in ? idx[(l0 + k) * 64 + lane] : 0u;
      t[k] = in ? cs[(l0 + k) * 64 + lane] : make_float2(1.0f, 0.0f);
    }
  };
  load_tables(0);
  const float sc0 = chan_scale[grp * kGroup + 2 * lane];
  const float sc1 = chan_scale[grp * kGroup + 2 * lane + 1];
  for (int r = 0; r < nrows; ++r) {
    float v[2];
    src.load2(row0 + r, grp * kGroup + 2 * lane, v);
    buf[r][2 * lane] = v[0];
    buf[r][2 * lane + 1] = v[1];
  }
  __syncthreads();
  for (int l0 = 0; l0 < L; l0 += LB) {
    if (l0 > 0) load_tables(l0);
#pragma unroll
    for (int k = 0; k < LB; ++k) {
      if (l0 + k >= L) break;
      const int i = pr[k] & 0xFF, j = pr[k] >> 8;
      for (int r = 0; r < nrows; ++r) {
        const float a = buf[r][i], b = buf[r][j];
        buf[r][i] = fmaf(t[k].x, a, t[k].y * b);
        buf[r][j] = fmaf(t[k].x, b, -t[k].y * a);
      }
      __syncthreads();
    }
  }
  for (int r = 0; r < nrows; ++r) {
    const float x0 = buf[r][2 * lane] * sc0;
    const float x1 = buf[r][2 * lane + 1] * sc1;
    float m = fmaxf(fabsf(x0), fabsf(x1));
    m = max_x<1>(m);
    m = max_x<2>(m);
    m = max_x<4>(m);
    m = max_x<8>(m);
    m = max_x<16>(m);
    m = max_x<32>(m);
    float xv[2] = {x0, x1};
    uint32_t b[2];
    encode<2>(xv, m, b);
    const uint32_t byte = pack2_bits_quad(b[0], b[1]);
    const int64_t row = row0 + r;
    q[row * (G * 64) + grp * 64 + lane] = uint8_t(byte);
    if (lane == 0) s[row * G + grp] = m * (1.0f / 7.0f);
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
namespace {

int grid_for_waves(int64_t waves_needed, int64_t cap_blocks) {
  int64_t blocks = (waves_needed + 3) / 4;  // 4 waves per 256-thread block
  if (blocks > cap_blocks) blocks = cap_blocks;
  if (blocks < 1) blocks = 1;
  return int(blocks);
}

// Row-major activations.  One row per wave while all (row, quad) items fit
// in one generation of resident waves (32 per CU), two rows up to two
// generations, else about three rows per wave: measured best at 2048 x 4096
// and 4096 x 14336 (more rows per wave leave the memory system less work in
// flight, fewer cost more setup; a deeper prefetch only added work at the
// end of each wave, and a wave covering 2 or 4 quads of a row instead of one
// was 7-14 % slower at 4096 x 14336).
template <int GS>
hipError_t launch_h128_act(const void* x, bool bf16, int64_t ldx, const uint32_t* sign_mask, int64_t rows,
                           int64_t G, uint8_t* q, float* s, float post, hipStream_t st) {
  constexpr int D = 1;
  constexpr int64_t kResidentWaves = 256 * 32;
  const int64_t Q = (G + 3) / 4;
  // rows per wave: 1 while the items fit one generation of resident waves, 2 up to two
  // generations (2048 x 4096: 6.05 us against 6.36 us with 3), else 3 (4096 x 14336)
  const int64_t rows_per_wave = Q * rows <= kResidentWaves ? 1 : Q * rows <= 2 * kResidentWaves ? 2 : 3;
  int64_t R = (rows + rows_per_wave - 1) / rows_per_wave;
  if (R < 1) R = 1;
  const int64_t blocks = (Q * R + 3) / 4;
  if (Q * R > 0x7FFFFFFF - 3 || G * 64 * (bf16 ? 4 : 8) >= (int64_t(1) << 31)) return hipErrorInvalidValue;
#define RW4_H128_ACT(B, S)                                                                              \
  hipLaunchKernelGGL((quant_h128_act_kernel<B, S, D, GS>), dim3(blocks), dim3(256), 0, st, x, ldx, rows, G, Q, R, \
                     sign_mask, q, s, post)
  if (bf16) {
    if (sign_mask) RW4_H128_ACT(true, true); else RW4_H128_ACT(true, false);
  } else {
    if (sign_mask) RW4_H128_ACT(false, true); else RW4_H128_ACT(false, false);
  }
#undef RW4_H128_ACT
  return hipGetLastError();
}

// Rotated Runtime Smooth over whole rows of K = 512 NC channels.
template <int NC>
hipError_t launch_rrs_full(const void* x, bool bf16, int64_t ldx, int64_t rows, uint8_t* q, float* s,
                           float* smooth, float post, hipStream_t st) {
  constexpr int64_t G = 4 * NC;
  constexpr int64_t kWaves = 256 * 12;
  const int64_t waves = rows < kWaves ? rows : kWaves;
  const int grid = int((waves + 3) / 4 > 0 ? (waves + 3) / 4 : 1);
  hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(256), 0, st, smooth, G, 0.0f);
  if (bf16) {
    hipLaunchKernelGGL((rrs_colmax_full_kernel<NC, true>), dim3(grid), dim3(256), 0, st, x, ldx, rows, smooth);
    hipLaunchKernelGGL((quant_rrs_full_kernel<NC, true>), dim3(grid), dim3(256), 0, st, x, ldx, rows,
                       (const float*)smooth, q, s, post);
  } else {
    hipLaunchKernelGGL((rrs_colmax_full_kernel<NC, false>), dim3(grid), dim3(256), 0, st, x, ldx, rows, smooth);
    hipLaunchKernelGGL((quant_rrs_full_kernel<NC, false>), dim3(grid), dim3(256), 0, st, x, ldx, rows,
                       (const float*)smooth, q, s, post);
  }
  return hipGetLastError();
}

template <int GS, class Src>
hipError_t launch_h128(const Src& src, int64_t rows, int64_t G, uint8_t* q, float* s, float post,
                       hipStream_t st) {
  // 16 groups per block, one quad of groups per wave: measured faster than
  // two quads per wave at both the 4096- and the 14336-channel shapes
  const int64_t bpr = (G + 15) / 16, blocks = rows * bpr;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((quant_h128_kernel<Src, 1, GS>), dim3(blocks), dim3(256), 0, st, src, G, bpr, q, s, post);
  return hipGetLastError();
}

template <int E, class Src>
hipError_t launch_rowh(const Src& src, int64_t rows, int log2b, bool rrs, uint8_t* q, float* s,
                       float* smooth, float post, hipStream_t st) {
  const int grid = grid_for_waves(rows, 256 * 16);
  if (rrs) {
    const int64_t G = E / 2;
    hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(256), 0, st, smooth, G, 0.0f);
    hipLaunchKernelGGL((rrs_colmax_kernel<E, Src>), dim3(grid), dim3(256), 0, st, src, rows, log2b,
                       smooth);
    hipLaunchKernelGGL((quant_rowh_kernel<E, Src, true>), dim3(grid), dim3(256), 0, st, src, rows,
                       log2b, q, s, (const float*)smooth, post);
  } else {
    hipLaunchKernelGGL((quant_rowh_kernel<E, Src, false>), dim3(grid), dim3(256), 0, st, src, rows,
                       log2b, q, s, (const float*)nullptr, post);
  }
  return hipGetLastError();
}

template <class Src>
hipError_t dispatch_rowh(const Src& src, int64_t K, int64_t rows, int log2b, bool rrs, uint8_t* q,
                         float* s, float* smooth, float post, hipStream_t st) {
  switch (K) {
    case 512: return launch_rowh<8>(src, rows, log2b, rrs, q, s, smooth, post, st);
    case 1024: return launch_rowh<16>(src, rows, log2b, rrs, q, s, smooth, post, st);
    case 2048: return launch_rowh<32>(src, rows, log2b, rrs, q, s, smooth, post, st);
    case 4096: return launch_rowh<64>(src, rows, log2b, rrs, q, s, smooth, post, st);
    case 8192: return launch_rowh<128>(src, rows, log2b, rrs, q, s, smooth, post, st);
    default: return hipErrorInvalidValue;
  }
}

template <class Src>
hipError_t launch_givens(const Src& src, int64_t rows, int64_t G, int L, const uint16_t* idx,
                         const float2* cs, const float* scale, uint8_t* q, float* s, hipStream_t st) {
  // few rows (decode): one row per wave, so the 8-layer dependency chain is
  // short and more waves run in parallel; many rows: 4 rows per wave
  if (rows <= 256) {
    const int64_t blocks = G * rows;
    hipLaunchKernelGGL((quant_givens_kernel<Src, 1>), dim3(blocks), dim3(64), 0, st, src, rows, G, L, idx,
                       cs, scale, q, s);
  } else {
    constexpr int ROWS = 4;
    const int64_t blocks = G * ((rows + ROWS - 1) / ROWS);
    hipLaunchKernelGGL((quant_givens_kernel<Src, ROWS>), dim3(blocks), dim3(64), 0, st, src, rows, G, L,
                       idx, cs, scale, q, s);
  }
  return hipGetLastError();
}

}  // namespace

bool rowh_supported(int64_t K) {
  return K == 512 || K == 1024 || K == 2048 || K == 4096 || K == 8192;
}

// Activations: X [M, K] row-major.
// group: 64, 128 or 256 for the block-128 Hadamard in per-group mode, else
// 128 (the caller checks).
hipError_t launch_quantize_act(const TransformDev& t, bool rrs, const void* x, bool bf16, int64_t M,
                               int64_t ldx, uint8_t* q, float* s, float* smooth, int group, hipStream_t st) {
  const int64_t K = t.K, G = K / kGroup;
  if (t.kind == TransformKind::Hadamard) {
    const float post = (rrs ? 1.0f : 1.0f / 7.0f) / sqrtf(float(t.block));
    int log2b = 0;
    while ((int64_t(1) << log2b) < t.block) ++log2b;
    if (t.block == 128 && !rrs) {
      if (group == 64) return launch_h128_act<64>(x, bf16, ldx, t.sign_mask, M, G, q, s, post, st);
      if (group == 256) return launch_h128_act<256>(x, bf16, ldx, t.sign_mask, M, G, q, s, post, st);
      return launch_h128_act<128>(x, bf16, ldx, t.sign_mask, M, G, q, s, post, st);
    }
    if (rrs && t.block == K && !t.sign_mask) {
      if (K == 2048) return launch_rrs_full<4>(x, bf16, ldx, M, q, s, smooth, post, st);
      if (K == 4096) return launch_rrs_full<8>(x, bf16, ldx, M, q, s, smooth, post, st);
      if (K == 8192) return launch_rrs_full<16>(x, bf16, ldx, M, q, s, smooth, post, st);
    }
    auto run = [&](const auto& src) { return dispatch_rowh(src, K, M, log2b, rrs, q, s, smooth, post, st); };
    if (t.sign_mask) {
      if (bf16) return run(SignedSrc<RowSrc<true>>{{x, ldx}, t.sign_mask});
      return run(SignedSrc<RowSrc<false>>{{x, ldx}, t.sign_mask});
    }
    if (bf16) return run(RowSrc<true>{x, ldx});
    return run(RowSrc<false>{x, ldx});
  }
  // Givens
  if (bf16)
    return launch_givens<RowSrc<true>>(RowSrc<true>{x, ldx}, M, G, t.layers, t.lut_idx,
                                              t.lut_cs, t.alpha_inv, q, s, st);
  return launch_givens<RowSrc<false>>(RowSrc<false>{x, ldx}, M, G, t.layers, t.lut_idx,
                                             t.lut_cs, t.alpha_inv, q, s, st);
}

// Weights: element (k, n) at w[k * sk + n * sn]; rows of the output are n.
// group: 128, or 64 / 256 for the block-128 Hadamard (the caller checks).
hipError_t launch_pack_weight(const TransformDev& t, const void* w, bool bf16, int64_t N, int64_t sk,
                              int64_t sn, uint8_t* q, float* s, int group, hipStream_t st) {
  const int64_t K = t.K, G = K / kGroup;
  if (t.kind == TransformKind::Hadamard) {
    const float post = (1.0f / 7.0f) / sqrtf(float(t.block));
    int log2b = 0;
    while ((int64_t(1) << log2b) < t.block) ++log2b;
    // W_tilde = R^T W with R = diag(signs) H / sqrt(b): H / sqrt(b) applied
    // to the rows of diag(signs) W, so the same sign flip on channel k
    auto run = [&](const auto& src) {
      if (t.block == 128 && group == 256) return launch_h128<256>(src, N, G, q, s, post, st);
      if (t.block == 128 && group == 64) return launch_h128<64>(src, N, G, q, s, post, st);
      if (t.block == 128) return launch_h128<128>(src, N, G, q, s, post, st);
      return dispatch_rowh(src, K, N, log2b, false, q, s, nullptr, post, st);
    };
    if (t.sign_mask) {
      if (bf16) return run(SignedSrc<StridedSrc<true>>{{w, sk, sn}, t.sign_mask});
      return run(SignedSrc<StridedSrc<false>>{{w, sk, sn}, t.sign_mask});
    }
    if (bf16) return run(StridedSrc<true>{w, sk, sn});
    return run(StridedSrc<false>{w, sk, sn});
  }
  if (bf16)
    return launch_givens<StridedSrc<true>>(StridedSrc<true>{w, sk, sn}, N, G, t.layers,
                                                 t.lut_idx, t.lut_cs, t.alpha, q, s, st);
  return launch_givens<StridedSrc<false>>(StridedSrc<false>{w, sk, sn}, N, G, t.layers,
                                                t.lut_idx, t.lut_cs, t.alpha, q, s, st);
}

}  // namespace rw4
