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
#include <type_traits>

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
    const uint32_t packed = pack8_bits(b, (sub & 2) != 0);
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
// which keeps the compiler's counted waits exact across the loop.  The lane
// stages are lane_stages_dpp (rw4_device.h): lane l stores its packed word
// at word h128_lane_word(l) of the group.
// ---------------------------------------------------------------------------

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
// ASYM (GS = 128 only): the asymmetric (s, z) encoder (encode8_asym) with
// the unsigned stored form; zs receives the zero points as floats.
template <bool BF16, bool SIGNED, int D, int GS, bool ASYM = false, bool MIXED = false>
__global__ __launch_bounds__(256) void quant_h128_act_kernel(const void* __restrict__ x, int64_t ldx,
                                                             int64_t rows, int64_t G, int64_t Q, int64_t R,
                                                             const uint32_t* __restrict__ sign_mask,
                                                             uint8_t* __restrict__ q, float* __restrict__ s,
                                                             float post_scale, float* __restrict__ zs = nullptr,
                                                             const int32_t* __restrict__ slot_of_group = nullptr,
                                                             int64_t n8 = 0, float post8h = 0.0f, float post8l = 0.0f) {
  static_assert(!ASYM || GS == 128, "asymmetric groups of 128");
  static_assert(!MIXED || (GS == 128 && !ASYM), "8-bit groups: symmetric groups of 128");
  constexpr int ES = BF16 ? 2 : 4;  // bytes per input element
  const int lane = threadIdx.x & 63;
  // wave index (4 waves per block), Q * R below 2^31 (checked on the host):
  // fits 32 bits without forming the thread index, 32-bit division
  const uint32_t w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4u + (threadIdx.x >> 6));
  if (w >= uint32_t(Q * R)) return;
  const int64_t quad = w % uint32_t(Q), r0 = w / uint32_t(Q);
  const int sub = lane & 15;
  const int64_t grp = quad * 4 + (lane >> 4);
  const int64_t K = G * kGroup;
  // byte offsets inside one row; lanes of groups past the end fall outside
  // the row's buffer range (their loads read zeros, their stores vanish)
  const uint32_t x_off = uint32_t((grp * kGroup + sub * 8) * ES);
  const uint32_t q_off = uint32_t(grp * 64 + h128_lane_word(sub) * 4);
  const bool role = (h128_lane_word(sub) & 2) != 0;  // bit 1 of the word index: its place in the word pair
  // MIXED: rows of G + n8 groups; a listed group (slot_of_group >= 0) keeps
  // its h plane in place and its l plane in the extra group G + slot
  const int64_t GX = MIXED ? G + n8 : G;
  const int32_t slot = MIXED && grp < G ? slot_of_group[grp] : -1;
  // uniform over a group's 16 lanes, so the packers' exchange with lane ^ 3 stays inside one branch
  const bool is8 = MIXED && slot >= 0 && slot < n8;
  const bool any8 = MIXED && __builtin_amdgcn_ballot_w64(is8) != 0;  // wave-uniform
  const uint32_t l_off = is8 ? uint32_t((G + slot) * 64 + h128_lane_word(sub) * 4) : kOutOfRange;
  const uint32_t sl_off = is8 && sub == 0 ? uint32_t((G + slot) * 4) : kOutOfRange;
  const int64_t GSN = GX * kGroup / GS;  // scale columns per row
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
  const float s7 = signed_const(1.0f / 7.0f, flip);  // the encoder's signed 1/7

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
      if constexpr (ASYM) {
        // true signs (the lane stages leave every value times flip), then
        // the group's range with zero inside it
        float hi = 0.0f, nlo = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[e] *= flip;
          hi = fmaxf(hi, v[e]);
          nlo = fmaxf(nlo, -v[e]);
        }
        hi = row16_max_dpp(hi);
        nlo = row16_max_dpp(nlo);
        uint32_t z;
        const uint32_t packed = encode8_asym(v, hi, nlo, z, role);
        const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + row * (G * 64), live ? G * 64 : 0);
        const __amdgpu_buffer_rsrc_t rs = buf_rsrc(s + row * G, live ? G * 4 : 0);
        const __amdgpu_buffer_rsrc_t rz = buf_rsrc(zs + row * G, live ? G * 4 : 0);
        __builtin_amdgcn_raw_buffer_store_b32(packed, rq, int(q_off), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((hi + nlo) * post_scale), rs, int(s_off), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(float(z)), rz, int(s_off), 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        continue;
      }
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
      const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + row * (GX * 64), live ? GX * 64 : 0);
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(s + row * GSN, live ? GSN * 4 : 0);
      if constexpr (MIXED) {
        if (any8) {
          // the 8-bit groups: q8 = rne(112 x~ / m) split as 15 h + l (h = rne(q8 / 15),
          // never a tie), 112 / m the reciprocal of m / 112 (tiny maxima lifted as
          // in encode8_rcp); the other groups of the wave as below
          uint32_t packed, packed_l = 0u;
          float sc = m * post_scale, sc_l = 0.0f;
          if (is8) {
            float mm = m;
            if (tiny_positive(m)) {
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] *= kTinyLift;
              mm = m * kTinyLift;
            }
            const float inv = mm > 0.0f ? __builtin_amdgcn_rcpf(mm * signed_const(1.0f / 112.0f, flip)) : 0.0f;
            uint32_t bh[8], bl[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int q8 = int(rne_code_bits(v[e], inv) - kRoundMagicBits);
              const int h = int(rne_code_bits(float(q8), 1.0f / 15.0f) - kRoundMagicBits);
              bh[e] = kRoundMagicBits + uint32_t(h);
              bl[e] = kRoundMagicBits + uint32_t(q8 - 15 * h);
            }
            packed = pack8_bits(bh, role);
            packed_l = pack8_bits(bl, role);
            sc = m * post8h;
            sc_l = m * post8l;
          } else {
            packed = encode8_rcp(v, m, s7, role);
          }
          __builtin_amdgcn_raw_buffer_store_b32(packed, rq, int(q_off), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(packed_l, rq, int(l_off), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rs, int(s_off), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc_l), rs, int(sl_off), 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          continue;
        }
      }
      const uint32_t packed = encode8_rcp(v, m, s7, role);
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
        qrow[c * 64 + lane] = pack8_bits(b, (lane & 2) != 0);
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
        qrow[c * 64 + lane] = pack8_bits(b, (lane & 2) != 0);
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
    const float k = mm > 0.0f ? __builtin_amdgcn_rcpf(mm * signed_const(1.0f / 7.0f, flip)) : 0.0f;
    const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + row * (G * 64), G * 64);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(s + row * G, G * 4);
    const float a_t = m * (1.0f / 7.0f);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint32_t b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = rne_code_bits(v[c][e], k);
      __builtin_amdgcn_raw_buffer_store_b32(pack8_bits(b, (h128_lane_word(lane & 15) & 2) != 0), rq, int(q_off[c]), 0, 0);
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
    const uint32_t byte = pack2_bits_quad(b[0], b[1], lane & 3, (lane & 8) != 0);
    const int64_t row = row0 + r;
    q[row * (G * 64) + grp * 64 + lane] = uint8_t(byte);
    if (lane == 0) s[row * G + grp] = m * (1.0f / 7.0f);
  }
}

// ---------------------------------------------------------------------------
// Rotated Runtime Smooth with the channel reorder (the Rotated Runtime Smooth
// page, Figure 4 (1)-(2)): per-channel maxima of |x~| over all rows of the
// call, channels ordered by decreasing maximum (equal maxima by increasing
// index), groups of 128 consecutive reordered channels with the group's
// largest maximum as smoothing scale, then the per-token quantizer on the
// reordered row.  Row transforms of any Hadamard block (quant_rowh layout:
// lane l holds channels 512 c + 8 l + e in natural order).
//   rrs_chanmax      per-block maxima of every channel      -> partial [P][K]
//   chanmax_reduce   maximum over the P partial rows         -> m [K]
//   rrs_rank         rank of every channel, group scales     -> order [K], s [K/128]
//   quant_rrs_order  transform, gather the row in order through LDS, smooth,
//                    per-token INT4, pack (codes in reordered channel order)
// ---------------------------------------------------------------------------
constexpr int kChanmaxBlocks = 256;

template <int E, class Src>
__global__ __launch_bounds__(256) void rrs_chanmax_kernel(Src src, int64_t M, int log2b, float* __restrict__ partial) {
  constexpr int K = E * 64;
  __shared__ float red[K];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  float cmax[E];
#pragma unroll
  for (int e = 0; e < E; ++e) cmax[e] = 0.0f;
  for (int64_t row = wave; row < M; row += n_waves) {
    float v[E];
    load_row<E>(src, row, lane, v);
    fwht_row<E>(v, lane, log2b);
#pragma unroll
    for (int e = 0; e < E; ++e) cmax[e] = fmaxf(cmax[e], fabsf(v[e]));
  }
  // the four waves of the block in turn: wave 0 stores, the others take the maximum
  for (int t = 0; t < 4; ++t) {
    if (w == t) {
#pragma unroll
      for (int c = 0; c < E / 8; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = c * 512 + lane * 8 + e;
          red[j] = t == 0 ? cmax[c * 8 + e] : fmaxf(red[j], cmax[c * 8 + e]);
        }
    }
    __syncthreads();
  }
  for (int j = threadIdx.x; j < K; j += blockDim.x) partial[int64_t(blockIdx.x) * K + j] = red[j];
}

// m[j] = max over the P partial rows.  A block of 16 waves takes 64
// channels; wave w reads partial rows w, w + 16, ... (64 consecutive floats
// per row, all of a lane's loads in flight at once), then the 16 waves
// combine in LDS.  (One thread per channel over all P rows left 16 blocks
// waiting on memory latency: 61 us at K = 4096.)
__global__ __launch_bounds__(1024) void chanmax_reduce_kernel(const float* __restrict__ partial, int P, int64_t K,
                                                              float* __restrict__ m) {
  __shared__ float red[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t j = int64_t(blockIdx.x) * 64 + lane;
  float v = 0.0f;
  if (j < K) {
    int p = w;
    for (; p + 15 * 16 < P; p += 16 * 16) {
      float t[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) t[u] = partial[int64_t(p + 16 * u) * K + j];
#pragma unroll
      for (int u = 0; u < 16; ++u) v = fmaxf(v, t[u]);
    }
    for (; p < P; p += 16) v = fmaxf(v, partial[int64_t(p) * K + j]);
  }
  red[w][lane] = v;
  __syncthreads();
  if (w == 0 && j < K) {
    float r = red[0][lane];
#pragma unroll
    for (int k = 1; k < 16; ++k) r = fmaxf(r, red[k][lane]);
    m[j] = r;
  }
}

// rank(j) = #{i : m_i > m_j} + #{i < j : m_i == m_j}: the position of
// channel j in decreasing order of the maxima, equal maxima by increasing
// index (unique ranks, so order is a permutation).  The maxima are >= +0,
// so their bit patterns order like the values, and the order is that of
// the 44-bit keys bits(m_i) 2^13 + (8191 - i) (K <= 8192): i precedes j
// exactly when key_i > key_j, one 64-bit comparison with no branch.  A
// block takes 16 channels; its 16 groups of 16 threads count over 16
// slices of the keys, then add up.  The channel of rank 128 g opens group
// g, and its maximum is the group's smoothing scale.
__global__ __launch_bounds__(256) void rrs_rank_kernel(const float* __restrict__ m, int64_t K,
                                                       int32_t* __restrict__ order, float* __restrict__ s_g) {
  extern __shared__ v4u32 keys4[];  // K keys (two per 16 bytes), then 256 partial counts
  int* cnt = reinterpret_cast<int*>(keys4 + K / 2);
  {
    // K <= 8192: at most 8 16-byte loads of 4 maxima per thread, all issued
    // before the first LDS store (one memory latency instead of one per load)
    const __amdgpu_buffer_rsrc_t rm = buf_rsrc(m, K * 4);
    v4u32 t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i4 = threadIdx.x + 256 * u;  // 16-byte chunk; past K / 4 reads zeros
      t[u] = __builtin_amdgcn_raw_buffer_load_b128(rm, int(i4 < K / 4 ? uint32_t(i4 * 16) : kOutOfRange), 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i4 = threadIdx.x + 256 * u;
      if (i4 < K / 4) {
        uint32_t w[8];  // keys of channels 4 i4 .. 4 i4 + 3 as (low, high) words
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t idx = uint32_t(i4 * 4 + q);
          w[2 * q] = (t[u][q] << 13) | (8191u - idx);
          w[2 * q + 1] = t[u][q] >> 19;
        }
        keys4[i4 * 2] = v4u32{w[0], w[1], w[2], w[3]};
        keys4[i4 * 2 + 1] = v4u32{w[4], w[5], w[6], w[7]};
      }
    }
  }
  __syncthreads();
  auto key = [](uint32_t lo, uint32_t hi) { return (uint64_t(hi) << 32) | lo; };
  const int c = threadIdx.x & 15, r = threadIdx.x >> 4;
  const int j = int(blockIdx.x) * 16 + c;  // < K: the grid has K / 16 blocks
  const v4u32 kw = keys4[j / 2];
  const uint64_t kj = (j & 1) ? key(kw[2], kw[3]) : key(kw[0], kw[1]);
  const int pairs = int(K / 32);  // 16-byte reads per slice of K / 16 keys (K % 128 == 0)
  const v4u32* k2 = keys4 + r * pairs;
  int n = 0;
#pragma unroll 8
  for (int i = 0; i < pairs; ++i) {
    const v4u32 w = k2[i];
    n += int(key(w[0], w[1]) > kj) + int(key(w[2], w[3]) > kj);
  }
  cnt[threadIdx.x] = n;
  __syncthreads();
  if (r == 0) {
    int rank = 0;
    for (int k = 0; k < 16; ++k) rank += cnt[k * 16 + c];
    order[rank] = int32_t(j);
    if ((rank & (kGroup - 1)) == 0) s_g[rank / kGroup] = __uint_as_float(uint32_t(kj >> 13));
  }
}

// The reordered row (lane l: reordered positions 512 c + 8 l + e, group
// 4 c + l / 16) smoothed by its groups' scales, then the per-token INT4
// encoder; stored scale a_t s_g (times post_scale).
template <int NC>
__device__ __forceinline__ void rrs_order_encode(float* v, const float* inv_s, const float* s_g, int lane,
                                                 int64_t row, uint8_t* __restrict__ q, float* __restrict__ s,
                                                 float post_scale) {
  constexpr int64_t G = 4 * NC;
  const int sub = lane & 15;
  float m = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[c * 8 + e] *= inv_s[c];
      m = fmaxf(m, fabsf(v[c * 8 + e]));
    }
  m = max_x<1>(m);
  m = max_x<2>(m);
  m = max_x<4>(m);
  m = max_x<8>(m);
  m = max_x<16>(m);
  m = max_x<32>(m);
  const float a_t = m * (1.0f / 7.0f);
  uint32_t* qrow = reinterpret_cast<uint32_t*>(q + row * (G * 64));
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    uint32_t b[8];
    encode<8>(&v[c * 8], m, b);
    qrow[c * 64 + lane] = pack8_bits(b, (lane & 2) != 0);
    if (sub == 0) s[row * G + c * 4 + (lane >> 4)] = a_t * (s_g[c] * post_scale);
  }
}

// Second pass: one wave per row.  The transformed row goes to the wave's
// LDS slice in natural channel order and is read back in the given order,
// so lane l then holds reordered positions 512 c + 8 l + e; their group is
// 4 c + l / 16, as in quant_rowh.
template <int E, class Src>
__global__ __launch_bounds__(256) void quant_rrs_order_kernel(Src src, int64_t M, int log2b,
                                                              const int32_t* __restrict__ order,
                                                              const float* __restrict__ smooth,
                                                              uint8_t* __restrict__ q, float* __restrict__ s,
                                                              float post_scale) {
  constexpr int K = E * 64;
  constexpr int NC = E / 8;
  __shared__ float rowbuf[4][K];
  __shared__ int32_t ord[K];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  for (int j = threadIdx.x; j < K; j += blockDim.x) ord[j] = order[j];
  __syncthreads();
  float inv_s[NC], s_g[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    s_g[c] = smooth[c * 4 + (lane >> 4)];
    inv_s[c] = safe_inv(s_g[c], 1.0f);
  }
  float* buf = rowbuf[w];
  for (int64_t row = wave; row < M; row += n_waves) {
    float v[E];
    load_row<E>(src, row, lane, v);
    fwht_row<E>(v, lane, log2b);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) buf[c * 512 + lane * 8 + e] = v[c * 8 + e];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[c * 8 + e] = buf[ord[c * 512 + lane * 8 + e]];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    rrs_order_encode<NC>(v, inv_s, s_g, lane, row, q, s, post_scale);
  }
}

// Full-row fast path of the reorder (block = K = 512 NC, row-major source
// without random signs): the register / DPP transform of quant_rrs_full
// (lane l holds the values of word rrs_word(l, c), times flip), with the
// next row's loads in flight while a row is transformed.
template <int NC, bool BF16>
__global__ __launch_bounds__(256) void rrs_chanmax_full_kernel(const void* __restrict__ x, int64_t ldx, int64_t M,
                                                               float* __restrict__ partial) {
  constexpr int K = 512 * NC;
  __shared__ float red[K];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // wave-uniform (the buffer descriptors built from it must be scalar)
  const int64_t wave = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int64_t n_waves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const float c1 = parity_sign(lane & 5), c2 = parity_sign(lane & 6);
  const float c7 = parity_sign(lane & 4), c8 = parity_sign(lane & 8);
  float cmax[NC][8];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) cmax[c][e] = 0.0f;
  RawFullRow<NC, BF16> raw = load_full_row<NC, BF16>(x, ldx, M, wave, lane);
  for (int64_t row = wave; row < M; row += n_waves) {
    float v[NC][8];
    unpack_full_row<NC, BF16>(raw, v);
    raw = load_full_row<NC, BF16>(x, ldx, M, row + n_waves, lane);
    fwht_row_full<NC>(v, c1, c2, c7, c8);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) cmax[c][e] = fmaxf(cmax[c][e], fabsf(v[c][e]));
  }
  // the four waves of the block in turn: wave 0 stores, the others take the maximum
  for (int t = 0; t < 4; ++t) {
    if (w == t) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float* r = red + 8 * rrs_word<NC>(lane, c);
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = t == 0 ? cmax[c][e] : fmaxf(r[e], cmax[c][e]);
      }
    }
    __syncthreads();
  }
  for (int j = threadIdx.x; j < K; j += blockDim.x) partial[int64_t(blockIdx.x) * K + j] = red[j];
}

template <int NC, bool BF16>
__global__ __launch_bounds__(256) void quant_rrs_order_full_kernel(const void* __restrict__ x, int64_t ldx, int64_t M,
                                                                   const int32_t* __restrict__ order,
                                                                   const float* __restrict__ smooth,
                                                                   uint8_t* __restrict__ q, float* __restrict__ s,
                                                                   float post_scale) {
  constexpr int K = 512 * NC;
  constexpr int E = 8 * NC;
  __shared__ float rowbuf[4][K];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t wave = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int64_t n_waves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  // this lane's source channels (reordered positions 512 c + 8 l + e), two
  // 16-bit indices per register (K <= 8192), so the gather reads LDS once
  // per element
  uint32_t ord2[E / 2];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int4* src = reinterpret_cast<const int4*>(order + c * 512 + lane * 8);
    const int4 o0 = src[0], o1 = src[1];
    ord2[c * 4 + 0] = uint32_t(o0.x) | (uint32_t(o0.y) << 16);
    ord2[c * 4 + 1] = uint32_t(o0.z) | (uint32_t(o0.w) << 16);
    ord2[c * 4 + 2] = uint32_t(o1.x) | (uint32_t(o1.y) << 16);
    ord2[c * 4 + 3] = uint32_t(o1.z) | (uint32_t(o1.w) << 16);
  }
  float inv_s[NC], s_g[NC];
  uint32_t woff[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    s_g[c] = smooth[c * 4 + (lane >> 4)];
    inv_s[c] = safe_inv(s_g[c], 1.0f);
    woff[c] = uint32_t(8 * rrs_word<NC>(lane, c));
  }
  const float c1 = parity_sign(lane & 5), c2 = parity_sign(lane & 6);
  const float c7 = parity_sign(lane & 4), c8 = parity_sign(lane & 8);
  const float flip = parity_sign(lane & 15);
  float* buf = rowbuf[w];
  RawFullRow<NC, BF16> raw = load_full_row<NC, BF16>(x, ldx, M, wave, lane);
  for (int64_t row = wave; row < M; row += n_waves) {
    float t[NC][8];
    unpack_full_row<NC, BF16>(raw, t);
    raw = load_full_row<NC, BF16>(x, ldx, M, row + n_waves, lane);
    fwht_row_full<NC>(t, c1, c2, c7, c8);
    // the row in natural channel order (true signs) in this wave's slice
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float4* d = reinterpret_cast<float4*>(buf + woff[c]);
      d[0] = make_float4(t[c][0] * flip, t[c][1] * flip, t[c][2] * flip, t[c][3] * flip);
      d[1] = make_float4(t[c][4] * flip, t[c][5] * flip, t[c][6] * flip, t[c][7] * flip);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    float v[E];
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      v[2 * i] = buf[ord2[i] & 0xFFFFu];
      v[2 * i + 1] = buf[ord2[i] >> 16];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    rrs_order_encode<NC>(v, inv_s, s_g, lane, row, q, s, post_scale);
  }
}

// Per-output-channel weights: the row transform, then one symmetric INT4
// scale over the whole transformed row (max / 7), stored in every group
// column (the Rotated Runtime Smooth experimental setup quantizes weights
// per channel; a channel permutation then only permutes the codes).
template <int E, class Src>
__global__ __launch_bounds__(256) void quant_row_perchannel_kernel(Src src, int64_t M, int log2b,
                                                                   uint8_t* __restrict__ q, float* __restrict__ s,
                                                                   float post_scale) {
  constexpr int NC = E / 8;
  constexpr int64_t G = E / 2;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const int sub = lane & 15;
  for (int64_t row = wave; row < M; row += n_waves) {
    float v[E];
    load_row<E>(src, row, lane, v);
    fwht_row<E>(v, lane, log2b);
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(v[e]));
    m = max_x<1>(m);
    m = max_x<2>(m);
    m = max_x<4>(m);
    m = max_x<8>(m);
    m = max_x<16>(m);
    m = max_x<32>(m);
    uint32_t* qrow = reinterpret_cast<uint32_t*>(q + row * (G * 64));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint32_t b[8];
      encode<8>(&v[c * 8], m, b);
      qrow[c * 64 + lane] = pack8_bits(b, (lane & 2) != 0);
      if (sub == 0) s[row * G + c * 4 + (lane >> 4)] = m * post_scale;
    }
  }
}

// Codes of every row taken in channel order: out[r, j] = code(q[r], order[j]).
// A block walks rows four at a time: their stored words are decoded into
// LDS as one byte per code (the code's 6-bit sign-magnitude field), then
// every thread gathers whole output words (8 fields) of all four rows and
// folds them into the stored form.  The next four rows' words are loaded
// while the current ones are gathered.  A thread's output words and their
// source channels are the same in every row, so it reads the order once
// (K <= 8192: at most 4 words of a row per thread).
constexpr int kPermuteRows = 4;
constexpr int kPermuteWords = 4;  // words of a row per thread (K <= 8192)
__global__ __launch_bounds__(256) void permute_codes_kernel(const uint8_t* __restrict__ q, int64_t rows, int64_t K,
                                                            const int32_t* __restrict__ order,
                                                            uint8_t* __restrict__ out) {
  extern __shared__ uint8_t pc_fields[];  // kPermuteRows rows of K fields
  const int W = int(K / 8);
  // source channel of this thread's output codes (word i = threadIdx.x + 256 u)
  uint16_t src[kPermuteWords][8];
#pragma unroll
  for (int u = 0; u < kPermuteWords; ++u) {
    const int i = int(threadIdx.x) + 256 * u;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      src[u][e] = uint16_t(i < W ? min(uint32_t(order[i * 8 + e]), uint32_t(K - 1)) : 0u);  // clamped into the row
  }
  // words of rows row0 .. row0 + 3; rows past the end and words past the row read zeros
  uint32_t wv[kPermuteRows][kPermuteWords];
  auto load = [&](int64_t row0) {
#pragma unroll
    for (int r = 0; r < kPermuteRows; ++r) {
      const int64_t row = row0 + r;
      const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + row * (K / 2), row < rows ? K / 2 : 0);
#pragma unroll
      for (int u = 0; u < kPermuteWords; ++u) {
        const int i = int(threadIdx.x) + 256 * u;
        wv[r][u] = __builtin_amdgcn_raw_buffer_load_b32(rq, int(i < W ? uint32_t(i * 4) : kOutOfRange), 0, 0);
      }
    }
  };
  const int64_t stride = int64_t(gridDim.x) * kPermuteRows;
  load(int64_t(blockIdx.x) * kPermuteRows);
  for (int64_t row0 = int64_t(blockIdx.x) * kPermuteRows; row0 < rows; row0 += stride) {
    const int nr = int(rows - row0 < kPermuteRows ? rows - row0 : kPermuteRows);
    __syncthreads();  // the previous rows' fields consumed
#pragma unroll
    for (int r = 0; r < kPermuteRows; ++r) {
#pragma unroll
      for (int u = 0; u < kPermuteWords; ++u) {
        const int i = int(threadIdx.x) + 256 * u;
        if (r < nr && i < W) {  // uniform over each 16-lane row (W is a multiple of 16): the exchange below is safe
          uint32_t lo, hi;
          pair_fields<true>(wv[r][u], xchg_lanes<3>(wv[r][u]), (i & 2) != 0, lo, hi);
          uint32_t f[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = field6(lo, hi, e);
          const uint32_t d0 = f[0] | (f[1] << 8) | (f[2] << 16) | (f[3] << 24);
          const uint32_t d1 = f[4] | (f[5] << 8) | (f[6] << 16) | (f[7] << 24);
          *reinterpret_cast<uint2*>(pc_fields + r * K + i * 8) = make_uint2(d0, d1);
        }
      }
    }
    load(row0 + stride);  // the next rows' words, in flight while these are gathered
    __syncthreads();
    for (int r = 0; r < nr; ++r) {
      const uint8_t* fr = pc_fields + r * K;
      uint32_t* dst = reinterpret_cast<uint32_t*>(out + (row0 + r) * (K / 2));
#pragma unroll
      for (int u = 0; u < kPermuteWords; ++u) {
        const int i = int(threadIdx.x) + 256 * u;
        if (i >= W) break;  // uniform over each 16-lane row, as above (pack8_fields exchanges with lane ^ 3)
        uint32_t f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = fr[src[u][e]];
        dst[i] = pack8_fields(f, (i & 2) != 0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Rotation without quantization: x~ = x R (Hadamard, optionally signed) or
// x R D^-1 (Givens), written as fp32 or bf16 (round to nearest even).  The
// query side of an INT4 KV cache: keys are stored rotated and quantized, the
// queries are rotated alike so that (q R)(k R)^T = q k^T (the OstQuant page,
// section 3.2, rotates queries and keys together after RoPE; the Rotated
// Runtime Smooth experiments quantize the KV cache in groups of 128).
// The transforms are the quantizers' own (same butterflies, same tables);
// only the epilogue differs: the normalization 1/sqrt(b) (the quantizers
// fold it into the stored scale) is applied, then the values are stored.
// ---------------------------------------------------------------------------
template <bool OUT_BF16>
__device__ __forceinline__ void store8(void* out, int64_t off, const float v[8]) {
  if constexpr (OUT_BF16) {
    __bf16 h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = static_cast<__bf16>(v[e]);  // round to nearest even
    *reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(out) + off) = *reinterpret_cast<const uint4*>(h);
  } else {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Block-128 Hadamard: 16 lanes per (row, group), 8 consecutive channels per
// lane, as quant_h128; the lane stages in the negating form leave lane l's
// values times (-1)^popcount(l & 15), undone with the normalization.
template <class Src, bool OUT_BF16>
__global__ __launch_bounds__(256) void rotate_h128_kernel(Src src, int64_t G, int64_t blocks_per_row,
                                                          void* __restrict__ out, int64_t ldo, float norm) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & 15;
  const int64_t row = int64_t(blockIdx.x) / blocks_per_row;
  const int64_t grp = (int64_t(blockIdx.x) - row * blocks_per_row) * 16 + wave * 4 + (lane >> 4);
  if (grp >= G) return;  // whole 16-lane groups leave together: the stages stay inside a group
  float v[8];
  src.load8(row, grp * kGroup + sub * 8, v);
  fwht8(v);
  const float c1 = (lane & 1) ? -1.0f : 1.0f, c2 = (lane & 2) ? -1.0f : 1.0f;
  const float c4 = (lane & 4) ? -1.0f : 1.0f, c8 = (lane & 8) ? -1.0f : 1.0f;
  const float scale = ((__builtin_popcount(lane & 15) & 1) ? -1.0f : 1.0f) * norm;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x = v[e];
    x = butterfly_neg_x<1>(x, c1);
    x = butterfly_neg_x<2>(x, c2);
    x = butterfly_neg_x<4>(x, c4);
    x = butterfly_neg_x<8>(x, c8);
    v[e] = x * scale;
  }
  store8<OUT_BF16>(out, row * ldo + grp * kGroup + sub * 8, v);
}

// Hadamard blocks of 2^log2b channels over whole rows of K = 64 E channels:
// one wave per row, lane l holds channels 512 c + 8 l + e (quant_rowh).
template <int E, class Src, bool OUT_BF16>
__global__ __launch_bounds__(256) void rotate_rowh_kernel(Src src, int64_t M, int log2b, void* __restrict__ out,
                                                          int64_t ldo, float norm) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t n_waves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  for (int64_t row = wave; row < M; row += n_waves) {
    float v[E];
    load_row<E>(src, row, lane, v);
    fwht_row<E>(v, lane, log2b);
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[c * 8 + e] *= norm;
      store8<OUT_BF16>(out, row * ldo + c * 512 + lane * 8, &v[c * 8]);
    }
  }
}

// Givens layers from the lookup table (as quant_givens with one row per
// wave), then the channel scale alpha^-1.
template <class Src, bool OUT_BF16>
__global__ __launch_bounds__(64) void rotate_givens_kernel(Src src, int64_t G, int L,
                                                           const uint16_t* __restrict__ lut_idx,
                                                           const float2* __restrict__ lut_cs,
                                                           const float* __restrict__ chan_scale,
                                                           void* __restrict__ out, int64_t ldo) {
  __shared__ float buf[kGroup];
  const int lane = threadIdx.x;
  const int64_t grp = blockIdx.x % G;
  const int64_t row = blockIdx.x / G;
  const uint16_t* idx = lut_idx + grp * L * 64;
  const float2* cs = lut_cs + grp * L * 64;
  float v[2];
  src.load2(row, grp * kGroup + 2 * lane, v);
  buf[2 * lane] = v[0];
  buf[2 * lane + 1] = v[1];
  __syncthreads();
  for (int l = 0; l < L; ++l) {
    const uint32_t pr = idx[l * 64 + lane];
    const float2 t = cs[l * 64 + lane];
    const int i = pr & 0xFF, j = pr >> 8;
    const float a = buf[i], b = buf[j];
    buf[i] = fmaf(t.x, a, t.y * b);
    buf[j] = fmaf(t.x, b, -t.y * a);
    __syncthreads();
  }
  const float x0 = buf[2 * lane] * chan_scale[grp * kGroup + 2 * lane];
  const float x1 = buf[2 * lane + 1] * chan_scale[grp * kGroup + 2 * lane + 1];
  const int64_t off = row * ldo + grp * kGroup + 2 * lane;
  if constexpr (OUT_BF16) {
    const __bf16 h[2] = {static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
    *reinterpret_cast<uint32_t*>(reinterpret_cast<__bf16*>(out) + off) = *reinterpret_cast<const uint32_t*>(h);
  } else {
    *reinterpret_cast<float2*>(reinterpret_cast<float*>(out) + off) = make_float2(x0, x1);
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

// The asymmetric form of launch_h128_act (groups of 128): codes, scales
// (range / 15 of the normalized transform) and zero points.
hipError_t launch_h128_act_asym(const void* x, bool bf16, int64_t ldx, const uint32_t* sign_mask, int64_t rows,
                                int64_t G, uint8_t* q, float* s, float* z, hipStream_t st) {
  constexpr int D = 1, GS = 128;
  constexpr int64_t kResidentWaves = 256 * 32;
  const int64_t Q = (G + 3) / 4;
  const int64_t rows_per_wave = Q * rows <= kResidentWaves ? 1 : Q * rows <= 2 * kResidentWaves ? 2 : 3;
  int64_t R = (rows + rows_per_wave - 1) / rows_per_wave;
  if (R < 1) R = 1;
  const int64_t blocks = (Q * R + 3) / 4;
  if (Q * R > 0x7FFFFFFF - 3 || G * 64 * (bf16 ? 4 : 8) >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const float post = (1.0f / 15.0f) / sqrtf(128.0f);
#define RW4_H128_ASYM(B, S)                                                                                   \
  hipLaunchKernelGGL((quant_h128_act_kernel<B, S, D, GS, true>), dim3(blocks), dim3(256), 0, st, x, ldx, rows, G, \
                     Q, R, sign_mask, q, s, post, z)
  if (bf16) {
    if (sign_mask) RW4_H128_ASYM(true, true); else RW4_H128_ASYM(true, false);
  } else {
    if (sign_mask) RW4_H128_ASYM(false, true); else RW4_H128_ASYM(false, false);
  }
#undef RW4_H128_ASYM
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

namespace {

template <class Src>
hipError_t launch_rotate_src(const TransformDev& t, const Src& src, int64_t M, void* out, bool out_bf16,
                             int64_t ldo, hipStream_t st) {
  const int64_t K = t.K, G = K / kGroup;
  const float norm = 1.0f / sqrtf(float(t.block));
  if (t.block == 128) {
    const int64_t bpr = (G + 15) / 16, blocks = M * bpr;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (out_bf16)
      hipLaunchKernelGGL((rotate_h128_kernel<Src, true>), dim3(blocks), dim3(256), 0, st, src, G, bpr, out, ldo, norm);
    else
      hipLaunchKernelGGL((rotate_h128_kernel<Src, false>), dim3(blocks), dim3(256), 0, st, src, G, bpr, out, ldo, norm);
    return hipGetLastError();
  }
  int log2b = 0;
  while ((int64_t(1) << log2b) < t.block) ++log2b;
  const int grid = grid_for_waves(M, 256 * 16);
  auto run = [&](auto e_const) {
    constexpr int E = decltype(e_const)::value;
    if (out_bf16)
      hipLaunchKernelGGL((rotate_rowh_kernel<E, Src, true>), dim3(grid), dim3(256), 0, st, src, M, log2b, out, ldo, norm);
    else
      hipLaunchKernelGGL((rotate_rowh_kernel<E, Src, false>), dim3(grid), dim3(256), 0, st, src, M, log2b, out, ldo, norm);
    return hipGetLastError();
  };
  switch (K) {
    case 512: return run(std::integral_constant<int, 8>{});
    case 1024: return run(std::integral_constant<int, 16>{});
    case 2048: return run(std::integral_constant<int, 32>{});
    case 4096: return run(std::integral_constant<int, 64>{});
    case 8192: return run(std::integral_constant<int, 128>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t rrs_reorder_workspace_bytes(int64_t K) {
  return (int64_t(kChanmaxBlocks) + 1) * K * 4 + (K / kGroup) * 4;
}

namespace {

template <class Src>
hipError_t launch_rrs_reorder_src(const Src& src, int64_t K, int log2b, int64_t M, uint8_t* q, float* s,
                                  int32_t* order, float* ws, float post, hipStream_t st) {
  float* partial = ws;
  float* m = ws + int64_t(kChanmaxBlocks) * K;
  float* smooth = m + K;
  const int grid = grid_for_waves(M, 256 * 16);
  const int rank_lds = int(K * 8 + 256 * 4);
  auto run = [&](auto e_const) {
    constexpr int E = decltype(e_const)::value;
    hipLaunchKernelGGL((rrs_chanmax_kernel<E, Src>), dim3(kChanmaxBlocks), dim3(256), 0, st, src, M, log2b, partial);
    hipLaunchKernelGGL(chanmax_reduce_kernel, dim3(unsigned((K + 63) / 64)), dim3(1024), 0, st,
                       (const float*)partial, kChanmaxBlocks, K, m);
    hipLaunchKernelGGL(rrs_rank_kernel, dim3(unsigned(K / 16)), dim3(256), rank_lds, st, (const float*)m, K, order,
                       smooth);
    hipLaunchKernelGGL((quant_rrs_order_kernel<E, Src>), dim3(grid), dim3(256), 0, st, src, M, log2b,
                       (const int32_t*)order, (const float*)smooth, q, s, post);
    return hipGetLastError();
  };
  switch (K) {
    case 512: return run(std::integral_constant<int, 8>{});
    case 1024: return run(std::integral_constant<int, 16>{});
    case 2048: return run(std::integral_constant<int, 32>{});
    case 4096: return run(std::integral_constant<int, 64>{});
    default: return hipErrorInvalidValue;
  }
}

template <int NC>
hipError_t launch_rrs_reorder_full(const void* x, bool bf16, int64_t ldx, int64_t M, uint8_t* q, float* s,
                                   int32_t* order, float* ws, float post, hipStream_t st) {
  constexpr int64_t K = 512 * NC;
  float* partial = ws;
  float* m = ws + int64_t(kChanmaxBlocks) * K;
  float* smooth = m + K;
  const int grid = grid_for_waves(M, 256 * 16);
  const int rank_lds = int(K * 8 + 256 * 4);
  if (bf16)
    hipLaunchKernelGGL((rrs_chanmax_full_kernel<NC, true>), dim3(kChanmaxBlocks), dim3(256), 0, st, x, ldx, M, partial);
  else
    hipLaunchKernelGGL((rrs_chanmax_full_kernel<NC, false>), dim3(kChanmaxBlocks), dim3(256), 0, st, x, ldx, M, partial);
  hipLaunchKernelGGL(chanmax_reduce_kernel, dim3(unsigned((K + 63) / 64)), dim3(1024), 0, st, (const float*)partial,
                     kChanmaxBlocks, K, m);
  hipLaunchKernelGGL(rrs_rank_kernel, dim3(unsigned(K / 16)), dim3(256), rank_lds, st, (const float*)m, K, order,
                     smooth);
  if (bf16)
    hipLaunchKernelGGL((quant_rrs_order_full_kernel<NC, true>), dim3(grid), dim3(256), 0, st, x, ldx, M,
                       (const int32_t*)order, (const float*)smooth, q, s, post);
  else
    hipLaunchKernelGGL((quant_rrs_order_full_kernel<NC, false>), dim3(grid), dim3(256), 0, st, x, ldx, M,
                       (const int32_t*)order, (const float*)smooth, q, s, post);
  return hipGetLastError();
}

template <class Src>
hipError_t launch_perchannel_src(const Src& src, int64_t K, int log2b, int64_t N, uint8_t* q, float* s, float post,
                                 hipStream_t st) {
  const int grid = grid_for_waves(N, 256 * 16);
  auto run = [&](auto e_const) {
    constexpr int E = decltype(e_const)::value;
    hipLaunchKernelGGL((quant_row_perchannel_kernel<E, Src>), dim3(grid), dim3(256), 0, st, src, N, log2b, q, s, post);
    return hipGetLastError();
  };
  switch (K) {
    case 512: return run(std::integral_constant<int, 8>{});
    case 1024: return run(std::integral_constant<int, 16>{});
    case 2048: return run(std::integral_constant<int, 32>{});
    case 4096: return run(std::integral_constant<int, 64>{});
    case 8192: return run(std::integral_constant<int, 128>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool rrs_reorder_supported(int64_t K) { return K == 512 || K == 1024 || K == 2048 || K == 4096; }

hipError_t launch_quantize_act_rrs_reorder(const TransformDev& t, const void* x, bool bf16, int64_t M, int64_t ldx,
                                           uint8_t* q, float* s, int32_t* order, void* workspace, hipStream_t st) {
  int log2b = 0;
  while ((int64_t(1) << log2b) < t.block) ++log2b;
  const float post = 1.0f / sqrtf(float(t.block));  // the per-token scale a_t carries the 1/7
  float* ws = static_cast<float*>(workspace);
  if (t.sign_mask) {
    if (bf16)
      return launch_rrs_reorder_src(SignedSrc<RowSrc<true>>{{x, ldx}, t.sign_mask}, t.K, log2b, M, q, s, order, ws,
                                    post, st);
    return launch_rrs_reorder_src(SignedSrc<RowSrc<false>>{{x, ldx}, t.sign_mask}, t.K, log2b, M, q, s, order, ws,
                                  post, st);
  }
  if (t.block == t.K && (t.K == 2048 || t.K == 4096)) {
    // whole-row transform: the register / DPP kernels of the RRS path
    if (t.K == 2048) return launch_rrs_reorder_full<4>(x, bf16, ldx, M, q, s, order, ws, post, st);
    return launch_rrs_reorder_full<8>(x, bf16, ldx, M, q, s, order, ws, post, st);
  }
  if (bf16) return launch_rrs_reorder_src(RowSrc<true>{x, ldx}, t.K, log2b, M, q, s, order, ws, post, st);
  return launch_rrs_reorder_src(RowSrc<false>{x, ldx}, t.K, log2b, M, q, s, order, ws, post, st);
}

hipError_t launch_pack_weight_per_channel(const TransformDev& t, const void* w, bool bf16, int64_t N, int64_t sk,
                                          int64_t sn, uint8_t* q, float* s, hipStream_t st) {
  int log2b = 0;
  while ((int64_t(1) << log2b) < t.block) ++log2b;
  const float post = (1.0f / 7.0f) / sqrtf(float(t.block));
  if (t.sign_mask) {
    if (bf16)
      return launch_perchannel_src(SignedSrc<StridedSrc<true>>{{w, sk, sn}, t.sign_mask}, t.K, log2b, N, q, s, post, st);
    return launch_perchannel_src(SignedSrc<StridedSrc<false>>{{w, sk, sn}, t.sign_mask}, t.K, log2b, N, q, s, post, st);
  }
  if (bf16) return launch_perchannel_src(StridedSrc<true>{w, sk, sn}, t.K, log2b, N, q, s, post, st);
  return launch_perchannel_src(StridedSrc<false>{w, sk, sn}, t.K, log2b, N, q, s, post, st);
}

hipError_t launch_permute_codes(const uint8_t* q, int64_t rows, int64_t K, const int32_t* order, uint8_t* out,
                                hipStream_t st) {
  const int64_t batches = (rows + kPermuteRows - 1) / kPermuteRows;
  const int64_t grid = batches < 1024 ? batches : 1024;
  const int lds = int(kPermuteRows * K);
  hipLaunchKernelGGL(permute_codes_kernel, dim3(unsigned(grid)), dim3(256), lds, st, q, rows, K, order, out);
  return hipGetLastError();
}

// Rotation without quantization of row-major activations X [M, K].
hipError_t launch_rotate_act(const TransformDev& t, const void* x, bool bf16, int64_t M, int64_t ldx, void* out,
                             bool out_bf16, int64_t ldo, hipStream_t st) {
  const int64_t K = t.K, G = K / kGroup;
  if (t.kind == TransformKind::Hadamard) {
    if (t.sign_mask) {
      if (bf16) return launch_rotate_src(t, SignedSrc<RowSrc<true>>{{x, ldx}, t.sign_mask}, M, out, out_bf16, ldo, st);
      return launch_rotate_src(t, SignedSrc<RowSrc<false>>{{x, ldx}, t.sign_mask}, M, out, out_bf16, ldo, st);
    }
    if (bf16) return launch_rotate_src(t, RowSrc<true>{x, ldx}, M, out, out_bf16, ldo, st);
    return launch_rotate_src(t, RowSrc<false>{x, ldx}, M, out, out_bf16, ldo, st);
  }
  const int64_t blocks = G * M;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
#define RW4_ROT_GIVENS(B, O)                                                                               \
  hipLaunchKernelGGL((rotate_givens_kernel<RowSrc<B>, O>), dim3(blocks), dim3(64), 0, st, RowSrc<B>{x, ldx}, G, \
                     t.layers, t.lut_idx, t.lut_cs, t.alpha_inv, out, ldo)
  if (bf16) {
    if (out_bf16) RW4_ROT_GIVENS(true, true); else RW4_ROT_GIVENS(true, false);
  } else {
    if (out_bf16) RW4_ROT_GIVENS(false, true); else RW4_ROT_GIVENS(false, false);
  }
#undef RW4_ROT_GIVENS
  return hipGetLastError();
}

bool rowh_supported(int64_t K) {
  return K == 512 || K == 1024 || K == 2048 || K == 4096 || K == 8192;
}

// Activations: X [M, K] row-major.
// group: 64, 128 or 256 for the block-128 Hadamard in per-group mode, else
// 128 (the caller checks).
// ---------------------------------------------------------------------------
// Mixed precision: block-128 Hadamard activations in groups of 128, with the
// groups named by slot_of_group (>= 0) kept at 8 bits (the independent-
// rotation article, section 4.1: mixed precision for extreme outliers).  An
// 8-bit group gets q8 = rne(112 x~ / max) (225 levels) split exactly as
// q8 = 15 h + l (h = rne(q8 / 15), never a tie): h is stored in place with
// scale 15 max / 112, l in the extra group G + slot with scale max / 112.
// Every other group is the plain INT4 group.  quant_h128_act_kernel's
// persistent layout in its MIXED form: a wave keeps one quad of groups, so
// only waves whose quad holds a listed group take the two-plane encoder
// (decided once per wave); rows hold G + n8 groups.
// ---------------------------------------------------------------------------
hipError_t launch_quantize_act_mixed(const TransformDev& t, const void* x, bool bf16, int64_t M, int64_t ldx,
                                     const int32_t* slot_of_group, int64_t n8, uint8_t* q, float* s, hipStream_t st) {
  if (t.kind != TransformKind::Hadamard || t.block != kGroup) return hipErrorInvalidValue;
  const int64_t G = t.K / kGroup;
  constexpr int D = 1, GS = 128;
  constexpr int64_t kResidentWaves = 256 * 32;
  const int64_t Q = (G + 3) / 4;
  const int64_t rows_per_wave = Q * M <= kResidentWaves ? 1 : Q * M <= 2 * kResidentWaves ? 2 : 3;
  int64_t R = (M + rows_per_wave - 1) / rows_per_wave;
  if (R < 1) R = 1;
  const int64_t blocks = (Q * R + 3) / 4;
  if (Q * R > 0x7FFFFFFF - 3 || (G + n8) * 64 * (bf16 ? 4 : 8) >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const float norm = 1.0f / sqrtf(128.0f);
  const float post4 = norm * (1.0f / 7.0f), post8h = norm * (15.0f / 112.0f), post8l = norm * (1.0f / 112.0f);
#define RW4_MIXED(B, S)                                                                                              \
  hipLaunchKernelGGL((quant_h128_act_kernel<B, S, D, GS, false, true>), dim3(blocks), dim3(256), 0, st, x, ldx, M, G, \
                     Q, R, t.sign_mask, q, s, post4, nullptr, slot_of_group, n8, post8h, post8l)
  if (bf16) {
    if (t.sign_mask) RW4_MIXED(true, true); else RW4_MIXED(true, false);
  } else {
    if (t.sign_mask) RW4_MIXED(false, true); else RW4_MIXED(false, false);
  }
#undef RW4_MIXED
  return hipGetLastError();
}

hipError_t launch_quantize_act_asym(const TransformDev& t, const void* x, bool bf16, int64_t M, int64_t ldx,
                                    uint8_t* q, float* s, float* z, hipStream_t st) {
  if (t.kind != TransformKind::Hadamard || t.block != kGroup) return hipErrorInvalidValue;
  return launch_h128_act_asym(x, bf16, ldx, t.sign_mask, M, t.K / kGroup, q, s, z, st);
}

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
