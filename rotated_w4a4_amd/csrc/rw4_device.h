// Device-side building blocks of the rotated W4A4 kernels (gfx950, wave64).
//
// Element sources, cross-lane exchanges for the Walsh-Hadamard butterflies,
// the round-to-nearest-even INT4 encoder and the packer of the stored form.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rw4 {

constexpr int kGroup = 128;
constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element sources.  A "row" is the K-vector that gets transformed and
// quantized: a token of X, or an output channel of W.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Row-major rows with a leading dimension; 8 consecutive elements per call
// through one (bf16) or two (fp32) 16-byte loads.  Requires 16-byte aligned
// rows (checked on the host).
template <bool BF16>
struct RowSrc {
  const void* p;
  int64_t ld;  // elements
  __device__ __forceinline__ void load8(int64_t row, int64_t k0, float v[8]) const {
    if constexpr (BF16) {
      const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + row * ld + k0);
      v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
      v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
      v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
      v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
    } else {
      const float4* q = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + row * ld + k0);
      const float4 a = q[0], b = q[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  }
  __device__ __forceinline__ void load2(int64_t row, int64_t k0, float v[2]) const {
    if constexpr (BF16) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(p) + row * ld + k0);
      v[0] = bf16_lo(u); v[1] = bf16_hi(u);
    } else {
      const float2 a = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(p) + row * ld + k0);
      v[0] = a.x; v[1] = a.y;
    }
  }
};

// Strided gather: element (row, k) at p[k * sk + row * sr].  Used for the
// offline weight pack, where W arrives as [K, N] or [N, K].
template <bool BF16>
struct StridedSrc {
  const void* p;
  int64_t sk, sr;
  __device__ __forceinline__ float at(int64_t row, int64_t k) const {
    const int64_t off = k * sk + row * sr;
    if constexpr (BF16) {
      return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(p)[off]) << 16);
    } else {
      return reinterpret_cast<const float*>(p)[off];
    }
  }
  __device__ __forceinline__ void load8(int64_t row, int64_t k0, float v[8]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = at(row, k0 + e);
  }
  __device__ __forceinline__ void load2(int64_t row, int64_t k0, float v[2]) const {
    v[0] = at(row, k0);
    v[1] = at(row, k0 + 1);
  }
};

// Randomized Hadamard: the inner source with the sign of channel k flipped
// where mask[k] = 0x80000000 (the +-1 diagonal applied before the block
// transform, to activations and to weight rows alike).  k0 is a multiple
// of 8 for load8 and of 2 for load2.
template <class Inner>
struct SignedSrc {
  Inner in;
  const uint32_t* mask;
  __device__ __forceinline__ void load8(int64_t row, int64_t k0, float v[8]) const {
    in.load8(row, k0, v);
    const uint4 a = *reinterpret_cast<const uint4*>(mask + k0);
    const uint4 b = *reinterpret_cast<const uint4*>(mask + k0 + 4);
    const uint32_t m[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ m[e]);
  }
  __device__ __forceinline__ void load2(int64_t row, int64_t k0, float v[2]) const {
    in.load2(row, k0, v);
    const uint2 a = *reinterpret_cast<const uint2*>(mask + k0);
    v[0] = __uint_as_float(__float_as_uint(v[0]) ^ a.x);
    v[1] = __uint_as_float(__float_as_uint(v[1]) ^ a.y);
  }
};

// ---------------------------------------------------------------------------
// Cross-lane exchange: value of lane (lane ^ M); every DPP source lane
// exists (bound_ctrl set only lets the compiler fuse the move into the
// consumer).  DPP quad permutes for
// M = 1, 2; DPP row rotate by 8 for M = 8 (inside a 16-lane row, lane i and
// i ^ 8 are 8 apart either way); ds_swizzle (bit-mask mode, within 32
// lanes) for 4 and 16; ds_bpermute for 32.
// ---------------------------------------------------------------------------
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  int x = __float_as_int(v);
  if constexpr (M == 1) {
    x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 8) {
    x = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true);  // row_ror:8 (lane ^ 8 in a row of 16)
  } else if constexpr (M < 32) {
    x = __builtin_amdgcn_ds_swizzle(x, (M << 10) | 0x1F);
  } else {
    const int lane = __lane_id();
    x = __builtin_amdgcn_ds_bpermute((lane ^ M) << 2, x);
  }
  return __int_as_float(x);
}

// One radix-2 butterfly stage of the Walsh-Hadamard transform across lanes
// that differ in lane bit M: the lane with the bit clear keeps a + b, the
// lane with the bit set keeps a - b (a = low partner, b = high partner).
template <int M>
__device__ __forceinline__ float butterfly_x(float v, int lane) {
  const float o = lane_xor<M>(v);
  const float sgn = (lane & M) ? -1.0f : 1.0f;
  return fmaf(sgn, v, o);
}

// The same stage in a cheaper form: x + c * partner with c = +1 on the low
// lane and -1 on the high lane, one fused multiply-add whose multiplicand
// comes straight from the cross-lane move.  The high lane gets the negated
// butterfly output; after stages on a set of lane bits, every value is off
// by (-1)^(number of those bits set in the lane index), which the caller
// folds into the quantizer (the absolute maximum does not change).
template <int M>
__device__ __forceinline__ float butterfly_neg_x(float v, float c) {
  return fmaf(lane_xor<M>(v), c, v);
}

// Butterfly stages on the low 3 index bits held in one lane's 8 registers.
__device__ __forceinline__ void fwht8(float v[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((e & h) == 0) {
        const float a = v[e], b = v[e | h];
        v[e] = a + b;
        v[e | h] = a - b;
      }
    }
  }
}

template <int M>
__device__ __forceinline__ float max_x(float m) {
  return fmaxf(m, lane_xor<M>(m));
}

// ---------------------------------------------------------------------------
// INT4 encoding.  fmaf(v, inv, 1.5 * 2^23) rounds v * inv to the nearest
// integer with ties to even (the float spacing is exactly 1 there and the
// constant's mantissa is even), so the low bits of the result hold the
// two's-complement code.  |v * inv| <= 7 (1 + 2^-23) by construction, so the
// code lies in [-7, 7] and no clamp is needed.
// ---------------------------------------------------------------------------
constexpr float kRoundMagic = 12582912.0f;      // 1.5 * 2^23
constexpr uint32_t kRoundMagicBits = 0x4B400000u;

__device__ __forceinline__ uint32_t rne_code_bits(float v, float inv) {
  return __float_as_uint(fmaf(v, inv, kRoundMagic));
}

// Two's-complement nibbles from 8 magic-rounded float bit patterns (code e
// at nibble e): Horner sum of the raw patterns, then subtract the magic
// constant from every nibble while adding 8 (offset binary, no borrows),
// then flip the nibble sign bits.
__device__ __forceinline__ uint32_t pack8_twos(const uint32_t b[8]) {
  uint32_t acc = b[7];
#pragma unroll
  for (int e = 6; e >= 0; --e) acc = (acc << 4) + b[e];
  constexpr uint32_t kOnes = 0x11111111u;
  constexpr uint32_t kFix = (8u - kRoundMagicBits) * kOnes;  // mod 2^32
  return (acc + kFix) ^ 0x88888888u;
}

// Stored form of 8 codes (one 32-bit word): sign-magnitude nibbles, nibble e
// = |c_e| in bits 0-2 and the sign of c_{(e-1) mod 8} in bit 3.  From the
// two's-complement nibbles t: s = the nibble sign bits; |c| per nibble is
// (t XOR 0xF) + 1 where negative, done for all nibbles at once (|c| <= 7, so
// nothing carries); the signs then move up one nibble, the top one wrapping
// to nibble 0.  Zero is stored with sign 0.
__device__ __forceinline__ uint32_t twos_to_stored(uint32_t t) {
  const uint32_t s = t & 0x88888888u;
  const uint32_t one = s >> 3;
  const uint32_t mag = (t ^ ((one << 4) - one)) + one;
  return mag | __builtin_amdgcn_alignbit(s, s, 28);  // rotate left by 4
}

__device__ __forceinline__ uint32_t pack8_bits(const uint32_t b[8]) { return twos_to_stored(pack8_twos(b)); }

// One byte of the stored form for codes 2l, 2l+1 of a word, held by lane l of
// a quad (lanes 4w..4w+3 hold word w): the low nibble takes the sign of code
// 2l-1, i.e. of the high code of the previous lane of the quad (cyclically).
__device__ __forceinline__ uint32_t pack2_bits_quad(uint32_t b0, uint32_t b1) {
  constexpr uint32_t kFix2 = (8u - kRoundMagicBits) * 0x11u;
  const uint32_t t = ((((b1 << 4) + b0) + kFix2) ^ 0x88u) & 0xFFu;  // two's complement byte
  const uint32_t s = t & 0x88u;
  const uint32_t one = s >> 3;
  const uint32_t mag = (t ^ ((one << 4) - one)) + one;
  // lane i of each quad reads lane (i + 3) % 4: quad_perm [3, 0, 1, 2]
  const uint32_t prev = uint32_t(__builtin_amdgcn_mov_dpp(int(s), 0x93, 0xF, 0xF, false));
  return (mag | ((s & 0x08u) << 4) | ((prev >> 4) & 0x08u)) & 0xFFu;
}

__device__ __forceinline__ float safe_inv(float m, float num) { return m > 0.0f ? num / m : 0.0f; }

// Encoder for a group (or row) whose absolute maximum is m >= 0.  When m is
// so small that 7 / m would overflow, the values are first scaled by 2^64
// (exact) so the reciprocal stays finite.  Codes are identical either way.
constexpr float kTinyMax = 0x1p-100f;
constexpr float kTinyLift = 0x1p64f;

// sign = -1 encodes the negated values (for inputs that carry a known sign
// flip); rounding to nearest even is symmetric, so the codes are exactly
// the negated codes.
template <int N>
__device__ __forceinline__ void encode(float v[N], float m, uint32_t b[N], float sign = 1.0f) {
  if (m > 0.0f && m < kTinyMax) {
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] *= kTinyLift;
    m *= kTinyLift;
  }
  const float inv = safe_inv(m, 7.0f) * sign;
#pragma unroll
  for (int e = 0; e < N; ++e) b[e] = rne_code_bits(v[e], inv);
}

// ---------------------------------------------------------------------------
// Lane stages of the block-128 activation quantizers (16 lanes x 8 values
// per group).  The four lane stages run along lane masks 1, 2, 7 and 8,
// each one DPP move (quad_perm, row_half_mirror, row_ror:8) fused into a
// v_fmac_f32: x += c_k * x[lane ^ m_k] with c_k = (-1)^parity(lane & t_k)
// for the dual functionals t = (5, 6, 4, 8) (parity(m_j & t_k) = [j == k]).
// The product of these stages is the Walsh-Hadamard transform of the
// 16-lane index up to a signed permutation: lane l ends with
// (-1)^popcount(l) times the outputs of Sylvester lane f(l), where f is
// GF(2)-linear with f(1) = 5, f(2) = 6, f(4) = 7, f(8) = 8.  The sign is
// undone in the encoder (the absolute maximum is unchanged) and the packed
// word is stored at word f(l) of the group.
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

// Packed word of 8 values whose group maximum is m, for the activation
// quantizers of the lane-stage layout.  Groups whose maximum is below
// 2^-100 are lifted by 2^64 (exact) so that 7 / m stays finite; rare, so
// the whole wave branches around it.  7 / m is the hardware reciprocal of
// m / 7: a few ulp from the rounded quotient, which moves v * 7 / m by
// ~1e-6 of a code step at most.  (The reciprocal flushes subnormal
// results, so it is taken of m / 7, whose reciprocal is normal for every
// finite m >= 2^-100; 1 / m is not, for m above 2^126.)
__device__ __forceinline__ uint32_t encode8_rcp(float (&v)[8], float m, float flip) {
  float mm = m;
  if (__builtin_amdgcn_ballot_w64(m > 0.0f && m < kTinyMax) != 0) {
    if (m > 0.0f && m < kTinyMax) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= kTinyLift;
      mm = m * kTinyLift;
    }
  }
  const float inv = mm > 0.0f ? flip * __builtin_amdgcn_rcpf(mm * (1.0f / 7.0f)) : 0.0f;
  uint32_t b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = rne_code_bits(v[e], inv);
  return pack8_bits(b);
}

// ---------------------------------------------------------------------------
// Asymmetric (s, z) encoder: 8 values t (true signs) of a group whose range,
// with zero kept inside it, is [-nlo, hi] (hi, nlo >= 0, reduced over the
// group).  With d = hi + nlo: z = rne(15 nlo / d) and code
// clamp(rne(15 t / d) + z, 0, 15), packed as plain nibbles (code e in
// nibble e).  15 / d is the hardware reciprocal of d / 15; groups with
// 0 < d < 2^-100 are lifted by 2^64 (exact) as in encode8_rcp; d = 0 gives
// z = 0 and codes 0.  Returns the word; z in z_out.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t encode8_asym(float (&t)[8], float hi, float nlo, uint32_t& z_out) {
  float d = hi + nlo, nl = nlo;
  if (__builtin_amdgcn_ballot_w64(d > 0.0f && d < kTinyMax) != 0) {
    if (d > 0.0f && d < kTinyMax) {
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] *= kTinyLift;
      d *= kTinyLift;
      nl *= kTinyLift;
    }
  }
  const float inv = d > 0.0f ? __builtin_amdgcn_rcpf(d * (1.0f / 15.0f)) : 0.0f;
  const uint32_t z = rne_code_bits(nl, inv) - kRoundMagicBits;
  uint32_t acc = 0;
#pragma unroll
  for (int e = 7; e >= 0; --e) {
    // rne(t inv) + z, clamped to [0, 15], in the magic-constant domain
    uint32_t b = rne_code_bits(t[e], inv) + z;
    b = b < kRoundMagicBits ? kRoundMagicBits : b;
    b = b > kRoundMagicBits + 15u ? kRoundMagicBits + 15u : b;
    acc = (acc << 4) + (b - kRoundMagicBits);
  }
  z_out = z;
  return acc;
}

}  // namespace rw4
