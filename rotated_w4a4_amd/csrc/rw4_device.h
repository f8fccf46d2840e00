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

// ---------------------------------------------------------------------------
// Stored form of the codes: 4 bits per code, 8 codes per 32-bit word (code
// e of word w = channel 8 w + e of the row), and the words of each 16-byte
// chunk paired as (4 j, 4 j + 3) and (4 j + 1, 4 j + 2): the first word of
// a pair (bit 1 of its index clear, "role 0") and its partner w ^ 3 ("role
// 1") share one bit pattern.  Its purpose: the GEMM reads codes as FP6
// E2M3 values (the gfx950 FP6 matrix cores run about 1.5x the FP8 rate),
// whose encodings are 6 bits wide.  Let f_k be the 6-bit E2M3 encoding of
// code k of a pair (k = 0..7 the role-0 word's codes, 8..15 its partner's):
// signed codes c as the subnormal c / 8 (sign bit 5, exponent bits 3-4
// zero, mantissa |c| in bits 0-2), unsigned codes u (0..15) as u / 8, whose
// encoding is u itself.  The pair's words a (role 0) and b (role 1) are the
// dense 96-bit string X = sum_k f_k << 6 k folded into 64 bits: with masks
// A and C (per code kind, below),
//   X[0:32] = a & A,   X[64:96] = b & C,   X[32:64] = (a & ~A) | (b & ~C).
// A marks the bits of X[0:32] that can be nonzero, C those of X[64:96];
// the bits of X[32:64] that can be nonzero are exactly ~A | ~C, and ~A, ~C
// are disjoint (signed: field offsets {3, 4} and {0, 5} of X[32:64]), so
// the GEMM opens a pair with four instructions and no rotation.  A packing
// lane holds one word's 8 codes and takes the 16 bits of X[32:64] it does
// not own from its partner's lane.
// ---------------------------------------------------------------------------
// Bitfield insert (mask ? a : b, bit by bit) and a funnel shift by a lane's
// own amount, written out: for masks and shifts that differ between lanes
// the compiler otherwise emits two instructions for each.
__device__ __forceinline__ uint32_t bfi32(uint32_t mask, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t alignbit_v(uint32_t hi, uint32_t lo, uint32_t shift) {
  uint32_t r;
  asm("v_alignbit_b32 %0, %1, %2, %3" : "=v"(r) : "v"(hi), "v"(lo), "v"(shift));
  return r;
}
// c with a lane's sign flip (+-1) applied, as a value the compiler cannot
// see through: 7 / m times the flip is then one reciprocal of m * (+-1/7)
// (rcp(-x) = -rcp(x) exactly), where the compiler otherwise computes the
// reciprocal for both signs and selects.  Never feed a transcendental
// result into inline asm: gfx950 needs a wait state between a
// transcendental instruction and a VALU reading its result, which the
// compiler does not insert for asm operands.
__device__ __forceinline__ float signed_const(float c, float flip) {
  uint32_t r;
  asm("v_xor_b32 %0, %1, %2" : "=v"(r) : "v"(__float_as_uint(c)), "v"(__float_as_uint(flip) & 0x80000000u));
  return __uint_as_float(r);
}

constexpr uint32_t kSgnA = 0xE79E79E7u, kSgnC = 0x9E79E79Eu;
constexpr uint32_t kUnsA = 0xCF3CF3CFu, kUnsC = 0x3CF3CF3Cu;

// The value of lane l ^ XOR of the 16-lane DPP row: XOR = 3 (quad_perm
// [3,2,1,0]) for packers whose lane l holds word w and lane l ^ 3 word
// w ^ 3; XOR = 12 (row_mirror, lane 15 - l, then the quad permutation) for
// packers that spread a word over a quad of lanes.  Every lane of the row
// must execute it.
template <int XOR>
__device__ __forceinline__ uint32_t xchg_lanes(uint32_t v) {
  static_assert(XOR == 3 || XOR == 12, "partner lane patterns");
  if constexpr (XOR == 3) {
    return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x1B, 0xF, 0xF, false));
  } else {
    const int t = __builtin_amdgcn_mov_dpp(int(v), 0x140, 0xF, 0xF, false);
    return uint32_t(__builtin_amdgcn_mov_dpp(t, 0x1B, 0xF, 0xF, false));
  }
}

// Stored word from the 48-bit field string of its 8 codes (lo: bits 0-31,
// hi: bits 32-47), role as above.  Role 0 holds X[0:48] (lo = X[0:32]) and
// needs X[48:64], the low 16 bits of its partner's lo; role 1 holds X[48:96]
// and needs X[32:48], its partner's hi.  Each lane offers both halves in
// one word (its lo's low 16 bits, its hi) and reads its partner's.
template <bool SIGNED, int XOR = 3>
__device__ __forceinline__ uint32_t pair_word(uint32_t lo, uint32_t hi, bool role) {
  constexpr uint32_t kA = SIGNED ? kSgnA : kUnsA, kC = SIGNED ? kSgnC : kUnsC;
  // v_perm_b32(P, Q, sel): selector bytes 0-3 pick bytes of Q, 4-7 of P
  const uint32_t mine = __builtin_amdgcn_perm(hi, lo, 0x05040100u);  // lo[0:16] | hi[0:16] << 16
  const uint32_t theirs = xchg_lanes<XOR>(mine);
  // X[32:64]: role 0 = hi[0:16] | partner lo[0:16] << 16, role 1 = partner hi | lo[0:16] << 16
  const uint32_t mid = __builtin_amdgcn_perm(theirs, mine, role ? 0x01000706u : 0x05040302u);
  const uint32_t own = alignbit_v(hi, lo, role ? 16u : 0u);  // X[0:32] or X[64:96]
  return bfi32(role ? kC : kA, own, mid);
}

// The 48-bit field string of a stored word's 8 codes (the inverse of
// pair_word) from the word w and its partner p.
template <bool SIGNED>
__device__ __forceinline__ void pair_fields(uint32_t w, uint32_t p, bool role, uint32_t& lo, uint32_t& hi) {
  constexpr uint32_t kA = SIGNED ? kSgnA : kUnsA, kC = SIGNED ? kSgnC : kUnsC;
  const uint32_t a = role ? p : w, b = role ? w : p;
  const uint32_t mid = (a & ~kA) | (b & ~kC);  // X[32:64]
  if (role) {
    const uint32_t x2 = b & kC;  // X[64:96]
    lo = __builtin_amdgcn_alignbit(x2, mid, 16);
    hi = x2 >> 16;
  } else {
    lo = a & kA;
    hi = mid & 0xFFFFu;
  }
}
// field k (0-7) of a 48-bit field string
__device__ __forceinline__ uint32_t field6(uint32_t lo, uint32_t hi, int k) {
  return k < 5 ? (lo >> (6 * k)) & 63u : k == 5 ? (lo >> 30) | ((hi & 15u) << 2) : (hi >> (6 * k - 32)) & 63u;
}

// Sign-magnitude 6-bit fields from 6-bit two's-complement codes offset by
// 32 (t: codes c + 32 in [25, 39], no field borrows from the next): with
// p = t ^ 32 (two's complement), a negative field is 0b111xxx with xxx =
// 8 - |c|; clearing bits 3-4 and replacing xxx by its negation mod 8 gives
// 0b100 |c|, the E2M3 encoding of c / 8.  ones: bit 0 of every field.
__device__ __forceinline__ uint32_t fp6_sign_magnitude(uint32_t t, uint32_t ones) {
  const uint32_t p = t ^ (ones << 5);
  const uint32_t n7 = (p >> 3) & (ones * 7u);        // 7 in negative fields
  const uint32_t q = p & ~(ones * 24u);               // bits 3-4 cleared
  return (q ^ n7) + (n7 & ones);                      // xxx -> (~xxx & 7) + 1 = |c|
}

// Fields of 6-bit stride from 8 magic-rounded float patterns (code e in the
// low bits of b[e]): Horner sums of the raw patterns over fields 0-5 (lo,
// field 5 cut at bit 32) and 5-7 (hi), then the magic constant removed
// from every field with 32 added (offset binary, no borrows).
constexpr uint32_t f6_rep(uint32_t v, int n) {
  uint32_t r = 0;
  for (int k = 0; k < n; ++k) r += v << (6 * k);
  return r;
}
__device__ __forceinline__ void horner6(const uint32_t b[8], uint32_t& lo, uint32_t& hi) {
  lo = b[5];
#pragma unroll
  for (int e = 4; e >= 0; --e) lo = (lo << 6) + b[e];
  hi = (((b[7] << 6) + b[6]) << 6) + b[5];
}

// Stored word of 8 signed codes from their magic-rounded patterns; role:
// bit 1 of the word's index in the row (the partner word w ^ 3 is packed by
// lane l ^ XOR at the same time).
template <int XOR = 3>
__device__ __forceinline__ uint32_t pack8_bits(const uint32_t b[8], bool role) {
  uint32_t lo, hi;
  horner6(b, lo, hi);
  constexpr uint32_t kOff = 32u - kRoundMagicBits;  // mod 2^32
  const uint32_t slo = fp6_sign_magnitude(lo + f6_rep(kOff, 6), f6_rep(1u, 5));
  const uint32_t shi = fp6_sign_magnitude(hi + f6_rep(kOff, 3), f6_rep(1u, 3));
  return pair_word<true, XOR>((slo & 0x3FFFFFFFu) | (shi << 30), shi >> 2, role);
}
// Stored word of 8 signed codes given as their 6-bit sign-magnitude fields
// (bits 0-2 |c|, bit 5 the sign, as field6 returns them).
__device__ __forceinline__ uint32_t pack8_fields(const uint32_t f[8], bool role) {
  uint32_t lo, hi;
  horner6(f, lo, hi);
  return pair_word<true>(lo, hi >> 2, role);
}
// Stored word of 8 unsigned codes (0..15) from their magic-rounded patterns.
__device__ __forceinline__ uint32_t pack8_ubits(const uint32_t b[8], bool role) {
  uint32_t lo, hi;
  horner6(b, lo, hi);
  constexpr uint32_t kOff = 0u - kRoundMagicBits;
  return pair_word<false>(lo + f6_rep(kOff, 6), (hi + f6_rep(kOff, 3)) >> 2, role);
}

// One byte of the stored form for codes 2l, 2l+1 of a word, held by lane l of
// a quad (lanes 4w..4w+3 hold word w of a 16-word group, role: bit 1 of w):
// the quad's 8 patterns are gathered into every lane (quad broadcasts),
// each lane packs the whole word (its partner w ^ 3 lies in the quad of
// lanes l ^ 12) and keeps byte l.
__device__ __forceinline__ uint32_t pack2_bits_quad(uint32_t b0, uint32_t b1, int l, bool role) {
  uint32_t b[8];
  b[0] = uint32_t(__builtin_amdgcn_mov_dpp(int(b0), 0x00, 0xF, 0xF, false));
  b[1] = uint32_t(__builtin_amdgcn_mov_dpp(int(b1), 0x00, 0xF, 0xF, false));
  b[2] = uint32_t(__builtin_amdgcn_mov_dpp(int(b0), 0x55, 0xF, 0xF, false));
  b[3] = uint32_t(__builtin_amdgcn_mov_dpp(int(b1), 0x55, 0xF, 0xF, false));
  b[4] = uint32_t(__builtin_amdgcn_mov_dpp(int(b0), 0xAA, 0xF, 0xF, false));
  b[5] = uint32_t(__builtin_amdgcn_mov_dpp(int(b1), 0xAA, 0xF, 0xF, false));
  b[6] = uint32_t(__builtin_amdgcn_mov_dpp(int(b0), 0xFF, 0xF, 0xF, false));
  b[7] = uint32_t(__builtin_amdgcn_mov_dpp(int(b1), 0xFF, 0xF, 0xF, false));
  return (pack8_bits<12>(b, role) >> (8 * l)) & 0xFFu;
}

__device__ __forceinline__ float safe_inv(float m, float num) { return m > 0.0f ? num / m : 0.0f; }

// Encoder for a group (or row) whose absolute maximum is m >= 0.  When m is
// so small that 7 / m would overflow, the values are first scaled by 2^64
// (exact) so the reciprocal stays finite.  Codes are identical either way.
constexpr float kTinyMax = 0x1p-100f;
constexpr float kTinyLift = 0x1p64f;
// 0 < m < kTinyMax for m >= +0 (or NaN, which is not tiny), as one unsigned
// comparison of the bit patterns: +0 wraps to the largest value
__device__ __forceinline__ bool tiny_positive(float m) {
  return __float_as_uint(m) - 1u < __float_as_uint(kTinyMax) - 1u;
}

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
// finite m >= 2^-100; 1 / m is not, for m above 2^126.)  s7 is the lane's
// signed 1/7, signed_const(1.0f / 7.0f, flip), made once by the caller.
__device__ __forceinline__ uint32_t encode8_rcp(float (&v)[8], float m, float s7, bool role) {
  float mm = m;
  if (__builtin_amdgcn_ballot_w64(tiny_positive(m)) != 0) {
    if (tiny_positive(m)) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= kTinyLift;
      mm = m * kTinyLift;
    }
  }
  // m = 0: the reciprocal is infinite and the select gives 0
  const float r = __builtin_amdgcn_rcpf(mm * s7);
  const float inv = mm > 0.0f ? r : 0.0f;
  uint32_t b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = rne_code_bits(v[e], inv);
  return pack8_bits(b, role);
}

// ---------------------------------------------------------------------------
// Asymmetric (s, z) encoder: 8 values t (true signs) of a group whose range,
// with zero kept inside it, is [-nlo, hi] (hi, nlo >= 0, reduced over the
// group).  With d = hi + nlo: z = rne(15 nlo / d) and code
// clamp(rne(15 t / d) + z, 0, 15), in the unsigned stored form.  15 / d is the hardware reciprocal of d / 15; groups with
// 0 < d < 2^-100 are lifted by 2^64 (exact) as in encode8_rcp; d = 0 gives
// z = 0 and codes 0.  Returns the word; z in z_out.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t encode8_asym(float (&t)[8], float hi, float nlo, uint32_t& z_out, bool role) {
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
  uint32_t b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // rne(t inv) + z, clamped to [0, 15], in the magic-constant domain
    b[e] = rne_code_bits(t[e], inv) + z;
    b[e] = b[e] < kRoundMagicBits ? kRoundMagicBits : b[e];
    b[e] = b[e] > kRoundMagicBits + 15u ? kRoundMagicBits + 15u : b[e];
  }
  z_out = z;
  return pack8_ubits(b, role);
}

}  // namespace rw4
