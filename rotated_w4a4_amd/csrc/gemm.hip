// W4A4 GEMM on the gfx950 FP6 matrix cores.
//
//   Y[m, n] = sum over 128-wide groups g of sa[m, g] * sw[n, g] * acc[m, n, g]
//   acc[m, n, g] = sum over k in g of qa[m, k] * qw[n, k]     (exact)
//
// (the Rotated Runtime Smooth page, main equation and Figure 4 (3): the
// GEMM block equals the quantization group and the scale multiplies the
// block's partial result; the QuIP#/QTIP page, section 4.2, folds the
// rotation into the weights so the GEMM itself is a plain product.)
//
// Operands.  A pair of words of the stored form (16 codes) opens into the
// dense string of the codes' FP6 E2M3 encodings with two masks and four
// instructions (rw4_device.h): a signed code c becomes the subnormal c / 8, an
// unsigned code u (asymmetric activations) the value u / 8.  The scaled
// MFMA with format FP6 E2M3 on both sides and E8M0 operand scale 2^3 on
// both therefore returns acc itself, exactly (integer products, partial
// sums below 128 * 15 * 7 < 2^24).  Both operands open the same way, so
// the order of codes inside an operand is the same on both sides and the
// dot product over the group is unchanged.  FP6 operands take 6 registers
// and issue at about 1.5 times the FP8 rate.
//
// Kernels:
//   gemm_f8_kernel     large products: 128 x 128 block tiles, 4 waves of 64 x 64
//                      (gemm_f8p_kernel: the same for 128-wide groups, with
//                      the LDS reads software-pipelined),
//                      v_mfma_scale_f32_32x32x64_f8f6f4 on FP6 (2 per group per
//                      32 x 32 tile); the scale products sa * sw of a tile
//                      come from one v_mfma_f32_32x32x16_bf16 on a 3-way
//                      bf16 split of each scale, split once per block and
//                      group into LDS; the VALU unpacks and accumulates.
//   gemm_small_kernel  M <= 64, and batches up to 1024 rows whose tiled grid
//                      would have fewer than 128 blocks (in 64-row chunks,
//                      grid y): 16 or 32 output channels per block, the
//                      eight waves split K; A and the scales staged in LDS
//                      per iteration, the weights read straight into
//                      registers, one v_mfma_scale_f32_16x16x128_f8f6f4 per
//                      128 codes.
// MFMA result layouts: for 32 x 32, lane l holds
// D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32], r = 0..15; for 16 x 16,
// D[4 (l / 16) + r][l % 16], r = 0..3.
#include <type_traits>

#include "rw4_device.h"
#include "rw4_internal.h"

namespace rw4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kF6Scale = 127 + 3;  // E8M0 encoding of 2^3: FP6 code c / 8 times 2^3 is c
constexpr int kF6 = 2;             // MFMA operand format FP6 E2M3

// 4 stored words (32 codes: the pairs (w0, w3) and (w1, w2)) -> the
// 6-register FP6 operand (the last two registers of the vector are not
// read by an FP6 MFMA).  Four instructions per pair: X[0:32] = a & A,
// X[64:96] = b & C, X[32:64] = (a & ~A) | (b & ~C).
template <bool SIGNED>
__device__ __forceinline__ void open_pair(uint32_t a, uint32_t b, uint32_t& d0, uint32_t& d1, uint32_t& d2) {
  constexpr uint32_t kA = SIGNED ? kSgnA : kUnsA, kC = SIGNED ? kSgnC : kUnsC;
  const uint32_t t = b & ~kC;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d1) : "v"(a), "s"(~kA), "v"(t));  // (a & ~A) | t
  d0 = a & kA;
  d2 = b & kC;
}
template <bool SIGNED = true, class W>
__device__ __forceinline__ v8i f6_operand(const W& w) {
  uint32_t d[6];
  open_pair<SIGNED>(uint32_t(w[0]), uint32_t(w[3]), d[0], d[1], d[2]);
  open_pair<SIGNED>(uint32_t(w[1]), uint32_t(w[2]), d[3], d[4], d[5]);
  return v8i{int(d[0]), int(d[1]), int(d[2]), int(d[3]), int(d[4]), int(d[5]), 0, 0};
}

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
// bf16 MFMA operands whose product over K slots 0..5 is
// a1 b1 + a1 b2 + a2 b1 + a1 b3 + a2 b2 + a3 b1 = x y up to ~2^-24 relative:
// rows get [a1 a1 a2 a1 a2 a3 0 0], columns [b1 b2 b1 b3 b2 b1 0 0].  From
// P = x1 | x2 << 16 and Q = x3 | x1 << 16 each operand dword is one byte
// permute with a selector fixed per wave (rows or columns).
struct SplitSel {
  uint32_t s0, s1, s2;
};
__device__ __forceinline__ SplitSel split_selectors(bool rows) {
  // v_perm_b32(P, Q, sel): selector byte values 0-3 pick bytes of Q, 4-7 of P
  // halves: x1 = P.lo (5,4), x2 = P.hi (7,6), x3 = Q.lo (1,0), x1' = Q.hi (3,2)
  return rows ? SplitSel{0x05040504u, 0x05040706u, 0x01000706u}   // (x1,x1) (x2,x1) (x2,x3)
              : SplitSel{0x07060504u, 0x01000504u, 0x05040706u};  // (x1,x2) (x1,x3) (x2,x1)
}
__device__ __forceinline__ uint4 split_operand(float x, const SplitSel& sel) {
  uint32_t a1, a2, a3;
  split3(x, a1, a2, a3);
  const uint32_t P = a1 | (a2 << 16), Q = a3 | (a1 << 16);
  return make_uint4(__builtin_amdgcn_perm(P, Q, sel.s0), __builtin_amdgcn_perm(P, Q, sel.s1),
                    __builtin_amdgcn_perm(P, Q, sel.s2), 0u);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS staging.  Packed tiles go from global memory straight into
// LDS (global_load_lds_dwordx4: no VGPR round trip, no VALU) through a
// 3-stage ring, one 128-wide group per stage, two groups in flight.  LDS
// rows hold 64 packed bytes as four 16-byte slots, the slot index
// XOR-swizzled by (row >> 2) & 3 so that 16 lanes reading 16 rows hit 16
// distinct 4-bank groups.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

// Buffer resource over [base, base + bytes) (bytes < 2^31, checked on the
// host): raw (stride 0) access; out-of-range lanes read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
// 16 bytes per lane from rsrc + voffset + soffset into LDS at lds_base + 16 lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, int(voff), int(soff), 0, 0);
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

// Block barrier for LDS hand-offs only: waits for this wave's LDS accesses
// (vmcnt left at its maximum), so the global loads of later stages stay in
// flight across it; __syncthreads() would drain them (its workgroup release
// fence waits for vmcnt(0)).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
  asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}

// Shared memory of one block: two stages of two groups each (packed A and
// B tiles of 128 rows x 64 bytes per group), and the split scale operands
// of the same four groups.  One object, so every group buffer is a fixed
// immediate offset from a per-lane base address.  After the main loop the
// tile area stages the output tile for wide stores.
constexpr int kTileBytes = 128 * 64;               // one operand of one group
constexpr int kGroupBytes = 2 * kTileBytes;        // A and B
constexpr int kStageBytes = 2 * kGroupBytes;       // two groups
constexpr int kSplitGroupBytes = 256 * 16;         // 128 row + 128 column operands
// NSPLIT split buffers: one per group buffer, or two (one per 64-wide
// half) for 64-wide scale groups.
template <int NSPLIT>
struct alignas(16) GemmSmem {
  uint8_t tile[2 * kStageBytes];
  uint8_t split[NSPLIT * kSplitGroupBytes];
};
static_assert(2 * kStageBytes <= 65536 && 8 * kSplitGroupBytes <= 65536, "ds offsets are 16-bit");
// group buffer q (0..3: stage q / 2, slot q % 2)
constexpr int tile_off(int q) { return q * kGroupBytes; }
constexpr int split_off(int q) { return q * kSplitGroupBytes; }
constexpr int split_off64(int q, int h) { return (2 * q + h) * kSplitGroupBytes; }

// LDS reads of one group for a wave, in two batches that each wait for
// their own results (the compiler cannot see these reads, so it adds no
// wait for the DMA stages still in flight).  Batch 1: the fragments of
// K-half 0 (A tiles 0/1, B tiles 0/1; tile 1 lies 32 rows = 2048 bytes
// further; B lies kTileBytes after A).  Batch 2, issued while the first
// half's MFMAs run: the fragments of K-half 1 and the 4 split-scale
// operands (tile 1 lies 32 entries = 512 bytes further; columns 2048 bytes
// after rows).  OT/OS: immediate byte offsets of the group's buffers.
template <int OT>
__device__ __forceinline__ void lds_read_half0(v4u (&f)[4], uint32_t a, uint32_t b) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%6\n"
      "ds_read_b128 %1, %4 offset:%7\n"
      "ds_read_b128 %2, %5 offset:%8\n"
      "ds_read_b128 %3, %5 offset:%9\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
      : "v"(a), "v"(b), "i"(OT), "i"(OT + 2048), "i"(OT + kTileBytes), "i"(OT + kTileBytes + 2048)
      : "memory");
}
template <int OT, int OS>
__device__ __forceinline__ void lds_read_half1(v4u (&f)[4], v4u (&p)[4], uint32_t a, uint32_t b, uint32_t sa,
                                               uint32_t sb) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%12\n"
      "ds_read_b128 %1, %8 offset:%13\n"
      "ds_read_b128 %2, %9 offset:%14\n"
      "ds_read_b128 %3, %9 offset:%15\n"
      "ds_read_b128 %4, %10 offset:%16\n"
      "ds_read_b128 %5, %10 offset:%17\n"
      "ds_read_b128 %6, %11 offset:%18\n"
      "ds_read_b128 %7, %11 offset:%19\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(p[0]), "=&v"(p[1]), "=&v"(p[2]), "=&v"(p[3])
      : "v"(a), "v"(b), "v"(sa), "v"(sb), "i"(OT), "i"(OT + 2048), "i"(OT + kTileBytes),
        "i"(OT + kTileBytes + 2048), "i"(OS), "i"(OS + 512), "i"(OS + 2048), "i"(OS + 2048 + 512)
      : "memory");
}
template <int OS>
__device__ __forceinline__ void lds_write_split(uint32_t addr, v4u v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OS) : "memory");
}

// Blocks are dispatched round-robin over the 8 XCDs (block b on XCD b % 8),
// each with its own L2.  Renumber so that every XCD gets one contiguous
// range of logical tiles, and walk the tiles in bands of 8 tile rows,
// column by column, so the tiles resident on one XCD share A row panels
// and B column panels.
__device__ __forceinline__ void tile_of_block(int64_t b, int64_t nb, int64_t tiles_m, int64_t& mt,
                                              int64_t& nt) {
  const int64_t x = b & 7, i = b >> 3, q = nb >> 3, r = nb & 7;
  const int64_t l = x * q + (x < r ? x : r) + i;
  const int64_t tiles_n = nb / tiles_m;
  constexpr int64_t kBand = 8;
  const int64_t band = l / (kBand * tiles_n);
  const int64_t m_first = band * kBand;
  const int64_t gm = tiles_m - m_first < kBand ? tiles_m - m_first : kBand;
  const int64_t li = l - band * kBand * tiles_n;
  mt = m_first + li % gm;
  nt = li / gm;
}

// GSZ: scale group width.  128: one scale pair per group buffer.  256: the
// two 128-groups of a stage share one scale pair; the accumulator runs over
// both (partial sums below 256 * 49 < 2^24, still exact) and the scale
// products and the epilogue run once per stage.  64: each K-half of a
// group has its own scale pair, so each K-half ends with the scale products
// and the epilogue; the split buffers double (96 KiB of LDS: one block per
// CU).
template <bool BF16, int GSZ>
__global__ __launch_bounds__(256, 2) void gemm_f8_kernel(const uint8_t* __restrict__ qa,
                                                         const float* __restrict__ sa,
                                                         const uint8_t* __restrict__ qw,
                                                         const float* __restrict__ sw, int64_t M,
                                                         int64_t N, int64_t K, void* __restrict__ y,
                                                         int64_t ldy, int64_t tiles_m) {
  constexpr bool G256 = GSZ == 256, G64 = GSZ == 64;
  __shared__ GemmSmem<G64 ? 8 : 4> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t G = K / kGroup;
  const int64_t GS = G256 ? G / 2 : G64 ? 2 * G : G;  // scale columns
  const int64_t rowbytes = K / 2;
  int64_t mt, nt;
  tile_of_block(blockIdx.x, gridDim.x, tiles_m, mt, nt);
  const int64_t m0 = mt * 128, n0 = nt * 128;

  // DMA sources: wave w fills rows [32 w, 32 w + 32) of the A and B tiles,
  // 16 rows per instruction; rows are clamped into range (every wave issues
  // the same instructions; data of clamped rows is never stored).  Buffer
  // ranges cover only the block's rows (<= 128 rows * K / 2 bytes).
  const int srow = lane >> 2;
  const int schunk = ((lane & 3) ^ ((lane >> 4) & 3)) * 16;
  const int64_t rows_a = M - m0 < 128 ? M - m0 : 128, rows_b = N - n0 < 128 ? N - n0 : 128;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(qa + m0 * rowbytes, rows_a * rowbytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(qw + n0 * rowbytes, rows_b * rowbytes);
  uint32_t a_src[2], b_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t r = (wave * 2 + i) * 16 + srow;
    a_src[i] = uint32_t((r < rows_a ? r : rows_a - 1) * rowbytes + schunk);
    b_src[i] = uint32_t((r < rows_b ? r : rows_b - 1) * rowbytes + schunk);
  }
  auto issue = [&](int q, int64_t g) {  // group g into group buffer q
    const uint32_t so = uint32_t((g < G ? g : G - 1) * 64);
    uint8_t* t = sm.tile + tile_off(q);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(ra, a_src[i], so, t + (wave * 2 + i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(rb, b_src[i], so, t + kTileBytes + (wave * 2 + i) * 1024);
  };

  // this thread splits one scale per group: sa of tile row tid (tid < 128)
  // or sw of tile column tid - 128 (waves 0-1 rows, waves 2-3 columns)
  const bool row_scale = wave < 2;
  const __amdgpu_buffer_rsrc_t rs =
      row_scale ? make_rsrc(sa + m0 * GS, rows_a * GS * 4) : make_rsrc(sw + n0 * GS, rows_b * GS * 4);
  uint32_t sc_off;  // byte offset of this thread's scale row
  {
    const int64_t r = row_scale ? tid : tid - 128;
    const int64_t lim = row_scale ? rows_a : rows_b;
    sc_off = uint32_t((r < lim ? r : lim - 1) * GS * 4);
  }
  auto sc_load = [&](int64_t g) {  // scale column g (clamped; past the end never read)
    return __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rs, int(sc_off), int((g < GS ? g : GS - 1) * 4), 0));
  };
  const SplitSel sel = split_selectors(row_scale);
  const uint32_t sp_addr = lds_off(sm.split + tid * 16);
  // written with an LDS store the compiler does not see (it would otherwise
  // wait for the DMA stages in flight, which never target the split
  // buffers); the next wait_vm_barrier completes it before any wave reads it
  auto put_split = [&](auto q_const, float x) {
    constexpr int q = decltype(q_const)::value;
    const uint4 o = split_operand(x, sel);
    lds_write_split<split_off(q)>(sp_addr, v4u{o.x, o.y, o.z, o.w});
  };
  auto put_split64 = [&](auto q_const, float x0, float x1) {  // the two halves of group buffer q
    constexpr int q = decltype(q_const)::value;
    const uint4 o0 = split_operand(x0, sel), o1 = split_operand(x1, sel);
    lds_write_split<split_off64(q, 0)>(sp_addr, v4u{o0.x, o0.y, o0.z, o0.w});
    lds_write_split<split_off64(q, 1)>(sp_addr, v4u{o1.x, o1.y, o1.z, o1.w});
  };

  // per-lane LDS read bases (group buffer 0).  Lanes 32..63 supply K slots
  // 8..15 of the bf16 scale-product MFMA with the same split operands as
  // lanes 0..31 (the product comes out doubled; see the epilogue).
  const int frow = lane & 31, h = lane >> 5;
  uint32_t ba0, ba1, bb0, bb1, bsa, bsb;
  {
    const uint32_t t0 = lds_off(sm.tile), s0 = lds_off(sm.split);
    const int ra_ = wm * 64 + frow, rb_ = wn * 64 + frow;
    const int xa = (ra_ >> 2) & 3, xb = (rb_ >> 2) & 3;
    // 16-byte slot (32 codes) of K-half ks for lane half h: the MFMA takes
    // K 0-31 from lanes 0-31 and K 32-63 from lanes 32-63.  With 64-wide
    // scale groups each K-half must be one 64-group (slots 2 ks, 2 ks + 1);
    // otherwise any split works and slot 2 h + ks is used.
    const int s0_ = G64 ? h : 2 * h, s1_ = G64 ? 2 + h : 2 * h + 1;
    ba0 = t0 + ra_ * 64 + ((s0_ ^ xa) * 16);
    ba1 = t0 + ra_ * 64 + ((s1_ ^ xa) * 16);
    bb0 = t0 + rb_ * 64 + ((s0_ ^ xb) * 16);
    bb1 = t0 + rb_ * 64 + ((s1_ ^ xb) * 16);
    bsa = s0 + (wm * 64 + frow) * 16;
    bsb = s0 + (wn * 64 + frow) * 16;  // + 2048 (column operands) in the read offsets
  }
  float yacc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) yacc[i][j][r] = 0.0f;

  // Scale products of the four 32 x 32 tiles from the split operands ps
  // (rows, rows, columns, columns), then y += acc * p.  Both lane halves
  // supply the same split operands (K slots 0-7 and 8-15), so the bf16
  // MFMA returns 2 sa sw; the integer MFMAs take the B-side scale 2^2
  // instead of 2^3 and return acc / 2 (exact), so the product is unchanged.
  v16f acc[2][2];
  auto epilogue = [&](v4u (&ps)[4]) {
    // tile by tile, one tile ahead of the accumulation (the scheduling
    // barriers keep at most two product tiles live)
    auto prod = [&](int t) {
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ps[t >> 1]),
                                                     __builtin_bit_cast(v8bf, ps[2 + (t & 1)]), v16f{}, 0,
                                                     0, 0);
    };
    auto accum = [&](int t, const v16f& p) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        yacc[t >> 1][t & 1][r] = fmaf(acc[t >> 1][t & 1][r], p[r], yacc[t >> 1][t & 1][r]);
    };
    v16f p0 = prod(0);
    v16f p1 = prod(1);
    __builtin_amdgcn_sched_barrier(0);
    accum(0, p0);
    p0 = prod(2);
    __builtin_amdgcn_sched_barrier(0);
    accum(1, p1);
    p1 = prod(3);
    __builtin_amdgcn_sched_barrier(0);
    accum(2, p0);
    accum(3, p1);
    __builtin_amdgcn_sched_barrier(0);
  };

  // One 128-group from group buffer q.  INIT: the accumulators start at
  // zero (else they continue); EPI: the scale products (split operands of
  // group buffer QS) and the epilogue follow.
  auto compute = [&](auto q_const, auto qs_const, auto init_const, auto epi_const) {
    constexpr int q = decltype(q_const)::value;
    constexpr int qs = decltype(qs_const)::value;
    constexpr bool init = decltype(init_const)::value;
    constexpr bool epi = decltype(epi_const)::value;
    v4u fr[4], ps[4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // fr: A tile 0, A tile 1, B tile 0, B tile 1 of this K-half
      if (ks == 0)
        lds_read_half0<tile_off(q)>(fr, ba0, bb0);
      else if constexpr (epi)
        lds_read_half1<tile_off(q), split_off(qs)>(fr, ps, ba1, bb1, bsa, bsb);
      else
        lds_read_half0<tile_off(q)>(fr, ba1, bb1);  // K-half 1 fragments only
      v8i oa[2], ob[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) oa[i] = f6_operand(fr[i]);
#pragma unroll
      for (int j = 0; j < 2; ++j) ob[j] = f6_operand(fr[2 + j]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const v16f c = (init && ks == 0) ? v16f{} : acc[i][j];
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(oa[i], ob[j], c, kF6, kF6, 0, kF6Scale,
                                                                     0, kF6Scale - 1);
        }
      // keep each half's unpack and MFMAs together (bounds register use)
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (epi) epilogue(ps);
    __builtin_amdgcn_sched_barrier(0);
  };

  // One 128-group with 64-wide scale groups: each K-half reads its own
  // splits and ends with its own epilogue.
  auto compute64 = [&](auto q_const) {
    constexpr int q = decltype(q_const)::value;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4u fr[4], ps[4];
      if (ks == 0)
        lds_read_half1<tile_off(q), split_off64(q, 0)>(fr, ps, ba0, bb0, bsa, bsb);
      else
        lds_read_half1<tile_off(q), split_off64(q, 1)>(fr, ps, ba1, bb1, bsa, bsb);
      v8i oa[2], ob[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) oa[i] = f6_operand(fr[i]);
#pragma unroll
      for (int j = 0; j < 2; ++j) ob[j] = f6_operand(fr[2 + j]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(oa[i], ob[j], v16f{}, kF6, kF6, 0, kF6Scale, 0,
                                                                     kF6Scale - 1);
      __builtin_amdgcn_sched_barrier(0);
      epilogue(ps);
    }
  };

  // Stage s holds groups 2s and 2s + 1 in group buffers 2 (s % 2) and
  // 2 (s % 2) + 1.  Iteration s: wait for stage s (everything this wave has
  // in flight) and a block barrier; issue the scale loads and DMA of stage
  // s + 1 into the other buffers (all waves finished reading them before
  // the barrier); compute the two groups; split the scales of stage s + 1.
  // Past the last group the loads are clamped to group G - 1 and never read.
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
  // With 256-wide scale groups (G even) stage s is scale column s: one split
  // per stage, in the stage's first buffer.
  using T = std::true_type;
  using F = std::false_type;
  if constexpr (G256) {
    put_split(Q0{}, sc_load(0));
  } else if constexpr (G64) {
    put_split64(Q0{}, sc_load(0), sc_load(1));
    put_split64(Q1{}, sc_load(2), sc_load(3));
  } else {
    put_split(Q0{}, sc_load(0));
    put_split(Q1{}, sc_load(1));
  }
  issue(0, 0);
  issue(1, 1);
  const int64_t S = (G + 1) / 2;
  auto stage = [&](auto q0, auto q1, auto n0_, auto n1_, int64_t s) {
    wait_vm_barrier<0>();
    if constexpr (G256) {
      const float x0 = sc_load(s + 1);
      issue(decltype(n0_)::value, 2 * s + 2);
      issue(decltype(n1_)::value, 2 * s + 3);
      compute(q0, q0, T{}, F{});
      compute(q1, q0, F{}, T{});
      put_split(n0_, x0);
    } else if constexpr (G64) {
      const float x0 = sc_load(4 * s + 4), x1 = sc_load(4 * s + 5);
      const float x2 = sc_load(4 * s + 6), x3 = sc_load(4 * s + 7);
      issue(decltype(n0_)::value, 2 * s + 2);
      issue(decltype(n1_)::value, 2 * s + 3);
      compute64(q0);
      if (2 * s + 1 < G) compute64(q1);
      put_split64(n0_, x0, x1);
      put_split64(n1_, x2, x3);
    } else {
      const float x0 = sc_load(2 * s + 2), x1 = sc_load(2 * s + 3);
      issue(decltype(n0_)::value, 2 * s + 2);
      issue(decltype(n1_)::value, 2 * s + 3);
      compute(q0, q0, T{}, T{});
      if (2 * s + 1 < G) compute(q1, q1, T{}, T{});
      put_split(n0_, x0);
      put_split(n1_, x1);
    }
  };
  for (int64_t s = 0; s < S; s += 2) {
    stage(Q0{}, Q1{}, Q2{}, Q3{}, s);
    if (s + 1 >= S) break;
    stage(Q2{}, Q3{}, Q0{}, Q1{}, s + 1);
  }
  // drain the trailing loads: no DMA may outlive the block's LDS allocation,
  // and the tile area is reused below
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
  asm volatile("s_barrier" ::: "memory");

  // Output: each wave stages its 64 x 64 tile in LDS (row-major), then
  // writes whole 16-byte chunks of rows; chunks that cross the right edge,
  // or a leading dimension that breaks 16-byte alignment, use element
  // stores.
  constexpr int E = BF16 ? 2 : 4;           // bytes per element
  constexpr int RB = 64 * E;                // bytes per staged row
  uint8_t* ot = sm.tile + wave * 64 * RB;   // 8 or 16 KB per wave
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i * 32 + (r >> 2) * 8 + h * 4 + (r & 3), col = j * 32 + frow;
        if constexpr (BF16)
          *reinterpret_cast<uint16_t*>(ot + row * RB + col * 2) = f32_to_bf16_rne(yacc[i][j][r]);
        else
          *reinterpret_cast<float*>(ot + row * RB + col * 4) = yacc[i][j][r];
      }
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0x0 << 8) | 0xF | (3 << 14));  // lgkmcnt(0)
  const int64_t wr0 = m0 + wm * 64, wc0 = n0 + wn * 64;
  constexpr int CPR = RB / 16;  // 16-byte chunks per row
  const bool aligned = ((ldy * E) % 16 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
#pragma unroll
  for (int it = 0; it < CPR; ++it) {
    const int idx = it * 64 + lane;
    const int row = idx / CPR, ch = idx % CPR;
    const int64_t m = wr0 + row, n = wc0 + ch * (16 / E);
    if (m >= M) continue;
    const v4u v = *reinterpret_cast<const v4u*>(ot + row * RB + ch * 16);
    uint8_t* dst = reinterpret_cast<uint8_t*>(y) + (m * ldy + n) * E;
    if (aligned && n + 16 / E <= N) {
      // streaming store: nothing in the kernel reads y back (3 % faster
      // at 2048 x 4096 x 4096 than a cached store, neutral at larger shapes)
      __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(dst));
    } else {
#pragma unroll
      for (int e = 0; e < 16 / E; ++e) {
        if (n + e < N) {
          if constexpr (BF16)
            reinterpret_cast<uint16_t*>(dst)[e] = uint16_t(v[e / 2] >> (16 * (e & 1)));
          else
            reinterpret_cast<uint32_t*>(dst)[e] = v[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// gemm_f8p_kernel: the 128-wide-group form of gemm_f8_kernel with its LDS
// reads software-pipelined.  The two DMA stages and their split buffers are
// four distinct __shared__ objects, so the compiler can tell that the DMA
// into one stage never writes what is being read from the other; the
// fragment reads are then ordinary loads that it schedules itself, issued
// a K-half (or a group) ahead of the MFMAs that consume them, with partial
// lgkmcnt waits (the asm reads of gemm_f8_kernel wait for all of their own
// results at once).  Bit-identical results; the pipelining measured 8-10 %
// faster at 4096 x 14336 x 4096 and 8192 x 4096 x 11008, and the wave-
// priority alternation below a further 8-19 %.
// ---------------------------------------------------------------------------
constexpr int kStageTileBytes = 2 * kGroupBytes;        // A and B tiles of two groups
constexpr int kStageSplitBytes = 2 * kSplitGroupBytes;  // their split scale operands

// ASYM: unsigned activation codes with zero points za [M][G] and the
// weight code sums cw [N][G]: every group's (halved) accumulators start at
// -za cw / 2 (exact, from a bf16 MFMA on the spare K slots 6 and 7 of the
// split scale operands: -za twice against cw / 4 split into two bf16 parts,
// in both lane halves), then the halved integer products add to them.
template <bool BF16, bool ASYM = false>
__global__ __launch_bounds__(256, 2) void gemm_f8p_kernel(const uint8_t* __restrict__ qa,
                                                          const float* __restrict__ sa,
                                                          const uint8_t* __restrict__ qw,
                                                          const float* __restrict__ sw, int64_t M,
                                                          int64_t N, int64_t K, void* __restrict__ y,
                                                          int64_t ldy, int64_t tiles_m,
                                                          const float* __restrict__ za = nullptr,
                                                          const float* __restrict__ cw = nullptr) {
  __shared__ __align__(16) uint8_t tA[kStageTileBytes];
  __shared__ __align__(16) uint8_t tB[kStageTileBytes];
  __shared__ __align__(16) uint8_t sA[kStageSplitBytes];
  __shared__ __align__(16) uint8_t sB[kStageSplitBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t G = K / kGroup;
  const int64_t rowbytes = K / 2;
  int64_t mt, nt;
  tile_of_block(blockIdx.x, gridDim.x, tiles_m, mt, nt);
  const int64_t m0 = mt * 128, n0 = nt * 128;

  // DMA sources as in gemm_f8_kernel: wave w fills rows [32 w, 32 w + 32)
  // of the A and B tiles, rows clamped into range
  const int srow = lane >> 2;
  const int schunk = ((lane & 3) ^ ((lane >> 4) & 3)) * 16;
  const int64_t rows_a = M - m0 < 128 ? M - m0 : 128, rows_b = N - n0 < 128 ? N - n0 : 128;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(qa + m0 * rowbytes, rows_a * rowbytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(qw + n0 * rowbytes, rows_b * rowbytes);
  uint32_t a_src[2], b_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t r = (wave * 2 + i) * 16 + srow;
    a_src[i] = uint32_t((r < rows_a ? r : rows_a - 1) * rowbytes + schunk);
    b_src[i] = uint32_t((r < rows_b ? r : rows_b - 1) * rowbytes + schunk);
  }
  auto issue = [&](uint8_t* T, int q, int64_t g) {  // group g into slot q of stage T
    const uint32_t so = uint32_t((g < G ? g : G - 1) * 64);
    uint8_t* t = T + q * kGroupBytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(ra, a_src[i], so, t + (wave * 2 + i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(rb, b_src[i], so, t + kTileBytes + (wave * 2 + i) * 1024);
  };

  // thread tid splits sa of tile row tid (tid < 128) or sw of column tid - 128
  const bool row_scale = wave < 2;
  const __amdgpu_buffer_rsrc_t rs =
      row_scale ? make_rsrc(sa + m0 * G, rows_a * G * 4) : make_rsrc(sw + n0 * G, rows_b * G * 4);
  uint32_t sc_off;
  {
    const int64_t r = row_scale ? tid : tid - 128;
    const int64_t lim = row_scale ? rows_a : rows_b;
    sc_off = uint32_t((r < lim ? r : lim - 1) * G * 4);
  }
  auto sc_load = [&](int64_t g) {
    return __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rs, int(sc_off), int((g < G ? g : G - 1) * 4), 0));
  };
  // ASYM: the zero point (rows) or weight code sum (columns) of the same
  // row or column
  const __amdgpu_buffer_rsrc_t rz =
      row_scale ? make_rsrc(za + m0 * G, ASYM ? rows_a * G * 4 : 0) : make_rsrc(cw + n0 * G, ASYM ? rows_b * G * 4 : 0);
  auto z_load = [&](int64_t g) {
    if constexpr (!ASYM) return 0.0f;
    return __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rz, int(sc_off), int((g < G ? g : G - 1) * 4), 0));
  };
  const SplitSel sel = split_selectors(row_scale);
  auto put_split = [&](uint8_t* S, int q, float x, float zx) {
    const uint4 o = split_operand(x, sel);
    uint32_t w = 0;
    if constexpr (ASYM) {
      // slots 6, 7: rows (-za, -za), columns cw / 4 as (rounded toward zero to
      // bf16, the exact rest): both lane halves supply them, so the products
      // add to -za cw / 2, the zero-point term of the halved accumulator
      if (row_scale) {
        const uint32_t nz = __float_as_uint(-zx) >> 16;  // small integers: exact in bf16
        w = nz | (nz << 16);
      } else {
        const float c4 = zx * 0.25f;  // exact
        const uint32_t hi = __float_as_uint(c4) & 0xFFFF0000u;
        w = (hi >> 16) | (__float_as_uint(c4 - __uint_as_float(hi)) & 0xFFFF0000u);
      }
    }
    *reinterpret_cast<v4u*>(S + q * kSplitGroupBytes + tid * 16) = v4u{o.x, o.y, o.z, w};
  };

  // byte offsets of this lane's fragments inside a group slot (as the read
  // bases of gemm_f8_kernel: K-half ks reads 16-byte slot 2 h + ks, XOR-
  // swizzled by (row >> 2) & 3; tile 1 lies 32 rows further, B after A)
  const int frow = lane & 31, h = lane >> 5;
  uint32_t oa0, oa1, ob0, ob1, osa, osb;
  {
    const int ra_ = wm * 64 + frow, rb_ = wn * 64 + frow;
    const int xa = (ra_ >> 2) & 3, xb = (rb_ >> 2) & 3;
    oa0 = ra_ * 64 + (((2 * h) ^ xa) * 16);
    oa1 = ra_ * 64 + (((2 * h + 1) ^ xa) * 16);
    ob0 = kTileBytes + rb_ * 64 + (((2 * h) ^ xb) * 16);
    ob1 = kTileBytes + rb_ * 64 + (((2 * h + 1) ^ xb) * 16);
    osa = (wm * 64 + frow) * 16;
    osb = 2048 + (wn * 64 + frow) * 16;
  }
  // Both lane halves supply the same split operands: the bf16 MFMA returns
  // 2 sa sw and the integer MFMAs return acc / 2 (B-side scale 2^2, exact).
  // ASYM: the accumulators start at -za cw / 2 (slots 6-7, see put_split),
  // and the scale products leave slots 6-7 out (row operands zeroed there).
  constexpr int kBScale = kF6Scale - 1;
  auto rd = [](const uint8_t* base, uint32_t off) { return *reinterpret_cast<const v4u*>(base + off); };
  auto read_half = [&](const uint8_t* T, int q, uint32_t oa, uint32_t ob, v4u (&f)[4]) {
    const uint8_t* b = T + q * kGroupBytes;
    f[0] = rd(b, oa);
    f[1] = rd(b, oa + 2048);
    f[2] = rd(b, ob);
    f[3] = rd(b, ob + 2048);
  };
  auto read_splits = [&](const uint8_t* S, int q, v4u (&p)[4]) {
    const uint8_t* b = S + q * kSplitGroupBytes;
    p[0] = rd(b, osa);
    p[1] = rd(b, osa + 512);
    p[2] = rd(b, osb);
    p[3] = rd(b, osb + 512);
  };

  float yacc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) yacc[i][j][r] = 0.0f;

  v16f acc[2][2];
  auto mfma_half = [&](const v4u (&f)[4], bool init) {
    v8i oa[2], ob[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) oa[i] = ASYM ? f6_operand<false>(f[i]) : f6_operand(f[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) ob[j] = f6_operand(f[2 + j]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(oa[i], ob[j], init ? v16f{} : acc[i][j], kF6, kF6,
                                                                   0, kF6Scale, 0, kBScale);
  };
  // scale products of the four 32 x 32 tiles (bf16 MFMA on the splits), then y += acc * p
  // ASYM: the accumulators of a group start at -za cw / 2 (K slots 6 and 7 only)
  auto init_acc = [&](const v4u (&ps)[4]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, v4u{0u, 0u, 0u, ps[i][3]}),
                                                           __builtin_bit_cast(v8bf, v4u{0u, 0u, 0u, ps[2 + j][3]}),
                                                           v16f{}, 0, 0, 0);
  };
  auto epilogue = [&](v4u (&ps)[4]) {
    if constexpr (ASYM) {
#pragma unroll
      for (int i = 0; i < 2; ++i) ps[i][3] = 0u;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v16f p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ps[t >> 1]),
                                                             __builtin_bit_cast(v8bf, ps[2 + (t & 1)]), v16f{}, 0,
                                                             0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        yacc[t >> 1][t & 1][r] = fmaf(acc[t >> 1][t & 1][r], p[r], yacc[t >> 1][t & 1][r]);
    }
  };

  // Stage s (groups 2s, 2s + 1) lives in tA/sA for even s, tB/sB for odd s.
  // Iteration s: wait for this wave's DMA and a block barrier; load the
  // scales and issue the DMA of stage s + 1 into the other arrays (every
  // wave finished reading them before the barrier); compute the two groups
  // with each K-half's fragments read one step ahead; split the scales of
  // stage s + 1.  Loads past the last group are clamped and never read.
  // the first stage's DMA goes out before the wait for its scales, so the
  // two memory latencies overlap
  issue(tA, 0, 0);
  issue(tA, 1, 1);
  {
    const float x0 = sc_load(0), x1 = sc_load(1), z0 = z_load(0), z1 = z_load(1);
    put_split(sA, 0, x0, z0);
    put_split(sA, 1, x1, z1);
  }
  const int64_t S = (G + 1) / 2;
  // Wave priority alternates stage by stage, opposite for odd and even
  // blocks.  Two blocks share a CU, and the arbiter otherwise lets the
  // older block's waves win: it finished ~7.6 us before the younger one at
  // 2048 x 4096 x 4096 (per-block timestamps), leaving one wave per SIMD for
  // the tail.  With the alternation the pair ends ~1.2 us apart.  Measured
  // over rotating 512 MiB buffer sets, on two boxes: 4096 x 14336 x 4096
  // -13 % and -19 %, 8192 x 4096 x 11008 -8 % and -10 %, 2048 x 4096 x 4096
  // -3 %.  Toggling every group instead of every stage was 20-40 % slower.
  const int prio_phase = int(blockIdx.x & 1);
  auto stage = [&](uint8_t* Tc, uint8_t* Sc, uint8_t* Tn, uint8_t* Sn, int64_t s) {
    if (((s + prio_phase) & 1) != 0)
      __builtin_amdgcn_s_setprio(2);
    else
      __builtin_amdgcn_s_setprio(0);
    wait_vm_barrier<0>();
    const float x0 = sc_load(2 * s + 2), x1 = sc_load(2 * s + 3);
    const float z0 = z_load(2 * s + 2), z1 = z_load(2 * s + 3);
    issue(Tn, 0, 2 * s + 2);
    issue(Tn, 1, 2 * s + 3);
    v4u f0[4], f1[4], ps[4];
    read_half(Tc, 0, oa0, ob0, f0);
    read_half(Tc, 0, oa1, ob1, f1);
    read_splits(Sc, 0, ps);
    if constexpr (ASYM) init_acc(ps);
    mfma_half(f0, !ASYM);
    const bool two = 2 * s + 1 < G;
    if (two) read_half(Tc, 1, oa0, ob0, f0);
    mfma_half(f1, false);
    epilogue(ps);
    if (two) {
      read_half(Tc, 1, oa1, ob1, f1);
      read_splits(Sc, 1, ps);
      if constexpr (ASYM) init_acc(ps);
      mfma_half(f0, !ASYM);
      mfma_half(f1, false);
      epilogue(ps);
    }
    put_split(Sn, 0, x0, z0);
    put_split(Sn, 1, x1, z1);
  };
  for (int64_t s = 0; s < S; s += 2) {
    stage(tA, sA, tB, sB, s);
    if (s + 1 >= S) break;
    stage(tB, sB, tA, sA, s + 1);
  }
  __builtin_amdgcn_s_setprio(0);
  // drain the trailing DMA before the stage arrays are reused for the output
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
  asm volatile("s_barrier" ::: "memory");

  // output: each wave stages its 64 x 64 tile (8 or 16 KB; waves 0-1 in tA,
  // 2-3 in tB), then writes whole 16-byte row chunks; chunks crossing the
  // right edge, or rows that break 16-byte alignment, use element stores
  constexpr int E = BF16 ? 2 : 4;
  constexpr int RB = 64 * E;
  static_assert(2 * 64 * RB <= kStageTileBytes, "two wave tiles per stage array");
  uint8_t* ot = (wave < 2 ? tA : tB) + (wave & 1) * 64 * RB;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i * 32 + (r >> 2) * 8 + h * 4 + (r & 3), col = j * 32 + frow;
        if constexpr (BF16)
          *reinterpret_cast<uint16_t*>(ot + row * RB + col * 2) = f32_to_bf16_rne(yacc[i][j][r]);
        else
          *reinterpret_cast<float*>(ot + row * RB + col * 4) = yacc[i][j][r];
      }
  __syncthreads();
  const int64_t wr0 = m0 + wm * 64, wc0 = n0 + wn * 64;
  constexpr int CPR = RB / 16;
  const bool aligned = ((ldy * E) % 16 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
#pragma unroll
  for (int it = 0; it < CPR; ++it) {
    const int idx = it * 64 + lane;
    const int row = idx / CPR, ch = idx % CPR;
    const int64_t m = wr0 + row, n = wc0 + ch * (16 / E);
    if (m >= M) continue;
    const v4u v = *reinterpret_cast<const v4u*>(ot + row * RB + ch * 16);
    uint8_t* dst = reinterpret_cast<uint8_t*>(y) + (m * ldy + n) * E;
    if (aligned && n + 16 / E <= N) {
      // streaming store: nothing in the kernel reads y back (3 % faster
      // at 2048 x 4096 x 4096 than a cached store, neutral at larger shapes)
      __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(dst));
    } else {
#pragma unroll
      for (int e = 0; e < 16 / E; ++e) {
        if (n + e < N) {
          if constexpr (BF16)
            reinterpret_cast<uint16_t*>(dst)[e] = uint16_t(v[e / 2] >> (16 * (e & 1)));
          else
            reinterpret_cast<uint32_t*>(dst)[e] = v[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small-M kernel (decode and small batches): one block of 8 waves per CT
// tiles of 16 output channels and one chunk of 16 MT rows of A (grid y).  K is cut into slices of 128 codes,
// one v_mfma_scale_f32_16x16x128_f8f6f4 per slice, 16-channel tile and
// 16-row A tile; lane l supplies row l % 16 and codes
// [32 (l / 16), 32 (l / 16) + 32) of the slice for both operands.  An
// iteration covers GB slices, NS consecutive ones per wave.
//
// Every block reads all of A and of sa, so these are the hot lines of the
// launch: per iteration the block stages its A slices and the scale columns
// they use (sa of every row, sw of its channels) into LDS with coalesced
// loads, instead of each wave fetching them lane by lane.  The weights are
// read once, straight into registers.  The loads of the next iteration are
// issued before the current one computes (two register stages).  All loads
// are buffer loads whose range or offset makes out-of-range lanes read
// zeros, so no branch surrounds a load and the waits count exactly.
// The partial sums of the waves are added in LDS at the end.
//
// GSZ 256: a scale column covers two consecutive slices, whose two MFMAs
// chain into one accumulator before the scale is applied.  GSZ 64: a slice
// has two scale columns; its MFMA runs twice, each time with the A
// fragments of the other 64-code half zeroed (lanes 0-31 supply codes 0-63
// of the slice, lanes 32-63 codes 64-127).
// ---------------------------------------------------------------------------
constexpr int kSmallWaves = 8;
constexpr int kSmallThreads = kSmallWaves * 64;
constexpr uint32_t kNoRead = 0x80000000u;  // buffer offset past every range: the load returns zeros

template <int GSZ, int MT, int CT>
struct SmallCfg {
  static constexpr int P = GSZ == 256 ? 2 : 1;                 // slices per scale column
  static constexpr int H = GSZ == 64 ? 2 : 1;                  // scale columns per slice
  static constexpr int NS = (MT == 4 ? 1 : 2) > P ? (MT == 4 ? 1 : 2) : P;  // slices per wave and iteration
  static constexpr int GB = kSmallWaves * NS;                   // slices per iteration
  static constexpr int CW = GB * H / P;                         // scale columns per iteration
  static constexpr int AROW = GB * 4;                           // 16-byte chunks of an A row slice
  static constexpr int AR = 16 * MT * AROW / kSmallThreads;     // A chunks staged per thread
  static constexpr int SAE = 16 * MT * CW, SWE = 16 * CT * CW;  // staged scales
  static constexpr int SAR = (SAE + kSmallThreads - 1) / kSmallThreads;
  static constexpr int SWR = (SWE + kSmallThreads - 1) / kSmallThreads;
  // LDS: A rows padded by one chunk, then sa as [column][row], sw as [column][channel]
  // (each padded to whole rounds of the block, the idle slots never read)
  static constexpr int A_BYTES = 16 * MT * (AROW + 1) * 16;
  static constexpr int SA_OFF = A_BYTES, SW_OFF = SA_OFF + SAR * kSmallThreads * 4;
  static constexpr int BYTES = SW_OFF + SWR * kSmallThreads * 4;
  static constexpr int RED_BYTES = kSmallWaves * CT * MT * 64 * 4 * 4;  // aliases the A rows
  static_assert(AR * kSmallThreads == 16 * MT * AROW, "A slice must split evenly over the block");
  static_assert(RED_BYTES <= A_BYTES, "reduction buffer must fit in the A staging area");
  static_assert(CT * MT <= kSmallWaves, "one wave per output tile in the epilogue");
};

template <int GSZ, int MT, int CT, bool ASYM = false>
struct SmallStage {
  using C = SmallCfg<GSZ, MT, CT>;
  float sa[C::SAR], sw[C::SWR];
  float za[ASYM ? C::SAR : 1], cw[ASYM ? C::SWR : 1];  // ASYM: zero points and weight code sums
  v4u a[C::AR];
  v4u b[CT][C::NS];
};

// ASYM (GSZ = 128): unsigned activation codes with zero points za and
// weight code sums cw, staged like sa and sw; each product starts at
// -za cw.
template <bool BF16, int GSZ, int MT, int CT, bool ASYM = false>
__global__ __launch_bounds__(kSmallThreads) void gemm_small_kernel(const uint8_t* __restrict__ qa,
                                                                   const float* __restrict__ sa,
                                                                   const uint8_t* __restrict__ qw,
                                                                   const float* __restrict__ sw, int64_t M,
                                                                   int64_t N, int64_t K, void* __restrict__ y,
                                                                   int64_t ldy, const float* __restrict__ za = nullptr,
                                                                   const float* __restrict__ cw = nullptr) {
  using C = SmallCfg<GSZ, MT, CT>;
  using Stage = SmallStage<GSZ, MT, CT, ASYM>;
  static_assert(!ASYM || GSZ == 128, "asymmetric groups of 128");
  constexpr int ZA_OFF = C::BYTES, CW_OFF = ZA_OFF + C::SAR * kSmallThreads * 4;
  constexpr int LDS_BYTES = ASYM ? CW_OFF + C::SWR * kSmallThreads * 4 : C::BYTES;
  __shared__ __align__(16) uint8_t lds[LDS_BYTES];
  v4u* const As = reinterpret_cast<v4u*>(lds);
  float* const saT = reinterpret_cast<float*>(lds + C::SA_OFF);
  float* const swT = reinterpret_cast<float*>(lds + C::SW_OFF);
  float* const zaT = reinterpret_cast<float*>(lds + ZA_OFF);
  float* const cwT = reinterpret_cast<float*>(lds + CW_OFF);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int am = lane & 15;   // A row within a 16-row tile; B channel within a 16-channel tile
  const int part = lane >> 4;  // 32-code quarter of the slice
  const int64_t SL = K / kGroup;             // slices
  const int64_t GS = SL * C::H / C::P;       // scale columns
  const int64_t rowbytes = K / 2;
  const int64_t n0 = int64_t(blockIdx.x) * 16 * CT;
  const int64_t nrows = N - n0 < 16 * CT ? N - n0 : 16 * CT;
  const int64_t m0 = int64_t(blockIdx.y) * 16 * MT;  // this block's chunk of A rows
  const int64_t mrows = M - m0 < 16 * MT ? M - m0 : 16 * MT;
  const int64_t NI = (SL + C::GB - 1) / C::GB;  // iterations
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(qa + m0 * rowbytes, mrows * rowbytes);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sa + m0 * GS, mrows * GS * 4);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(qw + n0 * rowbytes, nrows * rowbytes);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(sw + n0 * GS, nrows * GS * 4);
  const __amdgpu_buffer_rsrc_t rza = make_rsrc(za + m0 * GS, ASYM ? mrows * GS * 4 : 0);
  const __amdgpu_buffer_rsrc_t rcw = make_rsrc(cw + n0 * GS, ASYM ? nrows * GS * 4 : 0);

  // staged A chunk j of this thread: row, chunk within the row slice
  auto a_row = [&](int j) { return (j * kSmallThreads + tid) / C::AROW; };
  auto a_chunk = [&](int j) { return (j * kSmallThreads + tid) % C::AROW; };

  // every load of iteration it (it >= NI: all out of range); staging loads first
  auto issue = [&](Stage& S, int64_t it) {
    const int64_t s0 = it * C::GB;        // first slice
    const int64_t c0 = s0 * C::H / C::P;  // first scale column
#pragma unroll
    for (int j = 0; j < C::SAR; ++j) {
      const int idx = j * kSmallThreads + tid;
      const int64_t col = c0 + idx % C::CW;
      const bool ok = idx < C::SAE && col < GS;
      S.sa[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rsa, int(ok ? uint32_t(((idx / C::CW) * GS + col) * 4) : kNoRead), 0, 0));
      if constexpr (ASYM)
        S.za[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rza, int(ok ? uint32_t(((idx / C::CW) * GS + col) * 4) : kNoRead), 0, 0));
    }
#pragma unroll
    for (int j = 0; j < C::SWR; ++j) {
      const int idx = j * kSmallThreads + tid;
      const int64_t col = c0 + idx % C::CW;
      const bool ok = idx < C::SWE && col < GS;
      S.sw[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rsw, int(ok ? uint32_t(((idx / C::CW) * GS + col) * 4) : kNoRead), 0, 0));
      if constexpr (ASYM)
        S.cw[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rcw, int(ok ? uint32_t(((idx / C::CW) * GS + col) * 4) : kNoRead), 0, 0));
    }
#pragma unroll
    for (int j = 0; j < C::AR; ++j) {
      const int64_t byte = s0 * 64 + a_chunk(j) * 16;
      S.a[j] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                           ra, int(byte < rowbytes ? uint32_t(a_row(j) * rowbytes + byte) : kNoRead),
                                           0, 0));
    }
#pragma unroll
    for (int ns = 0; ns < C::NS; ++ns) {
      const int64_t sl = s0 + wave * C::NS + ns;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        S.b[ct][ns] = __builtin_bit_cast(
            v4u, __builtin_amdgcn_raw_buffer_load_b128(
                     rb, int(sl < SL ? uint32_t((ct * 16 + am) * rowbytes + sl * 64 + part * 16) : kNoRead), 0, 0));
    }
  };
  auto store = [&](const Stage& S) {
#pragma unroll
    for (int j = 0; j < C::SAR; ++j) {
      const int idx = j * kSmallThreads + tid;
      saT[idx < C::SAE ? (idx % C::CW) * (16 * MT) + idx / C::CW : idx] = S.sa[j];
      if constexpr (ASYM) zaT[idx < C::SAE ? (idx % C::CW) * (16 * MT) + idx / C::CW : idx] = S.za[j];
    }
#pragma unroll
    for (int j = 0; j < C::SWR; ++j) {
      const int idx = j * kSmallThreads + tid;
      swT[idx < C::SWE ? (idx % C::CW) * (16 * CT) + idx / C::CW : idx] = S.sw[j];
      if constexpr (ASYM) cwT[idx < C::SWE ? (idx % C::CW) * (16 * CT) + idx / C::CW : idx] = S.cw[j];
    }
#pragma unroll
    for (int j = 0; j < C::AR; ++j) As[a_row(j) * (C::AROW + 1) + a_chunk(j)] = S.a[j];
  };

  float yv[CT][MT][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) yv[ct][mt][r] = 0.0f;

  // y += acc * (sa * sw) of local scale column cl
  auto apply = [&](int ct, int mt, const v4f& acc, int cl) {
    const v4f s4 = *reinterpret_cast<const v4f*>(saT + cl * (16 * MT) + mt * 16 + part * 4);
    const float swv = swT[cl * (16 * CT) + ct * 16 + am];
#pragma unroll
    for (int r = 0; r < 4; ++r) yv[ct][mt][r] = fmaf(acc[r], s4[r] * swv, yv[ct][mt][r]);
  };
  auto a_frag = [&](int mt, int gl) {
    const v4u w = As[(mt * 16 + am) * (C::AROW + 1) + gl * 4 + part];
    return ASYM ? f6_operand<false>(w) : f6_operand(w);
  };
  // ASYM: the product of tile (ct, mt) in scale column cl starts at -za cw
  auto acc_init = [&](int ct, int mt, int cl) {
    if constexpr (!ASYM) return v4f{};
    const v4f z4 = *reinterpret_cast<const v4f*>(zaT + cl * (16 * MT) + mt * 16 + part * 4);
    const float c = cwT[cl * (16 * CT) + ct * 16 + am];
    return v4f{-z4[0] * c, -z4[1] * c, -z4[2] * c, -z4[3] * c};
  };
  auto compute = [&](const Stage& S) {
#pragma unroll
    for (int ns = 0; ns < C::NS; ns += C::P) {
      const int gl = wave * C::NS + ns;  // local slice
      v8i b[C::P][CT];
#pragma unroll
      for (int p = 0; p < C::P; ++p)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) b[p][ct] = f6_operand(S.b[ct][ns + p]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (GSZ == 64) {
          const v8i a = a_frag(mt, gl);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const v8i ah = (part >> 1) == h ? a : v8i{};
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
              apply(ct, mt,
                    __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ah, b[0][ct], v4f{}, kF6, kF6, 0, kF6Scale, 0,
                                                                     kF6Scale),
                    2 * gl + h);
          }
        } else {
          v8i a[C::P];
#pragma unroll
          for (int p = 0; p < C::P; ++p) a[p] = a_frag(mt, gl + p);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[0], b[0][ct], acc_init(ct, mt, gl / C::P),
                                                                       kF6, kF6, 0, kF6Scale, 0, kF6Scale);
            if constexpr (C::P == 2)
              acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[1], b[1][ct], acc, kF6, kF6, 0, kF6Scale, 0,
                                                                     kF6Scale);
            apply(ct, mt, acc, gl / C::P);
          }
        }
      }
    }
  };
  // one iteration: stage cur into LDS, issue the next iteration into nxt,
  // compute cur.  With 32 channels per block (CT = 2, several blocks per CU)
  // the barriers wait for LDS only, so nxt's loads stay in flight across
  // them (-11 % at 1 x 4096 x 14336); with one block per CU (CT = 1) the
  // draining __syncthreads() measured faster (5.2 against 5.6 us at
  // 1 x 4096 x 4096, 8.1 against 9.3 us at 64 x 4096 x 4096), also with a
  // third register stage.
  auto block_sync = [] {
    if constexpr (CT == 2)
      lds_barrier();
    else
      __syncthreads();
  };
  auto step = [&](Stage& cur, Stage& nxt, int64_t it) {
    store(cur);
    block_sync();
    issue(nxt, it + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(cur);
    block_sync();  // LDS free for the next store
  };

  Stage s0, s1;
  issue(s0, 0);
  __builtin_amdgcn_sched_barrier(0);
  for (int64_t it = 0; it < NI; it += 2) {
    step(s0, s1, it);
    if (it + 1 >= NI) break;
    step(s1, s0, it + 1);
  }

  float* const red = reinterpret_cast<float*>(lds);  // [wave][tile][lane][4]
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<v4f*>(red + ((wave * CT * MT + ct * MT + mt) * 64 + lane) * 4) =
          v4f{yv[ct][mt][0], yv[ct][mt][1], yv[ct][mt][2], yv[ct][mt][3]};
  __syncthreads();
  if (wave < CT * MT) {  // wave t adds up output tile t over the waves
    const int ct = wave / MT, mt = wave % MT;
    v4f v = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) v += *reinterpret_cast<const v4f*>(red + ((w * CT * MT + wave) * 64 + lane) * 4);
    const int64_t bn = n0 + ct * 16 + am;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = mt * 16 + part * 4 + r;
      if (m < mrows && bn < N) store_y<BF16>(y, ldy, m0 + m, bn, v[r]);
    }
  }
}

// ---------------------------------------------------------------------------
// decode_fused_kernel: quantize_act + w4a4_gemm of a decode-sized step
// (M <= 16 rows, block-128 Hadamard, 128-wide groups) in one launch (the
// independent-rotation article, section 3.2, fuses rotate, scale and
// quantize into one kernel; the QuIP#/QTIP page, section 6.1, precomputes
// fused kernels against launch latency).  It is gemm_small_kernel (MT = 1)
// with the activation side produced in place: in every K-iteration, each
// wave transforms and quantizes the M rows of exactly the two 128-channel
// slices its own MFMAs consume, straight into its part of the LDS A tile
// and scale column (no other wave reads them), while the block's weights
// stream in.  A pass of the quantizer takes four (slice, row) pairs, one
// per 16-lane DPP row, so a single row costs one pass for both slices.
// The activations of the next iteration are loaded during the current one.
// The transform and encoder are quant_h128_act's and the products and their
// order gemm_small_kernel's, so y equals quantize_act followed by
// w4a4_gemm.  PS: quantizer passes (2 M <= 4 PS); SG: random signs.
// ---------------------------------------------------------------------------
template <bool XBF16, int PS, bool SG>
struct FusedX {
  static constexpr int XW = XBF16 ? 1 : 2;  // 16-byte words per lane and pass
  v4u x[PS][XW];                            // pass p: pair 4 p + lane / 16, channels 8 (lane % 16) ..
  v4u sm[SG ? 2 : 1][2];                    // random signs of those channels in slices 0 and 1
};

template <bool BF16, int CT, bool XBF16, int PS, bool SG>
__global__ __launch_bounds__(kSmallThreads) void decode_fused_kernel(
    const void* __restrict__ x, int64_t ldx, const uint32_t* __restrict__ sign_mask, float post,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw, int64_t M, int64_t N, int64_t K,
    void* __restrict__ y, int64_t ldy) {
  constexpr int MT = 1, GSZ = 128;
  using C = SmallCfg<GSZ, MT, CT>;
  using Stage = SmallStage<GSZ, MT, CT>;
  using X = FusedX<XBF16, PS, SG>;
  static_assert(C::NS == 2, "two slices per wave and iteration");
  constexpr int ES = XBF16 ? 2 : 4;
  __shared__ __align__(16) uint8_t lds[C::BYTES];
  v4u* const As = reinterpret_cast<v4u*>(lds);
  uint8_t* const Ab = lds;
  float* const saT = reinterpret_cast<float*>(lds + C::SA_OFF);
  float* const swT = reinterpret_cast<float*>(lds + C::SW_OFF);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int am = lane & 15;
  const int part = lane >> 4;
  const int sub = lane & 15;
  const int64_t SL = K / kGroup;
  const int64_t GS = SL;
  const int64_t rowbytes = K / 2;
  const int64_t n0 = int64_t(blockIdx.x) * 16 * CT;
  const int64_t nrows = N - n0 < 16 * CT ? N - n0 : 16 * CT;
  const int64_t NI = (SL + C::GB - 1) / C::GB;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(qw + n0 * rowbytes, nrows * rowbytes);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(sw + n0 * GS, nrows * GS * 4);
  // rows 0..M-1 of pitch ldx (the host checks the range < 2^31 bytes)
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, ((M - 1) * ldx + K) * ES);
  const __amdgpu_buffer_rsrc_t rsm = make_rsrc(sign_mask, SG ? K * 4 : 0);

  // the weight side of iteration it: weights and their scales
  auto issue_b = [&](Stage& S, int64_t it) __attribute__((always_inline)) {
    const int64_t s0 = it * C::GB;
#pragma unroll
    for (int j = 0; j < C::SWR; ++j) {
      const int idx = j * kSmallThreads + tid;
      const int64_t col = s0 + idx % C::CW;
      const bool ok = idx < C::SWE && col < GS;
      S.sw[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rsw, int(ok ? uint32_t(((idx / C::CW) * GS + col) * 4) : kNoRead), 0, 0));
    }
#pragma unroll
    for (int ns = 0; ns < C::NS; ++ns) {
      const int64_t sl = s0 + wave * C::NS + ns;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        S.b[ct][ns] = __builtin_bit_cast(
            v4u, __builtin_amdgcn_raw_buffer_load_b128(
                     rb, int(sl < SL ? uint32_t((ct * 16 + am) * rowbytes + sl * 64 + part * 16) : kNoRead), 0, 0));
    }
  };
  auto store_b = [&](const Stage& S) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < C::SWR; ++j) {
      const int idx = j * kSmallThreads + tid;
      swT[idx < C::SWE ? (idx % C::CW) * (16 * CT) + idx / C::CW : idx] = S.sw[j];
    }
  };

  // the activation side of iteration it for this wave: pair q = 4 p + part
  // of pass p is (slice 2 wave + q % 2, row q / 2); rows past M read zeros
  // (past the buffer range), slices past K too
  X xs;
  auto issue_x = [&](int64_t it) __attribute__((always_inline)) {
    const int64_t g0 = it * C::GB + wave * C::NS;
#pragma unroll
    for (int p = 0; p < PS; ++p) {
      const int q = 4 * p + part;
      const int64_t g = g0 + (q & 1);
      const int64_t row = q >> 1;
      const uint32_t off = g < SL && row < M ? uint32_t((row * ldx + g * kGroup + sub * 8) * ES) : kNoRead;
#pragma unroll
      for (int i = 0; i < X::XW; ++i)
        xs.x[p][i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rx, int(off + 16 * i), 0, 0));
    }
    if constexpr (SG) {
#pragma unroll
      for (int ns = 0; ns < 2; ++ns) {
        const int64_t g = g0 + ns;
        const uint32_t off = g < SL ? uint32_t((g * kGroup + sub * 8) * 4) : kNoRead;
#pragma unroll
        for (int i = 0; i < 2; ++i)
          xs.sm[ns][i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rsm, int(off + 16 * i), 0, 0));
      }
    }
  };

  const int word = h128_lane_word(sub);
  const float c1 = parity_sign(lane & 5), c2 = parity_sign(lane & 6);
  const float c7 = parity_sign(lane & 4), c8 = parity_sign(lane & 8);
  const float flip = parity_sign(lane & 15);
  const float s7 = signed_const(1.0f / 7.0f, flip);  // the encoder's signed 1/7
  auto quantize = [&](int64_t it) __attribute__((always_inline)) {
    const int64_t g0 = it * C::GB + wave * C::NS;
    // slices past K: zero codes and scales (gemm_small_kernel's loads read zeros there)
#pragma unroll
    for (int ns = 0; ns < C::NS; ++ns) {
      if (g0 + ns >= SL) {
        const int gl = wave * C::NS + ns;
        for (int64_t m = 0; m < M; ++m) Ab[gl * 64 + m * (C::AROW + 1) * 16 + lane] = 0;
        if (lane < 16) saT[gl * 16 + lane] = 0.0f;
      }
    }
    auto load_v = [&](int p, float (&v)[8]) __attribute__((always_inline)) {
      if constexpr (XBF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = bf16_lo(xs.x[p][0][e]);
          v[2 * e + 1] = bf16_hi(xs.x[p][0][e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(xs.x[p][e >> 2][e & 3]);
      }
      if constexpr (SG) {
        const int ns = (4 * p + part) & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[e] = __uint_as_float(__float_as_uint(v[e]) ^ (ns ? xs.sm[1][e >> 2][e & 3] : xs.sm[0][e >> 2][e & 3]));
      }
      fwht8(v);
    };
    auto finish = [&](int p, float (&v)[8], float mx) __attribute__((always_inline)) {
      const int q = 4 * p + part;
      const int ns = q & 1;
      const int64_t m = q >> 1;
      const int gl = wave * C::NS + ns;
      const uint32_t packed = encode8_rcp(v, mx, s7, (word & 2) != 0);
      if (m < M && g0 + ns < SL) {
        *reinterpret_cast<uint32_t*>(Ab + gl * 64 + m * (C::AROW + 1) * 16 + word * 4) = packed;
        if (sub == 0) saT[gl * 16 + m] = mx * post;
      }
    };
    auto absmax8 = [](const float (&v)[8]) {
      float mx = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
      return mx;
    };
#pragma unroll
    for (int p = 0; p < PS; ++p) {
      if (2 * M <= 4 * p) break;
      float v[8];
      load_v(p, v);
      lane_stages_dpp(v, c1, c2, c7, c8);
      finish(p, v, row16_max_dpp(absmax8(v)));
    }
  };

  float yv[CT][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) yv[ct][r] = 0.0f;
  auto compute = [&](const Stage& S) __attribute__((always_inline)) {
#pragma unroll
    for (int ns = 0; ns < C::NS; ++ns) {
      const int gl = wave * C::NS + ns;
      v8i b[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) b[ct] = f6_operand(S.b[ct][ns]);
      const v8i a = f6_operand(As[am * (C::AROW + 1) + gl * 4 + part]);
      const v4f s4 = *reinterpret_cast<const v4f*>(saT + gl * 16 + part * 4);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const v4f acc =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[ct], v4f{}, kF6, kF6, 0, kF6Scale, 0, kF6Scale);
        const float swv = swT[gl * (16 * CT) + ct * 16 + am];
#pragma unroll
        for (int r = 0; r < 4; ++r) yv[ct][r] = fmaf(acc[r], s4[r] * swv, yv[ct][r]);
      }
    }
  };
  // one iteration: the next weights are requested, this iteration's
  // activations (loaded one iteration ago) are quantized into LDS, the next
  // activations requested, then the MFMAs (barriers as in gemm_small_kernel)
  auto block_sync = [] {
    if constexpr (CT == 2)
      lds_barrier();
    else
      __syncthreads();
  };
  auto step = [&](Stage& cur, Stage& nxt, int64_t it) __attribute__((always_inline)) {
    issue_b(nxt, it + 1);
    quantize(it);
    issue_x(it + 1);
    store_b(cur);
    block_sync();
    compute(cur);
    block_sync();  // LDS free for the next iteration
  };
  Stage s0, s1;
  issue_x(0);
  issue_b(s0, 0);
  for (int64_t it = 0; it < NI; it += 2) {
    step(s0, s1, it);
    if (it + 1 >= NI) break;
    step(s1, s0, it + 1);
  }
  float* const red = reinterpret_cast<float*>(lds);  // [wave][tile][lane][4]
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
    *reinterpret_cast<v4f*>(red + ((wave * CT + ct) * 64 + lane) * 4) = v4f{yv[ct][0], yv[ct][1], yv[ct][2], yv[ct][3]};
  __syncthreads();
  if (wave < CT) {  // wave t adds up output tile t over the waves
    const int ct = wave;
    v4f v = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) v += *reinterpret_cast<const v4f*>(red + ((w * CT + ct) * 64 + lane) * 4);
    const int64_t bn = n0 + ct * 16 + am;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = part * 4 + r;
      if (m < M && bn < N) store_y<BF16>(y, ldy, m, bn, v[r]);
    }
  }
}

hipError_t launch_decode_fused(const void* x, bool x_bf16, int64_t ldx, const uint32_t* sign_mask, float post,
                               const uint8_t* qw, const float* sw, int64_t M, int64_t N, int64_t K, void* y,
                               bool y_bf16, int64_t ldy, hipStream_t st) {
  const bool ct2 = N > 12288;  // the channel tiling of gemm_small_kernel for M <= 16
  const int64_t blocks = (N + (ct2 ? 31 : 15)) / (ct2 ? 32 : 16);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  auto run = [&](auto yb, auto ct, auto xb, auto mp, auto sg) {
    hipLaunchKernelGGL((decode_fused_kernel<decltype(yb)::value, decltype(ct)::value, decltype(xb)::value,
                                            decltype(mp)::value, decltype(sg)::value>),
                       dim3(unsigned(blocks)), dim3(kSmallThreads), 0, st, x, ldx, sign_mask, post, qw, sw, M, N, K,
                       y, ldy);
    return hipGetLastError();
  };
  using T = std::true_type;
  using F = std::false_type;
  auto by_sg = [&](auto yb, auto ct, auto xb, auto mp) { return sign_mask ? run(yb, ct, xb, mp, T{}) : run(yb, ct, xb, mp, F{}); };
  auto by_mp = [&](auto yb, auto ct, auto xb) {
    if (M <= 2) return by_sg(yb, ct, xb, std::integral_constant<int, 1>{});
    if (M <= 4) return by_sg(yb, ct, xb, std::integral_constant<int, 2>{});
    if (M <= 8) return by_sg(yb, ct, xb, std::integral_constant<int, 4>{});
    return by_sg(yb, ct, xb, std::integral_constant<int, 8>{});
  };
  auto by_x = [&](auto yb, auto ct) { return x_bf16 ? by_mp(yb, ct, T{}) : by_mp(yb, ct, F{}); };
  auto by_ct = [&](auto yb) {
    return ct2 ? by_x(yb, std::integral_constant<int, 2>{}) : by_x(yb, std::integral_constant<int, 1>{});
  };
  return y_bf16 ? by_ct(T{}) : by_ct(F{});
}

// Which kernel runs a product.  The tiled kernel gives one 128 x 128 tile per
// block; below about one block per CU its time is one block's K loop (about
// 30 us at K = 4096 for any M up to 1024 at N = 4096, measured), while the
// small-M kernel, run over 64-row chunks of A in one launch, streams the
// whole product at about 600 TOPS.  With ~4.5 TOPS per busy CU for the tiled
// kernel, the small kernel wins while the tiled grid has fewer than 128 blocks
// (measured crossover at N = 4096: M = 512, small 29.8 us against 31.2 us).
constexpr int64_t kSmallMaxM = 1024;
constexpr int64_t kTiledMinBlocks = 128;
__host__ __forceinline__ bool use_small_kernel(int64_t M, int64_t N) {
  if (M <= 64) return true;
  return M <= kSmallMaxM && ((M + 127) / 128) * ((N + 127) / 128) < kTiledMinBlocks;
}

template <int GSZ>
hipError_t launch_gemm_g(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                         int64_t M, int64_t N, int64_t K, void* y, bool y_bf16, int64_t ldy,
                         hipStream_t st) {
  if (use_small_kernel(M, N)) {  // 16 CT output channels per block, the rows in chunks of 16 MT (grid y)
    auto run = [&](auto mt_const, auto ct_const) {
      constexpr int MT = decltype(mt_const)::value, CT = decltype(ct_const)::value;
      const int64_t blocks = (N + 16 * CT - 1) / (16 * CT);
      const int64_t chunks = (M + 16 * MT - 1) / (16 * MT);
      if (blocks > 0x7FFFFFFF || chunks > 65535) return hipErrorInvalidValue;
      const dim3 grid{unsigned(blocks), unsigned(chunks), 1u};
      if (y_bf16)
        hipLaunchKernelGGL((gemm_small_kernel<true, GSZ, MT, CT>), grid, dim3(kSmallThreads), 0, st, qa, sa, qw,
                           sw, M, N, K, y, ldy);
      else
        hipLaunchKernelGGL((gemm_small_kernel<false, GSZ, MT, CT>), grid, dim3(kSmallThreads), 0, st, qa, sa, qw,
                           sw, M, N, K, y, ldy);
      return hipGetLastError();
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (M <= 16) return N > 12288 ? run(I1{}, I2{}) : run(I1{}, I1{});  // past 3 blocks per CU: 32 channels
    if (M <= 32) return run(I2{}, I1{});
    return run(std::integral_constant<int, 4>{}, I1{});
  }
  // per-block buffer ranges: 128 rows of K / 2 bytes, 128 rows of K / 128 scales
  if (K > (int64_t(1) << 24)) return hipErrorInvalidValue;
  const int64_t tiles_m = (M + 127) / 128, tiles_n = (N + 127) / 128;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if constexpr (GSZ == 128) {
    if (y_bf16)
      hipLaunchKernelGGL((gemm_f8p_kernel<true>), dim3(blocks), dim3(256), 0, st, qa, sa, qw, sw, M, N, K, y,
                         ldy, tiles_m);
    else
      hipLaunchKernelGGL((gemm_f8p_kernel<false>), dim3(blocks), dim3(256), 0, st, qa, sa, qw, sw, M, N, K, y,
                         ldy, tiles_m);
    return hipGetLastError();
  }
  if (y_bf16)
    hipLaunchKernelGGL((gemm_f8_kernel<true, GSZ>), dim3(blocks), dim3(256), 0, st, qa, sa, qw, sw, M, N,
                       K, y, ldy, tiles_m);
  else
    hipLaunchKernelGGL((gemm_f8_kernel<false, GSZ>), dim3(blocks), dim3(256), 0, st, qa, sa, qw, sw, M, N,
                       K, y, ldy, tiles_m);
  return hipGetLastError();
}

hipError_t launch_gemm_asym(const uint8_t* qa, const float* sa, const float* za, const uint8_t* qw, const float* sw,
                            const float* cw, int64_t M, int64_t N, int64_t K, void* y, bool y_bf16, int64_t ldy,
                            hipStream_t st) {
  if (use_small_kernel(M, N)) {
    auto run = [&](auto mt_const, auto ct_const) {
      constexpr int MT = decltype(mt_const)::value, CT = decltype(ct_const)::value;
      const int64_t blocks = (N + 16 * CT - 1) / (16 * CT);
      const int64_t chunks = (M + 16 * MT - 1) / (16 * MT);
      if (blocks > 0x7FFFFFFF || chunks > 65535) return hipErrorInvalidValue;
      const dim3 grid{unsigned(blocks), unsigned(chunks), 1u};
      if (y_bf16)
        hipLaunchKernelGGL((gemm_small_kernel<true, 128, MT, CT, true>), grid, dim3(kSmallThreads), 0, st, qa, sa,
                           qw, sw, M, N, K, y, ldy, za, cw);
      else
        hipLaunchKernelGGL((gemm_small_kernel<false, 128, MT, CT, true>), grid, dim3(kSmallThreads), 0, st, qa, sa,
                           qw, sw, M, N, K, y, ldy, za, cw);
      return hipGetLastError();
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (M <= 16) return N > 12288 ? run(I1{}, I2{}) : run(I1{}, I1{});
    if (M <= 32) return run(I2{}, I1{});
    return run(std::integral_constant<int, 4>{}, I1{});
  }
  if (K > (int64_t(1) << 24)) return hipErrorInvalidValue;
  const int64_t tiles_m = (M + 127) / 128, tiles_n = (N + 127) / 128;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (y_bf16)
    hipLaunchKernelGGL((gemm_f8p_kernel<true, true>), dim3(blocks), dim3(256), 0, st, qa, sa, qw, sw, M, N, K, y, ldy,
                       tiles_m, za, cw);
  else
    hipLaunchKernelGGL((gemm_f8p_kernel<false, true>), dim3(blocks), dim3(256), 0, st, qa, sa, qw, sw, M, N, K, y,
                       ldy, tiles_m, za, cw);
  return hipGetLastError();
}

// group: 64, 128 or 256 (K a multiple of 128 and of it, checked by the caller)
hipError_t launch_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                       int64_t M, int64_t N, int64_t K, int group, void* y, bool y_bf16, int64_t ldy,
                       hipStream_t st) {
  if (group == 256) return launch_gemm_g<256>(qa, sa, qw, sw, M, N, K, y, y_bf16, ldy, st);
  if (group == 128) return launch_gemm_g<128>(qa, sa, qw, sw, M, N, K, y, y_bf16, ldy, st);
  if (group == 64) return launch_gemm_g<64>(qa, sa, qw, sw, M, N, K, y, y_bf16, ldy, st);
  return hipErrorInvalidValue;
}

}  // namespace rw4
