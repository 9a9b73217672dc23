// Device helpers shared by the gfx950 kernels of the MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace moe {

typedef _Float16 f16;
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint2v __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 32;  // weights per quantisation block
constexpr int kMaxTopKLds = 32;  // top-k entries a wave can rank (the library's largest k)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even fp32 -> bf16 (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return uint16_t(u >> 16);
}

__device__ __forceinline__ float load_act(const float* p) { return *p; }
__device__ __forceinline__ float load_act(const uint16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ uint32_t pack_half2(f16 lo, f16 hi) {
  return uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
}

__device__ __forceinline__ half2v as_half2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t as_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// Wave-level reductions (wave64) through cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// 16x16x32 fp16 MFMA, fp32 accumulate.  Operand lane layout (gfx950):
//   A: lane l holds A[m = l%16][k = 8*(l/16) .. +7]
//   B: lane l holds B[k = 8*(l/16) .. +7][n = l%16]
//   D: lane l holds D[m = 4*(l/16) + j][n = l%16], j = 0..3
__device__ __forceinline__ float4v mfma16(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 32x32x16 fp16 MFMA, fp32 accumulate.  Operand lane layout (gfx950):
//   A: lane l holds A[m = l%32][k = 8*(l/32) .. +7]
//   B: lane l holds B[k = 8*(l/32) .. +7][n = l%32]
//   D: lane l holds D[m = 8*(j/4) + 4*(l/32) + j%4][n = l%32], j = 0..15
__device__ __forceinline__ float16v mfma32(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float16v mfma32_bf16(bf16x8 a, bf16x8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Tiled storage of one quantised matrix [rows][K] (K a multiple of 32).
// Rows go in groups of 16 (the last group of a matrix may be shorter);
// within a group the K axis is cut into units of 64 weights (two 32-weight
// blocks), and one unit of the whole group is contiguous, row after row:
//   low code plane (2 bits per weight): 16 bytes per row and unit,
//   scales (fp16, one per block):        4 bytes per row and unit,
//   3-bit high plane (1 bit per weight):  8 bytes per row and unit, each
//                                        block's word rearranged by
//                                        qt_high3_word.
// When K % 64 == 32 the last unit of a group holds one block (8, 2 and 4
// bytes per row).  A group occupies the bytes its rows take in row-major
// order, so buffer sizes, the offset of the high plane (rows * K / 4 bytes)
// and per-expert strides are those of the row-major layout; only the order
// within a group differs.  A wave that reads one unit of 16 rows (the GEMV
// and GEMM weight loads) then reads one 256-byte piece of codes instead of 16
// separate 16-byte pieces.  Within a block the bits are as in row-major
// storage: weight i of the block at bits 2i (low plane) and bit i (high).
// ---------------------------------------------------------------------------
struct QTile {
  int64_t g0;  // first row of the row's group
  int gsz;     // rows in the group
  int rr;      // row within the group
};

// rows = rows of the matrix; FULL: every group has 16 rows (rows % 16 == 0).
template <bool FULL>
__host__ __device__ __forceinline__ QTile qtile(int64_t row, int64_t rows) {
  QTile t;
  t.g0 = row & ~int64_t(15);
  t.gsz = FULL ? 16 : int(rows - t.g0 < 16 ? rows - t.g0 : 16);
  t.rr = int(row - t.g0);
  return t;
}

// Byte offset (in the low plane) of the 8 code bytes of block blk.
__host__ __device__ __forceinline__ int64_t qt_code_off(const QTile& t, int K, int blk) {
  const int nuf = K / 64, u = blk >> 1;
  const int64_t base = t.g0 * (K / 4);
  return u < nuf ? base + int64_t(u) * t.gsz * 16 + t.rr * 16 + (blk & 1) * 8
                 : base + int64_t(nuf) * t.gsz * 16 + t.rr * 8;
}

// Offset (in fp16 elements) of the scale of block blk.
__host__ __device__ __forceinline__ int64_t qt_scale_off(const QTile& t, int K, int blk) {
  const int nuf = K / 64, u = blk >> 1;
  const int64_t base = t.g0 * (K / 32);
  return u < nuf ? base + int64_t(u) * t.gsz * 2 + t.rr * 2 + (blk & 1) : base + int64_t(nuf) * t.gsz * 2 + t.rr;
}

// (4-bit: the high plane has the low plane's layout, so qt_code_off places
// its bytes too, from the plane's start.)
// Byte offset (in the 3-bit high plane) of the 4 high-plane bytes of block blk.
__host__ __device__ __forceinline__ int64_t qt_high_off(const QTile& t, int K, int blk) {
  const int nuf = K / 64, u = blk >> 1;
  const int64_t base = t.g0 * (K / 8);
  return u < nuf ? base + int64_t(u) * t.gsz * 8 + t.rr * 8 + (blk & 1) * 4
                 : base + int64_t(nuf) * t.gsz * 8 + t.rr * 4;
}

// ---------------------------------------------------------------------------
// Dequantisation of one 32-bit word of 2-bit codes into fp16 pairs.
//
// A word holds 16 codes, code i at bits 2i..2i+1.  Pair i (i = 0..7) is
// (code i, code i+8): low half from bits 2i, high half from bits 2i+16.
// For i <= 4 the code is OR-ed into the mantissa of the fp16 constant
// M_i = 2^(10-2i) whose unit in the last place is 4^-i, so the code lands
// with weight 1 and the half holds M_i + q exactly; subtracting M_i + 2
// leaves c = q - 2 exactly, and multiplying by the fp16 block scale gives
// c * s exactly (|c| <= 2).  Pairs 5..7 reuse M_0..M_2 on the word shifted
// right by 10.  Operand order within an MFMA k-slice therefore is
// k = {0,8,1,9,2,10,3,11} (first slice) and {4,12,5,13,6,14,7,15} (second);
// the activations are staged in LDS in the same order.
// ---------------------------------------------------------------------------

// d = (a & mask) | bits in one v_and_or_b32 (mask in a VGPR, bits in an SGPR:
// gfx9 VOP3 reads one scalar operand and no literal).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(mask), "s"(bits));
  return d;
}

// Same with every operand in VGPRs (for per-lane `bits`).
__device__ __forceinline__ uint32_t and_or_v(uint32_t a, uint32_t mask, uint32_t bits) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(mask), "v"(bits));
  return d;
}

__device__ __forceinline__ uint32_t magic_bits(int i) {
  // fp16 bit pattern of 2^(10-2i) in both halves
  const uint32_t e = uint32_t(25 - 2 * i) << 10;
  return e | (e << 16);
}
__device__ __forceinline__ f16 magic_val(int i) { return f16(float(1 << (10 - 2 * i))); }

// One word's dequantisation, split into a preparation (the shifted source
// words and the scale, once per word) and the 8 pairs (dq_pair: two or three
// VALU ops plus a packed subtract and multiply each), so that a caller can
// spread the pairs of one word between other work.  Pair i < NA takes its
// code bits from `a` (and `ha`), pair i >= NA from `b` (and `hb`), with
// M_{i} resp. M_{i - NA}.
struct DqSrc {
  uint32_t a, b;    // low two bits of the codes: the word and its shifted copy
  uint32_t ha, hb;  // 3-bit: bit 2 of the codes; 4-bit: bits 2..3; placed for pairs < NA and >= NA
  half2v s2;        // block scale in both halves
};

// 2-bit: pairs 0..4 from w, 5..7 from w >> 10.
__device__ __forceinline__ DqSrc dq2_src(uint32_t w, half2v s2) { return DqSrc{w, w >> 10, 0u, 0u, s2}; }

// 3-bit: w holds the low two bits of 16 codes (2-bit layout); hlo and hhi
// hold bit 2 of code i at bit 2i + 2 (pairs 0..3) and 2i - 6 (pairs 4..7),
// with bits on odd positions ignored (high3_slots).  Pairs 0..3 use M_0..M_3
// (bits up to 2i + 2 <= 8 stay inside the mantissa); pairs 4..7 use w >> 8
// with M_0..M_3.  c = q - 4; c * s rounds to fp16 for |c| = 3 (relative
// error <= 2^-11 per weight).
__device__ __forceinline__ DqSrc dq3_src(uint32_t w, uint32_t hlo, uint32_t hhi, half2v s2) {
  return DqSrc{w, w >> 8, hlo, hhi, s2};
}

// 4-bit: wl holds the low two bits of 16 codes and wh the high two bits, both
// in the 2-bit layout.  Pairs 0..3 use M_0..M_3 with the high bits moved to
// 2i+2 .. 2i+3 (wh << 2; bits up to 2i+3 <= 9 stay inside the mantissa, whose
// bit 2i has weight 1, so the half holds M_i + q, q <= 15); pairs 4..7 use
// wl >> 8 and wh >> 6 with M_0..M_3.  c = q - 8.  Bits that the shifts carry
// across the half boundary fall outside the masks.  Unlike the 2-bit case,
// c * s rounds to fp16 where |c| is not a power of two (as in the 3-bit
// case: relative error <= 2^-11 per weight).
__device__ __forceinline__ DqSrc dq4_src(uint32_t wl, uint32_t wh, half2v s2) {
  return DqSrc{wl, wl >> 8, wh << 2, wh >> 6, s2};
}

// Pair i (0..7) of a prepared word, (code i, code i + 8) as fp16 c * s, in
// dq_stages() dependent steps, so that a caller can interleave the steps of
// several pairs: step 0 starts the pair's work word t, the last leaves the
// fp16 pair in it.  Steps: [3-bit, 4-bit: high bits OR-ed into M_j], low bits
// OR-ed in, subtract M_j + 2^(QBITS-1), multiply by the scale.
template <int QBITS>
constexpr int dq_stages() { return QBITS == 2 ? 3 : 4; }

template <int QBITS>
__device__ __forceinline__ void dq_step(const DqSrc& d, int i, int k, uint32_t& t) {
  constexpr int NA = QBITS == 2 ? 5 : 4;
  constexpr int S = dq_stages<QBITS>();
  const int j = i < NA ? i : i - NA;
  const uint32_t src = i < NA ? d.a : d.b;
  if (k == S - 2) {
    const f16 off = magic_val(j) + f16(float(1 << (QBITS - 1)));
    t = as_u32(as_half2(t) - half2v{off, off});
  } else if (k == S - 1) {
    t = as_u32(as_half2(t) * d.s2);
  } else if constexpr (QBITS == 2) {
    t = and_or(src, 0x00030003u << (2 * j), magic_bits(j));
  } else if (k == 0) {
    constexpr uint32_t hmask = QBITS == 3 ? 0x00040004u : 0x000C000Cu;
    t = and_or(i < NA ? d.ha : d.hb, hmask << (2 * j), magic_bits(j));
  } else {
    t = and_or_v(src, 0x00030003u << (2 * j), t);
  }
}

template <int QBITS>
__device__ __forceinline__ half2v dq_pair(const DqSrc& d, int i) {
  uint32_t t = 0u;
#pragma unroll
  for (int k = 0; k < dq_stages<QBITS>(); ++k) dq_step<QBITS>(d, i, k, t);
  return as_half2(t);
}

// All 8 pairs of a prepared word into the two MFMA k-slices.
template <int QBITS>
__device__ __forceinline__ void dq_word(const DqSrc& d, half8& lo, half8& hi) {
  half2v p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = dq_pair<QBITS>(d, i);
  lo = half8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  hi = half8{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}

// Dequantise 2-bit word w (16 codes) with block scale s2 (scale in both
// halves) into two MFMA k-slices (8 fp16 each) in the permuted order.
__device__ __forceinline__ void dq2_word(uint32_t w, half2v s2, half8& lo, half8& hi) {
  dq_word<2>(dq2_src(w, s2), lo, hi);
}

// Spread the 16 bits of h to even bit positions: bit k -> bit 2k.
__host__ __device__ __forceinline__ uint32_t spread16(uint32_t h) {
  h &= 0xffffu;
  h = (h | (h << 8)) & 0x00ff00ffu;
  h = (h | (h << 4)) & 0x0f0f0f0fu;
  h = (h | (h << 2)) & 0x33333333u;
  h = (h | (h << 1)) & 0x55555555u;
  return h;
}

// The kernels' 3-bit high-plane word of a block: the block's 32 high bits
// (bit i = bit 2 of q for code i) rearranged once, at repack, so that bit i
// of codes 0..15 (the block's first 16-code word A) sits at bit 2i + 1 and
// bit i of codes 16..31 (word B) at bit 2i.  Shifted by a constant, the high
// bits of either word then line up with the fp16 mantissa slots of its pairs
// (dq3_src), with the other word's bits on odd positions outside the masks.
__host__ __device__ __forceinline__ uint32_t qt_high3_word(uint32_t h) {
  return (spread16(h & 0xffffu) << 1) | spread16(h >> 16);
}

// The high bits of 16-code word `second` (0 = A, 1 = B) of a block for
// dq3_src: bit 2 of code j at bit 2j + 2 (pairs 0..3, lo) and of code i at
// bit 2i - 6 (pairs 4..7, hi).
__device__ __forceinline__ void high3_slots(uint32_t hw, int second, uint32_t& lo, uint32_t& hi) {
  lo = second ? hw << 2 : hw << 1;
  hi = second ? hw >> 6 : hw >> 7;
}

__device__ __forceinline__ void dq3_word(uint32_t w, uint32_t hlo, uint32_t hhi, half2v s2, half8& lo, half8& hi) {
  dq_word<3>(dq3_src(w, hlo, hhi, s2), lo, hi);
}

__device__ __forceinline__ void dq4_word(uint32_t wl, uint32_t wh, half2v s2, half8& lo, half8& hi) {
  dq_word<4>(dq4_src(wl, wh, s2), lo, hi);
}

// Position of weight r (0..15) of a 16-weight group in the permuted order.
__host__ __device__ __forceinline__ int perm16(int r) { return r < 8 ? 2 * r : 2 * (r - 8) + 1; }

// Column position of h element i: the activations of the down projection are
// stored in the permuted 16-group order its MFMA operands use.
__device__ __forceinline__ int hcol(int i) { return (i & ~15) | perm16(i & 15); }

// 16 consecutive activations as loaded (bf16 or fp32), before conversion.
// Loading and converting are separate steps so that a batch of loads is in
// flight together: a conversion placed right after its load makes the wave
// wait for that load alone.
template <typename SRC>
struct Raw16 {
  uint4v q[sizeof(SRC) == 4 ? 4 : 2];
};

template <typename SRC>
__device__ __forceinline__ void load_raw16(const SRC* src, Raw16<SRC>& r) {
  const uint4v* p = reinterpret_cast<const uint4v*>(src);
#pragma unroll
  for (int i = 0; i < int(sizeof(r.q) / sizeof(r.q[0])); ++i) r.q[i] = p[i];
}

// -> the two permuted fp16 MFMA k-slices (lo = weights {0,8,1,9,2,10,3,11},
// hi = {4,12,5,13,6,14,7,15}).
template <typename SRC>
__device__ __forceinline__ void cvt_raw16(const Raw16<SRC>& r, half8& lo, half8& hi) {
  if constexpr (std::is_same<SRC, f16>::value) {  // already fp16: the permutation alone
    half8 a = __builtin_bit_cast(half8, r.q[0]), b = __builtin_bit_cast(half8, r.q[1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[2 * i] = a[i];
      lo[2 * i + 1] = b[i];
      hi[2 * i] = a[4 + i];
      hi[2 * i + 1] = b[4 + i];
    }
    return;
  }
  float v[16];
  if constexpr (sizeof(SRC) == 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < 4; ++u) v[4 * q + u] = __uint_as_float(r.q[q][u]);
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[8 * q + 2 * u] = __uint_as_float(r.q[q][u] << 16);
        v[8 * q + 2 * u + 1] = __uint_as_float(r.q[q][u] & 0xffff0000u);
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[2 * i] = f16(v[i]);
    lo[2 * i + 1] = f16(v[i + 8]);
    hi[2 * i] = f16(v[4 + i]);
    hi[2 * i + 1] = f16(v[12 + i]);
  }
}

template <typename SRC>
__device__ __forceinline__ void load_x16(const SRC* src, half8& lo, half8& hi) {
  Raw16<SRC> r;
  load_raw16(src, r);
  cvt_raw16(r, lo, hi);
}


// Exclusive scan over n <= 4096 ints held in LDS, 1024 threads.  Returns the
// total.  `tmp` has 1024 ints.
__device__ inline int block_exclusive_scan_lds(int* vals, int n, int* tmp) {
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;  // <= 4
  int local[4];
  int s = 0;
  for (int i = 0; i < per; ++i) {
    const int idx = tid * per + i;
    local[i] = idx < n ? vals[idx] : 0;
    s += local[i];
  }
  tmp[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += v;
    __syncthreads();
  }
  const int total = tmp[1023];
  int run = tmp[tid] - s;  // exclusive prefix of this thread's group
  __syncthreads();
  for (int i = 0; i < per; ++i) {
    const int idx = tid * per + i;
    if (idx < n) vals[idx] = run;
    run += local[i];
  }
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------------------
// DPP wave reductions (no LDS traffic).  Within each row of 16 lanes: xor 1
// and xor 2 through quad permutes, then rotations by 4 and 8; the four row
// results are combined from lanes 0, 16, 32, 48 with readlane, so the result
// is uniform across the wave.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xb1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4e>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x124>(v));  // row_ror:4
  v = max(v, dpp_u32<0x128>(v));  // row_ror:8
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0xb1>(v));
  v = min(v, dpp_u32<0x4e>(v));
  v = min(v, dpp_u32<0x124>(v));
  v = min(v, dpp_u32<0x128>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

// Order-preserving map of a finite float to an unsigned key (-0 folds to +0).
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over a wave (shuffle-up steps).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive scan of vals[0..n) in LDS by an NT-thread workgroup with two
// barriers: each wave scans a contiguous run, then the wave totals.  `tmp`
// holds NT / 64 ints.  Returns the total.  n <= 4 NT.
template <int NT = 1024>
__device__ inline int block_scan_fast(int* vals, int n, int* tmp) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int per = (n + NT - 1) / NT;  // values per thread, <= 4
  int local[4], s = 0;
  for (int i = 0; i < per; ++i) {
    const int idx = threadIdx.x * per + i;
    local[i] = idx < n ? vals[idx] : 0;
    s += local[i];
  }
  const int incl = wave_incl_scan(s);
  if (lane == 63) tmp[wv] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < NW; ++w) {
    const int t = tmp[w];
    base += w < wv ? t : 0;
    total += t;
  }
  int run = base + incl - s;
  for (int i = 0; i < per; ++i) {
    const int idx = threadIdx.x * per + i;
    if (idx < n) vals[idx] = run;
    run += local[i];
  }
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------------------
// Top-k of one token's logits on one wave, ties to the lower expert index,
// then the renormalised softmax weights of the selection.
// ---------------------------------------------------------------------------
// Inverse of float_key.
__device__ __forceinline__ float key_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Set bits of m below this lane.
__device__ __forceinline__ int bits_below(uint64_t m) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

// Lanes whose v >= t, as a mask in its own scalar register pair.  Written
// out so that the compares go to distinct registers and issue back to back
// (four per statement): compares through the shared VCC register, or each
// followed by its bit count, serialise on the vector-to-scalar latency.
__device__ __forceinline__ uint64_t ballot_ge(uint32_t v, uint32_t t) {
  uint64_t m;
  asm("v_cmp_le_u32_e64 %0, %1, %2" : "=s"(m) : "s"(t), "v"(v));
  return m;
}

__device__ __forceinline__ void ballot_ge4(const uint32_t* v, uint32_t t, uint64_t* m) {
  asm("v_cmp_le_u32_e64 %0, %4, %5\n\t"
      "v_cmp_le_u32_e64 %1, %4, %6\n\t"
      "v_cmp_le_u32_e64 %2, %4, %7\n\t"
      "v_cmp_le_u32_e64 %3, %4, %8"
      : "=&s"(m[0]), "=&s"(m[1]), "=&s"(m[2]), "=&s"(m[3])
      : "s"(t), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
}

// Number of keys >= t over the wave.
template <int V>
__device__ __forceinline__ int wave_count_ge(const uint32_t (&key)[V], uint32_t t) {
  uint64_t m[V];
  if constexpr (V % 4 == 0) {
#pragma unroll
    for (int v = 0; v < V; v += 4) ballot_ge4(key + v, t, m + v);
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) m[v] = ballot_ge(key[v], t);
  }
  int c = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) c += __builtin_popcountll(m[v]);
  return c;
}

// ---------------------------------------------------------------------------
// Top-k of one token's E logits on one wave: ranks ordered by (logit desc,
// expert index asc).  Lane l holds experts l + 64v (v < V) as
// order-preserving keys; 0 marks padding (every real key is >= 1).
// ---------------------------------------------------------------------------
template <int V>
struct WaveKeys {
  uint32_t key[V];
};

template <int V>
__device__ __forceinline__ void wave_keys(const float* __restrict__ row, int E, WaveKeys<V>& K) {
  const int lane = threadIdx.x & 63;
  float f[V];
#pragma unroll
  for (int v = 0; v < V; ++v) f[v] = row[min(lane + 64 * v, E - 1)];
  // Pin every load as unconditional, so the V loads are in flight together
  // (a load feeding only one side of a select is otherwise moved into a
  // branch with its own wait).
#pragma unroll
  for (int v = 0; v < V; ++v) asm volatile("" : "+v"(f[v]));
#pragma unroll
  for (int v = 0; v < V; ++v) K.key[v] = lane + 64 * v < E ? float_key(f[v]) : 0u;
}

// The selected set, as one lane mask per v: the k largest keys, ties at the
// k-th place going to the lowest expert indices.
//  1. The k-th largest key T by bisection, keeping count(>= lo) >= k and
//     count(>= hi + 1) < k with one ballot count per step; a cut point whose
//     count is exactly k ends it (the keys >= it are the top-k).  The search
//     starts at hi = the largest key and lo = the smallest maximum over 64/G
//     disjoint groups of G lanes, G the largest power of two with 64/G >= k
//     (at least 64/G >= k keys are >= lo).
//  2. Keys > T, then the lowest-index keys == T up to k.
template <int V>
__device__ __forceinline__ void wave_select(const WaveKeys<V>& K, int k, uint64_t (&msel)[V]) {
  const int lane = threadIdx.x & 63;
  uint32_t bk = K.key[0];
#pragma unroll
  for (int v = 1; v < V; ++v) bk = max(bk, K.key[v]);
  // group maxima: G lanes per group through the same DPP steps as wave_max_u32
  const int G = k <= 2 ? 32 : k <= 4 ? 16 : k <= 8 ? 8 : k <= 16 ? 4 : 2;  // k <= 32
  uint32_t gm = bk;
  if (G >= 2) gm = max(gm, dpp_u32<0xb1>(gm));   // quad_perm [1,0,3,2]: pairs
  if (G >= 4) gm = max(gm, dpp_u32<0x4e>(gm));   // quad_perm [2,3,0,1]: quads
  if (G >= 8) gm = max(gm, dpp_u32<0x124>(gm));  // row_ror:4: lanes 8i hold 8-lane groups
  if (G >= 16) gm = max(gm, dpp_u32<0x128>(gm)); // row_ror:8: lanes 16i hold rows
  uint32_t hi = wave_max_u32(bk);
  // k <= 2 (G >= 32): no group step; the search starts from the whole key range
  uint32_t lo = G >= 32 ? 1u : max(wave_min_u32(lane % G == 0 ? gm : 0xffffffffu), 1u);
  bool exact = false;
  while (lo < hi) {
    // cut at the midpoint of the logit values (a few steps cover the span
    // of the logits); when that does not split the key range, at the
    // midpoint of the keys (exact termination whatever the values)
    uint32_t mid = float_key(0.5f * key_float(lo) + 0.5f * key_float(hi));
    if (mid <= lo || mid > hi) mid = lo + (hi - lo + 1u) / 2u;
    const int c = wave_count_ge<V>(K.key, mid);
    if (c == k) {
      lo = mid;
      exact = true;
      break;
    }
    if (c > k) lo = mid;
    else hi = mid - 1u;
  }
  if (exact) {
    if constexpr (V % 4 == 0) {
#pragma unroll
      for (int v = 0; v < V; v += 4) ballot_ge4(K.key + v, lo, msel + v);
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) msel[v] = ballot_ge(K.key[v], lo);
    }
  } else {
    const int need = k - wave_count_ge<V>(K.key, lo + 1u);  // keys == lo to take, lowest index first
    int before = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const uint64_t eq = __ballot(K.key[v] == lo);
      msel[v] = __ballot(K.key[v] > lo || (K.key[v] == lo && before + bits_below(eq) < need));
      before += __builtin_popcountll(eq);
    }
  }
}

// Expert index of the n-th selected expert in index order (wave-uniform):
// the v holding it from the mask counts (scalar), then its lane from one
// ballot.
template <int V>
__device__ __forceinline__ int wave_nth_selected(const uint64_t (&msel)[V], int n) {
  const int lane = threadIdx.x & 63;
  int pre = 0, vs = 0, r = 0;
  uint64_t ms = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int c = __builtin_popcountll(msel[v]);
    const bool here = n >= pre && n < pre + c;
    vs = here ? v : vs;
    r = here ? n - pre : r;
    ms = here ? msel[v] : ms;
    pre += c;
  }
  const uint64_t hit = __ballot(((ms >> lane) & 1ull) && bits_below(ms) == r);
  return 64 * vs + int(__builtin_ctzll(hit));
}

// Ranks of the selection.  The k selected go to this wave's LDS slots in
// index order, each is ranked by counting the entries above it (larger key,
// or equal key and lower index), and lane j < k returns the rank-j expert,
// its logit (a -0 logit comes back as +0, which changes no weight) and its
// position in index order.
// tk: this wave's LDS scratch (index order / rank order).
template <int V>
__device__ __forceinline__ void wave_rank_s(const WaveKeys<V>& K, const uint64_t (&msel)[V], int k,
                                            uint2 (&tk)[2][kMaxTopKLds], float& my_val, int& my_idx,
                                            int& my_slot) {
  const int lane = threadIdx.x & 63;
  int base = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const uint64_t m = msel[v];
    if ((m >> lane) & 1ull) tk[0][base + bits_below(m)] = uint2{K.key[v], uint32_t(lane + 64 * v)};
    base += __builtin_popcountll(m);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < k) {
    const uint2 me = tk[0][lane];
    int rank = 0;
    for (int i = 0; i < k; ++i) {
      const uint2 o = tk[0][i];
      rank += (o.x > me.x || (o.x == me.x && i < lane)) ? 1 : 0;
    }
    tk[1][rank] = uint2{me.x, me.y | (uint32_t(lane) << 16)};  // expert < 2^16, slot in the high half
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint2 out = uint2{0u, 0u};
  if (lane < k) out = tk[1][lane];
  my_val = key_float(out.x);
  my_idx = int(out.y & 0xffffu);
  my_slot = int(out.y >> 16);
}

// The same with a scratch of the workgroup's (at most 16) waves.
template <int V>
__device__ __forceinline__ void wave_rank(const WaveKeys<V>& K, const uint64_t (&msel)[V], int k, float& my_val,
                                          int& my_idx, int& my_slot) {
  __shared__ uint2 tk_s[16][2][kMaxTopKLds];
  wave_rank_s<V>(K, msel, k, tk_s[threadIdx.x >> 6], my_val, my_idx, my_slot);
}

// Renormalised softmax weight of rank `lane` (lane < k):
// exp(l_j - l_0) / sum_{j' < k} exp(l_j' - l_0).
__device__ __forceinline__ float wave_topk_weight(float my_val, int k) {
  const float top = __shfl(my_val, 0, 64);
  const int lane = threadIdx.x & 63;
  const float p = lane < k ? expf(my_val - top) : 0.0f;
  const float sum = wave_sum(p);
  return p / sum;
}

// Lane j < k returns selection j: its expert and weight.  Every caller of
// the layer's selection goes through these routines, so all paths pick the
// same experts with the same weight bits.
template <int V>
__device__ __forceinline__ void wave_topk_softmax(const float* __restrict__ row, int E, int k, int& my_idx,
                                                  float& my_w) {
  WaveKeys<V> K;
  wave_keys<V>(row, E, K);
  uint64_t msel[V];
  wave_select<V>(K, k, msel);
  float my_val;
  int my_slot;
  wave_rank<V>(K, msel, k, my_val, my_idx, my_slot);
  my_w = wave_topk_weight(my_val, k);
}

}  // namespace moe
