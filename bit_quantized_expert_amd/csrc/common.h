// Device helpers shared by the gfx950 kernels of the MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Dequantise 2-bit word w (16 codes) with block scale s2 (scale in both
// halves) into two MFMA k-slices (8 fp16 each) in the permuted order.
__device__ __forceinline__ void dq2_word(uint32_t w, half2v s2, half8& lo, half8& hi) {
  const uint32_t w10 = w >> 10;
  half2v p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = i < 5 ? i : i - 5;
    const uint32_t src = i < 5 ? w : w10;
    const uint32_t v = and_or(src, 0x00030003u << (2 * j), magic_bits(j));
    const f16 off = magic_val(j) + f16(2.0f);
    half2v h = as_half2(v) - half2v{off, off};
    p[i] = h * s2;
  }
  lo = half8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  hi = half8{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}

// Spread the 16 bits of h to even bit positions: bit k -> bit 2k.
__device__ __forceinline__ uint32_t spread16(uint32_t h) {
  h &= 0xffffu;
  h = (h | (h << 8)) & 0x00ff00ffu;
  h = (h | (h << 4)) & 0x0f0f0f0fu;
  h = (h | (h << 2)) & 0x33333333u;
  h = (h | (h << 1)) & 0x55555555u;
  return h;
}

// 3-bit variant: w holds the low two bits of 16 codes (2-bit layout) and
// sp = spread16(high bits) holds bit 2 of code i at bit 2i.  Pairs 0..3 use
// M_0..M_3 with the high bits moved to 2i+2 (sp << 2; bits up to 2i+2 <= 8
// stay inside the mantissa); pairs 4..7 use w >> 8 and sp >> 6 with M_0..M_3
// (shifting right keeps bit 30, the high bit of code 15).  c = q - 4.
__device__ __forceinline__ void dq3_word(uint32_t w, uint32_t sp, half2v s2, half8& lo, half8& hi) {
  const uint32_t w8 = w >> 8, hs = sp << 2, h8 = sp >> 6;
  half2v p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = i < 4 ? i : i - 4;
    const uint32_t src = i < 4 ? w : w8;
    const uint32_t hsrc = i < 4 ? hs : h8;
    const uint32_t v = and_or_v(src, 0x00030003u << (2 * j), and_or(hsrc, 0x00040004u << (2 * j), magic_bits(j)));
    const f16 off = magic_val(j) + f16(4.0f);
    half2v h = as_half2(v) - half2v{off, off};
    p[i] = h * s2;
  }
  lo = half8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  hi = half8{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
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

// Exclusive scan of vals[0..n) in LDS by a 1024-thread workgroup with two
// barriers: each wave scans a contiguous run, then the wave totals.  `tmp`
// holds 16 ints.  Returns the total.  n <= 4096.
__device__ inline int block_scan_fast(int* vals, int n, int* tmp) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int per = (n + 1023) / 1024;  // values per thread, <= 4
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
  for (int w = 0; w < 16; ++w) {
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

// One wave: top-k of one token's logits.  Lane l holds experts l + 64v as
// order-preserving keys.  Each round takes the largest key (DPP max), then
// the lowest expert index holding it (a ballot per v, lowest v first, then
// the lowest lane) and zeroes that key (0 is below every finite key).  Lane
// j < k returns selection j; its value is recovered from the key (a -0
// logit comes back as +0, which changes no weight).
template <int V>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, float& my_val, int& my_idx) {
  const int lane = threadIdx.x & 63;
  uint32_t key[V];
  float f[V];
#pragma unroll
  for (int v = 0; v < V; ++v) f[v] = row[min(lane + 64 * v, E - 1)];
  // Pin every load as unconditional, so the V loads are in flight together
  // (a load feeding only one side of a select is otherwise moved into a
  // branch with its own wait).
#pragma unroll
  for (int v = 0; v < V; ++v) asm volatile("" : "+v"(f[v]));
#pragma unroll
  for (int v = 0; v < V; ++v) key[v] = lane + 64 * v < E ? float_key(f[v]) : 0u;
  uint32_t my_key = 0;
  my_idx = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t bk = key[0];
#pragma unroll
    for (int v = 1; v < V; ++v) bk = max(bk, key[v]);
    const uint32_t top = wave_max_u32(bk);
    int win = -1;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if (win < 0) {
        const uint64_t m = __ballot(key[v] == top);
        if (m) win = 64 * v + __builtin_ctzll(m);
      }
    }
    const int owner = win & 63, wv_ = win >> 6;
    if (lane == owner) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v == wv_) key[v] = 0u;
    }
    if (lane == j) {
      my_key = top;
      my_idx = win;
    }
  }
  my_val = key_float(my_key);
}

// Lane j < k returns selection j: its expert and weight
// exp(l_j - l_0) / sum_{j' < k} exp(l_j' - l_0).  Every caller of the
// layer's selection goes through this one function, so all paths pick the
// same experts with the same weight bits.
template <int V>
__device__ __forceinline__ void wave_topk_softmax(const float* __restrict__ row, int E, int k, int& my_idx,
                                                  float& my_w) {
  float my_val;
  wave_topk<V>(row, E, k, my_val, my_idx);
  const float top = __shfl(my_val, 0, 64);
  const int lane = threadIdx.x & 63;
  const float p = lane < k ? expf(my_val - top) : 0.0f;
  const float sum = wave_sum(p);
  my_w = p / sum;
}

}  // namespace moe
