// Block quantiser, dequantiser and repack for the 2-, 3- and 4-bit expert
// formats.
//
// Format: blocks of 32 weights along the reduction axis share one fp16 scale;
// code c in [-2^(b-1), 2^(b-1)-1] stored offset-binary.  The quantiser and the
// dequantiser use the canonical row-major layout of the C ABI: a low plane
// [rows][cols/4] bytes (weight k of a row at bits 2(k%4) of byte k/4), then
// for 3 bits a high plane [rows][cols/8] (bit 2 of q at bit k%8 of byte k/8)
// or for 4 bits a second plane [rows][cols/4] in the low plane's layout (bits
// 2..3 of q), and scales [rows][cols/32].  The repack kernel turns that into
// the kernels' own layout (tiled, common.h), once, when weights are uploaded.
// (The pages say experts are stored and read at 2 bits -- "How Strata runs a
// 125-billion-parameter model ...", intro and Step 1 byte table; the block
// layout is this library's own.)
#include "common.h"
#include "launch.h"

namespace moe {

// One thread per 32-weight block.
template <int QBITS>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, int64_t rows,
                                                      int cols, uint8_t* __restrict__ codes,
                                                      uint16_t* __restrict__ scales) {
  const int bpr = cols / kBlock;
  const int64_t nblk = rows * bpr;
  const int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  const int64_t r = b / bpr;
  const int j = int(b - r * bpr);
  const float4v* src = reinterpret_cast<const float4v*>(w + r * cols + int64_t(j) * kBlock);
  float v[kBlock];
#pragma unroll
  for (int i = 0; i < kBlock / 4; ++i) {
    float4v t = src[i];
    v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
  }
  // signed element of largest magnitude, first index on ties
  float m = v[0];
#pragma unroll
  for (int i = 1; i < kBlock; ++i)
    if (fabsf(v[i]) > fabsf(m)) m = v[i];
  constexpr int off = 1 << (QBITS - 1);
  constexpr float cmin = -float(off), cmax = float(off - 1);
  const f16 d16 = f16(m / cmin);  // m / c_min is exact (power of two); RNE to fp16
  const float d = float(d16);
  uint32_t q[kBlock];
#pragma unroll
  for (int i = 0; i < kBlock; ++i) {
    float c = 0.0f;
    if (d != 0.0f) c = fminf(fmaxf(__builtin_rintf(__fdiv_rn(v[i], d)), cmin), cmax);
    q[i] = uint32_t(int(c) + off);
  }
  // a zero scale is stored as +0 whatever the sign of the largest element
  scales[b] = d == 0.0f ? uint16_t(0) : __builtin_bit_cast(uint16_t, d16);
  // low plane: 8 bytes per block
  uint32_t lo0 = 0, lo1 = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    lo0 |= (q[i] & 3u) << (2 * i);
    lo1 |= (q[16 + i] & 3u) << (2 * i);
  }
  uint2v* dst = reinterpret_cast<uint2v*>(codes + b * 8);  // == r * cols / 4 + j * 8
  *dst = uint2v{lo0, lo1};
  if constexpr (QBITS == 3) {
    uint32_t hi = 0;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) hi |= ((q[i] >> 2) & 1u) << i;
    uint32_t* hdst = reinterpret_cast<uint32_t*>(codes + rows * cols / 4 + b * 4);
    *hdst = hi;
  }
  if constexpr (QBITS == 4) {  // bits 2..3 in a second plane of the low plane's layout
    uint32_t hi0 = 0, hi1 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      hi0 |= ((q[i] >> 2) & 3u) << (2 * i);
      hi1 |= ((q[16 + i] >> 2) & 3u) << (2 * i);
    }
    *reinterpret_cast<uint2v*>(codes + rows * cols / 4 + b * 8) = uint2v{hi0, hi1};
  }
}

// One thread per 32-weight block: out = (q - off) * scale, exact in fp32.
template <int QBITS>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ scales,
                                                     int64_t rows, int cols, float* __restrict__ out) {
  const int bpr = cols / kBlock;
  const int64_t nblk = rows * bpr;
  const int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  const int64_t base = b * kBlock;  // == r * cols + j * 32 (row-major output)
  const uint2v lo = *reinterpret_cast<const uint2v*>(codes + b * 8);
  uint32_t hi = 0;
  uint2v hi4 = uint2v{0u, 0u};
  if constexpr (QBITS == 3) hi = *reinterpret_cast<const uint32_t*>(codes + rows * cols / 4 + b * 4);
  if constexpr (QBITS == 4) hi4 = *reinterpret_cast<const uint2v*>(codes + rows * cols / 4 + b * 8);
  const float s = float(__builtin_bit_cast(f16, scales[b]));
  constexpr int off = 1 << (QBITS - 1);
  float4v* dst = reinterpret_cast<float4v*>(out + base);
#pragma unroll
  for (int i = 0; i < kBlock / 4; ++i) {
    float4v t;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = 4 * i + u;
      uint32_t q = ((k < 16 ? lo[0] : lo[1]) >> (2 * (k & 15))) & 3u;
      if constexpr (QBITS == 3) q |= ((hi >> k) & 1u) << 2;
      if constexpr (QBITS == 4) q |= (((k < 16 ? hi4[0] : hi4[1]) >> (2 * (k & 15))) & 3u) << 2;
      t[u] = float(int(q) - off) * s;
    }
    dst[i] = t;
  }
}

// One thread per 32-weight block: canonical row-major block -> the tiled
// placement of common.h.  The 3-bit high-plane word of a block (bit i = code
// i) is stored pre-spread for the unpack: bit i of codes 0..15 moves to bit
// 2i + 1 and bit i of codes 16..31 to bit 2i (qt_high3_word), so no unpack
// has to spread bits at run time.  Every other piece moves unchanged.
template <int QBITS>
__global__ __launch_bounds__(256) void repack_kernel(const uint8_t* __restrict__ codes,
                                                    const uint16_t* __restrict__ scales, int64_t rows, int cols,
                                                    uint8_t* __restrict__ tcodes, uint16_t* __restrict__ tscales) {
  const int bpr = cols / kBlock;
  const int64_t nblk = rows * bpr;
  const int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  const int64_t r = b / bpr;
  const int j = int(b - r * bpr);
  const QTile tl = qtile<false>(r, rows);
  tscales[qt_scale_off(tl, cols, j)] = scales[b];
  *reinterpret_cast<uint2v*>(tcodes + qt_code_off(tl, cols, j)) = *reinterpret_cast<const uint2v*>(codes + b * 8);
  const int64_t plane = rows * cols / 4;
  if constexpr (QBITS == 3) {
    const uint32_t h = *reinterpret_cast<const uint32_t*>(codes + plane + b * 4);
    *reinterpret_cast<uint32_t*>(tcodes + plane + qt_high_off(tl, cols, j)) = qt_high3_word(h);
  }
  if constexpr (QBITS == 4)
    *reinterpret_cast<uint2v*>(tcodes + plane + qt_code_off(tl, cols, j)) =
        *reinterpret_cast<const uint2v*>(codes + plane + b * 8);
}

hipError_t launch_repack(const uint8_t* codes, const uint16_t* scales, int64_t rows, int cols, int qbits,
                         uint8_t* tcodes, uint16_t* tscales, hipStream_t stream) {
  const int64_t nblk = rows * (cols / kBlock);
  if (nblk == 0) return hipSuccess;
  const dim3 grid(unsigned((nblk + 255) / 256));
  if (qbits == 2)
    repack_kernel<2><<<grid, 256, 0, stream>>>(codes, scales, rows, cols, tcodes, tscales);
  else if (qbits == 3)
    repack_kernel<3><<<grid, 256, 0, stream>>>(codes, scales, rows, cols, tcodes, tscales);
  else
    repack_kernel<4><<<grid, 256, 0, stream>>>(codes, scales, rows, cols, tcodes, tscales);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* w, int64_t rows, int cols, int qbits, uint8_t* codes,
                           uint16_t* scales, hipStream_t stream) {
  const int64_t nblk = rows * (cols / kBlock);
  if (nblk == 0) return hipSuccess;
  const dim3 grid(unsigned((nblk + 255) / 256));
  if (qbits == 2)
    quantize_kernel<2><<<grid, 256, 0, stream>>>(w, rows, cols, codes, scales);
  else if (qbits == 3)
    quantize_kernel<3><<<grid, 256, 0, stream>>>(w, rows, cols, codes, scales);
  else
    quantize_kernel<4><<<grid, 256, 0, stream>>>(w, rows, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint16_t* scales, int64_t rows, int cols,
                          int qbits, float* out, hipStream_t stream) {
  const int64_t nblk = rows * (cols / kBlock);
  if (nblk == 0) return hipSuccess;
  const dim3 grid(unsigned((nblk + 255) / 256));
  if (qbits == 2)
    dequant_kernel<2><<<grid, 256, 0, stream>>>(codes, scales, rows, cols, out);
  else if (qbits == 3)
    dequant_kernel<3><<<grid, 256, 0, stream>>>(codes, scales, rows, cols, out);
  else
    dequant_kernel<4><<<grid, 256, 0, stream>>>(codes, scales, rows, cols, out);
  return hipGetLastError();
}

}  // namespace moe
