// Expert FFN for decode-sized batches: fused dequant-GEMV on MFMA.
//
// The experts run straight from their 2-bit (or 3-bit) storage ("How Strata
// runs a 125-billion-parameter model ...", intro and Step 1 byte table: a
// token reads 0.66 GB of 2-bit expert weights).  With every expert resident
// in HBM the work is a stream of quantised weight rows:
//
//   gate/up kernel : h[m][i] = silu(x_m . W_gate[i]) * (x_m . W_up[i])
//   down kernel    : y[m][n] = h_m . W_down[n]
//
// Each wave owns 16 output rows and a tile of up to 16 tokens (padded), and
// runs v_mfma_f32_16x16x32_f16.  Lane (n = l%16, g = l/16) streams row n:
// in round r it loads the 64-weight unit u = 4r + g (16 bytes of 2-bit codes,
// a 128-bit load), so the 4 lanes of a row read 64 contiguous bytes per
// round.  Codes are unpacked in registers to exact fp16 c*s (see dq2_word);
// the activations sit in LDS as fp16 in the matching permuted order.  One
// workgroup = 4 waves = 64 rows of one expert (or of the shared expert).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

// ---------------------------------------------------------------------------
// Plan: active expert list (ascending ids with a non-empty segment) and the
// grouped-GEMM tile list.  One workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int E, int64_t T,
                                                   int has_shared, int tile_bm, int32_t* __restrict__ header,
                                                   int32_t* __restrict__ active, int32_t* __restrict__ tile_expert,
                                                   int32_t* __restrict__ tile_m0) {
  __shared__ int flag[kMaxExperts];
  __shared__ int ntile[kMaxExperts];
  __shared__ int tmp[1024];
  for (int e = threadIdx.x; e < E; e += 1024) {
    const int c = offsets[e + 1] - offsets[e];
    flag[e] = c > 0;
    ntile[e] = tile_bm > 0 ? (c + tile_bm - 1) / tile_bm : 0;
  }
  __syncthreads();
  const int n_active = block_exclusive_scan_lds(flag, E, tmp);
  const int n_routed_tiles = block_exclusive_scan_lds(ntile, E, tmp);
  for (int e = threadIdx.x; e < E; e += 1024) {
    const int c = offsets[e + 1] - offsets[e];
    if (c > 0) active[flag[e]] = e;
    if (tile_bm > 0) {
      int pos = ntile[e];
      for (int m0 = 0; m0 < c; m0 += tile_bm, ++pos) {
        tile_expert[pos] = e;
        tile_m0[pos] = m0;
      }
    }
  }
  int n_tiles = n_routed_tiles;
  if (tile_bm > 0 && has_shared) {
    const int st = int((T + tile_bm - 1) / tile_bm);
    for (int i = threadIdx.x; i < st; i += 1024) {
      tile_expert[n_routed_tiles + i] = -1;
      tile_m0[n_routed_tiles + i] = i * tile_bm;
    }
    n_tiles += st;
  }
  if (threadIdx.x == 0) {
    header[kHdrActive] = n_active;
    header[kHdrTiles] = n_tiles;
  }
}

hipError_t launch_plan(const int32_t* offsets, int E, int64_t T, int has_shared, int tile_bm, int32_t* header,
                       int32_t* active, int32_t* tile_expert, int32_t* tile_m0, hipStream_t stream) {
  plan_kernel<<<1, 1024, 0, stream>>>(offsets, E, T, has_shared, tile_bm, header, active, tile_expert, tile_m0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Slot resolution shared by both decode kernels.
// ---------------------------------------------------------------------------
struct Slot {
  bool valid, shared;
  int e, lo, m_total;
};

__device__ __forceinline__ Slot resolve_slot(const FfnArgs& a, int slot) {
  Slot s{false, false, 0, 0, 0};
  const int n_active = a.header[kHdrActive];
  if (slot < n_active) {
    s.valid = true;
    s.e = a.plan_active[slot];
    s.lo = a.offsets[s.e];
    s.m_total = a.offsets[s.e + 1] - s.lo;
  } else if (slot == n_active && a.has_shared) {
    s.valid = true;
    s.shared = true;
    s.m_total = int(a.T);
  }
  return s;
}

// Stage rows of fp16 activations (or fp32/bf16 inputs) into LDS in the
// permuted 16-group order.  src_row(r) gives the row pointer of tile row r.
template <typename SRC, typename RowFn>
__device__ __forceinline__ void stage_rows(f16* lds, int ldsw, int mnow, int K, RowFn src_row) {
  const int groups = K / 16;
  for (int it = threadIdx.x; it < mnow * groups; it += blockDim.x) {
    const int r = it / groups, gg = it - r * groups;
    const SRC* src = src_row(r) + gg * 16;
    float v[16];
    if constexpr (sizeof(SRC) == 4) {
      const float4v* p = reinterpret_cast<const float4v*>(src);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4v t = p[q];
        v[4 * q] = t[0]; v[4 * q + 1] = t[1]; v[4 * q + 2] = t[2]; v[4 * q + 3] = t[3];
      }
    } else {
      const uint4v* p = reinterpret_cast<const uint4v*>(src);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4v t = p[q];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t wd = t[u];
          if constexpr (std::is_same<SRC, f16>::value) {
            const half2v h = as_half2(wd);
            v[8 * q + 2 * u] = float(h[0]);
            v[8 * q + 2 * u + 1] = float(h[1]);
          } else {  // bf16
            v[8 * q + 2 * u] = __uint_as_float(wd << 16);
            v[8 * q + 2 * u + 1] = __uint_as_float(wd & 0xffff0000u);
          }
        }
      }
    }
    half8 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[2 * i] = f16(v[i]);
      lo[2 * i + 1] = f16(v[i + 8]);
      hi[2 * i] = f16(v[4 + i]);
      hi[2 * i + 1] = f16(v[12 + i]);
    }
    half8* dst = reinterpret_cast<half8*>(lds + r * ldsw + gg * 16);
    dst[0] = lo;
    dst[1] = hi;
  }
}

// One quantised unit of a row: UNIT = 64 weights (16 code bytes, 2 scales)
// or 32 (8 code bytes, 1 scale).  3-bit adds UNIT/32 high-plane words.
template <int QBITS, int UNIT>
struct Unit {
  uint32_t w[UNIT / 16];  // low-plane words, 16 codes each
  uint32_t h[UNIT / 32];  // high-plane words, 32 codes each (3-bit only)
  uint32_t s;             // fp16 scale bits (two for UNIT = 64)
};

template <int QBITS, int UNIT>
__device__ __forceinline__ void load_unit(Unit<QBITS, UNIT>& U, const uint8_t* codes, const uint16_t* scales,
                                          int rows, int K, int row, int u) {
  const uint8_t* lo = codes + int64_t(row) * (K / 4) + u * (UNIT / 4);
  if constexpr (UNIT == 64) {
    const uint4v c = *reinterpret_cast<const uint4v*>(lo);
    U.w[0] = c[0]; U.w[1] = c[1]; U.w[2] = c[2]; U.w[3] = c[3];
    U.s = *reinterpret_cast<const uint32_t*>(scales + int64_t(row) * (K / 32) + u * 2);
  } else {
    const uint2v c = *reinterpret_cast<const uint2v*>(lo);
    U.w[0] = c[0]; U.w[1] = c[1];
    U.s = scales[int64_t(row) * (K / 32) + u];
  }
  if constexpr (QBITS == 3) {
    const uint8_t* hp = codes + int64_t(rows) * (K / 4) + int64_t(row) * (K / 8) + u * (UNIT / 8);
    if constexpr (UNIT == 64) {
      const uint2v hv = *reinterpret_cast<const uint2v*>(hp);
      U.h[0] = hv[0]; U.h[1] = hv[1];
    } else {
      U.h[0] = *reinterpret_cast<const uint32_t*>(hp);
    }
  }
}

template <int QBITS, int UNIT>
__device__ __forceinline__ void zero_unit(Unit<QBITS, UNIT>& U) {
#pragma unroll
  for (int i = 0; i < UNIT / 16; ++i) U.w[i] = 0;
#pragma unroll
  for (int i = 0; i < UNIT / 32; ++i) U.h[i] = 0;
  U.s = 0;  // zero scale: every dequantised weight is 0
}

// Dequantise word d (16 codes) of a unit into two permuted MFMA k-slices.
template <int QBITS, int UNIT>
__device__ __forceinline__ void dq_unit_word(const Unit<QBITS, UNIT>& U, int d, half8& lo, half8& hi) {
  const uint32_t sbits = (UNIT == 64 && d >= 2) ? (U.s >> 16) : (U.s & 0xffffu);
  const half2v s2 = as_half2(sbits | (sbits << 16));
  if constexpr (QBITS == 2) {
    dq2_word(U.w[d], s2, lo, hi);
  } else {
    const uint32_t hb = (U.h[d >> 1] >> (16 * (d & 1))) & 0xffffu;
    dq3_word(U.w[d], spread16(hb), s2, lo, hi);
  }
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  grid = (ceil(max_rows / 64), slots), block = 256.
// ---------------------------------------------------------------------------
template <int QBITS, int UNIT, typename XT>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) f16 xs[];
  const Slot sl = resolve_slot(a, blockIdx.y);
  if (!sl.valid) return;
  const int rows = sl.shared ? a.Is : a.I;
  const int row_base = blockIdx.x * 64;
  if (row_base >= rows || sl.m_total == 0) return;
  const QMat G = sl.shared ? a.sg : a.rg;
  const QMat U = sl.shared ? a.su : a.ru;
  const int64_t ex = sl.shared ? 0 : sl.e;
  const uint8_t* gc = G.codes + ex * G.code_stride;
  const uint16_t* gs = G.scales + ex * G.scale_stride;
  const uint8_t* uc = U.codes + ex * U.code_stride;
  const uint16_t* us = U.scales + ex * U.scale_stride;
  const int H = a.H, ldsw = H + 8;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row = row_base + wv * 16 + n;
  const bool wave_on = row_base + wv * 16 < rows;
  const int n_units = H / UNIT, rounds = (n_units + 3) / 4;
  const XT* x = static_cast<const XT*>(a.x);
  f16* hout = sl.shared ? a.h_shared : a.h_routed;
  const int hw = sl.shared ? a.Is : a.I;

  for (int mc = 0; mc < sl.m_total; mc += kGemvMaxM) {
    const int mnow = min(kGemvMaxM, sl.m_total - mc);
    __syncthreads();
    stage_rows<XT>(xs, ldsw, mnow, H, [&](int r) -> const XT* {
      const int64_t t = sl.shared ? int64_t(mc + r) : int64_t(a.sorted_pair[sl.lo + mc + r] / a.k);
      return x + t * H;
    });
    __syncthreads();
    if (!wave_on) continue;
    float4v accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    const bool a_on = n < mnow;  // this lane's A row (token) exists
    const f16* xrow = xs + n * ldsw;
    constexpr int RB = 8;
    for (int r0 = 0; r0 < rounds; r0 += RB) {
      Unit<QBITS, UNIT> ug[RB], uu[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int u = (r0 + i) * 4 + g;
        if (r0 + i < rounds && u < n_units) {
          load_unit(ug[i], gc, gs, rows, H, row, u);
          load_unit(uu[i], uc, us, rows, H, row, u);
        } else {
          zero_unit(ug[i]);
          zero_unit(uu[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (r0 + i >= rounds) break;
        const int u = (r0 + i) * 4 + g;
        const bool on = a_on && u < n_units;
#pragma unroll
        for (int d = 0; d < UNIT / 16; ++d) {
          half8 glo, ghi, ulo, uhi, alo = {}, ahi = {};
          dq_unit_word(ug[i], d, glo, ghi);
          dq_unit_word(uu[i], d, ulo, uhi);
          if (on) {
            const half8* ap = reinterpret_cast<const half8*>(xrow + u * UNIT + 16 * d);
            alo = ap[0];
            ahi = ap[1];
          }
          accg = mfma16(alo, glo, accg);
          accg = mfma16(ahi, ghi, accg);
          accu = mfma16(alo, ulo, accu);
          accu = mfma16(ahi, uhi, accu);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = 4 * g + j;
      if (m < mnow) {
        const float hv = silu_f(accg[j]) * accu[j];
        const int64_t hr = sl.shared ? int64_t(mc + m) : int64_t(sl.lo + mc + m);
        hout[hr * hw + row] = f16(hv);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// down projection.  grid = (ceil(H / 64), slots), block = 256.
// ---------------------------------------------------------------------------
template <int QBITS, int UNIT>
__global__ __launch_bounds__(256) void gemv_down_kernel(FfnArgs a, int ldsw) {
  extern __shared__ __attribute__((aligned(16))) f16 hs[];
  const Slot sl = resolve_slot(a, blockIdx.y);
  if (!sl.valid) return;
  const int H = a.H;
  const int row_base = blockIdx.x * 64;
  if (row_base >= H || sl.m_total == 0) return;
  if (sl.shared && a.shared_out == nullptr) return;
  const int K = sl.shared ? a.Is : a.I;
  const QMat D = sl.shared ? a.sd : a.rd;
  const int64_t ex = sl.shared ? 0 : sl.e;
  const uint8_t* dc = D.codes + ex * D.code_stride;
  const uint16_t* ds = D.scales + ex * D.scale_stride;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row = row_base + wv * 16 + n;
  const bool wave_on = row_base + wv * 16 < H;
  const int n_units = K / UNIT, rounds = (n_units + 3) / 4;
  const f16* hin = sl.shared ? a.h_shared : a.h_routed;
  float* yout = sl.shared ? a.shared_out : a.y_sorted;

  for (int mc = 0; mc < sl.m_total; mc += kGemvMaxM) {
    const int mnow = min(kGemvMaxM, sl.m_total - mc);
    __syncthreads();
    stage_rows<f16>(hs, ldsw, mnow, K, [&](int r) -> const f16* {
      const int64_t hr = sl.shared ? int64_t(mc + r) : int64_t(sl.lo + mc + r);
      return hin + hr * K;
    });
    __syncthreads();
    if (!wave_on) continue;
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    const bool a_on = n < mnow;
    const f16* hrow = hs + n * ldsw;
    constexpr int RB = 4;
    for (int r0 = 0; r0 < rounds; r0 += RB) {
      Unit<QBITS, UNIT> ud[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int u = (r0 + i) * 4 + g;
        if (r0 + i < rounds && u < n_units) load_unit(ud[i], dc, ds, H, K, row, u);
        else zero_unit(ud[i]);
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (r0 + i >= rounds) break;
        const int u = (r0 + i) * 4 + g;
        const bool on = a_on && u < n_units;
#pragma unroll
        for (int d = 0; d < UNIT / 16; ++d) {
          half8 blo, bhi, alo = {}, ahi = {};
          dq_unit_word(ud[i], d, blo, bhi);
          if (on) {
            const half8* ap = reinterpret_cast<const half8*>(hrow + u * UNIT + 16 * d);
            alo = ap[0];
            ahi = ap[1];
          }
          acc = mfma16(alo, blo, acc);
          acc = mfma16(ahi, bhi, acc);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = 4 * g + j;
      if (m < mnow) {
        const int64_t yr = sl.shared ? int64_t(mc + m) : int64_t(sl.lo + mc + m);
        yout[yr * H + row] = acc[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <int QBITS>
static hipError_t launch_gemv_q(const FfnArgs& a, hipStream_t stream) {
  const int64_t P = a.T * a.k;
  const int slots = int(std::min<int64_t>(a.E, P)) + (a.has_shared ? 1 : 0);
  const int mrows = int(std::min<int64_t>(kGemvMaxM, std::max<int64_t>(a.T, 1)));
  const int max_rows = std::max(a.I, a.has_shared ? a.Is : 0);
  {
    const dim3 grid(unsigned((max_rows + 63) / 64), unsigned(slots));
    const size_t lds = size_t(mrows) * (a.H + 8) * sizeof(f16);
    const bool u64 = a.H % 64 == 0;
    if (a.x_bf16) {
      if (u64) gemv_gateup_kernel<QBITS, 64, uint16_t><<<grid, 256, lds, stream>>>(a);
      else gemv_gateup_kernel<QBITS, 32, uint16_t><<<grid, 256, lds, stream>>>(a);
    } else {
      if (u64) gemv_gateup_kernel<QBITS, 64, float><<<grid, 256, lds, stream>>>(a);
      else gemv_gateup_kernel<QBITS, 32, float><<<grid, 256, lds, stream>>>(a);
    }
  }
  {
    const int kmax = std::max(a.I, a.has_shared ? a.Is : 0);
    const int ldsw = kmax + 8;
    const dim3 grid(unsigned((a.H + 63) / 64), unsigned(slots));
    const size_t lds = size_t(mrows) * ldsw * sizeof(f16);
    // UNIT must divide both K values; 64 only when both are multiples of 64.
    const bool u64 = a.I % 64 == 0 && (!a.has_shared || a.Is % 64 == 0);
    if (u64) gemv_down_kernel<QBITS, 64><<<grid, 256, lds, stream>>>(a, ldsw);
    else gemv_down_kernel<QBITS, 32><<<grid, 256, lds, stream>>>(a, ldsw);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_gemv(const FfnArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  return a.qbits == 2 ? launch_gemv_q<2>(a, stream) : launch_gemv_q<3>(a, stream);
}

}  // namespace moe
