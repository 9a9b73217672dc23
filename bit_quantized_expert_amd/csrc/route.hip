// Router: logits, top-k selection with renormalised softmax weights, and the
// RMSNorm + bf16 glue between stacked layers.
//
// The router scores every expert of a layer for each token and the 10 best of
// 512 run ("How Strata runs a 125-billion-parameter model ...", intro and
// Step 2 "Mapped host doorbell and a single captured CUDA graph"); ranks 0..9
// are ordered by router weight (Step 2, "Verify-window route tail skip").
#include <float.h>
#include <limits.h>

#include "common.h"
#include "launch.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits on the vector ALUs: logits[t][e] = x[t] . W[e] + b[e].
// One wave per expert row, 4 rows per workgroup, up to TT tokens per
// workgroup (grid.y walks token chunks).  Lane l reads 8 consecutive weights
// at h = 8l + 512i (one 128-bit load of bf16, two of fp32), so a wave streams
// the row in 1 KB coalesced pieces.  For one token the activations come
// straight from global memory (the same 4 KB for every wave, L2-resident);
// for more tokens they are staged in LDS in K-chunks of KC.
// ---------------------------------------------------------------------------
template <typename T_>
__device__ __forceinline__ void load8(const T_* p, float* v) {
  if constexpr (sizeof(T_) == 2) {
    const uint4v u = *reinterpret_cast<const uint4v*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
    const float4v a = reinterpret_cast<const float4v*>(p)[0];
    const float4v b = reinterpret_cast<const float4v*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

template <typename XT, typename WT, int TT>
__global__ __launch_bounds__(256) void router_gemv_kernel(const XT* __restrict__ x, int64_t T, int H,
                                                         const WT* __restrict__ w, const float* __restrict__ bias,
                                                         int E, float* __restrict__ logits) {
  constexpr int KC = TT == 1 ? 0 : (32768 / (TT * int(sizeof(XT))));  // K chunk staged in LDS (32 KB)
  __shared__ __attribute__((aligned(16))) XT xs[TT == 1 ? 1 : TT * KC];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int e = blockIdx.x * 4 + wv;
  const int64_t t0 = int64_t(blockIdx.y) * TT;
  const int tt = int(min<int64_t>(TT, T - t0));
  float acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = 0.0f;
  const WT* wrow = w + int64_t(e < E ? e : 0) * H;
  if constexpr (TT == 1) {
    if (e < E) {
      for (int h = lane * 8; h < H; h += 512) {
        float wv8[8], xv8[8];
        load8(wrow + h, wv8);
        load8(x + t0 * H + h, xv8);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[0] += wv8[i] * xv8[i];
      }
    }
  } else {
    for (int k0 = 0; k0 < H; k0 += KC) {
      const int kc = min(KC, H - k0);
      __syncthreads();
      // stage x[t0 .. t0+tt)[k0 .. k0+kc) (8 elements per thread-step)
      for (int i = threadIdx.x * 8; i < TT * kc; i += 256 * 8) {
        const int r = i / kc, c = i - r * kc;
        if (r < tt) {
          const XT* src = x + (t0 + r) * H + k0 + c;
          *reinterpret_cast<uint4v*>(&xs[r * KC + c]) = *reinterpret_cast<const uint4v*>(src);
          if constexpr (sizeof(XT) == 4)
            *reinterpret_cast<uint4v*>(&xs[r * KC + c + 4]) = *reinterpret_cast<const uint4v*>(src + 4);
        }
      }
      __syncthreads();
      if (e < E) {
        for (int c = lane * 8; c < kc; c += 512) {
          float wv8[8];
          load8(wrow + k0 + c, wv8);
#pragma unroll
          for (int r = 0; r < TT; ++r) {
            if (r < tt) {
              float xv8[8];
              load8(&xs[r * KC + c], xv8);
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[r] += wv8[i] * xv8[i];
            }
          }
        }
      }
    }
  }
  if (e >= E) return;
  const float b = bias ? bias[e] : 0.0f;
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    if (i < tt) {
      const float s = wave_sum(acc[i]);
      if (lane == 0) logits[(t0 + i) * E + e] = s + b;
    }
  }
}

// ---------------------------------------------------------------------------
// Router logits on MFMA for bf16 activations and bf16 router weights
// (v_mfma_f32_16x16x32_bf16: bf16 x bf16 products are exact in fp32).
// Workgroup = 16 experts x 16 tokens, 8 waves; wave w takes the 32-wide
// K blocks w, w+8, w+16, ...  Partial tiles are summed through LDS in wave
// order, so a token's logits never depend on the other tokens.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void router_mfma_kernel(const uint16_t* __restrict__ x, int64_t T, int H,
                                                         const uint16_t* __restrict__ w,
                                                         const float* __restrict__ bias, int E,
                                                         float* __restrict__ logits) {
  __shared__ float red[8][4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * 16;
  const int64_t t0 = int64_t(blockIdx.y) * 16;
  const int nkb = H / 32;
  const bool b_on = e0 + n < E;
  const bool a_on = t0 + n < T;
  const uint16_t* wrow = w + int64_t(b_on ? e0 + n : 0) * H + 8 * g;
  const uint16_t* xrow = x + (a_on ? t0 + n : 0) * H + 8 * g;
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int B = 8;  // K blocks per load batch
  for (int kb0 = wv; kb0 < nkb; kb0 += 8 * B) {
    uint4v bw[B], ax[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {  // unconditional loads (clamped block, rows clamped above)
      const int kb = kb0 + 8 * i;
      const bool in = kb < nkb;
      const int kbc = in ? kb : 0;
      const uint4v wl = *reinterpret_cast<const uint4v*>(wrow + kbc * 32);
      const uint4v xl = *reinterpret_cast<const uint4v*>(xrow + kbc * 32);
      bw[i] = (in && b_on) ? wl : uint4v{0u, 0u, 0u, 0u};
      ax[i] = (in && a_on) ? xl : uint4v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < B; ++i)
      if (kb0 + 8 * i < nkb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ax[i]),
                                                      __builtin_bit_cast(bf16x8, bw[i]), acc, 0, 0, 0);
  }
  if (wv > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wv][j][lane] = acc[j];
  }
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int q = 1; q < 8; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += red[q][j][lane];
  if (!b_on) return;
  const float b = bias ? bias[e0 + n] : 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = t0 + 4 * g + j;
    if (t < T) logits[t * E + e0 + n] = acc[j] + b;
  }
}

hipError_t launch_router_mfma(const uint16_t* x, int64_t T, int H, const uint16_t* w, const float* bias, int E,
                              float* logits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid(unsigned((E + 15) / 16), unsigned((T + 15) / 16));
  router_mfma_kernel<<<grid, 512, 0, stream>>>(x, T, H, w, bias, E, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k with ties to the lower expert index, then softmax over the selected
// logits.  One wave per token; lane l holds experts l, l+64, l+128, ...
// ---------------------------------------------------------------------------
template <int V>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                  int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float val[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = lane + 64 * v;
    val[v] = e < E ? logits[t * E + e] : -INFINITY;
  }
  uint64_t taken = 0;
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (lane + 64 * v >= E) taken |= 1ull << v;
  float my_val = 0.0f;  // lane j keeps the j-th selection
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if (!((taken >> v) & 1ull) && (bi == INT_MAX || val[v] > bv)) {
        bv = val[v];
        bi = lane + 64 * v;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (oi != INT_MAX && (bi == INT_MAX || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi != INT_MAX && (bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (lane == j) {
      my_val = bv;
      my_idx = bi;
    }
  }
  const float top = __shfl(my_val, 0, 64);
  const float p = lane < k ? expf(my_val - top) : 0.0f;
  const float sum = wave_sum(p);
  if (lane < k) {
    idx_out[t * k + lane] = my_idx;
    w_out[t * k + lane] = p / sum;
  }
}

// ---------------------------------------------------------------------------
// a[t] = bf16_RNE(r[t] / sqrt(mean(r[t]^2) + 1e-6)); one workgroup per row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void rmsnorm_bf16_kernel(const float* __restrict__ r, int H,
                                                          uint16_t* __restrict__ a) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const float* row = r + t * H;
  float ss = 0.0f;
  for (int c = threadIdx.x; c < H; c += 256) ss += row[c] * row[c];
  ss = block_sum_256(ss, red);
  const float denom = sqrtf(ss / float(H) + 1e-6f);
  for (int c = threadIdx.x; c < H; c += 256) a[t * H + c] = f32_to_bf16_rne(row[c] / denom);
}

// ---------------------------------------------------------------------------
template <typename XT, typename WT>
static void router_launch(const void* x, int64_t T, int H, const void* w, const float* bias, int E, float* logits,
                          hipStream_t stream) {
  if (T == 1) {
    router_gemv_kernel<XT, WT, 1><<<dim3(unsigned((E + 3) / 4), 1), 256, 0, stream>>>(
        (const XT*)x, T, H, (const WT*)w, bias, E, logits);
  } else {
    router_gemv_kernel<XT, WT, 16><<<dim3(unsigned((E + 3) / 4), unsigned((T + 15) / 16)), 256, 0, stream>>>(
        (const XT*)x, T, H, (const WT*)w, bias, E, logits);
  }
}

hipError_t launch_router_gemv(const void* x, bool x_bf16, int64_t T, int H, const void* w, bool w_bf16,
                              const float* bias, int E, float* logits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (x_bf16 && w_bf16) router_launch<uint16_t, uint16_t>(x, T, H, w, bias, E, logits, stream);
  else if (x_bf16) router_launch<uint16_t, float>(x, T, H, w, bias, E, logits, stream);
  else if (w_bf16) router_launch<float, uint16_t>(x, T, H, w, bias, E, logits, stream);
  else router_launch<float, float>(x, T, H, w, bias, E, logits, stream);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w,
                       hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid(unsigned((T + 3) / 4));
  const int v = (E + 63) / 64;
  if (v <= 1) topk_kernel<1><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else if (v <= 2) topk_kernel<2><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else if (v <= 4) topk_kernel<4><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else if (v <= 8) topk_kernel<8><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else if (v <= 16) topk_kernel<16><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else if (v <= 32) topk_kernel<32><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else topk_kernel<64><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bf16(const float* r, int64_t T, int H, uint16_t* a, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  rmsnorm_bf16_kernel<<<dim3(unsigned(T)), 256, 0, stream>>>(r, H, a);
  return hipGetLastError();
}

}  // namespace moe
