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
// One wave per expert row, up to 16 tokens per workgroup; the activations
// are staged in LDS (fp32) in K-chunks of 512 and reused by the 4 waves.
// Used for decode-sized batches and for fp32 inputs.
// ---------------------------------------------------------------------------
constexpr int kRouteTT = 16;   // tokens per workgroup
constexpr int kRouteKC = 512;  // K chunk staged in LDS

template <typename XT, typename WT>
__global__ __launch_bounds__(256) void router_gemv_kernel(const XT* __restrict__ x, int64_t T, int H,
                                                         const WT* __restrict__ w, const float* __restrict__ bias,
                                                         int E, float* __restrict__ logits) {
  __shared__ float xs[kRouteTT][kRouteKC];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int e = blockIdx.x * 4 + wv;
  const int64_t t0 = int64_t(blockIdx.y) * kRouteTT;
  const int tt = int(min<int64_t>(kRouteTT, T - t0));
  float acc[kRouteTT];
#pragma unroll
  for (int i = 0; i < kRouteTT; ++i) acc[i] = 0.0f;
  for (int k0 = 0; k0 < H; k0 += kRouteKC) {
    const int kc = min(kRouteKC, H - k0);
    __syncthreads();
    for (int i = threadIdx.x; i < kRouteTT * kRouteKC; i += 256) {
      const int r = i / kRouteKC, c = i % kRouteKC;
      xs[r][c] = (r < tt && c < kc) ? load_act(x + (t0 + r) * H + k0 + c) : 0.0f;
    }
    __syncthreads();
    if (e < E) {
      for (int c = lane; c < kc; c += 64) {
        const float wv_ = load_act(w + int64_t(e) * H + k0 + c);
#pragma unroll
        for (int i = 0; i < kRouteTT; ++i) acc[i] += wv_ * xs[i][c];
      }
    }
  }
  if (e >= E) return;
  const float b = bias ? bias[e] : 0.0f;
#pragma unroll
  for (int i = 0; i < kRouteTT; ++i) {
    const float s = wave_sum(acc[i]);
    if (lane == 0 && i < tt) logits[(t0 + i) * E + e] = s + b;
  }
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
hipError_t launch_router_gemv(const void* x, bool x_bf16, int64_t T, int H, const void* w, bool w_bf16,
                              const float* bias, int E, float* logits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid(unsigned((E + 3) / 4), unsigned((T + kRouteTT - 1) / kRouteTT));
  if (x_bf16 && w_bf16)
    router_gemv_kernel<uint16_t, uint16_t><<<grid, 256, 0, stream>>>(
        (const uint16_t*)x, T, H, (const uint16_t*)w, bias, E, logits);
  else if (x_bf16)
    router_gemv_kernel<uint16_t, float><<<grid, 256, 0, stream>>>((const uint16_t*)x, T, H, (const float*)w,
                                                                  bias, E, logits);
  else if (w_bf16)
    router_gemv_kernel<float, uint16_t><<<grid, 256, 0, stream>>>((const float*)x, T, H, (const uint16_t*)w,
                                                                  bias, E, logits);
  else
    router_gemv_kernel<float, float><<<grid, 256, 0, stream>>>((const float*)x, T, H, (const float*)w, bias,
                                                               E, logits);
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
