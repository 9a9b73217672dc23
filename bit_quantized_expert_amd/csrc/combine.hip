// Weighted combine of the finished expert vectors, plus the optional
// residual + RMSNorm + bf16 glue of stacked layers.  The GPU sums the expert
// outputs of a layer ("How Strata runs a 125-billion-parameter model ...",
// Step 2, "Dynamic PCIe and CPU co-execution": finished vectors are written
// back for the GPU to sum).
//
//   out[t] = shared[t] + sum_{j<k} w[t][j] * y_sorted[pair_pos[t*k + j]]
//
// One workgroup per token row; each thread owns float4 columns.
#include "common.h"
#include "launch.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ pos,
                                                     const float* __restrict__ w, const float* __restrict__ shared,
                                                     int H, int k, float* __restrict__ out, float* __restrict__ res,
                                                     uint16_t* __restrict__ next_in) {
  __shared__ float red[4];
  __shared__ int s_pos[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    s_pos[threadIdx.x] = pos[t * k + threadIdx.x];
    s_w[threadIdx.x] = w[t * k + threadIdx.x];
  }
  __syncthreads();
  const int H4 = H / 4;
  float ss = 0.0f;
  for (int c = threadIdx.x; c < H4; c += 256) {
    float4v acc = shared ? reinterpret_cast<const float4v*>(shared + t * H)[c] : float4v{0.f, 0.f, 0.f, 0.f};
    // issue up to 8 row loads before using them (latency, not bandwidth, bounds one token)
    for (int j0 = 0; j0 < k; j0 += 8) {
      float4v v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = j0 + i < k ? s_pos[j0 + i] : -1;
        v[i] = p >= 0 ? reinterpret_cast<const float4v*>(y + int64_t(p) * H)[c] : float4v{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (j0 + i < k)  // pairs of out-of-range ids (p < 0) add 0
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(s_w[j0 + i], v[i][q], acc[q]);
    }
    if (out) reinterpret_cast<float4v*>(out + t * H)[c] = acc;
    if (res) {
      float4v r = reinterpret_cast<float4v*>(res + t * H)[c];
      r += acc;
      reinterpret_cast<float4v*>(res + t * H)[c] = r;
      ss += r[0] * r[0] + r[1] * r[1] + r[2] * r[2] + r[3] * r[3];
    }
  }
  if (!res || !next_in) return;  // uniform across the workgroup
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float denom = sqrtf((red[0] + red[1] + red[2] + red[3]) / float(H) + 1e-6f);
  for (int c = threadIdx.x; c < H4; c += 256) {
    const float4v r = reinterpret_cast<const float4v*>(res + t * H)[c];
    uint16_t* dst = next_in + t * H + 4 * c;
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[u] = f32_to_bf16_rne(r[u] / denom);
  }
}

hipError_t launch_combine(const float* y_sorted, const int32_t* pair_pos, const float* topk_w,
                          const float* shared_out, int64_t T, int H, int k, float* out, float* residual,
                          uint16_t* next_in, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  combine_kernel<<<dim3(unsigned(T)), 256, 0, stream>>>(y_sorted, pair_pos, topk_w, shared_out, H, k, out,
                                                        residual, next_in);
  return hipGetLastError();
}

}  // namespace moe
