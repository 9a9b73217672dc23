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

// Sum of squares of a float4, in one fixed order (the combine and the
// stand-alone residual RMSNorm must give the same bits).
__device__ __forceinline__ float sumsq4(float4v r) {
  return __builtin_fmaf(r[3], r[3], __builtin_fmaf(r[2], r[2], __builtin_fmaf(r[1], r[1], r[0] * r[0])));
}

// a = bf16_RNE(res / sqrt(ss_total / H + 1e-6)) for one row, ss per thread
// accumulated over the float4 columns c = threadIdx.x, +256, ...
__device__ __forceinline__ void rmsnorm_row(const float* __restrict__ res, int H, float ss, float* red,
                                            uint16_t* __restrict__ next_in) {
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float denom = sqrtf((red[0] + red[1] + red[2] + red[3]) / float(H) + 1e-6f);
  const int H4 = H / 4;
  for (int c = threadIdx.x; c < H4; c += 256) {
    const float4v r = reinterpret_cast<const float4v*>(res)[c];
    uint16_t* dst = next_in + 4 * c;
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[u] = f32_to_bf16_rne(r[u] / denom);
  }
}

// CPT float4 columns per thread per pass (all their loads in flight
// together); with H / 4 <= 256 * CPT the row is one pass and the updated
// residual stays in registers for the norm.  The pair slots and weights are
// uniform loads (no LDS staging, no barrier before the row loads).  JG pairs
// are loaded per group (the launch picks JG >= k where it can, so no row is
// loaded twice); RES: a residual row is read (only then).  YT: the expert
// rows are fp32, or fp16 (the grouped-GEMM layer, where these rows are most
// of the layer's memory traffic); the sum is fp32 either way.  ST: the
// shared rows' type (fp32, or fp16 beside fp16 expert rows).  shared points
// at [T][H] rows: the shared expert's output when has_shared, else any
// readable rows (their values are replaced by 0; they may be out or res, so
// the pointer is not restrict).
template <typename YT>
struct YRow;
template <>
struct YRow<float> {
  typedef float4v raw;
  static __device__ __forceinline__ float4v cvt(float4v v) { return v; }
};
template <>
struct YRow<f16> {
  typedef uint2v raw;  // four fp16
  static __device__ __forceinline__ float4v cvt(uint2v v) {
    const half2v a = as_half2(v[0]), b = as_half2(v[1]);
    return float4v{float(a[0]), float(a[1]), float(b[0]), float(b[1])};
  }
};

template <int CPT, int JG, bool RES, typename YT, typename ST>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y, const int32_t* __restrict__ pos,
                                                     const float* __restrict__ w, const ST* shared,
                                                     int has_shared, int H, int k, float* __restrict__ out,
                                                     float* __restrict__ res, uint16_t* __restrict__ next_in) {
  typedef typename YRow<YT>::raw Raw;
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const int32_t* pt = pos + t * k;
  const float* wt = w + t * k;
  const int H4 = H / 4;
  float ss = 0.0f;
  float4v rk[CPT];  // the updated residual of a one-pass row
  for (int c0 = 0; c0 < H4; c0 += 256 * CPT) {
    // every load unconditional (clamped columns and rows) so that they are in flight together:
    // latency, not bandwidth, bounds a few tokens.  Out-of-range pairs (p < 0) read row 0 and add 0.
    int cc[CPT];
    bool on[CPT];
    float4v acc[CPT], r[CPT];
    const ST* srow = shared + t * H;
    const float* rrow = RES ? res + t * H : nullptr;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = c0 + 256 * u + int(threadIdx.x);
      on[u] = c < H4;
      cc[u] = on[u] ? c : 0;
      acc[u] = YRow<ST>::cvt(reinterpret_cast<const typename YRow<ST>::raw*>(srow)[cc[u]]);  // zeroed below without a shared expert
      if constexpr (RES) r[u] = reinterpret_cast<const float4v*>(rrow)[cc[u]];
    }
    for (int j0 = 0; j0 < k; j0 += JG) {
      Raw v[JG][CPT];
      int pj[JG];
      float wj[JG];
      // the slots and weights first (uniform loads), then every row load
#pragma unroll
      for (int i = 0; i < JG; ++i) {
        const int j = min(j0 + i, k - 1);
        pj[i] = pt[j];
        wj[i] = wt[j];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < JG; ++i)
#pragma unroll
        for (int u = 0; u < CPT; ++u)
          v[i][u] = reinterpret_cast<const Raw*>(y + int64_t(pj[i] >= 0 ? pj[i] : 0) * H)[cc[u]];
      __builtin_amdgcn_sched_barrier(0);
      if (j0 == 0 && !has_shared) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) acc[u] = float4v{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < JG; ++i)
        if (j0 + i < k && pj[i] >= 0)  // pairs of out-of-range ids (p < 0) add 0
#pragma unroll
          for (int u = 0; u < CPT; ++u) {
            const float4v vf = YRow<YT>::cvt(v[i][u]);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[u][q] = __builtin_fmaf(wj[i], vf[q], acc[u][q]);
          }
    }
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      if (!on[u]) continue;
      if (out) reinterpret_cast<float4v*>(out + t * H)[cc[u]] = acc[u];
      if constexpr (RES) {
        r[u] += acc[u];
        reinterpret_cast<float4v*>(res + t * H)[cc[u]] = r[u];
        ss += sumsq4(r[u]);
        rk[u] = r[u];
      }
    }
  }
  if (!RES || !next_in) return;  // uniform across the workgroup
  if (H4 > 256 * CPT) {
    rmsnorm_row(res + t * H, H, ss, red, next_in + t * H);
    return;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float denom = sqrtf((red[0] + red[1] + red[2] + red[3]) / float(H) + 1e-6f);
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c = 256 * u + int(threadIdx.x);
    if (c >= H4) continue;
    uint16_t* dst = next_in + t * H + 4 * c;
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = f32_to_bf16_rne(rk[u][q] / denom);
  }
}

__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(const float* __restrict__ res, int H,
                                                              uint16_t* __restrict__ next_in) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const int H4 = H / 4;
  float ss = 0.0f;
  for (int c = threadIdx.x; c < H4; c += 256) ss += sumsq4(reinterpret_cast<const float4v*>(res + t * H)[c]);
  rmsnorm_row(res + t * H, H, ss, red, next_in + t * H);
}

hipError_t launch_residual_rmsnorm(const float* res, int64_t T, int H, uint16_t* next_in, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  residual_rmsnorm_kernel<<<dim3(unsigned(T)), 256, 0, stream>>>(res, H, next_in);
  return hipGetLastError();
}

template <typename YT, typename ST>
static hipError_t launch_combine_t(const YT* y_sorted, const int32_t* pair_pos, const float* topk_w,
                                   const ST* shared_out, int64_t T, int H, int k, float* out, float* residual,
                                   uint16_t* next_in, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid = dim3(unsigned(T));
  // rows standing in for a missing shared output: out or residual ([T][H] fp32, one is non-null; as
  // fp16 rows they are read within the first half of each fp32 row)
  const ST* sh = shared_out ? shared_out : reinterpret_cast<const ST*>(out ? out : residual);
  const int has_sh = shared_out != nullptr;
#define CB(JG_)                                                                                              \
  (residual ? combine_kernel<2, JG_, true, YT, ST><<<grid, 256, 0, stream>>>(y_sorted, pair_pos, topk_w, sh,      \
                                                                             has_sh, H, k, out, residual, next_in) \
            : combine_kernel<2, JG_, false, YT, ST><<<grid, 256, 0, stream>>>(y_sorted, pair_pos, topk_w, sh,     \
                                                                              has_sh, H, k, out, residual, next_in))
  if (k <= 4) CB(4);
  else if (k <= 8) CB(8);
  else if (k <= 10) CB(10);
  else CB(16);
#undef CB
  return hipGetLastError();
}

hipError_t launch_combine(const float* y_sorted, const int32_t* pair_pos, const float* topk_w,
                          const float* shared_out, int64_t T, int H, int k, float* out, float* residual,
                          uint16_t* next_in, hipStream_t stream) {
  return launch_combine_t<float, float>(y_sorted, pair_pos, topk_w, shared_out, T, H, k, out, residual, next_in,
                                        stream);
}

hipError_t launch_combine_f16y(const _Float16* y_sorted, const int32_t* pair_pos, const float* topk_w,
                               const _Float16* shared_out, int64_t T, int H, int k, float* out, float* residual,
                               uint16_t* next_in, hipStream_t stream) {
  return launch_combine_t<f16, f16>(y_sorted, pair_pos, topk_w, shared_out, T, H, k, out, residual, next_in,
                                    stream);
}

}  // namespace moe
