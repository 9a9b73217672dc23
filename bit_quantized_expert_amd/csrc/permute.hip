// Token-to-expert permutation: histogram, exclusive scan and a stable
// scatter of the (token, rank) pairs into expert-contiguous order.  This is
// this library's on-device counterpart of the per-layer partition of the 10
// selected experts ("How Strata runs a 125-billion-parameter model ...",
// Step 2, "Mapped host doorbell and a single captured CUDA graph"); here the
// IDs never leave the GPU.
//
// Pair p = t*k + j.  Within an expert's segment the pairs keep ascending p,
// so the result is unique.  IDs outside [0, E) are skipped and counted in the
// workspace header (word 0).
#include "common.h"
#include "launch.h"
#include "plan.h"

namespace moe {

// ---------------------------------------------------------------------------
// Stable placement of one batch of up to 1024 pairs (one per thread of a
// 1024-thread workgroup, pair order = thread order).  base[e] is the next
// free position of expert e and is advanced past the batch's pairs.
//   - Lanes of a wave holding the same expert find each other with one
//     ballot per bit of the expert index; a pair's rank is the number of
//     those lanes below it.
//   - The 16 waves then take turns in order: wave w reads base[e], places its
//     pairs at base[e] + rank, and the group's highest lane advances base[e]
//     (its read of the same word is an earlier instruction of the same wave).
// Only waves below nw hold pairs (the others place nothing and skip the
// turns after theirs).  Returns the pair's position, or -1 for e < 0 (an id
// outside [0, E)).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int stable_place_1024(int e, int nbits, int* base, int nw = 16) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint64_t same = __ballot(e >= 0);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bal = __ballot(bit);
    same &= bit ? bal : ~bal;
  }
  const int rank = __builtin_popcountll(same & ((1ull << lane) - 1ull));
  const bool last = (same >> lane) == 1ull;  // no higher lane of the group
  const int cnt = __builtin_popcountll(same);
  int pos = -1;
  for (int w = 0; w < nw; ++w) {
    if (wv == w && e >= 0) {
      const int b = base[e];
      pos = b + rank;
      if (last) base[e] = b + cnt;
    }
    __syncthreads();
  }
  return pos;
}

// bits of an expert index below E
__host__ __device__ __forceinline__ int expert_bits(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

// ---------------------------------------------------------------------------
// Single-workgroup permutation for small batches (P <= kSmallPairs).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void permute_small_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_pair,
                                                            int32_t* __restrict__ pair_pos,
                                                            int32_t* __restrict__ header) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int tmp[1024];
  __shared__ int err;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  if (tid == 0) err = 0;
  __syncthreads();
  for (int p = tid; p < P; p += 1024) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    else atomicAdd(&err, 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) counts[e] = cnt[e];
  const int total = block_exclusive_scan_lds(cnt, E, tmp);
  for (int e = tid; e < E; e += 1024) offsets[e] = cnt[e];
  if (tid == 0) {
    offsets[E] = total;
    header[0] = err;
  }
  __syncthreads();
  // stable scatter, 1024 pairs at a time; cnt[e] is the running base
  const int nbits = expert_bits(E);
  for (int p0 = 0; p0 < P; p0 += 1024) {
    const int p = p0 + tid;
    int e = -1;
    if (p < P) {
      e = idx[p];
      if (e < 0 || e >= E) e = -1;
    }
    const int pos = stable_place_1024(e, nbits, cnt);
    if (pos >= 0) sorted_pair[pos] = p;
    if (p < P) pair_pos[p] = pos;
  }
}

// ---------------------------------------------------------------------------
// Multi-workgroup permutation: per-chunk histograms, a column scan, and a
// stable per-chunk scatter.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ idx, int64_t P, int E,
                                                          int32_t* __restrict__ chunk_hist) {
  __shared__ int cnt[kMaxExperts + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int64_t p0 = int64_t(blockIdx.x) * kPermChunk;
  for (int i = tid; i < kPermChunk; i += 256) {
    const int64_t p = p0 + i;
    if (p >= P) break;
    const int e = idx[p];
    atomicAdd(&cnt[(e >= 0 && e < E) ? e : E], 1);
  }
  __syncthreads();
  int32_t* row = chunk_hist + int64_t(blockIdx.x) * (E + 1);
  for (int e = tid; e <= E; e += 256) row[e] = cnt[e];
}

// Column scan of the per-chunk histograms: chunk_hist[c][e] becomes the
// number of pairs of expert e in chunks before c.  Workgroup = CG experts x
// 1024 / CG chunk groups.  Column totals go to counts[e] (and, for the extra
// column E of out-of-range ids, to the header).
template <int CG>
__global__ __launch_bounds__(1024) void permute_colscan_kernel(int32_t* __restrict__ chunk_hist, int n_chunks,
                                                              int E, int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ header) {
  constexpr int RG = 1024 / CG;
  __shared__ int part[RG][CG];
  const int col = threadIdx.x % CG, grp = threadIdx.x / CG;
  const int e = blockIdx.x * CG + col;
  const int per = (n_chunks + RG - 1) / RG;
  const int c_lo = min(n_chunks, grp * per), c_hi = min(n_chunks, c_lo + per);
  int s = 0;
  if (e <= E)
    for (int c = c_lo; c < c_hi; ++c) s += chunk_hist[int64_t(c) * (E + 1) + e];
  part[grp][col] = s;
  __syncthreads();
  if (grp == 0) {
    int run = 0;
    for (int g = 0; g < RG; ++g) {
      const int v = part[g][col];
      part[g][col] = run;
      run += v;
    }
    if (e < E) counts[e] = run;
    else if (e == E) header[kHdrError] = run;
  }
  __syncthreads();
  if (e <= E) {
    int run = part[grp][col];
    for (int c = c_lo; c < c_hi; ++c) {
      int32_t* cell = chunk_hist + int64_t(c) * (E + 1) + e;
      const int v = *cell;
      *cell = run;
      run += v;
    }
  }
}

// offsets = exclusive scan of counts (one workgroup).
__global__ __launch_bounds__(1024) void offsets_scan_kernel(const int32_t* __restrict__ counts, int E,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int tmp[1024];
  for (int e = threadIdx.x; e < E; e += 1024) cnt[e] = counts[e];
  __syncthreads();
  const int total = block_exclusive_scan_lds(cnt, E, tmp);
  for (int e = threadIdx.x; e < E; e += 1024) offsets[e] = cnt[e];
  if (threadIdx.x == 0) offsets[E] = total;
}

__global__ __launch_bounds__(1024) void permute_scatter_kernel(const int32_t* __restrict__ idx, int64_t P, int E,
                                                              const int32_t* __restrict__ chunk_hist,
                                                              const int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_pair,
                                                              int32_t* __restrict__ pair_pos) {
  static_assert(kPermChunk == 1024, "one pair per thread");
  __shared__ int base[kMaxExperts];
  const int tid = threadIdx.x;
  const int32_t* row = chunk_hist + int64_t(blockIdx.x) * (E + 1);
  const int64_t p = int64_t(blockIdx.x) * kPermChunk + tid;
  int e = -1;
  if (p < P) {
    e = idx[p];
    if (e < 0 || e >= E) e = -1;
  }
  for (int i = tid; i < E; i += 1024) base[i] = offsets[i] + row[i];
  __syncthreads();
  const int pos = stable_place_1024(e, expert_bits(E), base);
  if (pos >= 0) sorted_pair[pos] = int32_t(p);
  if (p < P) pair_pos[p] = pos;
}

hipError_t launch_permute(const int32_t* idx, int64_t P, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, int32_t* header, int32_t* chunk_hist,
                          hipStream_t stream) {
  if (P <= kSmallPairs) {
    permute_small_kernel<<<1, 1024, 0, stream>>>(idx, int(P), E, counts, offsets, sorted_pair, pair_pos,
                                                 header);
    return hipGetLastError();
  }
  const int n_chunks = int((P + kPermChunk - 1) / kPermChunk);
  permute_hist_kernel<<<n_chunks, 256, 0, stream>>>(idx, P, E, chunk_hist);
  permute_colscan_kernel<64><<<(E + 1 + 63) / 64, 1024, 0, stream>>>(chunk_hist, n_chunks, E, counts, header);
  offsets_scan_kernel<<<1, 1024, 0, stream>>>(counts, E, offsets);
  permute_scatter_kernel<<<n_chunks, 1024, 0, stream>>>(idx, P, E, chunk_hist, offsets, sorted_pair, pair_pos);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The prefill layer's selection, permutation and plan in three launches (the
// stepwise calls keep the kernels above).  A chunk is kSelChunk consecutive
// tokens (at most 16 k <= 512 pairs):
//   1. select_hist_kernel: one workgroup per chunk, one wave per token: the
//      top-k and weights (the wave routines every path shares) and the
//      chunk's histogram row; a second workgroup per chunk writes the fp16
//      operand copy of the chunk's activations for the grouped GEMM (the x16
//      layout: permuted 16-groups);
//   2. permute_colscan_kernel over the chunk rows;
//   3. scatter_plan_kernel: one workgroup per chunk scans the counts into
//      offsets itself, then places the chunk's pairs (stable: ascending pair
//      index within each expert, the result of launch_permute); one more
//      workgroup writes the offsets and the plan (plan.h).
// ---------------------------------------------------------------------------
constexpr int kSelChunk = 16;

template <int V, typename XT>
__global__ __launch_bounds__(1024) void select_hist_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                          int k, int32_t* __restrict__ idx_out,
                                                          float* __restrict__ w_out, int32_t* __restrict__ chunk_hist,
                                                          const XT* __restrict__ x, int H, f16* __restrict__ x16,
                                                          int nc) {
  __shared__ int cnt[kMaxExperts + 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (int(blockIdx.x) >= nc) {  // workgroups nc..2nc-1: the fp16 copy of chunk blockIdx - nc's activations
    const int64_t t0 = int64_t(blockIdx.x - nc) * kSelChunk;
    const int64_t g0 = t0 * (H / 16);
    const int ng = int(min(int64_t(kSelChunk), T - t0)) * (H / 16);
    for (int g = tid; g < ng; g += 1024) {
      half8 lo, hi;
      load_x16<XT>(x + (g0 + g) * 16, lo, hi);
      half8* d = reinterpret_cast<half8*>(x16 + (g0 + g) * 16);
      d[0] = lo;
      d[1] = hi;
    }
    return;
  }
  const int64_t t0 = int64_t(blockIdx.x) * kSelChunk;
  const int nt = int(min(int64_t(kSelChunk), T - t0));
  for (int e = tid; e <= E; e += 1024) cnt[e] = 0;
  __syncthreads();
  if (wv < nt) {
    const int64_t t = t0 + wv;
    int my_idx;
    float my_w;
    wave_topk_softmax<V>(logits + t * E, E, k, my_idx, my_w);
    if (lane < k) {
      idx_out[t * k + lane] = my_idx;
      w_out[t * k + lane] = my_w;
      atomicAdd(&cnt[my_idx], 1);
    }
  }
  __syncthreads();
  int32_t* row = chunk_hist + int64_t(blockIdx.x) * (E + 1);
  for (int e = tid; e <= E; e += 1024) row[e] = cnt[e];  // column E (ids out of range) stays 0
}

__global__ __launch_bounds__(1024) void scatter_plan_kernel(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                           const int32_t* __restrict__ chunk_hist,
                                                           const int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_pair,
                                                           int32_t* __restrict__ pair_pos, PlanOut plan, int nc) {
  __shared__ int base[kMaxExperts + 1];
  __shared__ int flag[kMaxExperts];
  __shared__ int ntile[kMaxExperts];
  __shared__ int tmp[16];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) base[e] = counts[e];
  __syncthreads();
  const int total = block_scan_fast(base, E, tmp);
  if (blockIdx.x == nc) {  // the extra workgroup: offsets and the plan
    if (tid == 0) base[E] = total;
    __syncthreads();
    for (int e = tid; e <= E; e += 1024) offsets[e] = base[e];
    plan_from_offsets(base, E, T, plan.has_shared, plan.tile_bm, plan.header, plan.slots, plan.tile_desc,
                      plan_slots(E, T), nullptr, k, flag, ntile, tmp);
    return;
  }
  const int32_t* row = chunk_hist + int64_t(blockIdx.x) * (E + 1);
  for (int e = tid; e < E; e += 1024) base[e] += row[e];
  const int64_t p0 = int64_t(blockIdx.x) * kSelChunk * k;
  const int np = int(min(int64_t(kSelChunk), T - int64_t(blockIdx.x) * kSelChunk)) * k;
  const int64_t p = p0 + tid;
  int e = -1;
  if (tid < np) {
    e = idx[p];
    if (e < 0 || e >= E) e = -1;
  }
  __syncthreads();
  const int pos = stable_place_1024(e, expert_bits(E), base, (np + 63) / 64);
  if (pos >= 0) sorted_pair[pos] = int32_t(p);
  if (tid < np) pair_pos[p] = pos;
}

int select_chunks(int64_t T) { return int((T + kSelChunk - 1) / kSelChunk); }

hipError_t launch_select_plan(const float* logits, const void* x, int x_kind, int64_t T, int H, int E, int k,
                              int32_t* idx, float* w, int32_t* chunk_hist, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_pair, int32_t* pair_pos, f16* x16, const PlanOut& plan,
                              hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (k < 1 || k * kSelChunk > 1024 || H % 16 != 0) return hipErrorInvalidValue;
  const int nc = select_chunks(T);
  const int v = (E + 63) / 64;
#define SH(V_, XT_)                                                                                       \
  select_hist_kernel<V_, XT_><<<2 * nc, 1024, 0, stream>>>(logits, T, E, k, idx, w, chunk_hist,            \
                                                           static_cast<const XT_*>(x), H, x16, nc)
#define SHX(V_)                       \
  if (x_kind == kXBF16) SH(V_, uint16_t); \
  else if (x_kind == kXF16) SH(V_, f16);  \
  else SH(V_, float)
  if (v <= 1) { SHX(1); }
  else if (v <= 2) { SHX(2); }
  else if (v <= 4) { SHX(4); }
  else if (v <= 8) { SHX(8); }
  else if (v <= 16) { SHX(16); }
  else if (v <= 32) { SHX(32); }
  else { SHX(64); }
#undef SHX
#undef SH
  permute_colscan_kernel<16><<<(E + 1 + 15) / 16, 1024, 0, stream>>>(chunk_hist, nc, E, counts, plan.header);
  scatter_plan_kernel<<<nc + 1, 1024, 0, stream>>>(idx, T, k, E, chunk_hist, counts, offsets, sorted_pair, pair_pos,
                                                   plan, nc);
  return hipGetLastError();
}

}  // namespace moe
