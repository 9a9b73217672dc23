// Decode-layer selection on a single workgroup (T <= 16 tokens): top-k with
// renormalised softmax weights, the stable token-to-expert permutation and
// the slot table of the expert FFN -- everything between the router logits
// and the expert FFN in one launch.  Same rules as the standalone kernels:
// ranks ordered by router weight with ties to the lower expert index ("How
// Strata runs a 125-billion-parameter model ...", Step 2, "Verify-window
// route tail skip"), pairs grouped by expert in ascending (token, rank) order.
#include <limits.h>

#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kSelMaxT = 16;
static_assert(kMaxTopK <= kMaxTopKLds, "the wave top-k ranks at most kMaxTopKLds entries");

template <int V>
__global__ __launch_bounds__(1024) void select_small_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                           int has_shared, int32_t* __restrict__ idx_out,
                                                           float* __restrict__ w_out, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_pair,
                                                           int32_t* __restrict__ pair_pos,
                                                           int32_t* __restrict__ header, int4* __restrict__ slots) {
  __shared__ int cnt[kMaxExperts];
  __shared__ uint32_t tmask[kMaxExperts];  // bit t: token t chose the expert
  __shared__ int tmp[16];
  __shared__ int s_idx[kSelMaxT * kMaxTopK];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += 1024) {
    cnt[e] = 0;
    tmask[e] = 0u;
  }

  // ---- top-k of token wv (one wave per token)
  if (wv < T) {
    int my_idx;
    float my_w;
    wave_topk_softmax<V>(logits + int64_t(wv) * E, E, k, my_idx, my_w);
    if (lane < k) {
      idx_out[wv * k + lane] = my_idx;
      w_out[wv * k + lane] = my_w;
      s_idx[wv * k + lane] = my_idx;
    }
  }
  __syncthreads();

  // ---- histogram; then one scan of (count | active << 16): the low half
  // gives the offsets, the high half the slot of each active expert
  // (counts <= 1024 and active experts <= 4096, so neither half carries)
  const int P = T * k;
  for (int p = threadIdx.x; p < P; p += 1024) {
    atomicAdd(&cnt[s_idx[p]], 1);
    atomicOr(&tmask[s_idx[p]], 1u << (p / k));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 1024) {
    const int c = cnt[e];
    counts[e] = c;
    cnt[e] = c | (c > 0 ? 1 << 16 : 0);
  }
  __syncthreads();
  const int packed_total = block_scan_fast(cnt, E, tmp);
  const int total = packed_total & 0xffff, n_active = packed_total >> 16;
  for (int e = threadIdx.x; e < E; e += 1024) {
    const int off = cnt[e] & 0xffff;
    offsets[e] = off;
    const uint32_t m = tmask[e];  // a token picks an expert at most once: count = popcount
    if (m != 0u) slots[cnt[e] >> 16] = int4{e, off, __builtin_popcount(m), int(m)};
  }
  if (threadIdx.x == 0) offsets[E] = total;

  // ---- stable scatter (P <= 1024: one pair per thread).  The pairs of
  // expert e before pair (t, j) are those of the earlier tokens in e's token
  // mask.
  if (threadIdx.x < P) {
    const int p = threadIdx.x;
    const int e = s_idx[p];
    const int t = p / k;
    const int pos = (cnt[e] & 0xffff) + __builtin_popcount(tmask[e] & ((1u << t) - 1u));
    sorted_pair[pos] = p;
    pair_pos[p] = pos;
  }

  // ---- slot table tail: the shared expert after the active ones
  const int n_valid = n_active + (has_shared ? 1 : 0);
  if (threadIdx.x == 0) {
    if (has_shared) slots[n_active] = int4{-1, 0, T, int((1u << T) - 1u)};
    header[kHdrError] = 0;
    header[kHdrActive] = n_active;
    header[kHdrValid] = n_valid;
  }
  // slots past the valid ones are empty (m = 0) so any grid size is safe
  const int n_slots = min(E, P) + 1;
  for (int s = n_valid + threadIdx.x; s < n_slots; s += 1024) slots[s] = int4{0, 0, 0, 0};
}

hipError_t launch_select_small(const float* logits, int T, int E, int k, int has_shared, int32_t* idx, float* w,
                               int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                               int32_t* header, int4* slots, hipStream_t stream) {
  if (T > kSelMaxT || T * k > 1024) return hipErrorInvalidValue;
  const int v = (E + 63) / 64;
#define SEL(V_)                                                                                                \
  select_small_kernel<V_><<<1, 1024, 0, stream>>>(logits, T, E, k, has_shared, idx, w, counts, offsets,      \
                                                  sorted_pair, pair_pos, header, slots)
  if (v <= 1) SEL(1);
  else if (v <= 2) SEL(2);
  else if (v <= 4) SEL(4);
  else if (v <= 8) SEL(8);
  else if (v <= 16) SEL(16);
  else if (v <= 32) SEL(32);
  else SEL(64);
#undef SEL
  return hipGetLastError();
}

}  // namespace moe
