// Decode-layer selection on a single workgroup (T <= 16 tokens): top-k with
// renormalised softmax weights, the stable token-to-expert permutation and
// the slot table of the expert FFN -- everything between the router logits
// and the expert FFN in one launch.  Same rules as the standalone kernels:
// ranks ordered by router weight with ties to the lower expert index ("How
// Strata runs a 125-billion-parameter model ...", Step 2, "Verify-window
// route tail skip"), pairs grouped by expert in ascending (token, rank) order.
#include "select.h"

namespace moe {

static_assert(kMaxTopK <= kMaxTopKLds, "the wave top-k ranks at most kMaxTopKLds entries");

template <int V>
__global__ __launch_bounds__(1024) void select_small_kernel(SelOut o, int T, int E, int k, int has_shared) {
  __shared__ SelLds<kMaxExperts, 16> S;
  __shared__ SelRankLds tk[16];
  select_in_workgroup<V, 16, kMaxExperts>(o, T, E, k, has_shared, S, tk, true);
}

hipError_t launch_select_small(const float* logits, int T, int E, int k, int has_shared, int32_t* idx, float* w,
                               int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                               int32_t* header, int4* slots, int kc, hipStream_t stream) {
  if (T > kSelMaxT || T * k > 1024) return hipErrorInvalidValue;
  const int v = (E + 63) / 64;
  const SelOut o{logits, idx, w, counts, offsets, sorted_pair, pair_pos, header, slots, kc};
#define SEL(V_) select_small_kernel<V_><<<1, 1024, 0, stream>>>(o, T, E, k, has_shared)
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
