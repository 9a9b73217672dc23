// The per-call plan of the expert FFN, made from the expert segments of the
// permutation by one 1024-thread workgroup:
//   * slot table: the active experts in ascending id order, then the shared
//     expert, each int4 {expert or -1, first sorted position, rows, token
//     mask (T <= kGemvMaxM with sorted_pair given, else 0)}; slots past the
//     last valid one are zeroed;
//   * grouped-GEMM tile list (tile_bm > 0): int4 {expert (-1 = shared), first
//     row of the tile in the expert's rows, first sorted row (for the shared
//     expert: the first token), rows of the tile} of every tile_bm-row tile
//     of each expert's segment, then the shared expert's;
//   * header words: active experts, valid slots, tiles (the error word
//     belongs to the permutation and is left as it is).
#pragma once
#include "common.h"
#include "launch.h"

namespace moe {

// offsets: E + 1 ints (global or LDS); flag, ntile: E ints of LDS scratch;
// tmp: 16 ints of LDS.
__device__ inline void plan_from_offsets(const int32_t* offsets, int E, int64_t T, int has_shared, int tile_bm,
                                         int32_t* __restrict__ header, int4* __restrict__ slots,
                                         int4* __restrict__ tile_desc, int n_slots, const int32_t* __restrict__ sorted_pair, int k, int* flag,
                                         int* ntile, int* tmp) {
  for (int e = threadIdx.x; e < E; e += 1024) {
    const int c = offsets[e + 1] - offsets[e];
    flag[e] = c > 0;
    ntile[e] = tile_bm > 0 ? (c + tile_bm - 1) / tile_bm : 0;
  }
  __syncthreads();
  const int n_active = block_scan_fast(flag, E, tmp);
  const int n_routed_tiles = block_scan_fast(ntile, E, tmp);
  for (int e = threadIdx.x; e < E; e += 1024) {
    const int lo = offsets[e];
    const int c = offsets[e + 1] - lo;
    if (c > 0) {
      // token mask of the slot for small batches (the GEMV kernels then know
      // the slot's tokens without reading sorted_pair); 0 = not given.  Pair
      // ids that are not those of a permutation of T * k pairs cannot make a
      // correct result; their tokens are clamped into [0, T) so that no
      // kernel reads outside the activations.
      uint32_t mask = 0u;
      if (sorted_pair && T <= kGemvMaxM) {
        for (int q = lo; q < lo + c; ++q) {
          const int t = min(max(sorted_pair[q] / k, 0), int(T) - 1);
          mask |= 1u << t;
        }
      }
      slots[flag[e]] = int4{e, lo, c, int(mask)};
    }
    if (tile_bm > 0) {
      int pos = ntile[e];
      for (int m0 = 0; m0 < c; m0 += tile_bm, ++pos) tile_desc[pos] = int4{e, m0, lo + m0, min(tile_bm, c - m0)};
    }
  }
  const int n_valid = n_active + (has_shared ? 1 : 0);
  if (threadIdx.x == 0 && has_shared)
    slots[n_active] = int4{-1, 0, int(T), sorted_pair && T <= kGemvMaxM ? int((1u << T) - 1u) : 0};
  for (int s = n_valid + threadIdx.x; s < n_slots; s += 1024) slots[s] = int4{0, 0, 0, 0};
  int n_tiles = n_routed_tiles;
  if (tile_bm > 0 && has_shared) {
    const int st = int((T + tile_bm - 1) / tile_bm);
    for (int i = threadIdx.x; i < st; i += 1024)
      tile_desc[n_routed_tiles + i] = int4{-1, i * tile_bm, i * tile_bm, int(min(int64_t(tile_bm), T - i * tile_bm))};
    n_tiles += st;
  }
  if (threadIdx.x == 0) {
    header[kHdrActive] = n_active;
    header[kHdrValid] = n_valid;
    header[kHdrTiles] = n_tiles;
  }
}

// Slots the plan writes for T tokens: min(E, T * k) + 1 for every k <= 32.
__host__ __device__ inline int plan_slots(int E, int64_t T) {
  return int(T * 32 < int64_t(E) ? T * 32 : int64_t(E)) + 1;
}

}  // namespace moe
