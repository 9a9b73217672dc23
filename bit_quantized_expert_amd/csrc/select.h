// Decode-layer selection inside one workgroup (T <= 16 tokens): top-k with
// renormalised softmax weights, the stable token-to-expert permutation and
// the slot table of the expert FFN.  Same rules as the standalone kernels:
// ranks ordered by router weight with ties to the lower expert index ("How
// Strata runs a 125-billion-parameter model ...", Step 2, "Verify-window
// route tail skip"), pairs grouped by expert in ascending (token, rank) order.
//
// Two users: the one-workgroup selection kernel, and the persistent gate/up
// kernel of 2..16-token layers, whose workgroups each make the selection
// themselves (one of them also writes it out) instead of waiting for a
// separate launch.  The result is a pure function of the logits, so every
// workgroup finds the same one.
#pragma once

#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kSelMaxT = 16;

// Where the selection goes (workgroup `write` only).
struct SelOut {
  const float* logits;  // [T][E] router logits
  int32_t* idx;         // [T][k] experts, rank order
  float* w;             // [T][k] weights, rank order
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E + 1]
  int32_t* sorted_pair; // [T k]
  int32_t* pair_pos;    // [T k]
  int32_t* header;      // workspace header: error, active, valid
  int4* slots;          // slot table (min(E, T k) + 1 entries)
  int kc;               // route tail skip: an expert is computed only if some token ranks it
                        // below kc (0 or >= k: every selected expert is computed)
};

// LDS of the selection for up to EMAX experts and NW waves.
template <int EMAX, int NW>
struct SelLds {
  int cnt[EMAX];          // count | active << 16, then (scanned) offset | slot << 16
  uint32_t tmask[EMAX];   // bit t: token t chose the expert (a token picks an expert at most once)
  uint32_t hmask[EMAX];   // route tail skip: bit t: token t ranks the expert below kc
  uint16_t slot_e[EMAX];  // expert of active slot s
  int tmp[NW];
};

// Ranking scratch of one wave (the writing workgroup only; a caller may
// overlay it on LDS it uses after the selection).
typedef uint2 SelRankLds[2][kMaxTopKLds];

// Runs on all 64 NW threads of the workgroup; returns the number of active
// experts (uniform).  tk: NW wave scratches.  On return S.cnt[e] & 0xffff is e's first sorted
// position, S.tmask[e] its token mask and S.slot_e[s] the expert of active
// slot s (slots in ascending expert order; the shared expert, if any, is slot
// n_active).  V: key registers per lane (E <= 64 V <= EMAX).
template <int V, int NW, int EMAX>
__device__ int select_in_workgroup(const SelOut& o, int T, int E, int k, int has_shared, SelLds<EMAX, NW>& S,
                                   SelRankLds* tk, bool write) {
  constexpr int NT = 64 * NW;
  constexpr int TPW = (kSelMaxT + NW - 1) / NW;  // tokens per wave
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // route tail skip ("How Strata runs a 125-billion-parameter model ...",
  // Step 2, "Verify-window route tail skip"): an expert that no token ranks
  // below kc is dropped (its pairs add nothing); the selection, ranks and
  // weights written out are those of the full top-k
  const bool skip = o.kc > 0 && o.kc < k;
  for (int e = threadIdx.x; e < E; e += NT) {
    S.tmask[e] = 0u;
    if (skip) S.hmask[e] = 0u;
  }
  __syncthreads();

  // ---- top-k of tokens wv, wv + NW, ... (one wave per token at a time).
  // The logits of all of the wave's tokens are loaded first, so that their
  // loads are in flight together (a wave past the last token reloads it).
  float f[TPW][V];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const float* row = o.logits + int64_t(min(wv + NW * i, T - 1)) * E;
#pragma unroll
    for (int v = 0; v < V; ++v) f[i][v] = row[min(lane + 64 * v, E - 1)];
  }
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int v = 0; v < V; ++v) asm volatile("" : "+v"(f[i][v]));  // every load unconditional
  int my_idx[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = wv + NW * i;
    my_idx[i] = 0;
    if (t >= T) continue;  // uniform per wave
    WaveKeys<V> K;
#pragma unroll
    for (int v = 0; v < V; ++v) K.key[v] = lane + 64 * v < E ? float_key(f[i][v]) : 0u;
    uint64_t msel[V];
    wave_select<V>(K, k, msel);
#pragma unroll
    for (int v = 0; v < V; ++v)
      if ((msel[v] >> lane) & 1ull) atomicOr(&S.tmask[lane + 64 * v], 1u << t);
    if (skip) {  // the token's head ranks 0 .. kc - 1: its top-kc
      uint64_t mhead[V];
      wave_select<V>(K, o.kc, mhead);
#pragma unroll
      for (int v = 0; v < V; ++v)
        if ((mhead[v] >> lane) & 1ull) atomicOr(&S.hmask[lane + 64 * v], 1u << t);
    }
    if (write) {  // ranks and weights: only the workgroup that writes them out
      float my_val;
      int my_slot;
      wave_rank_s<V>(K, msel, k, tk[wv], my_val, my_idx[i], my_slot);
      const float my_w = wave_topk_weight(my_val, k);
      if (lane < k) {
        o.idx[t * k + lane] = my_idx[i];
        o.w[t * k + lane] = my_w;
      }
    }
  }
  __syncthreads();

  // ---- one scan of (count | active << 16): the low half gives the
  // offsets, the high half the slot of each active expert (counts <= 16 T
  // and active experts <= EMAX <= 4096, so neither half carries)
  auto count_of = [&](int e, uint32_t& m) {
    const bool active = skip ? S.hmask[e] != 0u : S.tmask[e] != 0u;
    if (skip && !active) S.tmask[e] = 0u;  // a dropped expert: no pairs, no slot
    m = S.tmask[e];
    const int c = __builtin_popcount(m);
    if (write) o.counts[e] = c;
    return c | (c > 0 ? 1 << 16 : 0);
  };
  auto place = [&](int e, uint32_t m, int sc) {  // sc: e's scanned (offset | slot << 16)
    if (m != 0u) S.slot_e[sc >> 16] = uint16_t(e);
    if (write) {
      const int off = sc & 0xffff;
      o.offsets[e] = off;
      if (m != 0u) o.slots[sc >> 16] = int4{e, off, __builtin_popcount(m), int(m)};
    }
  };
  int packed_total;
  if (E <= NT) {
    // one expert per thread: the count, the scan and the placement in one
    // pass with a single barrier (the wave totals)
    const int e = threadIdx.x;
    uint32_t m = 0u;
    const int v = e < E ? count_of(e, m) : 0;
    const int incl = wave_incl_scan(v);
    if (lane == 63) S.tmp[wv] = incl;
    __syncthreads();
    int base = 0;
    packed_total = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      const int t2 = S.tmp[w2];
      base += w2 < wv ? t2 : 0;
      packed_total += t2;
    }
    if (e < E) {
      const int sc = base + incl - v;
      S.cnt[e] = sc;
      place(e, m, sc);
    }
    if (write) __syncthreads();  // the scatter below reads other experts' offsets (uniform: write is)
  } else {
    for (int e = threadIdx.x; e < E; e += NT) {
      uint32_t m;
      S.cnt[e] = count_of(e, m);
    }
    __syncthreads();
    packed_total = block_scan_fast<NT>(S.cnt, E, S.tmp);
    for (int e = threadIdx.x; e < E; e += NT) place(e, S.tmask[e], S.cnt[e]);
    if (write) __syncthreads();
  }
  const int total = packed_total & 0xffff, n_active = packed_total >> 16;
  if (write) {
    if (threadIdx.x == 0) o.offsets[E] = total;
    // stable scatter: the pairs of expert e before pair (t, j) are those of
    // the earlier tokens in e's token mask
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + NW * i;
      if (t < T && lane < k) {
        const int e = my_idx[i], p = t * k + lane;
        if (S.tmask[e] == 0u) {  // dropped by the route tail skip: the combine adds nothing for it
          o.pair_pos[p] = -1;
        } else {
          const int pos = (S.cnt[e] & 0xffff) + __builtin_popcount(S.tmask[e] & ((1u << t) - 1u));
          o.sorted_pair[pos] = p;
          o.pair_pos[p] = pos;
        }
      }
    }
    // slot table tail: the shared expert after the active ones; slots past
    // the valid ones are empty (count 0) so any grid size is safe
    const int n_valid = n_active + (has_shared ? 1 : 0);
    if (threadIdx.x == 0) {
      if (has_shared) o.slots[n_active] = int4{-1, 0, T, int((1u << T) - 1u)};
      o.header[kHdrError] = 0;
      o.header[kHdrActive] = n_active;
      o.header[kHdrValid] = n_valid;
    }
    const int n_slots = min(E, T * k) + 1;
    for (int s2 = n_valid + int(threadIdx.x); s2 < n_slots; s2 += NT) o.slots[s2] = int4{0, 0, 0, 0};
  }
  __syncthreads();  // slot_e and the scanned counts are visible
  return n_active;
}

}  // namespace moe
