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
// round.  Codes are unpacked in registers to fp16 c*s (exact at 2 bits; see dq2_word);
// the activations sit in LDS as fp16 in the matching permuted order.  One
// workgroup = 4 waves = 64 rows of one expert (or of the shared expert).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "plan.h"
#include "select.h"

namespace moe {

// ---------------------------------------------------------------------------
// Plan: slot table and grouped-GEMM tile list from offsets (plan.h).  One
// workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int E, int64_t T,
                                                   int has_shared, int tile_bm, int32_t* __restrict__ header,
                                                   int4* __restrict__ slots, int4* __restrict__ tile_desc, int n_slots,
                                                   const int32_t* __restrict__ sorted_pair, int k) {
  __shared__ int flag[kMaxExperts];
  __shared__ int ntile[kMaxExperts];
  __shared__ int tmp[16];
  plan_from_offsets(offsets, E, T, has_shared, tile_bm, header, slots, tile_desc, n_slots, sorted_pair, k, flag,
                    ntile, tmp);
}

hipError_t launch_plan(const int32_t* offsets, int E, int64_t T, int has_shared, int tile_bm, int32_t* header,
                       int4* slots, int4* tile_desc, const int32_t* sorted_pair, int k,
                       hipStream_t stream) {
  const int n_slots = plan_slots(E, T);
  plan_kernel<<<1, 1024, 0, stream>>>(offsets, E, T, has_shared, tile_bm, header, slots, tile_desc, n_slots,
                                      sorted_pair, k);
  return hipGetLastError();
}

// One quantised unit of a row: UNIT = 64 weights (16 code bytes, 2 scales)
// or 32 (8 code bytes, 1 scale).  3-bit adds UNIT/32 high-plane words (one
// bit per code), 4-bit UNIT/16 (two bits per code, the low plane's layout).
template <int QBITS, int UNIT>
struct Unit {
  uint32_t w[UNIT / 16];                               // low-plane words, 16 codes each
  uint32_t h[QBITS == 4 ? UNIT / 16 : UNIT / 32];      // high-plane words (3- and 4-bit only)
  uint32_t s;                                          // fp16 scale bits (two for UNIT = 64)
};

// Unit u of row `row` of a matrix of `rows` rows in the tiled layout of
// common.h (rows are multiples of 32, so every 16-row group is full; UNIT 64
// is used only when K % 64 == 0, so its units are whole 64-weight units).
template <int QBITS, int UNIT>
__device__ __forceinline__ void load_unit(Unit<QBITS, UNIT>& U, const uint8_t* codes, const uint16_t* scales,
                                          int rows, int K, int row, int u) {
  const QTile tl = qtile<true>(row, rows);
  const int blk = UNIT == 64 ? 2 * u : u;
  const uint8_t* lo = codes + qt_code_off(tl, K, blk);
  if constexpr (UNIT == 64) {
    const uint4v c = *reinterpret_cast<const uint4v*>(lo);
    U.w[0] = c[0]; U.w[1] = c[1]; U.w[2] = c[2]; U.w[3] = c[3];
    U.s = *reinterpret_cast<const uint32_t*>(scales + qt_scale_off(tl, K, blk));
  } else {
    const uint2v c = *reinterpret_cast<const uint2v*>(lo);
    U.w[0] = c[0]; U.w[1] = c[1];
    U.s = scales[qt_scale_off(tl, K, blk)];
  }
  if constexpr (QBITS == 3) {
    const uint8_t* hp = codes + int64_t(rows) * (K / 4) + qt_high_off(tl, K, blk);
    if constexpr (UNIT == 64) {
      const uint2v hv = *reinterpret_cast<const uint2v*>(hp);
      U.h[0] = hv[0]; U.h[1] = hv[1];
    } else {
      U.h[0] = *reinterpret_cast<const uint32_t*>(hp);
    }
  }
  if constexpr (QBITS == 4) {
    const uint8_t* hp = codes + int64_t(rows) * (K / 4) + qt_code_off(tl, K, blk);
    if constexpr (UNIT == 64) {
      const uint4v hv = *reinterpret_cast<const uint4v*>(hp);
      U.h[0] = hv[0]; U.h[1] = hv[1]; U.h[2] = hv[2]; U.h[3] = hv[3];
    } else {
      const uint2v hv = *reinterpret_cast<const uint2v*>(hp);
      U.h[0] = hv[0]; U.h[1] = hv[1];
    }
  }
}

template <int QBITS, int UNIT>
__device__ __forceinline__ void zero_unit(Unit<QBITS, UNIT>& U) {
#pragma unroll
  for (int i = 0; i < UNIT / 16; ++i) U.w[i] = 0;
#pragma unroll
  for (int i = 0; i < int(sizeof(U.h) / sizeof(U.h[0])); ++i) U.h[i] = 0;
  U.s = 0;  // zero scale: every dequantised weight is 0
}

// Dequantise word d (16 codes) of a unit into two permuted MFMA k-slices.
template <int QBITS, int UNIT>
__device__ __forceinline__ void dq_unit_word(const Unit<QBITS, UNIT>& U, int d, half8& lo, half8& hi) {
  const uint32_t sbits = (UNIT == 64 && d >= 2) ? (U.s >> 16) : (U.s & 0xffffu);
  const half2v s2 = as_half2(sbits | (sbits << 16));
  if constexpr (QBITS == 2) {
    dq2_word(U.w[d], s2, lo, hi);
  } else if constexpr (QBITS == 4) {
    dq4_word(U.w[d], U.h[d], s2, lo, hi);
  } else {
    uint32_t hlo, hhi;
    high3_slots(U.h[d >> 1], d & 1, hlo, hhi);
    dq3_word(U.w[d], hlo, hhi, s2, lo, hi);
  }
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// Single-token gate/up + SwiGLU.  grid = (ceil(max_rows / 16), slots),
// block = 512.
//
// Unit u of a row (64 or 32 weights) is read in round r' = u / 4 by lane
// group g = u % 4.  Rounds fall in four classes c = r' % 4: waves 0..3 take
// the rounds of classes 0..3 of the workgroup's 16 gate rows, waves 4..7 the
// same for the up rows (the reduction axis split four ways and the two
// matrices apart: eight waves for one token), and the partial sums meet in
// LDS as ((c0 + c1) + c2) + c3 -- the order of the multi-token kernels, so a
// token's result does not depend on the batch.  The token is requested
// before anything else and converted to fp16 once per workgroup into LDS;
// every lane reads it as its MFMA row (only row 0 of the result is used).
// h is written in the permuted column order of the down projection.
//
// Slot source.  With `sl.logits` null, slot s of the slot table (standalone
// expert FFN: h row = the pair's sorted position).  With `sl.logits` set (the
// fused decode layer), every wave finds the token's selected set itself from
// the router logits (the shared selection routines, so the experts and
// weights are those of every other path): slot j < k is the j-th selected
// expert in ascending expert order, h row j; slot k is the shared expert.
// The ranking and the weights stay off that path: one wave of workgroup
// (0, 0) computes them while its weight loads are in flight and stores the
// rank-ordered selection and the rank <-> slot maps.
// ---------------------------------------------------------------------------
constexpr int k1tokWaves = 8;  // waves per workgroup of the single-token gate/up kernel

template <int QBITS, int UNIT, typename XT>
__global__ __launch_bounds__(64 * k1tokWaves) void gemv_gateup_1tok_kernel(FfnArgs a, Decode1Sel sl,
                                                                           const int4* __restrict__ slots) {
  // slots = a.slots, read-only here: the slot entry is a scalar load
  extern __shared__ __attribute__((aligned(16))) f16 xs1[];  // the token, fp16, permuted 16-groups
  __shared__ float red[4][2][16];
  constexpr int RB = 2;  // rounds per wave per load batch (rounds c and c + 4)
  constexpr int NT = 64 * k1tokWaves;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int ks = wv & 3, mat = wv >> 2;  // class ks; matrix 0 = gate, 1 = up
  const int n = lane & 15, g = lane >> 4;
  const int j = blockIdx.y;
  const int H = a.H;
  const int n_units = H / UNIT, rounds = (n_units + 3) / 4;
  const XT* xg = static_cast<const XT*>(a.x);

  // the token's first 16-groups, independent of the slot: raw loads now,
  // conversion into LDS once the weight loads are out
  const int ngrp = H / 16;
  Raw16<XT> xr;
  const int g0 = min(int(threadIdx.x), ngrp - 1);
  load_raw16(xg + g0 * 16, xr);

  bool shared;
  int64_t ex;
  int hrow;
  WaveKeys<8> K;
  uint64_t sel[8];
  bool rank_here = false;  // the one wave that also ranks the selection and stores it
  // route tail skip: the slots are the token's top-kc experts (ranks below
  // kc); ranks, weights and the selection written out stay those of the top-k
  const int kc = sl.kc > 0 && sl.kc < a.k ? sl.kc : a.k;
  if (sl.logits) {
    shared = j >= kc;
    if (blockIdx.x * 16 >= (shared ? a.Is : a.I)) return;
    ex = 0;
    hrow = shared ? 0 : j;
    if (!shared) {
      // one wave selects (the selection's ballot counts run on the CU's one
      // scalar unit, so several waves would queue behind each other there)
      __shared__ int s_ex;
      if (wv == 0) {
        wave_keys<8>(sl.logits, a.E, K);
        wave_select<8>(K, kc, sel);
        const int e = wave_nth_selected<8>(sel, j);  // slot j: the j-th selected expert in index order
        if (lane == 0) s_ex = e;
      }
      __syncthreads();
      ex = s_ex;
      rank_here = blockIdx.x == 0 && j == 0 && wv == 0;
    }
  } else {
    const int4 si = slots[j];
    if (si.z == 0) return;
    shared = si.x < 0;
    if (blockIdx.x * 16 >= (shared ? a.Is : a.I)) return;
    ex = shared ? 0 : si.x;
    hrow = shared ? 0 : si.y;
  }
  const int rows = shared ? a.Is : a.I;
  const int row = blockIdx.x * 16 + n;  // rows are multiples of 32: every row of the tile exists
  const QMat M = shared ? (mat == 0 ? a.sg : a.su) : (mat == 0 ? a.rg : a.ru);
  const uint8_t* wc = M.codes + ex * M.code_stride;
  const uint16_t* wsc = M.scales + ex * M.scale_stride;

  Unit<QBITS, UNIT> uw[RB];
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  // batch b0 (rounds (b0 + i) * 4 + ks): unconditional loads from a clamped
  // unit (a load under a branch costs a wait for every load in flight)
  auto issue = [&](int b0) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int rp = (b0 + i) * 4 + ks, u = rp * 4 + g;
      load_unit(uw[i], wc, wsc, rows, H, row, rp < rounds && u < n_units ? u : 0);
    }
  };
  // every lane reads the token's fragment (MFMA rows 1..15 repeat row 0;
  // only row 0 of the result is used)
  auto compute = [&](int b0) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int rp = (b0 + i) * 4 + ks;
      if (rp >= rounds) break;
      const int u = rp * 4 + g;
      const int ua = u < n_units ? u : 0;
      if (u >= n_units) zero_unit(uw[i]);  // units past K: zero weights
#pragma unroll
      for (int d = 0; d < UNIT / 16; ++d) {
        const half8* ap = reinterpret_cast<const half8*>(xs1 + ua * UNIT + 16 * d);
        half8 wlo, whi;
        dq_unit_word(uw[i], d, wlo, whi);
        acc = mfma16(ap[0], wlo, acc);
        acc = mfma16(ap[1], whi, acc);
      }
    }
  };
  issue(0);
  __builtin_amdgcn_sched_barrier(0);  // the first weight loads go out before anything waits on the token loads
  if (rank_here) {
    // ranks, weights and the slot maps, while this wave's weight loads are in flight
    float my_val;
    int my_idx, my_slot;
    if (kc == a.k) {
      wave_rank<8>(K, sel, a.k, my_val, my_idx, my_slot);
    } else {
      // the full top-k for the ranks and weights; a rank below kc is slot
      // (the number of the top-kc experts with a lower index)
      uint64_t selk[8];
      wave_select<8>(K, a.k, selk);
      wave_rank<8>(K, selk, a.k, my_val, my_idx, my_slot);
      const int v = my_idx >> 6, b = my_idx & 63;
      int below = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        below += u < v ? __builtin_popcountll(sel[u]) : u == v ? __builtin_popcountll(sel[u] & ((1ull << b) - 1ull)) : 0;
      my_slot = below;
    }
    const float my_w = wave_topk_weight(my_val, a.k);
    if (lane < a.k) {
      sl.idx[lane] = my_idx;
      sl.w[lane] = my_w;
    }
    if (lane < kc) {
      sl.slot_of_rank[lane] = my_slot;
      sl.slot_expert[my_slot] = my_idx;
    }
    if (lane == 0) sl.header[kHdrError] = 0;
  }
  // the token into LDS (first groups from the early loads, any others now)
  {
    half8 lo, hi;
    cvt_raw16(xr, lo, hi);
    if (int(threadIdx.x) < ngrp) {
      half8* dst = reinterpret_cast<half8*>(xs1 + threadIdx.x * 16);
      dst[0] = lo;
      dst[1] = hi;
    }
    for (int gi = NT + int(threadIdx.x); gi < ngrp; gi += NT) {
      Raw16<XT> r2;
      load_raw16(xg + gi * 16, r2);
      cvt_raw16(r2, lo, hi);
      half8* dst = reinterpret_cast<half8*>(xs1 + gi * 16);
      dst[0] = lo;
      dst[1] = hi;
    }
  }
  __syncthreads();
  compute(0);
  for (int b0 = RB; b0 * 4 < rounds; b0 += RB) {  // hidden > 2048: later batches
    issue(b0);
    compute(b0);
  }
  // row 0 of the result: lanes 0..15, element 0; the class partials meet in LDS
  if (wv > 0 && lane < 16) red[ks][mat][n] = acc[0];
  __syncthreads();
  if (wv == 0 && lane < 16) {
    float sg = acc[0], su = red[0][1][n];
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      sg += red[q][0][n];
      su += red[q][1][n];
    }
    f16* hout = shared ? a.h_shared : a.h_routed;
    hout[int64_t(hrow) * rows + hcol(row)] = f16(silu_f(sg) * su);
  }
}

// ---------------------------------------------------------------------------
// Single-token down projection of the k selected experts and the shared
// expert, combined inside the workgroup (the fused decode layer):
//   out[r] = shared[r] + sum_{j<k} w_j * y_j[r]
// in the combine's order (shared first, then ranks 0..k-1, one fma each).
// grid = H / 8: a workgroup owns 8 output rows of every slot (slot s < k =
// expert slot_expert[s], h row s; slot k = shared).  With one token the MFMA
// rows are free, so one MFMA serves two slots: B columns 0..7 are the 8 rows
// of slot s0 and columns 8..15 those of slot s1, A row 0 is h of s0 and A
// row 1 h of s1, and C[0][0..7], C[1][8..15] are the two slots' outputs
// (the other elements are not used).  Every output element goes through the
// same MFMA sequence as in the other down kernels, so the bits are the same,
// and every lane's dequantisation is used: 256 workgroups (all CUs) share
// the work that 128 did with 16 rows of one slot per MFMA.  Wave w takes
// pairs w, w + NW, ...: pair p < ceil(k/2) = slots (2p, 2p+1), then the
// shared expert alone (pairs mix no K).  The weight loads of a wave's first
// pair go out first; meanwhile the workgroup copies the h rows of all slots
// into LDS (their addresses depend on nothing), and the MFMA operands are
// read from there.  The rows of all slots meet in LDS for the combine.
// ---------------------------------------------------------------------------
struct DownSlot {
  const uint8_t* dc;
  const uint16_t* ds;
  int K, n_units, rounds;
};

// Down weights of slot s of the fused single-token layer (s < k: the
// expert slot_expert[s]; s == k: the shared expert).
template <int UNIT>
__device__ __forceinline__ DownSlot down_slot(const FfnArgs& a, const int32_t* __restrict__ slot_expert, int s) {
  const bool shared = s >= a.k;
  const QMat D = shared ? a.sd : a.rd;
  const int64_t ex = shared ? 0 : slot_expert[s];
  DownSlot r;
  r.K = shared ? a.Is : a.I;
  r.dc = D.codes + ex * D.code_stride;
  r.ds = D.scales + ex * D.scale_stride;
  r.n_units = r.K / UNIT;
  r.rounds = (r.n_units + 3) / 4;
  return r;
}

constexpr int kDcRows = 8;  // output rows per workgroup of the single-token down + combine

template <int QBITS, int UNIT>
__global__ __launch_bounds__(1024) void gemv_down_combine_1tok_kernel(FfnArgs a,
                                                                      const int32_t* __restrict__ slot_expert,
                                                                      const int32_t* __restrict__ slot_of_rank,
                                                                      const float* __restrict__ w,
                                                                      float* __restrict__ out,
                                                                      float* __restrict__ res, int ldh,
                                                                      int nthreads) {
  extern __shared__ __attribute__((aligned(16))) f16 hs[];  // [n_slots][ldh]
  __shared__ float ys[kMaxTopK + 1][kDcRows];
  __shared__ float s_w[kMaxTopK];
  __shared__ int s_slot[kMaxTopK];
  constexpr int RB = 4;
  const int nw = nthreads >> 6;  // == blockDim.x / 64 (blockDim would be a load from the packet)
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15, g = lane >> 4;
  const int half = n >> 3;  // B columns 0..7: first slot of the pair, 8..15: second
  const int H = a.H;
  const int row = blockIdx.x * kDcRows + (n & 7);  // H is a multiple of 32
  const int n_slots = a.k + (a.has_shared ? 1 : 0);
  const int n_rp = (a.k + 1) / 2;                        // pairs of routed slots
  const int n_pairs = n_rp + (a.has_shared ? 1 : 0);   // then the shared slot alone
  // Issue order: the combine's weights and slot map, then the h rows (their
  // addresses depend on nothing), then the slots' expert ids and, once they
  // are in, the weight loads; the LDS stores come last, so no load waits for
  // another before it is issued.
  float w_r = 0.0f;
  int slot_r = 0;
  if (threadIdx.x < a.k) {
    w_r = w[threadIdx.x];
    slot_r = slot_of_rank[threadIdx.x];
  }
  const int ch = ldh / 8;  // 16-byte chunks per LDS row (covers the longest K)
  const int items = n_slots * ch;
  constexpr int HB = 4;  // h chunks per thread per batch
  half8 hv[HB];
  bool hon[HB];
  auto load_h = [&](int base) {
#pragma unroll
    for (int q = 0; q < HB; ++q) {
      const int it = base + q * nthreads + int(threadIdx.x);
      const int s = min(it, items - 1) / ch, c = min(it, items - 1) - s * ch;
      const int Ks = s >= a.k ? a.Is : a.I;
      hon[q] = it < items && 8 * c < Ks;
      const f16* src = s >= a.k ? a.h_shared : a.h_routed + int64_t(s) * Ks;
      hv[q] = *reinterpret_cast<const half8*>(src + (8 * c < Ks ? 8 * c : 0));  // unconditional (clamped)
    }
  };
  auto store_h = [&](int base) {
#pragma unroll
    for (int q = 0; q < HB; ++q) {
      const int it = base + q * nthreads + int(threadIdx.x);
      if (hon[q]) *reinterpret_cast<half8*>(hs + it / ch * ldh + 8 * (it % ch)) = hv[q];
    }
  };
  load_h(0);

  // pair p: its two slots (the second is -1 when there is none)
  auto pair_slots = [&](int p, int& s0, int& s1) {
    s0 = p < n_rp ? 2 * p : a.k;
    s1 = p < n_rp && 2 * p + 1 < a.k ? 2 * p + 1 : -1;
  };
  Unit<QBITS, UNIT> ud[RB];
  int s0, s1;
  const uint8_t* dc;
  const uint16_t* ds;
  int K, n_units, rounds;
  // this lane's weight rows: slot s0 for columns 0..7, s1 for 8..15 (a
  // missing s1 reads s0's rows, whose columns are not used)
  auto set_pair = [&](int p) {
    pair_slots(p, s0, s1);
    const DownSlot d0 = down_slot<UNIT>(a, slot_expert, s0);
    const DownSlot d1 = down_slot<UNIT>(a, slot_expert, s1 >= 0 ? s1 : s0);
    dc = half ? d1.dc : d0.dc;
    ds = half ? d1.ds : d0.ds;
    K = d0.K;  // both slots of a pair have the same K
    n_units = d0.n_units;
    rounds = d0.rounds;
  };
  // unconditional loads from clamped units (a wave past the pairs loads the
  // last pair's weights and never uses them); units past K are zeroed at use
  // (a load under a branch costs a wait for every load in flight)
  set_pair(min(wv, n_pairs - 1));
  auto issue = [&](int r0) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int u = (r0 + i) * 4 + g;
      load_unit(ud[i], dc, ds, H, K, row, r0 + i < rounds && u < n_units ? u : 0);
    }
  };
  issue(0);
  __builtin_amdgcn_sched_barrier(0);
  store_h(0);
  for (int base = HB * nthreads; base < items; base += HB * nthreads) {  // more than one batch
    load_h(base);
    store_h(base);
  }
  __syncthreads();

  for (int p = wv; p < n_pairs; p += nw) {
    if (p != wv) {
      set_pair(p);
      issue(0);
    }
    // A row 0 = h of s0 (lanes n = 0), row 1 = h of s1 (lanes n = 1); the
    // other rows repeat s0 (their outputs are not used)
    const f16* hrow = hs + (n == 1 && s1 >= 0 ? s1 : s0) * ldh;
    float4v acc[4] = {};  // one accumulator per round class (round % 4), as in every down kernel
    static_assert(RB % 4 == 0, "a load batch holds whole round classes");
    for (int r0 = 0; r0 < rounds; r0 += RB) {
      if (r0 > 0) issue(r0);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (r0 + i >= rounds) break;
        const int u = (r0 + i) * 4 + g;
        const int ua = u < n_units ? u : 0;
        if (u >= n_units) zero_unit(ud[i]);
#pragma unroll
        for (int d = 0; d < UNIT / 16; ++d) {
          half8 blo, bhi;
          dq_unit_word(ud[i], d, blo, bhi);
          const half8* ap = reinterpret_cast<const half8*>(hrow + ua * UNIT + 16 * d);
          acc[i & 3] = mfma16(ap[0], blo, acc[i & 3]);
          acc[i & 3] = mfma16(ap[1], bhi, acc[i & 3]);
        }
      }
    }
    // lane n (g = 0) holds C[0][n] in element 0 and C[1][n] in element 1
    if (lane < 16) {
      const int e = half;
      const float y = ((acc[0][e] + acc[1][e]) + acc[2][e]) + acc[3][e];
      const int s = half ? s1 : s0;
      if (s >= 0) ys[s][n & 7] = y;
    }
  }
  if (threadIdx.x < a.k) {  // (stored here: an earlier store would wait on the loads behind it)
    s_w[threadIdx.x] = w_r;
    s_slot[threadIdx.x] = slot_r;
  }
  __syncthreads();
  if (threadIdx.x < kDcRows) {
    const int t = threadIdx.x;
    const int orow = blockIdx.x * kDcRows + t;
    const float r_in = res ? res[orow] : 0.0f;
    float v = a.has_shared ? ys[a.k][t] : 0.0f;
    for (int j0 = 0; j0 < a.k; j0 += 8) {  // the LDS reads of 8 ranks at a time, then their fmas in rank order
      float wj[8], yj[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = min(j0 + q, a.k - 1);
        wj[q] = s_w[j];
        yj[q] = ys[s_slot[j]][t];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (j0 + q < a.k) v = __builtin_fmaf(wj[q], yj[q], v);
    }
    if (out) out[orow] = v;
    if (res) res[orow] = r_in + v;
  }
}

// ---------------------------------------------------------------------------
// down projection: y[m][n] = h_m . W_down[n].  grid = (ceil(H / 64), slots),
// block = 256, 16 rows per wave.  The weight loads are issued first; the h
// operands (already in the permuted order) are read straight from global
// memory, so the kernel has no LDS and no barrier.
// ---------------------------------------------------------------------------
template <int QBITS, int UNIT>
__global__ __launch_bounds__(256) void gemv_down_kernel(FfnArgs a) {
  const int4 si = a.slots[blockIdx.y];
  const int m_total = si.z;
  if (m_total == 0) return;
  const bool shared = si.x < 0;
  if (shared && a.shared_out == nullptr) return;
  const int H = a.H;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row_w = blockIdx.x * 64 + wv * 16;
  if (row_w >= H) return;  // per wave: no barriers in this kernel
  const int K = shared ? a.Is : a.I;
  const QMat D = shared ? a.sd : a.rd;
  const int64_t ex = shared ? 0 : si.x;
  const uint8_t* dc = D.codes + ex * D.code_stride;
  const uint16_t* ds = D.scales + ex * D.scale_stride;
  const int n = lane & 15, g = lane >> 4;
  const int row = row_w + n;
  const int n_units = K / UNIT, rounds = (n_units + 3) / 4;
  const f16* hin = shared ? a.h_shared : a.h_routed;
  float* yout = shared ? a.shared_out : a.y_sorted;
  constexpr int RB = 4;

  for (int mc = 0; mc < m_total; mc += kGemvMaxM) {
    const int mnow = min(kGemvMaxM, m_total - mc);
    const bool a_on = n < mnow;
    const int nr = a_on ? n : 0;  // rows past the tokens read token 0's row (loads are unconditional)
    const f16* hrow = hin + (shared ? int64_t(mc + nr) : int64_t(si.y + mc + nr)) * K;
    float4v acc[4] = {};  // one accumulator per round class (round % 4)
    static_assert(RB % 4 == 0, "a load batch holds whole round classes");
    for (int r0 = 0; r0 < rounds; r0 += RB) {
      Unit<QBITS, UNIT> ud[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int u = (r0 + i) * 4 + g;
        if (r0 + i < rounds && u < n_units) load_unit(ud[i], dc, ds, H, K, row, u);
        else zero_unit(ud[i]);
      }
      half8 av[RB][UNIT / 16][2];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int u = (r0 + i) * 4 + g;
        const bool on = a_on && r0 + i < rounds && u < n_units;
        const int uc = on ? u : 0;  // unconditional loads from a clamped unit
#pragma unroll
        for (int d = 0; d < UNIT / 16; ++d) {
          const half8* ap = reinterpret_cast<const half8*>(hrow + uc * UNIT + 16 * d);
          const half8 l0 = ap[0], l1 = ap[1];
          av[i][d][0] = on ? l0 : half8{};
          av[i][d][1] = on ? l1 : half8{};
        }
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (r0 + i >= rounds) break;
#pragma unroll
        for (int d = 0; d < UNIT / 16; ++d) {
          half8 blo, bhi;
          dq_unit_word(ud[i], d, blo, bhi);
          acc[i & 3] = mfma16(av[i][d][0], blo, acc[i & 3]);
          acc[i & 3] = mfma16(av[i][d][1], bhi, acc[i & 3]);
        }
      }
    }
    const float4v y4 = ((acc[0] + acc[1]) + acc[2]) + acc[3];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = 4 * g + j;
      if (m < mnow) {
        const int64_t yr = shared ? int64_t(mc + m) : int64_t(si.y + mc + m);
        yout[yr * H + row] = y4[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Throughput versions for more than one token (decode batches, verify
// windows): NW waves of 16 rows each per workgroup, activations staged once
// in LDS for all of them, and a rolling pipeline that keeps the next D rounds
// of weight loads in flight while the current round is dequantised and fed
// to the MFMAs.  Accumulation classes and orders are those of the kernels
// above, so results are bit-identical to the single-token path.
// ---------------------------------------------------------------------------
constexpr int kTpD = 4;      // rounds of weight loads in flight in the per-slot gate/up kernel
constexpr int kTpNW = 4;     // row blocks (waves of gate rows) per workgroup of the per-slot kernels
constexpr int kTpMinW = 1;   // workgroups per CU asked of the per-slot gate/up kernel
constexpr int kTpEarly = 2;  // items per thread of an early activation staging
constexpr int kPersGrid = 512;       // persistent gate/up item groups of 8 waves (two per CU)
// Item groups per persistent gate/up workgroup: 2 (one 16-wave workgroup per
// CU) above 8 tokens, where the selection made by every workgroup then runs
// once per CU with one token per wave instead of two; 1 for fewer tokens
// (each wave already ranks one token at most, and the wider workgroup was
// measured slower there).
inline int pers_gateup_groups(int64_t T) { return T > 8 ? 2 : 1; }
// workgroups of the persistent gate/up launch for at most `slots` slots of
// n_rb items each
inline int pers_gateup_grid(int64_t slots, int n_rb, int ng) {
  return int(std::min<int64_t>(kPersGrid / ng, (slots * n_rb + ng - 1) / ng));
}
constexpr int kPersGridDown = 1024;  // persistent down workgroups (four per CU)
// NW row blocks of 16 per workgroup; waves 0..NW-1 take the gate rows of
// block wv, waves NW..2NW-1 the up rows (half the dequantisation per wave);
// the up sums reach the gate waves through LDS for the SwiGLU.
template <int QBITS, int UNIT, typename XT, int NW>
__global__ __launch_bounds__(128 * NW, kTpMinW) void gemv_gateup_tp_kernel(FfnArgs a) {
  extern __shared__ __attribute__((aligned(16))) f16 xs[];
  __shared__ float4v up_x[NW][64];  // the up waves' sums, per lane
  constexpr int kThreads = 128 * NW;  // the launch's block size (blockDim would be a load)
  constexpr int D = kTpD;
  static_assert(D % 4 == 0, "the pipeline depth is a multiple of the 4 accumulation classes");
  const int4 si = a.slots[blockIdx.y];
  const int m_total = si.z;
  if (m_total == 0) return;
  const bool shared = si.x < 0;
  const int rows = shared ? a.Is : a.I;
  const int row_base = blockIdx.x * 16 * NW;
  if (row_base >= rows) return;
  const int H = a.H, ldsw = H + 8;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int wr = wv % NW, mat = wv / NW;  // row block, matrix (0 gate, 1 up)
  const QMat Mq = shared ? (mat == 0 ? a.sg : a.su) : (mat == 0 ? a.rg : a.ru);
  const int64_t ex = shared ? 0 : si.x;
  const uint8_t* wc = Mq.codes + ex * Mq.code_stride;
  const uint16_t* wsc = Mq.scales + ex * Mq.scale_stride;
  const int n = lane & 15, g = lane >> 4;
  const int row = row_base + wr * 16 + n;
  const bool wave_on = row_base + wr * 16 < rows;
  const int n_units = H / UNIT, rounds = (n_units + 3) / 4;
  const XT* x = static_cast<const XT*>(a.x);
  f16* hout = shared ? a.h_shared : a.h_routed;
  const int hw = shared ? a.Is : a.I;
  // With a token mask in the slot (decode selection), the slot's tokens are
  // known without a load: the activations are requested before the weights,
  // so the staging waits for them alone (loads complete in issue order).
  __shared__ int s_tok[kGemvMaxM];
  const uint32_t tmask = uint32_t(si.w);
  if (tmask) {
    if (threadIdx.x < kGemvMaxM && ((tmask >> threadIdx.x) & 1u))
      s_tok[__builtin_popcount(tmask & ((1u << threadIdx.x) - 1u))] = int(threadIdx.x);
    __syncthreads();
  }
  constexpr int NB = sizeof(XT) == 4 ? 2 : 4;  // staging items per thread per batch
  constexpr int NBE = kTpEarly;             // items per thread of an early staging (registers held
                                                // across the weight loads)
  const int chunks = H / 16;

  for (int mc = 0; mc < m_total; mc += kGemvMaxM) {
    const int mnow = min(kGemvMaxM, m_total - mc);
    const int items = mnow * chunks;
    const bool early = tmask != 0u && items <= NBE * kThreads;
    Raw16<XT> raw0[NBE];
    if (early) {
#pragma unroll
      for (int q = 0; q < NBE; ++q) {
        const int it = min(q * kThreads + int(threadIdx.x), items - 1);
        const int r = it / chunks, gg = it - r * chunks;
        load_raw16(x + int64_t(s_tok[r]) * H + gg * 16, raw0[q]);
      }
    }
    Unit<QBITS, UNIT> uw[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int u = i * 4 + g;
      if (wave_on && i < rounds && u < n_units) load_unit(uw[i], wc, wsc, rows, H, row, u);
      else zero_unit(uw[i]);
    }
    __syncthreads();
    if (early) {
#pragma unroll
      for (int q = 0; q < NBE; ++q) {
        const int it = q * kThreads + int(threadIdx.x);
        if (it < items) {
          const int r = it / chunks, gg = it - r * chunks;
          half8 lo, hi;
          cvt_raw16(raw0[q], lo, hi);
          half8* dst = reinterpret_cast<half8*>(xs + r * ldsw + gg * 16);
          dst[0] = lo;
          dst[1] = hi;
        }
      }
    } else {
      // stage the tokens: per thread NB items at a time, the token ids, then
      // the activation loads, then the conversions, each step as one batch
      for (int base = 0; base < items; base += NB * kThreads) {
        int64_t tok[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          const int it = min(base + q * kThreads + int(threadIdx.x), items - 1);
          const int r = it / chunks;
          tok[q] = shared ? int64_t(mc + r) : int64_t(a.sorted_pair[si.y + mc + r] / a.k);
        }
        Raw16<XT> raw[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          const int it = min(base + q * kThreads + int(threadIdx.x), items - 1);
          const int r = it / chunks, gg = it - r * chunks;
          load_raw16(x + tok[q] * H + gg * 16, raw[q]);
        }
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          const int it = base + q * kThreads + int(threadIdx.x);
          if (it < items) {
            const int r = it / chunks, gg = it - r * chunks;
            half8 lo, hi;
            cvt_raw16(raw[q], lo, hi);
            half8* dst = reinterpret_cast<half8*>(xs + r * ldsw + gg * 16);
            dst[0] = lo;
            dst[1] = hi;
          }
        }
      }
    }
    __syncthreads();
    float4v acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};
    if (wave_on) {
      // Rows past the tokens (and units past K, whose weights are zero) read
      // a real, finite row: MFMA rows are independent and the extra rows of
      // the result are never stored, so no operand needs zeroing.
      const f16* xrow = xs + min(n, mnow - 1) * ldsw;
      for (int r0 = 0; r0 < rounds; r0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
          const int r = r0 + i;
          if (r >= rounds) break;
          const Unit<QBITS, UNIT> cw = uw[i];
          const int rn = r + D, un = rn * 4 + g;
          if (rn < rounds && un < n_units) load_unit(uw[i], wc, wsc, rows, H, row, un);
          const int u = r * 4 + g;
          const int ua = u < n_units ? u : 0;
#pragma unroll
          for (int d = 0; d < UNIT / 16; ++d) {
            half8 wlo, whi;
            dq_unit_word(cw, d, wlo, whi);
            const half8* ap = reinterpret_cast<const half8*>(xrow + ua * UNIT + 16 * d);
            const half8 alo = ap[0], ahi = ap[1];
            const int c = i & 3;  // class of round r = r0 + i (r0 is a multiple of D, D of 4)
            acc[c] = mfma16(alo, wlo, acc[c]);
            acc[c] = mfma16(ahi, whi, acc[c]);
          }
        }
      }
      float4v sum = acc[0];
#pragma unroll
      for (int c = 1; c < 4; ++c) sum += acc[c];
      if (mat == 1) up_x[wr][lane] = sum;
      acc[0] = sum;
    }
    __syncthreads();  // the up sums are in LDS
    if (wave_on && mat == 0) {
      const float4v sg = acc[0], su = up_x[wr][lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = 4 * g + j;
        if (m < mnow) {
          const float hv = silu_f(sg[j]) * su[j];
          const int64_t hr = shared ? int64_t(mc + m) : int64_t(si.y + mc + m);
          hout[hr * hw + hcol(row)] = f16(hv);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent gate/up for 2..kGemvMaxM tokens: the same per-row arithmetic as
// gemv_gateup_tp_kernel (8 waves, 64 rows per work item, gate and up waves,
// four round classes), but a fixed grid of G workgroups, each of NG item
// groups of 8 waves (pers_gateup_groups), and each group walks a contiguous run
// of the (slot, 64-row block) items.  The tokens of the workgroup's slots are
// staged in LDS once for its groups (rows indexed by token; a slot's MFMA
// rows pick its tokens through the token mask), and (SEL) the selection is
// made once for them.  The weight pipeline runs on across items: the next item's
// slot entry is requested when an item starts and its first D rounds of
// weights while the current item's last D rounds are computed.  So the
// first-load latency is paid once per workgroup instead of once per item.
// Requires H % (16 UNIT) == 0 (whole pipeline groups per item) and Is = I or
// no shared expert (one item size).
// ---------------------------------------------------------------------------
//
// SEL: the selection is made here, from the router logits, by every
// workgroup (the experts of each token, the slot table in LDS); the last
// workgroup also writes it out (topk_idx / topk_w, the permutation, the slot table and
// header for the down kernel and the combine).  E <= kSelPersMaxExperts.
// Otherwise the slot table and header come from a selection launch.
constexpr int kSelPersMaxExperts = 512;

template <int QBITS, int UNIT, typename XT, bool SEL, int NG>
__global__ __launch_bounds__(512 * NG) void gemv_gateup_pers_kernel(FfnArgs a, int n_rb, int G,
                                                                   const int4* __restrict__ slots,
                                                                   const int32_t* __restrict__ header, SelOut so) {
  // slots / header are a.slots / a.header, read-only here: scalar loads,
  // which wait on their own counter instead of behind the weight loads
  constexpr int NW = 4, D = 4, kThreads = 512 * NG;
  extern __shared__ __attribute__((aligned(16))) f16 xs[];  // [T][H + 8]
  // the up sums of the item loop; before it, the ranking scratch of the selection
  __shared__ union {
    float4v up_x[NG][NW][64];
    SelRankLds tk[8 * NG];
  } ux;
  __shared__ SelLds<SEL ? kSelPersMaxExperts : 1, SEL ? 8 * NG : 1> sel;
  const int H = a.H, ldsw = H + 8, T = int(a.T);
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int ig = wv / 8, wl = wv % 8;  // item group, wave in the group
  float4v(&up_x)[NW][64] = ux.up_x[ig];
  const int wr = wl % NW, mat = wl / NW;
  const int n = lane & 15, g = lane >> 4;
  const int n_units = H / UNIT, rounds = n_units / 4;  // a multiple of D (host-checked)
  // Token staging into LDS (fp16, permuted 16-groups; row = token id):
  // item i of a pass is chunk i % chunks of the (i / chunks)-th token of umask.
  const XT* xsrc = static_cast<const XT*>(a.x);
  const int chunks = H / 16;
  constexpr int NB = (sizeof(XT) == 4 ? 2 : 4) / NG;
  auto stage_load = [&](uint32_t umask, int items, int base, Raw16<XT>(&raw)[NB], int(&dst)[NB]) {
#pragma unroll
    for (int k2 = 0; k2 < NB; ++k2) {
      const int it = min(base + k2 * kThreads + int(threadIdx.x), items - 1);
      const int r = it / chunks, gg = it - r * chunks;
      uint32_t mm = umask;  // token of rank r: the r-th set bit
      for (int k3 = 0; k3 < r; ++k3) mm &= mm - 1u;
      const int tok = __builtin_ctz(mm);
      load_raw16(xsrc + int64_t(tok) * H + gg * 16, raw[k2]);
      dst[k2] = tok * ldsw + gg * 16;
    }
  };
  auto stage_store = [&](int items, int base, const Raw16<XT>(&raw)[NB], const int(&dst)[NB]) {
#pragma unroll
    for (int k2 = 0; k2 < NB; ++k2) {
      if (base + k2 * kThreads + int(threadIdx.x) < items) {
        half8 lo, hi;
        cvt_raw16(raw[k2], lo, hi);
        half8* d = reinterpret_cast<half8*>(xs + dst[k2]);
        d[0] = lo;
        d[1] = hi;
      }
    }
  };
  // SEL: every token is staged, and the first pass's loads are issued before
  // the selection (they do not depend on it), so their latency is hidden
  Raw16<XT> raw0[NB];
  int dst0[NB];
  if constexpr (SEL) stage_load(uint32_t((1ull << T) - 1u), T * chunks, 0, raw0, dst0);

  int n_active = 0, n_valid;
  if constexpr (SEL) {
    // the last workgroup writes the selection out: it has the fewest items
    // (none when there are fewer items than workgroups), so the ranks and
    // writes stay off the other workgroups' path
    n_active = select_in_workgroup<kSelPersMaxExperts / 64, 8 * NG, kSelPersMaxExperts>(
        so, T, a.E, a.k, a.has_shared, sel, ux.tk, blockIdx.x == gridDim.x - 1);
    n_valid = n_active + (a.has_shared ? 1 : 0);
  } else {
    n_valid = header[kHdrValid];
  }
  // slot s of the table: {expert or -1 (shared), first sorted position, tokens, token mask}
  auto slot_at = [&](int s) -> int4 {
    if constexpr (SEL) {
      if (s < n_active) {
        const int e = sel.slot_e[s];
        const uint32_t m = sel.tmask[e];
        return int4{e, sel.cnt[e] & 0xffff, __builtin_popcount(m), int(m)};
      }
      return s == n_active && a.has_shared ? int4{-1, 0, T, int((1u << T) - 1u)} : int4{0, 0, 0, 0};
    } else {
      return slots[s];
    }
  };
  // NG G workers take contiguous runs of the items: worker w = g G + b is
  // item group g of workgroup b, so that with fewer items than workers every
  // workgroup's first group has one before any second group does (a CU
  // streams one item's weights faster than two).  Every group runs as many
  // barrier pairs as its workgroup's first runs item iterations (the item
  // loop's barriers are the workgroup's): after its own items, bare ones.
  const int n_items = n_valid * n_rb, n_workers = NG * G;
  const int q = n_items / n_workers, rem = n_items - q * n_workers, b = blockIdx.x;
  auto first = [&](int w) { return w * q + min(w, rem); };
  const int n_iter = first(b + 1) - first(b);  // the first group's items: the most
  if (n_iter == 0) return;
  const int it0 = first(ig * G + b), it1 = first(ig * G + b + 1);  // the group's items
  const int it_first = it0 < it1 ? it0 : first(b);                  // a real item of the workgroup

  // an item's weight source for this wave (plain values: no aggregate copies)
  auto make = [&](int it, int4 si, const uint8_t*& wc, const uint16_t*& wsc, int& rows, int& row, bool& on) {
    const bool shared = si.x < 0;
    rows = shared ? a.Is : a.I;
    const int row_base = (it % n_rb) * 16 * NW + wr * 16;
    on = si.z > 0 && row_base < rows;
    row = row_base + n;
    const QMat Mq = shared ? (mat == 0 ? a.sg : a.su) : (mat == 0 ? a.rg : a.ru);
    const int64_t ex = shared ? 0 : si.x;
    wc = Mq.codes + ex * Mq.code_stride;
    wsc = Mq.scales + ex * Mq.scale_stride;
  };

  int4 si_cur = slot_at(it_first / n_rb);
  const uint8_t* c_wc;
  const uint16_t* c_wsc;
  int c_rows, c_row;
  bool c_on;
  make(it_first, si_cur, c_wc, c_wsc, c_rows, c_row, c_on);
  // Weight loads are unconditional (a wave past its rows reads the last row,
  // and the prefetch past a workgroup's last item rereads its own weights):
  // a load under a branch makes the compiler wait for every load in flight.
  // (A group without items loads nothing: the staging below waits for every
  // load anyway.)
  Unit<QBITS, UNIT> uw[D];
  if (it0 < it1) {
#pragma unroll
    for (int i = 0; i < D; ++i) load_unit(uw[i], c_wc, c_wsc, c_rows, H, min(c_row, c_rows - 1), i * 4 + g);
  }
  // the tokens into LDS: with SEL all of them (the first pass is loaded),
  // else the union of the workgroup's slots' token masks
  {
    uint32_t umask = uint32_t((1ull << T) - 1u);
    int base0 = 0;
    if constexpr (SEL) {
      stage_store(T * chunks, 0, raw0, dst0);
      base0 = NB * kThreads;
    } else {
      umask = 0u;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {  // the slots of every group's run
        const int r0 = first(gg * G + b), r1 = first(gg * G + b + 1);
        for (int sl = r0 / n_rb; r0 < r1 && sl <= (r1 - 1) / n_rb; ++sl) umask |= uint32_t(slot_at(sl).w);
      }
    }
    const int items = __builtin_popcount(umask) * chunks;
    for (int base = base0; base < items; base += NB * kThreads) {
      Raw16<XT> raw[NB];
      int dst[NB];
      stage_load(umask, items, base, raw, dst);
      stage_store(items, base, raw, dst);
    }
  }
  __syncthreads();
  // Nothing is in flight here (the staging waited for every load); saying so
  // keeps the compiler from assuming a pending staging load at the loop head,
  // where it would otherwise wait for all loads in flight every item.
  __builtin_amdgcn_s_waitcnt(0);

  for (int it = it0; it < it1; ++it) {
    const bool has_next = it + 1 < it1;
    const int4 si_next = slot_at(min(it + 1, it1 - 1) / n_rb);  // requested now, read at round rounds - D
    const bool shared = si_cur.x < 0;
    const int mnow = si_cur.z;
    // this lane's MFMA row: the slot's min(n, mnow - 1)-th token
    // (slot tables for at most kGemvMaxM tokens always carry the mask)
    int tok = 0;
    const uint32_t mask = uint32_t(si_cur.w);
    for (int bit = 0, c = 0; bit < kGemvMaxM; ++bit)
      if ((mask >> bit) & 1u) {
        if (c <= n) tok = bit;
        ++c;
      }
    const f16* xrow = xs + tok * ldsw;
    float4v acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};
    const uint8_t* n_wc = c_wc;
    const uint16_t* n_wsc = c_wsc;
    int n_rows = c_rows, n_row = c_row;
    bool n_on = false;
    for (int r0 = 0; r0 < rounds; r0 += D) {
      const bool last_group = r0 + D >= rounds;
      if (last_group && has_next) make(it + 1, si_next, n_wc, n_wsc, n_rows, n_row, n_on);
      // the loads of this group: this item's rounds r0 + D .., or the next item's first D
      const uint8_t* l_wc = last_group ? n_wc : c_wc;
      const uint16_t* l_wsc = last_group ? n_wsc : c_wsc;
      const int l_rows = last_group ? n_rows : c_rows;
      const int l_row = min(last_group ? n_row : c_row, l_rows - 1);
      const int l_r0 = last_group ? 0 : r0 + D;
      // Round r is dequantised from ring slot i, then the slot is reloaded
      // (reloading before the use would need a copy of the slot, and the
      // copies at the loop edge would wait for the loads just issued).
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const int r = r0 + i;
        if (c_on) {
          const int u = r * 4 + g;
#pragma unroll
          for (int d = 0; d < UNIT / 16; ++d) {
            half8 wlo, whi;
            dq_unit_word(uw[i], d, wlo, whi);
            const half8* ap = reinterpret_cast<const half8*>(xrow + u * UNIT + 16 * d);
            acc[i & 3] = mfma16(ap[0], wlo, acc[i & 3]);
            acc[i & 3] = mfma16(ap[1], whi, acc[i & 3]);
          }
        }
        load_unit(uw[i], l_wc, l_wsc, l_rows, H, l_row, (l_r0 + i) * 4 + g);
      }
    }
    if (c_on) {
      float4v sum = acc[0];
#pragma unroll
      for (int c = 1; c < 4; ++c) sum += acc[c];
      if (mat == 1) up_x[wr][lane] = sum;
      acc[0] = sum;
    }
    __syncthreads();  // the up sums are in LDS
    if (c_on && mat == 0) {
      const float4v su = up_x[wr][lane];
      f16* hout = shared ? a.h_shared : a.h_routed;
      const int hw = shared ? a.Is : a.I;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = 4 * g + j;
        if (m < mnow) {
          const float hv = silu_f(acc[0][j]) * su[j];
          const int64_t hr = shared ? int64_t(m) : int64_t(si_cur.y + m);
          hout[hr * hw + hcol(c_row)] = f16(hv);
        }
      }
    }
    __syncthreads();  // up_x is free for the next item
    c_wc = n_wc;
    c_wsc = n_wsc;
    c_rows = n_rows;
    c_row = n_row;
    c_on = n_on;
    si_cur = si_next;
  }
  for (int j = it1 - it0; j < n_iter; ++j) {  // the barriers of the first group's further items
    __syncthreads();
    __syncthreads();
  }
}

template <int QBITS, int UNIT, int NW>
__global__ __launch_bounds__(64 * NW) void gemv_down_tp_kernel(FfnArgs a, int ldsw) {
  extern __shared__ __attribute__((aligned(16))) f16 hs[];
  constexpr int kThreads = 64 * NW;  // the launch's block size (blockDim would be a load)
  constexpr int D = 4;
  const int4 si = a.slots[blockIdx.y];
  const int m_total = si.z;
  if (m_total == 0) return;
  const bool shared = si.x < 0;
  if (shared && a.shared_out == nullptr) return;
  const int H = a.H;
  const int row_base = blockIdx.x * 16 * NW;
  if (row_base >= H) return;
  const int K = shared ? a.Is : a.I;
  const QMat Dm = shared ? a.sd : a.rd;
  const int64_t ex = shared ? 0 : si.x;
  const uint8_t* dc = Dm.codes + ex * Dm.code_stride;
  const uint16_t* ds = Dm.scales + ex * Dm.scale_stride;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row = row_base + wv * 16 + n;
  const bool wave_on = row_base + wv * 16 < H;
  const int n_units = K / UNIT, rounds = (n_units + 3) / 4;
  const f16* hin = shared ? a.h_shared : a.h_routed;
  float* yout = shared ? a.shared_out : a.y_sorted;

  for (int mc = 0; mc < m_total; mc += kGemvMaxM) {
    const int mnow = min(kGemvMaxM, m_total - mc);
    Unit<QBITS, UNIT> ud[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int u = i * 4 + g;
      if (wave_on && i < rounds && u < n_units) load_unit(ud[i], dc, ds, H, K, row, u);
      else zero_unit(ud[i]);
    }
    __syncthreads();
    {
      // h rows are already in the MFMA operand order: plain 16-byte copies,
      // NB loads in flight per thread before their stores
      constexpr int NB = 8;
      const int chunks = K / 8, items = mnow * chunks;
      for (int base = 0; base < items; base += NB * kThreads) {
        half8 v[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          const int it = min(base + q * kThreads + int(threadIdx.x), items - 1);
          const int r = it / chunks, c8 = it - r * chunks;
          const int64_t hr = shared ? int64_t(mc + r) : int64_t(si.y + mc + r);
          v[q] = *reinterpret_cast<const half8*>(hin + hr * K + c8 * 8);
        }
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          const int it = base + q * kThreads + int(threadIdx.x);
          if (it < items) {
            const int r = it / chunks, c8 = it - r * chunks;
            *reinterpret_cast<half8*>(hs + r * ldsw + c8 * 8) = v[q];
          }
        }
      }
    }
    __syncthreads();
    if (!wave_on) continue;
    const f16* hrow = hs + min(n, mnow - 1) * ldsw;  // see the gate/up kernel: finite, never stored
    float4v acc[4] = {};  // one accumulator per round class (round % 4): r0 is a multiple of D, D of 4
    static_assert(D % 4 == 0, "the pipeline depth is a multiple of the 4 accumulation classes");
    for (int r0 = 0; r0 < rounds; r0 += D) {
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const int r = r0 + i;
        if (r >= rounds) break;
        const Unit<QBITS, UNIT> cd = ud[i];
        const int rn = r + D, un = rn * 4 + g;
        if (rn < rounds && un < n_units) load_unit(ud[i], dc, ds, H, K, row, un);
        const int u = r * 4 + g;
        const int ua = u < n_units ? u : 0;
#pragma unroll
        for (int d = 0; d < UNIT / 16; ++d) {
          half8 blo, bhi;
          dq_unit_word(cd, d, blo, bhi);
          const half8* ap = reinterpret_cast<const half8*>(hrow + ua * UNIT + 16 * d);
          const half8 alo = ap[0], ahi = ap[1];
          acc[i & 3] = mfma16(alo, blo, acc[i & 3]);
          acc[i & 3] = mfma16(ahi, bhi, acc[i & 3]);
        }
      }
    }
    const float4v y4 = ((acc[0] + acc[1]) + acc[2]) + acc[3];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = 4 * g + j;
      if (m < mnow) {
        const int64_t yr = shared ? int64_t(mc + m) : int64_t(si.y + mc + m);
        yout[yr * H + row] = y4[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent down projection for 2..kGemvMaxM tokens: the arithmetic of
// gemv_down_tp_kernel (16 output rows per wave, four round classes), with a
// fixed grid walking contiguous runs of (slot, 64-row block) items.  A slot
// has R = ceil(K / 256) rounds (the whole reduction axis in one ring), so
// while an item is computed the ring is refilled with the next item's
// weights (slot entries two items ahead are scalar loads).  The h rows of a
// slot are staged in LDS when the slot changes.  Requires Is = I (or no
// shared expert), I % 64 == 0 and ceil(I / 256) == R.
// ---------------------------------------------------------------------------
template <int QBITS, int R>
__global__ __launch_bounds__(256) void gemv_down_pers_kernel(FfnArgs a, int ldsw, int n_rb, int G,
                                                             const int4* __restrict__ slots,
                                                             const int32_t* __restrict__ header) {
  constexpr int NW = 4, UNIT = 64, kThreads = 256;
  extern __shared__ __attribute__((aligned(16))) f16 hs[];  // [<= kGemvMaxM][ldsw]
  const int H = a.H, K = a.I;
  const int n_units = K / UNIT;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int n = lane & 15, g = lane >> 4;
  const int n_items = header[kHdrValid] * n_rb;
  const int q = n_items / G, rem = n_items - q * G, b = blockIdx.x;
  const int it0 = b * q + min(b, rem), it1 = it0 + q + (b < rem ? 1 : 0);
  if (it0 >= it1) return;

  // item -> this wave's weight rows (loads always go to a real row and unit)
  auto src = [&](int it, int4 si, const uint8_t*& dc, const uint16_t*& dsc, int& row, bool& on) {
    const bool shared = si.x < 0;
    const QMat Dm = shared ? a.sd : a.rd;
    const int64_t ex = shared ? 0 : si.x;
    dc = Dm.codes + ex * Dm.code_stride;
    dsc = Dm.scales + ex * Dm.scale_stride;
    const int rb = (it % n_rb) * 16 * NW + wv * 16;
    on = si.z > 0 && rb < H && !(shared && a.shared_out == nullptr);
    row = min(rb + n, H - 1);
  };
  auto load_ring = [&](Unit<QBITS, UNIT> (&ud)[R], const uint8_t* dc, const uint16_t* dsc, int row) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int u = i * 4 + g;
      load_unit(ud[i], dc, dsc, H, K, row, u < n_units ? u : 0);
    }
  };

  int4 si_c = slots[it0 / n_rb];
  int4 si_n = slots[min(it0 + 1, it1 - 1) / n_rb];
  const uint8_t* c_dc;
  const uint16_t* c_dsc;
  int c_row;
  bool c_on;
  src(it0, si_c, c_dc, c_dsc, c_row, c_on);
  Unit<QBITS, UNIT> ud[R];
  load_ring(ud, c_dc, c_dsc, c_row);
  int staged = -1;  // slot index whose h rows are in LDS
  __builtin_amdgcn_s_waitcnt(0);  // (see the persistent gate/up kernel)

  for (int it = it0; it < it1; ++it) {
    const int4 si_nn = slots[min(it + 2, it1 - 1) / n_rb];  // two items ahead
    const int slot = it / n_rb;
    const bool shared = si_c.x < 0;
    const int mnow = si_c.z;
    if (slot != staged) {  // the slot's h rows into LDS (uniform over the workgroup)
      __syncthreads();
      const f16* hin = shared ? a.h_shared : a.h_routed;
      constexpr int NB = 4;
      const int chunks = K / 8, items = mnow * chunks;
      for (int base = 0; base < items; base += NB * kThreads) {
        half8 v[NB];
#pragma unroll
        for (int k2 = 0; k2 < NB; ++k2) {
          const int ii = min(base + k2 * kThreads + int(threadIdx.x), items - 1);
          const int r = ii / chunks, c8 = ii - r * chunks;
          const int64_t hr = shared ? int64_t(r) : int64_t(si_c.y + r);
          v[k2] = *reinterpret_cast<const half8*>(hin + hr * K + c8 * 8);
        }
#pragma unroll
        for (int k2 = 0; k2 < NB; ++k2) {
          const int ii = base + k2 * kThreads + int(threadIdx.x);
          if (ii < items) {
            const int r = ii / chunks, c8 = ii - r * chunks;
            *reinterpret_cast<half8*>(hs + r * ldsw + c8 * 8) = v[k2];
          }
        }
      }
      __syncthreads();
      staged = slot;
    }
    // the next item's weight source (its slot entry arrived during the previous item)
    const uint8_t* n_dc;
    const uint16_t* n_dsc;
    int n_row;
    bool n_on;
    src(min(it + 1, it1 - 1), si_n, n_dc, n_dsc, n_row, n_on);
    const f16* hrow = hs + min(n, mnow - 1) * ldsw;  // finite, never stored past mnow
    float4v acc[4] = {};
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int u = i * 4 + g;
      const bool valid = u < n_units;
      if (c_on) {
        const int ua = valid ? u : 0;
        if (!valid) zero_unit(ud[i]);  // units past K: the zero unit of the other down kernels
#pragma unroll
        for (int d = 0; d < UNIT / 16; ++d) {
          half8 blo, bhi;
          dq_unit_word(ud[i], d, blo, bhi);
          const half8* ap = reinterpret_cast<const half8*>(hrow + ua * UNIT + 16 * d);
          acc[i & 3] = mfma16(ap[0], blo, acc[i & 3]);
          acc[i & 3] = mfma16(ap[1], bhi, acc[i & 3]);
        }
      }
      load_unit(ud[i], n_dc, n_dsc, H, K, n_row, valid ? u : 0);  // the next item's round i
    }
    if (c_on) {
      const float4v y4 = ((acc[0] + acc[1]) + acc[2]) + acc[3];
      float* yout = shared ? a.shared_out : a.y_sorted;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = 4 * g + j;
        if (m < mnow) {
          const int64_t yr = shared ? int64_t(m) : int64_t(si_c.y + m);
          yout[yr * H + c_row] = y4[j];
        }
      }
    }
    si_c = si_n;
    si_n = si_nn;
    c_dc = n_dc;
    c_dsc = n_dsc;
    c_row = n_row;
    c_on = n_on;
  }
}

// ---------------------------------------------------------------------------
template <int QBITS>
static hipError_t launch_gemv_q(const FfnArgs& a, hipStream_t stream, int phases) {
  constexpr int NW = kTpNW;
  const int64_t P = a.T * a.k;
  const int slots = int(std::min<int64_t>(a.E, P)) + (a.has_shared ? 1 : 0);
  const int mrows = int(std::min<int64_t>(kGemvMaxM, std::max<int64_t>(a.T, 1)));
  const int max_rows = std::max(a.I, a.has_shared ? a.Is : 0);
  const bool one = a.T == 1;  // one token: latency-shaped kernels (no LDS on the gate/up side)
  if (phases & kPhaseGateUp) {
    const bool u64 = a.H % 64 == 0;
    if (one) {
      const dim3 grid(unsigned((max_rows + 15) / 16), unsigned(slots));
#define GU(U_, X_) \
  gemv_gateup_1tok_kernel<QBITS, U_, X_><<<grid, 64 * k1tokWaves, size_t(a.H) * 2, stream>>>(a, Decode1Sel{}, \
                                                                                               a.slots)
      if (a.x_kind == kXBF16) { if (u64) GU(64, uint16_t); else GU(32, uint16_t); }
      else if (a.x_kind == kXF16) { if (u64) GU(64, f16); else GU(32, f16); }
      else { if (u64) GU(64, float); else GU(32, float); }
#undef GU
    } else {
      const size_t lds = size_t(mrows) * (a.H + 8) * sizeof(f16);
      const bool pers = a.T <= kGemvMaxM && u64 && a.H % 1024 == 0 &&
                        (!a.has_shared || a.Is == a.I);
      if (pers) {
        const int n_rb = (a.I + 63) / 64;
        const int ng = pers_gateup_groups(a.T);
        const int G = pers_gateup_grid(slots, n_rb, ng);
        const size_t lds_p = size_t(a.T) * (a.H + 8) * sizeof(f16);
#define GP(X_, NG_) \
  gemv_gateup_pers_kernel<QBITS, 64, X_, false, NG_><<<G, 512 * NG_, lds_p, stream>>>(a, n_rb, G, a.slots, a.header, \
                                                                                    SelOut{})
        if (a.x_kind == kXBF16) { if (ng == 2) GP(uint16_t, 2); else GP(uint16_t, 1); }
        else if (a.x_kind == kXF16) { if (ng == 2) GP(f16, 2); else GP(f16, 1); }
        else { if (ng == 2) GP(float, 2); else GP(float, 1); }
#undef GP
      } else {
        const dim3 grid(unsigned((max_rows + 16 * NW - 1) / (16 * NW)), unsigned(slots));
#define GU(U_, X_) gemv_gateup_tp_kernel<QBITS, U_, X_, NW><<<grid, 128 * NW, lds, stream>>>(a)
        if (a.x_kind == kXBF16) { if (u64) GU(64, uint16_t); else GU(32, uint16_t); }
        else if (a.x_kind == kXF16) { if (u64) GU(64, f16); else GU(32, f16); }
        else { if (u64) GU(64, float); else GU(32, float); }
#undef GU
      }
    }
  }
  if (phases & kPhaseDown) {
    // UNIT must divide both K values; 64 only when both are multiples of 64.
    const bool u64 = a.I % 64 == 0 && (!a.has_shared || a.Is % 64 == 0);
    if (one) {
      const dim3 grid(unsigned((a.H + 63) / 64), unsigned(slots));
      if (u64) gemv_down_kernel<QBITS, 64><<<grid, 256, 0, stream>>>(a);
      else gemv_down_kernel<QBITS, 32><<<grid, 256, 0, stream>>>(a);
    } else {
      const int kmax = std::max(a.I, a.has_shared ? a.Is : 0);
      const int ldsw = kmax + 8;
      const size_t lds = size_t(mrows) * ldsw * sizeof(f16);
      const int rounds = (a.I / 64 + 3) / 4;
      const bool pers = a.T <= kGemvMaxM && a.I % 64 == 0 && rounds <= 4 &&
                        (!a.has_shared || a.Is == a.I);
      if (pers) {
        const int n_rb = (a.H + 63) / 64;
        const int G = int(std::min<int64_t>(kPersGridDown, int64_t(slots) * n_rb));
#define DP(R_) gemv_down_pers_kernel<QBITS, R_><<<G, 256, lds, stream>>>(a, ldsw, n_rb, G, a.slots, a.header)
        if (rounds == 1) DP(1);
        else if (rounds == 2) DP(2);
        else if (rounds == 3) DP(3);
        else DP(4);
#undef DP
      } else {
        const dim3 grid(unsigned((a.H + 16 * NW - 1) / (16 * NW)), unsigned(slots));
        if (u64) gemv_down_tp_kernel<QBITS, 64, NW><<<grid, 64 * NW, lds, stream>>>(a, ldsw);
        else gemv_down_tp_kernel<QBITS, 32, NW><<<grid, 64 * NW, lds, stream>>>(a, ldsw);
      }
    }
  }
  return hipGetLastError();
}

// The persistent gate/up kernel with the selection made inside it (see
// gemv_gateup_pers_kernel), for a 2..16-token layer whose shape the kernel
// takes; hipErrorNotSupported otherwise (then the caller launches the
// selection kernel and launch_ffn_gemv).
hipError_t launch_gateup_select(const FfnArgs& a, const SelOut& so, hipStream_t stream) {
  const int64_t P = a.T * a.k;
  const size_t lds_p = size_t(a.T) * (a.H + 8) * sizeof(f16);
  const bool ok = a.T >= 2 && a.T <= kGemvMaxM && a.H % 1024 == 0 &&
                  (!a.has_shared || a.Is == a.I) && a.E <= kSelPersMaxExperts && P <= 1024 &&
                  lds_p + 16384 <= kLdsBytes;
  if (!ok) return hipErrorNotSupported;
  const int slots = int(std::min<int64_t>(a.E, P)) + (a.has_shared ? 1 : 0);
  const int n_rb = (a.I + 63) / 64;
  const int ng = pers_gateup_groups(a.T);
  const int G = pers_gateup_grid(slots, n_rb, ng);
#define GS(Q_, X_, NG_) \
  gemv_gateup_pers_kernel<Q_, 64, X_, true, NG_><<<G, 512 * NG_, lds_p, stream>>>(a, n_rb, G, nullptr, nullptr, so)
#define GSX(Q_, X_)             \
  do {                          \
    if (ng == 2) GS(Q_, X_, 2); \
    else GS(Q_, X_, 1);         \
  } while (0)
#define GSQ(Q_)                          \
  if (a.x_kind == kXBF16) GSX(Q_, uint16_t); \
  else if (a.x_kind == kXF16) GSX(Q_, f16);  \
  else GSX(Q_, float)
  if (a.qbits == 2) {
    GSQ(2);
  } else if (a.qbits == 3) {
    GSQ(3);
  } else {
    GSQ(4);
  }
#undef GSQ
#undef GSX
#undef GS
  return hipGetLastError();
}

bool gemv_lds_ok(int64_t T, int H, int I, int Is) {
  const size_t m = size_t(std::max<int64_t>(1, std::min<int64_t>(T, kGemvMaxM)));
  const size_t kmax = size_t(std::max(I, Is));
  return m * (H + 8) * sizeof(f16) + 16384 <= kLdsBytes && m * (kmax + 8) * sizeof(f16) + 16384 <= kLdsBytes;
}

hipError_t launch_ffn_gemv(const FfnArgs& a, hipStream_t stream, int phases) {
  if (a.T == 0) return hipSuccess;
  return a.qbits == 2 ? launch_gemv_q<2>(a, stream, phases)
         : a.qbits == 3 ? launch_gemv_q<3>(a, stream, phases)
                        : launch_gemv_q<4>(a, stream, phases);
}

template <int QBITS>
static hipError_t launch_decode1_q(const FfnArgs& a_full, const Decode1Sel& sel, float* out, float* res,
                                   hipStream_t stream) {
  // the down + combine kernel sums the computed ranks only (all k, or the
  // ranks below kc under the route tail skip)
  FfnArgs a = a_full;
  if (sel.kc > 0 && sel.kc < a.k) a.k = sel.kc;
  const int slots = a.k + (a.has_shared ? 1 : 0);
  const int max_rows = std::max(a.I, a.has_shared ? a.Is : 0);
  {
    const bool u64 = a.H % 64 == 0;
    const dim3 grid(unsigned((max_rows + 15) / 16), unsigned(slots));
#define GU(U_, X_) \
  gemv_gateup_1tok_kernel<QBITS, U_, X_><<<grid, 64 * k1tokWaves, size_t(a.H) * 2, stream>>>(a_full, sel, a.slots)
    if (a.x_kind == kXBF16) { if (u64) GU(64, uint16_t); else GU(32, uint16_t); }
    else if (a.x_kind == kXF16) { if (u64) GU(64, f16); else GU(32, f16); }
    else { if (u64) GU(64, float); else GU(32, float); }
#undef GU
  }
  {
    const bool u64 = a.I % 64 == 0 && (!a.has_shared || a.Is % 64 == 0);
    const int pairs = (a.k + 1) / 2 + (a.has_shared ? 1 : 0);
    const int nw = std::min(pairs, 16);  // within the kernel's 1024-thread bound
    const dim3 grid(unsigned(a.H / kDcRows));
    const int ldh = std::max(a.I, a.has_shared ? a.Is : 0) + 8;
    const size_t lds = size_t(slots) * ldh * sizeof(_Float16);
#define DC(U_) \
  gemv_down_combine_1tok_kernel<QBITS, U_><<<grid, 64 * nw, lds, stream>>>(a, sel.slot_expert, sel.slot_of_rank, \
                                                                          sel.w, out, res, ldh, 64 * nw)
    if (u64) DC(64);
    else DC(32);
#undef DC
  }
  return hipGetLastError();
}

bool decode1_lds_ok(int H, int I, int Is, int k, bool has_shared) {
  const size_t slots = size_t(k) + (has_shared ? 1 : 0);
  const size_t ldh = size_t(std::max(I, has_shared ? Is : 0)) + 8;
  return size_t(H) * sizeof(f16) + 16384 <= kLdsBytes && slots * ldh * sizeof(f16) + 16384 <= kLdsBytes;
}

hipError_t launch_decode1_ffn(const FfnArgs& a, const Decode1Sel& sel, float* out, float* res, hipStream_t stream) {
  if (a.E > kDecode1MaxExperts || a.T != 1) return hipErrorInvalidValue;
  if (!decode1_lds_ok(a.H, a.I, a.Is, a.k, a.has_shared)) return hipErrorInvalidValue;
  return a.qbits == 2   ? launch_decode1_q<2>(a, sel, out, res, stream)
         : a.qbits == 3 ? launch_decode1_q<3>(a, sel, out, res, stream)
                        : launch_decode1_q<4>(a, sel, out, res, stream);
}

}  // namespace moe
