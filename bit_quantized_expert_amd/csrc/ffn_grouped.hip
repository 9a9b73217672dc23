// Expert FFN for prefill-sized batches: a grouped GEMM over the device-built
// tile list, fp16 MFMA (v_mfma_f32_32x32x16_f16) with fp32 accumulation, the
// 2/3/4-bit weights dequantised in registers straight into MFMA operands.
//
// The experts are computed from their quantised storage ("How Strata runs a
// 125-billion-parameter model ...", intro and Step 1 byte table); with many
// tokens per expert the work is a dense contraction per expert, so it runs
// on the matrix cores.  Each tile of the list is (expert or shared, first row
// m0) with BM = 128 (8 waves) or 96 (4 waves) rows of the expert's sorted
// segment.
//
//   gate/up : [BM x H] activations x [H x 32 W gate + 32 W up rows] -> SwiGLU
//             epilogue -> h (fp16, the permuted column order of the GEMV path)
//   down    : [BM x I] h x [I x 64 W down rows] -> y_sorted / shared_out (fp32,
//             or fp16 when the caller asks for y_sorted_h / shared_out_h)
//
// The activations keep the permuted 16-group k order the dequantiser
// produces (pairs (i, i+8)), so codes unpack straight into their slots.  The
// tile index is remapped so that the n-tiles of one M tile run on the same
// XCD (dispatch goes round-robin over the 8 XCDs): its activation tile is
// then fetched into one L2 instead of eight.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {


// The activations of the gate/up GEMM, converted once per call into x16: an
// fp16 copy of x [T][H] whose 16-element groups hold the permuted order the
// dequantiser produces (load_x16: {0,8,1,9,...} then {4,12,5,13,...}), so
// that staging an A tile is a plain copy for every n-tile that reads it.
template <typename XT>
__global__ __launch_bounds__(256) void x16_kernel(const XT* __restrict__ x, int64_t groups, f16* __restrict__ x16) {
  const int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (g >= groups) return;
  half8 lo, hi;
  load_x16<XT>(x + g * 16, lo, hi);
  half8* d = reinterpret_cast<half8*>(x16 + g * 16);
  d[0] = lo;
  d[1] = hi;
}

// ---------------------------------------------------------------------------
// The grouped GEMM.  A workgroup owns BM rows (128 with 8 waves, or 96 with
// 4 waves when experts hold few rows each: fewer padding rows per tile);
// each wave a BM x 64 block (BM/32 x 2 MFMA tiles of 32 x 32), so an A
// fragment read from LDS feeds two MFMAs and a B fragment BM/32.  Every
// output element goes through the same MFMA sequence for either BM.  The
// weights never pass through LDS: each wave loads and dequantises its own
// 64 columns straight into MFMA operands (lane (n, h) of a 32-column set
// takes 16 code bytes = words 4h .. 4h+3 of the row's 128-weight step; MFMA
// k-step kk pairs slice kk of lane h = 0 with slice kk of lane h = 1, and
// the A fragments are read from LDS in the same order).  K advances 128 per
// step; the activation tile is staged in LDS (fp16, permuted 16-groups) in
// two buffers (plain loop) or three (pipelined loop), one barrier per step.
// With NWV waves:
//   gate/up: wave w = gate rows nt*32*NWV + 32w .. +32 and the same up rows;
//   down   : wave w = output columns nt*64*NWV + 64w .. +64.
// ---------------------------------------------------------------------------
constexpr int kBK2 = 128, kLDA2 = kBK2 + 8;  // A row pitch in halves

template <int QBITS>
struct BRaw2 {
  uint4v c;                    // 16 code bytes: words 4h .. 4h+3
  uint32_t s;                  // two fp16 scales: blocks 2h, 2h + 1
  uint32_t hb[QBITS == 4 ? 4 : 2];  // high plane of the 64 codes: 3-bit one bit each, 4-bit two
  uint32_t v;                  // bit b: block 2h + b exists (else its scale reads as 0 in dq_b2)
};

// Where a lane's weights of step 0 start, for K a multiple of 64 (KM >= 1):
// with 16-row groups of whole 64-weight units, block 4 step + 2h of row r
// sits at a fixed offset plus step * 512 code bytes (step * 64 scales, step *
// 256 3-bit high-plane bytes), so a step's loads are base + step * stride.
// Rows past the matrix use row 0 (zeroed at dequantisation).
struct BSrc {
  const uint8_t* c;    // low plane
  const uint16_t* s;   // scales
  const uint8_t* hp;   // 3-bit high plane / 4-bit second plane
};

// (Unit h of the row, written out: with K == 64 unit 1 does not exist, and
// lane h = 1 only ever reads it at the half step, one unit back.)
template <int QBITS>
__device__ __forceinline__ BSrc bsrc_k64(const uint8_t* codes, const uint16_t* scales, int rows, int K, int row,
                                         int h, bool ok) {
  const QTile tl = qtile<true>(ok ? row : 0, rows);  // weight rows are multiples of 32: every group is full
  BSrc b;
  b.c = codes + tl.g0 * (K / 4) + h * 256 + tl.rr * 16;
  b.s = scales + tl.g0 * (K / 32) + h * 32 + tl.rr * 2;
  const uint8_t* plane = codes + int64_t(rows) * (K / 4);
  b.hp = QBITS == 3 ? plane + tl.g0 * (K / 8) + h * 128 + tl.rr * 8 : plane + tl.g0 * (K / 4) + h * 256 + tl.rr * 16;
  return b;
}

// KM >= 1: K is a multiple of 64 (even block count per row), so a lane's two
// blocks are in or out together and its 16 code bytes, 4 scale bytes (and
// 8 high-plane bytes) are aligned for single loads.
// A half step (K % 128 == 64, the last step: blocks 4 step and 4 step + 1
// only) is loaded by both lanes of a column from the first block: lane h then
// dequantises block 4 step + h alone (dq_b2 with sel), and the step runs half
// the MFMAs.  `step` is clamped to the last one (a prefetch past the end
// loads a real address and is zeroed).
template <int QBITS, int KM>
__device__ __forceinline__ void load_b2k(BRaw2<QBITS>& r, const BSrc& b, int K, int step, int nsteps, int h, bool ok) {
  const bool in = ok && step < nsteps;
  const int st = min(step, nsteps - 1);
  const bool half_step = KM == 2 && 4 * st + 2 >= K / 32;  // only blocks 4 step, 4 step + 1 (K % 128 == 64)
  const int back = half_step ? h : 0;                         // lane h = 1 reads its column's first block
  r.c = *reinterpret_cast<const uint4v*>(b.c + st * 512 - back * 256);
  r.s = *reinterpret_cast<const uint32_t*>(b.s + st * 64 - back * 32);
  if constexpr (QBITS == 3) {
    const uint2v hv = *reinterpret_cast<const uint2v*>(b.hp + st * 256 - back * 128);
    r.hb[0] = hv[0];
    r.hb[1] = hv[1];
  }
  if constexpr (QBITS == 4) {
    const uint4v hv = *reinterpret_cast<const uint4v*>(b.hp + st * 512 - back * 256);
    r.hb[0] = hv[0];
    r.hb[1] = hv[1];
    r.hb[2] = hv[2];
    r.hb[3] = hv[3];
  }
  r.v = in ? 3u : 0u;
}

// Any K (a multiple of 32): one load per block (8 code bytes, one scale: a K
// with an odd block count ends in a one-block unit), each unconditional from
// a clamped address; blocks of this lane b0 = 4 * step + 2h and b0 + 1, each
// zero past K or past the matrix.
template <int QBITS>
__device__ __forceinline__ void load_b2(BRaw2<QBITS>& r, const uint8_t* codes, const uint16_t* scales, int rows,
                                        int K, int row, int step, int h, bool ok) {
  const int nb = K / 32;
  const int b0 = 4 * step + 2 * h;
  const bool in0 = ok && b0 < nb, in1 = ok && b0 + 1 < nb;
  const int rr = in0 ? row : 0, bb0 = in0 ? b0 : 0, bb1 = in1 ? b0 + 1 : bb0;
  const QTile tl = qtile<true>(rr, rows);
  const uint2v c0 = *reinterpret_cast<const uint2v*>(codes + qt_code_off(tl, K, bb0));
  const uint2v c1 = *reinterpret_cast<const uint2v*>(codes + qt_code_off(tl, K, bb1));
  const uint32_t s0 = scales[qt_scale_off(tl, K, bb0)], s1 = scales[qt_scale_off(tl, K, bb1)];
  r.c = uint4v{c0[0], c0[1], c1[0], c1[1]};
  r.s = s0 | (s1 << 16);
  if constexpr (QBITS == 3) {
    const uint8_t* hp = codes + int64_t(rows) * (K / 4);
    r.hb[0] = *reinterpret_cast<const uint32_t*>(hp + qt_high_off(tl, K, bb0));
    r.hb[1] = *reinterpret_cast<const uint32_t*>(hp + qt_high_off(tl, K, bb1));
  }
  if constexpr (QBITS == 4) {
    const uint8_t* hp = codes + int64_t(rows) * (K / 4);
    const uint2v h0 = *reinterpret_cast<const uint2v*>(hp + qt_code_off(tl, K, bb0));
    const uint2v h1 = *reinterpret_cast<const uint2v*>(hp + qt_code_off(tl, K, bb1));
    r.hb[0] = h0[0];
    r.hb[1] = h0[1];
    r.hb[2] = h1[0];
    r.hb[3] = h1[1];
  }
  r.v = (in0 ? 1u : 0u) | (in1 ? 2u : 0u);
}

// word q (0..3) of a lane's step -> the prepared sources of its 8 pairs.
// sel (half steps, lane h = 1, q < 2): word q of the second block instead
// (block 4 step + 1).  MASK: blocks past K read as zero weights (any K); with
// K a multiple of 64 a lane's blocks are all real or belong to a column past
// the matrix or a step past the last, whose products are never stored, so
// the scale is only duplicated into both halves.
template <int QBITS, bool MASK = true>
__device__ __forceinline__ DqSrc dq_src_b2(const BRaw2<QBITS>& r, int q, bool sel) {
  const bool second = q >= 2 || sel;  // the lane's second block
  half2v s2;
  if constexpr (MASK) {
    const uint32_t sraw = second ? (r.s >> 16) : (r.s & 0xffffu);
    const uint32_t sbits = (r.v >> (q >> 1)) & 1u ? sraw : 0u;  // blocks past K: scale 0, weights 0
    s2 = as_half2(sbits | (sbits << 16));
  } else {
    s2 = as_half2(__builtin_amdgcn_perm(r.s, r.s, second ? 0x03020302u : 0x01000100u));
  }
  const uint32_t w = q < 2 && sel ? r.c[q + 2] : r.c[q];
  if constexpr (QBITS == 2) {
    return dq2_src(w, s2);
  } else if constexpr (QBITS == 4) {
    return dq4_src(w, q < 2 && sel ? r.hb[q + 2] : r.hb[q], s2);
  } else {
    uint32_t hlo, hhi;
    high3_slots(second ? r.hb[1] : r.hb[0], q & 1, hlo, hhi);
    return dq3_src(w, hlo, hhi, s2);
  }
}

// word q of a lane's step -> the two permuted k-slices
template <int QBITS, bool MASK = true>
__device__ __forceinline__ void dq_b2(const BRaw2<QBITS>& r, int q, bool sel, half8& lo, half8& hi) {
  dq_word<QBITS>(dq_src_b2<QBITS, MASK>(r, q, sel), lo, hi);
}

// silu(g) = g / (1 + e^-g) from the hardware exp2 and reciprocal (about 1e-7
// relative error, far below the fp16 rounding of h).
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * g));
}

// The main loop comes in two forms: the software-pipelined one (below) with
// 96-row tiles, and a plain one with 128-row tiles, where the pipeline's
// extra registers do not fit beside the accumulators (the compiler would
// spill).
template <int QBITS, int BM>
constexpr bool grouped_pipelined() { return BM == 96; }

// KM: 0 = any K (a multiple of 32), 1 = K a multiple of 64, 2 = K a multiple
// of 64 that may end in a half step (K % 128 == 64; the checks and selects of
// half steps cost VALU in every step, so only this instantiation has them).
template <int QBITS, bool GATEUP, int NWV, int KM, int BM>
__global__ __launch_bounds__(64 * NWV, NWV > 4 ? 1 : 2) void grouped_gemm2_kernel(FfnArgs a, int n_ntiles) {
  static_assert(BM % 32 == 0 && BM <= 128, "whole 32-row MFMA tiles");
  constexpr int NT = 64 * NWV;                         // threads
  constexpr int MI = BM / 32;                          // MFMA row tiles per wave
  constexpr int AITEMS = BM * (kBK2 / 16);             // A staging items (16-element groups) per step
  constexpr int AI = (AITEMS + NT - 1) / NT;           // per thread (the last may be past the tile)
  constexpr bool PIPE = grouped_pipelined<QBITS, BM>();
  __shared__ __attribute__((aligned(16))) f16 As[PIPE ? 3 : 2][BM * kLDA2];

  // ---- work item (XCD-aware remap over the real items)
  const int n_tiles = a.header[kHdrTiles];
  const int total = n_tiles * n_ntiles;
  const int per = (total + 7) / 8;
  const int b = blockIdx.x;
  if (b >= 8 * per) return;
  const int L = (b % 8) * per + b / 8;
  if (L >= total) return;
  const int tile = L / n_ntiles, nt = L - tile * n_ntiles;
  const int4 td = a.tile_desc[tile];  // {expert (-1 = shared), first row in the segment, first sorted row, rows}
  const int e = td.x, m0 = td.y;
  const bool shared = e < 0;
  const int lo = td.z - m0;  // first sorted row of the expert's segment (0 for the shared expert)
  const int rows_valid = td.w;
  const int H = a.H;
  const int K = GATEUP ? H : (shared ? a.Is : a.I);
  const int Nrows = GATEUP ? (shared ? a.Is : a.I) : H;  // rows of each weight matrix
  const int64_t ex = shared ? 0 : e;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;

  // ---- A sources (fp16 in the permuted order: the x16 copy of x, or h):
  // thread handles items tid + NT i (i < AI) of the BM x 8 groups; an item
  // past the tile loads a real row and is never stored
  const f16* asrc[AI];
  int arow[AI], agrp[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int item = min(tid + NT * i, AITEMS - 1);
    arow[i] = item >> 3;
    agrp[i] = item & 7;
    const int r = min(arow[i], rows_valid - 1);  // rows past the segment read a real row; never stored
    if constexpr (GATEUP) {
      const int64_t tok = shared ? int64_t(m0 + r) : int64_t(a.sorted_pair[lo + m0 + r] / a.k);
      asrc[i] = a.x16 + tok * H + agrp[i] * 16;
    } else {
      asrc[i] = (shared ? a.h_shared + int64_t(m0 + r) * K : a.h_routed + int64_t(lo + m0 + r) * K) + agrp[i] * 16;
    }
  }
  // ---- B sources: two 32-column sets per wave
  const uint8_t* bc[2];
  const uint16_t* bsc[2];
  int brow[2];
  bool bok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    QMat M;
    if constexpr (GATEUP) {
      M = j == 0 ? (shared ? a.sg : a.rg) : (shared ? a.su : a.ru);
      brow[j] = nt * (32 * NWV) + 32 * wv + n;
    } else {
      M = shared ? a.sd : a.rd;
      brow[j] = nt * (64 * NWV) + 64 * wv + 32 * j + n;
    }
    bc[j] = M.codes + ex * M.code_stride;
    bsc[j] = M.scales + ex * M.scale_stride;
    bok[j] = brow[j] < Nrows;
  }
  // a wave whose columns all lie past the matrix (the last n-tile of a
  // matrix whose rows are not a multiple of the tile) stages its share of A
  // and keeps the barriers, but loads and multiplies nothing
  const bool live = (GATEUP ? nt * (32 * NWV) + 32 * wv : nt * (64 * NWV) + 64 * wv) < Nrows;
  BSrc bsrc[2];
  if constexpr (KM >= 1) {
#pragma unroll
    for (int j = 0; j < 2; ++j) bsrc[j] = bsrc_k64<QBITS>(bc[j], bsc[j], Nrows, K, brow[j], h, bok[j]);
  }
  const int nsteps = (K + kBK2 - 1) / kBK2;
  auto load_b = [&](BRaw2<QBITS>& r, int j, int step) {
    if constexpr (KM >= 1) load_b2k<QBITS, KM>(r, bsrc[j], K, step, nsteps, h, bok[j]);
    else load_b2<QBITS>(r, bc[j], bsc[j], Nrows, K, brow[j], step, h, bok[j]);
  };

  auto load_a = [&](int step, uint4v (&r)[AI][2]) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      // K tail: the group's weights are zero, so any finite values do: the row's first group
      // (with K a multiple of 128 every step is whole)
      const int col = KM == 1 || step * kBK2 + agrp[i] * 16 < K ? step * kBK2 : -agrp[i] * 16;
      const uint4v* p = reinterpret_cast<const uint4v*>(asrc[i] + col);
      r[i][0] = p[0];
      r[i][1] = p[1];
    }
  };
  // rows past the tile's rows are zeroed once in every buffer and never
  // stored again (their MFMA products are discarded either way; zero operands
  // cost the matrix cores less power than copies of a real row)
  auto store_a = [&](const uint4v (&r)[AI][2], f16* buf) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      if ((AITEMS % NT != 0 && tid + NT * i >= AITEMS) || arow[i] >= rows_valid) continue;
      uint4v* d = reinterpret_cast<uint4v*>(buf + arow[i] * kLDA2 + agrp[i] * 16);
      d[0] = r[i][0];
      d[1] = r[i][1];
    }
  };
  if (rows_valid < BM) {
#pragma unroll
    for (int bb = 0; bb < (PIPE ? 3 : 2); ++bb)
#pragma unroll
      for (int i = 0; i < AI; ++i) {
        if ((AITEMS % NT != 0 && tid + NT * i >= AITEMS) || arow[i] < rows_valid) continue;
        uint4v* d = reinterpret_cast<uint4v*>(As[bb] + arow[i] * kLDA2 + agrp[i] * 16);
        d[0] = uint4v{0u, 0u, 0u, 0u};
        d[1] = uint4v{0u, 0u, 0u, 0u};
      }
  }

  float16v acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  uint4v ar[AI][2];
  if constexpr (PIPE) {
    // The loop runs over words: word q of step s is MFMA k-steps 2q (half 0)
    // and 2q + 1 (half 1), 2 MI MFMAs each.  It is software-pipelined so that
    // the MFMAs of one word overlap the work that feeds the next:
    //   * the next word's weights are dequantised during this word (column
    //     set j during half j), their steps spread over the half's MFMAs and
    //     taken four pairs at a time so that consecutive VALU ops are
    //     independent;
    //   * the next half's activation fragments are read from LDS during this
    //     half, each row tile's right after its last MFMA of this half, into
    //     the same registers;
    // each MFMA closing a group that a scheduling barrier keeps in this order
    // (left alone, the compiler issues the dequantisation in bursts between
    // MFMAs and waits for each LDS read right before its MFMA).
    // Rings: activations in three LDS buffers, staged two steps ahead (so the
    // next step's first fragments can be read before this step's barrier);
    // raw weights in two register sets (even and odd steps), reloaded two
    // steps ahead right after their last word is dequantised.  Every load is
    // unconditional (steps past K are clamped and zeroed): a reload before
    // the use needs a register copy, and those copies, like loads under a
    // branch, make the compiler wait for every load in flight.
    // A half step (KM == 2, K % 128 == 64) is always the last step; its words
    // 2 and 3 are not run, and the word dequantised after its word 1 is never
    // used.
    auto half_step = [&](int st) { return KM == 2 && 4 * st + 2 >= K / 32; };
    constexpr int S = dq_stages<QBITS>(), NOPS = 8 * S;  // dequantisation steps of one word
    BRaw2<QBITS> rawA[2], rawB[2];  // raw weights of the even and odd steps [column set]
    half8 bf[2][2][2];              // [word parity][half][column set]
    half8 af[MI];                   // [row tile], refilled for the next half right after its last use
    auto frag = [&](const f16* Ab, int i, int col) -> half8 {
      return *reinterpret_cast<const half8*>(Ab + (32 * i + n) * kLDA2 + col);
    };
    {  // the first two steps' activations and weights are all in flight together
      uint4v ar1[AI][2];
      load_a(0, ar);
      load_a(min(1, nsteps - 1), ar1);
      if (live) {
#pragma unroll
        for (int j = 0; j < 2; ++j) load_b(rawA[j], j, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j) load_b(rawB[j], j, 1);
      }
      store_a(ar, As[0]);
      store_a(ar1, As[1]);
    }
    __syncthreads();
    if (live) {
      const bool hs0 = half_step(0);
#pragma unroll
      for (int j = 0; j < 2; ++j) dq_b2<QBITS, KM == 0>(rawA[j], 0, hs0 && h, bf[0][0][j], bf[0][1][j]);
#pragma unroll
      for (int i = 0; i < MI; ++i) af[i] = frag(As[0], i, (hs0 ? 32 : 64) * h);
    }
    // one step; rc: its raw weights (reloaded two steps ahead), rn: the next step's
    auto run_step = [&](int step, BRaw2<QBITS>(&rc)[2], BRaw2<QBITS>(&rn)[2]) {
      load_a(min(step + 2, nsteps - 1), ar);  // activations two steps ahead (clamped at the end)
      __builtin_amdgcn_sched_barrier(0);
      if (live) {
        const f16* Ab = As[step % 3];
        const f16* An = As[(step + 1) % 3];
        const bool hs = half_step(step), hsn = half_step(step + 1);
        const int acol = (hs ? 32 : 64) * h, acoln = (hsn ? 32 : 64) * h;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q >= 2 && hs) break;
          const int c = q & 1;
          const bool last = q == 3;  // the next word is word 0 of the next step
          const int qn = last ? 0 : q + 1;
          const bool seln = (last ? hsn : hs) && h;
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            DqSrc d;
            uint32_t tw[8];
#pragma unroll
            for (int g = 0; g < 2 * MI; ++g) {
              const int i = g >> 1, j = g & 1;
              acc[i][j] = mfma32(af[i], bf[c][hf][j], acc[i][j]);
              // after its second MFMA, row tile i's fragment of the next half: half 1
              // of this word, or half 0 of the next word (read 2 MI - 2 MFMAs ahead)
              if (j == 1) {
                if (hf == 0) af[i] = frag(Ab, i, acol + 16 * q + 8);
                else if (last) af[i] = frag(An, i, acoln);
                else af[i] = frag(Ab, i, acol + 16 * (q + 1));
              }
              if (g == 0) {
                if (last) d = dq_src_b2<QBITS, KM == 0>(rn[hf], qn, seln);
                else d = dq_src_b2<QBITS, KM == 0>(rc[hf], qn, seln);
              }
              // this group's share of the word's dequantisation steps, taken four
              // pairs at a time step by step, so that consecutive VALU ops are
              // independent
#pragma unroll
              for (int o = g * NOPS / (2 * MI); o < (g + 1) * NOPS / (2 * MI); ++o) {
                const int stage = (o % (4 * S)) / 4, pi = (o / (4 * S)) * 4 + o % 4;
                dq_step<QBITS>(d, pi, stage, tw[pi]);
                if (stage == S - 1) {
                  const half2v v = as_half2(tw[pi]);
                  half8& dst = bf[c ^ 1][pi >> 2][hf];
                  dst[2 * (pi & 3)] = v[0];
                  dst[2 * (pi & 3) + 1] = v[1];
                }
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          if (q == 2) {  // this step's last word is dequantised: reload its set two steps ahead
#pragma unroll
            for (int j = 0; j < 2; ++j) load_b(rc[j], j, step + 2);
          }
        }
      }
      store_a(ar, As[(step + 2) % 3]);
      __syncthreads();
    };
    for (int s0 = 0; s0 < nsteps; s0 += 2) {
      run_step(s0, rawA, rawB);
      if (s0 + 1 < nsteps) run_step(s0 + 1, rawB, rawA);
    }
  } else {
    // B ring of one step: the weights of the next step are loaded right after
    // this step's are dequantised.  Every load is unconditional (steps past K
    // are clamped): a reload before the use needs a register copy, and those
    // copies, like loads under a branch, make the compiler wait for every load
    // in flight.
    BRaw2<QBITS> bring[2];
    load_a(0, ar);
    if (live) {
#pragma unroll
      for (int j = 0; j < 2; ++j) load_b(bring[j], j, 0);
    }
    store_a(ar, As[0]);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
      const int cur = step & 1;
      load_a(min(step + 1, nsteps - 1), ar);  // the next step's activations (the last step reloads its own)
      // keep the activation loads here, a whole step ahead of their LDS store
      // (the scheduler would otherwise sink them to their use)
      __builtin_amdgcn_sched_barrier(0);
      if (live) {
        const f16* Ab = As[cur];
        // half step (K % 128 == 64, the last step): lane h holds block 4 step + h, A columns
        // 32h .. 32h + 31, and words 2, 3 (k-steps 4 .. 7) are not run
        const bool half_step = KM == 2 && 4 * step + 2 >= K / 32;
        const bool sel = half_step && h;
        const int acol = (half_step ? 32 : 64) * h;
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // word q of each lane's step: k-steps 2q (lo) and 2q + 1 (hi)
          if (q >= 2 && half_step) break;
          half8 blo[2], bhi[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) dq_b2<QBITS, KM == 0>(bring[j], q, sel, blo[j], bhi[j]);
#pragma unroll
          for (int half_ = 0; half_ < 2; ++half_) {
            half8 af[MI];
#pragma unroll
            for (int i = 0; i < MI; ++i)
              af[i] = *reinterpret_cast<const half8*>(Ab + (32 * i + n) * kLDA2 + acol + 16 * q + 8 * half_);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], half_ ? bhi[j] : blo[j], acc[i][j]);
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) load_b(bring[j], j, step + 1);
      }
      store_a(ar, As[cur ^ 1]);  // (after the last step: a buffer nobody reads any more)
      __syncthreads();
    }

  }

  // ---- epilogue.  32 x 32 D layout: lane l holds column l % 32 and rows
  // 8*(q/4) + 4*(l/32) + q%4, q = 0..15.  fp16 outputs (h; the down rows a
  // layer hands to its combine) are transposed through the activation
  // buffers (free after the loop's last barrier) and leave as whole 16-byte
  // row pieces; fp32 rows are stored lane by lane.
  f16* o16 = nullptr;  // the tile's first output row (fp16), row pitch Nrows, or null
  if constexpr (GATEUP) {
    o16 = shared ? a.h_shared + int64_t(m0) * Nrows : a.h_routed + int64_t(lo + m0) * Nrows;
  } else {
    f16* y16 = shared ? a.shared_out_h : a.y_sorted_h;
    if (y16) o16 = y16 + int64_t(shared ? m0 : lo + m0) * Nrows;
  }
  if (o16 != nullptr) {
    constexpr int OW = (GATEUP ? 32 : 64) * NWV;              // output columns of the tile
    constexpr int AS_H = (PIPE ? 3 : 2) * BM * kLDA2;          // halves of the activation buffers
    constexpr int NPASS = BM * (OW + 8) <= AS_H ? 1 : 2;       // column passes
    constexpr int PW = OW / NPASS, OP = PW + 8;                // pass width, LDS row pitch (halves)
    constexpr int PPR = PW / 8;                                // 16-byte pieces per row
    static_assert(BM * OP <= AS_H && OW % NPASS == 0, "an output pass fits the activation buffers");
    f16* ot = &As[0][0];
    const int c0 = nt * OW;                // the tile's first output column
    const int wc = (GATEUP ? 32 : 64) * wv;  // this wave's first column in the tile
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
      if (live && wc >= pass * PW && wc < (pass + 1) * PW) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int m = 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
            if constexpr (GATEUP) {
              // h in the permuted 16-group column order (hcol keeps a 16-group in place)
              ot[m * OP + hcol(wc + n) - pass * PW] = f16(silu_fast(acc[i][0][q]) * acc[i][1][q]);
            } else {
#pragma unroll
              for (int j = 0; j < 2; ++j) ot[m * OP + wc + 32 * j + n - pass * PW] = f16(acc[i][j][q]);
            }
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int it = tid; it < BM * PPR; it += NT) {
        const int r = it / PPR, pc = it - r * PPR;
        const int col = c0 + pass * PW + 8 * pc;
        if (r < rows_valid && col < Nrows)
          *reinterpret_cast<uint4v*>(o16 + int64_t(r) * Nrows + col) =
              *reinterpret_cast<const uint4v*>(ot + r * OP + 8 * pc);
      }
      if (pass + 1 < NPASS) __syncthreads();
    }
    return;
  }
  if (!live) return;
  if constexpr (!GATEUP) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
        if (m >= rows_valid) continue;
        float* yrow = shared ? a.shared_out + int64_t(m0 + m) * H : a.y_sorted + int64_t(lo + m0 + m) * H;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (bok[j]) yrow[brow[j]] = acc[i][j][q];
      }
    }
  }
}

// Waves per workgroup: 8 (BM x 512 tiles, one workgroup per CU) with 128-row
// tiles; 4 (BM x 256, two workgroups per CU, so that one's prologue and
// epilogue overlap the other's MFMAs) with the 96-row tiles of short segments
// (measured on the 3-bit 4,096-token layer: gate/up -2%, down -8%; with
// 128-row tiles 4 waves were no faster, and a second step of weight loads in
// flight was no faster either).
constexpr int grouped_waves(int bm) { return bm == 96 ? 4 : 8; }

template <int QBITS, int BM>
static hipError_t launch_grouped_q(const FfnArgs& a, int64_t max_tiles, hipStream_t stream, int phases) {
  constexpr int W = grouped_waves(BM);
  if (phases & kPhaseGateUp) {
    const int rows = std::max(a.I, a.has_shared ? a.Is : 0);
    const int nn = (rows + 32 * W - 1) / (32 * W);
    const int64_t total = max_tiles * nn;
    const unsigned grid = unsigned((total + 7) / 8 * 8);
    if (a.H % 128 == 0) grouped_gemm2_kernel<QBITS, true, W, 1, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
    else if (a.H % 64 == 0) grouped_gemm2_kernel<QBITS, true, W, 2, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
    else grouped_gemm2_kernel<QBITS, true, W, 0, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
  }
  if (phases & kPhaseDown) {
    const int nn = (a.H + 64 * W - 1) / (64 * W);
    const int64_t total = max_tiles * nn;
    const unsigned grid = unsigned((total + 7) / 8 * 8);
    const bool k64 = a.I % 64 == 0 && (!a.has_shared || a.Is % 64 == 0);
    const bool k128 = a.I % 128 == 0 && (!a.has_shared || a.Is % 128 == 0);
    if (k128)
      grouped_gemm2_kernel<QBITS, false, W, 1, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
    else if (k64)
      grouped_gemm2_kernel<QBITS, false, W, 2, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
    else
      grouped_gemm2_kernel<QBITS, false, W, 0, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
  }
  return hipGetLastError();
}

// Rows per tile: 96 when the routed experts hold at most ~90 rows each on
// average (then most experts fit one 96-row tile, with fewer padding rows
// than in a 128-row one), else 128.
int grouped_tile_rows(int64_t T, int k, int E) {
  const int64_t P = T * k, active = std::max<int64_t>(1, std::min<int64_t>(E, P));
  return P <= 90 * active ? 96 : 128;
}

hipError_t launch_x16(const FfnArgs& a, hipStream_t stream) {
  const int64_t groups = a.T * (a.H / 16);
  if (groups == 0) return hipSuccess;
  if (a.x_kind == kXBF16)
    x16_kernel<uint16_t><<<unsigned((groups + 255) / 256), 256, 0, stream>>>(static_cast<const uint16_t*>(a.x), groups,
                                                                            a.x16);
  else if (a.x_kind == kXF16)
    x16_kernel<f16><<<unsigned((groups + 255) / 256), 256, 0, stream>>>(static_cast<const f16*>(a.x), groups, a.x16);
  else
    x16_kernel<float><<<unsigned((groups + 255) / 256), 256, 0, stream>>>(static_cast<const float*>(a.x), groups, a.x16);
  return hipGetLastError();
}

hipError_t launch_ffn_grouped(const FfnArgs& a, int64_t max_tiles, int bm, hipStream_t stream, int phases) {
  if (a.T == 0) return hipSuccess;
  if (bm != 96 && bm != 128) return hipErrorInvalidValue;
#define GQ(Q_) \
  return bm == 96 ? launch_grouped_q<Q_, 96>(a, max_tiles, stream, phases) \
                  : launch_grouped_q<Q_, 128>(a, max_tiles, stream, phases)
  if (a.qbits == 2) GQ(2);
  if (a.qbits == 4) GQ(4);
  GQ(3);
#undef GQ
}

}  // namespace moe
