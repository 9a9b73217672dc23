// Expert FFN for prefill-sized batches: a grouped GEMM over the device-built
// tile list, fp16 MFMA (v_mfma_f32_32x32x16_f16) with fp32 accumulation, the
// 2/3/4-bit weights dequantised in registers straight into MFMA operands.
//
// The experts are computed from their quantised storage ("How Strata runs a
// 125-billion-parameter model ...", intro and Step 1 byte table); with many
// tokens per expert the work is a dense contraction per expert, so it runs
// on the matrix cores.  Each tile of the list is (expert or shared, first row
// m0) with BM = 128 rows of the expert's sorted segment.
//
//   gate/up : [BM x H] activations x [H x 256 gate + 256 up rows] -> SwiGLU
//             epilogue -> h (fp16, the permuted column order of the GEMV path)
//   down    : [BM x I] h x [I x 512 down rows] -> y_sorted / shared_out (fp32;
//             routed rows in fp16 when the caller asks for y_sorted_h)
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

// Waves per workgroup: 8 (BM x 512 tiles, one workgroup per CU) with 128-row
// tiles; 4 (BM x 256, two workgroups per CU, so that one's prologue and
// epilogue overlap the other's MFMAs) with the 96-row tiles of short segments
// (measured on the 3-bit 4,096-token layer: gate/up -2%, down -8%; with
// 128-row tiles 4 waves were no faster).
#ifndef MOE_GROUPED2_WAVES
#define MOE_GROUPED2_WAVES(BM) ((BM) == 96 ? 4 : 8)
#endif
#ifndef MOE_GROUPED2_PD
#define MOE_GROUPED2_PD 1
#endif

// Raw A operand of one thread for one K step: two 16-element groups.
template <typename AT>
struct ARaw {
  uint4v v[2][sizeof(AT) == 4 ? 4 : 2];  // fp32: 64 B per group; 16-bit: 32 B
};

template <typename AT>
__device__ __forceinline__ void load_araw(const AT* src, ARaw<AT>& r, int i) {
  const uint4v* p = reinterpret_cast<const uint4v*>(src);
#pragma unroll
  for (int q = 0; q < (sizeof(AT) == 4 ? 4 : 2); ++q) r.v[i][q] = p[q];
}

// Convert one raw group to the two permuted fp16 slices (the order of
// load_x16: lo = weights {0,8,1,9,2,10,3,11}, hi = {4,12,5,13,6,14,7,15}).
template <typename AT>
__device__ __forceinline__ void cvt_araw(const ARaw<AT>& r, int i, half8& lo, half8& hi) {
  if constexpr (std::is_same<AT, f16>::value) {  // h: already fp16 in the permuted order
    lo = __builtin_bit_cast(half8, r.v[i][0]);
    hi = __builtin_bit_cast(half8, r.v[i][1]);
  } else {
    float v[16];
    if constexpr (sizeof(AT) == 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) v[4 * q + u] = __uint_as_float(r.v[i][q][u]);
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v[8 * q + 2 * u] = __uint_as_float(r.v[i][q][u] << 16);
          v[8 * q + 2 * u + 1] = __uint_as_float(r.v[i][q][u] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lo[2 * q] = f16(v[q]);
      lo[2 * q + 1] = f16(v[q + 8]);
      hi[2 * q] = f16(v[4 + q]);
      hi[2 * q + 1] = f16(v[12 + q]);
    }
  }
}

// ---------------------------------------------------------------------------
// The grouped GEMM.  A workgroup owns BM rows (128, or 96 when experts hold
// few rows each: fewer padding rows per tile) x 8 waves; each wave a
// BM x 64 block (BM/32 x 2 MFMA tiles of 32 x 32), so an A fragment read
// from LDS feeds two MFMAs and a B fragment BM/32.  Every output element
// goes through the same MFMA sequence for either BM.  The
// weights never pass through LDS: each wave loads and dequantises its own
// 64 columns straight into MFMA operands (lane (n, h) of a 32-column set
// takes 16 code bytes = words 4h .. 4h+3 of the row's 128-weight step; MFMA
// k-step kk pairs slice kk of lane h = 0 with slice kk of lane h = 1, and
// the A fragments are read from LDS in the same order).  K advances 128 per
// step; the activation tile is double-buffered in LDS (fp16, permuted
// 16-groups), one barrier per step.
//   gate/up: wave w = gate rows nt*256 + 32w .. +32 and the same up rows;
//   down   : wave w = output columns nt*512 + 64w .. +64.
// ---------------------------------------------------------------------------
constexpr int kBK2 = 128, kLDA2 = kBK2 + 8;  // A row pitch in halves

template <int QBITS>
struct BRaw2 {
  uint4v c;                    // 16 code bytes: words 4h .. 4h+3
  uint32_t s;                  // two fp16 scales: blocks 2h, 2h + 1
  uint32_t hb[QBITS == 4 ? 4 : 2];  // high plane of the 64 codes: 3-bit one bit each, 4-bit two
  uint32_t v;                  // bit b: block 2h + b exists (else its scale reads as 0 in dq_b2)
};

// KM >= 1: K is a multiple of 64 (even block count per row), so a lane's two
// blocks are in or out together and its 16 code bytes, 4 scale bytes (and
// 8 high-plane bytes) are aligned for single loads.
// A half step (K % 128 == 64, the last step: blocks 4 step and 4 step + 1
// only) is loaded by both lanes of a column from the first block: lane h then
// dequantises block 4 step + h alone (dq_b2 with sel), and the step runs half
// the MFMAs.
template <int QBITS, int KM>
__device__ __forceinline__ void load_b2(BRaw2<QBITS>& r, const uint8_t* codes, const uint16_t* scales, int rows,
                                        int K, int row, int step, int h, bool ok) {
  if constexpr (KM >= 1) {
    const int nb = K / 32;
    const bool half_step = KM == 2 && 4 * step + 2 >= nb;  // only blocks 4 step, 4 step + 1 (K % 128 == 64)
    const int b0 = 4 * step + (half_step ? 0 : 2 * h);
    const bool in = ok && b0 < nb;
    const int rr = in ? row : 0, bb = in ? b0 : 0;
    const QTile tl = qtile<true>(rr, rows);  // tiled layout (common.h); weight rows are multiples of 32
    // raw values only: a select on a loaded value here would wait for the
    // load; blocks past K are zeroed through their scale at dequantisation
    r.c = *reinterpret_cast<const uint4v*>(codes + qt_code_off(tl, K, bb));
    r.s = *reinterpret_cast<const uint32_t*>(scales + qt_scale_off(tl, K, bb));
    if constexpr (QBITS == 3) {
      const uint2v hv = *reinterpret_cast<const uint2v*>(codes + int64_t(rows) * (K / 4) + qt_high_off(tl, K, bb));
      r.hb[0] = hv[0];
      r.hb[1] = hv[1];
    }
    if constexpr (QBITS == 4) {
      const uint4v hv = *reinterpret_cast<const uint4v*>(codes + int64_t(rows) * (K / 4) + qt_code_off(tl, K, bb));
      r.hb[0] = hv[0];
      r.hb[1] = hv[1];
      r.hb[2] = hv[2];
      r.hb[3] = hv[3];
    }
    r.v = in ? 3u : 0u;
    return;
  }
  // blocks of this lane: b0 = 4 * step + 2h and b0 + 1, each zero past K or
  // past the matrix.  One load per block (8 code bytes, one scale: a K with
  // an odd block count ends in a one-block unit), each unconditional from a
  // clamped address.
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

// word q (0..3) of a lane's step -> the two permuted k-slices.  sel (half
// steps, lane h = 1, q < 2): word q of the second block instead (block
// 4 step + 1).
template <int QBITS>
__device__ __forceinline__ void dq_b2(const BRaw2<QBITS>& r, int q, bool sel, half8& lo, half8& hi) {
  const bool second = q >= 2 || sel;  // the lane's second block
  const uint32_t sraw = second ? (r.s >> 16) : (r.s & 0xffffu);
  const uint32_t sbits = (r.v >> (q >> 1)) & 1u ? sraw : 0u;  // blocks past K: scale 0, weights 0
  const half2v s2 = as_half2(sbits | (sbits << 16));
  const uint32_t w = q < 2 && sel ? r.c[q + 2] : r.c[q];
  if constexpr (QBITS == 2) {
    dq2_word(w, s2, lo, hi);
  } else if constexpr (QBITS == 4) {
    dq4_word(w, q < 2 && sel ? r.hb[q + 2] : r.hb[q], s2, lo, hi);
  } else {
    uint32_t hlo, hhi;
    high3_slots(r.hb[second ? 1 : 0], q & 1, hlo, hhi);
    dq3_word(w, hlo, hhi, s2, lo, hi);
  }
}

// KM: 0 = any K (a multiple of 32), 1 = K a multiple of 64, 2 = K a multiple
// of 64 that may end in a half step (K % 128 == 64; the checks and selects of
// half steps cost VALU in every step, so only this instantiation has them).
template <int QBITS, typename AT, bool GATEUP, int NWV, int PD, int KM, int BM>
__global__ __launch_bounds__(64 * NWV, sizeof(AT) == 4 || NWV > 4 ? 1 : 2) void grouped_gemm2_kernel(FfnArgs a,
                                                                                                 int n_ntiles) {
  static_assert(BM % 32 == 0 && BM <= 128, "whole 32-row MFMA tiles");
  constexpr int NT = 64 * NWV;                         // threads
  constexpr int MI = BM / 32;                          // MFMA row tiles per wave
  constexpr int AITEMS = BM * (kBK2 / 16);             // A staging items (16-element groups) per step
  constexpr int AI = (AITEMS + NT - 1) / NT;           // per thread (the last may be past the tile)
  __shared__ __attribute__((aligned(16))) f16 As[2][BM * kLDA2];

  // ---- work item (XCD-aware remap over the real items)
  const int n_tiles = a.header[kHdrTiles];
  const int total = n_tiles * n_ntiles;
  const int per = (total + 7) / 8;
  const int b = blockIdx.x;
  if (b >= 8 * per) return;
  const int L = (b % 8) * per + b / 8;
  if (L >= total) return;
  const int tile = L / n_ntiles, nt = L - tile * n_ntiles;
  const int e = a.tile_expert[tile], m0 = a.tile_m0[tile];
  const bool shared = e < 0;
  const int lo = shared ? 0 : a.offsets[e];
  const int m_count = shared ? int(a.T) : a.offsets[e + 1] - lo;
  const int rows_valid = min(BM, m_count - m0);
  const int H = a.H;
  const int K = GATEUP ? H : (shared ? a.Is : a.I);
  const int Nrows = GATEUP ? (shared ? a.Is : a.I) : H;  // rows of each weight matrix
  const int64_t ex = shared ? 0 : e;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;

  // ---- A sources: thread handles items tid + NT i (i < AI) of the BM x 8
  // groups; an item past the tile loads a real row and is never stored
  const AT* asrc[AI];
  int arow[AI], agrp[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int item = min(tid + NT * i, AITEMS - 1);
    arow[i] = item >> 3;
    agrp[i] = item & 7;
    const int r = min(arow[i], rows_valid - 1);  // rows past the segment read a real row; never stored
    if constexpr (GATEUP) {
      const int64_t tok = shared ? int64_t(m0 + r) : int64_t(a.sorted_pair[lo + m0 + r] / a.k);
      asrc[i] = static_cast<const AT*>(a.x) + tok * H;
    } else {
      const f16* hb = shared ? a.h_shared + int64_t(m0 + r) * K : a.h_routed + int64_t(lo + m0 + r) * K;
      asrc[i] = reinterpret_cast<const AT*>(hb);
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
  const int nsteps = (K + kBK2 - 1) / kBK2;

  using Raw = ARaw<AT>;
  constexpr int AR = (AI + 1) / 2;  // ARaw holds two groups
  auto load_a = [&](int step, Raw (&r)[AR]) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      int col = step * kBK2 + agrp[i] * 16;
      if (col >= K) col = 0;  // K tail: the matching weights are zero
      load_araw<AT>(asrc[i] + col, r[i >> 1], i & 1);
    }
  };
  auto store_a = [&](const Raw (&r)[AR], f16* buf) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      if (AITEMS % NT != 0 && tid + NT * i >= AITEMS) continue;
      half8 l8, h8;
      cvt_araw<AT>(r[i >> 1], i & 1, l8, h8);
      half8* d = reinterpret_cast<half8*>(buf + arow[i] * kLDA2 + agrp[i] * 16);
      d[0] = l8;
      d[1] = h8;
    }
  };

  float16v acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // B ring: the weights of steps step .. step + PD - 1 are in flight (a
  // ring of PD register sets; slot p holds steps p, p + PD, ...).  A slot is
  // dequantised in place and reloaded only after its step's MFMAs, and every
  // load is unconditional (steps past K are clamped in load_b2 / load_a): a
  // reload before the use needs a register copy, and those copies, like
  // loads under a branch, make the compiler wait for every load in flight.
  Raw ar[AR];
  BRaw2<QBITS> bring[PD][2];
  load_a(0, ar);
#pragma unroll
  for (int p = 0; p < PD; ++p)
#pragma unroll
    for (int j = 0; j < 2; ++j) load_b2<QBITS, KM>(bring[p][j], bc[j], bsc[j], Nrows, K, brow[j], p, h, bok[j]);
  store_a(ar, As[0]);
  __syncthreads();
  for (int s0 = 0; s0 < nsteps; s0 += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int step = s0 + p;
      if (step >= nsteps) break;
      const int cur = step & 1;
      load_a(min(step + 1, nsteps - 1), ar);  // the next step's activations (the last step reloads its own)
      // keep the activation loads here, a whole step ahead of their LDS store
      // (the scheduler would otherwise sink them to their use)
      __builtin_amdgcn_sched_barrier(0);
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
        for (int j = 0; j < 2; ++j) dq_b2<QBITS>(bring[p][j], q, sel, blo[j], bhi[j]);
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
      for (int j = 0; j < 2; ++j)
        load_b2<QBITS, KM>(bring[p][j], bc[j], bsc[j], Nrows, K, brow[j], step + PD, h, bok[j]);
      store_a(ar, As[cur ^ 1]);  // (after the last step: a buffer nobody reads any more)
      __syncthreads();
    }
  }

  // ---- epilogue.  32 x 32 D layout: lane l holds column l % 32 and rows
  // 8*(q/4) + 4*(l/32) + q%4, q = 0..15.
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int m = 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
      if (m >= rows_valid) continue;
      if constexpr (GATEUP) {
        const int gr = brow[0];
        if (bok[0]) {
          const float g = acc[i][0][q], u = acc[i][1][q];
          const float hv = g / (1.0f + expf(-g)) * u;
          const int hw = shared ? a.Is : a.I;
          f16* hout = shared ? a.h_shared + int64_t(m0 + m) * hw : a.h_routed + int64_t(lo + m0 + m) * hw;
          hout[hcol(gr)] = f16(hv);
        }
      } else if (!shared && a.y_sorted_h) {  // routed rows in fp16
        f16* yrow = a.y_sorted_h + int64_t(lo + m0 + m) * H;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (bok[j]) yrow[brow[j]] = f16(acc[i][j][q]);
      } else {
        float* yrow = shared ? a.shared_out + int64_t(m0 + m) * H : a.y_sorted + int64_t(lo + m0 + m) * H;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (bok[j]) yrow[brow[j]] = acc[i][j][q];
      }
    }
  }
}

template <int QBITS, typename XT, int BM>
static hipError_t launch_grouped_q(const FfnArgs& a, int64_t max_tiles, hipStream_t stream, int phases) {
  constexpr int W = MOE_GROUPED2_WAVES(BM), PD = MOE_GROUPED2_PD;
  if (phases & kPhaseGateUp) {
    const int rows = std::max(a.I, a.has_shared ? a.Is : 0);
    const int nn = (rows + 32 * W - 1) / (32 * W);
    const int64_t total = max_tiles * nn;
    const unsigned grid = unsigned((total + 7) / 8 * 8);
    if (a.H % 128 == 0) grouped_gemm2_kernel<QBITS, XT, true, W, PD, 1, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
    else if (a.H % 64 == 0) grouped_gemm2_kernel<QBITS, XT, true, W, PD, 2, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
    else grouped_gemm2_kernel<QBITS, XT, true, W, PD, 0, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
  }
  if (phases & kPhaseDown) {
    const int nn = (a.H + 64 * W - 1) / (64 * W);
    const int64_t total = max_tiles * nn;
    const unsigned grid = unsigned((total + 7) / 8 * 8);
    const bool k64 = a.I % 64 == 0 && (!a.has_shared || a.Is % 64 == 0);
    const bool k128 = a.I % 128 == 0 && (!a.has_shared || a.Is % 128 == 0);
    if (k128)
      grouped_gemm2_kernel<QBITS, f16, false, W, PD, 1, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
    else if (k64)
      grouped_gemm2_kernel<QBITS, f16, false, W, PD, 2, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
    else
      grouped_gemm2_kernel<QBITS, f16, false, W, PD, 0, BM><<<grid, 64 * W, 0, stream>>>(a, nn);
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

hipError_t launch_ffn_grouped(const FfnArgs& a, int64_t max_tiles, int bm, hipStream_t stream, int phases) {
  if (a.T == 0) return hipSuccess;
  if (bm != 96 && bm != 128) return hipErrorInvalidValue;
#define GQ(Q_, X_) \
  return bm == 96 ? launch_grouped_q<Q_, X_, 96>(a, max_tiles, stream, phases) \
                  : launch_grouped_q<Q_, X_, 128>(a, max_tiles, stream, phases)
  if (a.qbits == 2) {
    if (a.x_bf16) GQ(2, uint16_t);
    GQ(2, float);
  }
  if (a.qbits == 4) {
    if (a.x_bf16) GQ(4, uint16_t);
    GQ(4, float);
  }
  if (a.x_bf16) GQ(3, uint16_t);
  GQ(3, float);
#undef GQ
}

}  // namespace moe
