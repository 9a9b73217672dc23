// Expert FFN for prefill-sized batches: a grouped GEMM over the device-built
// tile list, weights dequantised into LDS, fp16 MFMA (v_mfma_f32_32x32x16_f16)
// with fp32 accumulation.
//
// The experts are computed from their quantised storage ("How Strata runs a
// 125-billion-parameter model ...", intro and Step 1 byte table); with many
// tokens per expert the work is a dense contraction per expert, so it runs
// on the matrix cores.  Each tile of the list is (expert or shared, first row
// m0) with BM = 128 rows of the expert's sorted segment.
//
//   gate/up : [BM x H] activations x [H x 128] (64 gate + 64 up rows) -> SwiGLU
//             epilogue -> h (fp16, the permuted column order of the GEMV path)
//   down    : [BM x I] h x [I x 128] down rows -> y_sorted / shared_out (fp32)
//
// Workgroup = 4 waves, 2 x 2, each wave a 64 x 64 output block made of 2 x 2
// MFMA tiles of 32 x 32; K advances 64 weights (two quantisation blocks) per
// step through double-buffered LDS with one barrier per step.  In LDS both
// operands keep the permuted 16-group k order the dequantiser produces (pairs
// (i, i+8)), so codes unpack straight into their slots.  The tile index is
// remapped so that the n-tiles of one M tile run on the same XCD (dispatch
// goes round-robin over the 8 XCDs): its activation tile is then fetched into
// one L2 instead of eight.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kBM = 128, kBN = 128, kBK = 64, kLDA = kBK + 8;  // row pitch in halves (144 B)
#ifndef MOE_GROUPED2
#define MOE_GROUPED2 1
#endif
#ifndef MOE_GROUPED2_WAVES
#define MOE_GROUPED2_WAVES 8
#endif
#ifndef MOE_GROUPED2_PD
#define MOE_GROUPED2_PD 1
#endif

// Raw (not yet dequantised) B operand of one thread for one K step.
struct BRaw {
  uint32_t w0, w1, hb, sb;
};

template <int QBITS>
__device__ __forceinline__ BRaw load_braw(const uint8_t* codes, const uint16_t* scales, int rows, int K, int row,
                                          int blk, bool valid) {
  BRaw r{0, 0, 0, 0};
  if (valid) {
    const uint2v c = *reinterpret_cast<const uint2v*>(codes + int64_t(row) * (K / 4) + blk * 8);
    r.w0 = c[0];
    r.w1 = c[1];
    r.sb = scales[int64_t(row) * (K / 32) + blk];
    if constexpr (QBITS == 3)
      r.hb = *reinterpret_cast<const uint32_t*>(codes + int64_t(rows) * (K / 4) + int64_t(row) * (K / 8) + blk * 4);
  }
  return r;
}

template <int QBITS>
__device__ __forceinline__ void dq_braw(const BRaw& r, half8* out4) {
  const half2v s2 = as_half2(r.sb | (r.sb << 16));
  if constexpr (QBITS == 2) {
    dq2_word(r.w0, s2, out4[0], out4[1]);
    dq2_word(r.w1, s2, out4[2], out4[3]);
  } else {
    dq3_word(r.w0, spread16(r.hb & 0xffffu), s2, out4[0], out4[1]);
    dq3_word(r.w1, spread16(r.hb >> 16), s2, out4[2], out4[3]);
  }
}

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

template <int QBITS, typename AT, bool GATEUP>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(FfnArgs a, int n_ntiles) {
  __shared__ __attribute__((aligned(16))) f16 As[2][kBM * kLDA];
  __shared__ __attribute__((aligned(16))) f16 Bs[2][kBN * kLDA];

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
  const int rows_valid = min(kBM, m_count - m0);
  const int H = a.H;
  const int K = GATEUP ? H : (shared ? a.Is : a.I);
  const int Nrows = GATEUP ? (shared ? a.Is : a.I) : H;  // rows of each weight matrix
  const int64_t ex = shared ? 0 : e;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;

  // ---- A sources: thread handles items tid and tid + 256 of the 128 x 4 groups
  const AT* asrc[2];
  int arow[2], agrp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int item = tid + 256 * i;
    arow[i] = item >> 2;
    agrp[i] = item & 3;
    const int r = min(arow[i], rows_valid - 1);  // rows past the segment read a real row; never stored
    if constexpr (GATEUP) {
      const int64_t tok = shared ? int64_t(m0 + r) : int64_t(a.sorted_pair[lo + m0 + r] / a.k);
      asrc[i] = static_cast<const AT*>(a.x) + tok * H;
    } else {
      const f16* hb = shared ? a.h_shared + int64_t(m0 + r) * K : a.h_routed + int64_t(lo + m0 + r) * K;
      asrc[i] = reinterpret_cast<const AT*>(hb);
    }
  }
  // ---- B source: thread -> (row of the 128-row tile, block 0/1 of the K step)
  const int brow = tid >> 1, bblk = tid & 1;
  const uint8_t* bc;
  const uint16_t* bs;
  int wrow;  // row inside its weight matrix
  if constexpr (GATEUP) {
    const QMat M = brow < 64 ? (shared ? a.sg : a.rg) : (shared ? a.su : a.ru);
    bc = M.codes + ex * M.code_stride;
    bs = M.scales + ex * M.scale_stride;
    wrow = nt * 64 + (brow & 63);
  } else {
    const QMat M = shared ? a.sd : a.rd;
    bc = M.codes + ex * M.code_stride;
    bs = M.scales + ex * M.scale_stride;
    wrow = nt * kBN + brow;
  }
  const bool brow_ok = wrow < Nrows;
  const int nkb = (K + kBK - 1) / kBK;
  const int nblk = K / 32;

  auto load_a = [&](int kb, ARaw<AT>& r) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int col = kb * kBK + agrp[i] * 16;
      if (col >= K) col = 0;  // K tail: the matching weights are zero
      load_araw<AT>(asrc[i] + col, r, i);
    }
  };
  auto store_a = [&](const ARaw<AT>& r, f16* buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      half8 l8, h8;
      cvt_araw<AT>(r, i, l8, h8);
      half8* d = reinterpret_cast<half8*>(buf + arow[i] * kLDA + agrp[i] * 16);
      d[0] = l8;
      d[1] = h8;
    }
  };
  auto load_b = [&](int kb) {
    const int blk = kb * 2 + bblk;
    return load_braw<QBITS>(bc, bs, Nrows, K, wrow, blk, brow_ok && blk < nblk);
  };
  auto store_b = [&](const BRaw& r, f16* buf) {
    half8 o[4];
    dq_braw<QBITS>(r, o);
    half8* d = reinterpret_cast<half8*>(buf + brow * kLDA + bblk * 32);
    d[0] = o[0];
    d[1] = o[1];
    d[2] = o[2];
    d[3] = o[3];
  };

  float16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // B columns of this wave: gate/up -> 32 gate + the same 32 up rows; down -> 64 rows
  const int bcol0 = GATEUP ? 32 * wn : 64 * wn;
  const int bcol1 = GATEUP ? 64 + 32 * wn : 64 * wn + 32;
  const int l32 = lane & 31, lh = lane >> 5;

  ARaw<AT> ar;
  BRaw br;
  load_a(0, ar);
  br = load_b(0);
  store_a(ar, As[0]);
  store_b(br, Bs[0]);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) {
      load_a(kb + 1, ar);
      br = load_b(kb + 1);
    }
    const f16* Ab = As[cur];
    const f16* Bb = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int ko = kk * 16 + 8 * lh;
      half8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const half8*>(Ab + (64 * wm + 32 * i + l32) * kLDA + ko);
      bf[0] = *reinterpret_cast<const half8*>(Bb + (bcol0 + l32) * kLDA + ko);
      bf[1] = *reinterpret_cast<const half8*>(Bb + (bcol1 + l32) * kLDA + ko);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
    if (kb + 1 < nkb) {
      store_a(ar, As[cur ^ 1]);
      store_b(br, Bs[cur ^ 1]);
    }
    __syncthreads();
  }

  // ---- epilogue.  32 x 32 D layout: lane l holds column l % 32 and rows
  // 8*(q/4) + 4*(l/32) + q%4, q = 0..15.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int m = 64 * wm + 32 * i + 8 * (q >> 2) + 4 * lh + (q & 3);
      if (m >= rows_valid) continue;
      if constexpr (GATEUP) {
        const int gr = nt * 64 + 32 * wn + l32;
        if (gr < Nrows) {
          const float g = acc[i][0][q], u = acc[i][1][q];
          const float hv = g / (1.0f + expf(-g)) * u;
          const int hw = shared ? a.Is : a.I;
          f16* hout = shared ? a.h_shared + int64_t(m0 + m) * hw : a.h_routed + int64_t(lo + m0 + m) * hw;
          hout[hcol(gr)] = f16(hv);
        }
      } else {
        float* yrow = shared ? a.shared_out + int64_t(m0 + m) * H : a.y_sorted + int64_t(lo + m0 + m) * H;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = nt * kBN + 64 * wn + 32 * j + l32;
          if (col < H) yrow[col] = acc[i][j][q];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Second design: operand traffic per MFMA halved.  A workgroup owns BM = 128
// rows x 4 waves; each wave a 128 x 64 block (4 x 2 MFMA tiles of 32 x 32),
// so an A fragment read from LDS feeds two MFMAs and a B fragment four.  The
// weights never pass through LDS: each wave loads and dequantises its own
// 64 columns straight into MFMA operands (lane (n, h) of a 32-column set
// takes 16 code bytes = words 4h .. 4h+3 of the row's 128-weight step; MFMA
// k-step kk pairs slice kk of lane h = 0 with slice kk of lane h = 1, and
// the A fragments are read from LDS in the same order).  K advances 128 per
// step; the activation tile is double-buffered in LDS (fp16, permuted
// 16-groups), one barrier per step.
//   gate/up: wave w = gate rows nt*128 + 32w .. +32 and the same up rows;
//   down   : wave w = output columns nt*256 + 64w .. +64.
// ---------------------------------------------------------------------------
constexpr int kBM2 = 128, kBK2 = 128, kLDA2 = kBK2 + 8;  // A row pitch in halves

template <int QBITS>
struct BRaw2 {
  uint4v c;        // 16 code bytes: words 4h .. 4h+3
  uint32_t s;      // two fp16 scales: blocks 2h, 2h + 1
  uint32_t hb[2];  // 3-bit: high-plane bits of the 64 codes
};

// K64: K is a multiple of 64 (even block count per row), so a lane's two
// blocks are in or out together and its 16 code bytes, 4 scale bytes (and
// 8 high-plane bytes) are aligned for single loads.
template <int QBITS, bool K64>
__device__ __forceinline__ void load_b2(BRaw2<QBITS>& r, const uint8_t* codes, const uint16_t* scales, int rows,
                                        int K, int row, int step, int h, bool ok) {
  if constexpr (K64) {
    const int nb = K / 32;
    const int b0 = 4 * step + 2 * h;
    const bool in = ok && b0 < nb;
    const int rr = in ? row : 0, bb = in ? b0 : 0;
    const uint4v c = *reinterpret_cast<const uint4v*>(codes + int64_t(rr) * (K / 4) + bb * 8);
    const uint32_t sv = *reinterpret_cast<const uint32_t*>(scales + int64_t(rr) * nb + bb);
    r.c = in ? c : uint4v{0u, 0u, 0u, 0u};
    r.s = in ? sv : 0u;
    if constexpr (QBITS == 3) {
      const uint2v hv = *reinterpret_cast<const uint2v*>(codes + int64_t(rows) * (K / 4) + int64_t(rr) * (K / 8) +
                                                        bb * 4);
      r.hb[0] = in ? hv[0] : 0u;
      r.hb[1] = in ? hv[1] : 0u;
    }
    return;
  }
  // blocks of this lane: b0 = 4 * step + 2h and b0 + 1, each zero past K or
  // past the matrix.  Every load stays inside its row (8-byte code loads,
  // 2-byte scale loads: rows of K / 4 code bytes are only 8-byte aligned)
  // and is unconditional from a clamped address.
  const int nb = K / 32;
  const int b0 = 4 * step + 2 * h;
  const bool in0 = ok && b0 < nb, in1 = ok && b0 + 1 < nb;
  const int rr = in0 ? row : 0, bb0 = in0 ? b0 : 0, bb1 = in1 ? b0 + 1 : bb0;
  const uint8_t* cr = codes + int64_t(rr) * (K / 4);
  const uint16_t* sr = scales + int64_t(rr) * nb;
  const uint2v c0 = *reinterpret_cast<const uint2v*>(cr + bb0 * 8);
  const uint2v c1 = *reinterpret_cast<const uint2v*>(cr + bb1 * 8);
  const uint32_t s0 = sr[bb0], s1 = sr[bb1];
  r.c = uint4v{in0 ? c0[0] : 0u, in0 ? c0[1] : 0u, in1 ? c1[0] : 0u, in1 ? c1[1] : 0u};
  r.s = (in0 ? s0 : 0u) | ((in1 ? s1 : 0u) << 16);
  if constexpr (QBITS == 3) {
    const uint32_t* hp = reinterpret_cast<const uint32_t*>(codes + int64_t(rows) * (K / 4) + int64_t(rr) * (K / 8));
    const uint32_t h0 = hp[bb0], h1 = hp[bb1];
    r.hb[0] = in0 ? h0 : 0u;
    r.hb[1] = in1 ? h1 : 0u;
  }
}

// word q (0..3) of a lane's step -> the two permuted k-slices
template <int QBITS>
__device__ __forceinline__ void dq_b2(const BRaw2<QBITS>& r, int q, half8& lo, half8& hi) {
  const uint32_t sbits = q < 2 ? (r.s & 0xffffu) : (r.s >> 16);
  const half2v s2 = as_half2(sbits | (sbits << 16));
  if constexpr (QBITS == 2) {
    dq2_word(r.c[q], s2, lo, hi);
  } else {
    const uint32_t hbits = (r.hb[q >> 1] >> (16 * (q & 1))) & 0xffffu;
    dq3_word(r.c[q], spread16(hbits), s2, lo, hi);
  }
}

template <int QBITS, typename AT, bool GATEUP, int NWV, int PD, bool K64>
__global__ __launch_bounds__(64 * NWV, sizeof(AT) == 4 || NWV > 4 ? 1 : 2) void grouped_gemm2_kernel(FfnArgs a,
                                                                                                 int n_ntiles) {
  constexpr int NT = 64 * NWV;              // threads
  constexpr int AI = kBM2 * (kBK2 / 16) / NT;  // A staging items (16-element groups) per thread
  __shared__ __attribute__((aligned(16))) f16 As[2][kBM2 * kLDA2];

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
  const int rows_valid = min(kBM2, m_count - m0);
  const int H = a.H;
  const int K = GATEUP ? H : (shared ? a.Is : a.I);
  const int Nrows = GATEUP ? (shared ? a.Is : a.I) : H;  // rows of each weight matrix
  const int64_t ex = shared ? 0 : e;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  static_assert(AI >= 1 && AI * NT == kBM2 * (kBK2 / 16), "A staging covers the tile");

  // ---- A sources: thread handles items tid + NT i (i < AI) of the 128 x 8 groups
  const AT* asrc[AI];
  int arow[AI], agrp[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int item = tid + NT * i;
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
      half8 l8, h8;
      cvt_araw<AT>(r[i >> 1], i & 1, l8, h8);
      half8* d = reinterpret_cast<half8*>(buf + arow[i] * kLDA2 + agrp[i] * 16);
      d[0] = l8;
      d[1] = h8;
    }
  };

  float16v acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // B ring: the weights of steps step .. step + PD - 1 are in flight (a
  // ring of PD register sets; slot p holds steps p, p + PD, ...).  Loads for
  // steps past K are clamped in load_b2 (zero weights from a valid address).
  Raw ar[AR];
  BRaw2<QBITS> bring[PD][2];
  load_a(0, ar);
#pragma unroll
  for (int p = 0; p < PD; ++p)
#pragma unroll
    for (int j = 0; j < 2; ++j) load_b2<QBITS, K64>(bring[p][j], bc[j], bsc[j], Nrows, K, brow[j], p, h, bok[j]);
  store_a(ar, As[0]);
  __syncthreads();
  for (int s0 = 0; s0 < nsteps; s0 += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int step = s0 + p;
      if (step >= nsteps) break;
      const int cur = step & 1;
      const bool more = step + 1 < nsteps;
      BRaw2<QBITS> bcur[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) bcur[j] = bring[p][j];
      if (more) load_a(step + 1, ar);
      if (step + PD < nsteps) {
#pragma unroll
        for (int j = 0; j < 2; ++j) load_b2<QBITS, K64>(bring[p][j], bc[j], bsc[j], Nrows, K, brow[j], step + PD, h,
                                                        bok[j]);
      }
      const f16* Ab = As[cur];
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // word q of each lane's step: k-steps 2q (lo) and 2q + 1 (hi)
        half8 blo[2], bhi[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) dq_b2<QBITS>(bcur[j], q, blo[j], bhi[j]);
#pragma unroll
        for (int half_ = 0; half_ < 2; ++half_) {
          half8 af[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const half8*>(Ab + (32 * i + n) * kLDA2 + 64 * h + 16 * q + 8 * half_);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], half_ ? bhi[j] : blo[j], acc[i][j]);
        }
      }
      if (more) store_a(ar, As[cur ^ 1]);
      __syncthreads();
    }
  }

  // ---- epilogue.  32 x 32 D layout: lane l holds column l % 32 and rows
  // 8*(q/4) + 4*(l/32) + q%4, q = 0..15.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
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
      } else {
        float* yrow = shared ? a.shared_out + int64_t(m0 + m) * H : a.y_sorted + int64_t(lo + m0 + m) * H;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (bok[j]) yrow[brow[j]] = acc[i][j][q];
      }
    }
  }
}

template <int QBITS, typename XT>
static hipError_t launch_grouped_q(const FfnArgs& a, int64_t max_tiles, hipStream_t stream, int phases) {
  // The wide-tile kernel pays off when the segments fill its 128-row tiles:
  // T * k pairs of at least one tile per expert on average.  Below that
  // (thin segments, e.g. uniform routing of a few thousand tokens) the
  // LDS-dequantising kernel's 128 x 128 tiles spread the weights over more
  // workgroups.
  const bool wide = MOE_GROUPED2 && a.T * a.k >= int64_t(kBM2) * a.E;
  if (phases & kPhaseGateUp) {
    const int rows = std::max(a.I, a.has_shared ? a.Is : 0);
    if (wide) {
      constexpr int W = MOE_GROUPED2_WAVES;
      const int nn = (rows + 32 * W - 1) / (32 * W);
      const int64_t total = max_tiles * nn;
      const unsigned grid = unsigned((total + 7) / 8 * 8);
      if (a.H % 64 == 0) grouped_gemm2_kernel<QBITS, XT, true, W, MOE_GROUPED2_PD, true><<<grid, 64 * W, 0, stream>>>(a, nn);
      else grouped_gemm2_kernel<QBITS, XT, true, W, MOE_GROUPED2_PD, false><<<grid, 64 * W, 0, stream>>>(a, nn);
    } else {
      const int nn = (rows + 63) / 64;
      const int64_t total = max_tiles * nn;
      const unsigned grid = unsigned((total + 7) / 8 * 8);
      grouped_gemm_kernel<QBITS, XT, true><<<grid, 256, 0, stream>>>(a, nn);
    }
  }
  if (phases & kPhaseDown) {
    if (wide) {
      constexpr int W = MOE_GROUPED2_WAVES;
      const int nn = (a.H + 64 * W - 1) / (64 * W);
      const int64_t total = max_tiles * nn;
      const unsigned grid = unsigned((total + 7) / 8 * 8);
      if (a.I % 64 == 0 && (!a.has_shared || a.Is % 64 == 0))
        grouped_gemm2_kernel<QBITS, f16, false, W, MOE_GROUPED2_PD, true><<<grid, 64 * W, 0, stream>>>(a, nn);
      else
        grouped_gemm2_kernel<QBITS, f16, false, W, MOE_GROUPED2_PD, false><<<grid, 64 * W, 0, stream>>>(a, nn);
    } else {
      const int nn = (a.H + kBN - 1) / kBN;
      const int64_t total = max_tiles * nn;
      const unsigned grid = unsigned((total + 7) / 8 * 8);
      grouped_gemm_kernel<QBITS, f16, false><<<grid, 256, 0, stream>>>(a, nn);
    }
  }
  return hipGetLastError();
}

hipError_t launch_ffn_grouped(const FfnArgs& a, int64_t max_tiles, hipStream_t stream, int phases) {
  if (a.T == 0) return hipSuccess;
  if (a.qbits == 2)
    return a.x_bf16 ? launch_grouped_q<2, uint16_t>(a, max_tiles, stream, phases)
                    : launch_grouped_q<2, float>(a, max_tiles, stream, phases);
  return a.x_bf16 ? launch_grouped_q<3, uint16_t>(a, max_tiles, stream, phases)
                  : launch_grouped_q<3, float>(a, max_tiles, stream, phases);
}

}  // namespace moe
