// Router: logits, top-k selection with renormalised softmax weights, and the
// RMSNorm + bf16 glue between stacked layers.
//
// The router scores every expert of a layer for each token and the 10 best of
// 512 run ("How Strata runs a 125-billion-parameter model ...", intro and
// Step 2 "Mapped host doorbell and a single captured CUDA graph"); ranks 0..9
// are ordered by router weight (Step 2, "Verify-window route tail skip").
#include <float.h>
#include <limits.h>

#include "common.h"
#include "launch.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits on the vector ALUs: logits[t][e] = x[t] . W[e] + b[e].
// One wave per expert row, 4 rows per workgroup, up to TT tokens per
// workgroup (grid.y walks token chunks).  Lane l reads 8 consecutive weights
// at h = 8l + 512i (one 128-bit load of bf16, two of fp32), so a wave streams
// the row in 1 KB coalesced pieces.  For one token the activations come
// straight from global memory (the same 4 KB for every wave, L2-resident);
// for more tokens they are staged in LDS in K-chunks of KC.
// ---------------------------------------------------------------------------
template <typename T_>
__device__ __forceinline__ void load8(const T_* p, float* v) {
  if constexpr (std::is_same<T_, f16>::value) {  // fp16 -> fp32 is exact
    const half8 u = *reinterpret_cast<const half8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = float(u[i]);
  } else if constexpr (sizeof(T_) == 2) {  // bf16 bits
    const uint4v u = *reinterpret_cast<const uint4v*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
    const float4v a = reinterpret_cast<const float4v*>(p)[0];
    const float4v b = reinterpret_cast<const float4v*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

template <typename XT, typename WT, int TT>
__global__ __launch_bounds__(256) void router_gemv_kernel(const XT* __restrict__ x, int64_t T, int H,
                                                         const WT* __restrict__ w, const float* __restrict__ bias,
                                                         int E, float* __restrict__ logits) {
  constexpr int KC = TT == 1 ? 0 : (32768 / (TT * int(sizeof(XT))));  // K chunk staged in LDS (32 KB)
  __shared__ __attribute__((aligned(16))) XT xs[TT == 1 ? 1 : TT * KC];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int e = blockIdx.x * 4 + wv;
  const int64_t t0 = int64_t(blockIdx.y) * TT;
  const int tt = int(min<int64_t>(TT, T - t0));
  float acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = 0.0f;
  const WT* wrow = w + int64_t(e < E ? e : 0) * H;
  if constexpr (TT == 1) {
    if (e < E) {
      for (int h = lane * 8; h < H; h += 512) {
        float wv8[8], xv8[8];
        load8(wrow + h, wv8);
        load8(x + t0 * H + h, xv8);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[0] += wv8[i] * xv8[i];
      }
    }
  } else {
    for (int k0 = 0; k0 < H; k0 += KC) {
      const int kc = min(KC, H - k0);
      __syncthreads();
      // stage x[t0 .. t0+tt)[k0 .. k0+kc) (8 elements per thread-step)
      for (int i = threadIdx.x * 8; i < TT * kc; i += 256 * 8) {
        const int r = i / kc, c = i - r * kc;
        if (r < tt) {
          const XT* src = x + (t0 + r) * H + k0 + c;
          *reinterpret_cast<uint4v*>(&xs[r * KC + c]) = *reinterpret_cast<const uint4v*>(src);
          if constexpr (sizeof(XT) == 4)
            *reinterpret_cast<uint4v*>(&xs[r * KC + c + 4]) = *reinterpret_cast<const uint4v*>(src + 4);
        }
      }
      __syncthreads();
      if (e < E) {
        for (int c = lane * 8; c < kc; c += 512) {
          float wv8[8];
          load8(wrow + k0 + c, wv8);
#pragma unroll
          for (int r = 0; r < TT; ++r) {
            if (r < tt) {
              float xv8[8];
              load8(&xs[r * KC + c], xv8);
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[r] += wv8[i] * xv8[i];
            }
          }
        }
      }
    }
  }
  if (e >= E) return;
  const float b = bias ? bias[e] : 0.0f;
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    if (i < tt) {
      const float s = wave_sum(acc[i]);
      if (lane == 0) logits[(t0 + i) * E + e] = s + b;
    }
  }
}

// ---------------------------------------------------------------------------
// Router logits on MFMA for bf16 activations and bf16 router weights
// (v_mfma_f32_16x16x32_bf16: bf16 x bf16 products are exact in fp32).
//
// Accumulation order, the same in both MFMA router kernels so that a token's
// logits are the same bits at every batch size: the 32-wide K blocks fall in
// 8 classes of ceil(nkb / 8) consecutive blocks; each class is one MFMA chain
// from zero in increasing block order; the class sums are added 0, 1, ..., 7
// (S = a0, S = S + a1, ...), then the bias.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int router_class_len(int nkb) { return (nkb + 7) / 8; }

// Few tokens: workgroup = EPW experts x 16 tokens on one 16 x 16 MFMA tile,
// 8 waves; wave w runs class w and the 8 partial tiles meet in LDS.  With
// EPW < 16 (a handful of tokens: the MFMA work is negligible, the weight
// rows are spread over more CUs) MFMA columns EPW..15 repeat real rows (the
// same addresses, no extra traffic) and are zeroed; every logit goes through
// the same MFMA sequence whatever EPW is.
template <int EPW>
__global__ __launch_bounds__(512) void router_mfma_kernel(const uint16_t* __restrict__ x, int64_t T, int H,
                                                         const uint16_t* __restrict__ w,
                                                         const float* __restrict__ bias, int E,
                                                         float* __restrict__ logits) {
  __shared__ float red[8][4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * EPW;
  const int64_t t0 = int64_t(blockIdx.y) * 16;
  const int nkb = H / 32, cl = router_class_len(nkb);
  const int c0 = min(nkb, wv * cl), c1 = min(nkb, c0 + cl);
  const int er = e0 + (EPW == 16 ? n : n % EPW);
  const bool b_on = (EPW == 16 || n < EPW) && er < E;
  const bool a_on = t0 + n < T;
  const uint16_t* wrow = w + int64_t(er < E ? er : 0) * H + 8 * g;
  const uint16_t* xrow = x + (a_on ? t0 + n : 0) * H + 8 * g;
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int B = 8;  // K blocks per load batch
  for (int kb0 = c0; kb0 < c1; kb0 += B) {
    uint4v bw[B], ax[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {  // unconditional loads (clamped block, rows clamped above)
      const int kb = kb0 + i;
      const bool in = kb < c1;
      const int kbc = in ? kb : kb0;
      const uint4v wl = *reinterpret_cast<const uint4v*>(wrow + kbc * 32);
      const uint4v xl = *reinterpret_cast<const uint4v*>(xrow + kbc * 32);
      bw[i] = (in && b_on) ? wl : uint4v{0u, 0u, 0u, 0u};
      ax[i] = (in && a_on) ? xl : uint4v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < B; ++i)
      if (kb0 + i < c1)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ax[i]),
                                                      __builtin_bit_cast(bf16x8, bw[i]), acc, 0, 0, 0);
  }
  if (wv > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wv][j][lane] = acc[j];
  }
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int q = 1; q < 8; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += red[q][j][lane];
  if (!b_on) return;
  const float b = bias ? bias[er] : 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = t0 + 4 * g + j;
    if (t < T) logits[t * E + er] = acc[j] + b;
  }
}

// Many tokens: a 128-token x ET-expert tile per workgroup (ET = 128, or 64
// when the 128-wide tiles would leave CUs without a workgroup), ET / 16
// waves of 32 tokens x 64 experts (2 x 4 MFMA blocks of 16 x 16).  The classes run
// one after another, so a wave keeps two accumulators per output (the class
// chain and the running sum S) instead of eight.  K advances RK blocks per
// step (within a class); the workgroup stages each step's activation and
// weight rows in LDS with row-contiguous 16-byte loads (a wave instruction
// covers two 256-byte row pieces) and the next step's loads are in flight
// during the MFMAs.  The logits tile goes out through LDS as whole 512-byte
// row pieces.  Tiles are handed out so that the expert tiles of one token
// tile run one after another on one XCD (its activations are read into one
// L2).
// ---------------------------------------------------------------------------
constexpr int kRtT = 128;  // tokens per tile
// LDS row pitch of the logits tile in floats
template <int ET>
constexpr int rt_out_pitch() { return ET + 4; }
constexpr int64_t kRouterGemmMinT = 2048;  // tokens from which the 128 x 128 tiles run
// experts per workgroup of the router at <= 16 tokens (one workgroup per CU
// at 512 experts); router_mfma_kernel's 16 x 16 tiles are below
constexpr int kRouterSmallEpw = 2;
// LDS row pitch of the staged operands in bf16: an odd number of 16-byte
// units, so the 16 rows of a fragment read hit distinct banks
template <int RK>
constexpr int rt_pitch() { return RK * 32 + 8; }
template <int RK, int ET>
constexpr size_t rt_lds() {
  return std::max(size_t(kRtT + ET) * rt_pitch<RK>() * 2, size_t(kRtT) * rt_out_pitch<ET>() * 4);
}

// RK = K blocks (of 32) per step; OCC = waves per SIMD the registers are
// budgeted for (RK = 2 fits 128 registers, 4 waves: two workgroups per CU;
// RK = 4 halves the steps and barriers but needs the 256 of 2 waves); PD =
// steps whose loads are in flight during a step's MFMAs (register sets of
// the staging ring: 2 fit beside RK = 4 in 256 registers, 1 beside RK = 2 in
// 128, where the second workgroup of the CU covers the latency).
// WHOLE: every class is PD whole steps of RK blocks (router_whole_classes;
// the 2048-wide hidden of the stack), so a step's blocks are unrolled and the
// fold runs once per ring turn.
template <int RK, int PD>
__host__ __device__ inline bool router_whole_classes(int H) {
  const int nkb = H / 32, cl = router_class_len(nkb);
  return cl % RK == 0 && nkb % cl == 0 && cl / RK == PD;
}

template <int RK, int OCC, int PD, int ET, bool WHOLE = false>
__global__ __launch_bounds__(4 * ET, OCC) void router_gemm_kernel(const uint16_t* __restrict__ x, int64_t T, int H,
                                                            const uint16_t* __restrict__ w,
                                                            const float* __restrict__ bias, int E,
                                                            float* __restrict__ logits, int n_et, int64_t total) {
  constexpr int kPitch = rt_pitch<RK>();
  constexpr int NT = 4 * ET;                // threads: ET / 16 waves
  constexpr int kOutPitch = rt_out_pitch<ET>();
  extern __shared__ __attribute__((aligned(16))) uint16_t rs[];  // [kRtT + ET][kPitch] bf16, then the out tile
  const int64_t per = (total + 7) / 8;
  const int64_t L = int64_t(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (L >= total) return;
  const int64_t tt = L / n_et;
  const int et = int(L - tt * n_et);
  const int64_t t0 = tt * kRtT;
  const int e0 = et * ET;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int wt = wv / (ET / 64), we = wv % (ET / 64);  // wave tile: tokens 32 wt .., experts 64 we ..
  const int nkb = H / 32, cl = router_class_len(nkb);

  // staging: 16-byte piece p = tid + NT q (q < NQ) of the step's
  // (kRtT + ET) rows x RK blocks: row p / (4 RK), piece p % (4 RK)
  // of the row's 64 RK bytes (block piece / 4 of the step, quarter piece % 4)
  constexpr int NQ = (kRtT + ET) * RK * 4 / NT, QX = kRtT * RK * 4 / NT;
  static_assert(NQ * NT == (kRtT + ET) * RK * 4 && QX * NT == kRtT * RK * 4,
                "staging covers the step; the first QX pieces of a thread are activation rows");
  // element offsets from the tile's first activation / weight row (rows
  // past the end read the last real row; their results are never stored)
  const uint16_t* xt = x + t0 * H;
  const uint16_t* wt_ = w + int64_t(e0) * H;
  const int t_last = int(min(T - t0, int64_t(kRtT))) - 1, e_last = min(E - e0, ET) - 1;
  int off[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int p = tid + NT * q, row = p / (4 * RK), pc = p % (4 * RK);
    off[q] = (row < kRtT ? min(row, t_last) : min(row - kRtT, e_last)) * H + pc * 8;
  }
  // Steps: class c has sp = ceil(cl / RK) steps, step i of the tile is step
  // i % sp of class i / sp and covers blocks b .. b + RK - 1 of it.  A ring
  // of PD register sets keeps the loads of steps i + 1 .. i + PD in flight
  // during step i's MFMAs.
  const int sp = (cl + RK - 1) / RK;
  const int n_cls = (nkb + cl - 1) / cl;  // non-empty classes (an empty class adds +0: S is never -0)
  const int n_steps = n_cls * sp;
  auto step_b = [&](int i) { return (i / sp) * cl + (i % sp) * RK; };
  auto step_end = [&](int i) { return min(nkb, (i / sp) * cl + cl); };
  uint4v stg[PD][NQ];
  // pieces of blocks at or past the class end (or of a step past the last)
  // read block 0 of their row instead and are never read back (the MFMA loop
  // stops at the class end).  The raw loaded values go straight to the LDS
  // stores: a select on them would make the loads wait here instead of under
  // the MFMAs.
  auto load_step = [&](uint4v (&st)[NQ], int i) {
    const bool real = i < n_steps;
    const int b = real ? step_b(i) : 0, cend = real ? step_end(i) : 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int kb = b + (tid + NT * q) % (4 * RK) / 4;
      const uint16_t* base = q < QX ? xt : wt_;  // pieces q < QX are activation rows
      st[q] = *reinterpret_cast<const uint4v*>(base + off[q] + (kb < cend ? b : 0) * 32);  // clamped, unconditional
    }
  };
  auto store_step = [&](const uint4v (&st)[NQ]) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int p = tid + NT * q, row = p / (4 * RK), pc = p % (4 * RK);
      *reinterpret_cast<uint4v*>(rs + row * kPitch + pc * 8) = st[q];
    }
  };

  float4v S[2][4], acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) S[i][j] = acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};
  // block k of the staged step: 2 x 4 MFMA tiles of the class chain
  auto mfma_block = [&](int k) {
    uint4v af[2], bf[4];
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
      af[i2] = *reinterpret_cast<const uint4v*>(rs + (32 * wt + 16 * i2 + n) * kPitch + k * 32 + 8 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[j] = *reinterpret_cast<const uint4v*>(rs + (kRtT + 64 * we + 16 * j + n) * kPitch + k * 32 + 8 * g);
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i2][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[i2]),
                                                             __builtin_bit_cast(bf16x8, bf[j]), acc[i2][j], 0, 0, 0);
  };
  auto fold = [&](int c) {  // the class is done: S += its chain
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        S[i2][j] = c == 0 ? acc[i2][j] : S[i2][j] + acc[i2][j];
        acc[i2][j] = float4v{0.f, 0.f, 0.f, 0.f};
      }
  };
  auto run_step = [&](uint4v (&st)[NQ], int i) {
    __syncthreads();  // the previous step's fragments are read
    store_step(st);
    __syncthreads();
    load_step(st, i + PD);  // the ring slot is free again: step i + PD's loads
    const int b = step_b(i), nsub = min(RK, step_end(i) - b);
    for (int k = 0; k < nsub; ++k) mfma_block(k);
    if (i % sp == sp - 1) {  // the class is done: S += its chain
      const int c = i / sp;
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          S[i2][j] = c == 0 ? acc[i2][j] : S[i2][j] + acc[i2][j];
          acc[i2][j] = float4v{0.f, 0.f, 0.f, 0.f};
        }
    }
  };
#pragma unroll
  for (int p = 0; p < PD; ++p) load_step(stg[p], p);
  if constexpr (WHOLE) {
    // whole classes of PD whole steps (the 2048-wide hidden of the stack): the
    // blocks of a step are unrolled and the class folds once per ring turn
    for (int c = 0; c < n_cls; ++c) {
#pragma unroll
      for (int p = 0; p < PD; ++p) {
        __syncthreads();  // the previous step's fragments are read
        store_step(stg[p]);
        __syncthreads();
        load_step(stg[p], c * PD + p + PD);  // the ring slot is free again
        // the blocks one after another, block k + 1's fragments read during block k's MFMAs (two
        // fragment sets: all RK blocks' would not fit beside the staging ring)
        uint4v fa[2][2], fb[2][4];
        auto frags = [&](int k, uint4v(&xa)[2], uint4v(&xb)[4]) {
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2)
            xa[i2] = *reinterpret_cast<const uint4v*>(rs + (32 * wt + 16 * i2 + n) * kPitch + k * 32 + 8 * g);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xb[j] = *reinterpret_cast<const uint4v*>(rs + (kRtT + 64 * we + 16 * j + n) * kPitch + k * 32 + 8 * g);
        };
        frags(0, fa[0], fb[0]);
#pragma unroll
        for (int k = 0; k < RK; ++k) {
          if (k + 1 < RK) frags(k + 1, fa[(k + 1) & 1], fb[(k + 1) & 1]);
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i2][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[k & 1][i2]),
                                                                   __builtin_bit_cast(bf16x8, fb[k & 1][j]),
                                                                   acc[i2][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      fold(c);
    }
  } else {
    // whole ring turns: a step past the last one stages block 0 and runs no
    // MFMA (its class fold adds +0), and every turn issues and waits for the
    // ring slots in the same order, so the compiler's wait counts stay exact
    for (int i = 0; i < n_steps; i += PD) {
#pragma unroll
      for (int p = 0; p < PD; ++p) run_step(stg[p], i + p);
    }
  }
  // logits tile through LDS: S block (i, j) element r = token 32 wt + 16 i + 4 g + r, expert 64 we + 16 j + n
  __syncthreads();
  float* os = reinterpret_cast<float*>(rs);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) os[(32 * wt + 16 * i + 4 * g + r) * kOutPitch + 64 * we + 16 * j + n] = S[i][j][r];
  __syncthreads();
  // 16-byte stores and bias loads when every logits row and the bias are 16-byte aligned
  const bool vec = E % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(bias) & 15) == 0;
#pragma unroll
  for (int q = 0; q < kRtT * ET / 4 / NT; ++q) {
    const int p = tid + NT * q, row = p / (ET / 4), c4 = (p % (ET / 4)) * 4;
    const int64_t t = t0 + row;
    const int e = e0 + c4;
    if (t >= T || e >= E) continue;
    float4v v = *reinterpret_cast<const float4v*>(os + row * kOutPitch + c4);
    if (vec && e + 3 < E) {
      const float4v bv = bias ? *reinterpret_cast<const float4v*>(bias + e) : float4v{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<float4v*>(logits + t * E + e) = v + bv;
    } else {
      for (int u = 0; u < 4 && e + u < E; ++u) logits[t * E + e + u] = v[u] + (bias ? bias[e + u] : 0.0f);
    }
  }
}

hipError_t launch_router_mfma(const uint16_t* x, int64_t T, int H, const uint16_t* w, const float* bias, int E,
                              float* logits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (T >= kRouterGemmMinT) {
    const int64_t n_tt = (T + kRtT - 1) / kRtT;
    const int n_et = (E + 127) / 128;
    const int64_t total = n_tt * n_et;
    const bool whole = router_whole_classes<4, 2>(H);
    if (total >= 512) {  // two resident workgroups per CU have work: the 128-register variant
      router_gemm_kernel<2, 4, 1, 128><<<unsigned((total + 7) / 8 * 8), 512, rt_lds<2, 128>(), stream>>>(
          x, T, H, w, bias, E, logits, n_et, total);
    } else if (total >= 256) {
      if (whole)
        router_gemm_kernel<4, 2, 2, 128, true><<<unsigned((total + 7) / 8 * 8), 512, rt_lds<4, 128>(), stream>>>(
            x, T, H, w, bias, E, logits, n_et, total);
      else
        router_gemm_kernel<4, 2, 2, 128><<<unsigned((total + 7) / 8 * 8), 512, rt_lds<4, 128>(), stream>>>(
            x, T, H, w, bias, E, logits, n_et, total);
    } else {  // fewer 128-wide tiles than CUs: 64-expert tiles, twice as many
      const int n_et64 = (E + 63) / 64;
      const int64_t total64 = n_tt * n_et64;
      if (whole)
        router_gemm_kernel<4, 2, 2, 64, true><<<unsigned((total64 + 7) / 8 * 8), 256, rt_lds<4, 64>(), stream>>>(
            x, T, H, w, bias, E, logits, n_et64, total64);
      else
        router_gemm_kernel<4, 2, 2, 64><<<unsigned((total64 + 7) / 8 * 8), 256, rt_lds<4, 64>(), stream>>>(
            x, T, H, w, bias, E, logits, n_et64, total64);
    }
    return hipGetLastError();
  }
  if (T <= 16) {
    constexpr int EPW = kRouterSmallEpw;
    router_mfma_kernel<EPW><<<dim3(unsigned((E + EPW - 1) / EPW)), 512, 0, stream>>>(x, T, H, w, bias, E, logits);
  } else {
    const dim3 grid(unsigned((E + 15) / 16), unsigned((T + 15) / 16));
    router_mfma_kernel<16><<<grid, 512, 0, stream>>>(x, T, H, w, bias, E, logits);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k with ties to the lower expert index, then softmax over the selected
// logits.  One wave per token, through the wave selection routines of
// common.h (the k-th largest key by bisection on ballot counts, then the
// ranking), so every path of the library selects the same experts with the
// same weight bits.
// ---------------------------------------------------------------------------
template <int V>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                  int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_idx;
  float my_w;
  wave_topk_softmax<V>(logits + t * E, E, k, my_idx, my_w);
  if (lane < k) {
    idx_out[t * k + lane] = my_idx;
    w_out[t * k + lane] = my_w;
  }
}

// ---------------------------------------------------------------------------
// a[t] = bf16_RNE(r[t] / sqrt(mean(r[t]^2) + 1e-6)); one workgroup per row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void rmsnorm_bf16_kernel(const float* __restrict__ r, int H,
                                                          uint16_t* __restrict__ a) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const float* row = r + t * H;
  float ss = 0.0f;
  for (int c = threadIdx.x; c < H; c += 256) ss += row[c] * row[c];
  ss = block_sum_256(ss, red);
  const float denom = sqrtf(ss / float(H) + 1e-6f);
  for (int c = threadIdx.x; c < H; c += 256) a[t * H + c] = f32_to_bf16_rne(row[c] / denom);
}

// ---------------------------------------------------------------------------
template <typename XT, typename WT>
static void router_launch(const void* x, int64_t T, int H, const void* w, const float* bias, int E, float* logits,
                          hipStream_t stream) {
  if (T == 1) {
    router_gemv_kernel<XT, WT, 1><<<dim3(unsigned((E + 3) / 4), 1), 256, 0, stream>>>(
        (const XT*)x, T, H, (const WT*)w, bias, E, logits);
  } else {
    router_gemv_kernel<XT, WT, 16><<<dim3(unsigned((E + 3) / 4), unsigned((T + 15) / 16)), 256, 0, stream>>>(
        (const XT*)x, T, H, (const WT*)w, bias, E, logits);
  }
}

hipError_t launch_router_gemv(const void* x, int x_kind, int64_t T, int H, const void* w, bool w_bf16,
                              const float* bias, int E, float* logits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (x_kind == kXBF16 && w_bf16) router_launch<uint16_t, uint16_t>(x, T, H, w, bias, E, logits, stream);
  else if (x_kind == kXBF16) router_launch<uint16_t, float>(x, T, H, w, bias, E, logits, stream);
  else if (x_kind == kXF16 && w_bf16) router_launch<f16, uint16_t>(x, T, H, w, bias, E, logits, stream);
  else if (x_kind == kXF16) router_launch<f16, float>(x, T, H, w, bias, E, logits, stream);
  else if (w_bf16) router_launch<float, uint16_t>(x, T, H, w, bias, E, logits, stream);
  else router_launch<float, float>(x, T, H, w, bias, E, logits, stream);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w,
                       hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid(unsigned((T + 3) / 4));
  const int v = (E + 63) / 64;
  if (v <= 1) topk_kernel<1><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else if (v <= 2) topk_kernel<2><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else if (v <= 4) topk_kernel<4><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else if (v <= 8) topk_kernel<8><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else if (v <= 16) topk_kernel<16><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else if (v <= 32) topk_kernel<32><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  else topk_kernel<64><<<grid, 256, 0, stream>>>(logits, T, E, k, idx, w);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bf16(const float* r, int64_t T, int H, uint16_t* a, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  rmsnorm_bf16_kernel<<<dim3(unsigned(T)), 256, 0, stream>>>(r, H, a);
  return hipGetLastError();
}

}  // namespace moe
