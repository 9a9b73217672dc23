// Internal launchers of the MoE kernels (host side).  The C ABI in abi.cpp
// validates arguments and then calls these; they only launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 4096;
constexpr int kMaxTopK = 32;
constexpr int kSmallPairs = 2048;   // single-workgroup permutation up to this many pairs
constexpr int kPermChunk = 1024;    // pairs per workgroup in the multi-workgroup permutation
constexpr int kGemvMaxM = 16;       // tokens per MFMA tile in the decode kernels
constexpr size_t kLdsBytes = 160 * 1024;  // LDS of a CU (the most one workgroup can have)

// Workspace header (int32 words at the start of the workspace).
enum HeaderWord { kHdrError = 0, kHdrActive = 1, kHdrTiles = 2, kHdrValid = 3, kHdrWords = 64 };

struct QMat {
  const uint8_t* codes;
  const uint16_t* scales;
  int64_t code_stride;   // bytes between experts
  int64_t scale_stride;  // fp16 elements between experts
};

// Everything the expert-FFN kernels read.  Slot s of the slot table is routed
// expert slots[s].x (or the shared expert when slots[s].x < 0).
// Activation element type of x.
enum XKind { kXF32 = 0, kXBF16 = 1, kXF16 = 2 };

struct FfnArgs {
  const void* x;
  int x_kind;  // XKind
  int64_t T;
  int H, I, Is, k, E, qbits, has_shared;
  QMat rg, ru, rd;  // routed gate / up / down
  QMat sg, su, sd;  // shared gate / up / down
  const int32_t* offsets;
  const int32_t* sorted_pair;
  const int32_t* header;       // workspace header (n_active, n_valid, n_tiles)
  const int4* slots;           // slot table, see launch_select_small
  const int4* tile_desc;       // grouped GEMM tiles: {expert (-1 = shared), first row of the
                               //   tile in the expert's rows, first sorted row, rows}
  _Float16* h_routed;          // [P][I] SwiGLU activations, sorted order, columns
                               //   permuted within groups of 16 (MFMA operand order)
  _Float16* h_shared;          // [T][Is]
  _Float16* x16;               // grouped GEMM: [T][H] fp16 copy of x in the permuted
                               //   16-group order (written by its gate/up launch)
  float* y_sorted;             // [P][H]
  _Float16* y_sorted_h;        // grouped GEMM: when non-null, the routed down output
                               //   goes here in fp16 instead of y_sorted
  float* shared_out;           // [T][H] or null
  _Float16* shared_out_h;      // grouped GEMM: when non-null, the shared down output goes
                               //   here in fp16 instead of shared_out
};

hipError_t launch_quantize(const float* w, int64_t rows, int cols, int qbits, uint8_t* codes,
                           uint16_t* scales, hipStream_t stream);
// Canonical row-major planes -> the tiled kernel layout of common.h.
hipError_t launch_repack(const uint8_t* codes, const uint16_t* scales, int64_t rows, int cols, int qbits,
                         uint8_t* tcodes, uint16_t* tscales, hipStream_t stream);
hipError_t launch_dequant(const uint8_t* codes, const uint16_t* scales, int64_t rows, int cols,
                          int qbits, float* out, hipStream_t stream);
hipError_t launch_router_gemv(const void* x, int x_kind, int64_t T, int H, const void* w, bool w_bf16,
                              const float* bias, int E, float* logits, hipStream_t stream);
hipError_t launch_router_mfma(const uint16_t* x, int64_t T, int H, const uint16_t* w, const float* bias,
                              int E, float* logits, hipStream_t stream);
hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w,
                       hipStream_t stream);
hipError_t launch_rmsnorm_bf16(const float* r, int64_t T, int H, uint16_t* a, hipStream_t stream);
hipError_t launch_permute(const int32_t* idx, int64_t P, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, int32_t* header, int32_t* chunk_hist,
                          hipStream_t stream);
// Builds the slot table (and, when tile_bm > 0, the grouped-GEMM tile list)
// from offsets, for the standalone expert FFN.  With sorted_pair given and
// T <= kGemvMaxM the slots carry their token masks (else mask 0); the
// persistent gate/up kernel relies on them.
hipError_t launch_plan(const int32_t* offsets, int E, int64_t T, int has_shared, int tile_bm,
                       int32_t* header, int4* slots, int4* tile_desc, const int32_t* sorted_pair, int k,
                       hipStream_t stream);
// Outputs of the plan (plan.h) for the fused prefill sequence below.
struct PlanOut {
  int has_shared, tile_bm;
  int32_t* header;
  int4* slots;
  int4* tile_desc;
};
// The prefill layer's top-k + softmax weights, stable permutation, plan and
// fp16 operand copy of x (x16) in three launches over chunks of 16 tokens
// (chunk_hist: select_chunks(T) x (E + 1) ints).  The same results as
// launch_topk, launch_permute, launch_plan and the grouped FFN's x16 copy.
// k <= 64 and H % 16 == 0 (else hipErrorInvalidValue, nothing launched).
int select_chunks(int64_t T);
hipError_t launch_select_plan(const float* logits, const void* x, int x_kind, int64_t T, int H, int E, int k,
                              int32_t* idx, float* w, int32_t* chunk_hist, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_pair, int32_t* pair_pos, _Float16* x16, const PlanOut& plan,
                              hipStream_t stream);
// Decode-layer selection on one workgroup (T <= 16): top-k + softmax weights,
// permutation and the slot table (int4 {expert or -1 for shared, first sorted
// position, token count, token mask: bit t set when token t uses the slot};
// empty slots have count 0).  Slot tables built by launch_plan carry the
// mask for T <= kGemvMaxM (0 otherwise: tokens then come from sorted_pair).
// kc: route tail skip (experts no token ranks below kc are dropped; 0 = off).
hipError_t launch_select_small(const float* logits, int T, int E, int k, int has_shared, int32_t* idx, float* w,
                               int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                               int32_t* header, int4* slots, int kc, hipStream_t stream);

// Routed + shared expert FFN on the decode kernels: h then y_sorted / shared_out.
enum { kPhaseGateUp = 1, kPhaseDown = 2 };
hipError_t launch_ffn_gemv(const FfnArgs& a, hipStream_t stream, int phases);
// The decode kernels stage up to 16 tokens of H (gate/up) or max(I, Is)
// (down) fp16 values per row in LDS: whether that fits for T tokens.
bool gemv_lds_ok(int64_t T, int H, int I, int Is);
// 2..16-token gate/up with the selection made in the kernel (select.h),
// when the shape allows it (else hipErrorNotSupported, nothing launched).
struct SelOut;
hipError_t launch_gateup_select(const FfnArgs& a, const SelOut& so, hipStream_t stream);
// Grouped-GEMM expert FFN over the tile list of launch_plan, built with
// tile_bm = grouped_tile_rows(T, k, E) (96 or 128) and launched with the same
// bm; max_tiles bounds the list for the launch grid.
int grouped_tile_rows(int64_t T, int k, int E);
// a.x -> a.x16 (the grouped gate/up GEMM's activations), part of the plan step.
hipError_t launch_x16(const FfnArgs& a, hipStream_t stream);
hipError_t launch_ffn_grouped(const FfnArgs& a, int64_t max_tiles, int bm, hipStream_t stream, int phases);
// The fused single-token decode FFN (needs E <= kDecode1MaxExperts): gate/up
// with the selection made from the router logits in every workgroup, then
// down + combine into out and/or res.  The selected experts occupy slots in
// ascending expert order; idx/w are the API's rank-ordered outputs.
constexpr int kDecode1MaxExperts = 512;
// LDS of the fused single-token kernels: the token (H fp16) in gate/up, the
// h rows of all k (+ shared) slots in down + combine; whether both fit.
bool decode1_lds_ok(int H, int I, int Is, int k, bool has_shared);
struct Decode1Sel {
  const float* logits;   // [E] router logits of the token
  int32_t* idx;          // [k] experts, rank order (written)
  float* w;              // [k] weights, rank order (written)
  int32_t* slot_of_rank; // [k] slot of rank r (written)
  int32_t* slot_expert;  // [k] expert of slot s (written)
  int32_t* header;       // workspace header: the error word is cleared
  int kc;                // route tail skip: only the token's ranks below kc are computed (its
                         //   top-kc experts are the slots); 0 or >= k: all k ranks
};
hipError_t launch_decode1_ffn(const FfnArgs& a, const Decode1Sel& sel, float* out, float* res, hipStream_t stream);
// res[t] -> a[t] = bf16_RNE(res[t] / sqrt(mean(res[t]^2) + 1e-6)) with the
// reduction order of the combine kernel (so both give the same bits).
hipError_t launch_residual_rmsnorm(const float* res, int64_t T, int H, uint16_t* next_in, hipStream_t stream);
hipError_t launch_combine(const float* y_sorted, const int32_t* pair_pos, const float* topk_w,
                          const float* shared_out, int64_t T, int H, int k, float* out, float* residual,
                          uint16_t* next_in, hipStream_t stream);
// The same combine over fp16 expert rows and fp16 shared rows (the grouped-GEMM
// layer's y_sorted_h and shared_out_h).
hipError_t launch_combine_f16y(const _Float16* y_sorted, const int32_t* pair_pos, const float* topk_w,
                               const _Float16* shared_out, int64_t T, int H, int k, float* out, float* residual,
                               uint16_t* next_in, hipStream_t stream);

}  // namespace moe
