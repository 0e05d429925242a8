// Host-side descriptor of one LoRA GEMM launch (see gemm.hip).
#pragma once
#include "common.h"
namespace lsl {
struct GemmDesc {
  const uint16_t* x = nullptr; int64_t ldx = 0;    // [M x K]
  int wfmt = LSL_WFMT_BF16; bool kn = false;        // weight format; stored [K x N] when kn
  const uint16_t* wb = nullptr; const uint8_t* wq = nullptr; const float* wa = nullptr;
  const uint8_t* wq8 = nullptr; const float* wsc = nullptr;  // NF4DQ absmax codes and block constants
  int64_t M = 0, N = 0, K = 0;
  int lora = 0;                                     // 0 none, 1 forward (masked B), 2 backward (A^T)
  const uint16_t* la = nullptr; int64_t ldla = 0; int kl = 0;
  const uint16_t* lb = nullptr; int r = 0; int nseg = 1; int64_t seg_end[4] = {0, 0, 0, 0};
  float scale = 0.f;
  uint16_t* y = nullptr; int64_t ldy = 0;
  const uint16_t* res = nullptr; int64_t ldres = 0;
  const uint16_t* bias = nullptr;                   // bf16 [N], added before the rounding (bf16 epilogue)
  // epilogue selection: 0 bf16 store (+ residual); 1 cross-entropy max/sum-exp
  // partials; 2 cross-entropy gradient chunk (hi into y, lo into y2);
  // 3 float accumulate into out32 (bf16 copy into y when y != NULL)
  int epi = 0;
  const int32_t* labels = nullptr; const float* lse = nullptr; const float* nvalid = nullptr;
  void* part = nullptr; float* zlab = nullptr; uint16_t* y2 = nullptr;
  float gscale = 1.f; int ignore = -100; int64_t vocab_off = 0, vocab = 0;
  float* out32 = nullptr; int64_t ldo32 = 0; int first = 1;
  // epilogue 3 only: the reduction is split acc_splits ways, split s accumulating
  // into out32 + s * o32_split (y must be NULL; the caller adds the splits)
  int acc_splits = 1; int64_t o32_split = 0;
  int64_t kwrap = 0;
  // split-K / stream-K scratch for the bf16 epilogue: gemm_split_bytes(M, N, K)
  // bytes; stream-K also takes gemm_counts_needed(M, N, K) arrival counts,
  // zero before the first launch and left zero by every launch
  float* split_ws = nullptr;
  unsigned* cnt = nullptr;
  // bf16 epilogue with its reduction split into float32 partials (gemm_splits > 1):
  // leave the partials in split_ws ([S][M][N]) and launch no reduce; the caller
  // sums them (the RMSNorm kernels that take split partials)
  bool defer_reduce = false;
};
lsl_status gemm_launch(const GemmDesc& d, hipStream_t s);
// The conditions gemm_launch rejects, checked without launching anything.
lsl_status gemm_check(const GemmDesc& d);
// Reduction splits gemm_launch uses for a bf16-epilogue GEMM of this shape, and
// the float32 scratch they need (0 when the GEMM is not split).
int gemm_splits(int64_t M, int64_t N, int64_t K);
size_t gemm_split_bytes(int64_t M, int64_t N, int64_t K);
size_t gemm_counts_needed(int64_t M, int64_t N, int64_t K);
// Tile shape gemm_launch picks for an M x N output (bn weight rows, bm tokens).
void gemm_tile_shape(int64_t M, int64_t N, int& bn, int& bm);
// cross-entropy GEMMs: whether the logits passes of an M x N x K problem run in
// the 256 x 256 tiles, the vocabulary tile width of the forward pass (its
// per-tile (max, sum) partials are [N / width][M]), and the number of
// reduction splits the float32 dH accumulation uses
bool gemm_ce_big(int64_t M, int64_t N, int64_t K);
int gemm_ce_tile_n(int64_t M, int64_t N, int64_t K);
int gemm_acc32_splits(int64_t M, int64_t N, int64_t K);
}  // namespace lsl
