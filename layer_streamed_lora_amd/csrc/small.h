// Host descriptors for the LoRA side products and the elementwise kernels.
#pragma once
#include "common.h"
namespace lsl {
struct SegEnds { int64_t e[4]; };

// C[t][j] = sum_k p[t][k] R[j][k] -> out bf16 [T x kl]; R = a_full [kl x K], or
// (b_full != NULL) the projection-masked B_full [K x r].
// ws: lora_nt_ws_bytes(T, K, kl) bytes; cnt: lora_counts_needed(T, .) arrival
// counts, zero before the call's first launch (each launch leaves them zero).
struct LoraNt {
  const uint16_t* p = nullptr; int64_t ldp = 0; int64_t T = 0, K = 0; int kl = 0;
  const uint16_t* a_full = nullptr;
  const uint16_t* b_full = nullptr; int r = 0; int nseg = 1; int64_t seg_end[4] = {0, 0, 0, 0};
  uint16_t* out = nullptr; int64_t ldo = 0;
  float* ws = nullptr;
  unsigned* cnt = nullptr;
};
// C[a][j] = sum_t p[t][a] q[t][j]; dA [kl x W] += s C^T, or dB [W x r] += s C (projection-selected)
struct LoraTn {
  const uint16_t* p = nullptr; int64_t ldp = 0; const uint16_t* q = nullptr; int64_t ldq = 0;
  int64_t T = 0, W = 0; int kl = 0;
  float scale = 0.f; float* dA = nullptr; float* dB = nullptr;
  int r = 0; int nseg = 1; int64_t seg_end[4] = {0, 0, 0, 0};
  float* ws = nullptr;
  unsigned* cnt = nullptr;
};
// the projection-masked transpose bt [kl x K] of B_full [K x r] (bt[j][k] =
// B[k][j % r] when row k belongs to projection j / r, else 0): the NT operand
// R of u = dy B
struct LoraBt {
  const uint16_t* b_full = nullptr; int r = 0; int kl = 0; int64_t K = 0;
  int nseg = 1; int64_t seg_end[4] = {0, 0, 0, 0};
  uint16_t* bt = nullptr;
};
// up to four of them in one launch
lsl_status lora_bt_group_launch(const LoraBt* jobs, int n, hipStream_t s);
size_t lora_nt_ws_bytes(int64_t T, int64_t K, int kl);
size_t lora_tn_ws_bytes(int64_t T, int64_t W, int kl);
// arrival counts a side product of T tokens and output width W (K for NT) may use
size_t lora_counts_needed(int64_t T, int64_t W);
// zero n counts (a fill kernel on the stream)
lsl_status lora_counts_zero(unsigned* cnt, size_t n, hipStream_t s);
lsl_status lora_nt_launch(const LoraNt& d, hipStream_t s);
lsl_status lora_tn_launch(const LoraTn& d, hipStream_t s);
// up to eight TN products in one launch; each needs its own ws (lora_tn_ws_bytes)
// and its own lora_tn_tiles(W) arrival counts
lsl_status lora_tn_group_launch(const LoraTn* d, int n, hipStream_t s);
size_t lora_tn_tiles(int64_t W);
// the conditions the launches reject, checked without launching anything
lsl_status lora_nt_check(const LoraNt& d);
lsl_status lora_tn_check(const LoraTn& d);

// zero (may be NULL): nzero 32-bit words the launch also sets to 0 (the layer's
// arrival counts, so that they need no launch of their own)
lsl_status rmsnorm_fwd_launch(const uint16_t* x, const uint16_t* w, int64_t T, int64_t H, float eps, uint16_t* y,
                              hipStream_t s, unsigned* zero = nullptr, int nzero = 0);
lsl_status rmsnorm_bwd_launch(const uint16_t* x, const uint16_t* w, const uint16_t* dy, const uint16_t* dres,
                              int64_t T, int64_t H, float eps, uint16_t* dx, hipStream_t s);
// The same two RMSNorm steps reading their input as the float32 split-K partials
// [S][T x H] of the GEMM before them (GemmDesc::defer_reduce): the input is summed
// (+ bias, + res) exactly as gemm_split_reduce would store it, written to h /
// dy_out, and normalised (forward) or back-propagated (backward) from those
// bf16 values, so every output has the bits of the unfused pair of launches.
lsl_status rmsnorm_fwd_split_launch(const float* part, int S, const uint16_t* bias, const uint16_t* res, int64_t ldres,
                                    uint16_t* h, const uint16_t* w, int64_t T, int64_t H, float eps, uint16_t* y,
                                    hipStream_t s);
lsl_status rmsnorm_bwd_split_launch(const uint16_t* x, const uint16_t* w, const float* part, int S,
                                    const uint16_t* dres, int64_t T, int64_t H, float eps, uint16_t* dy_out,
                                    uint16_t* dx, hipStream_t s);
// y = RoPE(x) for n_heads heads of head_dim from column 0 of each row (row
// stride ld for both; y may be x)
lsl_status rope_launch(const uint16_t* x, uint16_t* y, int64_t T, int64_t ld, int n_heads, int head_dim, int seq,
                       float theta, const lsl_rope_scaling* scaling, int inverse, hipStream_t s);
// RoPE of the q|k|v projection read as its float32 split-K partials [S][T x ld]
// (GemmDesc::defer_reduce): every column summed (+ bias) and rounded into qkv as
// gemm_split_reduce would, the first n_heads heads rotated from those values
// into y as rope_launch (forward) would.
lsl_status rope_split_launch(const float* part, int S, const uint16_t* bias, uint16_t* qkv, uint16_t* y, int64_t T,
                             int64_t ld, int n_heads, int head_dim, int seq, float theta,
                             const lsl_rope_scaling* scaling, hipStream_t s);
lsl_status swiglu_fwd_launch(const uint16_t* gu, int64_t T, int64_t I, uint16_t* a, hipStream_t s);
lsl_status swiglu_bwd_launch(const uint16_t* gu, const uint16_t* da, int64_t T, int64_t I, uint16_t* dgu, hipStream_t s);
}  // namespace lsl
