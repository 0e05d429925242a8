// Host descriptors for the LoRA side products and the elementwise kernels.
#pragma once
#include "common.h"
namespace lsl {
struct SegEnds { int64_t e[4]; };

// C[t][j] = sum_k p[t][k] R[j][k] -> out bf16 [T x kl]; R = a_full [kl x K], or
// (b_full != NULL) the projection-masked B_full [K x r].
struct LoraNt {
  const uint16_t* p = nullptr; int64_t ldp = 0; int64_t T = 0, K = 0; int kl = 0;
  const uint16_t* a_full = nullptr;
  const uint16_t* b_full = nullptr; int r = 0; int nseg = 1; int64_t seg_end[4] = {0, 0, 0, 0};
  uint16_t* out = nullptr; int64_t ldo = 0;
  float* ws = nullptr;
};
// C[a][j] = sum_t p[t][a] q[t][j]; dA [kl x W] += s C^T, or dB [W x r] += s C (projection-selected)
struct LoraTn {
  const uint16_t* p = nullptr; int64_t ldp = 0; const uint16_t* q = nullptr; int64_t ldq = 0;
  int64_t T = 0, W = 0; int kl = 0;
  float scale = 0.f; float* dA = nullptr; float* dB = nullptr;
  int r = 0; int nseg = 1; int64_t seg_end[4] = {0, 0, 0, 0};
  float* ws = nullptr;
};
size_t lora_nt_ws_bytes(int64_t T, int64_t K);
size_t lora_tn_ws_bytes(int64_t T, int64_t W);
lsl_status lora_nt_launch(const LoraNt& d, hipStream_t s);
lsl_status lora_tn_launch(const LoraTn& d, hipStream_t s);

lsl_status rmsnorm_fwd_launch(const uint16_t* x, const uint16_t* w, int64_t T, int64_t H, float eps, uint16_t* y, hipStream_t s);
lsl_status rmsnorm_bwd_launch(const uint16_t* x, const uint16_t* w, const uint16_t* dy, const uint16_t* dres,
                              int64_t T, int64_t H, float eps, uint16_t* dx, hipStream_t s);
lsl_status rope_launch(uint16_t* x, int64_t T, int64_t ld, int n_heads, int head_dim, int seq, float theta,
                       const lsl_rope_scaling* scaling, int inverse, hipStream_t s);
lsl_status swiglu_fwd_launch(const uint16_t* gu, int64_t T, int64_t I, uint16_t* a, hipStream_t s);
lsl_status swiglu_bwd_launch(const uint16_t* gu, const uint16_t* da, int64_t T, int64_t I, uint16_t* dgu, hipStream_t s);
}  // namespace lsl
