// HBM-bound steps of the decoder layer: RMSNorm forward/backward, rotary
// embedding, SwiGLU forward/backward, embedding gather and AdamW. One wave per
// row for the row reductions (wave64 shuffles, no LDS), 16-byte accesses.
#include "common.h"
#include "small.h"
#include "api_util.h"
#include <cmath>

namespace lsl {

// ---------------------------------------------------------------- RMSNorm
// One workgroup of RMS_THREADS threads per row. Thread t holds the row's
// 16-byte chunks t, t + 256, ... (columns 8 (t + 256 k) .. + 7, rows up to
// 256 * 8 * RMS_CHUNKS columns) in registers, so all of the row's loads are in
// flight together. Row sums are taken per thread in chunk order, then over the
// wave (butterfly), then over the four waves in wave order through LDS: the same
// order in every RMSNorm kernel here, so a kernel that reads its input as split
// partials gives the bits of the plain one.
constexpr int RMS_THREADS = 256, RMS_CHUNKS = 4;

LSL_DEV float row_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float t = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();  // red is written again by the next sum
  return t;
}

// The split-K sum of a GEMM's output fused into the RMSNorm that reads it.
// Eight columns of a row: the float32 partials of the S splits ([S][T][H] at
// part) added in split order, the bias added, rounded to bf16, the residual
// added and rounded again: the arithmetic of gemm_split_reduce, so the bf16
// values are the ones that kernel stores.
LSL_DEV u32x4 split_sum8(const float* __restrict__ part, int S, int64_t TH, int64_t off,
                         const uint16_t* __restrict__ bias, const uint16_t* __restrict__ res, int64_t col) {
  f32x4 a = *reinterpret_cast<const f32x4*>(part + off), b = *reinterpret_cast<const f32x4*>(part + off + 4);
  for (int sp = 1; sp < S; ++sp) {
    const f32x4 p = *reinterpret_cast<const f32x4*>(part + sp * TH + off);
    const f32x4 q = *reinterpret_cast<const f32x4*>(part + sp * TH + off + 4);
    a = f32x4{a[0] + p[0], a[1] + p[1], a[2] + p[2], a[3] + p[3]};
    b = f32x4{b[0] + q[0], b[1] + q[1], b[2] + q[2], b[3] + q[3]};
  }
  float e[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  if (bias) {
    const u32x4 bb = *reinterpret_cast<const u32x4*>(bias + col);
#pragma unroll
    for (int j = 0; j < 4; ++j) { e[2 * j] += lo_bf(bb[j]); e[2 * j + 1] += hi_bf(bb[j]); }
  }
  if (res) {
    const u32x4 rr = *reinterpret_cast<const u32x4*>(res);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[2 * j] = bf2f(f2bf(e[2 * j])) + lo_bf(rr[j]);
      e[2 * j + 1] = bf2f(f2bf(e[2 * j + 1])) + hi_bf(rr[j]);
    }
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack2(e[2 * j], e[2 * j + 1]);
  return o;
}

// Where an RMSNorm kernel takes its input row: a bf16 tensor, or (SPLIT) the
// split-K partials of the GEMM before it, summed as gemm_split_reduce would
// (+ bias, + res) and written to `out` as that kernel would store them.
struct RmsIn {
  const uint16_t* x;                                  // bf16 [T x H] (not SPLIT)
  const float* part; int S;                           // SPLIT: float32 [S][T][H]
  const uint16_t* bias; const uint16_t* res; int64_t ldres;
  uint16_t* out;                                      // SPLIT: the summed bf16 [T x H]
};
template <bool SPLIT>
LSL_DEV u32x4 rms_load(const RmsIn& in, int64_t T, int64_t H, int64_t row, int64_t col) {
  if constexpr (SPLIT) {
    const u32x4 v = split_sum8(in.part, in.S, T * H, row * H + col, in.bias,
                               in.res ? in.res + row * in.ldres + col : nullptr, col);
    *reinterpret_cast<u32x4*>(in.out + row * H + col) = v;
    return v;
  } else {
    return *reinterpret_cast<const u32x4*>(in.x + row * H + col);
  }
}

// y = bf16(x * r * w), r = 1 / sqrt(mean(x^2) + eps). Side job of workgroup 0:
// zero the caller's nzero words.
template <bool SPLIT>
__global__ __launch_bounds__(RMS_THREADS) void rmsnorm_fwd_kernel(const RmsIn in, const uint16_t* __restrict__ w,
                                                                  int64_t T, int64_t H, float eps,
                                                                  uint16_t* __restrict__ y, unsigned* __restrict__ zero,
                                                                  int nzero) {
  __shared__ float red[4];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0u;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  u32x4 v[RMS_CHUNKS];
#pragma unroll
  for (int k = 0; k < RMS_CHUNKS; ++k) {
    const int64_t col = (int64_t)(tid + RMS_THREADS * k) * 8;
    if (col < H) v[k] = rms_load<SPLIT>(in, T, H, row, col);
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < RMS_CHUNKS; ++k)
    if ((int64_t)(tid + RMS_THREADS * k) * 8 < H)
#pragma unroll
      for (int j = 0; j < 4; ++j) { float a = lo_bf(v[k][j]), b = hi_bf(v[k][j]); ss += a * a + b * b; }
  ss = row_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int k = 0; k < RMS_CHUNKS; ++k) {
    const int64_t col = (int64_t)(tid + RMS_THREADS * k) * 8;
    if (col >= H) continue;
    const u32x4 g = *reinterpret_cast<const u32x4*>(w + col);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack2(lo_bf(v[k][j]) * r * lo_bf(g[j]), hi_bf(v[k][j]) * r * hi_bf(g[j]));
    *reinterpret_cast<u32x4*>(y + row * H + col) = o;
  }
}

// dx = bf16(dres + r (w dy - x r^2 sum(x w dy) / H)); the row's x and dy chunks
// stay in registers between the two passes.
template <bool SPLIT>
__global__ __launch_bounds__(RMS_THREADS) void rmsnorm_bwd_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ w, const RmsIn dyin,
                                                                  const uint16_t* __restrict__ dres, int64_t T,
                                                                  int64_t H, float eps, uint16_t* __restrict__ dx) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  u32x4 xv[RMS_CHUNKS], dv[RMS_CHUNKS];
  float ss = 0.f, sd = 0.f;
#pragma unroll
  for (int k = 0; k < RMS_CHUNKS; ++k) {
    const int64_t c = (int64_t)(tid + RMS_THREADS * k) * 8;
    if (c >= H) continue;
    xv[k] = *reinterpret_cast<const u32x4*>(x + row * H + c);
    dv[k] = rms_load<SPLIT>(dyin, T, H, row, c);
    const u32x4 g = *reinterpret_cast<const u32x4*>(w + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = lo_bf(xv[k][j]), b = hi_bf(xv[k][j]);
      ss += a * a + b * b;
      sd += a * lo_bf(g[j]) * lo_bf(dv[k][j]) + b * hi_bf(g[j]) * hi_bf(dv[k][j]);
    }
  }
  ss = row_sum(ss, red);
  sd = row_sum(sd, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  const float c2 = r * r * sd / (float)H;
#pragma unroll
  for (int k = 0; k < RMS_CHUNKS; ++k) {
    const int64_t c = (int64_t)(tid + RMS_THREADS * k) * 8;
    if (c >= H) continue;
    const u32x4 g = *reinterpret_cast<const u32x4*>(w + c);
    const u32x4 rs = dres ? *reinterpret_cast<const u32x4*>(dres + row * H + c) : u32x4{0, 0, 0, 0};
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e0 = lo_bf(rs[j]) + r * (lo_bf(g[j]) * lo_bf(dv[k][j]) - lo_bf(xv[k][j]) * c2);
      const float e1 = hi_bf(rs[j]) + r * (hi_bf(g[j]) * hi_bf(dv[k][j]) - hi_bf(xv[k][j]) * c2);
      o[j] = pack2(e0, e1);
    }
    *reinterpret_cast<u32x4*>(dx + row * H + c) = o;
  }
}

static lsl_status rms_check(int64_t H, const char* what, int64_t T = 0) {
  if (H > (int64_t)RMS_THREADS * 8 * RMS_CHUNKS || H % 8)
    return set_error(LSL_ERR_UNSUPPORTED, "%s: hidden %lld (a multiple of 8 up to %d)", what, (long long)H,
                     RMS_THREADS * 8 * RMS_CHUNKS);
  if (T >= ((int64_t)1 << 31)) return set_error(LSL_ERR_UNSUPPORTED, "%s: %lld rows (one workgroup each)", what, (long long)T);
  return LSL_OK;
}

lsl_status rmsnorm_fwd_launch(const uint16_t* x, const uint16_t* w, int64_t T, int64_t H, float eps, uint16_t* y,
                              hipStream_t s, unsigned* zero, int nzero) {
  LSL_TRY(rms_check(H, "rmsnorm", T));
  if (T == 0) return LSL_OK;
  RmsIn in{};
  in.x = x;
  hipLaunchKernelGGL(rmsnorm_fwd_kernel<false>, dim3((unsigned)T), dim3(RMS_THREADS), 0, s, in, w, T, H, eps, y, zero,
                     zero ? nzero : 0);
  return check_launch("rmsnorm_fwd");
}
lsl_status rmsnorm_bwd_launch(const uint16_t* x, const uint16_t* w, const uint16_t* dy, const uint16_t* dres,
                              int64_t T, int64_t H, float eps, uint16_t* dx, hipStream_t s) {
  LSL_TRY(rms_check(H, "rmsnorm backward", T));
  if (T == 0) return LSL_OK;
  RmsIn in{};
  in.x = dy;
  hipLaunchKernelGGL(rmsnorm_bwd_kernel<false>, dim3((unsigned)T), dim3(RMS_THREADS), 0, s, x, w, in, dres, T, H, eps,
                     dx);
  return check_launch("rmsnorm_bwd");
}
lsl_status rmsnorm_fwd_split_launch(const float* part, int S, const uint16_t* bias, const uint16_t* res, int64_t ldres,
                                    uint16_t* h, const uint16_t* w, int64_t T, int64_t H, float eps, uint16_t* y,
                                    hipStream_t s) {
  LSL_TRY(rms_check(H, "rmsnorm (split sum)", T));
  if (S < 1) return set_error(LSL_ERR_INVALID_ARG, "rmsnorm (split sum): %d splits", S);
  if (T == 0) return LSL_OK;
  RmsIn in{};
  in.part = part; in.S = S; in.bias = bias; in.res = res; in.ldres = ldres; in.out = h;
  hipLaunchKernelGGL(rmsnorm_fwd_kernel<true>, dim3((unsigned)T), dim3(RMS_THREADS), 0, s, in, w, T, H, eps, y,
                     (unsigned*)nullptr, 0);
  return check_launch("rmsnorm_fwd (split sum)");
}
lsl_status rmsnorm_bwd_split_launch(const uint16_t* x, const uint16_t* w, const float* part, int S,
                                    const uint16_t* dres, int64_t T, int64_t H, float eps, uint16_t* dy_out,
                                    uint16_t* dx, hipStream_t s) {
  LSL_TRY(rms_check(H, "rmsnorm backward (split sum)", T));
  if (S < 1) return set_error(LSL_ERR_INVALID_ARG, "rmsnorm backward (split sum): %d splits", S);
  if (T == 0) return LSL_OK;
  RmsIn in{};
  in.part = part; in.S = S; in.out = dy_out;
  hipLaunchKernelGGL(rmsnorm_bwd_kernel<true>, dim3((unsigned)T), dim3(RMS_THREADS), 0, s, x, w, in, dres, T, H, eps,
                     dx);
  return check_launch("rmsnorm_bwd (split sum)");
}

// ---------------------------------------------------------------- RoPE
// The inverse frequencies theta^(-2i/d) (optionally rescaled the Llama-3.1 way)
// are computed on the host in float64 and passed by value. A workgroup takes
// ROPE_ROWS rows: first the float64 angle and its sine/cosine for each
// (row, i) into LDS, then every head's pairs (i, i + d/2) of those rows are
// rotated in float32 four at a time (8-byte accesses) and rounded to bf16 into
// y (the same row layout as x; y may be x).
struct RopeFreq {
  double inv[64];  // head_dim / 2 <= 64
};

static RopeFreq rope_freq(int head_dim, double theta, const lsl_rope_scaling* sc) {
  RopeFreq fr{};
  const double pi = 3.141592653589793;
  for (int i = 0; i < head_dim / 2; ++i) {
    double f = std::pow(theta, -2.0 * (double)i / (double)head_dim);
    if (sc && sc->factor != 0.f) {
      const double factor = sc->factor, low = sc->low_freq_factor, high = sc->high_freq_factor;
      const double orig = sc->original_max_position;
      const double wavelen = 2.0 * pi / f;
      if (wavelen > orig / low) {
        f = f / factor;
      } else if (wavelen >= orig / high) {
        const double m = (orig / wavelen - low) / (high - low);
        f = (1.0 - m) * f / factor + m * f;
      }
    }
    fr.inv[i] = f;
  }
  return fr;
}

// rows per workgroup: one row gives four times the workgroups of four rows and
// a quarter of the dependent load/store rounds per thread, which the launch's
// latency, not its bandwidth, pays for
#ifndef LSL_ROPE_ROWS
#define LSL_ROPE_ROWS 1
#endif
constexpr int ROPE_ROWS = LSL_ROPE_ROWS;

__global__ __launch_bounds__(256) void rope_kernel(const uint16_t* x, uint16_t* y, int64_t T, int64_t ld, int n_heads,
                                                   int head_dim, int seq, RopeFreq fr, int inverse) {
  __shared__ float cs[ROPE_ROWS][64], sn[ROPE_ROWS][64];
  const int half = head_dim >> 1;
  const int64_t r0 = (int64_t)blockIdx.x * ROPE_ROWS;
  for (int t = threadIdx.x; t < ROPE_ROWS * half; t += blockDim.x) {
    const int rr = t / half, i = t - rr * half;
    const int64_t row = r0 + rr;
    if (row >= T) continue;
    const double ang = (double)(row % seq) * fr.inv[i];
    double sd, cd;
    sincos(ang, &sd, &cd);
    cs[rr][i] = (float)cd;
    sn[rr][i] = inverse ? -(float)sd : (float)sd;
  }
  __syncthreads();
  const int q4 = half >> 2;          // groups of 4 pairs per head
  const int per_row = n_heads * q4;
  for (int t = threadIdx.x; t < ROPE_ROWS * per_row; t += blockDim.x) {
    const int rr = t / per_row, rem = t - rr * per_row;
    const int h = rem / q4, g = rem - h * q4;
    const int64_t row = r0 + rr;
    if (row >= T) continue;
    const int64_t off = row * ld + (int64_t)h * head_dim + 4 * g;
    const u32x2 a = *reinterpret_cast<const u32x2*>(x + off);
    const u32x2 b = *reinterpret_cast<const u32x2*>(x + off + half);
    float x1[4] = {lo_bf(a[0]), hi_bf(a[0]), lo_bf(a[1]), hi_bf(a[1])};
    float x2[4] = {lo_bf(b[0]), hi_bf(b[0]), lo_bf(b[1]), hi_bf(b[1])};
    float o1[4], o2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c = cs[rr][4 * g + e], s = sn[rr][4 * g + e];
      o1[e] = x1[e] * c - x2[e] * s;
      o2[e] = x2[e] * c + x1[e] * s;
    }
    *reinterpret_cast<u32x2*>(y + off) = u32x2{pack2(o1[0], o1[1]), pack2(o1[2], o1[3])};
    *reinterpret_cast<u32x2*>(y + off + half) = u32x2{pack2(o2[0], o2[1]), pack2(o2[2], o2[3])};
  }
}

// Four columns of a row of a split GEMM's output: the float32 partials of the S
// splits ([S][T][ld] at part) added in split order and the bias added, as
// gemm_split_reduce does before its rounding.
LSL_DEV void split_sum4(const float* __restrict__ part, int S, int64_t Tld, int64_t off,
                        const uint16_t* __restrict__ bias, int64_t col, float (&e)[4]) {
  f32x4 a = *reinterpret_cast<const f32x4*>(part + off);
  for (int sp = 1; sp < S; ++sp) {
    const f32x4 p = *reinterpret_cast<const f32x4*>(part + sp * Tld + off);
    a = f32x4{a[0] + p[0], a[1] + p[1], a[2] + p[2], a[3] + p[3]};
  }
  e[0] = a[0]; e[1] = a[1]; e[2] = a[2]; e[3] = a[3];
  if (bias) {
    const u32x2 b = *reinterpret_cast<const u32x2*>(bias + col);
    e[0] += lo_bf(b[0]); e[1] += hi_bf(b[0]); e[2] += lo_bf(b[1]); e[3] += hi_bf(b[1]);
  }
}

// The q|k|v projection's split-K sum fused with RoPE: every column of the
// [T x ld] output is summed (+ bias) and rounded as gemm_split_reduce would
// store it into qkv; the first n_heads heads of each row (q and k) are then
// rotated from those bf16 values exactly as rope_kernel rotates them, into y.
__global__ __launch_bounds__(256) void rope_split_kernel(const float* __restrict__ part, int S,
                                                         const uint16_t* __restrict__ bias, uint16_t* __restrict__ qkv,
                                                         uint16_t* __restrict__ y, int64_t T, int64_t ld, int n_heads,
                                                         int head_dim, int seq, RopeFreq fr) {
  __shared__ float cs[ROPE_ROWS][64], sn[ROPE_ROWS][64];
  const int half = head_dim >> 1;
  const int64_t r0 = (int64_t)blockIdx.x * ROPE_ROWS;
  for (int t = threadIdx.x; t < ROPE_ROWS * half; t += blockDim.x) {
    const int rr = t / half, i = t - rr * half;
    const int64_t row = r0 + rr;
    if (row >= T) continue;
    const double ang = (double)(row % seq) * fr.inv[i];
    double sd, cd;
    sincos(ang, &sd, &cd);
    cs[rr][i] = (float)cd;
    sn[rr][i] = (float)sd;
  }
  __syncthreads();
  const int64_t Tld = T * ld;
  const int q4 = half >> 2;
  const int per_row = n_heads * q4;
  for (int t = threadIdx.x; t < ROPE_ROWS * per_row; t += blockDim.x) {
    const int rr = t / per_row, rem = t - rr * per_row;
    const int h = rem / q4, g = rem - h * q4;
    const int64_t row = r0 + rr;
    if (row >= T) continue;
    const int64_t col = (int64_t)h * head_dim + 4 * g, off = row * ld + col;
    float e1[4], e2[4];
    split_sum4(part, S, Tld, off, bias, col, e1);
    split_sum4(part, S, Tld, off + half, bias, col + half, e2);
    const u32x2 a = u32x2{pack2(e1[0], e1[1]), pack2(e1[2], e1[3])};
    const u32x2 b = u32x2{pack2(e2[0], e2[1]), pack2(e2[2], e2[3])};
    *reinterpret_cast<u32x2*>(qkv + off) = a;
    *reinterpret_cast<u32x2*>(qkv + off + half) = b;
    float x1[4] = {lo_bf(a[0]), hi_bf(a[0]), lo_bf(a[1]), hi_bf(a[1])};
    float x2[4] = {lo_bf(b[0]), hi_bf(b[0]), lo_bf(b[1]), hi_bf(b[1])};
    float o1[4], o2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c = cs[rr][4 * g + e], s = sn[rr][4 * g + e];
      o1[e] = x1[e] * c - x2[e] * s;
      o2[e] = x2[e] * c + x1[e] * s;
    }
    *reinterpret_cast<u32x2*>(y + off) = u32x2{pack2(o1[0], o1[1]), pack2(o1[2], o1[3])};
    *reinterpret_cast<u32x2*>(y + off + half) = u32x2{pack2(o2[0], o2[1]), pack2(o2[2], o2[3])};
  }
  // the remaining columns (v): the sum alone
  const int64_t c0 = (int64_t)n_heads * head_dim;
  const int v4 = (int)((ld - c0) >> 2);
  for (int t = threadIdx.x; t < ROPE_ROWS * v4; t += blockDim.x) {
    const int rr = t / v4, g = t - rr * v4;
    const int64_t row = r0 + rr;
    if (row >= T) continue;
    const int64_t col = c0 + 4 * (int64_t)g, off = row * ld + col;
    float e[4];
    split_sum4(part, S, Tld, off, bias, col, e);
    *reinterpret_cast<u32x2*>(qkv + off) = u32x2{pack2(e[0], e[1]), pack2(e[2], e[3])};
  }
}

lsl_status rope_split_launch(const float* part, int S, const uint16_t* bias, uint16_t* qkv, uint16_t* y, int64_t T,
                             int64_t ld, int n_heads, int head_dim, int seq, float theta,
                             const lsl_rope_scaling* scaling, hipStream_t s) {
  if (head_dim % 8 || head_dim > 128 || ld % 4 || ld < (int64_t)n_heads * head_dim || S < 1)
    return set_error(LSL_ERR_UNSUPPORTED, "rope (split sum): head_dim %d, ld %lld, %d splits", head_dim, (long long)ld,
                     S);
  if (T == 0) return LSL_OK;
  const RopeFreq fr = rope_freq(head_dim, (double)theta, scaling);
  hipLaunchKernelGGL(rope_split_kernel, dim3((unsigned)((T + ROPE_ROWS - 1) / ROPE_ROWS)), dim3(256), 0, s, part, S,
                     bias, qkv, y, T, ld, n_heads, head_dim, seq, fr);
  return check_launch("rope (split sum)");
}

lsl_status rope_launch(const uint16_t* x, uint16_t* y, int64_t T, int64_t ld, int n_heads, int head_dim, int seq,
                       float theta, const lsl_rope_scaling* scaling, int inverse, hipStream_t s) {
  if (head_dim % 8 || head_dim > 128)
    return set_error(LSL_ERR_UNSUPPORTED, "rope: head_dim %d (a multiple of 8, at most 128)", head_dim);
  if (T == 0) return LSL_OK;
  const RopeFreq fr = rope_freq(head_dim, (double)theta, scaling);
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)((T + ROPE_ROWS - 1) / ROPE_ROWS)), dim3(256), 0, s, x, y, T, ld,
                     n_heads, head_dim, seq, fr, inverse);
  return check_launch("rope");
}

// ---------------------------------------------------------------- SwiGLU
LSL_DEV float sigm(float g) { return 1.0f / (1.0f + expf(-g)); }

// Grid (ceil(I / 2048), rows): a thread takes 8 columns of one row (no index
// division); rows past the grid's height are taken in steps of it.
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const uint16_t* __restrict__ gu, int64_t T, int64_t I,
                                                         uint16_t* __restrict__ a) {
  const int64_t c = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (c >= I) return;
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    u32x4 g = *reinterpret_cast<const u32x4*>(gu + t * 2 * I + c);
    u32x4 u = *reinterpret_cast<const u32x4*>(gu + t * 2 * I + I + c);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float g0 = lo_bf(g[j]), g1 = hi_bf(g[j]);
      o[j] = pack2(g0 * sigm(g0) * lo_bf(u[j]), g1 * sigm(g1) * hi_bf(u[j]));
    }
    *reinterpret_cast<u32x4*>(a + t * I + c) = o;
  }
}

__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t* __restrict__ gu,
                                                         const uint16_t* __restrict__ da, int64_t T, int64_t I,
                                                         uint16_t* __restrict__ dgu) {
  const int64_t c = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (c >= I) return;
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    u32x4 g = *reinterpret_cast<const u32x4*>(gu + t * 2 * I + c);
    u32x4 u = *reinterpret_cast<const u32x4*>(gu + t * 2 * I + I + c);
    u32x4 d = *reinterpret_cast<const u32x4*>(da + t * I + c);
    u32x4 og, ou;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float gg[2] = {lo_bf(g[j]), hi_bf(g[j])}, uu[2] = {lo_bf(u[j]), hi_bf(u[j])}, dd[2] = {lo_bf(d[j]), hi_bf(d[j])};
      float rg[2], ru[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float sg = sigm(gg[e]);
        rg[e] = dd[e] * uu[e] * sg * (1.0f + gg[e] * (1.0f - sg));
        ru[e] = dd[e] * gg[e] * sg;
      }
      og[j] = pack2(rg[0], rg[1]);
      ou[j] = pack2(ru[0], ru[1]);
    }
    *reinterpret_cast<u32x4*>(dgu + t * 2 * I + c) = og;
    *reinterpret_cast<u32x4*>(dgu + t * 2 * I + I + c) = ou;
  }
}

static dim3 swiglu_grid(int64_t T, int64_t I) {
  return dim3((unsigned)((I / 8 + 255) / 256), (unsigned)(T < 65535 ? T : 65535));
}
lsl_status swiglu_fwd_launch(const uint16_t* gu, int64_t T, int64_t I, uint16_t* a, hipStream_t s) {
  if (T == 0) return LSL_OK;
  hipLaunchKernelGGL(swiglu_fwd_kernel, swiglu_grid(T, I), dim3(256), 0, s, gu, T, I, a);
  return check_launch("swiglu_fwd");
}
lsl_status swiglu_bwd_launch(const uint16_t* gu, const uint16_t* da, int64_t T, int64_t I, uint16_t* dgu, hipStream_t s) {
  if (T == 0) return LSL_OK;
  hipLaunchKernelGGL(swiglu_bwd_kernel, swiglu_grid(T, I), dim3(256), 0, s, gu, da, T, I, dgu);
  return check_launch("swiglu_bwd");
}

// ---------------------------------------------------------------- embedding
__global__ void embed_kernel(const uint16_t* __restrict__ table, const int32_t* __restrict__ ids, int64_t T, int64_t H,
                             int64_t V, uint16_t* __restrict__ out) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t per = H / 8;
  if (idx >= T * per) return;
  int64_t t = idx / per, c = (idx - t * per) * 8;
  int64_t id = ids[t];
  u32x4 v = (id >= 0 && id < V) ? *reinterpret_cast<const u32x4*>(table + id * H + c) : u32x4{0, 0, 0, 0};
  *reinterpret_cast<u32x4*>(out + t * H + c) = v;
}

// ---------------------------------------------------------------- AdamW
__global__ void adamw_kernel(float* __restrict__ p, uint16_t* __restrict__ pb, const float* __restrict__ g,
                             float* __restrict__ m, float* __restrict__ v, int64_t n, float lr, float b1, float b2,
                             float eps, float decay, float bc1, float bc2) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float gi = g[i];
  float pi = p[i] * decay;
  float mi = b1 * m[i] + (1.0f - b1) * gi;
  float vi = b2 * v[i] + (1.0f - b2) * gi * gi;
  pi -= lr * (mi / bc1) / (sqrtf(vi / bc2) + eps);
  p[i] = pi; m[i] = mi; v[i] = vi;
  if (pb) pb[i] = f2bf(pi);
}

}  // namespace lsl

using namespace lsl;

extern "C" lsl_status lsl_embed_fwd(const uint16_t* table, const int32_t* ids, int64_t T, int64_t H, int64_t V,
                                    uint16_t* out, lsl_stream stream) {
  if (T < 0 || H <= 0 || V <= 0 || H % 8)
    return set_error(LSL_ERR_INVALID_ARG, "lsl_embed_fwd: bad sizes (H must be a multiple of 8)");
  if (T == 0) return LSL_OK;
  if (!table || !ids || !out || !aligned(table, 16) || !aligned(out, 16) || !aligned(ids, 4))
    return set_error(LSL_ERR_INVALID_ARG, "lsl_embed_fwd: null or misaligned pointer");
  int64_t n = T * (H / 8);
  hipLaunchKernelGGL(embed_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, table, ids, T,
                     H, V, out);
  return check_launch("embed");
}

extern "C" lsl_status lsl_adamw_step(float* p, uint16_t* p_bf16, const float* g, float* m, float* v, int64_t n,
                                     int32_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                                     lsl_stream stream) {
  if (n < 0 || step < 1) return set_error(LSL_ERR_INVALID_ARG, "lsl_adamw_step: n >= 0 and step >= 1 required");
  if (n == 0) return LSL_OK;
  if (!p || !g || !m || !v) return set_error(LSL_ERR_INVALID_ARG, "lsl_adamw_step: null pointer");
  float bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
  float bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
  float decay = 1.0f - lr * weight_decay;
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, p, p_bf16, g,
                     m, v, n, lr, beta1, beta2, eps, decay, bc1, bc2);
  return check_launch("adamw");
}
