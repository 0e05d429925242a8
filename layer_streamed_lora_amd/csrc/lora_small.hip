// The rank-r side products of LoRA on bf16 MFMA, with fixed-order split
// reductions (no atomics, so every run gives the same bits).
//
//   NT  (t, u):   C[t][j] = sum_k P[t][k] R[j][k]          P [T x K], j < kl <= 64
//        t = x A^T           R = A_full [kl x K]
//        u = dy B (per fused projection)  R[j][n] = B[n][j % r] if column n belongs to projection j / r
//   TN  (dA, dB): C[a][j] = sum_t P[t][a] Q[t][j]          P [T x W], Q [T x kl]
//        dA[j][k] += s C[k][j]              (P = x,  Q = u)
//        dB[n][i] += s C[n][p(n) r + i]     (P = dy, Q = t)
// The first kernel of each pair writes float32 partial sums per split of the
// reduction; the second adds the splits in index order and writes the result.
#include "common.h"
#include "small.h"

namespace lsl {

constexpr int SK_LDS = 72;  // LDS row stride (64 + 8 elements)

LSL_DEV f32x4 mfma16s(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct NtArgs {
  const uint16_t* p; int64_t ldp;   // [T x K]
  const uint16_t* rA;               // A_full [kl x K]  (mode 0)
  const uint16_t* rB; int r; int nseg; int64_t seg_end[4];  // B_full [K x r] (mode 1)
  int64_t T, K; int kl;
  int64_t k_per_split;
  float* part;                      // [S][T][kl]
};

// grid: (ceil(T/128), S); 4 waves, wave w owns rows 32w..32w+31 of the tile.
template <int MODE>
__global__ __launch_bounds__(256) void lora_nt_kernel(const NtArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ps[128 * SK_LDS];
  __shared__ __attribute__((aligned(16))) uint16_t Rs[64 * SK_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * 128;
  const int64_t kbeg = (int64_t)blockIdx.y * a.k_per_split;
  const int64_t kend = kbeg + a.k_per_split < a.K ? kbeg + a.k_per_split : a.K;
  f32x4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kbeg; k0 < kend; k0 += 64) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid + i * 256, row = c >> 3, col = (c & 7) * 8;
      int64_t gt = t0 + row;
      u32x4 v = gt < a.T ? *reinterpret_cast<const u32x4*>(a.p + gt * a.ldp + k0 + col) : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(Ps + row * SK_LDS + col) = v;
    }
    if constexpr (MODE == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int c = tid + i * 256, row = c >> 3, col = (c & 7) * 8;
        u32x4 v = row < a.kl ? *reinterpret_cast<const u32x4*>(a.rA + (int64_t)row * a.K + k0 + col) : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(Rs + row * SK_LDS + col) = v;
      }
    } else {
      // Rs[j][kk] = B[k0+kk][j % r] masked by projection; thread -> one kk, 16 j's
      int kk = tid & 63, jq = tid >> 6;  // jq: 16-wide j group
      int64_t n = k0 + kk;
      int seg = 0;
      while (seg < a.nseg - 1 && n >= a.seg_end[seg]) ++seg;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        int j = jq * 16 + jj;
        uint16_t v = 0;
        if (j < a.kl && j / a.r == seg) v = a.rB[n * a.r + (j % a.r)];
        Rs[j * SK_LDS + kk] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      int kofs = ks * 32 + (lane >> 4) * 8;
      bf16x8 rf[4], pf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) rf[i] = *reinterpret_cast<const bf16x8*>(Rs + (i * 16 + (lane & 15)) * SK_LDS + kofs);
#pragma unroll
      for (int i = 0; i < 2; ++i) pf[i] = *reinterpret_cast<const bf16x8*>(Ps + (wave * 32 + i * 16 + (lane & 15)) * SK_LDS + kofs);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16s(rf[i], pf[j], acc[i][j]);
    }
    __syncthreads();
  }
  // lane holds C[t][j..j+3], j = 16 i + 4 (lane >> 4)
  float* dst = a.part + (int64_t)blockIdx.y * a.T * a.kl;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int64_t t = t0 + wave * 32 + j * 16 + (lane & 15);
    if (t >= a.T) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = i * 16 + (lane >> 4) * 4;
      if (c < a.kl) *reinterpret_cast<f32x4*>(dst + t * a.kl + c) = acc[i][j];
    }
  }
}

// out[t][j] = bf16(sum_s part[s][t][j]) for j < kl
__global__ void nt_reduce_kernel(const float* __restrict__ part, int S, int64_t T, int kl, uint16_t* __restrict__ out, int64_t ldo) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * kl) return;
  int64_t t = i / kl; int j = (int)(i - t * kl);
  float s = 0.f;
  for (int k = 0; k < S; ++k) s += part[((int64_t)k * T + t) * kl + j];
  out[t * ldo + j] = f2bf(s);
}

struct TnArgs {
  const uint16_t* p; int64_t ldp;  // [T x W]
  const uint16_t* q; int64_t ldq;  // [T x kl]
  int64_t T, W; int kl;
  int64_t t_per_split;
  float* part;                     // [S][W][kl] (S > 1)
  // S == 1: the result goes straight to dA [kl x W] or dB [W x r] (+= scale C)
  float* dA; float* dB; float scale; int r; int nseg; SegEnds seg;
};

// grid: (ceil(W/128), S). 4 waves, wave w owns columns a = 32w..32w+31 of the tile.
template <bool DIRECT>
__global__ __launch_bounds__(256) void lora_tn_kernel(const TnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ps[128 * SK_LDS];  // [a][t]
  __shared__ __attribute__((aligned(16))) uint16_t Qs[64 * SK_LDS];   // [j][t]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t a0 = (int64_t)blockIdx.x * 128;
  const int64_t tbeg = (int64_t)blockIdx.y * a.t_per_split;
  const int64_t tend = tbeg + a.t_per_split < a.T ? tbeg + a.t_per_split : a.T;
  f32x4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t tt = tbeg; tt < tend; tt += 64) {
    {  // P: 4 t-rows x 8 a-cols per thread, stored transposed
      int q = tid >> 4, o = tid & 15;
      int64_t ac = a0 + o * 8;
      uint32_t w[4][4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        int64_t t = tt + q * 4 + rr;
        u32x4 v = (t < tend && ac < a.W) ? *reinterpret_cast<const u32x4*>(a.p + t * a.ldp + ac) : u32x4{0, 0, 0, 0};
        w[rr][0] = v[0]; w[rr][1] = v[1]; w[rr][2] = v[2]; w[rr][3] = v[3];
      }
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        uint32_t e[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) e[rr] = (cc & 1) ? (w[rr][cc >> 1] >> 16) : (w[rr][cc >> 1] & 0xFFFFu);
        *reinterpret_cast<u32x2*>(Ps + (o * 8 + cc) * SK_LDS + q * 4) = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
      }
    }
    {  // Q: 2 t-rows x 8 j-cols per thread, stored transposed
      int q = tid >> 3, o = tid & 7;
      uint32_t w[2][4];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        int64_t t = tt + q * 2 + rr;
        u32x4 v = (t < tend && o * 8 < a.kl) ? *reinterpret_cast<const u32x4*>(a.q + t * a.ldq + o * 8) : u32x4{0, 0, 0, 0};
        w[rr][0] = v[0]; w[rr][1] = v[1]; w[rr][2] = v[2]; w[rr][3] = v[3];
      }
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        uint32_t e0 = (cc & 1) ? (w[0][cc >> 1] >> 16) : (w[0][cc >> 1] & 0xFFFFu);
        uint32_t e1 = (cc & 1) ? (w[1][cc >> 1] >> 16) : (w[1][cc >> 1] & 0xFFFFu);
        *reinterpret_cast<uint32_t*>(Qs + (o * 8 + cc) * SK_LDS + q * 2) = e0 | (e1 << 16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      int kofs = ks * 32 + (lane >> 4) * 8;
      bf16x8 qf[4], pf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[i] = *reinterpret_cast<const bf16x8*>(Qs + (i * 16 + (lane & 15)) * SK_LDS + kofs);
#pragma unroll
      for (int i = 0; i < 2; ++i) pf[i] = *reinterpret_cast<const bf16x8*>(Ps + (wave * 32 + i * 16 + (lane & 15)) * SK_LDS + kofs);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16s(qf[i], pf[j], acc[i][j]);
    }
    __syncthreads();
  }
  // lane holds C[a][c..c+3], c = 16 i + 4 (lane >> 4)
  float* dst = a.part + (int64_t)blockIdx.y * a.W * a.kl;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int64_t ac = a0 + wave * 32 + j * 16 + (lane & 15);
    if (ac >= a.W) continue;
    int p = 0;
    if (DIRECT && a.dB)
      while (p < a.nseg - 1 && ac >= a.seg.e[p]) ++p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = i * 16 + (lane >> 4) * 4;
      if (c >= a.kl) continue;
      if (!DIRECT) {
        *reinterpret_cast<f32x4*>(dst + ac * a.kl + c) = acc[i][j];
      } else if (a.dA) {
#pragma unroll
        for (int e = 0; e < 4; ++e) a.dA[(int64_t)(c + e) * a.W + ac] += a.scale * acc[i][j][e];
      } else if (c >= p * a.r && c < (p + 1) * a.r) {
        f32x4* d = reinterpret_cast<f32x4*>(a.dB + ac * a.r + (c - p * a.r));
        f32x4 v = *d;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += a.scale * acc[i][j][e];
        *d = v;
      }
    }
  }
}

// dA[j][k] += s * sum_s part[s][k][j]
__global__ void tn_reduce_dA_kernel(const float* __restrict__ part, int S, int64_t W, int kl, float scale, float* __restrict__ dA) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= W * kl) return;
  int j = (int)(i / W); int64_t k = i - (int64_t)j * W;
  float s = 0.f;
  for (int q = 0; q < S; ++q) s += part[((int64_t)q * W + k) * kl + j];
  dA[i] += scale * s;
}

// dB[n][i] += s * sum_s part[s][n][p(n) r + i]
__global__ void tn_reduce_dB_kernel(const float* __restrict__ part, int S, int64_t W, int kl, int r, int nseg,
                                    SegEnds seg, float scale, float* __restrict__ dB) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= W * r) return;
  int64_t n = idx / r; int i = (int)(idx - n * r);
  int p = 0;
  while (p < nseg - 1 && n >= seg.e[p]) ++p;
  int j = p * r + i;
  float s = 0.f;
  for (int q = 0; q < S; ++q) s += part[((int64_t)q * W + n) * kl + j];
  dB[idx] += scale * s;
}

// ---------------------------------------------------------------- host side
// Splits of the reduction so that about `target_blocks` workgroups run, each
// taking at least `min_steps` 64-wide steps of the reduction.
static int pick_splits(int64_t tiles, int64_t red, int64_t target_blocks, int64_t min_steps) {
  int64_t steps = (red + 63) / 64;
  int64_t s = (target_blocks + tiles - 1) / tiles;
  int64_t cap = steps / min_steps;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
}
constexpr int64_t NT_TARGET = 256, NT_MIN_STEPS = 4, TN_TARGET = 256, TN_MIN_STEPS = 4;

size_t lora_nt_ws_bytes(int64_t T, int64_t K) {
  int64_t tiles = (T + 127) / 128;
  int S = pick_splits(tiles, K, NT_TARGET, NT_MIN_STEPS);
  return (size_t)S * T * 64 * sizeof(float);
}

size_t lora_tn_ws_bytes(int64_t T, int64_t W) {
  int64_t tiles = (W + 127) / 128;
  int S = pick_splits(tiles, T, TN_TARGET, TN_MIN_STEPS);
  return S > 1 ? (size_t)S * W * 64 * sizeof(float) : 0;
}

lsl_status lora_nt_launch(const LoraNt& d, hipStream_t s) {
  if (d.T == 0) return LSL_OK;
  if (d.K % 64 || d.kl <= 0 || d.kl > 64 || d.kl % 8)
    return set_error(LSL_ERR_UNSUPPORTED, "lora side product: K %% 64 and kl in [8, 64] multiple of 8 required");
  int64_t tiles = (d.T + 127) / 128;
  int S = pick_splits(tiles, d.K, NT_TARGET, NT_MIN_STEPS);
  int64_t steps = d.K / 64;
  int64_t per = ((steps + S - 1) / S) * 64;
  S = (int)((d.K + per - 1) / per);
  NtArgs a{};
  a.p = d.p; a.ldp = d.ldp; a.rA = d.a_full; a.rB = d.b_full; a.r = d.r; a.nseg = d.nseg;
  for (int i = 0; i < 4; ++i) a.seg_end[i] = d.seg_end[i];
  a.T = d.T; a.K = d.K; a.kl = d.kl; a.k_per_split = per; a.part = d.ws;
  dim3 grid((unsigned)tiles, (unsigned)S);
  if (d.b_full) hipLaunchKernelGGL(lora_nt_kernel<1>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(lora_nt_kernel<0>, grid, dim3(256), 0, s, a);
  int64_t n = d.T * d.kl;
  hipLaunchKernelGGL(nt_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const float*)d.ws, S, d.T, d.kl, d.out, d.ldo);
  return check_launch("lora_nt");
}

lsl_status lora_tn_launch(const LoraTn& d, hipStream_t s) {
  if (d.W == 0) return LSL_OK;
  if (d.kl <= 0 || d.kl > 64 || d.kl % 8 || d.W % 8)
    return set_error(LSL_ERR_UNSUPPORTED, "lora grad: kl in [8, 64] multiple of 8 and W %% 8 required");
  if (d.T == 0) return LSL_OK;
  int64_t tiles = (d.W + 127) / 128;
  int S = pick_splits(tiles, d.T, TN_TARGET, TN_MIN_STEPS);
  int64_t steps = (d.T + 63) / 64;
  int64_t per = ((steps + S - 1) / S) * 64;
  S = (int)((d.T + per - 1) / per);
  TnArgs a{};
  a.p = d.p; a.ldp = d.ldp; a.q = d.q; a.ldq = d.ldq; a.T = d.T; a.W = d.W; a.kl = d.kl;
  a.t_per_split = per; a.part = d.ws;
  a.dA = d.dA; a.dB = d.dA ? nullptr : d.dB; a.scale = d.scale; a.r = d.r; a.nseg = d.nseg;
  for (int i = 0; i < 4; ++i) a.seg.e[i] = d.seg_end[i];
  if (S == 1) {
    hipLaunchKernelGGL(lora_tn_kernel<true>, dim3((unsigned)tiles, 1), dim3(256), 0, s, a);
    return check_launch("lora_tn");
  }
  hipLaunchKernelGGL(lora_tn_kernel<false>, dim3((unsigned)tiles, (unsigned)S), dim3(256), 0, s, a);
  if (d.dA) {
    int64_t n = d.W * d.kl;
    hipLaunchKernelGGL(tn_reduce_dA_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)d.ws, S, d.W, d.kl, d.scale, d.dA);
  } else {
    int64_t n = d.W * d.r;
    hipLaunchKernelGGL(tn_reduce_dB_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)d.ws, S, d.W, d.kl, d.r, d.nseg, a.seg, d.scale, d.dB);
  }
  return check_launch("lora_tn");
}

}  // namespace lsl
