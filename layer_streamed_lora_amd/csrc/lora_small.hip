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
#include "api_util.h"

namespace lsl {

constexpr int SK_LDS = 72;  // LDS row stride (64 + 8 elements)

LSL_DEV f32x4 mfma16s(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct NtArgs {
  const uint16_t* p; int64_t ldp;   // [T x K]
  const uint16_t* rt;               // R [kl x K], row stride K (A_full, or the masked B transposed)
  int64_t T, K; int kl;
  int64_t k_per_split;              // multiple of 256
  float* part;                      // [S][T][kl] float32 partial sums (S > 1)
  uint16_t* out; int64_t ldo;       // S == 1: the bf16 result [T x kl]
};

// Raw buffer loads: bytes past the descriptor's end read as zeros.
LSL_DEV __amdgpu_buffer_rsrc_t small_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

// C[t][j] = sum_k P[t][k] R[j][k] for a 64-row tile and one split of K.
// grid (ceil(T/64), S), 4 waves; wave w takes the split's 64-wide K-steps
// w, w + 4, ... for all 64 rows and all kl columns, loading both operands from
// global memory (L2) straight into MFMA registers (each P element is read once;
// R is small and shared). The four waves' sums are added in wave order in LDS.
template <bool DIRECT>
__global__ __launch_bounds__(256) void lora_nt_kernel(const NtArgs a) {
  __shared__ f32x4 red[3][4][4][64];
  // the wave index is uniform in a wave: as a scalar, the K loop and the buffer
  // loads' offsets stay scalar (no per-lane loop around every load)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int64_t kbeg = (int64_t)blockIdx.y * a.k_per_split;
  const int64_t kend = kbeg + a.k_per_split < a.K ? kbeg + a.k_per_split : a.K;
  const __amdgpu_buffer_rsrc_t rp = small_rsrc(a.p, a.T * a.ldp * 2);
  const __amdgpu_buffer_rsrc_t rr = small_rsrc(a.rt, (int64_t)a.kl * a.K * 2);
  uint32_t po[4], ro[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    po[i] = (uint32_t)(((t0 + i * 16 + c16) * a.ldp + g * 8) * 2);   // rows >= T read zeros
    ro[i] = (uint32_t)(((int64_t)(i * 16 + c16) * a.K + g * 8) * 2);  // rows >= kl read zeros
  }
  f32x4 acc[4][4];  // [j block][row block]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = kbeg + wave * 64; k0 < kend; k0 += 256) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t so = (uint32_t)((k0 + ks * 32) * 2);
      bf16x8 pf[4], rf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rp, po[i], so, 0));
        rf[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rr, ro[i], so, 0));
      }
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) acc[jb][rb] = mfma16s(rf[jb], pf[rb], acc[jb][rb]);
    }
  }
  if (wave > 0)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) red[wave - 1][jb][rb][lane] = acc[jb][rb];
  __syncthreads();
  if (wave != 0) return;
  // lane holds C[j = 16 jb + 4 g + i][t = t0 + 16 rb + c16]
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const int j = jb * 16 + g * 4;
    if (j >= a.kl) continue;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int64_t t = t0 + rb * 16 + c16;
      f32x4 v = acc[jb][rb];
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        const f32x4 q = red[w][jb][rb][lane];
        v = f32x4{v[0] + q[0], v[1] + q[1], v[2] + q[2], v[3] + q[3]};
      }
      if (t >= a.T) continue;
      if (DIRECT) *reinterpret_cast<u32x2*>(a.out + t * a.ldo + j) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
      else *reinterpret_cast<f32x4*>(a.part + ((int64_t)blockIdx.y * a.T + t) * a.kl + j) = v;
    }
  }
}

// out[t][j] = bf16(sum over splits in order); 4 values per thread
__global__ void nt_reduce_kernel(const float* __restrict__ part, int S, int64_t T, int kl, uint16_t* __restrict__ out,
                                 int64_t ldo) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= T * kl) return;
  const int64_t t = i / kl;
  const int j = (int)(i - t * kl);
  f32x4 v = *reinterpret_cast<const f32x4*>(part + i);
  for (int k = 1; k < S; ++k) {
    const f32x4 q = *reinterpret_cast<const f32x4*>(part + (int64_t)k * T * kl + i);
    v = f32x4{v[0] + q[0], v[1] + q[1], v[2] + q[2], v[3] + q[3]};
  }
  *reinterpret_cast<u32x2*>(out + t * ldo + j) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
}

// Masked transpose of B_full [K x r] for u = dy B: bt[j][k] = B[k][j % r] when
// j / r is the projection owning row k (else 0), j < kl. 8 k per thread.
__global__ void lora_bt_kernel(const uint16_t* __restrict__ b, int r, int kl, int64_t K, int nseg, SegEnds seg,
                               uint16_t* __restrict__ bt) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t kc = K / 8;
  if (idx >= kl * kc) return;
  const int j = (int)(idx / kc);
  const int64_t k = (idx - (int64_t)j * kc) * 8;
  int p = 0;
  while (p < nseg - 1 && k >= seg.e[p]) ++p;  // segment ends are multiples of 8
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (j / r == p) {
    const uint16_t* src = b + k * r + (j % r);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (uint32_t)src[(2 * e) * r] | ((uint32_t)src[(2 * e + 1) * r] << 16);
  }
  *reinterpret_cast<u32x4*>(bt + (int64_t)j * K + k) = u32x4{w[0], w[1], w[2], w[3]};
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
// BUF: the split's rows are read through buffer descriptors (its bytes below
// 4 GiB): no per-load bounds branches.
template <bool DIRECT, bool BUF>
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

  // thread -> P: 4 t-rows x 8 a-cols; Q: 2 t-rows x 8 j-cols. The global loads
  // run two 64-token steps ahead of the MFMAs, in two register sets. With BUF,
  // rows past the split's end read zeros (t_per_split is a multiple of 64, so
  // that happens only past T); columns past W or kl read neighbouring data or
  // zeros and feed only outputs that are never stored.
  const int pq = tid >> 4, po = tid & 15, qq = tid >> 3, qo = tid & 7;
  const int64_t ac = a0 + po * 8;
  // (unused without BUF)
  const __amdgpu_buffer_rsrc_t rsp = small_rsrc(a.p + tbeg * a.ldp, (tend - tbeg) * a.ldp * 2);
  const __amdgpu_buffer_rsrc_t rsq = small_rsrc(a.q + tbeg * a.ldq, (tend - tbeg) * a.ldq * 2);
  uint32_t pofs[4], qofs[2];
  if constexpr (BUF) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) pofs[rr] = (uint32_t)(((int64_t)(pq * 4 + rr) * a.ldp + ac) * 2);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) qofs[rr] = (uint32_t)(((int64_t)(qq * 2 + rr) * a.ldq + qo * 8) * 2);
  }
  auto gload = [&](int64_t tt, u32x4 (&rp)[4], u32x4 (&rq)[2]) {
    if constexpr (BUF) {
      const uint32_t op = (uint32_t)((tt - tbeg) * a.ldp * 2), oq = (uint32_t)((tt - tbeg) * a.ldq * 2);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        rp[rr] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsp, pofs[rr] + op, 0, 0));
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
        rq[rr] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsq, qofs[rr] + oq, 0, 0));
    } else {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int64_t t = tt + pq * 4 + rr;
        rp[rr] = (t < tend && ac < a.W) ? *reinterpret_cast<const u32x4*>(a.p + t * a.ldp + ac) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int64_t t = tt + qq * 2 + rr;
        rq[rr] = (t < tend && qo * 8 < a.kl) ? *reinterpret_cast<const u32x4*>(a.q + t * a.ldq + qo * 8)
                                             : u32x4{0, 0, 0, 0};
      }
    }
  };
  // one 64-token step from the register set (rp, rq), which is then refilled
  // with the step two ahead
  auto step = [&](int64_t tt, u32x4 (&rp)[4], u32x4 (&rq)[2]) {
    // (nothing of this step moves into the previous one, where it would wait for
    // loads that are still in flight)
    __builtin_amdgcn_sched_barrier(0);
    // both tiles stored transposed ([col][t])
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      uint32_t e[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) e[rr] = (cc & 1) ? (rp[rr][cc >> 1] >> 16) : (rp[rr][cc >> 1] & 0xFFFFu);
      *reinterpret_cast<u32x2*>(Ps + (po * 8 + cc) * SK_LDS + pq * 4) = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const uint32_t e0 = (cc & 1) ? (rq[0][cc >> 1] >> 16) : (rq[0][cc >> 1] & 0xFFFFu);
      const uint32_t e1 = (cc & 1) ? (rq[1][cc >> 1] >> 16) : (rq[1][cc >> 1] & 0xFFFFu);
      *reinterpret_cast<uint32_t*>(Qs + (qo * 8 + cc) * SK_LDS + qq * 2) = e0 | (e1 << 16);
    }
    __syncthreads();
    // unconditional, so that every step has the same loads in flight and each
    // wait covers only the older register set (past the split: zeros, unused)
    gload(tt + 128, rp, rq);
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
  };
  u32x4 rpa[4], rqa[2], rpb[4], rqb[2];
  gload(tbeg, rpa, rqa);
  __builtin_amdgcn_sched_barrier(0);  // the first set's loads stay the older ones
  gload(tbeg + 64, rpb, rqb);
  // pairs of steps with no branch between them (so the loads in flight are the
  // same on every path into a step), then an odd last step
  int64_t tt = tbeg;
  for (; tt + 64 < tend; tt += 128) {
    step(tt, rpa, rqa);
    step(tt + 64, rpb, rqb);
  }
  if (tt < tend) step(tt, rpa, rqa);
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
  if (tiles <= 0) return 1;  // empty output
  int64_t steps = (red + 63) / 64;
  int64_t s = (target_blocks + tiles - 1) / tiles;
  int64_t cap = steps / min_steps;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
}
constexpr int64_t TN_TARGET = 256, TN_MIN_STEPS = 4;

// NT splits: about NT_BLOCKS workgroups of 64 rows, each split at least
// NT_MIN_K of K (so that each of its four waves takes NT_MIN_K / 256 steps)
#ifndef LSL_NT_BLOCKS
#define LSL_NT_BLOCKS 256
#endif
#ifndef LSL_NT_MIN_K
#define LSL_NT_MIN_K 1024
#endif
static int nt_splits(int64_t T, int64_t K) {
  const int64_t tiles = (T + 63) / 64;
  if (tiles == 0) return 1;  // no tokens
  int64_t S = (LSL_NT_BLOCKS + tiles - 1) / tiles;
  if (S > K / LSL_NT_MIN_K) S = K / LSL_NT_MIN_K;
  return S < 1 ? 1 : (int)S;
}

// [masked B^T, kl <= 64 rows] + [S][T][kl] partials
size_t lora_nt_ws_bytes(int64_t T, int64_t K) {
  const int S = nt_splits(T, K);
  return align256((size_t)64 * K * 2) + (S > 1 ? (size_t)S * T * 64 * sizeof(float) : 0);
}

size_t lora_tn_ws_bytes(int64_t T, int64_t W) {
  int64_t tiles = (W + 127) / 128;
  int S = pick_splits(tiles, T, TN_TARGET, TN_MIN_STEPS);
  return S > 1 ? (size_t)S * W * 64 * sizeof(float) : 0;
}

lsl_status lora_nt_check(const LoraNt& d) {
  if (d.T == 0) return LSL_OK;
  if (d.K % 64 || d.kl <= 0 || d.kl > 64 || d.kl % 8)
    return set_error(LSL_ERR_UNSUPPORTED, "lora side product: K %% 64 and kl in [8, 64] multiple of 8 required");
  if ((d.T + 64) * d.ldp * 2 >= ((int64_t)1 << 32))
    return set_error(LSL_ERR_UNSUPPORTED, "lora side product: operand larger than 4 GiB");
  return LSL_OK;
}

lsl_status lora_tn_check(const LoraTn& d) {
  if (d.W == 0) return LSL_OK;
  if (d.kl <= 0 || d.kl > 64 || d.kl % 8 || d.W % 8)
    return set_error(LSL_ERR_UNSUPPORTED, "lora grad: kl in [8, 64] multiple of 8 and W %% 8 required");
  return LSL_OK;
}

lsl_status lora_nt_launch(const LoraNt& d, hipStream_t s) {
  if (d.T == 0) return LSL_OK;
  LSL_TRY(lora_nt_check(d));
  char* ws = (char*)d.ws;
  NtArgs a{};
  a.p = d.p; a.ldp = d.ldp; a.T = d.T; a.K = d.K; a.kl = d.kl; a.out = d.out; a.ldo = d.ldo;
  if (d.b_full) {
    uint16_t* bt = (uint16_t*)ws;
    SegEnds se;
    for (int i = 0; i < 4; ++i) se.e[i] = d.seg_end[i];
    const int64_t n = (int64_t)d.kl * (d.K / 8);
    hipLaunchKernelGGL(lora_bt_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, d.b_full, d.r, d.kl, d.K,
                       d.nseg, se, bt);
    a.rt = bt;
  } else {
    a.rt = d.a_full;
  }
  a.part = (float*)(ws + align256((size_t)64 * d.K * 2));
  const int64_t tiles = (d.T + 63) / 64;
  int S = nt_splits(d.T, d.K);
  const int64_t per = (d.K / S + 255) / 256 * 256;
  S = (int)((d.K + per - 1) / per);
  a.k_per_split = per;
  if (S == 1) {
    hipLaunchKernelGGL(lora_nt_kernel<true>, dim3((unsigned)tiles, 1), dim3(256), 0, s, a);
    return check_launch("lora_nt");
  }
  hipLaunchKernelGGL(lora_nt_kernel<false>, dim3((unsigned)tiles, (unsigned)S), dim3(256), 0, s, a);
  const int64_t n4 = d.T * d.kl / 4;
  hipLaunchKernelGGL(nt_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, (const float*)a.part, S,
                     d.T, d.kl, d.out, d.ldo);
  return check_launch("lora_nt");
}

lsl_status lora_tn_launch(const LoraTn& d, hipStream_t s) {
  if (d.W == 0) return LSL_OK;
  LSL_TRY(lora_tn_check(d));
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
  // buffer descriptors address a split's rows with 32-bit offsets
  const int64_t lim = (int64_t)1 << 32;
  // (the loads run up to two steps past a split's rows)
  const bool buf = (per + 192) * d.ldp * 2 < lim && (per + 192) * d.ldq * 2 < lim;
  if (S == 1) {
    if (buf) hipLaunchKernelGGL((lora_tn_kernel<true, true>), dim3((unsigned)tiles, 1), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((lora_tn_kernel<true, false>), dim3((unsigned)tiles, 1), dim3(256), 0, s, a);
    return check_launch("lora_tn");
  }
  if (buf) hipLaunchKernelGGL((lora_tn_kernel<false, true>), dim3((unsigned)tiles, (unsigned)S), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((lora_tn_kernel<false, false>), dim3((unsigned)tiles, (unsigned)S), dim3(256), 0, s, a);
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
