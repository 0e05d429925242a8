// LoRA GEMM family on gfx950 bf16 MFMA (v_mfma_f32_16x16x32_bf16).
//
//   C[m][n] = sum_k X[m][k] * Wt[n][k]  (+ s * sum_j L[m][j] * Lt[n][j])  (+ residual)
//
// X is a bf16 activation [M x K] (k contiguous). Wt is the frozen weight seen as
// [N x K]: either stored that way (forward, y = x W^T: layout NK) or stored
// [K x N] (input gradient, dx = dy W: layout KN). It is bf16 or NF4; NF4 codes
// are dequantised while the tile is staged into LDS, w = bf16(code * absmax)
// (QLoRA NormalFloat with blockwise absmax, block 64), so the dense bf16 weight
// never exists in HBM. The LoRA term is one extra short K-step on the same
// tiles: forward L = t = x A^T, Lt = B masked per fused projection; backward
// L = u = dy B, Lt = A^T. Accumulation is float32 in MFMA registers; the output
// is rounded to bf16 once (plus once more after a fused residual add).
//
// Tiling: 128(n) x 128(m) per workgroup of 4 waves, 64 x 64 per wave, K-step 64,
// LDS double-buffered with one barrier per K-step. The MFMA A operand is the
// weight tile (rows n) and the B operand the activation tile (rows m), so each
// lane's four accumulators are four consecutive n of one output row m and the
// epilogue writes 8-byte chunks. Workgroups are mapped so that each XCD (L2)
// owns a contiguous range of weight tiles and all m-tiles of each: a weight
// tile is fetched from HBM by one XCD only.
#include "common.h"
#include "gemm.h"
#include "nf4.h"

namespace lsl {

constexpr int BM = 128, BN = 128, BK = 64, LDSW = BK + 8;  // LDS row stride in elements
constexpr int NTHREADS = 256;

struct GemmKArgs {
  const uint16_t* x; int64_t ldx;
  const uint16_t* wb; const uint8_t* wq; const float* wa;
  int64_t M, N, K;
  const uint16_t* la; int64_t ldla; int kl;   // LoRA A-side [M x kl]
  const uint16_t* lb;                         // fwd: B_full [N x r]; bwd: A_full [kl x N]
  int r; int nseg; int64_t seg_end[4];
  float scale;
  uint16_t* y; int64_t ldy;
  const uint16_t* res; int64_t ldres;
  int tiles_m, tiles_n;
  float cb[16];
  // cross-entropy epilogues
  const int32_t* labels; const float* lse; const float* nvalid;
  float2* part; float* zlab;
  uint16_t* y2;              // low half of the hi + lo gradient pair
  float gscale; int ignore; int64_t vocab_off, vocab;
  float* out32; int64_t ldo32; int first;
  int64_t kwrap;             // KN operand: reduction index k reads weight row k mod kwrap
};

enum { EPI_BF16 = 0, EPI_LSE = 1, EPI_CEGRAD = 2, EPI_ACC32 = 3 };

template <int WFMT, bool KN>
struct WLoader;

// ---- activation / bf16-NK loader: 128 rows x 64 k; 4 x 16B per thread
struct RowLoader {
  u32x4 v[4];
  LSL_DEV void load(const uint16_t* __restrict__ base, int64_t ld, int64_t rows, int64_t r0, int64_t k0, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid + i * NTHREADS;
      int row = c >> 3, col = (c & 7) * 8;
      int64_t gr = r0 + row;
      v[i] = gr < rows ? *reinterpret_cast<const u32x4*>(base + gr * ld + k0 + col) : u32x4{0, 0, 0, 0};
    }
  }
  LSL_DEV void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid + i * NTHREADS;
      int row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(lds + row * LDSW + col) = v[i];
    }
  }
};

template <>
struct WLoader<LSL_WFMT_BF16, false> {
  RowLoader r;
  LSL_DEV void load(const GemmKArgs& a, int64_t n0, int64_t k0, int tid) { r.load(a.wb, a.K, a.N, n0, k0, tid); }
  LSL_DEV void store(uint16_t* lds, const float2*, int tid) const { r.store(lds, tid); }
};

// NF4 [N x K]: thread -> row tid/2, 32 consecutive k (16 code bytes)
template <>
struct WLoader<LSL_WFMT_NF4, false> {
  u32x4 c; float am;
  LSL_DEV void load(const GemmKArgs& a, int64_t n0, int64_t k0, int tid) {
    int row = tid >> 1, half = tid & 1;
    int64_t n = n0 + row;
    if (n < a.N) {
      c = *reinterpret_cast<const u32x4*>(a.wq + n * (a.K >> 1) + (k0 >> 1) + half * 16);
      am = a.wa[n * (a.K >> 6) + (k0 >> 6)];
    } else {
      c = u32x4{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
      am = 0.f;
    }
  }
  LSL_DEV void store(uint16_t* lds, const float2* lut, int tid) const {
    int row = tid >> 1, half = tid & 1;
    uint32_t o[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float2 cv = lut[(c[j >> 2] >> ((j & 3) * 8)) & 0xFF];
      o[j] = pack2(cv.x * am, cv.y * am);
    }
    u32x4* d = reinterpret_cast<u32x4*>(lds + row * LDSW + half * 32);
    d[0] = u32x4{o[0], o[1], o[2], o[3]};
    d[1] = u32x4{o[4], o[5], o[6], o[7]};
    d[2] = u32x4{o[8], o[9], o[10], o[11]};
    d[3] = u32x4{o[12], o[13], o[14], o[15]};
  }
};

// Transposing store shared by the KN loaders: vals[r][c] = element (kk = 4q + r, j = 8o + c)
LSL_DEV void store_transposed_4x8(uint16_t* lds, const uint32_t w[4][4], int tid) {
  int q = tid >> 4, o = tid & 15;
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    uint32_t e[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) e[rr] = (cc & 1) ? (w[rr][cc >> 1] >> 16) : (w[rr][cc >> 1] & 0xFFFFu);
    u32x2 v = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
    *reinterpret_cast<u32x2*>(lds + (o * 8 + cc) * LDSW + q * 4) = v;
  }
}

// bf16 stored [K x N] (row = reduction index): thread -> 4 k-rows x 8 n-cols
template <>
struct WLoader<LSL_WFMT_BF16, true> {
  uint32_t w[4][4];
  LSL_DEV void load(const GemmKArgs& a, int64_t n0, int64_t k0, int tid) {
    int q = tid >> 4, o = tid & 15;
    int64_t n = n0 + o * 8;
    if (a.kwrap) k0 %= a.kwrap;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      u32x4 v = n < a.N ? *reinterpret_cast<const u32x4*>(a.wb + (k0 + q * 4 + rr) * a.N + n) : u32x4{0, 0, 0, 0};
      w[rr][0] = v[0]; w[rr][1] = v[1]; w[rr][2] = v[2]; w[rr][3] = v[3];
    }
  }
  LSL_DEV void store(uint16_t* lds, const float2*, int tid) const { store_transposed_4x8(lds, w, tid); }
};

// NF4 stored [K x N]: thread -> 4 k-rows x 8 n-cols (4 code bytes + absmax per row)
template <>
struct WLoader<LSL_WFMT_NF4, true> {
  uint32_t c[4]; float am[4];
  LSL_DEV void load(const GemmKArgs& a, int64_t n0, int64_t k0, int tid) {
    int q = tid >> 4, o = tid & 15;
    int64_t n = n0 + o * 8;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      int64_t kk = k0 + q * 4 + rr;
      if (n < a.N) {
        c[rr] = *reinterpret_cast<const uint32_t*>(a.wq + kk * (a.N >> 1) + (n >> 1));
        am[rr] = a.wa[kk * (a.N >> 6) + (n >> 6)];
      } else {
        c[rr] = 0x77777777u; am[rr] = 0.f;
      }
    }
  }
  LSL_DEV void store(uint16_t* lds, const float2* lut, int tid) const {
    uint32_t w[4][4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float2 cv = lut[(c[rr] >> (8 * j)) & 0xFF];
        w[rr][j] = pack2(cv.x * am[rr], cv.y * am[rr]);
      }
    store_transposed_4x8(lds, w, tid);
  }
};

LSL_DEV f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One 64-deep K-step on LDS tiles: acc[ni][mi] += Wt-frag[ni] x X-frag[mi]
LSL_DEV void mma_tile(const uint16_t* Ws, const uint16_t* Xs, f32x4 acc[4][4], int wn, int wm, int lane, int ksteps) {
  for (int ks = 0; ks < ksteps; ++ks) {
    bf16x8 af[4], bfr[4];
    int kofs = ks * 32 + (lane >> 4) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = *reinterpret_cast<const bf16x8*>(Ws + (wn * 64 + i * 16 + (lane & 15)) * LDSW + kofs);
      bfr[i] = *reinterpret_cast<const bf16x8*>(Xs + (wm * 64 + i * 16 + (lane & 15)) * LDSW + kofs);
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) acc[ni][mi] = mfma16(af[ni], bfr[mi], acc[ni][mi]);
  }
}

// Tile index remap: XCD x (= workgroup id mod 8) gets a contiguous range of
// tiles, ordered m-fastest so that the tiles sharing a weight tile run together.
LSL_DEV void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  int nt = tiles_m * tiles_n;
  int b = blockIdx.x;
  int per = nt / 8;
  int t = b;
  if (b < per * 8) t = (b & 7) * per + (b >> 3);
  tn = t / tiles_m;
  tm = t - tn * tiles_m;
}

template <int WFMT, bool KN, int LORA, int EPI>
__global__ __launch_bounds__(NTHREADS, 2) void gemm_kernel(const GemmKArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN * LDSW];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][BM * LDSW];
  __shared__ float2 lut[WFMT == LSL_WFMT_NF4 ? 256 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  int tm, tn;
  tile_coords(a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  if constexpr (WFMT == LSL_WFMT_NF4) lut[tid] = make_float2(a.cb[tid >> 4], a.cb[tid & 15]);

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = (int)(a.K / BK);
  RowLoader xl;
  WLoader<WFMT, KN> wl;
  xl.load(a.x, a.ldx, a.M, m0, 0, tid);
  wl.load(a, n0, 0, tid);
  __syncthreads();  // lut visible
  xl.store(Xs[0], tid);
  wl.store(Ws[0], lut, tid);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      xl.load(a.x, a.ldx, a.M, m0, (int64_t)(kt + 1) * BK, tid);
      wl.load(a, n0, (int64_t)(kt + 1) * BK, tid);
    }
    mma_tile(Ws[cur], Xs[cur], acc, wn, wm, lane, 2);
    if (more) {
      xl.store(Xs[cur ^ 1], tid);
      wl.store(Ws[cur ^ 1], lut, tid);
    }
    __syncthreads();
  }

  // ---- LoRA K-step (kl <= 64, zero padded to 64) into separate accumulators
  if constexpr (LORA != 0) {
    uint16_t* Ls = Xs[0];
    uint16_t* Lt = Ws[0];
    // L side: [128 m x kl]
    for (int c = tid; c < BM * 8; c += NTHREADS) {
      int row = c >> 3, col = (c & 7) * 8;
      int64_t gm = m0 + row;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (gm < a.M && col < a.kl) v = *reinterpret_cast<const u32x4*>(a.la + gm * a.ldla + col);
      *reinterpret_cast<u32x4*>(Ls + row * LDSW + col) = v;
    }
    if constexpr (LORA == 1) {
      // Lt[n][j] = B[n][j % r] if j / r is the projection owning column n
      for (int c = tid; c < BN * 64; c += NTHREADS) {
        int row = c >> 6, j = c & 63;
        int64_t gn = n0 + row;
        uint16_t v = 0;
        if (gn < a.N && j < a.kl) {
          int seg = 0;
          while (seg < a.nseg - 1 && gn >= a.seg_end[seg]) ++seg;
          if (j / a.r == seg) v = a.lb[gn * a.r + (j % a.r)];
        }
        Lt[row * LDSW + j] = v;
      }
    } else {
      // Lt[n][j] = A_full[j][n]
      for (int c = tid; c < BN * 64; c += NTHREADS) {
        int j = c >> 7, row = c & 127;
        int64_t gn = n0 + row;
        uint16_t v = 0;
        if (gn < a.N && j < a.kl) v = a.lb[(int64_t)j * a.N + gn];
        Lt[row * LDSW + j] = v;
      }
    }
    __syncthreads();
    f32x4 lacc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) lacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    mma_tile(Lt, Ls, lacc, wn, wm, lane, (a.kl + 31) / 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] += a.scale * lacc[i][j][e];
  }

  // ---- epilogue: lane holds C[m][n..n+3]
  if constexpr (EPI == EPI_LSE) {
    // Cross-entropy forward: per token m, max and sum of exp over this tile's
    // vocabulary entries n < N, and the label's logit if it falls in the tile.
    float2* red = reinterpret_cast<float2*>(Xs[0]);  // [2 (wn)][128 (m)]
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int64_t m = m0 + wm * 64 + mi * 16 + (lane & 15);
      const int lab = m < a.M ? a.labels[m] : -1;
      float mx = -INFINITY;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int64_t n = n0 + wn * 64 + ni * 16 + (lane >> 4) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (n + e < a.N) {
            mx = fmaxf(mx, acc[ni][mi][e]);
            if (n + e == lab) a.zlab[m] = acc[ni][mi][e];
          }
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float sm = 0.f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int64_t n = n0 + wn * 64 + ni * 16 + (lane >> 4) * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < a.N) sm += expf(acc[ni][mi][e] - mx);
        }
      }
      sm += __shfl_xor(sm, 16, 64);
      sm += __shfl_xor(sm, 32, 64);
      if ((lane >> 4) == 0) red[wn * BM + wm * 64 + mi * 16 + (lane & 15)] = make_float2(mx, sm);
    }
    __syncthreads();
    if (tid < BM && m0 + tid < a.M) {
      float2 p0 = red[tid], p1 = red[BM + tid];
      float mx = fmaxf(p0.x, p1.x);
      float sm = 0.f;
      if (mx != -INFINITY) {
        if (p0.x != -INFINITY) sm += p0.y * expf(p0.x - mx);
        if (p1.x != -INFINITY) sm += p1.y * expf(p1.x - mx);
      }
      a.part[(int64_t)tn * a.M + m0 + tid] = make_float2(mx, sm);
    }
    return;
  }
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int64_t n = n0 + wn * 64 + ni * 16 + (lane >> 4) * 4;
    if (n >= a.N) continue;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int64_t m = m0 + wm * 64 + mi * 16 + (lane & 15);
      if (m >= a.M) continue;
      float v0 = acc[ni][mi][0], v1 = acc[ni][mi][1], v2 = acc[ni][mi][2], v3 = acc[ni][mi][3];
      if constexpr (EPI == EPI_CEGRAD) {
        // G = coef * (softmax - onehot) for this vocabulary chunk, as a hi + lo
        // pair of bf16 matrices (about 16 significant bits for the dH product)
        const int lab = a.labels[m];
        const float nv = *a.nvalid;
        const bool valid = lab != a.ignore && lab >= 0 && lab < a.vocab;
        const float coef = (valid && nv > 0.f) ? a.gscale / nv : 0.f;
        const float l = a.lse[m];
        const int64_t nl = n + a.vocab_off;
        float g[4] = {v0, v1, v2, v3};
#pragma unroll
        for (int e = 0; e < 4; ++e) g[e] = coef * (expf(g[e] - l) - (nl + e == lab ? 1.f : 0.f));
        const uint32_t h0 = pack2(g[0], g[1]), h1 = pack2(g[2], g[3]);
        *reinterpret_cast<u32x2*>(a.y + m * a.ldy + n) = u32x2{h0, h1};
        *reinterpret_cast<u32x2*>(a.y2 + m * a.ldy + n) =
            u32x2{pack2(g[0] - lo_bf(h0), g[1] - hi_bf(h0)), pack2(g[2] - lo_bf(h1), g[3] - hi_bf(h1))};
      } else if constexpr (EPI == EPI_ACC32) {
        float* o = a.out32 + m * a.ldo32 + n;
        f32x4 prev = a.first ? f32x4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f32x4*>(o);
        f32x4 r = f32x4{prev[0] + v0, prev[1] + v1, prev[2] + v2, prev[3] + v3};
        *reinterpret_cast<f32x4*>(o) = r;
        if (a.y) *reinterpret_cast<u32x2*>(a.y + m * a.ldy + n) = u32x2{pack2(r[0], r[1]), pack2(r[2], r[3])};
      } else {
        if (a.res) {
          u32x2 r = *reinterpret_cast<const u32x2*>(a.res + m * a.ldres + n);
          v0 = bf2f(f2bf(v0)) + lo_bf(r[0]);
          v1 = bf2f(f2bf(v1)) + hi_bf(r[0]);
          v2 = bf2f(f2bf(v2)) + lo_bf(r[1]);
          v3 = bf2f(f2bf(v3)) + hi_bf(r[1]);
        }
        *reinterpret_cast<u32x2*>(a.y + m * a.ldy + n) = u32x2{pack2(v0, v1), pack2(v2, v3)};
      }
    }
  }
}

template <int WFMT, bool KN>
static void launch_lora_variant(const GemmKArgs& a, int lora, hipStream_t s, dim3 grid) {
  if (lora == 0) hipLaunchKernelGGL((gemm_kernel<WFMT, KN, 0, EPI_BF16>), grid, dim3(NTHREADS), 0, s, a);
  else if (lora == 1) hipLaunchKernelGGL((gemm_kernel<WFMT, KN, 1, EPI_BF16>), grid, dim3(NTHREADS), 0, s, a);
  else hipLaunchKernelGGL((gemm_kernel<WFMT, KN, 2, EPI_BF16>), grid, dim3(NTHREADS), 0, s, a);
}

lsl_status gemm_launch(const GemmDesc& d, hipStream_t s) {
  if (d.M == 0 || d.N == 0) return LSL_OK;
  if (d.K % BK || d.N % 8)
    return set_error(LSL_ERR_UNSUPPORTED, "gemm: K (%lld) must be a multiple of 64 and N (%lld) of 8",
                     (long long)d.K, (long long)d.N);
  if (d.lora && (d.kl <= 0 || d.kl > 64 || d.kl % 8))
    return set_error(LSL_ERR_UNSUPPORTED, "gemm: LoRA width %d must be a multiple of 8 in [8, 64]", d.kl);
  if (d.wfmt == LSL_WFMT_NF4 && d.kn && d.N % 64)
    return set_error(LSL_ERR_UNSUPPORTED, "gemm: NF4 transposed operand needs N %% 64 == 0");
  GemmKArgs a{};
  a.x = d.x; a.ldx = d.ldx;
  a.wb = d.wb; a.wq = d.wq; a.wa = d.wa;
  a.M = d.M; a.N = d.N; a.K = d.K;
  a.la = d.la; a.ldla = d.ldla; a.kl = d.kl; a.lb = d.lb; a.r = d.r; a.nseg = d.nseg;
  for (int i = 0; i < 4; ++i) a.seg_end[i] = d.seg_end[i];
  a.scale = d.scale;
  a.y = d.y; a.ldy = d.ldy; a.res = d.res; a.ldres = d.ldres;
  a.tiles_m = (int)((d.M + BM - 1) / BM);
  a.tiles_n = (int)((d.N + BN - 1) / BN);
  const Nf4Table& t = nf4_table();
  for (int i = 0; i < 16; ++i) a.cb[i] = t.cb[i];
  a.labels = d.labels; a.lse = d.lse; a.nvalid = d.nvalid; a.part = (float2*)d.part; a.zlab = d.zlab;
  a.y2 = d.y2; a.gscale = d.gscale; a.ignore = d.ignore; a.vocab_off = d.vocab_off; a.vocab = d.vocab;
  a.out32 = d.out32; a.ldo32 = d.ldo32; a.first = d.first; a.kwrap = d.kwrap;
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n));
  if (d.epi != EPI_BF16) {
    if (d.wfmt != LSL_WFMT_BF16 || d.lora) return set_error(LSL_ERR_UNSUPPORTED, "gemm: CE epilogues take a bf16 weight");
    if (d.epi == EPI_LSE && !d.kn) hipLaunchKernelGGL((gemm_kernel<LSL_WFMT_BF16, false, 0, EPI_LSE>), grid, dim3(NTHREADS), 0, s, a);
    else if (d.epi == EPI_CEGRAD && !d.kn) hipLaunchKernelGGL((gemm_kernel<LSL_WFMT_BF16, false, 0, EPI_CEGRAD>), grid, dim3(NTHREADS), 0, s, a);
    else if (d.epi == EPI_ACC32 && d.kn) hipLaunchKernelGGL((gemm_kernel<LSL_WFMT_BF16, true, 0, EPI_ACC32>), grid, dim3(NTHREADS), 0, s, a);
    else return set_error(LSL_ERR_UNSUPPORTED, "gemm: epilogue %d with layout %d", d.epi, (int)d.kn);
    return check_launch("gemm(ce)");
  }
  if (d.wfmt == LSL_WFMT_NF4) {
    if (d.kn) launch_lora_variant<LSL_WFMT_NF4, true>(a, d.lora, s, grid);
    else launch_lora_variant<LSL_WFMT_NF4, false>(a, d.lora, s, grid);
  } else {
    if (d.kn) launch_lora_variant<LSL_WFMT_BF16, true>(a, d.lora, s, grid);
    else launch_lora_variant<LSL_WFMT_BF16, false>(a, d.lora, s, grid);
  }
  return check_launch("gemm");
}

}  // namespace lsl
