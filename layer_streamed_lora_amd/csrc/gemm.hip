// LoRA GEMM family on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
//   C[m][n] = sum_k X[m][k] * Wt[n][k]  (+ s * sum_j L[m][j] * Lt[n][j])  (+ residual)
//
// X is a bf16 activation [M x K] (k contiguous). Wt is the frozen weight seen as
// [N x K]: either stored that way (forward, y = x W^T: layout NK) or stored
// [K x N] (input gradient, dx = dy W: layout KN). It is bf16 or NF4; NF4 codes
// are dequantised while the tile is staged into LDS, w = bf16(code * absmax)
// (QLoRA NormalFloat with blockwise absmax, block 64; the absmax itself is
// float32, or 8-bit codes times a float32 constant per 256 blocks), so the
// dense bf16 weight never exists in HBM. The LoRA term is one extra short K-step on the same
// tiles: forward L = t = x A^T, Lt = B masked per fused projection; backward
// L = u = dy B, Lt = A^T. Accumulation is float32 in MFMA registers; the output
// is rounded to bf16 once (plus once more after a fused residual add).
//
// Tiling: BN (weight rows) x BM (tokens) per workgroup of 4 waves; a wave owns
// 64 weight rows x BM/(4*64/BN) tokens, K-step 64; the next tile's global loads
// are issued into registers before the current tile's MFMAs and stored to LDS
// after them. The token tile is stored unpadded with a chunk swizzle, so its
// stores and the MFMA operand reads are free of bank conflicts. GEMMs with few
// output tiles split the reduction (float32 partials added in split order). The MFMA A operand is the weight tile
// and the B operand the token tile, so each lane's four accumulators are four
// consecutive n of one output row m and the epilogue writes 8-byte chunks.
// Loader addresses are set up once; a K-step only adds a uniform offset.
// NF4 dequantisation cost per weight is amortised over the BM tokens of the
// tile. Workgroups are mapped so that each XCD (L2) owns a contiguous range of
// weight tiles and all token tiles of each: a weight tile is fetched from HBM
// by one XCD only. The tile shape is a function of (M, N) only.
#include "common.h"
#include "gemm.h"
#include "nf4.h"
#include "api_util.h"

namespace lsl {

constexpr int BK = 64, LDSW = BK + 8;  // LDS row stride in elements
constexpr int NTHREADS = 256;
// at least two workgroups per CU: keeps each wave within 168 registers, so three
// workgroups (12 waves) fit on a CU, which hides the staging latency better
#ifndef LSL_GEMM_MINB
#define LSL_GEMM_MINB 2
#endif

struct GemmKArgs {
  const uint16_t* x; int64_t ldx;
  const uint16_t* wb; const uint8_t* wq; const float* wa;
  const uint8_t* wq8; const float* wsc;  // NF4DQ: 8-bit absmax codes, float32 block constants
  int64_t M, N, K;
  const uint16_t* la; int64_t ldla; int kl;   // LoRA A-side [M x kl]
  const uint16_t* lb;                         // fwd: B_full [N x r]; bwd: A_full [kl x N]
  int r; int nseg; int64_t seg_end[4];
  float scale;
  uint16_t* y; int64_t ldy;
  const uint16_t* res; int64_t ldres;
  const uint16_t* bias;      // bf16 [N] or NULL
  int tiles_m, tiles_n;
  float cb[16];
  // cross-entropy epilogues
  const int32_t* labels; const float* lse; const float* nvalid;
  float2* part; float* zlab;
  uint16_t* y2;              // low half of the hi + lo gradient pair
  float gscale; int ignore; int64_t vocab_off, vocab;
  float* out32; int64_t ldo32; int first; int64_t o32_split;  // split s accumulates at out32 + s o32_split
  int64_t kwrap;             // KN operand: reduction index k reads weight row k mod kwrap (K <= 2 kwrap)
  int ksplit; int kt_per_split;  // split-K: workgroup b takes split b / (tiles_m tiles_n)
  float* spart;                  // float32 partials [ksplit][M][N]; stream-K: tile slots
  int sk_g;                      // stream-K (large tile): number of workgroups, 0 when off
  unsigned* cnt;                 // stream-K: per-tile arrival counts (zero between launches)
};

enum { EPI_BF16 = 0, EPI_LSE = 1, EPI_CEGRAD = 2, EPI_ACC32 = 3 };

// 2 x bf16 halves: (lo of a, lo of b) and (hi of a, hi of b)
LSL_DEV uint32_t lo_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
LSL_DEV uint32_t hi_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Buffer resource over [base, base + bytes): loads whose per-lane (vector)
// offset is at or past the end return zeros, so partial tiles need no branches.
// The scalar offset of a buffer load is not part of that range check, so every
// loader keeps whatever can run past the end (rows past M or N, columns past N)
// in the vector offset and starts the descriptor at the uniform part of the
// address instead. The fourth descriptor word is the gfx9 raw-buffer format.
LSL_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
LSL_DEV u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
LSL_DEV u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}
LSL_DEV uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Chunk swizzle of the unpadded token tile (8 chunks of 16 B per 128-B row).
LSL_DEV int xswz(int r) { return (r ^ (r >> 3)) & 7; }

// ---- row-major bf16 tile loader: ROWS rows x 64 k, 16 B chunks, 8 chunks per
// row; thread -> rows tid/8 + 32 i. Chunk i reads through a descriptor that
// starts 32 i rows further on (and ends with the matrix), so the one per-lane
// offset covers every chunk and a row at or past `rows` reads zeros; per K-step
// only the scalar offset (the column k0) changes.
template <int ROWS>
struct RowLoader {
  static constexpr int CH = ROWS / 32;
  uint32_t voff;
  u32x4 v[CH];
  LSL_DEV void init(int64_t ld, int64_t r0, int tid) {
    voff = (uint32_t)(((r0 + (tid >> 3)) * ld + (tid & 7) * 8) * 2);
  }
  // base/ld/rows come straight from the kernel arguments, so the descriptors are uniform
  LSL_DEV void load(const uint16_t* base, int64_t ld, int64_t rows, int64_t k0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t left = rows - 32 * i;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + 32 * i * ld, left > 0 ? left * ld * 2 : 0);
      v[i] = bload16(rs, voff, (uint32_t)(k0 * 2));
    }
  }
  LSL_DEV void store(uint16_t* lds, int tid) const {
    const int r = tid >> 3, c = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < CH; ++i) *reinterpret_cast<u32x4*>(lds + (r + 32 * i) * LDSW + c) = v[i];
  }
  // unpadded [ROWS][64] layout, chunk c of row r at position c ^ xswz(r): each
  // wave store fills 8 whole rows (1 KB, no bank conflicts) and the 32-row MFMA
  // operand reads spread over all banks
  LSL_DEV void store_swz(uint16_t* lds, int tid) const {
    const int r = tid >> 3, c = tid & 7;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int row = r + 32 * i;
      *reinterpret_cast<u32x4*>(lds + row * 64 + 8 * (c ^ xswz(row))) = v[i];
    }
  }
};

template <int WFMT, bool KN, int BN>
struct WLoader;

template <int BN>
struct WLoader<LSL_WFMT_BF16, false, BN> {
  RowLoader<BN> r;
  LSL_DEV void init(const GemmKArgs& a, int64_t n0, int tid) { r.init(a.K, n0, tid); }
  LSL_DEV void load(const GemmKArgs& a, int64_t k0) { r.load(a.wb, a.K, a.N, k0); }
  LSL_DEV void store(uint16_t* lds, const float*, int tid) const { r.store(lds, tid); }
};

// NF4 [N x K]: each of the BN rows has 32 code bytes per K-step; TPR threads per
// row, BPT bytes (2 BPT weights) each. Rows past N are clamped to the last row:
// their outputs are never stored.
// absmax of NF4 block idx (flattened row-major): float32, or (NF4DQ) q * s
template <int WFMT>
LSL_DEV float block_absmax(const GemmKArgs& a, int64_t idx) {
  if constexpr (WFMT == LSL_WFMT_NF4DQ) return (float)a.wq8[idx] * a.wsc[idx >> 8];
  else return a.wa[idx];
}

template <int WFMT, int BN>
struct Nf4NkLoader {
  static constexpr int TPR = 256 / BN, BPT = 32 / TPR;
  const uint8_t* pc;
  int64_t ai;  // absmax index of the row's first block
  uint32_t c[BPT / 4];
  float am;
  LSL_DEV void init(const GemmKArgs& a, int64_t n0, int tid) {
    const int row = tid / TPR, part = tid % TPR;
    const int64_t n = n0 + row < a.N ? n0 + row : a.N - 1;
    pc = a.wq + n * (a.K >> 1) + part * BPT;
    ai = n * (a.K >> 6);
  }
  LSL_DEV void load(const GemmKArgs& a, int64_t k0) {
    if constexpr (BPT == 16) {
      u32x4 v = *reinterpret_cast<const u32x4*>(pc + (k0 >> 1));
      c[0] = v[0]; c[1] = v[1]; c[2] = v[2]; c[3] = v[3];
    } else {
      u32x2 v = *reinterpret_cast<const u32x2*>(pc + (k0 >> 1));
      c[0] = v[0]; c[1] = v[1];
    }
    am = block_absmax<WFMT>(a, ai + (k0 >> 6));
  }
  LSL_DEV void store(uint16_t* lds, const float* lut, int tid) const {
    const int row = tid / TPR, part = tid % TPR;
    uint32_t o[BPT];
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const uint32_t b = c[j >> 2] >> ((j & 3) * 8);  // element 2j in the high nibble
      o[j] = pack2(lut[(b >> 4) & 15] * am, lut[b & 15] * am);
    }
    u32x4* d = reinterpret_cast<u32x4*>(lds + row * LDSW + part * 2 * BPT);
#pragma unroll
    for (int i = 0; i < BPT / 4; ++i) d[i] = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
  }
};
template <int BN>
struct WLoader<LSL_WFMT_NF4, false, BN> : Nf4NkLoader<LSL_WFMT_NF4, BN> {};
template <int BN>
struct WLoader<LSL_WFMT_NF4DQ, false, BN> : Nf4NkLoader<LSL_WFMT_NF4DQ, BN> {};

// The [K x N] weight tile of this kernel in LDS: [64 k][64 n], rows unpadded,
// the 8-column chunk c of row r at chunk position c ^ kn64_swz(r). A
// transposing read (4 rows x 4 chunks per 32 lanes, rows r0 .. r0 + 3 with r0
// a multiple of 4, and rows r0 + 8 .. in the other half-wave) then touches 16
// distinct 16-byte bank groups, and so does each loader store below (16 lanes:
// the 8 chunks of an even and of an odd row).
LSL_DEV int kn64_swz(int r) { return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1); }
LSL_DEV int kn64_pos(int r, int c) { return r * 64 + 8 * (c ^ kn64_swz(r)); }

// bf16 stored [K x N] (row = reduction index): thread -> rows tid / 8 and
// tid / 8 + 32, columns 8 (tid % 8) .. + 7. Columns past N read zeros or
// neighbouring data; their outputs are never stored.
template <int BN>
struct WLoader<LSL_WFMT_BF16, true, BN> {
  static_assert(BN == 64, "the [K x N] tile layout is 64 columns wide");
  uint32_t voff[2];
  uint32_t w[2][4];
  LSL_DEV void init(const GemmKArgs& a, int64_t n0, int tid) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
      voff[rr] = (uint32_t)(((int64_t)((tid >> 3) + 32 * rr) * a.N + n0 + (tid & 7) * 8) * 2);
  }
  LSL_DEV void load(const GemmKArgs& a, int64_t k0) {
    const int64_t rows = a.kwrap ? a.kwrap : a.K;
    if (a.kwrap && k0 >= a.kwrap) k0 -= a.kwrap;  // K <= 2 kwrap (checked on the host)
    // descriptor from row k0 to the end of the matrix: the row and column offset
    // (in the vector offset) is range-checked
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.wb + k0 * a.N, (rows - k0) * a.N * 2);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      u32x4 v = bload16(rs, voff[rr], 0);
      w[rr][0] = v[0]; w[rr][1] = v[1]; w[rr][2] = v[2]; w[rr][3] = v[3];
    }
  }
  LSL_DEV void store(uint16_t* lds, const float*, int tid) const {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
      *reinterpret_cast<u32x4*>(lds + kn64_pos((tid >> 3) + 32 * rr, tid & 7)) =
          u32x4{w[rr][0], w[rr][1], w[rr][2], w[rr][3]};
  }
};

// NF4 stored [K x N]: thread -> rows tid / 8 and tid / 8 + 32, columns
// 8 (tid % 8) .. + 7 (4 code bytes and the absmax of each row); column groups
// past N are clamped to the last group (outputs not stored).
template <int WFMT, int BN>
struct Nf4KnLoader {
  static_assert(BN == 64, "the [K x N] tile layout is 64 columns wide");
  const uint8_t* pc;
  int64_t ai;  // absmax index of this thread's first row and column block
  int64_t rowc, rowa;
  uint32_t c[2];
  float am[2];
  LSL_DEV void init(const GemmKArgs& a, int64_t n0, int tid) {
    const int64_t n = n0 + (tid & 7) * 8 < a.N ? n0 + (tid & 7) * 8 : a.N - 8;
    rowc = a.N >> 1;
    rowa = a.N >> 6;
    pc = a.wq + (int64_t)(tid >> 3) * rowc + (n >> 1);
    ai = (int64_t)(tid >> 3) * rowa + (n >> 6);
  }
  LSL_DEV void load(const GemmKArgs& a, int64_t k0) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      c[rr] = *reinterpret_cast<const uint32_t*>(pc + (k0 + 32 * rr) * rowc);
      am[rr] = block_absmax<WFMT>(a, ai + (k0 + 32 * rr) * rowa);
    }
  }
  LSL_DEV void store(uint16_t* lds, const float* lut, int tid) const {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t b = c[rr] >> (8 * j);  // element 2j in the high nibble
        w[j] = pack2(lut[(b >> 4) & 15] * am[rr], lut[b & 15] * am[rr]);
      }
      *reinterpret_cast<u32x4*>(lds + kn64_pos((tid >> 3) + 32 * rr, tid & 7)) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
};
template <int BN>
struct WLoader<LSL_WFMT_NF4, true, BN> : Nf4KnLoader<LSL_WFMT_NF4, BN> {};
template <int BN>
struct WLoader<LSL_WFMT_NF4DQ, true, BN> : Nf4KnLoader<LSL_WFMT_NF4DQ, BN> {};

// 32 x 32 x 16 bf16 MFMA (on gfx950 twice the throughput of 16 x 16 x 32). Lane l
// holds A[l % 32][8 (l / 32) .. +7] and B[8 (l / 32) .. +7][l % 32]; accumulator
// element i is C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
LSL_DEV f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Tile geometry: WN x WM waves, each 64 (n) x WTM (m): 2 x MI blocks of 32 x 32.
template <int BN, int BM>
struct Geo {
  static constexpr int WN = BN / 64, WM = 4 / WN, WTM = BM / WM, MI = WTM / 32;
};

// ksteps x 16-deep MFMA steps on LDS tiles: acc[ni][mi] += Wt-block[ni] x X-block[mi].
// TRW: the weight tile is the swizzled [64 k][64 n] layout (kn64_pos) and read
// with transposing LDS reads (natural k order, so the token tile is unchanged).
// XSW: the token tile is the unpadded, swizzled [BM][64] layout (else [BM][LDSW]).
template <int MI, bool TRW = false, bool XSW = false>
LSL_DEV void mma_tile(const uint16_t* Ws, const uint16_t* Xs, f32x16 (&acc)[2][MI], int wn, int wm0, int lane,
                      int ksteps) {
  const int h8 = (lane >> 5) * 8, r32 = lane & 31;
  for (int ks = 0; ks < ksteps; ++ks) {
    const int kofs = ks * 16 + h8;
    bf16x8 af[2], bfr[MI];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (TRW) {
        // lanes 16-31 / 48-63 take columns 16..31 of the block; each 16-lane group
        // reads rows kofs .. kofs + 3 and kofs + 4 .. kofs + 7 of its 16 columns:
        // lane j gets row kofs + j / 4, columns 4 (j % 4) .. + 3 (half of a chunk)
        const int j = lane & 15, r = kofs + (j >> 2);
        const int c = wn * 8 + i * 4 + 2 * ((lane >> 4) & 1) + ((j & 3) >> 1), e = 4 * (j & 1);
        const u32x2 x = ld_tr4(Ws + kn64_pos(r, c) + e), y = ld_tr4(Ws + kn64_pos(r + 4, c) + e);
        af[i] = __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], y[0], y[1]});
      } else {
        af[i] = *reinterpret_cast<const bf16x8*>(Ws + (wn * 64 + i * 32 + r32) * LDSW + kofs);
      }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = wm0 + i * 32 + r32;
      if constexpr (XSW)
        bfr[i] = *reinterpret_cast<const bf16x8*>(Xs + row * 64 + 8 * ((2 * ks + (lane >> 5)) ^ xswz(row)));
      else
        bfr[i] = *reinterpret_cast<const bf16x8*>(Xs + row * LDSW + kofs);
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[ni][mi] = mfma32(af[ni], bfr[mi], acc[ni][mi]);
  }
}

// Tile index remap: XCD x (= workgroup id mod 8) gets a contiguous range of
// tiles. The tiles go in groups of GROUP_M token tiles: within a group
// m-fastest, so that the tiles sharing a weight tile run together, and group by
// group, so that the token rows in use (GROUP_M x BM rows, re-read by every
// weight tile) stay in L2/MALL however many tokens there are.
#ifndef LSL_GROUP_M
#define LSL_GROUP_M 2
#endif
LSL_DEV void tile_coords(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  int nt = tiles_m * tiles_n;
  int per = nt / 8;
  int t = b;
  if (b < per * 8) t = (b & 7) * per + (b >> 3);
  const int g = t / (LSL_GROUP_M * tiles_n);            // group of token tiles
  const int gm = min(LSL_GROUP_M, tiles_m - g * LSL_GROUP_M);
  const int i = t - g * LSL_GROUP_M * tiles_n;
  tn = i / gm;
  tm = g * LSL_GROUP_M + (i - tn * gm);
}

// y[m][n .. n + 3] = bf16(v (+ bias)) (+ residual, rounded again)
LSL_DEV void store_bf16x4(const GemmKArgs& a, int64_t m, int64_t n, float v0, float v1, float v2, float v3) {
  if (a.bias) {
    const u32x2 b = *reinterpret_cast<const u32x2*>(a.bias + n);
    v0 += lo_bf(b[0]); v1 += hi_bf(b[0]); v2 += lo_bf(b[1]); v3 += hi_bf(b[1]);
  }
  if (a.res) {
    u32x2 r = *reinterpret_cast<const u32x2*>(a.res + m * a.ldres + n);
    v0 = bf2f(f2bf(v0)) + lo_bf(r[0]);
    v1 = bf2f(f2bf(v1)) + hi_bf(r[0]);
    v2 = bf2f(f2bf(v2)) + lo_bf(r[1]);
    v3 = bf2f(f2bf(v3)) + hi_bf(r[1]);
  }
  *reinterpret_cast<u32x2*>(a.y + m * a.ldy + n) = u32x2{pack2(v0, v1), pack2(v2, v3)};
}

// Cross-entropy gradient for C[m][n .. n + 3] (logits of one vocabulary chunk):
// G = coef * (softmax - onehot), as a hi + lo pair of bf16 matrices (about 16
// significant bits for the dH product; the lo part only when y2 is set)
LSL_DEV void ce_grad4(const GemmKArgs& a, int64_t m, int64_t n, float v0, float v1, float v2, float v3) {
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
  if (a.y2)
    *reinterpret_cast<u32x2*>(a.y2 + m * a.ldy + n) =
        u32x2{pack2(g[0] - lo_bf(h0), g[1] - hi_bf(h0)), pack2(g[2] - lo_bf(h1), g[3] - hi_bf(h1))};
}

// float32 accumulation into split `split`'s partial sum (first: overwrite), with
// a bf16 copy of the sum when y is set
LSL_DEV void acc32_4(const GemmKArgs& a, int split, int64_t m, int64_t n, float v0, float v1, float v2, float v3) {
  float* o = a.out32 + split * a.o32_split + m * a.ldo32 + n;
  const f32x4 prev = a.first ? f32x4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f32x4*>(o);
  const f32x4 r = f32x4{prev[0] + v0, prev[1] + v1, prev[2] + v2, prev[3] + v3};
  *reinterpret_cast<f32x4*>(o) = r;
  if (a.y) *reinterpret_cast<u32x2*>(a.y + m * a.ldy + n) = u32x2{pack2(r[0], r[1]), pack2(r[2], r[3])};
}

// Cross-entropy forward, per token row of a tile: the row's max and sum of exp
// over the lane's logits (columns n < N; the label's logit is recorded where it
// falls), combined over the two lane halves holding the row. acc[ni][mi]
// element i is column nb + 32 ni + 8 (i / 4) + i % 4 of row mb + 32 mi.
template <int NI, int MI>
LSL_DEV void lse_rows(const GemmKArgs& a, const f32x16 (&acc)[NI][MI], int64_t mb, int64_t nb, float2 (&res)[MI]) {
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int64_t m = mb + mi * 32;
    const int lab = m < a.M ? a.labels[m] : -1;
    float mx = -INFINITY;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t n = nb + ni * 32 + 8 * (i >> 2) + (i & 3);
        if (n < a.N) {
          mx = fmaxf(mx, acc[ni][mi][i]);
          if (n == lab) a.zlab[m] = acc[ni][mi][i];
        }
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float sm = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t n = nb + ni * 32 + 8 * (i >> 2) + (i & 3);
          if (n < a.N) sm += expf(acc[ni][mi][i] - mx);
        }
    }
    sm += __shfl_xor(sm, 32, 64);
    res[mi] = make_float2(mx, sm);
  }
}

// (max, sum of exp) pairs of nw partial rows combined into one, in index order
LSL_DEV float2 lse_combine(const float2* p, int nw, int stride) {
  float mx = -INFINITY;
  for (int w = 0; w < nw; ++w) mx = fmaxf(mx, p[w * stride].x);
  float sm = 0.f;
  if (mx != -INFINITY)
    for (int w = 0; w < nw; ++w) {
      const float2 q = p[w * stride];
      if (q.x != -INFINITY) sm += q.y * expf(q.x - mx);
    }
  return make_float2(mx, sm);
}

// split-K: the float32 partial of this split (gemm_split_reduce adds the splits).
// Block (ni, mi), q < 4: the lane holds C[m][n .. n + 3], m = mb + 32 mi, n = nb + 32 ni + 8 q.
template <int MI>
LSL_DEV void store_split_partials(const GemmKArgs& a, const f32x16 (&acc)[2][MI], int64_t mb, int64_t nb, int split) {
  float* dst = a.spart + (int64_t)split * a.M * a.N;
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int64_t m = mb + mi * 32;
      if (m >= a.M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = nb + ni * 32 + 8 * q;
        if (n < a.N)
          *reinterpret_cast<f32x4*>(dst + m * a.N + n) =
              f32x4{acc[ni][mi][4 * q], acc[ni][mi][4 * q + 1], acc[ni][mi][4 * q + 2], acc[ni][mi][4 * q + 3]};
      }
    }
}

// segment (fused projection) owning output column n
LSL_DEV int lora_seg(const GemmKArgs& a, int64_t n) {
  int seg = 0;
  while (seg < a.nseg - 1 && n >= a.seg_end[seg]) ++seg;
  return seg;
}

// LoRA K-step operands in LDS ([rows][LDSW], k zero padded to 64): Ls = the
// A-side rows m0.. of la; Lt[n][j] = B[n][j % r] if j / r is the projection
// owning column n (LORA 1, forward), or A_full[j][n] (LORA 2, input gradient).
// Every operand moves in 16-byte chunks (kl and r are multiples of 8, so a chunk
// never straddles a projection), all of a thread's loads issued before its stores.
template <int LORA, int BN, int BM>
LSL_DEV void lora_stage(const GemmKArgs& a, uint16_t* Ls, uint16_t* Lt, int64_t m0, int64_t n0, int tid) {
  constexpr int LC = BM * 8 / NTHREADS;  // Ls chunks per thread
  u32x4 lv[LC];
#pragma unroll
  for (int i = 0; i < LC; ++i) {
    const int c = tid + i * NTHREADS, row = c >> 3, col = (c & 7) * 8;
    const int64_t gm = m0 + row;
    lv[i] = (gm < a.M && col < a.kl) ? *reinterpret_cast<const u32x4*>(a.la + gm * a.ldla + col) : u32x4{0, 0, 0, 0};
  }
  constexpr int TC = BN * 8 / NTHREADS;  // Lt chunks per thread
  u32x4 tv[TC];
  if constexpr (LORA == 1) {
    // thread -> row tid / (8 / TC), chunks TC (tid % (8 / TC)) .. + TC - 1
    const int row = tid / (8 / TC), c0 = (tid % (8 / TC)) * TC;
    const int64_t gn = n0 + row;
    const int seg = gn < a.N ? lora_seg(a, gn) : -1;
#pragma unroll
    for (int q = 0; q < TC; ++q) {
      const int j0 = (c0 + q) * 8;
      tv[q] = (seg >= 0 && j0 < a.kl && j0 / a.r == seg)
                  ? *reinterpret_cast<const u32x4*>(a.lb + gn * a.r + (j0 - seg * a.r))
                  : u32x4{0, 0, 0, 0};
    }
  } else {
    // thread -> reduction row j = c / (BN / 8), columns 8 (c % (BN / 8)) .. + 7 of A_full
#pragma unroll
    for (int q = 0; q < TC; ++q) {
      const int c = tid + q * NTHREADS, j = c / (BN / 8), nc = (c % (BN / 8)) * 8;
      const int64_t gn = n0 + nc;
      tv[q] = (j < a.kl && gn < a.N) ? *reinterpret_cast<const u32x4*>(a.lb + (int64_t)j * a.N + gn)
                                     : u32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int i = 0; i < LC; ++i) {
    const int c = tid + i * NTHREADS, row = c >> 3, col = (c & 7) * 8;
    *reinterpret_cast<u32x4*>(Ls + row * LDSW + col) = lv[i];
  }
  if constexpr (LORA == 1) {
    const int row = tid / (8 / TC), c0 = (tid % (8 / TC)) * TC;
#pragma unroll
    for (int q = 0; q < TC; ++q) *reinterpret_cast<u32x4*>(Lt + row * LDSW + (c0 + q) * 8) = tv[q];
  } else {
#pragma unroll
    for (int q = 0; q < TC; ++q) {  // transposed: Lt[n][j], eight 2-byte stores
      const int c = tid + q * NTHREADS, j = c / (BN / 8), nc = (c % (BN / 8)) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        Lt[(nc + e) * LDSW + j] = (uint16_t)((e & 1) ? (tv[q][e >> 1] >> 16) : (tv[q][e >> 1] & 0xFFFFu));
    }
  }
}

template <int WFMT, bool KN, int LORA, int EPI, int BN, int BM>
__global__ __launch_bounds__(NTHREADS, LSL_GEMM_MINB) void gemm_kernel(const GemmKArgs a) {
  using G = Geo<BN, BM>;
  constexpr int MI = G::MI;
  // weight tile: [BN][LDSW] (NK), or the swizzled [BK][64] layout read
  // transposed (KN); the LoRA step reuses it as [BN][LDSW]. Token tile:
  // swizzled [BM][64] (the LoRA step: [BM][LDSW]).
  constexpr int WSZ = BN * LDSW > BK * (BN + 32) ? BN * LDSW : BK * (BN + 32);
  __shared__ __attribute__((aligned(16))) uint16_t Ws[WSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[BM * LDSW];
  // NF4 codebook: 16 floats, so every lookup is a conflict-free broadcast read
  __shared__ float lut[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % G::WN, wm = wave / G::WN;
  const int wm0 = wm * G::WTM;
  int tm, tn;
  const int ntiles = a.tiles_m * a.tiles_n;
  const int split = (int)blockIdx.x / ntiles;
  tile_coords((int)blockIdx.x - split * ntiles, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  if constexpr (WFMT != LSL_WFMT_BF16)
    if (tid < 16) lut[tid] = a.cb[tid];

  f32x16 acc[2][MI];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto xstore = [&](const RowLoader<BM>& l, uint16_t* d) { l.store_swz(d, tid); };
  // ---- LoRA K-step first (kl <= 64, zero padded to 64), by split 0: the
  // accumulators start as s * (L Lt^T), so no second set of accumulators is live
  // during the main loop
  if constexpr (LORA != 0) if (split == 0) {
    uint16_t* Ls = Xs;
    uint16_t* Lt = Ws;
    lora_stage<LORA, BN, BM>(a, Ls, Lt, m0, n0, tid);
    __syncthreads();
    mma_tile<MI>(Lt, Ls, acc, wn, wm0, lane, (a.kl + 15) / 16);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= a.scale;
    // the main loop's first barrier (before any tile store) orders these LDS reads
  }

  // this workgroup's reduction steps [kt0, kt0 + KT)
  const int kt0 = split * a.kt_per_split;
  const int KT = min((int)(a.K / BK) - kt0, a.kt_per_split);
  // tile k + 1 is loaded into registers while tile k computes from the single
  // LDS buffer (two barriers per K-step; a second LDS buffer, or a second
  // register set two tiles ahead, measured slower: fewer workgroups per CU)
  RowLoader<BM> xl;
  WLoader<WFMT, KN, BN> wl;
  xl.init(a.ldx, m0, tid);
  wl.init(a, n0, tid);
  xl.load(a.x, a.ldx, a.M, (int64_t)kt0 * BK);
  wl.load(a, (int64_t)kt0 * BK);
  __syncthreads();  // lut visible
  xstore(xl, Xs);
  wl.store(Ws, lut, tid);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) {
      xl.load(a.x, a.ldx, a.M, (int64_t)(kt0 + kt + 1) * BK);
      wl.load(a, (int64_t)(kt0 + kt + 1) * BK);
    }
    mma_tile<MI, KN, true>(Ws, Xs, acc, wn, wm0, lane, 4);
    __syncthreads();
    if (more) {
      xstore(xl, Xs);
      wl.store(Ws, lut, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: for block (ni, mi) and q < 4, the lane holds C[m][n .. n+3] with
  // m = m0 + wm0 + 32 mi + lane % 32, n = n0 + 64 wn + 32 ni + 8 q + 4 (lane / 32)
  const int64_t mb = m0 + wm0 + (lane & 31);
  const int64_t nb = n0 + wn * 64 + (lane >> 5) * 4;
  if constexpr (EPI == EPI_LSE) {
    // Cross-entropy forward: per token m, max and sum of exp over this tile's
    // vocabulary entries n < N, and the label's logit if it falls in the tile.
    float2* red = reinterpret_cast<float2*>(Xs);  // [WN][BM]
    float2 rows[MI];
    lse_rows<2, MI>(a, acc, mb, nb, rows);
    if ((lane >> 5) == 0)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) red[wn * BM + wm0 + mi * 32 + (lane & 31)] = rows[mi];
    __syncthreads();
    for (int t = tid; t < BM; t += NTHREADS)
      if (m0 + t < a.M) a.part[(int64_t)tn * a.M + m0 + t] = lse_combine(red + t, G::WN, BM);
    return;
  }
  if (EPI == EPI_BF16 && a.ksplit > 1) {
    store_split_partials<MI>(a, acc, mb, nb, split);
    return;
  }
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t n = nb + ni * 32 + 8 * q;
    if (n >= a.N) continue;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int64_t m = mb + mi * 32;
      if (m >= a.M) continue;
      float v0 = acc[ni][mi][4 * q], v1 = acc[ni][mi][4 * q + 1], v2 = acc[ni][mi][4 * q + 2], v3 = acc[ni][mi][4 * q + 3];
      if constexpr (EPI == EPI_CEGRAD) {
        ce_grad4(a, m, n, v0, v1, v2, v3);
      } else if constexpr (EPI == EPI_ACC32) {
        acc32_4(a, split, m, n, v0, v1, v2, v3);
      } else {
        store_bf16x4(a, m, n, v0, v1, v2, v3);
      }
    }
  }
}

// y[m][n] = bf16(sum over splits in index order (+ bias)) (+ residual, rounded
// again), the same rounding as the unsplit bf16 epilogue. One thread per 4 outputs.
__global__ void gemm_split_reduce(const float* __restrict__ part, int S, int64_t M, int64_t N,
                                  const uint16_t* __restrict__ bias, const uint16_t* __restrict__ res, int64_t ldres,
                                  uint16_t* __restrict__ y, int64_t ldy) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= M * N) return;
  const int64_t m = i / N, n = i - m * N;
  f32x4 v = *reinterpret_cast<const f32x4*>(part + i);
  for (int s = 1; s < S; ++s) {
    const f32x4 p = *reinterpret_cast<const f32x4*>(part + (int64_t)s * M * N + i);
    v = f32x4{v[0] + p[0], v[1] + p[1], v[2] + p[2], v[3] + p[3]};
  }
  if (bias) {
    const u32x2 b = *reinterpret_cast<const u32x2*>(bias + n);
    v = f32x4{v[0] + lo_bf(b[0]), v[1] + hi_bf(b[0]), v[2] + lo_bf(b[1]), v[3] + hi_bf(b[1])};
  }
  if (res) {
    const u32x2 r = *reinterpret_cast<const u32x2*>(res + m * ldres + n);
    v = f32x4{bf2f(f2bf(v[0])) + lo_bf(r[0]), bf2f(f2bf(v[1])) + hi_bf(r[0]), bf2f(f2bf(v[2])) + lo_bf(r[1]),
              bf2f(f2bf(v[3])) + hi_bf(r[1])};
  }
  *reinterpret_cast<u32x2*>(y + m * ldy + n) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
}

// ---- Large-tile kernel for GEMMs with many output tiles: 256 weight rows x 256
// tokens per workgroup of 8 waves, each wave 128 weight rows x 64 tokens (4 x 2
// blocks of 32 x 32). The token tile (and a bf16 [N x K] weight tile) goes from
// global memory straight into LDS (buffer_load ... lds, no registers), into the
// same swizzled [256][64] layout as above; an NF4 tile is loaded into registers one
// K-step ahead of its dequantisation. Two LDS stages, one barrier per K-step:
//   step k: dequant codes(k + 1) -> W[k+1]; codes(k + 2) -> registers;
//           DMA tokens(k + 1) -> X[k+1]; MFMAs on X[k], W[k]; wait; barrier.
// Measured at 8192 tokens (gate|up 28672 x 4096, NF4): 27% less time than the
// 64 x 256 tile, whose token rows no longer stay in L2 at that size.
namespace big {
constexpr int BN = 256, BM = 256, NT = 512;
constexpr int XSZ = BM * BK;  // token stage [256][64], swizzled
constexpr int WSZ = BN * LDSW > BK * (BN + 32) ? BN * LDSW : BK * (BN + 32);

typedef __attribute__((address_space(3))) void lds_void;

// LDS DMA of a [256][64] bf16 tile (rows r0 .. r0 + 255 of a row-major matrix,
// 64 columns from k0) into the swizzled layout: wave w issues rows 8 (4 w + i) .. + 7,
// i < 4; lane l carries chunk (l % 8) ^ xswz(row) of row 8 (4 w + i) + l / 8, which
// lands at position l % 8 of that row. Rows at or past `rows` read zeros.
struct TileDma {
  uint32_t voff[4];
  int wave;
  LSL_DEV void init(int64_t ld, int64_t r0, int64_t rows_clamp, int w, int lane) {
    wave = w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (w * 4 + i) * 8 + (lane >> 3);
      int64_t g = r0 + row;
      if (rows_clamp > 0 && g >= rows_clamp) g = rows_clamp - 1;
      voff[i] = (uint32_t)((g * ld + ((lane & 7) ^ xswz(row)) * 8) * 2);
    }
  }
  LSL_DEV void issue(const uint16_t* base, int64_t ld, int64_t rows, int64_t k0, uint16_t* __restrict__ lds) const {
    // the host compilation pass has no LDS-load builtin; the device pass emits
    // buffer_load_dwordx4 ... lds
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, rows * ld * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (wave * 4 + i) * 8 * BK), 16, voff[i],
                                               (uint32_t)(k0 * 2), 0, 0);
#else
    (void)base; (void)ld; (void)rows; (void)k0; (void)lds;
#endif
  }
};

// Weight tile producers. kind: 0 registers + dequant (NF4 / NF4DQ, either
// layout; bf16 [K x N]), 1 LDS DMA (bf16 [N x K]).
template <int WFMT, bool KN>
struct BigW;

// codebook values of the 8 NF4 codes in one code dword (byte j: element 2j in
// the high nibble, 2j + 1 in the low one), and their bf16 products with the
// block's absmax. The codebook sits in LDS as 256 pairs, one per code byte, so
// a byte costs one 8-byte read and one address (about 3% of the large tile's
// time against one 4-byte read and address per nibble)
LSL_DEV void nf4_fetch(uint32_t cw, const float* lut, float (&v)[8]) {
  // lut: 256 pairs, entry b = the values of code byte b's high and low nibbles
  const float2* l2 = reinterpret_cast<const float2*>(lut);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float2 p = l2[(cw >> (j * 8)) & 255];
    v[2 * j] = p.x;
    v[2 * j + 1] = p.y;
  }
}
LSL_DEV u32x4 nf4_emit(const float (&v)[8], float am) {
  return u32x4{pack2(v[0] * am, v[1] * am), pack2(v[2] * am, v[3] * am), pack2(v[4] * am, v[5] * am),
               pack2(v[6] * am, v[7] * am)};
}

// NF4 [N x K]: thread -> row tid / 2, 16 code bytes (32 weights) at k 32 (tid % 2);
// rows past N clamped to the last row (their outputs are never stored)
template <int WFMT>
struct BigNf4Nk {
  static constexpr int kind = 0, nload = 2;
  const uint8_t* pc;
  int64_t ai;
  u32x4 c;
  float am;
  LSL_DEV void init(const GemmKArgs& a, int64_t n0, int tid, int, int) {
    const int row = tid >> 1, part = tid & 1;
    const int64_t n = n0 + row < a.N ? n0 + row : a.N - 1;
    pc = a.wq + n * (a.K >> 1) + part * 16;
    ai = n * (a.K >> 6);
  }
  LSL_DEV void load(const GemmKArgs& a, int64_t k0) {
    c = *reinterpret_cast<const u32x4*>(pc + (k0 >> 1));
    am = block_absmax<WFMT>(a, ai + (k0 >> 6));
  }
  // quarter i of the tile row, code dword i (8 weights): codebook values, then
  // the scaled bf16 weights as one 16-byte LDS store
  LSL_DEV void fetch(int i, const float* lut, float (&v)[8]) const { nf4_fetch(c[i], lut, v); }
  LSL_DEV void emit(int i, const float (&v)[8], uint16_t* __restrict__ lds, int tid) const {
    reinterpret_cast<u32x4*>(lds + (tid >> 1) * LDSW + (tid & 1) * 32)[i] = nf4_emit(v, am);
  }
  LSL_DEV void store(uint16_t* __restrict__ lds, const float* lut, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[8];
      fetch(i, lut, v);
      emit(i, v, lds, tid);
    }
  }
};
template <> struct BigW<LSL_WFMT_NF4, false> : BigNf4Nk<LSL_WFMT_NF4> {};
template <> struct BigW<LSL_WFMT_NF4DQ, false> : BigNf4Nk<LSL_WFMT_NF4DQ> {};

// The [K x N] weight tile in LDS: [64 k][256 n] with a row stride of KNW = 288
// elements (row r starts 4 r 16-byte bank groups further on, modulo 16), the
// 8-column chunk c of row r at chunk position c ^ 2 ((r >> 3) & 1). A
// transposing read takes rows r0 .. r0 + 3 (r0 a multiple of 4) x 4 chunks in
// lanes 0-31 and rows r0 + 8 .. r0 + 11 in lanes 32-63: both halves, and the
// lanes 0-15 + 32-47 pairing too, touch 16 distinct bank groups, and every
// offset but one base is an immediate. The loaders below give each thread one
// chunk position in four rows, so every 16 lanes of a store write 16
// consecutive chunks of one row: conflict-free too. Same size as [256][LDSW].
constexpr int KNW = BN + 32;
LSL_DEV int kn_pos(int r, int c) { return r * KNW + 8 * (c ^ (((r >> 3) & 1) << 1)); }
// row of load i (0..3) of thread tid: wave w takes rows 8 w .. 8 w + 7, lanes
// 0-31 the even and lanes 32-63 the odd ones; chunk tid % 32
LSL_DEV int kn_row(int tid, int i) { return 8 * (tid >> 6) + 2 * i + ((tid >> 5) & 1); }

// NF4 [K x N] (N % 64 == 0): thread -> chunk tid % 32 (8 columns, 4 code bytes
// and their absmax) of the rows kn_row(tid, i). Column groups past N are
// clamped to the last group (outputs not stored).
// Codes and absmax are read through buffer descriptors over the whole matrix
// with the lane's offset in the vector offset and the row's in the scalar
// offset: every row read is inside the matrix and the columns are clamped, so
// no range check is needed, and one 32-bit register per operand addresses all
// four rows.
template <int WFMT>
struct BigNf4Kn {
  // vector loads issued per load() (8, 12 for NF4DQ): the pipeline's wait for
  // the token DMA may count fewer of them, never more
  static constexpr int kind = 0, nload = 8;
  uint32_t vc, va;  // byte offsets of the lane's codes and absmax (code) in row 0
  uint32_t c[4];
  float am[4];
  LSL_DEV void init(const GemmKArgs& a, int64_t n0, int tid, int, int) {
    const int64_t n = n0 + (tid & 31) * 8 < a.N ? n0 + (tid & 31) * 8 : a.N - 8;
    const int64_t row = kn_row(tid, 0);
    vc = (uint32_t)(row * (a.N >> 1) + (n >> 1));
    va = (uint32_t)((row * (a.N >> 6) + (n >> 6)) * (WFMT == LSL_WFMT_NF4DQ ? 1 : 4));
  }
  LSL_DEV void load(const GemmKArgs& a, int64_t k0) {
    const int64_t rowc = a.N >> 1, rowa = a.N >> 6;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.wq, a.K * rowc);
#pragma unroll
    for (int i = 0; i < 4; ++i)  // rows kn_row(tid, 0) + 2 i
      c[i] = bload4(rc, vc, (uint32_t)((k0 + 2 * i) * rowc));
    if constexpr (WFMT == LSL_WFMT_NF4DQ) {
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.wq8, a.K * rowa);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t q = __builtin_amdgcn_raw_buffer_load_b8(rq, va, (uint32_t)((k0 + 2 * i) * rowa), 0);
        const int64_t idx = (int64_t)va + (k0 + 2 * i) * rowa;  // flattened absmax index
        am[i] = (float)q * a.wsc[idx >> 8];
      }
    } else {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.wa, a.K * rowa * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) am[i] = __uint_as_float(bload4(ra, va, (uint32_t)((k0 + 2 * i) * rowa * 4)));
    }
  }
  // quarter i: row kn_row(tid, i), its 8 codes' values, then the scaled bf16
  // weights as one 16-byte LDS store
  LSL_DEV void fetch(int i, const float* lut, float (&v)[8]) const { nf4_fetch(c[i], lut, v); }
  LSL_DEV void emit(int i, const float (&v)[8], uint16_t* __restrict__ lds, int tid) const {
    *reinterpret_cast<u32x4*>(lds + kn_pos(kn_row(tid, i), tid & 31)) = nf4_emit(v, am[i]);
  }
  LSL_DEV void store(uint16_t* __restrict__ lds, const float* lut, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[8];
      fetch(i, lut, v);
      emit(i, v, lds, tid);
    }
  }
};
template <> struct BigW<LSL_WFMT_NF4, true> : BigNf4Kn<LSL_WFMT_NF4> {};
template <> struct BigW<LSL_WFMT_NF4DQ, true> : BigNf4Kn<LSL_WFMT_NF4DQ> {};

// bf16 [K x N]: thread -> chunk tid % 32 (16 bytes) of the rows kn_row(tid, i);
// columns past N read zeros (buffer range) or neighbouring data, never stored
template <>
struct BigW<LSL_WFMT_BF16, true> {
  static constexpr int kind = 0, nload = 4;
  uint32_t voff;
  u32x4 v[4];
  LSL_DEV void init(const GemmKArgs& a, int64_t n0, int tid, int, int) {
    voff = (uint32_t)((((int64_t)kn_row(tid, 0)) * a.N + n0 + (tid & 31) * 8) * 2);
  }
  LSL_DEV void load(const GemmKArgs& a, int64_t k0) {
    // descriptor from row k0 to the end of the matrix: a column past N in the
    // last row reads zeros instead of the bytes after the matrix
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.wb + k0 * a.N, (a.K - k0) * a.N * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = bload16(rs, voff + (uint32_t)(2 * i * a.N * 2), 0);
  }
  LSL_DEV void fetch(int, const float*, float (&)[8]) const {}
  LSL_DEV void emit(int i, const float (&)[8], uint16_t* __restrict__ lds, int tid) const {
    *reinterpret_cast<u32x4*>(lds + kn_pos(kn_row(tid, i), tid & 31)) = v[i];
  }
  LSL_DEV void store(uint16_t* __restrict__ lds, const float*, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(lds + kn_pos(kn_row(tid, i), tid & 31)) = v[i];
  }
};

// bf16 [N x K]: LDS DMA like the token tile (rows past N clamped)
template <>
struct BigW<LSL_WFMT_BF16, false> {
  static constexpr int kind = 1, nload = 0;
  TileDma dma;
  LSL_DEV void init(const GemmKArgs& a, int64_t n0, int, int wave, int lane) { dma.init(a.K, n0, a.N, wave, lane); }
  LSL_DEV void issue(const GemmKArgs& a, int64_t k0, uint16_t* __restrict__ lds) const {
    dma.issue(a.wb, a.K, a.N, k0, lds);
  }
};

// nsub 16-deep MFMA sub-steps: acc[ni][mi] += W-block[ni] x X-block[mi] for the
// wave's 128 x 64 tile. WL: weight tile layout 0 padded [n][LDSW], 1 swizzled
// [n][64], 2 the swizzled [k][256] layout (kn_pos) read with transposing LDS reads.
struct NoPart {
  LSL_DEV void begin() const {}
  LSL_DEV void operator()(int) const {}
};
template <int WL, typename Part = NoPart>
LSL_DEV void mma_big(const uint16_t* __restrict__ Ws, const uint16_t* __restrict__ Xs, f32x16 (&acc)[4][2], int wn,
                     int wm, int lane, int nsub, Part&& part = Part()) {
  const int h = lane >> 5, r32 = lane & 31;
  auto frag = [&](int s, bf16x8 (&af)[4], bf16x8 (&bfr)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wn * 128 + i * 32 + r32;
      if constexpr (WL == 0) {
        af[i] = *reinterpret_cast<const bf16x8*>(Ws + row * LDSW + 16 * s + 8 * h);
      } else if constexpr (WL == 1) {
        af[i] = *reinterpret_cast<const bf16x8*>(Ws + row * BK + 8 * ((2 * s + h) ^ xswz(row)));
      } else {
        // lanes 16-31 / 48-63 take columns 16..31 of the block; each 16-lane group
        // reads rows kofs .. kofs + 3 and kofs + 4 .. kofs + 7 of its 16 columns:
        // lane j gets row kofs + j / 4, columns 4 (j % 4) .. + 3 (half of a chunk)
        const int j = lane & 15, r = 16 * s + 8 * h + (j >> 2);
        const int c = wn * 16 + i * 4 + 2 * ((lane >> 4) & 1) + ((j & 3) >> 1), e = 4 * (j & 1);
        const u32x2 lo = ld_tr4(Ws + kn_pos(r, c) + e), hi = ld_tr4(Ws + kn_pos(r + 4, c) + e);
        af[i] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wm * 64 + i * 32 + r32;
      bfr[i] = *reinterpret_cast<const bf16x8*>(Xs + row * BK + 8 * ((2 * s + h) ^ xswz(row)));
    }
  };
  // sub-step s + 1's fragments are read while sub-step s multiplies
  bf16x8 af[2][4], bfr[2][2];
  frag(0, af[0], bfr[0]);
  part.begin();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s >= nsub) break;
    if (s + 1 < nsub) frag(s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
    part(s);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) acc[ni][mi] = mfma32(af[s & 1][ni], bfr[s & 1][mi], acc[ni][mi]);
    if constexpr (!std::is_same<Part, NoPart>::value) {
      // issue order within the sub-step: each MFMA followed by two LDS reads
      // (next fragments, codebook values) and four VALU operations of the
      // weight conversion, then the weight store; nothing crosses sub-steps
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);    // LDS write
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// LoRA K-step operands: Ls = rows m0.. of la (k zero padded to 64) in the
// swizzled token layout; Lt as in lora_stage, [BN][LDSW] for the forward (LORA
// 1) and, for the input gradient (LORA 2), A_full's rows j < 64 in the swizzled
// [k][256] layout the KN main loop reads. 16-byte chunks, loads issued first.
template <int LORA>
LSL_DEV void lora_stage_big(const GemmKArgs& a, uint16_t* Ls, uint16_t* Lt, int64_t m0, int64_t n0, int tid) {
  constexpr int LC = BM * 8 / NT, TC = BN * 8 / NT;  // 4 and 4 chunks per thread
  u32x4 lv[LC], tv[TC];
#pragma unroll
  for (int i = 0; i < LC; ++i) {
    const int c = tid + i * NT, row = c >> 3, col = (c & 7) * 8;
    const int64_t gm = m0 + row;
    lv[i] = (gm < a.M && col < a.kl) ? *reinterpret_cast<const u32x4*>(a.la + gm * a.ldla + col) : u32x4{0, 0, 0, 0};
  }
  if constexpr (LORA == 1) {
    // thread -> row tid / 2, chunks 4 (tid % 2) .. + 3
    const int row = tid >> 1, c0 = (tid & 1) * 4;
    const int64_t gn = n0 + row;
    const int seg = gn < a.N ? lora_seg(a, gn) : -1;
#pragma unroll
    for (int q = 0; q < TC; ++q) {
      const int j0 = (c0 + q) * 8;
      tv[q] = (seg >= 0 && j0 < a.kl && j0 / a.r == seg)
                  ? *reinterpret_cast<const u32x4*>(a.lb + gn * a.r + (j0 - seg * a.r))
                  : u32x4{0, 0, 0, 0};
    }
  } else {
    // thread -> reduction row j = c / 32, columns 8 (c % 32) .. + 7
#pragma unroll
    for (int q = 0; q < TC; ++q) {
      const int c = tid + q * NT, j = c >> 5, nc = (c & 31) * 8;
      const int64_t gn = n0 + nc;
      tv[q] = (j < a.kl && gn < a.N) ? *reinterpret_cast<const u32x4*>(a.lb + (int64_t)j * a.N + gn)
                                     : u32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int i = 0; i < LC; ++i) {
    const int c = tid + i * NT, row = c >> 3, ch = c & 7;
    *reinterpret_cast<u32x4*>(Ls + row * BK + 8 * (ch ^ xswz(row))) = lv[i];
  }
  if constexpr (LORA == 1) {
    const int row = tid >> 1, c0 = (tid & 1) * 4;
#pragma unroll
    for (int q = 0; q < TC; ++q) *reinterpret_cast<u32x4*>(Lt + row * LDSW + (c0 + q) * 8) = tv[q];
  } else {
#pragma unroll
    for (int q = 0; q < TC; ++q) {
      const int c = tid + q * NT, j = c >> 5;
      *reinterpret_cast<u32x4*>(Lt + kn_pos(j, c & 31)) = tv[q];
    }
  }
}

// keeps the compiler from moving memory operations across this point
LSL_DEV void order_point() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// wait until at most n vector-memory loads are outstanding and all LDS stores
// are done, then the workgroup barrier (no release fence: the loads issued
// after the tile DMA stay in flight across it)
template <int N>
LSL_DEV void tile_barrier() {
  static_assert(N == 0 || N == 2 || N == 4 || N == 8, "tile_barrier: 0, 2, 4 or 8 loads");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace big

namespace big {

// The LDS stages of one workgroup.
struct Smem {
  uint16_t* xs0; uint16_t* xs1; uint16_t* ws0; uint16_t* ws1; const float* lut;
};

// acc = the sum over reduction steps [kb, kb + nsteps) of output tile (m0, n0),
// plus s * (L Lt^T) when kb == 0 and the GEMM has a LoRA term. On return every
// wave has passed the last step's barrier, so both stages are free again.
template <int WFMT, bool KN, int LORA>
LSL_DEV void tile_steps(const GemmKArgs& a, int64_t m0, int64_t n0, int kb, int nsteps, f32x16 (&acc)[4][2],
                        const Smem& sm, int tid) {
  using W = BigW<WFMT, KN>;
  constexpr int WL = KN ? 2 : (W::kind == 1 ? 1 : 0);
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  uint16_t* const Xs0 = sm.xs0; uint16_t* const Xs1 = sm.xs1;
  uint16_t* const Ws0 = sm.ws0; uint16_t* const Ws1 = sm.ws1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int KT = nsteps;
  const int64_t k0 = (int64_t)kb * BK;
  TileDma xd;
  xd.init(a.ldx, m0, 0, wave, lane);
  W wl;
  wl.init(a, n0, tid, wave, lane);
  // step 0's tiles are requested first, so their latency overlaps the LoRA step
  xd.issue(a.x, a.ldx, a.M, k0, Xs0);
  if constexpr (W::kind == 1) wl.issue(a, k0, Ws0);
  else wl.load(a, k0);

  // the LoRA K-step (with the tile's first reduction step), on the second
  // stage's buffers: the accumulators start as s * (L Lt^T)
  const bool lora_here = LORA != 0 && kb == 0;
  if constexpr (LORA != 0) if (lora_here) {
    lora_stage_big<LORA>(a, Xs1, Ws1, m0, n0, tid);
    __syncthreads();
    mma_big<LORA == 1 ? 0 : 2>(Ws1, Xs1, acc, wn, wm, lane, (a.kl + 15) / 16);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= a.scale;
    // stage 1 is next written after the prologue's barrier, which every wave
    // reaches only after these reads
  }

  // prologue: step 0 into stage 0; codes of step 1 into registers
  if constexpr (W::kind == 0) {
    if (!lora_here) __syncthreads();  // lut visible (the LoRA step's barrier did it otherwise)
    wl.store(Ws0, sm.lut, tid);
    if (KT > 1) wl.load(a, k0 + BK);
  }
  tile_barrier<0>();
  auto step = [&](int kt, const uint16_t* __restrict__ xc, const uint16_t* __restrict__ wc, uint16_t* __restrict__ xn,
                  uint16_t* __restrict__ wnx) {
    const bool next = kt + 1 < KT, next2 = kt + 2 < KT;
    if constexpr (W::kind == 1) {
      if (next) {
        wl.issue(a, k0 + (int64_t)(kt + 1) * BK, wnx);
        xd.issue(a.x, a.ldx, a.M, k0 + (int64_t)(kt + 1) * BK, xn);
      }
      mma_big<WL>(wc, xc, acc, wn, wm, lane, 4);
    } else {
      // step kt + 1's weights (held in registers) are converted and stored
      // between this step's MFMAs, a quarter per 16-deep sub-step. After the
      // last step the store goes to the idle stage and is never read.
      const W cur = wl;
      if (next) xd.issue(a.x, a.ldx, a.M, k0 + (int64_t)(kt + 1) * BK, xn);
      if (next2) {
        // the weight loads must issue after the DMA: the barrier below counts them
        order_point();
        wl.load(a, k0 + (int64_t)(kt + 2) * BK);
      }
      // quarter q's codebook values are read one sub-step before they are scaled
      // and stored, so the LDS latency hides behind that sub-step's MFMAs
      struct Part {
        const W& w;
        const float* lut;
        uint16_t* __restrict__ dst;
        int tid;
        float v[2][8];
        LSL_DEV void begin() { w.fetch(0, lut, v[0]); }
        LSL_DEV void operator()(int q) {
          if (q + 1 < 4) w.fetch(q + 1, lut, v[(q + 1) & 1]);
          w.emit(q, v[q & 1], dst, tid);
        }
      } part{cur, sm.lut, wnx, tid, {}};
      mma_big<WL>(wc, xc, acc, wn, wm, lane, 4, part);
    }
    // the DMA of step kt + 1 is complete once at most the weight loads issued
    // after it (step kt + 2) are outstanding
    if constexpr (W::kind == 0 && W::nload == 2) {
      if (next2) tile_barrier<2>(); else tile_barrier<0>();
    } else if constexpr (W::kind == 0 && W::nload == 4) {
      if (next2) tile_barrier<4>(); else tile_barrier<0>();
    } else if constexpr (W::kind == 0 && W::nload == 8) {
      if (next2) tile_barrier<8>(); else tile_barrier<0>();
    } else {
      tile_barrier<0>();
    }
  };
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, Xs0, Ws0, Xs1, Ws1);
    if (kt + 1 < KT) step(kt + 1, Xs1, Ws1, Xs0, Ws0);
  }
}

// bf16 epilogue of a finished tile (bias, residual), or its float32 split-K
// partial at `part` (row-major [M][N]) when part != NULL, for the column blocks
// ni0 .. ni0 + NI - 1 held in v[0 .. NI - 1]. Block (ni, mi), q < 4: the lane
// holds C[m][n .. n + 3] with m = m0 + 64 wm + 32 mi + lane % 32,
// n = n0 + 128 wn + 32 ni + 8 q + 4 (lane / 32).
template <int NI>
LSL_DEV void store_tile_bf16(const GemmKArgs& a, const f32x16 (&acc)[NI][2], int ni0, int64_t m0, int64_t n0, int tid,
                             float* part) {
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t mb = m0 + (wave >> 1) * 64 + (lane & 31);
  const int64_t nb = n0 + (wave & 1) * 128 + (lane >> 5) * 4;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n = nb + (ni0 + ni) * 32 + 8 * q;
      if (n >= a.N) continue;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int64_t m = mb + mi * 32;
        if (m >= a.M) continue;
        const f32x16& v = acc[ni][mi];
        if (part)
          *reinterpret_cast<f32x4*>(part + m * a.N + n) = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        else
          store_bf16x4(a, m, n, v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      }
    }
}

// Stream-K partial slots hold a tile's accumulators in register order: float4
// group g of thread t at (g NT + t) * 4, so every store and load is a
// contiguous 16-byte access per lane. They are written and read through
// (wt_store4 / wt_load4): the slot region is handed between workgroups on
// different XCDs within the launch.
constexpr int SLOT = BM * BN;
LSL_DEV void slot_store(__amdgpu_buffer_rsrc_t rs, int slot, const f32x16 (&acc)[4][2], int tid) {
  const uint32_t so = (uint32_t)slot * SLOT * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = (i * 2 + j) * 4 + q;
        const f32x16& v = acc[i][j];
        wt_store4(rs, (uint32_t)(g * NT + tid) * 16, so, f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]});
      }
}

// The last arrival's sum of a split tile: the partials in slots s0 .. s0 + nseg - 1,
// added in that order, then the bf16 epilogue; one half of the tile (column
// blocks 2 h, 2 h + 1) at a time, two slots' 32 loads in flight per lane (the
// segment loop's registers are free by now).
LSL_DEV void sk_fixup(const GemmKArgs& a, __amdgpu_buffer_rsrc_t rs, int s0, int nseg, int64_t m0, int64_t n0,
                      int tid) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x16 sum[2][2];
    for (int v = 0; v < nseg; v += 2) {
      f32x4 p[2][16];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (v + u < nseg) {
          const uint32_t so = (uint32_t)(s0 + v + u) * SLOT * 4;
#pragma unroll
          for (int c = 0; c < 16; ++c) p[u][c] = wt_load4(rs, (uint32_t)((h * 16 + c) * NT + tid) * 16, so);
        }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (v + u < nseg)
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const int i = c >> 3, j = (c >> 2) & 1, q = c & 3;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sum[i][j][4 * q + e] = v + u == 0 ? p[u][c][e] : sum[i][j][4 * q + e] + p[u][c][e];
          }
    }
    store_tile_bf16<2>(a, sum, 2 * h, m0, n0, tid, nullptr);
  }
}

// Stream-K schedule: the reduction steps of all tiles, tile after tile, form
// one range of U = tiles * KT units that G workgroups split evenly; workgroup w
// takes units [U w / G, U (w + 1) / G). owner(u) is the workgroup whose range
// holds unit u.
LSL_DEV int sk_owner(int u, int U, int G) { return ((u + 1) * G - 1) / U; }

}  // namespace big

// Stream-K over a.sk_g workgroups (bf16 epilogue): workgroup w (the dispatch
// order deals blocks to the XCDs in turn, so w gives each XCD a contiguous range
// of units) walks its units tile by tile. Tile t is (tm, tn) = (t % tiles_m,
// t / tiles_m): an XCD's tiles share weight tiles. A tile split over several
// workgroups is summed by the one that arrives last, in workgroup order.
template <int WFMT, bool KN, int LORA>
__global__ __launch_bounds__(big::NT, 1) void gemm_sk_kernel(const GemmKArgs a) {
  using namespace big;
  __shared__ __attribute__((aligned(16))) uint16_t Xs0[XSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Xs1[XSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Ws0[WSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Ws1[WSZ];
  __shared__ float2 lut2[256];
  float* const lut = reinterpret_cast<float*>(lut2);
  const Smem sm{Xs0, Xs1, Ws0, Ws1, lut};
  if constexpr (WFMT != LSL_WFMT_BF16)
    if (threadIdx.x < 256) lut2[threadIdx.x] = float2{a.cb[threadIdx.x >> 4], a.cb[threadIdx.x & 15]};
  f32x16 acc[4][2];
  const int KTall = (int)(a.K / BK);
  const int G = a.sk_g, b = (int)blockIdx.x;
  const int w = (b & 7) * (G >> 3) + (b >> 3);
  // U G < 2^31 (checked on the host)
  const int U = a.tiles_m * a.tiles_n * KTall;
  // the slots: (G + tiles - 1) x 256 KiB, below 4 GiB (tiles < G)
  const __amdgpu_buffer_rsrc_t rs = wt_rsrc(a.spart, (int64_t)(G + a.tiles_m * a.tiles_n - 1) * SLOT * 4);
  const int ue = U * (w + 1) / G;
  // tiles whose partials this workgroup adds up (it arrived last), summed after
  // its own segments so that the sum's registers are not live in the loop; with
  // fewer tiles than workgroups a workgroup has at most two segments
  int fix_t[2], fix_f[2], fix_n[2], nfix = 0;
  for (int u = U * w / G; u < ue;) {
    // thread-index arithmetic is redone per segment instead of being held in
    // registers across the loop (which would spill)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int t = u / KTall;
    const int kb = u - t * KTall;
    const int ke = min(KTall, kb + (ue - u));
    const int64_t m0 = (int64_t)(t % a.tiles_m) * BM, n0 = (int64_t)(t / a.tiles_m) * BN;
    tile_steps<WFMT, KN, LORA>(a, m0, n0, kb, ke - kb, acc, sm, tid);
    u += ke - kb;
    if (kb == 0 && ke == KTall) {
      store_tile_bf16<4>(a, acc, 0, m0, n0, tid, nullptr);
      continue;
    }
    // workgroups f .. l share tile t; their partials sit in slots f + t .. l + t
    slot_store(rs, w + t, acc, tid);
    const int f = sk_owner(t * KTall, U, G), l = sk_owner(t * KTall + KTall - 1, U, G);
    // (nfix < 2 always: the host launches stream-K only with fewer tiles than
    // workgroups, and a workgroup's units then span at most two tiles)
    if (last_arrival(a.cnt + t, l - f + 1) && nfix < 2) {
      fix_t[nfix] = t; fix_f[nfix] = f; fix_n[nfix] = l - f + 1;
      ++nfix;
    }
  }
  const int tid = threadIdx.x;
  for (int i = 0; i < nfix; ++i) {
    const int t = fix_t[i];
    sk_fixup(a, rs, fix_f[i] + t, fix_n[i], (int64_t)(t % a.tiles_m) * BM, (int64_t)(t / a.tiles_m) * BN, tid);
  }
}

template <int WFMT, bool KN, int LORA, int EPI = EPI_BF16>
__global__ __launch_bounds__(big::NT, 1) void gemm_big_kernel(const GemmKArgs a) {
  using namespace big;
  __shared__ __attribute__((aligned(16))) uint16_t Xs0[XSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Xs1[XSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Ws0[WSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Ws1[WSZ];
  __shared__ float2 lut2[256];
  float* const lut = reinterpret_cast<float*>(lut2);
  const Smem sm{Xs0, Xs1, Ws0, Ws1, lut};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (WFMT != LSL_WFMT_BF16)
    if (tid < 256) lut2[tid] = float2{a.cb[tid >> 4], a.cb[tid & 15]};
  f32x16 acc[4][2];
  const int KTall = (int)(a.K / BK);

  int tm, tn;
  const int ntiles = a.tiles_m * a.tiles_n;
  const int split = (int)blockIdx.x / ntiles;  // split-K: reduction steps [kt0, kt0 + KT)
  tile_coords((int)blockIdx.x - split * ntiles, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int kt0 = split * a.kt_per_split;
  tile_steps<WFMT, KN, LORA>(a, m0, n0, kt0, min(KTall - kt0, a.kt_per_split), acc, sm, tid);

  // epilogue: block (ni, mi), q < 4: the lane holds C[m][n .. n + 3] with
  // m = m0 + 64 wm + 32 mi + lane % 32, n = n0 + 128 wn + 32 ni + 8 q + 4 (lane / 32)
  const int wn = wave & 1, wm = wave >> 1;
  const int64_t mb = m0 + wm * 64 + (lane & 31);
  const int64_t nb = n0 + wn * 128 + (lane >> 5) * 4;
  if constexpr (EPI == EPI_LSE) {
    // cross-entropy forward: per token row, (max, sum of exp) over this tile's
    // vocabulary columns; the two column halves (wn) are combined through LDS,
    // which every wave has finished reading at the loop's last barrier
    float2* red = reinterpret_cast<float2*>(Xs0);  // [2][BM]
    float2 rows[2];
    lse_rows<4, 2>(a, acc, mb, nb, rows);
    if ((lane >> 5) == 0)
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) red[wn * BM + wm * 64 + mi * 32 + (lane & 31)] = rows[mi];
    __syncthreads();
    for (int t = tid; t < BM; t += NT)
      if (m0 + t < a.M) a.part[(int64_t)tn * a.M + m0 + t] = lse_combine(red + t, 2, BM);
    return;
  }
  if constexpr (EPI == EPI_CEGRAD || EPI == EPI_ACC32) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = nb + ni * 32 + 8 * q;
        if (n >= a.N) continue;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const int64_t m = mb + mi * 32;
          if (m >= a.M) continue;
          const f32x16& v = acc[ni][mi];
          if constexpr (EPI == EPI_CEGRAD) ce_grad4(a, m, n, v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
          else acc32_4(a, split, m, n, v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
      }
    return;
  }
  // split-K: this split's float32 partial (gemm_split_reduce adds the splits in order)
  store_tile_bf16<4>(a, acc, 0, m0, n0, tid, a.ksplit > 1 ? a.spart + (int64_t)split * a.M * a.N : nullptr);
}

template <int WFMT, bool KN, int BN, int BM>
static void launch_lora_variant(const GemmKArgs& a, int lora, hipStream_t s, dim3 grid) {
  if (lora == 0) hipLaunchKernelGGL((gemm_kernel<WFMT, KN, 0, EPI_BF16, BN, BM>), grid, dim3(NTHREADS), 0, s, a);
  else if (lora == 1) hipLaunchKernelGGL((gemm_kernel<WFMT, KN, 1, EPI_BF16, BN, BM>), grid, dim3(NTHREADS), 0, s, a);
  else hipLaunchKernelGGL((gemm_kernel<WFMT, KN, 2, EPI_BF16, BN, BM>), grid, dim3(NTHREADS), 0, s, a);
}

template <int BN, int BM>
static lsl_status launch_cfg(const GemmDesc& d, GemmKArgs& a, hipStream_t s) {
  a.tiles_m = (int)((d.M + BM - 1) / BM);
  a.tiles_n = (int)((d.N + BN - 1) / BN);
  const int KT = (int)(d.K / BK);
  a.ksplit = 1;
  a.kt_per_split = KT;
  if (d.epi == EPI_ACC32 && d.acc_splits > 1) {
    if (d.y) return set_error(LSL_ERR_UNSUPPORTED, "gemm: split float accumulation has no bf16 copy");
    a.kt_per_split = (KT + d.acc_splits - 1) / d.acc_splits;
    a.ksplit = (KT + a.kt_per_split - 1) / a.kt_per_split;
    if (d.first && a.ksplit != d.acc_splits)  // the first pass must initialise every split
      return set_error(LSL_ERR_UNSUPPORTED, "gemm: %d accumulation splits of %d steps", d.acc_splits, KT);
    a.o32_split = d.o32_split;
  }
  if (d.epi == EPI_BF16) {
    const int S = gemm_splits(d.M, d.N, d.K);
    if (S > 1) {
      if (!d.split_ws) return set_error(LSL_ERR_WORKSPACE, "gemm: split-K scratch missing");
      a.kt_per_split = (KT + S - 1) / S;
      a.ksplit = (KT + a.kt_per_split - 1) / a.kt_per_split;
      a.spart = d.split_ws;
    }
  }
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n * a.ksplit));
  if (d.epi != EPI_BF16) {
    if (d.wfmt != LSL_WFMT_BF16 || d.lora) return set_error(LSL_ERR_UNSUPPORTED, "gemm: CE epilogues take a bf16 weight");
    if (d.epi == EPI_LSE && !d.kn)
      hipLaunchKernelGGL((gemm_kernel<LSL_WFMT_BF16, false, 0, EPI_LSE, BN, BM>), grid, dim3(NTHREADS), 0, s, a);
    else if (d.epi == EPI_CEGRAD && !d.kn)
      hipLaunchKernelGGL((gemm_kernel<LSL_WFMT_BF16, false, 0, EPI_CEGRAD, BN, BM>), grid, dim3(NTHREADS), 0, s, a);
    else if (d.epi == EPI_ACC32 && d.kn)
      hipLaunchKernelGGL((gemm_kernel<LSL_WFMT_BF16, true, 0, EPI_ACC32, BN, BM>), grid, dim3(NTHREADS), 0, s, a);
    else
      return set_error(LSL_ERR_UNSUPPORTED, "gemm: epilogue %d with layout %d", d.epi, (int)d.kn);
    return check_launch("gemm(ce)");
  }
  if (d.wfmt == LSL_WFMT_NF4) {
    if (d.kn) launch_lora_variant<LSL_WFMT_NF4, true, BN, BM>(a, d.lora, s, grid);
    else launch_lora_variant<LSL_WFMT_NF4, false, BN, BM>(a, d.lora, s, grid);
  } else if (d.wfmt == LSL_WFMT_NF4DQ) {
    if (d.kn) launch_lora_variant<LSL_WFMT_NF4DQ, true, BN, BM>(a, d.lora, s, grid);
    else launch_lora_variant<LSL_WFMT_NF4DQ, false, BN, BM>(a, d.lora, s, grid);
  } else {
    if (d.kn) launch_lora_variant<LSL_WFMT_BF16, true, BN, BM>(a, d.lora, s, grid);
    else launch_lora_variant<LSL_WFMT_BF16, false, BN, BM>(a, d.lora, s, grid);
  }
  if (a.ksplit > 1 && !d.defer_reduce) {
    const int64_t n4 = d.M * d.N / 4;
    hipLaunchKernelGGL(gemm_split_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, (const float*)a.spart,
                       a.ksplit, d.M, d.N, d.bias, d.res, d.ldres, d.y, d.ldy);
  }
  return check_launch("gemm");
}

// Tile shape from the problem shape only: 64 weight rows, 256 tokens once there
// are at least 1024 tokens (128 below). Measured on MI355X at the Llama-8B
// layer shapes, this beat 128-row weight tiles and two-deep prefetching: with
// 64 x 64 wave tiles the loop is bound by LDS bandwidth, and the small LDS
// footprint (single buffer, 46 KB) lets three workgroups share a CU.
void gemm_tile_shape(int64_t M, int64_t N, int& bn, int& bm) {
  (void)N;
  bm = M >= 1024 ? 256 : 128;
  bn = 64;
}

// The large-tile kernel takes bf16-epilogue GEMMs with at least BIG_MIN_TILES
// output tiles of 256 x 256 (three quarters of the CUs); smaller ones keep the
// 64-row tiles (with split-K), which fill the chip better. Measured at 1024
// tokens: the input gradient of the Llama-8B down projection (224 tiles) takes
// 174 us here against 205 us with the 64-row tiles.
#ifndef LSL_BIG_MIN_TILES
#define LSL_BIG_MIN_TILES 192
#endif
// Stream-K in the large tile: when the tiles fill less than BIG_MIN_TILES of
// the SK_G workgroups (one per CU) and split-K (below) does not apply, the
// reduction steps of all tiles are dealt out evenly to SK_G workgroups instead,
// as long as each gets at least SK_MIN_STEPS steps. Each split tile costs a
// float32 partial per segment (256 KiB, written and read back once through one
// CU), about 30 us per launch in all. Measured at 1024 tokens of the Llama-8B
// layer before split-K existed: q|k|v forward 89 -> 87 us and input gradient
// 92 -> 82 us (24 steps each) against the 64-row tiles, but 65 -> 75 us for the
// o projection (16 steps) and 138 -> 160 us for the down projection's input
// gradient (224 tiles, one per workgroup). Since then it serves shapes below
// 1024 tokens (the Llama-8B layer at 512 tokens: the down forward and the
// gate|up and down input gradients). SK_G is the CU count of MI355X, so that
// the plan depends on the GEMM's shape only.
#ifndef LSL_SK_G
#define LSL_SK_G 256
#endif
#ifndef LSL_SK_MIN_STEPS
#define LSL_SK_MIN_STEPS 20
#endif
static_assert(LSL_SK_G % 8 == 0, "stream-K workgroups are dealt to 8 XCDs");
static_assert(LSL_BIG_MIN_TILES <= LSL_SK_G, "stream-K takes fewer tiles than workgroups");
// Split-K in the large tile: a GEMM of at least 1024 tokens with fewer than
// BIG_MIN_TILES tiles takes S = SK_G / tiles reduction splits (at least
// BIG_KSPLIT_MIN_STEPS K-steps each) when that fills at least BIG_MIN_TILES
// workgroups; each split's float32 partial is summed in split order by
// gemm_split_reduce, which reads them with the whole chip. This comes before
// stream-K: at 1024 tokens of the Llama-8B layer (A/B on one box, HIP events)
// the down forward went 159 -> 142 us, the q|k|v input gradient 83 -> 79 us and
// the gate|up input gradient 254 -> 248 us against stream-K, and the o
// projection 69.6 -> 66.5 us forward (69.2 -> 64.3 us input gradient) against
// the 64-row tiles.
#ifndef LSL_BIG_KSPLIT_MIN_STEPS
#define LSL_BIG_KSPLIT_MIN_STEPS 8
#endif
static int big_ksplit(int64_t M, int64_t tiles, int64_t K) {
  if (tiles <= 0 || M < 1024) return 1;
  int64_t S = LSL_SK_G / tiles;
  const int64_t KT = K / BK;
  if (S > KT / LSL_BIG_KSPLIT_MIN_STEPS) S = KT / LSL_BIG_KSPLIT_MIN_STEPS;
  if (S < 2 || tiles * S < LSL_BIG_MIN_TILES) return 1;
  const int64_t per = (KT + S - 1) / S;
  return (int)((KT + per - 1) / per);
}
// 0: the 64-row tiles; 1: the large tile, one workgroup per tile; -1: the
// large tile, stream-K over LSL_SK_G workgroups; 2: the large tile, split-K
static int gemm_big_plan(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + big::BM - 1) / big::BM) * ((N + big::BN - 1) / big::BN);
  if (tiles == 0) return 0;
  if (tiles >= LSL_BIG_MIN_TILES) return 1;
  if (big_ksplit(M, tiles, K) > 1) return 2;
  const int64_t units = tiles * (K / BK);
  // (fewer tiles than workgroups: a workgroup's units span at most two tiles;
  // units * SK_G < 2^31 keeps the kernel's unit arithmetic in 32 bits)
  if (units >= (int64_t)LSL_SK_MIN_STEPS * LSL_SK_G && units * LSL_SK_G < ((int64_t)1 << 31)) return -1;
  return 0;
}

size_t gemm_counts_needed(int64_t M, int64_t N, int64_t K) {
  if (gemm_big_plan(M, N, K) != -1) return 0;
  return (size_t)(((M + big::BM - 1) / big::BM) * ((N + big::BN - 1) / big::BN));
}

template <int WFMT, bool KN>
static void launch_big(const GemmKArgs& a, int lora, hipStream_t s, dim3 grid) {
  if (a.sk_g) {
    if (lora == 0) hipLaunchKernelGGL((gemm_sk_kernel<WFMT, KN, 0>), grid, dim3(big::NT), 0, s, a);
    else if (lora == 1) hipLaunchKernelGGL((gemm_sk_kernel<WFMT, KN, 1>), grid, dim3(big::NT), 0, s, a);
    else hipLaunchKernelGGL((gemm_sk_kernel<WFMT, KN, 2>), grid, dim3(big::NT), 0, s, a);
    return;
  }
  if (lora == 0) hipLaunchKernelGGL((gemm_big_kernel<WFMT, KN, 0>), grid, dim3(big::NT), 0, s, a);
  else if (lora == 1) hipLaunchKernelGGL((gemm_big_kernel<WFMT, KN, 1>), grid, dim3(big::NT), 0, s, a);
  else hipLaunchKernelGGL((gemm_big_kernel<WFMT, KN, 2>), grid, dim3(big::NT), 0, s, a);
}

static lsl_status launch_big_cfg(const GemmDesc& d, GemmKArgs& a, hipStream_t s, int plan) {
  a.tiles_m = (int)((d.M + big::BM - 1) / big::BM);
  a.tiles_n = (int)((d.N + big::BN - 1) / big::BN);
  a.ksplit = 1;
  a.kt_per_split = (int)(d.K / BK);
  a.sk_g = 0;
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n));
  if (plan == 2) {
    const int S = big_ksplit(d.M, (int64_t)a.tiles_m * a.tiles_n, d.K);
    const int KT = (int)(d.K / BK);
    if (!d.split_ws) return set_error(LSL_ERR_WORKSPACE, "gemm: split-K scratch missing");
    a.kt_per_split = (KT + S - 1) / S;
    a.ksplit = (KT + a.kt_per_split - 1) / a.kt_per_split;
    a.spart = d.split_ws;
    grid = dim3((unsigned)(a.tiles_m * a.tiles_n * a.ksplit));
  }
  if (plan == -1) {
    // at most two segments per workgroup (the kernel keeps two pending sums)
    if ((int64_t)a.tiles_m * a.tiles_n >= LSL_SK_G)
      return set_error(LSL_ERR_UNSUPPORTED, "gemm: stream-K needs fewer tiles than workgroups");
    a.sk_g = LSL_SK_G;
    a.spart = d.split_ws;
    a.cnt = d.cnt;
    grid = dim3(LSL_SK_G);
  }
  if (d.wfmt == LSL_WFMT_NF4) {
    if (d.kn) launch_big<LSL_WFMT_NF4, true>(a, d.lora, s, grid);
    else launch_big<LSL_WFMT_NF4, false>(a, d.lora, s, grid);
  } else if (d.wfmt == LSL_WFMT_NF4DQ) {
    if (d.kn) launch_big<LSL_WFMT_NF4DQ, true>(a, d.lora, s, grid);
    else launch_big<LSL_WFMT_NF4DQ, false>(a, d.lora, s, grid);
  } else {
    if (d.kn) launch_big<LSL_WFMT_BF16, true>(a, d.lora, s, grid);
    else launch_big<LSL_WFMT_BF16, false>(a, d.lora, s, grid);
  }
  if (a.ksplit > 1 && !d.defer_reduce) {
    const int64_t n4 = d.M * d.N / 4;
    hipLaunchKernelGGL(gemm_split_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, (const float*)a.spart,
                       a.ksplit, d.M, d.N, d.bias, d.res, d.ldres, d.y, d.ldy);
  }
  return check_launch("gemm(256 x 256 tiles)");
}

// Cross-entropy GEMMs (bf16 weight, no LoRA) in the large tile: the logits
// passes (forward log-sum-exp, gradient chunk) when the vocabulary gives enough
// tiles unsplit, the dH accumulation when its splits fill the chip.
bool gemm_ce_big(int64_t M, int64_t N, int64_t K) {
  (void)K;
  return ((M + big::BM - 1) / big::BM) * ((N + big::BN - 1) / big::BN) >= LSL_BIG_MIN_TILES;
}

int gemm_ce_tile_n(int64_t M, int64_t N, int64_t K) {
  if (gemm_ce_big(M, N, K)) return big::BN;
  int bn, bm;
  gemm_tile_shape(M, N, bn, bm);
  return bn;
}

// The float32 dH accumulation of the cross-entropy backward takes the large
// tile with its reduction split so that about BIG_SPLIT_TARGET workgroups run,
// each at least BIG_SPLIT_MIN_STEPS K-steps, when the splits fill the chip.
#ifndef LSL_BIG_SPLIT_MIN_TILES
#define LSL_BIG_SPLIT_MIN_TILES 32
#endif
#ifndef LSL_BIG_SPLIT_MIN_STEPS
#define LSL_BIG_SPLIT_MIN_STEPS 48
#endif
#ifndef LSL_BIG_SPLIT_TARGET
#define LSL_BIG_SPLIT_TARGET 256
#endif
static bool acc32_big(int64_t M, int64_t N, int S) {
  const int64_t tiles = ((M + big::BM - 1) / big::BM) * ((N + big::BN - 1) / big::BN);
  return tiles >= LSL_BIG_SPLIT_MIN_TILES && tiles * S >= LSL_BIG_MIN_TILES;
}

int gemm_acc32_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t steps = K / BK;
  const int64_t tiles = ((M + big::BM - 1) / big::BM) * ((N + big::BN - 1) / big::BN);
  if (tiles == 0) return 1;
  if (tiles >= LSL_BIG_SPLIT_MIN_TILES) {
    int64_t S = (LSL_BIG_SPLIT_TARGET + tiles - 1) / tiles;
    if (S > steps / LSL_BIG_SPLIT_MIN_STEPS) S = steps / LSL_BIG_SPLIT_MIN_STEPS;
    if (S < 1) S = 1;
    if (acc32_big(M, N, (int)S)) return (int)S;
  }
  // the 64-row tiles: about 768 workgroups, at least 32 K-steps each
  int bn, bm;
  gemm_tile_shape(M, N, bn, bm);
  const int64_t t64 = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  int64_t S = (768 + t64 - 1) / t64;
  if (S > steps / 32) S = steps / 32;
  return S < 1 ? 1 : (int)S;
}

static lsl_status launch_big_ce(const GemmDesc& d, GemmKArgs& a, hipStream_t s) {
  a.tiles_m = (int)((d.M + big::BM - 1) / big::BM);
  a.tiles_n = (int)((d.N + big::BN - 1) / big::BN);
  const int KT = (int)(d.K / BK);
  a.ksplit = 1;
  a.kt_per_split = KT;
  if (d.epi == EPI_ACC32 && d.acc_splits > 1) {
    if (d.y) return set_error(LSL_ERR_UNSUPPORTED, "gemm: split float accumulation has no bf16 copy");
    a.kt_per_split = (KT + d.acc_splits - 1) / d.acc_splits;
    a.ksplit = (KT + a.kt_per_split - 1) / a.kt_per_split;
    if (d.first && a.ksplit != d.acc_splits)  // the first pass must initialise every split
      return set_error(LSL_ERR_UNSUPPORTED, "gemm: %d accumulation splits of %d steps", d.acc_splits, KT);
    a.o32_split = d.o32_split;
  }
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n * a.ksplit));
  if (d.epi == EPI_LSE)
    hipLaunchKernelGGL((gemm_big_kernel<LSL_WFMT_BF16, false, 0, EPI_LSE>), grid, dim3(big::NT), 0, s, a);
  else if (d.epi == EPI_CEGRAD)
    hipLaunchKernelGGL((gemm_big_kernel<LSL_WFMT_BF16, false, 0, EPI_CEGRAD>), grid, dim3(big::NT), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_big_kernel<LSL_WFMT_BF16, true, 0, EPI_ACC32>), grid, dim3(big::NT), 0, s, a);
  return check_launch("gemm(ce, 256 x 256 tiles)");
}

// Split-K for GEMMs with few output tiles: enough reduction splits to give
// about SPLIT_TARGET workgroups, each taking at least SPLIT_MIN_STEPS K-steps.
#ifndef LSL_SPLIT_TARGET
#define LSL_SPLIT_TARGET 768
#endif
#ifndef LSL_SPLIT_MIN_STEPS
#define LSL_SPLIT_MIN_STEPS 32
#endif
int gemm_splits(int64_t M, int64_t N, int64_t K) {
  int bn, bm;
  gemm_tile_shape(M, N, bn, bm);
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int64_t steps = K / BK;
  if (tiles == 0) return 1;  // empty output
  const int plan = gemm_big_plan(M, N, K);
  if (plan == 2) return big_ksplit(M, ((M + big::BM - 1) / big::BM) * ((N + big::BN - 1) / big::BN), K);
  if (plan != 0) return 1;  // the large tile, unsplit or stream-K: no separate reduction pass
  int64_t S = (LSL_SPLIT_TARGET + tiles - 1) / tiles;
  if (S > steps / LSL_SPLIT_MIN_STEPS) S = steps / LSL_SPLIT_MIN_STEPS;
  if (S < 2) return 1;
  const int64_t per = (steps + S - 1) / S;
  return (int)((steps + per - 1) / per);
}

size_t gemm_split_bytes(int64_t M, int64_t N, int64_t K) {
  // stream-K: workgroup w's partial of tile t sits in slot w + t (the sum
  // rises by at least one from each segment of the schedule to the next)
  if (const size_t tiles = gemm_counts_needed(M, N, K)) return (LSL_SK_G + tiles - 1) * big::SLOT * sizeof(float);
  const int S = gemm_splits(M, N, K);
  return S > 1 ? (size_t)S * M * N * sizeof(float) : 0;
}

// Every condition gemm_launch can reject, checked without launching anything,
// so that an entry point can validate all of its GEMMs before the first launch.
lsl_status gemm_check(const GemmDesc& d) {
  if (d.M == 0 || d.N == 0) return LSL_OK;
  if (d.K % BK || d.N % 8 || d.K == 0)
    return set_error(LSL_ERR_UNSUPPORTED, "gemm: K (%lld) must be a multiple of 64 and N (%lld) of 8",
                     (long long)d.K, (long long)d.N);
  if (d.lora && (d.kl <= 0 || d.kl > 64 || d.kl % 8))
    return set_error(LSL_ERR_UNSUPPORTED, "gemm: LoRA width %d must be a multiple of 8 in [8, 64]", d.kl);
  if (d.wfmt != LSL_WFMT_BF16 && d.kn && d.N % 64)
    return set_error(LSL_ERR_UNSUPPORTED, "gemm: NF4 transposed operand needs N %% 64 == 0");
  if (d.kwrap && (d.kwrap % BK || d.K > 2 * d.kwrap || !d.kn))
    return set_error(LSL_ERR_UNSUPPORTED, "gemm: wrapped reduction needs kn, kwrap %% 64 == 0 and K <= 2 kwrap");
  // every operand is addressed through 32-bit buffer offsets (with one tile of slack)
  const int64_t lim = ((int64_t)1 << 32) - 1;
  if ((d.M + 256) * d.ldx * 2 > lim || (d.N + 128) * d.K * 2 > lim)
    return set_error(LSL_ERR_UNSUPPORTED, "gemm: operand larger than 4 GiB");
  if (d.epi == EPI_BF16) {
    if (gemm_split_bytes(d.M, d.N, d.K) && !d.split_ws) return set_error(LSL_ERR_WORKSPACE, "gemm: split-K scratch missing");
    if (gemm_counts_needed(d.M, d.N, d.K) && !d.cnt) return set_error(LSL_ERR_WORKSPACE, "gemm: stream-K arrival counts missing");
    return LSL_OK;
  }
  if (d.wfmt != LSL_WFMT_BF16 || d.lora) return set_error(LSL_ERR_UNSUPPORTED, "gemm: CE epilogues take a bf16 weight");
  if (!((d.epi == EPI_LSE && !d.kn) || (d.epi == EPI_CEGRAD && !d.kn) || (d.epi == EPI_ACC32 && d.kn)))
    return set_error(LSL_ERR_UNSUPPORTED, "gemm: epilogue %d with layout %d", d.epi, (int)d.kn);
  if (d.epi == EPI_ACC32 && d.acc_splits > 1) {
    if (d.y) return set_error(LSL_ERR_UNSUPPORTED, "gemm: split float accumulation has no bf16 copy");
    const int KT = (int)(d.K / BK);
    const int per = (KT + d.acc_splits - 1) / d.acc_splits;
    if (d.first && (KT + per - 1) / per != d.acc_splits)  // the first pass must initialise every split
      return set_error(LSL_ERR_UNSUPPORTED, "gemm: %d accumulation splits of %d steps", d.acc_splits, KT);
  }
  return LSL_OK;
}

lsl_status gemm_launch(const GemmDesc& d, hipStream_t s) {
  if (d.M == 0 || d.N == 0) return LSL_OK;
  LSL_TRY(gemm_check(d));
  GemmKArgs a{};
  a.x = d.x; a.ldx = d.ldx;
  a.wb = d.wb; a.wq = d.wq; a.wa = d.wa; a.wq8 = d.wq8; a.wsc = d.wsc;
  a.M = d.M; a.N = d.N; a.K = d.K;
  a.la = d.la; a.ldla = d.ldla; a.kl = d.kl; a.lb = d.lb; a.r = d.r; a.nseg = d.nseg;
  for (int i = 0; i < 4; ++i) a.seg_end[i] = d.seg_end[i];
  a.scale = d.scale;
  a.y = d.y; a.ldy = d.ldy; a.res = d.res; a.ldres = d.ldres; a.bias = d.bias;
  const Nf4Table& t = nf4_table();
  for (int i = 0; i < 16; ++i) a.cb[i] = t.cb[i];
  a.labels = d.labels; a.lse = d.lse; a.nvalid = d.nvalid; a.part = (float2*)d.part; a.zlab = d.zlab;
  a.y2 = d.y2; a.gscale = d.gscale; a.ignore = d.ignore; a.vocab_off = d.vocab_off; a.vocab = d.vocab;
  a.out32 = d.out32; a.ldo32 = d.ldo32; a.first = d.first; a.kwrap = d.kwrap;
  if (d.epi == EPI_BF16 && !d.kwrap)
    if (const int b = gemm_big_plan(d.M, d.N, d.K)) return launch_big_cfg(d, a, s, b);
  if (d.wfmt == LSL_WFMT_BF16 && !d.lora && !d.kwrap) {
    if ((d.epi == EPI_LSE || d.epi == EPI_CEGRAD) && !d.kn && gemm_ce_big(d.M, d.N, d.K))
      return launch_big_ce(d, a, s);
    if (d.epi == EPI_ACC32 && d.kn && acc32_big(d.M, d.N, d.acc_splits)) return launch_big_ce(d, a, s);
  }
  int bn, bm;
  gemm_tile_shape(d.M, d.N, bn, bm);
  return bm == 256 ? launch_cfg<64, 256>(d, a, s) : launch_cfg<64, 128>(d, a, s);
}

}  // namespace lsl
