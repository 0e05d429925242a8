// Causal grouped-query attention on gfx950 bf16 MFMA (16x16x32), head_dim 64 or 128.
//
// Forward (one pass, online softmax): a workgroup holds one (sequence, kv head,
// 16-query tile); its waves are the G query heads of that kv head (two per head
// at head_dim 128, each on half of every key tile), so the K/V tiles staged in
// LDS are shared by the whole group and all waves see the same causal range. Scores are computed transposed (S^T = K Q^T) so that each lane
// owns one query column: the running max/sum of the online softmax need one
// value per lane, and the probabilities feed the P V product straight from
// registers (the reduction index of an MFMA may be permuted freely as long as
// both operands use the same permutation; the V^T operand is read in that order
// from the row-major V tile with transposing LDS reads).
// The log-sum-exp per query row is saved for the backward.
//
// Backward (the standard gradient of softmax attention, recomputing P from the
// saved log-sum-exp): D_q = sum_d dO O; a dK/dV kernel owns a 32-key tile and
// sums over the G query heads (split over up to four head groups of waves,
// added in a fixed order at the end) and all query tiles; a dQ kernel owns
// query tiles like the forward. No atomics; every tile is staged row-major.
#include "common.h"
#include "api_util.h"

namespace lsl {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Block -> work item: the hardware deals consecutive blocks to the 8 XCDs in
// turn; XCD x gets the items [x n / 8, (x + 1) n / 8) (rounded), so that the
// blocks of one (sequence, kv head), which read the same K and V tiles, share
// an XCD's L2 instead of every XCD caching every head.
LSL_DEV int xcd_item(int b, int n) {
  const int per = n >> 3, rem = n & 7, x = b & 7, i = b >> 3;
  return x * per + min(x, rem) + i;
}

struct AttnArgs {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  int64_t ldq, ldk;
  const uint16_t* o; const uint16_t* dout;   // backward
  float* o32;                                // optional float32 copy of the output [T x n_q d]
  const float* lse; const float* dsum;       // [batch][n_q][seq]
  uint16_t* out; int64_t ldo;                // forward output o, or dq
  float* lse_out; float* dsum_out;
  uint16_t* dk; uint16_t* dv;
  int batch, seq, n_q, n_kv, group;
  float scale_log2;                          // log2(e) / sqrt(d)
  float scale;                               // 1 / sqrt(d)
  // balanced dK/dV (dkv_balanced): float32 partial slots and one arrival count
  // per (sequence, kv head, key tile), zeroed by the dsum kernel
  float* dkv_part; unsigned* dkv_cnt;
};

LSL_DEV f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 2^x on the hardware exponential (results below 2^-126 flush to zero, which
// a probability of that size may); exp2_ftz(-inf) = 0.
LSL_DEV float exp2_ftz(float x) { return __builtin_amdgcn_exp2f(x); }
LSL_DEV bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
LSL_DEV bf16x8 pack8(const f32x4& lo, const f32x4& hi) {
  return __builtin_bit_cast(bf16x8, u32x4{pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3])});
}
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): about 16 significant bits
// through two bf16 MFMAs, used where a reduction cancels (dS in dK and dQ).
LSL_DEV void split8(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
  hi = pack8(a, b);
  u32x4 h = __builtin_bit_cast(u32x4, hi);
  f32x4 ra = f32x4{a[0] - lo_bf(h[0]), a[1] - hi_bf(h[0]), a[2] - lo_bf(h[1]), a[3] - hi_bf(h[1])};
  f32x4 rb = f32x4{b[0] - lo_bf(h[2]), b[1] - hi_bf(h[2]), b[2] - lo_bf(h[3]), b[3] - hi_bf(h[3])};
  lo = pack8(ra, rb);
}

// A 64-row x D tile of a strided bf16 matrix moved global -> registers -> LDS
// (row-major, row stride D + 8) by the NT threads of a workgroup. Rows past
// `valid` read a clamped in-range row (callers mask them out), so the loads are
// branch-free and are only waited for at the LDS store: load() for the next
// tile is issued before the current one is computed.
template <int D, int NT>
struct TileStage {
  static constexpr int CHUNKS = 64 * D / 8;
  static constexpr int CPT = (CHUNKS + NT - 1) / NT;
  u32x4 v[CPT];
  LSL_DEV void load(const uint16_t* __restrict__ src, int64_t ld, int r0, int valid, int tid) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CHUNKS % NT == 0 || c < CHUNKS) {
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        const int64_t r = min(r0 + row, valid - 1);
        v[i] = *reinterpret_cast<const u32x4*>(src + r * ld + col);
      }
    }
  }
  LSL_DEV void store(uint16_t* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CHUNKS % NT == 0 || c < CHUNKS) {
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        *reinterpret_cast<u32x4*>(dst + row * (D + 8) + col) = v[i];
      }
    }
  }
};

// The same 64-row tile stage through a buffer descriptor over the sequence's
// rows: the per-thread offsets are set up once and a tile adds one scalar row
// offset; rows at or past the end read zeros (they meet only masked scores or
// zero probabilities).
template <int D, int NT>
struct BufTileStage {
  static constexpr int CHUNKS = 64 * D / 8;
  static constexpr int CPT = (CHUNKS + NT - 1) / NT;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff[CPT];
  u32x4 v[CPT];
  // src: row 0 of the sequence (head column offset included), rows rows of stride ld
  LSL_DEV void init(const uint16_t* src, int64_t ld, int rows, int tid) {
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), (short)0,
                                           (int)(uint32_t)((int64_t)rows * ld * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      voff[i] = (uint32_t)((row * ld + col) * 2);
    }
  }
  // rows r0 .. r0 + 63; r0 ld 2 is added to the vector offset, which the range
  // check covers
  LSL_DEV void load(int64_t ld, int r0, int tid) {
    const uint32_t o = (uint32_t)(r0 * ld * 2);
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (CHUNKS % NT == 0 || tid + i * NT < CHUNKS)
        v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i] + o, 0, 0));
  }
  template <int LDD>
  LSL_DEV void store(uint16_t* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CHUNKS % NT == 0 || c < CHUNKS) {
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        *reinterpret_cast<u32x4*>(dst + row * LDD + col) = v[i];
      }
    }
  }
};

// ---------------------------------------------------------------- forward
// grid (ceil(seq / (16 NQS)), n_kv, batch), block group*64 threads; wave = query
// head, 16 NQS queries per wave.
template <int D, int NQS, int NW>
__global__ __launch_bounds__(64 * NW) void attn_fwd_kernel(const AttnArgs a) {
  // K rows are read 16 at a time in 16-byte chunks (a 16-byte skew per row
  // spreads 16 rows over all banks); V is read with transposing reads of 8
  // rows x 32 bytes per half-wave (a 32-byte skew per row spreads those)
  constexpr int QT = 16 * NQS, LD = D + 8, LDV = D + 16;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * LDV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // item (b n_kv + kvh) n_qt + n_qt - 1 - qt: heaviest (latest) query tiles first
  const int n_qt = (a.seq + QT - 1) / QT;
  const int item = xcd_item((int)blockIdx.x, (int)gridDim.x);
  const int bk = item / n_qt, qt = n_qt - 1 - (item - bk * n_qt);
  const int kvh = bk % a.n_kv, b = bk / a.n_kv;
  const int h = kvh * a.group + wave;
  const int q0 = qt * QT;
  const int64_t rowbase = (int64_t)b * a.seq;
  const uint16_t* qp = a.q + rowbase * a.ldq + (int64_t)h * D;
  const uint16_t* kp = a.k + rowbase * a.ldk + (int64_t)kvh * D;
  const uint16_t* vp = a.v + rowbase * a.ldk + (int64_t)kvh * D;
  const int g = lane >> 4, c16 = lane & 15;

  bf16x8 qf[NQS][D / 32];
#pragma unroll
  for (int qs = 0; qs < NQS; ++qs) {
    const int64_t q = min(q0 + qs * 16 + c16, a.seq - 1);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qf[qs][ks] = ld8(qp + q * a.ldq + ks * 32 + g * 8);
  }
  f32x4 o[D / 16][NQS];
#pragma unroll
  for (int i = 0; i < D / 16; ++i)
#pragma unroll
    for (int qs = 0; qs < NQS; ++qs) o[i][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[NQS], l[NQS];
#pragma unroll
  for (int qs = 0; qs < NQS; ++qs) m[qs] = -INFINITY, l[qs] = 0.f;

  const int qmax = min(q0 + QT - 1, a.seq - 1);
  const int ntiles = qmax / 64 + 1;
  BufTileStage<D, 64 * NW> kst, vst;
  kst.init(kp, a.ldk, a.seq, tid);
  vst.init(vp, a.ldk, a.seq, tid);
  kst.load(a.ldk, 0, tid);
  vst.load(a.ldk, 0, tid);
  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = j * 64;
    kst.template store<LD>(Ks, tid);
    vst.template store<LDV>(Vs, tid);
    __syncthreads();
    if (j + 1 < ntiles) {
      kst.load(a.ldk, kv0 + 64, tid);
      vst.load(a.ldk, kv0 + 64, tid);
    }
    // S^T: lane holds kv = kv0 + kvs*16 + 4g + i, q = q0 + qs*16 + c16
    f32x4 sc[4][NQS];
#pragma unroll
    for (int kvs = 0; kvs < 4; ++kvs) {
#pragma unroll
      for (int qs = 0; qs < NQS; ++qs) sc[kvs][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const bf16x8 kf = ld8(Ks + (kvs * 16 + c16) * LD + ks * 32 + g * 8);
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) sc[kvs][qs] = mfma(kf, qf[qs][ks], sc[kvs][qs]);
      }
    }
    // only the tiles that reach the diagonal (or the sequence's end) are masked:
    // below it every key kv <= kv0 + 63 < q0 <= q is visible and inside the sequence
    const bool diag = kv0 + 63 > q0;
    bf16x8 pf[NQS][2], pl[NQS][2];
#pragma unroll
    for (int qs = 0; qs < NQS; ++qs) {
      const int q = q0 + qs * 16 + c16;
      if (diag) {
#pragma unroll
        for (int kvs = 0; kvs < 4; ++kvs)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kv = kv0 + kvs * 16 + g * 4 + i;
            if (!(kv <= q && kv < a.seq)) sc[kvs][qs][i] = -INFINITY;
          }
      }
      // the row maximum of the raw scores, scaled once (scaling by a positive
      // constant commutes with the maximum)
      float mt = fmaxf(fmaxf(sc[0][qs][0], sc[0][qs][1]), fmaxf(sc[0][qs][2], sc[0][qs][3]));
#pragma unroll
      for (int kvs = 1; kvs < 4; ++kvs)
        mt = fmaxf(mt, fmaxf(fmaxf(sc[kvs][qs][0], sc[kvs][qs][1]), fmaxf(sc[kvs][qs][2], sc[kvs][qs][3])));
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mn = fmaxf(m[qs], mt * a.scale_log2);  // finite: key 0 is visible to every query
      float ls = 0.f;
#pragma unroll
      for (int kvs = 0; kvs < 4; ++kvs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = exp2_ftz(fmaf(sc[kvs][qs][i], a.scale_log2, -mn));
          sc[kvs][qs][i] = pv;
          ls += pv;
        }
      // the running sums rescale only where some lane's maximum moved (exp2(0) = 1)
      if (__builtin_amdgcn_ballot_w64(mn != m[qs])) {
        const float alpha = exp2_ftz(m[qs] - mn);
        l[qs] *= alpha;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[ds][qs][i] *= alpha;
      }
      m[qs] = mn;
      l[qs] += ls;
      split8(sc[0][qs], sc[1][qs], pf[qs][0], pl[qs][0]);
      split8(sc[2][qs], sc[3][qs], pf[qs][1], pl[qs][1]);
    }
    // O^T += V^T P^T (reduction over the 64 keys in the permuted order of pf),
    // with P as a hi + lo pair of bf16 values: O then carries about 16
    // significant bits of P, so the backward's rowsum(dO O) is accurate where
    // dP - rowsum cancels
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 vf = ld_tr8(Vs, LDV, kk * 32, ds * 16, lane);
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
          o[ds][qs] = mfma(vf, pf[qs][kk], o[ds][qs]);
          o[ds][qs] = mfma(vf, pl[qs][kk], o[ds][qs]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int qs = 0; qs < NQS; ++qs) {
    float lt = l[qs] + __shfl_xor(l[qs], 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int q = q0 + qs * 16 + c16;
    if (q >= a.seq) continue;
    const float inv = 1.0f / lt;
    uint16_t* op = a.out + (rowbase + q) * a.ldo + (int64_t)h * D;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const f32x4& r = o[ds][qs];
      *reinterpret_cast<u32x2*>(op + ds * 16 + g * 4) = u32x2{pack2(r[0] * inv, r[1] * inv), pack2(r[2] * inv, r[3] * inv)};
      if (a.o32)
        *reinterpret_cast<f32x4*>(a.o32 + (rowbase + q) * ((int64_t)a.n_q * D) + (int64_t)h * D + ds * 16 + g * 4) =
            f32x4{r[0] * inv, r[1] * inv, r[2] * inv, r[3] * inv};
    }
    if (g == 0) a.lse_out[((int64_t)b * a.n_q + h) * a.seq + q] = (m[qs] + log2f(lt)) * LN2;
  }
}

// ---------------------------------------------------------------- forward, head_dim 128
// The same work split, with the K and V tiles moved global -> LDS by buffer loads
// that write LDS directly (no registers, no LDS store instructions), in two
// stages, and one barrier per 64-key tile. Rows are unpadded (256 bytes); the
// 16-byte chunk c of row r sits at position c ^ kv_sw(r). kv_sw is linear over
// the bits of r mod 16 (images 8, 4, 3, 6 of bits 0-3); with it both the row-wise
// K reads (16 rows, chunks ks*4 + g) and the transposing V reads (4 rows x two
// chunks per 16 lanes) ran with no LDS bank-conflict cycles on gfx950
// (SQ_LDS_BANK_CONFLICT), where rows padded by 16 bytes, the identity or a
// (r mod 8) << 1 swizzle left conflicts in one of the two.
LSL_DEV int kv_sw(int r) { return ((r & 1) ? 8 : 0) ^ ((r & 2) ? 4 : 0) ^ ((r & 4) ? 3 : 0) ^ ((r & 8) ? 6 : 0); }

typedef __attribute__((address_space(3))) void att_lds_void;

// one 64 x 128 tile = 16 loads of 4 rows (64 lanes x 16 bytes each); wave w
// issues loads w, w + NW, ... of K and of V. Lane l of load i fills position
// l % 16 of row 4 i + l / 16, i.e. global chunk (l % 16) ^ kv_sw(row).
template <int NW>
struct KvDma {
  static constexpr int PER = (16 + NW - 1) / NW;
  uint32_t voff[PER];
  int wave;
  LSL_DEV void init(int64_t ld, int w, int lane) {
    wave = w;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int r = 4 * (w + i * NW) + (lane >> 4);
      voff[i] = (uint32_t)(((int64_t)r * ld + (((lane & 15) ^ kv_sw(r)) * 8)) * 2);
    }
  }
  // tile rows r0 .. r0 + 63: r0 ld 2 goes into the vector offset, which the
  // descriptor's range check covers (rows at or past the end read zeros)
  LSL_DEV void issue(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint32_t r0off, uint16_t* ks,
                     uint16_t* vs) const {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ins = wave + i * NW;
      if (ins < 16) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (att_lds_void*)(ks + ins * 512), 16, voff[i] + r0off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (att_lds_void*)(vs + ins * 512), 16, voff[i] + r0off, 0, 0, 0);
      }
    }
#else
    (void)rk; (void)rv; (void)r0off; (void)ks; (void)vs;
#endif
  }
};

// V^T operand from the swizzled V tile (as ld_tr8: lane l, g = l / 16, gets
// column c0 + l % 16 at rows r0 + 4 g + s and r0 + 16 + 4 g + s, s < 4)
LSL_DEV bf16x8 ld_tr8_sw(const uint16_t* tile, int r0, int c0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int r = r0 + 4 * g + (j >> 2);
  const int chunk = (c0 >> 3) + ((j & 3) >> 1);
  const uint16_t* p = tile + r * 128 + ((chunk ^ kv_sw(r)) << 3) + 4 * (j & 1);
  const u32x2 x = ld_tr4(p), y = ld_tr4(p + 16 * 128);  // kv_sw(r + 16) = kv_sw(r)
  return __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], y[0], y[1]});
}

// the causal mask of a diagonal tile: score kb*16 + 4g + i of the lane (from the
// wave's first key) is visible when that offset is at most lim (the lane's last
// visible key, its query or the sequence's last key, minus the wave's first key
// and 4g)
template <int KB>
LSL_DEV void mask_tile(f32x4 (&sc)[KB], int lim) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (kb * 16 + i > lim) sc[kb][i] = -INFINITY;
}
// maximum / sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four row groups of
// a 16 x 16 block) by two cross-row swaps
LSL_DEV float max_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
LSL_DEV float sum_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The running maximum is moved (and O, l rescaled) only when a tile's maximum
// exceeds it by more than 2^RESCALE_LOG2 in probability: until then the
// probabilities are taken against the old maximum and stay below 2^8, far from
// float32 or bf16 overflow; the log-sum-exp m + log2(l) is the same either way.
constexpr float RESCALE_LOG2 = 8.f;

// grid (ceil(seq / 16), n_kv, batch) as one dimension, block NW KH waves: wave
// w = kh NW + hw is query head hw of the kv head for keys kv0 + 64 kh / KH ..
// of each 64-key tile (KH = 2: each wave takes half of every tile, and the two
// halves' (max, sum, output) are merged at the end in a fixed order).
template <int NW, int KH>
__global__ __launch_bounds__(64 * NW * KH) void attn_fwd_dma_kernel(const AttnArgs a) {
  constexpr int D = 128, QT = 16, NWT = NW * KH, KB = 4 / KH;  // 16-key blocks per wave and tile
  // two stages as separate arrays: the stage being read and the one being
  // filled are distinct objects, so reads of one need not wait for the other's loads
  __shared__ __attribute__((aligned(16))) uint16_t K0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t K1[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t V1[64 * D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = wave % NW, kh = wave / NW;
  // item (b n_kv + kvh) n_qt + n_qt - 1 - qt: heaviest (latest) query tiles first
  const int n_qt = (a.seq + QT - 1) / QT;
  const int item = xcd_item((int)blockIdx.x, (int)gridDim.x);
  const int bk = item / n_qt, qt = n_qt - 1 - (item - bk * n_qt);
  const int kvh = bk % a.n_kv, b = bk / a.n_kv;
  const int h = kvh * a.group + hw;
  const int q0 = qt * QT;
  const int64_t rowbase = (int64_t)b * a.seq;
  const uint16_t* qp = a.q + rowbase * a.ldq + (int64_t)h * D;
  const uint16_t* kp = a.k + rowbase * a.ldk + (int64_t)kvh * D;
  const uint16_t* vp = a.v + rowbase * a.ldk + (int64_t)kvh * D;
  const int g = lane >> 4, c16 = lane & 15;

  const int qmax = min(q0 + QT - 1, a.seq - 1);
  const int ntiles = qmax / 64 + 1;
  const uint32_t seqbytes = (uint32_t)((int64_t)a.seq * a.ldk * 2);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kp), (short)0, (int)seqbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vp), (short)0, (int)seqbytes, 0x00020000);
  KvDma<NWT> dma;
  dma.init(a.ldk, wave, lane);
  dma.issue(rk, rv, 0, K0, V0);

  bf16x8 qf[D / 32];
  {
    const int64_t q = min(q0 + c16, a.seq - 1);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qf[ks] = ld8(qp + q * a.ldq + ks * 32 + g * 8);
  }
  f32x4 o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // running maximum (scaled by log2 e / sqrt d) and the lane's partial sum
  const int q = q0 + c16;
  const int qlast = min(q, a.seq - 1);  // the lane's last visible key

  // one 64-key tile from stage (K, V) while the next tile's loads fill (Kn, Vn)
  auto tile = [&](const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, uint16_t* Kn, uint16_t* Vn,
                  int j) {
    const int kv0 = j * 64, kb0 = kv0 + kh * 16 * KB;  // the wave's first key
    // this wave's loads of tile j (and the queries) are done; after the barrier
    // every wave's are, and every wave has finished reading (Kn, Vn)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (j + 1 < ntiles) dma.issue(rk, rv, (uint32_t)((int64_t)(kv0 + 64) * a.ldk * 2), Kn, Vn);
    if (kb0 > qmax) return;  // no key of this wave's part is visible to the tile's queries
    // S^T: lane holds kv = kb0 + kb*16 + 4g + i, q = q0 + c16
    f32x4 sc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = kh * 16 * KB + kb * 16 + c16;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const bf16x8 kf = ld8(K + row * D + (((ks * 4 + g) ^ kv_sw(row)) << 3));
        sc[kb] = mfma(kf, qf[ks], sc[kb]);
      }
    }
    // only the parts that reach the diagonal (or the sequence's end) are masked
    if (kb0 + 16 * KB - 1 > q0) mask_tile<KB>(sc, qlast - kb0 - 4 * g);
    float mt = fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3]));
#pragma unroll
    for (int kb = 1; kb < KB; ++kb) mt = fmaxf(mt, fmaxf(fmaxf(sc[kb][0], sc[kb][1]), fmaxf(sc[kb][2], sc[kb][3])));
    mt = max_rows4(mt) * a.scale_log2;  // -inf where the lane's query sees none of these keys
    if (__builtin_amdgcn_ballot_w64(mt > m + RESCALE_LOG2)) {
      const float mn = fmaxf(m, mt);
      const float alpha = mn == -INFINITY ? 1.f : exp2_ftz(m - mn);  // exp2(-inf) = 0 from a first maximum
      l *= alpha;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[ds][i] *= alpha;
      m = mn;
    }
    // a lane that has seen no visible key has only -inf scores: 2^-inf = 0
    const float mref = m == -INFINITY ? 0.f : m;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = exp2_ftz(fmaf(sc[kb][i], a.scale_log2, -mref));
        sc[kb][i] = pv;
        ls += pv;
      }
    l += ls;
    bf16x8 pf[KB / 2], pl[KB / 2];
#pragma unroll
    for (int kk = 0; kk < KB / 2; ++kk) split8(sc[2 * kk], sc[2 * kk + 1], pf[kk], pl[kk]);
    // O^T += V^T P^T over the wave's keys (the permuted order of pf), with P as a
    // hi + lo pair of bf16 values: O then carries about 16 significant bits of P,
    // so the backward's rowsum(dO O) is accurate where dP - rowsum cancels
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
      for (int kk = 0; kk < KB / 2; ++kk) {
        const bf16x8 vf = ld_tr8_sw(V, kh * 16 * KB + kk * 32, ds * 16, lane);
        o[ds] = mfma(vf, pf[kk], o[ds]);
        o[ds] = mfma(vf, pl[kk], o[ds]);
      }
  };
  for (int j = 0; j < ntiles; j += 2) {
    tile(K0, V0, K1, V1, j);
    if (j + 1 < ntiles) tile(K1, V1, K0, V0, j + 1);
  }
  if constexpr (KH == 2) {
    // the second half's (max, partial sums, output) through LDS, in register
    // order (K0 / K1 hold the outputs of heads 0-1 / 2-3 of each group of four)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    static_assert(NW <= 8, "attn_fwd_dma_kernel: 8 query heads per kv head at most");
    float* red = reinterpret_cast<float*>((hw & 2) ? K1 : K0) + (hw & 1) * (D / 16) * 4 * 64;
    float* redml = reinterpret_cast<float*>(V0) + hw * 128;
    if (hw < 4) {
      if (kh == 1) {
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[(ds * 4 + i) * 64 + lane] = o[ds][i];
        redml[lane] = m;
        redml[64 + lane] = l;
      }
    }
    __syncthreads();
    if (hw < 4 && kh == 0) {
      const float m1 = redml[lane], l1 = redml[64 + lane];
      const float mn = fmaxf(m, m1);  // finite: key 0 is in the first half of tile 0
      const float a0 = exp2_ftz(m - mn), a1 = m1 == -INFINITY ? 0.f : exp2_ftz(m1 - mn);
      l = l * a0 + l1 * a1;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[ds][i] = o[ds][i] * a0 + red[(ds * 4 + i) * 64 + lane] * a1;
      m = mn;
    }
    if constexpr (NW > 4) {
      // heads 4..7: a second round through the same buffers
      __syncthreads();
      if (hw >= 4 && kh == 1) {
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[(ds * 4 + i) * 64 + lane] = o[ds][i];
        redml[lane] = m;
        redml[64 + lane] = l;
      }
      __syncthreads();
      if (hw >= 4 && kh == 0) {
        const float m1 = redml[lane], l1 = redml[64 + lane];
        const float mn = fmaxf(m, m1);
        const float a0 = exp2_ftz(m - mn), a1 = m1 == -INFINITY ? 0.f : exp2_ftz(m1 - mn);
        l = l * a0 + l1 * a1;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[ds][i] = o[ds][i] * a0 + red[(ds * 4 + i) * 64 + lane] * a1;
        m = mn;
      }
    }
    if (kh == 1) return;
  }
  const float lt = sum_rows4(l);
  if (q < a.seq) {
    const float inv = 1.0f / lt;
    uint16_t* op = a.out + (rowbase + q) * a.ldo + (int64_t)h * D;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const f32x4& r = o[ds];
      *reinterpret_cast<u32x2*>(op + ds * 16 + g * 4) = u32x2{pack2(r[0] * inv, r[1] * inv), pack2(r[2] * inv, r[3] * inv)};
      if (a.o32)
        *reinterpret_cast<f32x4*>(a.o32 + (rowbase + q) * ((int64_t)a.n_q * D) + (int64_t)h * D + ds * 16 + g * 4) =
            f32x4{r[0] * inv, r[1] * inv, r[2] * inv, r[3] * inv};
    }
    if (g == 0) a.lse_out[((int64_t)b * a.n_q + h) * a.seq + q] = (m + log2f(lt)) * LN2;
  }
}

// ---------------------------------------------------------------- backward
// D[b][h][q] = sum_d dO[q][d] * O[q][d]; one wave per (row, head).
template <int D>
__global__ void attn_dsum_kernel(const AttnArgs a) {
  if (a.dkv_cnt) {
    // the balanced dK/dV kernel's arrival counts start at zero
    const int64_t n = (int64_t)a.batch * a.n_kv * ((a.seq + 31) / 32);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
      a.dkv_cnt[i] = 0u;
  }
  int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  int64_t T = (int64_t)a.batch * a.seq;
  if (w >= T * a.n_q) return;
  int64_t row = w / a.n_q;
  int h = (int)(w - row * a.n_q);
  const uint16_t* op = a.o + row * a.ldo + (int64_t)h * D;
  const uint16_t* dp = a.dout + row * a.ldo + (int64_t)h * D;
  float s = 0.f;
  if (a.o32) {
    const float* o32 = a.o32 + row * ((int64_t)a.n_q * D) + (int64_t)h * D;
    for (int c = lane * 2; c < D; c += 128) {
      uint32_t dv = *reinterpret_cast<const uint32_t*>(dp + c);
      s += o32[c] * lo_bf(dv) + o32[c + 1] * hi_bf(dv);
    }
  } else {
    for (int c = lane * 2; c < D; c += 128) {
      uint32_t ov = *reinterpret_cast<const uint32_t*>(op + c), dv = *reinterpret_cast<const uint32_t*>(dp + c);
      s += lo_bf(ov) * lo_bf(dv) + hi_bf(ov) * hi_bf(dv);
    }
  }
  s = wave_sum(s);
  if (lane == 0) {
    int64_t b = row / a.seq, q = row - b * a.seq;
    a.dsum_out[(b * a.n_q + h) * a.seq + q] = s;
  }
}

// dK, dV for 32-key tiles of one kv head. block 128 * HG threads with HG =
// min(group, 4) head groups of two waves; wave (hg, w) owns keys kv0 + 16w .. +15
// and the query heads hg, hg + HG, ... of the kv head. A key tile's work is its
// units (query head sub-group, 64-query tile from the diagonal down: the next
// unit's tiles are fetched into registers while the current one is computed);
// the head groups' partial dK/dV are added in head-group order through LDS.
//
// One workgroup per key tile (grid ceil(seq/32) x n_kv x batch as one
// dimension, heaviest tiles first), or, BAL, the same number of workgroups per
// (sequence, kv head) walking equal ranges of the units in key-tile order: the
// first key tile of a sequence has all the query tiles and the last one, so at
// one workgroup per CU the kernel would otherwise last as long as its heaviest
// tile. A tile whose units span several workgroups is summed by the one that
// arrives last, adding their float32 partials in workgroup order.
constexpr int DKV_QT = 64;
LSL_DEV int dkv_owner(int u, int U, int G) { return (int)((((int64_t)u + 1) * G - 1) / U); }

template <int D, bool BAL>
__global__ __launch_bounds__(512) void attn_dkv_kernel(const AttnArgs a) {
  // head_dim 128: unpadded rows with the forward's chunk swizzle (conflict-free
  // for the row-wise and the transposing reads); 64: rows padded by 16 bytes
  constexpr bool SW = D == 128;
  constexpr int LD = SW ? D : D + 8;
  constexpr int SLOT = 2 * 32 * D;  // a partial: dK^T and dV^T of the tile, in register order
  auto at = [](int row, int col) { return SW ? row * LD + (((col >> 3) ^ kv_sw(row)) << 3) + (col & 7) : row * LD + col; };
  constexpr int CH = DKV_QT * D / 8 / 128;  // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * 2 * DKV_QT * LD];
  __shared__ float lse_s[4][DKV_QT], dsum_s[4][DKV_QT];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (a scalar)
  const int HG = blockDim.x >> 7, hg = wave >> 1, ws = wave & 1;
  const int n_kt = (a.seq + 31) / 32;
  const int item = xcd_item((int)blockIdx.x, (int)gridDim.x);
  const int bk = item / n_kt, wi = item - bk * n_kt;  // (sequence, kv head) block; index in it
  const int kvh = bk % a.n_kv, b = bk / a.n_kv;
  const int64_t rowbase = (int64_t)b * a.seq;
  uint16_t* Qs = lds + hg * 2 * DKV_QT * LD;
  uint16_t* Os = Qs + DKV_QT * LD;
  const int n_qt = (a.seq + DKV_QT - 1) / DKV_QT;
  const int hq = (a.group + HG - 1) / HG;  // query head sub-groups per head group
  // key tile kt's units: hq sub-groups x its query tiles from kt * 32 / 64 on
  auto units = [&](int kt) { return hq * (n_qt - kt / 2); };

  f32x4 dk[D / 16], dv[D / 16];  // dK^T, dV^T: lane holds [d = dd*16 + 4g + i][kv = kv0 + 16 ws + c16]
  // units [ia, ib) of key tile kt into dk, dv (summed over the head groups in
  // the hg = 0 waves; LDS is free again when it returns)
  auto segment = [&](int kt, int ia, int ib) {
    // lane arithmetic redone per segment rather than held across the segment
    // loop (which would spill)
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int lane = tid_o & 63, htid = tid_o & 127, g = lane >> 4, c16 = lane & 15;
    const int kv0 = kt * 32;
    const int mykv = kv0 + ws * 16 + c16;
    bf16x8 kf[D / 32], vf[D / 32];
    {
      const uint16_t* kp = a.k + (rowbase + mykv) * a.ldk + (int64_t)kvh * D;
      const uint16_t* vp = a.v + (rowbase + mykv) * a.ldk + (int64_t)kvh * D;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        kf[ks] = mykv < a.seq ? ld8(kp + ks * 32 + g * 8) : bf16x8{};
        vf[ks] = mykv < a.seq ? ld8(vp + ks * 32 + g * 8) : bf16x8{};
      }
    }
#pragma unroll
    for (int i = 0; i < D / 16; ++i) dk[i] = dv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int qt_begin = kv0 / DKV_QT;
    const int nq = n_qt - qt_begin;
    u32x4 pq[CH], po[CH];
    float plse = 0.f, pds = 0.f;
    // Prefetch into registers. Rows past the sequence and inactive head groups
    // load a clamped in-range row (masked out in the compute), so the loads need
    // no branches and nothing waits for them until the LDS store.
    auto fetch = [&](int it) {
      const int hl = min(hg + (it / nq) * HG, a.group - 1);
      const int q0 = (qt_begin + it % nq) * DKV_QT;
      const int h = kvh * a.group + hl;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int idx = htid + c * 128, row = idx / (D / 8), col = (idx % (D / 8)) * 8;
        const int64_t q = min(q0 + row, a.seq - 1);
        pq[c] = *reinterpret_cast<const u32x4*>(a.q + (rowbase + q) * a.ldq + (int64_t)h * D + col);
        po[c] = *reinterpret_cast<const u32x4*>(a.dout + (rowbase + q) * a.ldo + (int64_t)h * D + col);
      }
      if (htid < DKV_QT) {
        const int q = min(q0 + htid, a.seq - 1);
        plse = a.lse[((int64_t)b * a.n_q + h) * a.seq + q];
        pds = a.dsum[((int64_t)b * a.n_q + h) * a.seq + q];
      }
    };
    fetch(ia);
    for (int it = ia; it < ib; ++it) {
      const bool act = hg + (it / nq) * HG < a.group;
      const int q0 = (qt_begin + it % nq) * DKV_QT;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int idx = htid + c * 128, row = idx / (D / 8), col = (idx % (D / 8)) * 8;
        *reinterpret_cast<u32x4*>(Qs + at(row, col)) = pq[c];
        *reinterpret_cast<u32x4*>(Os + at(row, col)) = po[c];
      }
      if (htid < DKV_QT) {
        lse_s[hg][htid] = plse * LOG2E;
        dsum_s[hg][htid] = pds;
      }
      __syncthreads();
      if (it + 1 < ib) fetch(it + 1);
      if (act) {
        // only query tiles that reach the diagonal or the sequence's end are
        // masked: elsewhere every query q >= q0 >= kv0 + 31 sees every key of the
        // tile and is inside the sequence
        const bool diag = q0 < kv0 + 31 || q0 + DKV_QT > a.seq;
        // S[q][kv], dP[q][kv] for 64 queries: lane holds q = qs*16 + 4g + i, kv = mykv
        f32x4 p[4], ds[4];
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
          f32x4 sv = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) {
            const int off = at(qs * 16 + c16, ks * 32 + g * 8);
            sv = mfma(ld8(Qs + off), kf[ks], sv);
            dp = mfma(ld8(Os + off), vf[ks], dp);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ql = qs * 16 + g * 4 + i;
            const int q = q0 + ql;
            float x = fmaf(sv[i], a.scale_log2, -lse_s[hg][ql]);
            if (diag && !(mykv <= q && q < a.seq && mykv < a.seq)) x = -INFINITY;
            const float pv = exp2_ftz(x);
            p[qs][i] = pv;
            ds[qs][i] = pv * (dp[i] - dsum_s[hg][ql]);
          }
        }
        // dV^T += dO^T P, dK^T += Q^T dS: reduction over the 64 queries in two
        // 32-steps; the transposed operands come from the row-major tiles through
        // transposing LDS reads, in the permuted order of the P / dS registers.
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bf16x8 pb, pl, sb, sl;
          split8(p[2 * kk], p[2 * kk + 1], pb, pl);
          split8(ds[2 * kk], ds[2 * kk + 1], sb, sl);
#pragma unroll
          for (int dd = 0; dd < D / 16; ++dd) {
            bf16x8 oa, qa;
            if constexpr (SW) {
              oa = ld_tr8_sw(Os, kk * 32, dd * 16, lane);
              qa = ld_tr8_sw(Qs, kk * 32, dd * 16, lane);
            } else {
              oa = ld_tr8(Os, LD, kk * 32, dd * 16, lane);
              qa = ld_tr8(Qs, LD, kk * 32, dd * 16, lane);
            }
            dv[dd] = mfma(oa, pb, dv[dd]);
            dv[dd] = mfma(oa, pl, dv[dd]);
            dk[dd] = mfma(qa, sb, dk[dd]);
            dk[dd] = mfma(qa, sl, dk[dd]);
          }
        }
      }
      __syncthreads();
    }
    // add the head groups' partial sums in head-group order (LDS reused)
    f32x4* red = reinterpret_cast<f32x4*>(lds);
    auto slot = [&](int h, int which, int dd) { return (((h - 1) * 2 + ws) * 2 + which) * (D / 16) * 64 + dd * 64 + lane; };
    if (hg > 0) {
#pragma unroll
      for (int dd = 0; dd < D / 16; ++dd) {
        red[slot(hg, 0, dd)] = dk[dd];
        red[slot(hg, 1, dd)] = dv[dd];
      }
    }
    __syncthreads();
    if (hg == 0)
      for (int h = 1; h < HG; ++h)
#pragma unroll
        for (int dd = 0; dd < D / 16; ++dd) {
          const f32x4 rk = red[slot(h, 0, dd)], rv = red[slot(h, 1, dd)];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dk[dd][i] += rk[i];
            dv[dd][i] += rv[i];
          }
        }
    __syncthreads();
  };
  // the bf16 result of key tile kt from the hg = 0 waves' sums
  auto write = [&](int kt) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
    const int mykv = kt * 32 + ws * 16 + c16;
    if (hg != 0 || mykv >= a.seq) return;
    uint16_t* dkp = a.dk + (rowbase + mykv) * a.ldk + (int64_t)kvh * D;
    uint16_t* dvp = a.dv + (rowbase + mykv) * a.ldk + (int64_t)kvh * D;
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) {
      const f32x4& rk = dk[dd];
      const f32x4& rv = dv[dd];
      *reinterpret_cast<u32x2*>(dkp + dd * 16 + g * 4) =
          u32x2{pack2(rk[0] * a.scale, rk[1] * a.scale), pack2(rk[2] * a.scale, rk[3] * a.scale)};
      *reinterpret_cast<u32x2*>(dvp + dd * 16 + g * 4) = u32x2{pack2(rv[0], rv[1]), pack2(rv[2], rv[3])};
    }
  };

  if constexpr (!BAL) {
    // one workgroup per key tile, the heaviest (earliest) first
    segment(wi, 0, units(wi));
    write(wi);
  } else {
    // equal ranges of the block's units, G = n_kt workgroups; the partials of
    // key tile kt sit in slots f + kt .. l + kt of the block (f, l: its first and
    // last workgroup), (2 n_kt - 1) slots per block
    const int G = n_kt;
    int U = 0;
    for (int kt = 0; kt < n_kt; ++kt) U += units(kt);
    const int ub = (int)((int64_t)U * wi / G), ue = (int)((int64_t)U * (wi + 1) / G);
    float* part = a.dkv_part + (int64_t)bk * (2 * n_kt - 1) * SLOT;
    unsigned* cnt = a.dkv_cnt + (int64_t)bk * n_kt;
    const __amdgpu_buffer_rsrc_t rs = wt_rsrc(part, (int64_t)(2 * n_kt - 1) * SLOT * 4);
    // the first key tile of the range and its first unit
    int kt = 0, P = 0;
    while (P + units(kt) <= ub) { P += units(kt); ++kt; }
    // tiles whose partials this workgroup adds up (it arrived last): at most the
    // first and the last of its range (the others in it are whole)
    // (scalars, not an indexed array: an array indexed at run time lives in scratch)
    int fix_t0 = -1, fix_f0 = 0, fix_n0 = 0, fix_t1 = -1, fix_f1 = 0, fix_n1 = 0;
    for (int u = ub; u < ue; ++kt) {
      const int I = units(kt);
      const int ia = u - P, ib = min(I, ue - P);
      segment(kt, ia, ib);
      if (ia == 0 && ib == I) {
        write(kt);
      } else {
        const int lane = threadIdx.x & 63;
        if (hg == 0)
#pragma unroll
          for (int dd = 0; dd < D / 16; ++dd) {
            const uint32_t o = (uint32_t)((((ws * 2 + 0) * (D / 16) + dd) * 64 + lane) * 16);
            const uint32_t o2 = (uint32_t)((((ws * 2 + 1) * (D / 16) + dd) * 64 + lane) * 16);
            wt_store4(rs, o, (uint32_t)(wi + kt) * SLOT * 4, dk[dd]);
            wt_store4(rs, o2, (uint32_t)(wi + kt) * SLOT * 4, dv[dd]);
          }
        const int f = dkv_owner(P, U, G), l = dkv_owner(P + I - 1, U, G);
        if (last_arrival(cnt + kt, l - f + 1)) {
          if (fix_t0 < 0) { fix_t0 = kt; fix_f0 = f; fix_n0 = l - f + 1; }
          else { fix_t1 = kt; fix_f1 = f; fix_n1 = l - f + 1; }
        }
      }
      u = P + ib;
      P += I;
    }
    // the tiles' partials added in workgroup order by all threads: thread tid
    // takes float4 e = tid + 512 m of the slot, i.e. (half ws, dK or dV, dd, lane)
    const int nthr = (int)blockDim.x;
    for (int fi = 0; fi < 2; ++fi) {
      const int t = fi == 0 ? fix_t0 : fix_t1;
      if (t < 0) continue;
      const int ff = fi == 0 ? fix_f0 : fix_f1, fn = fi == 0 ? fix_n0 : fix_n1;
      constexpr int NE = SLOT / 4 / 128;  // float4 per thread at the smallest block (128 threads)
      f32x4 v[NE];
      for (int sp = 0; sp < fn; ++sp) {
        const uint32_t so = (uint32_t)(ff + sp + t) * SLOT * 4;
#pragma unroll
        for (int m = 0; m < NE; ++m) {
          if (tid + nthr * m >= SLOT / 4) break;
          const f32x4 q = wt_load4(rs, (uint32_t)(tid + nthr * m) * 16, so);
          v[m] = sp == 0 ? q : f32x4{v[m][0] + q[0], v[m][1] + q[1], v[m][2] + q[2], v[m][3] + q[3]};
        }
      }
#pragma unroll
      for (int m = 0; m < NE; ++m) {
        const int e = tid + nthr * m;
        if (e >= SLOT / 4) break;
        const int ln = e & 63, dd = (e >> 6) % (D / 16), which = (e >> 6) / (D / 16) % 2, hw = (e >> 6) / (D / 16) / 2;
        const int kv = t * 32 + hw * 16 + (ln & 15);
        if (kv >= a.seq) continue;
        const int d = dd * 16 + (ln >> 4) * 4;
        const float sc = which == 0 ? a.scale : 1.f;
        uint16_t* dst = (which == 0 ? a.dk : a.dv) + (rowbase + kv) * a.ldk + (int64_t)kvh * D + d;
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack2(v[m][0] * sc, v[m][1] * sc), pack2(v[m][2] * sc, v[m][3] * sc)};
      }
    }
  }
}

// dQ for one 16 NQS-query tile of each of the group's heads (wave = head), like
// the forward. grid (ceil(seq / (16 NQS)), n_kv, batch), block group*64 threads.
template <int D, int NQS, int NW>
__global__ __launch_bounds__(64 * NW) void attn_dq_kernel(const AttnArgs a) {
  constexpr int QT = 16 * NQS, LD = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_qt = (a.seq + QT - 1) / QT;
  const int item = xcd_item((int)blockIdx.x, (int)gridDim.x);
  const int bk = item / n_qt, qt = n_qt - 1 - (item - bk * n_qt);
  const int kvh = bk % a.n_kv, b = bk / a.n_kv;
  const int h = kvh * a.group + wave;
  const int q0 = qt * QT;
  const int64_t rowbase = (int64_t)b * a.seq;
  const int g = lane >> 4, c16 = lane & 15;
  const uint16_t* qp = a.q + rowbase * a.ldq + (int64_t)h * D;
  const uint16_t* dop = a.dout + rowbase * a.ldo + (int64_t)h * D;
  const uint16_t* kp = a.k + rowbase * a.ldk + (int64_t)kvh * D;
  const uint16_t* vp = a.v + rowbase * a.ldk + (int64_t)kvh * D;

  bf16x8 qf[NQS][D / 32], of[NQS][D / 32];
  float lse2[NQS], dsm[NQS];
#pragma unroll
  for (int qs = 0; qs < NQS; ++qs) {
    const int64_t q = min(q0 + qs * 16 + c16, a.seq - 1);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      qf[qs][ks] = ld8(qp + q * a.ldq + ks * 32 + g * 8);
      of[qs][ks] = ld8(dop + q * a.ldo + ks * 32 + g * 8);
    }
    lse2[qs] = a.lse[((int64_t)b * a.n_q + h) * a.seq + q] * LOG2E;
    dsm[qs] = a.dsum[((int64_t)b * a.n_q + h) * a.seq + q];
  }
  f32x4 dq[D / 16][NQS];
#pragma unroll
  for (int i = 0; i < D / 16; ++i)
#pragma unroll
    for (int qs = 0; qs < NQS; ++qs) dq[i][qs] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int qmax = min(q0 + QT - 1, a.seq - 1);
  const int ntiles = qmax / 64 + 1;
  TileStage<D, 64 * NW> kst, vst;
  kst.load(kp, a.ldk, 0, a.seq, tid);
  vst.load(vp, a.ldk, 0, a.seq, tid);
  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = j * 64;
    kst.store(Ks, tid);
    vst.store(Vs, tid);
    __syncthreads();
    if (j + 1 < ntiles) {
      kst.load(kp, a.ldk, kv0 + 64, a.seq, tid);
      vst.load(vp, a.ldk, kv0 + 64, a.seq, tid);
    }
    // S^T and dP^T: lane holds kv = kv0 + kvs*16 + 4g + i, q = q0 + qs*16 + c16
    bf16x8 dsf[NQS][2], dsl[NQS][2];
    f32x4 sc[4][NQS], dp[4][NQS];
#pragma unroll
    for (int kvs = 0; kvs < 4; ++kvs) {
#pragma unroll
      for (int qs = 0; qs < NQS; ++qs) sc[kvs][qs] = dp[kvs][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const bf16x8 ka = ld8(Ks + (kvs * 16 + c16) * LD + ks * 32 + g * 8);
        const bf16x8 va = ld8(Vs + (kvs * 16 + c16) * LD + ks * 32 + g * 8);
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
          sc[kvs][qs] = mfma(ka, qf[qs][ks], sc[kvs][qs]);
          dp[kvs][qs] = mfma(va, of[qs][ks], dp[kvs][qs]);
        }
      }
    }
    // only key tiles that reach the diagonal (or query rows past the sequence's
    // end) are masked: below it every key kv <= kv0 + 63 < q0 <= q is visible
    const bool diag = kv0 + 63 > q0 || q0 + QT > a.seq;
#pragma unroll
    for (int qs = 0; qs < NQS; ++qs) {
      const int q = q0 + qs * 16 + c16;
#pragma unroll
      for (int kvs = 0; kvs < 4; ++kvs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kv = kv0 + kvs * 16 + g * 4 + i;
          float x = fmaf(sc[kvs][qs][i], a.scale_log2, -lse2[qs]);
          if (diag && !(kv <= q && kv < a.seq && q < a.seq)) x = -INFINITY;
          const float pv = exp2_ftz(x);
          sc[kvs][qs][i] = pv * (dp[kvs][qs][i] - dsm[qs]);
        }
      split8(sc[0][qs], sc[1][qs], dsf[qs][0], dsl[qs][0]);
      split8(sc[2][qs], sc[3][qs], dsf[qs][1], dsl[qs][1]);
    }
    // dQ^T += K^T dS^T (reduction over 64 keys, permuted like the forward's P V)
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 ka = ld_tr8(Ks, LD, kk * 32, dd * 16, lane);
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
          dq[dd][qs] = mfma(ka, dsf[qs][kk], dq[dd][qs]);
          dq[dd][qs] = mfma(ka, dsl[qs][kk], dq[dd][qs]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int qs = 0; qs < NQS; ++qs) {
    const int q = q0 + qs * 16 + c16;
    if (q >= a.seq) continue;
    uint16_t* dqp = a.out + (rowbase + q) * a.ldq + (int64_t)h * D;
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) {
      const f32x4& r = dq[dd][qs];
      *reinterpret_cast<u32x2*>(dqp + dd * 16 + g * 4) =
          u32x2{pack2(r[0] * a.scale, r[1] * a.scale), pack2(r[2] * a.scale, r[3] * a.scale)};
    }
  }
}

// dQ at head_dim 128 with the forward's staging: K/V tiles by LDS-writing buffer
// loads (two stages, the conflict-free chunk swizzle), two waves per query head,
// each on half of every 64-key tile; the halves' dQ partials are added in order
// at the end.
template <int NW>
__global__ __launch_bounds__(128 * NW) void attn_dq_dma_kernel(const AttnArgs a) {
  constexpr int D = 128, QT = 16, KH = 2, NWT = NW * KH, KB = 4 / KH;
  __shared__ __attribute__((aligned(16))) uint16_t K0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t K1[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t V1[64 * D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = wave % NW, kh = wave / NW;
  const int n_qt = (a.seq + QT - 1) / QT;
  const int item = xcd_item((int)blockIdx.x, (int)gridDim.x);
  const int bk = item / n_qt, qt = n_qt - 1 - (item - bk * n_qt);
  const int kvh = bk % a.n_kv, b = bk / a.n_kv;
  const int h = kvh * a.group + hw;
  const int q0 = qt * QT;
  const int64_t rowbase = (int64_t)b * a.seq;
  const int g = lane >> 4, c16 = lane & 15;
  const uint16_t* qp = a.q + rowbase * a.ldq + (int64_t)h * D;
  const uint16_t* dop = a.dout + rowbase * a.ldo + (int64_t)h * D;
  const uint16_t* kp = a.k + rowbase * a.ldk + (int64_t)kvh * D;
  const uint16_t* vp = a.v + rowbase * a.ldk + (int64_t)kvh * D;

  const int qmax = min(q0 + QT - 1, a.seq - 1);
  const int ntiles = qmax / 64 + 1;
  const uint32_t seqbytes = (uint32_t)((int64_t)a.seq * a.ldk * 2);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kp), (short)0, (int)seqbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vp), (short)0, (int)seqbytes, 0x00020000);
  KvDma<NWT> dma;
  dma.init(a.ldk, wave, lane);
  dma.issue(rk, rv, 0, K0, V0);

  const int q = q0 + c16;
  const int qc = min(q, a.seq - 1);
  bf16x8 qf[D / 32], of[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    qf[ks] = ld8(qp + (int64_t)qc * a.ldq + ks * 32 + g * 8);
    of[ks] = ld8(dop + (int64_t)qc * a.ldo + ks * 32 + g * 8);
  }
  const float lse2 = a.lse[((int64_t)b * a.n_q + h) * a.seq + qc] * LOG2E;
  // D_q = sum_d dO O (O from the forward's float32 copy when there is one), over
  // the lane's 32 columns and then the query's four lanes; written for the dK/dV
  // kernel, which runs after this one
  float dsm = 0.f;
  if (a.o32) {
    const float* op = a.o32 + (rowbase + qc) * ((int64_t)a.n_q * D) + (int64_t)h * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const f32x4 o0 = *reinterpret_cast<const f32x4*>(op + ks * 32 + g * 8);
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(op + ks * 32 + g * 8 + 4);
      const u32x4 dv = __builtin_bit_cast(u32x4, of[ks]);
      dsm += o0[0] * lo_bf(dv[0]) + o0[1] * hi_bf(dv[0]) + o0[2] * lo_bf(dv[1]) + o0[3] * hi_bf(dv[1]);
      dsm += o1[0] * lo_bf(dv[2]) + o1[1] * hi_bf(dv[2]) + o1[2] * lo_bf(dv[3]) + o1[3] * hi_bf(dv[3]);
    }
  } else {
    const uint16_t* op = a.o + (rowbase + qc) * a.ldo + (int64_t)h * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const u32x4 ov = *reinterpret_cast<const u32x4*>(op + ks * 32 + g * 8);
      const u32x4 dv = __builtin_bit_cast(u32x4, of[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) dsm += lo_bf(ov[e]) * lo_bf(dv[e]) + hi_bf(ov[e]) * hi_bf(dv[e]);
    }
  }
  dsm = sum_rows4(dsm);
  if (kh == 0 && g == 0 && q < a.seq) a.dsum_out[((int64_t)b * a.n_q + h) * a.seq + q] = dsm;
  if (a.dkv_cnt && blockIdx.x == 0) {
    // the balanced dK/dV kernel's arrival counts start at zero
    const int64_t n = (int64_t)a.batch * a.n_kv * ((a.seq + 31) / 32);
    for (int64_t i = tid; i < n; i += blockDim.x) a.dkv_cnt[i] = 0u;
  }
  f32x4 dq[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) dq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the lane's last visible key; query rows past the sequence see none
  const int qlast = q < a.seq ? q : -1;

  auto tile = [&](const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, uint16_t* Kn, uint16_t* Vn,
                  int j) {
    const int kv0 = j * 64, kb0 = kv0 + kh * 16 * KB;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (j + 1 < ntiles) dma.issue(rk, rv, (uint32_t)((int64_t)(kv0 + 64) * a.ldk * 2), Kn, Vn);
    if (kb0 > qmax) return;
    // S^T and dP^T: lane holds kv = kb0 + kb*16 + 4g + i, q = q0 + c16
    f32x4 sc[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sc[kb] = dp[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = kh * 16 * KB + kb * 16 + c16;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const int off = row * D + (((ks * 4 + g) ^ kv_sw(row)) << 3);
        sc[kb] = mfma(ld8(K + off), qf[ks], sc[kb]);
        dp[kb] = mfma(ld8(V + off), of[ks], dp[kb]);
      }
    }
    if (kb0 + 16 * KB - 1 > q0 || q0 + QT > a.seq) mask_tile<KB>(sc, qlast - kb0 - 4 * g);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = exp2_ftz(fmaf(sc[kb][i], a.scale_log2, -lse2));
        sc[kb][i] = pv * (dp[kb][i] - dsm);
      }
    bf16x8 dsf[KB / 2], dsl[KB / 2];
#pragma unroll
    for (int kk = 0; kk < KB / 2; ++kk) split8(sc[2 * kk], sc[2 * kk + 1], dsf[kk], dsl[kk]);
    // dQ^T += K^T dS^T over the wave's keys (permuted like the forward's P V)
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd)
#pragma unroll
      for (int kk = 0; kk < KB / 2; ++kk) {
        const bf16x8 ka = ld_tr8_sw(K, kh * 16 * KB + kk * 32, dd * 16, lane);
        dq[dd] = mfma(ka, dsf[kk], dq[dd]);
        dq[dd] = mfma(ka, dsl[kk], dq[dd]);
      }
  };
  for (int j = 0; j < ntiles; j += 2) {
    tile(K0, V0, K1, V1, j);
    if (j + 1 < ntiles) tile(K1, V1, K0, V0, j + 1);
  }
  // the second half's partial through LDS in register order, added to the first's
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  static_assert(NW <= 8, "attn_dq_dma_kernel: 8 query heads per kv head at most");
#pragma unroll
  for (int round = 0; round < (NW + 3) / 4; ++round) {
    const bool mine = hw / 4 == round;
    float* red = reinterpret_cast<float*>((hw & 2) ? K1 : K0) + (hw & 1) * (D / 16) * 4 * 64;
    if (mine && kh == 1)
#pragma unroll
      for (int dd = 0; dd < D / 16; ++dd)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(dd * 4 + i) * 64 + lane] = dq[dd][i];
    __syncthreads();
    if (mine && kh == 0)
#pragma unroll
      for (int dd = 0; dd < D / 16; ++dd)
#pragma unroll
        for (int i = 0; i < 4; ++i) dq[dd][i] += red[(dd * 4 + i) * 64 + lane];
    __syncthreads();
  }
  if (kh == 1 || q >= a.seq) return;
  uint16_t* dqp = a.out + (rowbase + q) * a.ldq + (int64_t)h * D;
#pragma unroll
  for (int dd = 0; dd < D / 16; ++dd) {
    const f32x4& r = dq[dd];
    *reinterpret_cast<u32x2*>(dqp + dd * 16 + g * 4) =
        u32x2{pack2(r[0] * a.scale, r[1] * a.scale), pack2(r[2] * a.scale, r[3] * a.scale)};
  }
}

// ---------------------------------------------------------------- host
#ifndef LSL_ATT_QT
#define LSL_ATT_QT 16
#endif
constexpr int ATT_QT = LSL_ATT_QT;  // queries per wave in the forward and dQ kernels (16 or 32)

struct FwdKernel {
  template <int D, int NW> static void launch(dim3 g, dim3 b, hipStream_t s, const AttnArgs& a) {
    if constexpr (D == 128 && ATT_QT == 16)
      hipLaunchKernelGGL((attn_fwd_dma_kernel<NW, 2>), g, dim3(b.x * 2), 0, s, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<D, ATT_QT / 16, NW>), g, b, 0, s, a);
  }
};
struct DqKernel {
  template <int D, int NW> static void launch(dim3 g, dim3 b, hipStream_t s, const AttnArgs& a) {
    if constexpr (D == 128 && ATT_QT == 16)
      hipLaunchKernelGGL((attn_dq_dma_kernel<NW>), g, dim3(b.x * 2), 0, s, a);
    else
      hipLaunchKernelGGL((attn_dq_kernel<D, ATT_QT / 16, NW>), g, b, 0, s, a);
  }
};
// one instantiation per group size (1..8 query heads per kv head, checked by attn_check)
template <class K, int D>
static void launch_by_group(int group, dim3 g, dim3 b, hipStream_t s, const AttnArgs& a) {
  switch (group) {
    case 1: K::template launch<D, 1>(g, b, s, a); break;
    case 2: K::template launch<D, 2>(g, b, s, a); break;
    case 3: K::template launch<D, 3>(g, b, s, a); break;
    case 4: K::template launch<D, 4>(g, b, s, a); break;
    case 5: K::template launch<D, 5>(g, b, s, a); break;
    case 6: K::template launch<D, 6>(g, b, s, a); break;
    case 7: K::template launch<D, 7>(g, b, s, a); break;
    default: K::template launch<D, 8>(g, b, s, a); break;
  }
}

static lsl_status attn_check(const char* fn, int64_t ldq, int64_t ldk, int batch, int seq, int n_q, int n_kv, int d) {
  if (batch < 0 || seq < 0 || n_q <= 0 || n_kv <= 0 || n_q % n_kv)
    return set_error(LSL_ERR_INVALID_ARG, "%s: bad head counts (n_q %% n_kv must be 0)", fn);
  if (d != 64 && d != 128) return set_error(LSL_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128 supported)", fn, d);
  if (n_q / n_kv > 8) return set_error(LSL_ERR_UNSUPPORTED, "%s: more than 8 query heads per kv head", fn);
  // one-dimensional grids of (query or key tiles) x kv heads x sequences
  if ((int64_t)((seq + 15) / 16) * n_kv * batch >= ((int64_t)1 << 31))
    return set_error(LSL_ERR_UNSUPPORTED, "%s: too many tiles for one grid", fn);
  if (ldq < (int64_t)n_q * d || ldk < (int64_t)n_kv * d || ldq % 8 || ldk % 8)
    return set_error(LSL_ERR_INVALID_ARG, "%s: leading dimensions too small or not multiples of 8", fn);
  // the forward reads a sequence's K and V rows through 32-bit buffer offsets
  if ((int64_t)seq * ldk * 2 >= ((int64_t)1 << 32))
    return set_error(LSL_ERR_UNSUPPORTED, "%s: one sequence's K or V rows exceed 4 GiB", fn);
  return LSL_OK;
}

lsl_status attention_fwd_launch(const AttnArgs& a0, int d, hipStream_t s) {
  AttnArgs a = a0;
  if ((int64_t)a.batch * a.seq == 0) return LSL_OK;
  dim3 grid((unsigned)(((a.seq + ATT_QT - 1) / ATT_QT) * a.n_kv * a.batch));
  dim3 block((unsigned)(64 * a.group));
  if (d == 128) launch_by_group<FwdKernel, 128>(a.group, grid, block, s, a);
  else launch_by_group<FwdKernel, 64>(a.group, grid, block, s, a);
  return check_launch("attention_fwd");
}

lsl_status attention_bwd_launch(const AttnArgs& a0, int d, hipStream_t s) {
  AttnArgs a = a0;
  int64_t T = (int64_t)a.batch * a.seq;
  if (T == 0) return LSL_OK;
  dim3 gq((unsigned)(((a.seq + ATT_QT - 1) / ATT_QT) * a.n_kv * a.batch));
  if (d == 128 && ATT_QT == 16) {
    // the dQ kernel computes the row sums D itself (and zeroes the dK/dV
    // arrival counts); the dK/dV kernel reads them after it
    launch_by_group<DqKernel, 128>(a.group, gq, dim3(64 * a.group), s, a);
  } else {
    dim3 gs((unsigned)((T * a.n_q + 3) / 4));
    if (d == 128) hipLaunchKernelGGL(attn_dsum_kernel<128>, gs, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(attn_dsum_kernel<64>, gs, dim3(256), 0, s, a);
  }
  a.dsum = a.dsum_out;
  dim3 gk((unsigned)(((a.seq + 31) / 32) * a.n_kv * a.batch));
  dim3 bk((unsigned)(128 * std::min(a.group, 4)));
  if (a.dkv_cnt) {
    if (d == 128) hipLaunchKernelGGL((attn_dkv_kernel<128, true>), gk, bk, 0, s, a);
    else hipLaunchKernelGGL((attn_dkv_kernel<64, true>), gk, bk, 0, s, a);
  } else {
    if (d == 128) hipLaunchKernelGGL((attn_dkv_kernel<128, false>), gk, bk, 0, s, a);
    else hipLaunchKernelGGL((attn_dkv_kernel<64, false>), gk, bk, 0, s, a);
  }
  if (d == 64 || ATT_QT != 16) {
    if (d == 128) launch_by_group<DqKernel, 128>(a.group, gq, dim3(64 * a.group), s, a);
    else launch_by_group<DqKernel, 64>(a.group, gq, dim3(64 * a.group), s, a);
  }
  return check_launch("attention_bwd");
}

// The balanced dK/dV kernel runs when the key tiles are few (at most two per CU),
// so that one workgroup per key tile would leave the kernel waiting on its
// heaviest tiles; its scratch follows the row sums in the workspace.
static bool dkv_balanced(int batch, int seq, int n_kv) {
  const int64_t n_kt = (seq + 31) / 32;
  return n_kt >= 2 && (int64_t)batch * n_kv * n_kt <= 512;
}
static size_t dkv_cnt_bytes(int batch, int seq, int n_kv) {
  return align256((size_t)batch * n_kv * ((seq + 31) / 32) * sizeof(unsigned));
}
size_t attention_ws_bytes(int batch, int seq, int n_q, int n_kv, int d) {
  size_t bytes = align256((size_t)batch * n_q * seq * sizeof(float));
  if (dkv_balanced(batch, seq, n_kv))
    bytes += dkv_cnt_bytes(batch, seq, n_kv) +
             (size_t)batch * n_kv * (2 * ((seq + 31) / 32) - 1) * (2 * 32 * d) * sizeof(float);
  return bytes;
}

}  // namespace lsl

using namespace lsl;

extern "C" lsl_status lsl_attention_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ldq,
                                        int64_t ldk, int32_t batch, int32_t seq, int32_t n_q, int32_t n_kv,
                                        int32_t head_dim, uint16_t* o, int64_t ldo, float* lse, float* o32,
                                        lsl_stream stream) {
  const char* fn = "lsl_attention_fwd";
  LSL_TRY(attn_check(fn, ldq, ldk, batch, seq, n_q, n_kv, head_dim));
  if (ldo < (int64_t)n_q * head_dim || ldo % 8) return set_error(LSL_ERR_INVALID_ARG, "%s: bad ldo", fn);
  if ((int64_t)batch * seq == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {q, k, v, o, lse}));
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.ldq = ldq; a.ldk = ldk; a.out = o; a.ldo = ldo; a.lse_out = lse; a.o32 = o32;
  a.batch = batch; a.seq = seq; a.n_q = n_q; a.n_kv = n_kv; a.group = n_q / n_kv;
  a.scale = 1.0f / sqrtf((float)head_dim);
  a.scale_log2 = a.scale * LOG2E;
  return attention_fwd_launch(a, head_dim, (hipStream_t)stream);
}

extern "C" size_t lsl_attention_workspace_bytes(int32_t batch, int32_t seq, int32_t n_q, int32_t n_kv,
                                                 int32_t head_dim) {
  if (batch < 0 || seq < 0 || n_q <= 0) return 0;
  if (n_kv <= 0 || (head_dim != 64 && head_dim != 128)) return 0;
  return attention_ws_bytes(batch, seq, n_q, n_kv, head_dim);
}

extern "C" lsl_status lsl_attention_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                                        const uint16_t* dout, const float* lse, const float* o32, int64_t ldq,
                                        int64_t ldk, int64_t ldo, int32_t batch, int32_t seq, int32_t n_q,
                                        int32_t n_kv, int32_t head_dim, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                                        void* ws, size_t ws_bytes, lsl_stream stream) {
  const char* fn = "lsl_attention_bwd";
  LSL_TRY(attn_check(fn, ldq, ldk, batch, seq, n_q, n_kv, head_dim));
  if (ldo < (int64_t)n_q * head_dim || ldo % 8) return set_error(LSL_ERR_INVALID_ARG, "%s: bad ldo", fn);
  if ((int64_t)batch * seq == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {q, k, v, o, dout, lse, dq, dk, dv}));
  size_t need = attention_ws_bytes(batch, seq, n_q, n_kv, head_dim);
  if (!ws || ws_bytes < need) return set_error(LSL_ERR_WORKSPACE, "%s: workspace %zu < %zu", fn, ws_bytes, need);
  AttnArgs a{};
  if (dkv_balanced(batch, seq, n_kv)) {
    char* w = (char*)ws + align256((size_t)batch * n_q * seq * sizeof(float));
    a.dkv_cnt = (unsigned*)w;
    a.dkv_part = (float*)(w + dkv_cnt_bytes(batch, seq, n_kv));
  }
  a.q = q; a.k = k; a.v = v; a.ldq = ldq; a.ldk = ldk;
  a.o = o; a.dout = dout; a.ldo = ldo; a.lse = lse; a.dsum_out = (float*)ws; a.o32 = (float*)o32;
  a.out = dq; a.dk = dk; a.dv = dv;
  a.batch = batch; a.seq = seq; a.n_q = n_q; a.n_kv = n_kv; a.group = n_q / n_kv;
  a.scale = 1.0f / sqrtf((float)head_dim);
  a.scale_log2 = a.scale * LOG2E;
  return attention_bwd_launch(a, head_dim, (hipStream_t)stream);
}
