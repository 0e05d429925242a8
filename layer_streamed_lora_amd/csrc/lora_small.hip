// The rank-r side products of LoRA on bf16 MFMA, with fixed-order split
// reductions (no floating-point atomics, so every run gives the same bits).
//
//   NT  (t, u):   C[t][j] = sum_k P[t][k] R[j][k]          P [T x K], j < kl <= 64
//        t = x A^T           R = A_full [kl x K]
//        u = dy B (per fused projection)  R[j][n] = B[n][j % r] if column n belongs to projection j / r
//   TN  (dA, dB): C[a][j] = sum_t P[t][a] Q[t][j]          P [T x W], Q [T x kl]
//        dA[j][k] += s C[k][j]              (P = x,  Q = u)
//        dB[n][i] += s C[n][p(n) r + i]     (P = dy, Q = t)
//
// Both are short, bandwidth-bound reductions at a few thousand tokens, so they
// are split over many workgroups (NT over K, TN over T). Each workgroup writes
// a float32 partial sum in its registers' order (one contiguous 16-byte store
// per lane and float4, written through to the device's coherence point); the
// workgroup that finishes last for a tile (an integer arrival count per tile)
// reads the tile's partials back in the same order, many loads in flight, adds
// them in split order and writes the result, so no second kernel runs and the
// bits do not depend on which workgroup finished last. The arrival counts live
// in a caller-provided region that must be zero before the first launch; each
// launch leaves it zero.
#include "common.h"
#include "small.h"
#include "api_util.h"

namespace lsl {

LSL_DEV f32x4 mfma16s(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer loads: lanes whose (vector) offset is at or past the end read zeros.
LSL_DEV __amdgpu_buffer_rsrc_t small_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

// ---------------------------------------------------------------- NT
struct NtArgs {
  const uint16_t* p; int64_t ldp;   // [T x K]
  const uint16_t* rt;               // R [kl x K], row stride K (A_full, or the masked B transposed)
  int64_t T, K; int kl;
  int S, steps;                     // K split S ways, `steps` 64-wide steps each
  float* part;                      // S > 1: one NT_SLOT float32 slot per (64-row tile, split)
  unsigned* cnt;                    // one arrival count per 64-row tile (S > 1)
  uint16_t* out; int64_t ldo;       // the bf16 result [T x kl]
};

// a partial slot: the 64 x 64 float32 tile, lane l of wave w holding row block
// rb at float4 ((4 w + rb) 64 + l)
constexpr int NT_SLOT = 64 * 64;

// C[t][j] = sum_k P[t][k] R[j][k] for a 64-row tile and one split of K.
// grid (ceil(T/64), S), 4 waves; wave w takes the split's steps w, w + 4, ...,
// in halves of 32 k, the next half's 8 loads in flight during the current
// half's MFMAs (operands straight from L2 into MFMA registers: each P element
// is read once, R is small and shared). The waves' sums are added in wave order through LDS, wave
// w then holding the tile's columns 16 w .. 16 w + 15: with one split that is
// the result, else a partial for the last-arriving workgroup of the tile.
__global__ __launch_bounds__(256, 2) void lora_nt_kernel(const NtArgs a) {
  __shared__ f32x4 red[4][4][4][64];  // [wave][j block][row block][lane]
  // the wave index is uniform in a wave: as a scalar, the buffer loads' offsets stay scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int KT = (int)(a.K / 64);
  const int sb = (int)blockIdx.y * a.steps, se = min(KT, sb + a.steps);
  f32x4 acc[4][4];  // [j block][row block]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t rp = small_rsrc(a.p, a.T * a.ldp * 2);
  const __amdgpu_buffer_rsrc_t rr = small_rsrc(a.rt, (int64_t)a.kl * a.K * 2);
  // rows >= T and R rows >= kl read zeros (the row is in the vector offset, the
  // step's k in the scalar one)
  uint32_t pv[4], rv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pv[i] = (uint32_t)(((t0 + i * 16 + c16) * a.ldp + g * 8) * 2);
    rv[i] = (uint32_t)(((int64_t)(i * 16 + c16) * a.K + g * 8) * 2);
  }
  // half-steps (32 of the step's 64 k): h -> step sb + wave + 4 (h / 2), half h % 2;
  // the next half's 8 loads are in flight during the current half's MFMAs
  auto load = [&](int h, bf16x8 (&pf)[4], bf16x8 (&rf)[4]) {
    const uint32_t so = (uint32_t)(((sb + wave + 4 * (h >> 1)) * 64 + (h & 1) * 32) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pf[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rp, pv[i], so, 0));
      rf[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rr, rv[i], so, 0));
    }
  };
  auto mma = [&](const bf16x8 (&pf)[4], const bf16x8 (&rf)[4]) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[jb][rb] = mfma16s(rf[jb], pf[rb], acc[jb][rb]);
  };
  const int H = sb + wave < se ? 2 * ((se - sb - wave + 3) / 4) : 0;  // even
  bf16x8 pa[4], ra[4], pb[4], rb_[4];
  if (H > 0) load(0, pa, ra);
  for (int h = 0; h < H; h += 2) {
    load(h + 1, pb, rb_);
    mma(pa, ra);
    if (h + 2 < H) load(h + 2, pa, ra);
    mma(pb, rb_);
  }
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) red[wave][jb][rb][lane] = acc[jb][rb];
  __syncthreads();
  // wave w, lane: C[j = 16 w + 4 g + i][t = t0 + 16 rb + c16], the waves added in order
  f32x4 v[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    v[rb] = red[0][wave][rb][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 q = red[w][wave][rb][lane];
      v[rb] = f32x4{v[rb][0] + q[0], v[rb][1] + q[1], v[rb][2] + q[2], v[rb][3] + q[3]};
    }
  }
  const int j = wave * 16 + g * 4;
  const bool live = wave * 16 < a.kl;  // (uniform in the wave)
  if (a.S > 1) {
    const __amdgpu_buffer_rsrc_t rs = wt_rsrc(a.part, (int64_t)gridDim.x * a.S * NT_SLOT * 4);
    const uint32_t so = (blockIdx.x * (uint32_t)a.S + blockIdx.y) * NT_SLOT * 4;
    if (live)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) wt_store4(rs, (uint32_t)((wave * 4 + rb) * 64 + lane) * 16, so, v[rb]);
    if (!last_arrival(a.cnt + blockIdx.x, a.S)) return;
    if (!live) return;
    // the tile's S partials in split order, eight splits' loads in flight at a
    // time (the loop's registers are free by now)
    const uint32_t s0 = blockIdx.x * (uint32_t)a.S * NT_SLOT * 4;
    for (int sp = 0; sp < a.S; sp += 8) {
      f32x4 q[8][4];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (sp + u < a.S)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            q[u][rb] = wt_load4(rs, (uint32_t)((wave * 4 + rb) * 64 + lane) * 16, s0 + (uint32_t)(sp + u) * NT_SLOT * 4);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (sp + u < a.S)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            v[rb] = sp + u == 0 ? q[u][rb]
                                : f32x4{v[rb][0] + q[u][rb][0], v[rb][1] + q[u][rb][1], v[rb][2] + q[u][rb][2],
                                        v[rb][3] + q[u][rb][3]};
    }
  }
  if (!live || j >= a.kl) return;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int64_t t = t0 + rb * 16 + c16;
    if (t < a.T) *reinterpret_cast<u32x2*>(a.out + t * a.ldo + j) = u32x2{pack2(v[rb][0], v[rb][1]), pack2(v[rb][2], v[rb][3])};
  }
}

// Masked transpose of B_full [K x r] for u = dy B: bt[j][k] = B[k][j % r] when
// j / r is the projection owning row k (else 0), j < kl. 8 k per thread.
LSL_DEV void bt_chunk(const uint16_t* __restrict__ b, int r, int kl, int64_t K, int nseg, const SegEnds& seg,
                      uint16_t* __restrict__ bt, int64_t idx) {
  const int64_t kc = K / 8;
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
__global__ void lora_bt_kernel(const uint16_t* __restrict__ b, int r, int kl, int64_t K, int nseg, SegEnds seg,
                               uint16_t* __restrict__ bt) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= kl * (K / 8)) return;
  bt_chunk(b, r, kl, K, nseg, seg, bt, idx);
}
// up to four transposes in one launch (thread idx: the jobs' chunks one after another)
struct BtGroup {
  const uint16_t* b[4]; int r[4], kl[4], nseg[4]; int64_t K[4]; SegEnds seg[4]; uint16_t* bt[4];
  int n;
};
__global__ void lora_bt_group_kernel(const BtGroup g) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int i = 0; i < g.n; ++i) {
    const int64_t n = (int64_t)g.kl[i] * (g.K[i] / 8);
    if (idx < n) {
      bt_chunk(g.b[i], g.r[i], g.kl[i], g.K[i], g.nseg[i], g.seg[i], g.bt[i], idx);
      return;
    }
    idx -= n;
  }
}

// ---------------------------------------------------------------- TN
struct TnArgs {
  const uint16_t* p; int64_t ldp;  // [T x W]
  const uint16_t* q; int64_t ldq;  // [T x kl]
  int64_t T, W; int kl;
  int64_t t_per_split; int S;
  float* part;                     // S > 1: one TN_SLOT float32 slot per (128-column tile, split)
  unsigned* cnt;                   // one arrival count per 128-column tile (S > 1)
  // the result goes to dA [kl x W] or dB [W x r] (+= scale C)
  float* dA; float* dB; float scale; int r; int nseg; SegEnds seg;
};

// The tiles are stored row-major [64 t][cols] as loaded (one 16-byte store per
// chunk) and the MFMA operands, whose reduction index t runs down the rows, are
// read with transposing LDS reads (ld_tr8; both operands in the same permuted
// t order). Row strides: 144 elements for P (128 columns) and 80 for Q (64),
// 8 dwords past a multiple of 64 banks, so the 8 rows x 32 bytes of a
// transposing read's half-wave fall in distinct banks; a 16-lane store covers
// one P row, or two Q rows 4 apart (32 banks apart).
constexpr int TN_LDP = 144, TN_LDQ = 80;
// a partial slot: the workgroup's accumulators, float4 (i, j) of thread tid at
// ((2 i + j) 256 + tid)
constexpr int TN_SLOT = 8 * 256 * 4;
// Q row of load rr (0, 1) of thread tid: rows 0, 4, 1, 5, 2, 6, 3, 7 (+ 8 (tid / 64)) for
// tid / 8 = 0..7 of each wave, and 32 more for rr = 1
LSL_DEV int tn_qrow(int tid, int rr) {
  const int qq = tid >> 3;
  return 8 * (qq >> 3) + ((qq >> 1) & 3) + 4 * (qq & 1) + 32 * rr;
}

// Up to TN_GROUP_MAX products in one launch (the adapter gradients dA and dB of
// a layer's projections need no ordering among them): grid = the sum of tiles_i
// S_i workgroups in one dimension, product i taking workgroups [start_i,
// start_i + tiles_i S_i), workgroup start_i + b tile b % tiles_i, split b /
// tiles_i; each product has its own partial slots and arrival counts.
constexpr int TN_GROUP_MAX = 8;
struct TnGroup {
  TnArgs p[TN_GROUP_MAX];
  int tiles[TN_GROUP_MAX];
  int start[TN_GROUP_MAX];
  int n;
};
// 4 waves, wave w owns columns a = 32w..32w+31 of the tile.
// BUF: the split's rows are read through buffer descriptors (its bytes below
// 4 GiB): no per-load bounds branches.
template <bool BUF>
__global__ __launch_bounds__(256) void lora_tn_kernel(const TnGroup grp) {
  __shared__ __attribute__((aligned(16))) uint16_t Ps[64 * TN_LDP];  // [t][a]
  __shared__ __attribute__((aligned(16))) uint16_t Qs[64 * TN_LDQ];  // [t][j]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int pi = 0;  // (uniform in the workgroup)
  while (pi + 1 < grp.n && (int)blockIdx.x >= grp.start[pi + 1]) ++pi;
  const TnArgs& a = grp.p[pi];
  const int bi = (int)blockIdx.x - grp.start[pi];
  const int tile = bi % grp.tiles[pi], split = bi / grp.tiles[pi], ntiles = grp.tiles[pi];
  const int64_t a0 = (int64_t)tile * 128;
  const int64_t tbeg = (int64_t)split * a.t_per_split;
  const int64_t tend = tbeg + a.t_per_split < a.T ? tbeg + a.t_per_split : a.T;
  f32x4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // thread -> P: rows 4 (tid / 16) + rr (rr < 4), 8 a-columns at 8 (tid % 16);
  // Q: rows tn_qrow(tid, rr) (rr < 2), 8 j-columns at 8 (tid % 8). The global
  // loads run two 64-token steps ahead of the MFMAs, in two register sets. With
  // BUF, rows past the split's end read zeros (t_per_split is a multiple of 64,
  // so that happens only past T); columns past W or kl read neighbouring data
  // or zeros and feed only outputs that are never stored.
  const int pq = tid >> 4, po = tid & 15, qo = tid & 7;
  const int64_t ac = a0 + po * 8;
  // (unused without BUF)
  const __amdgpu_buffer_rsrc_t rsp = small_rsrc(a.p + tbeg * a.ldp, (tend - tbeg) * a.ldp * 2);
  const __amdgpu_buffer_rsrc_t rsq = small_rsrc(a.q + tbeg * a.ldq, (tend - tbeg) * a.ldq * 2);
  uint32_t pofs[4], qofs[2];
  if constexpr (BUF) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) pofs[rr] = (uint32_t)(((int64_t)(pq * 4 + rr) * a.ldp + ac) * 2);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) qofs[rr] = (uint32_t)(((int64_t)tn_qrow(tid, rr) * a.ldq + qo * 8) * 2);
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
        const int64_t t = tt + tn_qrow(tid, rr);
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
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) *reinterpret_cast<u32x4*>(Ps + (pq * 4 + rr) * TN_LDP + po * 8) = rp[rr];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) *reinterpret_cast<u32x4*>(Qs + tn_qrow(tid, rr) * TN_LDQ + qo * 8) = rq[rr];
    __syncthreads();
    // unconditional, so that every step has the same loads in flight and each
    // wait covers only the older register set (past the split: zeros, unused)
    gload(tt + 128, rp, rq);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 qf[4], pf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[i] = ld_tr8(Qs, TN_LDQ, kk * 32, i * 16, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i) pf[i] = ld_tr8(Ps, TN_LDP, kk * 32, wave * 32 + i * 16, lane);
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
  // lane holds C[a][c..c+3], a = a0 + 32 wave + 16 j + lane % 16, c = 16 i + 4 (lane / 16)
  if (a.S > 1) {
    const __amdgpu_buffer_rsrc_t rs = wt_rsrc(a.part, (int64_t)ntiles * a.S * TN_SLOT * 4);
    const uint32_t s0 = (uint32_t)tile * (uint32_t)a.S * TN_SLOT * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        wt_store4(rs, (uint32_t)((2 * i + j) * 256 + tid) * 16, s0 + (uint32_t)split * TN_SLOT * 4, acc[i][j]);
    if (!last_arrival(a.cnt + tile, a.S)) return;
    // the tile's S partials in split order, two splits' loads in flight at a time
    for (int sp = 0; sp < a.S; sp += 2) {
      f32x4 q[2][8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (sp + u < a.S)
#pragma unroll
          for (int c = 0; c < 8; ++c)
            q[u][c] = wt_load4(rs, (uint32_t)(c * 256 + tid) * 16, s0 + (uint32_t)(sp + u) * TN_SLOT * 4);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (sp + u < a.S)
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            f32x4& d = acc[c >> 1][c & 1];
            d = sp + u == 0 ? q[u][c] : f32x4{d[0] + q[u][c][0], d[1] + q[u][c][1], d[2] + q[u][c][2], d[3] + q[u][c][3]};
          }
    }
  }
  // the tile's sum, scaled, into dA / dB
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t aa = a0 + wave * 32 + j * 16 + (lane & 15);
    if (aa >= a.W) continue;
    int p = 0;
    if (a.dB)
      while (p < a.nseg - 1 && aa >= a.seg.e[p]) ++p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = i * 16 + (lane >> 4) * 4;
      if (c >= a.kl) continue;
      if (a.dA) {
#pragma unroll
        for (int e = 0; e < 4; ++e) a.dA[(int64_t)(c + e) * a.W + aa] += a.scale * acc[i][j][e];
      } else if (c >= p * a.r && c < (p + 1) * a.r) {
        f32x4* d = reinterpret_cast<f32x4*>(a.dB + aa * a.r + (c - p * a.r));
        f32x4 v = *d;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += a.scale * acc[i][j][e];
        *d = v;
      }
    }
  }
}

// zero n 32-bit words (the arrival counts, before a call's first split launch)
__global__ void zero_u32_kernel(unsigned* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------- host side
// NT: K split so that about NT_TARGET workgroups run (at most NT_MAX_S splits,
// at least one 64-wide step per wave)
#ifndef LSL_NT_TARGET
#define LSL_NT_TARGET 384
#endif
constexpr int64_t NT_TARGET = LSL_NT_TARGET, NT_MAX_S = 16;
static void nt_plan(int64_t T, int64_t K, int& S, int& steps) {
  const int64_t tiles = (T + 63) / 64, KT = K / 64;
  S = 1;
  steps = (int)KT;
  if (tiles <= 0 || KT <= 0) return;
  int64_t s = (NT_TARGET + tiles - 1) / tiles;
  if (s > NT_MAX_S) s = NT_MAX_S;
  if (s > KT / 4) s = KT / 4;
  if (s < 1) s = 1;
  steps = (int)((KT + s - 1) / s);
  S = (int)((KT + steps - 1) / steps);
}
static int nt_splits(int64_t T, int64_t K) {
  int S, steps;
  nt_plan(T, K, S, steps);
  return S;
}

// TN: splits of T so that about TN_TARGET workgroups run, each taking at least
// TN_MIN_STEPS 64-token steps
#ifndef LSL_TN_TARGET
#define LSL_TN_TARGET 256
#endif
constexpr int64_t TN_TARGET = LSL_TN_TARGET, TN_MIN_STEPS = 4;
static int tn_splits(int64_t W, int64_t T) {
  const int64_t tiles = (W + 127) / 128;
  const int64_t steps = (T + 63) / 64;
  if (tiles <= 0 || steps <= 0) return 1;  // empty output or no tokens
  int64_t s = (TN_TARGET + tiles - 1) / tiles;
  if (s > steps / TN_MIN_STEPS) s = steps / TN_MIN_STEPS;
  if (s < 1) s = 1;
  const int64_t per = (steps + s - 1) / s;
  return (int)((steps + per - 1) / per);
}

size_t lora_counts_needed(int64_t T, int64_t W) {
  const int64_t a = (T + 63) / 64, b = (W + 127) / 128;
  return (size_t)(a > b ? a : b);
}

// [masked B^T, kl <= 64 rows] + the partial slots
size_t lora_nt_ws_bytes(int64_t T, int64_t K, int kl) {
  (void)kl;
  const int S = nt_splits(T, K);
  return align256((size_t)64 * K * 2) + (S > 1 ? (size_t)((T + 63) / 64) * S * NT_SLOT * sizeof(float) : 0);
}

size_t lora_tn_ws_bytes(int64_t T, int64_t W, int kl) {
  (void)kl;
  const int S = tn_splits(W, T);
  return S > 1 ? (size_t)((W + 127) / 128) * S * TN_SLOT * sizeof(float) : 0;
}

lsl_status lora_counts_zero(unsigned* cnt, size_t n, hipStream_t s) {
  if (n == 0) return LSL_OK;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, cnt, (int)n);
  return check_launch("lora_counts_zero");
}

lsl_status lora_nt_check(const LoraNt& d) {
  if (d.T == 0) return LSL_OK;
  if (d.K % 64 || d.kl <= 0 || d.kl > 64 || d.kl % 8)
    return set_error(LSL_ERR_UNSUPPORTED, "lora side product: K %% 64 and kl in [8, 64] multiple of 8 required");
  if ((d.T + 64) * d.ldp * 2 >= ((int64_t)1 << 32))
    return set_error(LSL_ERR_UNSUPPORTED, "lora side product: operand larger than 4 GiB");
  if (nt_splits(d.T, d.K) > 1 && !d.cnt) return set_error(LSL_ERR_WORKSPACE, "lora side product: no arrival counts");
  return LSL_OK;
}

lsl_status lora_tn_check(const LoraTn& d) {
  if (d.W == 0) return LSL_OK;
  if (d.kl <= 0 || d.kl > 64 || d.kl % 8 || d.W % 8)
    return set_error(LSL_ERR_UNSUPPORTED, "lora grad: kl in [8, 64] multiple of 8 and W %% 8 required");
  if (d.T > 0 && tn_splits(d.W, d.T) > 1 && !d.cnt) return set_error(LSL_ERR_WORKSPACE, "lora grad: no arrival counts");
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
  a.cnt = d.cnt;
  nt_plan(d.T, d.K, a.S, a.steps);
  hipLaunchKernelGGL(lora_nt_kernel, dim3((unsigned)((d.T + 63) / 64), (unsigned)a.S), dim3(256), 0, s, a);
  return check_launch("lora_nt");
}

static TnArgs tn_args(const LoraTn& d, int& tiles, bool& buf) {
  tiles = (int)((d.W + 127) / 128);
  const int S = tn_splits(d.W, d.T);
  const int64_t steps = (d.T + 63) / 64;
  const int64_t per = ((steps + S - 1) / S) * 64;
  TnArgs a{};
  a.p = d.p; a.ldp = d.ldp; a.q = d.q; a.ldq = d.ldq; a.T = d.T; a.W = d.W; a.kl = d.kl;
  a.t_per_split = per; a.S = S; a.part = d.ws; a.cnt = d.cnt;
  a.dA = d.dA; a.dB = d.dA ? nullptr : d.dB; a.scale = d.scale; a.r = d.r; a.nseg = d.nseg;
  for (int i = 0; i < 4; ++i) a.seg.e[i] = d.seg_end[i];
  // buffer descriptors address a split's rows with 32-bit offsets
  // (the loads run up to two steps past a split's rows)
  const int64_t lim = (int64_t)1 << 32;
  buf = (per + 192) * d.ldp * 2 < lim && (per + 192) * d.ldq * 2 < lim;
  return a;
}

lsl_status lora_tn_group_launch(const LoraTn* d, int n, hipStream_t s) {
  if (n < 0 || n > TN_GROUP_MAX) return set_error(LSL_ERR_INVALID_ARG, "lora grad: 0..%d products", TN_GROUP_MAX);
  for (int i = 0; i < n; ++i) LSL_TRY(lora_tn_check(d[i]));
  TnGroup g{};
  bool buf = true;
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    if (d[i].W == 0 || d[i].T == 0) continue;
    bool b;
    g.p[g.n] = tn_args(d[i], g.tiles[g.n], b);
    buf = buf && b;
    g.start[g.n] = (int)blocks;
    blocks += (int64_t)g.tiles[g.n] * g.p[g.n].S;
    if (blocks >= ((int64_t)1 << 31)) return set_error(LSL_ERR_UNSUPPORTED, "lora grad: too many tiles");
    ++g.n;
  }
  if (g.n == 0) return LSL_OK;
  if (buf) hipLaunchKernelGGL((lora_tn_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, s, g);
  else hipLaunchKernelGGL((lora_tn_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, s, g);
  return check_launch("lora_tn");
}

lsl_status lora_tn_launch(const LoraTn& d, hipStream_t s) { return lora_tn_group_launch(&d, 1, s); }

size_t lora_tn_tiles(int64_t W) { return (size_t)((W + 127) / 128); }

lsl_status lora_bt_group_launch(const LoraBt* jobs, int n, hipStream_t s) {
  if (n < 1 || n > 4) return set_error(LSL_ERR_INVALID_ARG, "lora_bt_group: 1..4 transposes");
  BtGroup g{};
  int64_t total = 0;
  for (int i = 0; i < n; ++i) {
    const LoraBt& j = jobs[i];
    if (j.K % 8 || j.kl <= 0 || j.kl > 64 || j.r <= 0) return set_error(LSL_ERR_UNSUPPORTED, "lora_bt_group: shape");
    g.b[i] = j.b_full; g.r[i] = j.r; g.kl[i] = j.kl; g.nseg[i] = j.nseg; g.K[i] = j.K; g.bt[i] = j.bt;
    for (int q = 0; q < 4; ++q) g.seg[i].e[q] = j.seg_end[q];
    total += (int64_t)j.kl * (j.K / 8);
  }
  g.n = n;
  if (total == 0) return LSL_OK;
  hipLaunchKernelGGL(lora_bt_group_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, g);
  return check_launch("lora_bt_group");
}

}  // namespace lsl
