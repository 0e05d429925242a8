// Causal grouped-query attention on gfx950 bf16 MFMA (16x16x32), head_dim 64 or 128.
//
// Forward (one pass, online softmax): a workgroup holds one (sequence, kv head,
// 32-query tile); its G waves are the G query heads of that kv head, so the K/V
// tiles staged in LDS are shared by the whole group and all waves see the same
// causal range. Scores are computed transposed (S^T = K Q^T) so that each lane
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

// ---------------------------------------------------------------- forward
// grid (ceil(seq / (16 NQS)), n_kv, batch), block group*64 threads; wave = query
// head, 16 NQS queries per wave.
template <int D, int NQS, int NW>
__global__ __launch_bounds__(64 * NW) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int QT = 16 * NQS, LD = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qt = gridDim.x - 1 - blockIdx.x;  // heaviest (latest) query tiles first
  const int kvh = blockIdx.y, b = blockIdx.z;
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
    bf16x8 pf[NQS][2];
#pragma unroll
    for (int qs = 0; qs < NQS; ++qs) {
      const int q = q0 + qs * 16 + c16;
      float mt = -INFINITY;
#pragma unroll
      for (int kvs = 0; kvs < 4; ++kvs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kv = kv0 + kvs * 16 + g * 4 + i;
          const float x = (kv <= q && kv < a.seq) ? sc[kvs][qs][i] * a.scale_log2 : -INFINITY;
          sc[kvs][qs][i] = x;
          mt = fmaxf(mt, x);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mn = fmaxf(m[qs], mt);  // finite: key 0 is visible to every query
      const float alpha = exp2_ftz(m[qs] - mn);
      m[qs] = mn;
      float ls = 0.f;
#pragma unroll
      for (int kvs = 0; kvs < 4; ++kvs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = exp2_ftz(sc[kvs][qs][i] - mn);
          sc[kvs][qs][i] = pv;
          ls += pv;
        }
      l[qs] = l[qs] * alpha + ls;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[ds][qs][i] *= alpha;
      pf[qs][0] = pack8(sc[0][qs], sc[1][qs]);
      pf[qs][1] = pack8(sc[2][qs], sc[3][qs]);
    }
    // O^T += V^T P^T (reduction over the 64 keys in the permuted order of pf)
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 vf = ld_tr8(Vs, LD, kk * 32, ds * 16, lane);
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) o[ds][qs] = mfma(vf, pf[qs][kk], o[ds][qs]);
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

// ---------------------------------------------------------------- backward
// D[b][h][q] = sum_d dO[q][d] * O[q][d]; one wave per (row, head).
template <int D>
__global__ void attn_dsum_kernel(const AttnArgs a) {
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

// dK, dV for one 32-key tile of one kv head. grid (ceil(seq/32), n_kv, batch),
// block 128 * HG threads with HG = min(group, 4) head groups of two waves; wave
// (hg, w) owns keys kv0 + 16w .. +15 and the query heads hg, hg + HG, ... of the
// kv head. Each head group walks 64-query tiles from the diagonal down (the next
// tile is fetched into registers while the current one is computed); at the end
// the head groups' partial dK/dV are added in head-group order through LDS.
constexpr int DKV_QT = 64;
template <int D>
__global__ __launch_bounds__(512) void attn_dkv_kernel(const AttnArgs a) {
  constexpr int LD = D + 8;
  constexpr int CH = DKV_QT * D / 8 / 128;  // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * 2 * DKV_QT * LD];
  __shared__ float lse_s[4][DKV_QT], dsum_s[4][DKV_QT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int HG = blockDim.x >> 7, hg = wave >> 1, ws = wave & 1, htid = tid & 127;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int kv0 = blockIdx.x * 32;  // heaviest (earliest) key tiles are dispatched first
  const int64_t rowbase = (int64_t)b * a.seq;
  const int g = lane >> 4, c16 = lane & 15;
  const int mykv = kv0 + ws * 16 + c16;
  uint16_t* Qs = lds + hg * 2 * DKV_QT * LD;
  uint16_t* Os = Qs + DKV_QT * LD;

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
  f32x4 dk[D / 16], dv[D / 16];  // dK^T, dV^T: lane holds [d = dd*16 + 4g + i][kv = mykv]
#pragma unroll
  for (int i = 0; i < D / 16; ++i) dk[i] = dv[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int qt_begin = kv0 / DKV_QT;
  const int nq = (a.seq + DKV_QT - 1) / DKV_QT - qt_begin;
  const int iters = (a.group + HG - 1) / HG * nq;  // the same count for every head group
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

  fetch(0);
  for (int it = 0; it < iters; ++it) {
    const bool act = hg + (it / nq) * HG < a.group;
    const int q0 = (qt_begin + it % nq) * DKV_QT;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = htid + c * 128, row = idx / (D / 8), col = (idx % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(Qs + row * LD + col) = pq[c];
      *reinterpret_cast<u32x4*>(Os + row * LD + col) = po[c];
    }
    if (htid < DKV_QT) {
      lse_s[hg][htid] = plse * LOG2E;
      dsum_s[hg][htid] = pds;
    }
    __syncthreads();
    if (it + 1 < iters) fetch(it + 1);
    if (act) {
      // S[q][kv], dP[q][kv] for 64 queries: lane holds q = qs*16 + 4g + i, kv = mykv
      f32x4 p[4], ds[4];
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) {
        f32x4 sv = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          sv = mfma(ld8(Qs + (qs * 16 + c16) * LD + ks * 32 + g * 8), kf[ks], sv);
          dp = mfma(ld8(Os + (qs * 16 + c16) * LD + ks * 32 + g * 8), vf[ks], dp);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ql = qs * 16 + g * 4 + i;
          const int q = q0 + ql;
          const bool keep = mykv <= q && q < a.seq && mykv < a.seq;
          const float pv = exp2_ftz(keep ? sv[i] * a.scale_log2 - lse_s[hg][ql] : -INFINITY);
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
          const bf16x8 oa = ld_tr8(Os, LD, kk * 32, dd * 16, lane);
          const bf16x8 qa = ld_tr8(Qs, LD, kk * 32, dd * 16, lane);
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
  if (hg != 0 || mykv >= a.seq) return;
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
}

// dQ for one 16 NQS-query tile of each of the group's heads (wave = head), like
// the forward. grid (ceil(seq / (16 NQS)), n_kv, batch), block group*64 threads.
template <int D, int NQS, int NW>
__global__ __launch_bounds__(64 * NW) void attn_dq_kernel(const AttnArgs a) {
  constexpr int QT = 16 * NQS, LD = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qt = gridDim.x - 1 - blockIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
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
#pragma unroll
    for (int qs = 0; qs < NQS; ++qs) {
      const int q = q0 + qs * 16 + c16;
#pragma unroll
      for (int kvs = 0; kvs < 4; ++kvs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kv = kv0 + kvs * 16 + g * 4 + i;
          const bool keep = kv <= q && kv < a.seq && q < a.seq;
          const float pv = exp2_ftz(keep ? sc[kvs][qs][i] * a.scale_log2 - lse2[qs] : -INFINITY);
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

// ---------------------------------------------------------------- host
#ifndef LSL_ATT_QT
#define LSL_ATT_QT 16
#endif
constexpr int ATT_QT = LSL_ATT_QT;  // queries per wave in the forward and dQ kernels (16 or 32)

struct FwdKernel {
  template <int D, int NW> static void launch(dim3 g, dim3 b, hipStream_t s, const AttnArgs& a) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, ATT_QT / 16, NW>), g, b, 0, s, a);
  }
};
struct DqKernel {
  template <int D, int NW> static void launch(dim3 g, dim3 b, hipStream_t s, const AttnArgs& a) {
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
  if (ldq < (int64_t)n_q * d || ldk < (int64_t)n_kv * d || ldq % 8 || ldk % 8)
    return set_error(LSL_ERR_INVALID_ARG, "%s: leading dimensions too small or not multiples of 8", fn);
  return LSL_OK;
}

lsl_status attention_fwd_launch(const AttnArgs& a0, int d, hipStream_t s) {
  AttnArgs a = a0;
  if ((int64_t)a.batch * a.seq == 0) return LSL_OK;
  dim3 grid((unsigned)((a.seq + ATT_QT - 1) / ATT_QT), (unsigned)a.n_kv, (unsigned)a.batch);
  dim3 block((unsigned)(64 * a.group));
  if (d == 128) launch_by_group<FwdKernel, 128>(a.group, grid, block, s, a);
  else launch_by_group<FwdKernel, 64>(a.group, grid, block, s, a);
  return check_launch("attention_fwd");
}

lsl_status attention_bwd_launch(const AttnArgs& a0, int d, hipStream_t s) {
  AttnArgs a = a0;
  int64_t T = (int64_t)a.batch * a.seq;
  if (T == 0) return LSL_OK;
  dim3 gs((unsigned)((T * a.n_q + 3) / 4));
  if (d == 128) hipLaunchKernelGGL(attn_dsum_kernel<128>, gs, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(attn_dsum_kernel<64>, gs, dim3(256), 0, s, a);
  a.dsum = a.dsum_out;
  dim3 gk((unsigned)((a.seq + 31) / 32), (unsigned)a.n_kv, (unsigned)a.batch);
  dim3 bk((unsigned)(128 * std::min(a.group, 4)));
  if (d == 128) hipLaunchKernelGGL(attn_dkv_kernel<128>, gk, bk, 0, s, a);
  else hipLaunchKernelGGL(attn_dkv_kernel<64>, gk, bk, 0, s, a);
  dim3 gq((unsigned)((a.seq + ATT_QT - 1) / ATT_QT), (unsigned)a.n_kv, (unsigned)a.batch);
  if (d == 128) launch_by_group<DqKernel, 128>(a.group, gq, dim3(64 * a.group), s, a);
  else launch_by_group<DqKernel, 64>(a.group, gq, dim3(64 * a.group), s, a);
  return check_launch("attention_bwd");
}

size_t attention_ws_bytes(int batch, int seq, int n_q) { return align256((size_t)batch * n_q * seq * sizeof(float)); }

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

extern "C" size_t lsl_attention_workspace_bytes(int32_t batch, int32_t seq, int32_t n_q, int32_t, int32_t) {
  if (batch < 0 || seq < 0 || n_q <= 0) return 0;
  return attention_ws_bytes(batch, seq, n_q);
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
  size_t need = attention_ws_bytes(batch, seq, n_q);
  if (!ws || ws_bytes < need) return set_error(LSL_ERR_WORKSPACE, "%s: workspace %zu < %zu", fn, ws_bytes, need);
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.ldq = ldq; a.ldk = ldk;
  a.o = o; a.dout = dout; a.ldo = ldo; a.lse = lse; a.dsum_out = (float*)ws; a.o32 = (float*)o32;
  a.out = dq; a.dk = dk; a.dv = dv;
  a.batch = batch; a.seq = seq; a.n_q = n_q; a.n_kv = n_kv; a.group = n_q / n_kv;
  a.scale = 1.0f / sqrtf((float)head_dim);
  a.scale_log2 = a.scale * LOG2E;
  return attention_bwd_launch(a, head_dim, (hipStream_t)stream);
}
