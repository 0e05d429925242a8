// Causal grouped-query attention on gfx950 bf16 MFMA (16x16x32), head_dim 64 or 128.
//
// Forward (one pass, online softmax): a workgroup holds one (sequence, kv head,
// 32-query tile); its G waves are the G query heads of that kv head, so the K/V
// tiles staged in LDS are shared by the whole group and all waves see the same
// causal range. Scores are computed transposed (S^T = K Q^T) so that each lane
// owns one query column: the running max/sum of the online softmax need one
// value per lane, and the probabilities feed the P V product straight from
// registers (the reduction index of an MFMA may be permuted freely as long as
// both operands use the same permutation; V^T is staged in LDS to match).
// The log-sum-exp per query row is saved for the backward.
//
// Backward (the standard gradient of softmax attention, recomputing P from the
// saved log-sum-exp): D_q = sum_d dO O; a dK/dV kernel owns a 64-key tile (one
// 16-key slice per wave) and sums over the G query heads and all query tiles in
// a fixed order; a dQ kernel owns query tiles like the forward. No atomics.
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
LSL_DEV bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
// two 4-element (8-byte) pieces -> one fragment (the permuted reduction index)
LSL_DEV bf16x8 ld4x2(const uint16_t* p0, const uint16_t* p1) {
  u32x2 a = *reinterpret_cast<const u32x2*>(p0), b = *reinterpret_cast<const u32x2*>(p1);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}
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

// Stage rows [r0, r0+nrows) x D of a strided bf16 matrix (zero beyond `valid` rows)
// into LDS row-major [row][D + 8] and/or transposed [D][nrows + 8].
template <int D>
LSL_DEV void stage_rows(const uint16_t* __restrict__ src, int64_t ld, int r0, int nrows, int valid, uint16_t* rm,
                        uint16_t* tr, int tid, int nthreads) {
  const int chunks = nrows * (D / 8);
  for (int c = tid; c < chunks; c += nthreads) {
    int row = c / (D / 8), col = (c % (D / 8)) * 8;
    u32x4 v = (r0 + row) < valid ? *reinterpret_cast<const u32x4*>(src + (int64_t)(r0 + row) * ld + col) : u32x4{0, 0, 0, 0};
    if (rm) *reinterpret_cast<u32x4*>(rm + row * (D + 8) + col) = v;
    if (tr) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t w = v[e >> 1];
        tr[(col + e) * (nrows + 8) + row] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFF));
      }
    }
  }
}

// ---------------------------------------------------------------- forward
// grid (ceil(seq/32), n_kv, batch), block group*64 threads.
template <int D>
__global__ __launch_bounds__(512) void attn_fwd_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * 72];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nthreads = blockDim.x;
  const int qt = gridDim.x - 1 - blockIdx.x;  // heaviest (latest) query tiles first
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int h = kvh * a.group + wave;
  const int q0 = qt * 32;
  const int64_t rowbase = (int64_t)b * a.seq;
  const uint16_t* qp = a.q + rowbase * a.ldq + (int64_t)h * D;
  const uint16_t* kp = a.k + rowbase * a.ldk + (int64_t)kvh * D;
  const uint16_t* vp = a.v + rowbase * a.ldk + (int64_t)kvh * D;
  const int g = lane >> 4, c16 = lane & 15;

  bf16x8 qf[2][D / 32];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    int q = q0 + qs * 16 + c16;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[qs][ks] = q < a.seq ? ld8(qp + (int64_t)q * a.ldq + ks * 32 + g * 8) : bf16x8{};
  }
  f32x4 o[D / 16][2];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o[i][0] = o[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  const int qmax = min(q0 + 31, a.seq - 1);
  const int ntiles = qmax / 64 + 1;
  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = j * 64;
    stage_rows<D>(kp, a.ldk, kv0, 64, a.seq, Ks, nullptr, tid, nthreads);
    stage_rows<D>(vp, a.ldk, kv0, 64, a.seq, nullptr, Vt, tid, nthreads);
    __syncthreads();
    f32x4 s[4][2];
#pragma unroll
    for (int kvs = 0; kvs < 4; ++kvs) {
      s[kvs][0] = s[kvs][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        bf16x8 kf = ld8(Ks + (kvs * 16 + c16) * (D + 8) + ks * 32 + g * 8);
        s[kvs][0] = mfma(kf, qf[0][ks], s[kvs][0]);
        s[kvs][1] = mfma(kf, qf[1][ks], s[kvs][1]);
      }
    }
    bf16x8 pf[2][2], pl[2][2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int q = q0 + qs * 16 + c16;
      float mt = -INFINITY;
#pragma unroll
      for (int kvs = 0; kvs < 4; ++kvs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int kv = kv0 + kvs * 16 + g * 4 + i;
          float x = (kv <= q && kv < a.seq) ? s[kvs][qs][i] * a.scale_log2 : -INFINITY;
          s[kvs][qs][i] = x;
          mt = fmaxf(mt, x);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mn = fmaxf(m[qs], mt);
      const float alpha = exp2f(m[qs] - mn);
      m[qs] = mn;
      float ls = 0.f;
#pragma unroll
      for (int kvs = 0; kvs < 4; ++kvs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = exp2f(s[kvs][qs][i] - mn);
          s[kvs][qs][i] = p;
          ls += p;
        }
      l[qs] = l[qs] * alpha + ls;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[ds][qs][i] *= alpha;
      split8(s[0][qs], s[1][qs], pf[qs][0], pl[qs][0]);
      split8(s[2][qs], s[3][qs], pf[qs][1], pl[qs][1]);
    }
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const uint16_t* vr = Vt + (ds * 16 + c16) * 72;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 vf = ld4x2(vr + kk * 32 + g * 4, vr + kk * 32 + 16 + g * 4);
        o[ds][0] = mfma(vf, pf[0][kk], o[ds][0]);
        o[ds][0] = mfma(vf, pl[0][kk], o[ds][0]);
        o[ds][1] = mfma(vf, pf[1][kk], o[ds][1]);
        o[ds][1] = mfma(vf, pl[1][kk], o[ds][1]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
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

// dK, dV for one 64-key tile of one kv head. grid (ceil(seq/64), n_kv, batch), 4 waves;
// wave w owns keys kv0 + 16w .. +15. Loops over the group's query heads and over
// 32-query tiles from the diagonal down, in a fixed order.
template <int D>
__global__ __launch_bounds__(256) void attn_dkv_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Qs[32 * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * 40];
  __shared__ __attribute__((aligned(16))) uint16_t Os[32 * (D + 8)];   // dO
  __shared__ __attribute__((aligned(16))) uint16_t Ot[D * 40];         // dO^T
  __shared__ float lse_s[32], dsum_s[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kt = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int kv0 = kt * 64;
  const int64_t rowbase = (int64_t)b * a.seq;
  const int g = lane >> 4, c16 = lane & 15;
  const int mykv = kv0 + wave * 16 + c16;  // the key this lane's B-operand column is

  // K and V rows of this wave's 16 keys as B operands (rows kv, reduction d)
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
  f32x4 dk[D / 16], dv[D / 16];  // dK^T, dV^T: lane holds [d = ds*16 + 4g + i][kv = mykv]
#pragma unroll
  for (int i = 0; i < D / 16; ++i) dk[i] = dv[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int qt_begin = kv0 / 32;
  const int qt_end = (a.seq + 31) / 32;
  for (int hh = 0; hh < a.group; ++hh) {
    const int h = kvh * a.group + hh;
    const uint16_t* qp = a.q + rowbase * a.ldq + (int64_t)h * D;
    const uint16_t* dop = a.dout + rowbase * a.ldo + (int64_t)h * D;
    const float* lsep = a.lse + ((int64_t)b * a.n_q + h) * a.seq;
    const float* dsp = a.dsum + ((int64_t)b * a.n_q + h) * a.seq;
    for (int qt = qt_begin; qt < qt_end; ++qt) {
      const int q0 = qt * 32;
      stage_rows<D>(qp, a.ldq, q0, 32, a.seq, Qs, Qt, tid, 256);
      stage_rows<D>(dop, a.ldo, q0, 32, a.seq, Os, Ot, tid, 256);
      if (tid < 32) {
        int q = q0 + tid;
        lse_s[tid] = q < a.seq ? lsep[q] * LOG2E : 0.f;
        dsum_s[tid] = q < a.seq ? dsp[q] : 0.f;
      }
      __syncthreads();
      // S[q][kv] and dP[q][kv]: lane holds q = qs*16 + 4g + i, kv = mykv
      f32x4 s[2], dp[2];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        s[qs] = dp[qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          bf16x8 qa = ld8(Qs + (qs * 16 + c16) * (D + 8) + ks * 32 + g * 8);
          bf16x8 oa = ld8(Os + (qs * 16 + c16) * (D + 8) + ks * 32 + g * 8);
          s[qs] = mfma(qa, kf[ks], s[qs]);
          dp[qs] = mfma(oa, vf[ks], dp[qs]);
        }
      }
      bf16x8 pb[2], pbl[2], dsb[2], dsl[2];
      f32x4 p[2], ds[2];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ql = qs * 16 + g * 4 + i;
          const int q = q0 + ql;
          float pv = (mykv <= q && q < a.seq && mykv < a.seq) ? exp2f(s[qs][i] * a.scale_log2 - lse_s[ql]) : 0.f;
          p[qs][i] = pv;
          ds[qs][i] = pv * (dp[qs][i] - dsum_s[ql]);
        }
      split8(p[0], p[1], pb[0], pbl[0]);
      split8(ds[0], ds[1], dsb[0], dsl[0]);
      (void)pb[1]; (void)pbl[1]; (void)dsb[1]; (void)dsl[1];
      // dV^T += dO^T P ; dK^T += Q^T dS   (reduction over the 32 queries, permuted)
#pragma unroll
      for (int dd = 0; dd < D / 16; ++dd) {
        const uint16_t* otr = Ot + (dd * 16 + c16) * 40;
        const uint16_t* qtr = Qt + (dd * 16 + c16) * 40;
        bf16x8 oa = ld4x2(otr + g * 4, otr + 16 + g * 4);
        bf16x8 qa = ld4x2(qtr + g * 4, qtr + 16 + g * 4);
        dv[dd] = mfma(oa, pb[0], dv[dd]);
        dv[dd] = mfma(oa, pbl[0], dv[dd]);
        dk[dd] = mfma(qa, dsb[0], dk[dd]);
        dk[dd] = mfma(qa, dsl[0], dk[dd]);
      }
      __syncthreads();
    }
  }
  if (mykv < a.seq) {
    uint16_t* dkp = a.dk + (rowbase + mykv) * a.ldk + (int64_t)kvh * D;
    uint16_t* dvp = a.dv + (rowbase + mykv) * a.ldk + (int64_t)kvh * D;
    // lane holds d = dd*16 + 4g + i for key mykv: scatter 4 consecutive d
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) {
      const f32x4& rk = dk[dd];
      const f32x4& rv = dv[dd];
      *reinterpret_cast<u32x2*>(dkp + dd * 16 + g * 4) =
          u32x2{pack2(rk[0] * a.scale, rk[1] * a.scale), pack2(rk[2] * a.scale, rk[3] * a.scale)};
      *reinterpret_cast<u32x2*>(dvp + dd * 16 + g * 4) = u32x2{pack2(rv[0], rv[1]), pack2(rv[2], rv[3])};
    }
  }
}

// dQ for one 32-query tile of each of the group's heads (wave = head), like the forward.
// grid (ceil(seq/32), n_kv, batch), block group*64 threads.
template <int D>
__global__ __launch_bounds__(512) void attn_dq_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * (D + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * 72];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nthreads = blockDim.x;
  const int qt = gridDim.x - 1 - blockIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int h = kvh * a.group + wave;
  const int q0 = qt * 32;
  const int64_t rowbase = (int64_t)b * a.seq;
  const int g = lane >> 4, c16 = lane & 15;
  const uint16_t* qp = a.q + rowbase * a.ldq + (int64_t)h * D;
  const uint16_t* dop = a.dout + rowbase * a.ldo + (int64_t)h * D;
  const uint16_t* kp = a.k + rowbase * a.ldk + (int64_t)kvh * D;
  const uint16_t* vp = a.v + rowbase * a.ldk + (int64_t)kvh * D;

  bf16x8 qf[2][D / 32], of[2][D / 32];
  float lse2[2], dsm[2];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    int q = q0 + qs * 16 + c16;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      qf[qs][ks] = q < a.seq ? ld8(qp + (int64_t)q * a.ldq + ks * 32 + g * 8) : bf16x8{};
      of[qs][ks] = q < a.seq ? ld8(dop + (int64_t)q * a.ldo + ks * 32 + g * 8) : bf16x8{};
    }
    lse2[qs] = q < a.seq ? a.lse[((int64_t)b * a.n_q + h) * a.seq + q] * LOG2E : 0.f;
    dsm[qs] = q < a.seq ? a.dsum[((int64_t)b * a.n_q + h) * a.seq + q] : 0.f;
  }
  f32x4 dq[D / 16][2];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) dq[i][0] = dq[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int qmax = min(q0 + 31, a.seq - 1);
  const int ntiles = qmax / 64 + 1;
  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = j * 64;
    stage_rows<D>(kp, a.ldk, kv0, 64, a.seq, Ks, Kt, tid, nthreads);
    stage_rows<D>(vp, a.ldk, kv0, 64, a.seq, Vs, nullptr, tid, nthreads);
    __syncthreads();
    // S^T and dP^T: lane holds kv = kvs*16 + 4g + i, q = qs*16 + c16
    bf16x8 dsf[2][2], dsl[2][2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      f32x4 s[4], dp[4];
#pragma unroll
      for (int kvs = 0; kvs < 4; ++kvs) {
        s[kvs] = dp[kvs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          bf16x8 ka = ld8(Ks + (kvs * 16 + c16) * (D + 8) + ks * 32 + g * 8);
          bf16x8 va = ld8(Vs + (kvs * 16 + c16) * (D + 8) + ks * 32 + g * 8);
          s[kvs] = mfma(ka, qf[qs][ks], s[kvs]);
          dp[kvs] = mfma(va, of[qs][ks], dp[kvs]);
        }
      }
      const int q = q0 + qs * 16 + c16;
#pragma unroll
      for (int kvs = 0; kvs < 4; ++kvs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kv = kv0 + kvs * 16 + g * 4 + i;
          float pv = (kv <= q && kv < a.seq && q < a.seq) ? exp2f(s[kvs][i] * a.scale_log2 - lse2[qs]) : 0.f;
          s[kvs][i] = pv * (dp[kvs][i] - dsm[qs]);
        }
      split8(s[0], s[1], dsf[qs][0], dsl[qs][0]);
      split8(s[2], s[3], dsf[qs][1], dsl[qs][1]);
    }
    // dQ^T += K^T dS^T (reduction over 64 keys, permuted like the forward's P V)
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) {
      const uint16_t* kr = Kt + (dd * 16 + c16) * 72;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 ka = ld4x2(kr + kk * 32 + g * 4, kr + kk * 32 + 16 + g * 4);
        dq[dd][0] = mfma(ka, dsf[0][kk], dq[dd][0]);
        dq[dd][0] = mfma(ka, dsl[0][kk], dq[dd][0]);
        dq[dd][1] = mfma(ka, dsf[1][kk], dq[dd][1]);
        dq[dd][1] = mfma(ka, dsl[1][kk], dq[dd][1]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int q = q0 + qs * 16 + c16;
    if (q >= a.seq) continue;
    uint16_t* dp = a.out + (rowbase + q) * a.ldq + (int64_t)h * D;
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) {
      const f32x4& r = dq[dd][qs];
      *reinterpret_cast<u32x2*>(dp + dd * 16 + g * 4) =
          u32x2{pack2(r[0] * a.scale, r[1] * a.scale), pack2(r[2] * a.scale, r[3] * a.scale)};
    }
  }
}

// ---------------------------------------------------------------- host
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
  dim3 grid((unsigned)((a.seq + 31) / 32), (unsigned)a.n_kv, (unsigned)a.batch);
  dim3 block((unsigned)(64 * a.group));
  if (d == 128) hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, block, 0, s, a);
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
  dim3 gk((unsigned)((a.seq + 63) / 64), (unsigned)a.n_kv, (unsigned)a.batch);
  if (d == 128) hipLaunchKernelGGL(attn_dkv_kernel<128>, gk, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(attn_dkv_kernel<64>, gk, dim3(256), 0, s, a);
  dim3 gq((unsigned)((a.seq + 31) / 32), (unsigned)a.n_kv, (unsigned)a.batch);
  if (d == 128) hipLaunchKernelGGL(attn_dq_kernel<128>, gq, dim3(64 * a.group), 0, s, a);
  else hipLaunchKernelGGL(attn_dq_kernel<64>, gq, dim3(64 * a.group), 0, s, a);
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
