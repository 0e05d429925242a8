// Fused, vocabulary-chunked token cross-entropy (forward and backward).
//
// The pages measure what the naive logits term costs (bytes per logit element,
// "Exact Layer Streaming ...", abstract); here no [T x V] logits tensor is ever
// written. Forward: one MFMA GEMM pass z = hN W^T whose epilogue reduces every
// vocabulary tile to a (max, sum exp) pair per token and picks the
// label logit; a second kernel merges the tile pairs in index order into the
// log-sum-exp, and a single workgroup sums the loss in a fixed order.
// Backward: per vocabulary chunk, the GEMM recomputes z and writes
// G = s (softmax - onehot) for that chunk only (hi + lo bf16, L2/MALL resident),
// then dH += G W_chunk accumulates in float32 across chunks in chunk order.
#include "common.h"
#include "gemm.h"
#include "api_util.h"

namespace lsl {

#ifndef LSL_CE_CHUNK
#define LSL_CE_CHUNK 32768
#endif
constexpr int64_t CE_CHUNK = LSL_CE_CHUNK;  // vocabulary columns per backward chunk

struct CePlan {
  size_t nvalid, part, zlab, lossv, lse, g, dh32, total;
  int splits;
};

// dH = sum over chunks of G_c W_c is accumulated in `splits` float32 partial
// sums, each over its own share of every chunk's reduction (so that enough
// workgroups run on the T x H output), added in split order at the end.
static int ce_acc_splits(int64_t T, int64_t H, int64_t vc) { return gemm_acc32_splits(T, H, vc); }

static CePlan ce_plan(int64_t T, int64_t H, int64_t V) {
  CePlan p{};
  size_t off = 0;
  auto take = [&](size_t b) { size_t o = off; off = align256(off + b); return o; };
  p.nvalid = take(4);
  size_t common = off;
  const int bn = gemm_ce_tile_n(T, V, H);
  int64_t ntiles = (V + bn - 1) / bn;
  p.part = take((size_t)ntiles * T * 8);
  p.zlab = take((size_t)T * 4);
  p.lossv = take((size_t)T * 4);
  p.lse = take((size_t)T * 4);  // the log-probability call's own log-sum-exp
  size_t fwd_end = off;
  off = common;
  int64_t vc = V < CE_CHUNK ? V : CE_CHUNK;
  p.g = take((size_t)T * vc * 2);
  p.splits = ce_acc_splits(T, H, vc);
  p.dh32 = take((size_t)p.splits * T * H * 4);
  p.total = std::max(fwd_end, off);
  return p;
}

__global__ void ce_count_valid_kernel(const int32_t* __restrict__ labels, int64_t T, int ignore, int64_t V,
                                      float* __restrict__ nvalid) {
  __shared__ int cnt[256];
  int c = 0;
  for (int64_t t = threadIdx.x; t < T; t += 256) {
    int l = labels[t];
    c += (l != ignore && l >= 0 && l < V) ? 1 : 0;
  }
  cnt[threadIdx.x] = c;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) cnt[threadIdx.x] += cnt[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) *nvalid = (float)cnt[0];
}

// lse[t] = log sum over the per-tile partials (max, sum of exp); lossv[t] = lse - z_label
// (0 if ignored). A workgroup takes 64 rows; its 16 waves take every 16th tile
// (online max/sum merge), then wave 0 merges the 16 results in wave order, so
// the result depends on the tile count only.
constexpr int LSE_WAVES = 16;
__global__ __launch_bounds__(64 * LSE_WAVES) void ce_lse_kernel(const float2* __restrict__ part, int64_t ntiles,
                                                               int64_t T, const int32_t* __restrict__ labels,
                                                               const float* __restrict__ zlab, int ignore, int64_t V,
                                                               float* __restrict__ lse, float* __restrict__ lossv) {
  __shared__ float sm[LSE_WAVES][64], ss[LSE_WAVES][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 64 + lane;
  float m = -INFINITY, sum = 0.f;
  if (t < T) {
    for (int64_t i = w; i < ntiles; i += LSE_WAVES) {
      const float2 p = part[i * T + t];
      if (p.x == -INFINITY) continue;
      if (p.x > m) {
        sum = sum * expf(m - p.x) + p.y;
        m = p.x;
      } else {
        sum += p.y * expf(p.x - m);
      }
    }
  }
  sm[w][lane] = m;
  ss[w][lane] = sum;
  __syncthreads();
  if (w != 0 || t >= T) return;
  float mx = -INFINITY;
  for (int j = 0; j < LSE_WAVES; ++j) mx = fmaxf(mx, sm[j][lane]);
  float s = 0.f;
  for (int j = 0; j < LSE_WAVES; ++j)
    if (sm[j][lane] != -INFINITY) s += ss[j][lane] * expf(sm[j][lane] - mx);
  const float l = mx + logf(s);
  lse[t] = l;
  const int lab = labels[t];
  lossv[t] = (lab != ignore && lab >= 0 && lab < V) ? l - zlab[t] : 0.f;
}

// dH = bf16(sum of the split partial sums, in split order); 4 values per thread
__global__ void ce_dh_reduce_kernel(const float* __restrict__ part, int S, int64_t n, uint16_t* __restrict__ dh) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 v = *reinterpret_cast<const f32x4*>(part + i);
  for (int s = 1; s < S; ++s) {
    const f32x4 q = *reinterpret_cast<const f32x4*>(part + (int64_t)s * n + i);
    v = f32x4{v[0] + q[0], v[1] + q[1], v[2] + q[2], v[3] + q[3]};
  }
  *reinterpret_cast<u32x2*>(dh + i) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
}

// loss = sum(lossv) / nvalid, one workgroup, fixed summation order
__global__ void ce_loss_kernel(const float* __restrict__ lossv, int64_t T, const float* __restrict__ nvalid,
                               float* __restrict__ loss) {
  __shared__ float acc[256];
  float s = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += 256) s += lossv[t];
  acc[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if ((int)threadIdx.x < k) acc[threadIdx.x] += acc[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = *nvalid > 0.f ? acc[0] / *nvalid : 0.f;
}

// logp[t] = -lossv[t] (z_label - lse, 0 where ignored); seq_logp[b] = sum of
// sequence b's tokens, one workgroup per sequence, fixed summation order.
__global__ void ce_logp_kernel(const float* __restrict__ lossv, int64_t seq, float* __restrict__ logp,
                               float* __restrict__ seq_logp) {
  __shared__ float acc[256];
  const int64_t t0 = (int64_t)blockIdx.x * seq;
  float s = 0.f;
  for (int64_t j = threadIdx.x; j < seq; j += 256) {
    const float v = -lossv[t0 + j];
    logp[t0 + j] = v;
    s += v;
  }
  if (!seq_logp) return;
  acc[threadIdx.x] = s;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if ((int)threadIdx.x < k) acc[threadIdx.x] += acc[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) seq_logp[blockIdx.x] = acc[0];
}

static lsl_status ce_check(const char* fn, int64_t T, int64_t H, int64_t V) {
  if (T < 0 || H <= 0 || V <= 0) return set_error(LSL_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (H % 64 || V % 64) return set_error(LSL_ERR_UNSUPPORTED, "%s: hidden and vocab must be multiples of 64", fn);
  if (V > (int64_t)1 << 31) return set_error(LSL_ERR_UNSUPPORTED, "%s: vocab too large", fn);
  return LSL_OK;
}

}  // namespace lsl

using namespace lsl;

extern "C" size_t lsl_ce_workspace_bytes(int64_t T, int64_t H, int64_t V) {
  if (ce_check("lsl_ce_workspace_bytes", T, H, V) != LSL_OK) return 0;
  return ce_plan(T, H, V).total;
}

extern "C" lsl_status fused_ce_loss_fwd(const uint16_t* hN, const uint16_t* w_lm, const int32_t* labels, int64_t T,
                                        int64_t H, int64_t V, int32_t ignore_index, float* loss, float* lse, void* ws,
                                        size_t ws_bytes, lsl_stream stream) {
  const char* fn = "fused_ce_loss_fwd";
  LSL_TRY(ce_check(fn, T, H, V));
  LSL_TRY(check_ptrs(fn, {w_lm}));
  LSL_TRY(check_ptrs(fn, {loss}, 4));
  CePlan p = ce_plan(T, H, V);
  if (!ws || ws_bytes < p.total || !aligned(ws, 256))
    return set_error(LSL_ERR_WORKSPACE, "%s: workspace %zu < %zu (or not 256-byte aligned)", fn, ws_bytes, p.total);
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  float* nvalid = (float*)(w + p.nvalid);
  if (T == 0) {
    hipLaunchKernelGGL(ce_loss_kernel, dim3(1), dim3(256), 0, s, (const float*)nullptr, (int64_t)0,
                       (const float*)nvalid, loss);
    return check_launch(fn);
  }
  LSL_TRY(check_ptrs(fn, {hN}));
  LSL_TRY(check_ptrs(fn, {labels, lse}, 4));
  GemmDesc g;
  g.x = hN; g.ldx = H; g.wfmt = LSL_WFMT_BF16; g.wb = w_lm; g.M = T; g.N = V; g.K = H;
  g.epi = 1; g.labels = labels; g.part = w + p.part; g.zlab = (float*)(w + p.zlab); g.ignore = ignore_index;
  g.vocab = V;
  LSL_TRY(gemm_check(g));  // before anything is enqueued
  hipLaunchKernelGGL(ce_count_valid_kernel, dim3(1), dim3(256), 0, s, labels, T, ignore_index, V, nvalid);
  LSL_TRY(gemm_launch(g, s));
  const int bn = gemm_ce_tile_n(T, V, H);
  int64_t ntiles = (V + bn - 1) / bn;
  hipLaunchKernelGGL(ce_lse_kernel, dim3((unsigned)((T + 63) / 64)), dim3(64 * LSE_WAVES), 0, s, (const float2*)(w + p.part),
                     ntiles, T, labels, (const float*)(w + p.zlab), ignore_index, V, lse, (float*)(w + p.lossv));
  hipLaunchKernelGGL(ce_loss_kernel, dim3(1), dim3(256), 0, s, (const float*)(w + p.lossv), T, (const float*)nvalid,
                     loss);
  return check_launch(fn);
}

extern "C" lsl_status fused_ce_loss_bwd(const uint16_t* hN, const uint16_t* w_lm, const int32_t* labels,
                                        const float* lse, int64_t T, int64_t H, int64_t V, int32_t ignore_index,
                                        float grad_scale, uint16_t* dhN, void* ws, size_t ws_bytes,
                                        lsl_stream stream) {
  const char* fn = "fused_ce_loss_bwd";
  LSL_TRY(ce_check(fn, T, H, V));
  if (T == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {hN, w_lm, dhN}));
  LSL_TRY(check_ptrs(fn, {labels, lse}, 4));
  CePlan p = ce_plan(T, H, V);
  if (!ws || ws_bytes < p.total || !aligned(ws, 256))
    return set_error(LSL_ERR_WORKSPACE, "%s: workspace %zu < %zu (or not 256-byte aligned)", fn, ws_bytes, p.total);
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  float* nvalid = (float*)(w + p.nvalid);
  uint16_t* G = (uint16_t*)(w + p.g);
  float* dh32 = (float*)(w + p.dh32);
  const int64_t nchunks = (V + CE_CHUNK - 1) / CE_CHUNK;
  // the two GEMMs of vocabulary chunk c: G = coef (softmax - onehot) for the
  // chunk, bf16 [T x vc]; then dH (+)= G W_c in float32
  auto chunk = [&](int64_t c, GemmDesc& g1, GemmDesc& g2) {
    const int64_t v0 = c * CE_CHUNK;
    const int64_t vc = std::min(CE_CHUNK, V - v0);
    const uint16_t* wc = w_lm + v0 * H;
    g1.x = hN; g1.ldx = H; g1.wfmt = LSL_WFMT_BF16; g1.wb = wc; g1.M = T; g1.N = vc; g1.K = H;
    g1.epi = 2; g1.labels = labels; g1.lse = lse; g1.nvalid = nvalid; g1.gscale = grad_scale;
    g1.ignore = ignore_index; g1.vocab_off = v0; g1.vocab = V;
    g1.y = G; g1.ldy = vc;
    g2.x = G; g2.ldx = vc; g2.wfmt = LSL_WFMT_BF16; g2.kn = true; g2.wb = wc;
    g2.M = T; g2.N = H; g2.K = vc;
    g2.epi = 3; g2.out32 = dh32; g2.ldo32 = H; g2.first = c == 0 ? 1 : 0;
    g2.acc_splits = p.splits; g2.o32_split = T * H;
    g2.y = (p.splits == 1 && c == nchunks - 1) ? dhN : nullptr; g2.ldy = H;
  };
  for (int64_t c = 0; c < nchunks; ++c) {  // every chunk's conditions before anything is enqueued
    GemmDesc g1, g2;
    chunk(c, g1, g2);
    LSL_TRY(gemm_check(g1));
    LSL_TRY(gemm_check(g2));
  }
  hipLaunchKernelGGL(ce_count_valid_kernel, dim3(1), dim3(256), 0, s, labels, T, ignore_index, V, nvalid);
  for (int64_t c = 0; c < nchunks; ++c) {
    GemmDesc g1, g2;
    chunk(c, g1, g2);
    LSL_TRY(gemm_launch(g1, s));
    LSL_TRY(gemm_launch(g2, s));
  }
  if (p.splits > 1) {
    const int64_t n4 = T * H / 4;
    hipLaunchKernelGGL(ce_dh_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, dh32, p.splits,
                       T * H, dhN);
    return check_launch(fn);
  }
  return LSL_OK;
}

extern "C" lsl_status fused_ce_logprobs(const uint16_t* hN, const uint16_t* w_lm, const int32_t* labels, int64_t T,
                                        int64_t H, int64_t V, int32_t ignore_index, int32_t batch, float* logp,
                                        float* seq_logp, void* ws, size_t ws_bytes, lsl_stream stream) {
  const char* fn = "fused_ce_logprobs";
  LSL_TRY(ce_check(fn, T, H, V));
  if (batch <= 0 || T % batch) return set_error(LSL_ERR_INVALID_ARG, "%s: T must be a multiple of batch > 0", fn);
  if (T == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {hN, w_lm}));
  LSL_TRY(check_ptrs(fn, {labels, logp}, 4));
  if (seq_logp && !aligned(seq_logp, 4)) return set_error(LSL_ERR_INVALID_ARG, "%s: seq_logp misaligned", fn);
  CePlan p = ce_plan(T, H, V);
  if (!ws || ws_bytes < p.total || !aligned(ws, 256))
    return set_error(LSL_ERR_WORKSPACE, "%s: workspace %zu < %zu (or not 256-byte aligned)", fn, ws_bytes, p.total);
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  // the forward's first two stages: per-tile (max, sum exp) and the label logit,
  // then their ordered merge into lse and lossv = lse - z_label
  GemmDesc g;
  g.x = hN; g.ldx = H; g.wfmt = LSL_WFMT_BF16; g.wb = w_lm; g.M = T; g.N = V; g.K = H;
  g.epi = 1; g.labels = labels; g.part = w + p.part; g.zlab = (float*)(w + p.zlab); g.ignore = ignore_index;
  g.vocab = V;
  LSL_TRY(gemm_launch(g, s));
  const int bn = gemm_ce_tile_n(T, V, H);
  int64_t ntiles = (V + bn - 1) / bn;
  hipLaunchKernelGGL(ce_lse_kernel, dim3((unsigned)((T + 63) / 64)), dim3(64 * LSE_WAVES), 0, s,
                     (const float2*)(w + p.part), ntiles, T, labels, (const float*)(w + p.zlab), ignore_index, V,
                     (float*)(w + p.lse), (float*)(w + p.lossv));
  hipLaunchKernelGGL(ce_logp_kernel, dim3((unsigned)batch), dim3(256), 0, s, (const float*)(w + p.lossv),
                     T / batch, logp, seq_logp);
  return check_launch(fn);
}
