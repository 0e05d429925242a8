// Decoder layer forward / backward (with recompute) on one packed layer blob.
//
// The frozen weights of a layer live in one blob (lsl_layer_layout), so a
// streamed slot and a resident copy are byte-identical and the same kernels,
// with the same tiling, run on either: dispatch depends on (cfg, batch, seq)
// only. Per layer the forward is 4 fused LoRA GEMMs (qkv, o, gate|up, down),
// 4 rank-r side products, 2 RMSNorms, RoPE, attention and SwiGLU; residual adds
// are fused into the o and down GEMM epilogues.
#include "common.h"
#include "gemm.h"
#include "small.h"
#include "api_util.h"
#include <vector>

namespace lsl {
struct AttnArgs;
lsl_status attention_fwd_launch(const AttnArgs& a, int d, hipStream_t s);
}  // namespace lsl

extern "C" lsl_status lsl_attention_fwd(const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int32_t,
                                        int32_t, int32_t, int32_t, int32_t, uint16_t*, int64_t, float*, float*,
                                        lsl_stream);
extern "C" lsl_status lsl_attention_bwd(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                                        const uint16_t*, const float*, const float*, int64_t, int64_t, int64_t, int32_t, int32_t,
                                        int32_t, int32_t, int32_t, uint16_t*, uint16_t*, uint16_t*, void*, size_t,
                                        lsl_stream);
extern "C" size_t lsl_attention_workspace_bytes(int32_t, int32_t, int32_t, int32_t, int32_t);

namespace lsl {

// Optional GEMM timing (see lsl_timing_enable). Per calling thread, so layer
// calls on other threads neither see nor touch it.
struct Timing {
  int which = 0;
  std::vector<hipEvent_t> start, stop;
  int count = 0;
};
static thread_local Timing g_timing;

static void timing_mark(int which, bool begin, hipStream_t s) {
  if (g_timing.which != which || g_timing.count >= (int)g_timing.start.size()) return;
  if (begin) {
    (void)hipEventRecord(g_timing.start[g_timing.count], s);  // diagnostics only
  } else {
    (void)hipEventRecord(g_timing.stop[g_timing.count], s);
    ++g_timing.count;
  }
}

struct Dims {
  int64_t T, H, Q, KV, NQKV, I;
  int r, d;
};

static Dims dims_of(const lsl_layer_cfg* c, int batch, int seq) {
  Dims d;
  d.T = (int64_t)batch * seq;
  d.H = c->hidden;
  d.Q = (int64_t)c->n_q * c->head_dim;
  d.KV = (int64_t)c->n_kv * c->head_dim;
  d.NQKV = d.Q + 2 * d.KV;
  d.I = c->inter;
  d.r = c->lora_r;
  d.d = c->head_dim;
  return d;
}

static lsl_status check_cfg(const lsl_layer_cfg* c, const char* fn) {
  if (!c) return set_error(LSL_ERR_INVALID_ARG, "%s: cfg is NULL", fn);
  if (c->hidden <= 0 || c->n_q <= 0 || c->n_kv <= 0 || c->inter <= 0 || c->n_q % c->n_kv)
    return set_error(LSL_ERR_INVALID_ARG, "%s: bad layer sizes", fn);
  if (c->head_dim != 64 && c->head_dim != 128)
    return set_error(LSL_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128 supported)", fn, c->head_dim);
  if (c->n_q / c->n_kv > 8) return set_error(LSL_ERR_UNSUPPORTED, "%s: more than 8 query heads per kv head", fn);
  if (c->hidden % 64 || c->inter % 64)
    return set_error(LSL_ERR_UNSUPPORTED, "%s: hidden and inter must be multiples of 64", fn);
  if (c->hidden > 8192) return set_error(LSL_ERR_UNSUPPORTED, "%s: hidden %d > 8192", fn, c->hidden);
  if (c->lora_r != 8 && c->lora_r != 16)
    return set_error(LSL_ERR_UNSUPPORTED, "%s: fused layer supports LoRA rank 8 or 16 (got %d)", fn, c->lora_r);
  if (c->wfmt != LSL_WFMT_NF4 && c->wfmt != LSL_WFMT_BF16 && c->wfmt != LSL_WFMT_NF4DQ)
    return set_error(LSL_ERR_INVALID_ARG, "%s: unknown weight format %d", fn, c->wfmt);
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return set_error(LSL_ERR_INVALID_ARG, "%s: bad eps/theta", fn);
  if (c->qkv_bias != 0 && c->qkv_bias != 1) return set_error(LSL_ERR_INVALID_ARG, "%s: qkv_bias must be 0 or 1", fn);
  return check_rope_scaling(fn, &c->rope_scaling);
}

// Matrix shapes [n_out x k_in] of the four fused GEMMs.
static void mat_shape(const Dims& d, int i, int64_t& n, int64_t& k) {
  switch (i) {
    case LSL_M_QKV: n = d.NQKV; k = d.H; break;
    case LSL_M_O: n = d.H; k = d.Q; break;
    case LSL_M_GU: n = 2 * d.I; k = d.H; break;
    default: n = d.H; k = d.I; break;
  }
}

static void layout_of(const lsl_layer_cfg* c, lsl_layer_layout* L) {
  Dims d = dims_of(c, 1, 1);
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) { uint64_t o = off; off = align256(off + bytes); return o; };
  L->norm1_off = take(2 * d.H);
  L->norm2_off = take(2 * d.H);
  L->bias_off = c->qkv_bias ? take(2 * d.NQKV) : 0;
  for (int i = 0; i < 4; ++i) {
    int64_t n, k;
    mat_shape(d, i, n, k);
    L->scale_off[i] = 0;
    if (c->wfmt == LSL_WFMT_NF4) {
      L->w_off[i] = take((uint64_t)n * k / 2);
      L->absmax_off[i] = take((uint64_t)n * k / 64 * 4);
    } else if (c->wfmt == LSL_WFMT_NF4DQ) {
      const uint64_t nb = (uint64_t)n * k / 64;
      L->w_off[i] = take((uint64_t)n * k / 2);
      L->absmax_off[i] = take(nb);
      L->scale_off[i] = take((nb + 255) / 256 * 4);
    } else {
      L->w_off[i] = take((uint64_t)n * k * 2);
      L->absmax_off[i] = 0;
    }
  }
  L->total_bytes = off;
}

// The adapter gradients of the four projections (dA and dB each) run as one
// launch at the end of the backward, product j with its partial slots at
// ws_off[j] in the partial region (256-byte aligned, one after another) and
// its arrival counts at cnt_off[j]. Product 2 i is dA of projection
// 3 - i (dA [kl x k]: W = k), 2 i + 1 its dB (W = n), in the backward's order.
struct TnPlan {
  size_t ws_off[9];
  size_t cnt_off[9];
};
static TnPlan tn_plan(const Dims& d) {
  TnPlan t{};
  for (int j = 0; j < 8; ++j) {
    int64_t n, k;
    const int i = 3 - j / 2;
    mat_shape(d, i, n, k);
    const int nseg = i == LSL_M_QKV ? 3 : (i == LSL_M_GU ? 2 : 1);
    const int64_t W = (j & 1) ? n : k;
    t.ws_off[j + 1] = t.ws_off[j] + align256(lora_tn_ws_bytes(d.T, W, nseg * d.r));
    t.cnt_off[j + 1] = t.cnt_off[j] + lora_tn_tiles(W);
  }
  return t;
}

// Workspace plan (byte offsets, all 256-aligned).
// qkv holds the q|k|v GEMM output and qkr its RoPE'd q and k columns (same
// row stride; the v columns of qkr are unused); in the backward the attention
// writes dq and dk into dqkr and dv into dqkv, whose q and k columns then take
// the inverse RoPE of dqkr. So every rounding point keeps its own tensor.
struct Plan {
  size_t n1, tqkv, qkv, qkr, o, lse, to, h1, n2, tgu, gu, a, td;                    // forward
  size_t ud, da, dgu, ugu, dn2, dh1, uo, dob, dqkr, dqkv, uqkv, dn1, attn_ws, o32;  // backward
  size_t bt[4];                                                                   // backward: masked B^T
  size_t part, cnt, ncnt, total;
};

static Plan plan_of(const lsl_layer_cfg* c, int batch, int seq, int mode) {
  Dims d = dims_of(c, batch, seq);
  Plan p{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  const size_t T = (size_t)d.T;
  p.n1 = take(T * d.H * 2);
  p.tqkv = take(T * 3 * d.r * 2);
  p.qkv = take(T * d.NQKV * 2);
  p.qkr = take(T * d.NQKV * 2);
  p.o = take(T * d.Q * 2);
  p.lse = take((size_t)batch * c->n_q * seq * 4);
  p.to = take(T * d.r * 2);
  p.h1 = take(T * d.H * 2);
  p.n2 = take(T * d.H * 2);
  p.tgu = take(T * 2 * d.r * 2);
  p.gu = take(T * 2 * d.I * 2);
  p.a = take(T * d.I * 2);
  p.td = take(T * d.r * 2);
  // one region reused in turn by LoRA split partials and GEMM split-K partials
  const int r = d.r;
  size_t part = std::max({lora_nt_ws_bytes(d.T, d.H, 3 * r), lora_nt_ws_bytes(d.T, d.Q, r),
                          lora_nt_ws_bytes(d.T, d.H, 2 * r), lora_nt_ws_bytes(d.T, d.I, r),
                          gemm_split_bytes(d.T, d.NQKV, d.H), gemm_split_bytes(d.T, d.H, d.Q),
                          gemm_split_bytes(d.T, 2 * d.I, d.H), gemm_split_bytes(d.T, d.H, d.I)});
  if (mode == LSL_MODE_BWD) {
    p.ud = take(T * d.r * 2);
    p.da = take(T * d.I * 2);
    p.dgu = take(T * 2 * d.I * 2);
    p.ugu = take(T * 2 * d.r * 2);
    p.dn2 = take(T * d.H * 2);
    p.dh1 = take(T * d.H * 2);
    p.uo = take(T * d.r * 2);
    p.dob = take(T * d.Q * 2);
    p.dqkr = take(T * d.NQKV * 2);
    p.dqkv = take(T * d.NQKV * 2);
    p.uqkv = take(T * 3 * d.r * 2);
    p.dn1 = take(T * d.H * 2);
    p.attn_ws = take(lsl_attention_workspace_bytes(batch, seq, c->n_q, c->n_kv, c->head_dim));
    p.o32 = take(T * d.Q * 4);
    // the masked B^T of the four projections (u = dy B), made once per backward
    p.bt[LSL_M_QKV] = take((size_t)3 * d.r * d.NQKV * 2);
    p.bt[LSL_M_O] = take((size_t)d.r * d.H * 2);
    p.bt[LSL_M_GU] = take((size_t)2 * d.r * 2 * d.I * 2);
    p.bt[LSL_M_DOWN] = take((size_t)d.r * d.H * 2);
    part = std::max({part, lora_nt_ws_bytes(d.T, d.NQKV, 3 * r), lora_nt_ws_bytes(d.T, d.H, r),
                     lora_nt_ws_bytes(d.T, 2 * d.I, 2 * r), tn_plan(d).ws_off[8],
                     gemm_split_bytes(d.T, d.H, d.NQKV), gemm_split_bytes(d.T, d.Q, d.H),
                     gemm_split_bytes(d.T, d.H, 2 * d.I), gemm_split_bytes(d.T, d.I, d.H)});
  }
  p.part = take(part);
  // the arrival counts of the side products and of the stream-K GEMMs: a region
  // of their own (zeroed by the layer's first RMSNorm launch, left zero by every
  // launch that uses it; the launches that share it run one after another)
  p.ncnt = std::max({lora_counts_needed(d.T, std::max({d.NQKV, 2 * d.I, d.H, d.Q, d.I})),
                     mode == LSL_MODE_BWD ? tn_plan(d).cnt_off[8] : (size_t)0,
                     gemm_counts_needed(d.T, d.NQKV, d.H), gemm_counts_needed(d.T, d.H, d.Q),
                     gemm_counts_needed(d.T, 2 * d.I, d.H), gemm_counts_needed(d.T, d.H, d.I),
                     gemm_counts_needed(d.T, d.H, d.NQKV), gemm_counts_needed(d.T, d.Q, d.H),
                     gemm_counts_needed(d.T, d.H, 2 * d.I), gemm_counts_needed(d.T, d.I, d.H)});
  p.cnt = take(p.ncnt * sizeof(unsigned));
  p.total = off;
  return p;
}

struct LayerPtrs {
  const uint16_t* norm1; const uint16_t* norm2;
  const uint16_t* wb[4]; const uint8_t* wq[4]; const float* wa[4];
  const uint8_t* wq8[4]; const float* wsc[4];  // NF4DQ absmax codes and block constants
  const uint16_t* qkv_bias;                     // bf16 [NQKV] or NULL
};

static LayerPtrs ptrs_of(const lsl_layer_cfg* c, const void* blob) {
  lsl_layer_layout L;
  layout_of(c, &L);
  const char* b = (const char*)blob;
  LayerPtrs p{};
  p.norm1 = (const uint16_t*)(b + L.norm1_off);
  p.norm2 = (const uint16_t*)(b + L.norm2_off);
  p.qkv_bias = c->qkv_bias ? (const uint16_t*)(b + L.bias_off) : nullptr;
  for (int i = 0; i < 4; ++i) {
    if (c->wfmt == LSL_WFMT_NF4) {
      p.wq[i] = (const uint8_t*)(b + L.w_off[i]);
      p.wa[i] = (const float*)(b + L.absmax_off[i]);
    } else if (c->wfmt == LSL_WFMT_NF4DQ) {
      p.wq[i] = (const uint8_t*)(b + L.w_off[i]);
      p.wq8[i] = (const uint8_t*)(b + L.absmax_off[i]);
      p.wsc[i] = (const float*)(b + L.scale_off[i]);
    } else {
      p.wb[i] = (const uint16_t*)(b + L.w_off[i]);
    }
  }
  return p;
}

// y = x W_i^T + s t B_i^T (+ res); t = x A_i^T computed first.
// Forward of one fused LoRA linear: t = x A^T, y = x W^T + s t B^T (+ res).
// With y == nullptr only t is computed.
// dry: only check every launch's conditions (nothing is enqueued).
// t_ready: t already holds x A^T (kept from the forward of the same input), so
// only the GEMM runs.
// defer: a split GEMM leaves its float32 partials in part for the caller to sum.
static lsl_status fused_linear_fwd(const lsl_layer_cfg* c, const Dims& d, const LayerPtrs& W, const lsl_lora_set* lo,
                                   int i, const uint16_t* x, uint16_t* t, bool t_ready, uint16_t* y,
                                   const uint16_t* res, float* part, unsigned* cnt, hipStream_t s, bool dry,
                                   bool defer = false) {
  int64_t n, k;
  mat_shape(d, i, n, k);
  int nseg = i == LSL_M_QKV ? 3 : (i == LSL_M_GU ? 2 : 1);
  int kl = nseg * d.r;
  if (lo && !t_ready) {  // adapters on: t = x A^T first, then the GEMM's LoRA K-step
    LoraNt nt;
    nt.p = x; nt.ldp = k; nt.T = d.T; nt.K = k; nt.kl = kl; nt.a_full = lo->A[i];
    nt.out = t; nt.ldo = kl; nt.ws = part; nt.cnt = cnt;
    LSL_TRY(dry ? lora_nt_check(nt) : lora_nt_launch(nt, s));
  }
  if (!y) return LSL_OK;
  GemmDesc g;
  g.x = x; g.ldx = k; g.wfmt = c->wfmt; g.kn = false;
  g.wb = W.wb[i]; g.wq = W.wq[i]; g.wa = W.wa[i]; g.wq8 = W.wq8[i]; g.wsc = W.wsc[i];
  g.M = d.T; g.N = n; g.K = k;
  g.lora = lo ? 1 : 0; g.la = t; g.ldla = kl; g.kl = kl; g.lb = lo ? lo->B[i] : nullptr; g.r = d.r; g.nseg = nseg;
  if (i == LSL_M_QKV) { g.seg_end[0] = d.Q; g.seg_end[1] = d.Q + d.KV; g.seg_end[2] = d.NQKV; }
  else if (i == LSL_M_GU) { g.seg_end[0] = d.I; g.seg_end[1] = 2 * d.I; }
  else g.seg_end[0] = n;
  g.scale = c->lora_scale;
  g.y = y; g.ldy = n; g.res = res; g.ldres = n; g.split_ws = part; g.cnt = cnt; g.defer_reduce = defer;
  if (i == LSL_M_QKV) g.bias = W.qkv_bias;
  if (dry) return gemm_check(g);
  timing_mark(1 + i, true, s);
  lsl_status st = gemm_launch(g, s);
  timing_mark(1 + i, false, s);
  return st;
}

// Backward of one fused LoRA linear: u = dy B (per projection); dx = dy W + s u A;
// and the descriptors of dA += s u^T x and dB += s dy^T t (per projection) in
// tn[0], tn[1], with their partial slots and counts at tws, tcnt (the caller
// launches them with the other projections').
// bt: the projection's masked B^T, made beforehand (lora_bt_group_launch)
static lsl_status fused_linear_bwd(const lsl_layer_cfg* c, const Dims& d, const LayerPtrs& W, const lsl_lora_set* lo,
                                   const lsl_lora_grads* gr, int i, const uint16_t* x, const uint16_t* t,
                                   const uint16_t* dy, uint16_t* u, uint16_t* dx, float* part, unsigned* cnt,
                                   const uint16_t* bt, LoraTn (&tn)[2], float* const (&tws)[2],
                                   unsigned* const (&tcnt)[2], hipStream_t s, bool dry, bool defer = false) {
  int64_t n, k;
  mat_shape(d, i, n, k);
  int nseg = i == LSL_M_QKV ? 3 : (i == LSL_M_GU ? 2 : 1);
  int kl = nseg * d.r;
  int64_t se[4] = {n, 0, 0, 0};
  if (i == LSL_M_QKV) { se[0] = d.Q; se[1] = d.Q + d.KV; se[2] = d.NQKV; }
  else if (i == LSL_M_GU) { se[0] = d.I; se[1] = 2 * d.I; }
  LoraNt nt;
  nt.p = dy; nt.ldp = n; nt.T = d.T; nt.K = n; nt.kl = kl; nt.a_full = bt; nt.r = d.r; nt.nseg = nseg;
  for (int q = 0; q < 4; ++q) nt.seg_end[q] = se[q];
  nt.out = u; nt.ldo = kl; nt.ws = part; nt.cnt = cnt;
  LSL_TRY(dry ? lora_nt_check(nt) : lora_nt_launch(nt, s));
  if (dx) {
    GemmDesc g;
    g.x = dy; g.ldx = n; g.wfmt = c->wfmt; g.kn = true;
    g.wb = W.wb[i]; g.wq = W.wq[i]; g.wa = W.wa[i]; g.wq8 = W.wq8[i]; g.wsc = W.wsc[i];
    g.M = d.T; g.N = k; g.K = n;
    g.lora = 2; g.la = u; g.ldla = kl; g.kl = kl; g.lb = lo->A[i]; g.r = d.r;
    g.scale = c->lora_scale; g.y = dx; g.ldy = k; g.split_ws = part; g.cnt = cnt; g.defer_reduce = defer;
    if (dry) {
      LSL_TRY(gemm_check(g));
    } else {
      timing_mark(5 + i, true, s);
      lsl_status st = gemm_launch(g, s);
      timing_mark(5 + i, false, s);
      LSL_TRY(st);
    }
  }
  LoraTn& ta = tn[0];
  ta = LoraTn{};
  ta.p = x; ta.ldp = k; ta.q = u; ta.ldq = kl; ta.T = d.T; ta.W = k; ta.kl = kl;
  ta.scale = c->lora_scale; ta.dA = gr->dA[i]; ta.ws = tws[0]; ta.cnt = tcnt[0];
  LoraTn& tb = tn[1];
  tb = LoraTn{};
  tb.p = dy; tb.ldp = n; tb.q = t; tb.ldq = kl; tb.T = d.T; tb.W = n; tb.kl = kl;
  tb.scale = c->lora_scale; tb.dB = gr->dB[i]; tb.r = d.r; tb.nseg = nseg;
  for (int q = 0; q < 4; ++q) tb.seg_end[q] = se[q];
  tb.ws = tws[1]; tb.cnt = tcnt[1];
  LSL_TRY(lora_tn_check(ta));
  return lora_tn_check(tb);
}

// dry: check the conditions of every GEMM and side product, enqueue nothing
// (the other kernels' conditions follow from check_cfg)
// tp: where the four projections' t = x A^T go (the workspace, or the caller's
// t_keep buffer); t_ready: they already hold them (the backward's recompute with
// a t_keep buffer), so the side products are not computed again.
static lsl_status layer_forward(const lsl_layer_cfg* c, const LayerPtrs& W, const lsl_lora_set* lo, const uint16_t* x,
                                int batch, int seq, uint16_t* out, char* ws, const Plan& p, uint16_t* const (&tp)[4],
                                bool t_ready, float* o32, hipStream_t s, bool dry = false) {
  Dims d = dims_of(c, batch, seq);
  float* part = (float*)(ws + p.part);
  uint16_t* n1 = (uint16_t*)(ws + p.n1);
  uint16_t* qkv = (uint16_t*)(ws + p.qkv);
  uint16_t* o = (uint16_t*)(ws + p.o);
  uint16_t* h1 = (uint16_t*)(ws + p.h1);
  uint16_t* n2 = (uint16_t*)(ws + p.n2);
  uint16_t* gu = (uint16_t*)(ws + p.gu);
  uint16_t* a = (uint16_t*)(ws + p.a);
  unsigned* cnt = (unsigned*)(ws + p.cnt);
  const bool tr = t_ready;
  if (dry) {
    LSL_TRY(fused_linear_fwd(c, d, W, lo, LSL_M_QKV, n1, tp[LSL_M_QKV], tr, qkv, nullptr, part, cnt, s, true));
    LSL_TRY(fused_linear_fwd(c, d, W, lo, LSL_M_O, o, tp[LSL_M_O], tr, h1, x, part, cnt, s, true));
    LSL_TRY(fused_linear_fwd(c, d, W, lo, LSL_M_GU, n2, tp[LSL_M_GU], tr, gu, nullptr, part, cnt, s, true));
    return fused_linear_fwd(c, d, W, lo, LSL_M_DOWN, a, tp[LSL_M_DOWN], tr, out, h1, part, cnt, s, true);
  }
  // (also zeroes the arrival counts every later side product of the call uses)
  LSL_TRY(rmsnorm_fwd_launch(x, W.norm1, d.T, d.H, c->rms_eps, n1, s, cnt, (int)p.ncnt));
  // q and k heads are adjacent in each row and share the frequencies: one
  // launch; a split q|k|v projection's partials are summed by that launch
  const int sqkv = gemm_splits(d.T, d.NQKV, d.H);
  LSL_TRY(fused_linear_fwd(c, d, W, lo, LSL_M_QKV, n1, tp[LSL_M_QKV], tr, qkv, nullptr, part, cnt, s, false, sqkv > 1));
  uint16_t* qkr = (uint16_t*)(ws + p.qkr);
  if (sqkv > 1)
    LSL_TRY(rope_split_launch(part, sqkv, W.qkv_bias, qkv, qkr, d.T, d.NQKV, c->n_q + c->n_kv, d.d, seq, c->rope_theta,
                              &c->rope_scaling, s));
  else
    LSL_TRY(rope_launch(qkv, qkr, d.T, d.NQKV, c->n_q + c->n_kv, d.d, seq, c->rope_theta, &c->rope_scaling, 0, s));
  LSL_TRY(lsl_attention_fwd(qkr, qkr + d.Q, qkv + d.Q + d.KV, d.NQKV, d.NQKV, batch, seq, c->n_q, c->n_kv, d.d, o,
                            d.Q, (float*)(ws + p.lse), o32, s));
  // a split o projection's partials are summed (with the residual) by the
  // second RMSNorm, which writes h1 and n2
  const int so = gemm_splits(d.T, d.H, d.Q);
  LSL_TRY(fused_linear_fwd(c, d, W, lo, LSL_M_O, o, tp[LSL_M_O], tr, h1, x, part, cnt, s, false, so > 1));
  if (so > 1) LSL_TRY(rmsnorm_fwd_split_launch(part, so, nullptr, x, d.H, h1, W.norm2, d.T, d.H, c->rms_eps, n2, s));
  else LSL_TRY(rmsnorm_fwd_launch(h1, W.norm2, d.T, d.H, c->rms_eps, n2, s));
  LSL_TRY(fused_linear_fwd(c, d, W, lo, LSL_M_GU, n2, tp[LSL_M_GU], tr, gu, nullptr, part, cnt, s, false));
  LSL_TRY(swiglu_fwd_launch(gu, d.T, d.I, a, s));
  // out == nullptr (the backward's recompute): the layer output itself is not
  // needed, only the LoRA product t of the down projection (for its dB)
  return fused_linear_fwd(c, d, W, lo, LSL_M_DOWN, a, tp[LSL_M_DOWN], tr, out, h1, part, cnt, s, false);
}

// Byte offsets of the four projections' t (q|k|v, o, gate|up, down: [T x 3r],
// [T x r], [T x 2r], [T x r] bf16) inside a t_keep buffer; off[4] is its size.
static void tkeep_offsets(const Dims& d, size_t (&off)[5]) {
  const int nseg[4] = {3, 1, 2, 1};
  off[0] = 0;
  for (int i = 0; i < 4; ++i) off[i + 1] = off[i] + align256((size_t)d.T * nseg[i] * d.r * 2);
}

// the t pointers of a layer call: the caller's t_keep buffer, or the workspace
static void t_ptrs(const Dims& d, char* ws, const Plan& p, uint16_t* t_keep, uint16_t* (&tp)[4]) {
  if (t_keep) {
    size_t off[5];
    tkeep_offsets(d, off);
    for (int i = 0; i < 4; ++i) tp[i] = (uint16_t*)((char*)t_keep + off[i]);
  } else {
    tp[LSL_M_QKV] = (uint16_t*)(ws + p.tqkv);
    tp[LSL_M_O] = (uint16_t*)(ws + p.to);
    tp[LSL_M_GU] = (uint16_t*)(ws + p.tgu);
    tp[LSL_M_DOWN] = (uint16_t*)(ws + p.td);
  }
}

// Backward with recompute. dry: check every GEMM's and side product's
// conditions only. With dx == NULL (the first layer) the q|k|v input-gradient
// GEMM and the first RMSNorm's backward are skipped, as nothing reads dn1.
static lsl_status layer_backward(const lsl_layer_cfg* cfg, const LayerPtrs& W, const lsl_lora_set* lora,
                                 const uint16_t* x_in, const uint16_t* dy, int batch, int seq, uint16_t* dx,
                                 const lsl_lora_grads* grads, const uint16_t* t_keep, char* w, const Plan& p,
                                 hipStream_t s, bool dry) {
  Dims d = dims_of(cfg, batch, seq);
  // recompute the forward up to what the backward reads (every intermediate
  // except the layer output, whose down-projection GEMM is skipped; the LoRA
  // products t too unless the forward kept them)
  uint16_t* dn1 = (uint16_t*)(w + p.dn1);
  uint16_t* tp[4];
  t_ptrs(d, w, p, const_cast<uint16_t*>(t_keep), tp);
  LSL_TRY(layer_forward(cfg, W, lora, x_in, batch, seq, nullptr, w, p, tp, t_keep != nullptr, (float*)(w + p.o32), s,
                        dry));
  float* part = (float*)(w + p.part);
  unsigned* cnt = (unsigned*)(w + p.cnt);
  uint16_t* qkv = (uint16_t*)(w + p.qkv);
  uint16_t* qkr = (uint16_t*)(w + p.qkr);
  uint16_t* dqkr = (uint16_t*)(w + p.dqkr);
  uint16_t* dqkv = (uint16_t*)(w + p.dqkv);
  uint16_t* da = (uint16_t*)(w + p.da);
  uint16_t* dgu = (uint16_t*)(w + p.dgu);
  uint16_t* dn2 = (uint16_t*)(w + p.dn2);
  uint16_t* dh1 = (uint16_t*)(w + p.dh1);
  uint16_t* dob = (uint16_t*)(w + p.dob);
  const uint16_t* bt[4];
  for (int i = 0; i < 4; ++i) bt[i] = (const uint16_t*)(w + p.bt[i]);
  if (!dry) {
    // the four projections' masked B^T for u = dy B, in one launch
    LoraBt jobs[4];
    for (int i = 0; i < 4; ++i) {
      int64_t n, k;
      mat_shape(d, i, n, k);
      jobs[i].b_full = lora->B[i]; jobs[i].r = d.r; jobs[i].K = n; jobs[i].bt = (uint16_t*)(w + p.bt[i]);
      jobs[i].nseg = i == LSL_M_QKV ? 3 : (i == LSL_M_GU ? 2 : 1);
      jobs[i].kl = jobs[i].nseg * d.r;
      jobs[i].seg_end[0] = n;
      if (i == LSL_M_QKV) { jobs[i].seg_end[0] = d.Q; jobs[i].seg_end[1] = d.Q + d.KV; jobs[i].seg_end[2] = d.NQKV; }
      else if (i == LSL_M_GU) { jobs[i].seg_end[0] = d.I; jobs[i].seg_end[1] = 2 * d.I; }
    }
    LSL_TRY(lora_bt_group_launch(jobs, 4, s));
  }
  // the adapter gradients' descriptors, launched together at the end
  LoraTn tn[4][2];
  const TnPlan tnp = tn_plan(d);
  auto tws = [&](int j) { return (float*)((char*)part + tnp.ws_off[j]); };
  auto tcnt = [&](int j) { return cnt + tnp.cnt_off[j]; };
  auto tn_args = [&](int i, float* (&ws2)[2], unsigned* (&c2)[2]) {
    const int j = 2 * (3 - i);
    ws2[0] = tws(j); ws2[1] = tws(j + 1); c2[0] = tcnt(j); c2[1] = tcnt(j + 1);
  };
  float* twsp[4][2];
  unsigned* tcp[4][2];
  for (int i = 0; i < 4; ++i) tn_args(i, twsp[i], tcp[i]);
  // MLP
  LSL_TRY(fused_linear_bwd(cfg, d, W, lora, grads, LSL_M_DOWN, (uint16_t*)(w + p.a), tp[LSL_M_DOWN], dy,
                           (uint16_t*)(w + p.ud), da, part, cnt, bt[LSL_M_DOWN], tn[0], twsp[LSL_M_DOWN],
                           tcp[LSL_M_DOWN], s, dry));
  if (!dry) LSL_TRY(swiglu_bwd_launch((uint16_t*)(w + p.gu), da, d.T, d.I, dgu, s));
  // a split input-gradient GEMM's partials are summed by the RMSNorm backward
  // that follows it, which writes the GEMM's output (dn2, dn1) and its own
  const int sgu = gemm_splits(d.T, d.H, 2 * d.I), sqkv = gemm_splits(d.T, d.H, d.NQKV);
  LSL_TRY(fused_linear_bwd(cfg, d, W, lora, grads, LSL_M_GU, (uint16_t*)(w + p.n2), tp[LSL_M_GU], dgu,
                           (uint16_t*)(w + p.ugu), dn2, part, cnt, bt[LSL_M_GU], tn[1], twsp[LSL_M_GU], tcp[LSL_M_GU],
                           s, dry, sgu > 1));
  if (!dry && sgu > 1)
    LSL_TRY(rmsnorm_bwd_split_launch((uint16_t*)(w + p.h1), W.norm2, part, sgu, dy, d.T, d.H, cfg->rms_eps, dn2, dh1, s));
  else if (!dry)
    LSL_TRY(rmsnorm_bwd_launch((uint16_t*)(w + p.h1), W.norm2, dn2, dy, d.T, d.H, cfg->rms_eps, dh1, s));
  // attention block
  LSL_TRY(fused_linear_bwd(cfg, d, W, lora, grads, LSL_M_O, (uint16_t*)(w + p.o), tp[LSL_M_O], dh1,
                           (uint16_t*)(w + p.uo), dob, part, cnt, bt[LSL_M_O], tn[2], twsp[LSL_M_O], tcp[LSL_M_O], s,
                           dry));
  if (!dry) {
    LSL_TRY(lsl_attention_bwd(qkr, qkr + d.Q, qkv + d.Q + d.KV, (uint16_t*)(w + p.o), dob, (float*)(w + p.lse),
                              (const float*)(w + p.o32), d.NQKV, d.NQKV, d.Q, batch, seq, cfg->n_q, cfg->n_kv, d.d,
                              dqkr, dqkr + d.Q, dqkv + d.Q + d.KV, w + p.attn_ws, p.o32 - p.attn_ws, s));
    LSL_TRY(rope_launch(dqkr, dqkv, d.T, d.NQKV, cfg->n_q + cfg->n_kv, d.d, seq, cfg->rope_theta, &cfg->rope_scaling,
                        1, s));
  }
  LSL_TRY(fused_linear_bwd(cfg, d, W, lora, grads, LSL_M_QKV, (uint16_t*)(w + p.n1), tp[LSL_M_QKV], dqkv,
                           (uint16_t*)(w + p.uqkv), dx ? dn1 : nullptr, part, cnt, bt[LSL_M_QKV], tn[3],
                           twsp[LSL_M_QKV], tcp[LSL_M_QKV], s, dry, sqkv > 1));
  if (dx && !dry && sqkv > 1)
    LSL_TRY(rmsnorm_bwd_split_launch(x_in, W.norm1, part, sqkv, dh1, d.T, d.H, cfg->rms_eps, dn1, dx, s));
  else if (dx && !dry)
    LSL_TRY(rmsnorm_bwd_launch(x_in, W.norm1, dn1, dh1, d.T, d.H, cfg->rms_eps, dx, s));
  // dA and dB of all four projections in one launch: their inputs (the layer's
  // activations, the u and t products and the output gradients) all stay in
  // the workspace (or are the caller's dy) until the call ends
  if (!dry) LSL_TRY(lora_tn_group_launch(&tn[0][0], 8, s));
  return LSL_OK;
}

}  // namespace lsl

using namespace lsl;

extern "C" lsl_status lsl_layer_layout_get(const lsl_layer_cfg* cfg, lsl_layer_layout* out) {
  LSL_TRY(check_cfg(cfg, "lsl_layer_layout_get"));
  if (!out) return set_error(LSL_ERR_INVALID_ARG, "lsl_layer_layout_get: out is NULL");
  layout_of(cfg, out);
  return LSL_OK;
}

extern "C" size_t lsl_layer_workspace_bytes(const lsl_layer_cfg* cfg, int32_t batch, int32_t seq, int32_t mode) {
  if (check_cfg(cfg, "lsl_layer_workspace_bytes") != LSL_OK || batch < 0 || seq < 0) return 0;
  return plan_of(cfg, batch, seq, mode).total;
}

extern "C" lsl_status lsl_layer_workspace_map(const lsl_layer_cfg* cfg, int32_t batch, int32_t seq, int32_t mode,
                                              lsl_layer_ws_map* out) {
  const char* fn = "lsl_layer_workspace_map";
  LSL_TRY(check_cfg(cfg, fn));
  if (!out || batch < 0 || seq < 0 || (mode != LSL_MODE_FWD && mode != LSL_MODE_BWD))
    return set_error(LSL_ERR_INVALID_ARG, "%s: bad arguments", fn);
  const Plan p = plan_of(cfg, batch, seq, mode);
  *out = lsl_layer_ws_map{};
  out->n1 = p.n1; out->t_qkv = p.tqkv; out->qkv = p.qkv; out->qk_rope = p.qkr; out->attn = p.o; out->lse = p.lse;
  out->t_o = p.to; out->h1 = p.h1; out->n2 = p.n2; out->t_gu = p.tgu; out->gu = p.gu; out->act = p.a; out->t_down = p.td;
  if (mode == LSL_MODE_BWD) {
    out->u_down = p.ud; out->d_act = p.da; out->d_gu = p.dgu; out->u_gu = p.ugu; out->d_n2 = p.dn2; out->d_h1 = p.dh1;
    out->u_o = p.uo; out->d_attn = p.dob; out->d_qk_rope = p.dqkr; out->d_qkv = p.dqkv; out->u_qkv = p.uqkv;
    out->d_n1 = p.dn1; out->attn32 = p.o32;
  }
  return LSL_OK;
}

// lora may be NULL in the forward only (adapters off)
static lsl_status check_layer_call(const char* fn, const lsl_layer_cfg* cfg, const void* blob, const lsl_lora_set* lora,
                                   int32_t batch, int32_t seq, void* ws, size_t ws_bytes, int mode) {
  LSL_TRY(check_cfg(cfg, fn));
  if (batch < 0 || seq < 0) return set_error(LSL_ERR_INVALID_ARG, "%s: negative batch/seq", fn);
  if (!blob || !aligned(blob, 256)) return set_error(LSL_ERR_INVALID_ARG, "%s: layer blob NULL or not 256-byte aligned", fn);
  if (!lora && mode == LSL_MODE_BWD) return set_error(LSL_ERR_INVALID_ARG, "%s: lora set is NULL", fn);
  if (lora)
    for (int i = 0; i < 4; ++i) LSL_TRY(check_ptrs(fn, {lora->A[i], lora->B[i]}));
  size_t need = plan_of(cfg, batch, seq, mode).total;
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return set_error(LSL_ERR_WORKSPACE, "%s: workspace %zu < %zu (or not 256-byte aligned)", fn, ws_bytes, need);
  return LSL_OK;
}

extern "C" size_t lsl_layer_tkeep_bytes(const lsl_layer_cfg* cfg, int32_t batch, int32_t seq) {
  if (check_cfg(cfg, "lsl_layer_tkeep_bytes") != LSL_OK || batch < 0 || seq < 0) return 0;
  size_t off[5];
  tkeep_offsets(dims_of(cfg, batch, seq), off);
  return off[4];
}

extern "C" lsl_status decoder_layer_fwd(const lsl_layer_cfg* cfg, const void* layer_blob, const lsl_lora_set* lora,
                                        const uint16_t* x_in, int32_t batch, int32_t seq, uint16_t* x_out,
                                        uint16_t* t_keep, void* ws, size_t ws_bytes, lsl_stream stream) {
  const char* fn = "decoder_layer_fwd";
  LSL_TRY(check_layer_call(fn, cfg, layer_blob, lora, batch, seq, ws, ws_bytes, LSL_MODE_FWD));
  if (t_keep && !aligned(t_keep, 256)) return set_error(LSL_ERR_INVALID_ARG, "%s: t_keep not 256-byte aligned", fn);
  if ((int64_t)batch * seq == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {x_in, x_out}));
  Plan p = plan_of(cfg, batch, seq, LSL_MODE_FWD);
  const LayerPtrs W = ptrs_of(cfg, layer_blob);
  uint16_t* tp[4];
  t_ptrs(dims_of(cfg, batch, seq), (char*)ws, p, lora ? t_keep : nullptr, tp);
  const hipStream_t s = (hipStream_t)stream;
  LSL_TRY(layer_forward(cfg, W, lora, x_in, batch, seq, x_out, (char*)ws, p, tp, false, nullptr, s, true));
  return layer_forward(cfg, W, lora, x_in, batch, seq, x_out, (char*)ws, p, tp, false, nullptr, s);
}

extern "C" lsl_status decoder_layer_bwd(const lsl_layer_cfg* cfg, const void* layer_blob, const lsl_lora_set* lora,
                                        const uint16_t* x_in, const uint16_t* dy, int32_t batch, int32_t seq,
                                        uint16_t* dx, const lsl_lora_grads* grads, const uint16_t* t_keep, void* ws,
                                        size_t ws_bytes, lsl_stream stream) {
  const char* fn = "decoder_layer_bwd";
  LSL_TRY(check_layer_call(fn, cfg, layer_blob, lora, batch, seq, ws, ws_bytes, LSL_MODE_BWD));
  if (!grads) return set_error(LSL_ERR_INVALID_ARG, "%s: grads is NULL", fn);
  for (int i = 0; i < 4; ++i) LSL_TRY(check_ptrs(fn, {grads->dA[i], grads->dB[i]}));
  if (t_keep && !aligned(t_keep, 256)) return set_error(LSL_ERR_INVALID_ARG, "%s: t_keep not 256-byte aligned", fn);
  if ((int64_t)batch * seq == 0) return LSL_OK;
  LSL_TRY(check_ptrs(fn, {x_in, dy}));
  if (dx && !aligned(dx, 16)) return set_error(LSL_ERR_INVALID_ARG, "%s: dx misaligned", fn);
  const Plan p = plan_of(cfg, batch, seq, LSL_MODE_BWD);
  const LayerPtrs W = ptrs_of(cfg, layer_blob);
  const hipStream_t s = (hipStream_t)stream;
  // every launch's conditions first, so that a rejected call enqueues nothing
  LSL_TRY(layer_backward(cfg, W, lora, x_in, dy, batch, seq, dx, grads, t_keep, (char*)ws, p, s, true));
  return layer_backward(cfg, W, lora, x_in, dy, batch, seq, dx, grads, t_keep, (char*)ws, p, s, false);
}

static void timing_free() {
  for (auto e : g_timing.start) (void)hipEventDestroy(e);
  for (auto e : g_timing.stop) (void)hipEventDestroy(e);
  g_timing = Timing();
}

extern "C" lsl_status lsl_timing_enable(int32_t which, int32_t max_launches) {
  if (which < 1 || which > 8 || max_launches < 1 || max_launches > (1 << 20))
    return set_error(LSL_ERR_INVALID_ARG, "lsl_timing_enable: which in [1, 8], max_launches > 0");
  timing_free();
  g_timing.start.assign(max_launches, nullptr);
  g_timing.stop.assign(max_launches, nullptr);
  for (int i = 0; i < max_launches; ++i) {
    hipError_t e;
    if ((e = hipEventCreate(&g_timing.start[i])) != hipSuccess || (e = hipEventCreate(&g_timing.stop[i])) != hipSuccess) {
      timing_free();
      return set_error(LSL_ERR_HIP, "lsl_timing_enable: %s", hipGetErrorString(e));
    }
  }
  g_timing.which = which;
  return LSL_OK;
}

extern "C" lsl_status lsl_timing_read(double* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return set_error(LSL_ERR_INVALID_ARG, "lsl_timing_read: NULL argument");
  double t = 0.0;
  for (int i = 0; i < g_timing.count; ++i) {
    hipError_t e = hipEventSynchronize(g_timing.stop[i]);
    if (e != hipSuccess) return set_error(LSL_ERR_HIP, "lsl_timing_read: %s", hipGetErrorString(e));
    float ms = 0.f;
    if ((e = hipEventElapsedTime(&ms, g_timing.start[i], g_timing.stop[i])) != hipSuccess)
      return set_error(LSL_ERR_HIP, "lsl_timing_read: %s", hipGetErrorString(e));
    t += ms;
  }
  *total_ms = t;
  *launches = g_timing.count;
  g_timing.count = 0;
  return LSL_OK;
}

extern "C" lsl_status lsl_timing_disable(void) {
  timing_free();
  return LSL_OK;
}
