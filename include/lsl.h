/*
 * lsl.h - C ABI of the layer-streamed LoRA training library for AMD MI355X (gfx950).
 *
 * What the library computes: LoRA fine-tuning of a frozen decoder-only base whose
 * layers live in pinned host memory and are streamed, one layer per visit, into a
 * two-slot HBM pool, for the forward and the backward pass ("Exact Layer
 * Streaming: LoRA Fine-Tuning of an 8B Model on a 4 GB Laptop GPU", abstract;
 * "Soup CLI Lets You Fine-Tune an 8B LLM on a 4 GB Laptop GPU", section "How
 * Layer Streaming Works"; "Soup: Fine-Tuning an 8B LLM on a 4 GB Laptop GPU with
 * One YAML File", section "Layer Streaming: The Mechanism Behind the 4 GB Claim",
 * which describes a pinned host base store and two VRAM layer buffers).
 *
 * Conventions shared by every call:
 *  - Every call returns lsl_status. On any error nothing has been enqueued and
 *    lsl_last_error() returns a message (thread-local, valid until the next call
 *    on the same thread). No C++ exception crosses this boundary.
 *  - Compute calls are asynchronous on the caller's stream (a hipStream_t passed
 *    as lsl_stream; NULL is the null stream). They never synchronise the host and
 *    never allocate device memory: scratch space is a caller-provided workspace
 *    whose size the matching *_workspace_bytes call returns.
 *  - bfloat16 tensors are passed as uint16_t bit patterns, row-major, densely
 *    packed unless a leading dimension is given. Device pointers to bf16 data
 *    must be 16-byte aligned, float/int32 vectors (labels, lse, loss) 4-byte
 *    aligned (INVALID_ARG otherwise; there is no slower fallback path).
 *  - Kernel selection (tile shapes, splits, stream-K schedule, chunking) depends
 *    only on the shapes passed, never on pointer values, residency, the stream or
 *    the device, so a streamed and a resident run execute identical arithmetic
 *    and produce identical bits. No result is reduced with floating-point
 *    atomics: split partials are added in a fixed order, by a second kernel or
 *    by the workgroup that arrives last on a per-tile count (integer atomics).
 *  - The caller owns every buffer. The library keeps no device state beyond the
 *    allocation-free forward's scratch array; a pool object owns only its HIP
 *    events; the optional GEMM timing below is per calling thread.
 */
#ifndef LSL_H
#define LSL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lsl_status;
enum {
  LSL_OK = 0,
  LSL_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size */
  LSL_ERR_UNSUPPORTED = 2,  /* a shape this build does not support */
  LSL_ERR_NOT_PINNED = 3,   /* host pointer is not page-locked */
  LSL_ERR_WORKSPACE = 4,    /* workspace smaller than *_workspace_bytes */
  LSL_ERR_STATE = 5,        /* pool slot used out of order */
  LSL_ERR_HIP = 6           /* a HIP runtime call failed */
};

typedef void* lsl_stream; /* hipStream_t */

/* Message of the last error on this thread ("" when none). */
const char* lsl_last_error(void);
/* ABI version of this header (bumped on any incompatible change). */
int32_t lsl_abi_version(void);

typedef struct {
  int32_t cu_count;
  int32_t clock_khz;       /* peak shader clock */
  int32_t mem_clock_khz;
  int32_t mem_bus_bits;
  int64_t hbm_bytes;
  int32_t lds_bytes_per_cu;
  int32_t pad;
  char arch[64];           /* e.g. "gfx950:sramecc+:xnack-" */
} lsl_device_props;
/* Properties of `device`, for roofline arithmetic. */
lsl_status lsl_device_info(int32_t device, lsl_device_props* out);

/* ------------------------------------------------------------------ NF4
 * NF4 is the 4-bit NormalFloat format the pages quantise the 8B base to
 * ("Exact Layer Streaming ...", abstract). Definition (QLoRA, Dettmers et al.
 * 2023, section 3): 16 code values = standard-normal quantiles scaled to
 * [-1, 1] with an exact 0; blockwise absmax scaling over 64 consecutive
 * row-major elements, absmax stored as float32.
 * Packing: element 2j in the high nibble of byte j, element 2j+1 in the low one.
 */
/* The 16 float32 code values, ascending (host call, no GPU needed). */
lsl_status lsl_nf4_codebook(float out[16]);
/* Quantise w [rows x cols] bf16 (cols % 64 == 0) into codes [rows x cols/2] and
 * absmax [rows x cols/64]: n = w / absmax (IEEE float32 division; 0 when absmax
 * is 0), code = nearest code value, ties to the lower code. Device pointers. */
lsl_status lsl_nf4_quantize(const uint16_t* w, int64_t rows, int64_t cols,
                            uint8_t* codes, float* absmax, lsl_stream stream);
/* w' = bf16(code_value * absmax) (one float32 multiply, round to nearest even). */
lsl_status lsl_nf4_dequant(const uint8_t* codes, const float* absmax, int64_t rows,
                           int64_t cols, uint16_t* w, lsl_stream stream);

/* NF4 with 8-bit absmax codes: the storage behind the 3.60 GB store and 113 MB
 * layer buffers the pages report for Llama-3.1-8B ("Soup: ...", section "Layer
 * Streaming: The Mechanism Behind the 4 GB Claim"), which equal 4-bit codes +
 * one byte per 64 weights + one float32 per 256 absmax values. The pages fix
 * only those sizes; the 8-bit map is this library's reading, a linear one (not
 * QLoRA's 8-bit-float map of mean-centred constants, which has the same size).
 * The float32 absmax values, flattened row-major, are split into blocks of 256
 * (the last may be short); per block s = float32(max / 255),
 * q = round-half-even(absmax / s) (float32 division) clamped to [0, 255],
 * q = 0 when s = 0; absmax' = float32(q) * s. The 4-bit codes stay those of
 * lsl_nf4_quantize. */
/* absmax [n] float32 -> q [n] uint8, scale [ceil(n / 256)] float32. Device pointers. */
lsl_status lsl_nf4dq_quantize_absmax(const float* absmax, int64_t n, uint8_t* q, float* scale,
                                     lsl_stream stream);
/* w' = bf16(code_value * absmax') with absmax' = float32(q) * s of its block. */
lsl_status lsl_nf4dq_dequant(const uint8_t* codes, const uint8_t* q, const float* scale, int64_t rows,
                             int64_t cols, uint16_t* w, lsl_stream stream);

/* ------------------------------------------------------------------ weights */
enum { LSL_WFMT_NF4 = 0, LSL_WFMT_BF16 = 1, LSL_WFMT_NF4DQ = 2 };
/* A frozen weight [n_out x k_in] (n_out and k_in multiples of 64): NF4 (nf4
 * codes + absmax), bf16, or NF4 with 8-bit absmax codes (nf4 codes +
 * absmax_q + absmax_scale). Pointers not used by the format must be NULL.
 * bias (optional, NULL for none): a frozen bf16 vector [n_out] added to the
 * forward output before its rounding, as in the q/k/v projections of Qwen2
 * bases; it has no gradient and does not enter the backward. */
typedef struct {
  int32_t fmt;
  int32_t pad;
  int64_t n_out;
  int64_t k_in;
  const uint8_t* nf4;
  const float* absmax;
  const uint16_t* bf16;
  const uint8_t* absmax_q;
  const float* absmax_scale;
  const uint16_t* bias;
} lsl_weight;

/* ------------------------------------------------------------------ LoRA linear
 * y = x W^T + s (x A^T) B^T with frozen W and trainable A [r x k_in],
 * B [n_out x r] (LoRA, Hu et al. 2021; the pages train such adapters on the
 * frozen base: "Exact Layer Streaming ...", abstract).
 * Rounding: t = bf16(x A^T); y = bf16(x W^T + s t B^T (+ bias)) (float32
 * accumulation, one rounding). r is a multiple of 8 in [8, 64]; T >= 0 is any token count.
 */
size_t lsl_lora_linear_workspace_bytes(int64_t T, int64_t n_out, int64_t k_in, int32_t r);
/* Byte offset (a multiple of 256) in lora_linear_bwd's workspace where the call
 * leaves u = bf16(dy B) [T x r] (row-major), for callers that check or reuse it;
 * valid until the workspace is used again. */
size_t lsl_lora_linear_bwd_u_offset(int64_t T, int64_t n_out, int64_t k_in);
/* x [T x k_in], y [T x n_out], t_out [T x r] (kept for the backward). */
lsl_status lora_linear_fwd(const uint16_t* x, int64_t T, const lsl_weight* W,
                           const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                           uint16_t* y, uint16_t* t_out, void* ws, size_t ws_bytes,
                           lsl_stream stream);
/* The same forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument; its scratch (the side product's and the
 * GEMM's split partials and their arrival counts, lsl_lora_linear_workspace_bytes'
 * forward share) is a
 * device array of lsl_noalloc_scratch_bytes() bytes (88 MiB + 64 KiB) that the library
 * holds on each GPU it runs on until the process ends. It calls no allocating
 * routine. WORKSPACE if the shape needs more scratch than that. Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (two streams,
 * two threads) race and must be ordered by the caller. Results are bit for bit
 * those of lora_linear_fwd. */
lsl_status lora_linear_fwd_noalloc(const uint16_t* x, int64_t T, const lsl_weight* W,
                                   const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                                   uint16_t* y, uint16_t* t_out, lsl_stream stream);
size_t lsl_noalloc_scratch_bytes(void);
/* u = bf16(dy B); dx = bf16(dy W + s u A) (dx may be NULL);
 * dA += s u^T x and dB += s dy^T t (float32, accumulated into the caller's
 * buffers in a fixed order). W gets no gradient. */
lsl_status lora_linear_bwd(const uint16_t* x, const uint16_t* t, const uint16_t* dy, int64_t T,
                           const lsl_weight* W, const uint16_t* A, const uint16_t* B, int32_t r,
                           float scale, uint16_t* dx, float* dA, float* dB, void* ws,
                           size_t ws_bytes, lsl_stream stream);

/* ------------------------------------------------------------------ decoder layer
 * Pre-norm Llama/Qwen2 decoder layer: h = x + o(attn(rope(q(n1)), rope(k(n1)), v(n1))),
 * out = h + down(silu(gate(n2)) * up(n2)), n1 = rmsnorm(x), n2 = rmsnorm(h);
 * GQA causal attention (query head j reads kv head j / (n_q / n_kv)), scale
 * 1/sqrt(head_dim); rotate-half RoPE with angle pos * theta^(-2i/d) (frequencies
 * optionally rescaled, rope_scaling), positions restarting at 0 in each sequence;
 * optional frozen q/k/v bias; LoRA on all seven projections.
 * The pages stream exactly these "decoder layers" ("Soup CLI ...", section "How
 * Layer Streaming Works"). Supported: hidden and inter multiples of 64, hidden
 * at most 8192, head_dim 64 or 128, at most 8 query heads per kv head, LoRA
 * rank 8 or 16 (UNSUPPORTED otherwise).
 */
/* RoPE frequency scaling of Llama-3.1 checkpoints (their published rope_type
 * "llama3" configuration: 8, 1, 4, 8192). With f = theta^(-2i/d) and
 * wavelength 2 pi / f: f stays if the wavelength is below
 * original_max_position / high_freq_factor, becomes f / factor above
 * original_max_position / low_freq_factor, and in between
 * (1 - m) f / factor + m f with m = (original_max_position / wavelength -
 * low_freq_factor) / (high_freq_factor - low_freq_factor). factor == 0 means
 * no scaling; otherwise factor >= 1, 0 < low_freq_factor < high_freq_factor and
 * original_max_position > 0 are required. Computed in float64. */
typedef struct {
  float factor, low_freq_factor, high_freq_factor, original_max_position;
} lsl_rope_scaling;

typedef struct {
  int32_t hidden, n_q, n_kv, head_dim, inter;
  float rms_eps, rope_theta;
  int32_t wfmt;      /* LSL_WFMT_NF4, LSL_WFMT_BF16 or LSL_WFMT_NF4DQ */
  int32_t lora_r;
  float lora_scale;  /* alpha / r */
  int32_t qkv_bias;  /* 1: the blob holds a bf16 q|k|v bias [(n_q + 2 n_kv) d] (Qwen2 bases) */
  lsl_rope_scaling rope_scaling;  /* factor 0: none */
} lsl_layer_cfg;

/* Byte offsets inside one packed layer blob (every offset 256-byte aligned).
 * Matrices are stacked per fused GEMM: qkv = [Wq; Wk; Wv] [(n_q+2 n_kv) d x hidden],
 * o [hidden x n_q d], gu = [Wgate; Wup] [2 inter x hidden], down [hidden x inter].
 * For NF4 each matrix is codes at w_off[i] and float32 absmax at absmax_off[i];
 * for NF4DQ codes at w_off[i], uint8 absmax codes at absmax_off[i] and float32
 * block constants at scale_off[i]; for bf16 the matrix is at w_off[i] and
 * absmax_off[i] (and scale_off[i]) are 0. With qkv_bias the bf16 bias of the
 * stacked q|k|v rows is at bias_off (else bias_off is 0).
 * norm1/norm2 are bf16 [hidden]. The pinned host store and a resident copy use
 * this same layout, so a slot holds a byte-identical copy of one layer. */
enum { LSL_M_QKV = 0, LSL_M_O = 1, LSL_M_GU = 2, LSL_M_DOWN = 3 };
typedef struct {
  uint64_t norm1_off, norm2_off;
  uint64_t w_off[4];
  uint64_t absmax_off[4];
  uint64_t total_bytes;
  uint64_t scale_off[4];
  uint64_t bias_off;
} lsl_layer_layout;
lsl_status lsl_layer_layout_get(const lsl_layer_cfg* cfg, lsl_layer_layout* out);

/* Trainable adapters of one layer, grouped like the fused GEMMs:
 *   A[QKV] = [A_q; A_k; A_v]   [3r x hidden]    B[QKV] = [B_q; B_k; B_v] [(n_q+2n_kv)d x r]
 *   A[O]                       [r x n_q d]      B[O]                     [hidden x r]
 *   A[GU]  = [A_gate; A_up]    [2r x hidden]    B[GU]  = [B_gate; B_up]  [2 inter x r]
 *   A[DOWN]                    [r x inter]      B[DOWN]                  [hidden x r]
 * bf16 working copies; gradients have the same shapes in float32. */
typedef struct { const uint16_t* A[4]; const uint16_t* B[4]; } lsl_lora_set;
typedef struct { float* dA[4]; float* dB[4]; } lsl_lora_grads;

enum { LSL_MODE_FWD = 0, LSL_MODE_BWD = 1 };
size_t lsl_layer_workspace_bytes(const lsl_layer_cfg* cfg, int32_t batch, int32_t seq, int32_t mode);
/* Where decoder_layer_fwd / decoder_layer_bwd keep each intermediate inside
 * their workspace (byte offsets from ws; T = batch * seq, r = lora_r,
 * d = head_dim, NQKV = (n_q + 2 n_kv) d), so that every rounding point of the
 * layer can be read back and checked on its own. After decoder_layer_fwd the
 * forward entries hold that call's values; after decoder_layer_bwd the forward
 * entries hold the recomputed forward (the down projection's output is not
 * recomputed) and the backward entries the backward's values. They stay valid
 * until the workspace is used again. Backward entries are 0 in mode
 * LSL_MODE_FWD; with the adapters off, or with a t_keep buffer (which then
 * holds them), the t_* entries are not written. */
typedef struct {
  /* forward */
  uint64_t n1;        /* bf16 [T x hidden]  rmsnorm(x_in, norm1) */
  uint64_t t_qkv;     /* bf16 [T x 3r]      n1 [A_q; A_k; A_v]^T */
  uint64_t qkv;       /* bf16 [T x NQKV]    q|k|v projections (before RoPE) */
  uint64_t qk_rope;   /* bf16, row stride NQKV: the RoPE'd q and k columns (v columns unused) */
  uint64_t attn;      /* bf16 [T x n_q d]   attention output */
  uint64_t lse;       /* float [batch x n_q x seq] attention log-sum-exp */
  uint64_t t_o;       /* bf16 [T x r]       attn A_o^T */
  uint64_t h1;        /* bf16 [T x hidden]  x_in + o projection */
  uint64_t n2;        /* bf16 [T x hidden]  rmsnorm(h1, norm2) */
  uint64_t t_gu;      /* bf16 [T x 2r]      n2 [A_gate; A_up]^T */
  uint64_t gu;        /* bf16 [T x 2 inter] gate | up projections */
  uint64_t act;       /* bf16 [T x inter]   silu(gate) * up */
  uint64_t t_down;    /* bf16 [T x r]       act A_down^T */
  /* backward */
  uint64_t u_down;    /* bf16 [T x r]       dy B_down */
  uint64_t d_act;     /* bf16 [T x inter]   gradient of act */
  uint64_t d_gu;      /* bf16 [T x 2 inter] gradients of gate | up */
  uint64_t u_gu;      /* bf16 [T x 2r]      d_gate B_gate | d_up B_up */
  uint64_t d_n2;      /* bf16 [T x hidden] */
  uint64_t d_h1;      /* bf16 [T x hidden] */
  uint64_t u_o;       /* bf16 [T x r]       d_h1 B_o */
  uint64_t d_attn;    /* bf16 [T x n_q d]   gradient of the attention output */
  uint64_t d_qk_rope; /* bf16, row stride NQKV: gradients of the RoPE'd q and k columns */
  uint64_t d_qkv;     /* bf16 [T x NQKV]    dq, dk (inverse RoPE applied) and dv */
  uint64_t u_qkv;     /* bf16 [T x 3r]      per projection d_p B_p */
  uint64_t d_n1;      /* bf16 [T x hidden]  (written only when dx is not NULL) */
  uint64_t attn32;    /* float [T x n_q d]  attention output before its rounding */
} lsl_layer_ws_map;
lsl_status lsl_layer_workspace_map(const lsl_layer_cfg* cfg, int32_t batch, int32_t seq, int32_t mode,
                                   lsl_layer_ws_map* out);
/* Bytes of a t_keep buffer: the four projections' LoRA products t = x A^T
 * (q|k|v [T x 3r], o [T x r], gate|up [T x 2r], down [T x r], bf16, each
 * region 256-byte aligned, in that order), 0 for an invalid cfg. */
size_t lsl_layer_tkeep_bytes(const lsl_layer_cfg* cfg, int32_t batch, int32_t seq);
/* x_in, x_out [batch*seq x hidden] bf16. The caller keeps x_in as the
 * layer-boundary checkpoint for the backward ("Exact Layer Streaming ...",
 * abstract: the layer is recomputed in the backward). lora may be NULL: the
 * adapters are off and every projection is the frozen base alone (the
 * reference forward of preference training). t_keep may be NULL; otherwise
 * (256-byte aligned, lsl_layer_tkeep_bytes bytes, ignored when lora is NULL)
 * the forward leaves the rank-r products t = x A^T of the four projections
 * there instead of in the workspace, for decoder_layer_bwd of the same input. */
lsl_status decoder_layer_fwd(const lsl_layer_cfg* cfg, const void* layer_blob,
                             const lsl_lora_set* lora, const uint16_t* x_in, int32_t batch,
                             int32_t seq, uint16_t* x_out, uint16_t* t_keep, void* ws,
                             size_t ws_bytes, lsl_stream stream);
/* Recomputes the forward from x_in, then back-propagates dy. dx may be NULL
 * (first layer); adapter gradients are accumulated (+=) into grads. With
 * t_keep (as filled by decoder_layer_fwd for this x_in, lora, cfg, batch and
 * seq) the recompute takes the products t from there instead of computing
 * them again; the caller guarantees they are that forward's. The results are
 * the same bits either way (t is computed by the same launches from the same
 * bits); only the t_* workspace entries stay unwritten. */
lsl_status decoder_layer_bwd(const lsl_layer_cfg* cfg, const void* layer_blob,
                             const lsl_lora_set* lora, const uint16_t* x_in, const uint16_t* dy,
                             int32_t batch, int32_t seq, uint16_t* dx,
                             const lsl_lora_grads* grads, const uint16_t* t_keep, void* ws,
                             size_t ws_bytes, lsl_stream stream);

/* ------------------------------------------------------------------ layer pool
 * Two (or more) HBM slots, each holding one layer blob, filled from the pinned
 * host store by hipMemcpyAsync on a copy stream and ordered against compute by
 * events ("Soup: ...", section "Layer Streaming: The Mechanism Behind the 4 GB
 * Claim": a pinned base store and two VRAM buffers).
 * Slot life cycle: load_layer_async -> lsl_pool_acquire -> lsl_pool_release ->
 * load_layer_async ... . A load waits (on the copy stream) until the slot's
 * previous user released it; acquire makes the compute stream wait for the load.
 * The caller owns the slot memory and the copy stream. The copy stream must be
 * a non-blocking stream (hipStreamNonBlocking) that does not share a hardware
 * queue with the compute stream: HIP maps streams onto a few hardware queues
 * (GPU_MAX_HW_QUEUES, 4 by default) and two streams on one queue run one after
 * the other, which silently removes the overlap. Keeping one copy stream per
 * process, and few streams in all, avoids that.
 * Debugging aid: with the environment variable LSL_POISON_SLOTS set to a
 * non-zero value when the pool is created, every load first fills the whole
 * slot with 0xFF bytes on the copy stream (after the wait for the slot's
 * release), so a read outside the load/acquire/release window, or past the
 * layer's bytes, yields NaN weights instead of a silently stale layer (the
 * pages warn that streaming failures are silent: "Exact Layer Streaming ...",
 * abstract). Results are unchanged when the slots are used in order. */
typedef struct lsl_pool lsl_pool;
lsl_status lsl_pool_create(lsl_pool** out, void* const* slot_ptrs, int32_t n_slots,
                           size_t slot_bytes, lsl_stream copy_stream);
lsl_status lsl_pool_destroy(lsl_pool* pool);
/* Enqueue host->slot copy of `bytes` (<= slot_bytes) from page-locked host_ptr.
 * NOT_PINNED if host_ptr is pageable; STATE if the slot is loaded or acquired. */
lsl_status load_layer_async(lsl_pool* pool, int32_t slot, const void* host_ptr, size_t bytes);
/* Make `compute` wait for the slot's load; returns the slot's device pointer.
 * STATE unless the slot has been loaded and not yet acquired. */
lsl_status lsl_pool_acquire(lsl_pool* pool, int32_t slot, lsl_stream compute, void** slot_ptr);
/* Record on `compute` that the slot's contents are no longer needed.
 * STATE unless the slot is acquired. */
lsl_status lsl_pool_release(lsl_pool* pool, int32_t slot, lsl_stream compute);
/* Mark a released slot as still holding `host_ptr`'s layer, so it can be
 * acquired again without a copy (the layers kept across the turn of a sweep). */
lsl_status lsl_pool_reuse(lsl_pool* pool, int32_t slot);
/* Copy statistics: after enable, each of the next max_loads loads records a
 * start/end event pair on the copy stream; read waits for them and returns the
 * number of loads, bytes and summed copy seconds, then clears the record. */
lsl_status lsl_pool_stats_enable(lsl_pool* pool, int32_t max_loads);
lsl_status lsl_pool_stats_read(lsl_pool* pool, int32_t* loads, double* bytes, double* seconds);

/* ------------------------------------------------------------------ timing
 * Optional measurement of one GEMM of the decoder layer for roofline reports:
 * while enabled, decoder_layer_fwd/bwd record HIP events on their stream
 * around each launch of the selected GEMM (at most max_launches). The switch
 * and its events belong to the calling thread (layer calls made on other
 * threads neither see nor touch them); it is off by default.
 * which: 1..4 forward GEMM of group LSL_M_QKV..LSL_M_DOWN (+1),
 *        5..8 input-gradient GEMM of the same groups. */
lsl_status lsl_timing_enable(int32_t which, int32_t max_launches);
/* Waits for the recorded events; total milliseconds and launch count. */
lsl_status lsl_timing_read(double* total_ms, int32_t* launches);
lsl_status lsl_timing_disable(void);

/* ------------------------------------------------------------------ cross-entropy
 * Token cross-entropy over the vocabulary, fused with the lm_head product and
 * chunked over the vocabulary so no [T x V] logits tensor is ever stored (the
 * pages measure that tensor's cost: "Exact Layer Streaming ...", abstract).
 * z = hN W^T (float32, never rounded); lse_t = log sum_v exp(z_tv);
 * loss = mean over labels != ignore_index of (lse_t - z_t,label).
 * hN [T x H] bf16, w_lm [V x H] bf16, labels int32 [T].
 */
size_t lsl_ce_workspace_bytes(int64_t T, int64_t H, int64_t V);
/* loss: one float (device); lse: float [T] (device). */
lsl_status fused_ce_loss_fwd(const uint16_t* hN, const uint16_t* w_lm, const int32_t* labels,
                             int64_t T, int64_t H, int64_t V, int32_t ignore_index, float* loss,
                             float* lse, void* ws, size_t ws_bytes, lsl_stream stream);
/* dhN = bf16(grad_scale / N_valid * (softmax(z) - onehot(label)) W), zero rows for
 * ignored tokens; lse from fused_ce_loss_fwd. */
lsl_status fused_ce_loss_bwd(const uint16_t* hN, const uint16_t* w_lm, const int32_t* labels,
                             const float* lse, int64_t T, int64_t H, int64_t V,
                             int32_t ignore_index, float grad_scale, uint16_t* dhN, void* ws,
                             size_t ws_bytes, lsl_stream stream);
/* Per-token log-probabilities of the labels with the fused forward pass (no
 * logits tensor): logp[t] = z_t,label - lse_t (float32, 0 where the label is
 * ignore_index or outside the vocabulary), and, when seq_logp is not NULL,
 * seq_logp[b] = sum of logp over the T / batch tokens of sequence b (fixed
 * order). This is the reference score of preference training, computed on the
 * final hidden state of the adapter-off forward (decoder_layer_fwd with lora
 * NULL) of the same streamed base ("Soup: ...", section "Layer Streaming: The
 * Mechanism Behind the 4 GB Claim"; "Soup CLI ...", "Key Takeaways").
 * Workspace: lsl_ce_workspace_bytes(T, H, V). */
lsl_status fused_ce_logprobs(const uint16_t* hN, const uint16_t* w_lm, const int32_t* labels, int64_t T,
                             int64_t H, int64_t V, int32_t ignore_index, int32_t batch, float* logp,
                             float* seq_logp, void* ws, size_t ws_bytes, lsl_stream stream);

/* ------------------------------------------------------------------ support ops
 * The individual steps of the decoder layer, exported so each can be checked on
 * its own (same kernels the layer calls). */
/* y = bf16(x / sqrt(mean(x^2) + eps) * w), x, y [T x H], H a multiple of 8, at most 8192. */
lsl_status lsl_rmsnorm_fwd(const uint16_t* x, const uint16_t* w, int64_t T, int64_t H, float eps,
                           uint16_t* y, lsl_stream stream);
/* dx = bf16(dres + r (w dy - xh mean(xh w dy))), xh = x r; dres may be NULL. */
lsl_status lsl_rmsnorm_bwd(const uint16_t* x, const uint16_t* w, const uint16_t* dy,
                           const uint16_t* dres, int64_t T, int64_t H, float eps, uint16_t* dx,
                           lsl_stream stream);
/* In-place rotate-half RoPE on x [T rows, row stride ld elements], heads
 * [n_heads x head_dim] starting at column 0 of each row; position = row % seq.
 * inverse != 0 rotates by -angle (the backward). scaling may be NULL (none).
 * head_dim a multiple of 8, at most 128; ld a multiple of 4. */
lsl_status lsl_rope(uint16_t* x, int64_t T, int64_t ld, int32_t n_heads, int32_t head_dim,
                    int32_t seq, float theta, const lsl_rope_scaling* scaling, int32_t inverse,
                    lsl_stream stream);
/* Causal GQA attention. q [T x ldq] (n_q heads of d), k, v [T x ldk] (n_kv heads),
 * o [T x ldo]; lse float [batch x n_q x seq]. T = batch * seq. head_dim 64 or 128,
 * at most 8 query heads per kv head. o32 (may be NULL) receives the unrounded
 * output as float [T x n_q d], which the backward uses for rowsum(dout * o). */
lsl_status lsl_attention_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             int64_t ldq, int64_t ldk, int32_t batch, int32_t seq, int32_t n_q,
                             int32_t n_kv, int32_t head_dim, uint16_t* o, int64_t ldo, float* lse,
                             float* o32, lsl_stream stream);
size_t lsl_attention_workspace_bytes(int32_t batch, int32_t seq, int32_t n_q, int32_t n_kv,
                                     int32_t head_dim);
/* Gradients of sum(dout * o): o, dout [T x ldo]; dq [T x ldq] like q; dk, dv
 * [T x ldk] like k (dk, dv summed over the heads of each group). o32 (may be
 * NULL) is the forward's float output; without it rowsum(dout * o) uses o.
 * ws: lsl_attention_workspace_bytes() bytes of device scratch (any contents; the
 * call initialises what it needs): the row sums and, when the key tiles are few,
 * the float32 partials of key tiles whose dK/dV work is split over workgroups
 * (added in a fixed order, so the result does not depend on timing). */
lsl_status lsl_attention_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const uint16_t* o, const uint16_t* dout, const float* lse,
                             const float* o32, int64_t ldq, int64_t ldk, int64_t ldo, int32_t batch,
                             int32_t seq, int32_t n_q,
                             int32_t n_kv, int32_t head_dim, uint16_t* dq, uint16_t* dk,
                             uint16_t* dv, void* ws, size_t ws_bytes, lsl_stream stream);
/* gu [T x 2I] = [gate | up]; a = bf16(silu(gate) * up) [T x I]. */
lsl_status lsl_swiglu_fwd(const uint16_t* gu, int64_t T, int64_t I, uint16_t* a, lsl_stream stream);
/* dgu [T x 2I] = [bf16(da up s(g)(1 + g(1 - s(g)))) | bf16(da silu(g))]. */
lsl_status lsl_swiglu_bwd(const uint16_t* gu, const uint16_t* da, int64_t T, int64_t I,
                          uint16_t* dgu, lsl_stream stream);
/* out[t] = table[ids[t]] (frozen, resident embedding; ids outside [0, V) give zeros). */
lsl_status lsl_embed_fwd(const uint16_t* table, const int32_t* ids, int64_t T, int64_t H,
                         int64_t V, uint16_t* out, lsl_stream stream);
/* AdamW (decoupled decay) on n float32 master parameters; refreshes the bf16
 * working copy p_bf16 (may be NULL). step counts from 1. */
lsl_status lsl_adamw_step(float* p, uint16_t* p_bf16, const float* g, float* m, float* v,
                          int64_t n, int32_t step, float lr, float beta1, float beta2, float eps,
                          float weight_decay, lsl_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* LSL_H */
