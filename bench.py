"""Benchmark: layer-streamed LoRA training steps on one MI355X.

Workload: Llama-3.1-8B-shaped decoder (32 layers, hidden 4096, 32/8 heads of
128, SwiGLU 14336, vocab 128256, separate bf16 lm_head), frozen NF4 base
(block 64, float32 absmax) streamed layer by layer from a pinned host store
into 2 HBM slots, LoRA r=16 alpha=32 on all seven projections, batch 1 x seq
1024 uniform random tokens, fused chunked cross-entropy, full forward +
backward (recompute) + AdamW on the adapters. Synthetic random weights of that
architecture (no checkpoint): N(0, 0.02) base and embeddings.

Prints one JSON line. Other output goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA train tok/s (streamed fwd+bwd) + % bf16 MFMA peak + achieved H2D GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
# the timed kernel's instantiation: NF4 weight, [N x K] layout, forward LoRA step, bf16 epilogue
GU_LABEL = "gemm_big_kernel<NF4, NK, LoRA-fwd> gate|up"
COUNTERS = os.path.join(ROOT, "profiles", "gemm_gu_fwd_nf4_llama8b_s1024_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload(name):
    from synth.configs import WORKLOADS
    w = WORKLOADS[name]
    m = w.model
    return w, m.layer, m


def build_model(shape, ms, mode, seed=1234):
    import torch
    from synth.configs import PROJ_IN_OUT
    from layer_streamed_lora_amd.trainer import StreamedLoraModel
    m = StreamedLoraModel(shape, ms.n_layers, ms.vocab, ms.tied, ms.batch, ms.seq, mode=mode)
    g = torch.Generator(device="cuda").manual_seed(seed)
    for l in range(ms.n_layers):
        w = {p: (torch.randn((fout, fin), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
             for p, (fin, fout) in PROJ_IN_OUT(shape).items()}
        w["norm1"] = torch.ones(shape.hidden, dtype=torch.bfloat16, device="cuda")
        w["norm2"] = torch.ones(shape.hidden, dtype=torch.bfloat16, device="cuda")
        m.set_layer_weights(l, w)
        del w
    m.embed.copy_((torch.randn(m.embed.shape, generator=g, device="cuda") * 0.02).to(torch.bfloat16))
    if m.lm_head is not None:
        m.lm_head.copy_((torch.randn(m.lm_head.shape, generator=g, device="cuda") * 0.02).to(torch.bfloat16))
    lp = m.lora
    for l in range(ms.n_layers):
        for i in range(4):
            A = lp.view(lp.master, l, i, "A")
            A.copy_((torch.rand(A.shape, generator=g, device="cuda") * 2 - 1) / A.shape[1] ** 0.5)
            B = lp.view(lp.master, l, i, "B")
            B.copy_(torch.randn(B.shape, generator=g, device="cuda") * 0.01)
    lp.bf16.copy_(lp.master.to(torch.bfloat16))
    torch.cuda.synchronize()
    return m


def step_flops(shape, ms):
    """Algorithmic FLOPs of one optimizer step (per microbatch x n_micro):
    forward GEMMs, their recompute, input-gradient GEMMs, LoRA side products,
    attention (causal: half the dense score/value work), cross-entropy 3 passes."""
    T, H, I, r = ms.batch * ms.seq, shape.hidden, shape.inter, shape.lora_r
    q, kv, d = shape.n_q * shape.head_dim, shape.n_kv * shape.head_dim, shape.head_dim
    mats = [(q + 2 * kv, H, 3), (H, q, 1), (2 * I, H, 2), (H, I, 1)]   # (N, K, projections)
    base = sum(2 * T * n * k for n, k, _ in mats)
    lora = sum(2 * T * r * p * (k + n) for n, k, p in mats)        # t = xA^T and t B^T
    lora_bwd = sum(2 * T * r * p * (n + k) * 2 for n, k, p in mats)  # u, dx-term, dA, dB
    attn_fwd = 2 * 2 * ms.batch * shape.n_q * ms.seq * ms.seq * d / 2
    per_layer = 2 * (base + lora + attn_fwd) + (base + lora_bwd + 2.5 * attn_fwd)
    ce = 3 * 2 * T * H * ms.vocab
    return ms.n_micro * (ms.n_layers * per_layer + ce)


def pinned_h2d_peak(nbytes, stream, reps=20):
    """hipMemcpyAsync rate of a pinned buffer of nbytes on the given stream. The
    layer pool's own copy stream is passed: HIP maps streams onto a few hardware
    queues (4 by default), and streams that share one run one after the other,
    so every extra stream risks putting the copies behind the compute."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = stream
    with torch.cuda.stream(s):
        for _ in range(3):
            dst.copy_(src, non_blocking=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            dst.copy_(src, non_blocking=True)
        e1.record(s)
    e1.synchronize()
    return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def time_reference(m, inputs, steps, warmup):
    """The adapter-off streamed forward with per-token log-probabilities (the
    reference scores of preference training): ms per call over all microbatches."""
    import torch
    for _ in range(warmup):
        m.reference_logprobs(inputs)
    torch.cuda.synchronize()
    loads0 = m.loads
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        lp, _ = m.reference_logprobs(inputs)
    e1.record(stream)
    torch.cuda.synchronize()
    return {"ms": e0.elapsed_time(e1) / steps, "loads": (m.loads - loads0) // steps,
            "mean_logp": float(lp[:, :-1].mean().item())}


def time_steps(m, inputs, steps, warmup, timing_which=0, stats=False):
    import ctypes as C
    import torch
    from layer_streamed_lora_amd.ops import lib, _check
    for _ in range(warmup):
        m.step(inputs)
    torch.cuda.synchronize()
    if timing_which:
        n_launch = steps * m.n_layers * inputs[0].shape[0] * 2
        _check("lsl_timing_enable", lib().lsl_timing_enable(timing_which, n_launch))
    if stats and m.pool is not None:
        _check("lsl_pool_stats_enable", lib().lsl_pool_stats_enable(m.pool.handle, steps * 4 * m.n_layers * 8))
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        losses = m.step(inputs)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    out = {"ms_per_step": ms, "wall_s": wall, "loss": float(losses.mean().item())}
    if timing_which:
        tot, n = C.c_double(), C.c_int32()
        _check("lsl_timing_read", lib().lsl_timing_read(C.byref(tot), C.byref(n)))
        lib().lsl_timing_disable()
        out["kernel_ms_total"], out["kernel_launches"] = tot.value, n.value
    if stats and m.pool is not None:
        loads, b, s = C.c_int32(), C.c_double(), C.c_double()
        _check("lsl_pool_stats_read", lib().lsl_pool_stats_read(m.pool.handle, C.byref(loads), C.byref(b), C.byref(s)))
        lib().lsl_pool_stats_enable(m.pool.handle, 0)
        out["h2d_loads"], out["h2d_bytes"], out["h2d_copy_s"] = loads.value, b.value, s.value
    return out


def gemm_groups(m, inputs, shape, ms, steps=2):
    """Average duration and achieved TF/s of each of the layer's eight fused
    GEMMs (forward and input gradient of q|k|v, o, gate|up, down), LoRA K-step
    included, timed with HIP events around each launch over `steps` steps."""
    T, H, I, r = ms.batch * ms.seq, shape.hidden, shape.inter, shape.lora_r
    q, kv = shape.n_q * shape.head_dim, shape.n_kv * shape.head_dim
    mats = {"qkv": (q + 2 * kv, H, 3), "o": (H, q, 1), "gate|up": (2 * I, H, 2), "down": (H, I, 1)}
    out = {}
    for which in range(1, 9):
        name = list(mats)[(which - 1) % 4]
        n, k, nseg = mats[name]
        if which <= 4:   # y = x W^T + s t B^T: M = T, N = n, K = k (+ kl)
            flops = 2.0 * T * n * k + 2.0 * T * nseg * r * n
            label = f"fwd {name} {T}x{n}x{k}"
        else:            # dx = dy W + s u A: M = T, N = k, K = n (+ kl)
            flops = 2.0 * T * n * k + 2.0 * T * nseg * r * k
            label = f"dX {name} {T}x{k}x{n}"
        res = time_steps(m, inputs, steps, 0, timing_which=which)
        avg = res["kernel_ms_total"] / max(res["kernel_launches"], 1)
        tf = flops / (avg * 1e-3) / 1e12
        out[label] = {"avg_launch_ms": round(avg, 4), "TFLOP_s": round(tf, 1),
                      "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    return out


def t_sweep(args, sizes=(1024, 2048, 4096, 8192, 16384), emit=True):
    """Streamed and resident step time of the workload's model at growing token
    counts per layer visit (batch x 1024 tokens, one microbatch): where the
    layer copies start to hide behind compute."""
    import dataclasses
    import torch
    import synth
    from layer_streamed_lora_amd.trainer import StreamedLoraModel
    wl, shape, ms0 = workload(args.workload)
    rows = []
    for T in sizes:
        ms = dataclasses.replace(ms0, batch=T // 1024, seq=1024, n_micro=1)
        s_model = build_model(shape, ms, "streamed")
        r_model = StreamedLoraModel(shape, ms.n_layers, ms.vocab, ms.tied, ms.batch, ms.seq, mode="resident")
        r_model.copy_base_from(s_model)
        chunks = [synth.token_ids(T, ms.vocab, wl.wid, salt=0)]
        inputs = s_model.prepare_inputs(chunks)
        st = time_steps(s_model, inputs, args.steps, args.warmup)["ms_per_step"]
        rt = time_steps(r_model, inputs, args.steps, args.warmup)["ms_per_step"]
        rows.append({"tokens": T, "streamed_ms": round(st, 2), "resident_ms": round(rt, 2),
                     "streamed_over_resident": round(st / rt, 3), "streamed_tok_s": round(T / (st * 1e-3), 1)})
        log(f"  T {T}: streamed {st:.1f} ms, resident {rt:.1f} ms, ratio {st / rt:.2f}")
        del s_model, r_model, inputs
        torch.cuda.empty_cache()
    if emit:
        print(json.dumps({"t_sweep": rows, "workload": args.workload, "steps": args.steps, "warmup": args.warmup}),
              flush=True)
    return rows


def nf4dq_leg(args, T_inputs_seed):
    """The same model with double-quantized absmax (8-bit absmax codes, one
    float32 per 256): streamed step time, gate|up GEMM time and bytes moved."""
    import torch
    import synth
    wl, shape, ms = workload("llama8b_nf4dq")
    T = ms.batch * ms.seq
    log(f"building llama8b_nf4dq: {ms.n_layers} layers, {shape.wfmt} base")
    m = build_model(shape, ms, "streamed")
    chunks = [synth.token_ids(T, ms.vocab, T_inputs_seed, salt=i) for i in range(ms.n_micro)]
    inputs = m.prepare_inputs(chunks)
    res = time_steps(m, inputs, args.steps, args.warmup, timing_which=3)
    cs = time_steps(m, inputs, 1, 0, stats=True)
    g_ms = res["kernel_ms_total"] / max(res["kernel_launches"], 1)
    log(f"  nf4dq streamed: {res['ms_per_step']:.2f} ms/step, gate|up GEMM {g_ms * 1e3:.1f} us")
    out = {"workload": "llama8b_nf4dq: the same model, NF4 with double-quantized absmax",
           "ms_per_step": round(res["ms_per_step"], 3),
           "tok_s": round(T * ms.n_micro / (res["ms_per_step"] * 1e-3), 2),
           "blob_bytes": m.blob_bytes, "store_GB": round(m.blob_bytes * ms.n_layers / 1e9, 3),
           "h2d_bytes_per_step": cs.get("h2d_bytes"),
           "h2d_GBps_copy_engine": cs.get("h2d_copy_s") and round(cs["h2d_bytes"] / cs["h2d_copy_s"] / 1e9, 2),
           "gu_gemm_avg_launch_ms": round(g_ms, 4), "loss": round(res["loss"], 5)}
    del m, inputs
    torch.cuda.synchronize()
    return out


# the pages' own figures for these workloads' shapes ("Exact Layer Streaming ...",
# abstract): context only, other hardware and unstated sequence lengths
LEG_CONTEXT = {
    "qwen05b_bf16": {"pages_streamed_over_resident": 1.43,
                     "pages_note": "0.5B model, the one size with a resident baseline on the pages' 4 GB laptop GPU"},
    "qwen3b_bf16": {"pages_tok_s": 143.0,
                    "pages_note": "Qwen2.5-3B, un-quantized bf16 base, layer-streamed, RTX 3050 Laptop 4 GB (2.15 GB peak)"},
}


def model_leg(name, args):
    """One workload model streamed (2 slots) and resident with the same base:
    bit-exactness of one optimizer step, then `steps` timed steps of each (after
    one warm-up), and the layer copies of one step (copy-engine time)."""
    import torch
    import synth
    from layer_streamed_lora_amd.trainer import StreamedLoraModel
    wl, shape, ms = workload(name)
    T = ms.batch * ms.seq
    log(f"building {name}: {ms.n_layers} layers, {shape.wfmt} base, {ms.n_micro} x {ms.batch}x{ms.seq} tokens")
    s_model = build_model(shape, ms, "streamed", seed=2024 + wl.wid)
    r_model = StreamedLoraModel(shape, ms.n_layers, ms.vocab, ms.tied, ms.batch, ms.seq, mode="resident")
    r_model.copy_base_from(s_model)
    chunks = [synth.token_ids(T, ms.vocab, wl.wid, salt=i) for i in range(ms.n_micro)]
    inputs = s_model.prepare_inputs(chunks)
    ls, lr_ = s_model.step(inputs), r_model.step(inputs)
    torch.cuda.synchronize()
    exact = bool(torch.equal(ls, lr_) and torch.equal(s_model.lora.grad, r_model.lora.grad)
                 and torch.equal(s_model.lora.master, r_model.lora.master) and torch.equal(s_model.ckpt, r_model.ckpt))
    steps, warm = max(1, min(args.steps, 3)), 1
    st = time_steps(s_model, inputs, steps, warm)
    cs = time_steps(s_model, inputs, 1, 0, stats=True)
    rt = time_steps(r_model, inputs, steps, warm)
    ntok = T * ms.n_micro
    out = {"workload": (f"{name}: {ms.n_layers} layers, hidden {shape.hidden}, {shape.n_q}/{shape.n_kv} heads, "
                        f"MLP {shape.inter}, vocab {ms.vocab}{' tied' if ms.tied else ''}, {shape.wfmt} base, "
                        f"LoRA r{shape.lora_r}, {ms.n_micro} microbatch(es) of {ms.batch}x{ms.seq} tokens, AdamW"),
           "streamed_ms_per_step": round(st["ms_per_step"], 3), "resident_ms_per_step": round(rt["ms_per_step"], 3),
           "streamed_over_resident": round(st["ms_per_step"] / rt["ms_per_step"], 3),
           "streamed_tok_s": round(ntok / (st["ms_per_step"] * 1e-3), 1),
           "resident_tok_s": round(ntok / (rt["ms_per_step"] * 1e-3), 1),
           "bit_exact_vs_resident": exact, "blob_bytes": s_model.blob_bytes,
           "store_GB": round(s_model.blob_bytes * ms.n_layers / 1e9, 3),
           "h2d_loads_per_step": cs.get("h2d_loads"), "h2d_bytes_per_step": cs.get("h2d_bytes"),
           "h2d_GBps_copy_engine": cs.get("h2d_copy_s") and round(cs["h2d_bytes"] / cs["h2d_copy_s"] / 1e9, 2),
           "h2d_GBps_over_step": cs.get("h2d_bytes") and round(cs["h2d_bytes"] / (st["ms_per_step"] * 1e-3) / 1e9, 2),
           "steps": steps, "loss": round(st["loss"], 5), "context": LEG_CONTEXT.get(name)}
    log(f"  {name}: streamed {st['ms_per_step']:.2f} ms, resident {rt['ms_per_step']:.2f} ms, "
        f"ratio {out['streamed_over_resident']}, bit-exact {exact}")
    del s_model, r_model, inputs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def counters_traffic():
    """HBM bytes per launch of the timed GEMM from committed rocprofv3 counters,
    if they were taken on the current kernel source (else None)."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
        src = open(os.path.join(ROOT, "layer_streamed_lora_amd", "csrc", "gemm.hip"), "rb").read()
        if hashlib.sha256(src).hexdigest() != c.get("gemm_hip_sha256"):
            return None
        return c["hbm_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(shape, ms):
    """The CPU oracle on a bounded sample of the same step: one Llama-8B layer
    forward + backward (recompute) at all 1024 tokens, that layer's NF4 dequant
    (done on every visit, forward and backward), and the cross-entropy forward +
    backward for 32 of the 1024 tokens; scaled to 32 layers and 1024 tokens."""
    import numpy as np
    import oracle as O
    import synth
    from synth.configs import PROJ_IN_OUT
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        if info:
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '?')} threads, "
                             f"{i.get('architecture', '?')})" for i in info)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    T = ms.batch * ms.seq
    w = synth.layer_weights(shape, 5, 0, ones_norm=True)
    lora = {k: v.astype(np.float64) for k, v in synth.layer_lora(shape, 5, 0).items()}
    x = synth.activation((T, shape.hidden), 5, "x").astype(np.float64)
    dy = synth.activation((T, shape.hidden), 5, "dy").astype(np.float64) * 1e-3
    q = {p: O.nf4_quantize(w[p].astype(np.float64)) for p in PROJ_IN_OUT(shape)}
    t0 = time.perf_counter()
    wd = {p: O.nf4_dequant(*q[p]) for p in PROJ_IN_OUT(shape)}
    t_deq = time.perf_counter() - t0
    wd["norm1"], wd["norm2"] = w["norm1"].astype(np.float64), w["norm2"].astype(np.float64)
    t0 = time.perf_counter()
    O.decoder_layer_fwd(x, wd, lora, shape, ms.batch, ms.seq)
    O.decoder_layer_bwd(x, dy, wd, lora, shape, ms.batch, ms.seq)
    t_layer = time.perf_counter() - t0
    ntok = 32
    h = synth.activation((ntok, shape.hidden), 5, "x", salt=3).astype(np.float64)
    wlm = synth.normal_bf16((ms.vocab, shape.hidden), 0.02, 5, 1000, 52).astype(np.float64)
    labels = synth.token_ids(ntok, ms.vocab, 5)
    t0 = time.perf_counter()
    O.ce_loss_fwd(h, wlm, labels)
    O.ce_loss_bwd(h, wlm, labels)
    t_ce = time.perf_counter() - t0
    step_s = ms.n_layers * (t_layer + 2 * t_deq) + t_ce * (T / ntok)
    return {"value": T * ms.n_micro / (step_s * ms.n_micro), "unit": "tok/s", "cores": int(threads), "kind": "oracle",
            "blas": blas, "host_cpus": len(os.sched_getaffinity(0)),
            "sample": (f"1 of {ms.n_layers} layers fwd+bwd at {T} tokens ({t_layer:.1f} s) + its NF4 dequant x2 "
                       f"({2 * t_deq:.1f} s) + cross-entropy fwd+bwd on {ntok} of {T} tokens ({t_ce:.1f} s), "
                       f"scaled to {ms.n_layers} layers and {T} tokens (float64 numpy)"),
            "est_step_s": step_s}


# ---------------------------------------------------------------- profiling
# The timed kernel is recognised in rocprofv3 output by its name and its grid:
# one 256-thread workgroup per 256 x 64 (or 128 x 64 below 1024 rows) output tile.
CALIB_MIB = 256


def gu_kernel(shape, ms):
    """Name prefix and grid (work-items) of the gate|up forward GEMM launch: the
    library's 256 x 256-tile kernel once the output has at least 192 such tiles,
    else the 64-row tiles (256 tokens from 1024 tokens on, 128 below)."""
    T, N = ms.batch * ms.seq, 2 * shape.inter
    big = -(-T // 256) * -(-N // 256)
    if big >= 192:
        return "gemm_big_kernel<0, false, 1, 0>", big * 512
    bm = 256 if T >= 1024 else 128
    return "gemm_kernel<0, false, 1, 0,", -(-T // bm) * -(-N // 64) * 256


def gu_grid_items(shape, ms):
    return gu_kernel(shape, ms)[1]


def gu_algorithmic_bytes(shape, ms):
    """Bytes the gate|up forward launch must move at least once: x, the NF4
    codes and absmax, the LoRA B rows and x A^T, and the bf16 output."""
    T, K, N, kl = ms.batch * ms.seq, shape.hidden, 2 * shape.inter, 2 * shape.lora_r
    return T * K * 2 + N * K // 2 + N * K // 64 * 4 + N * kl * 2 + T * kl * 2 + T * N * 2


def calib_copy():
    """A plain copy kernel of known size for scaling the HBM byte counters:
    elementwise negation of CALIB_MIB MiB of bf16 (reads and writes that much)."""
    import torch
    n = CALIB_MIB << 20
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()


def _rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d, pattern):
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        sys.exit(f"no {pattern} under {d}")
    return hits[0]


def _grid_items(r):
    if "Grid_Size" in r:
        return int(float(r["Grid_Size"]))
    return int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])


def hbm_kernels(shape, ms):
    """Bandwidth-bound kernels of one step at the workload's shapes: (kernel name
    prefix in the trace, algorithmic HBM bytes per launch, what they are)."""
    from synth.configs import PROJ_IN_OUT
    T, H, I = ms.batch * ms.seq, shape.hidden, shape.inter
    nq, nkv, d = shape.n_q, shape.n_kv, shape.head_dim
    n_params = ms.n_layers * sum(shape.lora_r * (fin + fout) for fin, fout in PROJ_IN_OUT(shape).values())
    return [
        ("void lsl::rmsnorm_fwd_kernel<false>", 2 * T * H * 2 + 2 * H, "x read, y written, bf16 [T x H]"),
        ("void lsl::rmsnorm_bwd_kernel<false>", 4 * T * H * 2 + 2 * H, "x, dy, residual gradient read, dx written"),
        ("void lsl::rmsnorm_fwd_kernel<true>", None, "split partials and residual read, h and y written"),
        ("void lsl::rmsnorm_bwd_kernel<true>", None, "split partials, x, residual gradient read, dy and dx written"),
        ("lsl::swiglu_fwd_kernel", 3 * T * I * 2, "gate|up read, a written"),
        ("lsl::swiglu_bwd_kernel", 5 * T * I * 2, "gate|up and da read, dgate|dup written"),
        ("lsl::rope_kernel", (nq + nkv) * T * d * 2 * 2, "q and k heads read, rotated copy written (one launch)"),
        ("lsl::rope_split_kernel", None, "split partials read, q|k|v and the rotated q and k written"),
        ("lsl::adamw_kernel", n_params * (4 * 4 + 3 * 4 + 2), "master, grad, m, v read; master, m, v, bf16 copy written"),
    ]


def summarize_trace(d, args):
    """Markdown summary of a `rocprofv3 --kernel-trace --stats -f csv` run: the
    top kernels by total time, and the timed GEMM's dispatches (by grid)."""
    wl, shape, ms = workload(args.workload)
    if args.trace_tokens:  # the run's tokens per layer visit, in sequences of the workload's length
        import dataclasses
        ms = dataclasses.replace(ms, batch=args.trace_tokens // ms.seq)
    stats = _rows(_find(d, "*kernel_stats.csv"))
    out = ["| kernel | calls | total ms | avg us | % |", "|---|---:|---:|---:|---:|"]
    for r in stats[:25]:
        name = r["Name"] if len(r["Name"]) < 110 else r["Name"][:107] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                   f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    trace = _rows(_find(d, "*kernel_trace.csv"))
    kname, g = gu_kernel(shape, ms)
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
            if kname in r["Kernel_Name"] and _grid_items(r) == g]
    out.append("")
    if durs:
        out.append(f"gate|up forward GEMM dispatches ({kname.split('<')[0]}, {g} work-items): {len(durs)} calls, "
                   f"average {sum(durs) / len(durs):.1f} us, min {min(durs):.1f} us, max {max(durs):.1f} us")
    # attention: algorithmic FLOP / average duration against the bf16 MFMA peak (causal: half the
    # dense products; forward 2 products, dK/dV 4 (scores and dP recomputed), dQ 3)
    half = ms.batch * shape.n_q * ms.seq * ms.seq * shape.head_dim  # 2 B nq S^2 d / 2 per product
    out += ["", "| attention kernel | calls | avg us | algorithmic GFLOP per launch | TF/s | of bf16 peak |",
            "|---|---:|---:|---:|---:|---:|"]
    # (the kernel families: attn_fwd_kernel / attn_fwd_dma_kernel, attn_dkv_kernel, attn_dq_kernel /
    # attn_dq_dma_kernel; the forward's launches include the reference forwards and the recomputation)
    for prefix, nprod in (("void lsl::attn_fwd", 2), ("void lsl::attn_dkv", 4), ("void lsl::attn_dq", 3)):
        rows = [r for r in trace if r["Kernel_Name"].startswith(prefix)]
        if not rows:
            continue
        ds = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
        names = sorted({r["Kernel_Name"].split("(")[0][5:] for r in rows})
        avg = sum(ds) / len(ds)
        fl = nprod * half
        out.append(f"| `{', '.join(names)}` | {len(ds)} | {avg:.1f} | {fl / 1e9:.2f} | {fl / (avg * 1e-6) / 1e12:.0f} | "
                   f"{fl / (avg * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.2f} |")
    # bandwidth-bound kernels: algorithmic bytes / average duration against the 8 TB/s HBM peak
    out += ["", "| bandwidth-bound kernel | calls | avg us | algorithmic bytes per launch | GB/s | of 8 TB/s | bytes |",
            "|---|---:|---:|---:|---:|---:|---|"]
    for prefix, nbytes, what in hbm_kernels(shape, ms):
        ds = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
              if r["Kernel_Name"].startswith(prefix)]
        if not ds:
            continue
        avg = sum(ds) / len(ds)
        if nbytes is None:  # bytes depend on the split count: see --summarize-hbm-bytes
            out.append(f"| `{prefix}` | {len(ds)} | {avg:.1f} | - | - | - | {what} |")
            continue
        gbs = nbytes / (avg * 1e-6) / 1e9
        out.append(f"| `{prefix}` | {len(ds)} | {avg:.1f} | {nbytes:,} | {gbs:.0f} | {gbs / 8000:.2f} | {what} |")
    print("\n".join(out))


def summarize_copies(d, args):
    """Copy-engine timeline of a `rocprofv3 --kernel-trace --memory-copy-trace`
    run of `bench.py --no-resident --no-reference --steps K`: for each of the K timed steps
    (the layer copies before the final statistics step), copy-engine busy time,
    the idle gap at the turn of the sweep and at the step boundary, and the
    kernel time inside each gap."""
    wl, shape, ms = workload(args.workload)
    per_step = (2 * ms.n_layers - 4) * ms.n_micro
    cps = [r for r in _rows(_find(d, "*memory_copy_trace.csv")) if r["Direction"].endswith("HOST_TO_DEVICE")]
    kts = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in _rows(_find(d, "*kernel_trace.csv")))
    # layer copies: the pool's copies are the only ones taking over a millisecond
    big = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in cps
                 if int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) > 1_000_000)
    steps = args.steps
    timed = big[len(big) - (steps + 1) * per_step:len(big) - per_step]

    def kernel_ns(a, b):
        return sum(max(0, min(e, b) - max(s, a)) for s, e in kts if e > a and s < b)
    out = ["| step | span ms | copies | copy busy ms | GB/s while copying | largest gaps ms (kernel ms inside) | "
           "other gaps ms |", "|---|---:|---:|---:|---:|---|---:|"]
    for k in range(steps):
        c = timed[k * per_step:(k + 1) * per_step]
        nxt = timed[(k + 1) * per_step][0] if k + 1 < steps else None
        busy = sum(e - s for s, e in c) / 1e6
        gaps = [(c[i + 1][0] - c[i][1], c[i][1], c[i + 1][0]) for i in range(len(c) - 1)]
        if nxt is not None:
            gaps.append((nxt - c[-1][1], c[-1][1], nxt))
        gaps.sort(reverse=True)
        big2 = ", ".join(f"{g / 1e6:.2f} ({kernel_ns(a, b) / 1e6:.2f})" for g, a, b in gaps[:2])
        rest = sum(g for g, _, _ in gaps[2:]) / 1e6
        span = ((nxt if nxt is not None else c[-1][1]) - c[0][0]) / 1e6  # the last step ends at its last copy
        gbs = len(c) * args.blob_bytes / (busy * 1e-3) / 1e9 if args.blob_bytes else float("nan")
        out.append(f"| {k} | {span:.2f} | {len(c)} | {busy:.2f} | {gbs:.1f} | {big2} | {rest:.2f} |")
    print("\n".join(out))


def summarize_counters(fetch_dir, write_dir, args):
    """Scale the timed GEMM's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what
    the same counters read for the calibration copy, and write the counters file
    the benchmark reports as roofline traffic."""
    wl, shape, ms = workload(args.workload)
    kname, g = gu_kernel(shape, ms)
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _rows(_find(d, "*counter_collection.csv")) if r["Counter_Name"] == counter]
        copy = [float(r["Counter_Value"]) for r in rows if "neg_kernel" in r["Kernel_Name"]
                and _grid_items(r) >= 1 << 20]
        gemm = [float(r["Counter_Value"]) for r in rows if kname in r["Kernel_Name"] and _grid_items(r) == g]
        if not copy or not gemm:
            sys.exit(f"{counter}: copy dispatches {len(copy)}, gemm dispatches {len(gemm)}")
        kib_copy = sum(copy) / len(copy)
        scale = (CALIB_MIB << 20) / (kib_copy * 1024.0)
        res[counter] = {"gemm_kib_per_dispatch": sum(gemm) / len(gemm), "dispatches": len(gemm),
                        "copy_kib_per_dispatch": kib_copy, "copy_bytes_known": CALIB_MIB << 20, "scale": scale,
                        "gemm_bytes_per_dispatch": sum(gemm) / len(gemm) * 1024.0 * scale}
    src = open(os.path.join(ROOT, "layer_streamed_lora_amd", "csrc", "gemm.hip"), "rb").read()
    hbm = res["FETCH_SIZE"]["gemm_bytes_per_dispatch"] + res["WRITE_SIZE"]["gemm_bytes_per_dispatch"]
    doc = {"kernel": GU_LABEL, "workload": args.workload,
           "gemm_hip_sha256": hashlib.sha256(src).hexdigest(), "counters": res,
           "hbm_bytes_per_launch": round(hbm), "algorithmic_bytes_per_launch": gu_algorithmic_bytes(shape, ms),
           "commands": args.commands}
    with open(COUNTERS, "w") as f:
        json.dump(doc, f, indent=1)
    print(json.dumps(doc, indent=1))


def layer_only(args):
    """One resident decoder layer of the workload's shape (seeded N(0, 0.02) base,
    the benchmark's adapters) at batch x seq tokens: `steps` timed forward and
    backward (with recompute) calls after `warmup` untimed ones. For kernel
    traces and hardware counters of every kernel of a layer without building
    the whole model. Prints one JSON line."""
    import dataclasses
    import torch
    import synth
    from layer_streamed_lora_amd import model as M, _abi
    wl, shape, ms = workload(args.workload)
    if args.layer_seq:
        ms = dataclasses.replace(ms, batch=1, seq=args.layer_seq)
    T = ms.batch * ms.seq
    one = dataclasses.replace(ms, n_layers=1)
    m = build_model(shape, one, "resident")
    cfg, blob = m.cfg, m.blob_view(0)
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn((T, shape.hidden), generator=g, device="cuda").to(torch.bfloat16)
    dy = torch.randn((T, shape.hidden), generator=g, device="cuda").to(torch.bfloat16)
    out, dx = torch.empty_like(x), torch.empty_like(x)
    ws = torch.empty(M.layer_workspace_bytes(cfg, ms.batch, ms.seq, _abi.MODE_BWD), dtype=torch.uint8, device="cuda")
    lo, gr = m.lora.lora_set(0), m.lora.lora_grads(0)

    def fwd():
        M.decoder_layer_fwd(cfg, blob, lo, x, ms.batch, ms.seq, out=out, ws=ws)

    def bwd():
        M.decoder_layer_bwd(cfg, blob, lo, x, dy, ms.batch, ms.seq, gr, dx=dx, ws=ws)
    res = {"workload": f"one {args.workload} layer at {ms.batch}x{ms.seq} tokens, resident"}
    for name, fn in (("fwd", fwd), ("bwd", bwd)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[f"layer_{name}_ms"] = round(e0.elapsed_time(e1) / max(args.steps, 1), 4)
        log(f"  layer {name}: {res[f'layer_{name}_ms']} ms")
    print(json.dumps(res), flush=True)


def ce_only(args):
    """The fused cross-entropy of the workload's head (T tokens, hidden H, vocab
    V, its lm_head) on seeded inputs: `steps` timed forward + backward calls
    after `warmup`, for traces and HBM counters. Prints one JSON line."""
    import torch
    from layer_streamed_lora_amd import ops
    wl, shape, ms = workload(args.workload)
    T, H, V = ms.batch * ms.seq, shape.hidden, ms.vocab
    g = torch.Generator(device="cuda").manual_seed(11)
    h = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((V, H), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    labels = torch.randint(0, V, (T,), generator=g, device="cuda", dtype=torch.int32)
    ws = torch.empty(ops.ce_workspace_bytes(T, H, V), dtype=torch.uint8, device="cuda")

    def run():
        loss, lse = ops.fused_ce_loss_fwd(h, w, labels, ws=ws)
        ops.fused_ce_loss_bwd(h, w, labels, lse, ws=ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms_call = e0.elapsed_time(e1) / max(args.steps, 1)
    print(json.dumps({"workload": f"fused CE of {args.workload}: T {T}, H {H}, V {V}", "fwd_bwd_ms": round(ms_call, 4),
                      "logits_avoided_GB_naive_14B": round(14 * T * V / 1e9, 3)}), flush=True)


def summarize_ce_bytes(fetch_dir, write_dir, args):
    """HBM bytes per logit element of the fused cross-entropy (forward and
    backward) from two rocprofv3 --pmc runs of `--ce-only --calib-copy`
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), scaled by what the same
    counters read for the calibration copy. The CE kernels of one call are the
    lm_head GEMM passes and the small reductions around them."""
    wl, shape, ms = workload(args.workload)
    T, H, V = ms.batch * ms.seq, shape.hidden, ms.vocab
    ce_names = ("gemm_big_kernel<1", "gemm_kernel<1", "ce_")
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _rows(_find(d, "*counter_collection.csv")) if r["Counter_Name"] == counter]
        copy = [float(r["Counter_Value"]) for r in rows if "neg_kernel" in r["Kernel_Name"]
                and _grid_items(r) >= 1 << 20]
        ce = [r for r in rows if any(n in r["Kernel_Name"] for n in ce_names)]
        if not copy or not ce:
            sys.exit(f"{counter}: copy dispatches {len(copy)}, CE dispatches {len(ce)}")
        scale = (CALIB_MIB << 20) / (sum(copy) / len(copy) * 1024.0)
        calls = args.steps + args.warmup
        per_kernel = {}
        for r in ce:
            k = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("lsl::", "")
            per_kernel[k] = per_kernel.get(k, 0.0) + float(r["Counter_Value"]) * 1024.0 * scale / calls
        res[counter] = {"scale": scale, "bytes_per_call": sum(per_kernel.values()), "per_kernel": per_kernel}
    total = res["FETCH_SIZE"]["bytes_per_call"] + res["WRITE_SIZE"]["bytes_per_call"]
    doc = {"workload": f"fused CE, T {T}, H {H}, V {V} (forward + backward)", "counters": res,
           "hbm_bytes_per_call": round(total), "bytes_per_logit_element": round(total / (T * V), 3),
           "lm_head_bytes_per_call_algorithmic": 3 * V * H * 2,
           "pages_naive_bytes_per_logit_element": 14, "commands": args.commands}
    print(json.dumps(doc, indent=1))


def summarize_hbm_bytes(fetch_dir, write_dir, args):
    """HBM bytes per dispatch of the layer's bandwidth-bound kernels from two
    rocprofv3 --pmc runs of `--layer-only --calib-copy` (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch), scaled by what the same counters read for the
    calibration copy, beside each kernel's algorithmic bytes; with --trace-dir
    (a kernel-trace run of the same shapes) also the counter bytes over the
    kernel's average duration. Prints a markdown table."""
    wl, shape, ms = workload(args.workload)
    kernels = [k for k in hbm_kernels(shape, ms) if "adamw" not in k[0]]
    kernels.append(("lsl::gemm_split_reduce", None, "split partials read, bf16 result written"))
    got = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _rows(_find(d, "*counter_collection.csv")) if r["Counter_Name"] == counter]
        copy = [float(r["Counter_Value"]) for r in rows if "neg_kernel" in r["Kernel_Name"]
                and _grid_items(r) >= 1 << 20]
        if not copy:
            sys.exit(f"{counter}: no calibration copy dispatch")
        scale = (CALIB_MIB << 20) / (sum(copy) / len(copy) * 1024.0)
        for prefix, _, _ in kernels:
            vals = [float(r["Counter_Value"]) * 1024.0 * scale for r in rows if r["Kernel_Name"].startswith(prefix)]
            if vals:
                got.setdefault(prefix, {})[counter] = (sum(vals) / len(vals), len(vals), scale)
    durs = {}
    if args.trace_dir:
        trace = _rows(_find(args.trace_dir, "*kernel_trace.csv"))
        for prefix, _, _ in kernels:
            ds = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
                  if r["Kernel_Name"].startswith(prefix)]
            if ds:
                durs[prefix] = sum(ds) / len(ds)
    out = ["| kernel | dispatches | read MB | written MB | HBM MB per dispatch | algorithmic MB | "
           "HBM / algorithmic | trace avg us | HBM GB/s | of 8 TB/s |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for prefix, alg, what in kernels:
        g = got.get(prefix)
        if not g or "FETCH_SIZE" not in g or "WRITE_SIZE" not in g:
            continue
        rd, wr = g["FETCH_SIZE"][0], g["WRITE_SIZE"][0]
        tot = rd + wr
        avg = durs.get(prefix)
        gbs = tot / (avg * 1e-6) / 1e9 if avg else None
        out.append(f"| `{prefix}` | {g['FETCH_SIZE'][1]} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | {tot / 1e6:.1f} | "
                   + (f"{alg / 1e6:.1f} | {tot / alg:.2f}" if alg else "- | -") + " | "
                   + (f"{avg:.1f} | {gbs:.0f} | {gbs / 8000:.2f}" if avg else "- | - | -") + " |")
    print("\n".join(out))


def summarize_pmc(dirs, args):
    """Per-kernel averages of the hardware counters of one or more `rocprofv3
    --pmc` runs of this library's kernels (one row per kernel name and grid,
    values per dispatch), with derived ratios where their counters are present:
    MFMA utilisation (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs),
    the share of that time with VALU work issued beside it
    (SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES), VALU instructions
    per MFMA instruction, the LDS bank-conflict share (SQ_LDS_BANK_CONFLICT over
    SQ_ACTIVE_INST_LDS) and the wave-state shares (waiting on a counter,
    waiting to issue, issuing; over SQ_WAVE_CYCLES). rocprofv3 sums each
    counter over its dimensions, so GRBM_GUI_ACTIVE (one clock count per XCD) is
    divided by the XCD count before it is used as the dispatch's duration."""
    import collections
    simds = 4 * args.cus
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    names = []
    for d in dirs:
        for r in _rows(_find(d, "*counter_collection.csv")):
            if "lsl::" not in r["Kernel_Name"]:
                continue  # torch's and the runtime's own kernels
            k = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("lsl::", "") + f" grid {_grid_items(r)}"
            v = float(r["Counter_Value"])
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                v /= args.xcds
            per[k][r["Counter_Name"]].append(v)
            if r["Counter_Name"] not in names:
                names.append(r["Counter_Name"])

    def ratio(avg, num, den, scale=1.0):
        return avg[num] / (avg[den] * scale) if avg.get(num) is not None and avg.get(den) else None
    derived = [("MFMA util", lambda a: ratio(a, "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", simds)),
               ("VALU beside MFMA", lambda a: ratio(a, "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES")),
               ("VALU / MFMA instr", lambda a: ratio(a, "SQ_INSTS_VALU", "SQ_INSTS_MFMA")),
               ("LDS conflict / LDS active", lambda a: ratio(a, "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS")),
               ("waiting", lambda a: ratio(a, "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")),
               ("waiting to issue", lambda a: ratio(a, "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")),
               ("issuing", lambda a: ratio(a, "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES"))]
    rows = []
    for k, c in per.items():
        n = max(len(v) for v in c.values())
        avg = {cn: (sum(c[cn]) / len(c[cn]) if c.get(cn) else None) for cn in names}
        dv = [(dn, f(avg)) for dn, f in derived]
        key = avg.get("GRBM_GUI_ACTIVE") or avg.get("SQ_WAVE_CYCLES") or 0
        rows.append((-key * n, k, n, avg, dv))
    rows.sort()
    shown = [dn for dn, _ in derived if any(v is not None for _, _, _, _, dv in rows for d2, v in dv if d2 == dn)]
    out = ["| kernel | dispatches | " + " | ".join(names + shown) + " |",
           "|---|---:|" + "---:|" * (len(names) + len(shown))]
    for _, k, n, avg, dv in rows[:args.top]:
        vals = ["" if avg[cn] is None else f"{avg[cn]:.4g}" for cn in names]
        dd = dict(dv)
        vals += ["" if dd[dn] is None else f"{dd[dn]:.3f}" for dn in shown]
        out.append(f"| `{k[:110]}` | {n} | " + " | ".join(vals) + " |")
    print("\n".join(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama8b_nf4")
    ap.add_argument("--no-resident", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-nf4dq", action="store_true", help="skip the double-quantized-absmax variant")
    ap.add_argument("--no-reference", action="store_true", help="skip the adapter-off reference forward")
    ap.add_argument("--no-large-t", action="store_true", help="skip the 8 x 1024-token streamed/resident point")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the Qwen-0.5B and Qwen-3B streamed/resident legs")
    ap.add_argument("--t-sweep", action="store_true",
                    help="streamed vs resident step time from 1k to 16k tokens per layer visit, then exit")
    ap.add_argument("--sizes", type=int, nargs="*", default=[1024, 2048, 4096, 8192, 16384],
                    help="token counts of --t-sweep (multiples of 1024)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one plain copy kernel of known size first (for scaling HBM byte counters)")
    ap.add_argument("--summarize-trace", metavar="DIR", help="summarise a rocprofv3 kernel-trace csv run and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc csv runs into the committed counters file and exit")
    ap.add_argument("--commands", nargs="*", default=[], help="commands recorded in the counters file")
    ap.add_argument("--summarize-copies", metavar="DIR",
                    help="summarise a rocprofv3 kernel + memory-copy trace of a --no-resident run and exit")
    ap.add_argument("--blob-bytes", type=int, default=0, help="layer blob size, for --summarize-copies")
    ap.add_argument("--layer-only", action="store_true",
                    help="time one resident layer's forward and backward (for traces and counters), then exit")
    ap.add_argument("--layer-seq", type=int, default=0, help="tokens of --layer-only (default: the workload's)")
    ap.add_argument("--ce-only", action="store_true",
                    help="time the fused cross-entropy of the workload's head (for counters), then exit")
    ap.add_argument("--summarize-ce-bytes", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="HBM bytes per logit element of two --ce-only --pmc runs, then exit")
    ap.add_argument("--summarize-hbm-bytes", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="HBM bytes of the layer's bandwidth-bound kernels from two --pmc runs of "
                         "--layer-only --calib-copy, and exit")
    ap.add_argument("--trace-dir", metavar="DIR", help="kernel-trace run for --summarize-hbm-bytes durations")
    ap.add_argument("--trace-tokens", type=int, default=0,
                    help="tokens per layer visit of the run --summarize-trace reads (default: the workload's)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="per-kernel averages of rocprofv3 --pmc runs (markdown), then exit")
    ap.add_argument("--cus", type=int, default=256, help="compute units, for --summarize-pmc")
    ap.add_argument("--xcds", type=int, default=8, help="accelerator dies (XCDs), for --summarize-pmc")
    ap.add_argument("--top", type=int, default=30, help="kernels listed by --summarize-pmc")
    args = ap.parse_args()
    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc, args)
    if args.summarize_ce_bytes:
        return summarize_ce_bytes(*args.summarize_ce_bytes, args)
    if args.summarize_hbm_bytes:
        return summarize_hbm_bytes(*args.summarize_hbm_bytes, args)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args)
    if args.summarize_copies:
        return summarize_copies(args.summarize_copies, args)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters, args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (one process, one MI355X); "
              f"--gpus {args.gpus} / WORLD_SIZE {world} is not supported", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import layer_streamed_lora_amd as lsl
    import synth
    lsl.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calib_copy:
        calib_copy()
    if args.t_sweep:
        return t_sweep(args, args.sizes)
    if args.layer_only:
        return layer_only(args)
    if args.ce_only:
        return ce_only(args)
    wl, shape, ms = workload(args.workload)
    T = ms.batch * ms.seq
    log(f"building {args.workload}: {ms.n_layers} layers, hidden {shape.hidden}, {shape.wfmt} base")
    t0 = time.perf_counter()
    s_model = build_model(shape, ms, "streamed")
    log(f"  streamed model built in {time.perf_counter() - t0:.1f} s; blob {s_model.blob_bytes} B, "
        f"store {s_model.blob_bytes * ms.n_layers / 1e9:.3f} GB pinned")
    chunks = [synth.token_ids(T, ms.vocab, wl.wid, salt=i) for i in range(ms.n_micro)]
    inputs = s_model.prepare_inputs(chunks)
    # device memory of the streamed model: persistent buffers (2 slots, embedding,
    # lm_head, checkpoints, adapters and their optimizer state, workspace) and the
    # peak over one step (no optimizer update, so the state stays untouched)
    torch.cuda.synchronize()
    hbm_live = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    s_model.step(inputs, adamw=False)
    torch.cuda.synchronize()
    hbm_peak = torch.cuda.max_memory_allocated()
    log(f"  streamed model device memory: {hbm_live / 1e9:.2f} GB allocated, {hbm_peak / 1e9:.2f} GB peak in a step")

    bit_exact = None
    r_model = None
    if not args.no_resident:
        from layer_streamed_lora_amd.trainer import StreamedLoraModel
        r_model = StreamedLoraModel(shape, ms.n_layers, ms.vocab, ms.tied, ms.batch, ms.seq, mode="resident")
        r_model.copy_base_from(s_model)
        ls = s_model.step(inputs)
        lr_ = r_model.step(inputs)
        torch.cuda.synchronize()
        bit_exact = bool(torch.equal(ls, lr_) and torch.equal(s_model.lora.grad, r_model.lora.grad)
                         and torch.equal(s_model.lora.master, r_model.lora.master)
                         and torch.equal(s_model.ckpt, r_model.ckpt) and torch.equal(s_model.lse, r_model.lse))
        log(f"  streamed vs resident bit-exact: {bit_exact}")

    peak_h2d = pinned_h2d_peak(s_model.blob_bytes, s_model.pool.copy_stream)
    log(f"  pinned H2D (hipMemcpyAsync, {s_model.blob_bytes} B): {peak_h2d:.1f} GB/s")
    # the copy a GPU would make if N GPUs each pulled 1/N of every layer and
    # exchanged the rest over xGMI (cooperative streaming, not built here)
    slices = {}
    for n in (2, 4, 8):
        nb = (s_model.blob_bytes // n + 255) // 256 * 256
        slices[f"1/{n}"] = {"bytes": nb, "GBps": round(pinned_h2d_peak(nb, s_model.pool.copy_stream), 2)}
    log("  pinned H2D of layer slices: " + ", ".join(f"{k} {v['GBps']} GB/s" for k, v in slices.items()))
    res = time_steps(s_model, inputs, args.steps, args.warmup, timing_which=3)
    log(f"  streamed: {res['ms_per_step']:.2f} ms/step, loss {res['loss']:.4f}")
    # copy-engine statistics (an event pair per copy) in a separate, untimed step
    cs = time_steps(s_model, inputs, 1, 0, stats=True)
    res.update({k: cs[k] for k in ("h2d_loads", "h2d_bytes", "h2d_copy_s") if k in cs})
    resident = None
    gemms = None
    if r_model is not None:
        resident = time_steps(r_model, inputs, args.steps, args.warmup)
        log(f"  resident: {resident['ms_per_step']:.2f} ms/step")
        gemms = gemm_groups(r_model, inputs, shape, ms)
        log("  GEMMs: " + ", ".join(f"{k} {v['TFLOP_s']} TF/s" for k, v in gemms.items()))
    reference = None
    if not args.no_reference:
        reference = time_reference(s_model, inputs, args.steps, args.warmup)
        log(f"  reference forward (adapters off, streamed): {reference['ms']:.2f} ms per {T * ms.n_micro} tokens")

    variant = None
    if not args.no_nf4dq and args.workload == "llama8b_nf4":
        del r_model
        r_model = None
        torch.cuda.empty_cache()
        variant = nf4dq_leg(args, wl.wid)

    # the same model at 8 x 1024 tokens per layer visit, where the copies hide
    # behind compute (the full sweep: --t-sweep)
    large_t = None
    if not args.no_large_t and args.workload == "llama8b_nf4":
        del s_model
        torch.cuda.empty_cache()
        large_t = t_sweep(args, [8192], emit=False)[0]
    # the bf16-base workloads the pages quote (streaming overhead at 0.5B, tok/s at 3B)
    legs = None
    if not args.no_legs and args.workload == "llama8b_nf4":
        legs = {n: model_leg(n, args) for n in ("qwen05b_bf16", "qwen3b_bf16")}

    tok_s = T * ms.n_micro / (res["ms_per_step"] * 1e-3)
    flops = step_flops(shape, ms)
    # the timed kernel: forward gate|up GEMM, NF4 dequant fused, LoRA-up K-step fused
    K, N, kl = shape.hidden, 2 * shape.inter, 2 * shape.lora_r
    g_flops = 2.0 * T * K * N + 2.0 * T * kl * N
    g_ms = res["kernel_ms_total"] / max(res["kernel_launches"], 1)
    achieved = g_flops / (g_ms * 1e-3) / 1e12
    h2d_copy = res["h2d_bytes"] / res["h2d_copy_s"] / 1e9 if res.get("h2d_copy_s") else None
    step_bytes = res.get("h2d_bytes", 0)  # the statistics step moves one step's bytes
    h2d_eff = step_bytes / (res["ms_per_step"] * 1e-3) / 1e9 if step_bytes else None
    out = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: Llama-3.1-8B-shaped, 32 layers, NF4 base (block 64, fp32 absmax) "
                               f"streamed through 2 HBM slots, LoRA r16 a32 on all projections, "
                               f"{ms.batch}x{ms.seq} tokens, fused CE, AdamW",
                   "batch": ms.batch, "seq_len": ms.seq, "n_micro": ms.n_micro, "layers": ms.n_layers,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": GU_LABEL + " 1024x28672x4096",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": counters_traffic(),
                     "avg_launch_ms": round(g_ms, 4), "launches": res["kernel_launches"]},
        "mfma_frac_step": round(flops / (res["ms_per_step"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "gemms_resident": gemms,
        "h2d": {"achieved_GBps_copy_engine": h2d_copy and round(h2d_copy, 2),
                "achieved_GBps_over_step": h2d_eff and round(h2d_eff, 2),
                "pinned_peak_GBps": round(peak_h2d, 2), "pinned_slices": slices,
                "frac_of_pinned_peak": h2d_copy and round(h2d_copy / peak_h2d, 3),
                "bytes_per_step": step_bytes},
        "resident": resident and {"ms_per_step": round(resident["ms_per_step"], 3),
                                  "tok_s": round(T * ms.n_micro / (resident["ms_per_step"] * 1e-3), 2)},
        "streamed_over_resident": resident and round(res["ms_per_step"] / resident["ms_per_step"], 3),
        "bit_exact_vs_resident": bit_exact,
        "at_8192_tokens": large_t and dict(large_t, what="the same model at 8 x 1024 tokens per layer visit "
                                                         "(one microbatch), streamed and resident"),
        "hbm_streamed_GB": {"allocated": round(hbm_live / 1e9, 3), "peak_in_step": round(hbm_peak / 1e9, 3),
                            "pages_peak_vram_GB": 3.32},
        "loss": round(res["loss"], 5),
        "nf4dq": variant,
        "legs": legs,
        "reference_forward": reference and {
            "what": "adapter-off streamed forward + per-token log-probs (preference reference)",
            "ms": round(reference["ms"], 3), "tok_s": round(T * ms.n_micro / (reference["ms"] * 1e-3), 2),
            "layer_copies": reference["loads"], "mean_logp": round(reference["mean_logp"], 4)},
        "context": {"pages_tok_s": 119.6, "pages_hardware": "RTX 3050 Laptop 4 GB, seq/batch not stated"},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle sample ...")
        cb = cpu_baseline(shape, ms)
        cb["value"] = round(cb["value"], 4)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
