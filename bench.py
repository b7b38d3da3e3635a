"""Benchmark of the OmniQuant block-calibration step on one MI355X.

One step = quantized forward of a LLaMA-7B-shaped decoder block (LWC + LET,
W4A4, s_a on Q/K) on one 2048-token sample, the MSE against the full-precision
block output, the straight-through backward for every learnable parameter, and
the AdamW update.  The full-precision target is computed once, before timing.
Inputs are seeded synthetic tensors of the real shapes (random-init weights,
activations with systematic outlier channels) resident in HBM before timing.

Prints one JSON line.  Other workloads (--workload) are available for
exploration; the default is the headline one.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

def metric_of(c):
    """The metric string of a block workload, from its own shape and bit widths (the
    7B-shaped W4A4 block's is the headline metric above)."""
    shape = "LLaMA-2-70B-shaped" if c.d == 8192 else "LLaMA-7B-shaped"
    bits = "W%dA%d" % (c.wbits, c.abits) + ("g%d" % c.group if c.group else "")
    part = "FFN" if c.ffn_only else "block"
    return "LWC+LET %s fwd+bwd calib steps/s & TFLOP/s, %s, %s, 1 GPU" % (part, shape, bits)
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 matrix-core peak
PEAK_HBM_GBS = 8000.0


def workloads():
    import synth
    return {
        "llama7b_block_w4a4": synth.BLOCK_CFG4,
        "llama70b_block_w4a16": synth.BLOCK_CFG5_W4,
        "llama70b_block_w2a16": synth.BLOCK_CFG5_W2,
        "llama7b_ffn_w3a16": synth.FFN_CFG3_W3,
        "llama7b_ffn_w2a16": synth.FFN_CFG3_W2,
        "llama7b_block_w3a16g128": synth.BLOCK_CFG4_W3G128,
        "llama7b_block_w2a16g128": synth.BLOCK_CFG4_W2G128,
    }


def step_flops(c):
    """Algorithmic FLOPs of one step: GEMMs 6 T sum(W) (forward 2, backward 4);
    attention counts the causal half, forward 2 T^2 n_q hd, backward twice that."""
    import synth
    shapes = synth.block_weight_shapes(c)
    names = ("gate", "up", "down") if c.ffn_only else synth.WEIGHT_NAMES
    sw = sum(shapes[n][0] * shapes[n][1] for n in names)
    f = 6.0 * c.T * sw
    if not c.ffn_only:
        f += 3.0 * 2.0 * c.T * c.T * c.n_q * c.head_dim
    return f


def measured_traffic(workload):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by the copy-kernel calibration), or None when
    there is none for this workload or the GEMM source has changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm_traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "post_quantization_amd", "csrc", "gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("gemm_source_sha256") != sha:
        return None
    return rec["traffic_bytes_per_launch"]


def cpu_baseline(c, inp, tokens):
    """The oracle (never tuned for speed) on a bounded sample of the workload: one
    full step (forward, MSE, backward, AdamW) of the same block on `tokens` tokens
    (by default all of them: the workload's own step, about 20 s on 16 cores).  With
    fewer tokens the rate is scaled linearly to the full count, which is only an
    estimate: the weight-side quantizer work does not shrink with the tokens (the
    scaled rate then understates the full-size one) while attention grows with their
    square (it then overstates it)."""
    import numpy as np
    import synth
    from oracle import block as ob
    from oracle import optim
    from oracle.ops import ExactOps
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count()
    cs = synth.reduced(c, T=tokens)
    x = inp["x"][:tokens]
    Wd = {k: v for k, v in inp.items() if k.startswith("W_")}
    ystar = ob.reference(cs, x, Wd)
    shapes = synth.block_weight_shapes(cs)
    th = ob.init_theta(cs, shapes)
    t0 = time.perf_counter()
    loss, g, _, _ = ob.calib_step(cs, x, Wd, ystar, th, ExactOps(bf16=True))
    vec = ob.pack(cs, shapes, th)
    gv = ob.pack(cs, shapes, {k: np.asarray(v, np.float32) for k, v in g.items()})
    z = np.zeros_like(vec)
    optim.adamw(vec, gv, z, z, 1, c.lr_let)
    dt = time.perf_counter() - t0
    sec_full = dt * (c.T / tokens)
    if tokens == c.T:
        sample = ("one oracle step (fwd+MSE+bwd+AdamW) of the whole workload (%d tokens, "
                  "all weights full size): %.1f s measured" % (c.T, dt))
    else:
        sample = ("one oracle step (fwd+MSE+bwd+AdamW) on %d of %d tokens, all weights full "
                  "size; %.1f s measured, scaled x%.2f to the full token count (an estimate: "
                  "weight-side work does not scale with tokens, attention scales with their "
                  "square)" % (tokens, c.T, dt, c.T / tokens))
    return {"value": 1.0 / sec_full, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": sample, "host": platform.processor() or platform.machine()}


DECODE_WORKLOADS = {"llama7b_w4a16g128_decode": 1, "llama7b_w4a16g128_decode_t16": 16}


def decode_main(args):
    """Deployment form (packed 4-bit codes, g128 steps): the linear products of one
    7B-shaped block at T tokens (single-token decode by default), with the products
    that share their input stored as one weight (q|k|v and gate|up, rows
    concatenated: 4 launches), timed per launch with HIP events on the launching
    stream; tokens/s for a 32-block model."""
    import numpy as np
    import torch
    import post_quantization_amd as omq
    import synth

    T = DECODE_WORKLOADS[args.workload]
    c = synth.BLOCK_CFG4
    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = synth.block_inputs(c)
    shapes = synth.block_weight_shapes(c)
    layers = []
    fused = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")),
             ("down", ("down",)))
    for n, parts in fused:
        K = shapes[parts[0]][1]
        N = sum(shapes[p][0] for p in parts)
        W = torch.from_numpy(np.concatenate([inp["W_" + p] for p in parts], axis=0)) \
            .to(torch.bfloat16).to(dev)
        logits = torch.full((N * K // 128,), 4.0, dtype=torch.float32, device=dev)
        r = omq.lwc_fakequant(W, logits, logits, 4, out_dtype=torch.bfloat16, want_codes=True,
                              group=128)
        layers.append((n, N, K, omq.pack_codes(r["codes"], 4), r["h"], r["z"], r["codes"]))
    rng = np.random.default_rng(0)
    Xs = {K: torch.from_numpy(synth.to_bf16(rng.standard_normal((T, K)).astype(np.float32)))
          .to(torch.bfloat16).to(dev) for K in {k for _, _, k, *_ in layers}}
    Ys = {n: torch.empty(T, N, dtype=torch.float32, device=dev) for n, N, *_ in layers}

    def block():
        for n, N, K, words, h, z, _ in layers:
            omq.w4a16_gemm(Xs[K], words, N, h, z, 128, None, Ys[n])

    # per-launch durations: each product captured 20 times in a row into a HIP graph,
    # HIP events around the replays on the launching stream (events around single
    # launches of a few microseconds would mostly time the events)
    for _ in range(args.warmup):
        block()
    torch.cuda.synchronize()
    R = 20
    durs = []
    for n, N, K, words, h, z, _ in layers:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            omq.w4a16_gemm(Xs[K], words, N, h, z, 128, None, Ys[n])
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gl = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gl):
            for _ in range(R):
                omq.w4a16_gemm(Xs[K], words, N, h, z, 128, None, Ys[n])
        gl.replay()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(args.steps):
            gl.replay()
        a1.record()
        torch.cuda.synchronize()
        durs.append(a0.elapsed_time(a1) / (args.steps * R))
    # the block as a serving loop runs it: its launches captured once into a HIP
    # graph and replayed (no host work between the kernels)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        block()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        block()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_block = e0.elapsed_time(e1) / args.steps
    per_layer = [(N * K // 2 + N * (K // 128) * 8 + T * K * 2 + T * N * 4)
                 for _, N, K, *_ in layers]
    bytes_launch = sum(per_layer) / len(per_layer)
    avg_s = sum(durs) / len(durs) / 1e3             # mean launch duration over the products
    achieved = bytes_launch / avg_s / 1e9
    tok_s = T * 1000.0 / (ms_block * 32)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import export as ex
        t0 = time.perf_counter()
        for n, N, K, words, h, z, codes in layers:
            ex.wa16_linear(Xs[K].float().cpu().numpy(), ex.pack_codes(codes.cpu().numpy(), 4),
                           h.cpu().numpy(), z.cpu().numpy(), 4, K, 128)
        dt = time.perf_counter() - t0
        cpu = {"value": T / (dt * 32), "unit": "tokens/s", "cores": os.cpu_count(),
               "kind": "oracle",
               "sample": "the oracle's packed product (unpack, dequant, bf16, float64 matmul) "
                         "for the linears of one block at %d token(s), %.2f s, x32 blocks"
                         % (T, dt)}
    out = {
        "metric": "W4A16g128 decode tokens/s, LLaMA-7B-shaped linears (32 blocks), 1 GPU",
        "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_block, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "d": c.d, "F": c.F, "wbits": 4,
                   "lwc_group": 128, "step": "the linear products of one block (q|k|v, o, "
                                             "gate|up, down), replayed from a HIP graph"},
        "roofline": {"kernel": "k_w4a16_gemv (T <= 8) / k_w4a16_gemm", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "launches": len(durs) * R * args.steps,
                     "avg_launch_us": round(avg_s * 1e6, 2),
                     "bytes_per_launch": int(bytes_launch)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


EXPORT_WORKLOADS = {"llama7b_block_w4a16g128_export": 4}


def export_main(args):
    """Deployment export of a calibrated 7B-shaped weight-only block (fake quantizer
    with codes, packing, LET folds), weights resident in HBM, timed with HIP events."""
    import numpy as np
    import torch
    import post_quantization_amd as omq
    from post_quantization_amd import export
    import synth

    c = synth.replace(synth.BLOCK_CFG4_W3G128, wbits=EXPORT_WORKLOADS[args.workload])
    torch.cuda.set_device(0)
    inp = synth.block_inputs(c)
    W = [torch.from_numpy(inp["W_" + n]).to(torch.bfloat16).cuda() for n in synth.WEIGHT_NAMES]
    d = omq.BlockDesc(T=c.T, d=c.d, n_q=c.n_q, n_kv=c.n_kv, head_dim=c.head_dim, F=c.F,
                      wbits=c.wbits, abits=c.abits, group=c.group)
    offs, n_lwc, total = omq.block_theta_layout(d)
    rng = np.random.default_rng(0)
    th = rng.uniform(0.9, 1.1, total).astype(np.float32)
    th[:n_lwc] = 4.0
    theta = torch.from_numpy(th).cuda()
    for _ in range(args.warmup):
        export.export_block(d, W, theta)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        export.export_block(d, W, theta)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    shapes = synth.block_weight_shapes(c)
    nw = sum(a * b for a, b in shapes.values())
    # weight read 2 B, fake-quant weight 2 B and codes 1 B written, codes re-read 1 B,
    # packed codes written and re-read by the fold 2 x 0.5 B
    traffic = 7.0 * nw
    gbs = traffic / (ms * 1e-3) / 1e9
    out = {
        "metric": "W4A16g128 deployment export, LLaMA-7B-shaped block (blocks/s), 1 GPU",
        "value": round(1000.0 / ms, 3), "unit": "blocks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "d": c.d, "F": c.F, "wbits": c.wbits,
                   "lwc_group": c.group, "weights": nw},
        "roofline": {"kernel": "export pipeline (fake quantizer, pack, fold)", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_step": int(traffic)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


GEMM_WORKLOADS = {"llama7b_step_gemms": "BLOCK_CFG4"}


def gemm_main(args):
    """The matrix products of one 7B-shaped W4A4 calibration step, each alone: the
    backward's eight bf16 products through omq_gemm (main loop only, no fused
    straight-through epilogue) beside torch.matmul (hipBLASLt) on the same operand
    layouts, and the forward's four products on int8 codes through omq_code_gemm (and,
    for 4-bit codes, on codes two to a byte through omq_code_gemm4, the step's form).
    Per shape: the mean of `steps` launches after `warmup`, on HIP events."""
    import torch
    import post_quantization_amd as omq
    import synth

    c = getattr(synth, GEMM_WORKLOADS[args.workload])
    T, d, F = c.T, c.d, c.F
    nqkv = (c.n_q + 2 * c.n_kv) * c.head_dim
    dev = "cuda:0"
    torch.cuda.set_device(0)
    # (name, M, N, K, trans_a, trans_b): C[M x N] = op(A) op(B)^T; backward dX = dY W_hat
    # (rows = tokens), dW = dY^T X_hat (rows = output channels, both operands K-major)
    bwd = [("dX_down", T, F, d, 0, 1), ("dX_gate_up", T, d, 2 * F, 0, 1),
           ("dX_o", T, d, d, 0, 1), ("dX_qkv", T, d, nqkv, 0, 1),
           ("dW_down", d, F, T, 1, 1), ("dW_gate_up", 2 * F, d, T, 1, 1),
           ("dW_o", d, d, T, 1, 1), ("dW_qkv", nqkv, d, T, 1, 1)]
    fwd = [("Y_qkv", T, nqkv, d), ("Y_o", T, d, d), ("Y_gate_up", T, 2 * F, d), ("Y_down", T, d, F)]

    def timeit(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    g = torch.Generator(device=dev)
    g.manual_seed(0)
    rows, tot_o, tot_t, flops = [], 0.0, 0.0, 0.0
    for name, M, N, K, ta, tb in bwd:
        A = torch.randn((K, M) if ta else (M, K), generator=g, device=dev).to(torch.bfloat16)
        B = torch.randn((K, N) if tb else (N, K), generator=g, device=dev).to(torch.bfloat16)
        C = torch.empty(M, N, dtype=torch.float32, device=dev)
        f = 2.0 * M * N * K
        t_o = timeit(lambda: omq.gemm(A, B, C=C, trans_a=bool(ta), trans_b=bool(tb)))
        At, Bt = (A.t() if ta else A), (B if tb else B.t())
        t_t = timeit(lambda: torch.matmul(At, Bt))
        tot_o += t_o
        tot_t += t_t
        flops += f
        rows.append({"product": name, "M": M, "N": N, "K": K, "omq_us": round(t_o * 1e3, 1),
                     "omq_tflops": round(f / t_o / 1e9, 1), "hipblaslt_us": round(t_t * 1e3, 1),
                     "hipblaslt_tflops": round(f / t_t / 1e9, 1)})
    codes = []
    for name, M, N, K in fwd:
        qa = torch.randint(0, 16, (M, K), generator=g, dtype=torch.uint8, device=dev)
        qb = torch.randint(0, 16, (N, K), generator=g, dtype=torch.uint8, device=dev)
        ha, hb = torch.rand(M, device=dev), torch.rand(N, device=dev)
        za, zb = torch.full((M,), 7.0, device=dev), torch.full((N,), 8.0, device=dev)
        sa, sb = omq.code_rowsum(qa), omq.code_rowsum(qb)
        C = torch.empty(M, N, dtype=torch.float32, device=dev)
        t = timeit(lambda: omq.code_gemm(qa, ha, za, qb, hb, zb, sa, sb, C=C))
        row = {"product": name, "M": M, "N": N, "K": K, "omq_us": round(t * 1e3, 1),
               "omq_tops": round(2.0 * M * N * K / t / 1e9, 1)}
        if c.wbits <= 4 and c.abits <= 4:
            # the step's form: 4-bit codes two to a byte (omq_code_gemm4)
            pa = (qa[:, 0::2] | (qa[:, 1::2] << 4)).contiguous()
            pb = (qb[:, 0::2] | (qb[:, 1::2] << 4)).contiguous()
            t4 = timeit(lambda: omq.code_gemm4(pa, ha, za, pb, hb, zb, K, sa, sb, C=C))
            row.update({"packed_us": round(t4 * 1e3, 1),
                        "packed_tops": round(2.0 * M * N * K / t4 / 1e9, 1)})
        codes.append(row)
    tf = flops / tot_o / 1e9
    out = {
        "metric": "bf16 matrix-core TFLOP/s of the backward products of one LLaMA-7B-shaped W4A4 "
                  "calibration step (main loops alone), 1 GPU",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(tot_o, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "d": d, "F": F},
        "roofline": {"kernel": "k_gemm_bf16 main loop (omq_gemm)", "bound": "mfma",
                     "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "hipblaslt_ms": round(tot_t, 4),
        "hipblaslt_tflops": round(flops / tot_t / 1e9, 2),
        "products": rows, "code_products": codes, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


CALIB_WORKLOADS = {"llama7b_w4a4_model_calib": ("BLOCK_CFG4", 32, 20)}


def calib_main(args):
    """Sequential multi-block calibration with the pages' schedule (128 samples,
    batch 1, 20 epochs per block, AdamW) on a stack of --calib-blocks LLaMA-7B-shaped
    W4A4 blocks: per block the cached full-precision targets, the calibration steps,
    and the calibrated block's outputs for the next block.  The whole-model time is
    the measured per-block time times the model's 32 blocks (all blocks have the same
    shape and schedule)."""
    import torch
    import post_quantization_amd as omq
    from post_quantization_amd import driver
    import synth

    name, model_blocks, epochs = CALIB_WORKLOADS[args.workload]
    c = getattr(synth, name)
    torch.cuda.set_device(0)
    dev = "cuda:0"
    nb, ns = args.calib_blocks, args.calib_samples
    W = []
    for b in range(nb):
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + b)
        shapes = synth.block_weight_shapes(c)
        W.append([(torch.randn(shapes[n], generator=g, device=dev) * synth.WEIGHT_STD)
                  .to(torch.bfloat16) for n in synth.WEIGHT_NAMES])
    xs = synth.stack_samples_device(c, ns, dev)
    d = omq.BlockDesc(T=c.T, d=c.d, n_q=c.n_q, n_kv=c.n_kv, head_dim=c.head_dim, F=c.F,
                      wbits=c.wbits, abits=c.abits, ffn_only=c.ffn_only, group=c.group,
                      eps=c.eps, rope_theta=c.rope_theta, lr_lwc=c.lr_lwc, lr_let=c.lr_let)

    def on_block(b, x, th):
        print("block %d calibrated" % b, flush=True)

    # a short warm run (one block, 2 samples, 1 epoch) so the timed run starts warm
    driver.calibrate(d, W[:1], xs[:2], 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res = driver.calibrate(d, W, xs, epochs, on_block=on_block)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_block = wall / nb
    steps_per_block = ns * epochs
    model_h = per_block * model_blocks / 3600.0
    sps = steps_per_block / per_block
    tflops = step_flops(c) * sps / 1e12
    out = {
        "metric": "whole-model OmniQuant calibration time, LLaMA-7B-shaped W4A4 (32 blocks, "
                  "%d samples x %d epochs per block), 1 GPU" % (ns, epochs),
        "value": round(model_h, 4), "unit": "hours", "n_gpus": 1, "steps": nb, "warmup": 1,
        "ms_per_step": round(per_block * 1e3, 1), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "T": c.T, "d": c.d, "F": c.F, "wbits": c.wbits,
                   "abits": c.abits, "samples": ns, "epochs": epochs, "blocks_timed": nb,
                   "model_blocks": model_blocks, "optimizer": "adamw", "batch": 1},
        "seconds_per_block": [round(s, 3) for s in res.seconds],
        "calib_steps_per_s": round(sps, 3),
        "extrapolation": "measured seconds per block x %d blocks" % model_blocks,
        "roofline": {"kernel": "whole calibration step (every kernel of the step)",
                     "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the matrix-core kernels run 5-10% faster after ten or so steps (the clock settles
    # under load): the default warm-up lets it settle before the timed steps
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama7b_block_w4a4",
                    choices=list(workloads()) + list(DECODE_WORKLOADS) +
                    list(EXPORT_WORKLOADS) + list(CALIB_WORKLOADS) + list(GEMM_WORKLOADS))
    ap.add_argument("--calib-blocks", type=int, default=2,
                    help="blocks timed by the whole-model calibration workload")
    ap.add_argument("--calib-samples", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the oracle's timed step (0: the workload's own count)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (known bytes) to calibrate the "
                         "FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the block-calibration step runs on one GPU (blocks are sequential "
              "and the step is not sharded across GPUs); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import post_quantization_amd as omq
    import synth

    if args.workload in DECODE_WORKLOADS:
        decode_main(args)
        return
    if args.workload in EXPORT_WORKLOADS:
        export_main(args)
        return
    if args.workload in CALIB_WORKLOADS:
        calib_main(args)
        return
    if args.workload in GEMM_WORKLOADS:
        gemm_main(args)
        return

    if args.copy_calibration:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")    # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4,
                          "launches": 3}), flush=True)
        return

    c = workloads()[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = synth.block_inputs(c)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    W = [bf(inp["W_" + n]) if ("W_" + n) in inp else None for n in synth.WEIGHT_NAMES]
    x = bf(inp["x"])
    n_launch_cap = 64 * (args.steps + 1)
    timer = omq.GemmTimer(n_launch_cap)
    d = omq.BlockDesc(T=c.T, d=c.d, n_q=c.n_q, n_kv=c.n_kv, head_dim=c.head_dim, F=c.F,
                      wbits=c.wbits, abits=c.abits, ffn_only=c.ffn_only, group=c.group, eps=c.eps,
                      rope_theta=c.rope_theta, lr_lwc=c.lr_lwc, lr_let=c.lr_let)
    dt_ = omq.BlockDesc(T=c.T, d=c.d, n_q=c.n_q, n_kv=c.n_kv, head_dim=c.head_dim, F=c.F,
                        wbits=c.wbits, abits=c.abits, ffn_only=c.ffn_only, group=c.group, eps=c.eps,
                        rope_theta=c.rope_theta, lr_lwc=c.lr_lwc, lr_let=c.lr_let, timer=timer)
    from post_quantization_amd import driver
    # initial parameters: clipping logits 4.0, s = 1, delta = 0, s_a = 1
    theta = driver.init_theta(d, dev)
    dtheta = torch.zeros_like(theta)
    m = torch.zeros_like(theta)
    v = torch.zeros_like(theta)
    # the loss of every step (warm-up and timed) lands in its own slot: no host sync
    losses = torch.zeros(args.warmup + 2 * args.steps + 1, dtype=torch.float32, device=dev)
    slots = [losses[i:i + 1] for i in range(losses.numel())]
    ws = torch.empty(omq.block_workspace_size(d), dtype=torch.uint8, device=dev)
    y_t = torch.empty(c.T, c.d, dtype=torch.float32, device=dev)

    # full-precision target, once
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    omq.block_forward(d, x, W, None, y_t, ws)
    e1.record()
    torch.cuda.synchronize()
    fp_ms = e0.elapsed_time(e1)

    step = 0
    for _ in range(args.warmup):
        step += 1
        omq.block_step(d, x, y_t, W, theta, dtheta, m, v, step, slots[step - 1], ws)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step += 1
        omq.block_step(d, x, y_t, W, theta, dtheta, m, v, step, slots[step - 1], ws)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    loss_curve = [round(float(l), 6) for l in losses[:step].cpu()]
    # the same number of steps again with per-launch events (outside the timed
    # region, so the event records do not weigh on `value`)
    timer.reset()
    for _ in range(args.steps):
        step += 1
        omq.block_step(dt_, x, y_t, W, theta, dtheta, m, v, step, slots[step - 1], ws)
    torch.cuda.synchronize()
    durs = timer.durations_ms()
    kinds = timer.kinds()
    work = timer.work()
    gemm_ms = sum(t for t, k in zip(durs, kinds) if k in (omq.TIMED_GEMM, omq.TIMED_GEMM_I8))
    # the fake quantizers of the forward: algorithmic HBM bytes per launch over its time
    hbm = {}
    for name, kind in (("weight_fake_quant", omq.TIMED_WEIGHT_QUANT),
                       ("act_quant", omq.TIMED_ACT_QUANT)):
        d_ = [t for t, k in zip(durs, kinds) if k == kind]
        b_ = [b for b, k in zip(work, kinds) if k == kind]
        if d_:
            gbs = sum(b_) / (sum(d_) * 1e-3) / 1e9
            hbm[name] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "launches": len(d_), "avg_launch_us": round(sum(d_) / len(d_) * 1e3, 2),
                         "bytes_per_launch": round(sum(b_) / len(b_)),
                         "share_of_step": round(sum(d_) / (ms * args.steps), 4)}
    # the bf16 matrix-core GEMMs (every backward product; the forward's too unless
    # it runs on integer codes) and the int8 code products, each against its peak
    bf_d = [t for t, k in zip(durs, kinds) if k == omq.TIMED_GEMM]
    i8_d = [t for t, k in zip(durs, kinds) if k == omq.TIMED_GEMM_I8]
    n_l = len(bf_d)
    avg_dur_s = sum(bf_d) / n_l / 1e3
    flops_per_launch = (timer.struct.flops - timer.struct.flops_codes) / n_l
    achieved = flops_per_launch / avg_dur_s / 1e12
    codes_roof = None
    if i8_d:
        i8_ops = timer.struct.flops_codes / len(i8_d)
        i8_avg_s = sum(i8_d) / len(i8_d) / 1e3
        codes_roof = {
            "kernel": "k_gemm_bf16<..., I8 = 1> (the forward's products on int8 codes)",
            "bound": "mfma", "achieved": round(i8_ops / i8_avg_s / 1e12, 2),
            "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
            "frac": round(i8_ops / i8_avg_s / 1e12 / PEAK_INT8_TOPS, 4),
            "launches": len(i8_d), "avg_launch_us": round(i8_avg_s * 1e6, 2),
            "share_of_step": round(sum(i8_d) / (ms * args.steps), 4)}
    sps = 1000.0 / ms
    tflops = step_flops(c) * sps / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(c, inp, min(args.cpu_tokens or c.T, c.T))

    out = {
        "metric": metric_of(c),
        "value": round(sps, 4),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "T": c.T, "d": c.d, "n_q": c.n_q, "n_kv": c.n_kv,
                   "head_dim": c.head_dim, "F": c.F, "wbits": c.wbits, "abits": c.abits,
                   "lwc_group": c.group or "per_channel",
                   "optimizer": "adamw", "parallelism": "none"},
        "tflops": round(tflops, 2),
        "step_tflop": round(step_flops(c) / 1e12, 4),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "fp_target_ms": round(fp_ms, 3),
        "loss_per_step": loss_curve,
        "loss_note": "the loss before each step's update, warm-up steps first, from the "
                     "initialization (logits 4, s 1, delta 0, s_a 1) on one repeated sample; "
                     "the oracle's own trajectory rises the same way after a few steps",
        "roofline": {
            "kernel": "k_gemm_bf16 (the bf16 matrix-core GEMM launches of the timed steps)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(args.workload),
            "launches": n_l,
            "avg_launch_us": round(avg_dur_s * 1e6, 2),
            "share_of_step": round(sum(bf_d) / (ms * args.steps), 4),
            "gemm_share_of_step": round(gemm_ms / (ms * args.steps), 4),
        },
        "roofline_codes": codes_roof,
        "roofline_hbm": hbm or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
