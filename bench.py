"""Benchmark: denoised tokens/s of the token-skipping denoising path on one MI355X.

Default workload: the LLaDA-8B-shaped stack (32 layers, d 4096, 32 heads x 128,
SwiGLU 12288, vocab 126464, bf16, random init N(0, 0.02)), batch 1, prompt 256,
generation 256 in semi-autoregressive blocks of 32 over 64 denoising
iterations, 4 tokens unmasked per iteration.  Iteration 0 runs every layer on
every position; iterations 1..63 run layers 0-3 on all positions and layers
4-31 on the top 25% (k = 128) by importance = 0.5 * conf + 0.5 * L1 change of
the hidden state entering layer 4 (Eq. 1), skipped rows reusing cached K/V.
One bench step = one whole generation (64 iterations); value = generated
tokens / second.

Prints ONE JSON line (rank 0, N = 1).  `roofline` describes the dominant
kernel -- the gate/up + SwiGLU product of the skipped layers (128 active rows),
timed live with HIP events bracketing each of its launches; `kernels` gives the
same for every kernel class of the skipped-regime iteration (its algorithmic
bytes and flops over its average launch time, against the HBM or bf16 MFMA
roof); `cpu_baseline` times the CPU oracle on a bounded sample (16 layers
over all rows and over the active rows, scoring and selection, the LM head)
and extrapolates to a generation.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

from synth import workloads  # noqa: E402
from token_skipping_denoise_amd import _ffi, api  # noqa: E402

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # timing-only events: no cache writeback/invalidate


class HipEvents:
    """Raw hipEvent_t pairs (created through the HIP runtime) for the library's timing hook.  They
    only time work and are read after a full device synchronisation, so they skip the
    system-scope fence that would otherwise add cache maintenance inside the bracket."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.n = n
        self.start = (ctypes.c_void_p * n)()
        self.stop = (ctypes.c_void_p * n)()
        for arr in (self.start, self.stop):
            for i in range(n):
                ev = ctypes.c_void_p()
                if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
                arr[i] = ev

    def elapsed_ms(self, count: int) -> list[float]:
        out = []
        for i in range(count):
            ms = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.stop[i]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        for arr in (self.start, self.stop):
            for i in range(self.n):
                self.hip.hipEventDestroy(arr[i])


def llada_generation(dims, k_sparse=128, boundary=4, steps=64, block=32, nested=()):
    """Per-iteration (cfg kwargs) of the semi-autoregressive early-skip generation; `nested` adds
    later layers that narrow the active set ((layer, k), ...), on every iteration (a full step
    fills their caches)."""
    per_block = steps // ((dims.S - dims.prompt) // block)
    out = []
    for t in range(steps):
        lo = dims.prompt + (t // per_block) * block
        if t == 0:
            out.append(dict(boundary_layer=boundary, full_step=True, score=None, unmask_n=4, block_lo=lo,
                            block_hi=lo + block, nested=nested))
        else:
            sc = api.score_cfg(alpha=0.5, conf_inverted=False, var=api.VAR_L1N, sel=api.SEL_TOPK, k=k_sparse)
            out.append(dict(boundary_layer=boundary, full_step=False, score=sc, unmask_n=4, block_lo=lo,
                            block_hi=lo + block, nested=nested))
    return out


def run_generation(model, state, tok0, plan, ws, timing=None):
    state.tokens.copy_(tok0)
    state.c.have_prev = 0
    state.c.bnd_cur = 0
    for kw in plan:
        api.skip_step(model, state, api.step_cfg(ws=ws, timing=timing, **kw))


def ffn_up_bytes(dims, rows: int) -> float:
    """Algorithmic HBM bytes of one gate/up + SwiGLU launch: weights + input rows + output rows."""
    e = 2
    return (2 * dims.d_ff * dims.d + rows * dims.d + rows * dims.d_ff) * e


def kernel_work(dims, rows: int):
    """Per kernel class: (timing class, rows filter, algorithmic bytes, flops) of one launch in an
    early-skip iteration with `rows` active rows.  Bytes count what the method itself must move
    (weights, input and output rows, caches it reads), not split-K partials or scratch."""
    e, B, S, d, F, V = 2, dims.B, dims.S, dims.d, dims.d_ff, dims.vocab
    hqd, hkvd = dims.n_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    nqkv = hqd + 2 * hkvd
    R = rows

    def gemm(n, k, out_e=e):
        return (n * k + R * k) * e + R * n * out_e, 2.0 * R * n * k

    return {
        "qkv": (_ffi.TK_QKV, R) + gemm(nqkv, d),
        "attention": (_ffi.TK_ATTN, R, (2 * R * hqd + 2 * B * S * hkvd) * e, 4.0 * R * S * hqd),
        "o_proj": (_ffi.TK_O, R) + gemm(d, hqd),
        "ffn_up_swiglu": (_ffi.TK_FFN_UP, R, ffn_up_bytes(dims, R), 2.0 * R * 2 * F * d),
        "ffn_down": (_ffi.TK_FFN_DOWN, R) + gemm(d, F),
        "lm_head": (_ffi.TK_LM_HEAD, R) + gemm(V, d, 4),
        "vocab_conf": (_ffi.TK_VOCAB, R, 4.0 * R * V, 0.0),
        "score": (_ffi.TK_SCORE, 0, 3.0 * B * S * d * e + 8.0 * B * S, 0.0),
        "select": (_ffi.TK_SELECT, 0, 4.0 * B * S + 8.0 * B * rows, 0.0),  # scores in; indices + row positions out
    }


def kernel_table(lib, model, state, tok0, plan, ws, dims, rows: int):
    """Time every kernel class with HIP events around its launches over one eager generation each
    and report its share of the HBM or MFMA roof."""
    work = kernel_work(dims, rows)
    cap = max(1, (len(plan) - 1) * dims.n_layers)
    ev = HipEvents(cap)
    out = []
    try:
        for name, (tk, max_rows, nbytes, flops) in work.items():
            timing = _ffi.Timing(tk, max_rows, ev.n, 0, ctypes.cast(ev.start, ctypes.POINTER(ctypes.c_void_p)),
                                 ctypes.cast(ev.stop, ctypes.POINTER(ctypes.c_void_p)))
            run_generation(model, state, tok0, plan, ws, timing)
            torch.cuda.synchronize()
            if timing.count == 0:
                continue
            durs = ev.elapsed_ms(timing.count)
            us = sum(durs) / len(durs) * 1e3
            gbps = nbytes / (us * 1e-6) / 1e9
            tflops = flops / (us * 1e-6) / 1e12
            ai = flops / nbytes if nbytes else 0.0
            if name == "select":
                bound, frac = "latency", None
            elif ai > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
                bound, frac = "mfma", tflops / BF16_PEAK_TFLOPS
            else:
                bound, frac = "hbm", gbps / HBM_PEAK_GBS
            out.append({"kernel": name, "launches": timing.count, "avg_us": round(us, 2), "bytes": int(nbytes),
                        "gbps": round(gbps, 1), "tflops": round(tflops, 2), "bound": bound,
                        "frac": None if frac is None else round(frac, 4)})
    finally:
        ev.close()
    return out


def cpu_baseline(model_w_gpu, dims, k_sparse, boundary, steps, sample_layers=16):
    """Time the oracle (float64 NumPy, bf16 storage rounding) on a bounded sample of the generation and
    extrapolate to one generation.  The sample: `sample_layers` layers, each run once over all rows (as in
    the full first iteration and the layers below the boundary) and once over the active rows (as in the
    skipped regime); the importance score and top-k selection; the LM head with the confidence pass over
    all rows and over the active rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import synth
    from oracle.importance import VAR_L1N, importance_score
    from oracle.numerics import store_fn
    from oracle.selection import select_topk
    from oracle.transformer import layer_rows, lm_logits
    from oracle.vocab import conf_kl

    store = store_fn("bf16")
    B, S, d = dims.B, dims.S, dims.d
    x = synth.normal(synth.seed_of(900), (B * S, d), 1.0, torch.bfloat16).double().numpy()
    xp = x + synth.normal(synth.seed_of(903), (B * S, d), 1e-3, torch.float32).double().numpy()
    kc = synth.normal(synth.seed_of(901), (B, S, dims.n_kv_heads, dims.head_dim), 1.0, torch.bfloat16).double().numpy()
    vc = synth.normal(synth.seed_of(902), (B, S, dims.n_kv_heads, dims.head_dim), 1.0, torch.bfloat16).double().numpy()
    conf = synth.uniform01(synth.seed_of(904), (B * S,)).double().numpy()
    rows_all = np.arange(B * S)
    n_layers = min(sample_layers, len(model_w_gpu["layers"]))

    t_dense, t_sparse = [], []
    for layer in range(n_layers):
        lw = {k: v.detach().to("cpu", torch.float64).numpy() for k, v in model_w_gpu["layers"][layer].items()}
        for rows, acc in ((rows_all, t_dense), (rows_all[:k_sparse], t_sparse)):
            t0 = time.perf_counter()
            layer_rows(lw, x[rows], rows % S, rows // S, kc, vc, n_heads=dims.n_heads, n_kv_heads=dims.n_kv_heads,
                       rope_base=1e4, eps=1e-5, store=store)
            acc.append(time.perf_counter() - t0)
        del lw
    t0 = time.perf_counter()
    for b in range(B):
        sc = importance_score(x[b * S:(b + 1) * S], xp[b * S:(b + 1) * S], conf[b * S:(b + 1) * S], None,
                              alpha=0.5, var=VAR_L1N, conf_inverted=False)
        select_topk(sc, np.zeros(S, dtype=np.uint8), k_sparse)
    t_score = time.perf_counter() - t0
    head = model_w_gpu["lm_head"].detach().to("cpu", torch.float64).numpy()
    g = model_w_gpu["final_norm"].detach().to("cpu", torch.float64).numpy()
    t_head = []
    for rows in (rows_all, rows_all[:k_sparse]):
        t0 = time.perf_counter()
        conf_kl(lm_logits(x[rows], g, head, 1e-5, store), None, dims.mask_id)
        t_head.append(time.perf_counter() - t0)
    del head
    L = dims.n_layers
    td, ts = sum(t_dense) / len(t_dense), sum(t_sparse) / len(t_sparse)
    t_sample = sum(t_dense) + sum(t_sparse) + t_score + sum(t_head)
    t_gen = (L * td + t_head[0]) + (steps - 1) * (boundary * td + (L - boundary) * ts + t_score + t_head[1])
    n_threads = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"), default=1)
    gen_tokens = B * (S - dims.prompt)
    # the same oracle on one BLAS thread: one layer over all rows and over the active rows, and the
    # LM head + confidence pass over the active rows, extrapolated the same way
    from threadpoolctl import threadpool_limits
    lw = {k: v.detach().to("cpu", torch.float64).numpy() for k, v in model_w_gpu["layers"][0].items()}
    head = model_w_gpu["lm_head"].detach().to("cpu", torch.float64).numpy()
    with threadpool_limits(limits=1, user_api="blas"):
        t1 = []
        for rows in (rows_all, rows_all[:k_sparse]):
            t0 = time.perf_counter()
            layer_rows(lw, x[rows], rows % S, rows // S, kc, vc, n_heads=dims.n_heads, n_kv_heads=dims.n_kv_heads,
                       rope_base=1e4, eps=1e-5, store=store)
            t1.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        conf_kl(lm_logits(x[rows_all[:k_sparse]], g, head, 1e-5, store), None, dims.mask_id)
        t_head1 = time.perf_counter() - t0
    del lw, head
    th1_dense = t_head1 * (t_head[0] / t_head[1])   # the LM head scales with rows like the threaded one
    t_gen1 = (L * t1[0] + th1_dense) + (steps - 1) * (boundary * t1[0] + (L - boundary) * t1[1] + t_score + t_head1)
    single = {"value": gen_tokens / t_gen1, "cores": 1,
              "sample": (f"one BLAS thread: one layer over {B * S} rows ({t1[0]:.2f} s) and over {k_sparse} rows "
                         f"({t1[1]:.2f} s), LM head + confidence over {k_sparse} rows ({t_head1:.2f} s); extrapolated "
                         f"to one generation ({t_gen1:.0f} s)")}
    return {
        "value": gen_tokens / t_gen,
        "unit": "tokens/s",
        "cores": int(n_threads),
        "kind": "oracle",
        "sample": (f"oracle (float64 NumPy, bf16 storage rounding) timed for {t_sample:.1f} s: layers 0-{n_layers - 1} "
                   f"each over all {B * S} rows ({td:.2f} s/layer) and over {k_sparse} active rows ({ts:.2f} s/layer), "
                   f"importance score + top-{k_sparse} ({t_score:.2f} s), LM head + confidence over {B * S} rows "
                   f"({t_head[0]:.2f} s) and {k_sparse} rows ({t_head[1]:.2f} s); extrapolated to one "
                   f"{steps}-iteration generation ({t_gen:.0f} s); {n_threads} BLAS threads, "
                   f"os.cpu_count()={os.cpu_count()}"),
        "single_thread": single,
    }


def measured_peaks():
    """The measured denominators: the library's nontemporal read probe over 2 GiB (the way the
    products stream their weights), its device-copy probe (HBM read + write) and its MFMA-loop probe
    (bf16 32x32x16 MFMAs on register operands, 8 workgroups of 4 waves per CU)."""
    lib = _ffi.load()
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    work = ctypes.c_double()

    def rate(kind, iters):
        if lib.dllm_peak_probe(kind, buf.data_ptr(), buf.numel(), 1, ctypes.byref(work), stream) != 0:
            raise RuntimeError("dllm_peak_probe failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        lib.dllm_peak_probe(kind, buf.data_ptr(), buf.numel(), iters, ctypes.byref(work), stream)
        e1.record()
        torch.cuda.synchronize()
        return work.value / (e0.elapsed_time(e1) * 1e-3)

    read = rate(2, 5)
    copy = rate(0, 5)
    mfma = rate(1, 4000)
    del buf
    torch.cuda.empty_cache()
    return {"read_gbps": round(read / 1e9, 1), "read_frac_of_datasheet": round(read / 1e9 / HBM_PEAK_GBS, 4),
            "copy_gbps": round(copy / 1e9, 1), "copy_frac_of_datasheet": round(copy / 1e9 / HBM_PEAK_GBS, 4),
            "bf16_mfma_tflops": round(mfma / 1e12, 1),
            "bf16_mfma_frac_of_datasheet": round(mfma / 1e12 / BF16_PEAK_TFLOPS, 4),
            "how": "dllm_peak_probe: nontemporal read of 2 GiB x5; copy of 1 GiB into 1 GiB x5 (bytes read + "
                   "written); MFMA loop 2048 workgroups x 4 waves x 4 chains x 4000 steps; HIP events on the "
                   "launch stream. HBM-bound kernels are compared with the read rate (their traffic is reads)"}


def c2_layer_kernels(n_copies=6, k=64, reps=3):
    """One LLaDA-8B-shaped layer (d 4096, 32 heads, F 12288, S 512) with 64 of 512 rows active: the
    score, select and a5-a10 kernels of a step whose boundary is that layer, timed with HIP events
    around each launch.  n_copies distinct weight sets (0.74 GB each with the packed copies) are
    used in turn, so the 256 MB memory-side cache does not hold the weights between launches."""
    import synth
    dev = "cuda:0"
    dims = workloads.shrink(workloads.LLADA, n_layers=1, vocab=1024)
    B, S = dims.B, dims.S
    models, states, wss = [], [], []
    for c in range(n_copies):
        w = workloads.model_weights(dims, device=dev, seed_base=200 + c)
        m = api.Model(w, dims.n_heads, dims.n_kv_heads, dims.mask_id)
        tok = workloads.initial_tokens(dims, device=dev)
        st = api.State(m, tok, k_max=k)
        ws = api.alloc_workspace(m, B, S, k)
        api.skip_step(m, st, api.step_cfg(0, True, ws=ws))
        models.append(m)
        states.append(st)
        wss.append(ws)
    conf = synth.uniform01(synth.seed_of(2, 104), (B, S)).to(dev)
    sc = api.score_cfg(alpha=0.5, var=api.VAR_L1N, sel=api.SEL_TOPK, k=k)
    out = {}
    work = kernel_work(dims, k)
    n = n_copies * reps
    for name, (tk, _, nbytes, flops) in work.items():
        if name in ("lm_head", "vocab_conf"):
            continue
        ev = HipEvents(n + 1)
        timing = _ffi.Timing(tk, 0, ev.n, 0, ctypes.cast(ev.start, ctypes.POINTER(ctypes.c_void_p)),
                             ctypes.cast(ev.stop, ctypes.POINTER(ctypes.c_void_p)))
        for r in range(reps):
            for c in range(n_copies):
                states[c].conf.copy_(conf)
                states[c].tokens[:, 300 + r] = 7 + r   # a changed token, so the boundary state moves
                api.skip_step(models[c], states[c], api.step_cfg(0, False, sc, ws=wss[c], timing=timing))
        torch.cuda.synchronize()
        durs = ev.elapsed_ms(timing.count)
        ev.close()
        us = sorted(durs)[len(durs) // 2] * 1e3
        gbps = nbytes / (us * 1e-6) / 1e9
        out[name] = {"median_us": round(us, 2), "bytes": int(nbytes), "gbps": round(gbps, 1),
                     "frac_hbm": None if name == "select" else round(gbps / HBM_PEAK_GBS, 4)}
    # the whole step (embed, score, select, gather, the layer, a 1024-token LM head) per copy in turn
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for c in range(n_copies):
        api.skip_step(models[c], states[c], api.step_cfg(0, False, sc, ws=wss[c]))
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / n_copies
    del models, states, wss
    torch.cuda.empty_cache()
    return {"rows": k, "kernels": out, "step_us": round(step_us, 1),
            "layer_floor_us": round(2 * 218.1e6 / (HBM_PEAK_GBS * 1e9) * 1e6, 1),
            "how": (f"{n_copies} weight copies in turn ({reps} sparse steps each, median launch); the step also holds "
                    "the embedding of 512 rows and a 1024-token LM head")}


def profile_layer(which: str, calls: int):
    """A short program for counter collection: one layer of the given shape called ``calls`` times
    through dllm_layer_sparse, printing a line after each call.  ``llada128``: the LLaDA-8B layer
    (S 512) with 128 active rows, the skipped-regime shape of the default workload; ``llada512``:
    the same layer over all 512 rows (the dense layers); ``long205``: the long-context layer
    (batch 4, S 4096) with 205 active rows per sequence; ``dream1024``: one Dream-7B-shaped layer
    (batch 8, S 1024, GQA 28/4) over every row, the many-row regime of the lock ramp's first
    steps; ``step128``: whole sparse iterations of a one-layer model, for the scoring and
    selection kernels."""
    import synth
    dev = "cuda:0"
    if which == "step128":
        # sparse iterations of a one-layer LLaDA-8B-shaped model (1024-token vocabulary) with the
        # boundary at layer 0 and k = 128: the importance score and the selection at S = 512
        dims = workloads.shrink(workloads.LLADA, n_layers=1, vocab=1024)
        w = workloads.model_weights(dims, device=dev, seed_base=200)
        m = api.Model(w, dims.n_heads, dims.n_kv_heads, dims.mask_id)
        st = api.State(m, workloads.initial_tokens(dims, device=dev), k_max=128)
        ws = api.alloc_workspace(m, dims.B, dims.S, 128)
        api.skip_step(m, st, api.step_cfg(0, True, ws=ws))
        conf = synth.uniform01(synth.seed_of(2, 104), (dims.B, dims.S)).to(dev)
        sc = api.score_cfg(alpha=0.5, var=api.VAR_L1N, sel=api.SEL_TOPK, k=128)
        torch.cuda.synchronize()
        print(f"profile-layer {which}: B {dims.B} S {dims.S} k 128", flush=True)
        for i in range(calls):
            st.conf.copy_(conf)
            st.tokens[:, 300 + i % 64] = 7 + i   # a changed token, so the boundary state moves
            api.skip_step(m, st, api.step_cfg(0, False, sc, ws=ws))
            torch.cuda.synchronize()
            print(f"call {i + 1}/{calls} done", flush=True)
        return
    if which == "llada128":
        dims, n_act = workloads.LLADA_LAYER, [128]
    elif which == "llada512":
        dims, n_act = workloads.LLADA_LAYER, [512]
    elif which == "dream1024":
        dims = workloads.shrink(workloads.DREAM, n_layers=1)
        n_act = [dims.S] * dims.B
    else:
        dims, n_act = workloads.shrink(workloads.LLADA_LONG, n_layers=1), [205] * 4
    B, S, d = dims.B, dims.S, dims.d
    k_max = max(n_act)
    lw = workloads.layer_weights(dims, 0, device=dev)
    small = torch.zeros((8, d), dtype=torch.bfloat16, device=dev)
    model = api.Model({"embed": small, "final_norm": torch.ones(d, dtype=torch.bfloat16, device=dev),
                       "lm_head": small, "layers": [lw]}, dims.n_heads, dims.n_kv_heads, 7)
    kv = (B, S, dims.n_kv_heads, dims.head_dim)
    kc = synth.normal(synth.seed_of(dims.cfg_id, 1), kv, 1.0, torch.bfloat16).to(dev)
    vc = synth.normal(synth.seed_of(dims.cfg_id, 2), kv, 1.0, torch.bfloat16).to(dev)
    x0 = synth.normal(synth.seed_of(dims.cfg_id, 3), (B * k_max, d), 1.0, torch.bfloat16).to(dev)
    idx = torch.full((B, k_max), -1, dtype=torch.int32)
    for b in range(B):
        rows = synth.permutation(synth.seed_of(dims.cfg_id, 4, b), S)[:n_act[b]]
        idx[b, :n_act[b]] = torch.sort(rows).values.to(torch.int32)
    idx, nact = idx.to(dev), torch.tensor(n_act, dtype=torch.int32, device=dev)
    ws = api.alloc_workspace(model, B, S, k_max)
    torch.cuda.synchronize()
    print(f"profile-layer {which}: B {B} S {S} active {n_act}", flush=True)
    for i in range(calls):
        x = x0.clone()
        api.layer_sparse(model, 0, x, idx, nact, kc, vc, ws)
        torch.cuda.synchronize()
        print(f"call {i + 1}/{calls} done", flush=True)


DOMINANT_KERNEL = "dllm::(anonymous namespace)::k_gemm_packed<3, 64, 2>"
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_packed_swiglu_llada_128rows_hbm_bytes.md")
GEMM_SOURCE = os.path.join(ROOT, "token_skipping_denoise_amd", "csrc", "gemm_packed.hip")


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from its committed counter summary, or None when the
    summary is missing or was taken from a different kernel source."""
    import hashlib
    import re

    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch:\s*(\d+)\s+gemm_source_sha256:\s*([0-9a-f]{64})", text)
    if not m:
        return None
    with open(GEMM_SOURCE, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != m.group(2):
            return None
    return int(m.group(1))


def n_dus_rounds(block: int, a: int = 2) -> int:
    """Rounds of a dilated block (DUS summary, technical summary section 2): R = ceil(log_a block)."""
    R, p = 0, 1
    while p < block:
        p *= a
        R += 1
    return max(R, 1)


def dream_schedule(dims, device, n_steps=128, unmask=4, lock_max=0.8):
    """SureLock-style run on the Dream-7B shapes: step 0 full, then every unlocked row is recomputed
    (layers from 0, locked rows skip everything but stay attendable).  Random weights give
    near-uniform posteriors that never lock by themselves, so a seeded per-sequence permutation
    locks a growing share of all positions, f_t = lock_max * t / (n_steps - 1); the KL lock rule
    stays active on top.  Four positions of the generated half are unmasked per step by confidence."""
    import synth

    perms = [synth.permutation(synth.seed_of(dims.cfg_id, 30_000, b), dims.S) for b in range(dims.B)]
    lo, hi = dims.prompt, dims.S
    steps = []
    for t in range(n_steps):
        n = int(round(lock_max * t / (n_steps - 1) * dims.S))
        force = torch.zeros((dims.B, dims.S), dtype=torch.uint8)
        for b in range(dims.B):
            force[b, perms[b][:n]] = api.FORCE_EXCLUDED
        if t == 0:
            kw = dict(boundary_layer=0, full_step=True, score=None)
        else:
            kw = dict(boundary_layer=0, full_step=False,
                      score=api.score_cfg(alpha=0.0, var=api.VAR_NONE, sel=api.SEL_UNLOCKED, k=dims.S))
        kw.update(lock_kl_eps=1e-3, lock_conf_min=0.9, unmask_n=unmask, block_lo=lo, block_hi=hi)
        steps.append((kw, force.to(device), None))
    return steps


def long_schedule(dims, device, k_active=205, block=16, refresh_every=16):
    """Long-context run on the LLaDA-8B shapes with a dilated schedule: the generated half is cut
    into blocks of 16 decoded in ceil(log2 16) = 4 rounds (stride 8, 4, 2, 1); every step unmasks
    exactly the round's planned positions, which the library marks on the device
    (dllm_dus_mark).  Every 16th step refreshes everything (prompt included); the others
    recompute the planned positions plus the response rows whose hidden state at layer 0
    changed most (1 - cos), k_active = 5% of S rows per sequence in all."""
    n_rounds = n_dus_rounds(block)
    n_blocks = (dims.S - dims.prompt) // block
    base = torch.zeros((dims.B, dims.S), dtype=torch.uint8)
    base[:, :dims.prompt] = api.FORCE_EXCLUDED
    base = base.to(device)
    steps = []
    t = 0
    for blk in range(n_blocks):
        lo = dims.prompt + blk * block
        for r in range(n_rounds):
            if t % refresh_every == 0:
                kw = dict(boundary_layer=0, full_step=True, score=None)
            else:
                kw = dict(boundary_layer=0, full_step=False,
                          score=api.score_cfg(alpha=0.0, var=api.VAR_COS, sel=api.SEL_TOPK, k=k_active))
            kw.update(unmask_n=1, block_lo=lo, block_hi=lo + block, unmask_mode=api.UNMASK_FORCED)
            steps.append((kw, base, (lo, block, r)))
            t += 1
    return steps


def dcache_schedule(dims, device, k_active=64, refresh_every=16, block=32, unmask=4, feature="hidden"):
    """Per-layer cache run on the LLaDA-8B shapes (dLLM-Cache summary section 3): every 16th step
    is a full step that refreshes every layer's caches (prompt included); the others lock the
    prompt rows (long-interval prompt cache) and, at every layer, recompute the k_active = 25% of
    the 256 response rows whose hidden state entering the layer changed most (1 - cos) since
    they were last computed there, the rest taking their cached layer outputs.  Blocks of 32
    generated positions, four unmasked per step by confidence, 64 steps."""
    base = torch.zeros((dims.B, dims.S), dtype=torch.uint8)
    base[:, :dims.prompt] = api.FORCE_EXCLUDED
    base = base.to(device)
    n_steps = (dims.S - dims.prompt) // unmask
    per_block = block // unmask
    steps = []
    for t in range(n_steps):
        lo = dims.prompt + (t // per_block) * block
        if t % refresh_every == 0:
            kw = dict(boundary_layer=0, full_step=True, score=None)
        else:
            kw = dict(boundary_layer=0, full_step=False,
                      score=api.score_cfg(alpha=0.0, var=api.VAR_COS, sel=api.SEL_TOPK, k=k_active))
        kw.update(unmask_n=unmask, block_lo=lo, block_hi=lo + block, layer_cache=feature)
        steps.append((kw, base, None))
    return steps


def run_schedule(model, state, tok0, steps, ws, after_step=None, timing=None):
    state.tokens.copy_(tok0)
    state.c.have_prev = 0
    state.c.bnd_cur = 0
    if state.force is not None:
        state.force.zero_()
    for kw, force, plan in steps:
        if plan is not None:
            # a fresh base (prompt excluded), then this round's positions marked on the device
            state.force.copy_(force)
            api.dus_mark(state.force, plan[0], plan[1], plan[2])
        else:
            # the schedule's marks; rows the lock rule has already locked stay locked
            torch.maximum(state.force, force, out=state.force)
        api.skip_step(model, state, api.step_cfg(ws=ws, timing=timing, **kw))
        if after_step is not None:
            after_step(kw)


def vocab_pass_stats(model, state, tok0, steps, ws, dims, state_bytes):
    """Times the confidence/KL vocabulary pass over one run of the schedule.  Its algorithmic
    bytes per live row are 4 V (fp32 logits read) + 2 V state_bytes (previous logits read and
    rewritten); live rows are all B*S on a full step, else the selected ones."""
    ev = HipEvents(len(steps) + 1)
    rows = []

    def count_rows(kw):
        if kw.get("full_step"):
            rows.append(dims.B * dims.S)
        else:
            rows.append(int(state.n_active.sum()))

    timing = _ffi.Timing(_ffi.TK_VOCAB, 0, ev.n, 0, ctypes.cast(ev.start, ctypes.POINTER(ctypes.c_void_p)),
                         ctypes.cast(ev.stop, ctypes.POINTER(ctypes.c_void_p)))
    run_schedule(model, state, tok0, steps, ws, after_step=count_rows, timing=timing)
    torch.cuda.synchronize()
    n = timing.count
    durs = ev.elapsed_ms(n)
    ev.close()
    per_row = (4.0 + 2.0 * state_bytes) * dims.vocab
    total_bytes = per_row * sum(rows[:n])
    total_us = sum(durs) * 1e3
    gbps = total_bytes / (total_us * 1e-6) / 1e9
    return {"kernel": "vocab_conf_kl", "launches": n, "avg_us": round(total_us / max(n, 1), 2),
            "live_rows": int(sum(rows[:n])), "bytes_per_row": int(per_row), "bytes": int(total_bytes),
            "gbps": round(gbps, 1), "bound": "hbm", "frac": round(gbps / HBM_PEAK_GBS, 4)}


WORKLOAD_DESC = {
    "dream": ("Dream-7B-shaped 28-layer GQA 28/4 run, batch 8, prompt 512 + gen 512, 128 steps, locked share "
              "ramped 0 -> 80% of positions (seeded), unlocked rows recomputed, KL lock rule on"),
    "dcache": ("LLaDA-8B-shaped 32-layer per-layer cache run, batch 1, prompt 256 + gen 256, blocks of 32, 64 steps: "
               "full refresh every 16 steps, else prompt rows cached and at every layer the 64 response rows "
               "(25%) with the largest feature change (1 - cos) recomputed, the rest reusing cached outputs"),
    "long": ("LLaDA-8B-shaped 32-layer long-context run, batch 4, prompt 3584 + gen 512, dilated blocks of 16 "
             "(4 rounds), 128 steps, refresh every 16 steps, else 205 active rows (5%)"),
}


def many_row_gemm_stats(model, state, tok0, steps, ws, dims, tk, n_out, k_in):
    """A many-row product (timing class tk, n_out x k_in weights) over one run of the schedule: flops
    counted on the live rows of each step (all B*S on a full step, else the active rows), against the
    bf16 MFMA roof."""
    ev = HipEvents(len(steps) * dims.n_layers + 1)
    rows = []

    def count_rows(kw):
        rows.append(dims.B * dims.S if kw.get("full_step") else int(state.n_active.sum()))

    timing = _ffi.Timing(tk, 0, ev.n, 0, ctypes.cast(ev.start, ctypes.POINTER(ctypes.c_void_p)),
                         ctypes.cast(ev.stop, ctypes.POINTER(ctypes.c_void_p)))
    run_schedule(model, state, tok0, steps, ws, after_step=count_rows, timing=timing)
    torch.cuda.synchronize()
    durs = ev.elapsed_ms(timing.count)
    ev.close()
    per_step = timing.count // len(steps)
    flops = sum(2.0 * r * n_out * k_in * per_step for r in rows)
    total_us = sum(durs) * 1e3
    tflops = flops / (total_us * 1e-6) / 1e12
    return {"launches": timing.count, "avg_us": round(total_us / max(timing.count, 1), 2),
            "live_rows_per_step": [min(rows), max(rows)], "tflops": round(tflops, 1), "bound": "mfma",
            "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}


def oracle_rows_per_s(dims, n_rows, seed=950):
    """Oracle rows-per-second of one layer at these shapes (a sample of n_rows rows of one sequence
    over a full-length cache) and of the LM head + confidence pass; used to extrapolate a run."""
    import numpy as np

    import synth
    from oracle.numerics import store_fn
    from oracle.transformer import layer_rows, lm_logits
    from oracle.vocab import conf_kl

    store = store_fn("bf16")
    lw = {k: v.to(torch.float64).numpy() for k, v in workloads.layer_weights(dims, 0).items()}
    x = synth.normal(synth.seed_of(seed), (n_rows, dims.d), 1.0, torch.bfloat16).double().numpy()
    kc = synth.normal(synth.seed_of(seed, 1), (1, dims.S, dims.n_kv_heads, dims.head_dim), 1.0,
                      torch.bfloat16).double().numpy()
    vc = kc.copy()
    pos = np.arange(n_rows) * (dims.S // n_rows)
    t0 = time.perf_counter()
    layer_rows(lw, x, pos, np.zeros(n_rows, dtype=np.int64), kc, vc, n_heads=dims.n_heads,
               n_kv_heads=dims.n_kv_heads, rope_base=1e4, eps=1e-5, store=store)
    t_layer = time.perf_counter() - t0
    del lw
    head = synth.normal(synth.seed_of(seed, 2), (dims.vocab, dims.d), 0.02, torch.bfloat16).double().numpy()
    t0 = time.perf_counter()
    conf_kl(lm_logits(x, np.ones(dims.d), head, 1e-5, store), None, dims.vocab - 1)
    t_head = time.perf_counter() - t0
    return n_rows / t_layer, n_rows / t_head, t_layer + t_head


def run_workload(name, kl_state="f32", steps=1, warmup=1, kernel_timing=True, cache_feature="hidden"):
    """Dream-GQA lock ramp, long-context dilated run or per-layer cache run; eager launches (the steps
    are long enough that launch overhead is noise).  Returns the result dict."""
    dev = "cuda:0"
    if name == "dream":
        dims, k_max = workloads.DREAM, workloads.DREAM.S
    elif name == "dcache":
        dims, k_max = workloads.LLADA, 64
    else:
        dims, k_max = workloads.LLADA_LONG, 205
    t0 = time.perf_counter()
    w = workloads.model_weights(dims, device=dev)
    model = api.Model(w, dims.n_heads, dims.n_kv_heads, dims.mask_id)
    tok0 = workloads.initial_tokens(dims, device=dev)
    track_kl = name == "dream"
    state = api.State(model, tok0.clone(), k_max=k_max, track_kl=track_kl, kl_state=kl_state,
                      layer_cache=name == "dcache")
    ws = api.alloc_workspace(model, dims.B, dims.S, k_max)
    if name == "dream":
        sched = dream_schedule(dims, dev)
    elif name == "dcache":
        sched = dcache_schedule(dims, dev, k_active=k_max, feature=cache_feature)
    else:
        sched = long_schedule(dims, dev)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t0
    for _ in range(warmup):
        run_schedule(model, state, tok0, sched, ws)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps):
        run_schedule(model, state, tok0, sched, ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    gen_tokens = dims.B * (dims.S - dims.prompt)
    kernels = None
    if kernel_timing and name in ("long", "dcache"):
        kernels = kernel_table_schedule(model, state, tok0, sched, ws, dims, dims.B * k_max,
                                        only=("attention", "qkv", "ffn_up_swiglu") if name == "long" else None)
    elif kernel_timing and name == "dream":
        kernels = [vocab_pass_stats(model, state, tok0, sched, ws, dims, 2 if kl_state == "bf16" else 4)]
        kernels.append({"kernel": "ffn_up_swiglu (many rows)",
                        **many_row_gemm_stats(model, state, tok0, sched, ws, dims, _ffi.TK_FFN_UP, 2 * dims.d_ff,
                                              dims.d)})
    rows_per_step = [dims.B * dims.S if kw.get("full_step") else None for kw, _, _ in sched]
    del state, ws, model, w
    torch.cuda.empty_cache()
    return {
        "metric": "denoised tokens/s at 8B shapes on 1 MI355X",
        "value": round(gen_tokens * steps / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(elapsed / steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights N(0,0.02); prompt tokens uniform)",
        "config": {"workload": WORKLOAD_DESC[name], "batch": dims.B, "seq_len": dims.S, "layers": dims.n_layers,
                   "hidden": dims.d, "vocab": dims.vocab, "iterations_per_step": len(sched),
                   "setup_s": round(t_setup, 1), "launch": "eager",
                   "kl_state": kl_state if track_kl else None,
                   "layer_cache_feature": cache_feature if name == "dcache" else None},
        "kernels": kernels,
        "_full_steps": sum(1 for r in rows_per_step if r is not None),
    }


def workload_cpu_baseline(name, result):
    """The oracle's time for the run, extrapolated from one layer over a sample of rows and the LM
    head over the same rows (labelled as extrapolated): a full step computes every row of every
    layer, a sparse step the active rows (long context: 205 of each sequence; Dream: the unlocked
    rows of the ramp, 0.6 of all on average)."""
    dims = workloads.DREAM if name == "dream" else workloads.LLADA_LONG
    n_sample = 128 if name == "dream" else 64
    layer_rps, head_rps, t_sample = oracle_rows_per_s(dims, n_sample)
    n_steps = result["config"]["iterations_per_step"]
    n_full = result["_full_steps"]
    all_rows = dims.B * dims.S
    if name == "dream":
        sparse_rows = 0.6 * all_rows          # the locked share ramps 0 -> 0.8 linearly
    else:
        sparse_rows = dims.B * 205
    t_gen = (n_full * all_rows + (n_steps - n_full) * sparse_rows) * (dims.n_layers / layer_rps + 1.0 / head_rps)
    gen_tokens = dims.B * (dims.S - dims.prompt)
    return {"value": gen_tokens / t_gen, "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": (f"oracle (float64 NumPy, bf16 storage) timed for {t_sample:.1f} s: one layer over {n_sample} rows "
                       f"of one sequence against a {dims.S}-position cache ({layer_rps:.0f} rows/s) and the LM head + "
                       f"confidence over them ({head_rps:.0f} rows/s); extrapolated linearly in rows to the run's "
                       f"{n_full} full and {n_steps - n_full} sparse steps ({t_gen:.0f} s)")}


def _blas_threads():
    from threadpoolctl import threadpool_info
    return int(max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"), default=1))


def extra_workload(args):
    """One JSON line for --workload dream / long / dcache (dcache: the chosen feature, and the other
    feature's run beside it)."""
    res = run_workload(args.workload, args.kl_state, args.steps, args.warmup, not args.no_kernel_timing,
                       args.cache_feature)
    res.pop("_full_steps")
    if args.workload == "dcache":
        other = "value" if args.cache_feature == "hidden" else "hidden"
        alt = run_workload("dcache", args.kl_state, args.steps, args.warmup, not args.no_kernel_timing, other)
        res["other_feature"] = {"layer_cache_feature": other, "value": alt["value"], "ms_per_step": alt["ms_per_step"],
                                "kernels": alt["kernels"]}
    print(json.dumps(res), flush=True)


def kernel_table_schedule(model, state, tok0, steps, ws, dims, rows, only=None):
    """kernel_table for an explicit schedule: rows = the padded active rows of a sparse step."""
    work = kernel_work(dims, rows)
    cap = max(1, len(steps) * dims.n_layers)
    ev = HipEvents(cap)
    out = []
    try:
        for name, (tk, max_rows, nbytes, flops) in work.items():
            if name in ("score", "select") or (only is not None and name not in only):
                continue
            timing = _ffi.Timing(tk, max_rows, ev.n, 0, ctypes.cast(ev.start, ctypes.POINTER(ctypes.c_void_p)),
                                 ctypes.cast(ev.stop, ctypes.POINTER(ctypes.c_void_p)))
            run_schedule(model, state, tok0, steps, ws, timing=timing)
            torch.cuda.synchronize()
            if timing.count == 0:
                continue
            durs = ev.elapsed_ms(timing.count)
            us = sum(durs) / len(durs) * 1e3
            gbps = nbytes / (us * 1e-6) / 1e9
            tflops = flops / (us * 1e-6) / 1e12
            ai = flops / nbytes if nbytes else 0.0
            if ai > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
                bound, frac = "mfma", tflops / BF16_PEAK_TFLOPS
            else:
                bound, frac = "hbm", gbps / HBM_PEAK_GBS
            out.append({"kernel": name, "launches": timing.count, "avg_us": round(us, 2), "bytes": int(nbytes),
                        "gbps": round(gbps, 1), "tflops": round(tflops, 2), "bound": bound, "frac": round(frac, 4)})
    finally:
        ev.close()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3, help="timed generations")
    ap.add_argument("--warmup", type=int, default=1, help="untimed generations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--workload", choices=("llada", "dream", "long", "dcache"), default="llada",
                    help="llada: the 32-layer early-skip generation (default); dream: Dream-GQA lock ramp; "
                         "long: long-context dilated run; dcache: per-layer cache (dLLM-Cache) run")
    ap.add_argument("--nested", default="",
                    help="llada workload: nested boundaries 'layer:k[,layer:k]' that narrow the 128 active rows "
                         "at later layers (ES-dLLM per-layer selection), e.g. 16:64")
    ap.add_argument("--kl-state", choices=("f32", "bf16"), default="f32",
                    help="precision of the previous logits the KL lock rule compares against (dream workload)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy a 1 GiB buffer once (reference for the HBM byte counters) and exit")
    ap.add_argument("--cache-feature", choices=("hidden", "value"), default="hidden",
                    help="dcache workload: the feature a cached layer compares (its input, or its V projection)")
    ap.add_argument("--profile-layer", choices=("llada128", "llada512", "long205", "dream1024", "step128"), default=None,
                    help="only call one layer of that shape --steps times, a line per call (a short "
                         "program for counter collection), and exit")
    ap.add_argument("--no-extra", action="store_true",
                    help="llada workload: skip the extra measurements (measured peaks, the one-layer kernel "
                         "latencies, the Dream lock-ramp and long-context runs)")
    args = ap.parse_args()
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n}))
        return
    if args.profile_layer:
        profile_layer(args.profile_layer, args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(sequences shard with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.workload != "llada":
        extra_workload(args)
        return

    dims = workloads.LLADA
    dev = "cuda:0"
    k_sparse, boundary, n_iter = 128, 4, 64
    t0 = time.perf_counter()
    w = workloads.model_weights(dims, device=dev)
    model = api.Model(w, dims.n_heads, dims.n_kv_heads, dims.mask_id)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t0
    tok0 = workloads.initial_tokens(dims, device=dev)
    nested = tuple(tuple(int(v) for v in item.split(":")) for item in args.nested.split(",")) if args.nested else ()
    state = api.State(model, tok0.clone(), k_max=k_sparse, track_kl=False, n_nested=len(nested))
    ws = api.alloc_workspace(model, dims.B, dims.S, k_sparse)
    plan = llada_generation(dims, k_sparse, boundary, n_iter, nested=nested)

    # one eager generation first (first-touch of every buffer and kernel)
    run_generation(model, state, tok0, plan, ws)
    torch.cuda.synchronize()

    lib = _ffi.load()
    n_launch = (n_iter - 1) * (dims.n_layers - boundary)
    timing = None
    events = None
    if not args.no_kernel_timing:
        events = HipEvents(n_launch * args.steps if args.no_graph else n_launch)
        timing = _ffi.Timing(_ffi.TK_FFN_UP, k_sparse * dims.B, events.n, 0,
                             ctypes.cast(events.start, ctypes.POINTER(ctypes.c_void_p)),
                             ctypes.cast(events.stop, ctypes.POINTER(ctypes.c_void_p)))

    graph = None
    if not args.no_graph:
        # The whole generation (token reset + 64 iterations) is captured once and replayed:
        # the same kernels in the same order, without per-launch host overhead.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_generation(model, state, tok0, plan, ws)
        for _ in range(args.warmup):
            graph.replay()
    else:
        for _ in range(args.warmup):
            run_generation(model, state, tok0, plan, ws)
    torch.cuda.synchronize()

    t_start = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            run_generation(model, state, tok0, plan, ws, timing)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    if timing is not None and graph is not None:
        # Event records cannot be replayed from a captured graph: the dominant kernel is
        # timed over one eager generation issued right after the timed replays (same
        # kernels, same shapes, same stream).
        run_generation(model, state, tok0, plan, ws, timing)
        torch.cuda.synchronize()

    gen_tokens = dims.B * (dims.S - dims.prompt)
    value = gen_tokens * args.steps / elapsed
    roofline = None
    if timing is not None and timing.count > 0:
        durs = events.elapsed_ms(timing.count)
        avg_ms = sum(durs) / len(durs)
        bytes_per = ffn_up_bytes(dims, k_sparse * dims.B)
        achieved = bytes_per / (avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                    "kernel": DOMINANT_KERNEL + " (gate/up + SwiGLU of a skipped-regime layer, 128 active rows, "
                              "fragment-packed weights)",
                    "launches": timing.count, "avg_us": round(avg_ms * 1e3, 2),
                    "timed_in": ("eager generation right after the timed graph replays" if graph is not None
                                 else "timed region"),
                    "bytes_per_launch": int(bytes_per)}
        events.close()

    kernels = None
    if not args.no_kernel_timing:
        kernels = kernel_table(lib, model, state, tok0, plan, ws, dims, k_sparse * dims.B)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, dims, k_sparse, boundary, n_iter)

    line = {
        "metric": "denoised tokens/s at 8B shapes on 1 MI355X",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights N(0,0.02); prompt tokens uniform)",
        "config": {"workload": "LLaDA-8B-shaped 32-layer early-skip generation (prompt 256 + gen 256, blocks of 32, "
                               "64 iterations, layers 4-31 on top-128 rows)"
                               + ("".join(f"; from layer {nl} on the top {nk}" for nl, nk in nested)),
                   "batch": dims.B, "seq_len": dims.S, "layers": dims.n_layers, "hidden": dims.d,
                   "vocab": dims.vocab, "active_rows": k_sparse, "boundary_layer": boundary,
                   "iterations_per_step": n_iter, "setup_s": round(t_setup, 1),
                   "launch": "hip graph replay" if graph is not None else "eager",
                   "nested": [list(x) for x in nested] or None},
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "extra": None,
    }
    if not args.no_extra:
        del graph, state, ws, model, w
        torch.cuda.empty_cache()
        line["extra"] = extra_measurements(kernels, roofline, not args.no_cpu_baseline)
    print(json.dumps(line), flush=True)


def extra_measurements(kernels, roofline, with_cpu):
    """Beside the headline: the measured achievable peaks (and every kernel's fraction of them), the
    one-layer kernel latencies at 64 of 512 rows, and one timed run each of the Dream-7B-shaped
    lock ramp and the long-context dilated run with their dominant kernel's roofline and an
    extrapolated oracle baseline.  Each part that fails reports its error instead of a figure."""
    out = {}

    def part(key, fn):
        t0 = time.perf_counter()
        try:
            out[key] = fn()
        except Exception as e:  # noqa: BLE001 -- reported in the line, never hidden
            out[key] = {"error": f"{type(e).__name__}: {e}"}
            print(f"[bench] {key} failed: {type(e).__name__}: {e}", file=sys.stderr, flush=True)
        print(f"[bench] {key}: {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    part("measured_peaks", measured_peaks)
    pk = out.get("measured_peaks", {})
    if "read_gbps" in pk:
        for k in kernels or []:
            if k.get("bound") == "hbm":
                k["frac_of_measured"] = round(k["gbps"] / pk["read_gbps"], 4)
            elif k.get("bound") == "mfma":
                k["frac_of_measured"] = round(k["tflops"] / pk["bf16_mfma_tflops"], 4)
        if roofline:
            roofline["measured_peak"] = pk["read_gbps"]
            roofline["measured_peak_kind"] = "nontemporal HBM read probe"
            roofline["frac_of_measured"] = round(roofline["achieved"] / pk["read_gbps"], 4)
    part("one_layer_64_rows", c2_layer_kernels)

    def run(name):
        res = run_workload(name, steps=1, warmup=1)
        dom = None
        for k in res["kernels"] or []:
            if name == "dream" and k["kernel"].startswith("ffn_up"):
                dom = k
            if name == "long" and k["kernel"] == "attention":
                dom = k
        summary = {"value": res["value"], "unit": "tokens/s", "ms_per_step": res["ms_per_step"],
                   "config": res["config"], "dominant_kernel": dom, "kernels": res["kernels"]}
        if with_cpu:
            summary["cpu_baseline"] = workload_cpu_baseline(name, res)
        return summary

    part("dream_lock_ramp", lambda: run("dream"))
    part("long_context_dilated", lambda: run("long"))
    return out


if __name__ == "__main__":
    main()
