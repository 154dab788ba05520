"""Decode-throughput benchmark of the LowRAM decode step on one MI355X.

A step is one decode step of every layer (32 calls of lowram_decode_step,
one per layer, each for the whole batch) against a compressed cache resident
in HBM; tokens/s = batch / step time.  Default workload: 262144-token
context, batch 28, Llama-3-8B shape (32 layers, 32 query / 8 KV heads, head
dim 128), top-1024 chunks of 8, window 256, rank 512, value MLP 128-256-128,
12.5% residuals.  Every (sequence, layer) owns distinct device buffers.

Prints one JSON line with the step time, the per-kernel HIP-event timings of
the timed region, the roofline of the dominant kernel, the dense bf16
baseline and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
KERNELS = ("score", "select", "attend", "merge")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3_llama8b_262k")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None, help="fewer layers (debug only)")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--dense-batch", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-slices", type=int, default=10)
    ap.add_argument("--eager", action="store_true",
                    help="report the eager launches (with per-kernel events) instead of a hipGraph replay")
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--shared", type=int, default=0, metavar="Q",
                    help="time Q queries over one shared context (shared-prefix multi-query decode)")
    ap.add_argument("--fit", action="store_true",
                    help="time the randomised Cholesky-QR basis fit of one 262K-token layer group")
    ap.add_argument("--append", action="store_true",
                    help="time the window rollover (one chunk into the prefix) for one layer group")
    ap.add_argument("--build", action="store_true",
                    help="time the cache builder (one layer group of one sequence) instead of the decode step")
    ap.add_argument("--peaks", action="store_true",
                    help="measure achievable peaks: a streaming device copy and a large bf16 GEMM")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first copy a buffer of this size 3 times (HBM counter calibration)")
    return ap.parse_args()


TRAFFIC_FILES = {
    ("c3_llama8b_262k", 28): os.path.join(ROOT, "profiles", "decode_c3_262k_b28_hbm_traffic.txt"),
    ("c4_eq_int4_evict_262k", 16): os.path.join(ROOT, "profiles", "decode_c4_int4_evict_262k_b16_hbm_traffic.txt"),
}
KERNEL_SOURCES = {
    "attend": ("attend.hip", "attend_pipe.hip", "attend_ops.h", "window.h", "common.h", "internal.h"),
    "score": ("score_select.hip", "window.h", "common.h", "internal.h"),
    "select": ("score_select.hip", "window.h", "common.h", "internal.h"),
    "merge": ("attend.hip", "window.h", "common.h", "internal.h"),
    "predict": ("build.hip", "common.h", "internal.h"),
    "proj": ("build.hip", "common.h", "internal.h"),
}
BUILD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "build_c3_262k_hbm_traffic.txt")


def source_hash(kernel):
    """sha256[:16] of the kernel's source files with comments and blank space
    removed: a counter summary stays valid across comment edits, and goes
    stale with any change to the code itself."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "long_context_decode_landmark_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, nb, path=None):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a copy of known size), or None when
    there is none for the workload or the kernel's sources changed since."""
    path = path or TRAFFIC_FILES.get((workload, nb))
    if path is None:
        return None
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        f = ln.split()
        if len(f) == 6 and f[0] == "traffic" and f[1] == kernel and f[2] == workload and int(f[3]) == nb:
            return float(f[5]) if f[4] == source_hash(kernel) else None
    return None


COUNTER_FILES = {
    ("c3_llama8b_262k", 28): os.path.join(ROOT, "profiles", "decode_c3_262k_b28_counters.txt"),
    ("c4_eq_int4_evict_262k", 16): os.path.join(ROOT, "profiles", "decode_c4_int4_evict_262k_b16_counters.txt"),
}


def measured_mfma_flops(kernel, workload, nb):
    """MFMA flops per launch of `kernel` counted by rocprofv3 (512 x the
    SQ_INSTS_VALU_MFMA_MOPS_* counters) from the committed counter summary, or
    None when there is none for this workload or the sources changed since."""
    path = COUNTER_FILES.get((workload, nb))
    if path is None:
        return None
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        f = ln.split()
        if len(f) == 6 and f[0] == "mfma_flops" and f[1] == kernel and f[2] == workload and int(f[3]) == nb:
            return float(f[5]) if f[4] == source_hash(kernel) else None
    return None


def step_stats(ms):
    """Median, 10th and 90th percentile of per-step times (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_probe(mib):
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    print(f"copy probe: 3 copies of {n} bytes", file=sys.stderr)


def algorithmic(cfg, nb, window_stage="attend"):
    """Algorithmic HBM bytes and MFMA flops of one layer for `nb` sequences.

    Per (sequence, layer): landmarks read once; coefficients of the k*S
    selected tokens per KV head; this layer's basis blocks and MLP weights;
    residual rows (and indices, chunk offsets) of the selected tokens at the
    stored density; the exact window; q in, out.  Flops: landmark scores,
    reconstruction, the two MLP layers, attention.  The window's bytes and
    flops are counted in the stage whose launch runs its tiles
    (window_stage: "attend", or "score" when they ride in the score grid).
    """
    Hkv, Hq, d, H, r, S = cfg.n_heads_kv, cfg.n_heads_q, cfg.head_dim, cfg.mlp_hidden, cfg.rank, cfg.chunk
    k = min(cfg.topk, cfg.n_cand)
    kS = k * S
    rho = cfg.n_resid / cfg.prefix
    s_c = 0.5 + 2.0 / 32 if cfg.int4 else 2.0          # bytes per coefficient (+fp16 scale / 32)
    s_r = d * (0.5 + 2.0 / 32) if cfg.int4 else d * 2.0  # bytes per residual row
    b = {}
    b["score"] = cfg.n_cand * Hkv * d * 2 + (cfg.n_cand * Hkv * 4 if cfg.evict else 0) + Hq * d * 2
    b["attend"] = (Hkv * kS * r * s_c + Hkv * r * d * 2 + Hkv * (2 * d * H + H + d) * 2
                   + Hkv * kS * rho * (s_r + 4) + Hkv * k * 8 + Hq * d * 2)
    b["merge"] = Hq * d * 2
    b["select"] = 0.0
    f = {
        "score": 2.0 * Hq * cfg.n_cand * d,
        "attend": 2.0 * Hkv * kS * r * d + 4.0 * Hkv * kS * d * H + 4.0 * Hq * kS * d,
        "select": 0.0, "merge": 0.0,
    }
    b[window_stage] += 2 * Hkv * cfg.window * d * 2
    f[window_stage] += 4.0 * Hq * cfg.window * d
    return {kk: v * nb for kk, v in b.items()}, {kk: v * nb for kk, v in f.items()}


def window_stage(cfg, nb):
    """The stage whose launch runs the exact window's tiles in this process's
    decode step (the library's plan for this device, with the same
    LOWRAM_PIPE_CUS / LOWRAM_ATTEND overrides the library reads)."""
    import torch

    from long_context_decode_landmark_amd import native
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    env_cu = os.environ.get("LOWRAM_PIPE_CUS", "")
    if env_cu.isdigit() and 1 <= int(env_cu) <= 65536:
        n_cu = int(env_cu)
    mode = {"pipe": 1, "wave": 2}.get(os.environ.get("LOWRAM_ATTEND", ""), 0)
    plan = native.decode_plan(native.make_shape(cfg, batch=nb), n_cu, mode)
    return "score" if plan["window_kernel"] == 1 else "attend"


def build_device_cache(cfg, nb, n_layers, seed, dev, q_nb=None):
    """Distinct device buffers for every (sequence, layer); one drawn slice replicated.
    Queries: q_nb (default nb) query sets per layer."""
    import torch

    from long_context_decode_landmark_amd import native
    from synth import device as sd

    def rep(t):
        return t.unsqueeze(0).expand((nb,) + tuple(t.shape)).contiguous()

    base = sd.draw_layer(cfg, seed, dev)
    desc = torch.empty((cfg.n_heads_kv, cfg.n_chunks), dtype=torch.int32, device=dev)
    native.resid_chunk_desc(base["res_idx"], cfg.n_heads_kv, cfg.n_resid, cfg.n_chunks, cfg.chunk, desc)
    base["res_chunk_desc"] = desc
    coeff = sd.draw_coeff(cfg, seed + 1, dev)
    groups = []
    for _ in range((n_layers + cfg.group_layers - 1) // cfg.group_layers):
        if cfg.int4:
            groups.append({"coeff": rep(coeff[0]), "coeff_scale": rep(coeff[1])})
        else:
            groups.append({"coeff": rep(coeff)})
    layers, qs = [], []
    for li in range(n_layers):
        t = {kk: rep(v) for kk, v in base.items()}
        t.update(groups[li // cfg.group_layers])
        layers.append(t)
        qs.append(sd.draw_queries(cfg, nb if q_nb is None else q_nb, seed + 100 + li, dev))
    torch.cuda.synchronize()
    return layers, qs


def time_lowram(cfg, nb, n_layers, steps, warmup, seed, graph, shared=False):
    """Decode steps of nb sequences, or (shared) of nb queries over one context per layer."""
    import torch

    from long_context_decode_landmark_amd import native

    dev = torch.device("cuda:0")
    layers, qs = build_device_cache(cfg, 1 if shared else nb, n_layers, seed, dev, q_nb=nb)
    shape = native.make_shape(cfg, batch=nb)
    ws = torch.empty(native.workspace_bytes(shape), dtype=torch.uint8, device=dev)
    out = torch.empty_like(qs[0])
    caches = [native.make_cache(t) for t in layers]
    stream = torch.cuda.current_stream()

    def step(events=None):
        for li in range(n_layers):
            if shared:
                native.decode_shared(shape, caches[li], qs[li], out, ws,
                                     events=None if events is None else events[li])
            elif events is None:
                native.decode_step(shape, caches[li], qs[li], out, ws)
            else:
                native.decode_step_events(shape, caches[li], qs[li], out, ws, events[li])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # timed region: per-kernel events on the launch stream, step events around
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_layers)]
           for _ in range(steps)]
    for s in evs:
        for lay in s:
            for e in lay:
                e.record(stream)  # creates the underlying hipEvent
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for s in range(steps):
        step(evs[s])
    t1.record(stream)
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / steps
    eager_steps = [s[0][0].elapsed_time(s[-1][4]) for s in evs]
    kern = {k: 0.0 for k in KERNELS}
    for s in evs:
        for lay in s:
            for i, k in enumerate(KERNELS):
                kern[k] += lay[i].elapsed_time(lay[i + 1])
    kern = {k: v / (steps * n_layers) for k, v in kern.items()}  # ms per launch

    graph_ms, graph_steps = None, None
    if graph:
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(stream)
        with torch.cuda.stream(s2):
            step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        marks[0].record()
        for i in range(steps):
            g.replay()
            marks[i + 1].record()
        torch.cuda.synchronize()
        graph_ms = marks[0].elapsed_time(marks[-1]) / steps
        graph_steps = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]

    # one slice back to the host for the CPU baseline
    host = {kk: v[0].cpu() for kk, v in layers[0].items()}
    q0 = qs[0][:1].cpu()
    del layers, qs, caches, ws, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return step_ms, kern, graph_ms, host, q0, (graph_steps if graph_steps is not None else eager_steps)


def time_dense(cfg, nb, n_layers, steps, warmup, seed):
    """Dense bf16 GQA decode over the full cache; 2 distinct layer buffers
    (each far larger than the 256 MB Infinity Cache) cycled over the layers."""
    import torch

    from long_context_decode_landmark_amd import native

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    shp = (nb, cfg.n_heads_kv, cfg.ctx, cfg.head_dim)
    bufs = [(torch.randn(shp, generator=g, device=dev, dtype=torch.bfloat16),
             torch.randn(shp, generator=g, device=dev, dtype=torch.bfloat16)) for _ in range(2)]
    q = torch.randn((nb, cfg.n_heads_q, cfg.head_dim), generator=g, device=dev, dtype=torch.bfloat16)
    out = torch.empty_like(q)
    ds = native.dense_shape(nb, cfg.ctx, cfg.n_heads_q, cfg.n_heads_kv, cfg.head_dim)
    ws = torch.empty(native.dense_workspace_bytes(ds), dtype=torch.uint8, device=dev)

    def step():
        for li in range(n_layers):
            k, v = bufs[li % 2]
            native.dense_decode_step(ds, k, v, q, out, ws)

    for _ in range(warmup):
        step()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    bytes_layer = 2.0 * nb * cfg.n_heads_kv * cfg.ctx * cfg.head_dim * 2
    del bufs
    torch.cuda.empty_cache()
    return ms, bytes_layer * n_layers / (ms * 1e-3) / 1e9


def cpu_baseline(cfg, host, q0, n_slices):
    """The oracle on `n_slices` (sequence, layer) slices of the same workload."""
    import numpy as np
    import torch

    from oracle import decode

    def np_(t):
        if t.dtype in (torch.bfloat16, torch.int16):
            return t.contiguous().view(torch.int16).numpy().view(np.uint16)
        return t.contiguous().numpy()

    cache = {k: np_(v)[None] for k, v in host.items()}
    q = np_(q0)
    rng = np.random.default_rng(0)
    t0 = time.time()
    for i in range(n_slices):
        qi = q if i == 0 else np_(torch.randn((1, cfg.n_heads_q, cfg.head_dim)).to(torch.bfloat16))
        decode.decode_step(cfg, cache, qi)
    dt = (time.time() - t0) / n_slices
    del rng
    cores = len(os.sched_getaffinity(0))
    try:  # the BLAS pool the oracle's matmuls actually ran on
        from threadpoolctl import threadpool_info
        blas = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            cores = max(blas)
    except Exception:
        pass
    return {"value": 1.0 / (dt * cfg.n_layers), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n_slices} (sequence, layer) slices of the same workload (all {cfg.n_heads_kv} KV heads), "
                      f"{dt:.2f} s each, extrapolated x{cfg.n_layers} layers per token"}


BUILD_KERNELS = ("proj", "arrays", "predict", "select", "store")


def build_algorithmic(cfg, nb):
    """Algorithmic MFMA flops and HBM bytes of the builder's kernels, per launch.

    proj (one per group): C = X B^T over P tokens: 2 P D r flops; reads X (P x D
    bf16), B; writes C.  predict (one per layer): per (token, KV head) the
    rebuild 2 d r, the MLP 2 * 2 d H flops; reads C (once per head), this
    layer's values, writes the fp32 residual rows and error keys.
    """
    P, D, r, Hkv, d, H = cfg.prefix, cfg.group_dim, cfg.rank, cfg.n_heads_kv, cfg.head_dim, cfg.mlp_hidden
    s_c = 0.5 + 2.0 / 32 if cfg.int4 else 2.0
    f = {"proj": 2.0 * P * D * r, "predict": Hkv * P * (2.0 * d * r + 4.0 * d * H)}
    # predict: the coefficients once (all KV heads of a token share its row), the
    # layer's values, the fp32 residual rows and error keys written
    b = {"proj": P * D * 2.0 + r * D * 2.0 + P * r * s_c,
         "predict": P * r * s_c + Hkv * P * (d * 2.0 + d * 4.0 + 4.0)}
    return {k: v * nb for k, v in f.items()}, {k: v * nb for k, v in b.items()}


def build_cpu_baseline(cfg, n_tok):
    """The oracle's compression of the first n_tok prefix tokens of the group
    (projection) and of one (layer, KV head), scaled to the whole group."""
    import numpy as np
    from oracle import codecs, compress
    import synth
    sub = cfg.with_(name=cfg.name + "_cpu", ctx=n_tok + cfg.window, resid_frac=cfg.resid_frac)
    rng = np.random.default_rng(7)
    x = codecs.bf16_round(synth.exact_keys(sub, 0, 0, 0, n_tok, dtype=np.float32))
    B = codecs.bf16_round(synth.basis(cfg, 0, 0))
    t0 = time.perf_counter()
    c_st = compress.store_coeff(compress.project(x, B), cfg.int4)
    t_proj = time.perf_counter() - t0
    cols = synth.layer_cols(cfg, 0, 0)
    xh = np.concatenate([x[:, cols], rng.standard_normal((cfg.window, cfg.head_dim))])
    v = rng.standard_normal((n_tok + cfg.window, cfg.head_dim)) * 0.5
    mlp = tuple(codecs.bf16_encode(a) for a in synth.mlp_weights(cfg, 0, 0, 0))
    blk = codecs.bf16_encode(compress.basis_block(B, cols))
    t0 = time.perf_counter()
    compress.compress_from_kv(sub, xh, v, c_st, blk, mlp)
    t_head = time.perf_counter() - t0
    per_tok = (t_proj + cfg.group_layers * cfg.n_heads_kv * t_head) / n_tok
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": round(1.0 / per_tok, 1), "unit": "prefix tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"projection of {n_tok} tokens ({t_proj:.2f} s) and one (layer, KV head) compression of "
                      f"them ({t_head:.2f} s), scaled x{cfg.group_layers * cfg.n_heads_kv} heads per group"}


def bench_build(args):
    import torch
    import synth
    from long_context_decode_landmark_amd import native
    from synth import device as sd
    cfg = synth.CONFIGS[args.config]
    nb = args.batch or 1
    dev = torch.device("cuda:0")
    G, Hkv, d, r, P, W = cfg.group_layers, cfg.n_heads_kv, cfg.head_dim, cfg.rank, cfg.prefix, cfg.window
    nC, nR = cfg.n_chunks, cfg.n_resid
    inp = sd.draw_build_inputs(cfg, args.seed, dev, nb)
    shape = native.make_build_shape(cfg, batch=nb)
    bf = torch.bfloat16
    if cfg.int4:
        coeff = torch.empty((nb, P, r // 2), dtype=torch.uint8, device=dev)
        cscale = torch.empty((nb, P, r // 32), dtype=torch.int16, device=dev)
    else:
        coeff, cscale = torch.empty((nb, P, r), dtype=bf, device=dev), None
    ios = []
    for li in range(G):
        io = dict(keys=inp["keys"], group_basis=inp["group_basis"], coeff=coeff, coeff_scale=cscale,
                  **inp["layers"][li])
        io["basis"] = torch.empty((nb, Hkv, d, r), dtype=bf, device=dev)
        io["landmark"] = torch.empty((nb, Hkv, nC, d), dtype=bf, device=dev)
        io["res_idx"] = torch.empty((nb, Hkv, nR), dtype=torch.int32, device=dev)
        if cfg.int4:
            io["res_val"] = torch.empty((nb, Hkv, nR, d // 2), dtype=torch.uint8, device=dev)
            io["res_scale"] = torch.empty((nb, Hkv, nR, d // 32), dtype=torch.int16, device=dev)
        else:
            io["res_val"] = torch.empty((nb, Hkv, nR, d), dtype=bf, device=dev)
        io["res_chunk_desc"] = torch.empty((nb, Hkv, nC), dtype=torch.int32, device=dev)
        io["win_k"] = torch.empty((nb, Hkv, W, d), dtype=bf, device=dev)
        io["win_v"] = torch.empty((nb, Hkv, W, d), dtype=bf, device=dev)
        ios.append(io)
    ws = torch.empty(native.build_layer_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    acc = {k: 0.0 for k in BUILD_KERNELS}

    def step(ev=None):
        if ev is not None:
            ev[0][0].record()
        native.build_coeff(shape, inp["keys"], inp["group_basis"], coeff, cscale)
        if ev is not None:
            ev[0][1].record()
        for li in range(G):
            native.build_layer(shape, li, ios[li], ws, events=ev[1 + li] if ev is not None else None)

    for _ in range(args.warmup):
        step()
    # per-step events on the launch stream (recorded once here to create them)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)]] +
           [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(G)] for _ in range(args.steps)]
    for s_ in evs:
        for grp_ in s_:
            for e in grp_:
                e.record()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s_ in range(args.steps):
        step(evs[s_])
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / args.steps
    for s_ in evs:
        acc["proj"] += s_[0][0].elapsed_time(s_[0][1])
        for li in range(G):
            e = s_[1 + li]
            for j, k in enumerate(BUILD_KERNELS[1:]):
                acc[k] += e[j].elapsed_time(e[j + 1])
    launches = {"proj": args.steps, **{k: args.steps * G for k in BUILD_KERNELS[1:]}}
    per_launch = {k: acc[k] / launches[k] for k in BUILD_KERNELS}
    flops, byts = build_algorithmic(cfg, nb)
    share = {k: per_launch[k] * launches[k] for k in BUILD_KERNELS}
    dom = max(("proj", "predict"), key=lambda k: share[k])
    ach = flops[dom] / (per_launch[dom] * 1e-3) / 1e12
    res = {
        "metric": "cache build: prefix tokens compressed per second (all layers of one layer group)",
        "value": round(nb * P / (step_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (fp32-accurate residual prediction)" if not cfg.int4 else "bf16+int4",
        "data": "synthetic (seeded device draws: latent-structured keys, random values)",
        "config": {"workload": cfg.name + "_build", "batch": nb, "ctx": cfg.ctx, "prefix": P,
                   "group_layers": G, "heads_kv": Hkv, "rank": r, "resid_frac": cfg.resid_frac,
                   "int4": cfg.int4},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFS, 4),
                     "traffic": measured_traffic(dom, cfg.name + "_build", nb, BUILD_TRAFFIC_FILE)},
        "kernels": {k: {"ms_per_launch": round(per_launch[k], 5), "launches_per_step": launches[k] // args.steps,
                        "TFLOP/s": round(flops[k] / (per_launch[k] * 1e-3) / 1e12, 2) if k in flops else None,
                        "GB/s": round(byts[k] / (per_launch[k] * 1e-3) / 1e9, 1) if k in byts else None}
                    for k in BUILD_KERNELS},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = build_cpu_baseline(cfg, 65536)
    print(json.dumps(res))


def fit_cpu_baseline(cfg, n_tok):
    """The oracle's randomised Cholesky-QR fit and its exact SVD fit on the first
    n_tok tokens of the group (fp64 NumPy / LAPACK on the host), scaled to P."""
    import numpy as np
    from oracle import basis, codecs
    import synth
    x = codecs.bf16_round(synth.exact_keys(cfg, 0, 0, 0, n_tok, dtype=np.float32))
    om = np.random.default_rng(5).standard_normal((n_tok, cfg.rank))
    t0 = time.perf_counter()
    basis.randomized_cholqr(x, om, power=1)
    t_rand = time.perf_counter() - t0
    t0 = time.perf_counter()
    basis.svd_basis(x, cfg.rank)
    t_svd = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    scale = cfg.prefix / n_tok
    return {"value": round(cfg.prefix / (t_rand * scale), 1), "unit": "prefix tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"randomised CholQR (one power pass) of the first {n_tok} tokens x {cfg.group_dim} dims in "
                      f"{t_rand:.2f} s, scaled x{scale:.1f} (linear in tokens); exact SVD of the same sample "
                      f"{t_svd:.2f} s ({t_svd / t_rand:.1f}x the randomised fit)"}


def bench_fit(args):
    """lowram_fit_basis for one 262K-token layer group (keys 261888 x 4096,
    rank 512, one power pass): three MFMA GEMMs of 2 P D r flops each plus
    four fp64 Cholesky-QR passes."""
    import torch
    import synth
    from long_context_decode_landmark_amd import native
    from synth import device as sd
    cfg = synth.CONFIGS[args.config]
    P, D, r = cfg.prefix, cfg.group_dim, cfg.rank
    dev = torch.device("cuda:0")
    d_in = sd.draw_build_inputs(cfg, args.seed, dev, 1, layers=[])
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    om = torch.randn((1, r, P), generator=g, device=dev).to(torch.bfloat16)
    shape = native.fit_shape(1, cfg.ctx, P, D, r, 1)
    ws = torch.empty(native.fit_basis_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    out = torch.empty((1, r, D), dtype=torch.bfloat16, device=dev)
    status = torch.empty((1,), dtype=torch.int32, device=dev)
    for _ in range(args.warmup):
        native.fit_basis(shape, d_in["keys"], om, out, status, ws)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        native.fit_basis(shape, d_in["keys"], om, out, status, ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    gemm_flops = 3 * 2.0 * P * D * r
    ach = gemm_flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "basis fit: prefix tokens per second (randomised Cholesky-QR, one power pass, one layer group)",
        "value": round(P / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 GEMMs, fp64 Cholesky-QR", "data": "synthetic (seeded device draws)",
        "config": {"workload": cfg.name + "_fit", "prefix": P, "group_dim": D, "rank": r, "power": 1},
        "roofline": {"bound": "mfma", "kernel": "whole fit (GEMM flops)", "achieved": round(ach, 2),
                     "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFS, 4),
                     "traffic": None},
        "status": int(status.cpu()[0]),
    }
    if not args.no_cpu:
        res["cpu_baseline"] = fit_cpu_baseline(cfg, 32768)
    print(json.dumps(res))


def bench_append(args):
    """Window rollover at 262K, batch 28: one step moves the oldest 8 window
    tokens of every sequence into the prefix, for the G layers of one group
    (lowram_append_coeff once, lowram_append_layer per layer).  Every token is
    given a residual (threshold 0), the most work the step can do."""
    import torch
    import synth
    from long_context_decode_landmark_amd import native
    from synth import device as sd
    cfg = synth.CONFIGS[args.config]
    nb = args.batch or cfg.batch
    dev = torch.device("cuda:0")
    G, Hkv, d, r, P, W, S = cfg.group_layers, cfg.n_heads_kv, cfg.head_dim, cfg.rank, cfg.prefix, cfg.window, cfg.chunk
    n_app = args.warmup + args.steps
    assert n_app * S <= W, "more rollovers than window chunks"
    pcap, rcap = P + n_app * S, cfg.n_resid + n_app * S
    base = sd.draw_layer(cfg, args.seed, dev)
    bf = torch.bfloat16

    def rep(t, shape_):
        return t.unsqueeze(0).expand((nb,) + tuple(t.shape)).reshape(shape_) if t is not None else None

    coeff = torch.zeros((nb, pcap, r), dtype=bf, device=dev)
    coeff[:, :P] = sd.draw_coeff(cfg, args.seed + 1, dev).unsqueeze(0)
    basis_g = torch.randn((nb, r, cfg.group_dim), device=dev).mul_(1.0 / 64).to(bf)
    keys_all = torch.randn((nb, n_app * S, cfg.group_dim), device=dev).to(bf)
    layers = []
    for _ in range(G):
        L = {"coeff": coeff, "basis": rep(base["basis"], (nb, Hkv, d, r)).contiguous()}
        for k in ("w1", "b1", "w2", "b2"):
            L[k] = base[k].unsqueeze(0).expand((nb,) + tuple(base[k].shape)).contiguous()
        L["landmark"] = torch.zeros((nb, Hkv, pcap // S, d), dtype=bf, device=dev)
        L["res_idx"] = torch.zeros((nb, Hkv, rcap), dtype=torch.int32, device=dev)
        L["res_val"] = torch.zeros((nb, Hkv, rcap, d), dtype=bf, device=dev)
        L["res_chunk_desc"] = torch.zeros((nb, Hkv, pcap // S), dtype=torch.int32, device=dev)
        L["win_k"] = base["win_k"].unsqueeze(0).expand(nb, Hkv, W, d).contiguous()
        L["win_v"] = base["win_v"].unsqueeze(0).expand(nb, Hkv, W, d).contiguous()
        L["thresh"] = torch.zeros((nb, Hkv), dtype=torch.float32, device=dev)
        L["count"] = torch.full((nb, Hkv), cfg.n_resid, dtype=torch.int32, device=dev)
        L["dropped"] = torch.zeros((nb, Hkv), dtype=torch.int32, device=dev)
        layers.append(L)
    torch.cuda.synchronize()
    # one event set per timed step, so that the steps are enqueued back to back
    # (a host synchronisation between them would leave the GPU idle while the
    # next step's first launch is submitted, inside the first kernel's interval)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + G)] for _ in range(args.steps)]

    def step(k, ev):
        record = ev is not None
        P0, W0 = P + k * S, W - k * S
        sh = native.make_shape(cfg, batch=nb, prefix_len=P0, window=W0, n_cand=P0 // S, n_resid=rcap,
                               prefix_cap=pcap, window_cap=W)
        kn = keys_all[:, k * S:(k + 1) * S]
        if record:
            ev[0].record()
        native.append_coeff(sh, G, kn, basis_g, coeff)
        if record:
            ev[1].record()
        for li, L in enumerate(layers):
            io = dict(keys_new=kn, res_thresh=L["thresh"], res_count=L["count"], res_dropped=L["dropped"],
                      landmark=L["landmark"], res_idx=L["res_idx"], res_val=L["res_val"],
                      res_chunk_desc=L["res_chunk_desc"], win_k=L["win_k"], win_v=L["win_v"])
            native.append_layer(sh, G, li, L, io)
            if record:
                ev[2 + li].record()

    for k in range(args.warmup):
        step(k, None)
    for ev in evs:
        for e in ev:
            e.record()  # creates the underlying hipEvent
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i, k in enumerate(range(args.warmup, n_app)):
        step(k, evs[i])
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / args.steps
    per_layer_us = sum(ev[1].elapsed_time(ev[1 + G]) / G for ev in evs) / args.steps * 1e3
    coeff_us = sum(ev[0].elapsed_time(ev[1]) for ev in evs) / args.steps * 1e3
    # fp32 FMA work of the rollover kernel per layer: per (sequence, head, token) the
    # rebuild (d r) and the MLP (2 d H) multiply-adds
    H = cfg.mlp_hidden
    flops = 2.0 * nb * Hkv * S * (d * r + 2 * d * H)
    ach = flops / (per_layer_us * 1e-6) / 1e12
    res = {
        "metric": "window rollover: 8-token chunks moved into the compressed prefix per second (262K, batch 28)",
        "value": round(nb / (step_ms * 1e-3 / G), 1), "unit": "chunks/s per layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32 (bf16 storage)",
        "data": "synthetic (seeded device draws)",
        "config": {"workload": cfg.name + "_rollover", "batch": nb, "ctx": cfg.ctx, "group_layers": G,
                   "heads_kv": Hkv, "rank": r, "chunk": S},
        "roofline": {"bound": "alu", "kernel": "append", "achieved": round(ach, 3), "peak": 157.3,
                     "unit": "TFLOP/s", "frac": round(ach / 157.3, 4), "traffic": None},
        "kernels": {"append_coeff_us": round(coeff_us, 2), "append_layer_us": round(per_layer_us, 2)},
        "note": "step = one group (4 layers); a full 32-layer model rolls over 8 groups",
    }
    print(json.dumps(res))


def bench_shared(args, cfg, nq, n_layers):
    """Q queries over one 262K context per layer: every query's own top-k,
    rebuild and attention; the context is read by all of them."""
    step_ms, kern, _, _, _, _ = time_lowram(cfg, nq, n_layers, args.steps, args.warmup, args.seed, False,
                                            shared=True)
    byts, flops = algorithmic(cfg, nq)
    # the context's landmarks, weights and window are read once per layer, not once per query
    ctx = {"score": byts["score"] / nq, "attend": byts["attend"] / nq}
    per_kernel = {k: {"ms": round(kern[k], 5),
                      "TFLOP/s": round(flops[k] / (kern[k] * 1e-3) / 1e12, 2) if kern[k] > 0 else None}
                  for k in KERNELS}
    ach = flops["attend"] / (kern["attend"] * 1e-3) / 1e12
    res = {
        "metric": "shared-context decode tokens/sec: Q queries over one 262K context",
        "value": round(nq / (step_ms * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if not cfg.int4 else "bf16+int4",
        "data": "synthetic (seeded device draws, one context per layer)",
        "config": {"workload": cfg.name + "_shared", "queries": nq, "ctx": cfg.ctx, "layers": n_layers,
                   "heads_q": cfg.n_heads_q, "heads_kv": cfg.n_heads_kv, "topk": cfg.topk, "rank": cfg.rank},
        "roofline": {"bound": "mfma", "kernel": "attend", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFS, 4), "traffic": None},
        "context_bytes_per_layer_GB": {k: round(v / 1e9, 4) for k, v in ctx.items()},
        "kernels": per_kernel,
    }
    print(json.dumps(res))


def bench_peaks(args):
    """What the chip reaches on plain work, beside the published peaks: a
    device-to-device copy of 4 GiB (HBM read + write bytes / time), a
    streaming read of 8 GiB and a register-only MFMA loop (libpeaks.so), and
    an 8192^3 bf16 matrix product through torch (hipBLASLt; 2 n^3 flops / time)."""
    import ctypes

    import torch
    from long_context_decode_landmark_amd import build as lbuild
    dev = torch.device("cuda:0")
    if not os.path.exists(lbuild.PEAKS_LIB):
        raise RuntimeError(f"{lbuild.PEAKS_LIB} is not built: run __graft_entry__.build()")
    P = ctypes.CDLL(lbuild.PEAKS_LIB)
    P.peaks_read_gbs.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_double)]
    P.peaks_mfma_tfs.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
    rd_bytes = 8 << 30
    rbuf = torch.ones(rd_bytes, dtype=torch.uint8, device=dev)
    scratch = torch.empty(65536 * 256, dtype=torch.float32, device=dev)
    read = {}
    for n_wg in (2048, 8192):
        v = ctypes.c_double(0.0)
        rc = P.peaks_read_gbs(ctypes.c_void_p(rbuf.data_ptr()), rd_bytes, n_wg,
                              ctypes.c_void_p(scratch.data_ptr()), ctypes.byref(v))
        if rc != 0:
            raise RuntimeError(f"peaks_read_gbs failed ({rc})")
        read[n_wg] = v.value
    del rbuf
    torch.cuda.empty_cache()
    mf = {}
    for n_wg in (1024, 4096):
        v = ctypes.c_double(0.0)
        rc = P.peaks_mfma_tfs(n_wg, 20000, ctypes.c_void_p(scratch.data_ptr()), ctypes.byref(v))
        if rc != 0:
            raise RuntimeError(f"peaks_mfma_tfs failed ({rc})")
        mf[n_wg] = v.value
    del scratch
    n = 4 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(5, args.steps)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * n * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    m = 8192
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    x = torch.randn((m, m), generator=g, device=dev, dtype=torch.bfloat16)
    y = torch.randn((m, m), generator=g, device=dev, dtype=torch.bfloat16)
    z = torch.empty((m, m), device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(x, y, out=z)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        torch.mm(x, y, out=z)
    b.record()
    torch.cuda.synchronize()
    mm_tfs = 2.0 * m ** 3 * reps / (a.elapsed_time(b) * 1e-3) / 1e12
    print(json.dumps({
        "metric": "achievable peaks on this MI355X", "n_gpus": 1, "steps": reps,
        "copy": {"GB/s": round(copy_gbs, 1), "frac_of_8TB/s": round(copy_gbs / HBM_PEAK_GBS, 4),
                 "what": "device-to-device copy of 4 GiB, read + write bytes"},
        "read": {"GB/s": round(max(read.values()), 1), "frac_of_8TB/s": round(max(read.values()) / HBM_PEAK_GBS, 4),
                 "by_workgroups": {str(k): round(v, 1) for k, v in read.items()},
                 "what": "8 GiB streamed once with 16-byte non-temporal loads, contiguous per workgroup"},
        "mfma_loop": {"TFLOP/s": round(max(mf.values()), 1), "frac_of_2.5PF": round(max(mf.values()) / MFMA_BF16_PEAK_TFS, 4),
                      "by_workgroups": {str(k): round(v, 1) for k, v in mf.items()},
                      "what": "v_mfma_f32_16x16x32_bf16 on registers, 8 independent chains per wave, 4 waves per workgroup"},
        "bf16_gemm": {"TFLOP/s": round(mm_tfs, 1), "frac_of_2.5PF": round(mm_tfs / MFMA_BF16_PEAK_TFS, 4),
                      "what": "torch.mm bf16 8192 x 8192 x 8192 (hipBLASLt)"},
    }))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode step shards by "
              "sequence with no exchange, so N GPUs would each run this single-GPU workload.", file=sys.stderr)
        sys.exit(2)
    if args.peaks:
        bench_peaks(args)
        return
    if args.fit:
        bench_fit(args)
        return
    if args.append:
        bench_append(args)
        return
    if args.build:
        if args.copy_probe_mib:
            copy_probe(args.copy_probe_mib)
        bench_build(args)
        return
    import synth
    cfg = synth.CONFIGS[args.config]
    nb = args.batch or cfg.batch
    n_layers = args.layers or cfg.n_layers
    if args.shared:
        bench_shared(args, cfg, args.shared, n_layers)
        return

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    eager_ms, kern, graph_ms, host, q0, per_step = time_lowram(cfg, nb, n_layers, args.steps, args.warmup,
                                                               args.seed, not args.eager)
    # the step as a serving loop runs it: one hipGraph replay per decode step
    # (the same launches; the eager pass, with HIP events between kernels,
    # gives the per-kernel times)
    step_ms = graph_ms if graph_ms is not None else eager_ms
    byts, flops = algorithmic(cfg, nb, window_stage(cfg, nb))
    dom = max(KERNELS, key=lambda k: kern[k])
    t_dom = kern[dom] * 1e-3
    inten = flops[dom] / max(byts[dom], 1.0)
    bound = "hbm" if inten < MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
    if bound == "hbm":
        ach, peak, unit = byts[dom] / t_dom / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        ach, peak, unit = flops[dom] / t_dom / 1e12, MFMA_BF16_PEAK_TFS, "TFLOP/s"
    step_bytes = sum(byts.values()) * n_layers
    step_flops = sum(flops.values()) * n_layers
    t_roof = max(step_bytes / (HBM_PEAK_GBS * 1e9), step_flops / (MFMA_BF16_PEAK_TFS * 1e12))
    per_kernel = {k: {"ms": round(kern[k], 5),
                      "GB/s": round(byts[k] / (kern[k] * 1e-3) / 1e9, 1) if kern[k] > 0 else None,
                      "TFLOP/s": round(flops[k] / (kern[k] * 1e-3) / 1e12, 2) if kern[k] > 0 else None}
                  for k in KERNELS}

    res = {
        "metric": "decode tokens/sec at 262K ctx, batch 28; HBM GB/s & MFMA util vs peak",
        "value": round(nb / (step_ms * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if not cfg.int4 else "bf16+int4",
        "data": "synthetic (seeded device draws, distinct buffers per sequence and layer)",
        "config": {"workload": cfg.name, "batch": nb, "ctx": cfg.ctx, "layers": n_layers,
                   "heads_q": cfg.n_heads_q, "heads_kv": cfg.n_heads_kv, "topk": cfg.topk, "chunk": cfg.chunk,
                   "window": cfg.window, "rank": cfg.rank, "resid_frac": cfg.resid_frac,
                   "int4": cfg.int4, "evict": cfg.evict},
        "roofline": {"bound": bound, "kernel": dom, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                     "frac": round(ach / peak, 4), "traffic": measured_traffic(dom, cfg.name, nb)},
        "step_roofline": {"alg_bytes_GB": round(step_bytes / 1e9, 3), "alg_TFLOP": round(step_flops / 1e12, 3),
                          "t_roof_ms": round(t_roof * 1e3, 4), "frac": round(t_roof / (step_ms * 1e-3), 4),
                          "hbm_GB/s": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
                          "mfma_util": round(step_flops / (step_ms * 1e-3) / (MFMA_BF16_PEAK_TFS * 1e12), 4)},
        "kernels": per_kernel,
    }
    res["step_ms_stats"] = step_stats(per_step)
    counted = measured_mfma_flops(dom, cfg.name, nb)
    res["roofline"]["mfma_util_algorithmic"] = round(flops[dom] / t_dom / 1e12 / MFMA_BF16_PEAK_TFS, 4)
    res["roofline"]["mfma_util_counted"] = (round(counted / t_dom / 1e12 / MFMA_BF16_PEAK_TFS, 4)
                                            if counted is not None else None)
    res["timing"] = ("hipGraph replay of the whole step (all layers' launches)" if graph_ms is not None
                     else "eager launches with per-kernel HIP events")
    res["eager_ms_per_step"] = round(eager_ms, 4)
    if not args.no_dense:
        dnb = min(args.dense_batch, nb)
        dms, dgbs = time_dense(cfg, dnb, n_layers, max(3, args.steps // 4), 1, args.seed)
        res["dense_baseline"] = {"batch": dnb, "ms_per_step": round(dms, 3),
                                 "tokens/s": round(dnb / (dms * 1e-3), 2), "hbm_GB/s": round(dgbs, 1),
                                 "note": "dense bf16 cache needs 32 GiB per sequence at 262K: batch 8 is "
                                         "the largest that fits 288 GB"}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(cfg, host, q0, args.cpu_slices)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
