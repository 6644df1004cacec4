"""Benchmark of the canvas denoise step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--copy-mib M]

A step is one dg_denoise_step over the whole canvas (assemble, projections,
bidirectional canvas attention over the KV cache, output projection, fused
vocabulary head / confidence / self-conditioning, renoise), chained: step s
consumes step s-1's tokens and self-conditioning vector.  Inputs are seeded
synthetic tensors already resident in HBM.  Prints one JSON line.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DEFAULT_WORKLOAD = "canvas256_L8192_d2048_V262144"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "flash_vocab_traffic.json")
VOCAB_SOURCES = [os.path.join(ROOT, "uniform_state_discrete_amd", "csrc", f)
                 for f in ("k_vocab.hip", "vocab_common.h", "dg_common.h")]


def vocab_source_hash():
    """SHA-256 of the vocabulary kernel's sources and of the compile flags
    that shape its code (so a traffic record holds only for that code)."""
    from uniform_state_discrete_amd import build as B
    h = hashlib.sha256()
    for p in VOCAB_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    h.update(json.dumps([B.HIPCC_FLAGS, B.SOURCE_FLAGS.get("k_vocab.hip", [])]).encode())
    return h.hexdigest()


def algorithmic(cfg):
    """Per-step algorithmic work (what the method must compute / move)."""
    R = cfg.B * cfg.C
    fl_vocab = 4.0 * R * cfg.V * cfg.d                       # logits + P.E
    fl_attn = 4.0 * R * (cfg.L + cfg.C) * cfg.Hq * cfg.dh    # QK^T + PV
    fl_proj = 2.0 * R * cfg.d * (cfg.Hq + 2 * cfg.Hkv) * cfg.dh + 2.0 * R * cfg.Hq * cfg.dh * cfg.d
    by_E = cfg.V * cfg.d * 2.0
    by_cache = 2.0 * cfg.B * cfg.L * cfg.Hkv * cfg.dh * 2.0
    by_w = (2 * cfg.Hq + 2 * cfg.Hkv) * cfg.dh * cfg.d * 2.0
    return dict(fl_vocab=fl_vocab, fl_attn=fl_attn, fl_proj=fl_proj, flops=fl_vocab + fl_attn + fl_proj,
                by_E=by_E, by_cache=by_cache, bytes=by_E + by_cache + by_w)


def read_traffic(workload):
    """HBM bytes per flash-vocab launch from the committed rocprofv3 counter
    runs (one record per workload), or None when the record was taken on a
    different kernel source or is missing for this workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    recs = t.get("records", []) if isinstance(t, dict) else []
    h = vocab_source_hash()
    for r in recs:
        if r.get("workload") == workload and r.get("source_sha256") == h:
            return r.get("bytes_per_launch")
    return None


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def cpu_baseline(p, cfg, min_seconds=10.0):
    """The oracle, as it stands, timed on the host: whole denoise steps of the
    same workload (chained like the GPU's), repeated until min_seconds have
    passed (at least one step)."""
    import numpy as np
    from oracle import step
    from synth import from_storage
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    f = lambda a: from_storage(a, cfg.dtype).astype(np.float64)
    E, H, Kc, Vc = f(p.E), f(p.H[0]), f(p.Kc), f(p.Vc)
    W = {k: f(v) for k, v in p.W.items()}
    x = step.init_canvas(cfg.seed, 0, cfg.B, cfg.C, cfg.V)
    S = None
    n = 0
    t0 = time.perf_counter()
    while True:
        r = step.denoise_step(H, E, W, Kc, Vc, cfg.L, x, S, cfg.tau[0], cfg.seed, n + 1, 0, cfg.dtype)
        x, S = r["x_new"], r["S"]
        n += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": n / el, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} whole numpy fp64 oracle step(s) of {cfg.name}, chained, {el:.1f} s"}


def attention_hbm_shape(stream, reps=20):
    """The HBM-bound attention shape: the long-context cache (32768 rows, 8
    KV heads of 128, K/V ~ N(0, 1), bf16) read by 16 canvas queries of 32
    heads, so 64 query rows per KV head and about 64 flop per cache byte, far
    below the ridge.  Times dg_attn_bidir (attention kernel + split combine)
    with HIP events on the launch stream; returns the cache bytes streamed per
    second against the HBM peak."""
    import torch
    import uniform_state_discrete_amd as dg
    B, C, L, Hq, Hkv, dh = 1, 16, 32768, 32, 8, 128
    g = torch.Generator(device="cuda").manual_seed(3003)
    rnd = lambda *s: torch.randn(*s, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    Kc, Vc = rnd(B, Hkv, L + C, dh), rnd(B, Hkv, L + C, dh)
    q, kn, vn = rnd(B, C, Hq, dh), rnd(B, C, Hkv, dh), rnd(B, C, Hkv, dh)
    out = torch.empty_like(q)
    dims = dg.make_dims(B, C, L, L + C, 4096, Hq, Hkv, dh, 0, dg.DG_BF16)
    ws = dg.workspace(dg.dg_attn_workspace_bytes(dims))
    for _ in range(3):
        dg.dg_attn_bidir(dims, q, Kc, Vc, kn, vn, out, None, 0, ws, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        dg.dg_attn_bidir(dims, q, Kc, Vc, kn, vn, out, None, 0, ws, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    by = 2.0 * B * L * Hkv * dh * 2
    fl = 4.0 * B * C * (L + C) * Hq * dh
    return {"shape": f"canvas {C} x {Hq} heads over a {L}-row cache, {Hkv} KV heads, head_dim {dh}, bf16",
            "us": round(us, 2), "cache_bytes": by, "achieved_GBs": round(by / us / 1e3, 1),
            "hbm_frac": round(by / us / 1e3 / PEAK_HBM_GBS, 4),
            "mfma_frac": round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4)}


def block_loop_graph(stream, replays=3):
    """The block-diffusion workload (8 canvases of 256 tokens over their own
    4096-row caches, 4 blocks of 32 steps with tau annealed 0.5 -> 0.95, a
    causal append after each block) captured into one HIP graph by
    dg_graph_capture_block_loop; times whole-sequence replays with HIP events
    on the replay stream."""
    import torch
    import uniform_state_discrete_amd as dg
    from synth import config_by_name, gen_problem, tau_schedule
    c = config_by_name("blocks4_canvas8x256_L4096_d2048_V262144")
    p = gen_problem(c)
    W = {k: dg.to_device(v) for k, v in p.W.items()}
    W["E"] = dg.model_embedding(dg.to_device(p.E))
    Kc, Vc = dg.to_device(p.Kc), dg.to_device(p.Vc)
    H = torch.stack([dg.to_device(h) for h in p.H]).contiguous()
    del p
    dims = dg.make_dims(c.B, c.C, c.L, c.cap, c.d, c.Hq, c.Hkv, c.dh, c.V, dg.DG_BF16)
    ws = dg.workspace(dg.dg_workspace_bytes(dims))
    R = c.R
    i32 = dict(dtype=torch.int32, device="cuda")
    io = dict(H=H, k_cache=Kc, v_cache=Vc, tokens=torch.zeros((c.blocks, c.B, c.C), **i32),
              canvas=torch.zeros((2, c.B, c.C), **i32),
              selfcond=torch.zeros((2, c.B, c.C, c.d), dtype=torch.bfloat16, device="cuda"),
              max_logit=torch.empty(R, device="cuda"), conf=torch.empty(R, device="cuda"),
              argmax=torch.empty(R, **i32), mask=torch.empty(R, dtype=torch.uint8, device="cuda"))
    taus = tau_schedule(c)
    g = dg.dg_graph_capture_block_loop(dims, W, io, taus, c.steps, c.blocks, c.seed, ws, stream)
    g.launch(stream)                        # warm-up replay
    stream.synchronize()
    seq = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.launch(stream)
        e1.record(stream)
        stream.synchronize()
        seq.append(e0.elapsed_time(e1))
    ms = pct(seq, 50)
    g.close()
    n_steps = c.steps * c.blocks
    alg = algorithmic(c)
    return {"workload": c.name, "graph_replays": replays, "ms_per_sequence": round(ms, 3),
            "ms_per_sequence_p10": round(pct(seq, 10), 3), "ms_per_sequence_p90": round(pct(seq, 90), 3),
            "sequence": f"{c.blocks} blocks x ({c.steps} denoise steps + causal append) over {c.B} canvases",
            "steps_per_s": round(n_steps / (ms * 1e-3), 2),
            "canvas_tokens_per_s": round(n_steps * R / (ms * 1e-3), 1),
            "step_mfma_frac": round(alg["flops"] * n_steps / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def crossover_sweep(stream, reps=10):
    """Time of the fused vocabulary head (logits, softmax statistics, P.E over
    the 262144 x 2048 bf16 table) and of canvas attention (over an 8192-row
    cache, 16/8 heads of 128) as the number of canvas rows M grows: one user's
    canvas rows against many users' rows batched together.  While the kernels
    are bound by streaming E or the cache their time stays flat; past the
    ridge it grows with M."""
    import torch
    import uniform_state_discrete_amd as dg
    d, V = 2048, 262144
    g = torch.Generator(device="cuda").manual_seed(4004)
    E = (torch.randn(V, d, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    Et = dg.tiled_embedding(E)
    del E
    L, Hq, Hkv, dh = 8192, 16, 8, 128
    Kc = torch.randn(1, Hkv, L, dh, generator=g, device="cuda").to(torch.bfloat16) * (d ** -0.5)
    Vc = torch.randn(1, Hkv, L, dh, generator=g, device="cuda").to(torch.bfloat16) * (d ** -0.5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    out = []
    for M in (1, 8, 32, 64, 128, 156, 256, 512, 1024, 2048):
        Z = (torch.randn(M, d, generator=g, device="cuda") * 0.3).to(torch.bfloat16)
        st = [torch.empty(M, device="cuda") for _ in range(3)]
        am = torch.empty(M, dtype=torch.int32, device="cuda")
        S = torch.empty(M, d, dtype=torch.bfloat16, device="cuda")
        ws = dg.workspace(dg.dg_vocab_workspace_bytes(M, d, V, dg.DG_BF16))
        vu = timed(lambda: dg.dg_vocab_selfcond(M, d, V, Z, Et, st[0], am, st[1], st[2], S, ws, stream))
        q = torch.randn(1, M, Hq, dh, generator=g, device="cuda").to(torch.bfloat16)
        kn = torch.randn(1, M, Hkv, dh, generator=g, device="cuda").to(torch.bfloat16) * (d ** -0.5)
        vn = torch.randn(1, M, Hkv, dh, generator=g, device="cuda").to(torch.bfloat16) * (d ** -0.5)
        o = torch.empty_like(q)
        dims = dg.make_dims(1, M, L, L, d, Hq, Hkv, dh, 0, dg.DG_BF16)
        wa = dg.workspace(dg.dg_attn_workspace_bytes(dims))
        au = timed(lambda: dg.dg_attn_bidir(dims, q, Kc, Vc, kn, vn, o, None, 0, wa, stream))
        vfl = 4.0 * M * V * d
        afl = 4.0 * M * (L + M) * Hq * dh
        out.append({"rows": M, "vocab_us": round(vu, 2), "vocab_TFLOPs": round(vfl / vu / 1e6, 1),
                    "vocab_E_GBs": round(V * d * 2 / vu / 1e3, 1),
                    "attn_us": round(au, 2), "attn_TFLOPs": round(afl / au / 1e6, 1),
                    "attn_cache_GBs": round(2 * L * Hkv * dh * 2 / au / 1e3, 1)})
        print(json.dumps(out[-1]), flush=True)
    return out


def prompt_prefill(stream, cfg, W, H_row, n=4096, reps=5):
    """Causal prefill of an n-token prompt into an empty cache
    (dg_prefill_append with L = 0, C = n) on the bench model: assemble, Q/K/V
    projections, cache write and causal attention.  Beside it, the same
    attention shape with no mask (every key tile), to show what the causal
    key limit saves."""
    import torch
    import uniform_state_discrete_amd as dg
    Hq, Hkv, dh, d = cfg.Hq, cfg.Hkv, cfg.dh, cfg.d
    dims = dg.make_dims(1, n, 0, n, d, Hq, Hkv, dh, cfg.V, dg.DG_BF16)
    ws = dg.workspace(dg.dg_workspace_bytes(dims))
    Kc = torch.empty((1, Hkv, n, dh), dtype=torch.bfloat16, device="cuda")
    Vc = torch.empty_like(Kc)
    H = H_row.reshape(-1, d)[:1].expand(n, d).contiguous()   # hidden rows of the prompt
    g = torch.Generator(device="cuda").manual_seed(4096)
    toks = torch.randint(0, cfg.V, (1, n), generator=g, device="cuda", dtype=torch.int32)
    attn = torch.empty((1, n, Hq, dh), dtype=torch.bfloat16, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = timed(lambda: dg.dg_prefill_append(dims, W, H, toks, Kc, Vc, attn, ws, stream))
    q = torch.randn((1, n, Hq, dh), generator=g, device="cuda").to(torch.bfloat16)
    kn = Kc.transpose(1, 2).contiguous()
    vn = Vc.transpose(1, 2).contiguous()
    wa = dg.workspace(dg.dg_attn_workspace_bytes(dims))
    ms_causal = timed(lambda: dg.dg_attn_bidir(dims, q, Kc, Vc, kn, vn, attn, None, 1, wa, stream))
    ms_full = timed(lambda: dg.dg_attn_bidir(dims, q, Kc, Vc, kn, vn, attn, None, 0, wa, stream))
    fl = 2.0 * n * d * (Hq + 2 * Hkv) * dh + 2.0 * n * (n + 1) * Hq * dh   # projections + causal attention
    return {"prompt_tokens": n, "ms": round(ms, 4), "tokens_per_s": round(n / (ms * 1e-3), 1),
            "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "causal_attention_ms": round(ms_causal, 4), "unmasked_attention_ms": round(ms_full, 4)}


def copy_calibration(mib):
    """A plain device-to-device copy of known size, for scaling HBM counters."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4}))


# Untimed running of the step before the warm-up steps of each workload: after
# an idle host-side phase (input generation, upload) the first launches of
# the flash-vocab kernel run up to 40% slower; in a fresh process the time
# settles only after roughly half a second of continuous work (kernel traces
# of long chained runs).
SETTLE_S = 1.0


def run_workload(cfg, steps, warmup, replays, stream, keep_problem=False, settle_s=SETTLE_S):
    """The denoise step of one workload, chained over `steps` steps (step s
    consumes step s-1's tokens and self-conditioning vector):
      - settle: the chained step runs untimed for settle_s seconds, then the
        canvas is drawn again, so the timed steps start from the same state;
      - `warmup` untimed steps;
      - graph: the `steps` steps captured once into a HIP graph and replayed
        `replays` times, each replay timed with HIP events; median, p10 and
        p90 of the time per step (the headline);
      - eager, right after: the same `steps` steps between HIP events on the
        launch stream, with the per-kernel event hooks of the attention and
        flash-vocab kernels (the roofline's kernel time).
    Inputs are generated and uploaded before any timed region."""
    import numpy as np
    import torch

    import uniform_state_discrete_amd as dg
    from synth import gen_problem, tau_schedule

    p = gen_problem(cfg)
    W = {k: dg.to_device(v) for k, v in p.W.items()}
    W["E"] = dg.model_embedding(dg.to_device(p.E))   # once per model, outside any timed region
    Kc, Vc, H = dg.to_device(p.Kc), dg.to_device(p.Vc), dg.to_device(p.H[0])
    fdt = W["E"].dtype
    code = dg.DG_BF16 if cfg.dtype == "bf16" else dg.DG_F32
    dims = dg.make_dims(cfg.B, cfg.C, cfg.L, cfg.cap, cfg.d, cfg.Hq, cfg.Hkv, cfg.dh, cfg.V, code)
    ws = dg.workspace(dg.dg_workspace_bytes(dims))
    R = cfg.R
    tok = [torch.empty((cfg.B, cfg.C), dtype=torch.int32, device="cuda") for _ in range(2)]
    sc = [torch.zeros((cfg.B, cfg.C, cfg.d), dtype=fdt, device="cuda") for _ in range(2)]
    stats = dict(max_logit=torch.empty(R, device="cuda"), conf=torch.empty(R, device="cuda"),
                 lse=torch.empty(R, device="cuda"), argmax=torch.empty(R, dtype=torch.int32, device="cuda"),
                 mask=torch.empty(R, dtype=torch.uint8, device="cuda"))
    taus = tau_schedule(cfg)
    dg.dg_init_canvas(R, cfg.C, cfg.V, cfg.seed, 0, tok[0], stream)

    def mk_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)       # materialise the HIP event
        return evs

    ev = {k: mk_events(steps) for k in ("vb", "ve", "ab", "ae")}

    def run(s, strm, timed_index=None):
        a, b = s % 2, (s + 1) % 2
        io = dict(H=H, k_cache=Kc, v_cache=Vc, tokens_in=tok[a], selfcond_in=None if s == 0 else sc[a],
                  tokens_out=tok[b], selfcond_out=sc[b], **stats)
        if timed_index is not None:
            io.update(ev_vocab_begin=ev["vb"][timed_index], ev_vocab_end=ev["ve"][timed_index],
                      ev_attn_begin=ev["ab"][timed_index], ev_attn_end=ev["ae"][timed_index])
        dg.dg_denoise_step(dims, W, io, taus[s % cfg.steps], cfg.seed, s % cfg.steps + 1, 0, ws, strm)

    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < settle_s:
        for _ in range(8):
            run(n_settle, stream)
            n_settle += 1
        torch.cuda.synchronize()
    dg.dg_init_canvas(R, cfg.C, cfg.V, cfg.seed, 0, tok[0], stream)
    for s in range(warmup):
        run(s, stream)
    torch.cuda.synchronize()
    kept = [1.0 - float(stats["mask"].float().mean())]

    # the chained steps as one HIP graph, replayed: the headline time
    # (replays = 0: no graph; the eager time stands in, for profiler runs)
    per_step = []
    if replays > 0:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(g, stream=cap, capture_error_mode="relaxed"):
            for k in range(steps):
                run(k, cap)
        torch.cuda.synchronize()
        g.replay()                                   # warm-up replay
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream()
        for _ in range(replays):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            g.replay()
            e1.record(cur)
            torch.cuda.synchronize()
            per_step.append(e0.elapsed_time(e1) / steps)
        del g

    # right after, the same steps eager with HIP events around the attention
    # and flash-vocab kernels on the launch stream: the per-kernel times
    t0e, t1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t0e.record(stream)
    for k in range(steps):
        run(k, stream, k)
    t1e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_eager = t0e.elapsed_time(t1e) / steps
    kept.append(1.0 - float(stats["mask"].float().mean()))
    vocab_ms = [ev["vb"][k].elapsed_time(ev["ve"][k]) for k in range(steps)]
    attn_ms = [ev["ab"][k].elapsed_time(ev["ae"][k]) for k in range(steps)]

    if not per_step:
        per_step = [ms_eager]
    alg = algorithmic(cfg)
    v_avg = float(np.mean(vocab_ms))
    a_avg = float(np.mean(attn_ms))
    ms_med = pct(per_step, 50)
    achieved = alg["fl_vocab"] / (v_avg * 1e-3) / 1e12
    out = dict(
        workload=cfg.name, steps=steps, warmup=warmup, settle_steps=n_settle,
        ms_per_step=ms_med, ms_per_step_p10=pct(per_step, 10), ms_per_step_p90=pct(per_step, 90),
        graph_replays=replays, ms_per_step_eager=ms_eager, wall_s_timed_eager=wall,
        steps_per_s=1000.0 / ms_med, canvas_tokens_per_s=1000.0 / ms_med * R,
        step_mfma_frac=alg["flops"] / (ms_med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        step_hbm_frac=alg["bytes"] / (ms_med * 1e-3) / 1e9 / PEAK_HBM_GBS,
        flash_vocab_ms=v_avg, flash_vocab_ms_p10=pct(vocab_ms, 10), flash_vocab_ms_p90=pct(vocab_ms, 90),
        attention_ms=a_avg,
        attention_mfma_frac=alg["fl_attn"] / (a_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        attention_hbm_frac=alg["by_cache"] / (a_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
        kept_fraction=kept,
        roofline={"kernel": "flash-vocab (logits, softmax stats, P.E)", "bound": "mfma",
                  "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                  "frac": achieved / PEAK_BF16_TFLOPS, "traffic": read_traffic(cfg.name),
                  "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                  "algorithmic_bytes": alg["by_E"] + cfg.B * cfg.C * cfg.d * 2.0,
                  "algorithmic_flops": alg["fl_vocab"]})
    return out, (p, W, H) if keep_problem else None


def rounded(x, nd=4):
    if isinstance(x, float):
        return round(x, nd)
    if isinstance(x, dict):
        return {k: rounded(v, nd) for k, v in x.items()}
    if isinstance(x, list):
        return [rounded(v, nd) for v in x]
    return x


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--replays", type=int, default=10,
                    help="timed graph replays of the steps (0: no graph phase, eager time only)")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed chained steps before each workload's warm-up")
    ap.add_argument("--block-loop-only", action="store_true",
                    help="only time the block-diffusion graph replay (one JSON object)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attn-hbm", action="store_true", help="skip the HBM-bound attention shape")
    ap.add_argument("--no-block-loop", action="store_true", help="skip the block-diffusion graph replay")
    ap.add_argument("--no-prefill", action="store_true", help="skip the causal prompt prefill")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the 32k-vocabulary and long-context workloads")
    ap.add_argument("--sweep-rows", action="store_true",
                    help="only run the rows sweep of the vocabulary head and attention (one JSON line per size)")
    ap.add_argument("--copy-mib", type=int, default=0, help="only run a plain copy of this size")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return
    if args.sweep_rows:
        import torch
        torch.cuda.set_device(0)
        crossover_sweep(torch.cuda.current_stream())
        return

    import torch

    from synth import config_by_name

    if args.block_loop_only:
        torch.cuda.set_device(0)
        print(json.dumps({"block_loop_graph": block_loop_graph(torch.cuda.Stream())}), flush=True)
        return
    cfg = config_by_name(args.workload)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    r, keep = run_workload(cfg, args.steps, args.warmup, args.replays, stream, keep_problem=True,
                           settle_s=args.settle)
    p, W, H = keep
    out = {
        "metric": "canvas denoise steps/s (256 tok, V=262144) + % MFMA peak, % HBM peak",
        "value": round(r["steps_per_s"], 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; single-layer stand-in model, no trained weights)",
        "config": {"workload": cfg.name, "canvases": cfg.B, "canvas_tokens": cfg.C, "kv_cache": cfg.L,
                   "d_model": cfg.d, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv, "head_dim": cfg.dh,
                   "vocab": cfg.V, "tau": cfg.tau[0], "parallelism": "1 GPU"},
        "timing": "median of the graph replays (each replays the chained steps); p10/p90 beside it; "
                  f"before the warm-up steps the step runs untimed for {args.settle} s (settle_steps); "
                  "the roofline's kernel time is the mean over eager steps run right after the replays",
    }
    for k in ("ms_per_step_p10", "ms_per_step_p90", "graph_replays", "settle_steps", "ms_per_step_eager", "canvas_tokens_per_s",
              "step_mfma_frac", "step_hbm_frac", "flash_vocab_ms", "flash_vocab_ms_p10", "flash_vocab_ms_p90",
              "attention_ms", "attention_mfma_frac", "attention_hbm_frac", "kept_fraction", "wall_s_timed_eager"):
        out[k] = rounded(r[k])
    out["roofline"] = rounded(r["roofline"])
    if not args.no_other_workloads and args.workload == DEFAULT_WORKLOAD:
        others = []
        for name, steps in (("canvas256_L1024_d2048_V32768", 16), ("canvas256_L32768_d4096_V262144", 8)):
            o, _ = run_workload(config_by_name(name), steps, 2, 5, stream, settle_s=args.settle)
            others.append(rounded({k: o[k] for k in ("workload", "steps", "steps_per_s", "ms_per_step",
                                                     "ms_per_step_p10", "ms_per_step_p90", "ms_per_step_eager",
                                                     "canvas_tokens_per_s", "step_mfma_frac", "flash_vocab_ms",
                                                     "attention_ms", "attention_mfma_frac", "attention_hbm_frac",
                                                     "roofline")}))
            torch.cuda.empty_cache()
        out["other_workloads"] = others
    if not args.no_attn_hbm:
        out["attention_hbm_shape"] = attention_hbm_shape(stream)
    if not args.no_prefill:
        out["prompt_prefill"] = prompt_prefill(stream, cfg, W, H)
    if not args.no_block_loop:
        out["block_loop_graph"] = block_loop_graph(torch.cuda.Stream())
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
