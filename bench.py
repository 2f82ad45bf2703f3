"""Benchmark of the QuantWM hot path on one MI355X.

Default workload: the 1-minute rollout (40 heads, 1,560-token frames, 240
frames = 374,400 cached tokens).  One step is one generation step at the full
cache: quantize-append of the newest frame's Keys and Values (QSAC + INT2 +
PSAC for Keys, centre + INT2 for Values) at position 239, then attention of
the 1,560-query chunk over all 374,400 compressed tokens.  The frames before
it are appended frame by frame first (the rollout leg, timed step by step),
and every timed step rewrites the newest frame in place.  `value` is cached
tokens per second through that step, in Ktokens/s.

The bulk workloads (matrix_game, lingbot480p, lingbot720p, tiny): one step is
the quantize-append of every cached frame into a fresh cache plus attention of
the query chunk over it; `value` is cached tokens per second.

Inputs stay resident in HBM; calibration (statistics and centres) is done
once, untimed, through the library.  The line carries the append rate, the
attention TFLOP/s, the roofline object of the dominant kernel and the
oracle's CPU baseline on a bounded sample.

  python bench.py [--steps K] [--warmup W] [--config minute|matrix_game|lingbot480p|lingbot720p|tiny]
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

METRIC = "Ktokens/s quantize-append + dequant-attn TFLOP/s, % of HBM/MFMA roofline"
PEAK_FP16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="minute")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-measures", action="store_true",
                    help="skip the untimed quality measures (top-1 shift, logit MSE and the ablation appends), "
                         "so that a profiler's per-kernel averages cover the timed launches only")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the oracle sample (0: auto)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter scaling for profiles)")
    ap.add_argument("--seed", type=int, default=7)
    ap.add_argument("--no-rollout", action="store_true",
                    help="1-minute rollout: append the frames before the timed step without the per-step "
                         "attention (for profiler runs whose per-kernel averages should cover the timed "
                         "full-cache launches only)")
    ap.add_argument("--measure-frames", type=int, default=24,
                    help="1-minute rollout: frames of the prefix the quality measures run on")
    ap.add_argument("--epoch-frames", type=int, default=24,
                    help="1-minute rollout: also run it with a calibration epoch every this many frames "
                         "(0: skip)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (default: the step is also captured once per input copy "
                         "into a HIP graph, and value / ms_per_step come from graph replays)")
    return ap.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "video_world_model_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def append_bytes_per_token_head(w, cfg):
    """Algorithmic HBM bytes of append per token-head (K+V): inputs read once
    plus the compressed fields written."""
    b_in = 4 if w.io == "f32" else 2
    ng = w.head_dim // 16
    tpf = -(-w.frame_tokens // w.group_tokens)
    idx = (1 if w.c_k <= 256 else 2) + (1 if w.c_v <= 256 else 2)
    params = 2 * ng * 4 * tpf / w.frame_tokens
    coef = (w.rank + 2) if w.rank else 0
    return 2 * w.head_dim * b_in + idx + 2 * ng * 4 + params + coef


def top1_shift_per_mode(w, cfg, k, v, q, qh, kh, vh, seed, qwm, torch):
    """Share of (head, query) pairs whose highest-scoring cached token under
    the rebuilt keys differs from the one under the original keys, for the
    four modes of the method: QVG (nearest centre, no compensation), QSAC
    only, PSAC only, and both (QuantWM); then QuantWM over compensation ranks
    r in {0, 4, 8, 16, 32}, and QuantWM with the stage-2 score taken on the exact
    INT2 error in the diagonal and in the full quadratic form of Eq. 7.  Each
    setting calibrates and fills a cache of its own; the append of the three
    stage-2 scores is timed (HIP events, mean of three appends after one
    warm-up)."""
    import dataclasses

    import numpy as np
    dense = qwm.dense_top1(cfg, q, k)
    modes = {"qvg": (qwm.QVG_MODE, 0), "qsac_only": (0, 0), "psac_only": (qwm.QVG_MODE, w.rank),
             "quantwm": (0, w.rank)}
    modes.update({"quantwm_r%d" % r: (0, r) for r in (4, 16, 32) if r != w.rank})
    modes.update({"quantwm_exact": (qwm.EXACT_ERROR, w.rank), "quantwm_full": (qwm.FULL_QUADRATIC, w.rank)})
    timed = ("quantwm", "quantwm_exact", "quantwm_full")
    # logit MSE on the first 64 queries of every head: mean of (l - l~)^2 over
    # (head, query, cached token), l = tau q.k with the original keys
    q64 = q[:, :64]
    tau = 1.0 / math.sqrt(w.head_dim)
    ref = tau * torch.bmm(q64.float().contiguous(), k.float().transpose(1, 2).contiguous())
    top1, mse, app_ms = {}, {}, {}
    for name, (flags, rank) in modes.items():
        c = dataclasses.replace(cfg, flags=flags, rank=rank)
        try:
            qwm.layout(c)
        except qwm.QwmError as e:
            if e.status != qwm.ERR_UNSUPPORTED:
                raise
            # a setting the library does not run (r = 32 with 512 centres: the
            # append's codebook and fp64 U do not fit in one workgroup's LDS)
            top1[name] = mse[name] = None
            continue
        calib = qwm.alloc_calib(c)
        qwm.calibrate(c, calib, qh, kh, vh, seed=seed, iters=w.kmeans_iters)
        cache = qwm.Cache(c, calib)
        if name in timed:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
            for e in ev:
                cache.reset()
                e[0].record()
                qwm.append_kv(cache, k, v)
                e[1].record()
            torch.cuda.synchronize()
            app_ms[name] = round(float(np.mean([e[0].elapsed_time(e[1]) for e in ev[1:]])), 4)
        else:
            qwm.append_kv(cache, k, v)
        top1[name] = round(float((qwm.top1(cache, q) != dense).float().mean()), 5)
        lg = qwm.attention_logits(cache, q64)
        mse[name] = float("%.5g" % float(((lg - ref) ** 2).mean()))
        del lg
    torch.cuda.synchronize()
    return top1, mse, app_ms


def attn_flops(w, n_q, n_k):
    return 4.0 * n_q * n_k * w.head_dim * w.heads


def traffic_from_profiles(kernel, config, src_hash):
    """HBM bytes per launch of `kernel` (attention / append) from committed
    rocprofv3 counter runs, if they were taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % (kernel, config))
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    if d.get("kernel_source_hash") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def query_blocks(w):
    """Query blocks per head of the attention launch: each reads the whole
    compressed cache of its head once (blocks of at most 256 queries, balanced
    and rounded up to whole 32-query waves)."""
    return -(-w.n_q // 256)


def counter_gbs(kernel, config, src_hash, ms):
    """HBM GB/s of the kernel from the committed counter traffic (None when
    the counters were taken on other sources)."""
    t = traffic_from_profiles(kernel, config, src_hash)
    return None if t is None else round(t / (ms * 1e-3) / 1e9, 1)


def cpu_baseline(w, data, cfg_host, heads, seed):
    """The oracle (untuned) on a bounded sample: append + attention of
    `heads` heads of the same workload, scaled to Ktokens/s of the full step."""
    import numpy as np
    from oracle import attention as oa
    from oracle import calibrate as oc
    from oracle import codec
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    cores = len(os.sched_getaffinity(0))
    cal = oc.calibrate(data["q_hist"][:heads], data["k_hist"][:heads], data["v_hist"][:heads],
                       w.c_k, w.c_v, w.rank, w.io, seed=seed, iters=2)
    t0 = time.perf_counter()
    for h in range(heads):
        ko = codec.append_keys(data["k"][h], cal["mu_k"][h], cal["sens"][h], cal["u"][h], w.frame_tokens,
                               w.group_tokens, w.top_k, 0)
        vo = codec.append_values(data["v"][h], cal["mu_v"][h], w.frame_tokens, w.group_tokens)
        kr = oa.reconstruct_keys(ko["idx"], ko["codes"], ko["z"], ko["s"], ko["coef"], ko["coef_scale"],
                                 cal["mu_k"][h], cal["u"][h], w.frame_tokens, w.group_tokens)
        vr = oa.reconstruct_values(vo["idx"], vo["codes"], vo["z"], vo["s"], cal["mu_v"][h], w.frame_tokens,
                                   w.group_tokens)
        oa.softmax_attention(data["q"][h], kr, vr)
    dt = time.perf_counter() - t0
    step_s = dt * w.heads / heads
    return {"value": round(w.n_tokens / step_s / 1e3, 4), "unit": "Ktokens/s", "cores": int(min(cores, max(blas, 1))),
            "kind": "oracle",
            "sample": "%d of %d heads, all %d cached tokens: oracle append (K+V) + reconstruction attention of %d "
                      "queries, %.1f s on the host, scaled x%d to the full step; BLAS threads %d, affinity cores %d"
                      % (heads, w.heads, w.n_tokens, w.n_q, dt, w.heads // heads if w.heads % heads == 0 else 0,
                         blas, cores)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library runs on a single MI355X and has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np

    import workloads
    pool = None
    if args.config == "minute":
        # input generation runs in worker processes, forked before anything
        # touches the GPU
        import multiprocessing as mp
        pool = mp.get_context("fork").Pool(max(1, min(16, len(os.sched_getaffinity(0)))))
    import torch

    import video_world_model_amd as qwm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = workloads.WORKLOADS[args.config]
    if args.config == "minute":
        try:
            return generation_step(args, w, qwm, torch, np, workloads, pool)
        finally:
            pool.terminate()
    cfg = qwm.Config(heads=w.heads, head_dim=w.head_dim, frame_tokens=w.frame_tokens, max_frames=w.frames,
                     c_k=w.c_k, c_v=w.c_v, group_tokens=w.group_tokens, top_k=w.top_k, rank=w.rank, io=w.io)
    dt = cfg.torch_dtype
    t_gen = time.perf_counter()
    data = workloads.generate(w, threads=16)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)
    k, v, q = dev(data["k"]), dev(data["v"]), dev(data["q"])
    qh, kh, vh = dev(data["q_hist"]), dev(data["k_hist"]), dev(data["v_hist"])
    print("[bench] %s: generated in %.1fs" % (w.name, time.perf_counter() - t_gen), file=sys.stderr, flush=True)

    calib = qwm.alloc_calib(cfg)
    t_cal = time.perf_counter()
    energy = qwm.calibrate(cfg, calib, qh, kh, vh, seed=args.seed, iters=w.kmeans_iters)
    print("[bench] calibrated in %.1fs (top-%d energy mean %.3f)" % (time.perf_counter() - t_cal, w.rank,
          float(energy.mean())), file=sys.stderr, flush=True)

    # rotate input copies over > 512 MiB so the 256 MB MALL cannot serve them
    in_bytes = 2 * k.numel() * k.element_size()
    copies = max(1, math.ceil(512 * 2**20 / in_bytes))
    ks = [k] + [k.clone() for _ in range(copies - 1)]
    vs = [v] + [v.clone() for _ in range(copies - 1)]

    cache = qwm.Cache(cfg, calib)
    ws_bytes = qwm.workspace_bytes(cfg, w.n_tokens, w.n_q)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(w.heads, w.n_q, dtype=torch.float32, device="cuda")

    reset = cache.reset

    # per step: append (one kernel), attention call, attention kernel alone
    # (events recorded by the library around its main kernel, on its stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for e in ev:
        for x in e:
            x.record()  # creates the events the library records into
    torch.cuda.synchronize()

    def step(i, e=None):
        reset()
        kk, vv = ks[i % copies], vs[i % copies]
        if e: e[0].record()
        qwm.append_kv(cache, kk, vv)
        if e: e[1].record()
        if e: e[2].record()
        qwm.attention(cache, q, out=out, lse=lse, workspace=ws if ws_bytes else None,
                      kernel_events=(e[4], e[5]) if e else None)
        if e: e[3].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    wall_eager = wall

    # The same step captured into a HIP graph (one per rotated input copy:
    # reset, fused append, attention and its merge pass) and replayed: the
    # GPU work is identical, the launch gaps between the kernels go away.
    if not args.no_graph:
        graphs = []
        for i in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    app_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
    att_ms = [ev[i][2].elapsed_time(ev[i][3]) for i in range(args.steps)]
    attk_ms = [ev[i][4].elapsed_time(ev[i][5]) for i in range(args.steps)]
    ms_step = wall * 1e3 / args.steps
    tok_heads = w.n_tokens * w.heads
    app_bytes = tok_heads * append_bytes_per_token_head(w, cfg)
    flops = attn_flops(w, w.n_q, w.n_tokens)
    app_avg, att_avg, attk_avg = float(np.mean(app_ms)), float(np.mean(att_ms)), float(np.mean(attk_ms))
    achieved_tf = flops / (attk_avg * 1e-3) / 1e12
    app_gbs = app_bytes / (app_avg * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    # roofline of the dominant kernel: the fused append (HBM-bound) or the
    # attention kernel (fp16 MFMA), whichever takes longer per step
    if app_avg > attk_avg:
        roofline = {"kernel": "append_kv_kernel (quantize-append, Keys and Values)", "bound": "hbm",
                    "achieved": round(app_gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(app_gbs / PEAK_HBM_GBS, 4),
                    "traffic": traffic_from_profiles("append", args.config, src_hash),
                    "algorithmic_bytes_per_launch": round(app_bytes), "ms_per_launch": round(app_avg, 4)}
    else:
        roofline = {"kernel": "attn_bf16_kernel (dequant-attention)", "bound": "mfma",
                    "achieved": round(achieved_tf, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved_tf / PEAK_FP16_TFLOPS, 4),
                    "traffic": traffic_from_profiles("attention", args.config, src_hash),
                    "algorithmic_flops_per_launch": flops, "ms_per_launch": round(attk_avg, 4)}

    # one generation step's attention with the chunk's own keys and values:
    # the query chunk over the full compressed cache and the next frame in
    # bf16 (timed apart from the step, whole call including the merge)
    F = w.frame_tokens
    kl = dev(np.stack([workloads.kv_frames(w, h, "k", w.frames, w.frames + 1) for h in range(w.heads)]))
    vl = dev(np.stack([workloads.kv_frames(w, h, "v", w.frames, w.frames + 1) for h in range(w.heads)]))
    ws_l = torch.empty(max(qwm.workspace_bytes(cfg, w.n_tokens + F, w.n_q), 1), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        qwm.attention_local(cache, q, kl, vl, out=out, lse=lse, workspace=ws_l)
    el = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(10)]
    torch.cuda.synchronize()
    for e in el:
        e[0].record()
        qwm.attention_local(cache, q, kl, vl, out=out, lse=lse, workspace=ws_l)
        e[1].record()
    torch.cuda.synchronize()
    loc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in el]))
    loc_tf = attn_flops(w, w.n_q, w.n_tokens + F) / (loc_ms * 1e-3) / 1e12

    top1, logit_mse, stage2_ms = (None, None, None) if args.no_measures else \
        top1_shift_per_mode(w, cfg, k, v, q, qh, kh, vh, args.seed, qwm, torch)

    stored, resident, original = qwm.footprint(cfg, w.n_tokens)
    res = {
        "metric": METRIC,
        "value": round(w.n_tokens / (ms_step * 1e-3) / 1e3, 3),
        "unit": "Ktokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16" if w.io == "bf16" else "f32",
        "data": "synthetic (seeded workloads module: lognormal-scaled K/V with outlier channels, "
                "8-direction queries); centres and statistics calibrated by the library",
        "config": {"workload": w.name, "heads": w.heads, "head_dim": w.head_dim, "frame_tokens": w.frame_tokens,
                   "cached_frames": w.frames, "cached_tokens": w.n_tokens, "query_chunk": w.n_q,
                   "centroids_k": w.c_k, "centroids_v": w.c_v, "top_candidates": w.top_k, "rank": w.rank,
                   "group_tokens": w.group_tokens, "io_dtype": w.io, "parallelism": "single GPU",
                   "input_copies_rotated": copies,
                   "launch": "eager" if args.no_graph else "hip graph per step (one per input copy)"},
        "ms_per_step_eager": round(wall_eager * 1e3 / args.steps, 4),
        "append": {"ms": round(app_avg, 4), "ktokens_s": round(w.n_tokens / (app_avg * 1e-3) / 1e3, 3),
                   "token_heads_s": round(tok_heads / (app_avg * 1e-3), 1),
                   "algorithmic_gbs": round(app_gbs, 2), "frac_hbm": round(app_gbs / PEAK_HBM_GBS, 4),
                   "bytes_per_token_head": round(append_bytes_per_token_head(w, cfg), 2)},
        "attention": {"ms": round(att_avg, 4), "kernel_ms": round(attk_avg, 4),
                      "combine_ms": round(max(att_avg - attk_avg, 0.0), 4), "tflops": round(achieved_tf, 2),
                      "frac_mfma": round(achieved_tf / PEAK_FP16_TFLOPS, 4),
                      "flops_per_launch": flops,
                      "compressed_cache_gbs": round(stored / (attk_avg * 1e-3) / 1e9, 2),
                      "compressed_cache_streamed_gbs": round(stored * query_blocks(w) / (attk_avg * 1e-3) / 1e9, 2),
                      "counter_hbm_gbs": counter_gbs("attention", w.name, src_hash, attk_avg)},
        "attention_local": {"ms": round(loc_ms, 4), "local_tokens": F, "tflops": round(loc_tf, 2),
                            "frac_mfma": round(loc_tf / PEAK_FP16_TFLOPS, 4),
                            "flops_per_call": attn_flops(w, w.n_q, w.n_tokens + F)},
        "roofline": roofline,
        "compression": {"ratio": round(original / stored, 4), "ratio_resident": round(original / resident, 4),
                        "stored_bytes": stored, "original_bytes": original},
        "top1_shift": top1,
        "logit_mse": logit_mse,
        "append_ms_by_stage2_score": stage2_ms,
        "top8_energy_mean": round(float(energy.mean()), 4),
        "kernel_source_hash": src_hash,
        "cpu_baseline": None,
    }
    if args.copy_probe_mib:
        n = args.copy_probe_mib * 2**20 // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = n * 4
    if not args.no_cpu_baseline:
        # the whole Matrix-Game-2-like step (about 6 s of host work); one or
        # two heads of the larger workloads, scaled to the full step
        heads = args.cpu_heads or max(1, min(w.heads, {"tiny": 1, "matrix_game": w.heads}.get(w.name, 2)))
        res["cpu_baseline"] = cpu_baseline(w, data, cfg, heads, args.seed)
    print(json.dumps(res), flush=True)


def rollout_epochs(args, w, cfg, ks, vs, q, qh, out, lse, ws, qwm, torch):
    """The 1-minute rollout with calibration epochs: every `epoch_frames`
    frames the library calibrates again (Query statistics from the query
    history, centres from the last cached frame) and the frames that follow go
    to a new cache bound to that calibration; each step attends over all
    epochs' caches in one launch.  Calibration is host work and untimed (its
    mean wall time is reported apart)."""
    import numpy as np
    F, E = w.frame_tokens, args.epoch_frames
    n_ep = -(-w.frames // E)
    import dataclasses
    ecfg = dataclasses.replace(cfg, max_frames=E)
    caches, cal_s = [], []
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(w.frames)]
    for f in range(w.frames):
        if f % E == 0:
            t0 = time.perf_counter()
            calib = qwm.alloc_calib(ecfg)
            if f == 0:
                src = (qh, ks[0][:, :F], vs[0][:, :F])
            else:
                src = (qh, ks[0][:, (f - 1) * F:f * F], vs[0][:, (f - 1) * F:f * F])
            qwm.calibrate(ecfg, calib, *src, seed=args.seed + f, iters=w.kmeans_iters)
            caches.append(qwm.Cache(ecfg, calib))
            cal_s.append(time.perf_counter() - t0)
            print("[bench] epoch %d calibrated at frame %d in %.1fs" % (len(caches) - 1, f, cal_s[-1]),
                  file=sys.stderr, flush=True)
        e = ev[f]
        e[0].record()
        qwm.append_kv(caches[-1], ks[0][:, f * F:(f + 1) * F], vs[0][:, f * F:(f + 1) * F])
        e[1].record()
        qwm.attention_epochs(caches, q, out=out, lse=lse, workspace=ws)
        e[2].record()
    torch.cuda.synchronize()
    app = np.array([e[0].elapsed_time(e[1]) for e in ev])
    att = np.array([e[1].elapsed_time(e[2]) for e in ev])
    tf_final = attn_flops(w, w.n_q, w.frames * F) / (att[-1] * 1e-3) / 1e12
    return {"epoch_frames": E, "epochs": n_ep, "append_ms_median": round(float(np.median(app)), 4),
            "attention_ms_median": round(float(np.median(att)), 4),
            "attention_ms_final": round(float(att[-1]), 4), "attention_tflops_final": round(float(tf_final), 2),
            "calibration_s_mean": round(float(np.mean(cal_s)), 3),
            "launch": "one attention launch over all epochs' caches per step (combine pass included)"}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline_generation_step(w, seed, heads=2, prefix=None):
    """The oracle (untuned) on a bounded sample of the generation step: for
    the first `heads` heads, the quantize-append of the newest frame (Keys and
    Values) and the attention of the query chunk over the rebuilt first
    `prefix` cached frames (the rebuild from the stored fields plus the
    softmax).  The attention part is scaled to all cached frames (its cost is
    linear in the cached tokens) and the whole to all heads.  The oracle's
    append of the prefix frames is untimed setup."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import workloads
    from oracle import attention as oa
    from oracle import calibrate as oc
    from oracle import codec
    F, T, nf = w.frame_tokens, w.group_tokens, w.frames
    prefix = nf - 1 if prefix is None else min(prefix, nf - 1)
    t_app = t_att = 0.0
    for h in range(heads):
        k0 = workloads.kv_frames(w, h, "k", 0, prefix)
        v0 = workloads.kv_frames(w, h, "v", 0, prefix)
        k_last = workloads.kv_frames(w, h, "k", nf - 1, nf)
        v_last = workloads.kv_frames(w, h, "v", nf - 1, nf)
        q0 = workloads.queries(w, h, w.n_q, historical=False)
        qh0 = workloads.queries(w, h, w.n_q_hist, historical=True)
        cal = oc.calibrate(qh0[None], k0[None, :F], v0[None, :F], w.c_k, w.c_v, w.rank, w.io, seed=seed + 2 * h, iters=2)
        mk, mv, sk, uk = cal["mu_k"][0], cal["mu_v"][0], cal["sens"][0], cal["u"][0]

        def append(f, k, v):
            return f, codec.append_keys(k, mk, sk, uk, F, T, w.top_k, 0), codec.append_values(v, mv, F, T)
        with ThreadPoolExecutor(8) as ex:
            parts = sorted(ex.map(lambda f: append(f, k0[f * F:(f + 1) * F], v0[f * F:(f + 1) * F]), range(prefix)),
                           key=lambda x: x[0])
        ko = {key: np.concatenate([p[1][key] for p in parts]) for key in ("idx", "codes", "z", "s", "coef", "coef_scale")}
        vo = {key: np.concatenate([p[2][key] for p in parts]) for key in ("idx", "codes", "z", "s")}
        del parts
        t0 = time.perf_counter()
        append(nf - 1, k_last, v_last)
        t_app += time.perf_counter() - t0
        t0 = time.perf_counter()
        kr = oa.reconstruct_keys(ko["idx"], ko["codes"], ko["z"], ko["s"], ko["coef"], ko["coef_scale"], mk, uk, F, T)
        vr = oa.reconstruct_values(vo["idx"], vo["codes"], vo["z"], vo["s"], mv, F, T)
        oa.softmax_attention(q0, kr, vr)
        t_att += time.perf_counter() - t0
        del kr, vr
        print("[bench] oracle baseline head %d done" % h, file=sys.stderr, flush=True)
    step_s = (t_app + t_att * nf / prefix) * w.heads / heads  # prefix nf - 1: within 0.4 % of the whole cache
    blas = blas_threads()
    cores = len(os.sched_getaffinity(0))
    return {"value": round(w.n_tokens / step_s / 1e3, 4), "unit": "Ktokens/s", "cores": int(min(cores, max(blas, 1))),
            "kind": "oracle", "step_s": round(step_s, 2),
            "sample": "heads 0..%d of %d at the final generation step: the oracle's quantize-append of the newest "
                      "frame (%.2f s in all) and its attention of %d queries over the rebuilt first %d of %d cached "
                      "frames (%.2f s in all, scaled x%g to all frames: the cost is linear in the cached tokens), "
                      "timed; the step scaled x%g to all heads; BLAS threads %d, affinity cores %d"
                      % (heads - 1, w.heads, t_app, w.n_q, prefix, nf, t_att, nf / prefix, w.heads / heads, blas, cores)}


def generation_step(args, w, qwm, torch, np, workloads, pool):
    """The 1-minute rollout.  Inputs are generated frame by frame in worker
    processes; the library calibrates from the first frame; the rollout leg
    appends each frame and attends the query chunk over the cache so far
    (eager, timed per step); then the timed step: the newest frame's
    append at position nf - 1 and attention over the full cache, first eager
    with per-kernel HIP events, then as HIP graphs (one per rotated copy of the
    newest frame's inputs) for ms_per_step."""
    import dataclasses
    F, nf, H, d = w.frame_tokens, w.frames, w.heads, w.head_dim
    cfg = qwm.Config(heads=H, head_dim=d, frame_tokens=F, max_frames=nf, c_k=w.c_k, c_v=w.c_v,
                     group_tokens=w.group_tokens, top_k=w.top_k, rank=w.rank, io=w.io)
    t_gen = time.perf_counter()
    kd = torch.empty(H, nf * F, d, dtype=torch.bfloat16, device="cuda")
    vd = torch.empty_like(kd)
    loc = {}
    jobs = [(w, which, f) for f in range(nf + 1) for which in ("k", "v")]
    for (_, which, f), bits in zip(jobs, pool.imap(workloads.frame_bits, jobs, chunksize=2)):
        t = torch.from_numpy(bits).view(torch.bfloat16)
        if f < nf:
            (kd if which == "k" else vd)[:, f * F:(f + 1) * F].copy_(t)
        else:
            loc[which] = t.to("cuda")
        if which == "v" and f % 40 == 0:
            print("[bench] generated frame %d" % f, file=sys.stderr, flush=True)
    q = torch.from_numpy(np.stack([workloads.queries(w, h, w.n_q, False) for h in range(H)])).to("cuda").to(
        torch.bfloat16)
    qh = torch.from_numpy(np.stack([workloads.queries(w, h, w.n_q_hist, True) for h in range(H)])).to("cuda").to(
        torch.bfloat16)
    torch.cuda.synchronize()
    print("[bench] minute: generated in %.1fs" % (time.perf_counter() - t_gen), file=sys.stderr, flush=True)

    calib = qwm.alloc_calib(cfg)
    t_cal = time.perf_counter()
    energy = qwm.calibrate(cfg, calib, qh, kd[:, :F], vd[:, :F], seed=args.seed, iters=w.kmeans_iters)
    print("[bench] calibrated in %.1fs (top-%d energy mean %.3f)" % (time.perf_counter() - t_cal, w.rank,
          float(energy.mean())), file=sys.stderr, flush=True)
    cache = qwm.Cache(cfg, calib)
    ws = torch.empty(qwm.workspace_bytes(cfg, w.n_tokens + F, w.n_q), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(H, w.n_q, dtype=torch.float32, device="cuda")

    # ---- rollout leg: append frame f, attend over frames 0..f (eager) ----
    rollout = None
    if args.no_rollout:
        for f in range(nf):
            qwm.append_kv(cache, kd[:, f * F:(f + 1) * F], vd[:, f * F:(f + 1) * F])
    else:
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(nf)]
        for e in ev:
            for x in e:
                x.record()
        torch.cuda.synchronize()
        for f in range(nf):
            e = ev[f]
            e[0].record()
            qwm.append_kv(cache, kd[:, f * F:(f + 1) * F], vd[:, f * F:(f + 1) * F])
            e[1].record()
            qwm.attention(cache, q, out=out, lse=lse, workspace=ws, kernel_events=(e[3], e[4]))
            e[2].record()
            if f % 40 == 0:
                print("[bench] rollout frame %d" % f, file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        r_app = np.array([e[0].elapsed_time(e[1]) for e in ev])
        r_att = np.array([e[1].elapsed_time(e[2]) for e in ev])
        r_attk = np.array([e[3].elapsed_time(e[4]) for e in ev])
        r_tf = np.array([attn_flops(w, w.n_q, (f + 1) * F) for f in range(nf)]) / (r_attk * 1e-3) / 1e12
        rollout = {"steps": nf, "append_ms_median": round(float(np.median(r_app)), 4),
                   "attention_ms_median": round(float(np.median(r_att)), 4),
                   "attention_ms_final": round(float(r_att[-1]), 4),
                   "attention_tflops_final": round(float(r_tf[-1]), 2),
                   "attention_tflops_steady_median": round(float(np.median(r_tf[len(r_tf) // 2:])), 2),
                   "total_ms": round(float(r_app.sum() + r_att.sum()), 2),
                   "launch": "eager, one append and one attention call per generated frame"}
    torch.cuda.synchronize()

    # ---- the timed generation step at the full cache ----
    n_prev = (nf - 1) * F
    frame_bytes = 2 * H * F * d * 2
    copies = max(1, math.ceil(512 * 2**20 / frame_bytes))
    kl_c = [kd[:, n_prev:].clone() for _ in range(copies)]
    vl_c = [vd[:, n_prev:].clone() for _ in range(copies)]

    def step(i, e=None):
        cache.truncate(n_prev)
        if e: e[0].record()
        qwm.append_kv(cache, kl_c[i % copies], vl_c[i % copies])
        if e: e[1].record()
        qwm.attention(cache, q, out=out, lse=lse, workspace=ws, kernel_events=(e[2], e[3]) if e else None)

    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in sev:
        for x in e:
            x.record()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, sev[i])
    torch.cuda.synchronize()
    wall = wall_eager = time.perf_counter() - t0
    if not args.no_graph:
        graphs = []
        for i in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    app_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in sev]))
    attk_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in sev]))
    att_call_ms = float(np.mean([e[1].elapsed_time(e[3]) for e in sev]))  # append end to kernel end
    ms_step = wall * 1e3 / args.steps
    flops = attn_flops(w, w.n_q, w.n_tokens)
    tf = flops / (attk_ms * 1e-3) / 1e12
    app_bytes = H * F * append_bytes_per_token_head(w, cfg)
    app_gbs = app_bytes / (app_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    stored, resident, original = qwm.footprint(cfg, w.n_tokens)
    print("[bench] step %.3f ms (graph), %.3f ms eager; attention kernel %.3f ms, append %.4f ms"
          % (ms_step, wall_eager * 1e3 / args.steps, attk_ms, app_ms), file=sys.stderr, flush=True)

    # ---- one generation step with the chunk's own keys and values ----
    for _ in range(3):
        qwm.attention_local(cache, q, loc["k"], loc["v"], out=out, lse=lse, workspace=ws)
    el = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
    torch.cuda.synchronize()
    for e in el:
        e[0].record()
        qwm.attention_local(cache, q, loc["k"], loc["v"], out=out, lse=lse, workspace=ws)
        e[1].record()
    torch.cuda.synchronize()
    loc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in el]))
    loc_tf = attn_flops(w, w.n_q, w.n_tokens + F) / (loc_ms * 1e-3) / 1e12

    res = {
        "metric": METRIC,
        "value": round(w.n_tokens / (ms_step * 1e-3) / 1e3, 3),
        "unit": "Ktokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded workloads module: lognormal-scaled K/V with outlier channels, "
                "8-direction queries); centres and statistics calibrated by the library from the first frame",
        "config": {"workload": w.name, "heads": H, "head_dim": d, "frame_tokens": F, "cached_frames": nf,
                   "cached_tokens": w.n_tokens, "query_chunk": w.n_q, "centroids_k": w.c_k, "centroids_v": w.c_v,
                   "top_candidates": w.top_k, "rank": w.rank, "group_tokens": w.group_tokens, "io_dtype": w.io,
                   "parallelism": "single GPU",
                   "step": "generation step at the full cache: append of frame %d + attention over %d tokens"
                           % (nf, w.n_tokens),
                   "input_copies_rotated": copies,
                   "launch": "eager" if args.no_graph else "hip graph per step (one per input copy)"},
        "ms_per_step_eager": round(wall_eager * 1e3 / args.steps, 4),
        "append": {"ms": round(app_ms, 4), "tokens": F,
                   "token_heads_s": round(H * F / (app_ms * 1e-3), 1),
                   "algorithmic_gbs": round(app_gbs, 2), "frac_hbm": round(app_gbs / PEAK_HBM_GBS, 4),
                   "bytes_per_token_head": round(append_bytes_per_token_head(w, cfg), 2)},
        "attention": {"kernel_ms": round(attk_ms, 4), "call_ms": round(att_call_ms, 4),
                      "tflops": round(tf, 2), "frac_mfma": round(tf / PEAK_FP16_TFLOPS, 4),
                      "flops_per_launch": flops,
                      "compressed_cache_gbs": round(stored / (attk_ms * 1e-3) / 1e9, 2),
                      "compressed_cache_streamed_gbs": round(stored * query_blocks(w) / (attk_ms * 1e-3) / 1e9, 2),
                      "counter_hbm_gbs": counter_gbs("attention", w.name, src_hash, attk_ms)},
        "attention_local": {"ms": round(loc_ms, 4), "local_tokens": F, "tflops": round(loc_tf, 2),
                            "frac_mfma": round(loc_tf / PEAK_FP16_TFLOPS, 4)},
        "roofline": {"kernel": "attn_bf16_kernel (dequant-attention, full cache)", "bound": "mfma",
                     "achieved": round(tf, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_FP16_TFLOPS, 4),
                     "traffic": traffic_from_profiles("attention", w.name, src_hash),
                     "algorithmic_flops_per_launch": flops, "ms_per_launch": round(attk_ms, 4)},
        "rollout": rollout,
        "compression": {"ratio": round(original / stored, 4), "ratio_resident": round(original / resident, 4),
                        "stored_bytes": stored, "resident_bytes": resident, "original_bytes": original},
        "top8_energy_mean": round(float(energy.mean()), 4),
        "kernel_source_hash": src_hash,
        "cpu_baseline": None,
    }
    if args.epoch_frames:
        res["calibration_epochs"] = rollout_epochs(args, w, cfg, [kd], [vd], q, qh, out, lse, ws, qwm, torch)
    if not args.no_measures:
        # quality measures on the prefix of the first measure-frames frames
        mf = args.measure_frames
        wp = dataclasses.replace(w, frames=mf)
        cp = dataclasses.replace(cfg, max_frames=mf)
        print("[bench] quality measures on the first %d frames" % mf, file=sys.stderr, flush=True)
        kp, vp = kd[:, :mf * F], vd[:, :mf * F]
        top1, mse, s2 = top1_shift_per_mode(wp, cp, kp, vp, q, qh, kd[:, :F], vd[:, :F], args.seed, qwm, torch)
        res["measures"] = {"frames": mf, "top1_shift": top1, "logit_mse": mse, "append_ms_by_stage2_score": s2}
    if args.copy_probe_mib:
        n = args.copy_probe_mib * 2**20 // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = n * 4
    if not args.no_cpu_baseline:
        print("[bench] oracle baseline of the generation step (two heads, whole cache)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_generation_step(w, args.seed)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
