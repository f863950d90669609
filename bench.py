"""Benchmark: one tile-sparse video attention layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3a]

A step is one whole layer over one batch of synthetic input already resident
in HBM: tile map + gather, tile scores, top-k selection and the sparse
attention, all in the library's kernels. Prints ONE JSON line.

value = effective TFLOP/s of the whole layer (4*d * real query-key pairs the
attention visits / step time). ms_per_step is the median of K steps, each
timed with events on the stream the library launches on (the wall-clock
mean of the same K steps is reported beside it). The roofline object covers
the dominant kernel (the bf16 attention), timed the same way. The other
workloads are reported beside the headline, each with the same library's
dense path (sparsity 0) for the speed-up. The CPU baseline is the oracle on
a bounded sample of the headline workload.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
HBM_PEAK_GBS = 8000.0
# Workloads reported beside the headline by default.
DEFAULT_ALSO = "3b,2,4a,4b,5,3a-h3,3b-r2va,3a-fp8"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="3a")
    ap.add_argument("--also", default=DEFAULT_ALSO,
                    help="extra workloads reported beside, ',' list; a '-h3' suffix keeps "
                         "only heads 0-2 (one GPU's share of 24 heads over 8 GPUs); "
                         "'-r2va' runs the two-stream budget (32 reference tiles of the "
                         "reference-image segment and 32 video tiles per query tile); "
                         "'-fp8' runs the E4M3 attention variant (its gather also writes the "
                         "E4M3 tiles). Plain workloads also time their dense path.")
    ap.add_argument("--fp8", action="store_true",
                    help="with --profile-attn-only: run the E4M3 variant of the layer")
    ap.add_argument("--dense-steps", type=int, default=5,
                    help="timed steps of the headline's dense path")
    ap.add_argument("--also-steps", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-recall", action="store_true",
                    help="skip the teacher tile-map recall measurement")
    ap.add_argument("--profile-attn-only", action="store_true",
                    help="run only warmup+steps of the layer (for profilers)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="with --profile-attn-only: also run one plain device copy of this "
                         "many MiB (reference for the memory-traffic counters)")
    ap.add_argument("--overlap-probe", action="store_true",
                    help="only measure how exponentials share a SIMD with fp8 products "
                         "(vsa_mfma_probe kinds 1-3) and print one JSON line")
    return ap.parse_args()


_INPUTS = {}


def device_inputs(w):
    """Q, K, V of a workload on the device (bf16 or f32), drawn once per
    (seed, shape) and shared by every case that needs them; a workload with
    fewer heads takes the leading heads of a cached one (every head has its
    own random streams)."""
    import torch
    from workloads.inputs import make_qkv
    key = (w.seed, w.B, w.d, w.grid, tuple(w.prefix), w.dtype)
    hit = _INPUTS.get(key)
    if hit is not None and hit[0].shape[1] >= w.H:
        return [x[:, : w.H].contiguous() if x.shape[1] > w.H else x for x in hit]
    t0 = time.time()
    bits = w.dtype == "bf16"
    q, k, v = make_qkv(w, as_bf16_bits=bits)
    dev = [torch.from_numpy(x).cuda() for x in (q, k, v)]
    del q, k, v
    if bits:
        dev = [x.view(torch.bfloat16) for x in dev]
    torch.cuda.synchronize()
    log(f"[bench] inputs {w.name} ({w.H} heads) drawn in {time.time() - t0:.1f}s")
    _INPUTS[key] = dev
    return dev


def drop_inputs():
    import torch
    _INPUTS.clear()
    torch.cuda.empty_cache()


class Case:
    """Library buffers and inputs for one workload, resident on the GPU."""

    def __init__(self, wname: str, sparsity=None, heads=None, ref=None, workload=None,
                 fp8=False):
        import dataclasses

        import torch
        from block_sparse_video_map_amd import vsa
        from workloads import WORKLOADS
        from workloads.inputs import make_weights
        w = WORKLOADS[wname] if workload is None else workload
        if heads is not None:
            w = dataclasses.replace(w, H=heads)
        self.w = w
        self.sparsity = w.sparsity if sparsity is None else sparsity
        self.prob = vsa.Problem(w.B, w.H, w.d, w.grid, w.prefix, w.tile_shapes, w.dtype)
        mode = vsa.score_mode(w.scorer, w.tripool_mode)
        proj = w.d if w.scorer == "mean_gate" else w.proj_dim
        self.ref = ref
        self.fp8 = fp8
        self.layer = vsa.Layer(self.prob, self.sparsity, mode, proj, with_lse=False, ref=ref,
                               fp8=fp8)
        self.q, self.k, self.v = device_inputs(w)
        W = make_weights(w)
        if w.scorer == "mean_gate":
            self.wq, self.wk = torch.from_numpy(W["gate"]).cuda(), None
        else:
            self.wq = torch.from_numpy(W["proj_q"]).cuda()
            self.wk = torch.from_numpy(W["proj_k"]).cuda()
        torch.cuda.synchronize()

    def step(self):
        self.layer.forward(self.q, self.k, self.v, self.wq, self.wk)

    def flops(self) -> float:
        """Effective FLOPs of the attention on this case's selection."""
        import torch
        from block_sparse_video_map_amd import vsa
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.step()                    # the first (cold) call: code objects load here
        torch.cuda.synchronize()
        self.cold_ms = (time.perf_counter() - t0) * 1e3
        s2t = self.layer.slot_to_token.cpu().numpy()
        kv = None if self.sparsity == 0.0 else self.layer.kv_idx.cpu().numpy()
        if self.ref is not None:
            return vsa.vsa_count_flops_ref(self.prob, self.sparsity, self.layer.budget, s2t, kv,
                                           self.layer.ref_idx.cpu().numpy())
        return vsa.vsa_count_flops(self.prob, self.sparsity, s2t, kv)

    def time_steps(self, steps: int, warmup: int):
        """(median ms from events around each step on the launch stream, wall
        mean ms over the same steps)."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(steps):
            self.step()
            ev[i + 1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps * 1e3
        ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        return ms[len(ms) // 2], wall

    def stage_times(self, reps: int):
        """Median and mean ms per stage, from events on the launch stream."""
        import torch
        L = self.layer
        names = ["map_gather", "scores", "select", "attention"]
        fns = [lambda: L.map_tiles(self.q, self.k, self.v),
               lambda: L.tile_scores(self.wq, self.wk),
               L.select, L.attend]
        if self.sparsity == 0.0:
            names, fns = [names[0], names[3]], [fns[0], fns[3]]
        elif L.fused:                      # pooling, scores and top-k in one call
            names = [names[0], "score_select", names[3]]
            fns = [fns[0], lambda: L.score_select(self.wq, self.wk), fns[3]]
        elif L.gather_pool:                # gather with the tile means, gate, scores
            names = ["map_gather_scores", names[2], names[3]]
            fns = [lambda: L.map_tiles_scores(self.q, self.k, self.v, self.wq, self.wk),
                   fns[2], fns[3]]
        if self.fp8:                       # the gather writes the E4M3 tiles too
            names[0] = "map_gather_fp8"
            fns[0] = lambda: L.map_tiles_fp8(self.q, self.k, self.v)
        samples = {n: [] for n in names}
        for _ in range(reps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
            ev[0].record()
            for i, f in enumerate(fns):
                f()
                ev[i + 1].record()
            torch.cuda.synchronize()
            for i, n in enumerate(names):
                samples[n].append(ev[i].elapsed_time(ev[i + 1]))
        med = {n: float(sorted(v)[len(v) // 2]) for n, v in samples.items()}
        mean = {n: float(sum(v) / len(v)) for n, v in samples.items()}
        return med, mean

    def fused_select_ms(self, reps: int = 5):
        """Median ms of vsa_tile_select (pooling, scores and top-k in one call,
        no score matrix) beside the two calls it replaces, on this layer's
        tiles; None where the call does not take the problem."""
        import torch
        from block_sparse_video_map_amd import vsa
        L = self.layer
        if self.sparsity == 0.0 or not vsa.fused_select_supported(
                self.prob, L.mode, L.proj_dim, self.sparsity):
            return None
        kv = torch.empty_like(L.kv_idx)

        def fused():
            vsa.vsa_tile_select(self.prob, L.mode, L.proj_dim, L.qt, L.kt, L.slot_to_token,
                                self.wq, self.wk, self.sparsity, L.pooled, kv)

        def two():
            L.tile_scores(self.wq, self.wk)
            L.select()
        out = {}
        for name, fn in (("fused_call", fused), ("two_calls", two)):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            out[name + "_ms"] = round(sorted(ts)[len(ts) // 2], 4)
        out["lists_equal"] = bool(torch.equal(kv[: L.sizes.idx_elems],
                                              L.kv_idx[: L.sizes.idx_elems]))
        return out

    def stage_bytes(self) -> dict:
        """Algorithmic HBM bytes of the HBM-bound stages (each input read and
        each output written once)."""
        w, sz = self.w, self.layer.sizes
        es = 2 if w.dtype == "bf16" else 4
        ns = len(w.tile_shapes)
        heads = [h % ns for h in range(w.H)]
        tiles = sum(sz.n_tiles[s] for s in heads) * w.B
        vt = sum(sz.n_video_tiles[s] for s in heads) * w.B
        vt2 = sum(sz.n_video_tiles[s] ** 2 for s in heads) * w.B
        kk = sum(sz.n_video_tiles[s] * sz.k[s] for s in heads) * w.B
        nstat = {"triplet": 3, "maxmin": 2, "avg": 1}[w.tripool_mode]
        r = w.d if w.scorer == "mean_gate" else nstat * w.proj_dim
        out = {"map_gather": 3 * es * w.B * w.H * w.N * w.d + 3 * es * tiles * 64 * w.d}
        if self.sparsity != 0.0 and self.layer.gather_pool:
            # the gather with the pooling, descriptors written (and gated in place for
            # the mean gate) and read by the scores
            out.pop("map_gather")
            out["map_gather_scores"] = (3 * es * w.B * w.H * w.N * w.d + 3 * es * tiles * 64 * w.d
                                        + 4 * 8 * vt * r + 4 * vt2)
            out["select"] = 4 * vt2 + 4 * kk
        elif self.sparsity != 0.0 and self.layer.fused:
            # tiles read by the pooling, descriptors written and read back, lists written
            out["score_select"] = 2 * es * vt * 64 * w.d + 4 * 8 * vt * r + 4 * kk
        elif self.sparsity != 0.0:
            out["scores"] = 2 * es * vt * 64 * w.d + 2 * 8 * vt * r + 4 * vt2
            out["select"] = 4 * vt2 + 4 * kk
        return out

    def release(self):
        import torch
        del self.layer, self.q, self.k, self.v
        torch.cuda.empty_cache()


def dense_row(wname: str, steps: int, heads=None):
    """The same library's dense path (sparsity 0) on the workload's inputs."""
    c = Case(wname, sparsity=0.0, heads=heads)
    f = c.flops()
    ms, wall = c.time_steps(max(1, steps), 1)
    _, mean = c.stage_times(max(1, min(steps, 3)))
    c.release()
    return {"ms_per_step": round(ms, 3), "ms_per_step_wall_mean": round(wall, 3),
            "attention_ms": round(mean["attention"], 3), "steps": max(1, steps),
            "effective_tflop": f / 1e12,
            "effective_tflops_attention": f / mean["attention"] / 1e9}


def teacher_recall(wname: str):
    """Tile recall of the mean-gate and the TripPool selections against the
    teacher tile map (full attention max-pooled per tile pair), both at the
    workload's sparsity on the same synthetic inputs. A measurement: random
    untrained gates and projections, so the values are not the pages'."""
    import dataclasses

    import numpy as np
    import torch
    from block_sparse_video_map_amd import vsa
    from workloads import WORKLOADS
    w = WORKLOADS[wname]
    other = "trippool" if w.scorer == "mean_gate" else "mean_gate"
    base = Case(wname)
    alt = Case(wname, workload=dataclasses.replace(w, scorer=other))
    sels = {w.scorer: base, other: alt}
    for c in sels.values():
        c.step()
    sz = base.layer.sizes
    lse = torch.empty(w.B * w.H * sz.max_video_tiles * 64, dtype=torch.float32, device="cuda")
    teacher = torch.empty(sz.score_elems, dtype=torch.float32, device="cuda")
    top = torch.empty(sz.idx_elems, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    vsa.vsa_teacher_map(base.prob, base.layer.qt, base.layer.kt, base.layer.slot_to_token, 0.0,
                        lse, teacher)
    torch.cuda.synchronize()
    t_ms = (time.perf_counter() - t0) * 1e3
    vsa.vsa_select_topk(base.prob, teacher, base.sparsity, top)
    shp = (w.B * w.H, sz.max_video_tiles, sz.k_max)
    top = top.view(*shp).cpu().numpy()
    out = {}
    for name, c in sels.items():
        sel = c.layer.kv_idx[: sz.idx_elems].view(*shp).cpu().numpy()
        rec = []
        for bh in range(w.B * w.H):
            s = bh % w.H % len(w.tile_shapes)
            n, k = sz.n_video_tiles[s], sz.k[s]
            a, t = np.sort(sel[bh, :n, :k], axis=1), np.sort(top[bh, :n, :k], axis=1)
            hits = [np.intersect1d(x, y, assume_unique=True).size for x, y in zip(a, t)]
            rec.append(float(np.mean(hits)) / k)
        out[name] = round(float(np.mean(rec)), 4)
    alt.release()
    base.release()
    del lse, teacher
    out["teacher_map_ms"] = round(t_ms, 2)
    out["note"] = ("synthetic inputs, untrained gates/projections: a measurement of the "
                   "pipeline, not comparable to trained predictors")
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] + [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(wname: str, budget_s: float):
    """The oracle, as it stands (float64 NumPy), on a bounded sample of the
    workload: heads 0, 8 and 16, each with its full map, gather, pooling,
    scores and selection and then attention for as many query tiles (every
    prefix query tile first, then random video query tiles) as a third of
    the time budget allows. Reported as effective TFLOP/s of the sampled
    attention over the sampled time, and as milliseconds per layer
    extrapolated from the sample (per head: the measured pre-attention time
    plus the measured attention time per query tile times the head's query
    tiles; summed over the layer's heads)."""
    import numpy as np

    import oracle
    from workloads import WORKLOADS
    from workloads.inputs import head_qkv, make_weights
    w = WORKLOADS[wname]
    W = make_weights(w)
    heads = [h for h in (0, 8, 16) if h < w.H] or [0]
    per_head_budget = budget_s / len(heads)
    scale = 1.0 / np.sqrt(w.d)
    done_flops, sampled_s, n_done, pre_s, tile_s, tiles_all = 0, 0.0, 0, [], [], []
    for h in heads:
        q, k, v = head_qkv(w, 0, h)
        shape = w.tile_shapes[h % len(w.tile_shapes)]
        wq = W["gate"][h] if w.scorer == "mean_gate" else W["proj_q"][h]
        wk = None if w.scorer == "mean_gate" else W["proj_k"][h]
        t0 = time.perf_counter()
        r = oracle.head_forward(q, k, v, w.grid, w.prefix, shape, w.sparsity, w.scorer, wq,
                                wk, query_tiles=[], tripool_mode=w.tripool_mode)
        t_pre = time.perf_counter() - t0
        tm, allow = r["tmap"], r["allow"]
        order = list(range(tm.n_prefix_tiles)) + list(np.random.default_rng(h).permutation(
            np.arange(tm.n_prefix_tiles, tm.n_tiles)))
        real = tm.valid().sum(axis=1).astype(np.int64)
        t1 = time.perf_counter()
        n_tiles = 0
        for tq in order:
            oracle.sparse_attention(q, k, v, tm, allow, scale, query_tiles=[tq])
            done_flops += 4 * w.d * int(real[tq]) * int(allow[tq].astype(np.int64) @ real)
            n_tiles += 1
            if time.perf_counter() - t0 > per_head_budget:
                break
        t_att = time.perf_counter() - t1
        sampled_s += time.perf_counter() - t0
        n_done += n_tiles
        pre_s.append(t_pre)
        tile_s.append(t_att / max(1, n_tiles))
        tiles_all.append(tm.n_tiles)
    per_head_ms = (np.mean(pre_s) + np.mean(tile_s) * np.mean(tiles_all)) * 1e3
    return {"value": done_flops / sampled_s / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": (f"workload {wname}, heads {heads} of {w.H}: full map/gather/pool/score/"
                       f"select per head plus float64 attention of {n_done} query tiles "
                       f"(each head's prefix tiles first, then random video tiles) in "
                       f"{sampled_s:.1f}s"),
            "ms_per_layer_extrapolated": round(per_head_ms * w.H * w.B, 1),
            "seconds": round(sampled_s, 2), "cpu_model": cpu_model(),
            "nproc": os.cpu_count(), "blas_threads": blas_threads()}


def overlap_probe(iters: int = 20000) -> dict:
    """Shader cycles per trip of vsa_mfma_probe's fp8 kinds (median over
    workgroups of the span of their waves' loops), one workgroup per CU:
    four fp8 MFMAs per trip in one wave per SIMD (kind 1) or two (kind 2),
    two waves that each add 16 exponentials (kind 3), or one wave of products
    beside one that only runs the 16 exponentials (kind 4)."""
    import torch
    from block_sparse_video_map_amd import vsa
    cu, _, _ = vsa.vsa_device_clocks()
    rows = (("products, one wave per SIMD", 1, cu),
            ("products, two waves per SIMD", 2, cu),
            ("products + 16 exp in each wave, two waves per SIMD", 3, cu),
            ("products wave beside an exp wave on each SIMD", 4, cu))
    out = {"iters": iters, "mfma_cycles_per_trip_alone": 4 * 64, "rows": []}
    for name, kind, n_wg in rows:
        ticks = torch.zeros(4 * n_wg, dtype=torch.int64, device="cuda")
        vsa.vsa_mfma_probe(kind, iters, n_wg)        # warm-up
        vsa.vsa_mfma_probe(kind, iters, n_wg, ticks)
        torch.cuda.synchronize()
        tk = ticks.view(n_wg, 4).cpu().double()
        cyc = float(((tk[:, 1] - tk[:, 0]) / iters).median())
        out["rows"].append({"case": name, "kind": kind, "workgroups": n_wg,
                            "cycles_per_trip": round(cyc, 1)})
    return out


def measured_peak(reps: int = 5) -> dict:
    """The matrix-core rate the chip sustains under a pure MFMA load (bf16
    and fp8), and the clocks behind it: the engine clock the runtime reports
    (the maximum, which the published peaks assume), the clock the shader
    tick counter shows during the load, and the effective clock that the
    sustained bf16 rate implies at 4096 flop per clock per CU."""
    import torch
    from block_sparse_video_map_amd import vsa
    cu, clk_khz, wall_khz = vsa.vsa_device_clocks()
    n_wg = 2 * cu                                   # two waves on every SIMD
    out = {"cus": cu, "reported_clock_ghz": clk_khz / 1e6,
           "peak_at_reported_clock_tflops": {"bf16": cu * clk_khz * 1e3 * 4096 / 1e12,
                                             "fp8": cu * clk_khz * 1e3 * 8192 / 1e12}}
    ticks = torch.zeros(4 * n_wg, dtype=torch.int64, device="cuda")
    for kind, name, iters, per_clk in ((0, "bf16", 60000, 4096), (1, "fp8", 30000, 8192)):
        vsa.vsa_mfma_probe(kind, iters, n_wg)       # warm-up
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f = vsa.vsa_mfma_probe(kind, iters, n_wg, ticks)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        t = sorted(ms)[len(ms) // 2]
        rate = f / (t * 1e-3) / 1e12
        tk = ticks.view(n_wg, 4).cpu().double()
        dt, dr = tk[:, 1] - tk[:, 0], tk[:, 3] - tk[:, 2]
        ok = dr > 0
        tick_ghz = float((dt[ok] / dr[ok]).median()) * wall_khz / 1e6 if ok.any() else None
        out[f"probe_{name}"] = {"tflops": round(rate, 1), "ms": round(t, 4),
                                "effective_clock_ghz": round(rate * 1e12 / (cu * per_clk) / 1e9,
                                                             4),
                                "shader_tick_clock_ghz": None if tick_ghz is None
                                else round(tick_ghz, 4)}
    return out


def also_row(label: str, steps: int):
    """One workload reported beside the headline."""
    from block_sparse_video_map_amd.profsum import read_traffic
    name, heads, ref, sp, fp8 = label, None, None, None, False
    if name.endswith("-fp8"):         # E4M3 attention variant (reduced precision)
        name, fp8 = name[:-4], True
    if name.endswith("-h3"):          # one GPU's share when 8 GPUs split the heads
        name, heads = name[:-3], 3
    if name.endswith("-r2va"):        # two-stream budget: 32 + 32 tiles per query tile
        name, ref, sp = name[:-5], (1, 32), 0.9819
    plain = not (fp8 or heads or ref)
    c = Case(name, heads=heads, ref=ref, sparsity=sp, fp8=fp8)
    f = c.flops()
    ms, wall = c.time_steps(max(3, steps), 2)
    med, mean = c.stage_times(5)
    att = mean["attention"]
    row = {"ms_per_step": round(ms, 4), "ms_per_step_wall_mean": round(wall, 4),
           "effective_tflops_layer": f / ms / 1e9, "attention_ms": round(att, 4),
           "effective_tflops_attention": f / att / 1e9, "effective_tflop": f / 1e12,
           "stage_ms_median": med}
    if plain:
        row["fused_select"] = c.fused_select_ms()
    c.release()
    if fp8:
        row["precision"] = ("E4M3 Q/K/V and probabilities, fp32 accumulation, bf16 output: a "
                            "reduced-precision variant, not the headline")
        row["frac_of_fp8_peak"] = round(f / att / 1e9 / FP8_PEAK_TFLOPS, 4)
        rec = read_traffic(os.path.join(ROOT, "profiles", f"attn_fp8_{name}_traffic.md"),
                           "attn_fp8_kernel", name) if heads is None else None
        row["traffic"] = rec["bytes_per_launch"] if rec else None
    else:
        row["roofline_frac"] = round(f / att / 1e9 / BF16_PEAK_TFLOPS, 4)
    if plain:
        big = c.w.N * c.w.H > 4_000_000
        dense = dense_row(name, 1 if big else 3)
        row["dense"] = dense
        row["speedup_vs_dense_layer"] = round(dense["ms_per_step"] / ms, 3)
    return row


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {a.gpus}); the path shards by head "
              "across GPUs with no exchange; this benchmark runs one GPU.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    from block_sparse_video_map_amd import vsa
    from workloads import WORKLOADS

    if a.overlap_probe:
        print(json.dumps(overlap_probe()), flush=True)
        return
    w = WORKLOADS[a.workload]
    if a.fp8 and not a.profile_attn_only:
        print("--fp8 only applies to --profile-attn-only (the headline is the bf16 path)",
              file=sys.stderr)
        sys.exit(2)
    case = Case(a.workload, fp8=a.fp8)
    flops = case.flops()
    if a.profile_attn_only:
        case.time_steps(a.steps, a.warmup)
        if a.copy_calibration_mib:
            n = a.copy_calibration_mib * (1 << 20) // 4
            src = torch.ones(n, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            dst.copy_(src)
            torch.cuda.synchronize()
        log("[bench] profile run done")
        return
    cold_ms = case.cold_ms
    ms_step, wall_step = case.time_steps(a.steps, a.warmup)
    med, mean = case.stage_times(max(5, a.steps))
    kept, frac = vsa.vsa_kept_stats(case.prob, case.sparsity)
    sbytes = case.stage_bytes()
    stage_gbs = {n: {"bytes": b, "GB/s": round(b / (mean[n] * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(b / (mean[n] * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}
                 for n, b in sbytes.items()}
    attn_ms = mean["attention"]
    achieved = flops / (attn_ms * 1e-3) / 1e12
    log(f"[bench] {a.workload}: {ms_step:.3f} ms/step (event median), attention "
        f"{attn_ms:.3f} ms, {achieved:.1f} TFLOP/s on kept tiles")
    fused_sel = case.fused_select_ms()
    case.release()

    dense = dense_row(a.workload, a.dense_steps)
    log(f"[bench] dense: {dense['ms_per_step']:.2f} ms/step")

    extra = {}
    for label in [x for x in a.also.split(",") if x]:
        extra[label] = also_row(label, a.also_steps)
        log(f"[bench] {label}: {extra[label]['ms_per_step']:.3f} ms/step")

    log("[bench] matrix-core probe (measured-clock peak)")
    mpeak = measured_peak()
    log(f"[bench] probe {mpeak}")
    for e in extra.values():
        if "frac_of_fp8_peak" in e:
            e["frac_of_measured_fp8"] = round(e["effective_tflops_attention"]
                                              / mpeak["probe_fp8"]["tflops"], 4)

    recall = None
    if not a.no_recall:
        log("[bench] teacher tile-map recall")
        recall = teacher_recall(a.workload)
        log(f"[bench] recall {recall}")
    drop_inputs()

    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] cpu baseline (oracle, bounded sample)")
        cpu = cpu_baseline(a.workload, a.cpu_seconds)

    T, Hv, Wv = w.grid
    from block_sparse_video_map_amd.profsum import read_traffic
    kname = "attn_bf16_kernel<128>" if w.d == 128 else "attn_bf16_kernel<64>"
    rec = read_traffic(os.path.join(ROOT, "profiles", f"attn_bf16_{a.workload}_traffic.md"),
                       "attn_bf16_kernel", a.workload)
    traffic = rec["bytes_per_launch"] if rec else None
    line = {
        "metric": "effective TFLOP/s on kept tiles + ms/layer at ~105k tokens, "
                  "75% sparsity, 1 GPU",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_wall_mean": round(wall_step, 4),
        "timing": "median of the steps, each bracketed by events on the launch stream",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) + low-frequency 3D sinusoid per channel; "
                "random N(0,1/d) gates)",
        "config": {"workload": f"{a.workload}: {w.name}", "B": w.B, "H": w.H, "d": w.d,
                   "video_grid": [T, Hv, Wv], "prefix": list(w.prefix),
                   "tokens": w.N, "tile_shapes": [list(s) for s in w.tile_shapes],
                   "scorer": w.scorer, "sparsity": w.sparsity},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per launch (HBM, scaled rocprofv3 counters)",
                     "kernel": kname,
                     "per_launch_flop": flops, "avg_launch_ms": round(attn_ms, 4),
                     "tile_granular_flop": 4.0 * w.d * 64 * 64 * kept,
                     "peak_measured": mpeak["probe_bf16"]["tflops"],
                     "frac_of_measured": round(achieved / mpeak["probe_bf16"]["tflops"], 4)},
        "measured_peak": mpeak,
        "cpu_baseline": cpu,
        "effective_tflop_per_layer": flops / 1e12,
        "attention_ms": round(attn_ms, 4),
        "cold_ms_first_step": round(cold_ms, 3),
        "stage_ms_median": med,
        "fused_select": fused_sel,
        "stage_ms_mean": mean,
        "stage_hbm": stage_gbs,
        "kept_tile_pairs": kept, "kept_fraction_of_full": round(frac, 5),
        "dense": dense,
        "speedup_vs_dense_layer": round(dense["ms_per_step"] / ms_step, 3),
        "also": extra,
        "teacher_recall": recall,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
