"""Benchmark of one segment-relocated MLA attention layer on one MI355X.

A step is one pass of the whole hot path on resident inputs: plan build (segment
geometry and RoPE tables, protected row set, work list) followed by the forward
(per-segment rotate / attend / restore with the log-sum-exp merge, then the
row-replacement epilogue). The default workload is the Flash-like 32K layer
(64 heads, 56 Local / 8 Global, 512 + 64 latent, 8 x 4096 documents after a 256-row
prefix, 128 question rows, 10 % Local budget); the 128K layer is measured as a
secondary figure, its 8 Global heads alone (every row, the part the throughput target is
stated on) as the "target" figure, the Pro-like 64K layer with the E4M3 latent as the
"fp8" figure, the layer of 256 short documents (a 256-way merge per question row) as the
"many_short" figure, and the 32K request with sink + window heads (56 heads with 4 sink tokens
and a 256-token window beside 8 Global heads; and every head a 128-token window, the SWA
layer) as the "window_heads" figures. A row-window plan of the 128K layer's last row (decode: one new row against
131,584 keys) is the "decode" figure, its whole forward against the HBM roofline (latent
rows, W, and the row's q, out and z moved once). The main workload over a paged latent pool
(64-row pages in shuffled order) is the "paged" figure, and the main workload with its
projected state in groups of 8 heads (z and the cache per group) the "grouped" figure. The
main request as DeepSeek-V4 compressed-history layers (a CSA layer: 128-token window and
512-entry lists of 4-to-1 entries; an HCA layer: 128-token window and every 128-to-1 entry),
every row and the last row alone, are the "dual_pool" figures. The main request prefilled in
eight row windows on one plan moved by segmla_plan_set_window is the "chunked_prefill" figure.
Throughput is algorithmic
attention TFLOP/s, 2 * (576 + 576) FLOP per computed (row, head, key) triple, divided by the
step time.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-secondary]
                [--no-target] [--no-fp8] [--many-short NAME] [--window NAMES] [--no-cpu-baseline]
                [--decode-rows N] [--decode-only] [--paged-rows P] [--grouped NAME]
                [--dual SPECS] [--dual-only] [--chunks N]
"""
import argparse
import json
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "segmented-MLA attention TFLOP/s and µs/layer at 32K/128K ctx, 1 MI355X"
PEAK_FP8_TFLOPS = 5000.0  # dense fp8 MFMA (the E4M3 path dequantizes to bf16 MFMA)
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def attn_traffic():
    """HBM bytes per attention launch from the committed counter summary, or None when the
    kernel source changed since the counters were taken."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "attn_mfma_flash32k_traffic.md")
    src = os.path.join(ROOT, "segmented_attention_amd", "csrc", "k_attn_mfma.hip")
    try:
        fields = dict(line.split(": ", 1) for line in open(prof) if ": " in line and
                      line.split(": ", 1)[0] in ("kernel_source_sha256", "attn_traffic_bytes_per_launch"))
        if fields.get("kernel_source_sha256", "").strip() != hashlib.sha256(open(src, "rb").read()).hexdigest():
            return None
        return int(fields["attn_traffic_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def flops_per_pair(cfg):
    d_qk = cfg["d_nope"] + cfg["d_rope"]
    d_v = d_qk if cfg["v_has_rope"] else cfg["d_nope"]
    return 2.0 * (d_qk + d_v)


def measure_window(inp, cfg, n_rows, steps, warmup):
    """Decode-shaped forward: a plan for the last n_rows request rows only (their full
    causal context over every segment), built once; HIP-event times per forward. The
    algorithmic bytes are what the whole forward must move at least once: the latent rows
    the window sees, W (every head's projection slice), and the window's q, out and z."""
    import torch
    from segmented_attention_amd import segmla as S

    T, H = inp["T"], cfg["n_heads"]
    q0 = T - n_rows
    dt = inp["q"].dtype
    G = cfg.get("group_heads", 0)
    slots = H // G if G >= 2 else H  # z vectors per row (per head, or per group of heads)
    out = torch.empty((n_rows, H, inp["d_v"]), dtype=dt, device="cuda")
    z = torch.empty((n_rows, slots, cfg["d_state"]), dtype=dt, device="cuda")
    plan = S.Plan.for_inputs(inp, q_range=(q0, T))
    plan.build(inp["scores"])
    for _ in range(warmup):
        plan.forward(inp, out, z)
    torch.cuda.synchronize()
    S.segmla_profile_enable(plan.handle, True)
    for _ in range(steps):
        plan.forward(inp, out, z)
    ms, n_fwd, _ = S.segmla_profile_read(plan.handle)
    S.segmla_profile_enable(plan.handle, False)
    torch.cuda.synchronize()
    eager_us, graph_us = forward_eager_and_graph_us(plan, inp, out, z, steps)
    plan.close()
    n = max(1, n_fwd)
    attn_us, merge_us, epi_us = (1e3 * ms[i] / n for i in range(3))
    d_qk = cfg["d_nope"] + cfg["d_rope"]
    row_bytes = d_qk * 2 if cfg["kv_dtype"] == "bf16" else cfg["d_nope"] + 4 * (cfg["d_nope"] // 128) + 2 * cfg["d_rope"]
    w_bytes = H * cfg["d_state"] * inp["d_v"] * 2
    nbytes = T * row_bytes + w_bytes + n_rows * (H * (d_qk + inp["d_v"]) + slots * cfg["d_state"]) * 2
    fwd_us = attn_us + merge_us + epi_us
    gbps = nbytes / (fwd_us * 1e-6) / 1e9
    return dict(rows=n_rows, keys=T, attention_us=attn_us, merge_us=merge_us, epilogue_us=epi_us,
                forward_us=fwd_us, bytes=nbytes, gbps=gbps, forward_us_eager=eager_us,
                forward_us_graph=graph_us)


def forward_eager_and_graph_us(plan, inp, out, z, reps):
    """The same forward without per-stage events: back-to-back launches, and replays of a HIP
    graph that captured one forward (its three kernels launch as one graph, without the host
    launch path between them). HIP-event times over `reps` forwards."""
    import torch

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    eager = timed(lambda: plan.forward(inp, out, z))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.forward(inp, out, z)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    graph = timed(g.replay)
    del g
    return eager, graph


def measure_decode_walk(inp, cfg, n_steps, warmup=3):
    """Decode walk: one plan for the request's final length, moved row by row over the last
    n_steps + warmup rows with segmla_plan_set_window (no geometry, table or protected-set
    rebuild); each step is the window update plus the forward, timed with HIP events on the
    launch stream."""
    import torch
    from segmented_attention_amd import segmla as S

    T, H = inp["T"], cfg["n_heads"]
    first = T - n_steps - warmup
    dt = inp["q"].dtype
    out = torch.empty((1, H, inp["d_v"]), dtype=dt, device="cuda")
    z = torch.empty((1, H, cfg["d_state"]), dtype=dt, device="cuda")
    plan = S.Plan.for_inputs(inp, q_range=(first, first + 1))
    plan.build(inp["scores"], min_bytes=2 * S.segmla_plan_workspace_bytes(plan.handle))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
    for k in range(n_steps + warmup):
        t = first + k
        if k >= warmup:
            ev[k - warmup].record()
        if k > 0:
            plan.set_window(t, t + 1)
        plan.forward(inp, out, z)
    ev[n_steps].record()
    torch.cuda.synchronize()
    plan.close()
    steps = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n_steps)]
    return dict(steps=n_steps, step_us_median=statistics.median(steps), step_us_min=min(steps))


def measure_chunked(cfg_name, n_chunks, steps, warmup=2):
    """Chunked prefill: the request's rows in n_chunks consecutive windows computed one after
    another on one plan, moved from chunk to chunk by segmla_plan_set_window (geometry, RoPE
    tables and the protected set built once). HIP-event time of the whole sequence (window
    updates and forwards) per prefill; the algorithmic FLOP are the whole request's."""
    import torch
    from segmented_attention_amd import segmla as S
    from workload import config_by_name, make_inputs

    cfg = config_by_name(cfg_name)
    log("workload %s: chunked prefill in %d windows (set_window + forward)" % (cfg_name, n_chunks))
    inp = make_inputs(cfg, "cuda")
    T, H = inp["T"], cfg["n_heads"]
    dt = inp["q"].dtype
    out = torch.empty((T, H, inp["d_v"]), dtype=dt, device="cuda")
    z = torch.empty((T, H, cfg["d_state"]), dtype=dt, device="cuda")
    whole = S.Plan.for_inputs(inp)
    whole.build(inp["scores"])
    whole.forward(inp, out, z)
    torch.cuda.synchronize()
    ws = S.segmla_plan_workspace_bytes(whole.handle)
    pairs = sum(whole.pairs())
    whole.close()
    edges = [T * k // n_chunks for k in range(n_chunks + 1)]
    for k in range(n_chunks):  # room for every chunk's window (host-side sizing only)
        pk = S.Plan.for_inputs(inp, q_range=(edges[k], edges[k + 1]))
        ws = max(ws, S.segmla_plan_workspace_bytes(pk.handle))
        pk.close()
    plan = S.Plan.for_inputs(inp, q_range=(edges[0], edges[1]))
    plan.build(inp["scores"], min_bytes=ws)

    def prefill():
        for k in range(n_chunks):
            q0, q1 = edges[k], edges[k + 1]
            if k > 0 or plan.q0 != q0:
                plan.set_window(q0, q1)
            plan.forward(inp, out[q0:q1], z[q0:q1])

    for _ in range(warmup):
        prefill()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        prefill()
    b.record()
    torch.cuda.synchronize()
    plan.close()
    ms = a.elapsed_time(b) / steps
    flops = flops_per_pair(cfg) * pairs
    del inp, out, z
    torch.cuda.empty_cache()
    return {"workload": cfg_name, "chunks": n_chunks, "rows_per_chunk": edges[1] - edges[0],
            "ms_per_prefill": round(ms, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
            "over": "window updates and forwards of every chunk; the plan is built once"}


def measure_prefetch(cfg_name, steps):
    """The layer's forward alone, then with the next layer's artifacts (its latent rows and the
    cached state of its first document) staged from pinned host memory on the prefetch stream
    at the same time; HIP-event times on the launch stream, the transfer time on the prefetch
    stream."""
    import torch
    from segmented_attention_amd import segmla as S
    from workload import config_by_name, make_inputs

    cfg = config_by_name(cfg_name)
    inp = make_inputs(cfg, "cuda")
    T, H = inp["T"], cfg["n_heads"]
    dt = inp["q"].dtype
    out = torch.empty((T, H, inp["d_v"]), dtype=dt, device="cuda")
    z = torch.empty((T, H, cfg["d_state"]), dtype=dt, device="cuda")
    plan = S.Plan.for_inputs(inp)
    plan.build(inp["scores"])
    n_doc = int(inp["lens"][1])  # the first document after the prefix
    p0 = int(inp["pool_rows"][1])
    src = [inp["kv"].cpu().pin_memory(), inp["z_cached"][p0:p0 + n_doc].cpu().pin_memory()]
    dst = [torch.empty_like(src[0], device="cuda"), torch.empty_like(src[1], device="cuda")]
    nbytes = sum(x.numel() * x.element_size() for x in src)
    pf = S.Prefetcher()

    def timed(with_prefetch):
        ms, pms = [], []
        for _ in range(steps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if with_prefetch:
                pf.prefetch(list(zip(src, dst)))
            a.record()
            plan.forward(inp, out, z)
            b.record()
            if with_prefetch:
                pf.wait()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
            if with_prefetch:
                pms.append(pf.elapsed_ms())
        return statistics.median(ms[1:]), (statistics.median(pms[1:]) if pms else None)

    alone, _ = timed(False)
    shared, copy_ms = timed(True)
    pf.close()
    plan.close()
    del inp, out, z, src, dst
    torch.cuda.empty_cache()
    return dict(workload=cfg_name, forward_ms=round(alone, 3),
                forward_ms_with_prefetch=round(shared, 3), prefetch_bytes=nbytes,
                prefetch_ms=round(copy_ms, 3), prefetch_gbps=round(nbytes / copy_ms / 1e6, 1),
                source="pinned host memory")


def decode_json(name, d):
    return {
        "workload": name, "window_rows": d["rows"], "keys": d["keys"],
        "attention_us": round(d["attention_us"], 2), "split_merge_us": round(d["merge_us"], 2),
        "epilogue_us": round(d["epilogue_us"], 2), "forward_us_stage_events": round(d["forward_us"], 2),
        "forward_us": round(d["forward_us_eager"], 2),
        "forward_us_hip_graph": round(d["forward_us_graph"], 2),
        **({"stages": "one-row window: the split merge runs inside the projection kernel, so "
                      "epilogue_us holds both and split_merge_us is the cost of its events"}
           if d["rows"] == 1 else {}),
        **({"walk_step_us_median": round(d["walk"]["step_us_median"], 2),
            "walk_step_us_min": round(d["walk"]["step_us_min"], 2),
            "walk": "%d consecutive decode rows on one plan: window update + forward per row"
                    % d["walk"]["steps"]} if "walk" in d else {}),
        "roofline": {"bound": "hbm", "achieved": round(d["bytes"] / d["forward_us_eager"] / 1e3, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(d["bytes"] / d["forward_us_eager"] / 1e3 / PEAK_HBM_GBS, 4),
                     "bytes": int(d["bytes"]), "over": "whole forward, back-to-back launches"},
    }


def measure(cfg_name, steps, warmup, decode_rows=0, pool="identity", also_e4m3=False):
    import torch
    from segmented_attention_amd import segmla as S
    from workload import config_by_name, make_inputs

    cfg = config_by_name(cfg_name)
    log("workload %s: generating inputs (pool %s)" % (cfg_name, pool))
    inp = make_inputs(cfg, "cuda", pool=pool)
    T, H = inp["T"], cfg["n_heads"]
    dt = inp["q"].dtype
    out = torch.empty((T, H, inp["d_v"]), dtype=dt, device="cuda")
    G = cfg.get("group_heads", 0)
    z = torch.empty((T, H // G if G >= 2 else H, cfg["d_state"]), dtype=dt, device="cuda")
    plan = S.Plan.for_inputs(inp)

    def step():
        plan.build(inp["scores"])
        plan.forward(inp, out, z)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log("workload %s: timing %d steps" % (cfg_name, steps))
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    # kernel-level times from HIP events on the launch stream (separate profiled pass of
    # the same steps: the profiled forward waits for the previous one's events)
    S.segmla_profile_enable(plan.handle, True)
    attn_steps, fwd_steps = [], []
    prev = [0.0] * 4
    for _ in range(steps):
        step()
        ms, n_fwd, n_build = S.segmla_profile_read(plan.handle)  # cumulative; waits for the step
        attn_steps.append(ms[0] - prev[0])
        fwd_steps.append((ms[0] + ms[1] + ms[2]) - (prev[0] + prev[1] + prev[2]))
        prev = list(ms)
    S.segmla_profile_enable(plan.handle, False)
    torch.cuda.synchronize()
    g_pairs, l_pairs, w_pairs = plan.pairs()
    fpp = flops_per_pair(cfg)
    flops = fpp * (g_pairs + l_pairs + w_pairs)
    attn_ms = ms[0] / max(1, n_fwd)
    res = dict(
        cfg=cfg, T=T, n_protected=plan.n_protected, wall_s=wall, flops=flops,
        g_pairs=g_pairs, l_pairs=l_pairs, w_pairs=w_pairs,
        attn_ms=attn_ms, merge_ms=ms[1] / max(1, n_fwd), epi_ms=ms[2] / max(1, n_fwd),
        attn_ms_median=statistics.median(attn_steps), attn_ms_min=min(attn_steps),
        fwd_ms_median=statistics.median(fwd_steps), fwd_ms_min=min(fwd_steps),
        build_ms=ms[3] / max(1, n_build),
        attn_tflops=flops / (attn_ms * 1e-3) / 1e12,
        tflops=flops / wall / 1e12,
        tflops_576_512=(2.0 * (576 + 512)) * (g_pairs + l_pairs + w_pairs) / wall / 1e12,
    )
    plan.close()
    if also_e4m3:  # the same layer with the grouped state emitted as 1x128 E4M3 blocks
        log("workload %s: forward with the state emitted as E4M3 blocks" % cfg_name)
        pe = S.Plan.for_inputs(dict(inp, cfg=dict(cfg, z_e4m3=1)))
        pe.build(inp["scores"])
        zc = torch.empty(z.shape, dtype=torch.uint8, device="cuda")
        zsc = torch.empty(z.shape[:-1] + (cfg["d_state"] // 128,), dtype=torch.float32, device="cuda")
        for _ in range(warmup + 1):
            pe.forward(inp, out, zc, z_scale=zsc)
        torch.cuda.synchronize()
        S.segmla_profile_enable(pe.handle, True)
        for _ in range(steps):
            pe.forward(inp, out, zc, z_scale=zsc)
        ms_e, n_e, _ = S.segmla_profile_read(pe.handle)
        S.segmla_profile_enable(pe.handle, False)
        torch.cuda.synchronize()
        pe.close()
        res["epi_ms_e4m3"] = ms_e[2] / max(1, n_e)
        del zc, zsc
    if decode_rows > 0:
        log("workload %s: decode window of the last %d row(s)" % (cfg_name, decode_rows))
        res["decode"] = measure_window(inp, cfg, decode_rows, 20, 3)
        log("workload %s: decode walk over the last rows (set_window + forward)" % cfg_name)
        res["decode"]["walk"] = measure_decode_walk(inp, cfg, 16)
    del inp, out, z
    torch.cuda.empty_cache()
    return res


def dual_keys(inp, dual, rows):
    """Keys one head attends per row of `rows` in the dual-pool forward (host count for the
    FLOP figure): the raw window min(t, w) + 1, plus the entries of the row's walk (every
    available entry, or the list up to its first id that is not available)."""
    import numpy as np
    m, w = dual["ratio"], dual["window"]
    lens = np.asarray(inp["lens"], dtype=np.int64)
    offs = np.asarray(inp["offsets"], dtype=np.int64)
    cnt = lens // m
    base = np.concatenate([[0], np.cumsum(cnt)[:-1]])
    rows = np.asarray(rows, dtype=np.int64)
    s = np.searchsorted(offs, rows, side="right") - 1
    n_avail = base[s] + np.minimum(cnt[s], (rows - offs[s] + 1) // m)
    raw = np.minimum(rows, w) + 1
    if not dual["top_k"]:
        return raw + n_avail
    ids = dual["cidx"][torch_index(rows, dual["cidx"])].cpu().numpy().astype(np.int64)
    clen = dual["clen"][torch_index(rows, dual["clen"])].cpu().numpy().astype(np.int64)
    k = np.arange(ids.shape[1])[None, :]
    ok = (k < clen[:, None]) & (ids >= 0) & (ids < n_avail[:, None])
    lead = np.where(ok.all(axis=1), ids.shape[1], np.argmin(ok, axis=1))
    return raw + lead


def torch_index(rows, t):
    import torch
    return torch.as_tensor(rows, device=t.device)


def measure_dual(cfg_name, ratio, window, top_k, steps, warmup):
    """The compressed-history (dual-pool) attention of the workload's request: every row with
    all its heads (a CSA layer: ratio 4, 512-entry lists; an HCA layer: ratio 128, every
    available entry), and its last row alone (decode). Event-timed on the launch stream."""
    import numpy as np
    import torch
    from segmented_attention_amd import segmla as S
    from workload import config_by_name, make_dual_inputs, make_inputs

    cfg = config_by_name(cfg_name)
    kind = "csa" if top_k else "hca"
    log("workload %s: %s dual-pool layer (ratio %d, window %d, lists %d)"
        % (cfg_name, kind, ratio, window, top_k))
    inp = make_inputs(cfg, "cuda")
    dual = make_dual_inputs(inp, ratio, window, top_k, "cuda")
    T, H = inp["T"], cfg["n_heads"]
    res = {"workload": cfg_name, "layer": kind, "ratio": ratio, "window": window,
           "top_k": top_k, "rows": T, "heads": H}
    for q_range in (None, (T - 1, T)):
        q0, q1 = q_range if q_range else (0, T)
        plan = S.Plan.for_inputs(inp, q_range=q_range)
        plan.build(inp["scores"])
        d = S.Dual.for_inputs(plan, dual)
        d.build()
        out = torch.empty((q1 - q0, H, inp["d_v"]), dtype=torch.bfloat16, device="cuda")
        args = (inp["q"][q0:q1], inp["kv"], dual["ckv"], out,
                dual["cidx"][q0:q1] if top_k else None, dual["clen"][q0:q1] if top_k else None)
        n = steps if q_range is None else 50
        for _ in range(warmup):
            d.forward(*args)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for e0, e1 in evs:
            e0.record(st)
            d.forward(*args)
            e1.record(st)
        torch.cuda.synchronize()
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        keys = dual_keys(inp, dual, np.arange(q0, q1))
        pairs = float(keys.sum()) * H
        if q_range is None:
            med = statistics.median(ms)
            res.update({
                "keys_per_row_mean": round(float(keys.mean()), 1), "pairs": pairs,
                "attention_ms_median": round(med, 4), "attention_ms_min": round(min(ms), 4),
                "attention_tflops": round(flops_per_pair(cfg) * pairs / (med * 1e-3) / 1e12, 3),
                "attention_frac_bf16_peak": round(flops_per_pair(cfg) * pairs / (med * 1e-3) / 1e12
                                                  / PEAK_BF16_TFLOPS, 4),
            })
        else:
            # one row is one workgroup (64 heads): a latency figure, not a bandwidth one (its
            # keys are under 1 MB)
            res["decode"] = {"keys": int(keys.sum()), "workgroups": (H + 63) // 64,
                             "forward_us_median": round(statistics.median(ms) * 1e3, 2),
                             "forward_us_min": round(min(ms) * 1e3, 2)}
        d.close()
        plan.close()
        del out
    del inp, dual
    torch.cuda.empty_cache()
    return res


def cpu_baseline(cfg_name, budget_s=20.0):
    """The fp64 oracle, as it stands, on a bounded row sample of the same workload."""
    import numpy as np
    import torch
    from oracle import segmla_oracle as O
    from workload import config_by_name, make_inputs

    cfg = config_by_name(cfg_name)
    inp = make_inputs(cfg, "cuda")
    d = {k: v for k, v in inp.items() if not torch.is_tensor(v)}
    d["latent"] = inp["kv"].double().cpu().numpy()
    d["w"] = inp["w"].double().cpu().numpy()
    d["scores"] = inp["scores"].cpu().numpy()

    class Rows:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, i):
            return self.t[int(i)].double().cpu().numpy()

    d["q"], d["z_cached"] = Rows(inp["q"]), Rows(inp["z_cached"])
    T = inp["T"]
    g = O.geometry(d["kinds"], d["lens"], d["offsets"], d["pool_rows"], d["n_pool"])
    A = O.protected_rows(g, cfg["edge_rows"], cfg["tail_rows"], cfg["budget_permille"], (),
                         d["scores"])["A"]
    in_a = np.zeros(T, bool)
    in_a[A] = True
    rng = np.random.default_rng(123)
    # sample: rows spread uniformly over the request, protected and unprotected alike; the
    # row count is calibrated so that the timed oracle run takes about `budget_s`
    cand = rng.permutation(T)
    n_g, n_l = len(cfg["global_heads"]), cfg["n_heads"] - len(cfg["global_heads"])
    t0 = time.perf_counter()
    O.layer_forward(d, rows=[int(t) for t in cand[:4]])
    t4 = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.layer_forward(d, rows=[int(t) for t in cand[:36]])
    t36 = time.perf_counter() - t0
    per_row = max((t36 - t4) / 32.0, 1e-4)
    fixed = max(t4 - 4 * per_row, 0.0)
    n_rows = int(min(T, max(36, (budget_s - fixed) / per_row)))
    rows = sorted(int(t) for t in cand[:n_rows])
    t0 = time.perf_counter()
    O.layer_forward(d, rows=rows)
    secs = time.perf_counter() - t0
    pairs = sum((n_g + (n_l if in_a[t] else 0)) * (t + 1) for t in rows)
    flops = flops_per_pair(cfg) * pairs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    cpu_model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    del inp
    torch.cuda.empty_cache()
    return dict(value=flops / secs / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample="%d of %d request rows of %s (uniform random, seed 123; Global heads on each, "
                       "Local heads on the %d sampled rows in A), fp64 numpy incl. key re-rotation "
                       "of all rows; %.1f s on %d threads of %s"
                       % (len(rows), T, cfg_name, int(in_a[rows].sum()), secs, int(threads), cpu_model),
                seconds=secs)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="flash_32k_bf16")
    ap.add_argument("--secondary", default="long_128k_bf16")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--target", default="long_128k_global_bf16",
                    help="workload of the stated throughput target (the 128K layer's Global heads)")
    ap.add_argument("--no-target", action="store_true")
    ap.add_argument("--fp8", default="pro_64k_fp8", help="E4M3-latent workload reported alongside")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--window", default="flash_32k_window_bf16,swa_32k_bf16",
                    help="comma-separated workloads with sink + window heads reported alongside; "
                         "'' for none")
    ap.add_argument("--prefetch", type=int, default=1,
                    help="1: time the main workload's forward with a concurrent artifact prefetch")
    ap.add_argument("--many-short", default="many_short_bf16",
                    help="many-short-segments workload (256 documents, 256-way merge per row) "
                         "reported alongside; '' for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chunks", type=int, default=8,
                    help="chunked-prefill figure: the main workload in this many row windows (0: off)")
    ap.add_argument("--decode-rows", type=int, default=1,
                    help="decode window (last rows of the secondary workload) reported alongside; 0: none")
    ap.add_argument("--grouped", default="flash_32k_grouped_bf16",
                    help="also time this grouped-state workload (z per group of heads); '' for none")
    ap.add_argument("--pool", default="identity",
                    help="latent pool layout of the main workload: identity, shuffled, aliased or "
                         "paged:<rows per page>")
    ap.add_argument("--paged-rows", type=int, default=64,
                    help="also time the main workload over a paged latent pool of this many rows "
                         "per page; 0: none")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode window of the secondary workload (for kernel "
                         "traces of the decode path) and print its figures")
    ap.add_argument("--dual", default="csa:4:127:512,hca:128:127:0",
                    help="compressed-history (dual-pool) layers over the main workload's request, "
                         "kind:ratio:window:list width, comma-separated; '' for none")
    ap.add_argument("--dual-only", action="store_true",
                    help="time only the dual-pool layers (for their kernel traces)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size kernel "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library runs one layer on one GPU and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = src.clone()
        torch.cuda.synchronize()
        del src, dst
    if args.decode_only:
        from workload import config_by_name, make_inputs
        cfg = config_by_name(args.secondary)
        log("workload %s: generating inputs" % cfg["name"])
        inp = make_inputs(cfg, "cuda")
        log("workload %s: decode window of the last %d row(s)" % (cfg["name"], args.decode_rows))
        d = measure_window(inp, cfg, args.decode_rows, args.steps, args.warmup)
        print(json.dumps({"decode": decode_json(cfg["name"], d)}), flush=True)
        return
    duals = []
    for spec in [x for x in args.dual.split(",") if x]:
        _, ratio, window, top_k = spec.split(":")
        duals.append((int(ratio), int(window), int(top_k)))
    if args.dual_only:
        print(json.dumps({"dual_pool": [measure_dual(args.workload, *d, max(5, args.steps), 2)
                                        for d in duals]}), flush=True)
        return
    main_res = measure(args.workload, args.steps, args.warmup, pool=args.pool)
    # the target figure comes before the long layers (a chip that has run them for seconds
    # clocks lower) with at least 3 warm-up and 10 timed steps
    tgt = None
    if not args.no_target and args.target:
        tgt = measure(args.target, max(10, args.steps // 2), max(3, args.warmup))
    sec = None
    if not args.no_secondary and args.secondary:
        sec = measure(args.secondary, max(3, args.steps // 4), 1, decode_rows=args.decode_rows)
    f8 = None
    if not args.no_fp8 and args.fp8:
        f8 = measure(args.fp8, 10, 3)
    msh = None
    if args.many_short:
        msh = measure(args.many_short, max(3, args.steps // 4), 1)
    wins = [measure(name, max(3, args.steps // 2), 2) for name in args.window.split(",") if name]
    pfx = None
    if args.prefetch:
        log("workload %s: forward with a concurrent artifact prefetch" % args.workload)
        pfx = measure_prefetch(args.workload, 5)
    chk = measure_chunked(args.workload, args.chunks, max(3, args.steps // 4)) if args.chunks > 0 else None
    gr = None
    if args.grouped:
        gr = measure(args.grouped, max(2, args.steps // 2), 1, also_e4m3=True)
    pg = None
    if args.paged_rows > 0:
        pg = measure(args.workload, max(2, args.steps // 2), 1, pool="paged:%d" % args.paged_rows)
    dres = [measure_dual(args.workload, *d, max(5, args.steps // 2), 2) for d in duals]
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.workload)

    r = main_res
    cfg = r["cfg"]
    achieved = r["flops"] / (r["attn_ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(r["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall_s"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg["kv_dtype"] == "bf16" else cfg["kv_dtype"],
        "data": "synthetic",
        "config": {
            "workload": r["cfg"]["name"],
            **({"pool": args.pool} if args.pool != "identity" else {}),
            "rows": r["T"], "heads": cfg["n_heads"], "global_heads": len(cfg["global_heads"]),
            "latent": "%d+%d" % (cfg["d_nope"], cfg["d_rope"]),
            "protected_rows": r["n_protected"],
            "us_per_layer": round(r["wall_s"] * 1e6, 1),
            "flop_per_triple": flops_per_pair(cfg),
            "tflops_576_512_convention": round(r["tflops_576_512"], 3),
            "stage_ms": {"attention": round(r["attn_ms"], 4), "split_merge": round(r["merge_ms"], 4),
                         "epilogue": round(r["epi_ms"], 4), "plan_build": round(r["build_ms"], 4)},
            "event_ms_per_forward": {"attention_median": round(r["attn_ms_median"], 4),
                                     "attention_min": round(r["attn_ms_min"], 4),
                                     "forward_median": round(r["fwd_ms_median"], 4),
                                     "forward_min": round(r["fwd_ms_min"], 4)},
        },
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": attn_traffic() if r["cfg"]["name"] == "flash_32k_bf16" else None},
        "cpu_baseline": None if cpu is None else {k: (round(v, 6) if isinstance(v, float) else v)
                                                  for k, v in cpu.items() if k != "seconds"},
    }
    if sec is not None:
        line["secondary"] = {
            "workload": sec["cfg"]["name"], "rows": sec["T"], "protected_rows": sec["n_protected"],
            "tflops": round(sec["tflops"], 3), "us_per_layer": round(sec["wall_s"] * 1e6, 1),
            "attention_tflops": round(sec["attn_tflops"], 3),
            "attention_frac_bf16_peak": round(sec["attn_tflops"] / PEAK_BF16_TFLOPS, 4),
            "stage_ms": {"attention": round(sec["attn_ms"], 3), "epilogue": round(sec["epi_ms"], 3),
                         "plan_build": round(sec["build_ms"], 3)},
        }
    if sec is not None and "decode" in sec:
        line["decode"] = decode_json(sec["cfg"]["name"], sec["decode"])
    if tgt is not None:
        line["target"] = {
            "workload": tgt["cfg"]["name"], "rows": tgt["T"], "heads": tgt["cfg"]["n_heads"],
            "attention_ms": round(tgt["attn_ms"], 3), "attention_ms_median": round(tgt["attn_ms_median"], 3),
            "attention_ms_min": round(tgt["attn_ms_min"], 3), "attention_tflops": round(tgt["attn_tflops"], 3),
            "attention_frac_bf16_peak": round(tgt["attn_tflops"] / PEAK_BF16_TFLOPS, 4),
            "target_frac_bf16_peak": 0.5,
        }
    if msh is not None:
        line["many_short"] = {
            "workload": msh["cfg"]["name"], "rows": msh["T"],
            "segments": len(msh["cfg"]["segments"]), "protected_rows": msh["n_protected"],
            "tflops": round(msh["tflops"], 3), "us_per_layer": round(msh["wall_s"] * 1e6, 1),
            "attention_tflops": round(msh["attn_tflops"], 3),
            "attention_frac_bf16_peak": round(msh["attn_tflops"] / PEAK_BF16_TFLOPS, 4),
            "stage_ms": {"attention": round(msh["attn_ms"], 3), "split_merge": round(msh["merge_ms"], 3),
                         "epilogue": round(msh["epi_ms"], 3), "plan_build": round(msh["build_ms"], 3)},
        }
    if wins:
        line["window_heads"] = [{
            "workload": w["cfg"]["name"], "rows": w["T"], "heads": w["cfg"]["n_heads"],
            "global_heads": len(w["cfg"]["global_heads"]), "window_heads": len(w["cfg"]["window_heads"]),
            "n_sink": w["cfg"]["n_sink"], "window": w["cfg"]["window"],
            "pairs": {"global": w["g_pairs"], "local": w["l_pairs"], "window": w["w_pairs"]},
            "tflops": round(w["tflops"], 3), "us_per_layer": round(w["wall_s"] * 1e6, 1),
            "attention_tflops": round(w["attn_tflops"], 3),
            "attention_frac_bf16_peak": round(w["attn_tflops"] / PEAK_BF16_TFLOPS, 4),
            "stage_ms": {"attention": round(w["attn_ms"], 3), "epilogue": round(w["epi_ms"], 3),
                         "plan_build": round(w["build_ms"], 3)},
        } for w in wins]
    if pfx is not None:
        line["prefetch"] = pfx
    if chk is not None:
        chk["whole_request_ms"] = round(r["fwd_ms_median"] + r["build_ms"], 3)
        line["chunked_prefill"] = chk
    if gr is not None:
        line["grouped"] = {
            "workload": gr["cfg"]["name"], "group_heads": gr["cfg"]["group_heads"],
            "epilogue_ms": round(gr["epi_ms"], 3), "epilogue_ms_per_head_state": round(r["epi_ms"], 3),
            "epilogue_ms_e4m3_state": round(gr["epi_ms_e4m3"], 3),
            "attention_ms": round(gr["attn_ms"], 3), "us_per_layer": round(gr["wall_s"] * 1e6, 1),
        }
    if pg is not None:
        line["paged"] = {
            "workload": pg["cfg"]["name"], "page_rows": args.paged_rows,
            "layout": "shuffled pages, equal-length documents sharing pages",
            "attention_ms": round(pg["attn_ms"], 3), "attention_tflops": round(pg["attn_tflops"], 3),
            "attention_frac_bf16_peak": round(pg["attn_tflops"] / PEAK_BF16_TFLOPS, 4),
            "us_per_layer": round(pg["wall_s"] * 1e6, 1),
        }
    if f8 is not None:
        line["fp8"] = {
            "workload": f8["cfg"]["name"], "rows": f8["T"], "heads": f8["cfg"]["n_heads"],
            "latent": "e4m3 (1x128 blocks, fp32 scales) + bf16 rope", "protected_rows": f8["n_protected"],
            "tflops": round(f8["tflops"], 3), "us_per_layer": round(f8["wall_s"] * 1e6, 1),
            "attention_tflops": round(f8["attn_tflops"], 3),
            "attention_frac_bf16_peak": round(f8["attn_tflops"] / PEAK_BF16_TFLOPS, 4),
            "attention_frac_fp8_peak": round(f8["attn_tflops"] / PEAK_FP8_TFLOPS, 4),
            "stage_ms": {"attention": round(f8["attn_ms"], 3), "epilogue": round(f8["epi_ms"], 3),
                         "plan_build": round(f8["build_ms"], 3)},
        }
    if dres:
        line["dual_pool"] = dres
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
