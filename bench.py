"""Benchmark: SparK decode attention over the pruned key cache on one MI355X.

One step = the whole hot path on one LLaMA-3.1-8B-shaped layer (B=1,
S=32768, 32 query heads, 8 KV heads, D=128, window 32, lambda=0.5):
prefill prune (channel energy, per-token top-T, packing, recovery
statistics) followed by 64 decode steps. The decode steps rotate over R
replicas of the pruned cache (packed K, mask, V, r) totalling >= 768 MB, so
the 256 MB Infinity Cache cannot serve them and the reported bandwidth is
HBM bandwidth. Decode launches are replayed from a HIP graph (one graph per
step, 64 kernels); prefill is a second graph.

value = effective decode bytes / decode time, where the effective bytes of a
decode step are B*N_kv*S*(2T + 16 + 2D): packed K, the 16-byte mask and dense
V. Inputs are resident in HBM before timing starts.

Also reported (not the metric): the 128K-context layer at lambda=0.8, the
stacked-eviction workload (window eviction of B=8, S=32K to 4096 tokens per
KV head, then lambda=0.7 pruning and decode over the compacted cache) and the
32-layer stack (B=4, S=64K, lambda=0.8; one decode launch per layer per step).

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME] [--no-extra]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SparK decode attn effective KV GB/s & %HBM peak, S=32K, λ=0.5/0.8"
HBM_PEAK_GBS = 8000.0
MALL_DEFEAT_BYTES = 768e6
SAMPLE_SEED = 0x5EED5A3B1E0F2C47   # Philox key of the sampled-F legs
DECODE_SOURCES = ["sparse_decode_attention_amd/csrc/decode.hip", "sparse_decode_attention_amd/csrc/decode_common.h",
                  "sparse_decode_attention_amd/csrc/decode_fast.h", "sparse_decode_attention_amd/csrc/decode_fast_fixed.hip",
                  "sparse_decode_attention_amd/csrc/kernels.h", "sparse_decode_attention_amd/csrc/common.h",
                  "sparse_decode_attention_amd/csrc/spark_abi.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_llama8b_s32k_traffic.md")


def decode_source_sha() -> str:
    h = hashlib.sha256()
    for p in DECODE_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """(per-launch HBM bytes, profiled average duration in ns) of the decode
    kernel from the committed rocprofv3 summary, if it was taken on the
    current kernel source and this workload; (None, None) otherwise."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != decode_source_sha() or kv.get("workload") != workload:
        return None, None
    try:
        return float(kv["hbm_bytes_per_launch"]), float(kv["avg_duration_ns"])
    except (KeyError, ValueError):
        return None, None


# 32-bit VALU lane operations per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_GOPS = 256 * 64 * 2.4


def sampled_alu_ops_per_token(G, T, rec, valu_pv=None):
    """Algorithmic 32-bit VALU operations per (token, KV head) of the sampled
    decode: per 4-channel group a Philox4x32-10 block (10 rounds of two wide
    multiplies and two three-way xors), four uniforms (convert, scale), the
    transform (Exponential: log, fma each; Gaussian: two of log, scale, sqrt,
    sin, cos, two products), the kept-channel masks and 4 G FMAs; then the
    fixed-r part: G T FMAs and T subtractions of the kept channels, and, in
    the generic kernel (valu_pv), G 128 FMAs of P.V on the VALU (the
    matrix-core kernel for G = 4 and T in {26, 38, 48, 64} runs P.V on MFMA)."""
    if valu_pv is None:
        valu_pv = not (G == 4 and T in (26, 38, 48, 64))
    transform = 8 if rec == "exponential" else 14
    per_group = 40 + 8 + transform + 4 + 4 * G
    return 32 * per_group + G * T + T + (G * 128 if valu_pv else 0)


def effective_decode_bytes(w, T, Tv=None, nbv=None):
    """Packed K and its mask, then dense V (Tv and nbv None), packed V and
    its mask, or V pruned in 8-channel blocks (nbv blocks of 16 bytes and a
    2-byte block mask)."""
    v_bytes = 2 * w.D if Tv is None else 2 * Tv + 16
    if nbv is not None:
        v_bytes = 16 * nbv + 2
    return w.B * w.n_kv * w.S * (2 * T + 16 + v_bytes)


def effective_prefill_bytes(w, T):
    return w.B * w.n_kv * w.S * (2 * w.D + 2 * T + 16)


def decode_bucket(T: int) -> int:
    """Largest row length of the runtime-T decode variant that serves T."""
    return 32 if T <= 32 else 64 if T <= 64 else 96 if T <= 96 else 128


def decode_kernel_name(G: int, T: int, smode: int = 0, ragged: bool = False, vblocks: bool = False) -> str:
    """The matrix-core decode kernel the library launches, as
    decode_fast_kernel<G, TB, TFIX, ODD, SMODE, RG, VB> (VB: V pruned in
    8-channel blocks)."""
    if ragged:
        return f"decode_fast_kernel<{G}, 128, 0, true, 0, true, false>"
    odd = "true" if T & 1 else "false"
    if vblocks:
        if G == 4 and T in (26, 64):
            return f"decode_fast_kernel<4, {T}, {T}, false, 0, false, true>"
        return f"decode_fast_kernel<{G}, {decode_bucket(T)}, 0, {odd}, 0, false, true>"
    exact = (G == 4 and T in (26, 38, 48, 64)) or (not smode and (
        (G == 4 and T in (13, 51, 77, 90, 102, 115)) or (G in (1, 2, 8) and T in (26, 64))))
    if exact:
        return f"decode_fast_kernel<{G}, {T}, {T}, {odd}, {smode}, false, false>"
    if smode:
        return f"decode_kernel<{G}, {smode}, 0, false>"
    return f"decode_fast_kernel<{G}, {decode_bucket(T)}, 0, {odd}, 0, false, false>"


def run_leg(w, steps, warmup, rotate=True, seed=0, verbose=True, x=None, recovery="mean_retained",
            rng_seed=SAMPLE_SEED, lam_v=None, ratios=None, top_p=None, lam_vb=None):
    import torch
    from sparse_decode_attention_amd import gen, ops

    dev = torch.device("cuda:0")
    T = ops.num_kept(w.D, w.lam) if ratios is None else ops.num_kept_grouped(w.D, ratios)
    if top_p is not None:
        T = w.D            # ragged rows: sized (and replicas counted) for the longest row
    lam = w.lam if ratios is None else 1.0 - T / w.D
    if x is None:
        x = gen.torch_layer(w, dev, seed=seed, steps=w.steps)
    Tv = None if lam_v is None else ops.num_kept(w.D, lam_v)
    nbv = None if lam_vb is None else ops.num_kept_vblocks(w.D, lam_vb)
    dec_bytes = effective_decode_bytes(w, T, Tv, nbv)
    R = max(1, int(-(-MALL_DEFEAT_BYTES // dec_bytes))) if rotate else 1
    # replica 0 is written by the prefill every step; replicas 1..R-1 hold copies of it
    reps = []
    for i in range(R):
        reps.append({
            "k_packed": torch.empty((w.B, w.n_kv, w.S, T), dtype=torch.bfloat16, device=dev),
            "row_off": torch.empty((w.B, w.n_kv, w.S + 1), dtype=torch.int32, device=dev),
            "mask": torch.empty((w.B, w.n_kv, w.S, 4), dtype=torch.int32, device=dev),
            "chan_energy": torch.empty((w.B, w.n_kv, w.D), dtype=torch.float32, device=dev),
            "r": torch.empty((w.B, w.n_kv, w.D), dtype=torch.float32, device=dev),
            "cnt": torch.empty((w.B, w.n_kv, w.D), dtype=torch.int32, device=dev),
            "v": x["v"] if (i == 0 or Tv is not None or nbv is not None) else x["v"].clone(),
        })
        if nbv is not None:
            reps[-1].update({
                "v_packed": torch.empty((w.B, w.n_kv, w.S, 8 * nbv), dtype=torch.bfloat16, device=dev),
                "v_bmask": torch.empty((w.B, w.n_kv, ops.vblock_mask_stride(w.S)), dtype=torch.int16, device=dev),
                "r_v": torch.empty((w.B, w.n_kv, w.D), dtype=torch.float32, device=dev),
                "cnt_v": torch.empty((w.B, w.n_kv, w.D), dtype=torch.int32, device=dev),
            })
        if Tv is not None:
            reps[-1].update({
                "v_packed": torch.empty((w.B, w.n_kv, w.S, Tv), dtype=torch.bfloat16, device=dev),
                "v_mask": torch.empty((w.B, w.n_kv, w.S, 4), dtype=torch.int32, device=dev),
                "r_v": torch.empty((w.B, w.n_kv, w.D), dtype=torch.float32, device=dev),
                "cnt_v": torch.empty((w.B, w.n_kv, w.D), dtype=torch.int32, device=dev),
            })
    outs = torch.empty((w.steps, w.B, w.n_q, w.D), dtype=torch.float32, device=dev)

    sampled = recovery in ("gaussian", "exponential")

    def prefill():
        if top_p is not None:
            r0 = dict(reps[0])
            r0["k_packed"] = r0["k_packed"].view(w.B, w.n_kv, w.S * w.D)
            ops.prefill_prune_topp(x["q_win"], x["k"], w.n_kv, top_p, recovery=recovery, out=r0)
        elif ratios is not None:
            ops.prefill_prune_grouped(x["q_win"], x["k"], w.n_kv, ratios, recovery=recovery, out=reps[0])
        else:
            ops.prefill_prune(x["q_win"], x["k"], w.n_kv, w.lam, recovery=recovery, out=reps[0])
        if Tv is not None:
            r0 = reps[0]
            ops.prefill_prune_v(x["v"], lam_v, out={"v_packed": r0["v_packed"], "v_mask": r0["v_mask"],
                                                    "r_v": r0["r_v"], "cnt": r0["cnt_v"]})
        if nbv is not None:
            r0 = reps[0]
            ops.prefill_prune_vblocks(x["v"], lam_vb, out={"v_packed": r0["v_packed"], "v_bmask": r0["v_bmask"],
                                                           "r_v": r0["r_v"], "cnt": r0["cnt_v"]})

    def decode_all():
        for s in range(w.steps):
            rp = reps[s % R]
            if top_p is not None:
                ops.decode_attn_ragged(x["q_dec"][s], rp["k_packed"].view(w.B, w.n_kv, w.S * w.D), rp["row_off"],
                                       rp["mask"], rp["v"], rp["r"], out=outs[s])
            elif nbv is not None:
                ops.decode_attn_kvb(x["q_dec"][s], rp["k_packed"], rp["mask"], rp["r"], rp["v_packed"],
                                    rp["v_bmask"], rp["r_v"], lam, lam_vb, out=outs[s])
            elif Tv is not None:
                ops.decode_attn_kv(x["q_dec"][s], rp["k_packed"], rp["mask"], rp["r"], rp["v_packed"], rp["v_mask"],
                                   rp["r_v"], lam, lam_v, out=outs[s])
            elif sampled:
                ops.decode_attn_sampled(x["q_dec"][s], rp["k_packed"], rp["mask"], rp["v"], rp["chan_energy"],
                                        rp["r"], recovery, rng_seed, lam, out=outs[s])
            else:
                ops.decode_attn(x["q_dec"][s], rp["k_packed"], rp["mask"], rp["v"], rp["r"], lam, out=outs[s])

    # eager pass: fills every replica and allocates the cached workspaces
    prefill()
    for rp in reps[1:]:
        for n in ("k_packed", "mask", "chan_energy", "r", "cnt") + (("v_packed", "v_mask", "r_v") if Tv else ()) + \
                (("v_packed", "v_bmask", "r_v") if nbv else ()) + (("row_off",) if top_p is not None else ()):
            rp[n].copy_(reps[0][n])
    if top_p is not None:
        # the bytes a ragged decode reads: kept values, masks and row offsets, dense V
        kept = int(reps[0]["row_off"][..., -1].sum().item())
        dec_bytes = 2 * kept + w.B * w.n_kv * (w.S * (16 + 2 * w.D) + 4 * (w.S + 1))
        T = kept / (w.B * w.n_kv * w.S)
    decode_all()
    torch.cuda.synchronize()
    eager = outs.clone()

    s_cap = torch.cuda.Stream(dev)
    s_cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s_cap):
        g_pre, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_pre, stream=s_cap):
            prefill()
        with torch.cuda.graph(g_dec, stream=s_cap):
            decode_all()
    torch.cuda.current_stream(dev).wait_stream(s_cap)
    torch.cuda.synchronize()

    # graph replays must reproduce the eager results bit for bit
    for _ in range(2):
        g_pre.replay()
        g_dec.replay()
        torch.cuda.synchronize()
        if not torch.equal(outs, eager):
            raise RuntimeError("graph replay differs from eager decode")

    st = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        g_pre.replay()
        g_dec.replay()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(st)
        g_pre.replay()
        ev[i][1].record(st)
        g_dec.replay()
        ev[i][2].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    if not torch.equal(outs, eager):
        raise RuntimeError("timed replay differs from eager decode")

    pre_ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    dec_ms = sorted(e[1].elapsed_time(e[2]) for e in ev)
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in ev)
    med = lambda a: a[len(a) // 2]
    dec_launch_us = med(dec_ms) * 1e3 / w.steps
    res = {
        "T": T, "replicas": R, "replica_bytes": dec_bytes,
        "decode_bytes_per_step": dec_bytes,
        "decode_us_per_launch": dec_launch_us,
        "decode_GBps": dec_bytes / (dec_launch_us * 1e-6) / 1e9,
        "prefill_us": med(pre_ms) * 1e3,
        "prefill_GBps": effective_prefill_bytes(w, T) / (med(pre_ms) * 1e-3) / 1e9,
        "Tv": Tv, "nbv": nbv,
        "step_ms_median": med(step_ms),
        "step_ms_mean": sum(step_ms) / len(step_ms),
        "wall_s": wall,
        "tokens_heads_per_s": w.B * w.S * w.n_q / (dec_launch_us * 1e-6),
        "x": x, "reps": reps,
    }
    return res


def growth_leg(w, steps, warmup, x):
    """The serving loop with a growing cache: prefill w.S - w.steps prompt
    tokens into a cache of capacity w.S, then w.steps decode steps, each
    appending one generated token per (b, KV head) (pruned with the prefill's
    channel energy) and decoding the step's query over the grown cache. One
    graph holds the prefill, another the w.steps append + decode pairs."""
    import torch
    from sparse_decode_attention_amd import ops

    dev = torch.device("cuda:0")
    S0 = w.S - w.steps
    k0, v0 = x["k"][:, :, :S0].contiguous(), x["v"][:, :, :S0].contiguous()
    k_new = [x["k"][:, :, S0 + i].contiguous() for i in range(w.steps)]
    v_new = [x["v"][:, :, S0 + i].contiguous() for i in range(w.steps)]
    cache = ops.GrowingCache(x["q_win"], k0, v0, w.n_kv, w.lam, w.S)
    outs = torch.empty((w.steps, w.B, w.n_q, w.D), dtype=torch.float32, device=dev)
    ws = ops.workspace(dev, "decode", ops.decode_ws_bytes(w.B, w.S, w.n_q, w.n_kv, w.D))

    def steps_all():
        cache.S = S0
        for i in range(w.steps):
            cache.append(k_new[i], v_new[i])
            cache.decode(x["q_dec"][i], out=outs[i], ws=ws)

    steps_all()
    torch.cuda.synchronize()
    eager = outs.clone()
    s_cap = torch.cuda.Stream(dev)
    s_cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s_cap):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s_cap):
            steps_all()
    torch.cuda.current_stream(dev).wait_stream(s_cap)
    torch.cuda.synchronize()
    for _ in range(max(1, warmup)):
        g.replay()
    torch.cuda.synchronize()
    if not torch.equal(outs, eager):
        raise RuntimeError("growth graph replay differs from eager")
    st = torch.cuda.current_stream(dev)
    ms = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    ms.sort()
    us_step = ms[len(ms) // 2] * 1e3 / w.steps
    T = cache.T
    mean_S = S0 + (w.steps + 1) / 2
    step_bytes = w.B * w.n_kv * (mean_S * (2 * T + 16 + 2 * w.D) + 2 * T + 16 + 2 * w.D + 4 * w.D)
    return {"workload": w.name, "prompt_tokens": S0, "generated": w.steps, "T": T,
            "us_per_step_append_and_decode": round(us_step, 3), "GBps": round(step_bytes / (us_step * 1e-6) / 1e9, 2),
            "what": "graph of 64 (append + decode) pairs over one cache (no replica rotation, so the 256 MB "
                    "Infinity Cache may serve part of the 105 MB it reads); bytes per step: the mean cache read plus "
                    "the appended row"}


def sweep_leg(base, lams=(0.5, 0.8), lengths=(4096, 8192, 16384, 32768, 65536, 131072), steps=5, warmup=2):
    """Decode time against input length (the walkthrough's section 4.3
    throughput-vs-length curve, Fig. 4(b)) at fixed launch rules, with replica
    rotation: per lambda, t(S) at each S and the least-squares line
    t = fixed + bytes / rate over the points, which separates the per-launch
    fixed cost (start-up, split merge) from the streaming rate."""
    out = {}
    for lam in lams:
        pts = []
        for S in lengths:
            w = base.with_(S=S, lam=lam, steps=64)
            r = run_leg(w, steps, warmup, verbose=False)
            pts.append((S, r["decode_bytes_per_step"], r["decode_us_per_launch"]))
            del r
        n = len(pts)
        mx = sum(p[1] for p in pts) / n
        my = sum(p[2] for p in pts) / n
        sxx = sum((p[1] - mx) ** 2 for p in pts)
        sxy = sum((p[1] - mx) * (p[2] - my) for p in pts)
        slope = sxy / sxx                   # us per byte
        fixed = my - slope * mx
        out[f"lambda={lam}"] = {
            "points": [{"S": S, "bytes": b, "us_per_launch": round(t, 3), "GBps": round(b / (t * 1e-6) / 1e9, 1)}
                       for S, b, t in pts],
            "fit_fixed_us": round(fixed, 3),
            "fit_marginal_GBps": round(1e-3 / slope, 1),
        }
    return out


def stream_ceiling(nbytes: int, reps: int = 7, block_counts=(512, 1024, 2048, 4096)):
    """GB/s of a plain streaming read (spark_read_stream) of `nbytes`, rotated
    over >= 768 MB of buffers like the decode replicas: the practical HBM read
    rate at this working-set size, measured on the same device. The best
    (over launch sizes) of the median replay time. Returns (GB/s, blocks)."""
    import torch
    from sparse_decode_attention_amd import ops
    dev = torch.device("cuda:0")
    n = (nbytes // 16) * 8
    R = max(2, int(-(-MALL_DEFEAT_BYTES // nbytes)))
    xs = [torch.zeros(n, dtype=torch.bfloat16, device=dev) for _ in range(R)]
    sink = torch.zeros(max(block_counts), dtype=torch.int32, device=dev)
    best = (0.0, 0)
    for blocks in block_counts:
        def run():
            for xx in xs:
                ops.read_stream(xx, sink, blocks)
        run()
        torch.cuda.synchronize()
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                run()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3 / R)
        ts.sort()
        gbs = n * 2 / ts[len(ts) // 2] / 1e9
        if gbs > best[0]:
            best = (gbs, blocks)
        del g
    return best


def evict_leg(w, steps, warmup):
    """Stacked-eviction workload: window eviction of the S-token layer to
    `keep` tokens per KV head (timed on its own), then the pruned-cache decode
    over the compacted cache (run_leg on the kept K and V)."""
    import dataclasses

    import torch
    from sparse_decode_attention_amd import gen, ops

    dev = torch.device("cuda:0")
    x = gen.torch_layer(w, dev, seed=0, steps=w.steps)
    ev = ops.window_evict(x["q_win"], x["k"], x["v"], w.n_kv, w.keep)
    for _ in range(warmup):
        ops.window_evict(x["q_win"], x["k"], x["v"], w.n_kv, w.keep)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ops.window_evict(x["q_win"], x["k"], x["v"], w.n_kv, w.keep)
    e1.record()
    torch.cuda.synchronize()
    evict_us = e0.elapsed_time(e1) * 1e3 / steps
    wk = dataclasses.replace(w, S=w.keep)
    xk = {"q_win": x["q_win"], "k": ev["k"], "v": ev["v"], "q_dec": x["q_dec"]}
    del x
    leg = run_leg(wk, steps, warmup, x=xk)
    kv_read = 2 * w.B * w.n_kv * w.S * w.D * 2          # K twice
    return {"workload": w.name, "keep": w.keep, "lambda": w.lam, "T": leg["T"],
            "evict_us": round(evict_us, 1), "evict_K_read_GBps": round(kv_read / (evict_us * 1e-6) / 1e9, 1),
            "decode_GBps": round(leg["decode_GBps"], 2),
            "decode_pct_hbm_peak": round(100 * leg["decode_GBps"] / HBM_PEAK_GBS, 2),
            "decode_us_per_launch": round(leg["decode_us_per_launch"], 3),
            "prefill_us": round(leg["prefill_us"], 2), "replicas": leg["replicas"]}


def stack_leg(w, steps, warmup):
    """The 32-layer stack: every layer pruned once (prefill timed per layer),
    then each decode step runs one decode launch per layer over all layers'
    pruned caches (one graph of `layers` launches per step). The stack
    (about 21.7 GB at B=4, S=64K, lambda 0.8) is far beyond the 256 MB cache,
    so no replica rotation is needed."""
    import torch
    from sparse_decode_attention_amd import gen, ops

    dev = torch.device("cuda:0")
    T = ops.num_kept(w.D, w.lam)
    layers = []
    pre_ms = []
    for li in range(w.layers):
        x = gen.torch_layer(w, dev, seed=0, layer=li, steps=1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g = ops.prefill_prune(x["q_win"], x["k"], w.n_kv, w.lam)
        e1.record()
        torch.cuda.synchronize()
        pre_ms.append(e0.elapsed_time(e1))
        layers.append({"q": x["q_dec"][0], "k_packed": g["k_packed"], "mask": g["mask"], "v": x["v"], "r": g["r"]})
        del x, g
    torch.cuda.empty_cache()
    outs = torch.empty((w.layers, w.B, w.n_q, w.D), dtype=torch.float32, device=dev)

    def step():
        for li, L in enumerate(layers):
            ops.decode_attn(L["q"], L["k_packed"], L["mask"], L["v"], L["r"], w.lam, out=outs[li])
    step()
    torch.cuda.synchronize()
    eager = outs.clone()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(gr, stream=side):
            step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(warmup):
        gr.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    if not torch.equal(outs, eager):
        raise RuntimeError("stack graph replay differs from eager decode")
    ts.sort()
    step_ms = ts[len(ts) // 2]
    per_layer = effective_decode_bytes(w, T)
    pre_ms.sort()
    return {"workload": w.name, "layers": w.layers, "B": w.B, "S": w.S, "lambda": w.lam, "T": T,
            "decode_ms_per_step": round(step_ms, 4),
            "decode_GBps": round(per_layer * w.layers / (step_ms * 1e-3) / 1e9, 2),
            "decode_pct_hbm_peak": round(100 * per_layer * w.layers / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "stack_bytes": per_layer * w.layers,
            "prefill_us_per_layer_median": round(pre_ms[len(pre_ms) // 2] * 1e3, 1),
            "prefill_GBps_per_layer": round(effective_prefill_bytes(w, T) / (pre_ms[len(pre_ms) // 2] * 1e-3) / 1e9, 1)}


def cpu_baseline(w, x, reps, T):
    """The oracle (NumPy, float64) on the host cores: one prefill prune of the
    layer and 48 decode steps at full shape (about 10-15 s of CPU work)."""
    import numpy as np
    import torch

    import oracle
    from sparse_decode_attention_amd import gen

    def host(t):
        return gen.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))

    q_win, k, v = host(x["q_win"]), host(x["k"]), host(x["v"])
    n_dec = 48
    q_dec = host(x["q_dec"][:n_dec])
    t0 = time.perf_counter()
    pr = oracle.prune(q_win, k, w.n_kv, w.lam)
    r, _ = oracle.stats(k, pr["mask"], pr["A"])
    t1 = time.perf_counter()
    for s in range(n_dec):
        oracle.decode_attn(q_dec[s], pr["packed"], pr["mask"], v, r)
    t2 = time.perf_counter()
    # the oracle's masks must match the GPU's (a cheap end-to-end sanity check)
    gpu_words = reps[0]["mask"].cpu().numpy().view(np.uint32)
    if not np.array_equal(gpu_words, pr["words"]):
        raise RuntimeError("GPU masks differ from the oracle's")
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    dec_s = (t2 - t1) / n_dec
    return {
        "value": effective_decode_bytes(w, T) / dec_s / 1e9, "unit": "GB/s", "cores": blas, "kind": "oracle",
        "sample": f"{w.name}: 1 prefill prune+stats ({t1 - t0:.1f} s) and {n_dec} full-shape decode steps "
                  f"({dec_s:.2f} s each) in NumPy float64; decode effective bytes / decode time; "
                  f"BLAS threads {blas}, elementwise NumPy single-threaded, host has {os.cpu_count()} CPUs",
        "prefill_s": t1 - t0, "decode_s_per_step": dec_s, "cpu_model": cpu_model(),
    }


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def summarize(kt_dir: str, fetch_dir: str, write_dir: str, bench_log: str, workload: str, command: str) -> str:
    """Render profiles/decode_kernel_llama8b_s32k_traffic.md from three
    rocprofv3 runs of the same bench command (kernel trace, FETCH_SIZE pass,
    WRITE_SIZE pass) and the bench JSON line the kernel-trace run printed:
    per kernel of the library its profiled duration and HBM bytes per
    dispatch, the counters scaled by what they read for the plain 256 MiB
    device copy the run also performs."""
    import csv
    import glob

    if not command.strip():
        raise SystemExit("--summary-command must give the rocprofv3 command lines the summary is made from")

    def rows(d, name):
        out = []
        for f in glob.glob(os.path.join(d, "**", name), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    def short(name):
        return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")

    stats = [r for r in rows(kt_dir, "*kernel_stats.csv") if "spark::" in r["Name"]]
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    dec = [r for r in stats if "decode_fast_kernel" in r["Name"] or "decode_kernel" in r["Name"]]
    kname = short(dec[0]["Name"])
    avg_ns = float(dec[0]["AverageNs"])

    def per_dispatch(d, counter):
        """KiB per dispatch of every library kernel (dimension entries of one
        dispatch summed, then averaged over dispatches), and the copy's."""
        per, calib = {}, []
        for r in rows(d, "*counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= 131072:
                calib.append(float(r["Counter_Value"]))
            if "spark::" in r["Kernel_Name"]:
                k = per.setdefault(short(r["Kernel_Name"]), {})
                k[r["Dispatch_Id"]] = k.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return {n: sum(v.values()) / len(v) for n, v in per.items()}, max(calib)

    fetch, f_cal = per_dispatch(fetch_dir, "FETCH_SIZE")
    write, w_cal = per_dispatch(write_dir, "WRITE_SIZE")
    copy_bytes = 256 << 20
    f_scale, w_scale = copy_bytes / (f_cal * 1024), copy_bytes / (w_cal * 1024)
    line = None
    for ln in open(bench_log):
        if ln.startswith("{"):
            line = json.loads(ln)
    ev_us = line["decode_us_per_launch"]
    alg = line["roofline"]["algorithmic_bytes_per_launch"]
    fetch_b, write_b = fetch[kname] * 1024 * f_scale, write[kname] * 1024 * w_scale
    cmds = "\n".join("    " + c.strip() for c in command.split(";;"))
    table = ["| kernel | calls | profiled avg us | HBM read MB / dispatch | HBM write MB / dispatch |",
             "|---|---|---|---|---|"]
    for r in stats:
        n = short(r["Name"])
        fr = f"{fetch[n] * 1024 * f_scale / 1e6:.2f}" if n in fetch else "-"
        wr = f"{write[n] * 1024 * w_scale / 1e6:.2f}" if n in write else "-"
        table.append(f"| {n} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {fr} | {wr} |")
    text = f"""# Library kernels: time and HBM traffic, {workload}

Commands (three rocprofv3 runs of the same bench command: kernel trace,
FETCH_SIZE pass, WRITE_SIZE pass; then this summary):

{cmds}

{chr(10).join(table)}

Counter scale: a 256 MiB device copy (__amd_rocclr_copyBuffer, run by the
bench's --calib-copy-mb 256) reads FETCH_SIZE {f_cal:.0f} KiB and WRITE_SIZE
{w_cal:.0f} KiB, so fetch counts are multiplied by {f_scale:.3f} and write
counts by {w_scale:.3f}. (The derived FETCH_SIZE weighs every read request
that is not 32 bytes as 64 bytes; the L2's fills from HBM on this chip are
128-byte requests, so the raw counter shows half the bytes a copy of known
size reads.)

Decode: the profiled average duration against the HIP-event time per
launch that the same (profiled) bench run printed, over its graph of 64
launches; the profiler slows every dispatch, so both read above the
unprofiled bench's time.

- kernel: {kname}
- workload: {workload}
- source_sha256: {decode_source_sha()}
- avg_duration_ns: {avg_ns:.0f}
- hipevent_us_per_launch: {ev_us:.3f}
- profiler_overhead_us: {avg_ns / 1e3 - ev_us:.3f}
- algorithmic_bytes_per_launch: {alg}
- frac_hipevent: {alg / (ev_us * 1e-6) / 1e9 / HBM_PEAK_GBS:.4f}
- frac_profiled: {alg / (avg_ns * 1e-9) / 1e9 / HBM_PEAK_GBS:.4f}
- fetch_kib_per_dispatch_raw: {fetch[kname]:.1f}
- write_kib_per_dispatch_raw: {write[kname]:.1f}
- fetch_bytes_per_launch: {fetch_b:.0f}
- write_bytes_per_launch: {write_b:.0f}
- hbm_bytes_per_launch: {fetch_b + write_b:.0f}
"""
    return text


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_s32k_l05")
    ap.add_argument("--second", default="llama8b_s32k_l08", help="second reported workload ('' to skip)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 128K-context, stacked-eviction and 32-layer workloads")
    ap.add_argument("--no-sampled", action="store_true", help="skip the sampled recovery F legs")
    ap.add_argument("--no-vprune", action="store_true", help="skip the K-and-V-pruned leg")
    ap.add_argument("--no-grouped", action="store_true", help="skip the SparK-g leg")
    ap.add_argument("--no-topp", action="store_true", help="skip the SparK-p leg")
    ap.add_argument("--no-growth", action="store_true", help="skip the growing-cache serving loop")
    ap.add_argument("--no-shard", action="store_true", help="skip the TP-8 shard-shape leg")
    ap.add_argument("--no-sweep", action="store_true", help="skip the decode time vs input length sweep")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the other pruning ratios and group sizes (lambda 0.3 and 0.6; G = 8 and 1)")
    ap.add_argument("--warm", action="store_true", help="also report a run without replica rotation")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run a plain device copy of this size after the legs (counter calibration)")
    ap.add_argument("--summarize", nargs=4, metavar=("KT_DIR", "FETCH_DIR", "WRITE_DIR", "BENCH_LOG"),
                    help="write the rocprofv3 traffic summary under profiles/ and exit")
    ap.add_argument("--summary-command", default="",
                    help="the rocprofv3 command lines the summary is made from, separated by ';;' (required)")
    args = ap.parse_args()
    if args.summarize:
        txt = summarize(*args.summarize, args.workload, args.summary_command)
        open(TRAFFIC_FILE, "w").write(txt)
        print(txt)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the SparK hot path here is a single-GPU kernel set; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_decode_attention_amd import ops
    from sparse_decode_attention_amd.configs import WORKLOADS

    ops.lib()
    w = WORKLOADS[args.workload]
    print(f"bench: {w.name} steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    main_leg = run_leg(w, args.steps, args.warmup)
    T = main_leg["T"]
    line = {
        "metric": METRIC,
        "value": round(main_leg["decode_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_leg["step_ms_median"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "N_q": w.n_q, "N_kv": w.n_kv, "D": w.D,
                   "window": w.window, "lambda": w.lam, "T": T, "decode_steps_per_step": w.steps,
                   "storage": "bf16 q/k/v/packed, uint32 mask, fp32 r/out", "replicas": main_leg["replicas"]},
        "pct_hbm_peak": round(100 * main_leg["decode_GBps"] / HBM_PEAK_GBS, 2),
        "decode_us_per_launch": round(main_leg["decode_us_per_launch"], 3),
        "tokens_heads_per_s": main_leg["tokens_heads_per_s"],
        "tokens_kv_heads_per_s": w.B * w.S * w.n_kv / (main_leg["decode_us_per_launch"] * 1e-6),
        "prefill": {"us": round(main_leg["prefill_us"], 2), "GBps": round(main_leg["prefill_GBps"], 1),
                    "bytes": effective_prefill_bytes(w, T),
                    "tokens_kv_heads_per_s": w.B * w.S * w.n_kv / (main_leg["prefill_us"] * 1e-6)},
    }
    traffic, prof_ns = read_traffic(w.name)
    dec_bytes = main_leg["decode_bytes_per_step"]
    line["roofline"] = {"bound": "hbm", "achieved": round(main_leg["decode_GBps"], 2), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(main_leg["decode_GBps"] / HBM_PEAK_GBS, 4),
                        "traffic": traffic, "kernel": decode_kernel_name(w.G, T),
                        "algorithmic_bytes_per_launch": dec_bytes,
                        # the committed rocprofv3 summary's average duration (it includes the
                        # profiler's per-dispatch overhead) and the fraction it gives
                        "profiled_us": None if prof_ns is None else round(prof_ns / 1e3, 3),
                        "frac_profiled": None if prof_ns is None else
                        round(dec_bytes / (prof_ns * 1e-9) / 1e9 / HBM_PEAK_GBS, 4)}
    ceil, ceil_blocks = stream_ceiling(dec_bytes)
    ceil_1g, ceil_1g_blocks = stream_ceiling(1 << 30)
    line["stream_ceiling"] = {"GBps": round(ceil, 1), "bytes": dec_bytes,
                              "frac_of_ceiling": round(main_leg["decode_GBps"] / ceil, 4), "blocks": ceil_blocks,
                              "GBps_1GiB": round(ceil_1g, 1), "blocks_1GiB": ceil_1g_blocks,
                              "what": "spark_read_stream (nontemporal 16-byte requests) of the same bytes, rotated "
                                      "like the decode replicas, and of 1 GiB; best over launch sizes of the median replay"}
    if args.second:
        w2 = WORKLOADS[args.second]
        print(f"bench: {w2.name}", file=sys.stderr, flush=True)
        leg2 = run_leg(w2, args.steps, args.warmup)
        line["second"] = {"workload": w2.name, "lambda": w2.lam, "T": leg2["T"],
                          "GBps": round(leg2["decode_GBps"], 2),
                          "pct_hbm_peak": round(100 * leg2["decode_GBps"] / HBM_PEAK_GBS, 2),
                          "decode_us_per_launch": round(leg2["decode_us_per_launch"], 3),
                          "prefill_GBps": round(leg2["prefill_GBps"], 1), "replicas": leg2["replicas"]}
        del leg2
    if not args.no_sampled:
        line["sampled_f"] = {}
        for rec in ("gaussian", "exponential"):
            print(f"bench: sampled F ({rec}) on {w.name}", file=sys.stderr, flush=True)
            lg = run_leg(w, min(args.steps, 5), min(args.warmup, 2), x=main_leg["x"], recovery=rec)
            alu_ops = w.B * w.n_kv * w.S * sampled_alu_ops_per_token(w.G, T, rec)
            alu_gops = alu_ops / (lg["decode_us_per_launch"] * 1e-6) / 1e9
            line["sampled_f"][rec] = {
                "workload": w.name, "kernel": decode_kernel_name(w.G, T, ops.RECOVERY[rec]),
                "decode_us_per_launch": round(lg["decode_us_per_launch"], 3),
                "GBps": round(lg["decode_GBps"], 2),
                "roofline": {"bound": "alu", "achieved": round(alu_gops, 1), "peak": VALU_PEAK_GOPS, "unit": "Gop/s",
                             "frac": round(alu_gops / VALU_PEAK_GOPS, 4), "traffic": None,
                             "ops_per_token_head": sampled_alu_ops_per_token(w.G, T, rec)},
                "x_fixed_r_time": round(lg["decode_us_per_launch"] / main_leg["decode_us_per_launch"], 3),
                "prefill_us": round(lg["prefill_us"], 2), "seed": hex(SAMPLE_SEED)}
            del lg
        torch.cuda.empty_cache()
    if not args.no_variants:
        # the runtime-T variants of the matrix-core kernel: other pruning
        # ratios (G = 4) and other group sizes (G = 8: 64 query heads over 8
        # KV heads; G = 1: as many query as KV heads), same S and B
        line["variants"] = []
        main_us, main_bytes = main_leg["decode_us_per_launch"], main_leg["decode_bytes_per_step"]
        for name, wv, xv in (("lambda=0.3", w.with_(name=w.name + "_lam03", lam=0.3), main_leg["x"]),
                             ("lambda=0.6", w.with_(name=w.name + "_lam06", lam=0.6), main_leg["x"]),
                             ("G=8", w.with_(name=w.name + "_g8", n_q=8 * w.n_kv), None),
                             ("G=1", w.with_(name=w.name + "_g1", n_q=w.n_kv), None)):
            print(f"bench: variant {name} ({wv.name})", file=sys.stderr, flush=True)
            lg = run_leg(wv, min(args.steps, 5), min(args.warmup, 2), x=xv)
            Tv = lg["T"]
            kern = decode_kernel_name(wv.G, Tv)
            line["variants"].append({
                "variant": name, "workload": wv.name, "G": wv.G, "lambda": wv.lam, "T": Tv, "kernel": kern,
                "decode_us_per_launch": round(lg["decode_us_per_launch"], 3),
                "bytes_per_launch": lg["decode_bytes_per_step"], "GBps": round(lg["decode_GBps"], 2),
                "pct_hbm_peak": round(100 * lg["decode_GBps"] / HBM_PEAK_GBS, 2),
                # time relative to the headline leg over bytes relative to it: 1.0 is byte-proportional
                "time_over_bytes_vs_headline": round((lg["decode_us_per_launch"] / main_us) /
                                                     (lg["decode_bytes_per_step"] / main_bytes), 3),
                "replicas": lg["replicas"]})
            del lg
        torch.cuda.empty_cache()
    if not args.no_vprune:
        line["v_pruned"] = {}
        for lam_v in (0.5,):
            print(f"bench: K and V pruned, lambda_v={lam_v}, on {w.name}", file=sys.stderr, flush=True)
            lg = run_leg(w, min(args.steps, 5), min(args.warmup, 2), x=main_leg["x"], lam_v=lam_v)
            line["v_pruned"][f"lambda_v={lam_v}"] = {
                "workload": w.name, "kernel": f"decode_kernel<{w.G}, 0, 1, false>", "T_v": lg["Tv"],
                "decode_us_per_launch": round(lg["decode_us_per_launch"], 3),
                "bytes_per_launch": lg["decode_bytes_per_step"],
                "GBps": round(lg["decode_GBps"], 2), "pct_hbm_peak": round(100 * lg["decode_GBps"] / HBM_PEAK_GBS, 2),
                "x_dense_v_time": round(lg["decode_us_per_launch"] / main_leg["decode_us_per_launch"], 3),
                "prefill_us_k_and_v": round(lg["prefill_us"], 2), "replicas": lg["replicas"]}
            del lg
        torch.cuda.empty_cache()
        # V pruned in 8-channel blocks: the matrix-core kernel reads packed V
        # blocks with the dense V requests
        line["v_block_pruned"] = {}
        for lam_v in (0.5, 0.8):
            print(f"bench: K pruned, V pruned in blocks, lambda_v={lam_v}, on {w.name}", file=sys.stderr, flush=True)
            lg = run_leg(w, min(args.steps, 5), min(args.warmup, 2), x=main_leg["x"], lam_vb=lam_v)
            line["v_block_pruned"][f"lambda_v={lam_v}"] = {
                "workload": w.name, "kernel": decode_kernel_name(w.G, lg["T"], vblocks=True), "n_b": lg["nbv"],
                "decode_us_per_launch": round(lg["decode_us_per_launch"], 3),
                "bytes_per_launch": lg["decode_bytes_per_step"],
                "GBps": round(lg["decode_GBps"], 2), "pct_hbm_peak": round(100 * lg["decode_GBps"] / HBM_PEAK_GBS, 2),
                "x_dense_v_time": round(lg["decode_us_per_launch"] / main_leg["decode_us_per_launch"], 3),
                "prefill_us_k_and_v": round(lg["prefill_us"], 2), "replicas": lg["replicas"]}
            del lg
        torch.cuda.empty_cache()
    if not args.no_shard:
        # one GPU's share of a tensor-parallel split over the 8 KV heads: one KV
        # head and its 4 query heads at S = 32K (the kernel a TP-8 deployment runs)
        ws = w.with_(name=w.name + "_tp8_shard", n_q=w.G, n_kv=1)
        print(f"bench: TP-8 shard shape {ws.name}", file=sys.stderr, flush=True)
        lg = run_leg(ws, min(args.steps, 5), min(args.warmup, 2))
        line["tp8_shard"] = {"workload": ws.name, "B": ws.B, "N_q": ws.n_q, "N_kv": ws.n_kv, "S": ws.S,
                             "lambda": ws.lam, "decode_us_per_launch": round(lg["decode_us_per_launch"], 3),
                             "GBps": round(lg["decode_GBps"], 2), "bytes_per_launch": lg["decode_bytes_per_step"],
                             "replicas": lg["replicas"]}
        del lg
        torch.cuda.empty_cache()
    if not args.no_growth:
        print(f"bench: growing cache on {w.name}", file=sys.stderr, flush=True)
        line["growth"] = growth_leg(w, min(args.steps, 5), min(args.warmup, 2), main_leg["x"])
        line["growth"]["x_static_decode_time"] = round(line["growth"]["us_per_step_append_and_decode"] /
                                                       main_leg["decode_us_per_launch"], 3)
        torch.cuda.empty_cache()
    if not args.no_topp:
        print(f"bench: SparK-p 0.99 on {w.name}", file=sys.stderr, flush=True)
        lg = run_leg(w, min(args.steps, 5), min(args.warmup, 2), x=main_leg["x"], top_p=0.99)
        line["top_p"] = {
            "workload": w.name, "p": 0.99, "mean_kept": round(lg["T"], 2),
            "pruning_ratio": round(1 - lg["T"] / w.D, 4), "kernel": decode_kernel_name(w.G, w.D, ragged=True),
            "decode_us_per_launch": round(lg["decode_us_per_launch"], 3), "bytes_per_launch": lg["decode_bytes_per_step"],
            "GBps": round(lg["decode_GBps"], 2), "pct_hbm_peak": round(100 * lg["decode_GBps"] / HBM_PEAK_GBS, 2),
            "prefill_us": round(lg["prefill_us"], 2), "replicas": lg["replicas"]}
        del lg
        torch.cuda.empty_cache()
    if not args.no_grouped:
        ratios = [0.25, 0.5, 0.75, 1.0]
        print(f"bench: SparK-g {ratios} on {w.name}", file=sys.stderr, flush=True)
        lg = run_leg(w, min(args.steps, 5), min(args.warmup, 2), x=main_leg["x"], ratios=ratios)
        line["grouped"] = {
            "workload": w.name, "ratios": ratios, "T": lg["T"], "kernel": decode_kernel_name(w.G, lg["T"]),
            "decode_us_per_launch": round(lg["decode_us_per_launch"], 3), "GBps": round(lg["decode_GBps"], 2),
            "pct_hbm_peak": round(100 * lg["decode_GBps"] / HBM_PEAK_GBS, 2), "prefill_us": round(lg["prefill_us"], 2),
            "prefill_GBps": round(lg["prefill_GBps"], 1), "replicas": lg["replicas"]}
        del lg
        torch.cuda.empty_cache()
    if not args.no_extra:
        w3 = WORKLOADS["llama8b_s128k_l08"]
        print(f"bench: {w3.name}", file=sys.stderr, flush=True)
        leg3 = run_leg(w3, min(args.steps, 5), min(args.warmup, 2))
        line["s128k"] = {"workload": w3.name, "lambda": w3.lam, "T": leg3["T"],
                         "GBps": round(leg3["decode_GBps"], 2),
                         "pct_hbm_peak": round(100 * leg3["decode_GBps"] / HBM_PEAK_GBS, 2),
                         "decode_us_per_launch": round(leg3["decode_us_per_launch"], 3),
                         "prefill_us": round(leg3["prefill_us"], 2), "prefill_GBps": round(leg3["prefill_GBps"], 1),
                         "replicas": leg3["replicas"]}
        del leg3
        torch.cuda.empty_cache()
        print("bench: stacked eviction", file=sys.stderr, flush=True)
        line["evict_stack"] = evict_leg(WORKLOADS["snapkv_b8_s32k_keep4k_l07"], min(args.steps, 5),
                                        min(args.warmup, 2))
        torch.cuda.empty_cache()
        print("bench: 32-layer stack", file=sys.stderr, flush=True)
        line["layer_stack"] = stack_leg(WORKLOADS["llama8b_32L_b4_s64k_l08"], min(args.steps, 5),
                                        min(args.warmup, 2))
        torch.cuda.empty_cache()
    if not args.no_sweep:
        print("bench: decode time vs input length", file=sys.stderr, flush=True)
        line["length_sweep"] = sweep_leg(w, steps=min(args.steps, 5), warmup=min(args.warmup, 2))
        torch.cuda.empty_cache()
    if args.warm:
        wl = run_leg(w, args.steps, args.warmup, rotate=False)
        line["warm_single_replica_GBps"] = round(wl["decode_GBps"], 2)
        del wl
    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20)
        a = torch.empty(n // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        line["calib_copy_bytes"] = n
    if not args.no_cpu:
        print("bench: cpu oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, main_leg["x"], main_leg["reps"], T)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
