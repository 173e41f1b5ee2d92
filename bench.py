#!/usr/bin/env python3
"""Benchmark of the BSA hot path on one MI355X.

One step = bsa_select (pooling, pooled scores, softmax, top-k/CDF selection)
followed by bsa_attention (block-restricted flash attention) over one batch
of synthetic input already resident in HBM. Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload long|720p|480p|vc|tiny]

value = effective TFLOP/s of the whole step, with effective FLOP
4 * n_q * kept_keys * d per head (only kept query-block x key-block pairs
count). The CPU oracle is timed on a bounded sample of the same workload on
the host cores as a reported baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E, published
METRIC = "BSA effective TFLOP/s & ms/layer at 720p-scale (~92K/215K tokens), % MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "video_dit_block_bsa_amd", "csrc", f)
                  for f in ("attention.hip", "tile.h", "common.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_info() -> dict:
    """Compute-unit count and maximum engine clock of the GPU agent as
    rocminfo reports them (the peak figures assume 256 CUs at 2.4 GHz)."""
    import subprocess

    info = {"source": "rocminfo"}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        out = ""
    agent = None
    for block in out.split("*******"):
        if "gfx950" in block and "Compute Unit:" in block:
            agent = block
            break
    if agent:
        for line in agent.splitlines():
            key, _, val = line.strip().partition(":")
            val = val.strip().split()[0] if val.strip() else ""
            if key == "Marketing Name":
                info["name"] = line.split(":", 1)[1].strip()
            elif key == "Compute Unit" and val.isdigit():
                info["compute_units"] = int(val)
            elif key == "Max Clock Freq. (MHz)" and val.isdigit():
                info["max_clock_mhz"] = int(val)
    if "compute_units" not in info or not info.get("name"):
        import torch

        props = torch.cuda.get_device_properties(0)
        if "compute_units" not in info:
            info.update(source="torch", compute_units=props.multi_processor_count)
        info["name"] = info.get("name") or props.name
    return info


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def kernel_source_hash() -> str:
    """Hash of the attention kernel's sources (the kernel file and the
    headers it includes) without comments and blank lines, so that only a
    change to the code itself retires a counter record."""
    code = []
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            for line in f:
                line = line.split("//", 1)[0].rstrip()
                if line:
                    code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def traffic_for(workload_name: str):
    """HBM bytes per attention launch from committed rocprofv3 counter runs,
    or None if absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    w = rec.get("workloads", {}).get(workload_name)
    if not w:
        return None
    return w.get("hbm_bytes_per_launch")


LAUNCH_WORKGROUPS = 15 * 512  # workgroups per sparse attention launch (library constant)


def attention_launches(w) -> int:
    """Kernel launches per bsa_attention call, as the library makes them:
    launches of LAUNCH_WORKGROUPS workgroups, counted over batch*heads x the
    query-block workgroups of a head rounded up to a multiple of 8. A
    workgroup takes one query block, or with 64-token query blocks and
    128-token key blocks on grids the chunks divide (more than one block
    along w) a t-adjacent pair of them."""
    bh = w.batch * w.heads
    (ct, ch, cw), (kt, kh, kw) = w.chunk, w.kchunk
    divides = all(n % c == 0 for n, c in zip((w.T, w.H, w.W), w.chunk)) and \
        all(n % c == 0 for n, c in zip((w.T, w.H, w.W), w.kchunk))
    one_wide = w.W // cw == 1 or (w.H // ch) * (w.W // cw) == 1 or w.W // kw == 1 or \
        (w.H // kh) * (w.W // kw) == 1
    per_head = w.num_blocks
    if w.block_tokens != 128 and w.key_block_tokens == 128 and divides and not one_wide:
        nhw = (w.H // ch) * (w.W // cw)
        per_head = (w.num_blocks // nhw + 1) // 2 * nhw
    return -(-(bh * (-(-per_head // 8) * 8)) // LAUNCH_WORKGROUPS)


def roofline_record(flops: float, avg_ms: float, traffic, launches: int = 1) -> dict:
    """Roofline of the attention kernel (the step's dominant kernel) against
    both roofs, per launch: `flops` and `avg_ms` are one launch's effective
    flops and average duration (a bsa_attention call of `launches` launches
    of equal work). Effective flops go over the bf16 MFMA peak, HBM-side
    bytes counted by rocprofv3 (FETCH_SIZE and WRITE_SIZE per launch, or None
    without a current record) over the HBM peak. The binding roof is the one
    the kernel comes closer to; `achieved`, `peak`, `unit` and `frac`
    describe that roof."""
    sec = avg_ms * 1e-3
    tflops = flops / sec / 1e12
    frac_mfma = tflops / PEAK_BF16_TFLOPS
    gbps = None if traffic is None else traffic / sec / 1e9
    frac_hbm = None if gbps is None else gbps / PEAK_HBM_GBPS
    hbm = frac_hbm is not None and frac_hbm > frac_mfma
    return {
        "bound": "hbm" if hbm else "mfma",
        "kernel": "bsa_attention (block-sparse flash attention, attn_kernel<false, false, KeyMode>)",
        "achieved": round(gbps if hbm else tflops, 2),
        "peak": PEAK_HBM_GBPS if hbm else PEAK_BF16_TFLOPS,
        "unit": "GB/s" if hbm else "TFLOP/s",
        "frac": round(frac_hbm if hbm else frac_mfma, 4),
        "frac_mfma": round(frac_mfma, 4),
        "frac_hbm": None if frac_hbm is None else round(frac_hbm, 4),
        "achieved_tflops": round(tflops, 2),
        "achieved_hbm_gbps": None if gbps is None else round(gbps, 1),
        "traffic": traffic,
        "flops_per_launch": flops,
        "avg_launch_ms": round(avg_ms, 4),
        "launches_per_call": launches,
    }


def cpu_baseline(w, q, k, v, blocks: int, seconds: float):
    """Time the CPU oracle on one head: full selection for the head, then
    attention for query blocks 0, 1, ... until `blocks` are done or the
    attention part has run for `seconds`. Selection time is prorated to the
    blocks done. Returns the baseline record."""
    import numpy as np

    import oracle.bsa_oracle as O

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:  # threadpoolctl missing: report the visible cores
        threads = os.cpu_count() or 1
    kc = tuple(w.key_chunk) if w.key_chunk else (0, 0, 0)
    g = O.Geometry(w.T, w.H, w.W, *w.chunk, cond_frames=w.cond_frames, ctk=kc[0], chk=kc[1],
                   cwk=kc[2])
    sp = (O.SelectParams("topk", k=w.k) if w.mode == "topk"
          else O.SelectParams("cdf", p=w.p, k_min=w.k_min, k_max=w.k_max))
    scale = 1.0 / math.sqrt(w.head_dim)
    qf, kf, vf = (O.bf16_bits_to_f64(a[0, 0]) for a in (q, k, v))
    t0 = time.perf_counter()
    idx, cnt, _ = O.select_head(qf, kf, g, sp, scale)
    t_sel = time.perf_counter() - t0
    blocks = min(blocks, g.num_blocks)
    perm = O.block_token_order(g)
    kperm = O.block_token_order(O.key_geometry(g))
    t0 = time.perf_counter()
    done = 0
    while done < blocks and (done == 0 or time.perf_counter() - t0 < seconds):
        O.attend_query_block(qf, kf, vf, g, done, idx[done, : cnt[done]], scale, perm, kperm)
        done += 1
    t_att = time.perf_counter() - t0
    blocks = done
    t = t_att + t_sel * blocks / g.num_blocks
    flops = 4.0 * g.n * g.nk * w.head_dim * float(cnt[:blocks].sum())
    rate = flops / t
    return {
        "value": round(rate / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"head 0 of {w.name}: selection of all {g.num_blocks} query blocks "
                   f"({t_sel:.2f} s, prorated) + float64 attention of the first {blocks} "
                   f"query blocks ({t_att:.2f} s)"),
        "seconds": round(t_sel + t_att, 2),
        "rate_flop_per_s": rate,
    }


def backward_bench(w, problem, qd, kd, vd, idx, cnt, stride, ws_att, stream, eff, steps):
    """Training step of the attention on the same selection: bsa_attention_lse
    (forward that also writes the log-normaliser) then bsa_attention_bwd with
    a synthetic dO. Effective FLOP of the backward follow the usual count of
    five products (dV, dP, dQ, dK and the recomputed S: 2.5x the forward's);
    the kernels execute seven (S and dP are recomputed for dQ and for dK/dV)."""
    import numpy as np
    import torch

    from video_dit_block_bsa_amd import binding as B
    from video_dit_block_bsa_amd.inputs import make_grad

    dod = torch.from_numpy(make_grad(w.T, w.H, w.W, w.heads, w.head_dim, w.batch,
                                     seed=w.seed)).view(torch.bfloat16).cuda()
    o = torch.empty_like(qd)
    lse = torch.empty((w.batch, w.heads, w.seq_len), dtype=torch.float32, device="cuda")
    grads = [torch.empty_like(qd) for _ in range(3)]
    wsb = torch.empty(B.attention_bwd_workspace_bytes(problem), dtype=torch.uint8, device="cuda")

    def one(ev=None):
        if ev is not None:
            ev[0].record(stream)
        B.bsa_attention_lse(problem, qd, kd, vd, idx, cnt, stride, o, lse, ws_att, stream)
        if ev is not None:
            ev[1].record(stream)
        B.bsa_attention_bwd(problem, qd, kd, vd, o, dod, lse, idx, cnt, stride, *grads, wsb,
                            stream)
        if ev is not None:
            ev[2].record(stream)

    one()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for s in range(steps):
        one(events[s])
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    bwd_eff = 2.5 * eff
    log(f"[bench] training pass: forward with lse {fwd_ms:.3f} ms, backward {bwd_ms:.3f} ms "
        f"({bwd_eff / (bwd_ms * 1e-3) / 1e12:.1f} effective TFLOP/s)")
    del dod, o, lse, grads, wsb
    torch.cuda.empty_cache()
    return {
        "entry_points": "bsa_attention_lse + bsa_attention_bwd (selection fixed)",
        "steps": steps,
        "forward_lse_ms": round(fwd_ms, 4),
        "backward_ms": round(bwd_ms, 4),
        "effective_tflop": round(bwd_eff / 1e12, 4),
        "effective_tflops": round(bwd_eff / (bwd_ms * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100 * bwd_eff / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "executed_mfma_tflop": round(3.5 * eff / 1e12, 4),
        "dtype": "bf16",
    }


def cond_cache_bench(w, problem, params, qd, kd, vd, stride, full_ms, steps):
    """One denoising step with the condition-KV cache: bsa_select_noisy +
    bsa_attention_noisy over the noisy query blocks, condition pooled keys
    from a cache filled once (untimed), against the full step above."""
    import numpy as np
    import torch

    from video_dit_block_bsa_amd import binding as B

    rows = w.batch * w.heads * w.num_blocks
    idx = torch.empty((rows, stride), dtype=torch.int32, device="cuda")
    cnt = torch.empty((rows,), dtype=torch.int32, device="cuda")
    o = torch.empty_like(qd)
    ws = torch.empty(B.select_workspace_bytes(problem, params), dtype=torch.uint8, device="cuda")
    cache = torch.empty(B.cond_cache_bytes(problem) // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    B.bsa_pool_cond_keys(problem, kd, cache, stream)

    def one():
        B.bsa_select_noisy(problem, params, qd, kd, cache, idx, cnt, ws, stream)
        B.bsa_attention_noisy(problem, qd, kd, vd, idx, cnt, stride, o, ws, stream)

    one()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        one()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    cond_blocks = w.cond_blocks
    log(f"[bench] condition-KV cache step: {ms:.3f} ms (full step {full_ms:.3f} ms)")
    del idx, cnt, o, ws, cache
    return {
        "entry_points": "bsa_select_noisy + bsa_attention_noisy (bsa_pool_cond_keys once)",
        "steps": steps,
        "noisy_step_ms": round(ms, 4),
        "full_step_ms": round(full_ms, 4),
        "speedup": round(full_ms / ms, 3),
        "noisy_query_blocks": w.num_blocks - cond_blocks,
        "query_blocks": w.num_blocks,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--dense-steps", type=int, default=1,
                    help="timed dense_attention runs for the speedup figure (0 = skip)")
    ap.add_argument("--cpu-blocks", type=int, default=1 << 20,
                    help="at most this many query blocks in the CPU oracle sample (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="stop the CPU oracle sample after this much attention time")
    ap.add_argument("--backward-steps", type=int, default=5,
                    help="timed training forward (with lse) + backward passes (0 = skip)")
    ap.add_argument("--cond-cache-steps", type=int, default=5,
                    help="timed steps of the condition-KV cache path (noisy query blocks only; "
                         "workloads with condition frames; 0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first, so that "
                         "hardware byte counters can be calibrated against a known size")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path is "
              "built and measured on a single MI355X; see the design notes for how it would "
              "shard across GPUs.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from video_dit_block_bsa_amd import WORKLOADS, effective_flops
    from video_dit_block_bsa_amd import binding as B
    from video_dit_block_bsa_amd.inputs import make_qkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    w = WORKLOADS[args.workload]
    t0 = time.perf_counter()
    q, k, v = make_qkv(w.T, w.H, w.W, w.heads, w.head_dim, w.batch, kind=w.kind, seed=w.seed)
    log(f"[bench] inputs for {w.name} generated in {time.perf_counter() - t0:.1f} s")
    to_dev = lambda a: torch.from_numpy(a).view(torch.bfloat16).cuda()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    problem = B.Problem.from_workload(w)
    params = B.SelectParams.from_workload(w)
    stride = B.index_stride(problem, params)
    rows = w.batch * w.heads * w.num_blocks
    idx = torch.empty((rows, stride), dtype=torch.int32, device="cuda")
    cnt = torch.empty((rows,), dtype=torch.int32, device="cuda")
    o = torch.empty_like(qd)
    ws_sel = torch.empty(B.select_workspace_bytes(problem, params), dtype=torch.uint8, device="cuda")
    ws_att = torch.empty(B.attention_workspace_bytes(problem), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        B.bsa_select(problem, params, qd, kd, idx, cnt, ws_sel, stream)
        if ev is not None:
            ev[1].record(stream)
        B.bsa_attention(problem, qd, kd, vd, idx, cnt, stride, o, ws_att, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kept = int(cnt.sum().item())
    eff = effective_flops(w, kept)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sel_ms = [e[0].elapsed_time(e[1]) for e in events]
    att_ms = [e[1].elapsed_time(e[2]) for e in events]
    step_ms = [e[0].elapsed_time(e[2]) for e in events]
    ms_per_step = wall * 1e3 / args.steps
    value = eff / (ms_per_step * 1e-3) / 1e12
    att_avg = float(np.mean(att_ms))
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (select {np.mean(sel_ms):.3f} ms, "
        f"attention {att_avg:.3f} ms), {value:.1f} effective TFLOP/s")

    dense_ms = None
    if args.dense_steps > 0:
        ws_d = ws_att
        od = torch.empty_like(qd)
        B.dense_attention(problem, qd, kd, vd, od, ws_d, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.dense_steps):
            B.dense_attention(problem, qd, kd, vd, od, ws_d, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / args.dense_steps
        log(f"[bench] dense_attention: {dense_ms:.2f} ms")
        del od

    cache_rec = None
    if args.cond_cache_steps > 0 and w.cond_frames > 0:
        cache_rec = cond_cache_bench(w, problem, params, qd, kd, vd, stride, ms_per_step,
                                     args.cond_cache_steps)

    bwd = None
    if args.backward_steps > 0:
        bwd = backward_bench(w, problem, qd, kd, vd, idx, cnt, stride, ws_att, stream, eff,
                             args.backward_steps)

    launches = attention_launches(w)
    roofline = roofline_record(eff / launches, att_avg / launches, traffic_for(w.name), launches)
    cpu = None
    if args.cpu_blocks > 0:
        del qd, kd, vd
        torch.cuda.empty_cache()
        log("[bench] timing the CPU oracle sample ...")
        cpu = cpu_baseline(w, q, k, v, args.cpu_blocks, args.cpu_seconds)
        # The oracle's time for the whole layer (every head and query block)
        # at the sampled rate.
        cpu["ms_per_layer"] = round(eff / cpu.pop("rate_flop_per_s") * 1e3, 1)
        log(f"[bench] CPU oracle: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads "
            f"({cpu['seconds']} s; {cpu['ms_per_layer'] / 1e3:.0f} s per layer)")

    ct, ch, cw = w.chunk
    sel_desc = (f"top-k {w.k}" if w.mode == "topk"
                else f"CDF p={w.p} clamp [{w.k_min},{w.k_max}]")
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}: latent grid {w.T}x{w.H}x{w.W} ({w.seq_len} tokens, "
                         f"{w.num_blocks} blocks of [{ct},{ch},{cw}]"
                         + (f", {w.num_key_blocks} key blocks of [{','.join(map(str, w.kchunk))}]"
                            if w.key_chunk else "")
                         + f"), batch {w.batch}, "
                         f"{w.heads} heads, head_dim {w.head_dim}, {sel_desc}"
                         + (f", cond_frames {w.cond_frames}" if w.cond_frames else "")),
            "tokens": w.seq_len,
            "heads": w.heads,
            "kept_key_blocks": kept,
            "effective_tflop_per_step": round(eff / 1e12, 4),
        },
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "ms_per_step_min": round(float(np.min(step_ms)), 4),
        "device": device_info(),
        "select_ms": round(float(np.mean(sel_ms)), 4),
        "attention_ms": round(att_avg, 4),
        "dense_ms": None if dense_ms is None else round(dense_ms, 3),
        "speedup_vs_dense": None if dense_ms is None else round(dense_ms / ms_per_step, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "backward": bwd,
        "cond_cache": cache_rec,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
