"""Throughput of the whole hot path on one MI355X.

One step = score every reconstruction chunk of every layer of the cache
(kvz_score_chunk, L x n_chunks calls), select the global keep set
(kvz_select_threshold) and compact the kept K/V rows (kvz_compact), on
synthetic inputs already resident in device memory.

Prints one JSON line: context tokens scored and compacted per second, the
roofline of the dominant kernel (from HIP events recorded around each launch
inside the timed steps) and the CPU oracle's rate on a bounded sample.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0
METRIC = "context tokens scored+compacted/sec (8B shape, 128K ctx); % bf16 MFMA peak"


def score_flops(wl, n_in):
    """Algorithmic flops of one kvz_score_chunk call: one q.k product (2d
    flops) per visible (row, key) pair, pass 1 over context + causal chunk
    keys, pass 2 over context keys."""
    H, G, d, n_c = wl.heads, wl.group, wl.head_dim, wl.n_ctx
    vis_rows = G * (n_in * n_c + n_in * (n_in + 1) // 2)
    p1 = 2 * d * H * vis_rows
    p2 = 2 * d * H * G * n_in * n_c
    return p1, p2


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/<kernel>_<workload>_traffic.md), or None when that summary was
    taken on a different kernel source than the one built now."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    src = os.path.join(ROOT, "attention_score_reduction_amd", "csrc", "score.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("score.hip sha256") != sha:
        return None
    try:
        return int(fields["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, budget_s):
    """The oracle as it stands on a bounded sample: one (layer, head) pair,
    as many whole chunks as fit in about budget_s seconds; the full step is
    extrapolated linearly in (layer, head, chunk) units."""
    import numpy as np
    from attention_score_reduction_amd.inputs import HostGen
    from oracle import ras

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    gen = HostGen(wl)
    kc, _ = gen.context(0, [0])
    kc64 = ras.to_f64(kc, wl.dtype)
    S = np.zeros((1, wl.n_ctx))
    scale = 1 / math.sqrt(wl.head_dim)
    done = 0
    t_total = 0.0
    n_chunks = len(wl.chunks())
    while done < n_chunks:
        q, kin = gen.chunk_inputs(0, done, [0])
        q64, k64 = ras.to_f64(q, wl.dtype), ras.to_f64(kin, wl.dtype)
        t0 = time.perf_counter()
        ras.score_chunk(q64, kc64, k64, scale, S)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total > budget_s:
            break
    units_full = wl.layers * wl.heads * n_chunks
    t_full = t_total / done * units_full
    return {"value": wl.n_ctx / t_full, "unit": "context tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"scoring of {done} of {n_chunks} chunks for 1 of {wl.layers * wl.heads} "
                      f"(layer, head) pairs in {t_total:.1f} s, extrapolated x{units_full / done:.0f} "
                      f"to the full step (selection and compaction not included)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llama8b_128k")
    ap.add_argument("--layers", type=int, default=None, help="fewer layers (debug only)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-attention comparison after the timed steps")
    ap.add_argument("--no-attn", action="store_true",
                    help="skip the fused attention-output measurement after the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a 2 GiB device-to-device copy (a plain copy "
                         "kernel of known size, to scale the HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the per-head scoring would shard across GPUs without communication, but no "
              "multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_score_reduction_amd as kvz
    from attention_score_reduction_amd.inputs import WORKLOADS, device_tensors

    wl = WORKLOADS[args.workload]
    if args.layers:
        wl = wl.with_(layers=args.layers)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {wl.name} inputs on device", file=sys.stderr, flush=True)
    t0 = time.time()
    data = device_tensors(wl, device="cuda")
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f} s, "
          f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB", file=sys.stderr, flush=True)

    L, H, G, d, n_c = wl.layers, wl.heads, wl.group, wl.head_dim, wl.n_ctx
    chunks = wl.chunks()
    n_heads = L * H
    K = kvz.kvz_keep_count(n_heads * n_c, wl.keep_ratio)
    dt_code = 0 if wl.dtype == "bf16" else 1
    n_in_max = wl.n_prompt + max(m for _, m in chunks)
    ws_score = torch.empty(kvz.kvz_score_chunk_workspace(dt_code, H, G, n_in_max, d, n_c),
                           dtype=torch.uint8, device=dev)
    ws_sel = torch.empty(kvz.kvz_select_workspace(n_heads, n_c), dtype=torch.uint8, device=dev)
    per_layer_compact = wl.name.startswith("gemma")
    cmp_heads = H if per_layer_compact else n_heads
    ws_cmp = torch.empty(kvz.kvz_compact_workspace(cmp_heads, n_c), dtype=torch.uint8, device=dev)
    S = torch.zeros(n_heads, n_c, dtype=torch.float32, device=dev)
    mask = torch.empty(n_heads * n_c, dtype=torch.uint8, device=dev)
    offs = torch.empty(n_heads + 1, dtype=torch.int64, device=dev)
    tau = torch.empty(1, dtype=torch.float32, device=dev)
    tdt = data["kc"].dtype
    k_out = torch.empty(K, d, dtype=tdt, device=dev)
    v_out = torch.empty(K, d, dtype=tdt, device=dev)
    idx = torch.empty(K, dtype=torch.int32, device=dev)
    kc_flat = data["kc"].view(n_heads, n_c, d)
    vc_flat = data["vc"].view(n_heads, n_c, d)
    scale = 1 / math.sqrt(d)
    stream = torch.cuda.current_stream()

    def step():
        S.zero_()
        for l in range(L):
            Sl = S[l * H:(l + 1) * H]
            for k in range(len(chunks)):
                kvz.kvz_score_chunk(data["q"][l][k], data["kc"][l], data["kin"][l][k], Sl,
                                    wl.n_prompt, scale, ws=ws_score, stream=stream)
        kvz.kvz_select_threshold(S, K, mask, offs, tau, ws=ws_sel, stream=stream)
        if per_layer_compact:
            for l in range(L):
                kvz.kvz_compact(kc_flat[l * H:(l + 1) * H], vc_flat[l * H:(l + 1) * H], mask,
                                offs, k_out, v_out, idx, head_begin=l * H, ws=ws_cmp,
                                stream=stream)
        else:
            kvz.kvz_compact(kc_flat, vc_flat, mask, offs, k_out, v_out, idx, ws=ws_cmp,
                            stream=stream)

    for w in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup step {w} done", file=sys.stderr, flush=True)

    launches_per_step = L * len(chunks) * 3 + 16 + (3 * L if per_layer_compact else 3)
    kvz.kvz_prof_enable(True, launches_per_step * args.steps + 64)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step()
        torch.cuda.synchronize()
        print(f"[bench] step {s} done at {time.perf_counter() - t0:.2f} s", file=sys.stderr,
              flush=True)
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1000.0 / args.steps

    names = ["score_pass1", "score_combine", "score_pass2", "select_init", "select_hist",
             "select_pick", "select_fixup", "select_scan", "select_mask", "compact_count",
             "compact_scan", "compact_scatter"]
    kern = {}
    for nm in names:
        n, ms = kvz.kvz_prof_read(nm)
        if n:
            kern[nm] = {"launches": n, "total_ms_per_step": ms / args.steps, "avg_us": ms / n * 1e3}
    kvz.kvz_prof_enable(False)

    # HBM-bound kernels: algorithmic bytes per step / their time
    row_bytes = d * (2 if wl.dtype == "bf16" else 4)
    N = n_heads * n_c
    hbm_bytes = {
        # gather K and V rows, write them packed, idx, read the mask
        "compact_scatter": K * (4 * row_bytes + 4) + N,
        # reads of S: two radix-histogram passes and the mask pass; plus the
        # mask write.  When the K-th boundary splits a run of equal scores
        # (fp32 maxima collide on these caches) the tie fix-up re-reads only
        # the few tiles holding kept ties, which is left out
        "select_total": 3 * 4 * N + N,
    }
    hbm = {}
    if "compact_scatter" in kern:
        t = kern["compact_scatter"]["total_ms_per_step"] * 1e-3
        hbm["compact_scatter"] = {"bytes": hbm_bytes["compact_scatter"],
                                  "achieved_GBs": round(hbm_bytes["compact_scatter"] / t / 1e9, 1),
                                  "frac": round(hbm_bytes["compact_scatter"] / t / 1e9 / HBM_PEAK_GBS, 4)}
    sel_ms = sum(v["total_ms_per_step"] for k2, v in kern.items() if k2.startswith("select_"))
    if sel_ms:
        hbm["select_total"] = {"bytes": hbm_bytes["select_total"],
                               "achieved_GBs": round(hbm_bytes["select_total"] / (sel_ms * 1e-3) / 1e9, 1),
                               "frac": round(hbm_bytes["select_total"] / (sel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               "time_ms": round(sel_ms, 4)}

    # roofline of the dominant kernel (score passes: MFMA-bound)
    dom = max(kern, key=lambda k: kern[k]["total_ms_per_step"])
    full = [c for c in chunks if c[1] == wl.chunk]
    n_in = wl.n_prompt + (full[0][1] if full else chunks[0][1])
    p1, p2 = score_flops(wl, n_in)
    roof = None
    if dom in ("score_pass1", "score_pass2"):
        # per-launch figure for the full-length chunk; the ragged tail chunk
        # (if any) is counted by its own flops in the time-weighted average
        tot_flops = 0.0
        for (_, m) in chunks:
            a, b = score_flops(wl, wl.n_prompt + m)
            tot_flops += a if dom == "score_pass1" else b
        tot_flops *= L
        ach = tot_flops / (kern[dom]["total_ms_per_step"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(dom, wl.name), "kernel": dom,
                "flops_per_launch": p1 if dom == "score_pass1" else p2,
                "avg_launch_us": round(kern[dom]["avg_us"], 2)}
    # whole-score MFMA fraction over both passes (algorithmic flops)
    score_ms = sum(kern.get(k, {}).get("total_ms_per_step", 0.0)
                   for k in ("score_pass1", "score_combine", "score_pass2"))
    alg = 0.0
    for (_, m) in chunks:
        a, b = score_flops(wl, wl.n_prompt + m)
        alg += a + b
    alg *= L
    score_frac = alg / (score_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS if score_ms else None

    out = {
        "metric": METRIC,
        "value": round(n_c / (ms_per_step * 1e-3), 2),
        "unit": "context tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "kv_heads": H, "group": G, "head_dim": d,
                   "n_ctx": n_c, "chunk": wl.chunk, "n_prompt": wl.n_prompt,
                   "keep_ratio": wl.keep_ratio, "keep_count": K},
        "roofline": roof,
        "score_mfma_frac": round(score_frac, 4) if score_frac else None,
        "hbm_kernels": hbm,
        "head_token_scores_per_s": round(n_heads * n_c / (ms_per_step * 1e-3), 1),
        "kernels": {k: {kk: round(vv, 3) if isinstance(vv, float) else vv for kk, vv in v.items()}
                    for k, v in kern.items()},
    }
    # decode attention over the packed cache vs the full cache (one decode
    # token per query head, all layers), outside the headline step
    if not args.no_decode:
        import torch as _t
        gq = _t.Generator(device="cuda")
        gq.manual_seed(wl.seed + 100)
        q_dec = _t.randn(n_heads, G, d, generator=gq, device=dev).to(tdt)
        offs_full = _t.arange(n_heads + 1, device=dev, dtype=_t.int64) * n_c
        ws_dec = _t.empty(kvz.kvz_decode_workspace(n_heads, G, d, n_c), dtype=_t.uint8, device=dev)
        out_dec = _t.empty(n_heads, G, d, dtype=_t.float32, device=dev)

        def time_decode(k_rows, v_rows, offsets, reps=10):
            for _ in range(2):
                kvz.kvz_decode_packed(q_dec, k_rows, v_rows, offsets, n_c, out=out_dec, ws=ws_dec)
            _t.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                kvz.kvz_decode_packed(q_dec, k_rows, v_rows, offsets, n_c, out=out_dec, ws=ws_dec)
            _t.cuda.synchronize()
            return (time.perf_counter() - t0) / reps * 1e3

        t_full = time_decode(kc_flat.view(-1, d), vc_flat.view(-1, d), offs_full)
        t_kept = time_decode(k_out, v_out, offs)
        elt = 2 if wl.dtype == "bf16" else 4
        out["decode"] = {
            "full_cache_ms": round(t_full, 4), "kept_cache_ms": round(t_kept, 4),
            "speedup": round(t_full / t_kept, 3), "keep_ratio": wl.keep_ratio,
            "full_GBs": round(2 * N * d * elt / (t_full * 1e-3) / 1e9, 1),
            "kept_GBs": round(2 * K * d * elt / (t_kept * 1e-3) / 1e9, 1),
            "what": f"one decode token for all {G * n_heads} query heads over all {n_heads} "
                    "(layer, KV head) caches",
        }
    # fused reconstruction attention (scores plus the chunk's output
    # O = P [V_c; V_in]) on the first chunk of layer 0, outside the headline
    # step: per-kernel times of one call and the output pass's MFMA rate
    if not args.no_attn:
        import torch as _t
        k0 = 0
        n_in0 = wl.n_prompt + chunks[k0][1]
        gv = _t.Generator(device="cuda")
        gv.manual_seed(wl.seed + 200)
        v_in = _t.randn(H, n_in0, d, generator=gv, device=dev).to(tdt)
        o_buf = _t.empty(H, G, n_in0, d, dtype=_t.float32, device=dev)
        ws_attn = _t.empty(kvz.kvz_score_chunk_attn_workspace(dt_code, H, G, n_in0, d, n_c),
                           dtype=_t.uint8, device=dev)
        S_attn = _t.zeros(H, n_c, dtype=_t.float32, device=dev)

        def attn_call():
            kvz.kvz_score_chunk_attn(data["q"][0][k0], data["kc"][0], data["kin"][0][k0],
                                     data["vc"][0], v_in, S_attn, wl.n_prompt, O=o_buf,
                                     scale=scale, ws=ws_attn, stream=stream)

        attn_call()
        _t.cuda.synchronize()
        reps = 5
        kvz.kvz_prof_enable(True, 16 * reps)
        for _ in range(reps):
            attn_call()
        _t.cuda.synchronize()
        at = {}
        for nm in ("score_pass1", "score_combine", "score_pass2", "attn_pass3", "attn_reduce"):
            n_, ms_ = kvz.kvz_prof_read(nm)
            if n_:
                at[nm] = round(ms_ / n_ * 1e3, 2)
        kvz.kvz_prof_enable(False)
        # the output pass forms q.k once more and p.v once per visible (row, key) pair
        vis = H * G * (n_in0 * n_c + n_in0 * (n_in0 + 1) // 2)
        o_flops = 2 * d * vis * 2
        if "attn_pass3" in at:
            ach = o_flops / (at["attn_pass3"] * 1e-6) / 1e12
            out["attn_output"] = {
                "per_call_us": at, "call_us": round(sum(at.values()), 2),
                "pass3_flops": o_flops, "pass3_TFLOPs": round(ach, 2),
                "pass3_frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                "what": "kvz_score_chunk_attn on one 16+2048-row chunk of one layer "
                        "(all KV heads): scores plus O = P[V_c; V_in]"}
    if args.copy_calibration:
        nbytes = 2 << 30
        src_t = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst_t = torch.empty_like(src_t)
        for _ in range(3):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = nbytes
        del src_t, dst_t
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
