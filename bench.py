#!/usr/bin/env python3
"""Throughput of the DSA lightning-indexer hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input already resident in HBM:
preprocess + quantise (when the workload has it), KPool compression (when it has it),
scoring and top-k selection (with pool expansion). The metric is indexer query-key pairs
scored and top-k'd per second: pairs = sum over queries of their causal candidates (keys,
or pools for KPool). The default workload is 2 x 4096 tokens, 64 heads, head dim 128,
key LayerNorm + RoPE (64 dims) in fp32, FP8 E4M3 with per-vector UE8M0 scales, topk 512.

Prints ONE JSON line. The timed steps replay one step captured as a HIP graph. Per-kernel
times come from HIP events recorded on the stream the kernels run on, around each library
call, over the same number of eager steps queued behind a spin kernel, averaged. The
roofline entry is for the scoring kernel (MFMA-bound): algorithmic flops 2*H*D per pair.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..5]

Traffic counters (HBM bytes of the scoring kernel): run the bench twice under
`rocprofv3 --pmc FETCH_SIZE` and `rocprofv3 --pmc WRITE_SIZE` with `--copy-mb N`, which adds
one plain device-to-device copy of N MiB after the timed steps as the calibration kernel,
then `python bench.py --ingest-pmc FETCH_DB WRITE_DB --copy-mb N [--workload W]` scales the
scoring kernel's counters by the copy kernel's and records them in profiles/traffic.json
(keyed by workload, tied to the scoring kernel's source hash).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

PEAK_FLOPS = {"bf16": 2.5e15, "fp8": 5.0e15, "mxfp8": 5.0e15}    # MI355X dense MFMA
PEAK_HBM = 8.0e12                                                  # MI355X HBM3E bytes/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("score.hip", "device_common.h"):
        with open(os.path.join(ROOT, "sparse_attention_indexer_dsa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measure_peaks(prec, reps=5):
    """Rates this device sustains, to set the kernels against beside the published peaks:
    the scoring kernel's MFMA instruction with its operands in registers (dsa_bench_mfma,
    1024 workgroups x 4 waves, four accumulator chains each), and HBM read-only and copy
    sweeps over 1 GiB (dsa_bench_stream). Best of `reps` calls after a warm-up, each timed
    with events on the stream the library launches on."""
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    dev = torch.device("cuda")

    def best_rate(fn):
        fn()
        best = 0.0
        for _ in range(reps):
            st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            st.record()
            work = fn()
            en.record()
            en.synchronize()
            best = max(best, work / (st.elapsed_time(en) * 1e-3))
        return best

    blocks = 1024
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    iters = 8000 if prec == "bf16" else 4000
    mfma = best_rate(lambda: dsa.bench_mfma(prec, blocks, iters, out))
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    read = best_rate(lambda: dsa.bench_stream(src, dst, copy=False))
    copy = best_rate(lambda: dsa.bench_stream(src, dst, copy=True))

    def torch_copy():
        dst.copy_(src)
        return 2 * src.numel()
    tcopy = best_rate(torch_copy)
    del src, dst
    return {"mfma_tflops": round(mfma / 1e12, 1), "mfma_dtype": prec, "hbm_read_gbps": round(read / 1e9, 1),
            "hbm_copy_gbps": round(copy / 1e9, 1), "hbm_torch_copy_gbps": round(tcopy / 1e9, 1),
            "method": "dsa_bench_mfma (the scoring kernel's MFMA instruction, operands in registers), "
                      "dsa_bench_stream (1 GiB read-only and copy sweeps) and torch's device copy of the same "
                      "buffer; best of %d event-timed calls" % reps}


def pair_count(cu, kp):
    L = np.diff(np.asarray(cu, np.int64))
    if kp == 1:
        return int(np.sum(L * (L + 1) // 2))
    tot = 0
    for n in L:
        u = np.arange(n)
        tot += int(np.sum((u + 1) // kp))
    return tot


def device_inputs(inp, dev="cuda"):
    """Device tensors of a generated workload: bf16 inputs (held as uint16 bit patterns) as
    torch.bfloat16, everything else as it is."""
    import torch

    def put(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)
    d = {"q": put(inp["q"]), "k": put(inp["k"]), "w": put(inp["w"]), "cu": put(inp["cu_seqlens"])}
    for name in ("gamma", "beta", "cos", "sin", "bias", "gate"):
        if name in inp:
            d[name] = put(inp[name])
    return d


def run_gpu(inp, steps, warmup, copy_mb=0, fuse=False, softmax=False, attn_heads=0):
    import torch
    import sparse_attention_indexer_dsa_amd as dsa
    dsa.load()
    dev = "cuda"
    T, H, D = inp["q"].shape
    prec, kp, topk, max_seqlen = inp["precision"], inp["kpool"], inp["topk"], inp["max_seqlen"]
    B = len(inp["docs"])
    d = device_inputs(inp, dev)
    esz = 2 if prec == "bf16" else 1
    nsb = {"bf16": 0, "fp8": 1, "mxfp8": D // 32}[prec]
    odt = torch.bfloat16 if prec == "bf16" else torch.uint8
    ops = {}
    fused = inp["preprocess"] and kp == 1 and fuse
    if inp["preprocess"] and not fused:
        ops["q_op"] = torch.empty((T, H, D), dtype=odt, device=dev)
    if inp["preprocess"]:
        ops["k_op"] = torch.empty((T, D), dtype=odt, device=dev)
        if prec != "bf16":
            if not fused:
                ops["q_scale"] = torch.empty((T, H) if prec == "fp8" else (T, H, nsb), dtype=torch.uint8, device=dev)
            ops["k_scale"] = torch.empty((T,) if prec == "fp8" else (T, nsb), dtype=torch.uint8, device=dev)
        q_op, k_src = ops.get("q_op"), ops["k_op"]
    else:
        q_op, k_src = d["q"], d["k"]
    pool = {}
    if kp > 1:
        P = T // kp
        pool["pooled_op"] = torch.empty((P, D), dtype=odt, device=dev)
        pool["cu_pools"] = torch.empty(B + 1, dtype=torch.int32, device=dev)
        if prec != "bf16":
            pool["pooled_scale"] = torch.empty((P,) if prec == "fp8" else (P, nsb), dtype=torch.uint8, device=dev)
    ws = torch.empty(dsa.workspace_size(T, max_seqlen, topk, kp, H, D, B, prec), dtype=torch.uint8, device=dev)
    outs = dsa._alloc_outputs(None, T, topk, kp, dev)
    sm_out = torch.empty((T, topk), dtype=torch.float32, device=dev) if softmax else None
    attn = {}
    if attn_heads:
        # sparse attention over the selection: synthetic bf16 queries [T, heads, 576] and one
        # latent entry [576] per token, drawn on the device
        gen_t = torch.Generator(device=dev).manual_seed(7)
        attn["q"] = torch.randn((T, attn_heads, 576), generator=gen_t, device=dev).to(torch.bfloat16)
        attn["kv"] = torch.randn((T, 576), generator=gen_t, device=dev).to(torch.bfloat16)
        attn["out"] = torch.empty((T, attn_heads, 512), dtype=torch.bfloat16, device=dev)
        attn["lse"] = torch.empty((T, attn_heads), dtype=torch.float32, device=dev)
    k_op = pool["pooled_op"] if kp > 1 else (ops["k_op"] if inp["preprocess"] else d["k"])
    k_scale = pool.get("pooled_scale") if kp > 1 else ops.get("k_scale")

    def step(ev=None):
        i = 0
        if ev is not None:
            ev[i].record(); i += 1
        if inp["preprocess"]:
            # fused: only the keys here; the scoring kernel preprocesses the queries itself
            dsa.preprocess(None if fused else d["q"], d["k"], d["cu"],
                           ln_gamma=d.get("gamma") if inp["layernorm"] else None,
                           ln_beta=d.get("beta") if inp["layernorm"] else None, ln_eps=1e-6,
                           rope_cos=d.get("cos"), rope_sin=d.get("sin"), rope_dim=inp["rope_dim"],
                           rope_fp32=inp["rope_fp32"], precision=prec, out=ops)
        if ev is not None:
            ev[i].record(); i += 1
        if kp > 1:
            dsa.kpool(k_src, d["cu"], d["gate"], d["bias"], kp, precision=prec, out=pool)
        if ev is not None:
            ev[i].record(); i += 1
        if fused:
            dsa.score_fused(d["q"], k_op, d["w"], d["cu"], max_seqlen, ws, k_scale=k_scale, rope_cos=d.get("cos"),
                            rope_sin=d.get("sin"), rope_dim=inp["rope_dim"], rope_fp32=inp["rope_fp32"],
                            precision=prec)
        else:
            dsa.score(q_op, k_op, d["w"], d["cu"], max_seqlen, ws, q_scale=ops.get("q_scale"), k_scale=k_scale,
                      precision=prec, kpool=kp, cu_pools=pool.get("cu_pools"))
        if ev is not None:
            ev[i].record(); i += 1
        dsa.topk(ws, T, d["cu"], max_seqlen, topk, kpool=kp, cu_pools=pool.get("cu_pools"), kpool_tail=True,
                 out=outs)
        if ev is not None:
            ev[i].record(); i += 1
        if softmax:
            dsa.selection_softmax(outs["scores"], out=sm_out)
        if ev is not None:
            ev[i].record(); i += 1
        if attn_heads:
            dsa.sparse_attention(attn["q"], attn["kv"], outs["indices"], sm_scale=576 ** -0.5,
                                 lengths=outs["lengths"], out=attn["out"], lse=attn["lse"])
        if ev is not None:
            ev[i].record(); i += 1

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # One step captured as a HIP graph (the library allocates and synchronises nothing, so a
    # step captures as is): the timed steps replay it, without host gaps between kernels.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # Per-kernel durations: the same steps run eagerly with HIP events around every library
    # call on the stream the kernels run on, queued behind a spin kernel so that the stream
    # never waits for the host between a kernel and its events.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    torch.cuda._sleep(20_000_000)
    for s in range(steps):
        step(events[s])
    torch.cuda.synchronize()
    if copy_mb > 0:     # calibration kernel for the traffic counters (outside the timed steps)
        n = copy_mb << 20
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    names = ["preprocess", "kpool", "score", "topk", "softmax", "attention"]
    per = {n: float(np.mean([events[s][i].elapsed_time(events[s][i + 1]) for s in range(steps)])) / 1e3
           for i, n in enumerate(names)}
    # slots the attention reads per step (the selection's token lengths)
    per["attention_slots"] = int(outs["lengths"].sum().item()) if attn_heads else 0
    return (t1 - t0), per, fused


def algorithmic(inp, pairs, fused):
    """Algorithmic flops/bytes per launch of each kernel. Fused: the preprocessing kernel
    handles the keys only and the scoring kernel reads the raw (bf16) queries."""
    T, H, D = inp["q"].shape
    prec, kp, topk = inp["precision"], inp["kpool"], inp["topk"]
    esz = 2 if prec == "bf16" else 1
    nsb = {"bf16": 0, "fp8": 1, "mxfp8": D // 32}[prec]
    out = {"score_flops": 2.0 * H * D * pairs}
    if inp["preprocess"]:
        out["preprocess_bytes"] = float(T * D * 2 + T * D * esz + T * nsb)
        if not fused:
            out["preprocess_bytes"] += float(T * H * D * 2 + T * H * D * esz + T * H * nsb)
    if kp > 1:
        P = T // kp
        out["kpool_bytes"] = float(T * D * 2 + T * 2 + P * D * esz)
    width = topk if kp == 1 else topk * kp + kp - 1
    out["topk_bytes"] = float(pairs * 4 + T * topk * 4 + T * width * 4 + T * 4 + (T * topk * 4 if kp > 1 else 0))
    out["softmax_bytes"] = float(2 * T * topk * 4)     # the selected scores in, the weights out
    q_bytes = T * H * D * 2 if fused else T * H * D * esz + T * H * nsb
    out["score_bytes"] = float(q_bytes + T * H * 4 + (T // kp) * D * esz + pairs * 4)
    return out


def cpu_baseline(inp, budget_s):
    """The oracle on a bounded sample of the same workload: key side in full, then query rows in
    batches until the time budget is used; throughput extrapolated to the whole workload."""
    from threadpoolctl import threadpool_info
    from oracle import oracle as orc
    import gen
    import parity
    cfg = parity.config_of(inp)
    T = inp["q"].shape[0]
    kp, topk = inp["kpool"], inp["topk"]
    rng = np.random.default_rng(0)
    order = rng.permutation(T)
    t0 = time.perf_counter()
    o = parity.oracle_operands_rows(inp, cfg, order[:1])     # key side (LayerNorm/RoPE/quantise or KPool)
    t_keys = time.perf_counter() - t0
    cu = inp["cu_seqlens"]
    _, pos = orc.geometry(cu, T)
    done, pairs, t_rows = 0, 0, 0.0
    batch = 16
    while done < T and (t_rows < budget_s or done == 0):
        rows = np.sort(order[done:done + batch])
        t1 = time.perf_counter()
        qo = parity.oracle_operands_rows(inp, cfg, rows, keys=False) if cfg["preprocess"] else None
        if qo is not None:
            q_deq = qo["q_deq"]
        else:
            q_deq = {int(t): orc.dequantize(inp["q"][t], None, "bf16") for t in rows}
        orc.index_topk(q_deq, o["k_deq"], inp["w"].astype(np.float64), cu, topk, 1.0, kp, o.get("cu_pools"),
                       True, rows=rows)
        t_rows += time.perf_counter() - t1
        pairs += int(np.sum((pos[rows] + 1) // kp))
        done += rows.size
    total_pairs = pair_count(cu, kp)
    est = t_keys + t_rows * (total_pairs / max(pairs, 1))
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = int(blas[0]["num_threads"]) if blas else 1
    return {"value": total_pairs / est, "unit": "pairs/s", "cores": cores, "kind": "oracle",
            "blas_threads": cores, "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": (f"numpy fp64 oracle: full key side ({t_keys:.2f} s) + {done} random query rows "
                       f"({pairs} pairs, {t_rows:.2f} s), extrapolated to all {total_pairs} pairs"),
            "seconds": round(t_keys + t_rows, 2)}


def ingest_pmc(fetch_db, write_db, copy_mb, workload):
    """Scoring-kernel HBM bytes per launch from two rocprofv3 --pmc databases (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for the copy
    kernel of copy_mb MiB; recorded in profiles/traffic.json for the workload."""
    import sqlite3
    import gen

    def per_kernel(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, counter_name, value from counters_collection").fetchall()
        out = {}
        for name, cname, val in rows:
            if cname == counter:
                out.setdefault(name, []).append(float(val))
        return out

    res = {}
    for db, counter in ((fetch_db, "FETCH_SIZE"), (write_db, "WRITE_SIZE")):
        k = per_kernel(db, counter)
        score = [v for n, vs in k.items() if "score_kernel" in n for v in vs]
        copy = [v for n, vs in k.items() if "copybuffer" in n.lower() for v in vs]
        if not score or not copy:
            raise SystemExit(f"{db}: no {counter} records for the scoring or the copy kernel")
        copy_kib = max(copy)                       # the calibration copy is the largest copy
        if any(1024.0 < v < 0.99 * copy_kib for v in copy):
            raise SystemExit(f"{db}: copies of different sizes; record the counters with --no-peaks so the "
                             "calibration copy is the only large one")
        factor = copy_mb * 1024.0 / copy_kib
        res[counter] = {"kib_per_launch": float(np.mean(score)), "copy_kib": copy_kib, "factor": factor,
                        "bytes_per_launch": float(np.mean(score)) * 1024.0 * factor}
    name = gen.WORKLOADS[workload]["name"]
    rec = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    rec[name] = {"bytes_per_launch": res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"],
                 "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"], "copy_mb": copy_mb,
                 "source_hash": kernel_source_hash()}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    print(json.dumps({name: rec[name]}, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the on-device peak measurements")
    ap.add_argument("--copy-mb", type=int, default=0, help="calibration copy of this many MiB after timing")
    ap.add_argument("--fuse", action="store_true",
                    help="preprocess the queries inside the scoring kernel (dsa_index_score_fused) instead of in "
                         "the preprocessing kernel")
    ap.add_argument("--softmax", action="store_true",
                    help="also compute the softmax over each row's selection (dsa_index_selection_softmax) in "
                         "every step")
    ap.add_argument("--attention", type=int, default=0, metavar="HEADS",
                    help="also run the sparse MLA attention over each row's selection "
                         "(dsa_index_sparse_attention) with this many query heads in every step")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="record scoring-kernel traffic from two rocprofv3 --pmc databases and exit")
    args = ap.parse_args()
    if args.ingest_pmc:
        if args.copy_mb <= 0:
            raise SystemExit("--ingest-pmc needs the --copy-mb size of the calibration copy")
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.copy_mb, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the hot path runs on a "
              "single MI355X; sharding across GPUs is a design note, not a measured path)", file=sys.stderr)
        sys.exit(2)
    import gen
    inp = gen.workload(args.workload)
    T, H, D = inp["q"].shape
    kp = inp["kpool"]
    pairs = pair_count(inp["cu_seqlens"], kp)
    print(f"[bench] workload {args.workload}: {inp['name']} T={T} pairs={pairs}", file=sys.stderr, flush=True)
    elapsed, per, fused = run_gpu(inp, args.steps, args.warmup, args.copy_mb, args.fuse, args.softmax,
                                  args.attention)
    alg = algorithmic(inp, pairs, fused)
    prec = inp["precision"]
    kernels = {}
    for n in ("preprocess", "kpool", "score", "topk", "softmax"):
        if per[n] <= 0 or (n == "preprocess" and not inp["preprocess"]) or (n == "kpool" and kp == 1) or \
                (n == "softmax" and not args.softmax):
            continue
        k = {"ms": round(per[n] * 1e3, 4)}
        if n == "score":
            k["tflops"] = round(alg["score_flops"] / per[n] / 1e12, 1)
            k["frac_mfma"] = round(alg["score_flops"] / per[n] / PEAK_FLOPS[prec], 4)
        else:
            b = alg[f"{n}_bytes"]
            k["gbps"] = round(b / per[n] / 1e9, 1)
            k["frac_hbm"] = round(b / per[n] / PEAK_HBM, 4)
        kernels[n] = k
    if args.attention and per["attention"] > 0:
        # score and value products over every selected slot: 2 * heads * (576 + 512) flops each
        fl = 2.0 * per["attention_slots"] * args.attention * (576 + 512)
        kernels["attention"] = {"ms": round(per["attention"] * 1e3, 4), "tflops": round(fl / per["attention"] / 1e12, 1),
                                "frac_mfma": round(fl / per["attention"] / PEAK_FLOPS["bf16"], 4),
                                "heads": args.attention, "slots": per["attention_slots"]}
    achieved = alg["score_flops"] / per["score"] / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE)).get(inp["name"])
        if rec and rec.get("source_hash") == kernel_source_hash():
            traffic = rec.get("bytes_per_launch")
    line = {
        "metric": "indexer query-key pairs scored+top-k'd/sec",
        "value": pairs * args.steps / elapsed,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3", "mxfp8": "mxfp8-e4m3"}[prec],
        "data": "synthetic (seeded numpy draws with the workload's shapes and distributions)",
        "config": {"workload": inp["name"], "T": T, "H": H, "D": D, "docs": inp["docs"] if len(inp["docs"]) <= 16
                   else f"{len(inp['docs'])} docs", "topk": inp["topk"], "kpool": kp, "precision": prec,
                   "preprocess": bool(inp["preprocess"]), "query_preprocessing": "in the scoring kernel" if fused
                   else ("own kernel" if inp["preprocess"] else "none"), "pairs_per_step": pairs,
                   "selection_softmax": bool(args.softmax), "sparse_attention_heads": args.attention,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "score", "achieved": round(achieved, 2),
                     "peak": PEAK_FLOPS[prec] / 1e12, "unit": "TFLOP/s",
                     "frac": round(achieved * 1e12 / PEAK_FLOPS[prec], 4), "traffic": traffic},
        "kernels": kernels,
    }
    if not args.no_peaks:
        pk = measure_peaks(prec)
        line["peaks_measured"] = pk
        line["roofline"]["measured_peak"] = pk["mfma_tflops"]
        line["roofline"]["frac_of_measured"] = round(achieved / pk["mfma_tflops"], 4)
        hbm = max(pk["hbm_read_gbps"], pk["hbm_copy_gbps"], pk["hbm_torch_copy_gbps"])
        for k in kernels.values():
            if "gbps" in k:
                k["frac_hbm_measured"] = round(k["gbps"] / hbm, 4)
            if "tflops" in k and "heads" not in k:
                k["frac_mfma_measured"] = round(k["tflops"] / pk["mfma_tflops"], 4)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
