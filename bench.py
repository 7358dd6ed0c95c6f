"""Benchmark: fused compressed-BF16 GEMV over the Qwen3-4B layer set on one MI355X.

One step = one sweep of the whole hot path over one batch of synthetic input:
all 36 layers x 7 projections (q, k, v, o, gate, up, down) of a Qwen3-4B-shaped
decoder, each a batch-1 nwc_matvec over its own compressed matrix, back to
back on one stream.  The sweep reads ~4.9 GB of compressed weights, far more
than the 256 MB last-level cache, so every matrix is read cold from HBM.

Printed: one JSON line (the contract's fields plus roofline, cpu_baseline and
per-shape figures).  Inputs are generated and encoded before the timed region;
the timed region holds only kernel launches on resident data.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
CLOCK_HZ = 2.4e9  # MI355X peak engine clock, published
N_CU = 256
METRIC = "fused compressed GEMV µs & compressed GB/s (% of HBM peak), Qwen3-4B layer set"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("kernels.hip", "nwc_format.h"):
        h.update(open(os.path.join(ROOT, "decode_matvec_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(algo_bytes_per_launch: float):
    """HBM bytes per launch measured by rocprofv3 PMC (committed), if they are of this kernel source."""
    p = os.path.join(ROOT, "profiles", "matvec_qwen3_4b_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


FUSED_QWEN3 = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",)))


def build_layer_set(torch, nwc, S, C, dev, layers, with_bf16, fused=False, cols=0, rows=0):
    """The Qwen3-4B layer set, one compressed matrix per projection; with `fused`,
    also the projections that share an input in a decoder layer encoded as one
    matrix each (q||k||v and gate||up rows concatenated, one rank table), whose
    activation is the first member's."""
    mats, fmats = [], []
    t0 = time.time()
    for layer in range(layers):
        dense = {}
        for idx, (name, n, k) in enumerate(C.QWEN3_4B):
            ws, xs = C.qwen3_seed(layer, idx)
            w = S.blocked_normal_bf16(ws, (n, k), np.float32(C.sigma_for(k)))
            wt = torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16) if with_bf16 else None
            blob = nwc.encode(w, cols_per_lane=cols, rows_per_wave=rows)
            dm = nwc.DeviceMatrix(blob, dev)
            x = S.activation_bf16(xs, k)
            xd = torch.from_numpy(x.view(np.int16)).to(dev)
            y = torch.empty(n, dtype=torch.float32, device=dev)
            info = dm.info
            mats.append(dict(name=name, n=n, k=k, dm=dm, x=xd, y=y, info=info,
                             algo_bytes=info["coded_bits"] / 8.0 + 2 * k + 4 * n,
                             blob_bytes=info["total_bytes"],
                             w_bf16=wt if with_bf16 else None,
                             x_bf16=xd.view(torch.bfloat16).view(1, k) if with_bf16 else None))
            if fused:
                dense[name] = (w, xd)
            del w
        for fname, parts in FUSED_QWEN3 if fused else ():
            w = np.concatenate([dense[p][0] for p in parts]) if len(parts) > 1 else dense[parts[0]][0]
            n, k = w.shape
            dm = nwc.DeviceMatrix(nwc.encode(w), dev)
            fmats.append(dict(name=fname, n=n, k=k, dm=dm, x=dense[parts[0]][1],
                              y=torch.empty(n, dtype=torch.float32, device=dev), info=dm.info,
                              algo_bytes=dm.info["coded_bits"] / 8.0 + 2 * k + 4 * n,
                              blob_bytes=dm.info["total_bytes"]))
        if layer % 6 == 5 or layer == layers - 1:
            log(f"[bench] encoded {layer + 1}/{layers} layers ({time.time() - t0:.1f}s)")
    return mats, fmats


def time_region(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per call of fn


def cpu_baseline(S, C):
    """The oracle on host cores, on a bounded sample of the layer set: the plain C
    oracle (oracle/nwc_oracle.c) decodes each of layer 0's seven matrices from its
    row streams and computes the float64 matvec from the decoded weights, in row
    blocks on as many threads as the host gives this process (at most 16)."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import fast as OF
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    work, gbytes, weights = [], 0.0, 0
    for idx, (name, n, k) in enumerate(C.QWEN3_4B):
        ws, xs = C.qwen3_seed(0, idx)
        w = S.blocked_normal_bf16(ws, (n, k), np.float32(C.sigma_for(k)))  # the benchmarked weights
        r2s, s2r = OF.rank_table(OF.bf16_histogram(w, threads))
        blocks, bits = [], 0
        for r0, r1 in OF._blocks(n, k):
            stream, start, b = OF.encode_rows_bf16(w[r0:r1], s2r)
            blocks.append((r0, r1, stream, start, (w[r0:r1] & 0xFF).astype(np.uint8)))
            bits += b
        del w
        work.append((n, k, r2s, blocks, S.activation_bf16(xs, k)))
        gbytes += ((bits + 8 * n * k) / 8.0 + 2 * k + 4 * n) / 1e9
        weights += n * k

    def one(job):
        k, r2s, (r0, r1, stream, start, mant), x = job
        return OF.matvec_bf16(OF.decode_rows_bf16(stream, start, r1 - r0, k, r2s, mant), x, threads=1)

    jobs = [(k, r2s, b, x) for n, k, r2s, blocks, x in work for b in blocks]
    # The sample is decoded and multiplied repeatedly until about 10 s have passed.
    passes = 0
    with ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        while passes == 0 or time.perf_counter() - t0 < 10.0:
            list(ex.map(one, jobs))
            passes += 1
        dt = time.perf_counter() - t0
    return {"value": round(gbytes * passes / dt, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(), "host_cpus_usable": len(os.sched_getaffinity(0)),
            "sample": f"C oracle decode + float64 matvec of layer 0's 7 matrices ({weights / 1e6:.1f} M weights, "
                      f"the benchmarked weights), {len(jobs)} row blocks on {threads} threads, {passes} passes, "
                      f"{dt:.1f} s"}

def build_qwen25_step(torch, nwc, S, C, dev, layers, with_bf16, with_fused=False):
    """Qwen2.5-7B-shaped decode step: `layers` layers of 7 projections plus the
    152064 x 3584 lm_head, all N(0, 1/sqrt(K)), encoded and resident; with
    `with_fused`, also q||k||v and gate||up encoded as one matrix each."""
    t0 = time.time()

    def one(seed, n, k):
        w = S.blocked_normal_bf16(seed, (n, k), np.float32(C.sigma_for(k)))
        wt = torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16) if with_bf16 else None
        dm = nwc.DeviceMatrix(nwc.encode(w), dev)
        return dict(dm=dm, n=n, k=k, y=torch.empty(n, dtype=torch.float32, device=dev),
                    w_bf16=wt if with_bf16 else None, w_host=w if with_fused else None,
                    algo_bytes=dm.info["coded_bits"] / 8.0 + 2 * k + 4 * n, blob_bytes=dm.info["total_bytes"])

    def fused(L, name, parts):
        w = np.concatenate([L[p]["w_host"] for p in parts])
        dm = nwc.DeviceMatrix(nwc.encode(w), dev)
        n, k = w.shape
        return dict(dm=dm, n=n, k=k, y=torch.empty(n, dtype=torch.float32, device=dev),
                    algo_bytes=dm.info["coded_bits"] / 8.0 + 2 * k + 4 * n, blob_bytes=dm.info["total_bytes"])

    stack = []
    for layer in range(layers):
        L = {name: one(C.qwen25_seed(layer, idx), n, k) for idx, (name, n, k) in enumerate(C.QWEN25_7B)}
        if with_fused:
            L["qkv"] = fused(L, "qkv", ("q", "k", "v"))
            L["gate_up"] = fused(L, "gate_up", ("gate", "up"))
        for m in L.values():
            m.pop("w_host", None)
        stack.append(L)
        if layer % 7 == 6 or layer == layers - 1:
            log(f"[bench] encoded {layer + 1}/{layers} layers ({time.time() - t0:.1f}s)")
    head = one(C.QWEN25_LM_HEAD_SEED, C.QWEN25_7B_VOCAB, C.QWEN25_7B_HIDDEN)
    head.pop("w_host", None)
    h0 = torch.from_numpy(S.activation_bf16(C.QWEN25_X_SEED, C.QWEN25_7B_HIDDEN).view(np.int16)).to(dev)
    return stack, head, h0.view(torch.bfloat16)


def qwen25_step(torch, stack, head, h0, linear, fused=False, group=None):
    """One batch-1 decode step.  linear(m, x_bf16) -> fp32 output of matrix m;
    group(ms, x_bf16) -> fp32 outputs of the matrices ms, which read the same
    input (q, k, v; gate, up), in one launch.
    As in the Qwen2 architecture, RMS norms (unit weight) precede attention,
    the MLP and the lm_head; the residual stream stays fp32.  Attention at
    context length 1 returns v for every query head (softmax over one
    position), so each of the 4 KV heads feeds its 7 query heads."""
    F = torch.nn.functional

    def norm(h):
        return (h * torch.rsqrt(h.square().mean() + 1e-6)).to(torch.bfloat16)

    h = h0.float()
    for L in stack:
        hb = norm(h)
        if fused:  # q||k||v and gate||up as one matvec each (outputs split by rows)
            v = linear(L["qkv"], hb)[L["q"]["n"] + L["k"]["n"]:]
        elif group is not None:
            v = group([L["q"], L["k"], L["v"]], hb)[2]
        else:
            linear(L["q"], hb)
            linear(L["k"], hb)
            v = linear(L["v"], hb)
        attn = v.to(torch.bfloat16).view(4, 1, 128).expand(4, 7, 128).reshape(-1).contiguous()
        h = h + linear(L["o"], attn)
        hb = norm(h)
        if fused:
            gu = linear(L["gate_up"], hb)
            gate, up = gu[:L["gate"]["n"]], gu[L["gate"]["n"]:]
        elif group is not None:
            gate, up = group([L["gate"], L["up"]], hb)
        else:
            gate, up = linear(L["gate"], hb), linear(L["up"], hb)
        act = (F.silu(gate) * up).to(torch.bfloat16)
        h = h + linear(L["down"], act)
    return linear(head, norm(h))


def bench_qwen25_step(args, torch, nwc, S, C, dev):
    stack, head, h0 = build_qwen25_step(torch, nwc, S, C, dev, args.layers or C.QWEN25_7B_LAYERS,
                                        not args.no_bf16_baseline, with_fused=True)
    mats = [m for L in stack for name, m in L.items() if name not in ("qkv", "gate_up")] + [head]
    F = torch.nn.functional

    def nwc_linear(m, x):
        m["dm"].matvec(x, m["y"])
        return m["y"]

    def bf16_linear(m, x):
        return F.linear(x.view(1, -1), m["w_bf16"]).view(-1).float()

    def graph_of(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def nwc_group(ms_, x):
        nwc.matvec_group([m["dm"] for m in ms_], [x] * len(ms_), [m["y"] for m in ms_])
        return [m["y"] for m in ms_]

    # The step as the headline of this workload: q,k,v and gate,up each one
    # grouped launch (separately encoded matrices), 4 launches per layer.
    g_step = graph_of(lambda: qwen25_step(torch, stack, head, h0, nwc_linear, group=nwc_group))
    ms = time_region(torch, g_step.replay, args.steps, args.warmup)
    g_7 = graph_of(lambda: qwen25_step(torch, stack, head, h0, nwc_linear))
    ms_7 = time_region(torch, g_7.replay, args.steps, args.warmup)
    xs = {id(m): torch.zeros(m["k"], dtype=torch.bfloat16, device=dev) for m in mats}
    g_mv = graph_of(lambda: [m["dm"].matvec(xs[id(m)], m["y"]) for m in mats])
    ms_mv = time_region(torch, g_mv.replay, args.steps, args.warmup)
    g_fused = graph_of(lambda: qwen25_step(torch, stack, head, h0, nwc_linear, fused=True))
    ms_fused = time_region(torch, g_fused.replay, args.steps, args.warmup)
    algo = sum(m["algo_bytes"] for m in mats)
    out = {"metric": "Qwen2.5-7B-shaped batch-1 decode step, every linear through nwc_matvec",
           "value": round(1e3 / ms, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1/sqrt(K)) BF16 weights)",
           "config": {"workload": "qwen25_7b_decode_step", "layers": len(stack), "matrices": len(mats),
                      "batch": 1, "attention": "context length 1 stand-in (v repeated over the GQA heads)",
                      "glue": "RMS norms (unit weight), fp32 residual, silu(gate)*up, in torch"},
           "ms_matvecs_only": round(ms_mv, 4), "ms_glue": round(ms - ms_mv, 4),
           "compressed_GBps_matvecs": round(algo / (ms_mv * 1e-3) / 1e9, 1),
           "compressed_GB": round(algo / 1e9, 4), "blob_GB": round(sum(m["blob_bytes"] for m in mats) / 1e9, 4),
           "launches": "q,k,v one nwc_matvec_group launch, o, gate,up one launch, down; lm_head",
           "one_launch_per_matrix": {"ms_per_step": round(ms_7, 4), "tokens_per_s": round(1e3 / ms_7, 2)},
           "fused_projections": {"ms_per_step": round(ms_fused, 4), "tokens_per_s": round(1e3 / ms_fused, 2),
                                 "note": "q||k||v and gate||up each encoded as one matrix (one launch), "
                                         "4 launches per layer"},
           "timing": "HIP graph replay of the whole step (glue in torch); matvecs alone in a second graph",
           "kernel_source_hash": kernel_source_hash()}
    if not args.no_bf16_baseline:
        g_bf = graph_of(lambda: qwen25_step(torch, stack, head, h0, bf16_linear))
        ms_bf = time_region(torch, g_bf.replay, args.steps, args.warmup)
        y_nwc = qwen25_step(torch, stack, head, h0, nwc_linear)
        y_bf = qwen25_step(torch, stack, head, h0, bf16_linear)
        torch.cuda.synchronize()
        rel = float((y_nwc - y_bf).norm() / y_bf.norm())
        out["bf16_baseline"] = {"ms_per_step": round(ms_bf, 4), "tokens_per_s": round(1e3 / ms_bf, 2),
                                "speedup_compressed_vs_bf16": round(ms_bf / ms, 4),
                                "logits_rel_l2_vs_bf16_stack": rel,
                                "kernel": "torch.nn.functional.linear (hipBLASLt/rocBLAS), same glue"}
        # The library's plain BF16 GEMV with the same launch structure (grouped q,k,v and gate,up).
        for m in mats:
            m["y_plain"] = torch.empty(m["n"], dtype=torch.float32, device=dev)

        def plain_linear(m, x):
            nwc.bf16_gemv(m["w_bf16"], x, m["y_plain"])
            return m["y_plain"]

        def plain_group(ms_, x):
            nwc.bf16_gemv_group([m["w_bf16"] for m in ms_], [x] * len(ms_), [m["y_plain"] for m in ms_])
            return [m["y_plain"] for m in ms_]

        g_pl = graph_of(lambda: qwen25_step(torch, stack, head, h0, plain_linear, group=plain_group))
        ms_pl = time_region(torch, g_pl.replay, args.steps, args.warmup)
        out["bf16_plain_gemv_grouped"] = {"ms_per_step": round(ms_pl, 4), "tokens_per_s": round(1e3 / ms_pl, 2),
                                          "speedup_compressed_vs_plain": round(ms_pl / ms, 4),
                                          "kernel": "nwc_bf16_gemv_group / nwc_bf16_gemv, same launch structure"}
    print(json.dumps(out), flush=True)


def bench_prefill(args, torch, nwc, S, C, dev):
    """Prefill (several tokens at once) on the Qwen3-4B layer matrices: each
    matrix dequantized by nwc_dequant into one reused BF16 buffer, then
    torch.nn.functional.linear (hipBLASLt), against F.linear on the BF16
    weights; T = 16, 128, 512 tokens, over a rotation of 4 layers (0.8 GB of
    BF16 weights, so every call reads its weights from HBM)."""
    from decode_matvec_amd import prefill as P
    F = torch.nn.functional
    layers = args.layers or 4
    mats, _ = build_layer_set(torch, nwc, S, C, dev, layers, True)
    scratch = torch.empty(max(m["n"] * m["k"] for m in mats), dtype=torch.int16, device=dev)
    rows = {}
    for T in (16, 128, 512):
        xs = {k: torch.from_numpy(np.stack([S.activation_bf16(7000 + t, k) for t in range(T)]).view(np.int16))
              .to(dev).view(torch.bfloat16) for k in {m["k"] for m in mats}}

        def nwc_pass():
            for m in mats:
                P.prefill(m["dm"], xs[m["k"]], scratch=scratch)

        def bf16_pass():
            for m in mats:
                F.linear(xs[m["k"]], m["w_bf16"])

        def dequant_pass():
            for m in mats:
                m["dm"].dequant(scratch[: m["n"] * m["k"]].view(m["n"], m["k"]))

        res = {}
        for tag, fn in (("nwc", nwc_pass), ("bf16", bf16_pass), ("dequant_only", dequant_pass)):
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            res[tag] = time_region(torch, g.replay, args.steps, args.warmup) * 1e3 / layers  # us per layer
        rows[str(T)] = {"us_per_layer_nwc": round(res["nwc"], 2), "us_per_layer_bf16": round(res["bf16"], 2),
                        "us_per_layer_dequant": round(res["dequant_only"], 2),
                        "nwc_over_bf16": round(res["nwc"] / res["bf16"], 3)}
        log(f"[bench] prefill T={T}: {rows[str(T)]}")
    out = {"metric": "prefill: nwc_dequant + hipBLASLt GEMM vs BF16 GEMM, Qwen3-4B layer matrices",
           "value": rows["128"]["us_per_layer_nwc"], "unit": "us per layer (T=128)", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(rows["128"]["us_per_layer_nwc"] * layers / 1e3, 4),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1/sqrt(K)) BF16 weights)",
           "config": {"workload": "prefill", "layers": layers, "tokens": [16, 128, 512]},
           "per_tokens": rows, "kernel_source_hash": kernel_source_hash()}
    print(json.dumps(out), flush=True)


def bench_small_batch(args, torch, nwc, S, C, dev):
    """A few tokens at once on the Qwen3-4B layer matrices (12 layers in rotation: 1.85 GB of blobs, 2.4 GB
    of BF16, far beyond the last-level cache): nwc_matvec (B = 1) and the VALU batch path (B = 4) on the
    default encodings; the matrix-core path (B = 8, 16, 32) on encodings of 16 rows per wave; against
    torch.nn.functional.linear (hipBLASLt) on the BF16 weights with the same B."""
    F = torch.nn.functional
    layers = args.layers or 12
    mats, _ = build_layer_set(torch, nwc, S, C, dev, layers, True)
    mats16, _ = build_layer_set(torch, nwc, S, C, dev, layers, False, cols=16, rows=16)
    algo = sum(m["algo_bytes"] for m in mats)
    rows = {}
    for B in (1, 4, 8, 16, 32):
        ks = {m["k"] for m in mats}
        xs = {k: torch.from_numpy(np.stack([S.activation_bf16(9000 + t, k) for t in range(B)]).view(np.int16))
              .to(dev) for k in ks}
        ys = [torch.empty((B, m["n"]), dtype=torch.float32, device=dev) for m in mats]
        use = mats if B < 5 else mats16

        def nwc_pass():
            for m, y in zip(use, ys):
                if B == 1:
                    m["dm"].matvec(xs[m["k"]][0], y[0])
                else:
                    m["dm"].matvec_batch(xs[m["k"]], y)

        def bf16_pass():
            for m in mats:
                F.linear(xs[m["k"]].view(torch.bfloat16), m["w_bf16"])

        res = {}
        for tag, fn in (("nwc", nwc_pass), ("bf16", bf16_pass)):
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            res[tag] = time_region(torch, g.replay, args.steps, args.warmup) * 1e3 / layers  # us per layer
        path = "nwc_matvec" if B == 1 else "VALU batch (nwc_matvec_batch)" if B < 5 else \
            "matrix cores (nwc_matvec_batch, 16 rows per wave)"
        rows[str(B)] = {"path": path, "us_per_layer_nwc": round(res["nwc"], 2),
                        "us_per_token_layer_nwc": round(res["nwc"] / B, 2),
                        "us_per_layer_bf16_F_linear": round(res["bf16"], 2),
                        "nwc_speedup_vs_bf16": round(res["bf16"] / res["nwc"], 3),
                        "compressed_GBps_nwc": round(algo / layers / (res["nwc"] * 1e-6) / 1e9, 1)}
        log(f"[bench] small batch B={B}: {rows[str(B)]}")
    out = {"metric": "small batches on the Qwen3-4B layer matrices: us per layer, nwc vs BF16 F.linear",
           "value": rows["32"]["us_per_token_layer_nwc"], "unit": "us per token-layer (B=32)", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(rows["32"]["us_per_layer_nwc"] * layers / 1e3, 4), "higher_is_better": False,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1/sqrt(K)) BF16 weights)",
           "config": {"workload": "small_batch", "layers": layers, "batches": [1, 4, 8, 16, 32]},
           "per_batch": rows, "kernel_source_hash": kernel_source_hash()}
    print(json.dumps(out), flush=True)


def bench_tied_embedding(args, torch, nwc, S, C, dev):
    """Tied embedding / lm_head 151936 x 2560 N(0, 0.02): the lm_head GEMV (a
    ~575 MB blob, larger than the 256 MB last-level cache, so each call reads
    it from HBM), the gather of 4096 uniform token ids, a full dequantization;
    and the fp8 e4m3 variant: the 1024 x 1024 matrix and 9728 x 2560 matrices."""
    F = torch.nn.functional
    n, k = C.EMBED_VOCAB, C.EMBED_HIDDEN
    w = S.blocked_normal_bf16(C.EMBED["w_seed"], (n, k), 0.02)
    wt = torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16)
    dm = nwc.DeviceMatrix(nwc.encode(w), dev)
    del w
    x = torch.from_numpy(S.activation_bf16(C.EMBED["x_seed"], k).view(np.int16)).to(dev)
    y = torch.empty(n, dtype=torch.float32, device=dev)
    algo = dm.info["coded_bits"] / 8.0 + 2 * k + 4 * n

    def graph_of(fn, reps=1):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        torch.cuda.synchronize()
        return g

    # Work of a few microseconds is captured `reps` times per graph and the
    # time divided: one short launch per replay would time the host's graph
    # launches instead.
    def per_call_ms(fn, reps, steps=None, warmup=None):
        steps = args.steps if steps is None else steps
        warmup = args.warmup if warmup is None else warmup
        return time_region(torch, graph_of(fn, reps).replay, steps, warmup) / reps

    ms_mv = time_region(torch, graph_of(lambda: dm.matvec(x, y)).replay, args.steps, args.warmup)
    xb = x.view(torch.bfloat16).view(1, k)
    F.linear(xb, wt)
    torch.cuda.synchronize()
    ms_bf = time_region(torch, graph_of(lambda: F.linear(xb, wt)).replay, args.steps, args.warmup)
    ids = torch.from_numpy(S.token_ids(C.EMBED["ids_seed"], n, C.N_IDS)).to(dev)
    out = torch.empty((C.N_IDS, k), dtype=torch.int16, device=dev)
    ms_g = per_call_ms(lambda: dm.gather(ids, out), 8)
    ms_emb = per_call_ms(lambda: torch.index_select(wt, 0, ids), 8)
    full = torch.empty((n, k), dtype=torch.int16, device=dev)
    ms_dq = time_region(torch, graph_of(lambda: dm.dequant(full)).replay, max(2, args.steps // 4), 1)
    del full

    fp8 = {}
    for tag, (fn_, fk, seeds) in {"single_1024": (1024, 1024, [C.SINGLE["w_seed"]]),
                                   "gate_9728x2560": (9728, 2560, list(range(600000, 600012)))}.items():
        qs, ws16 = [], []
        for sd in seeds:
            if fn_ == 1024:
                wf = S.normal_bf16(sd, (fn_, fk), C.SINGLE["sigma"])
            else:
                wf = S.blocked_normal_bf16(sd, (fn_, fk), np.float32(C.sigma_for(fk)))
            qs.append(S.fp8_quantize(wf))
            ws16.append(wf)
        xf = torch.from_numpy(S.activation_bf16(C.SINGLE["x_seed"], fk).view(np.int16)).to(dev)
        yf = torch.empty(fn_, dtype=torch.float32, device=dev)
        fp8[tag] = {}
        # Both coders of the bytes: the unary rank code and the length-limited Huffman variant.
        for cname, coder in (("unary", nwc.NWC_CODER_UNARY), ("huffman", nwc.NWC_CODER_HUFFMAN)):
            dms = [nwc.DeviceMatrix(nwc.encode(q, elem=nwc.NWC_FP8_E4M3, coder=coder), dev) for q, _ in qs]
            scs = [torch.from_numpy(sc).to(dev) for _, sc in qs]
            reps = max(1, 32 // len(dms))
            msf = per_call_ms(lambda: [d.matvec(xf, yf, scale=sc) for d, sc in zip(dms, scs)], reps) / len(dms)
            fa = dms[0].info["coded_bits"] / 8.0 + 2 * fk + 4 * fn_
            fp8[tag][cname] = {"us": round(msf * 1e3, 3), "compressed_GBps": round(fa / (msf * 1e-3) / 1e9, 1),
                               "bits_per_weight_coded": round(dms[0].info["coded_bits"] / (fn_ * fk), 4),
                               "bits_per_weight_blob": round(dms[0].nbytes * 8 / (fn_ * fk), 4),
                               "rotation": len(dms)}
            del dms
        # The compressed BF16 matvec of the same weights, timed the same way: what fp8 is compared with.
        dms = [nwc.DeviceMatrix(nwc.encode(wf), dev) for wf in ws16]
        reps = max(1, 32 // len(dms))
        msb = per_call_ms(lambda: [d.matvec(xf, yf) for d in dms], reps) / len(dms)
        ba = dms[0].info["coded_bits"] / 8.0 + 2 * fk + 4 * fn_
        fp8[tag]["bf16_same_weights"] = {"us": round(msb * 1e3, 3),
                                         "compressed_GBps": round(ba / (msb * 1e-3) / 1e9, 1),
                                         "bits_per_weight_coded": round(dms[0].info["coded_bits"] / (fn_ * fk), 4),
                                         "rotation": len(dms)}
        del dms, ws16
    out_j = {"metric": "tied embedding 151936x2560: lm_head GEMV, 4096-id gather, dequant; fp8 e4m3 variant",
             "value": round(algo / (ms_mv * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
             "warmup": args.warmup, "ms_per_step": round(ms_mv, 4), "higher_is_better": True, "scaling": "weak",
             "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,0.02) BF16 weights)",
             "config": {"workload": "tied_embedding", "vocab": n, "hidden": k, "ids": C.N_IDS},
             "lm_head": {"us": round(ms_mv * 1e3, 2), "compressed_GBps": round(algo / (ms_mv * 1e-3) / 1e9, 1),
                         "hbm_frac_compressed": round(algo / (ms_mv * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "blob_MB": round(dm.info["total_bytes"] / 1e6, 1),
                         "geometry": {f: dm.info[f] for f in ("cols_per_lane", "rows_per_wave", "waves_per_group")},
                         "bf16_F_linear_us": round(ms_bf * 1e3, 2), "speedup_vs_bf16": round(ms_bf / ms_mv, 4)},
             "gather_4096": {"us": round(ms_g * 1e3, 2), "torch_index_select_on_bf16_us": round(ms_emb * 1e3, 2)},
             "dequant_full": {"us": round(ms_dq * 1e3, 1),
                              "GBps_written": round(2.0 * n * k / (ms_dq * 1e-3) / 1e9, 1)},
             "fp8": fp8, "kernel_source_hash": kernel_source_hash()}
    print(json.dumps(out_j), flush=True)


def measure_batch(torch, mats, args, ms_single, batch=4):
    """The layer-set sweep with `batch` activation rows per matrix through
    nwc_matvec_batch (each weight decoded once per row group of up to four
    activation rows), HIP-graph replayed like the batch-1 sweep."""
    for m in mats:
        k, n = m["k"], m["n"]
        ldx = (k + 7) // 8 * 8
        xb = torch.zeros((batch, ldx), dtype=torch.int16, device=m["x"].device)
        for b in range(batch):
            xb[b, :k] = torch.roll(m["x"], shifts=97 * b)
        m["xb"] = xb
        m["yb"] = torch.empty((batch, n), dtype=torch.float32, device=m["x"].device)

    def b_sweep():
        for m in mats:
            m["dm"].matvec_batch(m["xb"], m["yb"])

    b_sweep()
    torch.cuda.synchronize()
    bg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(bg):
        b_sweep()
    bms = time_region(torch, bg.replay, args.steps, args.warmup)
    algo = sum(m["algo_bytes"] for m in mats)
    for m in mats:
        del m["xb"], m["yb"]
    return {"batch": batch, "ms_per_sweep": round(bms, 4), "us_per_layer": round(bms * 1e3 / args.layers, 2),
            "us_per_layer_per_token": round(bms * 1e3 / args.layers / batch, 2),
            "weight_GBps": round(algo / (bms * 1e-3) / 1e9, 1),
            "speedup_vs_batch1_calls": round(batch * ms_single / bms, 3),
            "note": "nwc_matvec_batch, 4 activation rows per matrix; weights read and decoded once per sweep"}


def measure_fused(torch, fmats, args):
    def f_sweep():
        for m in fmats:
            m["dm"].matvec(m["x"], m["y"])

    fg = torch.cuda.CUDAGraph()
    f_sweep()
    torch.cuda.synchronize()
    with torch.cuda.graph(fg):
        f_sweep()
    fms = time_region(torch, fg.replay, args.steps, args.warmup)
    falgo = sum(m["algo_bytes"] for m in fmats)
    f_shape = {}
    for fname, _ in FUSED_QWEN3:
        group = [m for m in fmats if m["name"] == fname]
        gg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gg):
            for m in group:
                m["dm"].matvec(m["x"], m["y"])
        gus = time_region(torch, gg.replay, max(3, args.steps // 2), 1) * 1e3 / len(group)
        f_shape[fname] = {"shape": [group[0]["n"], group[0]["k"]], "us": round(gus, 3),
                          "compressed_GBps": round(group[0]["algo_bytes"] / (gus * 1e-6) / 1e9, 1)}
    fused = {"matvecs": len(fmats), "ms_per_sweep": round(fms, 4), "us_per_layer": round(fms * 1e3 / args.layers, 2),
             "GBps": round(falgo / (fms * 1e-3) / 1e9, 1),
             "hbm_frac_compressed": round(falgo / (fms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "per_shape": f_shape,
             "note": "same weights, q||k||v and gate||up each encoded as one matrix (one launch each)"}
    return fused


# ------------------------------------------------------------- profile summaries
# Host-only helpers that turn rocprofv3 CSV output of this script into the
# committed summaries under profiles/ (no GPU, no torch).

def _short_kernel(name: str) -> str:
    return name.replace("void (anonymous namespace)::", "").split("((anonymous")[0]


def summarize_traffic(fetch_csv, write_csv, profile_json, cmd_fetch, cmd_write):
    """FETCH_SIZE / WRITE_SIZE runs of `--profile-sweeps N --copy-calibration` -> HBM bytes per matvec
    dispatch, each counter scaled so that it reads the calibration copy's true size."""
    import csv
    import statistics
    meta = json.loads(open(profile_json).read().strip().splitlines()[-1])
    true_kib = meta["copy_calibration_bytes"] / 1024.0
    res = {}
    for cname, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == cname]
        first_mv = min(int(r["Dispatch_Id"]) for r in rows if "matvec" in r["Kernel_Name"])
        copies = [r for r in rows if int(r["Dispatch_Id"]) < first_mv and "copy" in r["Kernel_Name"].lower()]
        cal = max(float(r["Counter_Value"]) for r in copies)
        mv = [float(r["Counter_Value"]) for r in rows if "matvec" in r["Kernel_Name"]]
        res[cname] = {"scale": true_kib / cal, "cal_kib": cal, "dispatches": len(mv),
                      "mean_kib": statistics.mean(mv), "bytes": statistics.mean(mv) * 1024 * true_kib / cal}
    hbm = res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]
    algo, blob = meta["algo_bytes_per_launch"], meta["blob_bytes_per_launch"]
    d = {"kernel_source_hash": meta["kernel_source_hash"], "hbm_bytes_per_launch": round(hbm, 1),
         "fetch_bytes_per_launch": round(res["FETCH_SIZE"]["bytes"], 1),
         "write_bytes_per_launch": round(res["WRITE_SIZE"]["bytes"], 1),
         "fetch_scale": round(res["FETCH_SIZE"]["scale"], 4), "write_scale": round(res["WRITE_SIZE"]["scale"], 4),
         "algo_bytes_per_launch": round(algo, 1), "blob_bytes_per_launch": round(blob, 1),
         "dispatches": res["FETCH_SIZE"]["dispatches"]}
    json.dump(d, open(os.path.join(ROOT, "profiles", "matvec_qwen3_4b_traffic.json"), "w"), indent=1)
    with open(os.path.join(ROOT, "profiles", "matvec_qwen3_4b_traffic.md"), "w") as f:
        f.write("# matvec kernel HBM traffic, Qwen3-4B layer set (252 matvecs in 144 launches per step), MI355X\n\n"
                "Commands (from the repository root on an MI355X machine, with `TMPDIR=/tmp`):\n\n"
                f"    {cmd_fetch}\n    {cmd_write}\n\nSummarised with `python bench.py --summarize-traffic` "
                "(the counter CSVs and the JSON line the profiled run printed).\n\n"
                f"Kernel source hash: {meta['kernel_source_hash']}\n\n"
                "Counters are KiB per dispatch.  Each is scaled by the factor that maps its reading for the\n"
                "256 MiB device-to-device calibration copy in the same run to the copy's true size.\n\n"
                "| counter | calibration copy (KiB read) | true KiB | scale | matvec dispatches | mean KiB/dispatch | "
                "scaled bytes/dispatch |\n|---|---|---|---|---|---|---|\n")
        for cname in ("FETCH_SIZE", "WRITE_SIZE"):
            r = res[cname]
            f.write(f"| {cname} | {r['cal_kib']:.0f} | {true_kib:.0f} | {r['scale']:.3f} | {r['dispatches']} | "
                    f"{r['mean_kib']:.1f} | {r['bytes']:.0f} |\n")
        f.write(f"\nPer launch (mean over the step's launches: q,k,v group, o, gate,up group, down): HBM traffic "
                f"{hbm / 1e6:.3f} MB; algorithmic bytes "
                f"(coded bits/8 + 2K + 4N per matrix) {algo / 1e6:.3f} MB; blob bytes {blob / 1e6:.3f} MB.\n"
                f"Traffic / algorithmic = {hbm / algo:.3f}; traffic / blob = {hbm / blob:.3f}.\n")
    print(json.dumps(d, indent=1))


def summarize_counters(csv_path, profile_json, cmd):
    """One counter run of `--profile-sweeps N` with SQ counters -> instructions per 64 weights.

    Only instruction counts are reported: the counters are collected with the
    dispatches serialized, so cycle counters there do not describe the timed step."""
    import collections
    import csv
    import statistics
    meta = json.loads(open(profile_json).read().strip().splitlines()[-1])
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(csv_path)):
        if "matvec" in r["Kernel_Name"]:
            per[r["Counter_Name"]].append(float(r["Counter_Value"]))
    mean = {c: statistics.mean(v) for c, v in per.items()}
    w64 = meta["weights_per_launch"] / 64.0
    derived = {}
    if "SQ_INSTS_VALU" in mean:
        derived["VALU instructions per 64 weights (wave-level)"] = mean["SQ_INSTS_VALU"] / w64
    if "SQ_INSTS_LDS" in mean:
        derived["LDS instructions per 64 weights"] = mean["SQ_INSTS_LDS"] / w64
    if "SQ_INSTS_SALU" in mean:
        derived["SALU instructions per 64 weights"] = mean["SQ_INSTS_SALU"] / w64
    if "SQ_INSTS_VMEM_RD" in mean:
        derived["vector memory reads per 64 weights"] = mean["SQ_INSTS_VMEM_RD"] / w64
    if "SQ_LDS_BANK_CONFLICT" in mean and "SQ_LDS_IDX_ACTIVE" in mean:
        derived["LDS bank-conflict cycles / LDS active cycles"] = mean["SQ_LDS_BANK_CONFLICT"] / mean["SQ_LDS_IDX_ACTIVE"]
    with open(os.path.join(ROOT, "profiles", "matvec_qwen3_4b_counters.md"), "w") as f:
        f.write("# matvec kernel instruction and LDS counters, Qwen3-4B layer set (144 launches per step), MI355X\n\n"
                "Command (from the repository root on an MI355X machine, with `TMPDIR=/tmp`):\n\n"
                f"    {cmd}\n\nSummarised with `python bench.py --summarize-counters`.\n\n"
                f"Kernel source hash: {meta['kernel_source_hash']}\n\n"
                f"Mean per matvec launch ({len(next(iter(per.values())))} dispatches, "
                f"{meta['weights_per_launch'] / 1e6:.2f} M weights each on average).  Counter runs serialize the "
                "dispatches, so only instruction counts (not cycle counts) are used:\n\n"
                "| counter | mean per dispatch |\n|---|---|\n")
        for c in sorted(mean):
            f.write(f"| {c} | {mean[c]:.4g} |\n")
        f.write("\n| derived | value |\n|---|---|\n")
        for k, v in derived.items():
            f.write(f"| {k} | {v:.4g} |\n")
    print(json.dumps({"mean": mean, "derived": derived}, indent=1))


def summarize_workload(run_json, cmd):
    """The JSON line of `--workload qwen25_7b_step`, `tied_embedding` or `prefill` -> its summary under profiles/."""
    d = json.loads(open(run_json).read().strip().splitlines()[-1])
    wl = d["config"]["workload"]
    if wl == "qwen25_7b_decode_step":
        path = os.path.join(ROOT, "profiles", "qwen25_7b_decode_step.md")
        b = d.get("bf16_baseline") or {}
        f_ = d.get("fused_projections") or {}
        body = ("# Qwen2.5-7B-shaped batch-1 decode step, MI355X\n\n"
                f"Command (from the repository root on an MI355X machine):\n\n    {cmd}\n\n"
                "28 layers x {q 3584x3584, k/v 512x3584, o 3584x3584, gate/up 18944x3584, down 3584x18944} + lm_head\n"
                "152064x3584, N(0, 1/sqrt(K)); every linear through the library (q,k,v and gate,up grouped); glue in torch (RMS norms with unit\n"
                "weight, fp32 residual, context-1 attention stand-in = v repeated over the GQA heads, silu(gate)*up).\n"
                "The same step with `torch.nn.functional.linear` on the BF16 weights is the baseline.\n\n"
                "| | ms per token | tokens/s |\n|---|---|---|\n"
                f"| nwc step, q,k,v and gate,up grouped (4 launches per layer, graph replay) | {d['ms_per_step']} | "
                f"{d['value']} |\n"
                f"| nwc step, one launch per matrix (7 per layer) | {d['one_launch_per_matrix']['ms_per_step']} | "
                f"{d['one_launch_per_matrix']['tokens_per_s']} |\n"
                f"| the {d['config']['matrices']} matvecs alone, one launch each | {d['ms_matvecs_only']} | — |\n")
        if f_:
            body += (f"| nwc_matvec step, q\\|\\|k\\|\\|v and gate\\|\\|up fused (4 launches per layer) | "
                     f"{f_['ms_per_step']} | {f_['tokens_per_s']} |\n")
        if b:
            body += f"| BF16 `F.linear` step, same glue | {b['ms_per_step']} | {b['tokens_per_s']} |\n"
        p_ = d.get("bf16_plain_gemv_grouped")
        if p_:
            body += (f"| plain BF16 GEMV step (library's `nwc_bf16_gemv`, grouped like the headline) | "
                     f"{p_['ms_per_step']} | {p_['tokens_per_s']} |\n")
        body += (f"\nMatvecs {d['compressed_GBps_matvecs']} GB/s on {d['compressed_GB']} GB of algorithmic bytes "
                 f"({d['blob_GB']} GB of blobs)")
        if b:
            body += f"; logits relative L2 distance to the BF16 stack {b['logits_rel_l2_vs_bf16_stack']:.2e}"
        body += f".  Kernel source hash {d['kernel_source_hash']}.\n"
    elif wl == "tied_embedding":
        path = os.path.join(ROOT, "profiles", "tied_embedding_and_fp8.md")
        lm, fp8 = d["lm_head"], d["fp8"]
        body = ("# Tied embedding / lm_head 151936x2560 and the fp8 e4m3 variant, MI355X\n\n"
                f"Command (from the repository root on an MI355X machine):\n\n    {cmd}\n\n"
                "| operation | us | rate |\n|---|---|---|\n"
                f"| lm_head GEMV, nwc_matvec ({lm['blob_MB']} MB blob, > 256 MB last-level cache) | {lm['us']} | "
                f"{lm['compressed_GBps']} GB/s compressed ({100 * lm['hbm_frac_compressed']:.1f} % of 8 TB/s) |\n"
                f"| lm_head GEMV, BF16 `F.linear` | {lm['bf16_F_linear_us']} | nwc {lm['speedup_vs_bf16']}x faster |\n"
                f"| gather of 4096 ids, nwc_gather | {d['gather_4096']['us']} | torch index_select on the BF16 table: "
                f"{d['gather_4096']['torch_index_select_on_bf16_us']} us |\n"
                f"| dequantize the whole matrix | {d['dequant_full']['us']} | {d['dequant_full']['GBps_written']} GB/s written |\n")
        for k, byc in fp8.items():
            for cname, v in byc.items():
                if cname == "bf16_same_weights":
                    body += (f"| BF16 compressed matvec {k}, the same weights before fp8 quantization (rotation over "
                             f"{v['rotation']}) | {v['us']} | {v['compressed_GBps']} GB/s, "
                             f"{v['bits_per_weight_coded']} coded bits/weight |\n")
                    continue
                body += (f"| fp8 matvec {k}, {cname} coder (rotation over {v['rotation']}) | {v['us']} | "
                         f"{v['compressed_GBps']} GB/s, {v['bits_per_weight_coded']} coded bits/weight, "
                         f"{v['bits_per_weight_blob']} blob bits/weight |\n")
        body += ("\nThe 1024x1024 matrices (BF16 and fp8) fit in cache: their times are latency figures, not bandwidth "
                 f"claims.\nKernel source hash {d['kernel_source_hash']}.\n")
    elif wl == "prefill":
        path = os.path.join(ROOT, "profiles", "prefill_qwen3_4b.md")
        body = ("# Prefill on the Qwen3-4B layer matrices: nwc_dequant + hipBLASLt GEMM vs the BF16 GEMM, MI355X\n\n"
                f"Command (from the repository root on an MI355X machine):\n\n    {cmd}\n\n"
                f"{d['config']['layers']} layers x 7 matrices in rotation; every matrix dequantized into one reused BF16 "
                "buffer, then `torch.nn.functional.linear`; HIP-graph replay.\n\n"
                "| tokens | nwc us/layer | BF16 us/layer | of which dequant | nwc / BF16 |\n|---|---|---|---|---|\n")
        for t, r in d["per_tokens"].items():
            body += (f"| {t} | {r['us_per_layer_nwc']} | {r['us_per_layer_bf16']} | {r['us_per_layer_dequant']} | "
                     f"{r['nwc_over_bf16']} |\n")
        body += f"\nKernel source hash {d['kernel_source_hash']}.\n"
    elif wl == "small_batch":
        path = os.path.join(ROOT, "profiles", "small_batch_qwen3_4b.md")
        body = ("# Small batches on the Qwen3-4B layer matrices, MI355X\n\n"
                f"Command (from the repository root on an MI355X machine):\n\n    {cmd}\n\n"
                f"{d['config']['layers']} layers x 7 matrices in rotation (cold); B activation rows per matrix; "
                "HIP-graph replay.\n\n| B | path | us per layer | us per token-layer | BF16 `F.linear` us per layer "
                "| nwc speed-up | compressed GB/s |\n|---|---|---|---|---|---|---|\n")
        for b, r in d["per_batch"].items():
            body += (f"| {b} | {r['path']} | {r['us_per_layer_nwc']} | {r['us_per_token_layer_nwc']} | "
                     f"{r['us_per_layer_bf16_F_linear']} | {r['nwc_speedup_vs_bf16']} | {r['compressed_GBps_nwc']} |\n")
        body += f"\nKernel source hash {d['kernel_source_hash']}.\n"
    else:
        raise SystemExit(f"no summary for workload {wl}")
    with open(path, "w") as f:
        f.write(body + "\n```\n" + json.dumps(d) + "\n```\n")


def summarize_trace(prof_dir, profile_json, bench_json, cmd):
    """Kernel trace of `--profile-sweeps N` (the timed step's graph, replayed N times) -> per-launch-kind
    durations, their sum per step against the bench's ms_per_step, and the dominant kernel's bytes/time."""
    import collections
    import csv
    import statistics
    import glob

    def find(name):
        hits = sorted(glob.glob(os.path.join(prof_dir, "**", name), recursive=True))
        if not hits:
            raise SystemExit(f"{name} not found under {prof_dir}")
        return hits[0]

    trace = list(csv.DictReader(open(find("run_kernel_trace.csv"))))
    stats = list(csv.DictReader(open(find("run_kernel_stats.csv"))))
    meta = json.loads(open(profile_json).read().strip().splitlines()[-1])
    d = json.loads(open(bench_json).read().strip().splitlines()[-1])
    mv = [r for r in trace if "matvec" in r["Kernel_Name"]]
    mv.sort(key=lambda r: int(r["Start_Timestamp"]))
    per_sweep = meta["launches_per_sweep"]
    kinds = list(meta["per_launch_kind"])
    assert len(mv) == meta["profile_sweeps"] * per_sweep, (len(mv), meta["profile_sweeps"], per_sweep)
    # Dispatch i of a sweep is launch kind i % 4 (layer order q,k,v | o | gate,up | down).
    dur = collections.defaultdict(list)
    for i, r in enumerate(mv):
        dur[kinds[(i % per_sweep) % len(kinds)]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    layers = meta["layers"]
    step_from_medians = sum(statistics.median(v) for v in dur.values()) * layers / 1e6  # ms
    mean_all = statistics.mean(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in mv)
    sweeps = [mv[j * per_sweep:(j + 1) * per_sweep] for j in range(meta["profile_sweeps"])]
    span = [(int(s[-1]["End_Timestamp"]) - int(s[0]["Start_Timestamp"])) / 1e6 for s in sweeps]
    algo_launch = meta["algo_bytes_per_launch"]
    with open(os.path.join(ROOT, "profiles", "matvec_qwen3_4b_kernel_trace.md"), "w") as f:
        f.write("# matvec kernel trace -- Qwen3-4B layer set, the timed step only, MI355X\n\n"
                "Command (from the repository root on an MI355X machine, with `TMPDIR=/tmp`):\n\n"
                f"    {cmd}\n\nSummarised with `python bench.py --summarize-trace` from that run's CSVs and JSON "
                "line and the JSON line of a plain `python bench.py` run of the same source.\n\n"
                f"Kernel source hash: {meta['kernel_source_hash']} (bench run: {d['kernel_source_hash']})\n\n"
                f"The profiled run replays the step's HIP graph {meta['profile_sweeps']} times; the trace holds "
                f"exactly {len(mv)} matvec dispatches = {meta['profile_sweeps']} x {per_sweep} (36 layers x "
                "{q,k,v group, o, gate,up group, down}); nothing else runs between them.\n\n"
                "| launch kind | matrices | dispatches | median us | mean us | algorithmic MB | GB/s at the median |\n"
                "|---|---|---|---|---|---|---|\n")
        for k in kinds:
            v = dur[k]
            info = meta["per_launch_kind"][k]
            med = statistics.median(v) / 1e3
            f.write(f"| {k} | {'+'.join(info['matrices'])} | {len(v)} | {med:.2f} | {statistics.mean(v) / 1e3:.2f} | "
                    f"{info['algo_bytes'] / 1e6:.2f} | {info['algo_bytes'] / (med * 1e-6) / 1e9:.0f} |\n")
        f.write("\n| | ms per step |\n|---|---|\n"
                f"| sum of the per-kind medians x {layers} layers (kernel execution only) | {step_from_medians:.4f} |\n"
                f"| first-to-last dispatch span of one replay under the profiler (median of {len(span)}) | "
                f"{statistics.median(span):.4f} |\n"
                f"| bench.py `ms_per_step` (HIP events around graph replays, no profiler) | {d['ms_per_step']} |\n\n"
                f"All {len(mv)} matvec dispatches: mean {mean_all / 1e3:.3f} us.  Dominant kernel (the fused decode + "
                f"matvec, both entry points): {algo_launch / 1e6:.3f} MB algorithmic per launch / {mean_all / 1e3:.3f} us "
                f"= {algo_launch / (mean_all * 1e-9) / 1e9:.0f} GB/s "
                f"({algo_launch / (mean_all * 1e-9) / 1e9 / HBM_PEAK_GBPS:.4f} of 8 TB/s) from the trace; the bench "
                f"line's roofline gives {d['roofline']['achieved']} GB/s ({d['roofline']['frac']}) with launch gaps "
                "counted.\n\n`run_kernel_stats.csv`, matvec rows:\n\n"
                "| kernel | calls | avg us | min us | max us |\n|---|---|---|---|---|\n")
        for r in stats:
            if "matvec" in r["Name"]:
                f.write(f"| {_short_kernel(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                        f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |\n")
        keep = {k: d.get(k) for k in ("value", "unit", "ms_per_step", "us_per_layer", "roofline")}
        f.write(f"\nThe bench line (abridged):\n\n```\n{json.dumps(keep)}\n```\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=("qwen3_4b_layer_set", "qwen25_7b_step", "tied_embedding", "prefill",
                                           "small_batch"),
                    default="qwen3_4b_layer_set")
    ap.add_argument("--layers", type=int, default=0, help="layers of the workload (0: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16-baseline", action="store_true")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused-projection measurement")
    ap.add_argument("--profile-sweeps", type=int, default=0,
                    help="run this many eager sweeps and exit, untimed (for rocprofv3 counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before the sweeps, copy 256 MiB device->device once, a reference dispatch of known "
                         "size for scaling the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-traffic", nargs=5, metavar=("FETCH_CSV", "WRITE_CSV", "RUN_JSON", "CMD_F", "CMD_W"),
                    help="write profiles/matvec_qwen3_4b_traffic.{json,md} from two counter runs and exit")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("PROF_DIR", "PROFILE_JSON", "BENCH_JSON", "CMD"),
                    help="write profiles/matvec_qwen3_4b_kernel_trace.md from a kernel-trace run and exit")
    ap.add_argument("--summarize-workload", nargs=2, metavar=("RUN_JSON", "CMD"),
                    help="write the profiles/ summary of a qwen25_7b_step, tied_embedding or prefill run and exit")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("CSV", "RUN_JSON", "CMD"),
                    help="write profiles/matvec_qwen3_4b_counters.md from an SQ/GRBM counter run and exit")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_workload:
        summarize_workload(*args.summarize_workload)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth as S
    from synth import configs as C
    from decode_matvec_amd import nwc

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.workload == "qwen25_7b_step":
        bench_qwen25_step(args, torch, nwc, S, C, dev)
        return
    if args.workload == "tied_embedding":
        bench_tied_embedding(args, torch, nwc, S, C, dev)
        return
    if args.workload == "prefill":
        bench_prefill(args, torch, nwc, S, C, dev)
        return
    if args.workload == "small_batch":
        bench_small_batch(args, torch, nwc, S, C, dev)
        return
    args.layers = args.layers or C.QWEN3_4B_LAYERS
    mats, fmats = build_layer_set(torch, nwc, S, C, dev, args.layers,
                                  not args.no_bf16_baseline and not args.profile_sweeps,
                                  fused=not (args.profile_sweeps or args.no_fused))
    # The step as a decoder can launch it: in each layer the projections that
    # read one input (q, k, v; gate, up) run as one nwc_matvec_group launch, o
    # and down alone, in layer order -- 4 launches per layer.  Each matrix keeps
    # its own encoding and its own activation.
    by_layer = [{m["name"]: m for m in mats[7 * l:7 * l + 7]} for l in range(args.layers)]
    launch_groups = [[L[p] for p in parts] for L in by_layer for _, parts in FUSED_QWEN3]
    n_launch = len(launch_groups)

    def run_group(g):
        if len(g) == 1:
            g[0]["dm"].matvec(g[0]["x"], g[0]["y"])
        else:
            nwc.matvec_group([m["dm"] for m in g], [m["x"] for m in g], [m["y"] for m in g])

    def sweep():
        for g in launch_groups:
            run_group(g)

    def sweep_per_matrix():
        for m in mats:
            m["dm"].matvec(m["x"], m["y"])

    if args.profile_sweeps:
        if args.copy_calibration:
            src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        # The timed step's launches only: the sweep captured once (capture
        # launches nothing) and replayed N times, so a kernel trace holds
        # exactly N x launches_per_sweep matvec dispatches.
        pg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pg):
            sweep()
        torch.cuda.synchronize()
        for _ in range(args.profile_sweeps):
            pg.replay()
        torch.cuda.synchronize()
        print(json.dumps({"profile_sweeps": args.profile_sweeps, "launches_per_sweep": n_launch,
                          "matvecs_per_sweep": len(mats),
                          "algo_bytes_per_launch": sum(m["algo_bytes"] for m in mats) / n_launch,
                          "blob_bytes_per_launch": sum(m["blob_bytes"] for m in mats) / n_launch,
                          "weights_per_launch": sum(m["n"] * m["k"] for m in mats) / n_launch,
                          "per_launch_kind": {gname: {"matrices": list(parts),
                                                      "algo_bytes": sum(m["algo_bytes"] for m in launch_groups[i]),
                                                      "blob_bytes": sum(m["blob_bytes"] for m in launch_groups[i]),
                                                      "weights": sum(m["n"] * m["k"] for m in launch_groups[i])}
                                              for i, (gname, parts) in enumerate(FUSED_QWEN3)},
                          "layers": args.layers,
                          "copy_calibration_bytes": (64 << 20) * 4 if args.copy_calibration else 0,
                          "kernel_source_hash": kernel_source_hash()}), flush=True)
        return

    # The sweep is captured once as a HIP graph and replayed: 252 launches per
    # step from Python would otherwise be limited by host launch overhead,
    # not by the GPU.  The eager (per-call ctypes launch) rate is reported too.
    ms_eager = time_region(torch, sweep, max(2, args.steps // 4), 1)
    # One launch per matrix (252 per sweep), for comparison.
    sweep_per_matrix()
    torch.cuda.synchronize()
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        sweep_per_matrix()
    ms_one = time_region(torch, g1.replay, args.steps, args.warmup)
    del g1
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sweep()  # warm the launch path on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        sweep()
    torch.cuda.synchronize()
    ms = time_region(torch, graph.replay, args.steps, args.warmup)
    algo = sum(m["algo_bytes"] for m in mats)
    blob = sum(m["blob_bytes"] for m in mats)
    bf16_bytes = sum(2.0 * m["n"] * m["k"] for m in mats)
    value = algo / (ms * 1e-3) / 1e9

    per_shape = {}
    for name, n, k in C.QWEN3_4B:
        group = [m for m in mats if m["name"] == name]

        def g_sweep(group=group):
            for m in group:
                m["dm"].matvec(m["x"], m["y"])

        gg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gg):
            g_sweep()
        gms = time_region(torch, gg.replay, max(3, args.steps // 2), 1)
        us = gms * 1e3 / len(group)
        gb = sum(m["algo_bytes"] for m in group) / len(group)
        per_shape[name] = {"shape": [n, k], "us": round(us, 3),
                           "compressed_GBps": round(gb / (us * 1e-6) / 1e9, 1),
                           "effective_bf16_GBps": round(2.0 * n * k / (us * 1e-6) / 1e9, 1),
                           "blob_MB": round(group[0]["blob_bytes"] / 1e6, 3),
                           "bits_per_weight_coded": round(group[0]["info"]["coded_bits"] / (n * k), 4),
                           "bits_per_weight_blob": round(group[0]["blob_bytes"] * 8 / (n * k), 4),
                           "geometry": {f: group[0]["info"][f] for f in ("cols_per_lane", "rows_per_wave", "waves_per_group", "n_spans")}}

    # Each launch of the grouped step on its own: the 36 launches of one kind
    # (q,k,v group / o / gate,up group / down) replayed back to back.
    per_launch = {}
    for gi, (gname, parts) in enumerate(FUSED_QWEN3):
        gl = launch_groups[gi::len(FUSED_QWEN3)]
        gg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gg):
            for g in gl:
                run_group(g)
        gms = time_region(torch, gg.replay, max(3, args.steps // 2), 1)
        us = gms * 1e3 / len(gl)
        gb = sum(m["algo_bytes"] for g in gl for m in g) / len(gl)
        bb = sum(m["blob_bytes"] for g in gl for m in g) / len(gl)
        per_launch[gname] = {"matrices": list(parts), "us": round(us, 3), "algo_MB": round(gb / 1e6, 3),
                             "blob_MB": round(bb / 1e6, 3), "compressed_GBps": round(gb / (us * 1e-6) / 1e9, 1),
                             "blob_GBps": round(bb / (us * 1e-6) / 1e9, 1)}

    # Decode clocks per 64 weights: CU-clocks (time x MI355X's 2.4 GHz peak engine
    # clock x 256 CUs) over weights / 64, for the cold sweep and for one gate
    # matrix replayed while its 38 MB blob stays in the 256 MB last-level cache
    # (the decode-bound setting).
    n_w = sum(m["n"] * m["k"] for m in mats)

    def cu_clocks_per_64w(seconds, weights):
        return round(seconds * CLOCK_HZ * N_CU / (weights / 64.0), 2)

    gate = next(m for m in mats if m["name"] == "gate")
    hg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(hg):
        for _ in range(20):
            gate["dm"].matvec(gate["x"], gate["y"])
    hms = time_region(torch, hg.replay, max(3, args.steps // 2), 2) / 20
    decode_clocks = {"cold_sweep": cu_clocks_per_64w(ms * 1e-3, n_w),
                     "cache_resident_gate": cu_clocks_per_64w(hms * 1e-3, gate["n"] * gate["k"]),
                     "cache_resident_gate_us": round(hms * 1e3, 3), "clock_GHz": CLOCK_HZ / 1e9, "cus": N_CU}

    # The same layers as a decoder runs them: projections sharing an input fused
    # (q||k||v, gate||up), 4 launches per layer instead of 7.
    fused = measure_fused(torch, fmats, args) if fmats else None
    # Four tokens at once: each weight decoded once for four activation rows.
    batch4 = None if args.no_fused else measure_batch(torch, mats, args, ms)

    # Achievable bandwidth for the same launch pattern: a plain streaming read
    # (nwc_stream_read, 16-byte loads) of every blob in sweep order, and of 1 GiB.
    stream = None
    if not args.no_bf16_baseline:
        sink = torch.zeros(64, dtype=torch.int32, device=dev)
        sg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(sg):
            for m in mats:
                nwc.stream_read(m["dm"].d_blob, sink)
        sms = time_region(torch, sg.replay, max(3, args.steps // 2), 2)
        big = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
        bgr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(bgr):
            nwc.stream_read(big, sink)
        bigms = time_region(torch, bgr.replay, max(3, args.steps // 2), 2)
        stream = {"same_launches_GBps": round(blob / (sms * 1e-3) / 1e9, 1),
                  "one_GiB_GBps": round((1 << 30) / (bigms * 1e-3) / 1e9, 1),
                  "matvec_blob_GBps_over_stream_read": round(sms / ms, 4),
                  "kernel": "nwc_stream_read: plain streaming read of each blob (16-byte loads), same graph order"}
        del big

    bf16 = None
    if not args.no_bf16_baseline:
        F = torch.nn.functional

        def bf16_sweep():
            for m in mats:
                F.linear(m["x_bf16"], m["w_bf16"])

        bf16_sweep()  # library handles are created on first use, which capture forbids
        torch.cuda.synchronize()
        bg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(bg):
            bf16_sweep()
        bms = time_region(torch, bg.replay, args.steps, args.warmup)
        bf16 = {"ms_per_sweep": round(bms, 4),
                "GBps": round((bf16_bytes + sum(2.0 * (m["n"] + m["k"]) for m in mats)) / (bms * 1e-3) / 1e9, 1),
                "speedup_compressed_vs_bf16": round(bms / ms, 4),
                "kernel": "torch.nn.functional.linear (hipBLASLt/rocBLAS), same rotation"}

        # The library's plain BF16 GEMV (no decode), same weights and rotation: the uncompressed
        # reference on the same skeleton of 16-byte streaming loads.
        ys = [torch.empty(m["n"], dtype=torch.float32, device=dev) for m in mats]

        def plain_sweep():
            for m, yy in zip(mats, ys):
                nwc.bf16_gemv(m["w_bf16"], m["x_bf16"], yy)

        plain_sweep()
        torch.cuda.synchronize()
        pg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pg):
            plain_sweep()
        pms = time_region(torch, pg.replay, args.steps, args.warmup)
        bf16["plain_gemv"] = {"ms_per_sweep": round(pms, 4),
                              "GBps": round((bf16_bytes + sum(2.0 * (m["n"] + m["k"]) for m in mats)) / (pms * 1e-3) / 1e9, 1),
                              "speedup_compressed_vs_plain": round(pms / ms, 4),
                              "kernel": "nwc_bf16_gemv: plain BF16 GEMV, one launch per matrix, 16-byte streaming "
                                        "loads, no decode"}
        # The same plain GEMV with the launch structure of the timed step:
        # q,k,v and gate,up one launch each (nwc_bf16_gemv_group).
        ymap = {id(m): yy for m, yy in zip(mats, ys)}

        def plain_group_sweep():
            for g in launch_groups:
                if len(g) == 1:
                    nwc.bf16_gemv(g[0]["w_bf16"], g[0]["x_bf16"], ymap[id(g[0])])
                else:
                    nwc.bf16_gemv_group([m["w_bf16"] for m in g], [m["x_bf16"] for m in g],
                                        [ymap[id(m)] for m in g])

        plain_group_sweep()
        torch.cuda.synchronize()
        pgg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pgg):
            plain_group_sweep()
        pgms = time_region(torch, pgg.replay, args.steps, args.warmup)
        bf16["plain_gemv_grouped"] = {
            "ms_per_sweep": round(pgms, 4),
            "GBps": round((bf16_bytes + sum(2.0 * (m["n"] + m["k"]) for m in mats)) / (pgms * 1e-3) / 1e9, 1),
            "speedup_compressed_vs_plain_grouped": round(pgms / ms, 4),
            "kernel": "nwc_bf16_gemv_group / nwc_bf16_gemv: plain BF16 GEMV, 4 launches per layer as the timed step"}
        best = min(bms, pms, pgms)
        bf16["best_bf16_ms_per_sweep"] = round(best, 4)
        bf16["speedup_compressed_vs_best_bf16"] = round(best / ms, 4)
        del ys

    # The dominant kernel is the fused decode + matvec (the group launches and
    # the single-matrix launches run the same kernel body): algorithmic bytes
    # per launch over its average launch time in the timed step.
    algo_per_launch = algo / n_launch
    achieved = algo_per_launch / (ms * 1e-3 / n_launch) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_from_profiles(algo_per_launch)}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on host cores")
        cpu = cpu_baseline(S, C)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1/sqrt(K)) BF16 weights)",
        "config": {"workload": "qwen3_4b_layer_set", "layers": args.layers, "matrices": len(mats),
                   "launches": n_launch, "batch": 1,
                   "note": "36 x {q 4096x2560, k/v 1024x2560, o 2560x4096, gate/up 9728x2560, down 2560x9728}, "
                           "each matrix its own encoding and activation; per layer q,k,v one grouped launch, o, "
                           "gate,up one grouped launch, down (nwc_matvec_group / nwc_matvec); cold rotation"},
        "us_per_layer": round(ms * 1e3 / args.layers, 2),
        "timing": "HIP graph replay of the whole sweep on one stream; HIP events around the timed steps",
        "one_launch_per_matrix": {"ms_per_sweep": round(ms_one, 4), "launches": len(mats),
                                  "us_per_layer": round(ms_one * 1e3 / args.layers, 2),
                                  "GBps": round(algo / (ms_one * 1e-3) / 1e9, 1),
                                  "hbm_frac_compressed": round(algo / (ms_one * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "per_launch": per_launch,
        "ms_per_step_eager_launches": round(ms_eager, 4),
        "us_per_launch_avg": round(ms * 1e3 / n_launch, 3),
        "hbm_frac_compressed": round(value / HBM_PEAK_GBPS, 4),
        "effective_bf16_GBps": round(bf16_bytes / (ms * 1e-3) / 1e9, 1),
        "blob_GBps": round(blob / (ms * 1e-3) / 1e9, 1),
        "compressed_GB": round(algo / 1e9, 4), "blob_GB": round(blob / 1e9, 4), "bf16_GB": round(bf16_bytes / 1e9, 4),
        "per_shape": per_shape, "bf16_baseline": bf16, "stream_read_baseline": stream,
        "decode_cu_clocks_per_64_weights": decode_clocks, "roofline": roof, "cpu_baseline": cpu,
        "fused_projections": fused, "batch4": batch4,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
