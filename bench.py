"""Throughput of one EAGLE draft-and-verify cycle on one MI355X (batch 1 by
default; --batch B serves B sequences per cycle).

A step is one cycle: the draft passes and tree build (eagle_draft_tree) plus
the target verify pass, acceptance, KV compaction and the draft catch-up
(eagle_verify, or eagle_verify_batch for every lane of a batch), on seeded
synthetic weights and prompts already resident in HBM. Prints one JSON line
(see README of the driver contract):
  value       committed tokens/s over all lanes (tau x lanes x cycles/s; tau ~
              1 with random weights)
  roofline    the dominant kernel: the split-K projection of the target
              layers (q|k|v, o and down at M = tree rows), its algorithmic
              bytes / its device time from HIP events recorded around each of
              its launches inside the timed region, against 8 TB/s
  cpu_baseline  the CPU oracle timed on this host on a bounded sample
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0
# one in ROOF_EVERY dispatches of the roofline kernel carries HIP events in the
# timed region; 4 is coprime with the three projections of a layer, so q|k|v,
# o and down are sampled equally, and the events cost ~1.5% of a cycle
ROOF_EVERY = 4

WORKLOAD_TEXT = {
    "c1": "tiny fp32 Llama target (2 layers, H=256, V=1024), EAGLE-1 head, dynamic tree k=4 D=3 m=16, prompt 32",
    "c2": "Llama-2-7B-shaped bf16 target (32 layers, H=4096, 32 heads, FFN 11008, V=32000), EAGLE-1 head (FC 8192->4096 + 1 layer), static 26-node tree of depth 5, prompt 512, 256 generated",
    "c3": "Llama-2-7B-shaped bf16 target, EAGLE-1 head, EAGLE-2 dynamic tree k=10 D=6 m=60, prompt 1536, 512 generated",
    "c4": "Llama-3-8B-shaped bf16 target (GQA 32/8, FFN 14336, V=128256), EAGLE-3 head (FC 12288->4096 + 1 layer), k=8 D=7 m=64, context 4096",
    "c5": "Llama-2-70B-shaped bf16 target (80 layers, H=8192, GQA 64/8, FFN 28672), EAGLE-1 head, k=10 D=6 m=60, prompt 1024, 256 generated",
}


KERNEL_SOURCES = ["speculative_decoding_draft_amd/csrc/gemm.hip", "speculative_decoding_draft_amd/csrc/common.h"]


def stored_traffic(kernel_key: str):
    """HBM bytes per launch of a kernel from the counter summaries in profiles/
    (FETCH_SIZE and WRITE_SIZE runs scaled by a known-size copy), or None when
    none is recorded or the kernel's sources changed since the counters were
    taken (the summary records a hash of the sources)."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    digest = h.hexdigest()[:16]
    pat = re.compile(r"^traffic: (.+) = (\d+) bytes per launch; sources sha256 ([0-9a-f]+)\s*$")
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path, encoding="utf-8") as fh:
            for line in fh:
                m = pat.match(line)
                if m and m.group(1) == kernel_key and m.group(3) == digest:
                    return int(m.group(2))
    return None


def cycle_bytes(w: dict, ctx: int, lanes: int = 1) -> float:
    """Algorithmic HBM bytes of one cycle at context ctx: every weight byte the
    cycle must read (target layers + LM head once; draft layer + LM head +
    FC per draft pass), plus the KV cache reads (4 bytes per K/V element) of
    each of `lanes` sequences."""
    H, nq, nkv, F, V, L = (w[k] for k in ("hidden", "n_heads", "n_kv_heads", "ffn", "vocab", "n_layers"))
    d = H // nq
    esz = 2 if w["dtype"] == "bf16" else 4
    kin = 2 * H if w["head"] == "e3" else H
    layer = lambda k: k * (nq + 2 * nkv) * d + nq * d * H + 3 * H * F
    D = w["depth"]
    target = L * layer(H) + V * H
    draft = D * (layer(kin) + V * H)
    fc = D * H * 2 * H if w["head"] == "e1" else H * 3 * H
    kv = 2 * nkv * d * 4 * (L * ctx + D * ctx) * lanes
    return esz * (target + draft + fc) + kv


PEAK_BF16_TFLOPS = 2500.0   # dense MFMA, bf16


def prefill_flops(w: dict, n: int) -> float:
    """Algorithmic FLOPs of a prefill over n prompt tokens: every target
    projection and the LM head row of the last token (2 x weights x rows),
    causal attention (QK^T and PV over n(n+1)/2 visible pairs per head), and
    the draft catch-up over the n (feature, token) pairs (FC + draft layer)."""
    H, nq, nkv, F, V, L = (w[k] for k in ("hidden", "n_heads", "n_kv_heads", "ffn", "vocab", "n_layers"))
    d = H // nq
    kin = 2 * H if w["head"] == "e3" else H
    layer = lambda k: k * (nq + 2 * nkv) * d + nq * d * H + 3 * H * F
    fc = H * (3 * H if w["head"] == "e3" else 2 * H)
    pairs = n * (n + 1) / 2
    attn = 4.0 * pairs * d * nq
    return (2.0 * n * (L * layer(H) + layer(kin) + fc) + 2.0 * V * H * 2
            + attn * (L + 1))


def cpu_baseline(w: dict, budget_layers: int = 2) -> dict:
    """The oracle on this host: draft passes and verify of one cycle timed on a
    slice with `budget_layers` target layers (same width, tree, vocabulary;
    prompt 64), plus the measured time of one more target layer at the verify
    row count times the remaining layers."""
    import numpy as np
    import synth
    from oracle.loop import Session
    from oracle.model import Config, Weights, decoder_layer, causal_vis
    from synth import TARGET
    ws = synth.workloads.reduced(w["name"], n_layers=budget_layers, prompt_len=64, gen=8)
    cfg = Config(ws)
    W = Weights(cfg, cache_bytes=48 << 30)
    s = Session(ws, W)
    p = synth.prompt(1, ws["prompt_len"], ws["vocab"])
    s.prefill(p)
    s.draft_tree()
    s.verify()          # warm: weights generated and cached
    t0 = time.perf_counter()
    s.draft_tree()
    t1 = time.perf_counter()
    s.verify()
    t2 = time.perf_counter()
    M = len(s.rows["token"]) if hasattr(s, "rows") else 1 + ws["budget"]
    ctx = s.ctx
    kc = np.zeros((ctx + M, cfg.n_kv_heads, cfg.head_dim))
    vc = np.zeros_like(kc)
    h = np.random.default_rng(0).standard_normal((M, cfg.hidden))
    vis = np.ones((M, ctx + M), dtype=bool)
    decoder_layer(cfg, W, TARGET, 0, h, ctx + np.arange(M), kc, vc, ctx + np.arange(M), vis)
    t3 = time.perf_counter()
    decoder_layer(cfg, W, TARGET, 0, h, ctx + np.arange(M), kc, vc, ctx + np.arange(M), vis)
    t4 = time.perf_counter()
    per_cycle = (t1 - t0) + (t2 - t1) + (w["n_layers"] - budget_layers) * (t4 - t3)
    cores = len(os.sched_getaffinity(0))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        if os.environ.get(var, "").isdigit():
            cores = min(cores, int(os.environ[var]))   # BLAS threads actually used
            break
    return {"value": round(1.0 / per_cycle, 5), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"one cycle of {w['name']} (tau=1): draft passes {t1 - t0:.2f}s and verify "
                       f"{t2 - t1:.2f}s timed on a {budget_layers}-layer slice (full width, tree, "
                       f"vocab; prompt 64) + {w['n_layers'] - budget_layers} x {t4 - t3:.2f}s per "
                       f"target layer at {M} rows; numpy fp64, {cores} threads")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--profile-cycles", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: sampling-mode verification (rejection sampling over the tree)")
    ap.add_argument("--batch", type=int, default=1,
                    help="sequences served per cycle (lanes; each its own prompt)")
    ap.add_argument("--prefill-chunk", type=int, default=0,
                    help="prompt rows per prefill pass (0: the library default, 512)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device-to-device copies of MIB MiB (the known-size "
                         "kernel that scales the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration > 0:
        import torch
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 3}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 "
                                   "(multi-GPU sharding is design-only)"}))
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import speculative_decoding_draft_amd as E

    w = synth.workloads.get(args.config)
    if args.temperature > 0:
        w.update(temperature=args.temperature, seed=args.seed)
    B = args.batch
    w["batch"] = B
    cycles_needed = args.warmup + args.steps + max(0, args.profile_cycles) + 2 + 5   # + speedup-model cycles
    max_new = max(w["gen"], cycles_needed * (w["depth"] + 1))
    max_ctx = w["prompt_len"] + max_new + w["depth"] + 2
    eng = E.Engine(w, max_ctx=max_ctx, prefill_chunk=args.prefill_chunk)
    synth.fill_weights(eng.table, eng.weights.data_ptr(), w["weight_seed"], eng.stream.cuda_stream)
    torch.cuda.synchronize()
    eng.load()
    # lane b's prompt comes from seed + b (lane 0: the batch-1 prompt)
    prompts = [synth.prompt(args.seed + b, w["prompt_len"], w["vocab"]) for b in range(B)]
    prompt = prompts[0]
    # the first prefill loads the kernels; the second (it restarts the
    # sequence) is the timed one
    eng.prefill(prompt)
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    eng.prefill(prompt)
    torch.cuda.synchronize()
    prefill_ms = (time.perf_counter() - tp0) * 1e3
    for b in range(1, B):
        eng.prefill(prompts[b], lane=b)
    print(f"# {args.config}: prefill done, ctx {len(prompt)}, {prefill_ms:.1f} ms, {B} lane(s)",
          file=sys.stderr, flush=True)

    def cycle():
        eng.draft_tree(want=False)
        if B == 1:
            return len(eng.verify())
        return sum(len(n) for n in eng.verify_batch())

    def mean_ctx():
        return sum(len(eng.committed(b)) for b in range(B)) / B + len(prompt) - 1

    # the dominant kernel's launches carry HIP events from warmup on, so the
    # event pool is allocated before the timed region
    eng.profile(["gemm"], every=ROOF_EVERY)
    for _ in range(args.warmup):
        cycle()
    torch.cuda.synchronize()
    eng.profile(["gemm"], every=ROOF_EVERY)   # reset the counters; keep the class enabled
    ctx0 = mean_ctx()
    t0 = time.perf_counter()
    committed = 0
    for _ in range(args.steps):
        committed += cycle()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dt = t1 - t0
    g = eng.profile_read()["gemm"]
    eng.profile(False)
    ctx1 = mean_ctx()
    print(f"# timed {args.steps} cycles in {dt * 1e3:.1f} ms", file=sys.stderr, flush=True)

    # algorithmic bytes of the timed cycles (context grows by L+1 per cycle)
    avg_ctx = 0.5 * (ctx0 + ctx1)
    bytes_cycle = cycle_bytes(w, int(avg_ctx), B)
    gemm_gbps = g["bytes"] / (g["ms"] * 1e-3) / 1e9 if g["ms"] > 0 else 0.0
    mv = B * (1 + w["budget"])    # target rows of a verify pass
    mt = (mv + 15) // 16 if mv <= 80 else 4

    # breakdown window after the timed region: events around every launch
    prof = None
    if args.profile_cycles > 0:
        eng.profile(True)
        for _ in range(args.profile_cycles):
            cycle()
        prof = eng.profile_read()
        eng.profile(False)
    # draft-pass and target-pass times for the speedup model: D - 1 tree
    # passes in eagle_draft_tree; the target pass plus one catch-up draft
    # pass in eagle_verify
    model = None
    if w["depth"] >= 2 and w["budget"] > 0 and B == 1:
        from speculative_decoding_draft_amd import speedup as spm
        td = tv = 0.0
        n_model = 5
        for _ in range(n_model):
            torch.cuda.synchronize()
            a0 = time.perf_counter()
            eng.draft_tree(want=False)
            torch.cuda.synchronize()
            a1 = time.perf_counter()
            eng.verify()
            torch.cuda.synchronize()
            a2 = time.perf_counter()
            td += a1 - a0
            tv += a2 - a1
        t_draft = td / n_model / (w["depth"] - 1)
        model = spm.report(t_draft, tv / n_model - t_draft, w["depth"])
    cycles_s = args.steps / dt
    tau = committed / args.steps / B
    roof_key = (f"proj_kernel<{'bf16' if w['dtype'] == 'bf16' else 'f32'}, MT={mt}, EPI_PART> M={mv}")
    traffic = stored_traffic(roof_key)
    out = {
        "metric": ("committed tokens/sec + draft/verify cycles/sec at bs=1; % of HBM roofline"
                   if B == 1 else
                   f"committed tokens/sec + draft/verify cycles/sec at bs={B}; % of HBM roofline"),
        "value": round(committed / dt, 3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded N(0,0.02)-like weights, uniform random prompt)",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}"
                               + (f"; sampling at temperature {args.temperature}" if args.temperature > 0 else "")
                               + (f"; {B} sequences per cycle" if B > 1 else ""),
                   "global_batch": B, "seq_len": int(avg_ctx), "parallelism": "none (1 GPU)"},
        "cycles_per_s": round(cycles_s, 3),
        "tau": round(tau, 4),
        "cycle_hbm": {"bytes_per_cycle": bytes_cycle,
                      "achieved_GBps": round(bytes_cycle * cycles_s / 1e9, 1),
                      "frac": round(bytes_cycle * cycles_s / 1e9 / PEAK_GBPS, 4)},
        "roofline": {"bound": "hbm",
                     "kernel": (f"proj_kernel<{'bf16' if w['dtype'] == 'bf16' else 'f32'}, MT={mt}, EPI_PART>: "
                                f"target q|k|v, o and down projections at M={mv}"),
                     "achieved": round(gemm_gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gemm_gbps / PEAK_GBPS, 4), "traffic": traffic,
                     "launches": g["launches"], "avg_launch_us": round(g["ms"] * 1e3 / max(1, g["launches"]), 2),
                     "bytes_per_launch": round(g["bytes"] / max(1, g["launches"]))},
    }
    out["prefill_ms"] = round(prefill_ms, 3)
    # the prefill (one lane, the timed second run) against the dense bf16 MFMA peak
    pf = prefill_flops(w, len(prompt))
    out["prefill_roofline"] = {"bound": "mfma", "achieved": round(pf / (prefill_ms * 1e-3) / 1e12, 1),
                               "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(pf / (prefill_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                               "flops": pf, "tokens": len(prompt),
                               "chunk": args.prefill_chunk or 512}
    if model is not None:
        out["speedup_model"] = model
    if prof is not None:
        out["profile_ms_per_cycle"] = {k: round(v["ms"] / args.profile_cycles, 4) for k, v in prof.items()}
    if not args.no_cpu:
        # sequences are independent: the oracle's tokens/s is the same at any batch
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out))
    eng.close()


if __name__ == "__main__":
    main()
