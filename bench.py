"""Throughput of one EAGLE draft-and-verify cycle on one MI355X (batch 1 by
default; --batch B serves B sequences per cycle).

A step is one cycle: the draft passes and tree build (eagle_draft_tree) plus
the target verify pass, acceptance, KV compaction and the draft catch-up
(eagle_verify, or eagle_verify_batch for every lane of a batch), on seeded
synthetic weights and prompts already resident in HBM. For each prompt seed
(1, 2, 3 by default) the sequence is prefilled, advanced by untimed cycles to
the config's mean context (prompt + half the generation) less half the timed
cycles, warmed up, and K cycles are timed. Prints one JSON line:
  value       committed tokens/s over all lanes (tau x lanes x cycles/s; tau ~
              1 with random weights), from the median seed's timed cycles;
              every seed's figure is under "seeds"
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


def cycle_bytes(w: dict, ctx: int, lanes: int = 1, kv_elem_bytes: int = None) -> float:
    """Algorithmic HBM bytes of one cycle at context ctx: every weight byte the
    cycle must read (target layers + LM head once; draft layer + LM head +
    FC per draft pass), plus the KV cache reads of each of `lanes` sequences at
    the method's element size (2 bytes for bf16; the hi + lo planes this
    implementation keeps are 4 bytes per element, passed as kv_elem_bytes
    to count its KV traffic instead)."""
    H, nq, nkv, F, V, L = (w[k] for k in ("hidden", "n_heads", "n_kv_heads", "ffn", "vocab", "n_layers"))
    d = H // nq
    esz = 2 if w["dtype"] == "bf16" else 4
    kin = 2 * H if w["head"] == "e3" else H
    layer = lambda k: k * (nq + 2 * nkv) * d + nq * d * H + 3 * H * F
    D = w["depth"]
    target = L * layer(H) + V * H
    draft = D * (layer(kin) + V * H)
    fc = D * H * 2 * H if w["head"] == "e1" else H * 3 * H
    kv = 2 * nkv * d * (kv_elem_bytes or esz) * (L * ctx + D * ctx) * lanes
    return esz * (target + draft + fc) + kv


def plain_token_bytes(w: dict, ctx: int) -> float:
    """Algorithmic HBM bytes of one plain greedy decode step at context ctx:
    target layers and LM head once, plus the target KV at the method's
    element size."""
    H, nq, nkv, F, V, L = (w[k] for k in ("hidden", "n_heads", "n_kv_heads", "ffn", "vocab", "n_layers"))
    d = H // nq
    esz = 2 if w["dtype"] == "bf16" else 4
    layer = nq * d * H + 2 * nkv * d * H + nq * d * H + 3 * H * F
    return esz * (L * layer + V * H + 2 * nkv * d * L * ctx)


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
    model_name = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model_name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        if os.environ.get(var, "").isdigit():
            cores = min(cores, int(os.environ[var]))   # BLAS threads actually used
            break
    return {"value": round(1.0 / per_cycle, 5), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": model_name,
            "sample": (f"one cycle of {w['name']} (tau=1): draft passes {t1 - t0:.2f}s and verify "
                       f"{t2 - t1:.2f}s timed on a {budget_layers}-layer slice (full width, tree, "
                       f"vocab; prompt 64) + {w['n_layers'] - budget_layers} x {t4 - t3:.2f}s per "
                       f"target layer at {M} rows; numpy fp64, {cores} threads")}


def make_engine(w: dict, cycles: int, prefill_chunk: int = 0):
    """A loaded engine with the seeded weights, sized for the prompt plus
    `cycles` cycles of up to depth + 1 tokens each (and the generation)."""
    import torch
    import synth
    import speculative_decoding_draft_amd as E
    max_new = max(w["gen"], cycles * (w["depth"] + 1))
    max_ctx = w["prompt_len"] + max_new + w["depth"] + 2
    eng = E.Engine(w, max_ctx=max_ctx, prefill_chunk=prefill_chunk)
    synth.fill_weights(eng.table, eng.weights.data_ptr(), w["weight_seed"], eng.stream.cuda_stream)
    torch.cuda.synchronize()
    eng.load()
    return eng


def run_cycles(eng, B: int, n: int) -> int:
    """n cycles of every lane; returns the tokens committed."""
    committed = 0
    for _ in range(n):
        eng.draft_tree(want=False)
        if B == 1:
            committed += len(eng.verify())
        else:
            committed += sum(len(t) for t in eng.verify_batch())
    return committed


def mean_ctx(eng, B: int, prompt_len: int) -> float:
    """Mean context length over the lanes: prompt + committed tokens - 1 (the
    last committed token is the next cycle's root)."""
    return sum(len(eng.committed(b)) for b in range(B)) / B + prompt_len - 1


def timed_window(eng, w: dict, B: int, seed: int, steps: int, warmup: int, roof: bool):
    """Prefill every lane (lane b: prompt seed + b), advance to the config's
    mean context less half the timed cycles, warm up, then time `steps`
    cycles between stream synchronisations. Returns the window's figures."""
    import torch
    import synth
    P = w["prompt_len"]
    for b in range(B):
        eng.prefill(synth.prompt(seed + b, P, w["vocab"]), lane=b)
    target = P + w["gen"] / 2.0 - steps / 2.0
    while mean_ctx(eng, B, P) + warmup < target:
        # tau ~ 1: one cycle moves the context by one token, so advance in
        # batches of the remaining distance, re-reading the context after each
        run_cycles(eng, B, max(1, min(64, int(target - warmup - mean_ctx(eng, B, P)))))
    if roof:
        eng.profile(["gemm"], every=ROOF_EVERY)
    run_cycles(eng, B, warmup)
    torch.cuda.synchronize()
    if roof:
        eng.profile(["gemm"], every=ROOF_EVERY)   # reset the counters; keep the class enabled
    ctx0 = mean_ctx(eng, B, P)
    t0 = time.perf_counter()
    committed = run_cycles(eng, B, steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    g = eng.profile_read()["gemm"] if roof else None
    if roof:
        eng.profile(False)
    ctx1 = mean_ctx(eng, B, P)
    return dict(seed=seed, seconds=dt, committed=committed, ctx0=ctx0, ctx1=ctx1, gemm=g,
                cycles_per_s=steps / dt)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--profile-cycles", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--seeds", type=int, default=3,
                    help="prompt seeds seed .. seed + seeds - 1, each timed over --steps cycles")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra figures (whole generation, plain decode, second config)")
    ap.add_argument("--extra-config", default="c3",
                    help="second workload timed as an extra key (batch 1, greedy); '' for none")
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

    w = synth.workloads.get(args.config)
    if args.temperature > 0:
        w.update(temperature=args.temperature, seed=args.seed)
    B = args.batch
    w["batch"] = B
    P = w["prompt_len"]
    # advance to mid-generation, warm-up, timed, profile and speedup-model cycles
    cycles_needed = w["gen"] // 2 + args.warmup + args.steps + max(0, args.profile_cycles) + 8
    eng = make_engine(w, cycles_needed, args.prefill_chunk)
    prompt = synth.prompt(args.seed, P, w["vocab"])
    # the first prefill loads the kernels; the second (it restarts the
    # sequence) is the timed one
    eng.prefill(prompt)
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    eng.prefill(prompt)
    torch.cuda.synchronize()
    prefill_ms = (time.perf_counter() - tp0) * 1e3
    print(f"# {args.config}: prefill {P} tokens in {prefill_ms:.1f} ms, {B} lane(s)",
          file=sys.stderr, flush=True)

    windows = []
    for k in range(max(1, args.seeds)):
        win = timed_window(eng, w, B, args.seed + k, args.steps, args.warmup, roof=True)
        windows.append(win)
        print(f"# seed {win['seed']}: {args.steps} cycles at ctx {win['ctx0']:.0f}..{win['ctx1']:.0f} "
              f"in {win['seconds'] * 1e3:.1f} ms ({win['cycles_per_s']:.2f} cycles/s)",
              file=sys.stderr, flush=True)
    order = sorted(range(len(windows)), key=lambda i: windows[i]["cycles_per_s"])
    med = windows[order[len(order) // 2]]
    dt, committed, g = med["seconds"], med["committed"], med["gemm"]
    avg_ctx = 0.5 * (med["ctx0"] + med["ctx1"])
    bytes_cycle = cycle_bytes(w, int(avg_ctx), B)
    kv_planes = 4 if w["dtype"] == "bf16" else None
    traffic_cycle = cycle_bytes(w, int(avg_ctx), B, kv_elem_bytes=kv_planes)
    gemm_gbps = g["bytes"] / (g["ms"] * 1e-3) / 1e9 if g["ms"] > 0 else 0.0
    mv = B * (1 + w["budget"])    # target rows of a verify pass
    mt = (mv + 15) // 16 if mv <= 80 else 4

    # breakdown window after the timed region: events around every launch
    prof = None
    if args.profile_cycles > 0:
        eng.profile(True)
        run_cycles(eng, B, args.profile_cycles)
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
    roof_key = (f"proj_kernel<{'bf16' if w['dtype'] == 'bf16' else 'f32'}, MT={mt}, EPI_PART> "
                f"M={mv} {args.config}")
    traffic = stored_traffic(roof_key)
    cps = [x["cycles_per_s"] for x in windows]
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
        "data": "synthetic (seeded N(0,0.02)-like weights, uniform random prompts)",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}"
                               + (f"; sampling at temperature {args.temperature}" if args.temperature > 0 else "")
                               + (f"; {B} sequences per cycle" if B > 1 else ""),
                   "global_batch": B, "seq_len": int(avg_ctx), "parallelism": "none (1 GPU)"},
        "cycles_per_s": round(cycles_s, 3),
        "tau": round(tau, 4),
        "seeds": {"timed_seed": med["seed"], "median_cycles_per_s": round(cps[order[len(order) // 2]], 3),
                  "min_cycles_per_s": round(min(cps), 3), "max_cycles_per_s": round(max(cps), 3),
                  "per_seed": [{"seed": x["seed"], "cycles_per_s": round(x["cycles_per_s"], 3),
                                "tokens_per_s": round(x["committed"] / x["seconds"], 3),
                                "ctx": [round(x["ctx0"]), round(x["ctx1"])]} for x in windows]},
        "cycle_hbm": {"bytes_per_cycle": bytes_cycle,
                      "achieved_GBps": round(bytes_cycle * cycles_s / 1e9, 1),
                      "frac": round(bytes_cycle * cycles_s / 1e9 / PEAK_GBPS, 4),
                      "kv_bytes_per_element": 2 if w["dtype"] == "bf16" else 4,
                      "bytes_per_cycle_with_kv_planes": traffic_cycle},
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

    if not args.no_extra and B == 1 and args.temperature == 0:
        # the whole generation of the config (prompt seed `seed`): eagle_generate
        # times its cycle loop on the device (prefill excluded)
        toks, st = eng.generate(prompt, w["gen"])
        out["generation"] = {"tokens": len(toks), "cycles": st["cycles"],
                             "cycle_loop_s": round(st["seconds"], 5),
                             "tokens_per_s": round((st["committed"] - 1) / st["seconds"], 3),
                             "cycles_per_s": round(st["cycles"] / st["seconds"], 3),
                             "ctx": [P, P + len(toks)]}
        eng.close()
        del eng
        torch.cuda.empty_cache()
        # plain greedy decode on the GPU (budget 0: one token per target pass,
        # no drafting) over the same generation: the in-house speedup baseline
        wp = dict(w, tree="dynamic", static=None, budget=0)
        pe = make_engine(wp, 8)
        toks_p, stp = pe.generate(prompt, w["gen"])
        plain_tps = (stp["committed"] - 1) / stp["seconds"]
        mid = P + w["gen"] // 2
        out["plain_decode"] = {"tokens_per_s": round(plain_tps, 3),
                               "bytes_per_token": plain_token_bytes(w, mid),
                               "frac": round(plain_token_bytes(w, mid) * plain_tps / 1e9 / PEAK_GBPS, 4),
                               "same_tokens": toks_p == toks,
                               "speculative_over_plain": round(out["generation"]["tokens_per_s"] / plain_tps, 4)}
        pe.close()
        del pe
        torch.cuda.empty_cache()
        if args.extra_config and args.extra_config != args.config:
            wx = synth.workloads.get(args.extra_config)
            xe = make_engine(wx, wx["gen"] // 2 + args.warmup + args.steps + 8)
            xwin = timed_window(xe, wx, 1, args.seed, args.steps, args.warmup, roof=False)
            xctx = 0.5 * (xwin["ctx0"] + xwin["ctx1"])
            xb = cycle_bytes(wx, int(xctx))
            out["extra_config"] = {"workload": f"{args.extra_config}: {WORKLOAD_TEXT[args.extra_config]}",
                                   "seed": args.seed, "steps": args.steps,
                                   "cycles_per_s": round(xwin["cycles_per_s"], 3),
                                   "tokens_per_s": round(xwin["committed"] / xwin["seconds"], 3),
                                   "ctx": [round(xwin["ctx0"]), round(xwin["ctx1"])],
                                   "bytes_per_cycle": xb,
                                   "frac": round(xb * xwin["cycles_per_s"] / 1e9 / PEAK_GBPS, 4)}
            xe.close()
            del xe
            torch.cuda.empty_cache()
    else:
        eng.close()
    if not args.no_cpu:
        # sequences are independent: the oracle's tokens/s is the same at any batch
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
