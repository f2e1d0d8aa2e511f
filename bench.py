#!/usr/bin/env python3
"""Benchmark of batch-1 self-speculative greedy decoding on one MI355X.

Default workload (the Llama-3-8B-shaped configuration): 32 layers, d 4096,
32 query / 8 KV heads, FFN 14336, vocab 128256, bf16 weights drawn N(0, 0.02)
with residual-branch output projections x0.1; a 1024-token uniform-random
prompt; 512 generated tokens; the CLaSp DP skips 16 layers and re-runs every
32 verify rounds; draft exit threshold 0.7; at most 8 drafts per round.

One step = one full generation (prefill + layer selection + draft / verify /
accept rounds) of that workload; ``value`` = generated tokens / step time.
The same process also times the GPU's own greedy decoding (speedup), checks
that both produce identical tokens, times the draft gate/up GEMV launches
with HIP events on the engine stream (roofline), and times the CPU oracle
on a bounded sample (cpu_baseline).  Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0

WORKLOADS = {
    "llama3_8b": dict(shape="llama3_8b", prompt=1024, gen=512,
                      policy={"mode": "dp", "k_max": 8, "n_skip": 16, "interval": 32, "exit_tau": 0.7},
                      desc="Llama-3-8B shape, prompt 1024, 512 generated, CLaSp DP skip 16 every 32 "
                           "rounds, exit threshold 0.7, K <= 8"),
    # Workloads whose verifies carry many rows (K = 6 or 8, token trees) run
    # the full-model rows on the MFMA decode GEMM (one weight pass for all
    # rows, measured faster there); the 8B headline verifies about 2 rows per
    # round, where the vector-ALU GEMV is faster.
    "llama2_7b": dict(shape="llama2_7b", prompt=512, gen=256,
                      policy={"mode": "static", "k_max": 6, "skip": tuple(range(1, 32, 2)),
                              "decode_kernel": "mfma_verify"},
                      desc="Llama-2-7B shape, prompt 512, 256 generated, static skip of layers 1,3,..,31, K 6"),
    "tiny": dict(shape="tiny", prompt=32, gen=64, policy={"mode": "static", "k_max": 4, "skip": (1, 2)},
                 desc="4-layer float32 model, prompt 32, 64 generated, skip {1,2}, K 4"),
    # Llama-3-70B shape on one GPU (~141 GB of bf16 weights), the CLaSp DP
    # skipping 44 of 80 layers, re-run every 8, 32 or 128 verify rounds.
    "llama3_70b": dict(shape="llama3_70b", prompt=512, gen=256,
                       policy=[{"mode": "dp", "k_max": 8, "n_skip": 44, "interval": iv, "decode_kernel": "mfma_verify"}
                               for iv in (8, 32, 128)],
                       desc="Llama-3-70B shape, prompt 512, 256 generated, CLaSp DP skip 44 of 80, interval "
                            "8 / 32 / 128, K 8"),
    # Supplementary, not the headline configuration: the Llama-3-8B shape with
    # 16 planted identity layers (wo = w_down = 0, seeded set) and the LM head
    # scaled x10, so the layers the DP can skip are truly redundant and the
    # draft's top-1 probability can pass the exit threshold.  It shows the
    # engine's speculative ceiling when drafts are right.
    "llama3_8b_planted": dict(shape="llama3_8b", prompt=1024, gen=512, planted=16, head_scale=10.0,
                              policy={"mode": "dp", "k_max": 8, "n_skip": 16, "interval": 32, "exit_tau": 0.7},
                              desc="supplementary: Llama-3-8B shape with 16 planted identity layers and a x10 "
                                   "LM head, prompt 1024, 512 generated, CLaSp DP skip 16 every 32 rounds, exit "
                                   "threshold 0.7, K <= 8"),
    # CAS-Spec three-level cascade on the Llama-3-8B shape.  Levels as (layers
    # skipped in total, of which the last `exit` by early exit, int8
    # activations), fast -> precise: L1 skips 70% of 32 layers (4 by early
    # exit, 18 chosen by the DP), L2 skips 30% (DP) with int8 activations, L3
    # runs all layers with int8 activations.  DyTC routing with at most 8
    # drafts per round and a latency model fitted on this engine.
    # Speculative sampling at temperature 1 (the acceptance rule that keeps
    # the full model's distribution) with the headline draft policy; the AR
    # leg samples at the same temperature and seed.
    "llama3_8b_sampling": dict(shape="llama3_8b", prompt=1024, gen=512,
                               policy={"mode": "dp", "k_max": 8, "n_skip": 16, "interval": 32, "exit_tau": 0.7,
                                       "temperature": 1.0, "seed": 2025},
                               desc="Llama-3-8B shape, prompt 1024, 512 generated, speculative sampling at "
                                    "temperature 1, CLaSp DP skip 16 every 32 rounds, exit threshold 0.7, K <= 8"),
    # The headline policy with a W8A8 draft: the executed layers' projections
    # read an int8 copy of the weights (per-row scales) with int8
    # activations, halving the bytes a draft token streams.
    "llama3_8b_w8a8": dict(shape="llama3_8b", prompt=1024, gen=512,
                           policy={"mode": "dp", "k_max": 8, "n_skip": 16, "interval": 32, "exit_tau": 0.7,
                                   "quant": 2},
                           desc="Llama-3-8B shape, prompt 1024, 512 generated, CLaSp DP skip 16 every 32 rounds, "
                                "exit threshold 0.7, K <= 8, W8A8 draft (int8 weight copy + int8 activations)"),
    # Token trees of width 4 (depth 1) with the headline DP draft: the draft's
    # 4 most likely next tokens verified in one pass with a tree mask.
    "llama3_8b_tree": dict(shape="llama3_8b", prompt=1024, gen=512,
                           policy={"mode": "dp", "k_max": 1, "n_skip": 16, "interval": 32, "tree_width": 4,
                                   "decode_kernel": "mfma_verify"},
                           desc="Llama-3-8B shape, prompt 1024, 512 generated, CLaSp DP skip 16 every 32 rounds, "
                                "token tree of width 4 and depth 1 per round"),
    # Deeper trees: 3 branches of 4 tokens each (12 nodes + the pending
    # token: 13 verify rows, one MFMA weight pass).
    "llama3_8b_tree_deep": dict(shape="llama3_8b", prompt=1024, gen=512,
                                policy={"mode": "dp", "k_max": 1, "n_skip": 16, "interval": 32, "tree_width": 3,
                                        "tree_depth": 4, "decode_kernel": "mfma_verify"},
                                desc="Llama-3-8B shape, prompt 1024, 512 generated, CLaSp DP skip 16 every 32 "
                                     "rounds, token tree of width 3 and depth 4 per round"),
    # Batch > 1: eight independent sequences (seeded prompts of 1024 tokens,
    # 256 generated each) decoded together, every sequence with the headline
    # policy (its own CLaSp DP), or with one static skip set that lets all
    # eight share each draft pass.  The AR leg decodes the same eight
    # sequences batched.
    "llama3_8b_batch8": dict(shape="llama3_8b", prompt=1024, gen=256, batch=8,
                             policy={"mode": "dp", "k_max": 7, "n_skip": 16, "interval": 32, "exit_tau": 0.7,
                                     "decode_kernel": "mfma_verify"},
                             desc="Llama-3-8B shape, 8 sequences x (prompt 1024, 256 generated), each with "
                                  "CLaSp DP skip 16 every 32 rounds, exit threshold 0.7, K <= 7"),
    "llama3_8b_batch8_static": dict(shape="llama3_8b", prompt=1024, gen=256, batch=8,
                                    policy={"mode": "static", "k_max": 4, "skip": tuple(range(1, 32, 2)),
                                            "decode_kernel": "mfma"},
                                    desc="Llama-3-8B shape, 8 sequences x (prompt 1024, 256 generated), static "
                                         "skip of layers 1,3,..,31 shared by all, K 4"),
    # The same levels routed into token trees of width <= 4 (the tree
    # router prices each pass by its row count, factors measured on this
    # engine's verify), verify rows on the MFMA GEMM.
    "cascade_tree_8b": dict(shape="llama3_8b", prompt=(128, 512, 2048), gen=256,
                            policy={"mode": "cascade", "k_max": 8, "interval": 32, "tree_width": 4,
                                    "levels": [(22, 4, False), (10, 0, True), (0, 0, True)],
                                    "decode_kernel": "mfma_verify"},
                            desc="Llama-3-8B shape, CAS-Spec cascade levels as cascade_8b routed into token "
                                 "trees (width <= 4, DyTC tree router with measured row costs), K <= 8, "
                                 "prompts 128, 512, 2048 with 256 generated each"),
    "cascade_8b": dict(shape="llama3_8b", prompt=(128, 512, 2048), gen=256,
                       policy={"mode": "cascade", "k_max": 8, "interval": 32,
                               "levels": [(22, 4, False), (10, 0, True), (0, 0, True)]},
                       desc="Llama-3-8B shape, CAS-Spec cascade L1 (22 skipped: 4 early exit + 18 DP) / "
                            "L2 (10 skipped by DP, int8) / L3 (int8), DyTC routing, K <= 8, prompts 128, 512, "
                            "2048 with 256 generated each"),
}


def progress(msg):
    """One line on stderr as a piece of the benchmark finishes (stdout keeps
    the single JSON result line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(shape, w_gpu, prompt, policy, n_tokens, n_prompt):
    """Time the CPU oracle (float32, as it stands) on a bounded sample."""
    import numpy as np
    import lss_synth
    import oracle
    # BLAS threads: every CPU this process may run on, capped by the CPU
    # share the environment grants one GPU job (OMP_NUM_THREADS, 16 on the
    # GPU hosts); the host's total is reported beside it
    host_cpus = os.cpu_count()
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = host_cpus
    share = int(os.environ.get("OMP_NUM_THREADS") or allowed)
    threads = max(1, min(allowed, share))
    try:
        from threadpoolctl import threadpool_limits, threadpool_info
        limiter = threadpool_limits(limits=threads)
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        limiter, cores = None, threads
    progress("CPU oracle baseline: widening the weights")
    w_host = [(n, t.to("cpu")) for n, t in w_gpu]
    model = oracle.OracleModel(shape, lss_synth.LazyF32(w_host), dtype=np.float32, cache_layers=True)
    for l in range(shape.n_layers):           # widen every weight once (setup, not timed)
        model.layer(l)
    model._get("lm_head"); model._get("final_norm")
    pol = oracle.Policy(K=policy.get("k_max", 4), skip=tuple(policy.get("skip", ())),
                        dp_skip=policy.get("n_skip") if policy["mode"] == "dp" else None,
                        interval=policy.get("interval", 32), tau=policy.get("exit_tau", 0.0),
                        quant=int(policy.get("quant", 0)),
                        cascade=list(policy["levels"]) if policy["mode"] == "cascade" else None,
                        latency_beta=tuple(policy.get("beta", (1.0, 0.0, 1.0))),
                        temperature=float(policy.get("temperature", 0.0)), seed=int(policy.get("seed", 0)),
                        tree_width=int(policy.get("tree_width", 0)), tree_depth=int(policy.get("tree_depth", 1)),
                        row_cost=tuple(policy["row_cost"]) if policy.get("row_cost") else None)
    sample = np.asarray(prompt[:n_prompt])
    t0 = time.perf_counter()
    toks, recs = oracle.speculative_generate(model, sample, n_tokens, pol)
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "host_cpus": host_cpus, "affinity_cpus": allowed, "blas_threads": int(cores),
            "sample": f"oracle float32 speculative decoding (same policy) of {len(toks)} tokens after a "
                      f"{n_prompt}-token prompt of the same workload; prefill + layer selection + "
                      f"{len(recs)} rounds in {dt:.1f} s; BLAS threads {cores} = the CPUs this job may "
                      f"use (affinity {allowed}, job share {share}) of the host's {host_cpus}"}


GEMV_SECTIONS = ("scalars", "projection input format", "projections: shared definitions",
                 "decode GEMV (vector ALU)")
# the int8 GEMV also takes the activation rule (small kernels) and the load
# helper of the bf16 GEMV
GEMV8_SECTIONS = ("scalars", "projection input format", "small kernels", "projections: shared definitions",
                  "decode GEMV (vector ALU)", "int8 decode GEMV (W8A8 draft)")
TRAFFIC_RECORDS = (("draft_gemv_llama3_8b.md", GEMV_SECTIONS),
                   ("draft_gemv8_llama3_8b_w8a8.md", GEMV8_SECTIONS))


def gemv_source_hash(sections=GEMV_SECTIONS):
    """sha256 of kernel-source sections of lss_kernels.h (the named sections,
    in the given order) a recorded kernel is built from."""
    import hashlib
    src = os.path.join(ROOT, "layer_skip_self_amd", "csrc", "lss_kernels.h")
    mark = "// " + "-" * 64 + " "
    found, name = {}, None
    for line in open(src):
        if line.startswith(mark):
            name = line[len(mark):].strip()
        if name is not None:
            found[name] = found.get(name, "") + line
    h = hashlib.sha256()
    for n in sections:
        h.update(found[n].encode())
    return h.hexdigest()


def recorded_traffic(bytes_per_launch):
    """HBM bytes per launch of the timed draft gate/up kernel measured with
    rocprofv3 counters (the records in profiles/), or None when no record
    matches: its kernel's source sections changed since the counters were
    taken, or the launch is not the recorded one (another shape or kernel)."""
    for name, sections in TRAFFIC_RECORDS:
        rec = os.path.join(ROOT, "profiles", name)
        try:
            fields = {}
            for line in open(rec):
                if ":" in line and line.startswith("- "):
                    k, v = line[2:].split(":", 1)
                    fields[k.strip()] = v.strip().strip("`")
            if fields.get("kernel source sha256") != gemv_source_hash(sections):
                continue
            if int(fields["algorithmic bytes per launch"].split()[0]) != int(bytes_per_launch):
                continue
            return int(fields["traffic bytes per launch"])
        except (OSError, KeyError, ValueError):
            continue
    return None


def bench_batch(args, wl, shape, dev):
    """Batch > 1: wl["batch"] sequences decoded together (lss_generate_batch);
    value = generated tokens of all sequences per second."""
    import torch
    import lss_synth
    from layer_skip_self_amd import Engine
    S, G = wl["batch"], (wl["gen"] if args.gen is None else args.gen)
    weights = lss_synth.make_weights(shape, device=dev)
    prompts = [lss_synth.make_prompt(shape, wl["prompt"], seed=shape.prompt_seed + i) for i in range(S)]
    eng = Engine(shape, weights, max_seq=wl["prompt"] + G + 33, max_rows=64, max_seqs=S)
    pol = dict(wl["policy"])
    if args.decode_kernel:
        pol["decode_kernel"] = args.decode_kernel
    pol.setdefault("decode_kernel", "vector")

    def run(p):
        torch.cuda.synchronize()
        t = time.perf_counter()
        toks, st = eng.generate_batch(prompts, G, p)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t
        progress(f"{p['mode']} batch run: {len(prompts)} sequences x {G} tokens in {dt:.2f} s")
        return toks, st, dt

    for _ in range(args.warmup):
        run(pol)
    eng.profile_kernel("gate_up", rows=0)
    spec_t, toks, stats = 0.0, None, None
    for _ in range(args.steps):
        toks, stats, dt = run(pol)
        spec_t += dt
    k_ms, k_n, k_bytes = eng.profile_read()
    eng.profile_kernel("gate_up", enable=False)
    ar_pol = {"mode": "ar", "decode_kernel": pol["decode_kernel"]}
    ar_t, ar_toks = 0.0, None
    if args.ar_steps > 0:
        run(ar_pol)
        for _ in range(args.ar_steps):
            ar_toks, _, dt = run(ar_pol)
            ar_t += dt
    step_s = spec_t / args.steps
    value = S * G / step_s
    ar_value = S * G * args.ar_steps / ar_t if args.ar_steps > 0 else None
    rounds = sum(st["rounds"] for st in stats)
    accepted = sum(st["accepted"] for st in stats)
    drafted = sum(st["drafted"] for st in stats)
    avg_us = 1e3 * k_ms / max(k_n, 1)
    bpl = k_bytes / max(k_n, 1)
    achieved = bpl / (avg_us * 1e-6) / 1e9 if k_n else None
    out = {
        "metric": "gen tokens/s @bs1 (Llama-3-8B shape), speedup vs AR, draft GEMV HBM GB/s",
        "value": round(value, 3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * step_s, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": shape.dtype, "data": "synthetic (seeded random-init weights and uniform-random prompts)",
        "config": {"workload": wl["desc"], "global_batch": S, "seq_len": wl["prompt"] + G,
                   "parallelism": "none (1 GPU)"},
        "speedup_vs_ar": round(value / ar_value, 4) if ar_value else None,
        "ar_tokens_per_s": round(ar_value, 3) if ar_value else None,
        "lossless": toks == ar_toks if ar_toks is not None else None,
        "decoding": "greedy", "decode_kernel": pol["decode_kernel"],
        "mean_accepted": round(accepted / max(rounds, 1), 4),
        "drafted_per_round": round(drafted / max(rounds, 1), 4),
        "rounds": rounds, "dp_runs": sum(st["dp_runs"] for st in stats),
        "roofline": {
            "bound": "hbm",
            "kernel": "gate/up projection + SwiGLU, every launch of the step (draft and verify rows of all "
                      "sequences)",
            "achieved": round(achieved, 1) if achieved else None, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4) if achieved else None, "traffic": None,
            "bytes_per_launch": int(bpl), "avg_launch_us": round(avg_us, 3), "launches": k_n,
        },
    }
    if not args.no_cpu_baseline:
        # the oracle decodes a batch as independent sequences, one after the
        # other: its rate is the single-sequence rate of the same policy
        cb = cpu_baseline(shape, weights, prompts[0], pol, args.cpu_tokens, min(args.cpu_prompt, wl["prompt"]))
        cb["sample"] += "; the oracle decodes a batch's sequences one after another, so this is its batch rate too"
        out["cpu_baseline"] = cb
    eng.close()
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llama3_8b", choices=sorted(WORKLOADS))
    ap.add_argument("--ar-steps", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--cpu-prompt", type=int, default=64)
    ap.add_argument("--gen", type=int, default=None, help="override the generated length (profiling runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--decode-kernel", choices=("vector", "mfma", "mfma_verify"), default=None,
                    help="override the workload's decode-row kernel (A/B runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the engine runs on one GPU; --gpus must be 1 "
                                   "(multi-GPU sharding is a design note only)"}))
        sys.exit(2)

    import numpy as np
    import torch
    import lss_synth
    from layer_skip_self_amd import Engine

    wl = WORKLOADS[args.workload]
    shape = lss_synth.SHAPES[wl["shape"]]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if wl.get("batch"):
        return bench_batch(args, wl, shape, dev)
    planted = ()
    if wl.get("planted"):
        rng = np.random.default_rng(shape.weight_seed)
        planted = tuple(sorted(rng.choice(shape.n_layers, wl["planted"], replace=False).tolist()))
    weights = lss_synth.make_weights(shape, device=dev, planted_identity=planted,
                                     head_scale=wl.get("head_scale", 1.0))
    lens = wl["prompt"] if isinstance(wl["prompt"], tuple) else (wl["prompt"],)
    # one seeded prompt per length (the first uses the shape's prompt seed)
    prompts = [lss_synth.make_prompt(shape, n, seed=shape.prompt_seed + i) for i, n in enumerate(lens)]
    G = wl["gen"] if args.gen is None else args.gen
    max_seq = max(lens) + G + 33
    progress(f"weights of {wl['shape']} ready")
    eng = Engine(shape, weights, max_seq=max_seq, max_rows=64)
    policies = [dict(p) for p in (wl["policy"] if isinstance(wl["policy"], list) else [wl["policy"]])]
    for p in policies:
        if args.decode_kernel:
            p["decode_kernel"] = args.decode_kernel
        p.setdefault("decode_kernel", "vector")
    w8 = any(p.get("quant") == 2 or any(lv[2] == 2 for lv in p.get("levels", [])) for p in policies)
    if w8:
        eng.attach_w8()
    latency = None
    for policy in policies:
        if policy["mode"] != "cascade":
            continue
        # DyTC latency model of this engine: timed one-token drafts at the
        # levels' depths and at full depth (the verify), seq_len 128 .. 2048
        L = shape.n_layers
        depths = sorted({L - lv[0] for lv in policy["levels"]} | {L})
        cal_lens = tuple(n for n in (128, 512, 1024, 2048) if n + 40 <= max_seq)
        cal_prompt = lss_synth.make_prompt(shape, max(cal_lens), seed=shape.prompt_seed + 99)
        eng.set_decode_kernel(policy["decode_kernel"])
        beta, samples, err = eng.calibrate_latency(cal_prompt, cal_lens, depths)
        policy["beta"] = beta
        latency = {"beta": [float(b) for b in beta], "seq_lens": list(cal_lens), "depths": depths,
                   "samples": len(samples), "max_rel_err": round(err, 4)}
        if policy.get("tree_width"):
            rc = eng.calibrate_row_cost(cal_prompt[:min(cal_lens[-1], 1024)])
            policy["row_cost"] = rc
            latency["row_cost"] = [round(x, 4) for x in rc]
    runs = [(pol, i) for pol in policies for i in range(len(prompts))]   # (policy, prompt index)

    def run(pol, prompt):
        torch.cuda.synchronize()
        t = time.perf_counter()
        toks, st = eng.generate(prompt, G, pol)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t
        progress(f"{pol['mode']} run: prompt {len(prompt)}, {G} tokens in {dt:.2f} s")
        return toks, st, dt

    for _ in range(args.warmup):
        for pol, i in runs:
            run(pol, prompts[i])
    prof_kernel = "gate_up_int8" if w8 else "gate_up"      # the draft's gate/up kernel
    eng.profile_kernel(prof_kernel, rows=1)
    spec_t = [0.0] * len(runs)
    stats, spec_toks = [None] * len(runs), [None] * len(runs)
    torch.cuda.synchronize()
    t_all = time.perf_counter()
    for _ in range(args.steps):
        for j, (pol, i) in enumerate(runs):
            toks, st, dt = run(pol, prompts[i])
            spec_t[j] += dt
            stats[j] = st
            spec_toks[j] = toks
    torch.cuda.synchronize()
    t_all = time.perf_counter() - t_all
    k_ms, k_n, k_bytes = eng.profile_read()
    eng.profile_kernel(prof_kernel, enable=False)

    # the AR leg decodes the same way (greedy, or sampling at the same
    # temperature and seed)
    ar_pol = {"mode": "ar", "temperature": policies[0].get("temperature", 0.0), "seed": policies[0].get("seed", 0),
              "decode_kernel": policies[0]["decode_kernel"]}
    sampling = ar_pol["temperature"] > 0
    ar_t, ar_toks = [0.0] * len(prompts), [None] * len(prompts)
    if args.ar_steps > 0:
        for pr in prompts:
            run(ar_pol, pr)
    for _ in range(args.ar_steps):
        for i, pr in enumerate(prompts):
            ar_toks[i], _, dt = run(ar_pol, pr)
            ar_t[i] += dt
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    prefill_s = []
    for pr in prompts:
        pre = []
        for _ in range(3):
            torch.cuda.synchronize()
            t = time.perf_counter()
            eng.prefill(pr)
            torch.cuda.synchronize()
            pre.append(time.perf_counter() - t)
        prefill_s.append(min(pre))

    n_r = len(runs)
    step_s = t_all / args.steps
    value = n_r * G / step_s
    ar_step = sum(ar_t[i] for _, i in runs) / args.ar_steps if args.ar_steps > 0 else None
    ar_value = n_r * G / ar_step if ar_step else None
    rounds = sum(st["rounds"] for st in stats)
    accepted = sum(st["accepted"] for st in stats)
    drafted = sum(st["drafted"] for st in stats)
    emitted = sum(st["emitted"] for st in stats)
    dp_runs = sum(st["dp_runs"] for st in stats)
    avg_launch_us = 1e3 * k_ms / max(k_n, 1)
    bytes_per_launch = k_bytes / max(k_n, 1)
    achieved = bytes_per_launch / (avg_launch_us * 1e-6) / 1e9 if k_n else None
    per_run = []
    for j, (pol, i) in enumerate(runs):
        st = stats[j]
        sp = G * args.steps / spec_t[j]
        ar = G * args.ar_steps / ar_t[i] if args.ar_steps > 0 else None
        item = {"prompt": lens[i], "tokens_per_s": round(sp, 3),
                "ar_tokens_per_s": round(ar, 3) if ar else None,
                "speedup_vs_ar": round(sp / ar, 4) if ar else None,
                "lossless": spec_toks[j] == ar_toks[i] if args.ar_steps > 0 and not sampling else None,
                "mean_accepted": round(st["accepted"] / max(st["rounds"], 1), 4),
                "drafted_per_round": round(st["drafted"] / max(st["rounds"], 1), 4),
                "dp_runs": st["dp_runs"], "prefill_ms": round(1e3 * prefill_s[i], 3)}
        if len(policies) > 1:
            item["interval"] = pol.get("interval")
        per_run.append(item)
    prefill_total = sum(prefill_s[i] for _, i in runs)
    out = {
        "metric": "gen tokens/s @bs1 (Llama-3-8B shape), speedup vs AR, draft GEMV HBM GB/s",
        "value": round(value, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * step_s, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded random-init weights and uniform-random prompt)"
                + (f"; planted identity layers {list(planted)}" if planted else ""),
        "config": {"workload": wl["desc"], "global_batch": 1, "seq_len": max(lens) + G,
                   "parallelism": "none (1 GPU)"},
        "speedup_vs_ar": round(value / ar_value, 4) if ar_value else None,
        "ar_tokens_per_s": round(ar_value, 3) if ar_value else None,
        "lossless": all(r["lossless"] for r in per_run) if args.ar_steps > 0 and not sampling else None,
        "decoding": (f"speculative sampling, temperature {ar_pol['temperature']}, seed {ar_pol['seed']}"
                     if sampling else "greedy"),
        "decode_kernel": policies[0]["decode_kernel"],
        "mean_accepted": round(accepted / max(rounds, 1), 4),
        "tokens_per_round": round((emitted - n_r) / max(rounds, 1), 4),
        "drafted_per_round": round(drafted / max(rounds, 1), 4),
        "rounds": rounds,
        "dp_runs": dp_runs,
        "prefill_ms": round(1e3 * prefill_total, 3),
        "decode_tokens_per_s": round(n_r * (G - 1) / (step_s - prefill_total), 3),
        "draft_gemv_gbps": round(achieved, 1) if achieved else None,
        "roofline": {
            "bound": "hbm",
            "kernel": (f"k_gemv8<{shape.dtype},SWIGLU>: draft gate/up projection on the int8 weight copy + "
                       "SwiGLU, 1 row" if w8 else
                       "k_vgemm<SWIGLU,16>: draft gate/up projection (MFMA) + SwiGLU, 1 row"
                       if policies[0]["decode_kernel"] == "mfma" else
                       f"k_gemv<{shape.dtype},1,1,SWIGLU,8>: draft gate/up projection + SwiGLU, 1 row"),
            "achieved": round(achieved, 1) if achieved else None,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4) if achieved else None,
            "traffic": recorded_traffic(bytes_per_launch) if policies[0]["decode_kernel"] != "mfma" or w8 else None,
            "bytes_per_launch": int(bytes_per_launch),
            "avg_launch_us": round(avg_launch_us, 3),
            "launches": k_n,
        },
    }
    if n_r > 1:
        out["runs"] = per_run
    if latency is not None:
        out["latency_model"] = latency
    if not args.no_cpu_baseline:
        if shape.total_params() * 4 > 64e9:
            # the float32 oracle of this shape does not fit a bounded host sample
            out["cpu_baseline"] = {"value": None, "unit": "tokens/s", "cores": None, "kind": "oracle",
                                   "sample": "not run: the float32 oracle needs "
                                             f"{shape.total_params() * 4 / 1e9:.0f} GB of host memory"}
        else:
            out["cpu_baseline"] = cpu_baseline(shape, weights, prompts[0], policies[0], args.cpu_tokens,
                                               min(args.cpu_prompt, lens[0]))
    eng.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
