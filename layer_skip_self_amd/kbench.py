"""Kernel-level timing of the decode path at a model shape.

Projections: a teacher-forced verify of M rows (M - 1 forced draft tokens
after the pending one) after a prefill of ctx tokens, repeated; every launch of the
chosen projection family with exactly M rows is timed with HIP events on
the engine stream (``Engine.profile_kernel``), and its algorithmic bytes
(weights + activation rows read + rows written) give the achieved rate.
Run under ``rocprofv3 --kernel-trace --stats`` the same command gives the
tracer's per-kernel durations (attention and merge included), and under
``rocprofv3 --pmc FETCH_SIZE`` / ``WRITE_SIZE`` the HBM traffic;
``--calib-copy`` adds one 1 GiB device copy whose counters scale them.

    python -m layer_skip_self_amd.kbench --shape llama3_8b --ctx 1536 \\
        --rows 1,9 --kernel vector,mfma

Weights and prompt are the seeded synthetic ones of ``lss_synth``.
"""
import argparse
import json
import time

import numpy as np

PEAK_GBS = 8000.0


def _verify_loop(eng, M, reps, prompt, max_seq):
    """reps teacher-forced verifies of M rows, each after the previous
    round's accept (the context grows by the emitted tokens, at least one
    per round; the prompt is prefilled again when the cache is full)."""
    drafts = [int(t) for t in (np.arange(M - 1) * 7919 + 13) % 1000 + 100]
    for _ in range(reps):
        if eng.seq_len + M + 1 > max_seq:
            eng.prefill(prompt)
        eng.verify(drafts=drafts)
        eng.accept()


def main(argv=None):
    import torch
    import lss_synth
    from . import Engine

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shape", default="llama3_8b", choices=sorted(lss_synth.SHAPES))
    ap.add_argument("--ctx", type=int, default=1536, help="prompt length before the first verify")
    ap.add_argument("--rows", default="1,9", help="verify rows M (comma list)")
    ap.add_argument("--kernel", default="vector,mfma", help="decode kernels (vector, mfma; comma list)")
    ap.add_argument("--epilogues", default="qkv,resid,gate_up,lm_head")
    ap.add_argument("--reps", type=int, default=6)
    ap.add_argument("--kv", default="f32", choices=("f32", "bf16"))
    ap.add_argument("--calib-copy", action="store_true", help="one 1 GiB device-to-device copy first")
    ap.add_argument("--json", action="store_true", help="one JSON object per line instead of a table")
    args = ap.parse_args(argv)

    sh = lss_synth.SHAPES[args.shape]
    rows = [int(x) for x in args.rows.split(",")]
    kinds = args.kernel.split(",")
    epis = args.epilogues.split(",")
    if not torch.cuda.is_available():
        raise SystemExit("kbench needs a GPU")
    dev = torch.device("cuda:0")
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = lss_synth.make_weights(sh, device=dev)
    max_rows = max(16, max(rows))
    max_seq = min(4096, args.ctx + 256)
    eng = Engine(sh, w, max_seq=max_seq, max_rows=max_rows, kv_dtype=args.kv)
    prompt = lss_synth.make_prompt(sh, args.ctx)
    t_start = time.perf_counter()
    eng.prefill(prompt)
    for kind in kinds:
        eng.set_decode_kernel(kind)
        for M in rows:
            out = {"shape": args.shape, "ctx": args.ctx, "kernel": kind, "rows": M}
            for epi in epis:
                eng.profile_kernel(epi, rows=M)
                _verify_loop(eng, M, args.reps, prompt, max_seq)
                ms, n, b = eng.profile_read()
                eng.profile_kernel(epi, enable=False)
                us = 1e3 * ms / n if n else float("nan")
                gbs = (b / n) / (us * 1e-6) / 1e9 if n else float("nan")
                out[epi] = {"avg_us": round(us, 3), "launches": n, "bytes_per_launch": b // max(n, 1),
                            "gbs": round(gbs, 1), "frac": round(gbs / PEAK_GBS, 4)}
            if args.json:
                print(json.dumps(out), flush=True)
            else:
                cells = [f"{e} {out[e]['avg_us']:8.2f} us {out[e]['gbs']:7.0f} GB/s" for e in epis]
                print(f"{kind:6s} M={M:2d}: " + " | ".join(cells), flush=True)
    eng.close()
    if not args.json:
        print(f"done in {time.perf_counter() - t_start:.1f} s", flush=True)


if __name__ == "__main__":
    main()
