#!/usr/bin/env python3
"""Throughput of the looped nGPT forward pass on one MI355X, with roofline fractions.

Workload (seeded synthetic weights and prompts, nothing downloaded): the ~4B
looped nGPT (d=3072, 24/8 heads of 128, SwiGLU 8192, vocab 131072, 8/20/8
blocks, 3:1 sliding-window(4096):full attention), bf16, last-loop KV cache.

A step is one decode step at batch 1 (every block application of the input
stack, k passes of the recurrent core, the output stack, LM head and argmax)
with a 2560-token prompt already in the cache; the headline value is decode
tok/s at k=2. The breakdown adds decode at k=1/2/4 and the 2048-token prefill at
k=1/2/4 with their roofline fractions. The roofline entry is the dominant
decode kernel: its algorithmic bytes per launch over its average launch time,
from HIP events recorded around every launch on the stream the library uses
(an instrumented pass of the same decode steps, after the timed region).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--prompt", type=int, default=2560)
    p.add_argument("--prefill-len", type=int, default=2048)
    p.add_argument("--k", type=int, default=2, help="loop count of the headline decode value")
    p.add_argument("--loops", default="1,2,4")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-batched", action="store_true")
    p.add_argument("--no-mx", action="store_true", help="skip the MXFP8-weight decode measurement")
    p.add_argument("--no-spec", action="store_true", help="skip the self-speculative decoding measurement")
    p.add_argument("--no-sampling", action="store_true", help="skip the top-p sampler measurement")
    p.add_argument("--no-decode", action="store_true",
                   help="prefill only (for profiling): the JSON value is then the prefill rate at --k")
    p.add_argument("--batched-steps", type=int, default=16)
    p.add_argument("--no-long", action="store_true", help="skip the 131072-token prompt at k=4 with decode and "
                   "self-speculative decoding at that context (about 25 s)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run one device copy of 256 MiB first (counter calibration under rocprofv3)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the forward pass would shard by sequence, with no exchange between GPUs).", file=sys.stderr)
        sys.exit(2)
    import torch

    from looped_ngpt_language_amd import dory, synth

    loops = [int(x) for x in args.loops.split(",")]
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] calibration copy: 268435456 bytes read, 268435456 bytes written")
    shape = synth.DORY4B
    t0 = time.time()
    w = synth.make_weights(shape, seed=0)
    log(f"[bench] weights drawn in {time.time() - t0:.1f}s")
    prompt = synth.prompt_tokens(shape, max(args.prompt, args.prefill_len))
    max_len = args.prompt + max(args.warmup + args.steps, 48 + 4 + 1) + 32   # decode steps, or the speculative run
    t0 = time.time()
    # created in per-loop mode so the pool also holds a per-loop sequence (96 cache slots per page)
    m = dory.Model(shape, w, kv_mode="per_loop", max_loops=4, max_seqs=1, max_model_len=max_len,
                   max_tokens=max(args.prompt, args.prefill_len), device="cuda:0")
    m.set_kv_mode("last_loop")
    torch.cuda.synchronize()
    log(f"[bench] model uploaded in {time.time() - t0:.1f}s; workspace {m.ws_bytes / 2**30:.2f} GiB, "
        f"KV pool {m.kv_bytes / 2**30:.2f} GiB")
    st = m.stream
    res = {"decode": {}, "prefill": {}}

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ---------------------------------------------------------------- prefill
    if not args.no_prefill:
        toks = torch.from_numpy(prompt[:args.prefill_len]).to("cuda:0")
        logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda:0")
        for k in loops:
            m.set_loops(k)
            m.prefill(0, toks, 1, logits=logits)
            m.release(0)
            torch.cuda.synchronize()
            m.timing(reset=True)
            reps = 3
            e0, e1 = ev(), ev()
            e0.record(st)
            for _ in range(reps):
                m.prefill(0, toks, 1, logits=logits)
                m.release(0)
            e1.record(st)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            tim = m.timing(reset=True)
            flops = sum(v["flops"] for v in tim.values()) / reps
            tfs = flops / (ms * 1e-3) / 1e12
            res["prefill"][k] = {"tokens": args.prefill_len, "ms": ms, "tok_s": args.prefill_len / (ms * 1e-3),
                                 "tflop": flops / 1e12, "tflop_s": tfs, "mfma_frac": tfs / BF16_PEAK_TFLOPS}
            log(f"[bench] prefill T={args.prefill_len} k={k}: {ms:.2f} ms  {args.prefill_len / (ms * 1e-3):,.0f} tok/s  "
                f"{tfs:.1f} TFLOP/s ({100 * tfs / BF16_PEAK_TFLOPS:.1f}% of MFMA peak)")
            # instrumented pass: one prefill with an event pair around every launch
            m.set_timing(True)
            m.prefill(0, toks, 1, logits=logits)
            m.release(0)
            tim = m.timing(reset=True)
            m.set_timing(False)
            kern = {}
            for name, v in sorted(tim.items(), key=lambda x: -x[1]["ms"]):
                if v["timed_launches"]:
                    tf = v["flops"] / (v["ms"] * 1e-3) / 1e12 if v["ms"] else 0.0
                    kern[name] = {"ms": v["ms"], "tflop_s": tf, "launches": v["launches"]}
                    log(f"         {name:22s} {v['launches']:5d} launches  {v['ms']:8.2f} ms  {tf:7.1f} TFLOP/s")
            res["prefill"][k]["kernels"] = kern

    if args.no_decode:
        head = res["prefill"].get(args.k) or next(iter(res["prefill"].values()))
        dom_name, dom = max(head["kernels"].items(), key=lambda x: x[1]["ms"])
        print(json.dumps({
            "metric": f"prefill tok/s ({args.prefill_len}-token prompt, k={args.k})", "value": round(head["tok_s"], 1),
            "unit": "tok/s", "n_gpus": 1, "steps": 3, "warmup": 1, "ms_per_step": round(head["ms"], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded random weights and uniform-random prompt ids)",
            "config": {"workload": f"looped nGPT ~4B prefill, {args.prefill_len} tokens, k={args.k}"},
            "roofline": {"bound": "mfma", "kernel": dom_name, "achieved": round(dom["tflop_s"], 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(dom["tflop_s"] / BF16_PEAK_TFLOPS, 4), "traffic": None},
            "cpu_baseline": None}), flush=True)
        return

    # ---------------------------------------------------------------- decode
    ptoks = torch.from_numpy(prompt[:args.prompt]).to("cuda:0")
    ids = [torch.empty(1, dtype=torch.int32, device="cuda:0") for _ in range(2)]
    first = torch.empty(1, dtype=torch.int32, device="cuda:0")
    plog = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda:0")
    def decode_run(k, mode, m=m):
        m.set_kv_mode(mode)
        m.set_loops(k)
        _, pid = m.prefill(0, ptoks, 1, logits=plog)
        first.copy_(pid)
        cur = first
        for i in range(args.warmup):
            m.decode([0], cur, logits=None, out_ids=ids[i % 2])
            cur = ids[i % 2]
        torch.cuda.synchronize()
        m.timing(reset=True)
        e0, e1 = ev(), ev()
        e0.record(st)
        for i in range(args.steps):
            m.decode([0], cur, logits=None, out_ids=ids[i % 2])
            cur = ids[i % 2]
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        alg = m.timing(reset=True)
        step_bytes = sum(v["bytes"] for v in alg.values()) / args.steps
        # instrumented pass: same decode steps, an event pair around every launch
        n_inst = min(args.steps, 20)
        m.set_timing(True)
        for i in range(n_inst):
            m.decode([0], cur, logits=None, out_ids=ids[i % 2])
            cur = ids[i % 2]
        tim = m.timing(reset=True)
        m.set_timing(False)
        m.release(0)
        roles = {}
        for name, v in tim.items():
            if v["timed_launches"]:
                avg_ms = v["ms"] / v["timed_launches"]
                per_launch = v["bytes"] / v["launches"]
                roles[name] = {"launches_per_step": v["launches"] / n_inst, "avg_us": 1e3 * avg_ms,
                               "ms_per_step": v["ms"] / n_inst, "bytes_per_launch": per_launch,
                               "GBs": per_launch / (avg_ms * 1e-3) / 1e9}
        gbs = step_bytes / (ms * 1e-3) / 1e9
        log(f"[bench] decode bs1 k={k} {mode} ctx {args.prompt}: {ms:.3f} ms/step  {1e3 / ms:.1f} tok/s  "
            f"{step_bytes / 1e9:.2f} GB/step -> {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak)")
        for name, r in sorted(roles.items(), key=lambda x: -x[1]["ms_per_step"]):
            log(f"         {name:22s} {r['launches_per_step']:6.1f}/step  avg {r['avg_us']:8.2f} us  "
                f"{r['ms_per_step']:7.3f} ms/step  {r['GBs']:7.0f} GB/s")
        return {"ms_per_step": ms, "tok_s": 1e3 / ms, "bytes_per_step": step_bytes, "GBs": gbs,
                "hbm_frac": gbs / HBM_PEAK_GBS, "kernels": roles}

    for k in loops:
        res["decode"][k] = decode_run(k, "last_loop")
    res["decode_per_loop"] = {args.k: decode_run(args.k, "per_loop")}
    if not args.no_mx:
        # the same steps streaming MXFP8 copies of the weights (OCP MX, E4M3 + E8M0 per 32)
        mm = dory.Model(shape, None, kv_mode="last_loop", max_loops=4, max_seqs=1, max_model_len=max_len,
                        max_tokens=max(args.prompt, args.prefill_len), device="cuda:0", share_weights_from=m,
                        gemv_weights="mxfp8")
        log(f"[bench] MXFP8 context: workspace {mm.ws_bytes / 2**30:.2f} GiB")
        res["decode_mx"] = {k: decode_run(k, "last_loop", mm) for k in loops}
        mm.close()
        del mm

    if not args.no_sampling:
        res["sampling"] = bench_sampling(shape, args)
    if not args.no_spec:
        res["spec"] = bench_spec(m, ptoks, plog, res["decode"].get(4), args)

    if not args.no_batched:
        res["batched"] = bench_batched(m, shape, args, ev)
    if not args.no_long:
        res["long"] = bench_long(m, shape, args, ev)

    head = res["decode"].get(args.k) or next(iter(res["decode"].values()))
    dom_name, dom = max(head["kernels"].items(), key=lambda x: x[1]["ms_per_step"])
    roofline = {"bound": "hbm", "kernel": dom_name, "achieved": round(dom["GBs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(dom["GBs"] / HBM_PEAK_GBS, 4), "avg_us": round(dom["avg_us"], 3),
                "algorithmic_bytes_per_launch": round(dom["bytes_per_launch"]),
                "traffic": measured_traffic(dom_name)}

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(shape, w, prompt, args.k)

    out = {
        "metric": "decode tok/s (bs1, bs128) + prefill tok/s at k=1/2/4; % of HBM/MFMA roofline",
        "value": round(head["tok_s"], 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random weights and uniform-random prompt ids)",
        "config": {"workload": f"looped nGPT ~4B (d=3072, 8/20/8 blocks) decode, batch 1, k={args.k}, "
                               f"last-loop KV, {args.prompt}-token prompt in cache",
                   "global_batch": 1, "seq_len": args.prompt, "loops": args.k, "kv_mode": "last_loop"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "breakdown": {
            "decode_bs1": {str(k): {"tok_s": round(v["tok_s"], 2), "ms_per_step": round(v["ms_per_step"], 4),
                                    "GB_per_step": round(v["bytes_per_step"] / 1e9, 3),
                                    "hbm_frac": round(v["hbm_frac"], 4)} for k, v in res["decode"].items()},
            "decode_bs1_mxfp8": {str(k): {"tok_s": round(v["tok_s"], 2), "ms_per_step": round(v["ms_per_step"], 4),
                                          "GB_per_step": round(v["bytes_per_step"] / 1e9, 3),
                                          "hbm_frac": round(v["hbm_frac"], 4)}
                                 for k, v in res.get("decode_mx", {}).items()},
            "decode_bs1_per_loop": {str(k): {"tok_s": round(v["tok_s"], 2), "ms_per_step": round(v["ms_per_step"], 4),
                                             "GB_per_step": round(v["bytes_per_step"] / 1e9, 3),
                                             "hbm_frac": round(v["hbm_frac"], 4)}
                                    for k, v in res.get("decode_per_loop", {}).items()},
            "prefill": {str(k): {"tokens": v["tokens"], "tok_s": round(v["tok_s"], 1), "ms": round(v["ms"], 3),
                                 "tflop_s": round(v["tflop_s"], 1), "mfma_frac": round(v["mfma_frac"], 4)}
                        for k, v in res["prefill"].items()},
            "sampling_top_p": res.get("sampling"),
            "self_speculative_k1x4_k4": res.get("spec"),
            "decode_bs128_k2": res.get("batched"),
            "long_context_k4": res.get("long"),
        },
    }
    print(json.dumps(out), flush=True)


def bench_spec(m, ptoks, plog, plain4, args):
    """Self-speculative greedy decoding at batch 1 on the same context (k = 1 draft of 4 tokens,
    k = 4 verify, last-loop KV), with and without reuse of the draft's input-stack output,
    loop-1 state and cache in the verify pass; tok/s over 48 produced ids (host round trip per
    verify included), against plain k = 4 decode."""
    import torch
    out = {"plain_k4_tok_s": round(plain4["tok_s"], 2) if plain4 else None}
    m.set_kv_mode("last_loop")
    for reuse in (False, True):
        m.set_loops(4)
        _, pid = m.prefill(0, ptoks, 1, logits=plog)
        first = int(pid[0].item())
        m.spec_decode(0, first, 8, gamma=4, k_draft=1, k_verify=4, reuse=reuse)    # warm-up
        m.release(0)
        _, pid = m.prefill(0, ptoks, 1, logits=plog)
        first = int(pid[0].item())
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        got = m.spec_decode(0, first, 48, gamma=4, k_draft=1, k_verify=4, reuse=reuse)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        m.release(0)
        key = "reuse" if reuse else "no_reuse"
        out[f"{key}_tok_s"] = round(len(got) / dt, 2)
        out[f"{key}_tokens"] = int(len(got))
        log(f"[bench] self-speculative k=1 x4 / k=4, {'with' if reuse else 'without'} reuse: {len(got)} ids in "
            f"{dt:.3f} s -> {len(got) / dt:.1f} tok/s"
            + (f" ({len(got) / dt / plain4['tok_s']:.2f}x plain k=4)" if plain4 else ""))
    return out


def bench_sampling(shape, args):
    """Temperature 1.0 / top-p 0.95 draws (dory_sample) over the vocabulary, for 1 and 128 rows of
    seeded normal logits: microseconds per call (one workgroup per row; every pass over a row
    reads it from L2)."""
    import torch

    from looped_ngpt_language_amd import dory
    out = {}
    g = torch.Generator(device="cuda:0").manual_seed(3)
    for rows in (1, 128):
        logits = torch.randn(rows, shape.vocab, device="cuda:0", generator=g) * 2
        us = torch.rand(rows, device="cuda:0", generator=g)
        for _ in range(3):
            dory.sample(logits, us, 1.0, 0.95)
        n = 20
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            dory.sample(logits, us, 1.0, 0.95)
        b.record()
        torch.cuda.synchronize()
        t_us = a.elapsed_time(b) * 1e3 / n
        out[str(rows)] = {"us_per_call": round(t_us, 2), "rows": rows, "vocab": shape.vocab}
        log(f"[bench] top-p sampling, {rows} row(s) x {shape.vocab}: {t_us:.1f} us per call")
    return out


def bench_batched(m1, shape, args, ev):
    """Serving-style batched decode: 128 sequences with prompt lengths uniform in [256, 4096]
    (seeded), k = 2, one decode call per step for all sequences; per-loop vs last-loop KV."""
    import torch

    from looped_ngpt_language_amd import dory, synth
    n_seq, k, steps = 128, 2, args.batched_steps
    lens = synth.batch_prompt_lengths(n_seq, 256, 4096, seed=2)
    prompts = synth.batch_prompts(shape, lens, seed=1)
    extra = 2 + steps + 16
    kv_tokens = int(sum(((int(n) + extra + 15) // 16) * 16 for n in lens))
    mb = dory.Model(shape, None, kv_mode="per_loop", max_loops=k, max_seqs=n_seq, max_model_len=4096 + extra,
                    max_tokens=4096, kv_tokens=kv_tokens, device="cuda:0", share_weights_from=m1)
    out = {"sequences": n_seq, "loops": k, "prompt_tokens": int(sum(lens)), "steps": steps}
    st = mb.stream
    for mode in ("per_loop", "last_loop"):
        mb.set_kv_mode(mode)
        mb.set_loops(k)
        t0 = time.time()
        firsts = []
        for s_, p in enumerate(prompts):
            _, ids = mb.prefill(s_, torch.from_numpy(p).to("cuda:0"), 1)
            firsts.append(ids)
        cur = torch.cat(firsts)
        torch.cuda.synchronize()
        t_pf = time.time() - t0
        sids = list(range(n_seq))
        nxt = [torch.empty(n_seq, dtype=torch.int32, device="cuda:0") for _ in range(2)]
        for i in range(2):
            mb.decode(sids, cur, logits=None, out_ids=nxt[i % 2])
            cur = nxt[i % 2]
        torch.cuda.synchronize()
        mb.timing(reset=True)
        e0, e1 = ev(), ev()
        e0.record(st)
        for i in range(steps):
            mb.decode(sids, cur, logits=None, out_ids=nxt[i % 2])
            cur = nxt[i % 2]
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tim = mb.timing(reset=True)
        step_bytes = sum(v["bytes"] for v in tim.values()) / steps
        gbs = step_bytes / (ms * 1e-3) / 1e9
        kvb = mb.kv_bytes_in_use()
        # instrumented pass: a few more steps with an event pair around every launch
        n_inst = 4
        mb.set_timing(True)
        for i in range(n_inst):
            mb.decode(sids, cur, logits=None, out_ids=nxt[i % 2])
            cur = nxt[i % 2]
        inst = mb.timing(reset=True)
        mb.set_timing(False)
        roles = {}
        for name, v in inst.items():
            if v["timed_launches"]:
                avg_ms = v["ms"] / v["timed_launches"]
                per_launch = v["bytes"] / v["launches"]
                roles[name] = {"avg_us": round(1e3 * avg_ms, 2), "ms_per_step": round(v["ms"] / n_inst, 3),
                               "GBs": round(per_launch / (avg_ms * 1e-3) / 1e9, 1)}
        out[mode] = {"tok_s": round(n_seq * 1e3 / ms, 1), "ms_per_step": round(ms, 3),
                     "GB_per_step": round(step_bytes / 1e9, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "kv_bytes_in_use": kvb, "prefill_s": round(t_pf, 1), "kernels": roles}
        log(f"[bench] decode bs{n_seq} k={k} {mode}: {ms:.2f} ms/step  {n_seq * 1e3 / ms:,.0f} tok/s  "
            f"{step_bytes / 1e9:.1f} GB/step -> {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak); "
            f"KV in use {kvb / 1e9:.1f} GB; prefill of {int(sum(lens))} tokens took {t_pf:.1f} s")
        for name, r in sorted(roles.items(), key=lambda x: -x[1]["ms_per_step"]):
            log(f"         {name:22s} avg {r['avg_us']:9.2f} us  {r['ms_per_step']:7.3f} ms/step  {r['GBs']:7.0f} GB/s")
        for s_ in sids:
            mb.release(s_)
    mb.close()
    return out


def bench_long(m1, shape, args, ev):
    """131072-token uniform-random prompt at k = 4, last-loop KV (full layers attend over the
    whole prompt, sliding-window layers over 4096), prefilled in 8192-token chunks with
    sliding-window page recycling, then decode at batch 1 and self-speculative decoding (k = 1
    draft of 4 tokens, k = 4 verification) on the same weights. Reports the KV pool with and
    without recycling and the bytes in use."""
    import torch

    from looped_ngpt_language_amd import dory, synth
    T, k, n_dec, n_spec, chunk = 131072, 4, 16, 64, 8192
    mb = dory.Model(shape, None, kv_mode="last_loop", max_loops=4, max_seqs=1, max_model_len=T + 256,
                    max_tokens=chunk, device="cuda:0", share_weights_from=m1, swa_recycle=True)
    plain_bytes, _ = dory.query_sizes(dory.make_config(shape, max_seqs=1, max_model_len=T + 256, max_loops=4,
                                                       max_tokens=chunk), "last_loop", T + 256)
    mb.set_loops(k)
    st = mb.stream
    prompt = torch.from_numpy(synth.prompt_tokens(shape, T, seed=1)).to("cuda:0")
    mb.timing(reset=True)
    e0, e1 = ev(), ev()
    e0.record(st)
    for i in range(0, T, chunk):
        _, ids = mb.prefill(0, prompt[i:i + chunk], 1)
    e1.record(st)
    torch.cuda.synchronize()
    pf_ms = e0.elapsed_time(e1)
    tim = mb.timing(reset=True)
    flops = sum(v["flops"] for v in tim.values())
    tfs = flops / (pf_ms * 1e-3) / 1e12
    log(f"[bench] long prefill T={T} k={k} ({chunk}-token chunks): {pf_ms / 1e3:.2f} s  "
        f"{T / (pf_ms * 1e-3):,.0f} tok/s  {tfs:.1f} TFLOP/s ({100 * tfs / BF16_PEAK_TFLOPS:.1f}% of MFMA peak)")
    kv_after_prefill = mb.kv_bytes_in_use()
    base_len = mb.seq_len(0)
    cur = ids.clone()
    nxt = [torch.empty(1, dtype=torch.int32, device="cuda:0") for _ in range(2)]
    e0.record(st)
    for i in range(n_dec):
        mb.decode([0], cur, logits=None, out_ids=nxt[i % 2])
        cur = nxt[i % 2]
    e1.record(st)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / n_dec
    tim = mb.timing(reset=True)
    step_bytes = sum(v["bytes"] for v in tim.values()) / n_dec
    gbs = step_bytes / (dec_ms * 1e-3) / 1e9
    log(f"[bench] long decode ctx {T} k={k}: {dec_ms:.2f} ms/step  {1e3 / dec_ms:.1f} tok/s  "
        f"{step_bytes / 1e9:.1f} GB/step -> {gbs:.0f} GB/s")
    # instrumented pass: a few more steps with an event pair around every launch
    n_inst = 4
    mb.set_timing(True)
    for i in range(n_inst):
        mb.decode([0], cur, logits=None, out_ids=nxt[i % 2])
        cur = nxt[i % 2]
    inst = mb.timing(reset=True)
    mb.set_timing(False)
    long_roles = {}
    for name, v in sorted(inst.items(), key=lambda x: -x[1]["ms"]):
        if v["timed_launches"]:
            avg_ms = v["ms"] / v["timed_launches"]
            long_roles[name] = {"avg_us": round(1e3 * avg_ms, 2), "ms_per_step": round(v["ms"] / n_inst, 3),
                                "GBs": round(v["bytes"] / v["launches"] / (avg_ms * 1e-3) / 1e9, 1)}
            log(f"         {name:22s} avg {1e3 * avg_ms:9.2f} us  {v['ms'] / n_inst:7.3f} ms/step  "
                f"{long_roles[name]['GBs']:7.0f} GB/s")
    kv_decode = mb.kv_bytes_in_use()
    log(f"[bench] KV with sliding-window page recycling: pool {mb.kv_bytes / 1e9:.2f} GB (without: "
        f"{plain_bytes / 1e9:.2f} GB); in use {kv_after_prefill / 1e9:.2f} GB after the prompt, "
        f"{kv_decode / 1e9:.2f} GB while decoding")
    last = int(ids[0].item())
    spec = {}
    for reuse in (False, True):
        mb.truncate(0, base_len)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        got = mb.spec_decode(0, last, n_spec, gamma=4, k_draft=1, k_verify=4, reuse=reuse)
        torch.cuda.synchronize()
        sp_s = time.perf_counter() - t0
        spec[reuse] = (len(got), len(got) / sp_s)
        log(f"[bench] self-speculative (k=1 draft x4, k=4 verify, {'with' if reuse else 'without'} reuse): "
            f"{len(got)} tokens in {sp_s:.2f} s -> {len(got) / sp_s:.1f} tok/s "
            f"({len(got) / sp_s * dec_ms / 1e3:.2f}x plain k=4 decode)")
    got, spec_tok_s = [0] * spec[False][0], spec[False][1]
    mb_kv = mb.kv_bytes
    mb.close()
    return {"prompt_tokens": T, "loops": k, "prefill_s": round(pf_ms / 1e3, 3),
            "prefill_tok_s": round(T / (pf_ms * 1e-3), 1), "prefill_tflop_s": round(tfs, 1),
            "prefill_mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4), "decode_tok_s": round(1e3 / dec_ms, 2), "decode_kernels": long_roles,
            "decode_GB_per_step": round(step_bytes / 1e9, 2), "decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "spec_tok_s": round(spec_tok_s, 2), "spec_speedup": round(spec_tok_s * dec_ms / 1e3, 3),
            "spec_tokens": int(len(got)), "spec_reuse_tok_s": round(spec[True][1], 2),
            "spec_reuse_speedup": round(spec[True][1] * dec_ms / 1e3, 3), "kv_pool_GB": round(mb_kv / 1e9, 3),
            "kv_pool_without_recycling_GB": round(plain_bytes / 1e9, 3),
            "kv_in_use_after_prompt_GB": round(kv_after_prefill / 1e9, 3),
            "kv_in_use_decoding_GB": round(kv_decode / 1e9, 3)}


def measured_traffic(role):
    """HBM bytes per launch of the kernel behind `role` from the committed rocprofv3 counter passes
    (profiles/traffic.json), reported only while the kernel's source file is unchanged since then."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(role)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source_file"])
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if digest != rec["source_sha256"]:
        return None
    return {"fetch_bytes": rec["fetch_bytes"], "write_bytes": rec["write_bytes"],
            "bytes": rec["fetch_bytes"] + rec["write_bytes"], "kernel": rec["kernel"], "profile": rec["profile"]}


def cpu_baseline(shape, w, prompt, k, budget_s=12.0):
    """The oracle as it stands, on the host cores: a 16-token prompt, then decode steps for ~budget_s."""
    from threadpoolctl import threadpool_info

    from oracle import OracleModel
    om = OracleModel(shape, w, "last_loop", k)
    t0 = time.perf_counter()
    om.prefill(0, prompt[:16], 1)
    t_pf = time.perf_counter() - t0
    log(f"[bench] oracle prefill of 16 tokens at k={k}: {t_pf:.2f} s")
    n = 0
    tok = 1
    t0 = time.perf_counter()
    while n < 2 or (time.perf_counter() - t0 < budget_s and n < 200):
        _, ids = om.decode([0], [tok])
        tok = int(ids[0])
        n += 1
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    log(f"[bench] oracle decode: {n} steps, {dt / n:.3f} s/token on {threads} threads")
    return {"value": round(n / dt, 4), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "prefill_tok_s": round(16 / t_pf, 3),
            "sample": f"{n} decode steps ({dt:.1f} s) at batch 1, k={k}, last-loop KV, after a 16-token prompt "
                      f"(fp64 numpy oracle, same ~4B weights); cores = BLAS threads"}


if __name__ == "__main__":
    main()
