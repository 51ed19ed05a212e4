#!/usr/bin/env python3
"""Throughput of the looped nGPT forward pass on one MI355X, with roofline fractions.

Workload (seeded synthetic weights and prompts, nothing downloaded): the ~4B looped nGPT
(d=3072, 24/8 heads of 128, SwiGLU 8192, vocab 131072, 8/20/8 blocks, 3:1 sliding-window
(4096):full attention), bf16.

A step is one decode step at batch 1: every block application of the input stack, k passes of
the recurrent core, the output stack, the LM head and the argmax. The headline value is decode
tok/s at k=2, last-loop KV, over the 2560-token-prompt workload: the prompt is prefilled, then
--steps decode steps (300 by default) are timed from that context. The breakdown covers
  * decode at batch 1, k = 1/2/4, last-loop and per-loop KV: the 2560-token prompt with 300
    decode tokens and the 128-token prompt with 1024 decode tokens;
  * prefill of 2048 tokens (and of the 2560-token prompt) at k = 1/2/4;
  * batched decode of 128 ragged sequences (prompts of 256..4096 tokens), k = 1/2/4, both modes;
  * the 131072-token prompt at k = 4 prefilled as one chunk, decode and self-speculative
    decoding at that context (an 8192-token-chunk prefill is reported separately);
  * the mid-size model (d=1024), 512-token prompt and 128 decode tokens, k = 1/2/4, both modes;
  * MXFP8 decode weights, top-p sampling, self-speculative decoding with its cost breakdown.
Roofline fractions come from the library's algorithmic byte / flop accounting. The `roofline`
entry is the dominant decode kernel: its algorithmic bytes per launch over its average launch
time, from HIP events the dispatches record on the library's stream in an instrumented pass of
the same steps; it also carries the rocprofv3 average of the same kernel from the committed
profile while that kernel's source is unchanged. `gpu_clocks` holds the graphics and memory
clocks amd-smi read every few seconds while the GPU part ran.
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


def _clock_mhz(obj, prefix):
    """Current clocks (MHz) of every clock domain whose name starts with `prefix` ("gfx", "mem")
    in amd-smi's JSON clock report, whatever its nesting."""
    vals = []

    def num(v):
        if isinstance(v, dict):
            v = v.get("value")
        if isinstance(v, (int, float)):
            return float(v)
        if isinstance(v, str):
            try:
                return float(v.split()[0])
            except (ValueError, IndexError):
                return None
        return None

    def walk(o):
        if isinstance(o, dict):
            for k, v in o.items():
                if isinstance(k, str) and k.lower().startswith(prefix) and isinstance(v, dict):
                    c = num(v.get("clk", v.get("cur_clk")))
                    if c is not None:
                        vals.append(c)
                walk(v)
        elif isinstance(o, list):
            for v in o:
                walk(v)

    walk(obj)
    return vals


class ClockSampler:
    """Reads the GPU's current graphics and memory clocks with `amd-smi metric --clock --json`
    every few seconds from a background thread while the benchmark runs (amd-smi reads the
    driver's metrics; it launches no GPU work). Reports the spread of the readings."""

    def __init__(self, period_s=4.0):
        import threading
        self.period_s = period_s
        self.samples = []
        self.error = None
        self.raw = None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        import shutil
        import subprocess
        exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
        r = subprocess.run([exe, "metric", "--clock", "--json"], capture_output=True, text=True, timeout=30)
        if r.returncode != 0:
            raise RuntimeError(f"amd-smi exit {r.returncode}: {r.stderr.strip()[-200:]}")
        try:
            data = json.loads(r.stdout)
        except ValueError:  # warnings printed ahead of the JSON document
            lines = r.stdout.splitlines()
            first = next(i for i, ln in enumerate(lines) if ln.lstrip()[:1] in ("[", "{") and
                         not ln.lstrip().startswith("[W") and not ln.lstrip().startswith("[I"))
            data = json.loads("\n".join(lines[first:]))
        gfx, mem = _clock_mhz(data, "gfx"), _clock_mhz(data, "mem")
        if not gfx:
            self.raw = r.stdout[:600]
            raise RuntimeError("no gfx clock in amd-smi's report")
        return {"t": time.time(), "gfx_mhz": float(np.mean(gfx)), "mem_mhz": float(np.mean(mem)) if mem else None}

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception as e:  # a missing or changed tool must not end the benchmark
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period_s)

    def start(self):
        self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        self._thread.join(timeout=40)
        out = {"source": "amd-smi metric --clock --json", "samples": len(self.samples),
               "period_s": self.period_s}
        if self.samples:
            g = [x["gfx_mhz"] for x in self.samples]
            out.update({"gfx_mhz_min": round(min(g), 1), "gfx_mhz_median": round(float(np.median(g)), 1),
                        "gfx_mhz_max": round(max(g), 1)})
            mems = [x["mem_mhz"] for x in self.samples if x["mem_mhz"] is not None]
            if mems:
                out["mem_mhz_median"] = round(float(np.median(mems)), 1)
        if self.error:
            out["error"] = self.error
        if self.raw:
            out["raw_head"] = self.raw
        return out


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300, help="timed decode steps of the headline workload")
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
    p.add_argument("--no-short-prompt", action="store_true", help="skip the 128-token-prompt, 1024-step decode")
    p.add_argument("--no-per-loop", action="store_true", help="decode grid in last-loop mode only")
    p.add_argument("--no-mid", action="store_true", help="skip the mid-size (d=1024) model")
    p.add_argument("--no-decode", action="store_true",
                   help="prefill only (for profiling): the JSON value is then the prefill rate at --k")
    p.add_argument("--batched-steps", type=int, default=16)
    p.add_argument("--batched-loops", default="1,2,4")
    p.add_argument("--no-long", action="store_true", help="skip the 131072-token prompt at k=4 with decode and "
                   "self-speculative decoding at that context")
    p.add_argument("--no-long-chunked", action="store_true", help="skip the extra 8192-token-chunk long prefill")
    p.add_argument("--no-clocks", action="store_true", help="do not sample the GPU clocks with amd-smi")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run one device copy of 256 MiB first (counter calibration under rocprofv3)")
    return p.parse_args()


def ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def role_table(tim, n_steps):
    roles = {}
    for name, v in tim.items():
        if v["timed_launches"]:
            avg_ms = v["ms"] / v["timed_launches"]
            per_launch = v["bytes"] / v["launches"]
            roles[name] = {"launches_per_step": v["launches"] / n_steps, "avg_us": 1e3 * avg_ms,
                           "ms_per_step": v["ms"] / n_steps, "bytes_per_launch": per_launch,
                           "GBs": per_launch / (avg_ms * 1e-3) / 1e9}
    return roles


def log_roles(roles):
    for name, r in sorted(roles.items(), key=lambda x: -x[1]["ms_per_step"]):
        log(f"         {name:22s} {r['launches_per_step']:6.1f}/step  avg {r['avg_us']:8.2f} us  "
            f"{r['ms_per_step']:7.3f} ms/step  {r['GBs']:7.0f} GB/s")


def decode_run(m, k, mode, ptoks, steps, warmup, tag, n_rows=1):
    """Prefill `ptoks` into sequence 0, run `warmup` decode steps, release; prefill again and
    time `steps` decode steps from the prompt's context (HIP events on the library's stream);
    then an instrumented pass of a few more steps with an event pair around every launch."""
    import torch
    st = m.stream
    m.set_kv_mode(mode)
    m.set_loops(k)
    ids = [torch.empty(1, dtype=torch.int32, device="cuda:0") for _ in range(2)]
    plog = torch.empty((1, m.shape.vocab), dtype=torch.float32, device="cuda:0")
    if warmup:
        _, pid = m.prefill(0, ptoks, 1, logits=plog)
        cur = pid
        for i in range(warmup):
            m.decode([0], cur, logits=None, out_ids=ids[i % 2])
            cur = ids[i % 2]
        m.release(0)
    e0, e1 = ev(), ev()
    e0.record(st)
    _, pid = m.prefill(0, ptoks, 1, logits=plog)
    e1.record(st)
    torch.cuda.synchronize()
    pf_ms = e0.elapsed_time(e1)
    m.timing(reset=True)
    cur = pid
    e0.record(st)
    for i in range(steps):
        m.decode([0], cur, logits=None, out_ids=ids[i % 2])
        cur = ids[i % 2]
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    alg = m.timing(reset=True)
    step_bytes = sum(v["bytes"] for v in alg.values()) / steps
    n_inst = min(steps, 20)
    m.set_timing(True)
    for i in range(n_inst):
        m.decode([0], cur, logits=None, out_ids=ids[i % 2])
        cur = ids[i % 2]
    roles = role_table(m.timing(reset=True), n_inst)
    m.set_timing(False)
    m.release(0)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] {tag} decode bs1 k={k} {mode}, {len(ptoks)}-token prompt, {steps} steps: {ms:.3f} ms/step  "
        f"{1e3 / ms:.1f} tok/s  {step_bytes / 1e9:.2f} GB/step -> {gbs:.0f} GB/s "
        f"({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak); prompt prefill {pf_ms:.2f} ms")
    log_roles(roles)
    return {"ms_per_step": ms, "tok_s": 1e3 / ms, "bytes_per_step": step_bytes, "GBs": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS, "kernels": roles, "prompt_prefill_ms": pf_ms,
            "prompt_tokens": int(len(ptoks)), "steps": steps}


def short(v):
    return {"tok_s": round(v["tok_s"], 2), "ms_per_step": round(v["ms_per_step"], 4),
            "GB_per_step": round(v["bytes_per_step"] / 1e9, 3), "hbm_frac": round(v["hbm_frac"], 4),
            "prompt_tokens": v["prompt_tokens"], "steps": v["steps"],
            "prompt_prefill_tok_s": round(v["prompt_tokens"] / (v["prompt_prefill_ms"] * 1e-3), 1)}


def bench_prefill(m, shape, toks, loops):
    import torch
    out = {}
    st = m.stream
    logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda:0")
    T = len(toks)
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
        out[k] = {"tokens": T, "ms": ms, "tok_s": T / (ms * 1e-3), "tflop": flops / 1e12, "tflop_s": tfs,
                  "mfma_frac": tfs / BF16_PEAK_TFLOPS}
        log(f"[bench] prefill T={T} k={k}: {ms:.2f} ms  {T / (ms * 1e-3):,.0f} tok/s  "
            f"{tfs:.1f} TFLOP/s ({100 * tfs / BF16_PEAK_TFLOPS:.1f}% of MFMA peak)")
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
        out[k]["kernels"] = kern
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the forward pass would shard by sequence, with no exchange between GPUs).", file=sys.stderr)
        sys.exit(2)
    import torch

    from looped_ngpt_language_amd import dory, synth

    t_start = time.time()
    clocks = ClockSampler().start() if not args.no_clocks else None
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
    n_short_steps = 1024
    max_len = max(args.prompt + max(args.warmup, args.steps, 20 + args.steps) + 64,
                  128 + n_short_steps + 64, args.prompt + 48 + 64)
    t0 = time.time()
    # created in per-loop mode so the pool also holds a per-loop sequence (96 cache slots per page)
    m = dory.Model(shape, w, kv_mode="per_loop", max_loops=4, max_seqs=1, max_model_len=max_len,
                   max_tokens=max(args.prompt, args.prefill_len), device="cuda:0")
    m.set_kv_mode("last_loop")
    torch.cuda.synchronize()
    log(f"[bench] model uploaded in {time.time() - t0:.1f}s; workspace {m.ws_bytes / 2**30:.2f} GiB, "
        f"KV pool {m.kv_bytes / 2**30:.2f} GiB")
    res = {"decode": {}, "prefill": {}}

    # ---------------------------------------------------------------- prefill
    if not args.no_prefill:
        res["prefill"] = bench_prefill(m, shape, torch.from_numpy(prompt[:args.prefill_len]).to("cuda:0"), loops)

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

    # ---------------------------------------------------------------- decode, batch 1
    ptoks = torch.from_numpy(prompt[:args.prompt]).to("cuda:0")
    for k in loops:
        res["decode"][k] = decode_run(m, k, "last_loop", ptoks, args.steps, args.warmup, "cfg2a")
    if not args.no_per_loop:
        res["decode_per_loop"] = {k: decode_run(m, k, "per_loop", ptoks, args.steps, args.warmup, "cfg2a")
                                  for k in loops}
    if not args.no_short_prompt:
        stoks = torch.from_numpy(prompt[:128]).to("cuda:0")
        res["decode_short"] = {k: decode_run(m, k, "last_loop", stoks, n_short_steps, args.warmup, "cfg2b")
                               for k in loops}
    m.set_kv_mode("last_loop")
    if not args.no_mx:
        # the same steps streaming MXFP8 / MXFP4 copies of the weights (OCP MX: E4M3 or E2M1
        # elements, E8M0 scale per 32)
        for fmt in ("mxfp8", "mxfp4"):
            mm = dory.Model(shape, None, kv_mode="last_loop", max_loops=4, max_seqs=1, max_model_len=max_len,
                            max_tokens=max(args.prompt, args.prefill_len), device="cuda:0", share_weights_from=m,
                            gemv_weights=fmt)
            log(f"[bench] {fmt} context: workspace {mm.ws_bytes / 2**30:.2f} GiB")
            res[f"decode_{fmt}"] = {k: decode_run(mm, k, "last_loop", ptoks, min(args.steps, 100), args.warmup, fmt)
                                    for k in loops}
            mm.close()
            del mm

    if not args.no_sampling:
        res["sampling"] = bench_sampling(shape)
    if not args.no_spec:
        res["spec"] = bench_spec(m, ptoks, res["decode"].get(4), res["decode"].get(1))

    if not args.no_batched:
        res["batched"] = bench_batched(m, shape, args)
    if not args.no_long:
        res["long"] = bench_long(m, shape, args)
    if not args.no_mid:
        res["mid"] = bench_mid(args)

    head = res["decode"].get(args.k) or next(iter(res["decode"].values()))
    dom_name, dom = max(head["kernels"].items(), key=lambda x: x[1]["ms_per_step"])
    prof = profiled(dom_name)
    roofline = {"bound": "hbm", "kernel": dom_name, "achieved": round(dom["GBs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(dom["GBs"] / HBM_PEAK_GBS, 4), "avg_us": round(dom["avg_us"], 3),
                "algorithmic_bytes_per_launch": round(dom["bytes_per_launch"]),
                "traffic": prof["traffic"] if prof else None}
    if prof:
        achieved_prof = dom["bytes_per_launch"] / (prof["avg_us"] * 1e-6) / 1e9
        roofline.update({"profiled_avg_us": prof["avg_us"], "profiled_achieved": round(achieved_prof, 1),
                         "profiled_frac": round(achieved_prof / HBM_PEAK_GBS, 4), "profile": prof["profile"]})
    step_roofline = {"bound": "hbm", "achieved": round(head["GBs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["hbm_frac"], 4), "bytes_per_step": round(head["bytes_per_step"]),
                     "what": "algorithmic bytes of a whole decode step (recurrent-core weights streamed k times, "
                             "KV reads and writes, LM head) over the step time"}

    # the sampler stops before the host-side oracle timing, which it would disturb
    gpu_clocks = clocks.stop() if clocks else None

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(shape, w, prompt, args.k)

    bd = {
        "decode_bs1": {str(k): short(v) for k, v in res["decode"].items()},
        "decode_bs1_per_loop": {str(k): short(v) for k, v in res.get("decode_per_loop", {}).items()},
        "decode_bs1_128_prompt_1024_steps": {str(k): short(v) for k, v in res.get("decode_short", {}).items()},
        "decode_bs1_mxfp8": {str(k): short(v) for k, v in res.get("decode_mxfp8", {}).items()},
        "decode_bs1_mxfp4": {str(k): short(v) for k, v in res.get("decode_mxfp4", {}).items()},
        "prefill": {str(k): {"tokens": v["tokens"], "tok_s": round(v["tok_s"], 1), "ms": round(v["ms"], 3),
                             "tflop_s": round(v["tflop_s"], 1), "mfma_frac": round(v["mfma_frac"], 4)}
                    for k, v in res["prefill"].items()},
        "decode_bs1_kernels": {n: {kk: round(vv, 3) for kk, vv in r.items()} for n, r in head["kernels"].items()},
        "sampling_top_p": res.get("sampling"),
        "self_speculative_k1x4_k4": res.get("spec"),
        "decode_bs128": res.get("batched"),
        "long_context_k4": res.get("long"),
        "mid_model": res.get("mid"),
        "wall_s": round(time.time() - t_start, 1),
    }
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
                               f"last-loop KV, {args.prompt}-token prompt then {args.steps} decode tokens",
                   "global_batch": 1, "seq_len": args.prompt, "decode_tokens": args.steps, "loops": args.k,
                   "kv_mode": "last_loop"},
        "roofline": roofline,
        "step_roofline": step_roofline,
        "cpu_baseline": cpu,
        "gpu_clocks": gpu_clocks,
        "breakdown": bd,
    }
    print(json.dumps(out), flush=True)


def bench_spec(m, ptoks, plain4, plain1):
    """Self-speculative greedy decoding at batch 1 from the 2560-token context (k = 1 draft of 4
    tokens, k = 4 verify, last-loop KV), with and without reuse of the draft's input-stack
    output, loop-1 state and cache in the verify pass: tok/s over 48 produced ids (one host round
    trip per verify included) against plain k = 4 decode, and its cost model from the library's
    counters: acceptance rate, ids per round, the k = 1 draft step's GPU time and the verify
    chunk's GPU time against a plain k = 4 step."""
    import torch
    out = {"plain_k4_tok_s": round(plain4["tok_s"], 2) if plain4 else None}
    m.set_kv_mode("last_loop")
    plog = torch.empty((1, m.shape.vocab), dtype=torch.float32, device="cuda:0")
    for reuse in (False, True):
        m.set_loops(4)
        _, pid = m.prefill(0, ptoks, 1, logits=plog)
        first = int(pid[0].item())
        m.spec_decode(0, first, 8, gamma=4, k_draft=1, k_verify=4, reuse=reuse)    # warm-up
        m.release(0)
        _, pid = m.prefill(0, ptoks, 1, logits=plog)
        first = int(pid[0].item())
        torch.cuda.synchronize()
        m.spec_stats(reset=True)
        t0 = time.perf_counter()
        got = m.spec_decode(0, first, 48, gamma=4, k_draft=1, k_verify=4, reuse=reuse)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        s = m.spec_stats(reset=True)
        m.release(0)
        key = "reuse" if reuse else "no_reuse"
        draft_step_ms = s["draft_ms"] / max(1, s["drafted"])
        verify_ms = s["verify_ms"] / max(1, s["rounds"])
        entry = {"tok_s": round(len(got) / dt, 2), "tokens": int(len(got)), "rounds": s["rounds"],
                 "acceptance": round(s["accepted"] / max(1, s["drafted"]), 4),
                 "ids_per_round": round(s["produced"] / max(1, s["rounds"]), 3),
                 "draft_step_ms": round(draft_step_ms, 4), "verify_ms": round(verify_ms, 4),
                 "gpu_ms_per_id": round((s["draft_ms"] + s["verify_ms"]) / max(1, s["produced"]), 4)}
        if plain4:
            entry["verify_over_plain_k4_step"] = round(verify_ms / plain4["ms_per_step"], 3)
            entry["speedup_vs_plain_k4"] = round(len(got) / dt / plain4["tok_s"], 3)
        if plain1:
            entry["draft_over_plain_k1_step"] = round(draft_step_ms / plain1["ms_per_step"], 3)
        out[key] = entry
        log(f"[bench] self-speculative k=1 x4 / k=4, {'with' if reuse else 'without'} reuse: {entry}")
    return out


def bench_sampling(shape):
    """Temperature 1.0 / top-p 0.95 draws (dory_sample) over the vocabulary, for 1 and 128 rows of
    seeded normal logits: microseconds per call."""
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
        a, b = ev(), ev()
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


def bench_batched(m1, shape, args):
    """Serving-style batched decode: 128 sequences with prompt lengths uniform in [256, 4096]
    (seeded), one decode call per step for all sequences; per-loop vs last-loop KV at each k
    (per-loop contexts are laid out for exactly k loops, so the KV bytes compare the modes)."""
    import torch

    from looped_ngpt_language_amd import dory, synth
    n_seq, steps = 128, args.batched_steps
    lens = synth.batch_prompt_lengths(n_seq, 256, 4096, seed=2)
    prompts = [torch.from_numpy(p).to("cuda:0") for p in synth.batch_prompts(shape, lens, seed=1)]
    extra = 2 + steps + 8 + 16
    kv_tokens = int(sum(((int(n) + extra + 15) // 16) * 16 for n in lens))
    out = {"sequences": n_seq, "prompt_tokens": int(sum(lens)), "steps": steps}
    for k in [int(x) for x in args.batched_loops.split(",")]:
        for mode in ("last_loop", "per_loop"):
            mb = dory.Model(shape, None, kv_mode=mode, max_loops=k, max_seqs=n_seq, max_model_len=4096 + extra,
                            max_tokens=4096, kv_tokens=kv_tokens, device="cuda:0", share_weights_from=m1)
            st = mb.stream
            mb.set_loops(k)
            t0 = time.time()
            firsts = []
            for s_, p in enumerate(prompts):
                _, ids = mb.prefill(s_, p, 1)
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
            n_inst = 4
            mb.set_timing(True)
            for i in range(n_inst):
                mb.decode(sids, cur, logits=None, out_ids=nxt[i % 2])
                cur = nxt[i % 2]
            roles = role_table(mb.timing(reset=True), n_inst)
            mb.set_timing(False)
            out[f"k{k}_{mode}"] = {
                "tok_s": round(n_seq * 1e3 / ms, 1), "ms_per_step": round(ms, 3),
                "GB_per_step": round(step_bytes / 1e9, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "kv_bytes_in_use": kvb, "kv_pool_bytes": mb.kv_bytes, "prefill_s": round(t_pf, 1),
                "kernels": {n: {"avg_us": round(r["avg_us"], 2), "ms_per_step": round(r["ms_per_step"], 3),
                                "GBs": round(r["GBs"], 1)} for n, r in roles.items()}}
            log(f"[bench] decode bs{n_seq} k={k} {mode}: {ms:.2f} ms/step  {n_seq * 1e3 / ms:,.0f} tok/s  "
                f"{step_bytes / 1e9:.1f} GB/step -> {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak); "
                f"KV in use {kvb / 1e9:.1f} GB; prefill of {int(sum(lens))} tokens took {t_pf:.1f} s")
            if k == 2 and mode == "last_loop":
                log_roles(roles)
            for s_ in sids:
                mb.release(s_)
            mb.close()
            del mb
            torch.cuda.empty_cache()
    return out


def bench_long(m1, shape, args):
    """The 131072-token uniform-random prompt at k = 4, last-loop KV (full layers attend over the
    whole prompt, sliding-window layers over 4096), prefilled as one chunk with sliding-window
    page recycling on, then decode at batch 1 and self-speculative decoding (k = 1 draft of 4
    tokens, k = 4 verification) at that context. Also, separately labelled, the same prompt
    prefilled in 8192-token chunks (under last-loop KV a different computation: the chunks'
    earlier-loop queries read later loops' keys of earlier chunks). Reports the KV pool with and
    without recycling and the bytes in use."""
    import torch

    from looped_ngpt_language_amd import dory, synth
    T, k, n_dec, n_spec, chunk = 131072, 4, 16, 64, 8192
    mb = dory.Model(shape, None, kv_mode="last_loop", max_loops=4, max_seqs=1, max_model_len=T + 256,
                    max_tokens=T, device="cuda:0", share_weights_from=m1, swa_recycle=True)
    plain_bytes, _ = dory.query_sizes(dory.make_config(shape, max_seqs=1, max_model_len=T + 256, max_loops=4,
                                                       max_tokens=T), "last_loop", T + 256)
    log(f"[bench] long-context context: workspace {mb.ws_bytes / 2**30:.2f} GiB, KV pool {mb.kv_bytes / 2**30:.2f} GiB")
    mb.set_loops(k)
    st = mb.stream
    prompt = torch.from_numpy(synth.prompt_tokens(shape, T, seed=1)).to("cuda:0")
    out = {"prompt_tokens": T, "loops": k}

    def prefill(chunk_len):
        mb.timing(reset=True)
        e0, e1 = ev(), ev()
        e0.record(st)
        for i in range(0, T, chunk_len):
            _, ids = mb.prefill(0, prompt[i:i + chunk_len], 1)
        e1.record(st)
        torch.cuda.synchronize()
        pf_ms = e0.elapsed_time(e1)
        tim = mb.timing(reset=True)
        flops = sum(v["flops"] for v in tim.values())
        tfs = flops / (pf_ms * 1e-3) / 1e12
        log(f"[bench] long prefill T={T} k={k} ({chunk_len}-token chunks): {pf_ms / 1e3:.2f} s  "
            f"{T / (pf_ms * 1e-3):,.0f} tok/s  {tfs:.1f} TFLOP/s ({100 * tfs / BF16_PEAK_TFLOPS:.1f}% of MFMA peak)")
        return ids, {"prefill_s": round(pf_ms / 1e3, 3), "prefill_tok_s": round(T / (pf_ms * 1e-3), 1),
                     "prefill_tflop_s": round(tfs, 1), "prefill_mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4)}

    if not args.no_long_chunked:
        _, out["prefill_8192_token_chunks"] = prefill(chunk)
        mb.release(0)
    ids, one = prefill(T)
    out.update(one)
    out["prefill_chunk_tokens"] = T
    kv_after_prefill = mb.kv_bytes_in_use()
    base_len = mb.seq_len(0)
    cur = ids.clone()
    nxt = [torch.empty(1, dtype=torch.int32, device="cuda:0") for _ in range(2)]
    e0, e1 = ev(), ev()
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
    n_inst = 4
    mb.set_timing(True)
    for i in range(n_inst):
        mb.decode([0], cur, logits=None, out_ids=nxt[i % 2])
        cur = nxt[i % 2]
    roles = role_table(mb.timing(reset=True), n_inst)
    mb.set_timing(False)
    log_roles(roles)
    kv_decode = mb.kv_bytes_in_use()
    log(f"[bench] KV with sliding-window page recycling: pool {mb.kv_bytes / 1e9:.2f} GB (without: "
        f"{plain_bytes / 1e9:.2f} GB); in use {kv_after_prefill / 1e9:.2f} GB after the prompt, "
        f"{kv_decode / 1e9:.2f} GB while decoding")
    last = int(ids[0].item())
    spec = {}
    for reuse in (False, True):
        mb.truncate(0, base_len)
        torch.cuda.synchronize()
        mb.spec_stats(reset=True)
        t0 = time.perf_counter()
        got = mb.spec_decode(0, last, n_spec, gamma=4, k_draft=1, k_verify=4, reuse=reuse)
        torch.cuda.synchronize()
        sp_s = time.perf_counter() - t0
        s = mb.spec_stats(reset=True)
        spec["reuse" if reuse else "no_reuse"] = {
            "tok_s": round(len(got) / sp_s, 2), "speedup_vs_plain_k4": round(len(got) / sp_s * dec_ms / 1e3, 3),
            "acceptance": round(s["accepted"] / max(1, s["drafted"]), 4),
            "draft_step_ms": round(s["draft_ms"] / max(1, s["drafted"]), 4),
            "verify_ms": round(s["verify_ms"] / max(1, s["rounds"]), 4),
            "verify_over_plain_k4_step": round(s["verify_ms"] / max(1, s["rounds"]) / dec_ms, 3)}
        log(f"[bench] long-context self-speculative ({'with' if reuse else 'without'} reuse): "
            f"{spec['reuse' if reuse else 'no_reuse']}")
    out.update({"decode_tok_s": round(1e3 / dec_ms, 2), "decode_GB_per_step": round(step_bytes / 1e9, 2),
                "decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "decode_kernels": {n: {"avg_us": round(r["avg_us"], 2), "ms_per_step": round(r["ms_per_step"], 3),
                                       "GBs": round(r["GBs"], 1)} for n, r in roles.items()},
                "self_speculative": spec, "kv_pool_GB": round(mb.kv_bytes / 1e9, 3),
                "kv_pool_without_recycling_GB": round(plain_bytes / 1e9, 3),
                "kv_in_use_after_prompt_GB": round(kv_after_prefill / 1e9, 3),
                "kv_in_use_decoding_GB": round(kv_decode / 1e9, 3)})
    mb.close()
    del mb
    torch.cuda.empty_cache()
    out["context_262144_k1"] = bench_256k(m1, shape)
    return out


def bench_256k(m1, shape):
    """The longest context the pages give (256K): a 262112-token prompt prefilled as one chunk at
    k = 1, then 16 decode steps at batch 1 from that context (32 positions are left for them
    within the 262144-position limit; the down projection's activation operand, 262112 x 8192
    bf16, stays just under 4 GiB here, so the row-blocked GEMM path is taken only by a
    262144-token chunk)."""
    import torch

    from looped_ngpt_language_amd import dory, synth
    T, n_dec = 262144 - 32, 16
    mc = dory.Model(shape, None, kv_mode="last_loop", max_loops=1, max_seqs=1, max_model_len=262144, max_tokens=T,
                    device="cuda:0", share_weights_from=m1, swa_recycle=True)
    mc.set_loops(1)
    st = mc.stream
    prompt = torch.from_numpy(synth.prompt_tokens(shape, T, seed=1)).to("cuda:0")
    e0, e1 = ev(), ev()
    e0.record(st)
    _, ids = mc.prefill(0, prompt, 1)
    e1.record(st)
    torch.cuda.synchronize()
    pf_ms = e0.elapsed_time(e1)
    cur = ids.clone()
    nxt = [torch.empty(1, dtype=torch.int32, device="cuda:0") for _ in range(2)]
    e0.record(st)
    for i in range(n_dec):
        mc.decode([0], cur, logits=None, out_ids=nxt[i % 2])
        cur = nxt[i % 2]
    e1.record(st)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / n_dec
    out = {"prompt_tokens": T, "loops": 1, "prefill_s": round(pf_ms / 1e3, 3),
           "prefill_tok_s": round(T / (pf_ms * 1e-3), 1), "decode_tok_s": round(1e3 / dec_ms, 2),
           "kv_in_use_GB": round(mc.kv_bytes_in_use() / 1e9, 3)}
    log(f"[bench] 256K context, k=1: one-chunk prefill of {T} tokens {pf_ms / 1e3:.2f} s, decode "
        f"{1e3 / dec_ms:.1f} tok/s")
    mc.close()
    del mc
    torch.cuda.empty_cache()
    return out


def bench_mid(args):
    """The mid-size model (d=1024, 8/4 heads of 128, FFN 4096, vocab 32768, 8/20/8 blocks, window
    1024): 512-token prompt, 128 decode tokens at batch 1, k = 1/2/4, both KV modes."""
    import torch

    from looped_ngpt_language_amd import dory, synth
    shape = synth.MID
    w = synth.make_weights(shape, seed=0)
    m = dory.Model(shape, w, kv_mode="per_loop", max_loops=4, max_seqs=1, max_model_len=1024, max_tokens=512,
                   device="cuda:0")
    del w
    ptoks = torch.from_numpy(synth.prompt_tokens(shape, 512)).to("cuda:0")
    out = {}
    for mode in ("last_loop", "per_loop"):
        out[mode] = {str(k): short(decode_run(m, k, mode, ptoks, 128, args.warmup, "cfg1")) for k in (1, 2, 4)}
    m.close()
    return out


def profiled(role):
    """The rocprofv3 figures of the kernel behind `role` from the committed profile summaries
    (profiles/traffic.json): average dispatch time and counter bytes per launch, reported only
    while the kernel's source file is unchanged since then."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(role)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source_file"])
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return {"avg_us": rec.get("avg_us"), "profile": rec["profile"],
            "traffic": {"fetch_bytes": rec["fetch_bytes"], "write_bytes": rec["write_bytes"],
                        "bytes": rec["fetch_bytes"] + rec["write_bytes"], "kernel": rec["kernel"]}}


def cpu_baseline(shape, w, prompt, k, budget_s=12.0):
    """The oracle as it stands (fp64 numpy), on the host cores, on a bounded sample: a 16-token
    prompt, then decode steps for ~budget_s. The GPU decodes at a 2560-token context; building
    that context in the oracle (a ~30 TFLOP fp64 prefill) does not fit the sample's budget, and
    a decode step's cost is dominated by the weights it reads (the context's keys add ~5% at
    2560 tokens), so the sample decodes after a 16-token prompt. Also the tiny fp32 model's
    64-token prefill + 16 decode steps and the mid model's 64-token prefill + ~3 s of decode
    steps (k = 2), each on all threads and on one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from looped_ngpt_language_amd import synth
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
    tiny = {}
    tw = synth.make_weights(synth.TINY, seed=0, threads=1)
    tp = synth.prompt_tokens(synth.TINY, 64)
    for label, lim in (("all_threads", None), ("one_thread", 1)):
        with threadpool_limits(limits=lim):
            to = OracleModel(synth.TINY, tw, "last_loop", 2)
            t0 = time.perf_counter()
            _, ids = to.prefill(0, tp, 1)
            t1 = time.perf_counter()
            tk = int(ids[0])
            for _ in range(16):
                _, ids = to.decode([0], [tk])
                tk = int(ids[0])
            t2 = time.perf_counter()
        tiny[label] = {"prefill_tok_s": round(64 / (t1 - t0), 1), "decode_tok_s": round(16 / (t2 - t1), 1)}
    # the mid-size model (cfg 1 shapes): a 64-token prompt, then decode steps for ~3 s, on all
    # threads and on one thread
    mid = {}
    mw = synth.make_weights(synth.MID, seed=0)
    mp = synth.prompt_tokens(synth.MID, 64)
    for label, lim in (("all_threads", None), ("one_thread", 1)):
        with threadpool_limits(limits=lim):
            mo = OracleModel(synth.MID, mw, "last_loop", 2)
            t0 = time.perf_counter()
            _, ids = mo.prefill(0, mp, 1)
            t1 = time.perf_counter()
            tk, nd = int(ids[0]), 0
            while nd < 2 or (time.perf_counter() - t1 < 3.0 and nd < 64):
                _, ids = mo.decode([0], [tk])
                tk = int(ids[0])
                nd += 1
            t2 = time.perf_counter()
        mid[label] = {"prefill_tok_s": round(64 / (t1 - t0), 2), "decode_tok_s": round(nd / (t2 - t1), 2),
                      "decode_steps": nd}
    log(f"[bench] oracle mid model k=2: {mid}")
    return {"value": round(n / dt, 4), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "host_affinity": len(os.sched_getaffinity(0)),
            "prefill_tok_s": round(16 / t_pf, 3), "tiny_fp32_k2": tiny, "mid_bf16_k2_64_token_prompt": mid,
            "sample": f"{n} decode steps ({dt:.1f} s) at batch 1, k={k}, last-loop KV, after a 16-token prompt "
                      f"(fp64 numpy oracle, same ~4B weights; the GPU figure is at a 2560-token context); "
                      f"cores = BLAS threads used"}


if __name__ == "__main__":
    main()
