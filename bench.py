#!/usr/bin/env python3
"""Throughput of batched draft-token verification on one MI355X.

One step = one call of the verification path over one batch of synthetic
inputs already resident in HBM.  Default workload: sampling verification with
top-p, B=64, gamma=5, V=151936, bfloat16 logits, T=0.8, top-p 0.9 (the rows
the headline metric is quoted on).  Inputs rotate over several copies in HBM
(more than three times the 256 MB Infinity Cache in total) so every step reads
its logits from HBM, not from the cache.

Timing: after the warmup steps, the K timed steps are queued behind a short
GPU sleep (so the host is ahead and the steps run back to back) and timed with
one pair of HIP events on the launch stream.  That gives `value`,
`ms_per_step`, and the mean launch duration the roofline divides by: the K
launches run back to back, so total / K is the mean launch-to-launch time (for
the multi-kernel paths, of the whole call).  The same K steps are then run once
more with an event pair around every launch; those events add a gap of a
microsecond or two per launch, so that lap is reported beside it
(`config.launch_ms_*`) as a cross-check only.

Prints ONE JSON line: verified vocab rows/s (target + draft rows per second),
the dominant kernel's roofline (algorithmic HBM bytes per launch / its mean
launch time, against 8 TB/s), and the CPU oracle timed on a bounded sample of
the same workload (one thread and every host core).  The default run then
times the other workloads the same way (the four other verification
configurations, the draft-side sampler, the SSD fan-out lookup, the
vocabulary trim and the fused lm_head -> greedy verification, the latter
against the bf16 MFMA peak) and reports each under
config.workloads (step time, rows/s, GB/s and fraction of peak, counter
traffic, the oracle's rows/s).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified vocab rows/sec and achieved HBM GB/s (% of peak), 1 MI355X"
PEAK_GBS = 8000.0

WORKLOADS = {
    # name: (generator kwargs, description)
    "sample_topp": dict(desc="sampling verify + top-p, B=64 gamma=5 V=151936 bf16, T=0.8 top_p=0.9"),
    "sample_plain": dict(desc="sampling verify, B=1 gamma=3 V=49152 fp32, T=1, no top-p"),
    "greedy": dict(desc="greedy verify, B=128 gamma=6 V=128256 bf16"),
    "eagle_d2t": dict(desc="EAGLE3 d2t sampling verify, B=32 gamma=7 Vt=128256 bf16 Vd=32000 fp32, T=1"),
    "tree": dict(desc="greedy tree verify, B=16 N=32 V=49152 bf16"),
    "draft": dict(desc="draft-side sampler, B=64 V=151936 bf16, T=0.8 top_p=0.9 top_k=50"),
    "fanout": dict(desc="SSD fan-out lookup, B=64 gamma=7 f=3 L=8"),
    "trim": dict(desc="vocabulary-trim d2t builder, 2^24 Zipf(1.1) tokens over Vt=128256, P=0.95"),
    "lmhead": dict(desc="fused lm_head -> greedy verify, hidden [128, 7, 4096] x W [128256, 4096] bf16"),
}
PEAK_BF16_TFLOPS = 2500.0


def compulsory_bytes(w) -> int:
    """Every input byte read once plus every output byte written once."""
    if w["kind"] == "draft":
        B = w["logits"].shape[0]
        return int(w["logits"].nbytes + w["u"].nbytes + 3 * B * 4)       # logits, uniforms; token, prob, status
    if w["kind"] == "lmhead":
        # hidden and W read once, draft tokens read; tokens, lengths, argmax, max logit, status written
        B, R, d = w["hidden"].shape
        return int(w["hidden"].nbytes + w["W"].nbytes + w["tokens"].nbytes + B * R * 4 + B * 4 + 2 * B * R * 4 + B * 4)
    if w["kind"] == "trim":
        # the token stream read once; d2t, t2d, the kept count and the info written
        return int(w["tokens"].nbytes + 2 * 4 * w["Vt"] + 4 + 24)
    if w["kind"] == "fanout":
        B, g1, f = w["cand"].shape
        L = w["drafts"].shape[2]
        # tokens at n, lengths, the f candidates at n, one branch's drafts read; branch and drafts written
        return int(B * (4 + 4 + 4 * f + 4 * L) + B * (4 + 4 * L))
    n = w["target"].nbytes + w["tokens"].nbytes
    if w["kind"] == "sample":
        n += w["draft"].nbytes + w["u_accept"].nbytes + w["u_sample"].nbytes
        if w.get("d2t") is not None:
            n += w["d2t"].nbytes
        B, g = w["tokens"].shape
        n += B * (g + 1) * 4 + B * 4 + 2 * B * g * 4 + B * 4      # tokens, len, p/q, status
    elif w["kind"] == "greedy":
        B, g = w["tokens"].shape
        n += B * (g + 1) * 4 + 2 * B * 4
    else:
        B, N = w["tokens"].shape
        n += w["parents"].nbytes + 2 * B * N * 4 + 2 * B * 4
    return int(n)


def rows_per_step(w) -> int:
    if w["kind"] == "lmhead":
        return int(w["hidden"].shape[0] * w["hidden"].shape[1])
    if w["kind"] == "trim":
        return int(w["tokens"].shape[0])
    if w["kind"] == "fanout":
        return int(w["cand"].shape[0])
    if w["kind"] == "draft":
        return int(w["logits"].shape[0])
    if w["kind"] == "sample":
        B, g = w["tokens"].shape
        return B * (2 * g + 1)
    return int(w["target"].shape[0] * w["target"].shape[1])


def make_inputs(name, seed):
    from draft_token_verification_07_amd import synth
    return synth.WORKLOADS[name](seed)


def device_sets(w, nrot, dev):
    """The workload's tensors on the GPU, with nrot distinct copies of the
    logits (the bulk of the bytes) so consecutive steps read different memory."""
    import torch

    def t(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a.copy()).to(dev)

    if w["kind"] == "lmhead":
        # the weights (GBs) exceed the Infinity Cache: every step reads them from HBM
        base = dict(hidden=t(w["hidden"]), W=t(w["W"]), tokens=t(w["tokens"]))
        torch.cuda.synchronize()
        return [base]
    if w["kind"] == "trim":
        base = dict(tokens=t(w["tokens"]))
        sets = [base] + [dict(tokens=base["tokens"].clone()) for _ in range(nrot - 1)]
        torch.cuda.synchronize()
        return sets
    if w["kind"] == "fanout":
        base = {k: t(w[k]) for k in ("out_tokens", "accept_len", "cand", "drafts")}
        torch.cuda.synchronize()
        return [base]
    if w["kind"] == "draft":
        base = dict(logits=t(w["logits"]), u=t(w["u"]))
        sets = [base] + [dict(base, logits=base["logits"].clone()) for _ in range(nrot - 1)]
        torch.cuda.synchronize()
        return sets
    base = dict(target=t(w["target"]), tokens=t(w["tokens"].astype(np.int32)))
    if w["kind"] == "sample":
        base.update(draft=t(w["draft"]), u_accept=t(w["u_accept"]), u_sample=t(w["u_sample"]),
                    d2t=t(w.get("d2t")))
    if w["kind"] == "tree":
        base["parents"] = t(w["parents"].astype(np.int32))
    sets = [base]
    for _ in range(nrot - 1):
        c = dict(base)
        c["target"] = base["target"].clone()
        if "draft" in base:
            c["draft"] = base["draft"].clone()
        sets.append(c)
    torch.cuda.synchronize()
    return sets


def _batch(w) -> int:
    key = {"draft": "logits", "fanout": "cand", "trim": "tokens", "lmhead": "hidden"}.get(w["kind"], "target")
    return int(w[key].shape[0])


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, max_seqs: int, work_seconds: float, threads: int):
    """Time the oracle as it stands on the first max_seqs sequences with
    `threads` threads (sampling; the greedy and tree oracles are one
    thread), repeating the pass until about work_seconds of CPU time (wall
    time x threads used) have been spent."""
    import oracle
    oracle.build(force=False)
    B = _batch(w)
    s = min(B, max_seqs)
    sl = slice(0, s)

    def one_pass():
        if w["kind"] == "lmhead":
            R = w["hidden"].shape[1]
            z, _ = oracle.lmhead_logits(w["hidden"][0], w["W"])
            oracle.greedy_from_argmax(np.argmax(z, axis=1)[None], w["tokens"][:1], w["W"].shape[0])
            return R, 1
        if w["kind"] == "trim":
            n = min(w["tokens"].shape[0], 1 << 20)
            oracle.vocab_trim(w["tokens"][:n], w["Vt"], w["P"])
            return n, 1
        if w["kind"] == "fanout":
            oracle.fanout_lookup(w["out_tokens"][sl], w["accept_len"][sl], w["cand"][sl], w["drafts"][sl])
            return s, 1
        if w["kind"] == "draft":
            oracle.draft_sample(w["logits"][sl], w["u"][sl], w["temperature"], w["top_p"], top_k=w["top_k"])
            return s, 1
        if w["kind"] == "sample":
            oracle.verify_sample(w["target"][sl], w["draft"][sl], w["tokens"][sl], w["u_accept"][sl],
                                 w["u_sample"][sl], w["temperature"], w["top_p"], d2t=w.get("d2t"),
                                 nthreads=threads)
            return s * (2 * w["tokens"].shape[1] + 1), min(threads, s)
        if w["kind"] == "greedy":
            oracle.verify_greedy(w["target"][sl], w["tokens"][sl])
        else:
            oracle.verify_tree_greedy(w["target"][sl], w["tokens"][sl], w["parents"][sl])
        return s * w["target"].shape[1], 1

    rows = passes = 0
    used = 1
    t0 = time.perf_counter()
    while True:
        r, used = one_pass()
        rows += r
        passes += 1
        dt = time.perf_counter() - t0
        if dt * used >= work_seconds or dt >= 3.0 * work_seconds:
            break
    return dict(value=rows / dt, cores=used, passes=passes, seqs=s, wall_s=dt)


def cpu_baselines(w, max_seqs: int, work_seconds: float):
    """The oracle on one thread and on every host core this process may use."""
    ncores = min(len(os.sched_getaffinity(0)), 64)
    one = cpu_baseline(w, max(1, max_seqs // 8), work_seconds, 1)
    many = cpu_baseline(w, max_seqs, work_seconds, ncores) if w["kind"] == "sample" and ncores > 1 else one
    B = _batch(w)
    if w["kind"] == "trim":
        n = min(B, 1 << 20)
        return dict(value=one["value"], unit="tokens/s", cores=1, kind="oracle", value_1thread=one["value"],
                    cores_available=ncores, nproc=os.cpu_count(), cpu_model=cpu_model(),
                    sample="1 thread: %d pass(es) over the first %d of %d tokens, %.2f s wall"
                           % (one["passes"], n, B, one["wall_s"]))
    return dict(value=many["value"], unit="rows/s", cores=many["cores"], kind="oracle",
                value_1thread=one["value"], cores_available=ncores, nproc=os.cpu_count(), cpu_model=cpu_model(),
                sample="1 thread: %d pass(es) over the first %d of %d sequences, %.2f s wall; "
                       "%d threads: %d pass(es) over the first %d, %.2f s wall (same workload)"
                       % (one["passes"], one["seqs"], B, one["wall_s"], many["cores"], many["passes"],
                          many["seqs"], many["wall_s"]))


KERNELS = dict(sample_topp="topp_kernel", sample_plain="stats_kernel+tile_kernel+pick_kernel",
               eagle_d2t="stats_kernel+tile_kernel+pick_kernel", greedy="greedy_kernel",
               tree="greedy_kernel+seq_kernel", draft="draft_kernel", fanout="fanout_kernel",
               trim="trim_part_kernel+trim_reduce_kernel+trim_refine_kernel+trim_count_kernel+trim_write_kernel",
               lmhead="lmhead_dma_kernel+lmhead_reduce_kernel+seq_kernel")


def measure(name, args, dev, log):
    """Time one workload: W warmup steps, then K steps twice (throughput lap,
    then a lap with events around every launch).  Returns a dict."""
    import torch
    import draft_token_verification_07_amd as sv

    log("[bench] generating %s (seed %d)" % (name, args.seed))
    w = make_inputs(name, args.seed)
    nbytes = compulsory_bytes(w)
    # rotated copies keep the bulk inputs cold; the fan-out tables are a few KB
    nrot = 1 if w["kind"] in ("fanout", "lmhead") else max(1, int(math.ceil(args.cold_bytes / nbytes)))
    sets = device_sets(w, nrot, dev)
    stream = torch.cuda.current_stream(dev)

    # preallocated outputs and one workspace (calls on one stream share it)
    if w["kind"] == "lmhead":
        B, R, d = w["hidden"].shape
        need = sv.sv_workspace_bytes_lmhead(B * R, w["W"].shape[0])
        outs = (torch.empty((B, R), dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty((B, R), dtype=torch.int32, device=dev), torch.empty((B, R), dtype=torch.float32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev))

        def step(s):
            sv.spec_lmhead_verify_greedy(s["hidden"], s["W"], s["tokens"], ws=ws, out=outs)
    elif w["kind"] == "trim":
        Vt = w["Vt"]
        need = sv.sv_workspace_bytes_vocab_trim(Vt)
        outs = (torch.empty(Vt, dtype=torch.int32, device=dev), torch.empty(Vt, dtype=torch.int32, device=dev),
                torch.empty(1, dtype=torch.int32, device=dev), torch.empty(3, dtype=torch.int64, device=dev))

        def step(s):
            sv.spec_vocab_trim(s["tokens"], Vt, w["P"], ws=ws, out=outs)
    elif w["kind"] == "fanout":
        need = 256
        ctr = torch.zeros(2, dtype=torch.int64, device=dev)

        def step(s):
            sv.spec_fanout_lookup(s["out_tokens"], s["accept_len"], s["cand"], s["drafts"], counters=ctr)
        outs = None
    elif w["kind"] == "draft":
        B, V = w["logits"].shape
        need = sv.sv_workspace_bytes_draft(B, V)
        outs = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.float32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev))

        def step(s):
            sv.spec_draft_sample(s["logits"], s["u"], w["temperature"], w["top_p"], w["top_k"], ws=ws, out=outs)
    elif w["kind"] == "sample":
        B, g = w["tokens"].shape
        Vt = w["target"].shape[2]
        Vd = w["draft"].shape[2]
        need = sv.sv_workspace_bytes_sample(B, g, Vt, Vd, w["top_p"])
        outs = (torch.empty((B, g + 1), dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty((B, g), dtype=torch.float32, device=dev), torch.empty((B, g), dtype=torch.float32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev))

        def step(s):
            sv.spec_verify_sample(s["target"], s["draft"], s["tokens"], s["u_accept"], s["u_sample"],
                                  w["temperature"], w["top_p"], d2t=s["d2t"], ws=ws, out=outs)
    elif w["kind"] == "greedy":
        B, g = w["tokens"].shape
        need = sv.sv_workspace_bytes_greedy(B, g, w["target"].shape[2])
        outs = (torch.empty((B, g + 1), dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev))

        def step(s):
            sv.spec_verify_greedy(s["target"], s["tokens"], ws=ws, out=outs)
    else:
        B, N = w["tokens"].shape
        need = sv.sv_workspace_bytes_tree(B, N, w["target"].shape[2])
        outs = (torch.empty((B, N), dtype=torch.int32, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))

        def step(s):
            sv.spec_verify_tree_greedy(s["target"], s["tokens"], s["parents"], ws=ws, out=outs)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)

    for i in range(args.warmup):
        step(sets[i % nrot])
    torch.cuda.synchronize()

    K = args.steps
    t0e = torch.cuda.Event(enable_timing=True)
    t1e = torch.cuda.Event(enable_timing=True)

    def queue_ahead():
        # keep the GPU busy while the host queues the steps, so that they run
        # back to back and the events time the GPU, not Python
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(args.queue_ahead_cycles))

    # lap 1: throughput (no events between steps)
    torch.cuda.synchronize()
    queue_ahead()
    t0e.record(stream)
    for i in range(K):
        step(sets[i % nrot])
    t1e.record(stream)
    torch.cuda.synchronize()
    total_ms = t0e.elapsed_time(t1e)

    # lap 2: per-launch durations of the same K steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    queue_ahead()
    for i in range(K):
        ev[i][0].record(stream)
        step(sets[i % nrot])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_launch_ms = [a.elapsed_time(b) for a, b in ev]
    del sets, ws, outs
    torch.cuda.empty_cache()

    ms_per_step = total_ms / K
    rows = rows_per_step(w)
    # Average launch duration: the throughput lap's events bracket K launches
    # that run back to back on the launch stream, so total / K is the mean
    # launch-to-launch duration (for the multi-kernel paths, of the call).
    achieved = nbytes / (ms_per_step / 1e3) / 1e9
    res = dict(workload=name, desc=WORKLOADS[name]["desc"], kernel=KERNELS[name],
               logits_dtype=("-" if w["kind"] in ("fanout", "trim", "lmhead") else
                             str((w["logits"] if w["kind"] == "draft" else w["target"]).dtype).replace("uint16", "bf16")),
               rows_per_step=rows, bytes_per_step=nbytes, rotated_input_copies=nrot,
               ms_per_step=ms_per_step, rows_per_s=rows * K / (total_ms / 1e3),
               seqs_per_s=float(_batch(w) * K / (total_ms / 1e3)),
               achieved_GBps=achieved, bound="hbm", frac=achieved / PEAK_GBS,
               traffic=read_traffic(args.traffic_table, name),
               launch_ms_mean=float(np.mean(per_launch_ms)), launch_ms_median=float(np.median(per_launch_ms)),
               launch_ms_p10=float(np.percentile(per_launch_ms, 10)),
               launch_ms_p90=float(np.percentile(per_launch_ms, 90)))
    if w["kind"] == "lmhead":
        B, R, d = w["hidden"].shape
        flops = 2.0 * B * R * w["W"].shape[0] * d
        tf = flops / (ms_per_step / 1e3) / 1e12
        # frac is against the peak of the bound (the bf16 MFMA peak); the HBM
        # rate of the same step is kept beside it
        res.update(bound="mfma", flops_per_step=flops, achieved_TFLOPs=tf, mfma_frac=tf / PEAK_BF16_TFLOPS,
                   frac=tf / PEAK_BF16_TFLOPS, hbm_frac=achieved / PEAK_GBS)
        log("[bench] %s: %.2f us/step, %.0f TFLOP/s (%.3f of the bf16 MFMA peak), %.0f GB/s"
            % (name, ms_per_step * 1e3, tf, tf / PEAK_BF16_TFLOPS, achieved))
    else:
        log("[bench] %s: %.2f us/step, %.0f GB/s (%.3f of peak)" % (name, ms_per_step * 1e3, achieved,
                                                                   achieved / PEAK_GBS))
    return w, res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sample_topp", choices=sorted(WORKLOADS),
                    help="the workload of the headline value and roofline")
    ap.add_argument("--only", action="store_true", help="time the headline workload alone")
    ap.add_argument("--seed", type=int, default=2002)
    ap.add_argument("--cold-bytes", type=float, default=1.0e9,
                    help="total bytes of rotated input copies (> 3x the 256 MB Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=64)
    ap.add_argument("--cpu-work-seconds", type=float, default=10.0,
                    help="CPU time (wall x threads) to spend timing the oracle on the headline workload")
    ap.add_argument("--cpu-work-seconds-other", type=float, default=3.0,
                    help="the same for each of the other workloads")
    ap.add_argument("--queue-ahead-cycles", type=float, default=4e7,
                    help="GPU sleep queued before the timed steps (lets the host run ahead)")
    ap.add_argument("--copy-calibration", type=float, default=0.0,
                    help="instead of the benchmark, copy this many bytes device-to-device "
                         "(a kernel of known traffic, to scale rocprofv3 byte counters)")
    ap.add_argument("--traffic-table", default=os.path.join(ROOT, "profiles", "hbm_traffic.md"),
                    help="HBM bytes per launch measured with rocprofv3 counters (markdown table)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this verification path shards by sequence with no "
              "communication, and only --gpus 1 is run here.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration > 0:
        n = int(args.copy_calibration) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps(dict(copy_bytes_read=4 * n, copy_bytes_written=4 * n, launches=5)), flush=True)
        return
    import draft_token_verification_07_amd as sv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sv.lib()                                   # fails loudly without the HIP library

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    head = args.workload
    names = [head] + ([] if args.only else [n for n in ("greedy", "eagle_d2t", "tree", "sample_plain", "sample_topp",
                                                         "draft", "fanout", "trim", "lmhead") if n != head])
    results, inputs = {}, {}
    for name in names:
        inputs[name], results[name] = measure(name, args, dev, log)

    cpu = None
    if not args.no_cpu_baseline:
        for name in names:
            log("[bench] timing the CPU oracle on %s" % name)
            secs = args.cpu_work_seconds if name == head else args.cpu_work_seconds_other
            c = cpu_baselines(inputs[name], args.cpu_seqs, secs)
            results[name]["cpu_rows_per_s"] = c["value"]
            results[name]["cpu_rows_per_s_1thread"] = c["value_1thread"]
            results[name]["cpu_threads"] = c["cores"]
            if name == head:
                cpu = c

    r = results[head]
    K = args.steps
    cfg = dict(workload=head, desc=r["desc"], logits_dtype=r["logits_dtype"], rows_per_step=r["rows_per_step"],
               bytes_per_step=r["bytes_per_step"], rotated_input_copies=r["rotated_input_copies"],
               kernel=r["kernel"], launch_ms_mean=r["launch_ms_mean"], launch_ms_median=r["launch_ms_median"],
               launch_ms_p10=r["launch_ms_p10"], launch_ms_p90=r["launch_ms_p90"],
               step_GBps=r["achieved_GBps"], seqs_per_s=r["seqs_per_s"],
               workloads={n: {k: v for k, v in results[n].items() if k not in ("workload", "desc")}
                          for n in names if n != head})
    line = dict(metric=METRIC, value=r["rows_per_s"], unit="rows/s", n_gpus=1, steps=K, warmup=args.warmup,
                ms_per_step=r["ms_per_step"], higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="f32", data="synthetic", config=cfg,
                roofline=(dict(bound="mfma", achieved=r["achieved_TFLOPs"], peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                               frac=r["mfma_frac"], traffic=r["traffic"]) if r.get("bound") == "mfma" else
                          dict(bound="hbm", achieved=r["achieved_GBps"], peak=PEAK_GBS, unit="GB/s",
                               frac=r["frac"], traffic=r["traffic"])),
                cpu_baseline=cpu)
    print(json.dumps(line), flush=True)


# Sources each workload's kernels are built from: its own kernel file(s) plus
# the shared headers, host code and launch code.
SHARED_SOURCES = ("sv_host.h", "sv_host.cpp", "sv_common.h", "sv_rows.h", "sv_internal.h", "sv_api.hip")
KERNEL_SOURCES = {
    "sample_topp": ("sv_sample.hip",), "sample_plain": ("sv_sample.hip",), "eagle_d2t": ("sv_sample.hip",),
    "greedy": ("sv_greedy.hip",), "tree": ("sv_greedy.hip",), "draft": ("sv_draft.hip",),
    "fanout": ("sv_fanout.hip",), "trim": ("sv_trim.hip",), "lmhead": ("sv_lmhead.hip", "sv_greedy.hip"),
}


def sources_sha(workload: str) -> str:
    """Hash of the sources `workload`'s kernels are built from, so counter
    readings of an older kernel are not reported for a changed one."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "draft_token_verification_07_amd", "csrc")
    for f in sorted(SHARED_SOURCES + KERNEL_SOURCES[workload]):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(path: str, workload: str):
    """HBM bytes per launch for `workload` from the counter table, or None when
    the table is absent or was measured on other kernel sources.  Rows look
    like `| workload | sources | fetch KiB | write KiB | factor | bytes/launch |`."""
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    sha = sources_sha(workload)
    for ln in lines:
        cells = [c.strip() for c in ln.strip().strip("|").split("|")]
        if len(cells) >= 6 and cells[0] == workload and cells[1] == sha:
            try:
                return float(cells[5])
            except ValueError:
                return None
    return None


if __name__ == "__main__":
    main()
