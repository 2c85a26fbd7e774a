"""Benchmark of the batched verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]
                    [--mode sampled|greedy] [--no-cpu-baseline] [--no-ceiling] [--no-settle]

One step = one call of the verification library over a whole batch (all
rows of all B sequences: the fused row pass, the acceptance decisions, the
accept-prefix scan and the final draw).  Inputs are generated on the host by
the seeded workload generator, copied to HBM before timing, and two input
sets alternate so that consecutive steps never hit the same data in the
256 MB Infinity Cache.  Before the W warm-up steps a plain streaming read
of the same bytes runs for at least 50 ms (the GPU then runs the timed steps
at its loaded clocks) and measures the empirical read ceiling.

Printed: one JSON line (rank 0) with verify rounds/s as `value`, the
roofline of the dominant kernel (formula bytes per launch over the average
launch duration, from one pair of HIP events on the launch stream around the
timed launches, against 8 TB/s), the empirical ceiling of a plain read of
the same bytes on this GPU (context), and the fp64 CPU oracle timed on one
host thread and on the host's cores over a bounded sample of the same
workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = os.path.join(ROOT, "speculative_decoding_verification_row_amd", "csrc", "sv_verify.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha256() -> str:
    """SHA-256 of the kernel source's code: comments (// and /* */), trailing
    blanks and empty lines removed, so that an edit of a comment does not
    mark the committed counter figures stale, while any change of code does.
    (The source has no string literal that holds a comment marker.)"""
    import re
    with open(KERNEL_SRC, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode("utf-8")).hexdigest()


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    none were taken or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    e = data.get(f"{kernel}|{workload}")
    if not e or e.get("source_sha256") != source_sha256():
        return None
    return e.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> tuple:
    """(threads the multi-threaded oracle run uses, CPUs in this process's
    affinity mask).  The threads are the affinity mask's CPUs, capped by the
    host's CPU share for this process when OMP_NUM_THREADS states one (a
    shared GPU host gives each GPU a share of its cores)."""
    try:
        n_aff = len(os.sched_getaffinity(0))
    except AttributeError:
        n_aff = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    n = n_aff
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n), n_aff


def _time_oracle(once, target_seconds):
    once()
    reps, t0 = 0, time.perf_counter()
    while True:
        once()
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_seconds:
            return reps, el


def cpu_baseline(cfg, mode, target_seconds=10.0, logits=False, tau=1.0):
    """Time the fp64 oracle as it stands over a bounded sample of the
    workload (whole sequences of input set 0), scaled to rounds/s: once on one
    thread and once on the host's cores (cpu_threads; the oracle splits a
    batch over threads by whole sequences).  The logits oracle is numpy on
    one thread, so it is timed once."""
    import oracle
    import workloads
    B = cfg["B"]
    threads, n_aff = cpu_threads()
    if logits:
        threads = 1
    n_seq = min(B, max(1, 2 * threads))
    hb = workloads.make_batch(cfg["family"], B, cfg["K"], cfg["V"], seed=0, seqs=list(range(n_seq)), logits=logits)
    sampled = mode == "sampled"

    def run(nthreads, seqs):
        sl = slice(0, seqs)
        args = (hb.target_probs[sl], hb.draft_probs[sl] if sampled or logits else None, hb.draft_tokens[sl],
                hb.uniforms[sl])

        def once():
            if logits:
                from oracle.logits import verify_sample_logits
                verify_sample_logits(args[0], args[1], args[2], args[3], tau)
            elif sampled:
                oracle.verify_sample(*args, threads=nthreads, diagnostics=False)
            else:
                oracle.verify_greedy(args[0], args[2], threads=nthreads)
        reps, el = _time_oracle(once, target_seconds)
        return reps * seqs / el / B, f"{seqs} of {B} sequences of input set 0, repeated {reps}x in {el:.1f}s " \
                                     f"on {nthreads} thread(s), scaled by {seqs}/{B} to whole rounds"

    v1, s1 = run(1, min(n_seq, 2))
    out = {"value": v1, "unit": "rounds/s", "cores": 1, "kind": "oracle", "sample": s1,
           "cpu_model": cpu_model(), "affinity_cpus": n_aff}
    if threads > 1:
        vn, sn = run(threads, n_seq)
        out.update(value=vn, cores=threads, sample=sn, single_thread={"value": v1, "sample": s1})
    return out


def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "speculative_decoding_verification_row_amd", "libsv_probe.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    P, SZ, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    L.sv_probe_blocks.argtypes = [SZ, SZ, I32, I32]
    L.sv_probe_blocks.restype = ctypes.c_int64
    L.sv_probe_read.argtypes = [P, SZ, P, SZ, I32, I32, P, P]
    L.sv_probe_read.restype = I32
    return L


def _probe_buffers(sets, sampled):
    bufs = []
    for db in sets:
        t, d = db["tp"], db["dp"] if sampled else None
        bufs.append((t.data_ptr(), t.numel() * 4, d.data_ptr() if d is not None else None,
                     d.numel() * 4 if d is not None else 0))
    return bufs


def settle_device(sets, sampled, min_ms=50.0):
    """Stream the step's operand bytes with the read probe (one-shot shape)
    for at least min_ms of wall clock before the warm-up steps, so that the
    timed steps run at the GPU's loaded clocks.  Measured: straight after the
    inputs are generated (the GPU idle while the host hashes them), 5 warm-up
    steps of the headline workload leave the next 20 at 228.6-231.9 us per
    launch, against 221.2 us over 400 after 40."""
    import torch
    L = _probe_lib()
    if L is None:
        return {"note": "libsv_probe.so not built; no settle"}
    bufs = _probe_buffers(sets, sampled)
    b0, b1 = bufs[0][1], bufs[0][3]
    stream = torch.cuda.current_stream()
    nb = L.sv_probe_blocks(b0, b1, 0, 0)
    res = torch.empty(max(nb, 1), dtype=torch.float32, device=sets[0]["tp"].device)
    t0, n = time.perf_counter(), 0
    while True:
        for _ in range(8):
            x = bufs[n % len(bufs)]
            assert L.sv_probe_read(x[0], x[1], x[2], x[3], 0, 0, res.data_ptr(), stream.cuda_stream) == 0
            n += 1
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) * 1e3
        if el >= min_ms:
            return {"launches": n, "ms": round(el, 1)}


def stream_ceiling(sets, sampled, steps=20):
    """The empirical ceiling of one read pass on this GPU: the streaming-read
    probe (libsv_probe.so; no arithmetic but a keep-alive sum) over the same
    operand bytes as a step, in both launch shapes (one block per 32 KB
    chunk, and one persistent block per CU), two input sets alternating, one
    pair of HIP events around the timed launches.  Context for the roofline,
    never its peak."""
    import torch
    L = _probe_lib()
    if L is None:
        return {"note": "libsv_probe.so not built"}
    bufs = _probe_buffers(sets, sampled)
    b0, b1 = bufs[0][1], bufs[0][3]
    stream = torch.cuda.current_stream()
    out = {"bytes_per_launch": b0 + b1, "unit": "GB/s", "steps": steps}
    for name, mode, bpc in (("one_shot", 0, 0), ("persistent", 1, 1)):
        nb = L.sv_probe_blocks(b0, b1, mode, bpc)
        res = torch.empty(max(nb, 1), dtype=torch.float32, device=sets[0]["tp"].device)

        def launch(k):
            x = bufs[k % len(bufs)]
            rc = L.sv_probe_read(x[0], x[1], x[2], x[3], mode, bpc, res.data_ptr(), stream.cuda_stream)
            assert rc == 0, f"probe launch failed ({rc})"
        for k in range(4):
            launch(k)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(steps):
            launch(k)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        out[name] = {"us": round(us, 2), "gbs": round((b0 + b1) / us / 1e3, 1)}
    best = max(out["one_shot"]["gbs"], out["persistent"]["gbs"])
    out["gbs"] = best
    out["frac_of_peak"] = round(best / PEAK_HBM_GBS, 4)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--mode", default=None, choices=[None, "sampled", "greedy"])
    ap.add_argument("--sets", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gen-workers", type=int, default=1,
                    help="forked processes generating the inputs; more speed up the large "
                         "workloads, but forked workers die under rocprofv3 counter collection")
    ap.add_argument("--logits", action="store_true",
                    help="sampled verification given logits (warped in the library) instead of probabilities")
    ap.add_argument("--temperature", type=float, default=1.0, help="temperature of --logits")
    ap.add_argument("--stats", action="store_true",
                    help="sampled or greedy verification that also writes the per-row statistics (argmax, max, "
                         "sum p, sum q, sum min, sum max(0, p - q), p(t), q(t)): the full fused pass")
    ap.add_argument("--early-exit", action="store_true",
                    help="sampled verification through the early-exit entry point (reads only the rows the "
                         "outputs depend on; its byte count is those rows)")
    ap.add_argument("--decoder", action="store_true",
                    help="time rounds of the multi-round driver (B=1, K=4, V=32000) instead")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read probe (the empirical ceiling reported beside the roofline)")
    ap.add_argument("--no-settle", action="store_true",
                    help="skip the >= 50 ms of streaming reads that bring the GPU to its loaded clocks "
                         "before the warm-up steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy 5 times (reference for "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the verification step is sharded over sequences with "
              "no exchange, and this build runs on a single MI355X; use --gpus 1.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    from workloads.device import device_batch
    import speculative_decoding_verification_row_amd as sv

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", flush=True)
        sys.exit(1)
    sv.load_library()
    if args.decoder:
        return decoder_bench(args)
    cfg = dict(workloads.CONFIGS[args.workload])
    mode = args.mode or ("sampled" if "sampled" in cfg["modes"] else "greedy")
    if args.logits:
        if cfg["family"] not in ("c1", "c3"):
            raise SystemExit("--logits takes workload 1 or 3 (families with logits)")
        mode = "sampled"
    sampled = mode == "sampled"
    if args.early_exit and not sampled:
        raise SystemExit("--early-exit takes the sampled mode (probabilities or --logits)")
    if args.stats and (args.logits or args.early_exit):
        raise SystemExit("--stats takes the probability passes (the logits and early-exit passes write none)")
    B, K, V = cfg["B"], cfg["K"], cfg["V"]
    dev = torch.device("cuda:0")
    workload = f"B={B} K={K} V={V} {mode}" + (f" logits tau={args.temperature:g}" if args.logits else "")
    if args.early_exit:
        workload += " early-exit"
    if args.stats:
        workload += " stats"
    log(f"workload {args.workload}: {workload}; generating {args.sets} input sets")

    sets = []
    for s in range(args.sets):
        sets.append(device_batch(cfg["family"], B, K, V, seed=s, device=dev, sampled=sampled,
                                 workers=args.gen_workers, logits=args.logits,
                                 progress=lambda d, n: log(f"    {d}/{n} sequences")))
        log(f"  set {s} ready ({sets[-1]['sha256'][:12]})")
    n_out = torch.empty(B, dtype=torch.int32, device=dev)
    x_out = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ws = sv.workspace_for(B, K, V, sampled, dev, stream)
    st_out = torch.empty((B, K + 1, 48), dtype=torch.uint8, device=dev) if args.stats else None

    def step(db):
        if args.logits:
            f = sv.sv_verify_sample_logits_early_batched if args.early_exit else sv.sv_verify_sample_logits_batched
            f(db["tp"], db["dp"], db["dt"], db["u"], args.temperature,
              n_accepted=n_out, next_token=x_out, workspace=ws, stream=stream)
        elif args.early_exit:
            sv.sv_verify_sample_early_batched(db["tp"], db["dp"], db["dt"], db["u"], n_accepted=n_out,
                                              next_token=x_out, workspace=ws, stream=stream)
        elif sampled:
            sv.sv_verify_sample_batched(db["tp"], db["dp"], db["dt"], db["u"], n_accepted=n_out,
                                        next_token=x_out, workspace=ws, stats=st_out, stream=stream)
        else:
            sv.sv_verify_greedy_batched(db["tp"], db["dt"], n_accepted=n_out, next_token=x_out,
                                        workspace=ws, stats=st_out, stream=stream)

    # The read probe runs before the warm-up steps: first a settle of at
    # least 50 ms, then (unless --no-ceiling) the ceiling measurement.
    settle = settle_device(sets, sampled) if not args.no_settle else None
    ceil = None
    if not args.no_ceiling:
        log("streaming-read probe over the same bytes (empirical ceiling, context)")
        ceil = stream_ceiling(sets, sampled)
    for w in range(args.warmup):
        step(sets[w % len(sets)])
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")

    # One pair of HIP events on the launch stream around the K back-to-back
    # launches: the average launch duration then includes the gaps between
    # launches, and the timed work is exactly what a caller sees (an event pair
    # per launch would add its own packets between the launches).
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for k in range(args.steps):
        step(sets[k % len(sets)])
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = ev0.elapsed_time(ev1) / args.steps
    assert sv.sv_workspace_error(ws) == 0, "device fault word set during the benchmark"

    # spot check of the last step's outputs against the oracle (2 sequences)
    last = sets[(args.steps - 1) % len(sets)]
    spot = spot_check(cfg, mode, last, n_out, x_out, seed=(args.steps - 1) % len(sets),
                      logits=args.logits, tau=args.temperature, stats=st_out)

    fbytes = workloads.formula_bytes(B, K, V, sampled)
    formula = fbytes
    if args.early_exit:
        # the early exit's algorithmic bytes: the rows the outputs depend on
        # (pairs 0..n, and row K after full acceptance), averaged over the
        # input sets, which the timed steps use equally often
        need = []
        for db in sets:
            step(db)
            n = n_out.cpu().numpy().astype(np.int64)
            need.append(int(((np.where(n < K, 2 * (n + 1), 2 * K + 1)) * V * 4).sum()))
        fbytes = int(round(sum(need) / len(need)))
    achieved = fbytes / (avg_ms * 1e-3) / 1e9
    kernel = "sv_logits_kernel" if args.logits else ("sv_sample_kernel" if sampled else "sv_greedy_kernel")
    rounds_per_s = args.steps / wall
    line = {
        "metric": f"verify rounds/s + HBM GB/s (% of peak), {workload}",
        "value": round(rounds_per_s, 2),
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload, "B": B, "K": K, "V": V, "mode": mode,
                   "recipe": cfg["family"], "input_sets": args.sets},
        "hbm_gbs": round(fbytes * rounds_per_s / 1e9, 1),
        "pct_of_peak": round(100.0 * fbytes * rounds_per_s / 1e9 / PEAK_HBM_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for(kernel, workload),
                     "kernel": kernel, "kernel_avg_us": round(avg_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": fbytes},
        **({"formula_bytes_per_launch": formula} if args.early_exit else {}),
        "accumulation": "f64",
        "parity_spot": spot,
        "context": {"pages_cpu_latency_us": {"greedy": 33, "sampled": 117,
                                             "hardware": "Raspberry Pi 5, V=32000, K=4, one sequence"}},
    }
    if args.copy_calibration:
        # a plain copy kernel of known size: 1 GiB read + 1 GiB written per
        # launch (an elementwise kernel; a device-to-device copy_ may run on a
        # DMA engine that the counters do not see)
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = src.numel() * 4
    if settle is not None:
        line["settle"] = settle
    if ceil is not None:
        if "gbs" in ceil:
            ceil["kernel_frac_of_ceiling"] = round(achieved / ceil["gbs"], 4)
        line["stream_ceiling"] = ceil
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(cfg, mode, logits=args.logits, tau=args.temperature)
    print(json.dumps(line), flush=True)


def decoder_bench(args):
    """Rounds of the multi-round driver (SpeculativeDecoder) at the card's own
    shape, B=1, K=4, V=32000 (workload 1), with callbacks that hand back
    device-resident rows of that workload, so that the figure is the driver
    and the verification, not a model.  Two input sets alternate."""
    import numpy as np
    import torch
    import speculative_decoding_verification_row_amd as sv
    import workloads
    from workloads.device import device_batch
    cfg = workloads.CONFIGS[1]
    K, V = cfg["K"], cfg["V"]
    mode = args.mode or "sampled"
    sampled = mode == "sampled"
    dev = torch.device("cuda:0")
    sets = [device_batch(cfg["family"], 1, K, V, seed=s, device=dev, sampled=sampled) for s in range(2)]
    turn = [0]

    def draft_step(prefix, k):
        db = sets[turn[0] % 2]
        return db["dt"][0], (db["dp"][0] if sampled else None)

    def target_step(prefix, proposed):
        db = sets[turn[0] % 2]
        turn[0] += 1
        return db["tp"][0]

    dec = sv.SpeculativeDecoder(draft_step, target_step, k=K, greedy=not sampled, seed=0, device=dev)
    dec.generate([1], max_new=args.warmup * (K + 1))
    torch.cuda.synchronize()
    dec.stats = sv.DecodeStats()
    max_new = args.steps * (K + 1)
    t0 = time.perf_counter()
    out = dec.generate([1], max_new=max_new)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rounds = dec.stats.rounds
    # the verification kernel alone on the same inputs (one event pair)
    ws = sv.workspace_for(1, K, V, sampled, dev)
    n_out = torch.empty(1, dtype=torch.int32, device=dev)
    x_out = torch.empty(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def verify(db):
        if sampled:
            sv.sv_verify_sample_batched(db["tp"], db["dp"], db["dt"], db["u"], n_accepted=n_out,
                                        next_token=x_out, workspace=ws, stream=stream)
        else:
            sv.sv_verify_greedy_batched(db["tp"], db["dt"], n_accepted=n_out, next_token=x_out,
                                        workspace=ws, stream=stream)

    for j in range(20):
        verify(sets[j % 2])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for j in range(rounds):
        verify(sets[j % 2])
    e1.record(stream)
    torch.cuda.synchronize()
    kern_us = e0.elapsed_time(e1) * 1e3 / rounds
    round_us = wall / rounds * 1e6
    line = {
        "metric": f"speculative decoding driver rounds/s, B=1 K={K} V={V} {mode}, device-resident callbacks",
        "value": round(rounds / wall, 1), "unit": "rounds/s", "n_gpus": 1, "steps": rounds,
        "warmup": args.warmup, "ms_per_step": round(round_us / 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"B=1 K={K} V={V} {mode} decoder rounds", "recipe": cfg["family"]},
        "tokens_per_round": round((len(out) - 1) / rounds, 3),
        "verify_launch_us": round(kern_us, 2),
        "host_us_per_round": round(round_us - kern_us, 2),
        "mean_accepted": round(dec.stats.mean_accepted(), 3),
    }
    print(json.dumps(line), flush=True)


def spot_check(cfg, mode, db, n_out, x_out, seed, logits=False, tau=1.0, stats=None):
    """Two sequences of the last step against the oracle (and, with row
    statistics, their masses and argmax)."""
    import numpy as np
    import oracle
    import workloads
    seqs = [0, cfg["B"] - 1]
    hb = workloads.make_batch(cfg["family"], cfg["B"], cfg["K"], cfg["V"], seed=seed, seqs=seqs, logits=logits)
    n = n_out.cpu().numpy()[seqs]
    x = x_out.cpu().numpy()[seqs]
    if logits:
        from oracle.logits import verify_sample_logits
        o = verify_sample_logits(hb.target_probs, hb.draft_probs, hb.draft_tokens, hb.uniforms, tau)
        d = o["diag"]   # fp32 logit weights in the kernel: the contract's 1e-5 band
        bnd = (d["accept_margin"] <= 1e-5) | (d["draw_margin"] <= 1e-5) | (d["draw_kind"] >= 4)
    elif mode == "sampled":
        o = oracle.verify_sample(hb.target_probs, hb.draft_probs, hb.draft_tokens, hb.uniforms)
        d = o["diag"]   # fp64 masses on both sides: a 1e-9 band
        bnd = (d["accept_margin"] <= 1e-9) | (d["draw_margin"] <= 1e-9)
    else:
        o = oracle.verify_greedy(hb.target_probs, hb.draft_tokens)
        bnd = np.zeros(len(seqs), bool)
    ok = (n == o["n_accepted"]) & (x == o["next_token"])
    if not np.all(ok | bnd):
        raise SystemExit(f"benchmark outputs differ from the oracle: gpu {n},{x} oracle "
                         f"{o['n_accepted']},{o['next_token']}")
    if stats is not None:
        import speculative_decoding_verification_row_amd as sv
        g = sv.stats_to_numpy(stats)[seqs]
        ref = o["stats"]
        if not (np.array_equal(g["argmax"], ref["argmax"]) and
                float(np.max(np.abs(g["sum_p"] - ref["sum_p"]) / ref["sum_p"])) <= 1e-9):
            raise SystemExit("benchmark row statistics differ from the oracle")
    return f"{int(ok.sum())}/{len(seqs)} sequences identical to the oracle ({int(bnd.sum())} boundary)"


if __name__ == "__main__":
    main()
