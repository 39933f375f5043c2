"""Benchmark of the attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one fa_fwd call over the whole batch of the full workload
(B16 N4096 H16 d128 bf16, non-causal, seeded N(0,1) inputs resident in HBM before
timing; the tile configuration is the one the library's autotuner picks on those buffers
before timing -- every compiled configuration timed in interleaved rounds -- or, with
--no-tune, the built-in choice).  Prints ONE JSON line with the throughput in TFLOP/s
(4 * B * H * Nq * Nk * d per step), the roofline figures of the kernel and the
fp64 oracle timed on a bounded sample on the host cores.

Other modes (used to produce the committed profiles and the secondary measurements):
    --workload NAME     time another named workload (tiny, slice, full, small_head, varlen,
                        causal, gqa); causal counts only the visible (query, key) pairs
    --splits N          key-range splits per query tile (fa_fwd_ext num_splits): 0 = the
                        library's automatic choice (default), 1 = no split
    --pass bwd          time the backward pass (fa_bwd: preprocess, main and dQ kernels) on
                        the workload instead, with O and LSE from one forward call and a
                        seeded dO; FLOPs counted as 2.5x the forward's (five products
                        instead of two, the pages' convention)
    --atomic-dq         with --pass bwd: dQ by atomic adds instead of the separate dQ pass
    --copy-bytes N      run only a plain device copy of N bytes (the counter calibration)
    --no-cpu-baseline   skip the oracle timing
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA: 256 CU x 4 SIMD x 1024 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
HEADLINE_METRIC = "fwd TFLOP/s (4BHN\u00b2d) at B16\u00b7N4096\u00b7H16\u00b7d128 bf16; % of MFMA bf16 peak"
WORKLOAD_NAMES = {
    "full": "full B16 N4096 H16 d128 bf16 non-causal",
    "tiny": "tiny B1 N128 H2 d64 bf16",
    "slice": "slice B1 Nq64 Nk4096 H1 d128 bf16",
    "small_head": "small_head B64 N512 H16 d32 fp16",
    "varlen": "varlen 8 seqs U[512,8192] H16 d128 bf16",
    "causal": "causal B16 N4096 H16 d128 bf16 (top-left causal mask)",
    "gqa": "gqa B16 N4096 H16 Hkv2 d128 bf16 non-causal",
}


def device_peak():
    """Dense bf16 MFMA peak from the device's own CU count and maximum clock (rocminfo), as
    CUs x 4 SIMD x 1024 FLOP/clk x clock; None when rocminfo is unavailable."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    cus = clock = None
    in_gpu = False
    for line in txt.splitlines():
        line = line.strip()
        if line.startswith("Name:") and "gfx" in line:
            in_gpu = True
        elif in_gpu and line.startswith("Max Clock Freq. (MHz):"):
            clock = int(line.split(":")[1].split()[0])
        elif in_gpu and line.startswith("Compute Unit:"):
            cus = int(line.split(":")[1].split()[0])
        if cus and clock:
            break
    if not (cus and clock):
        return None
    return {"cus": cus, "max_clock_mhz": clock, "peak_tflops": round(cus * 4 * 1024 * clock * 1e6 / 1e12, 1)}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _code_only(text):
    """C++ source with comments and whitespace removed (string literals kept), so that
    editing a comment does not count as a kernel change."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            i = text.find("*/", i + 2)
            i = n if i < 0 else i + 2
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return "".join(out)


def kernel_source_hash():
    """Hash of the forward kernel's device sources (the kernel template, the shared argument
    header and the instantiation units), comments and whitespace aside; counter-derived
    traffic is only reported for the same kernel."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "exact_attention_17_amd", "csrc", "*"))):
        base = os.path.basename(p)
        if base == "fa_internal.h" or (base.startswith("fa_fwd_") and base.endswith((".h", ".hip"))):
            with open(p, encoding="utf-8") as f:
                h.update(base.encode())
                h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload, cfg, splits):
    """HBM bytes per launch from a committed rocprofv3 counter summary of the workload
    (profiles/fa_fwd_<workload>_traffic.txt for the tile the tuner picked when it was taken,
    profiles/fa_fwd_<workload>_<tile>_traffic.txt for other tiles; "key: value" lines): the one
    taken on the current kernel sources with this tile configuration and split count, else None."""
    tile = ",".join(str(x) for x in cfg.as_tuple())
    paths = [os.path.join(ROOT, "profiles", "fa_fwd_%s_traffic.txt" % workload),
             os.path.join(ROOT, "profiles", "fa_fwd_%s_%s_traffic.txt" % (workload, tile.replace(",", "-")))]
    for path in paths:
        vals = {}
        try:
            with open(path) as f:
                for line in f:
                    if line.startswith("#") or ":" not in line:
                        continue
                    key, val = line.split(":", 1)
                    vals[key.strip()] = val.strip()
        except OSError:
            continue
        if vals.get("kernel_source_hash") != kernel_source_hash() or vals.get("workload") != workload:
            continue
        if vals.get("tile") != tile or vals.get("num_splits") != str(splits):
            continue
        try:
            return int(float(vals["hbm_bytes_per_launch"]))
        except (KeyError, ValueError):
            continue
    return None


def copy_calibration(nbytes, reps):
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log("copy calibration: %d launches of a %d-byte device copy" % (reps, n * 4))


def cpu_baseline(w, target_s=12.0):
    """The oracle, as it stands, on sampled query rows of batch entry 0 (each row against all
    keys): calibrate on a few rows, then run about target_s seconds."""
    import numpy as np

    import oracle
    from exact_attention_17_amd import inputs
    if w["cu_seqlens"] is not None:
        s0, s1 = int(w["cu_seqlens"][0]), int(w["cu_seqlens"][1])
        q, k, v = (inputs.to_f64(t[None, s0:s1]) for t in (w["q"], w["k"], w["v"]))
        nq = nk = s1 - s0
    else:
        q, k, v = (inputs.to_f64(t[0:1]) for t in (w["q"], w["k"], w["v"]))
        nq, nk = w["seqlen_q"], w["seqlen_k"]
    heads, d, causal = w["heads"], w["d_head"], w["causal"]
    rng = np.random.default_rng(0)
    picked = []

    def rows(n):
        r = [(0, int(rng.integers(heads)), int(rng.integers(nq))) for _ in range(n)]
        picked[:] = r
        return r

    def run(n):
        oracle.attention_rows(q, k, v, w["scale"], rows(n), causal=causal)

    run(8)  # warm (threads, pages)
    n = 64
    t0 = time.perf_counter()
    run(n)
    t = time.perf_counter() - t0
    n = int(min(max(n * target_s / max(t, 1e-6), 64), 200000))
    t0 = time.perf_counter()
    run(n)
    t = time.perf_counter() - t0
    # work of the sampled rows: each row against its visible keys
    flops = 4.0 * d * sum((min(i + 1, nk) if causal else nk) for (_, _, i) in picked)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d random query rows of batch entry 0 (%s %d keys, d %d), fp64, %.1f s"
                      % (n, "visible ones of" if causal else "all", nk, d, t)}


def setup(name, dev, splits=0, which="fwd", atomic_dq=False, tune=True, tune_rounds=5):
    """Inputs of a named workload resident on `dev`, output buffers, and the step the benchmark
    times: one fa_fwd_ext call (or, for which="bwd", one fa_bwd call after one forward call).
    With tune, the library's autotuner first times every compiled tile configuration on these
    buffers (fa_fwd_autotune_ext, interleaved median timing) and the step then runs its pick.
    The parity tests launch through this same function.  Returns a dict with w (the workload),
    o, lse, step, cfg (the forward tile configuration), source (where the library took it from:
    default, tuned, FA_FWD_CONFIG or forced), splits, tuned (the tuner's report or None), flops,
    nbytes, stream and desc."""
    import torch

    from exact_attention_17_amd import fa, inputs, metrics

    w = inputs.workload(name)
    qd, kd, vd = w["q"].to(dev), w["k"].to(dev), w["v"].to(dev)
    cu = w["cu_seqlens"].to(dev) if w["cu_seqlens"] is not None else None
    o = torch.empty_like(qd)
    lse = torch.empty((w["batch"], w["heads"], w["seqlen_q"]), dtype=torch.float32, device=dev)
    causal, hkv = w["causal"], w["heads_kv"]
    if cu is None:
        flops = metrics.fwd_flops(w["batch"], w["heads"], w["seqlen_q"], w["seqlen_k"], w["d_head"], causal)
        nbytes = metrics.fwd_bytes(w["batch"], w["heads"], w["seqlen_q"], w["seqlen_k"], w["d_head"],
                                   heads_kv=hkv)
    else:
        flops = metrics.varlen_fwd_flops(w["lengths"], w["heads"], w["d_head"], causal)
        nbytes = metrics.varlen_fwd_bytes(w["lengths"], w["heads"], w["d_head"], heads_kv=hkv)
    dtype_code = fa.FA_FP16 if w["dtype"] == "fp16" else fa.FA_BF16
    shape = (w["batch"], w["seqlen_q"], w["seqlen_k"], w["heads"], w["d_head"])
    stream = torch.cuda.current_stream(dev)
    # Split workspace, allocated before timing (the library allocates nothing).  With the
    # automatic count (splits = 0) every tile configuration may pick its own: room for the
    # largest count, within 256 MiB (the library lowers a count to what the workspace holds).
    want = splits if splits > 0 else fa.FA_MAX_SPLITS
    ws_bytes = fa.fa_fwd_workspace_bytes(w["batch"], w["seqlen_q"], w["heads"], w["d_head"], want)
    ws_bytes = min(ws_bytes, 256 << 20) // 16 * 16
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    tuned = None
    if tune and which == "fwd":
        chosen, ms = fa.fa_fwd_autotune_ext(qd, kd, vd, o, lse, scale=w["scale"], causal=causal, cu_seqlens=cu,
                                            max_seqlen=w["max_seqlen"], num_splits=splits, workspace=workspace,
                                            rounds=tune_rounds, stream=stream)
        ranking = fa.fa_fwd_tune_ranking()
        tuned = {"tuned": True, "candidates": len(ranking), "rounds": tune_rounds, "median_ms": round(ms, 5),
                 "runner_up": {"tile": list(ranking[1][0].as_tuple()), "median_ms": round(ranking[1][1], 5)}
                 if len(ranking) > 1 else None}
    cfg, auto_splits, source = fa.fa_fwd_query_config(*shape, dtype_code, n_heads_kv=hkv, varlen=cu is not None,
                                                      causal=causal)
    if splits == 0:  # the count fa_fwd_ext will use: the automatic one, lowered to the workspace
        splits = auto_splits
        while splits > 1 and fa.fa_fwd_workspace_bytes(w["batch"], w["seqlen_q"], w["heads"], w["d_head"],
                                                       splits) > ws_bytes:
            splits -= 1
        req_splits = 0
    else:
        req_splits = splits

    def step():
        fa.fa_fwd_ext(qd, kd, vd, o, lse, scale=w["scale"], causal=causal, cu_seqlens=cu,
                      max_seqlen=w["max_seqlen"], num_splits=req_splits, workspace=workspace, stream=stream)

    out = dict(w=w, o=o, lse=lse, step=step, cfg=cfg, source=source, splits=splits, tuned=tuned, flops=flops,
               nbytes=nbytes, stream=stream, desc="fa_fwd_ext tiles %r (%s), %d split(s)" % (cfg, source, splits))
    if which == "bwd":
        step()  # O and LSE of this workload
        g = torch.Generator().manual_seed(int(w["seed"]) + 1000)
        dout = torch.randn(tuple(qd.shape), generator=g, dtype=torch.float32).to(qd.dtype).to(dev)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        bws = torch.empty(fa.fa_bwd_workspace_bytes(w["batch"], w["seqlen_q"], w["heads"], w["d_head"],
                                                    atomic_dq), dtype=torch.uint8, device=dev)
        # algorithmic bytes: Q, K, V, O, dO read and dQ, dK, dV written (16-bit), LSE read and
        # D, L log2(e) written once (fp32 per query row)
        out["flops"] = flops * 5 // 2
        out["nbytes"] = 2 * nbytes + 2 * 4 * qd.numel() // w["d_head"]

        def bstep():
            fa.fa_bwd(qd, kd, vd, o, lse, dout, dq, dk, dv, scale=w["scale"], causal=causal, cu_seqlens=cu,
                      max_seqlen=w["max_seqlen"], atomic_dq=atomic_dq, workspace=bws, stream=stream)
        out.update(step=bstep, dq=dq, dk=dk, dv=dv, desc="fa_bwd atomic_dq=%d" % int(bool(atomic_dq)))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clock needs about twenty launches of the full workload to settle: with five
    # warmup steps the timed region ran about 8% (causal: 17%) slower than in steady state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="full")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd")
    ap.add_argument("--atomic-dq", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tune", action="store_true", help="time the built-in tile choice, without tuning")
    ap.add_argument("--tune-rounds", type=int, default=5)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(every (batch, head, query tile) is independent; see the sharding notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from exact_attention_17_amd import fa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.lib()
    if args.copy_bytes:
        copy_calibration(args.copy_bytes, max(args.steps, 1))
        return

    dev = torch.device("cuda:0")
    log("generating inputs for workload %s" % args.workload)
    st = setup(args.workload, dev, splits=args.splits, which=args.which, atomic_dq=args.atomic_dq,
               tune=not args.no_tune, tune_rounds=args.tune_rounds)
    if st["tuned"]:
        log("tuned over %d configurations: %r, median %.4f ms" % (st["tuned"]["candidates"], st["cfg"],
                                                                 st["tuned"]["median_ms"]))
    w, cfg, splits, flops, nbytes, step = st["w"], st["cfg"], st["splits"], st["flops"], st["nbytes"], st["step"]
    stream = st["stream"]
    causal, hkv = w["causal"], w["heads_kv"]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: events on the stream the kernel is launched on.
    # (an event between launches as well, for the per-launch median and minimum)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_launch = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    tflops = flops / (ms * 1e-3) / 1e12
    log("%s %s: %.4f ms per step (wall %.4f ms), %.1f TFLOP/s, %.1f%% of %.1f, forward tiles %r, splits %d"
        % (args.workload, args.which, ms, wall * 1e3 / args.steps, tflops, 100 * tflops / PEAK_BF16_TFLOPS,
           PEAK_BF16_TFLOPS, cfg, splits))

    traffic = read_traffic(args.workload, cfg, splits) if args.which == "fwd" else None
    cpu = None
    if not args.no_cpu_baseline and args.which == "fwd":
        log("timing the fp64 oracle on a bounded sample")
        cpu = cpu_baseline(w)
        log("oracle: %.3g TFLOP/s on %d threads (%s)" % (cpu["value"], cpu["cores"], cpu["sample"]))

    wl = WORKLOAD_NAMES[args.workload]
    metric = HEADLINE_METRIC if args.workload == "full" and args.which == "fwd" else \
        "%s TFLOP/s (%s x 4 d x visible query-key pairs per batch and head) on %s; %% of MFMA bf16 peak" % (
            args.which, "2.5" if args.which == "bwd" else "1", wl)
    out = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded N(0,1), rounded to %s)" % w["dtype"],
        "config": {"workload": wl, "batch": w["batch"], "seq_len_q": w["seqlen_q"], "seq_len_k": w["seqlen_k"],
                   "heads": w["heads"], "heads_kv": hkv, "d_head": w["d_head"], "causal": causal,
                   "tile": ({"br": cfg.br, "bc": cfg.bc, "waves": cfg.waves, "stages": cfg.stages,
                             "schedule": cfg.schedule, "tuned": st["source"] == "tuned", "source": st["source"]}
                            if args.which == "fwd" else
                            {"dkdv_keys_per_workgroup": 64 if w["d_head"] == 32 else 128,
                             "dq_pass_rows_per_workgroup": 256 if w["d_head"] == 128 else 128}),
                   "num_splits": splits, "pass": args.which,
                   "atomic_dq": bool(args.atomic_dq) if args.which == "bwd" else None, "parallelism": "single GPU"},
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "algorithmic_bytes": nbytes,
                     "algorithmic_flops": flops,
                     # the HBM roofline beside it: algorithmic bytes per launch over its time
                     "hbm_achieved_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "cpu_baseline": cpu,
        "tuning": st["tuned"],
        "launch_ms": {"median": round(per_launch[len(per_launch) // 2], 5), "min": round(per_launch[0], 5)},
        "device_peak": device_peak(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
