#!/usr/bin/env python
"""Benchmark of the tree-attention + tree-verification hot path on one MI355X.

Metric (per layer): draft tokens per second of tree attention + verification,
B N / (t_attn + t_verify), over one batch of draft trees; tree build and KV
compaction sit outside it and are reported beside it (the whole step). Inputs
are seeded synthetic tensors (``workloads``), resident in HBM before timing.

The headline line is the mixed serving batch (32 sequences, prefixes of 512 to
16384 tokens, 32-node trees, half greedy and half sampling at T = 0.7), the
largest of the five workloads that fits one GPU; ``per_config`` repeats the
measurement on every workload.

To keep the 256 MB Infinity Cache from serving repeated steps, each timed loop
cycles through R device replicas of every input (R * replica >= --rotate-gib).
Each replica's step is captured once in a HIP graph; a timed loop replays the
graphs back to back, bracketed by torch.cuda.synchronize() on both sides, with
HIP events on the stream the graphs run on.

Prints ONE JSON line. Its "roofline" object is for the attention call (the
dominant kernel, tree_attn_kernel, plus the split-K combine when prefixes are
split) and "cpu_baseline" is the CPU oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
PMC_COPY_BYTES = 256 << 20  # calibration copy of --profile-kernels
BF16_DENSE_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP8_DENSE_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
HEADLINE = "mixed_serving_b32"
METRIC = "tree-attn+verify draft tokens/s per layer; achieved HBM GB/s vs MI355X peak"


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def clone_device_workload(dw):
    import copy

    c = copy.copy(dw)
    for name, val in vars(dw).items():
        if hasattr(val, "clone") and hasattr(val, "device"):
            setattr(c, name, val.clone())
    return c


def algorithmic_work(w, host):
    """Bytes / flops the method must move / compute per step (per stage)."""
    import numpy as np

    B, d, Hq, Hkv, V = w.B, w.d, w.Hq, w.Hkv, w.V
    L = w.prefix_lens.astype(np.int64)
    T = w.T_b.astype(np.int64)
    attn_bytes = int((L * Hkv * d * 2 * 2).sum() + (T * Hkv * d * 2 * 2).sum() + 2 * (T * Hq * d * 2).sum())
    # visible tree keys per node = depth + 1 (root, ancestors, itself)
    tree_keys = int(sum((host["depth"][b, : T[b]] + 1).sum() for b in range(B)))
    attn_flops = int(4 * d * Hq * ((T * L).sum() + tree_keys))
    ver_rows = 0
    for b in range(B):
        ver_rows += int(T[b])
        if w.modes[b] == 1:
            par = host["parents"][b, 1 : T[b]]
            ver_rows += len(set(int(p) for p in par))  # q rows of internal nodes
    verify_bytes = ver_rows * V * 4
    build_rows = int(sum(1 + (int(w.depth[b]) - 1) * int(w.topk[b]) for b in range(B)))
    build_bytes = build_rows * w.draft_logprobs.shape[-1] * 4  # draft rows: V, or the truncated vocabulary
    return dict(attn_bytes=attn_bytes, attn_flops=attn_flops, verify_bytes=verify_bytes, build_bytes=build_bytes)


def pmc_traffic(workload):
    """HBM bytes per attention call (main kernel + combine) from the committed rocprofv3 --pmc summary of this
    workload, or None when there is none or the kernel source changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"tree_attn_kernel_{workload}_pmc.md")
    src = os.path.join(ROOT, "tree_attention_verification_03_amd", "csrc", "tree_attention.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- `"):
                k, _, v = line[3:].partition("`:")
                fields[k.strip()] = v.strip().strip("`")
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != digest:
        return None
    try:
        return int(float(fields["traffic_bytes_per_call"]))
    except (KeyError, ValueError):
        return None



def measure_fp8(w, steps, bf16_call_ms, args, torch):
    """The FP8-KV variant of the attention call (spec_tree_attention_fp8) on the same trees and queries, E4M3
    pools drawn for the workload's shape: back-to-back calls in one graph over >= --rotate-gib of pools."""
    import numpy as np

    from tree_attention_verification_03_amd import ops
    from workloads.synth import fp8_kv_pools

    eprint("[bench] FP8-KV variant: drawing E4M3 pools")
    k8, v8, ks, vs = fp8_kv_pools(w.k_pages.shape, seed=1)
    dev = steps[0].dw.device
    per = k8.nbytes + v8.nbytes
    Rf = int(min(512, max(2, np.ceil(args.rotate_gib * 2**30 / per))))
    kt, vt = torch.from_numpy(k8).to(dev), torch.from_numpy(v8).to(dev)
    pools = [(kt, vt)] + [(kt.clone(), vt.clone()) for _ in range(Rf - 1)]
    kst, vst = torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev)

    def call(i):
        st = steps[i % len(steps)]
        o, d = st.o, st.dw
        k, v = pools[i]
        ops.spec_tree_attention_fp8(d.q, k, v, kst, vst, d.page_table, d.prefix_lens, o.parents, d.T_b, d.w.sm_scale,
                                    o.attn_out, o.lse, None, st.ws_attn)

    for i in range(Rf):
        call(i)
    torch.cuda.synchronize()

    def chain():
        for i in range(Rf):
            call(i)

    g = capture(chain, torch)
    time_graphs([g], 2, torch)
    ms = time_graphs([g], max(4, args.steps // Rf), torch)[0] / Rf
    L = w.prefix_lens.astype(np.int64)
    T = w.T_b.astype(np.int64)
    nbytes = int((L * w.Hkv * w.d * 2).sum() + (T * w.Hkv * w.d * 2).sum() + 2 * (T * w.Hq * w.d * 2).sum())
    host_depth = steps[0].o.depth.cpu().numpy()
    tree_keys = int(sum((host_depth[b, : T[b]] + 1).sum() for b in range(w.B)))
    flops = int(4 * w.d * w.Hq * ((T * L).sum() + tree_keys))
    t = ms * 1e-3
    eprint(f"[bench] FP8-KV attention call, back-to-back: {ms * 1e3:.2f} us per call ({Rf} pool replicas)")
    bound = "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (FP8_DENSE_TFLOPS * 1e12) else "mfma"
    del pools, g
    return dict(attn_us=round(ms * 1e3, 3), speedup_vs_bf16=round(bf16_call_ms / ms, 3), bound=bound,
                bytes_per_call=nbytes, achieved_gbs=round(nbytes / t / 1e9, 1),
                hbm_frac=round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4), flops_per_call=flops,
                achieved_tflops=round(flops / t / 1e12, 2), fp8_mfma_frac=round(flops / t / 1e12 / FP8_DENSE_TFLOPS, 4),
                kernel="tree_attn_fp8_kernel + tree_attn_combine (E4M3 K/V with per-head scales, E4M3 MFMA)",
                replicas=Rf)

def time_graphs(graphs, n, torch):
    """Replay graphs round-robin n times; returns (gpu ms per replay, wall ms per replay)."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s.record()
    for i in range(n):
        graphs[i % len(graphs)].replay()
    e.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / n
    return s.elapsed_time(e) / n, wall


def capture(fn, torch):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def cpu_baseline(w, seconds):
    """The oracle as it stands, on the host cores: whole oracle steps of the same workload, at least one, until
    ``seconds`` have passed; attention + verification timed apart from the tree build (the metric's steps)."""
    import numpy as np

    import oracle
    from workloads.synth import bf16_bits_to_f32

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(cores) if threadpool_limits else None
    qf = bf16_bits_to_f32(w.q).astype(np.float64)
    kf, vf = bf16_bits_to_f32(w.k_pages), bf16_bits_to_f32(w.v_pages)
    steps = 0
    t_build = t_av = 0.0
    t0 = time.perf_counter()
    while True:
        ta = time.perf_counter()
        trees = [oracle.tree.build_tree(w.draft_logprobs[b], int(w.root_tokens[b]), int(w.topk[b]), int(w.depth[b]),
                                        int(w.num_draft[b]), w.max_topk, token_map=w.token_map) for b in range(w.B)]
        par = np.full((w.B, w.max_T), -1, dtype=np.int32)
        for b, t in enumerate(trees):
            par[b, : len(t.parents)] = t.parents
        tb = time.perf_counter()
        oracle.attention.tree_attention(qf, kf, vf, w.page_table, w.prefix_lens, par, w.T_b, w.sm_scale)
        for b, t in enumerate(trees):
            oracle.verify.verify_sequence(w.target[b], w.draft_probs[b], t.q_row, t.tokens, t.parents, int(w.T_b[b]),
                                          int(w.modes[b]), w.philox_key, w.philox_offset, b)
        tc = time.perf_counter()
        t_build += tb - ta
        t_av += tc - tb
        steps += 1
        if tc - t0 >= seconds:
            break
    threads = cores
    if threadpool_info:
        info = threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
    if ctx is not None:
        ctx.unregister() if hasattr(ctx, "unregister") else None
    n_draft = int(w.num_draft.sum())
    return dict(value=round(n_draft * steps / t_av, 3), unit="draft tokens/s", cores=threads, kind="oracle",
                cpu=platform.processor() or platform.machine(),
                whole_step_draft_tokens_per_s=round(n_draft * steps / (t_av + t_build), 3),
                sample=f"{steps} full oracle step(s) on the same {w.name} workload: tree attention over all "
                f"{w.B} x {w.Hq} sequence x head pairs + verification of all {w.B} trees took {t_av:.1f} s "
                f"(the value: {n_draft} draft tokens per step / that time), the tree build {t_build:.1f} s more")


def measure(spec, args, torch, profile_mode=False):
    """Measure one workload; returns (result dict, workload) or None in profile mode."""
    import numpy as np

    from tree_attention_verification_03_amd import ops
    from tree_attention_verification_03_amd.pipeline import DeviceWorkload, SpecTreeStep
    from workloads.synth import from_spec

    eprint(f"[bench] workload {spec.name}: generating inputs")
    w = from_spec(spec, draft_vocab=args.draft_vocab)
    dw0 = DeviceWorkload(w, logits=args.verify_logits)
    per_replica = sum(t.numel() * t.element_size() for t in vars(dw0).values() if hasattr(t, "element_size"))
    R = max(2, int(np.ceil(args.rotate_gib * 2**30 / per_replica)))
    R = min(R, 512)
    eprint(f"[bench] replica {per_replica / 2**20:.1f} MiB x {R} replicas")
    replicas = [dw0] + [clone_device_workload(dw0) for _ in range(R - 1)]
    steps = [SpecTreeStep(d, attn_status=False, verify_from_logits=args.verify_logits) for d in replicas]
    compact = bool(spec.compact)

    # eager warm-up and the reference outputs of replica 0
    for st in steps:
        st.run(compact=compact)
    torch.cuda.synchronize()
    ref = {k: getattr(steps[0].o, k).clone() for k in ("accept_len", "out_tokens", "attn_out")}
    host = {k: getattr(steps[0].o, k).cpu().numpy() for k in ("depth", "parents")}

    def attn_only(st):
        o, d = st.o, st.dw
        return lambda: ops.spec_tree_attention(d.q, d.k_pages, d.v_pages, d.page_table, d.prefix_lens, o.parents,
                                               d.T_b, d.w.sm_scale, o.attn_out, o.lse, None, st.ws_attn)

    def attn_verify(st):
        def f():
            attn_only(st)()
            st.verify()
        return f

    if profile_mode:
        if args.profile_op == "attention_fp8":
            from workloads.synth import fp8_kv_pools

            k8, v8, ks, vs = fp8_kv_pools(w.k_pages.shape, seed=1)
            dev = dw0.device
            kt, vt = torch.from_numpy(k8).to(dev), torch.from_numpy(v8).to(dev)
            Rf = int(min(512, max(2, np.ceil(args.rotate_gib * 2**30 / (k8.nbytes + v8.nbytes)))))
            pools = [(kt, vt)] + [(kt.clone(), vt.clone()) for _ in range(Rf - 1)]
            kst, vst = torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev)

            def fp8_call(i):
                st = steps[i % R]
                return lambda: ops.spec_tree_attention_fp8(st.dw.q, pools[i % Rf][0], pools[i % Rf][1], kst, vst,
                                                           st.dw.page_table, st.dw.prefix_lens, st.o.parents,
                                                           st.dw.T_b, w.sm_scale, st.o.attn_out, st.o.lse, None,
                                                           st.ws_attn)
            for i in range(args.profile_kernels):
                fp8_call(i)()
        else:
            op = {"attention": attn_only, "verify": lambda st: st.verify, "build": lambda st: st.build}[args.profile_op]
            for i in range(args.profile_kernels):
                op(steps[i % R])()
        torch.cuda.synchronize()
        src = torch.empty(PMC_COPY_BYTES, dtype=torch.uint8, device=dw0.device)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        eprint(f"[bench] profile mode: {args.profile_kernels} {args.profile_op} calls, one "
               f"{PMC_COPY_BYTES >> 20} MiB copy")
        return None

    class _Eager:
        def __init__(self, f):
            self.replay = f

    make = (lambda f: _Eager(f)) if args.eager else (lambda f: capture(f, torch))
    if not args.eager:
        eprint("[bench] capturing HIP graphs")
    av = [make(attn_verify(st)) for st in steps]
    full = [make(lambda st=st: st.run(compact=compact)) for st in steps]
    stage = {"build": [make(st.build) for st in steps], "attention": [make(attn_only(st)) for st in steps],
             "verify": [make(st.verify) for st in steps]}
    attn_chain = None
    if not args.eager:
        def all_attn():
            for st in steps:
                attn_only(st)()

        # one graph holding the attention call of every replica: back-to-back kernels, no per-graph gaps
        attn_chain = capture(all_attn, torch)
        # a replay must reproduce the eager result
        full[0].replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            got = getattr(steps[0].o, k)
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               v.view(torch.int16) if v.dtype == torch.bfloat16 else v), f"graph replay differs: {k}"

    # the metric's step: attention + verification, W untimed, then exactly K timed
    time_graphs(av, args.warmup, torch)
    eprint(f"[bench] timing {args.steps} attention + verify steps")
    gpu_ms, wall_ms = time_graphs(av, args.steps, torch)
    time_graphs(full, max(3, args.warmup // 4), torch)
    full_gpu_ms, full_wall_ms = time_graphs(full, args.steps, torch)
    stage_ms = {}
    for name, gs in stage.items():
        time_graphs(gs, max(5, args.warmup // 4), torch)
        stage_ms[name] = time_graphs(gs, max(20, args.steps // 2), torch)[0]
        eprint(f"[bench] stage {name}: {stage_ms[name] * 1e3:.2f} us")

    attn_call_ms = stage_ms["attention"]
    if attn_chain is not None:
        reps = max(4, args.steps // R)
        time_graphs([attn_chain], 2, torch)
        attn_call_ms = time_graphs([attn_chain], reps, torch)[0] / R
        eprint(f"[bench] attention call, back-to-back: {attn_call_ms * 1e3:.2f} us per call")

    fp8 = measure_fp8(w, steps, attn_call_ms, args, torch) if (w.d == 128 and not args.eager and not args.no_fp8) else None

    work = algorithmic_work(w, host)
    n_draft = int(w.num_draft.sum())
    t_attn = attn_call_ms * 1e-3
    attn_gbs = work["attn_bytes"] / t_attn / 1e9
    attn_tfs = work["attn_flops"] / t_attn / 1e12
    t_hbm = work["attn_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = work["attn_flops"] / (BF16_DENSE_TFLOPS * 1e12)
    traffic = pmc_traffic(spec.name) if not (args.verify_logits or args.draft_vocab) else None
    if t_hbm >= t_mfma:
        roof = dict(bound="hbm", achieved=round(attn_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(attn_gbs / HBM_PEAK_GBS, 4), traffic=traffic)
    else:
        roof = dict(bound="mfma", achieved=round(attn_tfs, 2), peak=BF16_DENSE_TFLOPS, unit="TFLOP/s",
                    frac=round(attn_tfs / BF16_DENSE_TFLOPS, 4), traffic=traffic)
    roof.update(kernel="tree_attn_kernel + tree_attn_combine (one spec_tree_attention call)",
                bytes_per_launch=work["attn_bytes"], flops_per_launch=work["attn_flops"],
                avg_launch_us=round(t_attn * 1e6, 3),
                timing="HIP events around a graph of back-to-back spec_tree_attention calls, one per replica; a "
                       "call is the main kernel plus, for split prefixes, the combine kernel",
                traffic_unit="HBM bytes per call, both kernels (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)")
    res = dict(
        workload=spec.name, value=round(n_draft / (gpu_ms * 1e-3), 1), ms_per_step=round(gpu_ms, 5),
        wall_ms_per_step=round(wall_ms, 5), verified_seqs_per_s=round(w.B / (gpu_ms * 1e-3), 1),
        full_step_us=round(full_gpu_ms * 1e3, 3),
        full_step_draft_tokens_per_s=round(n_draft / (full_gpu_ms * 1e-3), 1),
        stage_us={k: round(v * 1e3, 3) for k, v in stage_ms.items()},
        verify_hbm_gbs=round(work["verify_bytes"] / (stage_ms["verify"] * 1e-3) / 1e9, 1),
        roofline=roof, replicas=R, batch=w.B, draft_tokens=n_draft)
    if fp8 is not None:
        res["fp8_variant"] = fp8
    del av, full, stage, attn_chain, steps, replicas, dw0
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, w


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default=HEADLINE, help="headline workload, name or index (0-4)")
    ap.add_argument("--per-config", choices=["all", "none"], default="all",
                    help="also measure every other workload (the line's per_config object)")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle: whole oracle steps until this many seconds have passed (at least one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-KV attention variant's timing")
    ap.add_argument("--verify-logits", action="store_true",
                    help="verify with spec_tree_verify_logits (sampling distributions formed from the target logits and "
                         "temperatures inside the library) instead of supplied probabilities")
    ap.add_argument("--draft-vocab", type=int, default=None, metavar="N",
                    help="truncated draft vocabulary: draft rows over N tokens with a token map into the target's "
                         "vocabulary (frequency-ranked speculative sampling)")
    ap.add_argument("--details", default=None, help="write the line and per-stage details as JSON to this path")
    ap.add_argument("--profile-kernels", type=int, default=0, metavar="N",
                    help="profiling mode (run under rocprofv3): N eager calls of --profile-op over the replicas of the "
                         "--config workload, then one 256 MiB device-to-device copy whose counters calibrate "
                         "FETCH_SIZE / WRITE_SIZE; no timing")
    ap.add_argument("--profile-op", choices=["attention", "attention_fp8", "verify", "build"], default="attention")
    args = ap.parse_args()

    if args.gpus != 1:
        eprint("bench.py: this build runs on exactly one GPU; --gpus must be 1 (no multi-GPU path is built).")
        sys.exit(2)

    import torch

    from workloads import CONFIGS, get_config

    cfg_key = int(args.config) if args.config.isdigit() else args.config
    spec = get_config(cfg_key)
    if args.profile_kernels:
        measure(spec, args, torch, profile_mode=True)
        return

    head, w = measure(spec, args, torch)
    per_config = {spec.name: {k: v for k, v in head.items() if k != "workload"}}
    if args.per_config == "all":
        for other in CONFIGS:
            if other.name != spec.name:
                r, _ = measure(other, args, torch)
                per_config[other.name] = {k: v for k, v in r.items() if k != "workload"}

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "prefix": [int(w.prefix_lens.min()), int(w.prefix_lens.max())],
                   "draft_tokens": int(w.num_draft.max()), "vocab": w.V,
                   "step": "tree attention + verification (the metric); tree build"
                           + (" and KV compaction" if spec.compact else "") + " in full_step_us",
                   "replicas": head["replicas"], "graphs": not args.eager,
                   "verify_input": "target logits + temperature" if args.verify_logits else "target probabilities",
                   "draft_vocab": int(w.draft_logprobs.shape[-1])},
        "verified_seqs_per_s": head["verified_seqs_per_s"],
        "full_step_us": head["full_step_us"],
        "full_step_draft_tokens_per_s": head["full_step_draft_tokens_per_s"],
        "stage_us": head["stage_us"],
        "verify_hbm_gbs": head["verify_hbm_gbs"],
        "roofline": head["roofline"],
        "fp8_variant": head.get("fp8_variant"),
        "per_config": per_config,
    }
    if not args.no_cpu_baseline:
        eprint(f"[bench] CPU oracle baseline (at least one whole oracle step, ~{args.cpu_seconds:.0f} s or more)")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    if args.details:
        with open(args.details, "w") as f:
            json.dump(line, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
