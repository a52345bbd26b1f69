#!/usr/bin/env python
"""Benchmark of the tree-attention + tree-verification hot path on one MI355X.

A step is one pass of the whole path over one batch: EAGLE-2 tree build (one
call per depth + finish), tree attention over the paged prefix, verification
(+ accepted-path KV compaction on workloads that include it). Inputs are
seeded synthetic tensors (``workloads``), resident in HBM before timing.

To keep the 256 MB Infinity Cache from serving repeated steps, the timed loop
cycles through R device replicas of every input (R * replica >= --rotate-gib).
Each replica's step is captured once in a HIP graph; the timed region replays
the graphs back to back, bracketed by torch.cuda.synchronize() on both sides.

Prints ONE JSON line (see the "roofline" and "cpu_baseline" objects for the
dominant kernel's roofline and the CPU oracle baseline).
"""
from __future__ import annotations

import argparse
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
    """HBM bytes per attention launch from the committed rocprofv3 --pmc summary of this workload, or
    None when there is none or the kernel source changed since the counters were taken."""
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
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


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
    """The oracle as it stands, on the host cores, over whole steps of the same workload."""
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
    t0 = time.perf_counter()
    while True:
        trees = [oracle.tree.build_tree(w.draft_logprobs[b], int(w.root_tokens[b]), int(w.topk[b]), int(w.depth[b]),
                                        int(w.num_draft[b]), w.max_topk, token_map=w.token_map) for b in range(w.B)]
        par = np.full((w.B, w.max_T), -1, dtype=np.int32)
        for b, t in enumerate(trees):
            par[b, : len(t.parents)] = t.parents
        oracle.attention.tree_attention(qf, kf, vf, w.page_table, w.prefix_lens, par, w.T_b, w.sm_scale)
        for b, t in enumerate(trees):
            oracle.verify.verify_sequence(w.target[b], w.draft_probs[b], t.q_row, t.tokens, t.parents, int(w.T_b[b]),
                                          int(w.modes[b]), w.philox_key, w.philox_offset, b)
        steps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    threads = cores
    if threadpool_info:
        info = threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
    if ctx is not None:
        ctx.unregister() if hasattr(ctx, "unregister") else None
    return dict(value=round(w.B * int(w.num_draft.mean()) * steps / el, 3), unit="draft tokens/s", cores=threads,
                kind="oracle", cpu=platform.processor() or platform.machine(),
                sample=f"{steps} full oracle step(s) (tree build + attention over all {w.Hq} heads + verify) on the "
                f"same {w.name} workload, {el:.1f} s")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="llama2_7b_layer_b1", help="workload name or index (0-4)")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--verify-logits", action="store_true",
                    help="verify with spec_tree_verify_logits (sampling distributions formed from the target logits and "
                         "temperatures inside the library) instead of supplied probabilities")
    ap.add_argument("--draft-vocab", type=int, default=None, metavar="N",
                    help="truncated draft vocabulary: draft rows over N tokens with a token map into the target's "
                         "vocabulary (frequency-ranked speculative sampling)")
    ap.add_argument("--details", default=None, help="write per-stage details as JSON to this path")
    ap.add_argument("--profile-kernels", type=int, default=0, metavar="N",
                    help="profiling mode (run under rocprofv3): N eager attention calls over the replicas, then one "
                         "256 MiB device-to-device copy whose counters calibrate FETCH_SIZE / WRITE_SIZE; no timing")
    args = ap.parse_args()

    if args.gpus != 1:
        eprint("bench.py: this build runs on exactly one GPU; --gpus must be 1 (no multi-GPU path is built).")
        sys.exit(2)

    import numpy as np
    import torch

    from tree_attention_verification_03_amd import ops
    from tree_attention_verification_03_amd.pipeline import DeviceWorkload, SpecTreeStep
    from workloads import get_config
    from workloads.synth import from_spec

    cfg_key = int(args.config) if args.config.isdigit() else args.config
    spec = get_config(cfg_key)
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

    if args.profile_kernels:
        for i in range(args.profile_kernels):
            attn_only(steps[i % R])()
        torch.cuda.synchronize()
        src = torch.empty(PMC_COPY_BYTES, dtype=torch.uint8, device=dw0.device)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        eprint(f"[bench] profile mode: {args.profile_kernels} attention calls, one {PMC_COPY_BYTES >> 20} MiB copy")
        return

    if args.eager:
        full_fns = [lambda st=st: st.run(compact=compact) for st in steps]

        class _G:
            def __init__(self, f):
                self.replay = f

        full = [_G(f) for f in full_fns]
        stage = {"build": [_G(st.build) for st in steps], "attention": [_G(attn_only(st)) for st in steps],
                 "verify": [_G(st.verify) for st in steps]}
    else:
        eprint("[bench] capturing HIP graphs")
        full = [capture(lambda st=st: st.run(compact=compact), torch) for st in steps]
        stage = {"build": [capture(st.build, torch) for st in steps],
                 "attention": [capture(attn_only(st), torch) for st in steps],
                 "verify": [capture(st.verify, torch) for st in steps]}

        def all_attn():
            for st in steps:
                attn_only(st)()

        # one graph holding the attention launch of every replica: back-to-back kernels, no per-graph gaps
        attn_chain = capture(all_attn, torch)
        # a replay must reproduce the eager result
        full[0].replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            got = getattr(steps[0].o, k)
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               v.view(torch.int16) if v.dtype == torch.bfloat16 else v), f"graph replay differs: {k}"

    time_graphs(full, args.warmup, torch)
    eprint(f"[bench] timing {args.steps} steps")
    gpu_ms, wall_ms = time_graphs(full, args.steps, torch)
    stage_ms = {}
    for name, gs in stage.items():
        time_graphs(gs, max(10, args.warmup // 2), torch)
        stage_ms[name] = time_graphs(gs, args.steps, torch)[0]
        eprint(f"[bench] stage {name}: {stage_ms[name] * 1e3:.2f} us")

    attn_launch_ms = stage_ms["attention"]
    if not args.eager:
        reps = max(4, args.steps // R)
        time_graphs([attn_chain], 2, torch)
        attn_launch_ms = time_graphs([attn_chain], reps, torch)[0] / R
        eprint(f"[bench] attention kernel, back-to-back launches: {attn_launch_ms * 1e3:.2f} us per launch")

    work = algorithmic_work(w, host)
    n_draft = int(w.num_draft.sum())
    ms_step = wall_ms
    value = n_draft / (ms_step * 1e-3)
    t_attn = attn_launch_ms * 1e-3
    attn_gbs = work["attn_bytes"] / t_attn / 1e9
    attn_tfs = work["attn_flops"] / t_attn / 1e12
    t_hbm = work["attn_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = work["attn_flops"] / (BF16_DENSE_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        roof = dict(bound="hbm", achieved=round(attn_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(attn_gbs / HBM_PEAK_GBS, 4), traffic=pmc_traffic(spec.name))
    else:
        roof = dict(bound="mfma", achieved=round(attn_tfs, 2), peak=BF16_DENSE_TFLOPS, unit="TFLOP/s",
                    frac=round(attn_tfs / BF16_DENSE_TFLOPS, 4), traffic=pmc_traffic(spec.name))
    roof.update(kernel="tree_attn_kernel (+ tree_attn_combine when the prefix is split)",
                bytes_per_launch=work["attn_bytes"], flops_per_launch=work["attn_flops"],
                avg_launch_us=round(t_attn * 1e6, 3),
                timing="HIP events around a graph of back-to-back spec_tree_attention calls, one per replica; a "
                       "call is the main kernel plus, for split prefixes, the combine kernel",
                traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)")

    line = {
        "metric": "tree-attn+verify draft tokens/s per layer; achieved HBM GB/s vs MI355X peak",
        "value": round(value, 1),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "prefix": int(w.prefix_lens.max()), "draft_tokens": int(w.num_draft.max()), "vocab": w.V,
                   "step": "tree build + tree attention + verify" + (" + KV compaction" if compact else ""),
                   "replicas": R, "graphs": not args.eager,
                   "verify_input": "target logits + temperature" if args.verify_logits else "target probabilities",
                   "draft_vocab": int(w.draft_logprobs.shape[-1])},
        "gpu_ms_per_step": round(gpu_ms, 5),
        "stage_us": {k: round(v * 1e3, 3) for k, v in stage_ms.items()},
        "attn_verify_draft_tokens_per_s": round(n_draft / ((stage_ms["attention"] + stage_ms["verify"]) * 1e-3), 1),
        "verified_seqs_per_s": round(w.B / (ms_step * 1e-3), 1),
        "roofline": roof,
        "verify_hbm_gbs": round(work["verify_bytes"] / (stage_ms["verify"] * 1e-3) / 1e9, 1),
    }
    if not args.no_cpu_baseline:
        eprint(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    if args.details:
        with open(args.details, "w") as f:
            json.dump(dict(line=line, work=work), f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
