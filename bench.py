"""Benchmark: DDTree tree-verify steps/s on one MI355X.

One step = ddtree_build -> ddtree_tree_attention -> ddtree_vocab_reduce ->
ddtree_verify_greedy (or ddtree_verify_sample when the workload samples), then
accept_len and bonus reaching the host and a stream synchronisation (the
serving loop's per-step sync).  By default the walk kernel stores the two
results straight into pinned host memory and the host busy-polls for the
synchronisation; --result-copy adds an explicit device-to-host copy instead,
--host-wait auto sleeps until signalled.  By default each step is a captured HIP
graph replayed once per step (--eager launches every call from Python).  Inputs are seeded synthetic tensors of
the workload's shapes, resident in HBM before timing starts; several copies
of the input set are rotated so that consecutive steps do not find their
inputs in the 256 MB last-level cache.

The build's inputs are the draft top-K of the synthetic draft logits, computed
once with ddtree_draft_topk before timing (the draft side of a real step); the
same call is timed on its own and reported as "draft_topk" (not in the step).

Prints one JSON line: steps/s, a roofline entry for the tree-attention call
(algorithmic bytes / measured duration vs 8 TB/s), and the CPU oracle timed on
the host cores for the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-verify steps/s at 1 GPU (budget=32); KV+vocab HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15         # dense bf16
MFMA_F32_PEAK = 157.3e12


def describe(cfg):
    ctx = cfg.ctx if not isinstance(cfg.ctx, tuple) else f"U[{cfg.ctx[0]},{cfg.ctx[1]}]"
    mode = "greedy" if cfg.temperature == 0 else f"T={cfg.temperature} rejection sampling"
    return (f"{cfg.name}: batch {cfg.B}, context {ctx}, {cfg.Hq}/{cfg.Hkv} heads, head_dim "
            f"{cfg.Dh}, {cfg.dtype}; depth {cfg.D}, budget {cfg.budget}, top-k cap {cfg.K}; "
            f"vocab {cfg.V}; {mode}")


def algorithmic_bytes(cfg, total_ctx):
    """Bytes the step must move at least once (context KV once, tree Q/K/V/O, logits once)."""
    e = 2 if cfg.dtype == "bf16" else 4
    kv = 2 * total_ctx * cfg.Hkv * cfg.Dh * e
    tree_qkvo = cfg.B * cfg.N * cfg.Dh * e * (2 * cfg.Hq + 2 * cfg.Hkv)
    logits = cfg.B * cfg.N * cfg.V * e
    residual = cfg.B * cfg.V * e if cfg.temperature > 0 else 0
    return {"attention": kv + tree_qkvo, "vocab": logits, "residual": residual,
            "total": kv + tree_qkvo + logits + residual}


def attention_flops(cfg, total_ctx):
    return 4.0 * cfg.N * total_ctx * cfg.Hq * cfg.Dh


def set_host_wait(mode):
    """Before the HIP runtime starts: 'spin' makes host waits on the device (the
    per-step stream synchronisation) busy-poll instead of sleeping until an
    interrupt, the usual setting of a latency-bound serving loop.  Returns the
    mode in effect."""
    if mode != "spin":
        return "auto"
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        return "spin" if hip.hipSetDeviceFlags(ctypes.c_uint(1)) == 0 else "auto"
    except OSError:
        return "auto"


TOP_P = 0.9   # nucleus mass of the top-p figure (sampling workloads)


def run_gpu(cfg, steps, warmup, rotate, graph=True, result_copy=False):
    import torch
    import tree_verification_build_amd as lib
    import workloads

    dev = "cuda:0"
    inp = workloads.make_inputs(cfg)
    tot_ctx = int(inp["ctx_offsets"][-1])

    def d(x, dt=None):
        x = np.ascontiguousarray(x)
        if dt == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x.view(np.int64) if x.dtype == np.uint64 else x).to(dev)

    base = {k: d(inp[k], cfg.dtype) for k in ("q", "k_ctx", "v_ctx", "k_tree", "v_tree")}
    small = {k: d(inp[k]) for k in ("root_tok", "prefix_len", "ctx_offsets", "uniforms")}
    # the build's inputs: the draft top-K of the first D draft rows, computed on the
    # GPU over every row (the target-logit planting reads the draft ranking)
    dl = d(inp["draft_logits"])
    tok_all, lp_all = lib.ddtree_draft_topk(dl, cfg.K)
    torch.cuda.synchronize()
    inp["draft_tok_all"] = tok_all.cpu().numpy()
    small["draft_tok"] = tok_all[:, :cfg.D].contiguous()
    small["draft_lp"] = lp_all[:, :cfg.D].contiguous()
    # the target logits depend on the tree shape: build it once on the GPU
    t0 = lib.ddtree_build(small["draft_lp"], small["draft_tok"], small["root_tok"],
                          small["prefix_len"], cfg.budget)
    torch.cuda.synchronize()
    tn = t0.to_numpy()
    logits_np, _ = workloads.make_target_logits(cfg, inp, tn["depth"], tn["num_nodes"])
    base["logits"] = d(logits_np, cfg.dtype)
    del logits_np

    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(rotate - 1)]
    tree = lib.alloc_tree(cfg.B, cfg.budget, cfg.D, cfg.K, dev)
    # accept_len and bonus land in pinned host memory, written by the walk
    # kernel itself (the device-to-host transfer is its stores); with
    # --result-copy they stay on the device and one copy per step brings them over
    if result_copy:
        result = torch.empty((2, cfg.B), dtype=torch.int32, device=dev)
    else:
        result = torch.empty((2, cfg.B), dtype=torch.int32, pin_memory=True)
    outputs = {"accept_len": result[0],
               "path_nodes": torch.empty((cfg.B, cfg.D + 1), dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((cfg.B, cfg.D + 1), dtype=torch.int32, device=dev),
               "bonus": result[1]}
    attn_out = torch.empty_like(base["q"])
    ws_a = torch.empty(max(16, lib.ddtree_tree_attention_workspace_size(
        cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.Dh, inp["ctx_offsets"])), dtype=torch.uint8,
        device=dev)
    ws_v = torch.empty(max(16, lib.ddtree_vocab_reduce_workspace_size(cfg.B, cfg.N, cfg.V)),
                       dtype=torch.uint8, device=dev)
    host_result = torch.empty((2, cfg.B), dtype=torch.int32, pin_memory=True) if result_copy \
        else result
    stream = torch.cuda.current_stream()
    T = cfg.temperature

    def attention(s):
        lib.ddtree_tree_attention(s["q"], s["k_ctx"], s["v_ctx"], small["ctx_offsets"],
                                  inp["ctx_offsets"], s["k_tree"], s["v_tree"], tree,
                                  out=attn_out, workspace=ws_a)

    def vocab(s):
        return lib.ddtree_vocab_reduce(s["logits"], tree.num_nodes, T, workspace=ws_v)

    def step(i):
        s = sets[i % rotate]
        lib.ddtree_build(small["draft_lp"], small["draft_tok"], small["root_tok"],
                         small["prefix_len"], cfg.budget, tree=tree)
        attention(s)
        v = vocab(s)
        if T > 0:
            lib.ddtree_verify_sample(tree, s["logits"], v["maxv"], v["R"], v["R_blocks"], T,
                                     small["uniforms"], outputs=outputs)
        else:
            lib.ddtree_verify_greedy(tree, v["argmax"], outputs=outputs)
        if result_copy:
            host_result.copy_(result, non_blocking=True)

    for i in range(warmup):
        step(i)
        stream.synchronize()
    torch.cuda.synchronize()
    if graph:
        # one captured step per input set; replaying it is the serving loop
        graphs = []
        for i in range(rotate):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(warmup):
            graphs[i % rotate].replay()
            stream.synchronize()
        run = lambda i: graphs[i % rotate].replay()  # noqa: E731
    else:
        run = step
    # timed: per-step synchronised serving loop (step + D2H of accept_len/bonus + sync)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        run(i)
        stream.synchronize()
    t_sync = time.perf_counter() - t_start
    # pipelined: the same steps without the per-step synchronisation
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    t_pipe = time.perf_counter() - t_start

    # sampling workloads: the same step with the lazy walk, which reduces only the
    # target rows it visits (no vocabulary pass over every node); same sync loop
    t_lazy = None
    if T > 0:
        def step_lazy(i):
            s = sets[i % rotate]
            lib.ddtree_build(small["draft_lp"], small["draft_tok"], small["root_tok"],
                             small["prefix_len"], cfg.budget, tree=tree)
            attention(s)
            lib.ddtree_verify_sample_lazy(tree, s["logits"], T, small["uniforms"],
                                          outputs=outputs)
        run_lazy = step_lazy
        if graph:
            lazy_graphs = []
            for i in range(rotate):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step_lazy(i)
                lazy_graphs.append(g)
            run_lazy = lambda i: lazy_graphs[i % rotate].replay()  # noqa: E731
        for i in range(warmup):
            run_lazy(i)
            stream.synchronize()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(steps):
            run_lazy(i)
            stream.synchronize()
        t_lazy = time.perf_counter() - t_start

    # greedy workloads: the same step with the vocabulary reduction and the walk in
    # one call (ddtree_vocab_verify_greedy: the slice merge and the walk share a
    # launch; same outputs); same synchronised loop
    t_fused = None
    if T == 0:
        f_am = torch.empty((cfg.B, cfg.N), dtype=torch.int32, device=dev)
        f_mx = torch.empty((cfg.B, cfg.N), dtype=torch.float32, device=dev)

        def step_fused(i):
            s = sets[i % rotate]
            lib.ddtree_build(small["draft_lp"], small["draft_tok"], small["root_tok"],
                             small["prefix_len"], cfg.budget, tree=tree)
            attention(s)
            lib.ddtree_vocab_verify_greedy(s["logits"], tree, workspace=ws_v, outputs=outputs,
                                           argmax=f_am, maxv=f_mx)
        run_fused = step_fused
        if graph:
            fused_graphs = []
            for i in range(rotate):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step_fused(i)
                fused_graphs.append(g)
            run_fused = lambda i: fused_graphs[i % rotate].replay()  # noqa: E731
        for i in range(warmup):
            run_fused(i)
            stream.synchronize()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(steps):
            run_fused(i)
            stream.synchronize()
        t_fused = time.perf_counter() - t_start

    # sampling workloads: the step with top-p (p = 0.9) nuclei: vocabulary pass, the
    # per-node nucleus, then the walk on it; same synchronised loop
    t_topp = None
    if T > 0:
        nuc = None

        def step_topp(i):
            nonlocal nuc
            s = sets[i % rotate]
            lib.ddtree_build(small["draft_lp"], small["draft_tok"], small["root_tok"],
                             small["prefix_len"], cfg.budget, tree=tree)
            attention(s)
            v = vocab(s)
            nuc = lib.ddtree_vocab_top_p(s["logits"], tree.num_nodes, v["maxv"], v["R"], T,
                                         TOP_P, outputs=nuc)
            lib.ddtree_verify_sample_top_p(tree, s["logits"], v["maxv"], nuc, T,
                                           small["uniforms"], outputs=outputs)
        step_topp(0)                 # eager once: allocates the nucleus outputs
        torch.cuda.synchronize()
        run_topp = step_topp
        if graph:
            topp_graphs = []
            for i in range(rotate):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step_topp(i)
                topp_graphs.append(g)
            run_topp = lambda i: topp_graphs[i % rotate].replay()  # noqa: E731
        for i in range(warmup):
            run_topp(i)
            stream.synchronize()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(steps):
            run_topp(i)
            stream.synchronize()
        t_topp = time.perf_counter() - t_start

    # kernel durations: a HIP graph of back-to-back calls over the rotated input sets,
    # replayed between two HIP events on this stream (no host gaps fall inside)
    def timed_calls(fn, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(rotate):
                fn(sets[i])
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * rotate)
    reps = max(1, steps // rotate)
    attn_ms = timed_calls(attention, reps)
    vocab_ms = timed_calls(vocab, reps)
    # the commit that follows a step (not part of it): the last step's walk, its
    # path rows into a compact cache (request b's position p at row
    # b * (D + 1) + p - prefix_len[b])
    walk = {k: v.to(dev) for k, v in outputs.items()}
    cb = (torch.arange(cfg.B, dtype=torch.int64, device=dev) * (cfg.D + 1)
          - small["prefix_len"].to(torch.int64))
    kcache = torch.empty((cfg.B * (cfg.D + 1), cfg.Hkv, cfg.Dh), dtype=base["k_tree"].dtype,
                         device=dev)
    vcache = torch.empty_like(kcache)
    nxt = torch.empty((cfg.B,), dtype=torch.int32, device=dev)
    nroot = torch.empty_like(nxt)
    commit_ms = timed_calls(lambda s: lib.ddtree_commit(
        tree, walk, s["k_tree"], s["v_tree"], kcache, vcache, cb, 1 << 30,
        next_prefix_len=nxt, next_root=nroot), reps)
    commit_rows = int(walk["accept_len"].sum().item()) + cfg.B
    commit_bytes = commit_rows * 2 * 2 * cfg.Hkv * cfg.Dh * base["k_tree"].element_size()
    del sets
    if graph:
        del graphs
    lin = run_linear(cfg, inp, tok_all, stream) if T > 0 else None
    # the draft top-K over the D draft rows of each request (outside the step),
    # over enough copies that the last-level cache does not hold them
    rows_d = dl[:, :cfg.D].contiguous()
    ncopy = max(2, min(64, -(-(1 << 30) // (rows_d.numel() * 4))))
    dsets = [rows_d] + [rows_d.clone() for _ in range(ncopy - 1)]
    tk_ws = torch.empty(max(16, lib.ddtree_draft_topk_workspace_size(
        cfg.B * cfg.D, cfg.V, cfg.K)), dtype=torch.uint8, device=dev)
    tk_tok = torch.empty((cfg.B, cfg.D, cfg.K), dtype=torch.int32, device=dev)
    tk_lp = torch.empty((cfg.B, cfg.D, cfg.K), dtype=torch.float32, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x in dsets:
            lib.ddtree_draft_topk(x, cfg.K, tokens=tk_tok, logprobs=tk_lp, workspace=tk_ws)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    treps = max(1, 200 // ncopy)
    e0.record(stream)
    for _ in range(treps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    topk_ms = e0.elapsed_time(e1) / (treps * ncopy)
    return {"t_sync": t_sync, "t_pipe": t_pipe, "t_lazy": t_lazy, "t_topp": t_topp,
            "t_fused": t_fused, "linear": lin,
            "attn_ms": attn_ms, "vocab_ms": vocab_ms, "commit_ms": commit_ms,
            "commit_rows": commit_rows, "commit_bytes": commit_bytes,
            "topk_ms": topk_ms, "topk_bytes": rows_d.numel() * 4,
            "total_ctx": tot_ctx, "accept_len_mean": float(host_result[0].float().mean())}


def run_linear(cfg, inp, tok_all, stream, reps=50):
    """Linear speculative sampling on the workload's draft rows: a chain of D
    drafted tokens per request (the draft's top-1 at each depth), target rows =
    the draft rows plus the workload's target noise, both in the workload's dtype.
    Times the vocabulary pass over the D+1 target and D draft rows plus the walk
    (graph of back-to-back calls between two HIP events)."""
    import torch
    import tree_verification_build_amd as lib
    import workloads
    dev = "cuda:0"
    B, D, T = cfg.B, cfg.D, cfg.temperature
    chain = workloads.config(cfg.name, budget=D)
    depth = np.tile(np.arange(D + 1, dtype=np.int32), (B, 1))
    tl, _ = workloads.make_target_logits(chain, inp, depth, np.full(B, D + 1, np.int32))
    dl = np.ascontiguousarray(inp["draft_logits"][:, :D])
    if cfg.dtype == "bf16":
        dl = workloads.f32_to_bf16_bits(dl)
        tg = torch.from_numpy(tl.view(np.int16)).view(torch.bfloat16).to(dev)
        dg = torch.from_numpy(dl.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        tg, dg = torch.from_numpy(tl).to(dev), torch.from_numpy(dl).to(dev)
    x = tok_all[:, :D, 0].contiguous()
    u = torch.from_numpy(np.ascontiguousarray(inp["uniforms"][:, :D + 1]).view(np.int64)).to(dev)
    nq = torch.full((B,), D + 1, dtype=torch.int32, device=dev)
    npd = torch.full((B,), D, dtype=torch.int32, device=dev)
    out = {"accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
           "out_tokens": torch.empty((B, D + 1), dtype=torch.int32, device=dev),
           "bonus": torch.empty((B,), dtype=torch.int32, device=dev)}

    def call():
        ts = lib.ddtree_vocab_reduce(tg, nq, T)
        ds = lib.ddtree_vocab_reduce(dg, npd, T)
        lib.ddtree_verify_linear_sample(tg, dg, x, T, u, target_stats=ts, draft_stats=ds,
                                        outputs=out)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"ms_per_call": round(ms, 4), "accept_len_mean": float(out["accept_len"].float().mean()),
            "calls": "ddtree_vocab_reduce (target D+1 rows, draft D rows) + "
                     "ddtree_verify_linear_sample",
            "chain": f"{B} requests x {D} drafted tokens (draft top-1), V {cfg.V}, T {T}"}


def run_copy_calibration(mib, reps=20):
    """A plain device-to-device copy of a known size (for scaling HBM counters)
    and its bandwidth, the practical ceiling of a streaming kernel here."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"copy_bytes_read": n, "copy_bytes_written": n, "copies": reps + 1,
            "copy_GBs": round(2 * n / (ms * 1e-3) / 1e9, 1)}


def traffic_profile(cfg_name):
    """The committed counter summary of the tree-attention call on this workload."""
    return os.path.join(ROOT, "profiles", f"tree_attention_{cfg_name}_hbm_traffic.md")


TRAFFIC_PROFILE = traffic_profile("single")


def attention_source_digest():
    import hashlib
    p = os.path.join(ROOT, "tree_verification_build_amd", "csrc", "attention.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def measured_traffic(cfg_name):
    """HBM bytes per tree-attention call from the committed counter summary, or
    None when it covers another workload or an older attention source."""
    try:
        text = open(traffic_profile(cfg_name)).read()
    except OSError:
        return None
    vals = dict(line.split(":", 1) for line in text.splitlines()
                if line.startswith(("workload:", "source_digest:", "traffic_bytes_per_call:")))
    vals = {k.strip(): v.strip() for k, v in vals.items()}
    if vals.get("workload") != cfg_name or vals.get("source_digest") != attention_source_digest():
        return None
    try:
        return int(vals["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def run_cpu_baseline(cfg, seconds):
    """The oracle as it stands, same workload, on the host cores (one step = build,
    float64 attention, vocabulary pass, walk)."""
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    # the oracle's draft top-K gives the build's inputs (outside the timed step,
    # as on the GPU)
    inp = oracle.attach_draft_topk(workloads.make_inputs(cfg), cfg.D, cfg.K)
    t = oracle.build_tree(inp["draft_lp"], inp["draft_tok"], inp["root_tok"], inp["prefix_len"],
                          cfg.budget)
    logits, _ = workloads.make_target_logits(cfg, inp, t["depth"], t["num_nodes"])
    n = 0
    t0 = time.perf_counter()
    while True:
        tr = oracle.build_tree(inp["draft_lp"], inp["draft_tok"], inp["root_tok"],
                               inp["prefix_len"], cfg.budget)
        oracle.tree_attention(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"],
                              inp["k_tree"], inp["v_tree"], tr["vis"], tr["num_nodes"],
                              dtype=cfg.dtype)
        vr = oracle.vocab_reduce(logits, tr["num_nodes"], cfg.temperature, dtype=cfg.dtype)
        if cfg.temperature > 0:
            oracle.verify_sample(tr, logits, vr["maxv"], vr["R"], cfg.temperature,
                                 inp["uniforms"], cfg.D, dtype=cfg.dtype)
        else:
            oracle.verify_greedy(tr, vr["argmax"], cfg.D)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 1000:
            break
    return {"value": n / el, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} full oracle steps of the {cfg.name} workload in {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="single")
    ap.add_argument("--rotate", type=int, default=0, help="input sets (0: >= 1 GiB in total)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every call from Python instead of replaying a HIP graph")
    ap.add_argument("--host-wait", choices=("spin", "auto"), default="spin",
                    help="how the host waits for each step: busy-poll (spin) or the runtime's "
                         "default sleep-until-signalled (auto)")
    ap.add_argument("--result-copy", action="store_true",
                    help="keep accept_len/bonus in device memory and copy them to the host "
                         "each step (default: the walk writes them to pinned host memory)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter scaling) and print it")
    args = ap.parse_args()
    if args.copy_calibration:
        print(json.dumps(run_copy_calibration(args.copy_calibration)), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the verify path here is built and timed on a "
              "single MI355X (no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    host_wait = set_host_wait(args.host_wait)
    import workloads
    cfg = workloads.config(args.config)
    offs = np.concatenate([[0], np.cumsum(workloads.ctx_lengths(cfg))])
    ab = algorithmic_bytes(cfg, int(offs[-1]))
    rotate = args.rotate or int(max(1, min(32, np.ceil(2 ** 30 / ab["total"]))))
    r = run_gpu(cfg, args.steps, args.warmup, rotate, graph=not args.eager,
                result_copy=args.result_copy)
    steps_s = args.steps / r["t_sync"]
    attn_gbs = ab["attention"] / (r["attn_ms"] * 1e-3) / 1e9
    vocab_gbs = ab["vocab"] / (r["vocab_ms"] * 1e-3) / 1e9
    flops = attention_flops(cfg, r["total_ctx"])
    mfma_peak = MFMA_BF16_PEAK if cfg.dtype == "bf16" else MFMA_F32_PEAK
    line = {
        "metric": METRIC,
        "value": round(steps_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * r["t_sync"] / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": describe(cfg), "B": cfg.B, "ctx_tokens": r["total_ctx"],
                   "heads_q": cfg.Hq, "heads_kv": cfg.Hkv, "head_dim": cfg.Dh, "depth": cfg.D,
                   "budget": cfg.budget, "topk_cap": cfg.K, "vocab": cfg.V,
                   "temperature": cfg.temperature, "input_sets_rotated": rotate,
                   "launch": "eager" if args.eager else "hip_graph", "host_wait": host_wait,
                   "result_to_host": "copy" if args.result_copy else "pinned_store"},
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(cfg.name), "kernel": "ddtree_tree_attention",
                     "bytes_per_launch": ab["attention"], "avg_ms": round(r["attn_ms"], 5)},
        "pipelined_steps_per_s": round(args.steps / r["t_pipe"], 2),
        "vocab_reduce": {"achieved_GBs": round(vocab_gbs, 1), "avg_ms": round(r["vocab_ms"], 5),
                         "bytes_per_launch": ab["vocab"]},
        "attention_plus_vocab_GBs": round((ab["attention"] + ab["vocab"]) /
                                          ((r["attn_ms"] + r["vocab_ms"]) * 1e-3) / 1e9, 1),
        "mfma_util": round(flops / (r["attn_ms"] * 1e-3) / mfma_peak, 4),
        "draft_topk": {"achieved_GBs": round(r["topk_bytes"] / (r["topk_ms"] * 1e-3) / 1e9, 1),
                       "avg_ms": round(r["topk_ms"], 5), "bytes_per_launch": r["topk_bytes"],
                       "in_step": False},
        "commit": {"avg_ms": round(r["commit_ms"], 5), "rows": r["commit_rows"],
                   "bytes_per_launch": r["commit_bytes"], "in_step": False},
        "accept_len_mean": r["accept_len_mean"],
    }
    if r["linear"] is not None:
        line["linear_speculative_sampling"] = r["linear"]
    if r["t_fused"] is not None:
        line["fused_greedy_step"] = {
            "steps_per_s": round(args.steps / r["t_fused"], 2),
            "ms_per_step": round(r["t_fused"] / args.steps * 1e3, 4),
            "step": "build, attention, ddtree_vocab_verify_greedy (vocabulary reduction and "
                    "greedy walk in one call; same outputs)"}
    if r["t_lazy"] is not None:
        line["lazy_sampling_walk"] = {
            "steps_per_s": round(args.steps / r["t_lazy"], 2),
            "ms_per_step": round(r["t_lazy"] / args.steps * 1e3, 4),
            "step": "build, attention, ddtree_verify_sample_lazy (target rows reduced only "
                    "where the walk goes; same outputs)"}
    if r["t_topp"] is not None:
        line["top_p_sampling_walk"] = {
            "top_p": TOP_P,
            "steps_per_s": round(args.steps / r["t_topp"], 2),
            "ms_per_step": round(r["t_topp"] / args.steps * 1e3, 4),
            "step": "build, attention, ddtree_vocab_reduce, ddtree_vocab_top_p, "
                    "ddtree_verify_sample_top_p"}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = run_cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
