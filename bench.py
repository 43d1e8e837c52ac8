"""Benchmark: DDTree tree-verify steps/s on one MI355X, every workload.

One step = ddtree_build -> ddtree_tree_attention -> the vocabulary reduction
and the walk, then accept_len and bonus reaching the host, which waits for
them before the next step (the serving loop's per-step wait).  Greedy workloads reduce
and walk with ddtree_vocab_verify_greedy (one launch; the same argmax, max and
walk outputs as ddtree_vocab_reduce + ddtree_verify_greedy, whose step is
reported beside it as "separate_calls_step"); sampling workloads call
ddtree_vocab_reduce, then ddtree_verify_sample.  The walk kernel stores the two results straight
into pinned host memory, accept_len last after a system-scope release, and
the host waits by polling accept_len there (filled with -1 before the step);
--step-wait sync synchronises the stream instead (reported beside the polled
rate as "stream_sync_step"), --result-copy adds an explicit device-to-host copy
and a synchronisation, --host-wait auto lets stream synchronisations sleep
until signalled.  Each step is a captured HIP graph replayed once per
step (--eager launches every call from Python).  Inputs are seeded synthetic
tensors of the workload's shapes, resident in HBM before timing starts; several
copies of the input set are rotated so that consecutive steps do not find their
inputs in the 256 MB last-level cache.

The build's inputs are the draft top-K of the synthetic draft logits, computed
once with ddtree_draft_topk before timing (the draft side of a real step); the
same call is timed on its own and reported as "draft_topk" (not in the step).

Default run (--config all): the single-request workload gives the headline
line's fields (value, roofline, cpu_baseline); every workload (tiny, single,
batched, long, ragged) also gets an entry in "configs" with its steps/s,
kernel rooflines and CPU baseline.  Timing protocol per workload: --warmup
untimed steps, then --reps repetitions of exactly --steps waited-for steps
(value = median rate); a sustained figure times repetitions of at least
max(--steps, 200) steps and 1 s each; kernel durations come from HIP events
around graphs of back-to-back calls on the calls' stream (--eager: the same
calls launched from Python, no graph anywhere).  The CPU baseline is
the oracle on a bounded sample of the same workload, timed single-threaded on
one core and on all cores of the process's affinity set.
"""
import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-verify steps/s at 1 GPU (budget=32); KV+vocab HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15         # dense bf16
MFMA_F32_PEAK = 157.3e12
HEADLINE = "single"
ALL_CONFIGS = ("tiny", "single", "batched", "long", "ragged")
TOP_P = 0.9   # nucleus mass of the top-p figure (sampling workloads)


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


def summary(rates):
    """Median, spread and count of per-repetition rates."""
    return {"median": round(statistics.median(rates), 2), "min": round(min(rates), 2),
            "max": round(max(rates), 2), "reps": len(rates)}


# ---------------------------------------------------------------------------- GPU side

class Workload:
    """Device inputs, buffers and the step functions of one workload."""

    def __init__(self, cfg, rotate, result_copy=False, eager=False, step_wait="sync"):
        import torch
        import tree_verification_build_amd as lib
        import workloads
        self.cfg, self.lib, self.torch = cfg, lib, torch
        dev = self.dev = "cuda:0"
        inp = self.inp = workloads.make_inputs(cfg)
        self.total_ctx = int(inp["ctx_offsets"][-1])
        d = self.d
        base = {k: d(inp[k], cfg.dtype) for k in ("q", "k_ctx", "v_ctx", "k_tree", "v_tree")}
        small = self.small = {k: d(inp[k]) for k in ("root_tok", "prefix_len", "ctx_offsets",
                                                     "uniforms")}
        # the build's inputs: the draft top-K of the first D draft rows, computed on the
        # GPU over every row (the target-logit planting reads the draft ranking)
        dl = self.draft_logits = d(inp["draft_logits"])
        tok_all, lp_all = lib.ddtree_draft_topk(dl, cfg.K)
        torch.cuda.synchronize()
        self.tok_all = tok_all
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
        self.rotate = rotate
        self.sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(rotate - 1)]
        self.tree = lib.alloc_tree(cfg.B, cfg.budget, cfg.D, cfg.K, dev)
        # accept_len and bonus land in pinned host memory, written by the walk kernel
        # itself (the device-to-host transfer is its stores); with result_copy they stay
        # on the device and one copy per step brings them over
        self.result_copy = result_copy
        self.eager = eager
        # polling needs the walk's own stores in pinned memory
        self.step_wait = "sync" if result_copy else step_wait
        if result_copy:
            self.result = torch.empty((2, cfg.B), dtype=torch.int32, device=dev)
            self.host_result = torch.empty((2, cfg.B), dtype=torch.int32, pin_memory=True)
        else:
            self.result = torch.empty((2, cfg.B), dtype=torch.int32, pin_memory=True)
            self.host_result = self.result
        self.outputs = {"accept_len": self.result[0],
                        "path_nodes": torch.empty((cfg.B, cfg.D + 1), dtype=torch.int32,
                                                  device=dev),
                        "out_tokens": torch.empty((cfg.B, cfg.D + 1), dtype=torch.int32,
                                                  device=dev),
                        "bonus": self.result[1]}
        self.attn_out = torch.empty_like(base["q"])
        self.ws_a = torch.empty(max(16, lib.ddtree_tree_attention_workspace_size(
            cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.Dh, inp["ctx_offsets"])), dtype=torch.uint8,
            device=dev)
        self.ws_v = torch.empty(max(16, lib.ddtree_vocab_reduce_workspace_size(
            cfg.B, cfg.N, cfg.V)), dtype=torch.uint8, device=dev)
        self.f_am = torch.empty((cfg.B, cfg.N), dtype=torch.int32, device=dev)
        self.f_mx = torch.empty((cfg.B, cfg.N), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream()
        self.nuc = None

    def d(self, x, dt=None):
        torch = self.torch
        x = np.ascontiguousarray(x)
        if dt == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(self.dev)
        return torch.from_numpy(x.view(np.int64) if x.dtype == np.uint64 else x).to(self.dev)

    # -- the calls of a step
    def build(self):
        s = self.small
        self.lib.ddtree_build(s["draft_lp"], s["draft_tok"], s["root_tok"], s["prefix_len"],
                              self.cfg.budget, tree=self.tree)

    def attention(self, s):
        self.lib.ddtree_tree_attention(s["q"], s["k_ctx"], s["v_ctx"], self.small["ctx_offsets"],
                                       self.inp["ctx_offsets"], s["k_tree"], s["v_tree"],
                                       self.tree, out=self.attn_out, workspace=self.ws_a)

    def vocab(self, s):
        return self.lib.ddtree_vocab_reduce(s["logits"], self.tree.num_nodes,
                                            self.cfg.temperature, workspace=self.ws_v)

    def step(self, i):
        """build -> attention -> vocabulary reduction -> walk (one verify step)."""
        s = self.sets[i % self.rotate]
        lib, T = self.lib, self.cfg.temperature
        self.build()
        self.attention(s)
        v = self.vocab(s)
        if T > 0:
            lib.ddtree_verify_sample(self.tree, s["logits"], v["maxv"], v["R"], v["R_blocks"], T,
                                     self.small["uniforms"], outputs=self.outputs)
        else:
            lib.ddtree_verify_greedy(self.tree, v["argmax"], outputs=self.outputs)
        if self.result_copy:
            self.host_result.copy_(self.result, non_blocking=True)

    def step_fused(self, i):
        """greedy: the vocabulary reduction and the walk in one call."""
        s = self.sets[i % self.rotate]
        self.build()
        self.attention(s)
        self.lib.ddtree_vocab_verify_greedy(s["logits"], self.tree, workspace=self.ws_v,
                                            outputs=self.outputs, argmax=self.f_am,
                                            maxv=self.f_mx)
        if self.result_copy:
            self.host_result.copy_(self.result, non_blocking=True)

    def step_lazy(self, i):
        """sampling: the walk reduces only the target rows it visits."""
        s = self.sets[i % self.rotate]
        self.build()
        self.attention(s)
        self.lib.ddtree_verify_sample_lazy(self.tree, s["logits"], self.cfg.temperature,
                                           self.small["uniforms"], outputs=self.outputs)

    def step_topp(self, i):
        """sampling with top-p nuclei: vocabulary pass, nucleus per node, walk."""
        s = self.sets[i % self.rotate]
        lib, T = self.lib, self.cfg.temperature
        self.build()
        self.attention(s)
        v = self.vocab(s)
        self.nuc = lib.ddtree_vocab_top_p(s["logits"], self.tree.num_nodes, v["maxv"], v["R"], T,
                                          TOP_P, outputs=self.nuc)
        lib.ddtree_verify_sample_top_p(self.tree, s["logits"], v["maxv"], self.nuc, T,
                                       self.small["uniforms"], outputs=self.outputs)

    # -- timing helpers
    def graphs_of(self, fn):
        """One captured graph per input set; replaying graph i % rotate is step i."""
        torch = self.torch
        gs = []
        for i in range(self.rotate):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(i)
            gs.append(g)
        torch.cuda.synchronize()
        return lambda i: gs[i % self.rotate].replay()

    def replayable(self, fn):
        """fn captured into a HIP graph, returned as its replay (eager: fn itself)."""
        if self.eager:
            return fn
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g):
            fn()
        return g.replay

    def loop_rates(self, run, steps, reps, wait=None):
        """`reps` repetitions of exactly `steps` steps; steps/s of each.  After
        each step the host waits for its results: "poll" spins on accept_len in
        pinned memory (filled with -1 before the step; the walk stores it last,
        after the other results and a system-scope release), "sync"
        synchronises the stream, "none" does not wait (pipelined steps)."""
        torch, stream = self.torch, self.stream
        wait = wait or self.step_wait
        acc = self.host_result[0].numpy() if wait == "poll" else None
        rates = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                if wait == "poll":
                    acc.fill(-1)
                    run(i)
                    t1 = time.perf_counter()
                    while (acc < 0).any():
                        if time.perf_counter() - t1 > 5.0:
                            raise RuntimeError(f"step {i}: no accept lengths after 5 s")
                else:
                    run(i)
                    if wait == "sync":
                        stream.synchronize()
            torch.cuda.synchronize()
            rates.append(steps / (time.perf_counter() - t0))
        return rates

    def sustained(self, run, min_steps, min_seconds, reps):
        """Repetitions of at least min_steps steps and min_seconds each."""
        est = self.loop_rates(run, min_steps, 1)[0]
        steps = max(min_steps, int(np.ceil(est * min_seconds)))
        return steps, self.loop_rates(run, steps, reps)

    def call_ms(self, fn, min_calls=200, reps=5):
        """Average duration of one call: a graph of back-to-back calls over the
        rotated input sets, replayed between two HIP events on this stream
        (eager: the same calls launched from Python); median over repetitions
        of at least min_calls calls."""
        torch, stream = self.torch, self.stream

        def calls():
            for i in range(self.rotate):
                fn(self.sets[i])
        once = self.replayable(calls)
        once()
        torch.cuda.synchronize()
        per = max(1, -(-min_calls // self.rotate))
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(per):
                once()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / (per * self.rotate))
        return statistics.median(out), out


def run_gpu(cfg, args, rotate):
    """Every GPU figure of one workload."""
    import torch
    w = Workload(cfg, rotate, result_copy=args.result_copy, eager=args.eager,
                 step_wait=args.step_wait)
    T = cfg.temperature
    main_step = w.step_fused if T == 0 else w.step
    for i in range(args.warmup):
        main_step(i)
        w.stream.synchronize()
    run = main_step if args.eager else w.graphs_of(main_step)
    for i in range(args.warmup):
        run(i)
        w.stream.synchronize()
    r = {"total_ctx": w.total_ctx}
    # the contract's loop: --reps repetitions of exactly --steps steps, the host
    # waiting for each step's accept lengths before the next
    r["rates"] = w.loop_rates(run, args.steps, args.reps)
    r["step_wait"] = w.step_wait
    if w.step_wait != "sync":
        # the same steps, each followed by a stream synchronisation instead
        r["sync_rates"] = w.loop_rates(run, args.steps, args.reps, wait="sync")
    r["accept_len_mean"] = float(w.host_result[0].float().mean())
    r["tree_stats"] = {"num_nodes_mean": float(w.tree.num_nodes.float().mean()),
                       "max_depth_mean": float(w.tree.max_depth.float().mean()),
                       "max_depth_min": int(w.tree.max_depth.min())}
    r["sustained_steps"], r["sustained"] = w.sustained(run, max(args.steps, 200),
                                                       args.min_seconds, args.reps)
    # the same steps without the per-step synchronisation
    r["pipelined"] = w.loop_rates(run, r["sustained_steps"], 3, wait="none")
    # kernel durations
    r["attn_ms"], r["attn_reps"] = w.call_ms(w.attention)
    r["vocab_ms"], r["vocab_reps"] = w.call_ms(w.vocab)
    r["decode_loop"] = run_decode_loop(w, max(100, args.steps))
    r["decode_loop_graph"] = run_decode_loop_graph(w, max(100, args.steps))
    if not args.no_extras:
        extra_steps = max(args.steps, 100)
        if T == 0:
            f = w.step if args.eager else w.graphs_of(w.step)
            f(0)
            r["separate"] = w.loop_rates(f, extra_steps, 3)
        else:
            f = w.step_lazy if args.eager else w.graphs_of(w.step_lazy)
            f(0)
            r["lazy"] = w.loop_rates(f, extra_steps, 3)
            w.step_topp(0)        # eager once: allocates the nucleus outputs
            torch.cuda.synchronize()
            f = w.step_topp if args.eager else w.graphs_of(w.step_topp)
            f(0)
            r["topp"] = w.loop_rates(f, extra_steps, 3)
            r["linear"] = run_linear(w)
        r.update(run_commit(w))
        r.update(run_topk(w))
    r["inputs"] = w.inp       # host copies, reused by the CPU baseline
    del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return r


DECODE_WARMUP = 3   # untimed chained steps before the graph-replayed decode loop's timed ones
# untimed steps before the eager loop's: in a fresh process its first eager launches of
# the range-form attention stall once or twice for tens of milliseconds (at the first
# call and near the 90th), a start-up cost of the launch path, not a per-step one
EAGER_DECODE_WARMUP = 120


def run_decode_loop(w, steps):
    """A decode loop over growing per-request cache slabs: each step builds the
    tree from the previous step's bonus token and prefix length, runs the tree
    attention over the slabs with ddtree_tree_attention_ranges (its split plan
    made anew on the host from the grown lengths), the vocabulary pass and the
    walk, then ddtree_commit appends the accepted path's K/V and gives the next
    (prefix length, root).  The accept lengths come back to the host each step
    (a copy into pinned memory and a stream synchronisation) to update the
    host's copy of the lengths, as a serving loop does.  Eager launches: the
    plan changes every step.  Inputs rotate over the workload's sets."""
    torch, lib, cfg = w.torch, w.lib, w.cfg
    dev, B, D, T = w.dev, cfg.B, cfg.D, cfg.temperature
    lens = np.diff(w.inp["ctx_offsets"]).astype(np.int64)
    cap = int(lens.max()) + (EAGER_DECODE_WARMUP + steps) * (D + 1) + 1
    base = np.arange(B, dtype=np.int64) * cap
    s0 = w.sets[0]
    kslab = torch.empty((B * cap, cfg.Hkv, cfg.Dh), dtype=s0["k_ctx"].dtype, device=dev)
    vslab = torch.empty_like(kslab)
    offs = w.inp["ctx_offsets"]
    for b in range(B):
        kslab[base[b]:base[b] + lens[b]] = s0["k_ctx"][offs[b]:offs[b + 1]]
        vslab[base[b]:base[b] + lens[b]] = s0["v_ctx"][offs[b]:offs[b + 1]]
    start_h = base.astype(np.int32)
    start_d = torch.from_numpy(start_h).to(dev)
    base_d = torch.from_numpy(base).to(dev)
    prefix_h = lens.astype(np.int32)
    prefix_d = [torch.from_numpy(prefix_h.copy()).to(dev), torch.empty((B,), dtype=torch.int32,
                                                                     device=dev)]
    root_d = [w.small["root_tok"].clone(), torch.empty((B,), dtype=torch.int32, device=dev)]
    walk = {"accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
            "path_nodes": torch.empty((B, D + 1), dtype=torch.int32, device=dev),
            "out_tokens": torch.empty((B, D + 1), dtype=torch.int32, device=dev),
            "bonus": torch.empty((B,), dtype=torch.int32, device=dev)}
    acc_h = torch.empty((B,), dtype=torch.int32, pin_memory=True)
    ws = torch.empty(16, dtype=torch.uint8, device=dev)
    regrown = 0
    sm = w.small
    torch.cuda.synchronize()
    tokens = 0
    for i in range(EAGER_DECODE_WARMUP + steps):
        if i == EAGER_DECODE_WARMUP:
            # untimed steps first: the first calls of a process pay one-time costs
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            tokens = 0
            grown0 = int(prefix_h.astype(np.int64).sum())
            per_step = []
        ts = time.perf_counter()
        s = w.sets[i % w.rotate]
        cur, nxt = i % 2, 1 - i % 2
        need = lib.ddtree_tree_attention_ranges_workspace_size(B, cfg.N, cfg.Hq, cfg.Hkv, cfg.Dh,
                                                               prefix_h)
        if need > ws.numel():
            ws = torch.empty(2 * need, dtype=torch.uint8, device=dev)
            regrown += 1
        lib.ddtree_build(sm["draft_lp"], sm["draft_tok"], root_d[cur], prefix_d[cur], cfg.budget,
                         tree=w.tree)
        lib.ddtree_tree_attention_ranges(s["q"], kslab, vslab, start_d, prefix_d[cur], start_h,
                                         prefix_h, s["k_tree"], s["v_tree"], w.tree,
                                         out=w.attn_out, workspace=ws)
        if T > 0:
            v = w.vocab(s)
            lib.ddtree_verify_sample(w.tree, s["logits"], v["maxv"], v["R"], v["R_blocks"], T,
                                     sm["uniforms"], outputs=walk)
        else:
            lib.ddtree_vocab_verify_greedy(s["logits"], w.tree, workspace=w.ws_v, outputs=walk,
                                           argmax=w.f_am, maxv=w.f_mx)
        lib.ddtree_commit(w.tree, walk, s["k_tree"], s["v_tree"], kslab, vslab, base_d, cap,
                          next_prefix_len=prefix_d[nxt], next_root=root_d[nxt])
        acc_h.copy_(walk["accept_len"], non_blocking=True)
        w.stream.synchronize()
        a = acc_h.numpy()
        prefix_h = (prefix_h + a + 1).astype(np.int32)
        tokens += int(a.sum()) + B
        if i >= EAGER_DECODE_WARMUP:
            per_step.append(time.perf_counter() - ts)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    consistent = bool(np.array_equal(prefix_d[(EAGER_DECODE_WARMUP + steps) % 2].cpu().numpy(),
                                     prefix_h))
    del kslab, vslab
    return {"steps": steps, "untimed_first": EAGER_DECODE_WARMUP, "steps_per_s": round(steps / dt, 2),
            "ms_per_step": round(1e3 * dt / steps, 4),
            "median_ms_per_step": round(1e3 * float(np.median(per_step)), 4),
            "max_ms_per_step": round(1e3 * float(np.max(per_step)), 4),
            "tokens_per_s": round(tokens / dt, 1),
            "accept_len_mean": round((tokens - steps * B) / (steps * B), 4),
            "ctx_growth": [grown0, int(prefix_h.astype(np.int64).sum())],
            "workspace_regrown": regrown, "host_lengths_match_device": consistent,
            "step": "build (previous bonus and prefix), ddtree_tree_attention_ranges over the "
                    "slabs (plan made anew), vocabulary pass and walk (one launch when greedy), "
                    "ddtree_commit, accept lengths to the host, synchronise; eager launches"}


def run_decode_loop_graph(w, steps):
    """The decode loop of run_decode_loop with each step a replayed HIP graph:
    build from the previous step's (prefix length, root) on the device,
    ddtree_tree_attention_ranges_capped over the slabs (the lengths read on the
    device when the kernels run, the slab capacities as bounds, so the captured
    call stays valid as the caches grow), vocabulary pass and walk,
    ddtree_commit appending the accepted K/V and writing the next (prefix
    length, root).  One graph per (input set, step parity): the (prefix, root)
    and walk buffers alternate between steps.  The host waits for every step's
    accept lengths by polling them in pinned memory (the walk's completion
    protocol) and keeps its own copy of the lengths; nothing else crosses."""
    torch, lib, cfg = w.torch, w.lib, w.cfg
    dev, B, D, T = w.dev, cfg.B, cfg.D, cfg.temperature
    lens = np.diff(w.inp["ctx_offsets"]).astype(np.int64)
    cap = int(lens.max()) + (DECODE_WARMUP + steps) * (D + 1) + 1
    base = np.arange(B, dtype=np.int64) * cap
    s0 = w.sets[0]
    kslab = torch.empty((B * cap, cfg.Hkv, cfg.Dh), dtype=s0["k_ctx"].dtype, device=dev)
    vslab = torch.empty_like(kslab)
    offs = w.inp["ctx_offsets"]
    for b in range(B):
        kslab[base[b]:base[b] + lens[b]] = s0["k_ctx"][offs[b]:offs[b + 1]]
        vslab[base[b]:base[b] + lens[b]] = s0["v_ctx"][offs[b]:offs[b + 1]]
    start_h = base.astype(np.int32)
    caps_h = np.full(B, cap, dtype=np.int32)
    start_d = torch.from_numpy(start_h).to(dev)
    base_d = torch.from_numpy(base).to(dev)
    prefix_d = [torch.from_numpy(lens.astype(np.int32)).to(dev),
                torch.empty((B,), dtype=torch.int32, device=dev)]
    root_d = [w.small["root_tok"].clone(), torch.empty((B,), dtype=torch.int32, device=dev)]
    walks = [{"accept_len": torch.empty((B,), dtype=torch.int32, pin_memory=True),
              "bonus": torch.empty((B,), dtype=torch.int32, pin_memory=True),
              "path_nodes": torch.empty((B, D + 1), dtype=torch.int32, device=dev),
              "out_tokens": torch.empty((B, D + 1), dtype=torch.int32, device=dev)}
             for _ in range(2)]
    ws = torch.empty(max(16, lib.ddtree_tree_attention_ranges_workspace_size(
        B, cfg.N, cfg.Hq, cfg.Hkv, cfg.Dh, caps_h)), dtype=torch.uint8, device=dev)
    sm = w.small
    keep = []

    def step(si, p):
        s = w.sets[si]
        lib.ddtree_build(sm["draft_lp"], sm["draft_tok"], root_d[p], prefix_d[p], cfg.budget,
                         tree=w.tree)
        lib.ddtree_tree_attention_ranges_capped(s["q"], kslab, vslab, start_d, prefix_d[p],
                                                start_h, caps_h, s["k_tree"], s["v_tree"],
                                                w.tree, out=w.attn_out, workspace=ws)
        if T > 0:
            v = w.vocab(s)
            keep.append(v)
            lib.ddtree_verify_sample(w.tree, s["logits"], v["maxv"], v["R"], v["R_blocks"], T,
                                     sm["uniforms"], outputs=walks[p])
        else:
            lib.ddtree_vocab_verify_greedy(s["logits"], w.tree, workspace=w.ws_v,
                                           outputs=walks[p], argmax=w.f_am, maxv=w.f_mx)
        lib.ddtree_commit(w.tree, walks[p], s["k_tree"], s["v_tree"], kslab, vslab, base_d, cap,
                          next_prefix_len=prefix_d[1 - p], next_root=root_d[1 - p])

    graphs = {}
    for si in range(w.rotate):
        for p in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(si, p)
            graphs[si, p] = g
    torch.cuda.synchronize()
    # capturing ran nothing: the slabs and lengths are still the initial ones
    prefix_h = lens.astype(np.int32)
    acc = [x["accept_len"].numpy() for x in walks]
    tokens = 0
    torch.cuda.synchronize()
    for i in range(DECODE_WARMUP + steps):
        if i == DECODE_WARMUP:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            tokens = 0
            grown0 = int(prefix_h.astype(np.int64).sum())
        p = i % 2
        a = acc[p]
        a.fill(-1)
        graphs[i % w.rotate, p].replay()
        t1 = time.perf_counter()
        while (a < 0).any():
            if time.perf_counter() - t1 > 5.0:
                raise RuntimeError(f"decode step {i}: no accept lengths after 5 s")
        prefix_h = (prefix_h + a + 1).astype(np.int32)
        tokens += int(a.sum()) + B
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    consistent = bool(np.array_equal(prefix_d[(DECODE_WARMUP + steps) % 2].cpu().numpy(),
                                     prefix_h))
    del graphs, kslab, vslab, keep
    return {"steps": steps, "untimed_first": DECODE_WARMUP, "steps_per_s": round(steps / dt, 2),
            "ms_per_step": round(1e3 * dt / steps, 4),
            "tokens_per_s": round(tokens / dt, 1),
            "accept_len_mean": round((tokens - steps * B) / (steps * B), 4),
            "ctx_growth": [grown0, int(prefix_h.astype(np.int64).sum())],
            "host_lengths_match_device": consistent,
            "step": "build from the device's (prefix length, root), "
                    "ddtree_tree_attention_ranges_capped over the slabs (lengths read on the "
                    "device, slab capacities as bounds), vocabulary pass and walk, "
                    "ddtree_commit; one replayed HIP graph per step, the host polling the "
                    "accept lengths in pinned memory"}


def run_commit(w):
    """ddtree_commit of the last step's walk into a compact cache (request b's
    position p at row b * (D + 1) + p - prefix_len[b]); not part of the step."""
    torch, lib, cfg = w.torch, w.lib, w.cfg
    dev = w.dev
    walk = {k: v.to(dev) for k, v in w.outputs.items()}
    cb = (torch.arange(cfg.B, dtype=torch.int64, device=dev) * (cfg.D + 1)
          - w.small["prefix_len"].to(torch.int64))
    kcache = torch.empty((cfg.B * (cfg.D + 1), cfg.Hkv, cfg.Dh), dtype=w.sets[0]["k_tree"].dtype,
                         device=dev)
    vcache = torch.empty_like(kcache)
    nxt = torch.empty((cfg.B,), dtype=torch.int32, device=dev)
    nroot = torch.empty_like(nxt)
    ms, _ = w.call_ms(lambda s: lib.ddtree_commit(
        w.tree, walk, s["k_tree"], s["v_tree"], kcache, vcache, cb, 1 << 30,
        next_prefix_len=nxt, next_root=nroot), reps=3)
    rows = int(walk["accept_len"].sum().item()) + cfg.B
    return {"commit_ms": ms, "commit_rows": rows,
            "commit_bytes": rows * 2 * 2 * cfg.Hkv * cfg.Dh * kcache.element_size()}


def run_topk(w):
    """The draft top-K over the D draft rows of each request (outside the step),
    over enough copies that the last-level cache does not hold them."""
    torch, lib, cfg = w.torch, w.lib, w.cfg
    dev = w.dev
    rows_d = w.draft_logits[:, :cfg.D].contiguous()
    ncopy = max(2, min(64, -(-(1 << 30) // (rows_d.numel() * 4))))
    dsets = [rows_d] + [rows_d.clone() for _ in range(ncopy - 1)]
    tk_ws = torch.empty(max(16, lib.ddtree_draft_topk_workspace_size(
        cfg.B * cfg.D, cfg.V, cfg.K)), dtype=torch.uint8, device=dev)
    tk_tok = torch.empty((cfg.B, cfg.D, cfg.K), dtype=torch.int32, device=dev)
    tk_lp = torch.empty((cfg.B, cfg.D, cfg.K), dtype=torch.float32, device=dev)
    def calls():
        for x in dsets:
            lib.ddtree_draft_topk(x, cfg.K, tokens=tk_tok, logprobs=tk_lp, workspace=tk_ws)
    once = w.replayable(calls)
    once()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    treps = max(1, 200 // ncopy)
    e0.record(w.stream)
    for _ in range(treps):
        once()
    e1.record(w.stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (treps * ncopy)
    del dsets
    return {"topk_ms": ms, "topk_bytes": rows_d.numel() * 4}


def run_linear(w, reps=50):
    """Linear speculative sampling on the workload's draft rows: a chain of D
    drafted tokens per request (the draft's top-1 at each depth), target rows =
    the draft rows plus the workload's target noise, both in the workload's dtype.
    Times the vocabulary pass over the D+1 target and D draft rows plus the walk
    (graph of back-to-back calls between two HIP events)."""
    import workloads
    torch, lib, cfg, inp = w.torch, w.lib, w.cfg, w.inp
    dev = w.dev
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
    x = w.tok_all[:, :D, 0].contiguous()
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
    once = w.replayable(call)
    once()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(w.stream)
    for _ in range(reps):
        once()
    e1.record(w.stream)
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


# ---------------------------------------------------------------------------- counter summaries

KERNEL_SOURCES = {"tree_attention": "attention.hip", "vocab_reduce": "vocab.hip"}


def traffic_profile(cfg_name, kernel="tree_attention"):
    """The committed counter summary of a call on this workload."""
    return os.path.join(ROOT, "profiles", f"{kernel}_{cfg_name}_hbm_traffic.md")


TRAFFIC_PROFILE = traffic_profile("single")


def source_digest(kernel="tree_attention"):
    import hashlib
    p = os.path.join(ROOT, "tree_verification_build_amd", "csrc", KERNEL_SOURCES[kernel])
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def attention_source_digest():
    return source_digest("tree_attention")


def measured_traffic(cfg_name, kernel="tree_attention"):
    """HBM bytes per call from the committed counter summary, or None when it
    covers another workload or an older kernel source."""
    try:
        text = open(traffic_profile(cfg_name, kernel)).read()
    except OSError:
        return None
    vals = dict(line.split(":", 1) for line in text.splitlines()
                if line.startswith(("workload:", "source_digest:", "traffic_bytes_per_call:")))
    vals = {k.strip(): v.strip() for k, v in vals.items()}
    if vals.get("workload") != cfg_name or vals.get("source_digest") != source_digest(kernel):
        return None
    try:
        return int(vals["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------- CPU baseline

# Oracle sample per workload: the first `requests` requests of the batch and, for
# attention, the first `heads` query heads (None: all).  Times are scaled to the
# whole step: attention by (total context x query heads) over the sample's, the
# other stages by requests.
CPU_SAMPLE = {"tiny": (None, None), "single": (None, None), "batched": (2, None),
              "long": (None, 1), "ragged": (2, None)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _subset_inputs(cfg, inp, reqs):
    """The workload's inputs restricted to requests `reqs` (contexts repacked)."""
    import dataclasses
    offs = inp["ctx_offsets"]
    sub = {k: np.ascontiguousarray(inp[k][reqs]) for k in
           ("q", "k_tree", "v_tree", "draft_logits", "root_tok", "uniforms", "prefix_len",
            "ctx_lens")}
    sub["k_ctx"] = np.concatenate([inp["k_ctx"][offs[b]:offs[b + 1]] for b in reqs])
    sub["v_ctx"] = np.concatenate([inp["v_ctx"][offs[b]:offs[b + 1]] for b in reqs])
    sub["ctx_offsets"] = np.concatenate([[0], np.cumsum(sub["ctx_lens"])]).astype(np.int32)
    return dataclasses.replace(cfg, B=len(reqs)), sub


def cpu_sample_step(cfg, inp, reqs, heads):
    """One oracle step on the sample; returns the seconds of each stage (the
    draft top-K and the target logits are inputs, outside the timed stages)."""
    import oracle
    import workloads
    scfg, sub = _subset_inputs(cfg, inp, reqs)
    oracle.attach_draft_topk(sub, cfg.D, cfg.K)
    t0 = time.perf_counter()
    tr = oracle.build_tree(sub["draft_lp"], sub["draft_tok"], sub["root_tok"], sub["prefix_len"],
                           cfg.budget)
    t1 = time.perf_counter()
    logits, _ = workloads.make_target_logits(scfg, sub, tr["depth"], tr["num_nodes"])
    t2 = time.perf_counter()
    oracle.tree_attention(sub["q"], sub["k_ctx"], sub["v_ctx"], sub["ctx_offsets"], sub["k_tree"],
                          sub["v_tree"], tr["vis"], tr["num_nodes"], dtype=cfg.dtype, heads=heads)
    t3 = time.perf_counter()
    vr = oracle.vocab_reduce(logits, tr["num_nodes"], cfg.temperature, dtype=cfg.dtype)
    t4 = time.perf_counter()
    if cfg.temperature > 0:
        oracle.verify_sample(tr, logits, vr["maxv"], vr["R"], cfg.temperature, sub["uniforms"],
                             cfg.D, dtype=cfg.dtype)
    else:
        oracle.verify_greedy(tr, vr["argmax"], cfg.D)
    t5 = time.perf_counter()
    return {"build": t1 - t0, "attention": t3 - t2, "vocab": t4 - t3, "walk": t5 - t4,
            "ctx": int(sub["ctx_offsets"][-1])}


def cpu_leg(cfg, inp, seconds, cores):
    """Oracle steps/s (scaled from the sample) with `cores` CPUs: the BLAS/OpenMP
    pools limited to that many threads and the process pinned to that many CPUs
    of its affinity set."""
    from threadpoolctl import threadpool_limits
    nreq, nheads = CPU_SAMPLE.get(cfg.name, (None, None))
    reqs = list(range(cfg.B if nreq is None else min(nreq, cfg.B)))
    heads = None if nheads is None else list(range(min(nheads, cfg.Hq)))
    total_ctx = int(inp["ctx_offsets"][-1])
    allowed = sorted(os.sched_getaffinity(0))
    use = allowed[:cores]
    os.sched_setaffinity(0, use)
    try:
        with threadpool_limits(limits=len(use)):
            runs, t_start = [], time.perf_counter()
            while True:
                runs.append(cpu_sample_step(cfg, inp, reqs, heads))
                if time.perf_counter() - t_start >= seconds:
                    break
    finally:
        os.sched_setaffinity(0, allowed)
    st = {k: statistics.median(r[k] for r in runs) for k in ("build", "attention", "vocab",
                                                               "walk")}
    fr = cfg.B / len(reqs)
    fa = (total_ctx * cfg.Hq) / (max(1, runs[0]["ctx"]) * (cfg.Hq if heads is None else len(heads)))
    step = (st["build"] + st["vocab"] + st["walk"]) * fr + st["attention"] * fa
    sample = (f"oracle step on requests 0..{len(reqs) - 1} of {cfg.B}"
              + ("" if heads is None else f", attention on {len(heads)} of {cfg.Hq} query heads")
              + f"; median of {len(runs)} runs, stage times scaled to the whole step "
                "(attention by context x heads, other stages by requests)")
    if len(reqs) == cfg.B and heads is None:
        sample = f"full oracle step of the {cfg.name} workload; median of {len(runs)} runs"
    return {"value": 1.0 / step, "unit": "steps/s", "cores": len(use), "kind": "oracle",
            "sample": sample, "stage_seconds_per_step": {
                "build": round(st["build"] * fr, 5), "attention": round(st["attention"] * fa, 5),
                "vocab": round(st["vocab"] * fr, 5), "walk": round(st["walk"] * fr, 5)}}


def run_cpu_baseline(cfg, seconds, inp=None):
    """The oracle as it stands on the host cores: single-threaded on one core,
    and on every core of the affinity set (both scaled from the same sample)."""
    import workloads
    if inp is None:
        inp = workloads.make_inputs(cfg)
    ncores = len(os.sched_getaffinity(0))
    one = cpu_leg(cfg, inp, seconds, 1)
    allc = cpu_leg(cfg, inp, seconds, ncores)
    out = dict(allc)
    out["single_core"] = {"value": one["value"], "cores": 1,
                          "stage_seconds_per_step": one["stage_seconds_per_step"]}
    out["cpu_model"] = cpu_model()
    return out


# ---------------------------------------------------------------------------- records

STEP_WAIT_TEXT = {
    "poll": "host polls accept_len in pinned memory (the walk stores it last, after a "
            "system-scope release)",
    "sync": "stream synchronisation",
}


def config_record(cfg, r, args, rotate):
    ab = algorithmic_bytes(cfg, r["total_ctx"])
    med = statistics.median(r["rates"])
    attn_gbs = ab["attention"] / (r["attn_ms"] * 1e-3) / 1e9
    vocab_gbs = ab["vocab"] / (r["vocab_ms"] * 1e-3) / 1e9
    mfma_peak = MFMA_BF16_PEAK if cfg.dtype == "bf16" else MFMA_F32_PEAK
    flops = attention_flops(cfg, r["total_ctx"])
    rec = {
        "workload": describe(cfg),
        "steps_per_s": round(med, 2),
        "ms_per_step": round(1e3 / med, 4),
        "steps": args.steps,
        "reps": summary(r["rates"]),
        "sustained": dict(summary(r["sustained"]), steps_per_rep=r["sustained_steps"]),
        "pipelined_steps_per_s": round(statistics.median(r["pipelined"]), 2),
        "step_wait": STEP_WAIT_TEXT[r.get("step_wait", "sync")],
        "ctx_tokens": r["total_ctx"],
        "input_sets_rotated": rotate,
        "attention": {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                      "traffic": measured_traffic(cfg.name, "tree_attention"),
                      "bytes_per_launch": ab["attention"], "avg_ms": round(r["attn_ms"], 5),
                      "avg_ms_reps": [round(x, 5) for x in r["attn_reps"]]},
        "vocab_reduce": {"bound": "hbm", "achieved": round(vocab_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(vocab_gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(cfg.name, "vocab_reduce"),
                         "bytes_per_launch": ab["vocab"], "avg_ms": round(r["vocab_ms"], 5),
                         "avg_ms_reps": [round(x, 5) for x in r["vocab_reps"]]},
        "attention_plus_vocab": {
            "achieved_GBs": round((ab["attention"] + ab["vocab"]) /
                                  ((r["attn_ms"] + r["vocab_ms"]) * 1e-3) / 1e9, 1),
            "frac": round((ab["attention"] + ab["vocab"]) /
                          ((r["attn_ms"] + r["vocab_ms"]) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "mfma_util": round(flops / (r["attn_ms"] * 1e-3) / mfma_peak, 4),
        "accept_len_mean": r["accept_len_mean"],
        "tree_stats": r["tree_stats"],
        "decode_loop": r["decode_loop"],
        "decode_loop_graph": r["decode_loop_graph"],
    }
    rec["step"] = ("build, attention, ddtree_vocab_verify_greedy (vocabulary reduction and "
                   "greedy walk in one launch)" if cfg.temperature == 0 else
                   "build, attention, ddtree_vocab_reduce, ddtree_verify_sample")
    if "sync_rates" in r:
        m = statistics.median(r["sync_rates"])
        rec["stream_sync_step"] = {"steps_per_s": round(m, 2), "ms_per_step": round(1e3 / m, 4),
                                   "reps": summary(r["sync_rates"]),
                                   "step": "the same steps, each followed by a stream "
                                           "synchronisation instead of the poll"}
    if "separate" in r:
        m = statistics.median(r["separate"])
        rec["separate_calls_step"] = {
            "steps_per_s": round(m, 2), "ms_per_step": round(1e3 / m, 4),
            "step": "build, attention, ddtree_vocab_reduce, ddtree_verify_greedy (same outputs "
                    "as the one-launch reduction and walk)"}
    if "lazy" in r:
        m = statistics.median(r["lazy"])
        rec["lazy_sampling_walk"] = {
            "steps_per_s": round(m, 2), "ms_per_step": round(1e3 / m, 4),
            "step": "build, attention, ddtree_verify_sample_lazy (target rows reduced only "
                    "where the walk goes; same outputs)"}
    if "topp" in r:
        m = statistics.median(r["topp"])
        rec["top_p_sampling_walk"] = {
            "top_p": TOP_P, "steps_per_s": round(m, 2), "ms_per_step": round(1e3 / m, 4),
            "step": "build, attention, ddtree_vocab_reduce, ddtree_vocab_top_p, "
                    "ddtree_verify_sample_top_p"}
    if "linear" in r:
        rec["linear_speculative_sampling"] = r["linear"]
    if "commit_ms" in r:
        rec["commit"] = {"avg_ms": round(r["commit_ms"], 5), "rows": r["commit_rows"],
                         "bytes_per_launch": r["commit_bytes"], "in_step": False}
    if "topk_ms" in r:
        rec["draft_topk"] = {"achieved_GBs": round(r["topk_bytes"] / (r["topk_ms"] * 1e-3) / 1e9, 1),
                             "avg_ms": round(r["topk_ms"], 5), "bytes_per_launch": r["topk_bytes"],
                             "in_step": False}
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed steps per repetition")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--reps", type=int, default=5, help="repetitions of --steps steps")
    ap.add_argument("--min-seconds", type=float, default=1.0,
                    help="minimum length of a sustained repetition")
    ap.add_argument("--config", default="all", help="a workload name, or 'all'")
    ap.add_argument("--rotate", type=int, default=0, help="input sets (0: >= 1 GiB in total)")
    ap.add_argument("--cpu-seconds", type=float, default=3.0,
                    help="oracle time per CPU leg and workload (at least one sample step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the figures outside the step (fused, lazy, top-p, linear, commit, "
                         "draft top-K)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every call from Python instead of replaying a HIP graph")
    ap.add_argument("--host-wait", choices=("spin", "auto"), default="spin",
                    help="how the host waits for each step: busy-poll (spin) or the runtime's "
                         "default sleep-until-signalled (auto)")
    ap.add_argument("--step-wait", choices=("poll", "sync"), default="poll",
                    help="how the host waits for each step's results: poll accept_len in "
                         "pinned memory (default) or synchronise the stream")
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
    names = ALL_CONFIGS if args.config == "all" else (args.config,)
    head = HEADLINE if HEADLINE in names else names[0]
    order = [head] + [n for n in names if n != head]
    records = {}
    for name in order:
        cfg = workloads.config(name)
        offs = np.concatenate([[0], np.cumsum(workloads.ctx_lengths(cfg))])
        ab = algorithmic_bytes(cfg, int(offs[-1]))
        rotate = args.rotate or int(max(1, min(32, np.ceil(2 ** 30 / ab["total"]))))
        print(f"[bench] {name}: GPU", file=sys.stderr, flush=True)
        r = run_gpu(cfg, args, rotate)
        rec = config_record(cfg, r, args, rotate)
        if not args.no_cpu_baseline:
            print(f"[bench] {name}: CPU oracle", file=sys.stderr, flush=True)
            rec["cpu_baseline"] = run_cpu_baseline(cfg, args.cpu_seconds, r["inputs"])
        del r
        records[name] = rec
        print(f"[bench] {name}: {rec['steps_per_s']} steps/s", file=sys.stderr, flush=True)
    h = records[head]
    hcfg = workloads.config(head)
    line = {
        "metric": METRIC,
        "value": h["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": hcfg.dtype,
        "data": "synthetic",
        "config": {"workload": h["workload"], "B": hcfg.B, "ctx_tokens": h["ctx_tokens"],
                   "heads_q": hcfg.Hq, "heads_kv": hcfg.Hkv, "head_dim": hcfg.Dh,
                   "depth": hcfg.D, "budget": hcfg.budget, "topk_cap": hcfg.K,
                   "vocab": hcfg.V, "temperature": hcfg.temperature,
                   "input_sets_rotated": h["input_sets_rotated"],
                   "launch": "eager" if args.eager else "hip_graph", "host_wait": host_wait,
                   "step_wait": h["step_wait"],
                   "result_to_host": "copy" if args.result_copy else "pinned_store",
                   "value_is": f"median steps/s over {args.reps} repetitions of {args.steps} "
                               "steps, each waited for on the host (step_wait)"},
        "roofline": dict(h["attention"], kernel="ddtree_tree_attention"),
        "reps": h["reps"],
        "sustained": h["sustained"],
        "pipelined_steps_per_s": h["pipelined_steps_per_s"],
        "vocab_reduce": h["vocab_reduce"],
        "attention_plus_vocab": h["attention_plus_vocab"],
        "mfma_util": h["mfma_util"],
        "accept_len_mean": h["accept_len_mean"],
    }
    if "cpu_baseline" in h:
        line["cpu_baseline"] = h["cpu_baseline"]
    line["configs"] = [dict(name=n, **records[n]) for n in names]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
