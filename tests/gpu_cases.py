"""Shared machinery of the GPU parity tests: run the HIP path through the C-ABI
binding and the CPU oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

import oracle
import workloads

DEV = "cuda:0"


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev_tensor(arr, dtype):
    """numpy storage array -> device tensor (bf16 from uint16 bits)."""
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    if a.dtype == np.uint64:
        return torch.from_numpy(a.view(np.int64)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def attn_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


class Case:
    """Inputs, oracle tree and target logits of one workload."""

    def __init__(self, cfg, with_kv=True):
        self.cfg = cfg
        self.inp = oracle.attach_draft_topk(workloads.make_inputs(cfg, with_kv=with_kv),
                                            cfg.D, cfg.K)
        i = self.inp
        self.tree = oracle.build_tree(i["draft_lp"], i["draft_tok"], i["root_tok"],
                                      i["prefix_len"], cfg.budget)
        self.logits, self.planted = workloads.make_target_logits(cfg, i, self.tree["depth"],
                                                                 self.tree["num_nodes"])
        self._d = {}

    def d(self, name):
        """Device copy of an input (cached)."""
        if name not in self._d:
            i, c = self.inp, self.cfg
            if name in ("q", "k_ctx", "v_ctx", "k_tree", "v_tree"):
                self._d[name] = dev_tensor(i[name], c.dtype)
            elif name == "logits":
                self._d[name] = dev_tensor(self.logits, c.dtype)
            elif name == "uniforms":
                self._d[name] = dev_tensor(i["uniforms"], None)
            else:
                self._d[name] = dev_tensor(i[name], None)
        return self._d[name]

    def gpu_tree(self):
        import tree_verification_build_amd as lib
        c = self.cfg
        return lib.ddtree_build(self.d("draft_lp"), self.d("draft_tok"), self.d("root_tok"),
                                self.d("prefix_len"), c.budget)

    def gpu_attention(self, tree, want_lse=True):
        import tree_verification_build_amd as lib
        return lib.ddtree_tree_attention(self.d("q"), self.d("k_ctx"), self.d("v_ctx"),
                                         self.d("ctx_offsets"), self.inp["ctx_offsets"],
                                         self.d("k_tree"), self.d("v_tree"), tree,
                                         want_lse=want_lse)

    def oracle_attention(self, requests=None, heads=None):
        i, c = self.inp, self.cfg
        return oracle.tree_attention(i["q"], i["k_ctx"], i["v_ctx"], i["ctx_offsets"],
                                     i["k_tree"], i["v_tree"], self.tree["vis"],
                                     self.tree["num_nodes"], dtype=c.dtype, requests=requests,
                                     heads=heads)


def assert_tree_equal(got: dict, ref: dict):
    for k in ("token", "parent", "depth", "rank", "position", "first_child", "next_sibling",
              "num_nodes", "max_depth"):
        if not np.array_equal(got[k], ref[k]):
            bad = np.argwhere(got[k] != ref[k])[:4]
            raise AssertionError(f"{k}: first mismatches at {bad.tolist()}: got "
                                 f"{[got[k][tuple(i)] for i in bad]}, expected "
                                 f"{[ref[k][tuple(i)] for i in bad]}")
    assert np.array_equal(got["score"].view(np.uint32), ref["score"].view(np.uint32)), "score bits"
    assert np.array_equal(got["vis"], ref["vis"]), "vis"


def assert_attention_close(o_gpu, o_ref, dtype, mask=None):
    """The attention tolerance: max-abs 2e-2 (bf16) / 1e-4 (fp32), also relative to max|o_ref|."""
    tol = 2e-2 if dtype == "bf16" else 1e-4
    sel = ~np.isnan(o_ref) if mask is None else mask
    err = np.abs(o_gpu[sel] - o_ref[sel]).max()
    scale = np.abs(o_ref[sel]).max()
    assert err <= tol, f"max abs error {err} > {tol}"
    assert err <= tol * scale, f"max abs error {err} > {tol} * max|o| ({scale})"
    return err, scale
