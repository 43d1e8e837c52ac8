"""The seeded input generators: determinism, storage rounding and the top-k stand-in."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10).astype(np.float32)
    x[:4] = [0.0, -0.0, 1e-40, -3.3895314e38]
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(workloads.bf16_bits_to_f32(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_inputs_are_deterministic_and_shaped():
    cfg = workloads.config("ragged", B=3, ctx=(5, 20), V=300, Hq=2, Hkv=1, Dh=16)
    a = workloads.make_inputs(cfg)
    b = workloads.make_inputs(cfg)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    B, N = cfg.B, cfg.N
    assert a["q"].shape == (B, N, 2, 16) and a["q"].dtype == np.uint16
    assert a["k_ctx"].shape == (int(a["ctx_offsets"][-1]), 1, 16)
    assert np.all((a["ctx_lens"] >= 5) & (a["ctx_lens"] <= 20))
    assert a["uniforms"].shape == (B, N, 2) and a["uniforms"].dtype == np.uint64
    assert a["draft_logits"].shape == (B, cfg.D + 1, cfg.V)
    assert a["draft_logits"].dtype == np.float32
    # the generator holds no step arithmetic: no top-K or log-probs in it
    assert not {"draft_lp", "draft_tok", "draft_tok_all"} & set(a)


def test_uniform_streams_are_per_request():
    u0 = workloads.uniforms_for(7, 0, 5)
    u1 = workloads.uniforms_for(7, 1, 5)
    assert u0.shape == (5, 2) and not np.array_equal(u0, u1)
    assert np.array_equal(u0, workloads.uniforms_for(7, 0, 5))
