"""The seeded input generator: determinism, ranges and the bf16 rounding
(checked against torch's own fp32 -> bfloat16 conversion)."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    gen = np.random.default_rng(0)
    x = np.concatenate([gen.standard_normal(100_000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, 3.0e38, -1e-40, 65504.0], np.float32)])
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = workloads.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_uniforms_range_and_determinism():
    u1 = workloads.uniforms(workloads.rng(7, 1), (1000, 3))
    u2 = workloads.uniforms(workloads.rng(7, 1), (1000, 3))
    u3 = workloads.uniforms(workloads.rng(7, 2), (1000, 3))
    assert u1.dtype == np.float32 and np.array_equal(u1, u2) and not np.array_equal(u1, u3)
    assert (u1 >= 0).all() and (u1 < 1).all()
    assert np.array_equal(u1 * 2**24, np.floor(u1 * 2**24))  # exact 24-bit values


def test_small_case_shapes():
    c = workloads.make_verify_case(3, 4, 50, "bf16", seed=1, verify_len=[0, 2, 4],
                                   temperature=[0.0, 1.0, 0.5])
    assert c.target.shape == (3, 5, 50) and c.target.dtype == np.uint16
    assert c.draft.shape == (3, 4, 50) and c.draft_tokens.shape == (3, 4)
    assert (c.draft_tokens >= 0).all() and (c.draft_tokens < 50).all()
    # at T = 0 the draft tokens are the draft argmaxes
    assert np.array_equal(c.draft_tokens[0], np.argmax(workloads.as_f32(c.draft[0]), axis=1))
    c2 = workloads.make_verify_case(3, 4, 50, "bf16", seed=1, verify_len=[0, 2, 4],
                                    temperature=[0.0, 1.0, 0.5])
    assert np.array_equal(c.target, c2.target) and np.array_equal(c.draft_tokens, c2.draft_tokens)


def test_named_small_workloads():
    t = workloads.tiny_chain()
    assert t.target.shape == (1, 5, 32) and t.target.dtype == np.float32
    g = workloads.truncated_geometric(workloads.rng(0, 6), 0.3, 7, 200_000)
    k = np.arange(8)
    w = 0.3 * 0.7 ** k
    assert abs(g.mean() - (k * w).sum() / w.sum()) < 0.02
    assert g.min() == 0 and g.max() == 7


def test_algorithmic_bytes():
    assert workloads.algorithmic_bytes(np.array([0, 7]), 10, 2, 2) == (1 + 15) * 10 * 2
