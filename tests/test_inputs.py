"""The seeded input generator shared by the oracle and the HIP path."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * rng.choice([1e-3, 1.0, 1e3], 100000)).astype(np.float32)
    # include exact ties of the bf16 grid
    ties = (np.arange(-50, 50, dtype=np.float32) * 2 ** -8 + 1.0 + 2 ** -9).astype(np.float32)
    x = np.concatenate([x, ties])
    ours = workloads.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_dapo_lengths_drawn_first():
    w = workloads.WORKLOADS["dapo_long"]
    rng = np.random.default_rng(w.seed)
    L = rng.integers(1024, 4096, endpoint=True, size=w.n_resp)
    assert L.tolist() == [3597, 1827, 1359, 1941, 2295, 3526, 2410, 1306,
                          2053, 2868, 3522, 3262, 4075, 1601, 3728, 1193]
    assert int(L.sum()) == 40563


def test_tiny_draws_are_seeded_and_shaped():
    w = workloads.WORKLOADS["tiny_f32"]
    a = workloads.generate(w)
    b = workloads.generate(w)
    assert a.q.shape == (192, 2, 64) and a.k.shape == (192, 2, 64)
    np.testing.assert_array_equal(a.q, b.q)
    rng = np.random.default_rng(0)
    np.testing.assert_array_equal(a.q, rng.standard_normal((192, 2, 64), dtype=np.float32))
    wb = workloads.WORKLOADS["tiny_bf16"]
    c = workloads.generate(wb)
    np.testing.assert_array_equal(c.q, workloads.round_to_bf16(a.q))


def test_workload_sizes():
    W = workloads.WORKLOADS
    assert W["qwen3_8b"].packed_len == 40960 and W["qwen3_8b"].replicated_len == 294912
    assert W["moe_30b"].packed_len == 81920 and W["moe_30b"].replicated_len == 589824
    assert W["gemma_global"].packed_len == 122880
    assert W["tiny_f32"].packed_len == 192 and W["tiny_f32"].replicated_len == 384
