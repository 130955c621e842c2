"""Input generators: encodings and mask structure (no attention arithmetic here)."""
import numpy as np
import torch

from workloads import CONFIGS, bf16_bits, bf16_to_f32, causal_mask, make_workload


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -2.00390625, 0.0, -0.0], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(x), want)
    assert np.array_equal(bf16_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_dropped_sentinel_is_exact_in_fp16():
    assert float(np.float16(-30000.0)) == -30000.0


def test_causal_mask_shape_and_values():
    m = causal_mask(5, 3, 10)
    assert m.dtype == np.float16 and m.shape == (3, 10)
    for i in range(3):
        assert np.all(m[i, : 5 + i + 1] == 0) and np.all(m[i, 5 + i + 1:] == -30000)


def test_workloads_are_seeded_and_shaped():
    a = make_workload("tiny", cache=False)
    b = make_workload("tiny", cache=False)
    assert np.array_equal(a.Q, b.Q) and np.array_equal(a.V, b.V)
    s = CONFIGS["gqa4k"]
    w = make_workload("gqa4k")
    assert w.Q.shape == (s.N, s.n_q, s.d) and w.K.shape == (s.N, s.n_kv, s.d)
    assert w.Q.dtype == np.uint16
    # chunks tile the prompt exactly
    for name, spec in CONFIGS.items():
        ends = [q + c for q, c in spec.chunks]
        starts = [q for q, _ in spec.chunks]
        assert ends[-1] == spec.N and starts[1:] == ends[:-1], name
