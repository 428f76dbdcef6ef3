"""Input generators: determinism, rounding, shapes and value ranges."""
import numpy as np
import torch

from linear_attention_recurrence_gated_amd import workloads as w


def test_bf16_round_matches_torch_rne():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10.0 ** r.integers(-8, 8, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-40], dtype=np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = w.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    bits = w.bf16_bits(got)
    assert np.array_equal(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy(), got)


def test_same_seed_same_bytes():
    a = w.make_prefill([70, 0, 33], H=3, d=16, seed=5, init_std=0.02)
    b = w.make_prefill([70, 0, 33], H=3, d=16, seed=5, init_std=0.02)
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.g, b.g), (a.beta, b.beta), (a.s_init, b.s_init)]:
        assert x.tobytes() == y.tobytes()
    assert list(a.cu_seqlens) == [0, 70, 70, 103]
    c = w.make_prefill([70, 0, 33], H=3, d=16, seed=6, init_std=0.02)
    assert c.q.tobytes() != a.q.tobytes()


def test_tiny_fp32_shapes_and_ranges():
    c = w.prefill_t64_d16_fp32()
    assert c.q.shape == (64, 1, 16) and c.v.shape == (64, 1, 16) and c.g.shape == (64, 1)
    assert c.dtype == "fp32" and c.cu_seqlens is None and c.s_init is None
    assert np.allclose(np.linalg.norm(c.k.astype(np.float64), axis=-1), 1.0, atol=1e-6)
    assert np.all((c.g > 0) & (c.g < 1)) and np.all((c.beta > 0) & (c.beta < 1))


def test_prefill_bf16_values_are_exact_and_normalised():
    c = w.prefill_t4096_h48(T=256, H=4)
    for x in (c.q, c.k, c.v):
        w.bf16_bits(x)  # raises if any value is not bf16-exact
    n = np.linalg.norm(c.k.astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1.0) < 2 ** -7)
    lg = np.log(c.g.astype(np.float64))
    assert -3.0 < lg.mean() < -1.5  # g = exp(-softplus(x + 2)): strong decay


def test_varlen_lengths_in_range_and_fixed():
    lens = w.varlen_lengths()
    assert len(lens) == 8 and all(1024 <= x <= 65536 for x in lens)
    assert lens == w.varlen_lengths()


def test_decode_shapes():
    c = w.make_decode(3, 2, 5, 16)
    assert c.q.shape == (3, 2, 5, 16) and c.g.shape == (3, 2, 5) and c.s_init.shape == (2, 5, 16, 16)
    assert abs(float(c.s_init.std()) - 0.02) < 0.005
