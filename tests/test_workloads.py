"""The seeded input generator: determinism, shapes and the bf16 rounding rule."""
import numpy as np

import workloads


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                     -2.5, 3.140625, 0.0, -0.0], dtype=np.float32)
    bits = workloads.round_to_bf16_bits(vals)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)... check by value
    assert bits.tolist()[0] == 0x3F80
    assert bits.tolist()[1] == 0x3F80
    assert bits.tolist()[2] == 0x3F82
    assert bits.tolist()[3] == 0x3F81
    assert bits.tolist()[4] == 0xC020
    assert bits.tolist()[5] == 0x4049
    assert bits.tolist()[6] == 0x0000
    assert bits.tolist()[7] == 0x8000


def test_generate_deterministic_and_thread_independent():
    cfg = workloads.config("qwen15_moe_decode").scaled(hidden_size=64, intermediate_size=32,
                                                        shared_intermediate_size=48)
    a = workloads.generate(cfg, seed=0, threads=1)
    b = workloads.generate(cfg, seed=0, threads=4)
    c = workloads.generate(cfg, seed=1, threads=2)
    assert set(a) == {"x", "router_weight", "w13", "w2", "shared_w13", "shared_w2", "shared_gate"}
    for k in a:
        assert a[k].dtype == np.uint16
        assert (a[k] == b[k]).all()
        assert not (a[k] == c[k]).all()
    assert a["w13"].shape == (60, 64, 64)
    assert a["w2"].shape == (60, 64, 32)
    assert a["shared_w13"].shape == (96, 64)


def test_generate_distributions():
    cfg = workloads.config("tiny_fp32")
    a = workloads.generate(cfg)
    assert a["x"].dtype == np.float32
    assert abs(a["x"].std() - 1.0) < 0.05
    assert abs(a["w13"].std() - 0.02) < 0.001
    assert a["w13"].shape == (8, 512, 128) and a["w2"].shape == (8, 128, 256)


def test_zipf_bias():
    cfg = workloads.config("qwen3_30b_a3b_prefill_zipf")
    b = workloads.zipf_bias(cfg, 0)
    assert b.dtype == np.float32 and b.shape == (128,)
    assert (b == np.float32(-1e4)).sum() == 16
    rest = np.sort(b[b > -1000])[::-1]
    ranks = np.arange(1, 113)
    assert np.allclose(rest, -1.2 * np.log(ranks), rtol=1e-6, atol=1e-6)
