"""K-blocked expert weights (MOE_DTYPE_BF16_KB32) on the GPU, through the C ABI.

The packed layout only moves bytes: moe_pack_weights must equal the plain
reshape of its definition (include/moe.h), and a layer run on packed weights
must give bit for bit the outputs of the same layer on row-major weights (the
same tiles sum the same products in the same order; only the addresses of the
weight fetches differ).  The row-major layer is checked against the float64
oracle in test_gpu_parity.py, every token at full size, so the packed layer
that bench.py times is checked through it."""
import numpy as np
import pytest
import torch

import route_dispatch_grouped_amd as rdg
import workloads
from gpu_common import device_inputs, full_inputs, log, to_device

pytestmark = pytest.mark.gpu

BF16_SMALL = {
    "multi_tile": dict(base="qwen3_30b_a3b_prefill", num_tokens=1000, hidden_size=512, num_experts=8, top_k=2,
                       intermediate_size=384),
    "decode_shared": dict(base="qwen15_moe_decode", num_tokens=16, hidden_size=256, num_experts=60, top_k=4,
                          intermediate_size=192, shared_intermediate_size=320),
    "mid_rows": dict(base="qwen3_30b_a3b_prefill", num_tokens=333, hidden_size=128, num_experts=16, top_k=3,
                     intermediate_size=128),
    "pipe_tiles": dict(base="qwen3_30b_a3b_prefill", num_tokens=8192, hidden_size=512, num_experts=16, top_k=8,
                       intermediate_size=256),
    "big_short_k": dict(base="qwen3_30b_a3b_prefill", num_tokens=600, hidden_size=64, num_experts=2, top_k=1,
                        intermediate_size=64),
    # K not a multiple of 32 in both GEMMs: the packed weights' last block is padded
    "h1000_i80": dict(base="qwen3_30b_a3b_prefill", num_tokens=1200, hidden_size=1000, num_experts=4, top_k=2,
                      intermediate_size=80),
    "h136_decode": dict(base="qwen15_moe_decode", num_tokens=16, hidden_size=136, num_experts=60, top_k=4,
                        intermediate_size=96, shared_intermediate_size=176),
    "tp8_pipe": dict(base="qwen3_30b_a3b_prefill", num_tokens=4096, hidden_size=512, num_experts=16, top_k=8,
                     intermediate_size=96),
    # packed w2 under a down projection that reads row-major h in whole lines
    "rowmajor_h_down": dict(base="qwen3_30b_a3b_prefill", num_tokens=2048, hidden_size=160, num_experts=8, top_k=2,
                            intermediate_size=256),
}


def small_cfg(name):
    kw = dict(BF16_SMALL[name])
    base = kw.pop("base")
    return workloads.config(base).scaled(name=name, **kw)


def kb32_reference(w: np.ndarray) -> np.ndarray:
    """The definition of include/moe.h, written out: dst[g][b][r][i] =
    src[g][r][32 b + i], zero past k."""
    G, R, K = w.shape
    KB = (K + 31) // 32
    pad = np.zeros((G, R, KB * 32), dtype=w.dtype)
    pad[:, :, :K] = w
    return pad.reshape(G, R, KB, 32).transpose(0, 2, 1, 3).copy()


@pytest.mark.parametrize("G,R,K", [(3, 64, 64), (2, 50, 40), (1, 7, 8), (4, 96, 1000), (1, 2048, 1408)])
def test_pack_weights_matches_its_definition(G, R, K):
    rng = np.random.default_rng(G * 1000 + R + K)
    w = rng.integers(0, 2 ** 16, size=(G, R, K), dtype=np.uint16)
    p = rdg.pack_weights(to_device(w))
    got = p.data.view(torch.int16).cpu().numpy().view(np.uint16)
    assert got.shape == (G * ((K + 31) // 32) * R * 32,)
    assert (got == kb32_reference(w).reshape(-1)).all()
    assert p.shape == (G, R, K)


def layer_outputs(cfg, dev, pack):
    layer = rdg.MoeLayer(dev["router_weight"], dev["w13"], dev["w2"], cfg.top_k, router_bias=dev.get("router_bias"),
                         shared_w13=dev.get("shared_w13"), shared_w2=dev.get("shared_w2"),
                         shared_gate=dev.get("shared_gate"), renormalize=cfg.renormalize, pack=pack)
    out = layer(dev["x"]).clone()
    torch.cuda.synchronize()
    return out


def check_bit_equal(cfg, dev):
    a = layer_outputs(cfg, dev, pack=False)
    b = layer_outputs(cfg, dev, pack=True)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    return a


@pytest.mark.parametrize("name", list(BF16_SMALL))
def test_packed_layer_bit_equal_to_row_major(name):
    cfg = small_cfg(name)
    log(f"[packed] {name}: {cfg}")
    inp = workloads.generate(cfg, seed=1)
    dev = device_inputs(inp)
    check_bit_equal(cfg, dev)
    # the grouped FFN stage alone, fp32 and bf16 expert outputs
    r = rdg.moe_router_topk(dev["x"], dev["router_weight"], cfg.top_k)
    plan = rdg.moe_dispatch_plan(r["topk_ids"], r["topk_weights"], cfg.num_experts)
    w13p, w2p = rdg.pack_weights(dev["w13"]), rdg.pack_weights(dev["w2"])
    for out_dtype in (torch.float32, torch.bfloat16):
        y = rdg.moe_grouped_ffn(dev["x"], plan["packed_ids"], plan["offsets"], dev["w13"], dev["w2"], cfg.top_k,
                                out_dtype=out_dtype)
        yp = rdg.moe_grouped_ffn(dev["x"], plan["packed_ids"], plan["offsets"], w13p, w2p, cfg.top_k,
                                 out_dtype=out_dtype)
        assert torch.equal(y.view(torch.int16), yp.view(torch.int16)), out_dtype


@pytest.mark.parametrize("shape", [(1500, 384, 6, 2, 256), (2400, 640, 10, 4, 320), (1000, 200, 5, 3, 144),
                                   (2048, 192, 24, 6, 208), (1200, 136, 8, 2, 400), (2500, 512, 20, 8, 160)],
                         ids=lambda t: "T%d_H%d_E%d_k%d_I%d" % t)
def test_packed_layer_bit_equal_mixed_shapes(shape):
    """Layers of the mixed parity shapes (whole-line A, padded K loops, K
    tails, down on the plain 256-row kernel) on packed weights."""
    T, H, E, k, I = shape
    cfg = workloads.config("qwen3_30b_a3b_prefill").scaled(name="packed_mixed", num_tokens=T, hidden_size=H,
                                                            num_experts=E, top_k=k, intermediate_size=I)
    check_bit_equal(cfg, device_inputs(workloads.generate(cfg, seed=3)))


@pytest.mark.parametrize("name", ["qwen15_moe_decode", "qwen3_30b_a3b_prefill", "qwen3_30b_a3b_prefill_zipf",
                                  "dwdp_h4096_e64"])
def test_packed_layer_bit_equal_at_full_size(name):
    cfg, inp = full_inputs(name)
    dev = device_inputs(inp)
    out = check_bit_equal(cfg, dev)
    log(f"[packed] {name}: packed and row-major outputs equal, rms {float(out.float().pow(2).mean().sqrt()):.3e}")
    del dev
    torch.cuda.empty_cache()


def test_mixed_packed_and_row_major_weights_rejected():
    cfg = small_cfg("mid_rows")
    dev = device_inputs(workloads.generate(cfg, seed=2))
    with pytest.raises(ValueError):
        rdg.moe_forward(dev["x"], dev["router_weight"], rdg.pack_weights(dev["w13"]), dev["w2"], cfg.top_k)
