"""Entry points on caller streams other than torch's current one, and
forwards from several host threads, through the C ABI.

Each entry point is called with ``stream=`` a side stream that is still busy
with earlier work, and torch's current stream then at once allocates and
fills fresh memory: the temporaries the binding hands the library (the
workspaces it drops on return) must not be given to that allocation while the
side stream's kernels still use them.  Every result must equal the same call
on torch's current stream, bit for bit.  Two host threads forwarding layers
with a shared expert on two streams, one of them capturing a graph, must not
see each other's work either.
"""
import threading

import numpy as np
import pytest
import torch

import workloads
from gpu_common import device_inputs, log, to_device

pytestmark = pytest.mark.gpu

rdg = pytest.importorskip("route_dispatch_grouped_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from conftest import ensure_library
    ensure_library()
    yield
    torch.cuda.synchronize()


def _busy(stream, mb=256):
    """Queue some milliseconds of unrelated work on `stream`, so that what is
    enqueued after it has not started when the host returns."""
    with torch.cuda.stream(stream):
        a = torch.empty((mb << 20) // 4, dtype=torch.float32, device="cuda")
        for _ in range(8):
            a.fill_(1.0)
            a.mul_(1.0001)
    return a


def _clobber(n_bytes):
    """Allocate and fill memory on torch's current stream (the memory the
    caching allocator hands out first if a dropped temporary were reusable)."""
    out = []
    for size in (n_bytes, n_bytes // 2, 1 << 20, 4096):
        t = torch.empty(max(size, 256), dtype=torch.uint8, device="cuda")
        t.fill_(0xA5)
        out.append(t)
    return out


def _same(a, b, name):
    assert set(a) == set(b), name
    for k in a:
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), f"{name}: {k}"


@pytest.mark.parametrize("name", ["prefill", "decode_shared"])
def test_entry_points_on_a_busy_side_stream(name):
    if name == "prefill":
        cfg = workloads.config("qwen3_30b_a3b_prefill").scaled(num_tokens=2048, hidden_size=512, num_experts=16,
                                                                top_k=4, intermediate_size=256)
    else:
        cfg = workloads.config("qwen15_moe_decode").scaled(num_tokens=16, hidden_size=256, num_experts=60, top_k=4,
                                                            intermediate_size=192, shared_intermediate_size=320)
    log(f"[streams] {name}: {cfg}")
    inp = workloads.generate(cfg, seed=31)
    d = device_inputs(inp)
    k, E = cfg.top_k, cfg.num_experts
    shared = dict(shared_w13=d.get("shared_w13"), shared_w2=d.get("shared_w2"), shared_gate=d.get("shared_gate"))

    def calls(stream):
        r = rdg.moe_router_topk(d["x"], d["router_weight"], k, shared_gate=d.get("shared_gate"), return_probs=True,
                                stream=stream)
        yield "router", r
        if E % 4 == 0:
            yield "router_grouped", rdg.moe_router_topk_grouped(d["x"], d["router_weight"], k, 4, 2, stream=stream)
        plan = rdg.moe_dispatch_plan(r["topk_ids"], r["topk_weights"], E, stream=stream)
        yield "plan", plan
        yield "ep", rdg.moe_ep_routing_table(r["topk_ids"], r["topk_weights"], cfg.num_tokens, k, E // 4, E // 2,
                                             stream=stream)
        yield "ranks", rdg.moe_ep_rank_counts(plan["offsets"], 4, stream=stream)
        y = rdg.moe_grouped_ffn(d["x"], plan["packed_ids"], plan["offsets"], d["w13"], d["w2"], k, stream=stream)
        yield "ffn", {"y": y}
        yield "combine", {"out": rdg.moe_combine(y, plan["inv"], r["topk_weights"], stream=stream)}
        f = rdg.moe_forward(d["x"], d["router_weight"], d["w13"], d["w2"], k, return_routing=True, stream=stream,
                            **shared)
        yield "forward", f

    ref = {}
    for nm, res in calls(None):
        ref[nm] = {kk: v.clone() for kk, v in res.items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    keep = []
    got = {}
    for nm, res in calls(side):
        keep.append(_busy(side, 64))  # the next call queues behind more work
        keep.append(_clobber(64 << 20))
        got[nm] = res
    side.synchronize()
    torch.cuda.synchronize()
    for nm in ref:
        _same(got[nm], ref[nm], nm)


def _layer(cfg, seed):
    inp = workloads.generate(cfg, seed=seed)
    d = device_inputs(inp)
    layer = rdg.MoeLayer(d["router_weight"], d["w13"], d["w2"], cfg.top_k, router_bias=d.get("router_bias"),
                         shared_w13=d.get("shared_w13"), shared_w2=d.get("shared_w2"),
                         shared_gate=d.get("shared_gate"), renormalize=cfg.renormalize)
    return layer, d["x"]


def test_two_host_threads_with_shared_experts_one_capturing():
    """Thread A captures a forward of layer A into a graph on its stream while
    thread B runs eager forwards of layer B on another stream; then both run
    again concurrently (A replaying).  Each layer has a shared expert, which
    goes through the library's second stream of its caller stream.  Every
    result equals its layer run alone, bit for bit."""
    cfg_a = workloads.config("qwen15_moe_decode").scaled(num_tokens=16, hidden_size=256, num_experts=60, top_k=4,
                                                          intermediate_size=192, shared_intermediate_size=320)
    cfg_b = workloads.config("qwen15_moe_decode").scaled(num_tokens=40, hidden_size=512, num_experts=20, top_k=3,
                                                          intermediate_size=128, shared_intermediate_size=512)
    la, xa = _layer(cfg_a, 41)
    lb, xb = _layer(cfg_b, 42)
    ref_a = la(xa).clone()
    ref_b = lb(xb).clone()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for s in (sa, sb):
        s.wait_stream(torch.cuda.current_stream())
    # warm-up on both streams (the library makes each caller stream's
    # shared-expert stream there, outside any capture)
    with torch.cuda.stream(sa):
        la(xa)
    with torch.cuda.stream(sb):
        lb(xb)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    outs_b, errors, box = [], [], {}
    start = threading.Barrier(2)

    def run_a():
        try:
            start.wait()
            with torch.cuda.graph(graph, stream=sa, capture_error_mode="thread_local"):
                box["out"] = la(xa)
            for _ in range(5):
                with torch.cuda.stream(sa):
                    graph.replay()
                sa.synchronize()
                box.setdefault("replays", []).append(box["out"].clone())
        except Exception as e:  # reported below
            errors.append(("A", repr(e)))

    def run_b():
        try:
            start.wait()
            with torch.cuda.stream(sb):
                for _ in range(12):
                    outs_b.append(lb(xb).clone())
            sb.synchronize()
        except Exception as e:
            errors.append(("B", repr(e)))

    ta, tb = threading.Thread(target=run_a), threading.Thread(target=run_b)
    ta.start()
    tb.start()
    ta.join(timeout=120)
    tb.join(timeout=120)
    assert not ta.is_alive() and not tb.is_alive(), "a host thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    assert len(box.get("replays", [])) == 5 and len(outs_b) == 12
    for i, o in enumerate(box["replays"]):
        assert torch.equal(o, ref_a), f"replay {i}"
    for i, o in enumerate(outs_b):
        assert torch.equal(o, ref_b), f"thread B forward {i}"
