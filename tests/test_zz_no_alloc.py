"""moe_dispatch_plan_noalloc (the dispatch plan with the library's fixed
device scratch instead of a workspace, for callers that cannot allocate)
against moe_dispatch_plan, through the C ABI, bit for bit: two calls in a row
into the same preallocated outputs, the second with a smaller input, and the
size limit rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import oracle

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


def _ids(T, E, k, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    return torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()


def test_noalloc_plan_equals_workspace_plan():
    lib = rdg.load_library()
    assert lib.moe_dispatch_noalloc_max_workspace() == 8 << 20
    E = 128
    Pmax = 8192 * 8
    out = {
        "counts": torch.full((E,), -1, dtype=torch.int32, device="cuda"),
        "offsets": torch.full((E + 1,), -1, dtype=torch.int32, device="cuda"),
        "perm": torch.full((Pmax,), -1, dtype=torch.int32, device="cuda"),
        "inv": torch.full((Pmax,), -1, dtype=torch.int32, device="cuda"),
        "packed_ids": torch.full((Pmax,), -1, dtype=torch.int32, device="cuda"),
        "packed_w": torch.full((Pmax,), -1.0, dtype=torch.float32, device="cuda"),
    }
    # the large call, then a smaller one into the same buffers (segmented
    # passes both), then one on the single-workgroup path (P <= 4096)
    for T, k, seed in ((8192, 8, 1), (3001, 8, 2), (1000, 4, 3)):
        P = T * k
        ids, w = _ids(T, E, k, seed)
        view = {n: (t[:P] if t.numel() >= Pmax else t) for n, t in out.items()}
        rdg.moe_dispatch_plan_noalloc(ids, w, E, view)
        ref = rdg.moe_dispatch_plan(ids, w, E)
        torch.cuda.synchronize()
        for n in ("counts", "offsets", "perm", "inv", "packed_ids", "packed_w"):
            assert torch.equal(view[n].view(torch.int32), ref[n].view(torch.int32)), (T, n)
        # and the oracle's plan of the same ids
        o = oracle.dispatch_plan(ids.cpu().numpy(), w.cpu().numpy(), E)
        for n in ("counts", "offsets", "perm", "inv", "packed_ids"):
            assert (view[n].cpu().numpy() == o[n]).all(), (T, n)


def test_noalloc_plan_rejects_sizes_past_the_fixed_scratch():
    lib = rdg.load_library()
    P16 = ctypes.c_void_p(4096)
    # E = 512: each 128-assignment segment needs 2 * 512 ints of scratch, so
    # 8 MiB covers 2048 segments (262144 assignments); one more is rejected
    st = lib.moe_dispatch_plan_noalloc(P16, None, 262144 + 128, 1, 512, P16, P16, P16, P16, P16, None, None)
    assert st == 2 and "dispatch scratch" in lib.moe_last_error_message().decode()
