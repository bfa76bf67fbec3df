"""The extend work list the metadata kernel writes into the plan: every
(request, query tile) item exactly once, request by request -- requests
longest first (ties: lower index first), each request's tiles from its last
(heaviest: a tile's weight is the number of keys its last row attends to) to
its first -- so the workgroups resident together on an XCD share one
request's K/V pages in its L2; batches past the fused-metadata limit (1024
requests) keep request order, tiles last to first.  Covers small and large
fused batches and batches past the limit."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests.gpu_problem import GpuProblem

PLAN_EXT_COUNT, PLAN_EXT_TQ, PLAN_HDR, DEC_MAX_WG, FUSE_MAX_B = 4, 5, 80, 2048, 1024


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _spec(name, B, new, pfx, seed):
    return workloads.Spec(name, "extend", B, 8, 2, 128, 16, "bf16", "bf16", seed=seed,
                          new_len_args=new, prefix_len_args=pfx)


CASES = {
    "llama_extend": workloads.WORKLOADS["llama3_8b_extend"],
    "b64": _spec("ext_b64", 64, (300, 600), (0, 900), 111),
    "b200_ties": _spec("ext_b200", 200, (400, 700), (0, 300), 112),
    "b1024": _spec("ext_b1024", 1024, (0, 40), (1, 60), 115),
    "large_b1100": _spec("ext_b1100", 1100, (0, 2), (1, 50), 113),
    "large_b1500": _spec("ext_b1500", 1500, (1, 90), (0, 60), 114),
}


def expected_items(seq_lens, extend_lens, tq, ranked):
    B = len(seq_lens)
    order = sorted(range(B), key=lambda b: (-int(seq_lens[b]), b)) if ranked else list(range(B))
    items = []
    for b in order:
        n = int(extend_lens[b])
        items.extend((b, ti) for ti in reversed(range((n + tq - 1) // tq)))
    return np.array(items, dtype=np.int32).reshape(-1, 2)


@pytest.mark.parametrize("name", list(CASES))
def test_extend_items_request_by_request(name):
    layout = workloads.make_layout(CASES[name])
    prob = GpuProblem(layout, fill=False)
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    plan = prob.md.plan.cpu().numpy()
    B = layout.spec.batch
    count, tq = int(plan[PLAN_EXT_COUNT]), int(plan[PLAN_EXT_TQ])
    want = expected_items(np.asarray(layout.seq_lens), np.asarray(layout.extend_lens), tq,
                          ranked=B <= FUSE_MAX_B)
    print(f"[items] {name}: B={B} count={count} tq={tq}", flush=True)
    assert count == len(want)
    off = PLAN_HDR + 2 * (B + 1) + 2 * DEC_MAX_WG
    got = plan[off:off + 2 * count].reshape(-1, 2)
    assert np.array_equal(got, want)
