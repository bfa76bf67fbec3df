"""The extend work list the metadata kernel writes into the plan: every
(request, query tile) item exactly once, heaviest first (a tile's weight is
the number of keys its last row attends to; ties keep request order), or in
request order when there are more items than the in-LDS sort holds.  Covers
the rank sort (<= 512 items), the bitonic sort (<= 2048), the unsorted list,
and the same for batches past the fused-metadata limit (1024 requests)."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests.gpu_problem import GpuProblem

PLAN_EXT_COUNT, PLAN_EXT_TQ, PLAN_HDR, DEC_MAX_WG, SORT_MAX = 4, 5, 80, 2048, 2048


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _spec(name, B, new, pfx, seed):
    return workloads.Spec(name, "extend", B, 8, 2, 128, 16, "bf16", "bf16", seed=seed,
                          new_len_args=new, prefix_len_args=pfx)


CASES = {
    "rank_llama_extend": workloads.WORKLOADS["llama3_8b_extend"],
    "bitonic_b64": _spec("ext_b64", 64, (300, 600), (0, 900), 111),
    "request_order_b200": _spec("ext_b200", 200, (400, 700), (0, 300), 112),
    "large_bitonic_b1100": _spec("ext_b1100", 1100, (0, 2), (1, 50), 113),
    "large_request_order_b1500": _spec("ext_b1500", 1500, (1, 90), (0, 60), 114),
}


def expected_items(seq_lens, extend_lens, tq, sort):
    items, keys = [], []
    for b, (L, n) in enumerate(zip(seq_lens, extend_lens)):
        for ti in range((n + tq - 1) // tq):
            last = L - n + min((ti + 1) * tq, n)
            items.append((b, ti))
            keys.append(min(last, (1 << 20) - 1))
    if sort:
        order = sorted(range(len(items)), key=lambda i: (-keys[i], i))
        items = [items[i] for i in order]
    return np.array(items, dtype=np.int32).reshape(-1, 2)


@pytest.mark.parametrize("name", list(CASES))
def test_extend_items_heaviest_first(name):
    layout = workloads.make_layout(CASES[name])
    prob = GpuProblem(layout, fill=False)
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    plan = prob.md.plan.cpu().numpy()
    B = layout.spec.batch
    count, tq = int(plan[PLAN_EXT_COUNT]), int(plan[PLAN_EXT_TQ])
    want = expected_items(np.asarray(layout.seq_lens), np.asarray(layout.extend_lens), tq, sort=None)
    print(f"[items] {name}: B={B} count={count} tq={tq}", flush=True)
    assert count == len(want)
    want = expected_items(np.asarray(layout.seq_lens), np.asarray(layout.extend_lens), tq,
                          sort=count <= SORT_MAX)
    off = PLAN_HDR + 2 * (B + 1) + 2 * DEC_MAX_WG
    got = plan[off:off + 2 * count].reshape(-1, 2)
    assert np.array_equal(got, want)
