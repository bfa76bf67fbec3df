"""Large batches through the C ABI: more requests than one metadata
workgroup scans in a pass (multi-chunk scan, separate gather kernel) and more
extend items than the in-LDS sort holds (items left in request order).

Metadata must be bit-exact; attention within max-abs 2e-2 / rel-RMS 5e-3 of
the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.oracle_ref import LSE_ATOL, TOL, errors, oracle_full

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_attention_02_amd as pka
    from tests.gpu_problem import GpuProblem


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[case] {request.node.name}", flush=True)


CASES = {
    "decode_b3000_p16": workloads.Spec("decode_b3000", "decode", 3000, 8, 2, 128, 16, "bf16", "bf16",
                                       seed=101, seq_len_kind="uniform", seq_len_args=(1, 120)),
    "decode_b1100_p1": workloads.Spec("decode_b1100", "decode", 1100, 8, 8, 64, 1, "bf16", "bf16",
                                      seed=102, seq_len_kind="uniform", seq_len_args=(1, 90)),
    "extend_b1500_p16": workloads.Spec("extend_b1500", "extend", 1500, 8, 2, 128, 16, "bf16", "bf16",
                                       seed=103, new_len_args=(0, 70), prefix_len_args=(0, 60)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_large_batch_metadata_bit_exact(name):
    layout = workloads.make_layout(CASES[name])
    spec = layout.spec
    prob = GpuProblem(layout, fill=False)
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    ref = oracle.metadata(layout.seq_lens, None if spec.mode == "decode" else layout.extend_lens,
                          layout.page_table, spec.page_size, layout.num_pages)
    for k, v in ref.items():
        got = getattr(prob.md, k).cpu().numpy()
        assert np.array_equal(got[:v.size], v), k


@pytest.mark.parametrize("name", list(CASES))
def test_large_batch_attention(name):
    layout = workloads.make_layout(CASES[name])
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values)
    prob.attention_step(save=True)
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    ref, ref_lse = oracle_full(layout, values)
    got = prob.out_np()
    max_abs, rel = errors(got, ref)
    print(f"[parity] {name}: B={layout.batch} N={layout.num_q_tokens} max_abs={max_abs:.2e} rel={rel:.2e}",
          flush=True)
    bad = np.argwhere(~np.isfinite(got).all(axis=(1, 2)))[:, 0]
    if bad.size:
        qo = np.concatenate([[0], np.cumsum(layout.extend_lens)])
        reqs = np.searchsorted(qo, bad, side="right") - 1
        info = [(int(r), int(t - qo[r]), int(layout.seq_lens[r]), int(layout.extend_lens[r])) for t, r in
                zip(bad[:20], reqs[:20])]
        print(f"[diag] {bad.size} non-finite rows; (request, token, L, n): {info}", flush=True)
        print(f"[diag] requests hit: {sorted(set(int(r) for r in reqs))[:40]}", flush=True)
    assert np.all(np.isfinite(got))
    assert max_abs <= TOL["bf16"][0] and rel <= TOL["bf16"][1], (max_abs, rel)
    np.testing.assert_allclose(prob.lse_np(), ref_lse, rtol=0, atol=LSE_ATOL)
