"""Extend (prefill) over an fp8 e4m3fn cache, through the C ABI.

The cache holds the quantised K/V (written by the library's save_kv); the
oracle attends to the same codes dequantised exactly (code value x scale in
fp64).  Gates: max-abs 5e-2, rel-RMS 2e-2 against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import workloads
from tests.oracle_ref import LSE_ATOL, TOL, errors, oracle_full

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests.gpu_problem import GpuProblem
    from tests.test_gpu_parity import _sampled


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[case] {request.node.name}", flush=True)


BASE = workloads.Spec("fp8_extend", "extend", 3, 32, 8, 128, 128, "bf16", "fp8", seed=91,
                      new_len_args=(1, 200), prefix_len_args=(0, 300))


def _run(spec, seq_lens=None, extend_lens=None, name=""):
    layout = workloads.make_layout(spec, seq_lens=seq_lens, extend_lens=extend_lens)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values, prefix_only=True)
    prob.attention_step(save=True)
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    ref, ref_lse = oracle_full(layout, values)
    got = prob.out_np()
    max_abs, rel = errors(got, ref)
    print(f"[parity] {name or spec.name}: max_abs={max_abs:.2e} rel={rel:.2e}", flush=True)
    assert np.all(np.isfinite(got))
    assert max_abs <= TOL["fp8"][0] and rel <= TOL["fp8"][1], (max_abs, rel)
    np.testing.assert_allclose(prob.lse_np(), ref_lse, rtol=0, atol=LSE_ATOL)


@pytest.mark.parametrize("P", [1, 16, 64, 128])
def test_fp8_extend_page_sizes(P):
    _run(BASE.replace(page_size=P, seed=91 + P), name=f"fp8 extend P={P}")


@pytest.mark.parametrize("hq,hkv,d,P", [(8, 8, 128, 64), (64, 8, 128, 16), (8, 2, 64, 32), (16, 2, 64, 128)])
def test_fp8_extend_groups_and_dims(hq, hkv, d, P):
    _run(BASE.replace(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=P, seed=95),
         name=f"fp8 extend {hq}/{hkv} d={d} P={P}")


def test_fp8_extend_ragged():
    lens_new = [1, 0, 33, 64, 65, 130, 7]
    prefix = [0, 5, 0, 63, 64, 1, 300]
    spec = BASE.replace(batch=len(lens_new), page_size=64, seed=96)
    _run(spec, seq_lens=[p + n if p + n > 0 else 1 for p, n in zip(prefix, lens_new)],
         extend_lens=[n if p + n > 0 else 0 for p, n in zip(prefix, lens_new)], name="fp8 extend ragged")


def test_fp8_extend_prefill_batch_sampled():
    """The 8-request prefill batch (new U[512, 2048] on prefixes U[0, 4096],
    page 128) with an fp8 cache, on sampled requests, heads and tokens."""
    spec = workloads.WORKLOADS["llama3_8b_extend"].replace(name="extend_fp8kv_b8_g4_d128_p128", kv_dtype="fp8")
    _sampled("llama3_8b_extend", lambda L: [int(np.argmax(L)), int(np.argmin(L)), 5], heads=[0, 7, 18, 31],
             tokens=lambda n: sorted(set(list(range(0, n, 41)) + [n - 1])), spec=spec)
