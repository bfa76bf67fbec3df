"""The cache write inside forward(save_kv_cache=True), through the C ABI.

The pools start with every prefix token written and the new tokens' slots
still holding the NaN sentinel, so only the forward pass's own write (fused
into the decode kernel for bf16 / fp8 caches, a separate kernel otherwise)
can put them there.  Pools must then equal the oracle's cache write bit for
bit, and outputs must be within the oracle tolerances (bf16/fp32: max-abs
2e-2, rel-RMS 5e-3; fp8: 5e-2, 2e-2).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.oracle_ref import LSE_ATOL, TOL, errors, oracle_full, oracle_pools, raw_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests.gpu_problem import GpuProblem


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[case] {request.node.name}", flush=True)


CASES = {
    "decode_bf16_p16": workloads.WORKLOADS["llama3_8b_decode"].replace(batch=11, seq_len_args=(1, 900)),
    "decode_bf16_p1_g16": workloads.WORKLOADS["qwen3_235b_decode"].replace(batch=5, seq_len_kind="uniform",
                                                       seq_len_args=(1, 700)),
    "decode_fp8_p64": workloads.WORKLOADS["long_fp8_decode"].replace(batch=7, seq_len_args=(1, 1500)),
    "decode_fp8_d64_g32": workloads.Spec("fp8_d64_g32", "decode", 4, 64, 2, 64, 32, "bf16", "fp8",
                                         seed=61, seq_len_kind="uniform", seq_len_args=(1, 600)),
    "decode_f32": workloads.WORKLOADS["tiny_decode"],
    "extend_bf16": workloads.WORKLOADS["llama3_8b_extend"].replace(batch=3, new_len_args=(1, 200),
                                                prefix_len_args=(0, 300)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_forward_writes_the_new_tokens(name):
    spec = CASES[name]
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values, prefix_only=True)
    prob.attention_step(save=True)
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    kp, vp = oracle_pools(layout, raw_np(values.k_all), raw_np(values.v_all), values.k_scale,
                          values.v_scale)
    for got, ref in ((prob.k_pool, kp), (prob.v_pool, vp)):
        g = raw_np(got)
        if g.dtype == np.float32:
            g, ref = g.view(np.uint32), ref.view(np.uint32)
        np.testing.assert_array_equal(g, ref)
    out_ref, lse_ref = oracle_full(layout, values)
    max_abs, rel = errors(prob.out_np(), out_ref)
    tol_abs, tol_rel = TOL[spec.kv_dtype]
    print(f"[parity] {name}: max_abs={max_abs:.2e} rel={rel:.2e}", flush=True)
    assert max_abs <= tol_abs and rel <= tol_rel, (max_abs, rel)
    np.testing.assert_allclose(prob.lse_np(), lse_ref, rtol=0, atol=LSE_ATOL)


def test_without_the_write_the_sentinel_is_read():
    """Control: the same batch with save_kv_cache=False attends to the NaN
    sentinel in every new token's slot."""
    spec = CASES["decode_bf16_p16"]
    layout = workloads.make_layout(spec)
    prob = GpuProblem(layout, prefix_only=True)
    prob.attention_step(save=False)
    torch.cuda.synchronize()
    assert torch.isnan(prob.out.float()).any(dim=-1).all()


@pytest.mark.parametrize("cfg", ["llama3_8b_decode", "long_fp8_decode"])
def test_full_size_new_token_rows(cfg):
    """Full-size decode batches: every new token's slot holds exactly the
    oracle's encoding of that token (bf16 copy or fp8 quantisation)."""
    spec = workloads.WORKLOADS[cfg]
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values, prefix_only=True)
    prob.step()
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    for new, pool, scale in ((prob.k_new, prob.k_pool, values.k_scale),
                             (prob.v_new, prob.v_pool, values.v_scale)):
        got = raw_np(pool[prob.new_slots])
        src = raw_np(new)
        want = src if spec.kv_dtype == "bf16" else oracle.fp8_quantize(src, scale)
        np.testing.assert_array_equal(got, want.reshape(got.shape))
