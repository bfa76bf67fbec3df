"""Decode as one tile stream per wave, through the C ABI: the shapes that make a
wave cross many units (pieces of requests, column passes) in a row.

- hundreds of 1-5 token requests, so most units are a single tile and the
  next unit's queries are fetched in the step that reads the current one's;
- the same with the new-token write fused into decode (every unit opening
  writes its request's new row first);
- query-head groups of 24 and 48 (waves with 16- and 8-column passes) on the
  decode path and for speculative verify;
- one long request surrounded by tiny ones (a share holding both);
- KV-head counts that pack 1 to 8 shares into one workgroup.

Outputs are checked against the fp64 oracle (bf16: max-abs 2e-2, rel-RMS 5e-3;
fp8: 5e-2, 2e-2; lse within 4e-3), pools byte for byte after the fused write.
"""
import numpy as np
import pytest
import torch

import workloads
from tests.oracle_ref import LSE_ATOL, TOL, errors, oracle_full, oracle_pools, raw_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_attention_02_amd as pka
    from tests.gpu_problem import GpuProblem


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[case] {request.node.name}", flush=True)


DEC = workloads.Spec("stream_decode", "decode", 1, 8, 2, 128, 16, "bf16", "bf16", seed=141)


def _run(spec, seq_lens=None, extend_lens=None, mode=None, spec_mode="prefill", prefix_only=False,
         name=""):
    layout = workloads.make_layout(spec, seq_lens=seq_lens, extend_lens=extend_lens)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values, prefix_only=prefix_only)
    if mode is not None:
        prob.mode = mode
        prob.md = pka.Batch(prob.ctx, mode, layout.batch, layout.num_q_tokens, layout.kv_pages)
        prob.metadata_step()
    prob.attention_step(save=True, spec_mode=spec_mode)
    torch.cuda.synchronize()
    status = prob.md.status()
    ref, ref_lse = oracle_full(layout, values)
    got = prob.out_np()
    max_abs, rel = errors(got, ref)
    tol_abs, tol_rel = TOL[spec.kv_dtype]
    print(f"[parity] {name or spec.name}: B={layout.batch} max_abs={max_abs:.2e} rel={rel:.2e}", flush=True)
    assert status == 0, status
    assert np.all(np.isfinite(got))
    assert max_abs <= tol_abs and rel <= tol_rel, (max_abs, rel)
    np.testing.assert_allclose(prob.lse_np(), ref_lse, rtol=0, atol=LSE_ATOL)
    return prob, layout, values


@pytest.mark.parametrize("kv,P", [("bf16", 1), ("bf16", 16), ("fp8", 4)])
def test_many_tiny_requests(kv, P):
    rng = np.random.default_rng(142)
    lens = rng.integers(1, 6, size=300).tolist()
    _run(DEC.replace(batch=len(lens), kv_dtype=kv, page_size=P, seed=142), seq_lens=lens,
         name=f"300 tiny requests {kv} P={P}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_many_tiny_requests_fused_write(kv):
    """The new tokens' slots start as NaN sentinels: only the write fused into
    the decode kernel fills them, before the tile holding them is loaded."""
    rng = np.random.default_rng(143)
    lens = rng.integers(1, 6, size=257).tolist()
    prob, layout, values = _run(DEC.replace(batch=len(lens), kv_dtype=kv, page_size=2, seed=143),
                                seq_lens=lens, prefix_only=True, name=f"fused write, tiny {kv}")
    kp, vp = oracle_pools(layout, raw_np(values.k_all), raw_np(values.v_all), values.k_scale,
                          values.v_scale)
    assert raw_np(prob.k_pool).tobytes() == kp.tobytes()
    assert raw_np(prob.v_pool).tobytes() == vp.tobytes()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("hq,hkv", [(48, 2), (48, 1), (96, 2)])
def test_groups_with_uneven_passes(hq, hkv, kv):
    _run(DEC.replace(batch=7, num_q_heads=hq, num_kv_heads=hkv, kv_dtype=kv,
                     seq_len_kind="uniform", seq_len_args=(1, 700), seed=144),
         name=f"decode {hq}/{hkv} {kv}")


@pytest.mark.parametrize("hq,hkv", [(48, 2), (24, 1)])
def test_verify_groups_with_uneven_passes(hq, hkv):
    spec = workloads.Spec("stream_verify", "extend", 6, hq, hkv, 128, 16, "bf16", "bf16", seed=145,
                          new_len_args=(0, 6), prefix_len_args=(1, 600))
    _run(spec, mode="target_verify", spec_mode="decode", prefix_only=True,
         name=f"verify {hq}/{hkv}")


def test_long_request_among_tiny_ones():
    lens = [3, 1, 2] * 20 + [9000] + [1, 4, 2] * 20
    _run(DEC.replace(batch=len(lens), page_size=16, seed=146), seq_lens=lens, name="long among tiny")


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("hq,hkv", [(3, 3), (12, 6), (16, 8), (32, 16), (24, 12)])
def test_workgroup_layouts(hq, hkv, kv):
    """KV-head counts giving 1, 2, 4 and 8 units per share and odd counts: the
    MFMA kernel packs 8 / units-per-share shares into one 8-wave workgroup
    (waves wv and wv ^ 4 then balance each other); the fp32 kernel runs
    workgroups of at most 4 waves."""
    qd = "f32" if kv == "f32" else "bf16"
    _run(DEC.replace(batch=9, num_q_heads=hq, num_kv_heads=hkv, q_dtype=qd, kv_dtype=kv,
                     seq_len_kind="uniform", seq_len_args=(1, 1200), seed=147),
         name=f"decode {hq}/{hkv} {kv}")
