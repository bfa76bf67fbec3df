"""Key and value heads of different widths (192-wide query/key heads, 128-wide
value/output heads), through the C ABI.

The pages have one backend picked for models whose K and V head widths
differ ("sglang-101 s4.2 --attention-backend", backend table and "How SGLang
picks a default"); here the same paged path (metadata, cache write, decode,
extend, speculative verify on the decode path) runs with head_dim = 192 and
v_head_dim = 128.  The cache write must be bit-exact; outputs are held to the
same gates as the equal-width workloads (bf16 / fp32: max-abs 2e-2, rel-RMS
5e-3; fp8: 5e-2, 2e-2) against the fp64 oracle.
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
    from tests.test_gpu_parity import _sampled


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[case] {request.node.name}", flush=True)


DEC = workloads.Spec("asym_decode_small", "decode", 7, 16, 4, 192, 16, "bf16", "bf16", seed=121,
                     seq_len_kind="uniform", seq_len_args=(1, 1500), v_head_dim=128)
EXT = workloads.Spec("asym_extend_small", "extend", 3, 16, 16, 192, 128, "bf16", "bf16", seed=122,
                     new_len_args=(1, 300), prefix_len_args=(0, 400), v_head_dim=128)


def _run(spec, mode=None, spec_mode="prefill", seq_lens=None, extend_lens=None, name=""):
    layout = workloads.make_layout(spec, seq_lens=seq_lens, extend_lens=extend_lens)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values, prefix_only=True)
    if mode is not None:
        prob.mode = mode
        prob.md = pka.Batch(prob.ctx, mode, layout.batch, layout.num_q_tokens, layout.kv_pages)
        prob.metadata_step()
    prob.attention_step(save=True, spec_mode=spec_mode)
    torch.cuda.synchronize()
    status = prob.md.status()
    ref, ref_lse = oracle_full(layout, values)
    got = prob.out_np()
    assert got.shape[-1] == spec.value_dim
    max_abs, rel = errors(got, ref)
    tol_abs, tol_rel = TOL[spec.kv_dtype]
    print(f"[parity] {name or spec.name}: max_abs={max_abs:.2e} rel={rel:.2e}", flush=True)
    assert status == 0, status
    assert np.all(np.isfinite(got))
    assert max_abs <= tol_abs and rel <= tol_rel, (max_abs, rel)
    np.testing.assert_allclose(prob.lse_np(), ref_lse, rtol=0, atol=LSE_ATOL)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_asym_save_kv_bit_exact(kv):
    spec = DEC.replace(kv_dtype=kv, batch=5, seq_len_args=(1, 300))
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values)
    kp, vp = oracle_pools(layout, raw_np(values.k_all), raw_np(values.v_all), values.k_scale,
                          values.v_scale)
    gk, gv = raw_np(prob.k_pool), raw_np(prob.v_pool)
    assert gk.shape[-1] == 192 and gv.shape[-1] == 128
    assert gk.tobytes() == kp.tobytes()
    assert gv.tobytes() == vp.tobytes()


@pytest.mark.parametrize("kv,P,hq,hkv", [
    ("bf16", 16, 16, 4), ("bf16", 1, 16, 16), ("bf16", 128, 32, 2),
    ("fp8", 64, 16, 4), ("fp8", 1, 8, 8),
])
def test_asym_decode(kv, P, hq, hkv):
    _run(DEC.replace(kv_dtype=kv, page_size=P, num_q_heads=hq, num_kv_heads=hkv, seed=121 + P),
         name=f"asym decode {kv} P={P} {hq}/{hkv}")


def test_asym_decode_f32():
    _run(DEC.replace(q_dtype="f32", kv_dtype="f32", batch=4, page_size=4, seq_len_args=(1, 400)),
         name="asym decode f32")


@pytest.mark.parametrize("kv,P,hq,hkv", [
    ("bf16", 128, 16, 16), ("bf16", 16, 16, 16), ("bf16", 1, 32, 8), ("bf16", 64, 64, 4),
    ("fp8", 128, 16, 16), ("fp8", 4, 16, 4),
])
def test_asym_extend(kv, P, hq, hkv):
    _run(EXT.replace(kv_dtype=kv, page_size=P, num_q_heads=hq, num_kv_heads=hkv, seed=122 + P),
         name=f"asym extend {kv} P={P} {hq}/{hkv}")


def test_asym_extend_f32():
    _run(EXT.replace(q_dtype="f32", kv_dtype="f32", page_size=8, new_len_args=(1, 40),
                     prefix_len_args=(0, 60)), name="asym extend f32")


def test_asym_extend_ragged():
    lens_new = [1, 0, 33, 64, 65, 130, 7]
    prefix = [0, 5, 0, 63, 64, 1, 300]
    spec = EXT.replace(batch=len(lens_new), page_size=32, seed=126)
    _run(spec, seq_lens=[p + n if p + n > 0 else 1 for p, n in zip(prefix, lens_new)],
         extend_lens=[n if p + n > 0 else 0 for p, n in zip(prefix, lens_new)], name="asym extend ragged")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_asym_verify_on_decode_path(kv):
    spec = EXT.replace(kv_dtype=kv, batch=6, page_size=16, num_q_heads=16, num_kv_heads=4,
                       new_len_args=(2, 8), prefix_len_args=(1, 900), seed=127)
    _run(spec, mode="target_verify", spec_mode="decode", name=f"asym verify {kv}")


def test_asym_extend_workload_sampled():
    """The 8-request prefill batch (new U[512, 2048] on prefixes U[0, 4096],
    16 heads, 192 / 128 widths, page 128) on sampled requests and tokens."""
    spec = workloads.EXTRA["asym_extend"]
    _sampled(None, lambda L: [int(np.argmax(L)), int(np.argmin(L)), 5], heads=[0, 7, 15],
             tokens=lambda n: sorted(set(list(range(0, n, 37)) + [n - 1])), spec=spec)


def test_asym_decode_workload_sampled():
    """64 decode requests, contexts U[512, 8192], 16 heads, 192 / 128 widths,
    page 128, on sampled requests."""
    spec = workloads.EXTRA["asym_decode"]
    _sampled(None, lambda L: [int(np.argmax(L)), int(np.argmin(L)), 0, 33], spec=spec)
