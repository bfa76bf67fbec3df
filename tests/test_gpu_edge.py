"""GPU edge cases, invariances, dispatch and device status, through the C ABI.

Every output is compared with the fp64 oracle on the same seeded inputs
(bf16/fp32: max-abs 2e-2, rel-RMS 5e-3; fp8: 5e-2, 2e-2).
"""
import numpy as np
import pytest
import torch

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


def run_and_check(spec, seq_lens=None, extend_lens=None, spec_mode="prefill", mode=None,
                  pool_pages=None):
    layout = workloads.make_layout(spec, seq_lens=seq_lens, extend_lens=extend_lens,
                                   pool_pages=pool_pages)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values)
    if mode is not None:
        prob.mode = mode
        prob.md = pka.Batch(prob.ctx, mode, layout.batch, layout.num_q_tokens, layout.kv_pages)
        prob.metadata_step()
    prob.attention_step(save=True, spec_mode=spec_mode)
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    ref, ref_lse = oracle_full(layout, values)
    got = prob.out_np()
    max_abs, rel = errors(got, ref)
    tol_abs, tol_rel = TOL[spec.kv_dtype]
    print(f"[parity] {spec.name} L={list(layout.seq_lens)[:6]}: max_abs={max_abs:.2e} rel={rel:.2e}", flush=True)
    assert np.all(np.isfinite(got))
    assert max_abs <= tol_abs and rel <= tol_rel, (max_abs, rel)
    np.testing.assert_allclose(prob.lse_np(), ref_lse, rtol=0, atol=LSE_ATOL)
    return prob, layout, values


BASE_DEC = workloads.Spec("edge_decode", "decode", 1, 8, 2, 128, 16, "bf16", "bf16", seed=21)


@pytest.mark.parametrize("P", [1, 16, 64])
def test_decode_boundary_lengths(P):
    lens = [1, 2, P - 1 if P > 1 else 3, P, P + 1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 200]
    spec = BASE_DEC.replace(batch=len(lens), page_size=P)
    run_and_check(spec, seq_lens=lens)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 2), (32, 1), (64, 2)])
def test_decode_group_sizes(hq, hkv, kv):
    spec = BASE_DEC.replace(batch=5, num_q_heads=hq, num_kv_heads=hkv, kv_dtype=kv,
                            seq_len_kind="uniform", seq_len_args=(1, 300), seed=22)
    run_and_check(spec)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_decode_head_dim_64(kv):
    spec = BASE_DEC.replace(batch=6, head_dim=64, kv_dtype=kv, page_size=32,
                            seq_len_kind="uniform", seq_len_args=(1, 400), seed=23)
    run_and_check(spec)


def test_decode_single_long_request_is_split():
    """One request spread over many workgroups exercises the merge."""
    spec = BASE_DEC.replace(batch=1, num_q_heads=32, num_kv_heads=8, page_size=16, seed=24)
    run_and_check(spec, seq_lens=[20000])


def test_decode_peaked_softmax_and_shifted_values():
    """A large scale makes the softmax nearly one-hot; V ~ N(1, 1) keeps the
    output away from zero so max-abs is meaningful."""
    spec = BASE_DEC.replace(batch=4, scale=1.0, v_mean=1.0, seq_len_kind="uniform",
                            seq_len_args=(100, 3000), seed=25)
    run_and_check(spec)


def test_decode_zero_scale_is_mean_of_v():
    spec = BASE_DEC.replace(batch=3, scale=0.0, seq_len_kind="uniform", seq_len_args=(1, 500), seed=26)
    run_and_check(spec)


BASE_EXT = workloads.Spec("edge_extend", "extend", 3, 8, 2, 128, 128, "bf16", "bf16", seed=31,
                          new_len_args=(1, 200), prefix_len_args=(0, 300))


@pytest.mark.parametrize("P", [1, 16, 128])
def test_extend_page_sizes(P):
    run_and_check(BASE_EXT.replace(page_size=P))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("P", [2, 32, 256])
def test_other_page_sizes(P, kv):
    """Page sizes outside the workloads' (2, 32, 256): decode (pages smaller
    than, equal to and larger than a 32-token tile) and extend (pages
    smaller and larger than a 64-key tile)."""
    run_and_check(BASE_DEC.replace(batch=7, page_size=P, kv_dtype=kv, seq_len_kind="uniform",
                                   seq_len_args=(1, 900), seed=29))
    run_and_check(BASE_EXT.replace(page_size=P, kv_dtype=kv, seed=30))


def test_extend_ragged_new_and_prefix():
    lens_new = [1, 0, 33, 64, 65, 130, 7]
    prefix = [0, 5, 0, 63, 64, 1, 300]
    spec = BASE_EXT.replace(batch=len(lens_new), seed=32)
    run_and_check(spec, seq_lens=[p + n if p + n > 0 else 1 for p, n in zip(prefix, lens_new)],
                  extend_lens=[n if p + n > 0 else 0 for p, n in zip(prefix, lens_new)])


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (16, 2, 128), (48, 8, 128), (8, 2, 64), (64, 2, 128)])
def test_extend_group_sizes_and_dims(hq, hkv, d):
    spec = BASE_EXT.replace(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seed=33)
    run_and_check(spec)


def test_extend_fp32():
    spec = BASE_EXT.replace(q_dtype="f32", kv_dtype="f32", head_dim=64, page_size=4, seed=34)
    run_and_check(spec)


def test_extend_negative_scale():
    run_and_check(BASE_EXT.replace(scale=-0.05, seed=35))


# ------------------------------------------------------------- invariances

def _outputs(spec, seq_lens, extend_lens=None, pool_pages=None, seed_perm=None):
    layout = workloads.make_layout(spec.replace(seed=seed_perm) if seed_perm else spec,
                                   seq_lens=seq_lens, extend_lens=extend_lens, pool_pages=pool_pages)
    values = workloads.make_values(workloads.make_layout(spec, seq_lens=seq_lens,
                                                         extend_lens=extend_lens), device="cuda")
    prob = GpuProblem(layout, values)
    prob.attention_step(save=True)
    torch.cuda.synchronize()
    return prob.out.clone(), prob.lse.clone()


@pytest.mark.parametrize("mode", ["decode", "extend"])
def test_page_placement_is_bit_identical(mode):
    """Same logical data in different physical pages: identical bits (the work
    partition and every reduction order depend only on logical positions)."""
    if mode == "decode":
        spec, lens, ext = BASE_DEC.replace(batch=6, page_size=16), [5, 900, 33, 1, 2048, 17], None
    else:
        spec, lens, ext = BASE_EXT.replace(batch=3, page_size=16), [300, 90, 500], [200, 90, 64]
    a = _outputs(spec, lens, ext, pool_pages=400)
    b = _outputs(spec, lens, ext, pool_pages=400, seed_perm=777)
    c = _outputs(spec, lens, ext, pool_pages=900, seed_perm=778)
    for x in (b, c):
        assert torch.equal(a[0], x[0]) and torch.equal(a[1], x[1])


def test_runs_are_deterministic():
    spec = workloads.WORKLOADS["llama3_8b_decode"].replace(batch=12, seq_len_args=(1, 3000))
    layout = workloads.make_layout(spec)
    prob = GpuProblem(layout)
    outs = []
    for _ in range(3):
        prob.step()
        torch.cuda.synchronize()
        outs.append(prob.out.clone())
    assert all(torch.equal(outs[0], o) for o in outs[1:])


# ---------------------------------------------------------------- dispatch

def test_extend_with_one_new_token_matches_decode():
    spec = BASE_DEC.replace(batch=5, seq_len_kind="uniform", seq_len_args=(1, 700), seed=41)
    dec, layout, values = run_and_check(spec)
    ext = GpuProblem(layout, values)
    ext.mode = "extend"
    ext.md = pka.Batch(ext.ctx, "extend", layout.batch, layout.num_q_tokens, layout.kv_pages)
    ext.metadata_step()
    ext.attention_step(save=True)
    torch.cuda.synchronize()
    max_abs, rel = errors(ext.out_np(), dec.out_np())
    assert max_abs <= 1e-2 and rel <= 5e-3, (max_abs, rel)


@pytest.mark.parametrize("mode,spec_mode", [("target_verify", "prefill"), ("draft_extend", "prefill"),
                                            ("target_verify", "decode"), ("draft_extend", "decode")])
def test_speculative_modes_route_by_spec_mode(mode, spec_mode):
    if spec_mode == "decode":  # the decode path: one query token per request
        spec = BASE_EXT.replace(batch=4, new_len_args=(1, 1), prefix_len_args=(0, 400), seed=42)
    else:                      # the prefill (extend) path: a few chained draft tokens
        spec = BASE_EXT.replace(batch=4, new_len_args=(2, 8), prefix_len_args=(0, 400), seed=43)
    assert pka.select_path(mode, spec_mode) == ("decode" if spec_mode == "decode" else "extend")
    run_and_check(spec, mode=mode, spec_mode=spec_mode)


def test_idle_and_empty_batches_launch_nothing():
    spec = BASE_DEC.replace(batch=2, seq_len_kind="uniform", seq_len_args=(5, 50))
    layout = workloads.make_layout(spec)
    prob = GpuProblem(layout)
    prob.out.fill_(0.5)  # defined contents (torch.empty may hold NaN, which never compares equal)
    before = prob.out.clone()
    pka.forward(prob.ctx, "idle", prob.md, None, None, None, None, None, None)
    empty = pka.Batch(prob.ctx, "decode", 0, 0, 0)
    pka.forward(prob.ctx, "decode", empty, prob.values.q[:0], prob.k_new[:0], prob.v_new[:0],
                prob.k_pool, prob.v_pool, prob.out[:0])
    torch.cuda.synchronize()
    assert torch.equal(before, prob.out)


# ------------------------------------------------------------ device status

def test_out_of_range_page_ids_are_clamped_and_flagged():
    """Bad page ids never lead to an access outside the pool: the metadata
    kernel clamps them and raises a sticky flag."""
    spec = BASE_DEC.replace(batch=3, seq_len_kind="uniform", seq_len_args=(20, 60))
    layout = workloads.make_layout(spec)
    prob = GpuProblem(layout)
    bad = prob.page_table.clone()
    bad[1, 0] = layout.num_pages + 5
    bad[2, 1] = -3
    prob.md.init(prob.seq_lens, None, bad)
    prob.attention_step(save=True)
    flags = prob.md.status()
    assert flags & 2, flags  # PKA_DEV_BAD_PAGE


def test_lengths_beyond_the_page_table_are_flagged():
    spec = BASE_DEC.replace(batch=2, seq_len_kind="uniform", seq_len_args=(20, 40))
    layout = workloads.make_layout(spec)
    prob = GpuProblem(layout)
    lens = prob.seq_lens.clone()
    lens[0] = layout.page_table.shape[1] * spec.page_size + 100  # more pages than the row holds
    prob.md.init(lens, None, prob.page_table)
    prob.attention_step(save=False)
    assert prob.md.status() & 4  # PKA_DEV_TABLE_SHORT
