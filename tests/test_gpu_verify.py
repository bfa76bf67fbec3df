"""Speculative verify on the decode path, through the C ABI.

A TARGET_VERIFY / DRAFT_EXTEND batch with the decode speculative-attention
mode goes to the decode path ("[SGLang] Hybrid Attention", section on
_select_backend) carrying n_b query tokens per request; token i sees the
cache up to position L_b - n_b + i.  Outputs are compared with the fp64
oracle's extend semantics (bf16 / fp32: max-abs 2e-2, rel-RMS 5e-3; fp8:
5e-2, 2e-2), and with the extend path on the same batch.
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


def _verify_problem(spec, mode="target_verify", seq_lens=None, extend_lens=None):
    layout = workloads.make_layout(spec, seq_lens=seq_lens, extend_lens=extend_lens)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values, prefix_only=True)
    prob.mode = mode
    prob.md = pka.Batch(prob.ctx, mode, layout.batch, layout.num_q_tokens, layout.kv_pages)
    prob.metadata_step()
    return prob, layout, values


def _check(prob, layout, values, name):
    prob.attention_step(save=True, spec_mode="decode")
    torch.cuda.synchronize()
    status = prob.md.status()
    ref, ref_lse = oracle_full(layout, values)
    got = prob.out_np()
    max_abs, rel = errors(got, ref)
    tol_abs, tol_rel = TOL[layout.spec.kv_dtype]
    print(f"[parity] {name}: n={list(layout.extend_lens)[:8]} max_abs={max_abs:.2e} rel={rel:.2e}", flush=True)
    assert status == 0, status
    assert np.all(np.isfinite(got))
    assert max_abs <= tol_abs and rel <= tol_rel, (max_abs, rel)
    np.testing.assert_allclose(prob.lse_np(), ref_lse, rtol=0, atol=LSE_ATOL)


BASE = workloads.Spec("verify", "extend", 6, 32, 8, 128, 16, "bf16", "bf16", seed=81,
                      new_len_args=(2, 8), prefix_len_args=(1, 900))


@pytest.mark.parametrize("name,spec", [
    ("bf16_p16_g4", BASE),
    ("bf16_p1_g16", BASE.replace(num_q_heads=64, num_kv_heads=4, page_size=1, seed=82)),
    ("fp8_p64_g8", BASE.replace(num_q_heads=64, num_kv_heads=8, page_size=64, kv_dtype="fp8", seed=83)),
    ("bf16_d64_g2", BASE.replace(num_q_heads=8, num_kv_heads=4, head_dim=64, page_size=32, seed=84)),
    ("f32_p1_g2", BASE.replace(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=1, q_dtype="f32",
                               kv_dtype="f32", seed=85)),
])
@pytest.mark.parametrize("mode", ["target_verify", "draft_extend"])
def test_verify_on_decode_path(name, spec, mode):
    prob, layout, values = _verify_problem(spec, mode)
    _check(prob, layout, values, f"{name}/{mode}")


@pytest.mark.parametrize("name,spec", [
    # 4 tokens x 4 heads = 16 columns: one 16-column block per wave
    ("llama_n4_g4", BASE.replace(batch=64, new_len_args=(4, 4), prefix_len_args=(0, 600), seed=90)),
    # 8 tokens x 4 heads = 32 columns: both blocks of one wave
    ("llama_n8_g4", BASE.replace(batch=64, new_len_args=(8, 8), prefix_len_args=(0, 600), seed=91)),
    # 4 tokens x 16 heads = 64 columns: two waves of two blocks per KV head, fp8 cache
    ("fp8_n4_g16", BASE.replace(batch=9, num_q_heads=64, num_kv_heads=4, page_size=64, kv_dtype="fp8",
                                new_len_args=(4, 4), prefix_len_args=(0, 2000), seed=92)),
    # 8 tokens x 8 heads = 64 columns: two waves of two blocks per KV head, bf16 cache
    ("bf16_n8_g8", BASE.replace(batch=12, num_q_heads=64, num_kv_heads=8, page_size=16,
                                new_len_args=(8, 8), prefix_len_args=(0, 1500), seed=93)),
    # 16 tokens x 16 heads = 256 columns: four waves per KV head, each taking
    # two 32-column passes over its tiles
    ("bf16_n16_g16", BASE.replace(batch=5, num_q_heads=32, num_kv_heads=2, page_size=1,
                                  new_len_args=(16, 16), prefix_len_args=(0, 1200), seed=94)),
    # 64-wide heads, 8 tokens x 4 heads = 32 columns
    ("bf16_d64_n8_g4", BASE.replace(batch=10, num_q_heads=16, num_kv_heads=4, head_dim=64, page_size=32,
                                    new_len_args=(8, 8), prefix_len_args=(0, 900), seed=95)),
])
def test_verify_column_passes_in_parallel_waves(name, spec):
    """Uniform draft lengths whose columns need one or several 16-column
    blocks: a wave takes up to two adjacent blocks over one tile stream, and
    further passes go to parallel waves of one workgroup."""
    prob, layout, values = _verify_problem(spec)
    _check(prob, layout, values, name)


def test_verify_long_requests_are_split_and_merged():
    """Long contexts spread over many workgroups: every query token's rows
    come from partials, including pieces where some tokens see no key."""
    spec = BASE.replace(batch=3, seed=86)
    prob, layout, values = _verify_problem(spec, seq_lens=[30000, 12000, 4100],
                                           extend_lens=[8, 3, 16])
    _check(prob, layout, values, "long_split")


def test_verify_ragged_token_counts():
    """n_b from 0 to 16 in one batch, lengths around tile and page edges."""
    lens_new = [0, 1, 2, 5, 16, 7, 1, 12]
    prefix = [40, 0, 31, 33, 64, 500, 2, 95]
    spec = BASE.replace(batch=len(lens_new), seed=87)
    prob, layout, values = _verify_problem(spec, seq_lens=[p + n if p + n > 0 else 1 for p, n in zip(prefix, lens_new)],
                                           extend_lens=lens_new)
    _check(prob, layout, values, "ragged")


def test_verify_matches_the_extend_path():
    spec = BASE.replace(batch=5, seed=88)
    prob, layout, values = _verify_problem(spec)
    prob.attention_step(save=True, spec_mode="decode")
    torch.cuda.synchronize()
    dec = prob.out.clone()
    prob.attention_step(save=False, spec_mode="prefill")
    torch.cuda.synchronize()
    max_abs, rel = errors(dec.float().cpu().numpy().astype(np.float64), prob.out_np())
    assert max_abs <= 1e-2 and rel <= 5e-3, (max_abs, rel)


def test_more_than_16_tokens_is_flagged():
    spec = BASE.replace(batch=2, seed=89)
    prob, layout, values = _verify_problem(spec, seq_lens=[300, 100], extend_lens=[20, 3])
    prob.out.fill_(0.0)
    prob.attention_step(save=True, spec_mode="decode")
    torch.cuda.synchronize()
    assert prob.md.status() & 1  # PKA_DEV_BAD_LENGTH
    ref, _ = oracle_full(layout, values)
    got = prob.out_np()
    # the first 16 rows of request 0 and all rows of request 1 are computed
    rows = list(range(16)) + [20, 21, 22]
    max_abs, rel = errors(got[rows], ref[rows])
    assert max_abs <= 2e-2 and rel <= 5e-3, (max_abs, rel)
    assert np.all(got[16:20] == 0)


def test_verify_rows_sized_by_max_q_per_request():
    """A context built for 4 draft tokens per request sizes the decode
    partials for 4 rows (a quarter of the 16-row default) and computes the
    same batch within the gates; a batch with more rows on average than that
    is refused before any launch."""
    spec = BASE.replace(batch=24, new_len_args=(1, 4), prefix_len_args=(1, 1500), seed=96)
    prob, layout, values = _verify_problem(spec)
    ctx4 = pka.Context(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                       layout.num_pages, spec.q_dtype, spec.kv_dtype, spec.softmax_scale,
                       max_q_per_request=4)
    full = prob.ctx.sizes("target_verify", layout.batch, layout.num_q_tokens, layout.kv_pages)
    four = ctx4.sizes("target_verify", layout.batch, layout.num_q_tokens, layout.kv_pages)
    assert four.workspace_bytes * 4 == full.workspace_bytes
    prob.ctx = ctx4
    prob.md = pka.Batch(ctx4, "target_verify", layout.batch, layout.num_q_tokens, layout.kv_pages)
    prob.metadata_step()
    _check(prob, layout, values, "max_q_per_request=4")
    many = BASE.replace(batch=8, new_len_args=(5, 6), prefix_len_args=(1, 300), seed=97)
    prob5, layout5, _ = _verify_problem(many)
    prob5.ctx = pka.Context(many.num_q_heads, many.num_kv_heads, many.head_dim, many.page_size,
                            layout5.num_pages, many.q_dtype, many.kv_dtype, many.softmax_scale,
                            max_q_per_request=4)
    prob5.md = pka.Batch(prob5.ctx, "target_verify", layout5.batch, layout5.num_q_tokens, layout5.kv_pages)
    with pytest.raises(pka.PkaError) as e:
        prob5.attention_step(save=False, spec_mode="decode")
    assert e.value.status == -2
