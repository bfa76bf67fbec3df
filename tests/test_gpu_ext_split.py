"""Extend path with a key-range split, through the C ABI.

A batch of few query rows per request (at most 16 on average: speculative
verify sent down the prefill path, short continuations) has one or two items
per request and KV head, so a long request's item would stream its keys
alone.  With a workspace of pka_batch_sizes' size the extend call cuts each
item's key range into chunks computed by workgroups of their own and merges
their partials (the forward_extend semantics of "[SGLang] Hybrid Attention"
are unchanged: every row attends causally to its prefix and to the new
tokens up to itself).  Outputs and lse are compared with the fp64 oracle
(bf16: max-abs 2e-2, rel-RMS 5e-3; fp8: 5e-2, 2e-2) and with the same batch
run unsplit (a workspace too small for the partials).
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


BASE = workloads.Spec("ext_split", "extend", 12, 32, 8, 128, 16, "bf16", "bf16", seed=301,
                      new_len_args=(1, 16), prefix_len_args=(0, 3000))


def _problem(spec, mode, seq_lens=None, extend_lens=None):
    layout = workloads.make_layout(spec, seq_lens=seq_lens, extend_lens=extend_lens)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values, prefix_only=True)
    prob.mode = mode
    prob.md = pka.Batch(prob.ctx, mode, layout.batch, layout.num_q_tokens, layout.kv_pages)
    prob.metadata_step()
    return prob, layout, values


def _check(prob, layout, values, name):
    d = prob.ctx.describe(prob.mode, layout.batch, layout.num_q_tokens)
    assert "chunks per item" in d, d  # the batch takes the split
    prob.attention_step(save=True, spec_mode="prefill")
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    ref, ref_lse = oracle_full(layout, values)
    got = prob.out_np()
    max_abs, rel = errors(got, ref)
    tol_abs, tol_rel = TOL[layout.spec.kv_dtype]
    print(f"[parity] {name}: n={list(layout.extend_lens)[:8]} L={list(layout.seq_lens)[:6]} "
          f"max_abs={max_abs:.2e} rel={rel:.2e}", flush=True)
    assert np.all(np.isfinite(got))
    assert max_abs <= tol_abs and rel <= tol_rel, (max_abs, rel)
    np.testing.assert_allclose(prob.lse_np(), ref_lse, rtol=0, atol=LSE_ATOL)


@pytest.mark.parametrize("name,spec,mode", [
    # ragged draft counts (0 .. 16), short and long prefixes: chunks without
    # a start tile stay empty
    ("verify_p16_g4", BASE, "target_verify"),
    ("draft_extend_p16_g4", BASE.replace(seed=302), "draft_extend"),
    # 16-head groups, page size 1
    ("verify_p1_g16", BASE.replace(batch=6, num_q_heads=64, num_kv_heads=4, page_size=1,
                                   new_len_args=(4, 4), seed=303), "target_verify"),
    # one page per key tile
    ("verify_p128", BASE.replace(batch=8, page_size=128, new_len_args=(8, 8), seed=304), "target_verify"),
    # fp8 cache
    ("verify_fp8_p64", BASE.replace(batch=8, page_size=64, kv_dtype="fp8", seed=305), "target_verify"),
    # 192-wide keys, 128-wide values
    ("verify_dk192_dv128", BASE.replace(batch=6, num_q_heads=16, num_kv_heads=16, head_dim=192,
                                        v_head_dim=128, page_size=128, seed=306), "target_verify"),
    # 64-wide heads
    ("verify_d64", BASE.replace(batch=8, num_q_heads=8, num_kv_heads=4, head_dim=64, page_size=32,
                                seed=307), "target_verify"),
    # a plain extend batch of short continuations
    ("extend_short_rows", BASE.replace(batch=10, page_size=32, new_len_args=(1, 20), seed=308), "extend"),
    # negative softmax scale
    ("verify_negative_scale", BASE.replace(batch=6, scale=-0.05, seed=309), "target_verify"),
    # 32 and 42 requests: four and three chunks per item
    ("verify_b32_c4", BASE.replace(batch=32, prefix_len_args=(0, 1500), seed=312), "target_verify"),
    ("verify_b42_c3", BASE.replace(batch=42, new_len_args=(1, 6), prefix_len_args=(0, 1200), seed=313),
     "target_verify"),
])
def test_split_extend_matches_oracle(name, spec, mode):
    prob, layout, values = _problem(spec, mode)
    _check(prob, layout, values, name)


def test_split_edges():
    """Prefixes of 0, 1, 63, 64, 65 and 4,000 tokens (a single start tile,
    starts on and around tile edges, many tiles per chunk), requests without
    rows and a request of 16 rows."""
    prefix = [0, 1, 63, 64, 65, 4000, 200, 0]
    lens_new = [3, 16, 1, 0, 5, 2, 0, 1]
    spec = BASE.replace(batch=len(prefix), seed=310)
    prob, layout, values = _problem(spec, "target_verify",
                                    seq_lens=[max(p + n, 1) for p, n in zip(prefix, lens_new)],
                                    extend_lens=lens_new)
    _check(prob, layout, values, "edges")


def test_split_and_unsplit_agree():
    """The same batch with and without the split: the same attention, up to
    rounding (the chunks' bf16 partial rows are merged in fp32)."""
    prob, layout, values = _problem(BASE.replace(seed=311), "target_verify")
    prob.attention_step(save=True, spec_mode="prefill")
    torch.cuda.synchronize()
    split = prob.out.float().clone()
    split_lse = prob.lse.clone()
    tiny = torch.empty(16, dtype=torch.uint8, device="cuda")  # too small for the partials: unsplit
    pka.attn_extend(prob.ctx, prob.md, values.q, prob.k_pool, prob.v_pool, prob.out, prob.lse,
                    workspace=tiny)
    torch.cuda.synchronize()
    whole = prob.out.float()
    max_abs, rel = errors(split.cpu().numpy().astype(np.float64), whole.cpu().numpy().astype(np.float64))
    assert max_abs <= 1e-2 and rel <= 5e-3, (max_abs, rel)
    assert float((split_lse - prob.lse).abs().max()) <= LSE_ATOL

