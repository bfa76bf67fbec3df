"""Capture one step (metadata + forward with the cache write) in a HIP graph
and replay it, through the C ABI.

Nothing on the path allocates, synchronises or records a memset, so the whole
step can be captured once and replayed while the caller updates the inputs in
place (new queries, decode lengths that grow by one token).  Every replay is
compared bit for bit with the same step run eagerly on the same inputs, with
eager work and synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

import workloads
from tests.oracle_ref import LSE_ATOL, TOL, errors, oracle_full, oracle_requests

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests.gpu_problem import GpuProblem


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _capture(prob):
    # warm up eagerly on a side stream (first-call host work happens here)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prob.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        prob.step()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name,spec", [
    ("decode_bf16_p16", workloads.WORKLOADS["llama3_8b_decode"].replace(batch=9, seq_len_args=(40, 900), seed=71)),
    ("decode_fp8_p64", workloads.WORKLOADS["long_fp8_decode"].replace(batch=5, seq_len_args=(100, 3000), seed=72)),
    ("extend_bf16_p128", workloads.WORKLOADS["llama3_8b_extend"].replace(batch=3, new_len_args=(1, 150),
                                                      prefix_len_args=(0, 300), seed=73)),
])
def test_graph_replays_match_eager(name, spec):
    layout = workloads.make_layout(spec)
    prob = GpuProblem(layout)
    g = _capture(prob)
    gen = torch.Generator(device="cuda").manual_seed(5)
    grow = None
    if spec.mode == "decode":
        # requests whose last page has room for two more tokens (the page
        # table holds no page beyond the last one in use)
        P = spec.page_size
        grow = torch.tensor([1 <= int(L) % P <= P - 2 for L in layout.seq_lens], device="cuda")
        assert bool(grow.any())
    for r in range(3):
        # eager work between replays: new queries, longer decode contexts
        q_new = torch.randn(prob.values.q.shape, generator=gen, device="cuda").to(prob.values.q.dtype)
        prob.values.q.copy_(q_new)
        if grow is not None and r > 0:
            prob.seq_lens += grow.to(torch.int32)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got, got_lse = prob.out.clone(), prob.lse.clone()
        assert prob.md.status() == 0
        prob.step()  # the same step, eagerly, on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(got, prob.out), f"replay {r} differs from the eager step"
        assert torch.equal(got_lse, prob.lse)
        print(f"[graph] {name} replay {r}: bit-identical to eager", flush=True)


def test_graph_replay_matches_oracle():
    """The replayed step is also right: one replay checked against the oracle."""
    spec = workloads.WORKLOADS["llama3_8b_decode"].replace(batch=6, seq_len_args=(10, 700), seed=74)
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values)
    g = _capture(prob)
    prob.out.zero_()
    g.replay()
    torch.cuda.synchronize()
    ref, ref_lse = oracle_full(layout, values)
    max_abs, rel = errors(prob.out_np(), ref)
    print(f"[parity] graph replay: max_abs={max_abs:.2e} rel={rel:.2e}", flush=True)
    assert max_abs <= TOL["bf16"][0] and rel <= TOL["bf16"][1]
    np.testing.assert_allclose(prob.lse_np(), ref_lse, rtol=0, atol=LSE_ATOL)


def _capture_fused(prob, noalloc=False):
    """Capture the one-call step (forward_with_metadata with the cache write)."""
    import paged_kv_attention_02_amd as pka

    def step():
        if noalloc:
            pka.forward_with_metadata_noalloc(prob.ctx, prob.mode, prob.md, prob.seq_lens, None,
                                              prob.page_table, prob.values.q, prob.k_new, prob.v_new,
                                              prob.k_pool, prob.v_pool, prob.out, prob.lse)
        else:
            prob.fused_step()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g, step


@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_replay_with_fewer_live_requests(noalloc):
    """A step captured for 64 requests replayed with 64, 33 and 17 live ones.
    Padding convention: a padded request has seq_len 1 and its page-table row
    points at one reserved page no live request uses (the reserved page takes
    the padded rows' cache writes; their outputs are unspecified).  Each
    replay's live rows equal the same padded step run eagerly bit for bit, and
    the oracle within the gates."""
    spec = workloads.WORKLOADS["llama3_8b_decode"].replace(batch=64, seq_len_args=(30, 1500), seed=75)
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values)
    g, step = _capture_fused(prob, noalloc)
    reserved = int(layout.page_table[63, 0])  # a page of a request that is padding below
    full_lens, full_table = prob.seq_lens.clone(), prob.page_table.clone()
    for live in (64, 33, 17):
        prob.seq_lens.copy_(full_lens)
        prob.page_table.copy_(full_table)
        if live < 64:
            prob.seq_lens[live:] = 1
            prob.page_table[live:, 0] = reserved
        prob.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert prob.md.status() == 0
        got, got_lse = prob.out[:live].clone(), prob.lse[:live].clone()
        prob.out.fill_(float("nan"))
        step()  # the same padded step, eagerly
        torch.cuda.synchronize()
        assert torch.equal(got, prob.out[:live]) and torch.equal(got_lse, prob.lse[:live]), live
        ref = oracle_requests(layout, values, list(range(live)))
        ref_out = np.concatenate([ref[b][1] for b in range(live)])
        ref_lse = np.concatenate([ref[b][2] for b in range(live)])
        out = got.float().cpu().numpy().astype(np.float64)
        max_abs, rel = errors(out, ref_out)
        print(f"[graph] 64-request graph, {live} live: bit-identical to eager; max_abs={max_abs:.2e} "
              f"rel={rel:.2e}", flush=True)
        assert max_abs <= TOL["bf16"][0] and rel <= TOL["bf16"][1]
        np.testing.assert_allclose(got_lse.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)
