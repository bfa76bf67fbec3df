"""The entry point that allocates nothing, through the C ABI.

pka_forward_with_metadata_noalloc takes pka_forward_with_metadata's
arguments minus the workspace: the decode path's split partials live in the
library's per-device scratch array.  Its outputs, metadata and cache writes
must equal those of pka_forward_with_metadata on the same inputs (the same
kernels and partition; only the partials' address differs), over two calls
in a row with a smaller batch second, for a decode batch (metadata built in
the decode launch), a verify batch on the decode path and an extend batch
(no scratch used).  A batch whose partials exceed the array is refused.
"""
import numpy as np
import pytest
import torch

import workloads
from tests.oracle_ref import TOL, errors, oracle_full

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_attention_02_amd as pka
    from tests.gpu_problem import GpuProblem, sentinel_pool_gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[case] {request.node.name}", flush=True)


MD_ARRAYS = ("kv_indptr", "kv_indices", "kv_last_page_len", "qo_indptr", "out_cache_loc")


def _problem(spec, mode, max_q=0):
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values, prefix_only=True)  # new tokens' slots hold the sentinel
    if max_q:
        # a verify caller's context: its draft-token count sizes the partial rows
        prob.ctx = pka.Context(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                               layout.num_pages, spec.q_dtype, spec.kv_dtype, spec.softmax_scale,
                               values.k_scale, values.v_scale, max_q_per_request=max_q)
    prob.mode = mode
    prob.md = pka.Batch(prob.ctx, mode, layout.batch, layout.num_q_tokens, layout.kv_pages)
    return prob, layout, values


def _run(prob, noalloc, spec_mode):
    """One step through either entry point, from sentinel new-token slots
    and zeroed metadata; returns everything the step writes."""
    for pool in (prob.k_pool, prob.v_pool):
        pool[prob.new_slots] = sentinel_pool_gpu((1,) + tuple(pool.shape[1:]), prob.spec.kv_dtype, pool.device)
    for name in MD_ARRAYS:
        getattr(prob.md, name).zero_()
    prob.out.fill_(float("nan"))
    prob.lse.fill_(float("nan"))
    ext = None if prob.mode == "decode" else prob.extend_lens
    args = (prob.ctx, prob.mode, prob.md, prob.seq_lens, ext, prob.page_table, prob.values.q,
            prob.k_new, prob.v_new, prob.k_pool, prob.v_pool, prob.out, prob.lse)
    if noalloc:
        pka.forward_with_metadata_noalloc(*args, save_kv_cache=True, spec_mode=spec_mode)
    else:
        pka.forward_with_metadata(*args, save_kv_cache=True, spec_mode=spec_mode)
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    return {"out": prob.out.clone(), "lse": prob.lse.clone(), "k_pool": prob.k_pool.clone(),
            "v_pool": prob.v_pool.clone(), **{n: getattr(prob.md, n).clone() for n in MD_ARRAYS}}


def _same(a, b):
    """Byte equality of every output (NaN sentinels included)."""
    for k in a:
        assert torch.equal(a[k].contiguous().view(torch.uint8), b[k].contiguous().view(torch.uint8)), k


LLAMA = workloads.WORKLOADS["llama3_8b_decode"]
CASES = {
    # metadata built in the decode launch, new tokens written by it
    "decode": (LLAMA.replace(batch=64, seq_len_args=(1, 3000), seed=201),
               LLAMA.replace(batch=23, seq_len_args=(1, 1200), seed=202), "decode", "prefill"),
    # fp8 cache, Qwen-shaped head groups
    "decode_fp8": (workloads.WORKLOADS["long_fp8_decode"].replace(batch=12, seq_len_args=(1, 9000), seed=203),
                   workloads.WORKLOADS["long_fp8_decode"].replace(batch=5, seq_len_args=(1, 4000), seed=204),
                   "decode", "prefill"),
    # several query rows per request on the decode path (metadata kernel first)
    "verify": (workloads.Spec("v", "extend", 48, 32, 8, 128, 16, "bf16", "bf16", seed=205,
                              new_len_args=(4, 4), prefix_len_args=(1, 2000)),
               workloads.Spec("v", "extend", 9, 32, 8, 128, 16, "bf16", "bf16", seed=206,
                              new_len_args=(1, 4), prefix_len_args=(1, 700)), "target_verify", "decode", 4),
    # extend path: no scratch is used
    "extend": (workloads.WORKLOADS["llama3_8b_extend"].replace(batch=3, new_len_args=(1, 300),
                                                              prefix_len_args=(0, 400), seed=207),
               workloads.WORKLOADS["llama3_8b_extend"].replace(batch=2, new_len_args=(1, 100),
                                                              prefix_len_args=(0, 200), seed=208),
               "extend", "prefill"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_workspace_entry_point(name):
    big, small, mode, spec_mode, *max_q = CASES[name]
    for spec in (big, small):  # two calls in a row, the second on a smaller batch
        prob, layout, values = _problem(spec, mode, *max_q)
        want = _run(prob, noalloc=False, spec_mode=spec_mode)
        got = _run(prob, noalloc=True, spec_mode=spec_mode)
        _same(want, got)
        ref, _ = oracle_full(layout, values)
        max_abs, rel = errors(got["out"].float().cpu().numpy(), ref)
        tol_abs, tol_rel = TOL[spec.kv_dtype]
        print(f"[noalloc] {name} B={layout.batch}: identical to the workspace call; "
              f"max_abs={max_abs:.2e} rel={rel:.2e}", flush=True)
        assert max_abs <= tol_abs and rel <= tol_rel
        del prob
    torch.cuda.empty_cache()


def test_noalloc_refuses_batches_beyond_the_scratch():
    """16 query rows per request of 96 requests over 32-head groups need more
    partial rows than the array holds (the requests' own slots alone take
    96 x 16 x 128 bf16 rows and lse, 51 MB, and every share adds 16 x 128):
    refused, nothing launched (outputs untouched)."""
    spec = workloads.Spec("v", "extend", 96, 128, 4, 128, 16, "bf16", "bf16", seed=209,
                          new_len_args=(16, 16), prefix_len_args=(600, 1200))
    prob, layout, values = _problem(spec, "target_verify")
    need = prob.ctx.sizes("target_verify", layout.batch, layout.num_q_tokens, layout.kv_pages).workspace_bytes
    assert need > pka.NOALLOC_SCRATCH_BYTES
    prob.out.fill_(3.0)
    with pytest.raises(pka.PkaError) as e:
        pka.forward_with_metadata_noalloc(prob.ctx, "target_verify", prob.md, prob.seq_lens, prob.extend_lens,
                                          prob.page_table, prob.values.q, prob.k_new, prob.v_new, prob.k_pool,
                                          prob.v_pool, prob.out, prob.lse, spec_mode="decode")
    assert e.value.status == -3 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((prob.out == 3.0).all())
