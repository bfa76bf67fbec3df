"""GPU parity: the HIP library, called through its C ABI, against the oracle.

Metadata and the cache write must be bit-exact; attention outputs must be
within max-abs 2e-2 / relative RMS 5e-3 (bf16 and fp32 caches) or 5e-2 / 2e-2
(fp8 caches) of the fp64 oracle, on the same seeded inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.oracle_ref import LSE_ATOL, TOL, errors, oracle_full, oracle_pools, oracle_requests, raw_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_attention_02_amd as pka
    from tests.gpu_problem import GpuProblem


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[case] {request.node.name}", flush=True)


def _small(name, **kw):
    return workloads.WORKLOADS[name].replace(**kw)


# Reduced shapes of the five workloads (same heads, dims, page sizes and
# dtypes; fewer/shorter requests) for element-by-element parity.
SMALL = {
    "tiny": (workloads.WORKLOADS["tiny_decode"], None),
    "llama_b9": (_small("llama3_8b_decode", batch=9, seq_len_args=(1, 700)), None),
    "qwen_b5_p1": (_small("qwen3_235b_decode", batch=5, seq_len_kind="uniform", seq_len_args=(1, 900)), None),
    "fp8_b6_p64": (_small("long_fp8_decode", batch=6, seq_len_args=(1, 1500)), None),
    "extend_b3": (_small("llama3_8b_extend", batch=3, new_len_args=(1, 300), prefix_len_args=(0, 500)), None),
}


def _check_close(name, gpu, ref, kv_dtype):
    max_abs, rel = errors(gpu, ref)
    tol_abs, tol_rel = TOL[kv_dtype]
    print(f"[parity] {name}: max_abs={max_abs:.3e} rel_rms={rel:.3e} (gates {tol_abs}, {tol_rel})",
          flush=True)
    assert np.all(np.isfinite(gpu)), "non-finite output"
    assert max_abs <= tol_abs and rel <= tol_rel, (max_abs, rel)


# ------------------------------------------------------------- metadata

@pytest.mark.parametrize("cfg", list(workloads.WORKLOADS))
def test_metadata_bit_exact(cfg):
    layout = workloads.make_layout(workloads.WORKLOADS[cfg])
    spec = layout.spec
    ctx = pka.Context(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                      layout.num_pages, spec.q_dtype, spec.kv_dtype, spec.softmax_scale,
                      1.0 if spec.kv_dtype != "fp8" else 0.01, 1.0 if spec.kv_dtype != "fp8" else 0.01)
    i32 = dict(dtype=torch.int32, device="cuda")
    ext = None if spec.mode == "decode" else torch.tensor(layout.extend_lens, **i32)
    md = pka.Batch(ctx, spec.mode, layout.batch, layout.num_q_tokens, layout.kv_pages)
    md.init(torch.tensor(layout.seq_lens, **i32), ext, torch.tensor(layout.page_table, **i32))
    assert md.status() == 0
    ref = oracle.metadata(layout.seq_lens, None if spec.mode == "decode" else layout.extend_lens,
                          layout.page_table, spec.page_size, layout.num_pages)
    got = {k: getattr(md, k).cpu().numpy() for k in ref}
    for k, v in ref.items():
        assert np.array_equal(got[k][:v.size], v), k


# ----------------------------------------------------------- cache write

@pytest.mark.parametrize("name", ["tiny", "llama_b9", "fp8_b6_p64", "extend_b3"])
def test_save_kv_bit_exact(name):
    spec, _ = SMALL[name]
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values)
    kp, vp = oracle_pools(layout, raw_np(values.k_all), raw_np(values.v_all), values.k_scale,
                          values.v_scale)
    gk, gv = raw_np(prob.k_pool), raw_np(prob.v_pool)
    # untouched slots keep their NaN sentinel on both sides: compare bytes
    assert gk.tobytes() == kp.tobytes()
    assert gv.tobytes() == vp.tobytes()


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -4, float(np.float32(5.3 / 448.0)), 0.0131, 3.7])
def test_fp8_quantiser_exhaustive(scale):
    """All 65,536 bf16 bit patterns through the library's cache write."""
    Hkv, D = 8, 128
    rows = 65536 // (Hkv * D)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).reshape(rows, Hkv, D).cuda()
    ctx = pka.Context(8, Hkv, D, 1, rows, "bf16", "fp8", 0.1, scale, scale)
    i32 = dict(dtype=torch.int32, device="cuda")
    md = pka.Batch(ctx, "extend", 1, rows, rows)
    md.init(torch.tensor([rows], **i32), torch.tensor([rows], **i32),
            torch.arange(rows, **i32)[None, :].contiguous())
    kp = torch.zeros((rows, Hkv, D), dtype=torch.uint8, device="cuda")
    vp = torch.zeros_like(kp)
    pka.save_kv(ctx, md, x, x, kp, vp)
    assert md.status() == 0
    expect = oracle.fp8_quantize(bits, scale)
    got = kp.cpu().numpy().reshape(-1)
    bad = np.nonzero(got != expect)[0]
    assert bad.size == 0, [(hex(int(bits[i])), hex(int(got[i])), hex(int(expect[i]))) for i in bad[:8]]
    assert np.array_equal(vp.cpu().numpy().reshape(-1), expect)


def test_fp8_decode_of_every_code_is_exact():
    """One cached token per request: the output is v_scale * V exactly, so the
    kernel's fp8 -> bf16 conversion is checked for every finite code."""
    Hkv, D, G = 1, 128, 2
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)  # 254 codes
    B = (codes.size + D - 1) // D
    vcodes = np.resize(codes, (B, Hkv, D)).astype(np.uint8)
    ctx = pka.Context(G * Hkv, Hkv, D, 1, B, "bf16", "fp8", 0.1, 1.0, 1.0)
    i32 = dict(dtype=torch.int32, device="cuda")
    md = pka.Batch(ctx, "decode", B, B, B)
    md.init(torch.ones(B, **i32), None, torch.arange(B, **i32)[:, None].contiguous())
    kp = torch.zeros((B, Hkv, D), dtype=torch.uint8, device="cuda")
    vp = torch.from_numpy(vcodes).cuda()
    q = torch.randn((B, G * Hkv, D), device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    pka.attn_decode(ctx, md, q, kp, vp, out)
    got = out.float().cpu().numpy()
    want = oracle.fp8_value(vcodes.reshape(-1)).reshape(B, Hkv, D)
    for h in range(G * Hkv):
        assert np.array_equal(got[:, h, :], want[:, h // G, :])


# ------------------------------------------------------------- attention

@pytest.mark.parametrize("name", list(SMALL))
def test_attention_parity_small(name):
    spec, _ = SMALL[name]
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values)
    prob.attention_step(save=True)
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    ref_out, ref_lse = oracle_full(layout, values)
    _check_close(name, prob.out_np(), ref_out, spec.kv_dtype)
    np.testing.assert_allclose(prob.lse_np(), ref_lse, rtol=0, atol=LSE_ATOL)


def test_attention_parity_llama_decode_full():
    spec = workloads.WORKLOADS["llama3_8b_decode"]
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values)
    prob.step()
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    ref_out, ref_lse = oracle_full(layout, values)
    _check_close("config2", prob.out_np(), ref_out, spec.kv_dtype)
    np.testing.assert_allclose(prob.lse_np(), ref_lse, rtol=0, atol=LSE_ATOL)


def _sampled(cfg, requests, heads=None, tokens=None, spec=None):
    spec = workloads.WORKLOADS[cfg] if spec is None else spec
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    prob = GpuProblem(layout, values)
    prob.step()
    torch.cuda.synchronize()
    assert prob.md.status() == 0
    out, lse = prob.out_np(), prob.lse_np()
    assert np.all(np.isfinite(out))
    L = layout.seq_lens
    reqs = sorted(set(requests(L)))
    ref = oracle_requests(layout, values, reqs, heads=heads, tokens=tokens)
    qo = np.concatenate([[0], np.cumsum(layout.extend_lens)])
    hs = list(range(spec.num_q_heads)) if heads is None else list(heads)
    g_all, r_all = [], []
    for b, (ts, ro, rl) in ref.items():
        rows = qo[b] + ts
        g_all.append(out[rows][:, hs, :])
        r_all.append(ro)
        np.testing.assert_allclose(lse[rows][:, hs], rl, rtol=0, atol=LSE_ATOL)
    what = f"all {len(reqs)} requests" if len(reqs) == layout.batch else f"requests {reqs}"
    _check_close(f"{spec.name} {what}", np.concatenate(g_all), np.concatenate(r_all), spec.kv_dtype)


def test_attention_parity_qwen_decode_full():
    """The Qwen3-235B-shaped batch at full size: every request, every head
    (the oracle takes each request on its own, ~1.4 M cached tokens)."""
    _sampled("qwen3_235b_decode", lambda L: range(len(L)))


def test_attention_parity_fp8_long_decode_full():
    """The long-context fp8 batch at full size: every request, every head."""
    _sampled("long_fp8_decode", lambda L: range(len(L)))


def test_attention_parity_extend_full():
    """The prefill batch at full size: every request, every head and every
    new token (13,360 tokens x 32 heads; ~670 GFLOP of fp64 oracle work, the
    oracle taking one request at a time on all host threads), so every
    (request, query tile, KV head) item and every XCD chunk of the grid is
    compared."""
    _sampled("llama3_8b_extend", lambda L: range(len(L)))
