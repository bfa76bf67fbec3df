"""Pins of the CPU oracle against facts fixed by mathematics or the pages.

Each test ties the oracle to something other than itself: closed forms
(one token, identical keys), invariances (page placement, page size, shift of
K, linearity in V), an independent pure-Python brute force, and a library
special case (torch's CPU scaled-dot-product attention in fp64).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import brute

RNG = np.random.default_rng(12345)


def storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact storage of values that are representable in the dtype."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), x), "value not exact in fp32"
    if dtype == "f32":
        return np.ascontiguousarray(f)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return np.ascontiguousarray((u >> 16).astype(np.uint16))


def grid_values(shape, step=2.0 ** -6, span=64, rng=RNG):
    """Random multiples of a power of two: exact in bf16 and fp32."""
    return rng.integers(-span, span + 1, size=shape).astype(np.float64) * step


def place(seq_lens, P, pool_pages=None, rng=RNG, shuffle=True):
    pages = [(L + P - 1) // P for L in seq_lens]
    need = sum(pages)
    pool_pages = pool_pages or need + 3
    perm = rng.permutation(pool_pages)[:need] if shuffle else np.arange(need)
    table = np.full((len(seq_lens), max(pages)), -1, dtype=np.int32)
    off = 0
    for b, k in enumerate(pages):
        table[b, :k] = perm[off:off + k]
        off += k
    return table, pool_pages


def build_pools(seq_lens, table, P, pool_pages, k_all, v_all, src, kv, ks=1.0, vs=1.0):
    """Oracle cache write of every token; unused slots hold NaN."""
    Hkv, Dk, Dv = k_all.shape[1], k_all.shape[2], v_all.shape[2]
    md = oracle.metadata(seq_lens, seq_lens, table, P, pool_pages)
    nanbits = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}[kv]
    dt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[kv]
    kp = np.full((pool_pages * P, Hkv, Dk), nanbits, dtype=dt)
    vp = np.full((pool_pages * P, Hkv, Dv), nanbits, dtype=dt)
    oracle.save_kv(md["out_cache_loc"], k_all, v_all, src, kv, kp, vp, ks, vs)
    return kp, vp


def run(seq_lens, ext, P, q, k_all, v_all, dtype="f32", kv=None, scale=0.125, shuffle=True,
        ks=1.0, vs=1.0, table=None, pool_pages=None, rng=RNG):
    kv = kv or dtype
    if table is None:
        table, pool_pages = place(seq_lens, P, rng=rng, shuffle=shuffle)
    kp, vp = build_pools(seq_lens, table, P, pool_pages, k_all, v_all, dtype, kv, ks, vs)
    return oracle.attention(seq_lens, ext, table, P, pool_pages, q, dtype, kp, vp, kv, scale,
                            ks, vs)


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("dv", [16, 8, 24])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_cached_token_returns_v(dtype, dv):
    D, Hq, Hkv = 16, 4, 2  # key width D; value width dv (may differ)
    q = storage(grid_values((1, Hq, D)), dtype)
    k = storage(grid_values((1, Hkv, D)), dtype)
    v = storage(grid_values((1, Hkv, dv)), dtype)
    out, lse = run([1], None, 1, q, k, v, dtype)
    vv = (v.astype(np.float64) if dtype == "f32" else oracle.bf16_value(v))
    qq = (q.astype(np.float64) if dtype == "f32" else oracle.bf16_value(q))
    kk = (k.astype(np.float64) if dtype == "f32" else oracle.bf16_value(k))
    for h in range(Hq):
        g = h // (Hq // Hkv)
        assert np.array_equal(out[0, h], vv[0, g])
        s0 = 0.125 * sum(qq[0, h, d] * kk[0, g, d] for d in range(D))
        assert lse[0, h] == pytest.approx(s0, abs=1e-15)


@pytest.mark.parametrize("dv", [32, 12])
@pytest.mark.parametrize("scale", [0.125, 0.0])
def test_identical_keys_give_mean_of_v(scale, dv):
    L, D, Hq, Hkv = 57, 32, 2, 1
    q = storage(grid_values((1, Hq, D)), "f32")
    k1 = grid_values((1, Hkv, D))
    k = storage(np.repeat(k1, L, axis=0), "f32")
    v = storage(grid_values((L, Hkv, dv)), "f32")
    out, lse = run([L], None, 4, q, k, v, "f32", scale=scale)
    mean_v = v.astype(np.float64).mean(axis=0)[0]
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], mean_v, rtol=0, atol=1e-14)
        s = scale * float(np.dot(q[0, h].astype(np.float64), k1[0, 0]))
        assert lse[0, h] == pytest.approx(s + math.log(L), abs=1e-12)


# -------------------------------------------------------------- invariances

def _random_problem(seq_lens, ext, Hq=4, Hkv=2, D=32, dtype="bf16", rng=RNG):
    N = len(seq_lens) if ext is None else int(sum(ext))
    T = int(sum(seq_lens))
    q = storage(grid_values((N, Hq, D), rng=rng), dtype)
    k = storage(grid_values((T, Hkv, D), rng=rng), dtype)
    v = storage(grid_values((T, Hkv, D), rng=rng), dtype)
    return q, k, v


def test_page_placement_permutation_is_bit_identical():
    seq_lens, ext = [29, 64, 3], [5, 64, 1]
    q, k, v = _random_problem(seq_lens, ext)
    rng = np.random.default_rng(7)
    a = run(seq_lens, ext, 8, q, k, v, "bf16", shuffle=False)
    b = run(seq_lens, ext, 8, q, k, v, "bf16", shuffle=True, rng=rng)
    c = run(seq_lens, ext, 8, q, k, v, "bf16", shuffle=True, rng=rng)
    for x in (b, c):
        assert np.array_equal(a[0], x[0]) and np.array_equal(a[1], x[1])


def test_page_size_is_bit_identical():
    seq_lens = [1, 16, 17, 129, 300]
    q, k, v = _random_problem(seq_lens, None)
    ref = run(seq_lens, None, 1, q, k, v, "bf16")
    for P in (16, 128):
        x = run(seq_lens, None, P, q, k, v, "bf16")
        assert np.array_equal(ref[0], x[0]) and np.array_equal(ref[1], x[1])


def test_shift_of_keys_leaves_output_unchanged():
    L, D, Hq, Hkv = 40, 16, 3, 1
    q = storage(grid_values((1, Hq, D)), "f32")
    k = grid_values((L, Hkv, D))
    u = grid_values((1, Hkv, D), step=2.0 ** -3)
    v = storage(grid_values((L, Hkv, D)), "f32")
    a, la = run([L], None, 1, q, storage(k, "f32"), v, "f32")
    b, lb = run([L], None, 1, q, storage(k + u, "f32"), v, "f32")
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    shift = 0.125 * (q[0].astype(np.float64) @ u[0, 0])
    np.testing.assert_allclose(lb[0] - la[0], shift, atol=1e-12)


def test_linearity_in_v():
    seq_lens, ext = [33, 10], [4, 10]
    q, k, v1 = _random_problem(seq_lens, ext, dtype="f32")
    v2 = storage(grid_values(v1.shape), "f32")
    comb = storage(3.0 * v1.astype(np.float64) - 2.0 * v2.astype(np.float64), "f32")
    table, pp = place(seq_lens, 4)
    o1 = run(seq_lens, ext, 4, q, k, v1, "f32", table=table, pool_pages=pp)[0]
    o2 = run(seq_lens, ext, 4, q, k, v2, "f32", table=table, pool_pages=pp)[0]
    o3 = run(seq_lens, ext, 4, q, k, comb, "f32", table=table, pool_pages=pp)[0]
    np.testing.assert_allclose(o3, 3.0 * o1 - 2.0 * o2, rtol=0, atol=1e-12)


def test_extend_with_one_new_token_equals_decode():
    seq_lens = [7, 33, 100]
    q, k, v = _random_problem(seq_lens, None)
    table, pp = place(seq_lens, 4)
    dec = run(seq_lens, None, 4, q, k, v, "bf16", table=table, pool_pages=pp)
    ext = run(seq_lens, [1, 1, 1], 4, q, k, v, "bf16", table=table, pool_pages=pp)
    assert np.array_equal(dec[0], ext[0]) and np.array_equal(dec[1], ext[1])


def test_extend_first_row_without_prefix_returns_v0():
    seq_lens, ext = [12, 5], [12, 5]
    q, k, v = _random_problem(seq_lens, ext)
    out, _ = run(seq_lens, ext, 4, q, k, v, "bf16")
    vv = oracle.bf16_value(v)
    G = 2
    for h in range(4):
        assert np.array_equal(out[0, h], vv[0, h // G])  # request 0, token 0
        assert np.array_equal(out[12, h], vv[12, h // G])  # request 1, token 0


def test_extend_is_causal_bottom_right():
    """Changing a key after a query's position cannot change that query."""
    seq_lens, ext = [20], [6]  # prefix 14, queries at positions 14..19
    q, k, v = _random_problem(seq_lens, ext, dtype="f32")
    table, pp = place(seq_lens, 4)
    a = run(seq_lens, ext, 4, q, k, v, "f32", table=table, pool_pages=pp)[0]
    k2, v2 = k.copy(), v.copy()
    k2[17:] += 1.0
    v2[17:] -= 2.0
    b = run(seq_lens, ext, 4, q, k2, v2, "f32", table=table, pool_pages=pp)[0]
    assert np.array_equal(a[:3], b[:3])  # positions 14, 15, 16
    assert not np.array_equal(a[3:], b[3:])


def test_gqa_mapping_matches_replicated_heads():
    """Head h of a GQA batch equals head h of an MHA batch whose KV head h is
    a copy of GQA KV head h // G (contiguous groups)."""
    seq_lens, ext = [25, 9], [3, 9]
    Hq, Hkv, D = 8, 2, 16
    G = Hq // Hkv
    q, k, v = _random_problem(seq_lens, ext, Hq=Hq, Hkv=Hkv, D=D)
    table, pp = place(seq_lens, 4)
    a = run(seq_lens, ext, 4, q, k, v, "bf16", table=table, pool_pages=pp)
    k_rep = np.ascontiguousarray(np.repeat(k, G, axis=1))
    v_rep = np.ascontiguousarray(np.repeat(v, G, axis=1))
    b = run(seq_lens, ext, 4, q, k_rep, v_rep, "bf16", table=table, pool_pages=pp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------- brute force

CASES = [
    dict(seq_lens=[5, 12], ext=None, P=1, Hq=4, Hkv=2, D=8, dtype="f32", kv="f32"),
    dict(seq_lens=[3, 9, 17], ext=None, P=4, Hq=4, Hkv=1, D=8, dtype="bf16", kv="bf16"),
    dict(seq_lens=[11, 6], ext=[4, 6], P=2, Hq=2, Hkv=2, D=8, dtype="bf16", kv="bf16"),
    dict(seq_lens=[9, 14], ext=None, P=4, Hq=4, Hkv=2, D=8, dtype="bf16", kv="fp8"),
    dict(seq_lens=[10], ext=[3], P=8, Hq=6, Hkv=3, D=4, dtype="bf16", kv="fp8"),
    # value width different from the key width
    dict(seq_lens=[7, 13], ext=[2, 5], P=4, Hq=4, Hkv=2, D=12, DV=8, dtype="bf16", kv="bf16"),
    dict(seq_lens=[6, 9], ext=None, P=2, Hq=2, Hkv=1, D=6, DV=10, dtype="f32", kv="f32"),
    dict(seq_lens=[11], ext=[4], P=4, Hq=4, Hkv=2, D=8, DV=4, dtype="bf16", kv="fp8"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_brute_force_agrees(case):
    rng = np.random.default_rng(99)
    seq_lens, ext, P = case["seq_lens"], case["ext"], case["P"]
    N = len(seq_lens) if ext is None else sum(ext)
    T = sum(seq_lens)
    dt = case["dtype"]
    q = storage(rng.standard_normal((N, case["Hq"], case["D"])).astype(np.float32)
                .astype(np.float64) if dt == "f32" else grid_values((N, case["Hq"], case["D"]), rng=rng), dt)
    k = storage(grid_values((T, case["Hkv"], case["D"]), rng=rng), dt)
    v = storage(grid_values((T, case["Hkv"], case.get("DV", case["D"])), rng=rng), dt)
    ks = vs = 1.0
    if case["kv"] == "fp8":
        ks, vs = 0.0078125 * 1.3, 0.0078125 * 0.7
    table, pp = place(seq_lens, P, rng=rng)
    kp, vp = build_pools(seq_lens, table, P, pp, k, v, dt, case["kv"], ks, vs)
    out, lse = oracle.attention(seq_lens, ext, table, P, pp, q, dt, kp, vp, case["kv"], 0.3, ks, vs)
    bo, bl = brute.attention(seq_lens, ext, table, P, q, dt, kp, vp, case["kv"], 0.3, ks, vs)
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-12)


# ------------------------------------------------------- library special case

def _sdpa_reference(q, k, v, mask, scale):
    import torch
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=None if mask is None else torch.from_numpy(mask), scale=scale).numpy()


@pytest.mark.parametrize("dv", [16, 24])
def test_torch_sdpa_decode_and_extend_fp64(dv):
    """P = 1 with contiguous slots and K/V heads repeated per group is torch's
    dense SDPA: no mask for decode, an explicit bottom-right mask for extend.
    SDPA takes a value width different from the key width as well."""
    rng = np.random.default_rng(5)
    Hq, Hkv, D, G = 4, 2, 16, 2
    for mode in ("decode", "extend"):
        L, n = 23, (1 if mode == "decode" else 7)
        q = storage(rng.standard_normal((n, Hq, D)).astype(np.float32).astype(np.float64), "f32")
        k = storage(rng.standard_normal((L, Hkv, D)).astype(np.float32).astype(np.float64), "f32")
        v = storage(rng.standard_normal((L, Hkv, dv)).astype(np.float32).astype(np.float64), "f32")
        table = np.arange(L, dtype=np.int32)[None, :]
        ext = None if mode == "decode" else [n]
        out, _ = run([L], ext, 1, q, k, v, "f32", scale=0.25, table=table, pool_pages=L)
        qq = q.astype(np.float64).transpose(1, 0, 2)[None]  # [1, Hq, n, D]
        kk = np.repeat(k.astype(np.float64), G, axis=1).transpose(1, 0, 2)[None]
        vv = np.repeat(v.astype(np.float64), G, axis=1).transpose(1, 0, 2)[None]
        mask = None
        if mode == "extend":
            pos = (L - n) + np.arange(n)[:, None]
            mask = np.arange(L)[None, :] <= pos  # bottom-right causal
        ref = _sdpa_reference(np.ascontiguousarray(qq), np.ascontiguousarray(kk),
                              np.ascontiguousarray(vv), mask, 0.25)[0].transpose(1, 0, 2)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------- metadata

def test_metadata_invariants_and_slots():
    rng = np.random.default_rng(3)
    for P in (1, 2, 16, 64):
        seq_lens = rng.integers(1, 300, size=9).astype(np.int32)
        ext = np.minimum(seq_lens, rng.integers(0, 40, size=9)).astype(np.int32)
        table, pp = place(seq_lens.tolist(), P, rng=rng)
        md = oracle.metadata(seq_lens, ext, table, P, pp)
        ip = md["kv_indptr"]
        assert ip[0] == 0 and np.all(np.diff(ip) >= 1)
        assert ip[-1] == sum((int(L) + P - 1) // P for L in seq_lens)
        lpl = md["kv_last_page_len"]
        assert np.all((lpl >= 1) & (lpl <= P))
        # tokens covered by the pages equal the sequence length
        assert np.array_equal((np.diff(ip) - 1) * P + lpl, seq_lens)
        assert np.all((md["kv_indices"] >= 0) & (md["kv_indices"] < pp))
        qo = md["qo_indptr"]
        assert qo[0] == 0 and np.array_equal(np.diff(qo), ext)
        # the new tokens' slots are the last n_b positions, read through kv_indices
        loc = md["out_cache_loc"]
        for b in range(len(seq_lens)):
            for i in range(int(ext[b])):
                pos = int(seq_lens[b]) - int(ext[b]) + i
                page = md["kv_indices"][ip[b] + pos // P]
                assert loc[qo[b] + i] == page * P + pos % P
        assert len(set(loc.tolist())) == len(loc)  # distinct slots


def test_metadata_page_size_one_is_token_slots():
    seq_lens = [5, 1, 8]
    table, pp = place(seq_lens, 1)
    md = oracle.metadata(seq_lens, None, table, 1, pp)
    assert np.all(md["kv_last_page_len"] == 1)
    assert np.array_equal(md["kv_indices"], np.concatenate([table[b, :L] for b, L in enumerate(seq_lens)]))
    # decode: the new token is the last slot of each request
    ip = md["kv_indptr"]
    assert np.array_equal(md["out_cache_loc"], md["kv_indices"][ip[1:] - 1])


def test_metadata_rejects_inconsistent_batches():
    table = np.array([[0, 1]], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.metadata([0], None, table, 4, 2)  # empty decode request
    with pytest.raises(ValueError):
        oracle.metadata([9], None, table, 4, 2)  # needs 3 pages, row holds 2
    with pytest.raises(ValueError):
        oracle.metadata([5], [6], table, 4, 2)  # more new tokens than tokens
    with pytest.raises(ValueError):
        oracle.metadata([5], None, np.array([[0, 7]], dtype=np.int32), 4, 2)  # page out of pool
