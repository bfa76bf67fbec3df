"""Test-side glue: build oracle inputs from a seeded workload.

Only tests and the benchmark's CPU-baseline leg use this; it calls nothing but
the oracle and the seeded generators.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads

NAN_BITS = {"f32": None, "bf16": 0x7FC0, "fp8": 0x7F}
RAW_NP = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


def raw_np(t) -> np.ndarray:
    """Raw storage of a torch tensor as numpy (bf16 -> uint16 bit patterns)."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(t.dtype)


def sentinel_pool(slots: int, heads: int, dim: int, kv_dtype: str) -> np.ndarray:
    """A pool whose every slot holds NaN, so stray reads show up as NaN."""
    if kv_dtype == "f32":
        return np.full((slots, heads, dim), np.nan, dtype=np.float32)
    return np.full((slots, heads, dim), NAN_BITS[kv_dtype], dtype=RAW_NP[kv_dtype])


def oracle_pools(layout: workloads.Layout, k_all: np.ndarray, v_all: np.ndarray, k_scale=1.0,
                 v_scale=1.0):
    """Oracle cache write of every token of every request (prefix and new)."""
    spec = layout.spec
    md = oracle.metadata(layout.seq_lens, layout.seq_lens, layout.page_table, spec.page_size,
                         layout.num_pages)
    slots = layout.num_pages * spec.page_size
    kp = sentinel_pool(slots, spec.num_kv_heads, spec.head_dim, spec.kv_dtype)
    vp = sentinel_pool(slots, spec.num_kv_heads, spec.value_dim, spec.kv_dtype)
    oracle.save_kv(md["out_cache_loc"], k_all, v_all, spec.q_dtype, spec.kv_dtype, kp, vp,
                   k_scale, v_scale)
    return kp, vp


def oracle_full(layout: workloads.Layout, values: workloads.Values, threads: int = 0):
    """Whole-batch oracle output (small and medium shapes)."""
    spec = layout.spec
    q = raw_np(values.q)
    kp, vp = oracle_pools(layout, raw_np(values.k_all), raw_np(values.v_all), values.k_scale,
                          values.v_scale)
    ext = None if spec.mode == "decode" else layout.extend_lens
    return oracle.attention(layout.seq_lens, ext, layout.page_table, spec.page_size,
                            layout.num_pages, q, spec.q_dtype, kp, vp, spec.kv_dtype,
                            spec.softmax_scale, values.k_scale, values.v_scale, threads=threads)


def oracle_requests(layout: workloads.Layout, values: workloads.Values, requests, heads=None,
                    tokens=None, threads: int = 0):
    """Oracle output for a few requests of a large batch.

    Each selected request is re-packed into a compact single-request problem
    (its own tokens, contiguous pages); attention of a request does not depend
    on where its pages sit in the pool.  ``tokens(n_b)`` may pick a subset of
    the request's new tokens.  Returns {b: (token_idx, out [t, H, Dv], lse [t, H])}.
    """
    spec = layout.spec
    offs = workloads.request_token_offsets(layout)
    qo = np.concatenate([[0], np.cumsum(layout.extend_lens.astype(np.int64))])
    P = spec.page_size
    res = {}
    for b in requests:
        L, n = int(layout.seq_lens[b]), int(layout.extend_lens[b])
        pages = (L + P - 1) // P
        sub = workloads.Layout(spec, np.array([L], np.int32), np.array([n], np.int32),
                               np.arange(pages, dtype=np.int32)[None, :], pages)
        k = raw_np(values.k_all[offs[b]:offs[b + 1]])
        v = raw_np(values.v_all[offs[b]:offs[b + 1]])
        kp, vp = oracle_pools(sub, k, v, values.k_scale, values.v_scale)
        q = raw_np(values.q[qo[b]:qo[b + 1]])
        ext = None if spec.mode == "decode" else sub.extend_lens
        Hq = spec.num_q_heads
        hs = list(range(Hq)) if heads is None else list(heads)
        ts = list(range(n)) if tokens is None else list(tokens(n))
        sel = np.array([t * Hq + h for t in ts for h in hs], dtype=np.int64)
        out, lse = oracle.attention(sub.seq_lens, ext, sub.page_table, P, pages, q, spec.q_dtype,
                                    kp, vp, spec.kv_dtype, spec.softmax_scale, values.k_scale,
                                    values.v_scale, sel=sel, threads=threads)
        res[b] = (np.asarray(ts, dtype=np.int64), out.reshape(len(ts), len(hs), spec.value_dim),
                  lse.reshape(len(ts), len(hs)))
    return res


def errors(gpu: np.ndarray, ref: np.ndarray):
    """(max-abs, relative RMS) of gpu vs ref over the whole tensor."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    diff = g - r
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.sqrt(np.sum(r * r)))
    rel = float(np.sqrt(np.sum(diff * diff)) / denom) if denom > 0 else float(np.sqrt(np.sum(diff * diff)))
    return max_abs, rel


# Gates: bf16/fp32 caches and fp8 caches.
TOL = {"f32": (2e-2, 5e-3), "bf16": (2e-2, 5e-3), "fp8": (5e-2, 2e-2)}

# Absolute tolerance of the log-sum-exp output (not a gate of the method, a
# check of the normaliser): the kernels round the softmax weights to bf16
# before summing them, and bf16's unit roundoff 2^-8 bounds the relative
# error of that sum, i.e. |d lse| <= ln(1 + 2^-8) = 3.9e-3.
LSE_ATOL = 4e-3
