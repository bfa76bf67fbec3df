"""Seeded synthetic inputs for paged KV attention.

This module is shared by the HIP path's tests/benchmark and by the oracle's
tests.  It only *draws* inputs (lengths, page placement, Q/K/V values and the
per-tensor fp8 scales that the workload recipe fixes); it holds none of the
attention arithmetic, no metadata construction and no quantiser.

Recipe (all draws seeded, in this order):
  1. lengths      numpy PCG64(seed): uniform integers (inclusive ends) or
                  log-uniform round(exp(U(ln a, ln b)));
  2. placement    the same numpy generator: a permutation of the page pool,
                  the first sum(ceil(L_b/P)) entries handed out to requests in
                  order (pool = ceil(1.25 * needed pages) unless fixed);
  3. values       torch.Generator(device).manual_seed(seed): Q, then K, then V,
                  each N(0,1) in fp32 (V optionally shifted), then rounded to
                  the workload's Q dtype (bf16 with round-to-nearest-even).
The fp8 per-tensor scales are absmax(K)/448 and absmax(V)/448 over every
cached K/V value, as fp32 (the long-context fp8 decode recipe).

Shapes follow the pages' model families (Llama-3-8B and Qwen3-235B GQA,
head_dim 128): "sglang-101 s4.2 --attention-backend", section "How SGLang picks
a default" names MHA models such as Llama and Qwen.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

FP8_E4M3FN_MAX = 448.0

DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and draw recipe of one synthetic workload."""

    name: str
    mode: str  # "decode" or "extend"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    q_dtype: str  # "f32" or "bf16"
    kv_dtype: str  # "f32", "bf16" or "fp8"
    seed: int
    # decode: lengths of the whole cached context including the new token.
    seq_len_kind: str = "fixed"  # fixed | uniform | loguniform
    seq_len_args: tuple = ()
    # extend: new tokens and cached prefix are drawn separately.
    new_len_args: tuple = ()
    prefix_len_args: tuple = ()
    pool_pages: Optional[int] = None  # None -> ceil(1.25 * needed pages)
    scale: Optional[float] = None  # None -> 1/sqrt(head_dim)
    v_mean: float = 0.0
    q_mult: float = 1.0
    v_head_dim: Optional[int] = None  # None -> head_dim

    @property
    def value_dim(self) -> int:
        return self.head_dim if self.v_head_dim is None else self.v_head_dim

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


# The seeded workloads the path is checked and measured on, named by shape.
WORKLOADS = {
    "tiny_decode": Spec("tiny_decode_f32_b2_g2_d64_p1", "decode", 2, 4, 2, 64, 1, "f32", "f32", seed=1,
            seq_len_kind="fixed", seq_len_args=(37, 100), pool_pages=256, scale=1.0 / 8.0),
    "llama3_8b_decode": Spec("llama3_8b_decode_bf16_b64_g4_d128_p16", "decode", 64, 32, 8, 128, 16, "bf16", "bf16",
            seed=2, seq_len_kind="uniform", seq_len_args=(512, 4096)),
    "qwen3_235b_decode": Spec("qwen3_235b_decode_bf16_b128_g16_d128_p1", "decode", 128, 64, 4, 128, 1, "bf16", "bf16",
            seed=3, seq_len_kind="loguniform", seq_len_args=(2048, 32768)),
    "llama3_8b_extend": Spec("extend_bf16_b8_g4_d128_p128", "extend", 8, 32, 8, 128, 128, "bf16", "bf16", seed=4,
            new_len_args=(512, 2048), prefix_len_args=(0, 4096)),
    "long_fp8_decode": Spec("long_decode_fp8kv_b16_g8_d128_p64", "decode", 16, 64, 8, 128, 64, "bf16", "fp8", seed=5,
            seq_len_kind="uniform", seq_len_args=(32768, 131072)),
}

# A small-context decode shaped after the pages' L4 log line: 33 running
# requests, 20,422 cached tokens (about 619 each), Qwen3-8B-like 32/8 heads.
EXTRA = {
    "l4_log_decode": Spec("l4_log_decode_bf16_b33_g4_d128_p1", "decode", 33, 32, 8, 128, 1, "bf16",
                          "bf16", seed=11, seq_len_kind="uniform", seq_len_args=(519, 719)),
    # Key and value heads of different widths (the pages have a backend picked
    # for such models): 192-wide query/key heads (128 + a 64-wide rotary part)
    # against 128-wide values, 16 heads of one rank, plain multi-head (G = 1),
    # pages of 128 tokens (the native page size the pages give that backend).
    "asym_extend": Spec("asym_extend_bf16_b8_h16_dk192_dv128_p128", "extend", 8, 16, 16, 192, 128,
                        "bf16", "bf16", seed=12, new_len_args=(512, 2048),
                        prefix_len_args=(0, 4096), v_head_dim=128),
    "asym_decode": Spec("asym_decode_bf16_b64_h16_dk192_dv128_p128", "decode", 64, 16, 16, 192, 128,
                        "bf16", "bf16", seed=13, seq_len_kind="uniform",
                        seq_len_args=(512, 8192), v_head_dim=128),
    # Speculative verify on the Llama-shaped cache: 64 requests, each with 4
    # chained draft tokens (topk = 1) on a cached prefix uniform in
    # [508, 4092] (contexts of 512 ... 4096 tokens, as the decode batch).
    "llama3_8b_verify": Spec("verify_bf16_b64_g4_d128_p16_n4", "extend", 64, 32, 8, 128, 16, "bf16",
                             "bf16", seed=14, new_len_args=(4, 4), prefix_len_args=(508, 4092)),
}


@dataclasses.dataclass
class Layout:
    """Integer part of a workload: lengths and page placement (host arrays)."""

    spec: Spec
    seq_lens: np.ndarray  # int32 [B]: L_b, tokens attended (includes new tokens)
    extend_lens: np.ndarray  # int32 [B]: n_b, new tokens (decode: all ones)
    page_table: np.ndarray  # int32 [B, cols]: physical page ids, -1 past the end
    num_pages: int

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_q_tokens(self) -> int:
        return int(self.extend_lens.sum())

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.sum())

    @property
    def prefix_lens(self) -> np.ndarray:
        return (self.seq_lens - self.extend_lens).astype(np.int32)

    @property
    def kv_pages(self) -> int:
        P = self.spec.page_size
        return int(sum((int(L) + P - 1) // P for L in self.seq_lens))


def _draw_ints(rng: np.random.Generator, kind: str, args: Sequence, n: int) -> np.ndarray:
    if kind == "fixed":
        assert len(args) == n, (args, n)
        return np.asarray(args, dtype=np.int64)
    lo, hi = args
    if kind == "uniform":
        return rng.integers(lo, hi, size=n, endpoint=True).astype(np.int64)
    if kind == "loguniform":
        u = rng.uniform(math.log(lo), math.log(hi), size=n)
        return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)
    raise ValueError(kind)


def make_layout(spec: Spec, seq_lens: Optional[Sequence[int]] = None,
                extend_lens: Optional[Sequence[int]] = None,
                pool_pages: Optional[int] = None) -> Layout:
    """Draw lengths, then page placement.  Explicit lengths override the draw."""
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    B, P = spec.batch, spec.page_size
    if seq_lens is not None:
        L = np.asarray(seq_lens, dtype=np.int64)
        n = (np.ones_like(L) if extend_lens is None else np.asarray(extend_lens, dtype=np.int64))
    elif spec.mode == "decode":
        L = _draw_ints(rng, spec.seq_len_kind, spec.seq_len_args, B)
        n = np.ones(B, dtype=np.int64)
    else:
        n = _draw_ints(rng, "uniform", spec.new_len_args, B)
        p = _draw_ints(rng, "uniform", spec.prefix_len_args, B)
        L = p + n
    B = int(L.shape[0])
    pages = [(int(x) + P - 1) // P for x in L]
    need = int(sum(pages))
    if pool_pages is None:
        pool_pages = spec.pool_pages if (spec.pool_pages is not None and seq_lens is None) else None
    if pool_pages is None:
        pool_pages = max(1, math.ceil(1.25 * need))
    assert pool_pages >= need, (pool_pages, need)
    perm = rng.permutation(pool_pages)[:need]
    cols = max(1, max(pages) if pages else 1)
    table = np.full((B, cols), -1, dtype=np.int32)
    off = 0
    for b, k in enumerate(pages):
        table[b, :k] = perm[off:off + k]
        off += k
    return Layout(spec, L.astype(np.int32), n.astype(np.int32), table, int(pool_pages))


@dataclasses.dataclass
class Values:
    """Floating-point part of a workload, as torch tensors on one device."""

    q: "object"  # [N, Hq, D] in the Q dtype
    k_all: "object"  # [sum L, Hkv, D] in the Q dtype, request-major, position order
    v_all: "object"  # [sum L, Hkv, Dv]
    k_scale: float  # fp32 per-tensor fp8 scale (1.0 for non-fp8 caches)
    v_scale: float


def torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_values(layout: Layout, device="cpu") -> Values:
    """Draw Q, then K, then V (N(0,1) fp32, rounded to the Q dtype)."""
    import torch
    spec = layout.spec
    g = torch.Generator(device=device)
    g.manual_seed(spec.seed)
    N, T = layout.num_q_tokens, layout.total_tokens
    Hq, Hkv, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    dt = torch_dtype(spec.q_dtype)

    def draw(rows, heads, mean=0.0, mult=1.0, width=D):
        x = torch.randn((rows, heads, width), generator=g, device=device, dtype=torch.float32)
        if mult != 1.0:
            x.mul_(mult)
        if mean != 0.0:
            x.add_(mean)
        return x.to(dt)

    q = draw(N, Hq, mult=spec.q_mult)
    k = draw(T, Hkv)
    v = draw(T, Hkv, mean=spec.v_mean, width=spec.value_dim)
    ks = vs = 1.0
    if spec.kv_dtype == "fp8":
        ks = float(np.float32(float(k.abs().amax().float()) / FP8_E4M3FN_MAX))
        vs = float(np.float32(float(v.abs().amax().float()) / FP8_E4M3FN_MAX))
    return Values(q, k, v, ks, vs)


def new_token_rows(layout: Layout) -> np.ndarray:
    """Indices into k_all/v_all of the new tokens, in query-token order."""
    rows: List[int] = []
    off = 0
    for L, n in zip(layout.seq_lens.tolist(), layout.extend_lens.tolist()):
        rows.extend(range(off + L - n, off + L))
        off += L
    return np.asarray(rows, dtype=np.int64)


def request_token_offsets(layout: Layout) -> np.ndarray:
    """Start row of each request in k_all/v_all (length B+1)."""
    return np.concatenate([[0], np.cumsum(layout.seq_lens.astype(np.int64))])
