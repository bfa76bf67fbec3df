"""Build and run one seeded workload through the HIP library (GPU tests,
smoke check and benchmark share this).  Pools start as NaN sentinels, every
cached token is written by the library's own save_kv, and the batch's
metadata is built by the library's own metadata kernels."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_attention_02_amd as pka
import workloads

KV_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


def sentinel_pool_gpu(shape, kv_dtype: str, device="cuda"):
    if kv_dtype == "fp8":
        return torch.full(shape, 0x7F, dtype=torch.uint8, device=device)
    return torch.full(shape, float("nan"), dtype=KV_TORCH[kv_dtype], device=device)


class GpuProblem:
    def __init__(self, layout: workloads.Layout, values: workloads.Values = None, device="cuda",
                 fill: bool = True, prefix_only: bool = False, max_q_per_request: int = 0):
        spec = layout.spec
        self.layout, self.spec = layout, spec
        if values is None:
            values = workloads.make_values(layout, device=device)
        self.values = values
        self.ctx = pka.Context(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                               layout.num_pages, spec.q_dtype, spec.kv_dtype, spec.softmax_scale,
                               values.k_scale, values.v_scale, v_head_dim=spec.value_dim,
                               max_q_per_request=max_q_per_request)
        self.k_pool = sentinel_pool_gpu(self.ctx.pool_shape(), spec.kv_dtype, device)
        self.v_pool = sentinel_pool_gpu(self.ctx.v_pool_shape(), spec.kv_dtype, device)
        i32 = dict(dtype=torch.int32, device=device)
        self.seq_lens = torch.tensor(layout.seq_lens, **i32)
        self.extend_lens = torch.tensor(layout.extend_lens, **i32)
        self.page_table = torch.tensor(layout.page_table, **i32)
        B, kvp = layout.batch, layout.kv_pages
        if fill:
            self.fill_pools(prefix_only)
        self.mode = spec.mode
        self.md = pka.Batch(self.ctx, self.mode, B, layout.num_q_tokens, kvp, device=device)
        self.md.init(self.seq_lens, None if self.mode == "decode" else self.extend_lens,
                     self.page_table)
        rows = torch.from_numpy(workloads.new_token_rows(layout)).to(device)
        self.k_new = values.k_all.index_select(0, rows).contiguous()
        self.v_new = values.v_all.index_select(0, rows).contiguous()
        self.out = torch.empty((layout.num_q_tokens, spec.num_q_heads, spec.value_dim),
                               dtype=workloads.torch_dtype(spec.q_dtype), device=device)
        self.lse = torch.empty((layout.num_q_tokens, spec.num_q_heads), dtype=torch.float32,
                               device=device)

    def fill_pools(self, prefix_only: bool = False):
        """Write every cached token (prefix and new) with the library's save_kv.

        prefix_only: afterwards put the sentinel back into the new tokens'
        slots, so only a forward pass with save_kv_cache=True fills them."""
        layout = self.layout
        B = layout.batch
        fill = pka.Batch(self.ctx, "extend", B, layout.total_tokens, layout.kv_pages,
                         device=self.seq_lens.device)
        fill.init(self.seq_lens, self.seq_lens, self.page_table)
        pka.save_kv(self.ctx, fill, self.values.k_all, self.values.v_all, self.k_pool, self.v_pool)
        torch.cuda.synchronize()
        status = fill.status()
        assert status == 0, f"device status {status} while filling the pools"
        if prefix_only:
            rows = torch.from_numpy(workloads.new_token_rows(layout)).to(self.seq_lens.device)
            self.new_slots = fill.out_cache_loc.index_select(0, rows).long()
            for pool in (self.k_pool, self.v_pool):
                pool[self.new_slots] = sentinel_pool_gpu((1,) + tuple(pool.shape[1:]),
                                                         self.spec.kv_dtype, pool.device)

    def metadata_step(self):
        self.md.init(self.seq_lens, None if self.mode == "decode" else self.extend_lens,
                     self.page_table)

    def attention_step(self, save: bool = True, spec_mode: str = "prefill", lse: bool = True):
        pka.forward(self.ctx, self.mode, self.md, self.values.q, self.k_new, self.v_new,
                    self.k_pool, self.v_pool, self.out, self.lse if lse else None,
                    save_kv_cache=save, spec_mode=spec_mode)

    def step(self):
        """One pass of the whole path: metadata, cache write, attention."""
        self.metadata_step()
        self.attention_step(save=True)

    def fused_step(self, save: bool = True, lse: bool = True, page_table=None, seq_lens=None,
                   spec_mode: str = "prefill"):
        """The same pass as step(), through the one-call entry point
        (pka_forward_with_metadata)."""
        pt = self.page_table if page_table is None else page_table
        sl = self.seq_lens if seq_lens is None else seq_lens
        pka.forward_with_metadata(self.ctx, self.mode, self.md, sl,
                                  None if self.mode == "decode" else self.extend_lens, pt,
                                  self.values.q, self.k_new, self.v_new, self.k_pool, self.v_pool,
                                  self.out, self.lse if lse else None, save_kv_cache=save,
                                  spec_mode=spec_mode)

    def out_np(self) -> np.ndarray:
        return self.out.float().cpu().numpy().astype(np.float64)

    def lse_np(self) -> np.ndarray:
        return self.lse.cpu().numpy().astype(np.float64)
