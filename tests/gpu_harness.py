"""Put a synthetic workload on the GPU in the library's layout and run the
library's entry points on it.  Used by the GPU tests, smoke() and bench.py.

Only the input generator and the C-ABI binding are used here: the cache is
uploaded in the generator's plain paged layout and converted on the device by
fsa_import_kv_plain; the page metadata is built by fsa_build_page_meta.
"""
from __future__ import annotations

import numpy as np
import torch

import free_sparse_attention_amd as fsa


def to_dev_bf16(a: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16 numpy) -> device bfloat16 tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bits(t: torch.Tensor) -> np.ndarray:
    """Device bf16 tensor -> uint16 numpy bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(t: torch.Tensor) -> np.ndarray:
    b = bits(t).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


class DeviceWorkload:
    """A workload resident in HBM: q, K/V caches (library layout), metadata, page table, lengths."""

    def __init__(self, wl, device="cuda", build_meta=True, replicas: int = 1):
        self.wl = wl
        self.device = device
        self.dims = fsa.dims(wl.batch, wl.hq, wl.hkv, wl.d, wl.max_pages, wl.pool_pages)
        self.q = to_dev_bf16(wl.q, device)
        self.page_table = torch.from_numpy(wl.page_table).to(device)
        self.seq_lens = torch.from_numpy(wl.seq_lens.astype(np.int32)).to(device)
        self.max_seq_len = int(wl.seq_lens.max())
        kp = to_dev_bf16(wl.k_pool, device)
        vp = to_dev_bf16(wl.v_pool, device)
        self.k_cache = torch.empty_like(kp)
        self.v_cache = torch.empty_like(vp)
        fsa.import_kv_plain(self.dims, kp, vp, self.k_cache, self.v_cache)
        del kp, vp
        self.meta = torch.zeros(fsa.meta_bytes(self.dims) // 2, dtype=torch.bfloat16, device=device)
        if build_meta:
            fsa.build_page_meta(self.dims, self.k_cache, self.page_table, self.seq_lens, self.meta)
        torch.cuda.synchronize()

    def meta_pages(self, meta=None) -> np.ndarray:
        """Library metadata as bf16 bits [B][Hkv][max_pages][2][D] (index 0 = min, 1 = max)."""
        wl = self.wl
        T = -(-wl.max_pages // 16)
        ns = 2 * wl.d // 32
        m = bits(self.meta if meta is None else meta).reshape(wl.batch, wl.hkv, T, ns, 16, 32)
        m = m.transpose(0, 1, 2, 4, 3, 5).reshape(wl.batch, wl.hkv, T * 16, 2 * wl.d)[:, :, :wl.max_pages]
        return m.reshape(wl.batch, wl.hkv, wl.max_pages, 2, wl.d)

    # ------------------------------------------------------------ entry points
    def cfg(self, cfg=None):
        return fsa.cfg(*(cfg if cfg is not None else self.wl.cfg))

    def scores(self, cfg=None, q=None, max_seq_len=None):
        wl = self.wl
        s = torch.full((wl.batch, wl.hkv, wl.max_pages), float("nan"), dtype=torch.float32, device=self.device)
        fsa.quest_scores(self.dims, self.cfg(cfg), max_seq_len or self.max_seq_len, self.q if q is None else q,
                         self.meta, self.seq_lens, s)
        return s

    def select(self, scores, cfg=None, max_seq_len=None):
        wl = self.wl
        c = self.cfg(cfg)
        msl = max_seq_len or self.max_seq_len
        n_items = fsa.max_work_items(self.dims, c, msl)
        sel = torch.full((wl.batch, wl.hkv, max(c.budget_pages, 1)), -7, dtype=torch.int32, device=self.device)
        work = torch.full((wl.batch, wl.hkv, n_items, 4), -7, dtype=torch.int32, device=self.device)
        counts = torch.full((wl.batch, wl.hkv, 2), -7, dtype=torch.int32, device=self.device)
        fsa.select_pages(self.dims, c, msl, scores, self.page_table, self.seq_lens,
                         sel if c.budget_pages > 0 else None, work, counts)
        return sel[..., :c.budget_pages], work, counts

    def workspace(self, cfg=None, max_seq_len=None):
        n = fsa.sparse_decode_workspace_bytes(self.dims, self.cfg(cfg), max_seq_len or self.max_seq_len)
        return torch.empty(n, dtype=torch.uint8, device=self.device)

    def sparse(self, cfg=None, q=None, max_seq_len=None, ws=None, out=None, want_sel=True):
        wl = self.wl
        c = self.cfg(cfg)
        msl = max_seq_len or self.max_seq_len
        if ws is None:
            ws = self.workspace(cfg, msl)
        if out is None:
            out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.bfloat16, device=self.device)
        sel = None
        if want_sel and c.budget_pages > 0:
            sel = torch.full((wl.batch, wl.hkv, c.budget_pages), -7, dtype=torch.int32, device=self.device)
        fsa.sparse_decode_attn(self.dims, c, wl.sm_scale, msl, self.q if q is None else q, self.k_cache,
                               self.v_cache, self.meta, self.page_table, self.seq_lens, out, sel, ws)
        return out, sel

    def dense_workspace(self, max_seq_len=None):
        n = fsa.dense_decode_workspace_bytes(self.dims, max_seq_len or self.max_seq_len)
        return torch.zeros(n, dtype=torch.uint8, device=self.device)

    def dense(self, q=None, max_seq_len=None, ws=None, out=None):
        wl = self.wl
        msl = max_seq_len or self.max_seq_len
        if ws is None:
            ws = self.dense_workspace(msl)
        if out is None:
            out = torch.empty((wl.batch, wl.hq, wl.d), dtype=torch.bfloat16, device=self.device)
        fsa.dense_decode_attn(self.dims, wl.sm_scale, msl, self.q if q is None else q, self.k_cache,
                              self.v_cache, self.page_table, self.seq_lens, out, ws)
        return out
