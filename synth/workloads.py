"""Seeded synthetic workloads shaped like the decode configurations under study.

Every workload is a batch of decode queries over a paged KV cache:

* ``q``          bf16 bits ``[B][Hq][D]``
* ``k_pool``     bf16 bits ``[pool][Hkv][S][D]`` (plain layout: token-major inside a page)
* ``v_pool``     bf16 bits ``[pool][Hkv][S][D]``
* ``page_table`` int32 ``[B][max_pages]`` logical page -> physical pool page (-1 = unmapped)
* ``seq_lens``   int32 ``[B]``, the number of cached tokens including the current one
* ``cfg``        ``(prefix_tokens, window_tokens, budget_pages)`` of the layer

Values (the stream numbers are fixed below; ``seed`` selects the workload):

* q, V ~ N(0, 1); K = s[g, c] * N(0, 1) with the per-(KV head, channel) scale
  s = exp(sigma * N(0, 1)) (LogNormal(0, sigma)); sigma = 0 gives s = 1.
* Needles: in each sequence ``n_needles`` distinct full pages inside the middle
  region [prefix, L - window) are drawn uniformly, and one uniformly drawn slot
  of each gets, for every KV head g, the key
  ``bf16(k + 4 * sqrt(D) * u_g)`` where k is the key already there and u_g is the
  unit vector along the sum of the group's query heads.
* Page tables are either contiguous (``b * max_pages + p``) or a Fisher-Yates
  permutation of the whole pool handed out to the sequences in order.

All random draws go through the counter-based generator, so a value depends
only on (seed, stream, logical index).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from . import core

# stream numbers (per layer, add 100 * layer)
S_Q, S_K, S_V, S_KSCALE, S_NEEDLE_PAGE, S_NEEDLE_SLOT = 1, 2, 3, 4, 5, 6
S_PERM, S_LENS, S_LAYER_CFG, S_STEP_Q = 7, 8, 9, 12


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    layer: int
    batch: int
    hq: int
    hkv: int
    d: int
    page: int
    seq_lens: np.ndarray
    max_pages: int
    pool_pages: int
    page_table: np.ndarray
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    cfg: tuple
    sm_scale: float
    needles: list
    k_scale: np.ndarray | None
    permuted: bool

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    def keys(self):
        """Stream keys of this workload's layer (K and V) and of its queries."""
        off = 100 * self.layer
        return (core.stream_key(self.seed, S_K + off), core.stream_key(self.seed, S_V + off),
                core.stream_key(self.seed, S_Q + off))

    def step_q(self, step: int) -> np.ndarray:
        """Query of decode step ``step`` (step 0 is ``self.q``)."""
        if step == 0:
            return self.q
        key = core.stream_key(self.seed, S_STEP_Q + 100 * self.layer)
        n = self.batch * self.hq * self.d
        return core.normal_bf16(key, n, idx0=step * n).reshape(self.batch, self.hq, self.d)

    def append_tokens(self, step: int, n_new: int = 1):
        """K/V of the ``n_new`` tokens appended at decode step ``step``.

        Token positions are seq_lens[b] + step * n_new + i, drawn with the same
        value rule as the prefilled cache.  Returns bf16 bits [B][n_new][Hkv][D] twice.
        """
        kk, kv, _ = self.keys()
        kn = np.empty((self.batch, n_new, self.hkv, self.d), np.uint16)
        vn = np.empty_like(kn)
        for b in range(self.batch):
            t0 = int(self.seq_lens[b]) + step * n_new
            kn[b] = core.fill_tokens(kk, b, t0, n_new, self.hkv, self.d, self.k_scale)
            vn[b] = core.fill_tokens(kv, b, t0, n_new, self.hkv, self.d, None)
        return kn, vn


def _permutation(seed: int, stream: int, n: int) -> np.ndarray:
    draws = core.raw_u64(core.stream_key(seed, stream), max(n - 1, 0))
    perm = np.arange(n, dtype=np.int64)
    # Fisher-Yates: position i swaps with j uniform in [0, i]
    for k, i in enumerate(range(n - 1, 0, -1)):
        j = int(draws[k] % np.uint64(i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return perm


def build(*, name="custom", seed=0, layer=0, batch=1, hq=8, hkv=2, d=64, page=16,
          seq_lens=(4096,), prefix=64, window=256, budget=32, k_sigma=0.0,
          n_needles=0, permuted=False, extra_tokens=0, sm_scale=None) -> Workload:
    """Generate one layer's inputs.  ``extra_tokens`` reserves mapped pages for appends."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (batch,)
    assert hq % hkv == 0
    off = 100 * layer
    pages_needed = [(int(L) + extra_tokens + page - 1) // page for L in seq_lens]
    max_pages = max(pages_needed)
    page_table = np.full((batch, max_pages), -1, dtype=np.int32)
    if permuted:
        pool_pages = sum(pages_needed)
        perm = _permutation(seed, S_PERM + off, pool_pages)
        o = 0
        for b, n in enumerate(pages_needed):
            page_table[b, :n] = perm[o:o + n]
            o += n
    else:
        pool_pages = batch * max_pages
        for b, n in enumerate(pages_needed):
            page_table[b, :n] = b * max_pages + np.arange(n)

    k_scale = None
    if k_sigma > 0:
        z = core.normal_f64(core.stream_key(seed, S_KSCALE + off), hkv * d)
        k_scale = np.exp(k_sigma * z).reshape(hkv, d)

    q = core.normal_bf16(core.stream_key(seed, S_Q + off), batch * hq * d).reshape(batch, hq, d)
    kk = core.stream_key(seed, S_K + off)
    kv = core.stream_key(seed, S_V + off)
    k_pool = np.zeros((pool_pages, hkv, page, d), np.uint16)
    v_pool = np.zeros((pool_pages, hkv, page, d), np.uint16)
    for b in range(batch):
        L = int(seq_lens[b])
        core.fill_pool_seq(kk, b, 0, L, hkv, d, page, page_table[b], k_scale, k_pool)
        core.fill_pool_seq(kv, b, 0, L, hkv, d, page, page_table[b], None, v_pool)

    needles = []
    G = hq // hkv
    for b in range(batch):
        L = int(seq_lens[b])
        lo_page = -(-prefix // page)              # first page fully at or after the prefix
        hi_page = max(L - window, 0) // page      # pages ending at or before L - window
        cand = np.arange(lo_page, hi_page)
        pos = np.zeros(0, np.int64)
        if n_needles > 0 and len(cand) > 0:
            m = min(n_needles, len(cand))
            kp = core.stream_key(seed, S_NEEDLE_PAGE + off)
            draws = core.raw_u64(kp, m, idx0=b * 4096)
            pool = cand.copy()
            chosen = []
            for i in range(m):  # partial Fisher-Yates over the candidate pages
                j = i + int(draws[i] % np.uint64(len(pool) - i))
                pool[i], pool[j] = pool[j], pool[i]
                chosen.append(int(pool[i]))
            slots = core.raw_u64(core.stream_key(seed, S_NEEDLE_SLOT + off), m, idx0=b * 4096)
            pos = np.sort(np.array([p * page + int(s % np.uint64(page)) for p, s in zip(chosen, slots)]))
            qf = core.bf16_bits_to_f64(q[b]).reshape(hkv, G, d).sum(axis=1)   # [hkv][d]
            u = qf / np.linalg.norm(qf, axis=1, keepdims=True)
            for t in pos:
                phys = page_table[b, t // page]
                slot = t % page
                k_old = core.bf16_bits_to_f64(k_pool[phys, :, slot, :])        # [hkv][d]
                k_pool[phys, :, slot, :] = core.f64_to_bf16_bits(k_old + 4.0 * math.sqrt(d) * u)
        needles.append(pos)

    return Workload(name=name, seed=seed, layer=layer, batch=batch, hq=hq, hkv=hkv, d=d, page=page,
                    seq_lens=seq_lens, max_pages=max_pages, pool_pages=pool_pages,
                    page_table=page_table, q=q, k_pool=k_pool, v_pool=v_pool,
                    cfg=(int(prefix), int(window), int(budget)),
                    sm_scale=float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(d)),
                    needles=needles, k_scale=k_scale, permuted=permuted)


def sweep_layer_cfg(seed: int, layer: int):
    """Per-layer (prefix, window, budget) of the 12-layer sweep, drawn from ``seed``."""
    u = core.raw_u64(core.stream_key(seed, S_LAYER_CFG), 3, idx0=3 * layer)
    prefixes, windows, budgets = (0, 64, 128), (512, 1024, 2048, 4096, 8192), (64, 128, 256, 512)
    return (prefixes[int(u[0] % np.uint64(3))], windows[int(u[1] % np.uint64(5))],
            budgets[int(u[2] % np.uint64(4))])


def ragged_lens(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    u = core.raw_u64(core.stream_key(seed, S_LENS), batch)
    return (lo + (u % np.uint64(hi - lo + 1)).astype(np.int64)).astype(np.int32)


# Named workloads.  Sizes follow the decode configurations studied: a tiny
# case, batch-4 decode at 64k and 256k context, a 12-layer sweep at 128k and a
# ragged 16-sequence serving batch with appends.
WORKLOADS = {
    "tiny": dict(seed=0, batch=1, hq=8, hkv=2, d=64, seq_lens=(4096,), prefix=64, window=256,
                 budget=32, k_sigma=0.0, n_needles=8, permuted=False),
    "ctx64k": dict(seed=1, batch=4, hq=16, hkv=4, d=128, seq_lens=(65536,) * 4, prefix=128,
                   window=1024, budget=128, k_sigma=0.5, n_needles=64, permuted=False),
    "ctx256k": dict(seed=2, batch=4, hq=32, hkv=4, d=128, seq_lens=(262144,) * 4, prefix=128,
                    window=4096, budget=256, k_sigma=0.5, n_needles=64, permuted=True),
}


def make_workload(name: str, layer: int = 0, **overrides) -> Workload:
    """Build a named workload.  ``sweep12`` takes ``layer`` in 0..11; ``ragged16``
    reserves room for 64 appended tokens per sequence."""
    if name in WORKLOADS:
        spec = dict(WORKLOADS[name])
    elif name == "sweep12":
        p, w, bud = sweep_layer_cfg(3, layer)
        spec = dict(seed=3, layer=layer, batch=4, hq=16, hkv=4, d=128, seq_lens=(131072,) * 4,
                    prefix=p, window=w, budget=bud, k_sigma=0.5, n_needles=64, permuted=False)
    elif name == "ragged16":
        spec = dict(seed=4, batch=16, hq=32, hkv=8, d=128,
                    seq_lens=tuple(ragged_lens(4, 16, 16384, 262144)), prefix=128, window=2048,
                    budget=256, k_sigma=0.5, n_needles=64, permuted=True, extra_tokens=64)
    else:
        raise KeyError(name)
    spec.update(overrides)
    return build(name=name, **spec)
