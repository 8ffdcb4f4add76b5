"""CPU oracle of combined sparse decode attention: plain, slow, float64.

TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path imports or
calls this module; only the tests, the smoke check and the CPU-baseline leg of
the benchmark do.  It shares no code with the GPU library: it reads the plain
paged pool that the input generator writes (``[pool][Hkv][S][D]`` bf16 bits,
token-major inside a page) and follows the method step by step.

Method (all from the paper "Accelerating Long-Context Decoding in Large-Scale
Hybrid LLMs Without Retraining", Batista, Vatai and Wahib):

* Abstract: each remaining full-attention layer attends, at each decode step,
  to a sliding window of recent tokens, a pinned prefix and a fixed budget of
  the most relevant context tokens; window and budget are set per layer.
* Analysis page, "Methodology", and the digest page, "The Move": the relevant
  tokens are chosen query-aware, Quest style, as a paged top-k.
* Digest page, "Why It Matters": the KV cache stays full size, so any page can
  be selected.

Quest's page criterion (Tang et al., ICML 2024): for every page keep the
elementwise minimum m and maximum M of its keys; the upper bound on q.k over
the page is sum_i max(q_i m_i, q_i M_i).

Readings where the pages leave a step open:

* the budget counts pages of S tokens;
* one selection per (sequence, KV head), shared by the group's query heads;
  a page's group score is the largest of the per-head bounds;
* candidates are the pages that intersect the middle region [P, L - W);
* the union of prefix, window and selected pages is taken token by token;
* k = min(budget, candidates); equal scores go to the lower logical page id;
* softmax scale is an explicit argument (1/sqrt(D) in the workloads);
* a zero in the page metadata is stored as +0.

Parity status of each function is stated in its docstring ("pinned by ..." or
"parity unpinned").
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 of float64 values (through fp32), returned as float64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Step 1: page metadata (Quest's per-page elementwise key minimum and maximum)
# --------------------------------------------------------------------------

def gather_keys(pool: np.ndarray, page_table: np.ndarray, b: int, g: int, L: int) -> np.ndarray:
    """Keys (or values) of tokens [0, L) of sequence b, KV head g: float64 [L][D].

    Token t lives in physical page page_table[b][t // S], slot t % S.
    Pinned by: page-table permutation invariance of every later result.
    """
    S = pool.shape[2]
    n = -(-L // S)
    phys = page_table[b, :n]
    blocks = bf16_to_f64(pool[phys, g])          # [n][S][D]
    return blocks.reshape(n * S, -1)[:L]


def page_minmax(keys: np.ndarray, S: int):
    """Elementwise min and max of the keys of every page, over its valid tokens.

    keys: float64 [L][D] of one (sequence, KV head).  Returns (m, M), each [n][D].
    The last page may be partial: only tokens < L count.  A zero result is
    returned as +0 (x + 0.0 turns -0 into +0 and leaves every other value alone).
    Pinned by: brute-force containment and attainment tests, and append-vs-rebuild.
    """
    L, D = keys.shape
    n = -(-L // S)
    m = np.empty((n, D))
    M = np.empty((n, D))
    for p in range(n):
        blk = keys[p * S:min(p * S + S, L)]
        m[p] = blk.min(axis=0) + 0.0
        M[p] = blk.max(axis=0) + 0.0
    return m, M


def build_meta(k_pool: np.ndarray, page_table: np.ndarray, seq_lens: np.ndarray) -> dict:
    """Metadata of every mapped page in use: {(phys, g): (m[D], M[D])} float64."""
    out = {}
    S = k_pool.shape[2]
    for b, L in enumerate(seq_lens):
        L = int(L)
        for g in range(k_pool.shape[1]):
            m, M = page_minmax(gather_keys(k_pool, page_table, b, g, L), S)
            for p in range(m.shape[0]):
                out[(int(page_table[b, p]), g)] = (m[p], M[p])
    return out


# --------------------------------------------------------------------------
# Step 2: regions and candidate pages
# --------------------------------------------------------------------------

def regions(L: int, prefix: int, window: int):
    """(Pe, Ws): the prefix is [0, Pe), the window [Ws, L), the middle [Pe, Ws)."""
    Pe = min(prefix, L)
    Ws = max(0, L - window)
    return Pe, Ws


def candidate_pages(L: int, prefix: int, window: int, S: int) -> np.ndarray:
    """Logical pages that intersect the middle region [Pe, Ws) (empty if Pe >= Ws)."""
    Pe, Ws = regions(L, prefix, window)
    if Pe >= Ws:
        return np.zeros(0, np.int64)
    return np.arange(Pe // S, -(-Ws // S), dtype=np.int64)


# --------------------------------------------------------------------------
# Step 3: Quest bound per query head, group score
# --------------------------------------------------------------------------

def quest_bound(q: np.ndarray, m: np.ndarray, M: np.ndarray) -> np.ndarray:
    """U[h][p] = sum_i max(q[h,i] * m[p,i], q[h,i] * M[p,i]).

    q: float64 [G][D]; m, M: float64 [C][D].  Quest's upper bound on q_h . k
    over every key k of page p.  Pinned by: brute-force bound invariant, tight
    single-token and constant-page cases, K = 0, positive-q closed form, and the
    hand-worked fixture in tests/golden/.
    """
    lo = q[:, None, :] * m[None, :, :]
    hi = q[:, None, :] * M[None, :, :]
    return np.maximum(lo, hi).sum(axis=2)


def group_score(U: np.ndarray) -> np.ndarray:
    """Score of each page for the KV-head group: the largest per-head bound.

    Parity unpinned: the pages do not say how a query group shares one
    selection; taking the maximum keeps the bound valid for every head.
    """
    return U.max(axis=0)


# --------------------------------------------------------------------------
# Step 4: top-k page selection
# --------------------------------------------------------------------------

def select_topk(scores: np.ndarray, pages: np.ndarray, budget: int) -> np.ndarray:
    """The k = min(budget, C) pages with the largest scores, ascending by id.

    Order: larger score first, equal scores by lower logical page id; -0 == +0.
    Pinned by: a rank-counting brute force on tiny inputs with forced ties, and
    the all-equal (K = 0) closed form (the first k candidates).
    """
    k = min(int(budget), len(pages))
    order = np.lexsort((pages, -(scores + 0.0)))
    return np.sort(pages[order[:k]])


def selection_margin(scores: np.ndarray, budget: int) -> float:
    """(s_(k) - s_(k+1)) / |s_(k)| over the sorted scores; inf when nothing is left out."""
    k = min(int(budget), len(scores))
    if k >= len(scores) or k == 0:
        return float("inf")
    s = np.sort(scores)[::-1]
    return float((s[k - 1] - s[k]) / max(abs(s[k - 1]), 1e-300))


# --------------------------------------------------------------------------
# Step 5: attended token set (union of prefix, window and selected pages)
# --------------------------------------------------------------------------

def attended_mask(L: int, prefix: int, window: int, S: int, selected) -> np.ndarray:
    """Boolean mask over tokens [0, L): prefix, window and every token of a selected page.

    Pinned by: the per-token brute force and the count closed form in the tests.
    """
    Pe, Ws = regions(L, prefix, window)
    mask = np.zeros(L, dtype=bool)
    mask[:Pe] = True
    mask[Ws:L] = True
    for p in selected:
        mask[int(p) * S:min(int(p) * S + S, L)] = True
    return mask


# --------------------------------------------------------------------------
# Step 6: attention over the attended set (two-pass softmax)
# --------------------------------------------------------------------------

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, mask: np.ndarray, sm_scale: float) -> np.ndarray:
    """out[h] = sum_t softmax_t(sm_scale * q_h . k_t) v_t over the masked tokens.

    Two passes, float64: the maximum logit first, then the weighted sums.
    Pinned by: torch CPU scaled_dot_product_attention in float64 with a
    boolean mask, constant-V and equal-logit closed forms.
    """
    idx = np.nonzero(mask)[0]
    Ks, Vs = K[idx], V[idx]
    z = sm_scale * (q @ Ks.T)                 # [G][T]
    mu = z.max(axis=1, keepdims=True)
    w = np.exp(z - mu)
    return (w @ Vs) / w.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# Whole decode step for one (sequence, KV head) unit
# --------------------------------------------------------------------------

def unit_inputs(wl, b: int, g: int, q_bits=None):
    """float64 q of the group [G][D] and K, V of the sequence [L][D]."""
    G = wl.hq // wl.hkv
    qb = wl.q if q_bits is None else q_bits
    q = bf16_to_f64(qb[b, g * G:(g + 1) * G])
    L = int(wl.seq_lens[b])
    K = gather_keys(wl.k_pool, wl.page_table, b, g, L)
    V = gather_keys(wl.v_pool, wl.page_table, b, g, L)
    return q, K, V


def sparse_decode_unit(q, K, V, L, cfg, S, sm_scale, selected=None) -> dict:
    """Decode one (sequence, KV head): scores, selection, mask and output.

    ``selected`` overrides the oracle's own selection (used to check attention
    on the exact page set another implementation chose).
    """
    prefix, window, budget = cfg
    m, M = page_minmax(K, S)
    cand = candidate_pages(L, prefix, window, S)
    U = quest_bound(q, m[cand], M[cand])
    s = group_score(U)
    sel = select_topk(s, cand, budget) if selected is None else np.asarray(selected)
    mask = attended_mask(L, prefix, window, S, sel)
    out = attend(q, K, V, mask, sm_scale)
    return dict(candidates=cand, scores=s, bounds=U, selected=sel, mask=mask, out=out,
                margin=selection_margin(s, budget), meta=(m, M))


def dense_decode_unit(q, K, V, sm_scale) -> np.ndarray:
    """Plain attention over all tokens [0, L)."""
    return attend(q, K, V, np.ones(K.shape[0], dtype=bool), sm_scale)
