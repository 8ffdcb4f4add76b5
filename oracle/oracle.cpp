/*
 * CPU oracle of combined sparse decode attention: plain, slow C++ in double.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path links,
 * loads or calls this file; only the tests, the smoke check and the CPU
 * baseline of the benchmark do.  It shares no code with the GPU library: it
 * reads the plain paged pool the input generator writes (bf16 bits,
 * [pool][Hkv][S][D], token-major inside a page) and follows the method step
 * by step, every step exposed as its own function.
 *
 * The method (paper "Accelerating Long-Context Decoding in Large-Scale Hybrid
 * LLMs Without Retraining", Batista, Vatai and Wahib):
 *   - Abstract: each remaining full-attention layer attends, at every decode
 *     step, to a sliding window of recent tokens, a pinned prefix and a fixed
 *     budget of the most relevant context tokens; window and budget are set
 *     per layer.
 *   - Analysis page, "Methodology", and digest page, "The Move": the relevant
 *     tokens are chosen query-aware, Quest style, as a paged top-k.
 *   - Digest page, "Why It Matters": the KV cache stays full size, so any page
 *     can be chosen.
 * Quest's criterion (Tang et al., ICML 2024): per page the elementwise
 * minimum m and maximum M of its keys; sum_i max(q_i m_i, q_i M_i) bounds q.k
 * over every key of the page.
 *
 * Readings where the pages leave a step open (each is a choice, stated once):
 *   - the budget counts pages of S tokens;
 *   - one selection per (sequence, KV head), shared by the query heads of its
 *     group (query head h belongs to KV head h / G, G = Hq / Hkv); a page's
 *     group score is the largest of its per-head bounds;
 *   - candidates are the pages meeting the middle region [min(P, L), L - W);
 *   - prefix, window and selected pages are united token by token;
 *   - k = min(budget, candidates); equal scores go to the lower logical page
 *     id, and -0 equals +0;
 *   - the softmax scale is an explicit argument;
 *   - a zero in the metadata is stored as +0.
 *
 * Parity of each function: see the "pinned by" note above it, or "parity
 * unpinned".  Built with g++ into liboracle.so and called through ctypes.
 */
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <limits>
#include <thread>
#include <vector>

namespace {

// ------------------------------------------------------------------ numbers

// Exact value of one bf16 bit pattern: the pattern is the upper half of an
// IEEE binary32, which a double holds exactly.
double bf16_value(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

// ------------------------------------------------------------------ step 1: page metadata

// Elementwise minimum and maximum over the valid tokens [p S, min(p S + S, L))
// of page p, for every page p < ceil(L / S).  keys(t, i) gives channel i of
// token t.  A zero result is stored as +0 (adding +0.0 turns -0 into +0 and
// leaves every other value as it is).
template <class Keys>
void page_minmax(const Keys& keys, int L, int D, int S, double* m, double* M) {
  const int n = (L + S - 1) / S;
  for (int p = 0; p < n; ++p) {
    const int t_end = std::min(p * S + S, L);
    for (int i = 0; i < D; ++i) {
      double lo = keys(p * S, i), hi = lo;
      for (int t = p * S + 1; t < t_end; ++t) {
        const double v = keys(t, i);
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
      m[(size_t)p * D + i] = lo + 0.0;
      M[(size_t)p * D + i] = hi + 0.0;
    }
  }
}

// ------------------------------------------------------------------ step 2: regions and candidates

// The prefix is [0, Pe), the window [Ws, L), the middle region [Pe, Ws).
void regions(int L, int P, int W, int* Pe, int* Ws) {
  *Pe = std::min(P, L);
  *Ws = std::max(0, L - W);
}

// Candidate pages: those meeting the middle region, [c_lo, c_lo + C).
int candidates(int L, int P, int W, int S, int* c_lo) {
  int Pe, Ws;
  regions(L, P, W, &Pe, &Ws);
  *c_lo = Pe / S;
  if (Pe >= Ws) return 0;
  return (Ws + S - 1) / S - Pe / S;
}

// ------------------------------------------------------------------ step 3: Quest bound, group score

// U = sum_i max(q_i m_i, q_i M_i) for one head and one page.
double quest_bound_one(const double* q, const double* m, const double* M, int D) {
  double u = 0.0;
  for (int i = 0; i < D; ++i) u += std::max(q[i] * m[i], q[i] * M[i]);
  return u;
}

// ------------------------------------------------------------------ step 4: top-k selection

struct Scored {
  double s;
  int32_t page;
};

// Larger score first; equal scores (-0 == +0 under ==) by lower page id.
bool ranks_before(const Scored& a, const Scored& b) {
  if (a.s != b.s) return a.s > b.s;
  return a.page < b.page;
}

// The k = min(budget, C) best pages in ascending page order, and the margin
// (s_(k) - s_(k+1)) / |s_(k)| of the sorted scores (infinity when no
// candidate is left out, or nothing is taken).
int select_topk(const double* s, const int32_t* pages, int C, int budget, int32_t* sel, double* margin) {
  std::vector<Scored> v(C);
  for (int i = 0; i < C; ++i) v[i] = Scored{s[i], pages[i]};
  std::sort(v.begin(), v.end(), ranks_before);
  const int k = std::min(budget, C);
  std::vector<int32_t> out(k);
  for (int i = 0; i < k; ++i) out[i] = v[i].page;
  std::sort(out.begin(), out.end());
  for (int i = 0; i < k; ++i) sel[i] = out[i];
  if (margin) {
    if (k == 0 || k >= C) {
      *margin = std::numeric_limits<double>::infinity();
    } else {
      const double a = v[k - 1].s, b = v[k].s;
      *margin = (a - b) / std::max(std::fabs(a), 1e-300);
    }
  }
  return k;
}

// ------------------------------------------------------------------ step 5: attended tokens

// mask[t] = 1 for t in the prefix, the window, or a selected page; 0 otherwise.
void attended_mask(int L, int P, int W, int S, const int32_t* sel, int k, uint8_t* mask) {
  int Pe, Ws;
  regions(L, P, W, &Pe, &Ws);
  for (int t = 0; t < L; ++t) mask[t] = (t < Pe || t >= Ws) ? 1 : 0;
  for (int j = 0; j < k; ++j)
    for (int t = sel[j] * S; t < std::min(sel[j] * S + S, L); ++t) mask[t] = 1;
}

// ------------------------------------------------------------------ step 6: attention

// out[h] = sum_t e^(z_t - mu) v_t / sum_t e^(z_t - mu) over the masked tokens,
// z_t = scale q_h . k_t, mu = max z: two passes in double (not online, not
// split).  keys(t, i) / vals(t, i) give channel i of token t.
template <class Keys, class Vals>
void attend(const double* q, int G, int D, const Keys& keys, const Vals& vals, const uint8_t* mask, int L,
            double scale, double* out) {
  std::vector<int> toks;
  for (int t = 0; t < L; ++t)
    if (mask[t]) toks.push_back(t);
  std::vector<double> z(toks.size());
  for (int h = 0; h < G; ++h) {
    const double* qh = q + (size_t)h * D;
    double mu = -std::numeric_limits<double>::infinity();
    for (size_t j = 0; j < toks.size(); ++j) {
      double dot = 0.0;
      for (int i = 0; i < D; ++i) dot += qh[i] * keys(toks[j], i);
      z[j] = scale * dot;
      mu = std::max(mu, z[j]);
    }
    double den = 0.0;
    std::vector<double> num(D, 0.0);
    for (size_t j = 0; j < toks.size(); ++j) {
      const double w = std::exp(z[j] - mu);
      den += w;
      for (int i = 0; i < D; ++i) num[i] += w * vals(toks[j], i);
    }
    for (int i = 0; i < D; ++i) out[(size_t)h * D + i] = num[i] / den;
  }
}

// Channel i of token t of sequence b, KV head g, read through the page table
// from the plain pool [pool][Hkv][S][D].
struct PoolRows {
  const uint16_t* pool;
  const int32_t* pt_row;
  int hkv, D, S, g;
  double operator()(int t, int i) const {
    const size_t phys = (size_t)pt_row[t / S];
    return bf16_value(pool[((phys * hkv + g) * S + t % S) * D + i]);
  }
};

// A gathered [L][D] array of doubles.
struct ArrayRows {
  const double* a;
  int D;
  double operator()(int t, int i) const { return a[(size_t)t * D + i]; }
};

// ------------------------------------------------------------------ one (sequence, KV head) unit

struct UnitIn {
  const double* q;  // [G][D] of the group
  PoolRows K, V;
  int G, D, S, L, P, W, budget;
  double scale;
  const double* meta;     // [n][2][D] min then max, or null: computed from K
  const int32_t* sel_in;  // attend over these pages instead of the oracle's own selection, or null
  int n_sel_in;
  int dense;              // attend over every token [0, L)
};

struct UnitOut {
  double* scores;   // [max_pages]: the candidates' group scores at their page ids, or null
  int32_t* sel;     // [budget]: the oracle's selection ascending, then -1, or null
  double* margin;   // or null
  double* meta;     // [n][2][D], or null
  double* out;      // [G][D]
  int k;
};

void decode_unit(const UnitIn& in, UnitOut& o) {
  const int D = in.D, S = in.S, L = in.L, G = in.G;
  const int n = (L + S - 1) / S;
  std::vector<double> m_own, M_own;
  const double *m, *M;
  size_t stride = 0;  // doubles between consecutive pages' min rows
  if (in.meta) {
    m = in.meta;
    M = in.meta + D;
    stride = 2 * (size_t)D;
  } else {
    m_own.resize((size_t)n * D);
    M_own.resize((size_t)n * D);
    page_minmax(in.K, L, D, S, m_own.data(), M_own.data());
    m = m_own.data();
    M = M_own.data();
    stride = D;
  }
  if (o.meta)
    for (int p = 0; p < n; ++p)
      for (int i = 0; i < D; ++i) {
        o.meta[((size_t)p * 2 + 0) * D + i] = m[p * stride + i];
        o.meta[((size_t)p * 2 + 1) * D + i] = M[p * stride + i];
      }
  int c_lo;
  const int C = candidates(L, in.P, in.W, S, &c_lo);
  std::vector<double> s(C);
  std::vector<int32_t> pages(C);
  for (int c = 0; c < C; ++c) {
    const int p = c_lo + c;
    pages[c] = p;
    double best = -std::numeric_limits<double>::infinity();
    for (int h = 0; h < G; ++h)
      best = std::max(best, quest_bound_one(in.q + (size_t)h * D, m + p * stride, M + p * stride, D));
    s[c] = best;
    if (o.scores) o.scores[p] = best;
  }
  std::vector<int32_t> sel(std::max(C, 1));
  double margin;
  const int k = select_topk(s.data(), pages.data(), C, in.budget, sel.data(), &margin);
  o.k = k;
  if (o.sel) {
    for (int j = 0; j < k; ++j) o.sel[j] = sel[j];
    for (int j = k; j < in.budget; ++j) o.sel[j] = -1;
  }
  if (o.margin) *o.margin = margin;
  std::vector<uint8_t> mask(L);
  if (in.dense) {
    std::fill(mask.begin(), mask.end(), 1);
  } else if (in.sel_in) {
    attended_mask(L, in.P, in.W, S, in.sel_in, in.n_sel_in, mask.data());
  } else {
    attended_mask(L, in.P, in.W, S, sel.data(), k, mask.data());
  }
  attend(in.q, G, D, in.K, in.V, mask.data(), L, in.scale, o.out);
}

}  // namespace

extern "C" {

// ---------------------------------------------------------------- single steps on arrays

/* Exact values of n bf16 bit patterns.  Pinned by fixed bit patterns whose
 * values the bf16 format defines (tests/golden/bf16_patterns.json). */
void ora_bf16_decode(const uint16_t* bits, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_value(bits[i]);
}

/* Keys (or values) of tokens [0, L) of sequence b, KV head g, gathered through
 * the page table row: out [L][D].  Pinned by page-table permutation invariance
 * of the metadata and of every later result. */
void ora_gather(const uint16_t* pool, const int32_t* pt_row, int hkv, int D, int S, int g, int L, double* out) {
  const PoolRows r{pool, pt_row, hkv, D, S, g};
  for (int t = 0; t < L; ++t)
    for (int i = 0; i < D; ++i) out[(size_t)t * D + i] = r(t, i);
}

/* Per-page elementwise min and max of keys [L][D] over each page's valid
 * tokens: m, M [ceil(L/S)][D].  Pinned by brute-force containment and
 * attainment, the partial last page, the zero sign, and append-vs-rebuild. */
void ora_page_minmax(const double* keys, int L, int D, int S, double* m, double* M) {
  page_minmax(ArrayRows{keys, D}, L, D, S, m, M);
}

/* Number of candidate pages of a sequence of length L, and the first one.
 * Pinned by the per-page brute force of which pages meet the middle region. */
int ora_candidates(int L, int P, int W, int S, int* c_lo) { return candidates(L, P, W, S, c_lo); }

/* U[h][c] = sum_i max(q[h][i] m[c][i], q[h][i] M[c][i]) for G heads and C
 * pages.  Pinned by the brute-force bound invariant, tight single-token and
 * constant-page cases, the K = 0, q >= 0 and q <= 0 closed forms and the
 * hand-worked fixture. */
void ora_quest_bound(const double* q, const double* m, const double* M, int G, int C, int D, double* U) {
  for (int h = 0; h < G; ++h)
    for (int c = 0; c < C; ++c)
      U[(size_t)h * C + c] = quest_bound_one(q + (size_t)h * D, m + (size_t)c * D, M + (size_t)c * D, D);
}

/* s[c] = max_h U[h][c]: the group's score of page c.  The aggregation is a
 * reading (parity unpinned by the pages); pinned as an operation by the
 * hand-worked fixture and the every-head bound test. */
void ora_group_score(const double* U, int G, int C, double* s) {
  for (int c = 0; c < C; ++c) {
    double best = -std::numeric_limits<double>::infinity();
    for (int h = 0; h < G; ++h) best = std::max(best, U[(size_t)h * C + c]);
    s[c] = best;
  }
}

/* Top-k selection: writes the k = min(budget, C) selected pages ascending and
 * returns k.  Pinned by a rank-counting brute force with forced ties and
 * signed zeros, the all-equal closed form and the hand-worked fixtures. */
int ora_select_topk(const double* s, const int32_t* pages, int C, int budget, int32_t* sel) {
  return select_topk(s, pages, C, budget, sel, nullptr);
}

/* Margin (s_(k) - s_(k+1)) / |s_(k)| of the scores sorted in decreasing
 * order, k = min(budget, C); infinity when nothing is left out or taken.
 * Pinned by the hand-worked fixture (tests/golden/handworked.json). */
double ora_selection_margin(const double* s, int C, int budget) {
  std::vector<int32_t> pages(C), sel(std::max(C, 1));
  for (int i = 0; i < C; ++i) pages[i] = i;
  double margin;
  select_topk(s, pages.data(), C, budget, sel.data(), &margin);
  return margin;
}

/* Attended-token mask over [0, L).  Pinned by the per-token brute force, the
 * count closed form and the hand-worked fixture. */
void ora_attended_mask(int L, int P, int W, int S, const int32_t* sel, int k, uint8_t* mask) {
  attended_mask(L, P, W, S, sel, k, mask);
}

/* Two-pass softmax attention of G heads q [G][D] over the masked tokens of
 * K, V [L][D]: out [G][D].  Pinned by torch CPU scaled_dot_product_attention
 * in float64, the constant-V and equal-logit closed forms and the hand-worked
 * fixture. */
void ora_attend(const double* q, const double* K, const double* V, const uint8_t* mask, int L, int G, int D,
                double scale, double* out) {
  attend(q, G, D, ArrayRows{K, D}, ArrayRows{V, D}, mask, L, scale, out);
}

// ---------------------------------------------------------------- whole units, from the pool

/* Page metadata of every (sequence, KV head) unit, from the pool:
 * meta [B][Hkv][max_pages][2][D] (pages past a sequence's length untouched),
 * computed on nthreads threads over units. */
void ora_build_meta(const uint16_t* k_pool, const int32_t* page_table, const int32_t* seq_lens, int B, int hkv, int D,
                    int S, int max_pages, double* meta, int nthreads) {
  const int units = B * hkv;
  auto work = [&](int u) {
    const int b = u / hkv, g = u % hkv;
    const int L = seq_lens[b], n = (L + S - 1) / S;
    std::vector<double> m((size_t)n * D), M((size_t)n * D);
    page_minmax(PoolRows{k_pool, page_table + (size_t)b * max_pages, hkv, D, S, g}, L, D, S, m.data(), M.data());
    double* dst = meta + (size_t)u * max_pages * 2 * D;
    for (int p = 0; p < n; ++p) {
      memcpy(dst + ((size_t)p * 2) * D, m.data() + (size_t)p * D, D * sizeof(double));
      memcpy(dst + ((size_t)p * 2 + 1) * D, M.data() + (size_t)p * D, D * sizeof(double));
    }
  };
  const int nt = std::max(1, std::min(nthreads, units));
  std::vector<std::thread> th;
  for (int w = 0; w < nt; ++w)
    th.emplace_back([&, w] {
      for (int u = w; u < units; u += nt) work(u);
    });
  for (auto& t : th) t.join();
}

/* The decode step of the listed (sequence b, KV head g) units, each on its
 * own, spread over nthreads threads (units[2 j], units[2 j + 1]):
 *   q_bits      bf16 [B][Hq][D]; the group of KV head g is query heads
 *               g G .. g G + G - 1
 *   k_pool, v_pool  bf16 [pool][Hkv][S][D]; page_table [B][max_pages]
 *   meta        [B][Hkv][max_pages][2][D] from ora_build_meta, or null to
 *               compute each unit's metadata from the pool
 *   sel_in      [n_units][sel_stride] pages to attend instead of the
 *               oracle's own selection (-1 ends a row early), or null
 *   dense       1: attend to every token [0, L) (full attention)
 * Outputs per listed unit j (each may be null but out):
 *   scores [j][max_pages] candidates' group scores at their page ids (other
 *   entries untouched); sel [j][budget] the oracle's own selection, ascending,
 *   -1 padded; margin [j]; k [j]; meta_out [j][max_pages][2][D] (pages past the
 *   length untouched); out [j][G][D].
 * Returns 0, or -1 on an inconsistent argument. */
int ora_decode_units(const uint16_t* q_bits, const uint16_t* k_pool, const uint16_t* v_pool, const int32_t* page_table,
                     const int32_t* seq_lens, int B, int hq, int hkv, int D, int S, int max_pages, int prefix,
                     int window, int budget, double scale, const double* meta, const int32_t* units, int n_units,
                     const int32_t* sel_in, int sel_stride, int dense, double* scores, int32_t* sel, double* margin,
                     int32_t* k_out, double* meta_out, double* out, int nthreads) {
  if (hkv < 1 || hq % hkv != 0 || D < 1 || S < 1 || n_units < 0 || budget < 0) return -1;
  const int G = hq / hkv;
  for (int j = 0; j < n_units; ++j) {
    const int b = units[2 * j], g = units[2 * j + 1];
    if (b < 0 || b >= B || g < 0 || g >= hkv || seq_lens[b] < 1 || (seq_lens[b] + S - 1) / S > max_pages) return -1;
  }
  auto work = [&](int j) {
    const int b = units[2 * j], g = units[2 * j + 1];
    std::vector<double> q((size_t)G * D);
    for (int h = 0; h < G; ++h)
      for (int i = 0; i < D; ++i) q[(size_t)h * D + i] = bf16_value(q_bits[((size_t)b * hq + g * G + h) * D + i]);
    const int32_t* pt_row = page_table + (size_t)b * max_pages;
    UnitIn in{q.data(),
              PoolRows{k_pool, pt_row, hkv, D, S, g},
              PoolRows{v_pool, pt_row, hkv, D, S, g},
              G, D, S, seq_lens[b], prefix, window, budget, scale,
              meta ? meta + ((size_t)b * hkv + g) * max_pages * 2 * D : nullptr,
              nullptr, 0, dense};
    int n_sel = 0;
    if (sel_in) {
      in.sel_in = sel_in + (size_t)j * sel_stride;
      while (n_sel < sel_stride && in.sel_in[n_sel] >= 0) ++n_sel;
      in.n_sel_in = n_sel;
    }
    UnitOut o{scores ? scores + (size_t)j * max_pages : nullptr, sel ? sel + (size_t)j * budget : nullptr,
              margin ? margin + j : nullptr, meta_out ? meta_out + (size_t)j * max_pages * 2 * D : nullptr,
              out + (size_t)j * G * D, 0};
    decode_unit(in, o);
    if (k_out) k_out[j] = o.k;
  };
  const int nt = std::max(1, std::min(nthreads, std::max(n_units, 1)));
  std::vector<std::thread> th;
  for (int w = 0; w < nt; ++w)
    th.emplace_back([&, w] {
      for (int j = w; j < n_units; j += nt) work(j);
    });
  for (auto& t : th) t.join();
  return 0;
}

}  // extern "C"
