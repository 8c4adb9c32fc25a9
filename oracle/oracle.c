/*
 * CPU oracle for filter-first constrained beam search over semantic IDs.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It is deliberately plain and slow: double precision,
 * library qsort, binary search, no blocking or fusion.
 *
 * What it computes (ZeroGR: Filtering-First Constrained Decoding for
 * Generative Recommendation, paper-daily page):
 *   - "what problem" section: a beam's legal next tokens are exactly those
 *     that still lead to a real catalog item (worked example: if the only
 *     items under 3-5 are 3-5-1 and 3-5-4, the legal set after 3-5 is {1, 4}).
 *   - "overall pipeline" section: per step, read each beam's legal tokens,
 *     score only those (z_v = W_t[v] . h), apply log-softmax over the legal
 *     tokens only, add the result to the beam's cumulative log-prob and pick
 *     the next beams by the new cumulative value.
 *   - "does filter-first change results" section: the softmax denominator
 *     covers the legal tokens only.
 *   - "why slice the index per step" section: the row of a beam in the step-t
 *     table is its length-(t-1) prefix; rows are numbered here by the
 *     lexicographic rank of that prefix among all distinct prefixes of that
 *     length, and the item id of a full SID is its lexicographic rank (the
 *     last step stores no item ids, so the position is the id).
 *
 * The trie is held as its node sets per depth: depth_keys[t] lists the
 * distinct length-t prefixes in lexicographic order (each packed into one
 * 64-bit integer, `bits` bits per token, so numeric order equals
 * lexicographic order for prefixes of one length).  The children of a
 * depth-(t-1) node p are the depth-t nodes whose key shifted right by `bits`
 * equals p: one contiguous run, found by binary search, already in token
 * order.  A node's number is its index in depth_keys[t].
 *
 * Two more modes, for comparisons only (orc_step_mode): score-first, where
 * the softmax denominator covers the whole codebook before the illegal
 * tokens are dropped ("does filter-first change results" section), and
 * unconstrained search, where every codebook token is a candidate ("is it
 * really better" section).
 *
 * Selection: every candidate of a request is ranked by (cumulative score
 * descending, beam index ascending, token ascending) and the first K are kept
 * in that order; fewer than K candidates keep them all.  The fixed tie-break
 * is the reading taken where the pages say nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MAX_L 8

typedef struct {
  int32_t L, V, bits;
  int64_t N;
  uint64_t* depth_keys[ORC_MAX_L + 1]; /* depth t = 0..L */
  int64_t depth_count[ORC_MAX_L + 1];
  int64_t* input_row_of_item; /* [N]: catalog row of the item with lexicographic rank i */
} orc_catalog;

typedef struct {
  uint64_t key;
  int64_t row;
} orc_keyed_row;

static int cmp_keyed_row(const void* a, const void* b) {
  const orc_keyed_row* x = (const orc_keyed_row*)a;
  const orc_keyed_row* y = (const orc_keyed_row*)b;
  if (x->key < y->key) return -1;
  if (x->key > y->key) return 1;
  return (x->row < y->row) ? -1 : (x->row > y->row);
}

static uint64_t pack_prefix(const orc_catalog* c, const int32_t* tok, int32_t len) {
  uint64_t k = 0;
  for (int32_t i = 0; i < len; ++i) k = (k << c->bits) | (uint64_t)(uint32_t)tok[i];
  return k;
}

/* first index in a[0..n) with a[i] >= x */
static int64_t lower_bound_u64(const uint64_t* a, int64_t n, uint64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (a[mid] < x)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

void orc_free(orc_catalog* c) {
  if (!c) return;
  for (int t = 0; t <= ORC_MAX_L; ++t) free(c->depth_keys[t]);
  free(c->input_row_of_item);
  free(c);
}

/*
 * Build the per-depth node sets from the catalog sids[N][L].
 * Returns 0 and *out on success; 1 bad arguments; 2 a token outside [0, V);
 * 3 two catalog rows with the same SID; 4 out of memory.
 */
int orc_build(const int32_t* sids, int64_t N, int32_t L, int32_t V, orc_catalog** out) {
  if (!sids || !out || N < 1 || L < 1 || L > ORC_MAX_L || V < 2) return 1;
  int bits = 0;
  while ((1LL << bits) < V) ++bits;
  if ((int64_t)bits * L > 63) return 1;
  orc_catalog* c = (orc_catalog*)calloc(1, sizeof(orc_catalog));
  if (!c) return 4;
  c->L = L;
  c->V = V;
  c->bits = bits;
  c->N = N;
  orc_keyed_row* kr = (orc_keyed_row*)malloc((size_t)N * sizeof(orc_keyed_row));
  c->input_row_of_item = (int64_t*)malloc((size_t)N * sizeof(int64_t));
  if (!kr || !c->input_row_of_item) {
    free(kr);
    orc_free(c);
    return 4;
  }
  for (int64_t i = 0; i < N; ++i) {
    for (int32_t l = 0; l < L; ++l) {
      const int32_t v = sids[i * L + l];
      if (v < 0 || v >= V) {
        free(kr);
        orc_free(c);
        return 2;
      }
    }
    kr[i].key = pack_prefix(c, sids + i * L, L);
    kr[i].row = i;
  }
  qsort(kr, (size_t)N, sizeof(orc_keyed_row), cmp_keyed_row);
  for (int64_t i = 1; i < N; ++i) {
    if (kr[i].key == kr[i - 1].key) {
      free(kr);
      orc_free(c);
      return 3;
    }
  }
  for (int64_t i = 0; i < N; ++i) c->input_row_of_item[i] = kr[i].row;
  /* depth t node set: distinct values of key >> (bits * (L - t)), in sorted order */
  for (int32_t t = 0; t <= L; ++t) {
    const int shift = bits * (L - t);
    uint64_t* nodes = (uint64_t*)malloc((size_t)N * sizeof(uint64_t));
    if (!nodes) {
      free(kr);
      orc_free(c);
      return 4;
    }
    int64_t n = 0;
    for (int64_t i = 0; i < N; ++i) {
      const uint64_t p = (shift >= 64) ? 0 : (kr[i].key >> shift);
      if (n == 0 || nodes[n - 1] != p) nodes[n++] = p;
    }
    c->depth_keys[t] = nodes;
    c->depth_count[t] = n;
  }
  free(kr);
  *out = c;
  return 0;
}

int64_t orc_count(const orc_catalog* c, int32_t depth) {
  if (!c || depth < 0 || depth > c->L) return -1;
  return c->depth_count[depth];
}

/* catalog row of the item whose lexicographic rank (item id) is `item` */
int64_t orc_input_row(const orc_catalog* c, int64_t item) {
  if (!c || item < 0 || item >= c->N) return -1;
  return c->input_row_of_item[item];
}

/* Node number of a length-len prefix (its rank among distinct length-len prefixes), or -1. */
int64_t orc_node(const orc_catalog* c, const int32_t* prefix, int32_t len) {
  if (!c || len < 0 || len > c->L) return -1;
  for (int32_t i = 0; i < len; ++i)
    if (prefix[i] < 0 || prefix[i] >= c->V) return -1;
  const uint64_t k = pack_prefix(c, prefix, len);
  const int64_t i = lower_bound_u64(c->depth_keys[len], c->depth_count[len], k);
  return (i < c->depth_count[len] && c->depth_keys[len][i] == k) ? i : -1;
}

/*
 * Legal next tokens after a length-len prefix (the filter): the last tokens of
 * the depth-(len+1) nodes under it, ascending.  Writes at most cap tokens and
 * returns the full count (0 when the prefix is not in the catalog).
 */
int64_t orc_legal(const orc_catalog* c, const int32_t* prefix, int32_t len, int32_t* tokens, int64_t cap) {
  if (!c || len < 0 || len >= c->L) return -1;
  if (orc_node(c, prefix, len) < 0) return 0;
  const uint64_t p = pack_prefix(c, prefix, len);
  const uint64_t* a = c->depth_keys[len + 1];
  const int64_t n = c->depth_count[len + 1];
  const int64_t lo = lower_bound_u64(a, n, p << c->bits);
  const int64_t hi = lower_bound_u64(a, n, (p + 1) << c->bits);
  const uint64_t mask = (c->bits >= 64) ? ~0ULL : ((1ULL << c->bits) - 1ULL);
  for (int64_t i = lo; i < hi && i - lo < cap; ++i) tokens[i - lo] = (int32_t)(a[i] & mask);
  return hi - lo;
}

typedef struct {
  double score;
  int32_t beam;
  int32_t token;
} orc_cand;

static int cmp_cand(const void* a, const void* b) {
  const orc_cand* x = (const orc_cand*)a;
  const orc_cand* y = (const orc_cand*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  if (x->beam != y->beam) return (x->beam < y->beam) ? -1 : 1;
  return (x->token < y->token) ? -1 : (x->token > y->token);
}

/*
 * One decode step t (1-based) of one request, in one of three modes:
 *   ORC_FILTER_FIRST (0)  the method: score only the legal tokens, softmax
 *                         over the legal tokens only ("overall pipeline").
 *   ORC_SCORE_FIRST (1)   the order the method replaces: every codebook token
 *                         is scored and the softmax denominator covers all V
 *                         of them; only then are the illegal tokens dropped
 *                         ("does filter-first change results" section).
 *   ORC_UNCONSTRAINED (2) the speed reference: softmax over all V tokens and
 *                         every token is a candidate; the catalog is not
 *                         consulted, so a code need not be a real item ("is
 *                         it really better" section).
 *   W      [V][d]   step-t weights (values as stored, widened to float)
 *   prefix [k_in][t-1] each beam's tokens so far; cum [k_in] its cumulative
 *          log-prob; h [k_in][d] its hidden vector.  Beams are given in rank
 *          order; a beam with cum = -inf is dead and contributes nothing.
 * All candidates are written to cand_* (beam, token, log-prob, new score) in
 * beam order then token order; at most cap of them; *n_cand gets the full count.
 * The selection (at most K) goes to sel_* in rank order with the node number
 * of the extended prefix (the next row; at t = L the item id; -1 when the
 * extended prefix is not in the catalog, which only the unconstrained mode
 * produces); *n_sel its size.
 * Returns 0, or 1 on bad arguments, 4 out of memory.
 */
int orc_step_mode(const orc_catalog* c, int32_t mode, int32_t t, const float* W, int32_t d,
                  int32_t k_in, const int32_t* prefix, const double* cum, const float* h,
                  int32_t K, int64_t cap, int32_t* cand_beam, int32_t* cand_token,
                  double* cand_logp, double* cand_score, int64_t* n_cand, int32_t* sel_beam,
                  int32_t* sel_token, double* sel_score, int64_t* sel_node, int32_t* n_sel) {
  if (!c || t < 1 || t > c->L || !W || d < 1 || k_in < 1 || !cum || !h || K < 1) return 1;
  if (mode < 0 || mode > 2) return 1;
  if (t > 1 && !prefix) return 1;
  const int32_t plen = t - 1;
  int32_t* legal = (int32_t*)malloc((size_t)c->V * sizeof(int32_t));
  double* z = (double*)malloc((size_t)c->V * sizeof(double));
  double* lp = (double*)malloc((size_t)c->V * sizeof(double));
  int64_t total = 0;
  for (int32_t k = 0; k < k_in; ++k) {
    if (isinf(cum[k]) && cum[k] < 0) continue;
    if (mode != 0) {  /* at most V candidates per beam */
      total += c->V;
      continue;
    }
    const int64_t n = orc_legal(c, prefix ? prefix + (int64_t)k * plen : NULL, plen, legal, c->V);
    total += (n > 0) ? n : 0;
  }
  orc_cand* all = (orc_cand*)malloc((size_t)(total > 0 ? total : 1) * sizeof(orc_cand));
  int32_t* ext = (int32_t*)malloc((size_t)(t + 1) * sizeof(int32_t));
  if (!legal || !z || !lp || !all || !ext) {
    free(legal);
    free(z);
    free(lp);
    free(all);
    free(ext);
    return 4;
  }
  int64_t m_all = 0;
  for (int32_t k = 0; k < k_in; ++k) {
    if (isinf(cum[k]) && cum[k] < 0) continue;
    const int32_t* pk = prefix ? prefix + (int64_t)k * plen : NULL;
    const float* hk = h + (int64_t)k * d;
    int64_t n;
    if (mode == 0) {
      n = orc_legal(c, pk, plen, legal, c->V);
      if (n <= 0) continue;
      /* score only the legal tokens */
      double zmax = -INFINITY;
      for (int64_t j = 0; j < n; ++j) {
        const float* w = W + (int64_t)legal[j] * d;
        double acc = 0.0;
        for (int32_t i = 0; i < d; ++i) acc += (double)w[i] * (double)hk[i];
        z[j] = acc;
        if (acc > zmax) zmax = acc;
      }
      /* log-softmax over the legal tokens only */
      double s = 0.0;
      for (int64_t j = 0; j < n; ++j) s += exp(z[j] - zmax);
      const double lse = zmax + log(s);
      for (int64_t j = 0; j < n; ++j) lp[j] = z[j] - lse;
    } else {
      /* score every token of the codebook: z[v] = W[v] . h */
      double zmax_all = -INFINITY;
      for (int32_t v = 0; v < c->V; ++v) {
        const float* wv = W + (int64_t)v * d;
        double dot = 0.0;
        for (int32_t i = 0; i < d; ++i) dot += (double)wv[i] * (double)hk[i];
        z[v] = dot;
        if (dot > zmax_all) zmax_all = dot;
      }
      /* log-softmax over all V tokens */
      double s_all = 0.0;
      for (int32_t v = 0; v < c->V; ++v) s_all += exp(z[v] - zmax_all);
      const double lse_all = zmax_all + log(s_all);
      if (mode == 1) {
        /* then drop the illegal tokens */
        n = orc_legal(c, pk, plen, legal, c->V);
        if (n <= 0) continue;
      } else {
        n = c->V;
        for (int32_t v = 0; v < c->V; ++v) legal[v] = v;
      }
      for (int64_t j = 0; j < n; ++j) lp[j] = z[legal[j]] - lse_all;
    }
    for (int64_t j = 0; j < n; ++j) {
      const double logp = lp[j];
      const double score = cum[k] + logp;
      if (m_all < cap) {
        if (cand_beam) cand_beam[m_all] = k;
        if (cand_token) cand_token[m_all] = legal[j];
        if (cand_logp) cand_logp[m_all] = logp;
        if (cand_score) cand_score[m_all] = score;
      }
      all[m_all].score = score;
      all[m_all].beam = k;
      all[m_all].token = legal[j];
      ++m_all;
    }
  }
  if (n_cand) *n_cand = m_all;
  qsort(all, (size_t)m_all, sizeof(orc_cand), cmp_cand);
  const int32_t keep = (m_all < K) ? (int32_t)m_all : K;
  for (int32_t r = 0; r < keep; ++r) {
    if (sel_beam) sel_beam[r] = all[r].beam;
    if (sel_token) sel_token[r] = all[r].token;
    if (sel_score) sel_score[r] = all[r].score;
    if (sel_node) {
      for (int32_t i = 0; i < plen; ++i) ext[i] = prefix[(int64_t)all[r].beam * plen + i];
      ext[plen] = all[r].token;
      sel_node[r] = orc_node(c, ext, t);
    }
  }
  if (n_sel) *n_sel = keep;
  free(legal);
  free(z);
  free(lp);
  free(all);
  free(ext);
  return 0;
}

/* The method's step (filter-first). */
int orc_step(const orc_catalog* c, int32_t t, const float* W, int32_t d, int32_t k_in,
             const int32_t* prefix, const double* cum, const float* h, int32_t K, int64_t cap,
             int32_t* cand_beam, int32_t* cand_token, double* cand_logp, double* cand_score,
             int64_t* n_cand, int32_t* sel_beam, int32_t* sel_token, double* sel_score,
             int64_t* sel_node, int32_t* n_sel) {
  return orc_step_mode(c, 0, t, W, d, k_in, prefix, cum, h, K, cap, cand_beam, cand_token,
                       cand_logp, cand_score, n_cand, sel_beam, sel_token, sel_score, sel_node,
                       n_sel);
}
