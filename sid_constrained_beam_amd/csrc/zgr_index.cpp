// Host construction and HBM upload of the per-step filter index.
//
// ZeroGR description, "why slice the index per step": decoding step t only
// asks which tokens may follow a length-(t-1) prefix, so the index is one
// table per step.  A row is a length-(t-1) prefix; it records the legal next
// tokens and, for each, the row of the extended prefix in table t+1.  Dense
// tables (many legal tokens) keep a bitmap whose columns are in codebook
// order, the order of the full projection's output; sparse tables keep the
// sorted legal tokens, and an entry's position in the array is its next-step
// row, so no successor array and no item ids are stored (second ZeroGR
// description, ai-papers-daily digest).
//
// Rows of table t are numbered by the lexicographic rank of their prefix, so
// an entry's next row is simply its index in the concatenation of all rows'
// entries (CSR order) and the last table's entry index is the item id.  A
// dense row's entries are counted by popcount: next row = row_ptr[r] + number
// of set bits below the token.  The per-step format is picked by size unless
// forced ("sparse or dense per step by legal-token density, to save memory").
#include <algorithm>
#include <cstring>
#include <mutex>
#include <thread>
#include <unordered_map>

#include "zgr_internal.h"

namespace {

int hw_threads() {
  const unsigned n = std::thread::hardware_concurrency();
  return (int)std::max(1u, std::min(n, 16u));
}

template <class F>
void par_chunks(int64_t n, F&& fn) {
  const int T = (n < (1 << 16)) ? 1 : hw_threads();
  if (T == 1) {
    fn(0, n, 0);
    return;
  }
  std::vector<std::thread> th;
  const int64_t chunk = (n + T - 1) / T;
  for (int t = 0; t < T; ++t) {
    const int64_t lo = t * chunk, hi = std::min(n, lo + chunk);
    if (lo >= hi) break;
    th.emplace_back([&fn, lo, hi, t] { fn(lo, hi, t); });
  }
  for (auto& x : th) x.join();
}

// Stable LSD radix sort of (key, original row) by key, skipping digits that are
// zero in every key.
void sort_keys(std::vector<uint64_t>& key, std::vector<int32_t>& row) {
  const int64_t n = (int64_t)key.size();
  uint64_t any = 0;
  for (int64_t i = 0; i < n; ++i) any |= key[i];
  std::vector<uint64_t> k2(n);
  std::vector<int32_t> r2(n);
  const int T = (n < (1 << 16)) ? 1 : hw_threads();
  const int64_t chunk = (n + T - 1) / T;
  std::vector<int64_t> hist((size_t)T * 256);
  for (int shift = 0; shift < 64; shift += 8) {
    if (((any >> shift) & 0xFF) == 0) continue;
    std::fill(hist.begin(), hist.end(), 0);
    auto count = [&](int t) {
      const int64_t lo = t * chunk, hi = std::min(n, lo + chunk);
      int64_t* h = &hist[(size_t)t * 256];
      for (int64_t j = lo; j < hi; ++j) ++h[(key[j] >> shift) & 0xFF];
    };
    auto scatter = [&](int t) {
      const int64_t lo = t * chunk, hi = std::min(n, lo + chunk);
      int64_t* h = &hist[(size_t)t * 256];
      for (int64_t j = lo; j < hi; ++j) {
        const int64_t p = h[(key[j] >> shift) & 0xFF]++;
        k2[p] = key[j];
        r2[p] = row[j];
      }
    };
    if (T == 1) {
      count(0);
    } else {
      std::vector<std::thread> th;
      for (int t = 0; t < T; ++t) th.emplace_back(count, t);
      for (auto& x : th) x.join();
    }
    int64_t acc = 0;
    for (int b = 0; b < 256; ++b)
      for (int t = 0; t < T; ++t) {
        int64_t& h = hist[(size_t)t * 256 + b];
        const int64_t c = h;
        h = acc;
        acc += c;
      }
    if (T == 1) {
      scatter(0);
    } else {
      std::vector<std::thread> th;
      for (int t = 0; t < T; ++t) th.emplace_back(scatter, t);
      for (auto& x : th) x.join();
    }
    key.swap(k2);
    row.swap(r2);
  }
}

std::mutex g_live_mu;
std::unordered_map<const zgr_index*, uint64_t>& live_map() {
  static std::unordered_map<const zgr_index*, uint64_t> m;
  return m;
}

}  // namespace

namespace zgr {
void index_register(const zgr_index* idx, uint64_t generation) {
  std::lock_guard<std::mutex> g(g_live_mu);
  live_map()[idx] = generation;
}
void index_unregister(const zgr_index* idx) {
  std::lock_guard<std::mutex> g(g_live_mu);
  live_map().erase(idx);
}
bool index_alive(const zgr_index* idx, uint64_t generation) {
  std::lock_guard<std::mutex> g(g_live_mu);
  auto it = live_map().find(idx);
  return it != live_map().end() && it->second == generation;
}
}  // namespace zgr

extern "C" int32_t zgr_index_build_host(const int32_t* sids, int64_t N, int32_t L, int32_t V,
                                        const int32_t* fmt, int64_t* rank_of_input,
                                        zgr_index** out) {
  using namespace zgr;
  if (!sids || !out) return fail(ZGR_E_ARG, "zgr_index_build_host: null sids or out");
  *out = nullptr;
  if (N < 1) return fail(ZGR_E_ARG, "zgr_index_build_host: N must be >= 1");
  if (N >= INT32_MAX) return fail(ZGR_E_SHAPE, "zgr_index_build_host: N must be < 2^31 - 1");
  if (L < 1 || L > kMaxL) return fail(ZGR_E_ARG, "zgr_index_build_host: L must be in [1, 8]");
  if (V < 2 || V > 65536) return fail(ZGR_E_ARG, "zgr_index_build_host: V must be in [2, 65536]");
  int bits = 0;
  while ((1 << bits) < V) ++bits;
  if (bits * L > 64) return fail(ZGR_E_SHAPE, "zgr_index_build_host: ceil(log2 V) * L > 64");
  if (fmt) {
    for (int l = 0; l < L; ++l)
      if (fmt[l] < ZGR_FMT_AUTO || fmt[l] > ZGR_FMT_SPARSE)
        return fail(ZGR_E_ARG, "zgr_index_build_host: fmt[t] must be AUTO, DENSE or SPARSE");
  }
  std::vector<uint64_t> key;
  std::vector<int32_t> row;
  try {
    key.resize(N);
    row.resize(N);
  } catch (...) {
    return fail(ZGR_E_NOMEM, "zgr_index_build_host: host allocation");
  }
  std::vector<int64_t> bad(hw_threads() + 1, -1);
  par_chunks(N, [&](int64_t lo, int64_t hi, int t) {
    for (int64_t i = lo; i < hi; ++i) {
      uint64_t k = 0;
      for (int l = 0; l < L; ++l) {
        const int32_t v = sids[i * L + l];
        if ((v < 0 || v >= V) && bad[t] < 0) bad[t] = i;
        k = (k << bits) | (uint64_t)(uint32_t)v;
      }
      key[i] = k;
      row[i] = (int32_t)i;
    }
  });
  for (int64_t b : bad)
    if (b >= 0)
      return fail(ZGR_E_TOKEN_RANGE, "zgr_index_build_host: catalog row " + std::to_string(b) +
                                         " has a token outside [0, V)");
  sort_keys(key, row);
  for (int64_t i = 1; i < N; ++i)
    if (key[i] == key[i - 1])
      return fail(ZGR_E_DUP_SID, "zgr_index_build_host: catalog rows " + std::to_string(row[i - 1]) +
                                     " and " + std::to_string(row[i]) + " share one SID");
  if (rank_of_input)
    par_chunks(N, [&](int64_t lo, int64_t hi, int) {
      for (int64_t i = lo; i < hi; ++i) rank_of_input[row[i]] = i;
    });
  row.clear();
  row.shrink_to_fit();

  zgr_index* idx = new (std::nothrow) zgr_index();
  if (!idx) return fail(ZGR_E_NOMEM, "zgr_index_build_host: host allocation");
  idx->L = L;
  idx->V = V;
  idx->bits = bits;
  idx->N = N;
  const uint64_t tmask = (1ULL << bits) - 1ULL;
  auto token_at = [&](uint64_t k, int l) { return (uint32_t)((k >> (bits * (L - 1 - l))) & tmask); };
  // First level at which key i differs from key i-1 (0 for the first key).
  auto first_diff = [&](int64_t i) -> int {
    if (i == 0) return 0;
    const uint64_t x = key[i] ^ key[i - 1];
    const int msb = 63 - __builtin_clzll(x);
    return L - 1 - msb / bits;
  };
  // Table l (step l+1): rows = distinct length-l prefixes, entries = distinct length-(l+1) prefixes.
  int64_t rows[kMaxL] = {0}, nnz[kMaxL] = {0};
  rows[0] = 1;
  for (int64_t i = 0; i < N; ++i) {
    const int f = first_diff(i);
    for (int l = f; l < L; ++l) {
      ++nnz[l];
      if (l >= f + 1) ++rows[l];
    }
  }
  try {
    for (int l = 0; l < L; ++l) {
      idx->host[l].rows = rows[l];
      idx->host[l].nnz = nnz[l];
      idx->host[l].row_ptr.assign(rows[l] + 1, 0);
      idx->host[l].tok.resize(nnz[l]);
    }
  } catch (...) {
    delete idx;
    return fail(ZGR_E_NOMEM, "zgr_index_build_host: host allocation");
  }
  int64_t e[kMaxL] = {0}, r[kMaxL] = {0};
  r[0] = 1;  // the single root row of table 1 starts at entry 0
  for (int64_t i = 0; i < N; ++i) {
    const int f = first_diff(i);
    for (int l = f; l < L; ++l) {
      HostTable& h = idx->host[l];
      if (l >= f + 1) h.row_ptr[r[l]++] = (int32_t)e[l];
      h.tok[e[l]++] = (uint16_t)token_at(key[i], l);
    }
  }
  key.clear();
  key.shrink_to_fit();
  const int32_t words = (V + 31) / 32;
  for (int l = 0; l < L; ++l) {
    HostTable& h = idx->host[l];
    h.row_ptr[h.rows] = (int32_t)h.nnz;
    int32_t mx = 0;
    for (int64_t q = 0; q < h.rows; ++q) mx = std::max(mx, h.row_ptr[q + 1] - h.row_ptr[q]);
    h.max_legal = mx;
    const int64_t dense_bytes = h.rows * (int64_t)words * 4;
    const int64_t sparse_bytes = h.nnz * 2;
    const int32_t want = fmt ? fmt[l] : ZGR_FMT_AUTO;
    h.fmt = (want == ZGR_FMT_AUTO) ? (dense_bytes < sparse_bytes ? ZGR_FMT_DENSE : ZGR_FMT_SPARSE)
                                   : want;
    h.stride = (h.fmt == ZGR_FMT_DENSE) ? V : mx;
    if (h.fmt == ZGR_FMT_DENSE) {
      try {
        h.bits.assign((size_t)h.rows * words, 0u);
      } catch (...) {
        delete idx;
        return fail(ZGR_E_NOMEM, "zgr_index_build_host: host allocation");
      }
      par_chunks(h.rows, [&](int64_t lo, int64_t hi, int) {
        for (int64_t q = lo; q < hi; ++q)
          for (int32_t j = h.row_ptr[q]; j < h.row_ptr[q + 1]; ++j)
            h.bits[q * words + h.tok[j] / 32] |= 1u << (h.tok[j] % 32);
      });
    }
  }
  static uint64_t gen_counter = 0;
  idx->generation = __atomic_add_fetch(&gen_counter, 1, __ATOMIC_RELAXED);
  index_register(idx, idx->generation);
  *out = idx;
  return ZGR_OK;
}

extern "C" int32_t zgr_index_to_device(zgr_index* idx, void* stream) {
  using namespace zgr;
  if (!idx) return fail(ZGR_E_ARG, "zgr_index_to_device: null index");
  if (idx->on_device) return fail(ZGR_E_STATE, "zgr_index_to_device: index already on device");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipGetDevice(&idx->device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  auto upload = [&](const void* src, size_t bytes, void** dst) -> int32_t {
    *dst = nullptr;
    if (bytes == 0) return ZGR_OK;
    hipError_t err = hipMalloc(dst, bytes);
    if (err != hipSuccess) {
      *dst = nullptr;
      (void)hipGetLastError();
      return fail(ZGR_E_NOMEM, "zgr_index_to_device: hipMalloc of " + std::to_string(bytes) + " bytes");
    }
    idx->allocations.push_back(*dst);
    err = hipMemcpyAsync(*dst, src, bytes, hipMemcpyHostToDevice, s);
    if (err != hipSuccess) return hip_fail(err, "hipMemcpyAsync H2D");
    return ZGR_OK;
  };
  const int32_t words = (idx->V + 31) / 32;
  for (int l = 0; l < idx->L; ++l) {
    const HostTable& h = idx->host[l];
    DevTable& d = idx->dev[l];
    d.fmt = h.fmt;
    d.stride = h.stride;
    d.words = words;
    d.V = idx->V;
    d.rows = h.rows;
    void *rp = nullptr, *tk = nullptr, *bt = nullptr, *rk = nullptr;
    int32_t rc = upload(h.row_ptr.data(), h.row_ptr.size() * 4, &rp);
    if (rc == ZGR_OK && h.fmt == ZGR_FMT_SPARSE) rc = upload(h.tok.data(), h.tok.size() * 2, &tk);
    std::vector<uint16_t> rank;
    if (rc == ZGR_OK && h.fmt == ZGR_FMT_DENSE) {
      rc = upload(h.bits.data(), h.bits.size() * 4, &bt);
      // rank directory: set bits of the row before each word (a dense entry's
      // next row is row_ptr[r] + rank + popcount within its word)
      rank.resize(h.bits.size());
      for (int64_t q = 0; q < h.rows; ++q) {
        uint32_t acc = 0;
        for (int32_t w = 0; w < words; ++w) {
          rank[q * words + w] = (uint16_t)acc;
          acc += (uint32_t)__builtin_popcount(h.bits[q * words + w]);
        }
      }
      if (rc == ZGR_OK) rc = upload(rank.data(), rank.size() * 2, &rk);
      if (rc == ZGR_OK) {
        hipError_t se = hipStreamSynchronize(s);  // rank is a temporary
        if (se != hipSuccess) rc = hip_fail(se, "hipStreamSynchronize");
      }
    }
    if (rc != ZGR_OK) {
      (void)hipStreamSynchronize(s);
      for (void* p : idx->allocations) (void)hipFree(p);
      idx->allocations.clear();
      return rc;
    }
    d.row_ptr = (const int32_t*)rp;
    d.tok = (const uint16_t*)tk;
    d.bits = (const uint32_t*)bt;
    d.rank = (const uint16_t*)rk;
  }
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize after index upload");
  idx->on_device = true;
  return ZGR_OK;
}

extern "C" int32_t zgr_index_upload(const int32_t* sids, int64_t N, int32_t L, int32_t V,
                                    const int32_t* fmt, void* stream, zgr_index** out,
                                    int64_t* rank_of_input) {
  using namespace zgr;
  if (!out) return fail(ZGR_E_ARG, "zgr_index_upload: null out");
  zgr_index* idx = nullptr;
  int32_t rc = zgr_index_build_host(sids, N, L, V, fmt, rank_of_input, &idx);
  if (rc != ZGR_OK) return rc;
  rc = zgr_index_to_device(idx, stream);
  if (rc != ZGR_OK) {
    zgr_index_free(idx);
    return rc;
  }
  *out = idx;
  return ZGR_OK;
}

extern "C" int32_t zgr_index_stats(const zgr_index* idx, int32_t t, zgr_step_stats* out) {
  using namespace zgr;
  if (!idx || !out) return fail(ZGR_E_ARG, "zgr_index_stats: null argument");
  if (t < 1 || t > idx->L) return fail(ZGR_E_ARG, "zgr_index_stats: t out of range");
  const HostTable& h = idx->host[t - 1];
  const int64_t words = (idx->V + 31) / 32;
  out->rows = h.rows;
  out->nnz = h.nnz;
  out->fmt = h.fmt;
  out->stride = h.stride;
  out->max_legal = h.max_legal;
  out->reserved = 0;
  out->bytes = (h.rows + 1) * 4 + (h.fmt == ZGR_FMT_DENSE ? h.rows * words * 6 : h.nnz * 2);
  return ZGR_OK;
}

extern "C" int32_t zgr_index_host_table(const zgr_index* idx, int32_t t, const int32_t** row_ptr,
                                        const uint16_t** tok, const uint32_t** bits) {
  using namespace zgr;
  if (!idx) return fail(ZGR_E_ARG, "zgr_index_host_table: null index");
  if (t < 1 || t > idx->L) return fail(ZGR_E_ARG, "zgr_index_host_table: t out of range");
  const HostTable& h = idx->host[t - 1];
  if (row_ptr) *row_ptr = h.row_ptr.data();
  if (tok) *tok = h.tok.data();
  if (bits) *bits = h.fmt == ZGR_FMT_DENSE ? h.bits.data() : nullptr;
  return ZGR_OK;
}

extern "C" int32_t zgr_index_shape(const zgr_index* idx, int32_t* L, int32_t* V, int64_t* N) {
  using namespace zgr;
  if (!idx) return fail(ZGR_E_ARG, "zgr_index_shape: null index");
  if (L) *L = idx->L;
  if (V) *V = idx->V;
  if (N) *N = idx->N;
  return ZGR_OK;
}

extern "C" void zgr_index_free(zgr_index* idx) {
  if (!idx) return;
  zgr::index_unregister(idx);
  if (!idx->allocations.empty()) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (idx->device >= 0 && cur != idx->device) (void)hipSetDevice(idx->device);
    (void)hipDeviceSynchronize();
    for (void* p : idx->allocations) (void)hipFree(p);
    if (cur >= 0 && cur != idx->device) (void)hipSetDevice(cur);
  }
  delete idx;
}
