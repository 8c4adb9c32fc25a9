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
#include <chrono>
#include <cstring>
#include <mutex>
#include <thread>
#include <unordered_map>

#include "zgr_internal.h"

namespace {

// Bytes of a table in HBM: row_ptr, then the sorted tokens (sparse), the
// bitmap and its rank directory (dense), or the next-row matrix.
int64_t table_device_bytes(const zgr::HostTable& h, int32_t words) {
  const int64_t rp = (h.rows + 1) * 4;
  if (h.fmt == ZGR_FMT_SPARSE) return rp + h.nnz * 2 + (int64_t)h.sdir.size() * 2;
  if (h.fmt == ZGR_FMT_DENSE_NEXT) return rp + h.rows * (int64_t)h.stride * 4;
  return rp + h.rows * (int64_t)words * 6;
}

using Clock = std::chrono::steady_clock;
double ms_since(Clock::time_point t0) {
  return std::chrono::duration<double, std::milli>(Clock::now() - t0).count();
}

constexpr int kMaxThreads = 64;

// Threads for n items: an explicit request is honoured (capped at 64 and at
// n); 0 picks the hardware thread count (capped at 16) for large inputs and
// one thread below 2^16 items.
int pick_threads(int32_t requested, int64_t n) {
  int T;
  if (requested > 0) {
    T = std::min(requested, kMaxThreads);
  } else {
    const unsigned hw = std::thread::hardware_concurrency();
    T = (n < (1 << 16)) ? 1 : (int)std::max(1u, std::min(hw, 16u));
  }
  return (int)std::max<int64_t>(1, std::min<int64_t>(T, n));
}

// Chunk t of T equal chunks of [0, n).
inline void chunk_of(int64_t n, int T, int t, int64_t* lo, int64_t* hi) {
  const int64_t c = (n + T - 1) / T;
  *lo = std::min(n, t * c);
  *hi = std::min(n, *lo + c);
}

// fn(t) for t in [0, T) on T threads (inline when T = 1).
template <class F>
void run_par(int T, F&& fn) {
  if (T == 1) {
    fn(0);
    return;
  }
  std::vector<std::thread> th;
  th.reserve(T);
  for (int t = 0; t < T; ++t) th.emplace_back([&fn, t] { fn(t); });
  for (auto& x : th) x.join();
}

// fn(lo, hi, t) over T chunks of [0, n).
template <class F>
void par_chunks(int T, int64_t n, F&& fn) {
  run_par(T, [&](int t) {
    int64_t lo, hi;
    chunk_of(n, T, t, &lo, &hi);
    if (lo < hi) fn(lo, hi, t);
  });
}

// Stable LSD radix sort of (key, original row) by key on T threads, skipping
// digits that are zero in every key.
void sort_keys(std::vector<uint64_t>& key, std::vector<int32_t>& row, int T) {
  const int64_t n = (int64_t)key.size();
  std::vector<uint64_t> any_t(T, 0);
  par_chunks(T, n, [&](int64_t lo, int64_t hi, int t) {
    uint64_t a = 0;
    for (int64_t i = lo; i < hi; ++i) a |= key[i];
    any_t[t] = a;
  });
  uint64_t any = 0;
  for (uint64_t a : any_t) any |= a;
  std::vector<uint64_t> k2(n);
  std::vector<int32_t> r2(n);
  std::vector<int64_t> hist((size_t)T * 256);
  for (int shift = 0; shift < 64; shift += 8) {
    if (((any >> shift) & 0xFF) == 0) continue;
    std::fill(hist.begin(), hist.end(), 0);
    par_chunks(T, n, [&](int64_t lo, int64_t hi, int t) {
      int64_t* h = &hist[(size_t)t * 256];
      for (int64_t j = lo; j < hi; ++j) ++h[(key[j] >> shift) & 0xFF];
    });
    int64_t acc = 0;
    for (int b = 0; b < 256; ++b)
      for (int t = 0; t < T; ++t) {
        int64_t& h = hist[(size_t)t * 256 + b];
        const int64_t c = h;
        h = acc;
        acc += c;
      }
    par_chunks(T, n, [&](int64_t lo, int64_t hi, int t) {
      int64_t* h = &hist[(size_t)t * 256];
      for (int64_t j = lo; j < hi; ++j) {
        const int64_t p = h[(key[j] >> shift) & 0xFF]++;
        k2[p] = key[j];
        r2[p] = row[j];
      }
    });
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

namespace {

// The rebuild pipeline of a catalog, on the host:
//   keys    pack each SID into a 64-bit key (token range check)
//   sort    radix sort of (key, catalog row)
//   layout  two passes over the sorted keys in T chunks: count each chunk's
//           entries and rows per table, prefix-sum the counts into chunk
//           offsets, then every chunk fills its part of row_ptr and tok
//   encode  per table: largest row, format, and for dense tables the bitmap
//           and its rank directory
int32_t build_host(const int32_t* sids, int64_t N, int32_t L, int32_t V, const int32_t* fmt,
                   int64_t* rank_of_input, const zgr_build_opts* opts, zgr_build_times* times,
                   zgr_index** out) {
  using namespace zgr;
  if (!sids || !out) return fail(ZGR_E_ARG, "zgr_index_build_host: null sids or out");
  *out = nullptr;
  if (N < 1) return fail(ZGR_E_ARG, "zgr_index_build_host: N must be >= 1");
  if (N >= INT32_MAX) return fail(ZGR_E_SHAPE, "zgr_index_build_host: N must be < 2^31 - 1");
  if (L < 1 || L > kMaxL) return fail(ZGR_E_ARG, "zgr_index_build_host: L must be in [1, 8]");
  if (V < 2 || V > 65536) return fail(ZGR_E_ARG, "zgr_index_build_host: V must be in [2, 65536]");
  if (opts && opts->host_threads < 0)
    return fail(ZGR_E_ARG, "zgr_index_build_host: host_threads must be >= 0");
  const int32_t slices = opts ? opts->slices : ZGR_SLICES_AUTO;
  if (slices < ZGR_SLICES_AUTO || slices > ZGR_SLICES_NEVER)
    return fail(ZGR_E_ARG, "zgr_index_build_host: slices must be ZGR_SLICES_AUTO, _ALWAYS or _NEVER");
  int bits = 0;
  while ((1 << bits) < V) ++bits;
  if (bits * L > 64) return fail(ZGR_E_SHAPE, "zgr_index_build_host: ceil(log2 V) * L > 64");
  if (fmt) {
    for (int l = 0; l < L; ++l)
      if (fmt[l] < ZGR_FMT_AUTO || fmt[l] > ZGR_FMT_DENSE_NEXT)
        return fail(ZGR_E_ARG, "zgr_index_build_host: fmt[t] must be AUTO, DENSE, SPARSE or DENSE_NEXT");
  }
  const int T = pick_threads(opts ? opts->host_threads : 0, N);
  zgr_build_times tm{};
  tm.threads = T;
  const auto t_all = Clock::now();
  auto t0 = t_all;

  std::vector<uint64_t> key;
  std::vector<int32_t> row;
  try {
    key.resize(N);
    row.resize(N);
  } catch (...) {
    return fail(ZGR_E_NOMEM, "zgr_index_build_host: host allocation");
  }
  std::vector<int64_t> bad(T, -1);
  std::vector<char> ordered(T, 1);  // chunk's keys non-decreasing
  par_chunks(T, N, [&](int64_t lo, int64_t hi, int t) {
    uint64_t prev = 0;
    bool ord = true;
    for (int64_t i = lo; i < hi; ++i) {
      uint64_t k = 0;
      for (int l = 0; l < L; ++l) {
        const int32_t v = sids[i * L + l];
        if ((v < 0 || v >= V) && bad[t] < 0) bad[t] = i;
        k = (k << bits) | (uint64_t)(uint32_t)v;
      }
      key[i] = k;
      row[i] = (int32_t)i;
      if (i > lo && k < prev) ord = false;
      prev = k;
    }
    ordered[t] = ord;
  });
  for (int64_t b : bad)
    if (b >= 0)
      return fail(ZGR_E_TOKEN_RANGE, "zgr_index_build_host: catalog row " + std::to_string(b) +
                                         " has a token outside [0, V)");
  // A catalog already in SID order (the usual case when a rebuild starts from
  // the previous index's order) needs no sort.
  bool sorted = true;
  for (int t = 0; t < T && sorted; ++t) {
    int64_t lo, hi;
    chunk_of(N, T, t, &lo, &hi);
    if (lo < hi && (!ordered[t] || (lo > 0 && key[lo] < key[lo - 1]))) sorted = false;
  }
  tm.keys_ms = ms_since(t0);
  t0 = Clock::now();
  if (!sorted) {
    try {
      sort_keys(key, row, T);
    } catch (...) {
      return fail(ZGR_E_NOMEM, "zgr_index_build_host: host allocation");
    }
  }
  tm.sort_ms = ms_since(t0);
  t0 = Clock::now();

  const uint64_t tmask = (1ULL << bits) - 1ULL;
  auto token_at = [&](uint64_t k, int l) { return (uint32_t)((k >> (bits * (L - 1 - l))) & tmask); };
  // First level at which sorted key i differs from key i-1 (0 for the first
  // key).  Keys are distinct once the duplicate check has passed.
  auto first_diff = [&](int64_t i) -> int {
    if (i == 0) return 0;
    const uint64_t x = key[i] ^ key[i - 1];
    const int msb = 63 - __builtin_clzll(x);
    return L - 1 - msb / bits;
  };
  // Pass 1: per chunk, entries and new rows of every table, and the first
  // duplicate.  Table l (step l+1) has an entry for every distinct length-(l+1)
  // prefix and a row for every distinct length-l prefix.
  struct Count {
    int64_t nnz[kMaxL];
    int64_t rows[kMaxL];
    int64_t dup;
  };
  Count zero{};
  zero.dup = -1;
  std::vector<Count> cnt(T, zero);  // empty chunks keep zero counts
  par_chunks(T, N, [&](int64_t lo, int64_t hi, int t) {
    Count c{};
    c.dup = -1;
    for (int64_t i = lo; i < hi; ++i) {
      if (i > 0 && key[i] == key[i - 1]) {
        if (c.dup < 0) c.dup = i;
        continue;
      }
      const int f = first_diff(i);
      for (int l = f; l < L; ++l) ++c.nnz[l];
      for (int l = f + 1; l < L; ++l) ++c.rows[l];
    }
    cnt[t] = c;
  });
  for (int t = 0; t < T; ++t)
    if (cnt[t].dup >= 0) {
      const int64_t i = cnt[t].dup;
      return fail(ZGR_E_DUP_SID, "zgr_index_build_host: catalog rows " + std::to_string(row[i - 1]) +
                                     " and " + std::to_string(row[i]) + " share one SID");
    }
  if (rank_of_input)
    par_chunks(T, N, [&](int64_t lo, int64_t hi, int) {
      for (int64_t i = lo; i < hi; ++i) rank_of_input[row[i]] = i;
    });
  row.clear();
  row.shrink_to_fit();

  // Chunk offsets.  Row 0 of table 1 is the empty prefix; for deeper tables
  // the first key opens row 0, so row_ptr[q] is written when row q opens.
  std::vector<Count> off(T);
  int64_t rows[kMaxL] = {0}, nnz[kMaxL] = {0};
  for (int l = 0; l < L; ++l) {
    int64_t e = 0, r = (l == 0) ? 1 : 0;
    for (int t = 0; t < T; ++t) {
      off[t].nnz[l] = e;
      off[t].rows[l] = r;
      e += cnt[t].nnz[l];
      r += cnt[t].rows[l];
    }
    nnz[l] = e;
    rows[l] = r;
  }
  zgr_index* idx = new (std::nothrow) zgr_index();
  if (!idx) return fail(ZGR_E_NOMEM, "zgr_index_build_host: host allocation");
  idx->L = L;
  idx->V = V;
  idx->bits = bits;
  idx->N = N;
  try {
    for (int l = 0; l < L; ++l) {
      idx->host[l].rows = rows[l];
      idx->host[l].nnz = nnz[l];
      idx->host[l].row_ptr.resize(rows[l] + 1);
      idx->host[l].tok.resize(nnz[l]);
    }
  } catch (...) {
    delete idx;
    return fail(ZGR_E_NOMEM, "zgr_index_build_host: host allocation");
  }
  // Pass 2: fill.
  par_chunks(T, N, [&](int64_t lo, int64_t hi, int t) {
    int64_t e[kMaxL], r[kMaxL];
    int32_t* rp[kMaxL];
    uint16_t* tk[kMaxL];
    for (int l = 0; l < L; ++l) {
      e[l] = off[t].nnz[l];
      r[l] = off[t].rows[l];
      rp[l] = idx->host[l].row_ptr.data();
      tk[l] = idx->host[l].tok.data();
    }
    for (int64_t i = lo; i < hi; ++i) {
      const int f = first_diff(i);
      const uint64_t k = key[i];
      for (int l = f; l < L; ++l) {
        if (l > f) rp[l][r[l]++] = (int32_t)e[l];
        tk[l][e[l]++] = (uint16_t)token_at(k, l);
      }
    }
  });
  idx->host[0].row_ptr[0] = 0;
  for (int l = 0; l < L; ++l) idx->host[l].row_ptr[rows[l]] = (int32_t)nnz[l];
  key.clear();
  key.shrink_to_fit();
  tm.layout_ms = ms_since(t0);
  t0 = Clock::now();

  const int32_t words = (V + 31) / 32;
  for (int l = 0; l < L; ++l) {
    HostTable& h = idx->host[l];
    const int Tr = std::min<int64_t>(T, std::max<int64_t>(1, h.rows / 256));
    std::vector<int32_t> mx_t(Tr, 0);
    par_chunks(Tr, h.rows, [&](int64_t lo, int64_t hi, int t) {
      int32_t m = 0;
      for (int64_t q = lo; q < hi; ++q) m = std::max(m, h.row_ptr[q + 1] - h.row_ptr[q]);
      mx_t[t] = m;
    });
    h.max_legal = *std::max_element(mx_t.begin(), mx_t.end());
    const int64_t dense_bytes = h.rows * (int64_t)words * 4;
    const int64_t sparse_bytes = h.nnz * 2;
    const int32_t want = fmt ? fmt[l] : ZGR_FMT_AUTO;
    h.fmt = (want == ZGR_FMT_AUTO) ? (dense_bytes < sparse_bytes ? ZGR_FMT_DENSE : ZGR_FMT_SPARSE)
                                   : want;
    const bool next_matrix = h.fmt == ZGR_FMT_DENSE_NEXT;
    h.stride = (h.fmt != ZGR_FMT_SPARSE) ? V : h.max_legal;
    const bool want_sdir = h.fmt == ZGR_FMT_SPARSE &&
                           (slices == ZGR_SLICES_ALWAYS ||
                            (slices == ZGR_SLICES_AUTO && V >= 1024 && h.nnz >= 32 * h.rows));
    if (want_sdir) {
      // Slice directory: a row's legal tokens below the end of each codebook
      // eighth (tokens are sorted, so one walk per row).  Counts below 7/8 of
      // V stay under 2^16 for any V <= 65536.
      try {
        h.sdir.assign((size_t)h.rows * kSlices, 0);
      } catch (...) {
        delete idx;
        return fail(ZGR_E_NOMEM, "zgr_index_build_host: host allocation");
      }
      const int32_t span = (V + kSlices - 1) / kSlices;
      par_chunks(Tr, h.rows, [&](int64_t lo, int64_t hi, int) {
        for (int64_t q = lo; q < hi; ++q) {
          const int32_t b0 = h.row_ptr[q], b1 = h.row_ptr[q + 1];
          int32_t j = b0;
          for (int x = 0; x + 1 < kSlices; ++x) {
            while (j < b1 && (int32_t)h.tok[j] < (x + 1) * span) ++j;
            h.sdir[q * kSlices + x] = (uint16_t)(j - b0);
          }
        }
      });
    }
    if (h.fmt != ZGR_FMT_SPARSE) {
      try {
        h.bits.assign((size_t)h.rows * words, 0u);
        h.rank.resize((size_t)h.rows * words);
        if (next_matrix) h.next.assign((size_t)h.rows * V, -1);
      } catch (...) {
        delete idx;
        return fail(ZGR_E_NOMEM, "zgr_index_build_host: host allocation");
      }
      if (next_matrix)
        // the alternative dense encoding: every (row, token) cell holds the
        // entry's next row, -1 where the token is not legal
        par_chunks(Tr, h.rows, [&](int64_t lo, int64_t hi, int) {
          for (int64_t q = lo; q < hi; ++q)
            for (int32_t j = h.row_ptr[q]; j < h.row_ptr[q + 1]; ++j) h.next[q * V + h.tok[j]] = j;
        });
      // Bitmap, then the rank directory: set bits of the row before each word
      // (a dense entry's next row is row_ptr[r] + rank + popcount below the
      // token inside its word).
      par_chunks(Tr, h.rows, [&](int64_t lo, int64_t hi, int) {
        for (int64_t q = lo; q < hi; ++q) {
          uint32_t* bq = &h.bits[q * words];
          for (int32_t j = h.row_ptr[q]; j < h.row_ptr[q + 1]; ++j)
            bq[h.tok[j] / 32] |= 1u << (h.tok[j] % 32);
          uint32_t acc = 0;
          for (int32_t w = 0; w < words; ++w) {
            h.rank[q * words + w] = (uint16_t)acc;
            acc += (uint32_t)__builtin_popcount(bq[w]);
          }
        }
      });
    }
  }
  tm.encode_ms = ms_since(t0);
  for (int l = 0; l < L; ++l) {
    const HostTable& h = idx->host[l];
    tm.device_bytes += table_device_bytes(h, words);
  }
  tm.build_ms = ms_since(t_all);
  static uint64_t gen_counter = 0;
  idx->generation = __atomic_add_fetch(&gen_counter, 1, __ATOMIC_RELAXED);
  idx->times = tm;
  index_register(idx, idx->generation);
  if (times) *times = tm;
  *out = idx;
  return ZGR_OK;
}

// Pinned host staging of an upload: two buffers used in turn.  While the DMA
// engine copies one buffer to HBM, host threads fill the other; an event per
// buffer says when the DMA engine is done with it.
struct Staging {
  void* buf[2] = {nullptr, nullptr};
  hipEvent_t ev[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  size_t cap = 0;
  int cur = 0;
  ~Staging() {
    for (int i = 0; i < 2; ++i) {
      if (ev[i]) {
        (void)hipEventSynchronize(ev[i]);
        (void)hipEventDestroy(ev[i]);
      }
      if (buf[i]) (void)hipHostFree(buf[i]);
    }
  }
};

int32_t upload_index(zgr_index* idx, void* stream, const zgr_build_opts* opts, zgr_build_times* times) {
  using namespace zgr;
  if (!idx) return fail(ZGR_E_ARG, "zgr_index_to_device: null index");
  if (idx->on_device) return fail(ZGR_E_STATE, "zgr_index_to_device: index already on device");
  const int32_t mode = opts ? opts->upload : ZGR_UPLOAD_STAGED;
  if (mode != ZGR_UPLOAD_STAGED && mode != ZGR_UPLOAD_DIRECT)
    return fail(ZGR_E_ARG, "zgr_index_to_device: upload must be ZGR_UPLOAD_STAGED or ZGR_UPLOAD_DIRECT");
  if (opts && (opts->host_threads < 0 || opts->staging_bytes < 0))
    return fail(ZGR_E_ARG, "zgr_index_to_device: negative host_threads or staging_bytes");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipGetDevice(&idx->device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  zgr_build_times& tm = idx->times;
  tm.upload = mode;
  auto t0 = Clock::now();

  struct Piece {
    const void* src;
    size_t bytes;
    void** dst;
  };
  std::vector<Piece> pieces;
  void* ptrs[kMaxL][6] = {};
  size_t total = 0;
  for (int l = 0; l < idx->L; ++l) {
    const HostTable& h = idx->host[l];
    pieces.push_back({h.row_ptr.data(), h.row_ptr.size() * 4, &ptrs[l][0]});
    if (h.fmt == ZGR_FMT_SPARSE) {
      pieces.push_back({h.tok.data(), h.tok.size() * 2, &ptrs[l][1]});
      if (!h.sdir.empty()) pieces.push_back({h.sdir.data(), h.sdir.size() * 2, &ptrs[l][5]});
    } else if (h.fmt == ZGR_FMT_DENSE_NEXT) {
      pieces.push_back({h.next.data(), h.next.size() * 4, &ptrs[l][4]});
    } else {
      pieces.push_back({h.bits.data(), h.bits.size() * 4, &ptrs[l][2]});
      pieces.push_back({h.rank.data(), h.rank.size() * 2, &ptrs[l][3]});
    }
  }
  auto release = [&]() {
    (void)hipStreamSynchronize(s);
    for (void* q : idx->allocations) (void)hipFree(q);
    idx->allocations.clear();
  };
  for (Piece& pc : pieces) {
    if (pc.bytes == 0) continue;
    hipError_t err = hipMalloc(pc.dst, pc.bytes);
    if (err != hipSuccess) {
      *pc.dst = nullptr;
      (void)hipGetLastError();
      release();
      return fail(ZGR_E_NOMEM, "zgr_index_to_device: hipMalloc of " + std::to_string(pc.bytes) + " bytes");
    }
    idx->allocations.push_back(*pc.dst);
    total += pc.bytes;
  }
  tm.alloc_ms = ms_since(t0);
  t0 = Clock::now();
  if (mode == ZGR_UPLOAD_DIRECT) {
    for (Piece& pc : pieces) {
      if (pc.bytes == 0) continue;
      e = hipMemcpyAsync(*pc.dst, pc.src, pc.bytes, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) {
        release();
        return hip_fail(e, "hipMemcpyAsync H2D");
      }
    }
  } else {
    const int64_t want = (opts && opts->staging_bytes > 0) ? opts->staging_bytes : (64LL << 20);
    const int T = pick_threads(opts ? opts->host_threads : 0, (int64_t)total / 4096);
    Staging st;
    st.cap = (size_t)std::max<int64_t>(4096, std::min<int64_t>(want, (int64_t)total));
    for (int i = 0; i < 2; ++i) {
      e = hipHostMalloc(&st.buf[i], st.cap, hipHostMallocDefault);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&st.ev[i], hipEventDisableTiming);
      if (e != hipSuccess) {
        st.buf[i] = nullptr;
        (void)hipGetLastError();
        release();
        return fail(ZGR_E_NOMEM, "zgr_index_to_device: pinned staging allocation");
      }
    }
    for (Piece& pc : pieces) {
      for (size_t o = 0; o < pc.bytes; o += st.cap) {
        const size_t n = std::min(st.cap, pc.bytes - o);
        const int b = st.cur;
        if (st.pending[b]) {
          e = hipEventSynchronize(st.ev[b]);
          if (e != hipSuccess) {
            release();
            return hip_fail(e, "hipEventSynchronize");
          }
        }
        const char* src = (const char*)pc.src + o;
        char* dst = (char*)st.buf[b];
        const int Tc = (n >= (4u << 20)) ? T : 1;
        par_chunks(Tc, (int64_t)n, [&](int64_t lo, int64_t hi, int) {
          std::memcpy(dst + lo, src + lo, (size_t)(hi - lo));
        });
        e = hipMemcpyAsync((char*)*pc.dst + o, st.buf[b], n, hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipEventRecord(st.ev[b], s);
        if (e != hipSuccess) {
          release();
          return hip_fail(e, "hipMemcpyAsync H2D from staging");
        }
        st.pending[b] = true;
        st.cur ^= 1;
      }
    }
  }
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    release();
    return hip_fail(e, "hipStreamSynchronize after index upload");
  }
  tm.upload_ms = ms_since(t0);
  tm.device_bytes = (int64_t)total;
  const int32_t words = (idx->V + 31) / 32;
  for (int l = 0; l < idx->L; ++l) {
    const HostTable& h = idx->host[l];
    DevTable& d = idx->dev[l];
    d.fmt = h.fmt;
    d.stride = h.stride;
    d.words = words;
    d.V = idx->V;
    d.rows = h.rows;
    d.row_ptr = (const int32_t*)ptrs[l][0];
    d.tok = (const uint16_t*)ptrs[l][1];
    d.bits = (const uint32_t*)ptrs[l][2];
    d.rank = (const uint16_t*)ptrs[l][3];
    d.next = (const int32_t*)ptrs[l][4];
    d.sdir = (const uint16_t*)ptrs[l][5];
  }
  idx->on_device = true;
  if (times) *times = tm;
  return ZGR_OK;
}

}  // namespace

extern "C" int32_t zgr_index_build_host(const int32_t* sids, int64_t N, int32_t L, int32_t V,
                                        const int32_t* fmt, int64_t* rank_of_input,
                                        zgr_index** out) {
  return build_host(sids, N, L, V, fmt, rank_of_input, nullptr, nullptr, out);
}

extern "C" int32_t zgr_index_build_host_ex(const int32_t* sids, int64_t N, int32_t L, int32_t V,
                                           const int32_t* fmt, int64_t* rank_of_input,
                                           const zgr_build_opts* opts, zgr_build_times* times,
                                           zgr_index** out) {
  return build_host(sids, N, L, V, fmt, rank_of_input, opts, times, out);
}

extern "C" int32_t zgr_index_to_device(zgr_index* idx, void* stream) {
  return upload_index(idx, stream, nullptr, nullptr);
}

extern "C" int32_t zgr_index_to_device_ex(zgr_index* idx, void* stream, const zgr_build_opts* opts,
                                          zgr_build_times* times) {
  return upload_index(idx, stream, opts, times);
}

extern "C" int32_t zgr_index_upload(const int32_t* sids, int64_t N, int32_t L, int32_t V,
                                    const int32_t* fmt, void* stream, zgr_index** out,
                                    int64_t* rank_of_input) {
  return zgr_index_upload_ex(sids, N, L, V, fmt, stream, nullptr, nullptr, out, rank_of_input);
}

extern "C" int32_t zgr_index_upload_ex(const int32_t* sids, int64_t N, int32_t L, int32_t V,
                                       const int32_t* fmt, void* stream,
                                       const zgr_build_opts* opts, zgr_build_times* times,
                                       zgr_index** out, int64_t* rank_of_input) {
  using namespace zgr;
  if (!out) return fail(ZGR_E_ARG, "zgr_index_upload: null out");
  *out = nullptr;
  if (opts && (opts->upload != ZGR_UPLOAD_STAGED && opts->upload != ZGR_UPLOAD_DIRECT))
    return fail(ZGR_E_ARG, "zgr_index_upload: upload must be ZGR_UPLOAD_STAGED or ZGR_UPLOAD_DIRECT");
  if (opts && opts->staging_bytes < 0)
    return fail(ZGR_E_ARG, "zgr_index_upload: negative staging_bytes");
  zgr_index* idx = nullptr;
  int32_t rc = build_host(sids, N, L, V, fmt, rank_of_input, opts, nullptr, &idx);
  if (rc != ZGR_OK) return rc;
  rc = upload_index(idx, stream, opts, times);
  if (rc != ZGR_OK) {
    zgr_index_free(idx);
    return rc;
  }
  *out = idx;
  return ZGR_OK;
}

extern "C" int32_t zgr_index_times(const zgr_index* idx, zgr_build_times* out) {
  using namespace zgr;
  if (!idx || !out) return fail(ZGR_E_ARG, "zgr_index_times: null argument");
  *out = idx->times;
  return ZGR_OK;
}

extern "C" int32_t zgr_index_device_table(const zgr_index* idx, int32_t t, const void** row_ptr,
                                          const void** tok, const void** bits, const void** rank,
                                          const void** next) {
  using namespace zgr;
  if (!idx) return fail(ZGR_E_ARG, "zgr_index_device_table: null index");
  if (t < 1 || t > idx->L) return fail(ZGR_E_ARG, "zgr_index_device_table: t out of range");
  if (!idx->on_device) return fail(ZGR_E_STATE, "zgr_index_device_table: index is not on a device");
  const DevTable& d = idx->dev[t - 1];
  if (row_ptr) *row_ptr = d.row_ptr;
  if (tok) *tok = d.tok;
  if (bits) *bits = d.bits;
  if (rank) *rank = d.rank;
  if (next) *next = d.next;
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
  out->slice_dir = h.sdir.empty() ? 0 : 1;
  out->bytes = table_device_bytes(h, (int32_t)words);
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
  if (bits) *bits = h.fmt != ZGR_FMT_SPARSE ? h.bits.data() : nullptr;
  return ZGR_OK;
}

extern "C" int32_t zgr_index_host_slices(const zgr_index* idx, int32_t t, const uint16_t** sdir) {
  using namespace zgr;
  if (!idx || !sdir) return fail(ZGR_E_ARG, "zgr_index_host_slices: null argument");
  if (t < 1 || t > idx->L) return fail(ZGR_E_ARG, "zgr_index_host_slices: t out of range");
  const HostTable& h = idx->host[t - 1];
  *sdir = h.sdir.empty() ? nullptr : h.sdir.data();
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
