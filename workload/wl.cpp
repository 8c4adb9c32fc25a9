// Seeded synthetic inputs for filter-first constrained beam search over
// semantic IDs: the item catalog (one SID of L tokens per item), the per-step
// projection weights W_t [V][d] and the per-beam hidden vectors that stand in
// for the trained decoder.
//
// This module only draws inputs.  It holds none of the search's arithmetic
// (no index, no scoring, no normalisation, no selection), so both the CPU
// oracle and the HIP library can be fed from it without sharing method code.
//
// Randomness is counter based: every value is a pure function of
// (seed, field ids, element index) through the SplitMix64 output function
// (Steele, Lea, Flood, "Fast splittable pseudorandom number generators",
// OOPSLA 2014; constants as published by Vigna).  Results do not depend on
// thread count or call order.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

inline uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ULL;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ULL;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBULL;
  return x ^ (x >> 31);
}
inline uint64_t mix(uint64_t h, uint64_t v) { return sm64(h ^ sm64(v)); }

// Field tags keep the catalog, weight and hidden streams apart.
constexpr uint64_t TAG_ITEM = 0x4954454dULL;    // per-item draws
constexpr uint64_t TAG_PERM = 0x5045524dULL;    // per-prefix permutations
constexpr uint64_t TAG_W = 0x57454947ULL;       // projection weights
constexpr uint64_t TAG_HIDDEN = 0x48494444ULL;  // hidden vectors

// uniform in [0, 1) with 53 random bits
inline double unit_open1(uint64_t r) { return (double)(r >> 11) * (1.0 / 9007199254740992.0); }
// uniform in (0, 1]
inline double unit_open0(uint64_t r) { return (double)((r >> 11) + 1) * (1.0 / 9007199254740992.0); }

// Standard normal from two counters (Box-Muller, cosine branch), in double.
inline double normal(uint64_t base, uint64_t i) {
  const double u1 = unit_open0(mix(base, 2 * i));
  const double u2 = unit_open1(mix(base, 2 * i + 1));
  return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586476925286766559 * u2);
}

inline uint32_t f32_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}
inline float bits_f32(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// float -> bfloat16, round to nearest even (inputs here are finite).
inline uint16_t to_bf16(float f) {
  const uint32_t u = f32_bits(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
inline float from_bf16(uint16_t h) { return bits_f32((uint32_t)h << 16); }

// float -> IEEE binary16, round to nearest even, with subnormals.
inline uint16_t to_f16(float f) {
  const uint32_t u = f32_bits(f);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const int32_t e = (int32_t)((u >> 23) & 0xFF);
  uint32_t m = u & 0x7FFFFFu;
  if (e == 0xFF) return (uint16_t)(sign | 0x7C00u | (m ? 0x200u : 0u));
  int32_t he = e - 127 + 15;
  if (he >= 31) return (uint16_t)(sign | 0x7C00u);
  if (he <= 0) {
    // subnormal result: value = m24 * 2^(e-150); unit of f16 subnormal = 2^-24
    if (he < -10) return (uint16_t)sign;  // below half the smallest subnormal
    m |= 0x800000u;
    const int shift = 14 - he;  // 24-bit mantissa -> units of 2^-24
    const uint32_t q = m >> shift;
    const uint32_t rem = m & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    uint32_t r = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
    return (uint16_t)(sign | r);  // r may carry into the exponent: still correct
  }
  uint32_t q = ((uint32_t)he << 10) | (m >> 13);
  const uint32_t rem = m & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) q += 1;  // may round up to inf
  return (uint16_t)(sign | q);
}
inline float from_f16(uint16_t h) {
  const uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu;
  const uint32_t m = h & 0x3FFu;
  if (e == 0) {
    const float v = (float)m * (1.0f / 16777216.0f);  // m * 2^-24, exact
    return (sign ? -v : v);
  }
  if (e == 31) return bits_f32(sign | 0x7F800000u | (m << 13));
  return bits_f32(sign | ((e - 15 + 127) << 23) | (m << 13));
}

// Store one value as dtype (0 f32, 1 bf16, 2 f16); return the stored value widened to float.
inline float store(int32_t dtype, double v, void* out, int64_t k) {
  const float f = (float)v;
  if (dtype == 0) {
    ((float*)out)[k] = f;
    return f;
  }
  if (dtype == 1) {
    const uint16_t h = to_bf16(f);
    ((uint16_t*)out)[k] = h;
    return from_bf16(h);
  }
  const uint16_t h = to_f16(f);
  ((uint16_t*)out)[k] = h;
  return from_f16(h);
}

template <class F>
void parallel_for(int64_t n, int32_t n_threads, F&& fn) {
  if (n_threads <= 1 || n < 4096) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> th;
  const int64_t chunk = (n + n_threads - 1) / n_threads;
  for (int32_t t = 0; t < n_threads; ++t) {
    const int64_t lo = t * chunk, hi = std::min(n, lo + chunk);
    if (lo >= hi) break;
    th.emplace_back([&fn, lo, hi] { fn(lo, hi); });
  }
  for (auto& x : th) x.join();
}

// Keyed bijection of [0, V): balanced 4-round Feistel network on the smallest
// even bit width covering V, with cycle walking back into [0, V).
inline uint32_t keyed_perm(uint64_t key, uint32_t V, uint32_t x) {
  if (V <= 1) return 0;
  int b = 0;
  while ((1u << b) < V) ++b;
  if (b & 1) ++b;
  const int h = b / 2;
  const uint32_t mask = (1u << h) - 1u;
  do {
    uint32_t lo = x & mask, hi = x >> h;
    for (uint64_t r = 0; r < 4; ++r) {
      const uint32_t f = (uint32_t)(mix(key, (r << 32) | lo) & mask);
      const uint32_t nlo = hi ^ f;
      hi = lo;
      lo = nlo;
    }
    x = (hi << h) | lo;
  } while (x >= V);
  return x;
}

struct LevelDist {
  int32_t kind;     // 0 Zipf(param) over all V ranks, 1 uniform over V, 2 uniform over first m ranks
  double param;     // Zipf exponent, or the fraction of ranks for kind 2
  std::vector<double> cdf;
  uint32_t m = 0;
  void init(uint32_t V) {
    if (kind == 0) {
      cdf.resize(V);
      double acc = 0.0;
      for (uint32_t k = 0; k < V; ++k) {
        acc += std::pow((double)(k + 1), -param);
        cdf[k] = acc;
      }
      for (uint32_t k = 0; k < V; ++k) cdf[k] /= acc;
    } else if (kind == 2) {
      m = (uint32_t)std::llround(param * (double)V);
      if (m < 1) m = 1;
      if (m > V) m = V;
    }
  }
  uint32_t rank(double u, uint32_t V) const {
    if (kind == 0) {
      const uint32_t k = (uint32_t)(std::upper_bound(cdf.begin(), cdf.end(), u) - cdf.begin());
      return k < V ? k : V - 1;
    }
    if (kind == 1) return std::min<uint32_t>((uint32_t)(u * V), V - 1);
    return std::min<uint32_t>((uint32_t)(u * m), m - 1);
  }
};

struct Catalog {
  int32_t L;
  uint32_t V;
  int bits;
  uint64_t seed;
  std::vector<LevelDist> lv;

  // Draw attempt a of item i into sid[L]; return the SID packed with `bits` per level.
  uint64_t draw(int64_t i, uint64_t a, int32_t* sid) const {
    const uint64_t k = mix(mix(mix(seed, TAG_ITEM), (uint64_t)i), a);
    uint64_t pk = mix(seed, TAG_PERM);
    uint64_t key = 0;
    for (int32_t l = 0; l < L; ++l) {
      const double u = unit_open1(mix(k, (uint64_t)l));
      const uint32_t r = lv[l].rank(u, V);
      const uint32_t tok = keyed_perm(mix(pk, (uint64_t)l), V, r);
      sid[l] = (int32_t)tok;
      pk = mix(pk, tok);
      key = (key << bits) | tok;
    }
    return key;
  }
};

// Parallel stable LSD radix sort of (key, id) pairs on the low `key_bits` bits.
void radix_sort_pairs(std::vector<uint64_t>& key, std::vector<int64_t>& id, int key_bits, int32_t n_threads) {
  const int64_t n = (int64_t)key.size();
  std::vector<uint64_t> k2(n);
  std::vector<int64_t> i2(n);
  const int T = std::max(1, std::min<int32_t>(n_threads, (int32_t)((n + 65535) / 65536)));
  const int64_t chunk = (n + T - 1) / T;
  std::vector<int64_t> hist((size_t)T * 256);
  for (int shift = 0; shift < key_bits; shift += 8) {
    std::fill(hist.begin(), hist.end(), 0);
    auto count = [&](int t) {
      const int64_t lo = t * chunk, hi = std::min(n, lo + chunk);
      int64_t* h = &hist[(size_t)t * 256];
      for (int64_t j = lo; j < hi; ++j) h[(key[j] >> shift) & 0xFF]++;
    };
    {
      std::vector<std::thread> th;
      for (int t = 0; t < T; ++t) th.emplace_back(count, t);
      for (auto& x : th) x.join();
    }
    int64_t acc = 0;
    for (int b = 0; b < 256; ++b)
      for (int t = 0; t < T; ++t) {
        const int64_t c = hist[(size_t)t * 256 + b];
        hist[(size_t)t * 256 + b] = acc;
        acc += c;
      }
    auto scatter = [&](int t) {
      const int64_t lo = t * chunk, hi = std::min(n, lo + chunk);
      int64_t* h = &hist[(size_t)t * 256];
      for (int64_t j = lo; j < hi; ++j) {
        const int64_t p = h[(key[j] >> shift) & 0xFF]++;
        k2[p] = key[j];
        i2[p] = id[j];
      }
    };
    {
      std::vector<std::thread> th;
      for (int t = 0; t < T; ++t) th.emplace_back(scatter, t);
      for (auto& x : th) x.join();
    }
    key.swap(k2);
    id.swap(i2);
  }
}

// Open-addressing set of packed SIDs (stored +1 so that 0 marks an empty slot).
struct KeySet {
  std::vector<uint64_t> slot;
  uint64_t mask;
  explicit KeySet(int64_t n) {
    uint64_t cap = 1024;
    while (cap < (uint64_t)n * 2) cap <<= 1;
    slot.assign(cap, 0);
    mask = cap - 1;
  }
  bool contains(uint64_t k) const {
    const uint64_t s = k + 1;
    for (uint64_t p = sm64(k) & mask;; p = (p + 1) & mask) {
      if (slot[p] == s) return true;
      if (slot[p] == 0) return false;
    }
  }
  void insert(uint64_t k) {
    const uint64_t s = k + 1;
    for (uint64_t p = sm64(k) & mask;; p = (p + 1) & mask) {
      if (slot[p] == s) return;
      if (slot[p] == 0) {
        slot[p] = s;
        return;
      }
    }
  }
};

}  // namespace

extern "C" {

// Draw N distinct SIDs of L tokens from [0, V).
//   kind[l], param[l]: level-l token law over a keyed permutation of [0, V)
//     seeded by (seed, l, prefix tokens): 0 = Zipf(param) over ranks 1..V,
//     1 = uniform over V, 2 = uniform over the first round(param*V) ranks.
//   A SID that repeats an earlier one is redrawn with the next attempt number,
//   in rounds: within a round the lowest item index keeps a repeated SID.
// sids_out: [N][L] int32 (host).  Returns the number of rounds, or -1 on bad args.
int32_t wl_catalog(int64_t N, int32_t L, int32_t V, const int32_t* kind, const double* param,
                   uint64_t seed, int32_t n_threads, int32_t* sids_out) {
  if (N < 0 || L < 1 || V < 1 || !kind || !param || !sids_out) return -1;
  Catalog cat;
  cat.L = L;
  cat.V = (uint32_t)V;
  cat.bits = 0;
  while ((1u << cat.bits) < (uint32_t)V) ++cat.bits;
  if (cat.bits == 0) cat.bits = 1;
  if (cat.bits * L > 63) return -1;
  cat.seed = seed;
  cat.lv.resize(L);
  for (int32_t l = 0; l < L; ++l) {
    cat.lv[l].kind = kind[l];
    cat.lv[l].param = param[l];
    if (kind[l] < 0 || kind[l] > 2) return -1;
    cat.lv[l].init((uint32_t)V);
  }
  KeySet accepted(N);
  std::vector<int64_t> pending(N);
  for (int64_t i = 0; i < N; ++i) pending[i] = i;
  int32_t rounds = 0;
  for (uint64_t a = 0; !pending.empty(); ++a) {
    ++rounds;
    if (rounds > 100000) return -1;
    const int64_t n = (int64_t)pending.size();
    std::vector<uint64_t> key(n);
    std::vector<int64_t> id(pending);
    parallel_for(n, n_threads, [&](int64_t lo, int64_t hi) {
      for (int64_t j = lo; j < hi; ++j) key[j] = cat.draw(id[j], a, sids_out + id[j] * L);
    });
    radix_sort_pairs(key, id, cat.bits * L, n_threads);
    // Within a group of equal keys the stable sort keeps ids ascending: the first wins.
    std::vector<uint8_t> keep(n, 0);
    parallel_for(n, n_threads, [&](int64_t lo, int64_t hi) {
      for (int64_t j = lo; j < hi; ++j)
        keep[j] = (j == 0 || key[j] != key[j - 1]) && !accepted.contains(key[j]);
    });
    std::vector<int64_t> next;
    for (int64_t j = 0; j < n; ++j) {
      if (keep[j])
        accepted.insert(key[j]);
      else
        next.push_back(id[j]);
    }
    pending.swap(next);
  }
  return rounds;
}

// Projection weights of step t: W_t[v][i] ~ N(0, std^2), v < V, i < d, stored
// as dtype (0 f32, 1 bf16, 2 f16) into out_bits and, if out_f32 is not NULL,
// the stored values widened to float (exact).
void wl_weights(uint64_t seed, int32_t t, int32_t V, int32_t d, double std_dev, int32_t dtype,
                void* out_bits, float* out_f32, int32_t n_threads) {
  parallel_for(V, n_threads, [&](int64_t lo, int64_t hi) {
    for (int64_t v = lo; v < hi; ++v) {
      const uint64_t base = mix(mix(mix(seed, TAG_W), (uint64_t)t), (uint64_t)v);
      for (int32_t i = 0; i < d; ++i) {
        const int64_t k = v * d + i;
        const float f = store(dtype, std_dev * normal(base, (uint64_t)i), out_bits, k);
        if (out_f32) out_f32[k] = f;
      }
    }
  });
}

// Hidden vectors of M beams at step t: beam j belongs to request req[j] and has
// prefix tokens prefix[j*ld + 0 .. t-2].  h ~ N(0, std^2) seeded by
// (seed, request, step, prefix tokens).  Layout [M][d] as dtype, plus optional
// widened floats.
void wl_hidden(uint64_t seed, int32_t t, int64_t M, const int64_t* req, const int32_t* prefix,
               int64_t ld, int32_t d, double std_dev, int32_t dtype, void* out_bits, float* out_f32,
               int32_t n_threads) {
  parallel_for(M, n_threads, [&](int64_t lo, int64_t hi) {
    for (int64_t j = lo; j < hi; ++j) {
      uint64_t base = mix(mix(mix(seed, TAG_HIDDEN), (uint64_t)req[j]), (uint64_t)t);
      for (int32_t l = 0; l + 1 < t; ++l) base = mix(base, (uint64_t)(uint32_t)prefix[j * ld + l]);
      for (int32_t i = 0; i < d; ++i) {
        const int64_t k = j * d + i;
        const float f = store(dtype, std_dev * normal(base, (uint64_t)i), out_bits, k);
        if (out_f32) out_f32[k] = f;
      }
    }
  });
}

// Round float values to dtype and back (exposed so tests can pin the rounding
// against independent converters).
void wl_round(int32_t dtype, const float* in, int64_t n, uint16_t* bits_out, float* out_f32) {
  for (int64_t k = 0; k < n; ++k) {
    uint16_t h;
    float f;
    if (dtype == 1) {
      h = to_bf16(in[k]);
      f = from_bf16(h);
    } else {
      h = to_f16(in[k]);
      f = from_f16(h);
    }
    if (bits_out) bits_out[k] = h;
    if (out_f32) out_f32[k] = f;
  }
}

// The keyed permutation, exposed for its bijectivity test.
uint32_t wl_perm(uint64_t key, uint32_t V, uint32_t x) { return keyed_perm(key, V, x); }

}  // extern "C"
