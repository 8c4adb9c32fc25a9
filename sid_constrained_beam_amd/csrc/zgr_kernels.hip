// HIP kernels (gfx950) of one filter-first constrained beam-search step.
//
// ZeroGR description, "overall pipeline": per step each beam's legal tokens
// are read from the index, scored (only the legal ones on sparse steps; the
// full projection followed by a pick of the legal columns on dense steps),
// normalised by a log-softmax over the legal tokens only, added to the beam's
// cumulative log-prob, and the next beams are picked by the new value.
// "Why fewer scores is not faster": every beam owns the same number of
// candidate slots (the step's largest legal count; a dense step uses the
// whole codebook with slot = token), a candidate's slot depends only on its
// beam and its rank, empty slots are minus infinity and never picked, and
// filter, score and select all address those slots directly, with weight rows
// read in place: no compacted candidate list and no temporary matrix.
//
// Kernels of a step:
//   k_units            per beam: legal count n_b and its number of work units;
//                      an exclusive scan over the M beams (not over candidates:
//                      slot addresses never depend on other beams).
//   k_score_selective  persistent grid over (beam, tile) units: each unit
//                      reads the beam's legal tokens (sparse: tok[row_ptr[r]+j];
//                      dense: set bits of the row's bitmap) and computes
//                      z = W_t[token] . h_beam with the weight row read in place
//                      by a group of lanes (16-byte loads), h kept in registers,
//                      a lane-group shuffle reduction, z stored at the slot.
//   k_gemm_nt          full projection Z = H . W_t^T on MFMA (fp32, bf16, f16
//                      inputs; fp32 accumulate), Z row = beam, column = token.
//   k_beam_reduce      per beam: max and sum-exp over the legal slots only,
//                      lse, cand = cum + (z - lse), then the beam's best
//                      min(K, n_b) candidates as 64-bit keys (LDS radix select).
//   k_request_select   per request: the best K keys over its beams (LDS radix
//                      select), bitonic sort, decode (parent, token, cum) and
//                      advance: next row = row_ptr[r] + slot (sparse: the
//                      position is the next row) or row_ptr[r] + popcount of
//                      the bitmap below the token (dense); prefix gather.
//
// Ranking key (64 bits, larger = better): high word = order-preserving image
// of the float cand, low word = ~(beam_rank * S_t + slot).  Keys are unique,
// so every selection is exact and deterministic; equal scores fall to the
// lower beam rank, then the lower slot (slot order = token order).
#include <hip/hip_runtime.h>

#include "zgr_internal.h"

namespace zgr {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// ---------------------------------------------------------------- element helpers

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Load 16 bytes and widen to float: 4 (f32) or 8 (bf16 / f16) values.
template <int DT>
__device__ __forceinline__ void load16(const void* p, float* out) {
  if constexpr (DT == ZGR_F32) {
    const float4 v = *(const float4*)p;
    out[0] = v.x;
    out[1] = v.y;
    out[2] = v.z;
    out[3] = v.w;
  } else {
    const uint4 v = *(const uint4*)p;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == ZGR_BF16) {
        out[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        out[2 * i + 1] = bf16_to_f32(w[i] >> 16);
      } else {
        out[2 * i] = f16_to_f32(w[i] & 0xFFFFu);
        out[2 * i + 1] = f16_to_f32(w[i] >> 16);
      }
    }
  }
}

// ---------------------------------------------------------------- keys

__device__ __forceinline__ uint32_t ord_of(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_of_ord(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t make_key(float cand, uint32_t slotcode) {
  return ((uint64_t)ord_of(cand) << 32) | (uint64_t)(0xFFFFFFFFu - slotcode);
}

// ---------------------------------------------------------------- block helpers (256 threads)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Fixed-order block reductions (deterministic).
__device__ float block_max(float v, float* sh) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, sh[i]);
  return r;
}
__device__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r += sh[i];
  return r;
}
__device__ int block_sum_i(int v, int* sh) {
  v = wave_sum_i(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) r += sh[i];
  return r;
}
// Exclusive prefix over the block's threads; *total gets the sum.
__device__ int block_excl_scan(int v, int* sh, int* total) {
  const int incl = wave_incl_scan(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 63) sh[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    if (i < w) before += sh[i];
    all += sh[i];
  }
  *total = all;
  return before + incl - v;
}

// State of an LDS radix select for the `need` largest of a set of distinct
// 64-bit keys, 8 bits per pass from the top.
struct RadixSel {
  uint64_t prefix;
  uint64_t mask;
  int need;
};

// One histogram pass has been accumulated in hist[256]; pick the digit that
// holds the need-th largest key and narrow the state.  Returns true when every
// key matching the new prefix is selected (no further pass needed).
__device__ bool radix_narrow(RadixSel& s, int shift, int* hist, int* sh) {
  // thread d looks at digit 255 - d: inclusive prefix over threads = count of
  // keys whose digit is >= 255 - d
  const int d = 255 - (int)threadIdx.x;
  const int c = hist[d];
  int total;
  const int excl = block_excl_scan(c, sh, &total);
  __shared__ int pick_digit, pick_above, pick_count;
  if (excl < s.need && excl + c >= s.need) {
    pick_digit = d;
    pick_above = excl;
    pick_count = c;
  }
  __syncthreads();
  s.prefix |= (uint64_t)pick_digit << shift;
  s.mask |= (uint64_t)0xFF << shift;
  s.need -= pick_above;
  const bool done = (pick_count == s.need);
  __syncthreads();
  return done;
}

// ---------------------------------------------------------------- k_units

__global__ __launch_bounds__(1024) void k_units(const int32_t* __restrict__ row_in, int32_t M,
                                                DevTable tab, int32_t* __restrict__ nlegal,
                                                int32_t* __restrict__ unit_start,
                                                int32_t* __restrict__ err) {
  const int per = (M + 1023) / 1024;
  const int b0 = threadIdx.x * per, b1 = min(M, b0 + per);
  const int dense_units = (tab.V + kDenseTile - 1) / kDenseTile;
  auto units_of = [&](int b, bool record) -> int {
    const int r = row_in[b];
    int n = 0;
    if (r >= 0 && r < tab.rows) {
      n = tab.row_ptr[r + 1] - tab.row_ptr[r];
    } else if (r >= tab.rows && record) {
      atomicOr(err, 1);
    }
    if (record) nlegal[b] = n;
    if (n == 0) return 0;
    return tab.fmt == ZGR_FMT_DENSE ? dense_units : (n + kSparseTile - 1) / kSparseTile;
  };
  int mine = 0;
  for (int b = b0; b < b1; ++b) mine += units_of(b, true);
  // block-wide exclusive scan of 1024 per-thread totals
  __shared__ int wsum[16];
  const int incl = wave_incl_scan(mine);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int i = 0; i < 16; ++i) {
    if (i < w) before += wsum[i];
    total += wsum[i];
  }
  int run = before + incl - mine;
  for (int b = b0; b < b1; ++b) {
    unit_start[b] = run;
    run += units_of(b, false);
  }
  if (threadIdx.x == 0) unit_start[M] = total;
}

// ---------------------------------------------------------------- k_score_selective

constexpr int pow2_floor(int x) {
  int p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}

template <int DT, int D>
struct SelShape {
  static constexpr int ES = (DT == ZGR_F32) ? 4 : 2;   // bytes per element
  static constexpr int VEC = 16 / ES;                  // elements per 16-byte load
  static constexpr int RAW = D * ES / 64;              // lanes per row at 64 bytes each
  // lanes per candidate: a power of two (shuffle groups), at most one wave
  static constexpr int G = RAW < 1 ? 1 : (RAW > 64 ? 64 : pow2_floor(RAW));
  static constexpr int NV = D * ES / (16 * G);         // 16-byte loads per lane per row
  static constexpr int NG = kThreads / G;              // candidates in flight per block
  static_assert(D * ES % (16 * G) == 0, "hidden size must split into 16-byte lane chunks");
};

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void k_score_selective(
    const int32_t* __restrict__ unit_start, int32_t M, DevTable tab,
    const int32_t* __restrict__ row_in, const void* __restrict__ hidden,
    const void* __restrict__ W, float* __restrict__ z, int64_t ldz) {
  using S = SelShape<DT, D>;
  constexpr int G = S::G, NV = S::NV, VEC = S::VEC, NG = S::NG, ES = S::ES;
  __shared__ uint16_t lst[kDenseTile];
  __shared__ int lst_count;
  const int gl = threadIdx.x % G;   // lane within the candidate group
  const int grp = threadIdx.x / G;  // group within the block
  const int lane = threadIdx.x & 63;
  const int total = unit_start[M];
  const char* Wb = (const char*)W;
  for (int u = blockIdx.x; u < total; u += gridDim.x) {
    // beam owning unit u: the last b with unit_start[b] <= u
    int lo = 0, hi = M;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (unit_start[mid] <= u)
        lo = mid;
      else
        hi = mid;
    }
    const int b = lo;
    const int tile = u - unit_start[b];
    const int r = row_in[b];
    // this lane's share of h_b, widened to float, kept in registers
    float h[NV * VEC];
    const char* hb = (const char*)hidden + (int64_t)b * D * ES;
#pragma unroll
    for (int c = 0; c < NV; ++c) load16<DT>(hb + (int64_t)(c * G + gl) * 16, &h[c * VEC]);
    float* zb = z + (int64_t)b * ldz;
    auto score = [&](int token, int slot) {
      const char* wr = Wb + (int64_t)token * D * ES;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        float w[VEC];
        load16<DT>(wr + (int64_t)(c * G + gl) * 16, w);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc = fmaf(w[e], h[c * VEC + e], acc);
      }
#pragma unroll
      for (int o = G / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
      if (gl == 0) zb[slot] = acc;
    };
    if (tab.fmt == ZGR_FMT_SPARSE) {
      const int base = tab.row_ptr[r];
      const int n = tab.row_ptr[r + 1] - base;
      const int j0 = tile * kSparseTile, j1 = min(n, j0 + kSparseTile);
      for (int j = j0 + grp; j < j1; j += NG) score(tab.tok[base + j], j);
    } else {
      // compact this tile's set bits into an LDS token list (a local, per-tile
      // list; slots stay token-addressed)
      const int v0 = tile * kDenseTile;
      const int w0 = v0 >> 5;
      const int nw = min(kDenseTile / 32, tab.words - w0);
      __syncthreads();  // previous unit's readers are done with lst
      if (threadIdx.x < 64) {
        const uint32_t word = (lane < nw) ? tab.bits[(int64_t)r * tab.words + w0 + lane] : 0u;
        const int pc = __popc(word);
        const int incl = wave_incl_scan(pc);
        int pos = incl - pc;
        uint32_t x = word;
        while (x) {
          const int k = __ffs(x) - 1;
          x &= x - 1;
          lst[pos++] = (uint16_t)(v0 + lane * 32 + k);
        }
        if (lane == 63) lst_count = incl;
      }
      __syncthreads();
      const int cnt = lst_count;
      for (int i = grp; i < cnt; i += NG) {
        const int v = lst[i];
        score(v, v);
      }
    }
  }
}

// ---------------------------------------------------------------- k_beam_reduce

// Visit every legal candidate of row r: fn(slot, token).  Sparse: slot = rank
// j, token = tok[row_ptr[r] + j]; dense: slot = token = set bit of the row.
template <class F>
__device__ __forceinline__ void for_each_legal(const DevTable& tab, int r, F&& fn) {
  if (tab.fmt == ZGR_FMT_SPARSE) {
    const int base = tab.row_ptr[r];
    const int n = tab.row_ptr[r + 1] - base;
    for (int j = threadIdx.x; j < n; j += kThreads) fn(j, (int)tab.tok[base + j]);
  } else {
    const uint32_t* row = tab.bits + (int64_t)r * tab.words;
    for (int w = threadIdx.x; w < tab.words; w += kThreads) {
      uint32_t x = row[w];
      while (x) {
        const int v = (w << 5) + __ffs(x) - 1;
        x &= x - 1;
        fn(v, v);
      }
    }
  }
}

// z source: token-indexed (full projection, or any dense step) or slot-indexed
// (selective projection on a sparse step).
template <bool TOKEN_IDX>
__global__ __launch_bounds__(kThreads) void k_beam_reduce(
    DevTable tab, int32_t M, int32_t k_in, int32_t K, const int32_t* __restrict__ row_in,
    const float* __restrict__ cum_in, const float* __restrict__ z, int64_t ldz,
    float* __restrict__ slot_dbg, uint64_t* __restrict__ bkeys, int32_t* __restrict__ bcount,
    int32_t* __restrict__ err) {
  __shared__ float shf[kWaves];
  __shared__ int shi[kWaves + 1];
  __shared__ int hist[256];
  __shared__ int pos;
  const int b = blockIdx.x;
  const int r = row_in[b];
  const bool live = r >= 0 && r < tab.rows;
  if (!live) {
    if (threadIdx.x == 0) {
      bcount[b] = 0;
      if (r >= tab.rows) atomicOr(err, 1);
    }
    if (slot_dbg)
      for (int j = threadIdx.x; j < tab.stride; j += kThreads)
        slot_dbg[(int64_t)b * tab.stride + j] = -INFINITY;
    return;
  }
  const int n = tab.row_ptr[r + 1] - tab.row_ptr[r];
  const float* zb = z + (int64_t)b * ldz;
  auto zval = [&](int slot, int token) -> float { return TOKEN_IDX ? zb[token] : zb[slot]; };
  // log-softmax over the legal tokens only
  float m = -INFINITY;
  for_each_legal(tab, r, [&](int slot, int token) { m = fmaxf(m, zval(slot, token)); });
  m = block_max(m, shf);
  float s = 0.f;
  for_each_legal(tab, r, [&](int slot, int token) { s += __expf(zval(slot, token) - m); });
  s = block_sum(s, shf);
  const float lse = m + __logf(s);
  const float cum = cum_in[b];
  if (slot_dbg) {
    float* dbg = slot_dbg + (int64_t)b * tab.stride;
    for (int j = threadIdx.x; j < tab.stride; j += kThreads) dbg[j] = -INFINITY;
    __syncthreads();
    for_each_legal(tab, r, [&](int slot, int token) { dbg[slot] = zval(slot, token) - lse; });
  }
  const uint32_t code0 = (uint32_t)(b % k_in) * (uint32_t)tab.stride;
  auto key_of = [&](int slot, int token) {
    return make_key(cum + (zval(slot, token) - lse), code0 + (uint32_t)slot);
  };
  uint64_t* out = bkeys + (int64_t)b * K;
  if (threadIdx.x == 0) pos = 0;
  __syncthreads();
  if (n <= K) {
    for_each_legal(tab, r, [&](int slot, int token) {
      const int p = atomicAdd(&pos, 1);
      if (p < K) out[p] = key_of(slot, token);
    });
    if (threadIdx.x == 0) bcount[b] = n;
    return;
  }
  RadixSel sel{0, 0, K};
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[threadIdx.x] = 0;
    __syncthreads();
    for_each_legal(tab, r, [&](int slot, int token) {
      const uint64_t k = key_of(slot, token);
      if ((k & sel.mask) == sel.prefix) atomicAdd(&hist[(k >> shift) & 0xFF], 1);
    });
    __syncthreads();
    if (radix_narrow(sel, shift, hist, shi)) break;
  }
  for_each_legal(tab, r, [&](int slot, int token) {
    const uint64_t k = key_of(slot, token);
    if ((k & sel.mask) >= sel.prefix) {
      const int p = atomicAdd(&pos, 1);
      if (p < K) out[p] = k;
    }
  });
  if (threadIdx.x == 0) bcount[b] = K;
}

// ---------------------------------------------------------------- k_request_select

constexpr int kMaxSort = 1024;

__device__ void bitonic_sort_desc(uint64_t* a, int P) {
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += kThreads) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t x = a[i], y = a[l];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            a[i] = y;
            a[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_request_select(
    DevTable tab, int32_t t, int32_t L, int32_t k_in, int32_t K,
    const int32_t* __restrict__ row_in, const uint64_t* __restrict__ bkeys,
    const int32_t* __restrict__ bcount, int32_t* __restrict__ parent_out,
    int32_t* __restrict__ token_out, int32_t* __restrict__ row_out, float* __restrict__ cum_out,
    const int32_t* __restrict__ prefix_in, int32_t* __restrict__ prefix_out) {
  __shared__ uint64_t sel[kMaxSort];
  __shared__ int hist[256];
  __shared__ int shi[kWaves + 1];
  __shared__ int pos;
  const int q = blockIdx.x;  // request
  const int b0 = q * k_in;
  int mine = 0;
  for (int i = threadIdx.x; i < k_in; i += kThreads) mine += bcount[b0 + i];
  const int C = block_sum_i(mine, shi);
  const int nsel = min(C, K);
  const int slots = k_in * K;
  auto for_each_key = [&](auto&& fn) {
    for (int i = threadIdx.x; i < slots; i += kThreads) {
      const int bb = i / K, j = i - bb * K;
      if (j < bcount[b0 + bb]) fn(bkeys[(int64_t)(b0 + bb) * K + j]);
    }
  };
  if (threadIdx.x == 0) pos = 0;
  __syncthreads();
  if (C <= K) {
    for_each_key([&](uint64_t k) {
      const int p = atomicAdd(&pos, 1);
      if (p < K) sel[p] = k;
    });
  } else {
    RadixSel rs{0, 0, K};
    for (int shift = 56; shift >= 0; shift -= 8) {
      hist[threadIdx.x] = 0;
      __syncthreads();
      for_each_key([&](uint64_t k) {
        if ((k & rs.mask) == rs.prefix) atomicAdd(&hist[(k >> shift) & 0xFF], 1);
      });
      __syncthreads();
      if (radix_narrow(rs, shift, hist, shi)) break;
    }
    for_each_key([&](uint64_t k) {
      if ((k & rs.mask) >= rs.prefix) {
        const int p = atomicAdd(&pos, 1);
        if (p < K) sel[p] = k;
      }
    });
  }
  __syncthreads();
  int P = 1;
  while (P < K) P <<= 1;
  for (int i = nsel + threadIdx.x; i < P; i += kThreads) sel[i] = 0;  // 0 sorts last
  __syncthreads();
  bitonic_sort_desc(sel, P);
  const uint32_t S = (uint32_t)tab.stride;
  for (int o = threadIdx.x; o < K; o += kThreads) {
    const int64_t oi = (int64_t)q * K + o;
    if (o < nsel) {
      const uint64_t key = sel[o];
      const uint32_t code = 0xFFFFFFFFu - (uint32_t)key;
      const int bl = (int)(code / S);
      const int slot = (int)(code - (uint32_t)bl * S);
      const int b = b0 + bl;
      const int r = row_in[b];
      int token, next;
      if (tab.fmt == ZGR_FMT_SPARSE) {
        next = tab.row_ptr[r] + slot;
        token = tab.tok[next];
      } else {
        token = slot;
        const uint32_t* row = tab.bits + (int64_t)r * tab.words;
        int below = 0;
        const int wfull = slot >> 5;
        for (int w = 0; w < wfull; ++w) below += __popc(row[w]);
        below += __popc(row[wfull] & ((1u << (slot & 31)) - 1u));
        next = tab.row_ptr[r] + below;
      }
      parent_out[oi] = b;
      token_out[oi] = token;
      row_out[oi] = next;
      cum_out[oi] = float_of_ord((uint32_t)(key >> 32));
      if (prefix_out) {
        for (int l = 0; l < t - 1; ++l) prefix_out[oi * L + l] = prefix_in[(int64_t)b * L + l];
        prefix_out[oi * L + t - 1] = token;
        for (int l = t; l < L; ++l) prefix_out[oi * L + l] = -1;
      }
    } else {
      parent_out[oi] = -1;
      token_out[oi] = -1;
      row_out[oi] = -1;
      cum_out[oi] = -INFINITY;
      if (prefix_out)
        for (int l = 0; l < L; ++l) prefix_out[oi * L + l] = -1;
    }
  }
}

// ---------------------------------------------------------------- k_gemm_nt (MFMA)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kTileM = 128, kTileN = 128, kTileKBytes = 128;
constexpr int kLdsRow = kTileKBytes + 16;  // padded row pitch in bytes

// C[m][n] = sum_k A[m][k] * B[n][k]: A = hidden [M][D], B = W_t [N][D], both
// k-contiguous.  128x128 block tile, 4 waves each owning 64x64 as 2x2 MFMA
// 32x32 blocks, 128-byte k-slices staged through LDS with a register prefetch
// of the next slice.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_gemm_nt(const void* __restrict__ A,
                                                      const void* __restrict__ Bm,
                                                      float* __restrict__ C, int32_t M, int32_t N,
                                                      int32_t D, int64_t ldc) {
  constexpr int ES = (DT == ZGR_F32) ? 4 : 2;
  constexpr int TK = kTileKBytes / ES;  // k elements per slice
  __shared__ __attribute__((aligned(16))) char As[kTileM * kLdsRow];
  __shared__ __attribute__((aligned(16))) char Bs[kTileN * kLdsRow];
  const int nbm = (M + kTileM - 1) / kTileM;
  const int tm = blockIdx.x % nbm, tn = blockIdx.x / nbm;
  const int m0 = tm * kTileM, n0 = tn * kTileN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const char* Ab = (const char*)A;
  const char* Bb = (const char*)Bm;
  const int64_t rowbytes = (int64_t)D * ES;
  // global -> register staging: 4 x 16 bytes of A and of B per thread
  uint4 ra[4], rb[4];
  auto gload = [&](int kbyte) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = threadIdx.x + i * kThreads;
      const int row = c >> 3, col = (c & 7) * 16;
      const int gm = m0 + row, gn = n0 + row;
      ra[i] = (gm < M) ? *(const uint4*)(Ab + gm * rowbytes + kbyte + col) : make_uint4(0, 0, 0, 0);
      rb[i] = (gn < N) ? *(const uint4*)(Bb + gn * rowbytes + kbyte + col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = threadIdx.x + i * kThreads;
      const int row = c >> 3, col = (c & 7) * 16;
      *(uint4*)(As + row * kLdsRow + col) = ra[i];
      *(uint4*)(Bs + row * kLdsRow + col) = rb[i];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int half = lane >> 5, l32 = lane & 31;
  gload(0);
  for (int kb = 0; kb < (int)rowbytes; kb += kTileKBytes) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (kb + kTileKBytes < rowbytes) gload(kb + kTileKBytes);
    if constexpr (DT == ZGR_F32) {
      // per 8-wide k chunk: lanes 0-31 hold k 0..3, lanes 32-63 k 4..7 of their
      // row; four 32x32x2 MFMAs pair (k, k+4) - the same pairing for A and B.
#pragma unroll
      for (int kc = 0; kc < TK / 8; ++kc) {
        const int off = kc * 32 + half * 16;
        f32x4 a[2], bv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a[i] = *(const f32x4*)(As + (wm * 64 + i * 32 + l32) * kLdsRow + off);
          bv[i] = *(const f32x4*)(Bs + (wn * 64 + i * 32 + l32) * kLdsRow + off);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], bv[j][s], acc[i][j], 0, 0, 0);
      }
    } else {
      // per 16-wide k chunk: lanes 0-31 hold k 0..7, lanes 32-63 k 8..15.
#pragma unroll
      for (int kc = 0; kc < TK / 16; ++kc) {
        const int off = kc * 32 + half * 16;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint4 ua = *(const uint4*)(As + (wm * 64 + i * 32 + l32) * kLdsRow + off);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint4 ub = *(const uint4*)(Bs + (wn * 64 + j * 32 + l32) * kLdsRow + off);
            if constexpr (DT == ZGR_BF16) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, ua), __builtin_bit_cast(bf16x8, ub), acc[i][j], 0, 0, 0);
            } else {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(f16x8, ua), __builtin_bit_cast(f16x8, ub), acc[i][j], 0, 0, 0);
            }
          }
        }
      }
    }
  }
  // 32x32 accumulator layout: lane -> column l32, register v -> row 8*(v/4) + 4*half + v%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (row < M && col < N) C[(int64_t)row * ldc + col] = acc[i][j][v];
      }
    }
}

// ---------------------------------------------------------------- decode helpers

__global__ void k_decode_init(int32_t* row, float* cum, int32_t B, int32_t K) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B * K) {
    row[i] = (i < B) ? 0 : -1;
    cum[i] = (i < B) ? 0.f : -INFINITY;
  }
}

__global__ void k_decode_final(const int32_t* row, const float* cum, const int32_t* prefix,
                               int32_t B, int32_t K, int32_t L, int32_t top_k, int64_t* item_out,
                               int32_t* sid_out, float* score_out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * top_k) return;
  const int q = i / top_k, o = i - q * top_k;
  const int src = q * K + o;
  const int r = row[src];
  item_out[i] = r;
  if (score_out) score_out[i] = cum[src];
  if (sid_out)
    for (int l = 0; l < L; ++l) sid_out[(int64_t)i * L + l] = (r >= 0) ? prefix[(int64_t)src * L + l] : -1;
}

template <int DT, int D>
hipError_t launch_sel_typed(const StepArgs& a, hipStream_t s) {
  const int grid = a.n_cu * 8;
  hipLaunchKernelGGL((k_score_selective<DT, D>), dim3(grid), dim3(kThreads), 0, s, a.unit_start, a.M,
                     a.tab, a.row_in, a.hidden, a.W, a.z, a.ldz);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_sel_d(const StepArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_sel_typed<DT, 64>(a, s);
    case 128: return launch_sel_typed<DT, 128>(a, s);
    case 256: return launch_sel_typed<DT, 256>(a, s);
    case 512: return launch_sel_typed<DT, 512>(a, s);
    case 768: return launch_sel_typed<DT, 768>(a, s);
    case 1024: return launch_sel_typed<DT, 1024>(a, s);
    case 2048: return launch_sel_typed<DT, 2048>(a, s);
    case 4096: return launch_sel_typed<DT, 4096>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool supported_hidden_size(int d) {
  return d == 64 || d == 128 || d == 256 || d == 512 || d == 768 || d == 1024 || d == 2048 ||
         d == 4096;
}

hipError_t launch_selective_score(const StepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_units, dim3(1), dim3(1024), 0, s, a.row_in, a.M, a.tab, a.nlegal,
                     a.unit_start, a.err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.dtype) {
    case ZGR_F32: return launch_sel_d<ZGR_F32>(a, s);
    case ZGR_BF16: return launch_sel_d<ZGR_BF16>(a, s);
    case ZGR_F16: return launch_sel_d<ZGR_F16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_full_projection(const StepArgs& a, hipStream_t s) {
  const int V = a.tab.V;
  const int nbm = (a.M + kTileM - 1) / kTileM, nbn = (V + kTileN - 1) / kTileN;
  const dim3 grid(nbm * nbn);
  switch (a.dtype) {
    case ZGR_F32:
      hipLaunchKernelGGL(k_gemm_nt<ZGR_F32>, grid, dim3(kThreads), 0, s, a.hidden, a.W, a.z, a.M, V,
                         a.d, a.ldz);
      break;
    case ZGR_BF16:
      hipLaunchKernelGGL(k_gemm_nt<ZGR_BF16>, grid, dim3(kThreads), 0, s, a.hidden, a.W, a.z, a.M, V,
                         a.d, a.ldz);
      break;
    case ZGR_F16:
      hipLaunchKernelGGL(k_gemm_nt<ZGR_F16>, grid, dim3(kThreads), 0, s, a.hidden, a.W, a.z, a.M, V,
                         a.d, a.ldz);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_beam_reduce(const StepArgs& a, bool token_indexed, hipStream_t s) {
  if (token_indexed)
    hipLaunchKernelGGL(k_beam_reduce<true>, dim3(a.M), dim3(kThreads), 0, s, a.tab, a.M, a.k_in, a.K,
                       a.row_in, a.cum_in, a.z, a.ldz, a.slot_dbg, a.bkeys, a.bcount, a.err);
  else
    hipLaunchKernelGGL(k_beam_reduce<false>, dim3(a.M), dim3(kThreads), 0, s, a.tab, a.M, a.k_in, a.K,
                       a.row_in, a.cum_in, a.z, a.ldz, a.slot_dbg, a.bkeys, a.bcount, a.err);
  return hipGetLastError();
}

hipError_t launch_request_select(const StepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_request_select, dim3(a.B), dim3(kThreads), 0, s, a.tab, a.t, a.L, a.k_in, a.K,
                     a.row_in, a.bkeys, a.bcount, a.parent_out, a.token_out, a.row_out, a.cum_out,
                     a.prefix_in, a.prefix_out);
  return hipGetLastError();
}

hipError_t launch_decode_init(int32_t* row, float* cum, int32_t B, int32_t K, hipStream_t s) {
  const int n = B * K;
  hipLaunchKernelGGL(k_decode_init, dim3((n + 255) / 256), dim3(256), 0, s, row, cum, B, K);
  return hipGetLastError();
}

hipError_t launch_decode_final(const int32_t* row, const float* cum, const int32_t* prefix,
                               int32_t B, int32_t K, int32_t L, int32_t top_k, int64_t* item_out,
                               int32_t* sid_out, float* score_out, hipStream_t s) {
  const int n = B * top_k;
  hipLaunchKernelGGL(k_decode_final, dim3((n + 255) / 256), dim3(256), 0, s, row, cum, prefix, B, K,
                     L, top_k, item_out, sid_out, score_out);
  return hipGetLastError();
}

}  // namespace zgr
