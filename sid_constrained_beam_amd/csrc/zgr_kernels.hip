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
//   k_units            sparse steps, per beam: its run of legal tokens (the
//                      row, or its tokens in one codebook eighth when the
//                      table has a slice directory) and the run's work units;
//                      an exclusive scan per 1,024-beam chunk (not over
//                      candidates: slot addresses never depend on other
//                      beams) and each unit's place.
//   k_score_sparse     persistent grid over a sparse step's units, a slice per
//                      XCD when sliced: each wave scores its units' candidates,
//                      z = W_t[token] . h_beam with the weight row read in
//                      place by a group of lanes (16-byte loads), h kept in
//                      registers, a lane-group shuffle reduction, z stored at
//                      the slot (the token's rank in the row).
//   k_score_selective  the same on dense rows: persistent grid over (beam,
//                      tile) pairs, the set bits of a 1024-token tile of the
//                      row's bitmap, tiles split over the XCDs so each XCD's L2
//                      holds its tiles' weight rows; z stored at the token's
//                      legal rank.
//   k_score_staged     comparison on dense rows: weight-row tiles staged in LDS
//                      once per group of beams held in registers.
//   k_gemm_nt          full projection Z = H . W_t^T on MFMA (fp32, bf16, f16
//                      inputs; fp32 accumulate), Z row = beam, column = token;
//   k_gemm_small       the same product for few beams (first step): 16x16 MFMA.
//   k_request_step     one block per request: legal-only log-sum-exp of each
//                      beam, cand = cum + (z - lse) for every legal candidate,
//                      the best K by an LDS distance histogram, rank sort, decode
//                      (parent, token, cum) and advance: next row = row_ptr[r]
//                      + slot (sparse: the position is the next row) or
//                      row_ptr[r] + rank directory + popcount (dense); prefix
//                      gather.  On light sparse steps it also does the
//                      selective projection itself (one launch per step).
//
// Ranking key (64 bits, larger = better): high word = order-preserving image
// of the float cand, low word = ~(beam_rank * S_t + slot).  Keys are unique,
// so every selection is exact and deterministic; equal scores fall to the
// lower beam rank, then the lower slot (slot order = token order).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "zgr_internal.h"

namespace zgr {

namespace {

constexpr int kThreads = 256;
// Selective scoring: candidates a lane group scores at once when a row takes
// at most 6 loads per lane (a power of two)
constexpr int kSelU = 2;
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

// ---------------------------------------------------------------- wave / block helpers

// Value of x held by lane (lane ^ O), for a compile-time O in {1, ..., 32}, every
// lane of the wave active.  Within a 16-lane row the exchange is a DPP move
// (O = 1, 2: quad permutations 0xB1 and 0x4E; O = 4: row_shl:4 into banks 0
// and 2, row_shr:4 into banks 1 and 3; O = 8: row_ror:8), so it stays off the
// LDS crossbar; O = 16 and 32 cross rows and use a permute.
template <int O>
__device__ __forceinline__ int xor_lane(int x) {
  static_assert(O == 1 || O == 2 || O == 4 || O == 8 || O == 16 || O == 32, "lane xor");
  if constexpr (O == 1) return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false);
  else if constexpr (O == 2) return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false);
  else if constexpr (O == 4) {
    const int t = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xf, 0x5, false);
    return __builtin_amdgcn_update_dpp(t, x, 0x114, 0xf, 0xa, false);
  } else if constexpr (O == 8) return __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false);
  else return __shfl_xor(x, O);
}
template <int O>
__device__ __forceinline__ float xor_lane(float v) {
  return __int_as_float(xor_lane<O>(__float_as_int(v)));
}
template <int O>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  return (uint32_t)xor_lane<O>((int)v);
}
template <int O>
__device__ __forceinline__ uint64_t xor_lane(uint64_t v) {
  const uint32_t lo = xor_lane<O>((uint32_t)v), hi = xor_lane<O>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
// Calls f(integral_constant<O>) for O, O/2, ..., 1: the butterfly stages of a
// reduction over an aligned group of 2*O lanes.
template <int O, typename F>
__device__ __forceinline__ void xor_down(F&& f) {
  if constexpr (O >= 1) {
    f(std::integral_constant<int, O>{});
    xor_down<O / 2>(f);
  }
}
// The same stages for a group width W known only at run time (a power of two
// in [1, 64], equal across the wave): the switch falls through from the widest
// stage the width needs down to offset 1, so each stage is compiled once.
template <typename F>
__device__ __forceinline__ void xor_down_width(int W, F&& f) {
  switch (W) {
    case 64: f(std::integral_constant<int, 32>{}); [[fallthrough]];
    case 32: f(std::integral_constant<int, 16>{}); [[fallthrough]];
    case 16: f(std::integral_constant<int, 8>{}); [[fallthrough]];
    case 8: f(std::integral_constant<int, 4>{}); [[fallthrough]];
    case 4: f(std::integral_constant<int, 2>{}); [[fallthrough]];
    case 2: f(std::integral_constant<int, 1>{}); [[fallthrough]];
    default: break;
  }
}
// Sum of v over an aligned group of G lanes (G a power of two, at most 64),
// every lane of the group active; every lane ends with the sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  xor_down<G / 2>([&](auto o) { v += xor_lane<decltype(o)::value>(v); });
  return v;
}
// Inclusive prefix sum over the 64 lanes, with DPP moves only (no LDS
// crossbar permutes): shifts by 1, 2, 4 and 8 within each 16-lane row (a
// lane without a source adds 0), then lane 15 of rows 0 and 2 is broadcast
// into rows 1 and 3, and lane 31 (the total of rows 0-1) into rows 2 and 3.
// DPP controls: row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 =
// 0x143; row masks 0xa (rows 1, 3) and 0xc (rows 2, 3).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

// Exclusive prefix over the NT threads of a block (fixed order); *total = sum.
// sh must hold NT/64 ints.
template <int NT>
__device__ int block_excl_scan(int v, int* sh, int* total) {
  constexpr int NW = NT / 64;
  const int incl = wave_incl_scan(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 63) sh[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < w) before += sh[i];
    all += sh[i];
  }
  *total = all;
  return before + incl - v;
}

template <int NT>
__device__ uint64_t block_max_u64(uint64_t v, uint64_t* sh) {
  constexpr int NW = NT / 64;
  xor_down<32>([&](auto o) {
    const uint64_t u = xor_lane<decltype(o)::value>(v);
    v = u > v ? u : v;
  });
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = sh[i] > r ? sh[i] : r;
  return r;
}
template <int NT>
__device__ uint64_t block_min_u64(uint64_t v, uint64_t* sh) {
  constexpr int NW = NT / 64;
  xor_down<32>([&](auto o) {
    const uint64_t u = xor_lane<decltype(o)::value>(v);
    v = u < v ? u : v;
  });
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = sh[i] < r ? sh[i] : r;
  return r;
}

// State of a radix select for the `need` largest of a set of distinct 64-bit
// keys, 8 bits per pass from the top: keys whose bits under `mask` equal
// `prefix` are still undecided; keys above that prefix are already selected.
struct RadixSel {
  uint64_t prefix;
  uint64_t mask;
  int need;
};

// hist[256] holds the digit counts of the undecided keys at `shift`: pick the
// digit holding the need-th largest and narrow.  True when every key under the
// new prefix is selected.
template <int NT>
__device__ bool radix_narrow(RadixSel& s, int shift, const int* hist, int* sh) {
  const int d = 255 - (int)threadIdx.x;  // thread i looks at digit 255 - i
  const int c = (threadIdx.x < 256) ? hist[d] : 0;
  int total;
  const int excl = block_excl_scan<NT>(c, sh, &total);
  __shared__ int pick_digit, pick_above, pick_count;
  if (threadIdx.x < 256 && excl < s.need && excl + c >= s.need) {
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

// ---------------------------------------------------------------- dense rows
//
// A dense row is read one 32-token word at a time: the word's legal bits and
// the row's legal count before the word (legal rank of its first set bit).
// With the bitmap encoding both are stored (bitmap + rank directory).  With
// the next-row matrix encoding they come from the word's 32 cells: a cell
// >= 0 is a legal token, and its value minus the row's base is its legal
// rank (a row's entries are numbered consecutively in token order).
struct DWord {
  uint32_t bits;
  int rank;
};

__device__ __forceinline__ bool is_dense(int fmt) { return fmt != ZGR_FMT_SPARSE; }

// NX selects the encoding at compile time, so the bitmap instantiations of
// every kernel carry none of the next-row matrix code (nor its registers).
template <bool NX>
__device__ __forceinline__ DWord dense_word(const DevTable& tab, int64_t r, int w) {
  if constexpr (!NX) {
    const int64_t i = r * tab.words + w;
    return {tab.bits[i], (int)tab.rank[i]};
  } else {
    const int32_t* nx = tab.next + r * (int64_t)tab.V + (w << 5);
    const int nk = min(32, tab.V - (w << 5));
    uint32_t b = 0;
    int first = -1;
    if (nk == 32 && (tab.V & 3) == 0) {
      // highest quad first, so `first` ends at the word's lowest legal token
      for (int q = 7; q >= 0; --q) {
        const int4 v = ((const int4*)nx)[q];
        const int c[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 3; k >= 0; --k)
          if (c[k] >= 0) {
            b |= 1u << (4 * q + k);
            first = c[k];
          }
      }
    } else {
      for (int k = nk - 1; k >= 0; --k) {
        const int v = nx[k];
        if (v >= 0) {
          b |= 1u << k;
          first = v;
        }
      }
    }
    return {b, first >= 0 ? first - tab.row_ptr[r] : 0};
  }
}

// ---------------------------------------------------------------- k_units

// Before the selective projection of a sparse step: every beam's run of
// legal tokens (the whole row, or with a slice directory its tokens in one
// eighth of the codebook) and the run's units of up to kSparseTile
// candidates.  Block (chunk q, slice x) takes beams [1024 q, 1024 q + 1024)
// of slice x, one per thread: it scans its beams' units, writes the chunk's
// unit total to ctot[x][q] and each unit's place (beam, first entry of the
// token list, first slot, size) to umeta[x][q][unit], so the projection reads
// a unit's place with one load and no block scans more than 1,024 beams.
// Blocks are numbered q * slices + x.
template <bool SLICED>
__global__ __launch_bounds__(1024) void k_units(const int32_t* __restrict__ row_in, int32_t M,
                                                DevTable tab, int32_t* __restrict__ ctot,
                                                int4* __restrict__ umeta, int64_t chunk_cap,
                                                int32_t* __restrict__ err) {
  constexpr int NSL = SLICED ? kSlices : 1;
  const int x = (int)blockIdx.x % NSL, q = (int)blockIdx.x / NSL;
  const int nq = (M + 1023) / 1024;
  __shared__ int sh[16];
  const int b = q * 1024 + (int)threadIdx.x;
  int n = 0, first = 0, sb = 0;
  if (b < M) {
    const int r = row_in[b];
    const bool live = r >= 0 && r < tab.rows;
    if (r >= tab.rows && x == 0) atomicOr(err, 1);
    const int rr = live ? r : 0;
    const int lo = tab.row_ptr[rr], hi = tab.row_ptr[rr + 1];
    n = live ? hi - lo : 0;
    if constexpr (SLICED) {
      // the row's run of slice x: entries [first, end) of the row (entry i of
      // the directory: the row's tokens below the end of slice i)
      const uint4 d = *reinterpret_cast<const uint4*>(tab.sdir + (int64_t)rr * kSlices);
      const uint32_t w[4] = {d.x, d.y, d.z, d.w};
      auto entry = [&](int i) { return (int)((i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu)); };
      first = (live && x > 0) ? entry(x - 1) : 0;
      const int end = (x + 1 < kSlices) ? entry(x) : n;
      n = live ? end - first : 0;
    }
    sb = lo + first;
  }
  const int units = (n + kSparseTile - 1) / kSparseTile;
  int tot;
  const int s0 = block_excl_scan<1024>(units, sh, &tot);
  if (threadIdx.x == 0) ctot[x * nq + q] = tot;
  int4* um = umeta + ((int64_t)x * nq + q) * chunk_cap;
  for (int k = 0; k < units; ++k)
    um[s0 + k] = make_int4(b, sb + k * kSparseTile, first + k * kSparseTile,
                           min(kSparseTile, n - k * kSparseTile));
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
  static constexpr int NG = kThreads / G;              // lane groups per block
  // candidates a lane group scores at once (their row loads in flight together)
  static constexpr int U = NV <= 6 ? (kSelU < G ? kSelU : G) : 1;
  static_assert(D * ES % (16 * G) == 0, "hidden size must split into 16-byte lane chunks");
};

// Sums of U candidates' partial dot products over a group of G lanes (U a
// power of two, U <= G): U - 1 shuffles halve the vector (each lane keeps
// the half that its partner does not), then a butterfly over the remaining
// G / U lanes.  Lane gl ends with the sum of candidate gl / (G / U).
template <int U, int N, int O>
__device__ __forceinline__ void group_halve(float (&acc)[U], int gl) {
  if constexpr (N > 1) {
    const bool hi = (gl & O) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float send = hi ? acc[i] : acc[i + N / 2];
      const float keep = hi ? acc[i + N / 2] : acc[i];
      acc[i] = keep + xor_lane<O>(send);
    }
    group_halve<U, N / 2, O / 2>(acc, gl);
  }
}
template <int G, int U>
__device__ __forceinline__ float group_sum_multi(float (&acc)[U], int gl) {
  group_halve<U, U, G / 2>(acc, gl);
  return group_sum<G / U>(acc[0]);
}

typedef __bf16 __attribute__((ext_vector_type(2))) bf16x2_t;

// A lane group's gather-dot: the group's share of one beam's hidden vector
// in registers (load_h), then U candidates at once (score): tok(u) gives
// candidate u's token (callers clamp it to a real candidate, so every load is
// in bounds) and slot(u) its z index; only the first nvalid are stored.  The
// hidden share and the weight loads stay packed as loaded (16-bit types: two
// values per register) and are widened element by element in the FMA chain,
// which halves their registers; the FMA order is the element order.
template <int DT, int D>
struct GatherDot {
  using S = SelShape<DT, D>;
  static constexpr int G = S::G, NV = S::NV, ES = S::ES, U = S::U;
  const char* Wb;
  const char* hidden;
  int gl;  // lane within the candidate group
  uint4 h[NV];
  __device__ __forceinline__ void load_h(int b) {
    const char* hb = hidden + (int64_t)b * D * ES;
#pragma unroll
    for (int c = 0; c < NV; ++c) h[c] = *(const uint4*)(hb + (int64_t)(c * G + gl) * 16);
  }
  // acc += the dot product of two packed 16-byte chunks, in element order
  static __device__ __forceinline__ float dot16(const uint4& w, const uint4& x, float acc) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w}, b[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == ZGR_F32) {
        acc = fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), acc);
      } else if constexpr (DT == ZGR_BF16) {
        // two bf16 products (exact in f32) and the sum in one instruction
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[i]),
                                              __builtin_bit_cast(bf16x2_t, b[i]), acc, false);
      } else {
        acc = fmaf(f16_to_f32(a[i] & 0xFFFFu), f16_to_f32(b[i] & 0xFFFFu), acc);
        acc = fmaf(f16_to_f32(a[i] >> 16), f16_to_f32(b[i] >> 16), acc);
      }
    }
    return acc;
  }
  template <typename Tok, typename Slot>
  __device__ __forceinline__ void score(float* zb, Tok&& tok, Slot&& slot, int nvalid) {
    const char* wr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) wr[u] = Wb + (int64_t)tok(u) * D * ES;
    uint4 w[U][NV];
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
      for (int u = 0; u < U; ++u) w[u][c] = *(const uint4*)(wr[u] + (int64_t)(c * G + gl) * 16);
    // the packed hidden share is opaque to the compiler here, so it widens it
    // at each use instead of hoisting a widened copy (twice the registers)
    if constexpr (DT != ZGR_F32) {
#pragma unroll
      for (int c = 0; c < NV; ++c) asm volatile("" : "+v"(h[c].x), "+v"(h[c].y), "+v"(h[c].z), "+v"(h[c].w));
    }
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc[u] = 0.f;
#pragma unroll
      for (int c = 0; c < NV; ++c) acc[u] = dot16(w[u][c], h[c], acc[u]);
    }
    const float v = group_sum_multi<G, U>(acc, gl);
    const int mine = gl / (G / U);
    if (gl % (G / U) == 0 && mine < nvalid) zb[slot(mine)] = v;
  }
};

// Selective projection of a sparse step: units (a beam's run of up to
// kSparseTile candidates, placed by k_units) in one contiguous range per
// block, each wave taking every NW-th unit of the range on its own (no block
// barrier).  With a slice directory the blocks are dealt to the XCDs in turn
// (block i runs on XCD i mod 8), so block i takes slice i mod kSlices: the
// units of the beams' runs of legal tokens in that eighth of the codebook,
// whose weight rows then stay in the XCD's own L2 (the grid is a multiple of
// kSlices).  A kernel of its own, so its register count (and so its
// occupancy) is not the dense path's.
// Beam chunks of the unit kernel a sparse projection can take (its LDS
// prefix of chunk totals): M <= 1024 kMaxUnitChunks beams.
constexpr int kMaxUnitChunks = kMaxUnitChunksHost;

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void k_score_sparse(
    const int32_t* __restrict__ ctot, const int4* __restrict__ umeta, int64_t chunk_cap,
    int32_t M, DevTable tab, const void* __restrict__ hidden, const void* __restrict__ W,
    float* __restrict__ z, int64_t ldz) {
  using GD = GatherDot<DT, D>;
  constexpr int G = GD::G, U = GD::U;
  constexpr int NW = kThreads / 64, GW = 64 / G;  // waves per block, lane groups per wave
  GD gd;
  gd.Wb = (const char*)W;
  gd.hidden = (const char*)hidden;
  gd.gl = threadIdx.x % G;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x / 64, wg = (threadIdx.x % 64) / G;
  // slice x of the blocks' residues mod nsl (one slice, whole rows, without
  // a directory); the slice's units are numbered over its beam chunks in
  // order, from the chunks' totals (prefix in LDS, by wave 0)
  __shared__ int cpre[kMaxUnitChunks + 1];
  const int nsl = tab.sdir != nullptr ? kSlices : 1;
  const int x = (int)blockIdx.x % nsl;
  const int lb = (int)blockIdx.x / nsl, nb = (int)gridDim.x / nsl;
  const int nq = (M + 1023) / 1024;
  if (wv == 0) {
    int carry = 0;
    for (int i0 = 0; i0 < nq; i0 += 64) {
      const int v = i0 + lane < nq ? ctot[x * nq + i0 + lane] : 0;
      const int incl = wave_incl_scan(v);
      if (i0 + lane < nq) cpre[i0 + lane] = carry + incl - v;
      carry += __shfl(incl, 63);
    }
    if (lane == 0) cpre[nq] = carry;
  }
  __syncthreads();
  const int total = cpre[nq];
  const int chunk = (total + nb - 1) / nb;
  const int u0 = lb * chunk, u1 = min(total, u0 + chunk);
  const int4* um = umeta + (int64_t)x * nq * chunk_cap;
  // unit u of the slice: chunk q (the last with cpre[q] <= u), its unit u - cpre[q]
  auto place_of = [&](int u) {
    int lo = 0, hi = nq;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cpre[mid] <= u)
        lo = mid;
      else
        hi = mid;
    }
    return (int64_t)lo * chunk_cap + (u - cpre[lo]);
  };
  // each wave takes every NW-th unit of the block's range on its own (no
  // block barrier); lane i holds the place of the wave's i-th unit of a
  // round, and the next unit's tokens load while a unit is scored, so a
  // unit waits only on its weight rows
  for (int ub = u0 + wv; ub < u1; ub += NW * 64) {
    const int ui = ub + lane * NW;
    const int4 m = ui < u1 ? um[place_of(ui)] : make_int4(0, 0, 0, 0);
    const int nr = min(64, (u1 - ub + NW - 1) / NW);
    int tk;
    {
      const int e0 = __builtin_amdgcn_readlane(m.y, 0), cnt = __builtin_amdgcn_readlane(m.w, 0);
      tk = lane < cnt ? (int)tab.tok[e0 + lane] : 0;
    }
    for (int i = 0; i < nr; ++i) {
      const int b = __builtin_amdgcn_readlane(m.x, i);
      const int j0 = __builtin_amdgcn_readlane(m.z, i), cnt = __builtin_amdgcn_readlane(m.w, i);
      int tk_next = 0;
      if (i + 1 < nr) {
        const int e0n = __builtin_amdgcn_readlane(m.y, i + 1);
        const int cntn = __builtin_amdgcn_readlane(m.w, i + 1);
        tk_next = lane < cntn ? (int)tab.tok[e0n + lane] : 0;
      }
      gd.load_h(b);
      float* zb = z + (int64_t)b * ldz;
      // the trip count is uniform over the wave (the token shuffle needs
      // every lane); a group past the unit's end stores nothing
      for (int jb = 0; jb < cnt; jb += GW * U) {
        const int j = jb + wg;
        const int nv = min(U, (cnt - j + GW - 1) / GW);
        gd.score(
            zb, [&](int u) { return __shfl(tk, min(j + u * GW, cnt - 1)); },
            [&](int u) { return j0 + j + u * GW; }, nv);
      }
      tk = tk_next;
    }
  }
}

template <int DT, int D, bool NX>
__global__ __launch_bounds__(kThreads) void k_score_selective(
    const int32_t* __restrict__ unit_start, int32_t M, DevTable tab,
    const int32_t* __restrict__ row_in, const void* __restrict__ hidden,
    const void* __restrict__ W, float* __restrict__ z, int64_t ldz, int32_t tt) {
  using S = SelShape<DT, D>;
  constexpr int G = S::G, NV = S::NV, VEC = S::VEC, NG = S::NG, ES = S::ES;
  __shared__ uint16_t lst[kDenseTile];
  __shared__ int lpos[kDenseTile];
  __shared__ int lst_count;
  const int gl = threadIdx.x % G;   // lane within the candidate group
  const int grp = threadIdx.x / G;  // group within the block
  const int lane = threadIdx.x & 63;
  const char* Wb = (const char*)W;
  float h[NV * VEC];  // this lane's share of the unit's hidden vector
  auto load_h = [&](int b) {
    const char* hb = (const char*)hidden + (int64_t)b * D * ES;
#pragma unroll
    for (int c = 0; c < NV; ++c) load16<DT>(hb + (int64_t)(c * G + gl) * 16, &h[c * VEC]);
  };
  // U candidates of one beam per lane group: tok(u) gives candidate u's token
  // (callers clamp it to a real candidate, so every load is in bounds), and
  // slot(u) its z index; only the first nvalid are stored
  constexpr int U = S::U;
  auto score_u = [&](float* zb, auto&& tok, auto&& slot, int nvalid) {
    const char* wr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) wr[u] = Wb + (int64_t)tok(u) * D * ES;
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = 0.f;
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      float w[U][VEC];
#pragma unroll
      for (int u = 0; u < U; ++u) load16<DT>(wr[u] + (int64_t)(c * G + gl) * 16, w[u]);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[u] = fmaf(w[u][e], h[c * VEC + e], acc[u]);
    }
    const float v = group_sum_multi<G, U>(acc, gl);
    const int mine = gl / (G / U);
    if (gl % (G / U) == 0 && mine < nvalid) zb[slot(mine)] = v;
  };

  // Dense rows: every live beam has the same tiles of tt tokens (a multiple
  // of 32, at most kDenseTile; the host sizes a tile's weight rows to a
  // fraction of one XCD's L2), so (tile, beam) pairs are enumerated
  // directly.  With at least 8 tiles and enough beams to keep every block
  // busy, the blocks of one XCD (blocks are dealt to the 8 XCDs in turn) take
  // only the tiles of their own residue, one tile at a time, so the weight
  // rows a tile gathers stay in that XCD's L2 instead of every XCD streaming
  // all of W_t.  Otherwise one flat range with a beam's tiles side by side
  // (neighbouring blocks share its bitmap row and hidden vector).
  const int tiles = (tab.V + tt - 1) / tt;
  const bool by_xcd = tiles >= 8 && (gridDim.x & 7) == 0 && M >= (int)gridDim.x / 8;
  const int stride_b = by_xcd ? (int)gridDim.x / 8 : (int)gridDim.x;
  const int first_b = by_xcd ? (int)blockIdx.x / 8 : (int)blockIdx.x;
  const int t_step = by_xcd ? 8 : 1;
  const int t_first = by_xcd ? (int)blockIdx.x % 8 : 0;
  // Wave 0 fetches the next pair's bitmap words while the block scores the
  // current pair (pf_pb: the pair they belong to, -1 = none).
  int pf_pb = -1;
  DWord pf_dw{0u, 0};
  for (int tile = t_first; tile < tiles; tile += t_step) {
    // without the XCD split, pairs run over (tile, beam) in one flat range
    const int nb = by_xcd ? M : M * tiles;
    for (int pb = first_b; pb < nb; pb += stride_b) {
      const int b = by_xcd ? pb : pb / tiles;  // flat range: a beam's tiles side by side
      const int tl = by_xcd ? tile : pb % tiles;
      const int r = row_in[b];
      if (r < 0 || r >= tab.rows) continue;  // the request kernel reports bad rows
      load_h(b);
      float* zb = z + (int64_t)b * ldz;
      // this tile's set bits as an LDS token list with their legal ranks
      // (z of a dense row is stored by legal rank)
      const int v0 = tl * tt;
      const int w0 = v0 >> 5;
      const int nw = min(tt >> 5, tab.words - w0);
      __syncthreads();  // previous pair's readers are done with lst
      if (threadIdx.x < 64) {
        const DWord dw = (pf_pb == pb) ? pf_dw : (lane < nw) ? dense_word<NX>(tab, r, w0 + lane) : DWord{0u, 0};
        // the next pair of this block within the tile (its loads overlap the scoring below)
        pf_pb = -1;
        const int pn = pb + stride_b;
        if (pn < nb) {
          const int bn = by_xcd ? pn : pn / tiles;
          const int tn = by_xcd ? tile : pn % tiles;
          const int rn = row_in[bn];
          const int wn0 = (tn * tt) >> 5;
          if (rn >= 0 && rn < tab.rows) {
            pf_pb = pn;
            pf_dw = (lane < min(tt >> 5, tab.words - wn0)) ? dense_word<NX>(tab, rn, wn0 + lane) : DWord{0u, 0};
          }
        }
        const uint32_t word = dw.bits;
        int rk = dw.rank;
        const int pc = __popc(word);
        const int incl = wave_incl_scan(pc);
        int pos = incl - pc;
        uint32_t x = word;
        while (x) {
          const int k = __ffs(x) - 1;
          x &= x - 1;
          lst[pos] = (uint16_t)(v0 + lane * 32 + k);
          lpos[pos++] = rk++;
        }
        if (lane == 63) lst_count = incl;
      }
      __syncthreads();
      const int cnt = lst_count;
      for (int i = grp; i < cnt; i += NG * U) {
        const int nv = min(U, (cnt - i + NG - 1) / NG);
        score_u(
            zb, [&](int u) { return (int)lst[min(i + u * NG, cnt - 1)]; },
            [&](int u) { return lpos[i + u * NG]; }, nv);
      }
    }
    if (!by_xcd) break;  // the flat range covered every tile
  }
}

// LDS-staged projection of a dense step (a comparison, chosen only when a
// plan is told to): the weight rows are staged in LDS and shared by the
// beams of a block.  A block (kStageThreads threads, one per CU) takes work
// items (a group of BG beams, a codebook slice): the blocks of XCD x (blocks
// are dealt to the 8 XCDs in turn) take slice x, an eighth of the row's
// bitmap words, so an XCD reads only its slice's weight rows and its blocks
// stream them in the same order.  Each wave keeps BW beams' hidden vectors in
// registers (lane l holds 16-byte chunks l, 64 + l, ... of each) and their
// bitmap words of a 64-word part of the slice in LDS.  The slice's rows are
// read TT at a time, a contiguous run of W_t, in coalesced 16-byte loads by
// the whole block (three tiles in flight in registers, three LDS buffers, one
// barrier per tile), and every legal (beam, token) pair of the tile is scored
// from LDS: a round takes the next legal token of each of the wave's beams,
// and one reduction sums the round's BW dot products.  A weight row then
// leaves L2 once per work item instead of once per legal pair: the traffic
// drops by the expected number of the block's beams that have the token
// legal (BG times the row density), at the price of a block barrier per tile
// and registers that allow two waves per SIMD.
constexpr int kStageThreads = 512;
constexpr int kStageTileBytes = 32 * 1024;  // one LDS buffer (three per block)
constexpr int kStageOut = 256;              // scores a wave holds before it stores them

template <int DT, int D>
struct StagedShape {
  static constexpr int ES = (DT == ZGR_F32) ? 4 : 2;
  static constexpr int RB = D * ES;      // bytes per weight row
  static constexpr int NV = RB / 1024;   // 16-byte chunks of a row per lane
  static constexpr int BW0 = 32 / (NV > 0 ? NV : 1);
  static constexpr int BW = pow2_floor(BW0 > 8 ? 8 : (BW0 < 1 ? 1 : BW0));  // beams per wave
  static constexpr int TT0 = kStageTileBytes / RB;
  static constexpr int TT = TT0 > 32 ? 32 : TT0;                 // tokens per tile
  static constexpr int TB = TT * RB;                             // bytes per tile
  static constexpr int LPT = TB / (16 * kStageThreads);          // 16-byte loads per thread
  static constexpr int NWV = kStageThreads / 64;
  static constexpr int BG = NWV * BW;  // beams per work item
  // f16 inputs would widen the hidden shares to f32 (twice the registers)
  static constexpr bool OK =
      DT != ZGR_F16 && RB % 1024 == 0 && LPT >= 1 && TB % (16 * kStageThreads) == 0;
};

template <int DT, int D, bool NX>
__global__ __launch_bounds__(kStageThreads) void k_score_staged(int32_t M, DevTable tab,
                                                                const int32_t* __restrict__ row_in,
                                                                const void* __restrict__ hidden,
                                                                const void* __restrict__ W,
                                                                float* __restrict__ z, int64_t ldz) {
  using SS = StagedShape<DT, D>;
  static_assert(SS::OK, "staged projection shape");
  constexpr int NV = SS::NV, BW = SS::BW, TT = SS::TT, LPT = SS::LPT, BG = SS::BG;
  constexpr int RC = SS::RB / 16;  // 16-byte chunks per row
  constexpr int GL = 64 / BW;      // lanes per beam after the reduction
  __shared__ uint4 stage[3][SS::TB / 16];
  // Each wave's scores wait in LDS (value, slot * BW + beam) and go to z in
  // batches, so no global store is in flight while the tile loads are: the
  // loads' wait then covers only the older tile.
  __shared__ float ov[SS::NWV][kStageOut];
  __shared__ int od[SS::NWV][kStageOut];
  __shared__ uint32_t wsh[SS::NWV][BW][64];
  __shared__ int rsh[SS::NWV][BW][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nx = (gridDim.x & 7) == 0 ? 8 : 1;
  const int x = (int)blockIdx.x % nx;
  const int sw = (tab.words + nx - 1) / nx;  // words per slice
  const int ws0 = x * sw, ws1 = min(tab.words, ws0 + sw);
  const int ngroups = (M + BG - 1) / BG;
  for (int g = (int)blockIdx.x / nx; g < ngroups; g += (int)gridDim.x / nx) {
    const int b0 = g * BG + wv * BW;  // the wave's first beam
    // rows in one load (lane i: beam b0 + i), hidden vectors beside them
    const int rl = (lane < BW && b0 + lane < M) ? row_in[b0 + lane] : -1;
    uint4 h[BW][NV];
#pragma unroll
    for (int i = 0; i < BW; ++i) {
      const char* hb = (const char*)hidden + (int64_t)min(b0 + i, M - 1) * SS::RB;
#pragma unroll
      for (int c = 0; c < NV; ++c) h[i][c] = *(const uint4*)(hb + (int64_t)(c * 64 + lane) * 16);
    }
    int rq[BW];
#pragma unroll
    for (int i = 0; i < BW; ++i) {
      const int r = __builtin_amdgcn_readlane(rl, i);
      rq[i] = (r >= 0 && r < tab.rows) ? r : -1;  // the request kernel reports bad rows
    }
    float* zw = z + (int64_t)b0 * ldz;
    int cnt = 0;  // scores waiting in the wave's LDS buffer
    auto flush = [&]() {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int j = lane; j < cnt; j += 64) {
        const int d = od[wv][j];
        zw[(int64_t)(d % BW) * ldz + d / BW] = ov[wv][j];
      }
      // the stores complete here, so no store is outstanding behind a tile's
      // loads when the pipeline waits for them (vmcnt 0; expcnt, lgkmcnt not waited)
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      cnt = 0;
    };
    for (int sw0 = ws0; sw0 < ws1; sw0 += 64) {
      const int nwd = min(64, ws1 - sw0);
      // the beams' bitmap words of this part (lane w: word sw0 + w) and
      // their ranks, kept in the wave's LDS (registers hold the hidden shares)
#pragma unroll
      for (int i = 0; i < BW; ++i) {
        const DWord d = (rq[i] >= 0 && lane < nwd) ? dense_word<NX>(tab, rq[i], sw0 + lane) : DWord{0u, 0};
        wsh[wv][i][lane] = d.bits;
        rsh[wv][i][lane] = d.rank;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int v0 = sw0 * 32;
      const int ntile = (nwd * 32 + TT - 1) / TT;
      // every thread issues all its loads (a chunk past row V - 1 reads the
      // last chunk of W_t instead; those rows are never scored), so the
      // compiler's wait for a tile counts only the loads issued after it
      struct Tile {
        uint4 v[LPT];
      };
      auto load_tile = [&](int k) {
        const int t0 = min(v0 + k * TT, tab.V - 1);
        const int lastc = min(TT, tab.V - t0) * RC - 1;  // last chunk of rows below V
        const uint4* src = (const uint4*)W + (int64_t)t0 * RC;
        Tile r;
#pragma unroll
        for (int j = 0; j < LPT; ++j) r.v[j] = src[min(j * kStageThreads + (int)threadIdx.x, lastc)];
        return r;
      };
      auto store_tile = [&](int sb, const Tile& r) {
#pragma unroll
        for (int j = 0; j < LPT; ++j) stage[sb][j * kStageThreads + threadIdx.x] = r.v[j];
      };
      auto compute = [&](int k, int sb) {
        const int tw = (k * TT) >> 5, off = (k * TT) & 31;
        uint32_t tb[BW];
        int tr[BW];
#pragma unroll
        for (int i = 0; i < BW; ++i) {
          const uint32_t wb = (uint32_t)__builtin_amdgcn_readfirstlane((int)wsh[wv][i][tw]);
          const int wr = __builtin_amdgcn_readfirstlane(rsh[wv][i][tw]);
          tb[i] = TT == 32 ? wb : (wb >> off) & ((1u << (TT & 31)) - 1u);
          tr[i] = wr + __popc(wb & ((1u << off) - 1u));
        }
        const uint4* st = stage[sb];
        for (;;) {
          uint32_t any = 0;
#pragma unroll
          for (int i = 0; i < BW; ++i) any |= tb[i];
          if (!any) break;
          if (cnt + BW > kStageOut) flush();
          float acc[BW];
          int dst = 0;
          bool put = false;
#pragma unroll
          for (int i = 0; i < BW; ++i) {
            acc[i] = 0.f;
            if (tb[i]) {
              const int t = __builtin_ctz(tb[i]);
              tb[i] &= tb[i] - 1u;
              const uint4* row = st + t * RC;
#pragma unroll
              for (int c = 0; c < NV; ++c) acc[i] = GatherDot<DT, D>::dot16(row[c * 64 + lane], h[i][c], acc[i]);
              if (lane == i * GL) {
                dst = tr[i] * BW + i;
                put = true;
              }
              ++tr[i];
            }
          }
          // lane i * GL ends with beam i's sum
          const float v = group_sum_multi<64, BW>(acc, lane);
          const uint64_t pm = __ballot(put);
          if (put) {
            const int j = cnt + __popcll(pm & ((1ull << lane) - 1ull));
            ov[wv][j] = v;
            od[wv][j] = dst;
          }
          cnt += __popcll(pm);
        }
      };
      // three tiles in flight in registers, three LDS buffers, one barrier
      // per tile; loads past the last tile read clamped rows, so every
      // iteration issues the same loads
      Tile r0 = load_tile(0), r1 = load_tile(1), r2 = load_tile(2);
      store_tile(0, r0);
      __syncthreads();
      for (int k = 0; k < ntile; k += 3) {
        // buffer 0 holds tile k; r1, r2 tiles k + 1, k + 2 (in flight)
        r0 = load_tile(k + 3);
        compute(k, 0);
        store_tile(1, r1);
        __syncthreads();
        if (k + 1 >= ntile) break;
        r1 = load_tile(k + 4);
        compute(k + 1, 1);
        store_tile(2, r2);
        __syncthreads();
        if (k + 2 >= ntile) break;
        r2 = load_tile(k + 5);
        compute(k + 2, 2);
        store_tile(0, r0);
        __syncthreads();
      }
    }
    flush();
  }
}

// ---------------------------------------------------------------- naive compaction baseline
//
// The selective projection organised the way the ZeroGR description says a
// straightforward implementation does it ("why fewer scores is not faster":
// all beams' candidates are first packed into one compact list and a
// temporary matrix is built): a scan of the legal counts over every beam
// gives each candidate's list position (a beam's position depends on all the
// beams before it), the list is sized from that count on the host, the
// candidates' weight rows are copied into a temporary [candidates x d]
// matrix, each row is dotted with its beam's hidden vector, and the score is
// scattered back to the beam's slot.  Used only to measure the padded-slot
// design against it.

// Legal counts of every beam and their exclusive scan (one block).
__global__ __launch_bounds__(1024) void k_naive_scan(const int32_t* __restrict__ row_in, int32_t M,
                                                     DevTable tab, int32_t* __restrict__ start,
                                                     int32_t* __restrict__ err) {
  __shared__ int sh[16];
  const int per = (M + 1023) / 1024;
  const int b0 = threadIdx.x * per, b1 = min(M, b0 + per);
  auto count = [&](int b) {
    const int r = row_in[b];
    if (r >= 0 && r < tab.rows) return tab.row_ptr[r + 1] - tab.row_ptr[r];
    if (r >= tab.rows) atomicOr(err, 1);
    return 0;
  };
  int mine = 0;
  for (int b = b0; b < b1; ++b) mine += count(b);
  int total;
  int run = block_excl_scan<1024>(mine, sh, &total);
  for (int b = b0; b < b1; ++b) {
    start[b] = run;
    const int r = row_in[b];
    run += (r >= 0 && r < tab.rows) ? tab.row_ptr[r + 1] - tab.row_ptr[r] : 0;
  }
  if (threadIdx.x == 0) start[M] = total;
}

// The compact list: (beam, token) of every legal candidate at start[b] + its
// legal rank.  One wave per beam.
__global__ __launch_bounds__(256) void k_naive_compact(const int32_t* __restrict__ row_in, int32_t M,
                                                       DevTable tab, const int32_t* __restrict__ start,
                                                       int32_t* __restrict__ lbeam,
                                                       int32_t* __restrict__ ltok) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= M) return;  // wave-uniform
  const int r = row_in[b];
  if (r < 0 || r >= tab.rows) return;
  const int s0 = start[b];
  if (tab.fmt == ZGR_FMT_SPARSE) {
    const int base = tab.row_ptr[r], n = tab.row_ptr[r + 1] - base;
    for (int j = lane; j < n; j += 64) {
      lbeam[s0 + j] = b;
      ltok[s0 + j] = tab.tok[base + j];
    }
  } else {
    for (int w = lane; w < tab.words; w += 64) {
      const DWord dw = tab.next ? dense_word<true>(tab, r, w) : dense_word<false>(tab, r, w);
      uint32_t x = dw.bits;
      int j = s0 + dw.rank;
      while (x) {
        const int v = (w << 5) + __ffs(x) - 1;
        x &= x - 1;
        lbeam[j] = b;
        ltok[j] = v;
        ++j;
      }
    }
  }
}

// The temporary matrix: tmp[c] = W[ltok[c]], rows copied in 16-byte pieces.
__global__ __launch_bounds__(256) void k_naive_gather(const uint4* __restrict__ W, int32_t row_vec,
                                                      const int32_t* __restrict__ ltok, int64_t n,
                                                      uint4* __restrict__ tmp) {
  const int64_t total = n * row_vec;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = i / row_vec, q = i - c * row_vec;
    tmp[i] = W[(int64_t)ltok[c] * row_vec + q];
  }
}

// z of every list entry: its temporary-matrix row dotted with its beam's
// hidden vector (a group of lanes per entry), scattered to the beam's slot.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void k_naive_dot(const void* __restrict__ tmp,
                                                        const void* __restrict__ hidden,
                                                        const int32_t* __restrict__ lbeam,
                                                        const int32_t* __restrict__ start, int64_t n,
                                                        float* __restrict__ z, int64_t ldz) {
  using Sh = SelShape<DT, D>;
  constexpr int G = Sh::G, NV = Sh::NV, VEC = Sh::VEC, ES = Sh::ES, NG = Sh::NG;
  const int gl = threadIdx.x % G, grp = threadIdx.x / G;
  for (int64_t c = (int64_t)blockIdx.x * NG + grp; c < n; c += (int64_t)gridDim.x * NG) {
    const int b = lbeam[c];
    const char* tr = (const char*)tmp + c * D * ES;
    const char* hb = (const char*)hidden + (int64_t)b * D * ES;
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      float w[VEC], h[VEC];
      load16<DT>(tr + (int64_t)(q * G + gl) * 16, w);
      load16<DT>(hb + (int64_t)(q * G + gl) * 16, h);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc = fmaf(w[e], h[e], acc);
    }
    acc = group_sum<G>(acc);
    if (gl == 0) z[(int64_t)b * ldz + (c - start[b])] = acc;
  }
}

// ---------------------------------------------------------------- k_request_step

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kKeyCap = kKeyCapHost;      // candidates of a part whose keys fit in LDS (40 KiB: two
                                          // blocks per compute unit)
constexpr int kMergeCap = kMergeCapHost;  // the parts' best keys a merge holds in LDS (112 KiB)
// unit partials of the log-sum-exp pass that fit beside the unit prefix in the
// selection's LDS (before the selection needs it)
constexpr int kUnitCap = 1400;
constexpr int kMaxK = 1024;
// candidates of a wave-sized log-sum-exp unit (four passes of eight per lane)
constexpr int kWaveUnit = 4 * 8 * 64;
// word partials a thread of a pruned request joins (its beam's share of them)
constexpr int kPruneWords = kPruneWordsHost;

// Distance histogram: 64 exact bins for distances below 64 ulps, then 64
// sub-bins per octave (monotone in the distance; 1728 bins used).
constexpr int kDistBins = 2 * kSelThreads;
constexpr int kBoundary = kDistBins / 2;  // boundary keys resolved by rank counting
// At most this many stored keys: every key is ranked directly (the number of
// keys above it), which yields the sorted selection in one pass.  The pass
// moves 8 C^2 bytes through LDS, so it only pays for small C.
constexpr int kSmallSel = 128;

__device__ __forceinline__ int dist_bin(uint32_t d) {
  if (d < 64u) return (int)d;
  const int e = 31 - __clz(d);
  return ((e - 5) << 6) | (int)((d >> (e - 6)) & 63u);
}

// How z reaches the request kernel: token-indexed rows (full projection, or a
// dense step), slot-indexed rows (selective projection of a sparse step), or
// computed by the request kernel itself (selective projection of a light
// sparse step: gather-dot in the block, no separate launches); kZParts is the
// merge of a request split over several blocks.
// kZSlotBig: kZSlot with the merge-sized key array (one block per CU), for
// requests so large that small parts would repeat their fixed cost too often.
// kZPrune: dense rank-indexed rows after the full projection, whose epilogue
// left each (beam, 32-token word) its legal (max, sum of exp): the request
// reads only the scores of the K words whose best candidates rank highest
// (merge-sized key array, so a request of K <= 448 stays in one block).
enum ZMode { kZToken = 0, kZSlot = 1, kZScore = 2, kZParts = 3, kZSlotBig = 4, kZPrune = 5 };

// Combine two (max, sum of exp(x - max)) partials; lanes that saw nothing hold
// (-inf, 0).  Symmetric, so both butterfly partners get identical bits.
__device__ __forceinline__ void lse_combine(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  const float e1 = (m == mn) ? 1.f : __expf(m - mn);
  const float e2 = (m2 == mn) ? 1.f : __expf(m2 - mn);
  s = s * e1 + s2 * e2;
  m = mn;
}

// Join of two (max, sum of exp) pairs with one exponential: the pair with the
// larger max keeps its sum, the other's is scaled by exp(-|difference|); two
// empty pairs (max -inf) give (-inf, 0).
__device__ __forceinline__ void ms_join(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  const float e = __expf(-fabsf(m - m2));
  s = (mn == -INFINITY) ? 0.f : ((m >= m2) ? fmaf(s2, e, s) : fmaf(s, e, s2));
  m = mn;
}

// N pairs per lane, reduced over lanes by halving: at lane offset O a lane
// keeps the half of its pairs that its partner does not (the upper half where
// lane & O is set) and joins its partner's copy of that half.  Offsets run
// 1, 2, 4, ... (exchanges within a 16-lane row are DPP moves), so after
// log2(N) stages lane l holds pair rev(l mod N) (its low log2(N) bits
// reversed), reduced over the lanes that differ from it in those bits.
template <int A, int N, int O>
__device__ __forceinline__ void ms_halve(float (&m)[A], float (&s)[A], int l) {
  if constexpr (N > 1) {
    const bool hi = (l & O) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const float sm = hi ? m[i] : m[i + N / 2], ss = hi ? s[i] : s[i + N / 2];
      float km = hi ? m[i + N / 2] : m[i], ks = hi ? s[i + N / 2] : s[i];
      ms_join(km, ks, xor_lane<O>(sm), xor_lane<O>(ss));
      m[i] = km;
      s[i] = ks;
    }
    ms_halve<A, N / 2, O * 2>(m, s, l);
  }
}

// One block per part of a request, the step after scoring.  A request's
// candidates are numbered flat: beams in rank order, each beam's candidates in
// slot order (sparse: legal rank; dense: token order, z stored by legal rank).
// Part p of P takes the flat range [Cq p / P, Cq (p + 1) / P) of the request's
// Cq candidates, so parts carry equal work however unevenly the legal tokens
// fall on the beams, and one beam may span several parts:
//   1. every beam of the request: row of table t, legal count, row base,
//      cumulative score; the candidate prefix over the beams;
//   2. (kZScore) z = W_t[token] . h_beam for the candidates of the beams this
//      part touches, the weight row read in place by a lane group;
//   3. legal-only log-sum-exp of those beams over all their candidates (also
//      the ones in neighbouring parts): every beam is cut into units of SEG
//      candidates counted from its first candidate (SEG depends only on the
//      request), a 16-lane group reduces a unit with contiguous loads to an
//      online (max, sum of exp), and one wave joins a beam's units in a fixed
//      butterfly, so every part that touches a beam computes the same value;
//      the same pass leaves the part's (z, beam*S + slot) in keys[] when they
//      fit in LDS;
//   4. cand = cum + (z - lse) as a 64-bit key (ord(cand), ~(beam*S + slot));
//      the K largest through a distance histogram (in LDS, or by passes over
//      z when they do not fit);
//   5. with P > 1 a part hands its best K to the merge (MODE kZParts, one
//      block per request); otherwise sort by rank counting, decode and
//      advance: next row = row_ptr[r] + slot (sparse: the position is the
//      next row) or row_ptr[r] + legal rank (dense); prefix gather.
// Scores z[b][j] are stored by legal rank j on sparse selective steps and on
// every dense step; after a full projection of a sparse step, and in the
// score-first comparison, they are token-indexed (kZToken).  On dense rows
// the token of rank j is the row's j-th set bit; the rank directory gives each
// word's first rank.
// The part kernels of heavy steps (scores already in z) are compiled for 8
// waves per SIMD, i.e. two 1024-thread blocks per compute unit (their LDS
// allows two); left to itself the compiler takes about 106 scalar registers,
// which leaves room for 7 waves and so one block.
constexpr int request_waves_per_eu(int mode) { return (mode == kZToken || mode == kZSlot) ? 8 : 1; }

template <int MODE, int DT, int D, bool NX>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(request_waves_per_eu(MODE))))
void k_request_step(
    DevTable tab, int32_t t, int32_t L, int32_t k_in, int32_t K, const int32_t* __restrict__ row_in,
    const float* __restrict__ cum_in, const void* __restrict__ hidden, const void* __restrict__ W,
    float* __restrict__ z, int64_t ldz, int32_t P, uint64_t* __restrict__ part_keys,
    int32_t* __restrict__ part_cnt, float2* __restrict__ part_ms, int32_t* __restrict__ parent_out,
    int32_t* __restrict__ token_out, int32_t* __restrict__ row_out, float* __restrict__ cum_out,
    const int32_t* __restrict__ prefix_in, int32_t* __restrict__ prefix_out,
    float* __restrict__ slot_dbg, const float* __restrict__ lse_ext, int32_t ztok,
    const float2* __restrict__ zms, int32_t* __restrict__ err) {
  constexpr int NT = kSelThreads;
  constexpr bool TOKEN_IDX = (MODE == kZToken);
  constexpr bool MERGE = (MODE == kZParts);
  constexpr bool PRUNE = (MODE == kZPrune);
  constexpr int KEYCAP = (MERGE || MODE == kZSlotBig || PRUNE) ? kMergeCap : kKeyCap;
  __shared__ uint64_t keys[KEYCAP];
  // sel (the selection) and dhist (the distance histogram, then the boundary
  // keys) from phase 4 on; before that the log-sum-exp pass keeps its unit
  // partials and the unit prefix over the beams here
  __shared__ __attribute__((aligned(16))) uint64_t selhist[kMaxK + kDistBins / 2];
  uint64_t* sel = selhist;
  int* dhist = reinterpret_cast<int*>(selhist + kMaxK);
  float2* upart = reinterpret_cast<float2*>(selhist);             // [kUnitCap]
  int* upre = reinterpret_cast<int*>(selhist + kUnitCap);          // [kMaxK + 1]
  __shared__ int cpre[kMaxK + 1];  // candidate prefix over the request's beams
  __shared__ int brow[kMaxK];
  __shared__ int bbase[kMaxK];
  __shared__ float bcum[kMaxK];
  __shared__ float blse[kMaxK];
  __shared__ int mpre[kMaxParts + 1], mcn[kMaxParts];  // merge: the parts' key counts and prefix
  __shared__ int hist[256];
  __shared__ int sh[kSelWaves];
  __shared__ int pos, pos2, pick_bin, pick_above, bl_lo_sh, bl_hi_sh, multi_sh;
  __shared__ float pm[kSelWaves], ps[kSelWaves];
  __shared__ float2 zms_sh;  // single-beam part: (max, sum of exp) of its own range
  __shared__ unsigned int omax_sh;
  const int q = MERGE ? blockIdx.x : blockIdx.x / P;
  const int part = MERGE ? 0 : blockIdx.x - q * P;
  const int b0 = q * k_in;  // the request's first beam
  const bool dense = tab.fmt != ZGR_FMT_SPARSE;
  const bool all_legal = tab.fmt == kFmtAll;
  const uint32_t S = (uint32_t)tab.stride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // 0. the merge's part counts and first keys: their addresses are known
  //    before the beams' rows, so they overlap the row lookups below
  constexpr int U = 8;  // phase-3 loads issued together per thread
  // a single-beam request split over parts selects by the score alone (cand
  // is monotone in z within a beam): each part reduces only its own range to
  // a (max, sum of exp) partial, and the merge joins the partials into the
  // normaliser (fixed order) and forms the cumulative scores
  const bool zkey = k_in == 1 && P > 1;
  int mcnt = 0;
  uint64_t mkey0 = 0;
  float2 mms = make_float2(-INFINITY, 0.f);
  if constexpr (MERGE) {
    if ((int)threadIdx.x < P) mcnt = part_cnt[q * P + threadIdx.x];
    if (zkey && (int)threadIdx.x < P) mms = part_ms[q * P + threadIdx.x];
    if ((int)threadIdx.x < P * K) mkey0 = part_keys[(int64_t)q * P * K + threadIdx.x];
  }

  // 1. the request's beams
  int cnt = 0;
  if ((int)threadIdx.x < k_in) {
    int r = row_in[b0 + threadIdx.x];
    if (all_legal && r > 0) r = 0;  // every live beam has the one all-legal row
    int base = 0;
    if (r >= 0 && r < tab.rows) {
      base = tab.row_ptr[r];
      cnt = tab.row_ptr[r + 1] - base;
    } else {
      if (r >= tab.rows && !MERGE) atomicOr(err, 1);
      r = -1;
    }
    brow[threadIdx.x] = r;
    bbase[threadIdx.x] = base;
    bcum[threadIdx.x] = cum_in[b0 + threadIdx.x];
  }
  int Cq;
  const int exc = block_excl_scan<NT>(cnt, sh, &Cq);
  if ((int)threadIdx.x < k_in) cpre[threadIdx.x] = exc;
  // 2. this part's candidates [f0, f1) and the beams they fall on
  //    [bl_lo, bl_hi]: the beams holding f0 and f1 - 1 say so themselves
  int f0 = MERGE ? 0 : (int)((int64_t)Cq * part / P);
  int f1 = MERGE ? 0 : (int)((int64_t)Cq * (part + 1) / P);
  if (cnt > 0 && exc <= f0 && f0 < exc + cnt) bl_lo_sh = threadIdx.x;
  if (cnt > 0 && exc <= f1 - 1 && f1 - 1 < exc + cnt) bl_hi_sh = threadIdx.x;
  // units of the log-sum-exp pass: SEG candidates from each beam's first,
  // reduced by GL lanes with UL loads each per pass; GL follows the
  // request's mean legal count (1 lane for the one or two legal tokens of a
  // late step, 16 for rows of hundreds) and SEG = GL * UL * 2^s is the
  // smallest that keeps any part's units within kUnitCap.  A part touches
  // its own ceil(Cq / P) candidates plus at most two beams' worth (S each)
  // beyond them, so its units are at most that over SEG plus one per beam.
  // Both depend only on the request, so every part reduces a beam the same
  // way.
  // (4 in the part kernels compiled for two blocks per CU: with 8 they spill)
  constexpr int UL = (MODE == kZSlot || MODE == kZToken) ? 4 : 8;
  const int mean_n = Cq / max(1, k_in);
  const int GL = mean_n >= 64 ? 16 : (mean_n >= 8 ? 4 : 1);
  const int64_t touch = ((int64_t)Cq + P - 1) / P + 2 * (int64_t)S;
  // scores at their slots, rows of 64 or more on average that either fit one
  // wave-sized unit (the slot stride is at most 2,048) or hold 256 or more on
  // average: wave-sized units of 2,048 candidates, one wave each (below)
  const bool wave_units =
      !TOKEN_IDX && MODE != kZScore && GL == 16 && ((int)S <= kWaveUnit || mean_n >= 256);
  int SEG = wave_units ? kWaveUnit : GL * UL;
  while ((touch + SEG - 1) / SEG + k_in + 1 > kUnitCap) SEG *= 2;
  if (!MERGE && !zkey && !PRUNE) {  // uniform; split single-beam parts reduce only their own range
    int Uq;
    const int uex = block_excl_scan<NT>((cnt + SEG - 1) / SEG, sh, &Uq);
    if ((int)threadIdx.x < k_in) upre[threadIdx.x] = uex;
    if (threadIdx.x == 0) upre[k_in] = Uq;
  }
  if (threadIdx.x == 0) {
    cpre[k_in] = Cq;
    pos = 0;
    multi_sh = 0;
    omax_sh = 0u;
    zms_sh = make_float2(-INFINITY, 0.f);
  }
  __syncthreads();
  auto beam_of = [&](int f) {  // the beam of flat candidate f < Cq: last b with cpre[b] <= f
    int lo = 0, hi = k_in;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cpre[mid] <= f)
        lo = mid;
      else
        hi = mid;
    }
    return lo;
  };
  //    (and all those beams' candidates [e0, e1))
  int C = f1 - f0;
  const int bl_lo = C > 0 ? bl_lo_sh : 0;
  const int bl_hi = C > 0 ? bl_hi_sh : -1;
  const int e0 = C > 0 ? cpre[bl_lo] : 0, e1 = C > 0 ? cpre[bl_hi + 1] : 0;
  bool store = C <= KEYCAP;
  auto code_of = [&](int b, int slot) { return (uint32_t)b * S + (uint32_t)slot; };

  //    (kZScore) selective projection inside the block: U2 candidates per
  //    lane group with their token and row loads issued together; z goes to
  //    its slot and, for this part's candidates, to keys[]
  if constexpr (MODE == kZScore) {
    using Sh = SelShape<DT, D>;
    constexpr int G = Sh::G, NV = Sh::NV, VEC = Sh::VEC, ES = Sh::ES;
    constexpr int NGB = NT / G;
    constexpr int U2 = NV <= 8 ? 2 : 1;  // two candidates' rows in flight unless that spills
    const int gl = threadIdx.x % G, grp = threadIdx.x / G;
    for (int f00 = e0 + grp; f00 < e1; f00 += NGB * U2) {
      int bls[U2], js[U2], toks[U2];
#pragma unroll
      for (int u = 0; u < U2; ++u) {
        const int f = f00 + u * NGB;
        bls[u] = f < e1 ? beam_of(f) : bl_lo;
        js[u] = f < e1 ? f - cpre[bls[u]] : 0;
        toks[u] = f < e1 ? (int)tab.tok[bbase[bls[u]] + js[u]] : 0;
      }
      float acc[U2];
#pragma unroll
      for (int u = 0; u < U2; ++u) acc[u] = 0.f;
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        float h[U2][VEC], w[U2][VEC];
#pragma unroll
        for (int u = 0; u < U2; ++u) {
          const char* hb = (const char*)hidden + (int64_t)(b0 + bls[u]) * D * ES;
          const char* wr = (const char*)W + (int64_t)toks[u] * D * ES;
          load16<DT>(hb + (int64_t)(c * G + gl) * 16, h[u]);
          load16<DT>(wr + (int64_t)(c * G + gl) * 16, w[u]);
        }
#pragma unroll
        for (int u = 0; u < U2; ++u)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[u] = fmaf(w[u][e], h[u][e], acc[u]);
      }
#pragma unroll
      for (int u = 0; u < U2; ++u) {
        acc[u] = group_sum<G>(acc[u]);
        const int f = f00 + u * NGB;
        if (gl == 0 && f < e1) {
          z[(int64_t)(b0 + bls[u]) * ldz + js[u]] = acc[u];
          if (store && f >= f0 && f < f1)
            keys[f - f0] = ((uint64_t)__float_as_uint(acc[u]) << 32) | code_of(bls[u], js[u]);
        }
      }
    }
    __syncthreads();
  }

  // Dense rank-indexed scores get their slot codes after phase 3 (below):
  // LPW lanes share a (beam, word) pair, each walking its own 32/LPW bits.
  // LPW grows while the pairs leave threads idle, so a full row at the first
  // step needs no long serial walks.  The first round's bitmap words are
  // loaded now so that phase 3 hides their latency.
  const int nbl = bl_hi - bl_lo + 1;  // beams this part touches (0 when C = 0)
  const bool code_pass = !MERGE && !PRUNE && dense && store && !TOKEN_IDX;
  const int pairs = nbl * tab.words;
  int LPW = 1;
  while (LPW < 32 && pairs * LPW * 2 <= NT) LPW *= 2;
  DWord dwpf{0u, 0};
  if (code_pass && (int)threadIdx.x < pairs * LPW) {
    const int pr = threadIdx.x / LPW, bl = bl_lo + pr / tab.words, w = pr % tab.words;
    if (brow[bl] >= 0) dwpf = dense_word<NX>(tab, brow[bl], w);
  }

  // 3. legal-only log-sum-exp of the beams bl_lo..bl_hi over [e0, e1)
  //    (omax_t: the best candidate of this thread's beams, cand being
  //    monotone in z within a beam; joined over the block below with one LDS
  //    atomic per wave, not one per beam on a single address)
  uint32_t omax_t = 0u;
  auto final_lse = [&](int b, float m, float s) {
    const float l = lse_ext ? lse_ext[b0 + b] : m + __logf(s);
    blse[b] = l;
    omax_t = max(omax_t, ord_of(bcum[b] + (m - l)));
  };
  if constexpr (!MERGE && !PRUNE) {
    if ((zkey || (k_in == 1 && P == 1)) && !(TOKEN_IDX && dense)) {
      // this part's own range only, coalesced, with its keys' scores (a
      // single-beam request in one part: its whole row, by every thread)
      float m = -INFINITY, s = 0.f;
      const float* zb = z + (int64_t)b0 * ldz;
      for (int i0 = threadIdx.x; i0 < C; i0 += NT * U) {
        float zv[U];
        int tk[U];
        if constexpr (TOKEN_IDX) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int i = i0 + u * NT;
            tk[u] = i < C ? (int)tab.tok[bbase[0] + f0 + i] : 0;
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * NT;
          if (i < C) {
            if (MODE == kZScore && store)
              zv[u] = __uint_as_float((uint32_t)(keys[i] >> 32));
            else
              zv[u] = zb[TOKEN_IDX ? tk[u] : f0 + i];
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * NT;
          if (i < C) {
            const float x = zv[u];
            if (x > m) {
              s = s * __expf(m - x) + 1.f;
              m = x;
            } else {
              s += __expf(x - m);
            }
            if (MODE != kZScore && store)
              keys[i] = ((uint64_t)__float_as_uint(x) << 32) | (dense ? 0u : code_of(0, f0 + i));
          }
        }
      }
      xor_down<32>([&](auto o) {
        constexpr int X = decltype(o)::value;
        lse_combine(m, s, xor_lane<X>(m), xor_lane<X>(s));
      });
      if (lane == 0) {
        pm[wave] = m;
        ps[wave] = s;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        float mm = pm[0], ss = ps[0];
        for (int w = 1; w < kSelWaves; ++w) lse_combine(mm, ss, pm[w], ps[w]);
        if (zkey) {
          zms_sh = make_float2(mm, ss);
          omax_sh = ord_of(mm);
        } else if (C > 0) {
          final_lse(0, mm, ss);
        }
      }
    } else if (TOKEN_IDX && dense) {
      // token-indexed rows of a dense table (the score-first comparison; its
      // normaliser over the whole codebook is given): keys from a walk of the
      // beams' bitmap words, the beams' best score by an exact atomic max
      uint32_t* bmo = reinterpret_cast<uint32_t*>(sel);  // sel is free until phase 4
      for (int i = threadIdx.x; i < nbl; i += NT) bmo[i] = 0u;
      __syncthreads();
      for (int u = threadIdx.x; u < pairs; u += NT) {
        const int bl = bl_lo + u / tab.words, w = u % tab.words;
        const int r = brow[bl];
        if (r < 0) continue;
        const DWord dw = dense_word<NX>(tab, r, w);
        const float* zb = z + (int64_t)(b0 + bl) * ldz;
        uint32_t x = dw.bits;
        int f = cpre[bl] + dw.rank;
        uint32_t mo = 0u;
        while (x) {
          const int v = (w << 5) + __ffs(x) - 1;
          x &= x - 1;
          const float zv = zb[v];
          mo = max(mo, ord_of(zv));
          if (store && f >= f0 && f < f1) keys[f - f0] = ((uint64_t)__float_as_uint(zv) << 32) | code_of(bl, v);
          ++f;
        }
        if (mo) atomicMax(&bmo[bl - bl_lo], mo);
      }
      __syncthreads();
      for (int bl = bl_lo + threadIdx.x; bl <= bl_hi; bl += NT)
        if (brow[bl] >= 0 && cpre[bl + 1] > cpre[bl]) {
          if (zkey)
            omax_sh = bmo[0];  // single beam, score-first: keys by the score alone
          else
            final_lse(bl, float_of_ord(bmo[bl - bl_lo]), 1.f);
        }
    } else if (wave_units) {
      // rows of 64 or more legal tokens on average: wave-sized units, SEG
      // candidates from each beam's first (SEG is the request's), one wave
      // each.  Lane i reads the unit's scores i, i + 64, ... in passes of 8
      // (contiguous per load), each pass reduced to (max, sum of exp) without
      // branches and joined in order, then the wave's lanes in a fixed
      // butterfly; a beam of several units is joined below in unit order:
      // the same value in every part that touches the beam.  The part's own
      // candidates also go to keys[].
      // (when every row fits one unit, the waves walk the beams directly)
      const int u_lo = C > 0 ? upre[bl_lo] : 0, u_hi = C > 0 ? upre[bl_hi + 1] : 0;
      const bool one_unit = (int)S <= SEG;
      const int w_hi = one_unit ? (C > 0 ? bl_hi + 1 : 0) : u_hi;
      for (int u = (one_unit ? bl_lo : u_lo) + wave; u < w_hi; u += kSelWaves) {  // uniform over the wave
        int b = u;
        if (!one_unit) {
          int lo = bl_lo, hi = bl_hi + 1;  // the unit's beam: last b with upre[b] <= u
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (upre[mid] <= u)
              lo = mid;
            else
              hi = mid;
          }
          b = lo;
        }
        const int n_b = cpre[b + 1] - cpre[b];
        if (n_b == 0) continue;  // a dead beam (direct walk only)
        const int j0 = one_unit ? 0 : (u - upre[b]) * SEG, j1 = min(n_b, j0 + SEG);
        const float* zb = z + (int64_t)(b0 + b) * ldz;
        float m = -INFINITY, sm = 0.f;
        for (int jb = j0; jb < j1; jb += 64 * UL) {
          float zv[UL];
#pragma unroll
          for (int i = 0; i < UL; ++i) {
            const int j = jb + i * 64 + lane;
            zv[i] = j < j1 ? zb[j] : -INFINITY;
          }
          float pm = zv[0];
#pragma unroll
          for (int i = 1; i < UL; ++i) pm = fmaxf(pm, zv[i]);
          float ps = 0.f;
          if (pm != -INFINITY) {
#pragma unroll
            for (int i = 0; i < UL; ++i) ps += __expf(zv[i] - pm);
          }
          lse_combine(m, sm, pm, ps);
#pragma unroll
          for (int i = 0; i < UL; ++i) {
            const int j = jb + i * 64 + lane;
            const int f = cpre[b] + j;
            if (store && j < j1 && f >= f0 && f < f1) {
              // sparse rows: slot = legal rank; dense rows (rank-indexed
              // scores): the code goes in after this pass
              const uint32_t code = dense ? 0u : code_of(b, j);
              keys[f - f0] = ((uint64_t)__float_as_uint(zv[i]) << 32) | code;
            }
          }
        }
        xor_down<32>([&](auto o) {
          constexpr int X = decltype(o)::value;
          lse_combine(m, sm, xor_lane<X>(m), xor_lane<X>(sm));
        });
        if (lane == 0) {
          if (one_unit || upre[b + 1] - upre[b] == 1) {
            final_lse(b, m, sm);
          } else {
            upart[u - u_lo] = make_float2(m, sm);
            multi_sh = 1;
          }
        }
      }
      __syncthreads();
      // beams of several units: one wave joins the unit partials in order
      for (int b = bl_lo + wave; multi_sh && b <= bl_hi; b += kSelWaves) {
        const int nu = upre[b + 1] - upre[b];
        if (nu < 2) continue;  // uniform over the wave
        float m = -INFINITY, sm = 0.f;
        for (int i = lane; i < nu; i += 64) {
          const float2 pq = upart[upre[b] - u_lo + i];
          lse_combine(m, sm, pq.x, pq.y);
        }
        xor_down<32>([&](auto o) {
          constexpr int X = decltype(o)::value;
          lse_combine(m, sm, xor_lane<X>(m), xor_lane<X>(sm));
        });
        if (lane == 0) final_lse(b, m, sm);
      }
    } else {
      // unit u of the part (u_lo + u is the request's unit) to a 16-lane
      // group; the group's lanes read the unit's scores at a stride of 16
      // (contiguous per load), each keeping an online (max, sum of exp)
      const int NGR = NT / GL;
      const int u_lo = C > 0 ? upre[bl_lo] : 0, u_hi = C > 0 ? upre[bl_hi + 1] : 0;
      const int gl = threadIdx.x % GL, grp = threadIdx.x / GL;
      auto unit_beam = [&](int u) {  // last b with upre[b] <= u
        int lo = bl_lo, hi = bl_hi + 1;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (upre[mid] <= u)
            lo = mid;
          else
            hi = mid;
        }
        return lo;
      };
      for (int u = u_lo + grp; u < u_hi; u += NGR) {  // uniform over the group
        const int b = unit_beam(u);
        const int ua = u - upre[b];
        const int n_b = cpre[b + 1] - cpre[b];
        const int j0 = ua * SEG, j1 = min(n_b, j0 + SEG);
        const float* zb = z + (int64_t)(b0 + b) * ldz;
        float m = -INFINITY, s = 0.f;
        for (int jb = j0; jb < j1; jb += GL * UL) {
          float zv[UL];
          int tk[UL];
          if constexpr (TOKEN_IDX) {
#pragma unroll
            for (int i = 0; i < UL; ++i) {
              const int j = jb + i * GL + gl;
              tk[i] = j < j1 ? (int)tab.tok[bbase[b] + j] : 0;
            }
          }
#pragma unroll
          for (int i = 0; i < UL; ++i) {
            const int j = jb + i * GL + gl;
            const int f = cpre[b] + j;
            if (j < j1) {
              if (MODE == kZScore && store && f >= f0 && f < f1)
                zv[i] = __uint_as_float((uint32_t)(keys[f - f0] >> 32));
              else
                zv[i] = zb[TOKEN_IDX ? tk[i] : j];
            }
          }
#pragma unroll
          for (int i = 0; i < UL; ++i) {
            const int j = jb + i * GL + gl;
            if (j < j1) {
              const float x = zv[i];
              if (x > m) {
                s = s * __expf(m - x) + 1.f;
                m = x;
              } else {
                s += __expf(x - m);
              }
              const int f = cpre[b] + j;
              if (MODE != kZScore && store && f >= f0 && f < f1) {
                // sparse rows: slot = legal rank; dense rows (rank-indexed
                // scores): the code goes in after this pass
                const uint32_t code = dense ? 0u : code_of(b, j);
                keys[f - f0] = ((uint64_t)__float_as_uint(x) << 32) | code;
              }
            }
          }
        }
        xor_down_width(GL, [&](auto o) {
          constexpr int X = decltype(o)::value;
          lse_combine(m, s, xor_lane<X>(m), xor_lane<X>(s));
        });
        if (gl == 0) {
          if (upre[b + 1] - upre[b] == 1) {
            final_lse(b, m, s);
          } else {
            upart[u - u_lo] = make_float2(m, s);
            multi_sh = 1;
          }
        }
      }
      __syncthreads();
      // beams of a few units: one thread joins their partials in order;
      // beams of many: one wave, in a fixed butterfly
      constexpr int kJoinSerial = 16;
      if (multi_sh) {
        for (int b = bl_lo + (int)threadIdx.x; b <= bl_hi; b += NT) {
          const int nu = upre[b + 1] - upre[b];
          if (nu < 2 || nu > kJoinSerial) continue;
          float m = -INFINITY, s = 0.f;
          for (int i = 0; i < nu; ++i) {
            const float2 pq = upart[upre[b] - u_lo + i];
            lse_combine(m, s, pq.x, pq.y);
          }
          final_lse(b, m, s);
        }
        for (int b = bl_lo + wave; b <= bl_hi; b += kSelWaves) {
          const int nu = upre[b + 1] - upre[b];
          if (nu <= kJoinSerial) continue;  // uniform over the wave
          float m = -INFINITY, s = 0.f;
          for (int i = lane; i < nu; i += 64) {
            const float2 pq = upart[upre[b] - u_lo + i];
            lse_combine(m, s, pq.x, pq.y);
          }
          xor_down<32>([&](auto o) {
            constexpr int X = decltype(o)::value;
            lse_combine(m, s, xor_lane<X>(m), xor_lane<X>(s));
          });
          if (lane == 0) final_lse(b, m, s);
        }
      }
    }
  }
  if constexpr (PRUNE) {
    // Word-level pruning.  The full projection's epilogue left zms[beam][w]
    // = the legal (max, sum of exp) of the 32-token word w of the beam's row.
    //  a. a beam's log-sum-exp joins its words' partials: G threads per beam,
    //     each over PW consecutive words in order, then a fixed butterfly
    //  b. a word's best candidate is cum + (max - lse), the same arithmetic as
    //     its key below; the word's key takes the word's first code, so words
    //     order exactly as their best candidates' keys do
    //  c. the K-th largest word key (radix select): the words at or above it
    //     hold the request's whole top K, since a candidate in any other word
    //     lies below K better candidates (the best of each kept word)
    //  d. the kept words in (beam, word) order, their legal counts and a flat
    //     prefix; this part takes its share [f0, f1) of that list
    //  e. and loads those scores only
    const int NWD = tab.words;
    int kp2 = 1;
    while (kp2 < k_in) kp2 <<= 1;
    const int G = min(64, NT / kp2);
    const int PW = (NWD + G - 1) / G;  // at most kPruneWords (checked by the host)
    const int pb = (int)threadIdx.x / G, pg = (int)threadIdx.x - pb * G;
    const bool plive = pb < k_in && brow[min(pb, k_in - 1)] >= 0;
    float wmax[kPruneWords];
    float m = -INFINITY, sm = 0.f;
    {
      float2 pq[kPruneWords];
      const float2* zp = zms + (int64_t)(b0 + min(pb, k_in - 1)) * NWD;
#pragma unroll
      for (int u = 0; u < kPruneWords; ++u) {
        const int w = pg * PW + u;
        pq[u] = (plive && u < PW && w < NWD) ? zp[w] : make_float2(-INFINITY, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kPruneWords; ++u) {
        wmax[u] = pq[u].x;
        lse_combine(m, sm, pq[u].x, pq[u].y);
      }
    }
    xor_down_width(G, [&](auto o) {
      constexpr int X = decltype(o)::value;
      lse_combine(m, sm, xor_lane<X>(m), xor_lane<X>(sm));
    });
    const bool pcand = plive && cpre[pb + 1] > cpre[pb];
    if (pcand && pg == 0) final_lse(pb, m, sm);
    __syncthreads();
    const float pl = pcand ? blse[pb] : 0.f, pc = pcand ? bcum[pb] : 0.f;
    uint64_t wkey[kPruneWords];  // 0: an empty word
    int nonempty = 0;
#pragma unroll
    for (int u = 0; u < kPruneWords; ++u) {
      const bool ok = wmax[u] != -INFINITY;  // only real words of live beams
      wkey[u] = ok ? make_key(pc + (wmax[u] - pl), code_of(pb, (pg * PW + u) << 5)) : 0ull;
      nonempty += ok ? 1 : 0;
    }
    int ne_total;
    (void)block_excl_scan<NT>(nonempty, sh, &ne_total);
    const bool keep_all = ne_total <= K;  // uniform
    // radix select, 8 bits per pass from the top, two barriers per pass: the
    // counts, then wave 0 scans the 256 digits (four per lane, descending),
    // publishes the digit holding the need-th largest and clears the bins
    RadixSel rs{0, 0, K};
    if (!keep_all) {
      __shared__ int rp_digit, rp_above, rp_count;
      __shared__ uint64_t rp_prefix, rp_mask;
      if (threadIdx.x < 256) hist[threadIdx.x] = 0;
      __syncthreads();
      auto count = [&](int shift) {
#pragma unroll
        for (int u = 0; u < kPruneWords; ++u)
          if (wkey[u] != 0ull && (wkey[u] & rs.mask) == rs.prefix) atomicAdd(&hist[(wkey[u] >> shift) & 0xFF], 1);
      };
      auto scan = [&]() {  // wave 0
        int c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = hist[255 - 4 * lane - i];
        const int tot = c[0] + c[1] + c[2] + c[3];
        int run = wave_incl_scan(tot) - tot;  // digits above this lane's four
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (run < rs.need && run + c[i] >= rs.need) {
            rp_digit = 255 - 4 * lane - i;
            rp_above = run;
            rp_count = c[i];
          }
          run += c[i];
          hist[255 - 4 * lane - i] = 0;
        }
      };
      auto take = [&](int shift) {
        rs.prefix |= (uint64_t)rp_digit << shift;
        rs.mask |= (uint64_t)0xFF << shift;
        rs.need -= rp_above;
        return rp_count == rs.need;  // every key under the prefix is kept
      };
      if (kp2 * G <= 64) {
        // every word key lives in wave 0 (a single-beam request): its passes
        // run there alone, ordered by LDS waits instead of block barriers
        if (wave == 0) {
          for (int shift = 56; shift >= 0; shift -= 8) {
            count(shift);
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            scan();
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            if (take(shift)) break;  // uniform over the wave
          }
          if (lane == 0) {
            rp_prefix = rs.prefix;
            rp_mask = rs.mask;
          }
        }
        __syncthreads();
        rs.prefix = rp_prefix;
        rs.mask = rp_mask;
      } else {
        for (int shift = 56; shift >= 0; shift -= 8) {
          count(shift);
          __syncthreads();
          if (wave == 0) scan();
          __syncthreads();
          if (take(shift)) break;  // uniform
        }
      }
    }
    auto kept = [&](uint64_t k) { return k != 0ull && (keep_all || (k & rs.mask) >= rs.prefix); };
    int nkeep = 0;
#pragma unroll
    for (int u = 0; u < kPruneWords; ++u) nkeep += kept(wkey[u]) ? 1 : 0;
    int NU;
    int kpos = block_excl_scan<NT>(nkeep, sh, &NU);  // NU <= K: the keys are distinct
    int* uinfo = reinterpret_cast<int*>(selhist);  // [kMaxK] beam << 16 | word
    uint32_t* ubits = reinterpret_cast<uint32_t*>(uinfo + kMaxK);
    int* urank = reinterpret_cast<int*>(ubits + kMaxK);
    int* ucum = urank + kMaxK;
#pragma unroll
    for (int u = 0; u < kPruneWords; ++u)
      if (kept(wkey[u])) {
        if (kpos < kMaxK) uinfo[kpos] = (pb << 16) | (pg * PW + u);
        ++kpos;
      }
    NU = min(NU, kMaxK);
    __syncthreads();
    int ucnt = 0;
    if ((int)threadIdx.x < NU) {
      const int info = uinfo[threadIdx.x];
      const DWord dw = dense_word<NX>(tab, brow[info >> 16], info & 0xFFFF);
      ubits[threadIdx.x] = dw.bits;
      urank[threadIdx.x] = dw.rank;
      ucnt = __popc(dw.bits);
    }
    int Cp;
    const int uex = block_excl_scan<NT>(ucnt, sh, &Cp);
    if ((int)threadIdx.x < NU) ucum[threadIdx.x] = uex;
    f0 = (int)((int64_t)Cp * part / P);
    f1 = (int)((int64_t)Cp * (part + 1) / P);
    if (f1 - f0 > KEYCAP) {  // the host sizes P so that this cannot happen
      if (threadIdx.x == 0) atomicOr(err, 1);
      f1 = f0 + KEYCAP;
    }
    C = f1 - f0;
    store = true;
    __syncthreads();
    // four threads per kept word, eight bit positions each: their eight loads
    // go out together, clamped to the word's candidates (always in bounds)
    for (int i2 = threadIdx.x; i2 < NU * 4; i2 += NT) {
      const int u = i2 >> 2, lo = (i2 & 3) * 8;
      const int fb = ucum[u];
      const uint32_t bits = ubits[u];
      const int nc = __popc(bits);
      if (fb + nc <= f0 || fb >= f1) continue;
      const int info = uinfo[u];
      const int bl = info >> 16, w = info & 0xFFFF;
      const float* zb = z + (int64_t)(b0 + bl) * ldz + urank[u];
      const int k0 = __popc(bits & ((1u << lo) - 1u));
      float zv[8];
      int kk[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kk[i] = k0 + __popc((bits >> lo) & ((1u << i) - 1u));
        zv[i] = zb[min(kk[i], nc - 1)];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int f = fb + kk[i];
        if (((bits >> (lo + i)) & 1u) && f >= f0 && f < f1)
          keys[f - f0] = ((uint64_t)__float_as_uint(zv[i]) << 32) | code_of(bl, (w << 5) + lo + i);
      }
    }
  }
  {
    uint32_t o = omax_t;
    xor_down<32>([&](auto d) { o = max(o, xor_lane<decltype(d)::value>(o)); });
    if (lane == 0 && o != 0u) atomicMax(&omax_sh, o);
  }
  __syncthreads();
  if (code_pass) {
    // a bit's legal rank is the word's count before it plus the set bits below
    // it; only this part's flat range [f0, f1) is coded
    const int nb = 32 / LPW;
    const uint32_t sub_mask = (nb == 32) ? 0xFFFFFFFFu : ((1u << nb) - 1u);
    uint32_t* key_lo = reinterpret_cast<uint32_t*>(keys);
    for (int u = threadIdx.x; u < pairs * LPW; u += NT) {
      const int pr = u / LPW, sub = u - pr * LPW;
      const int bl = bl_lo + pr / tab.words, w = pr % tab.words;
      const int r = brow[bl];
      if (r < 0) continue;
      const DWord dw = (u == (int)threadIdx.x) ? dwpf : dense_word<NX>(tab, r, w);
      const int lo = sub * nb;  // <= 31
      uint32_t x = (dw.bits >> lo) & sub_mask;
      int f = cpre[bl] + dw.rank + __popc(dw.bits & ((1u << lo) - 1u));
      if (f >= f1 || f + __popc(x) <= f0) continue;
      const uint32_t code0 = code_of(bl, (w << 5) + lo);
      // the key's high half (the score) was stored with a zero low half above:
      // the code goes into the low half alone, with no read of the key
      while (x) {
        const int k = __ffs(x) - 1;
        x &= x - 1;
        if (f >= f0 && f < f1) key_lo[2 * (f - f0)] = code0 + (uint32_t)k;
        ++f;
      }
    }
    __syncthreads();
  }
  if constexpr (MERGE) {
    if (zkey) {
      // the single beam's normaliser: the parts' partials joined in a fixed
      // butterfly over wave 0 (lane i holds part i), or the given one
      if (wave == 0) {
        float m = (lane < P) ? mms.x : -INFINITY, s = (lane < P) ? mms.y : 0.f;
        xor_down<32>([&](auto o) {
          constexpr int X = decltype(o)::value;
          lse_combine(m, s, xor_lane<X>(m), xor_lane<X>(s));
        });
        if (lane == 0) blse[0] = lse_ext ? lse_ext[b0] : m + __logf(s);
      }
      __syncthreads();
    }
  }
  if (slot_dbg && (MERGE ? zkey : !zkey)) {
    // each beam's row is written by one part: the one holding its first
    // candidate (beams without candidates: part b mod P); a single beam
    // split over parts by the merge
    for (int b = wave; b < k_in; b += kSelWaves) {
      const int r = brow[b];
      const int n = cpre[b + 1] - cpre[b];
      const bool mine =
          MERGE || (PRUNE ? b % P == part : ((n > 0) ? (cpre[b] >= f0 && cpre[b] < f1) : (b % P == part)));
      if (!mine) continue;
      float* dbg = slot_dbg + (int64_t)(b0 + b) * S;
      const float* zb = z + (int64_t)(b0 + b) * ldz;
      const bool tix = MERGE ? ztok != 0 : TOKEN_IDX;  // the merge is told the score layout
      const float l = n > 0 ? blse[b] : 0.f;
      for (int j = lane; j < (int)S; j += 64) {
        float v = -INFINITY;
        if (r >= 0 && n > 0) {
          if (!dense) {
            if (j < n) v = (tix ? zb[tab.tok[bbase[b] + j]] : zb[j]) - l;
          } else {
            const DWord dw = dense_word<NX>(tab, r, j >> 5);
            const uint32_t x = dw.bits;
            if ((x >> (j & 31)) & 1u)
              v = (tix ? zb[j] : zb[dw.rank + __popc(x & ((1u << (j & 31)) - 1u))]) - l;
          }
        }
        dbg[j] = v;
      }
    }
  }
  uint32_t omax = omax_sh;

  if constexpr (MERGE) {
    // the parts' keys (already final) into LDS, in part order
    const int exp_ = block_excl_scan<NT>(mcnt, sh, &C);
    if ((int)threadIdx.x < P) {
      mpre[threadIdx.x] = exp_;
      mcn[threadIdx.x] = mcnt;
    }
    __syncthreads();
    uint32_t o = 0;
    for (int f = threadIdx.x; f < P * K; f += NT) {
      const int pi = f / K, i = f - pi * K;
      if (i < mcn[pi]) {
        const uint64_t kk = (f == (int)threadIdx.x) ? mkey0 : part_keys[(int64_t)(q * P + pi) * K + i];
        keys[mpre[pi] + i] = kk;
        o = max(o, (uint32_t)(kk >> 32));
      }
    }
    xor_down<32>([&](auto d) { o = max(o, xor_lane<decltype(d)::value>(o)); });
    if (lane == 0) sh[wave] = (int)o;
    __syncthreads();
    omax = 0;
    for (int i = 0; i < kSelWaves; ++i) omax = max(omax, (uint32_t)sh[i]);
    store = true;
    __syncthreads();
  }

  // 4. keys: ord(cum + (z - lse)) over ~(beam*S + slot); the K largest.
  // Log-scaled histogram of each key's distance below the best key's ord:
  // bins above the boundary bin are taken whole, the boundary bin is resolved
  // exactly among its own keys.
  // Few stored keys skip the histogram: each is ranked directly below.
  auto bin_of = [&](uint64_t k) { return dist_bin(omax - (uint32_t)(k >> 32)); };
  const bool small = store && C <= kSmallSel;
  const bool histo = C > K && !small;
  if (histo) {
    for (int i = threadIdx.x; i < kDistBins; i += NT) dhist[i] = 0;
    __syncthreads();
  }
  if (MERGE) {
    if (histo) {
      for (int i = threadIdx.x; i < C; i += NT) atomicAdd(&dhist[bin_of(keys[i])], 1);
      __syncthreads();
    }
  } else if (store) {
    for (int i = threadIdx.x; i < C; i += NT) {
      const uint64_t e = keys[i];
      const uint32_t code = (uint32_t)e;
      const int bl = (int)(code / S);
      const float zv = __uint_as_float((uint32_t)(e >> 32));
      const uint64_t k = zkey ? make_key(zv, code) : make_key(bcum[bl] + (zv - blse[bl]), code);
      keys[i] = k;
      if (histo) atomicAdd(&dhist[bin_of(k)], 1);
    }
    __syncthreads();
  }
  // without room in LDS, keys are recomputed from z in every pass, over this
  // part's flat range; on dense rows LPE threads share a bitmap word (each
  // walks 32 / LPE of its bits) while that leaves no thread idle
  int LPE = 1;
  if (dense)
    while (LPE < 32 && pairs * LPE * 2 <= NT) LPE *= 2;
  auto enumerate = [&](auto&& fn) {
    if (!dense) {
      for (int f = f0 + threadIdx.x; f < f1; f += NT) {
        const int bl = beam_of(f), i = f - cpre[bl];
        const float* zb = z + (int64_t)(b0 + bl) * ldz;
        const float zv = TOKEN_IDX ? zb[tab.tok[bbase[bl] + i]] : zb[i];
        fn(zkey ? make_key(zv, code_of(bl, i)) : make_key(bcum[bl] + (zv - blse[bl]), code_of(bl, i)));
      }
      return;
    }
    for (int f2 = threadIdx.x; f2 < pairs * LPE; f2 += NT) {
      const int pr = f2 / LPE, sub = f2 - pr * LPE;
      const int bl = bl_lo + pr / tab.words, i = pr % tab.words;
      const int r = brow[bl];
      if (r < 0) continue;
      const float c = bcum[bl], l = blse[bl];
      const float* zb = z + (int64_t)(b0 + bl) * ldz;
      const DWord dw = dense_word<NX>(tab, r, i);
      const int nb = 32 / LPE, lo = sub * nb;  // this thread's bits [lo, lo + nb)
      uint32_t y = (dw.bits >> lo) & (nb == 32 ? 0xFFFFFFFFu : ((1u << nb) - 1u));
      int j = dw.rank + __popc(dw.bits & ((1u << lo) - 1u));
      while (y) {
        const int v = (i << 5) + lo + __ffs(y) - 1;
        y &= y - 1;
        const int f = cpre[bl] + j;
        if (f >= f0 && f < f1) {
          const float zv = TOKEN_IDX ? zb[v] : zb[j];
          fn(zkey ? make_key(zv, code_of(bl, v)) : make_key(c + (zv - l), code_of(bl, v)));
        }
        ++j;
      }
    }
  };
  const int nsel = min(C, K);
  if (small) {
    // rank of a key = number of keys above it (keys are distinct); G lanes
    // share a key, each counting over a strided part; the K best land in
    // sel[] already in order
    int G = 1;
    while (G < 64 && G * 2 * max(C, 1) <= NT) G *= 2;
    const int per = NT / G;
    for (int i0 = 0; i0 < C; i0 += per) {
      const int i = i0 + (int)threadIdx.x / G, g = (int)threadIdx.x % G;
      const uint64_t mine = i < C ? keys[i] : 0ull;
      int rank = 0;
      if (i < C)
        for (int j0 = g; j0 < C; j0 += 8 * G) {
          // eight independent LDS reads in flight: the reads are
          // unconditional (clamped index), the bound applies to the count
          uint64_t kk[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) kk[u] = keys[min(j0 + u * G, C - 1)];
#pragma unroll
          for (int u = 0; u < 8; ++u) rank += (j0 + u * G < C && kk[u] > mine) ? 1 : 0;
        }
      xor_down_width(G, [&](auto o) { rank += xor_lane<decltype(o)::value>(rank); });
      if (i < C && g == 0 && rank < K) sel[rank] = mine;
    }
  } else if (C <= K) {
    for (int i = threadIdx.x; i < C; i += NT) sel[i] = keys[i];  // C <= K <= kKeyCap: stored
  } else {
    if (!store) {
      enumerate([&](uint64_t k) { atomicAdd(&dhist[bin_of(k)], 1); });
      __syncthreads();
    }
    // thread i owns bins 2i, 2i+1 (bin order = decreasing key)
    const int h0 = dhist[2 * threadIdx.x], h1 = dhist[2 * threadIdx.x + 1];
    int tot;
    const int ex2 = block_excl_scan<NT>(h0 + h1, sh, &tot);
    if (ex2 < K && ex2 + h0 + h1 >= K) {
      if (ex2 + h0 >= K) {
        pick_bin = 2 * threadIdx.x;
        pick_above = ex2;
      } else {
        pick_bin = 2 * threadIdx.x + 1;
        pick_above = ex2 + h0;
      }
    }
    if (threadIdx.x == 0) {
      pos = 0;
      pos2 = 0;
    }
    __syncthreads();
    const int bstar = pick_bin, above = pick_above, need = K - above;
    uint64_t* bnd = (uint64_t*)dhist;  // the histogram is done: its space holds the boundary keys
    if (store) {
      for (int i0 = 0; i0 < C; i0 += NT) {
        const int i = i0 + threadIdx.x;
        const uint64_t k = i < C ? keys[i] : 0ull;
        const int bn = i < C ? bin_of(k) : kDistBins;
        // the wave's selected and boundary keys as two lane masks: a lane's
        // append position is the count of its category's lanes below it
        const uint64_t m1 = __ballot(bn < bstar), m2 = __ballot(bn == bstar);
        if ((m1 | m2) == 0) continue;  // wave-uniform: nothing to keep here
        int b1 = 0, b2 = 0;
        if (lane == 0) {
          if (m1) b1 = atomicAdd(&pos, __popcll(m1));
          if (m2) b2 = atomicAdd(&pos2, __popcll(m2));
        }
        // lane 0's results to the whole wave (scalar read, every lane is active)
        b1 = __builtin_amdgcn_readfirstlane(b1);
        b2 = __builtin_amdgcn_readfirstlane(b2);
        const uint64_t lower = (1ull << lane) - 1ull;
        const int a1 = b1 + __popcll(m1 & lower), a2 = b2 + __popcll(m2 & lower);
        if (bn < bstar && a1 < kMaxK) sel[a1] = k;
        if (bn == bstar && a2 < kBoundary) bnd[a2] = k;
      }
    } else {
      enumerate([&](uint64_t k) {
        const int bn = bin_of(k);
        if (bn < bstar) {
          const int p = atomicAdd(&pos, 1);
          if (p < kMaxK) sel[p] = k;
        }
        if (bn == bstar) {
          const int a2 = atomicAdd(&pos2, 1);
          if (a2 < kBoundary) bnd[a2] = k;
        }
      });
    }
    __syncthreads();
    const int nb = pos2;
    if (nb <= kBoundary) {
      // exact among the boundary keys: rank = keys above it (keys are distinct)
      if ((int)threadIdx.x < nb) {
        const uint64_t k = bnd[threadIdx.x];
        int rk = 0;
        for (int j = 0; j < nb; ++j) rk += bnd[j] > k ? 1 : 0;
        if (rk < need) sel[above + rk] = k;
      }
    } else {
      // very many keys in one bin (e.g. exactly tied scores): radix select
      // over the full keys of that bin
      RadixSel rs{0, 0, need};
      for (int shift = 56; shift >= 0; shift -= 8) {
        if (threadIdx.x < 256) hist[threadIdx.x] = 0;
        __syncthreads();
        auto count = [&](uint64_t k) {
          if (bin_of(k) == bstar && (k & rs.mask) == rs.prefix) atomicAdd(&hist[(k >> shift) & 0xFF], 1);
        };
        if (store) {
          for (int i = threadIdx.x; i < C; i += NT) count(keys[i]);
        } else {
          enumerate(count);
        }
        __syncthreads();
        if (radix_narrow<NT>(rs, shift, hist, sh)) break;
      }
      if (threadIdx.x == 0) pos = above;
      __syncthreads();
      auto take = [&](uint64_t k) {
        if (bin_of(k) == bstar && (k & rs.mask) >= rs.prefix) {
          const int p = atomicAdd(&pos, 1);
          if (p < kMaxK) sel[p] = k;
        }
      };
      if (store) {
        for (int i = threadIdx.x; i < C; i += NT) take(keys[i]);
      } else {
        enumerate(take);
      }
    }
  }
  __syncthreads();

  if (!MERGE && P > 1) {
    // a part: its best keys go to the merge (in any order)
    for (int i = threadIdx.x; i < nsel; i += NT) part_keys[(int64_t)blockIdx.x * K + i] = sel[i];
    if (threadIdx.x == 0) {
      part_cnt[blockIdx.x] = nsel;
      if (zkey) part_ms[blockIdx.x] = zms_sh;
    }
    return;
  }

  // 5. sorted position of a selected key = number of selected keys above it;
  //    G = NT / nsel lanes (a power of two, within one wave) share a key,
  //    each counting over a strided part of the selection (the direct ranking
  //    above already left them in order).  Rank counting moves 8 nsel^2 bytes
  //    through LDS, so more than 256 keys go through a bitonic network in
  //    place instead.
  const bool in_order = small;
  const bool bitonic = !in_order && nsel > 256;
  const uint64_t* sorted = (in_order || bitonic) ? sel : keys;
  if (bitonic) {
    int n2 = 1;
    while (n2 < nsel) n2 <<= 1;  // <= kMaxK
    for (int i = nsel + threadIdx.x; i < n2; i += NT) sel[i] = 0ull;  // padding sorts last
    __syncthreads();
    for (int k2 = 2; k2 <= n2; k2 <<= 1)
      for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1) {
        for (int i = threadIdx.x; i < n2; i += NT) {
          const int l = i ^ j2;
          if (l > i) {
            const uint64_t x = sel[i], y = sel[l];
            // descending where (i & k2) == 0, so the last round is descending
            if (((i & k2) == 0) ? (x < y) : (x > y)) {
              sel[i] = y;
              sel[l] = x;
            }
          }
        }
        __syncthreads();
      }
  } else if (!in_order) {
    int G = 1;
    while (G < 64 && G * 2 * max(nsel, 1) <= NT) G *= 2;
    const int i = threadIdx.x / G, g = threadIdx.x - i * G;
    uint64_t mine = 0;
    int rank = 0;
    if (i < nsel) {
      mine = sel[i];
      for (int j = g; j < nsel; j += G) rank += sel[j] > mine ? 1 : 0;
    }
    xor_down_width(G, [&](auto o) { rank += xor_lane<decltype(o)::value>(rank); });
    __syncthreads();
    if (i < nsel && g == 0) keys[rank] = mine;
    __syncthreads();
  }
  for (int o = threadIdx.x; o < K; o += NT) {
    const int64_t oi = (int64_t)q * K + o;
    if (o < nsel) {
      const uint64_t key = sorted[o];
      const uint32_t code = 0xFFFFFFFFu - (uint32_t)key;
      const int bl = (int)(code / S);
      const int slot = (int)(code - (uint32_t)bl * S);
      const int b = b0 + bl;
      const int r = brow[bl];
      int token, next;
      if (!dense) {
        next = bbase[bl] + slot;  // the entry's position is its next row
        token = tab.tok[next];
      } else {
        token = slot;
        // entries of the row before this token: the count before its word,
        // then popcount within the word
        const DWord dw = dense_word<NX>(tab, r, slot >> 5);
        next = all_legal ? 0 : bbase[bl] + dw.rank + __popc(dw.bits & ((1u << (slot & 31)) - 1u));
      }
      parent_out[oi] = b;
      token_out[oi] = token;
      row_out[oi] = next;
      // split single-beam requests ranked by the score: cum = cum_in + (z - lse)
      cum_out[oi] = zkey ? bcum[bl] + (float_of_ord((uint32_t)(key >> 32)) - blse[bl])
                         : float_of_ord((uint32_t)(key >> 32));
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

constexpr int kTileKBytes = 128;
constexpr int kLdsRow = kTileKBytes + 16;  // padded row pitch in bytes

// C[m][n] = sum_k A[m][k] * B[n][k]: A = hidden [M][D], B = W_t [N][D], both
// k-contiguous.  BM x BN block tile, 4 waves in 2x2 each owning (BM/2)x(BN/2)
// (8 waves in 2x4 for 16-bit 128x128 tiles, see gemm_threads) as MFMA 32x32
// blocks, 128-byte k-slices staged through LDS with a register
// prefetch of the next slice.
// compact != 0 (dense table): only legal columns are written, at their legal
// rank within the beam's row (rank directory + popcount below the column);
// dead beams are skipped.  The tile's rows, bitmap words and rank entries are
// loaded into LDS before the k loop so the epilogue does not wait on them.
// compact == 0: full rows, column = token.
// SP: sparse table (compact == 2): the tile is staged in LDS after the k
// loop and only the rows' legal columns are written, at their slot (the
// token's position in the row), so the scores of a sparse step take the
// same layout as under the selective projection; each row's first token in
// the tile's column range is found before the product.
// Tile order of the tiled GEMM.  Blocks are dealt to the 8 XCDs in turn;
// with at least 8 row blocks, XCD x takes the row blocks tm = x (mod 8) and
// walks them in groups of up to 16, every column tile of a group with the
// group's row blocks side by side, so the blocks an XCD runs at once share
// their hidden rows and weight rows in its L2 (consecutive blocks on
// different XCDs would each stream the same hidden rows).  Blocks padding the
// last group of an XCD have no tile (tm = -1).
struct GemmOrder {
  int nbm, nbn, gm, nlr_pad;
  __host__ __device__ GemmOrder(int M, int N, int BM, int BN) {
    nbm = (M + BM - 1) / BM;
    nbn = (N + BN - 1) / BN;
    const int nlr = (nbm + 7) / 8;
    gm = nlr < 16 ? nlr : 16;
    nlr_pad = (nlr + gm - 1) / gm * gm;
  }
  __host__ __device__ bool by_xcd() const { return nbm >= 8; }
  __host__ __device__ int64_t blocks() const {
    return by_xcd() ? (int64_t)8 * nlr_pad * nbn : (int64_t)nbm * nbn;
  }
  __device__ void tile(int bid, int& tm, int& tn) const {
    if (!by_xcd()) {
      tm = bid % nbm;
      tn = bid / nbm;
      return;
    }
    const int x = bid & 7, j = bid >> 3;
    const int tmi = j % gm, rest = j / gm;
    tn = rest % nbn;
    const int lr = (rest / nbn) * gm + tmi;
    tm = lr * 8 + x;
    if (tm >= nbm) tm = -1;
  }
};

// Threads of a GEMM block: 16-bit 128x128 tiles run 8 waves (2 x 4, 64x32
// each), which hide more of the k loop's load latency (the 1e7-item
// V = 4,096 step 2: 34.7 -> 31.0 us); fp32 and 64x64 tiles keep 4 (2 x 2).
constexpr int gemm_threads(int dt, int bm) { return (bm == 128 && dt != ZGR_F32) ? 512 : kThreads; }

template <int DT, int BM, int BN, bool NX, bool SP>
__global__ __launch_bounds__(gemm_threads(DT, BM)) void k_gemm_nt(const void* __restrict__ A,
                                                      const void* __restrict__ Bm,
                                                      float* __restrict__ C, int32_t M, int32_t N,
                                                      int32_t D, int64_t ldc, int32_t compact,
                                                      DevTable tab,
                                                      const int32_t* __restrict__ row_in,
                                                      float2* __restrict__ zms) {
  constexpr int ES = (DT == ZGR_F32) ? 4 : 2;
  constexpr int TK = kTileKBytes / ES;  // k elements per slice
  constexpr int NT = gemm_threads(DT, BM);
  constexpr int NWX = NT / 128;  // waves along N (two along M)
  constexpr int WM = BM / 2, WN = BN / NWX, IB = WM / 32, JB = WN / 32;
  constexpr int NA = BM * 8 / NT, NB = BN * 8 / NT;  // 16-byte chunks per thread
  constexpr int TW = BN / 32;                                     // bitmap words per tile row
  constexpr int STAGE = (BM + BN) * kLdsRow;
  constexpr int CTILE = SP ? BM * (BN + 1) * 4 : 0;  // staged output tile (sparse epilogue)
  // 64x64 tiles keep two stages (slice s is read from one while slice s + 1
  // is written to the other, one barrier per slice); 128x128 tiles one, so
  // that three blocks fit a CU's LDS (two stages measured slower there:
  // 71.2 against 65.8 us for the f16 step 2 of the dense-early catalog)
  constexpr int NST = BM * BN <= 64 * 64 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) char smem[NST * STAGE > CTILE ? NST * STAGE : CTILE];
  __shared__ int2 tword[BM * TW];  // a tile row's bitmap word and its legal rank, together
  int tm, tn;
  GemmOrder(M, N, BM, BN).tile((int)blockIdx.x, tm, tn);
  if (tm < 0) return;  // padding block (before any barrier)
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / NWX, wn = wave % NWX;
  const char* Ab = (const char*)A;
  const char* Bb = (const char*)Bm;
  const int64_t rowbytes = (int64_t)D * ES;
  // compact epilogue: the tile rows' bitmap words and ranks are loaded into
  // registers now (thread i < BM owns tile row i) and reach LDS only after
  // the k loop, so their two dependent loads overlap the product
  static_assert(BM <= NT, "one tile row per thread");
  DWord pdw[TW];
#pragma unroll
  for (int k = 0; k < TW; ++k) pdw[k] = DWord{0u, 0};
  int sp_base = 0, sp_n = 0, sp_lo = 0;  // sparse: the row's entries, first one in the tile
  if (compact == 1 && (int)threadIdx.x < BM) {
    const int gm = m0 + threadIdx.x;
    const int r = gm < M ? row_in[gm] : -1;
    if (r >= 0 && r < tab.rows) {
#pragma unroll
      for (int k = 0; k < TW; ++k) {
        const int wd = (n0 >> 5) + k;
        if (wd < tab.words) pdw[k] = dense_word<NX>(tab, r, wd);
      }
    }
  }
  if constexpr (SP) {
    if ((int)threadIdx.x < BM) {
      const int gm = m0 + threadIdx.x;
      const int r = gm < M ? row_in[gm] : -1;
      if (r >= 0 && r < tab.rows) {
        sp_base = tab.row_ptr[r];
        sp_n = tab.row_ptr[r + 1] - sp_base;
        int lo = 0, hi = sp_n;  // first entry with token >= n0
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((int)tab.tok[sp_base + mid] < n0)
            lo = mid + 1;
          else
            hi = mid;
        }
        sp_lo = lo;
      }
    }
  }
  // global -> register staging of A and B slices.  Each load's row pointer
  // is formed once; rows past M or N read zeros.  A tile wholly inside both
  // (every tile but the edges) issues its loads without per-load guards.
  uint4 ra[NA], rb[NB];
  const char* pa[NA];
  const char* pb[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int c = threadIdx.x + i * NT;
    const int gm = m0 + (c >> 3);
    pa[i] = gm < M ? Ab + (int64_t)gm * rowbytes + (c & 7) * 16 : nullptr;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int c = threadIdx.x + i * NT;
    const int gn = n0 + (c >> 3);
    pb[i] = gn < N ? Bb + (int64_t)gn * rowbytes + (c & 7) * 16 : nullptr;
  }
  const bool whole = m0 + BM <= M && n0 + BN <= N;  // uniform over the block
  auto gload = [&](int kbyte) {
    if (whole) {
#pragma unroll
      for (int i = 0; i < NA; ++i) ra[i] = *(const uint4*)(pa[i] + kbyte);
#pragma unroll
      for (int i = 0; i < NB; ++i) rb[i] = *(const uint4*)(pb[i] + kbyte);
    } else {
#pragma unroll
      for (int i = 0; i < NA; ++i) ra[i] = pa[i] ? *(const uint4*)(pa[i] + kbyte) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < NB; ++i) rb[i] = pb[i] ? *(const uint4*)(pb[i] + kbyte) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int st) {
    char* As = smem + st * STAGE;
    char* Bs = As + BM * kLdsRow;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = threadIdx.x + i * NT;
      *(uint4*)(As + (c >> 3) * kLdsRow + (c & 7) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = threadIdx.x + i * NT;
      *(uint4*)(Bs + (c >> 3) * kLdsRow + (c & 7) * 16) = rb[i];
    }
  };
  f32x16 acc[IB][JB];
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int half = lane >> 5, l32 = lane & 31;
  // k loop over 128-byte slices.  Two stages: the MFMAs read slice s from
  // one while the registers loaded during slice s - 1 fill the other with
  // slice s + 1 and the loads of slice s + 2 are issued.  One stage: the
  // slice is stored after a barrier and the next slice's loads are issued.
  const int nsl = (int)(rowbytes / kTileKBytes);
  gload(0);
  if constexpr (NST == 2) {
    sstore(0);
    if (nsl > 1) gload(kTileKBytes);
    __syncthreads();
  }
  for (int sl = 0; sl < nsl; ++sl) {
    if constexpr (NST == 1) {
      __syncthreads();
      sstore(0);
      __syncthreads();
      if (sl + 1 < nsl) gload((sl + 1) * kTileKBytes);
    }
    const char* As = smem + (sl & (NST - 1)) * STAGE;
    const char* Bs = As + BM * kLdsRow;
    if constexpr (DT == ZGR_F32) {
      // per 8-wide k chunk: lanes 0-31 hold k 0..3, lanes 32-63 k 4..7 of their
      // row; four 32x32x2 MFMAs pair (k, k+4) - the same pairing for A and B.
#pragma unroll
      for (int kc = 0; kc < TK / 8; ++kc) {
        const int off = kc * 32 + half * 16;
        f32x4 a[IB], bv[JB];
#pragma unroll
        for (int i = 0; i < IB; ++i) a[i] = *(const f32x4*)(As + (wm * WM + i * 32 + l32) * kLdsRow + off);
#pragma unroll
        for (int j = 0; j < JB; ++j) bv[j] = *(const f32x4*)(Bs + (wn * WN + j * 32 + l32) * kLdsRow + off);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < IB; ++i)
#pragma unroll
            for (int j = 0; j < JB; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], bv[j][s], acc[i][j], 0, 0, 0);
      }
    } else {
      // per 16-wide k chunk: lanes 0-31 hold k 0..7, lanes 32-63 k 8..15.
#pragma unroll
      for (int kc = 0; kc < TK / 16; ++kc) {
        const int off = kc * 32 + half * 16;
        uint4 ua[IB], ub[JB];
#pragma unroll
        for (int i = 0; i < IB; ++i) ua[i] = *(const uint4*)(As + (wm * WM + i * 32 + l32) * kLdsRow + off);
#pragma unroll
        for (int j = 0; j < JB; ++j) ub[j] = *(const uint4*)(Bs + (wn * WN + j * 32 + l32) * kLdsRow + off);
#pragma unroll
        for (int i = 0; i < IB; ++i)
#pragma unroll
          for (int j = 0; j < JB; ++j) {
            if constexpr (DT == ZGR_BF16) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, ua[i]), __builtin_bit_cast(bf16x8, ub[j]), acc[i][j], 0, 0, 0);
            } else {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(f16x8, ua[i]), __builtin_bit_cast(f16x8, ub[j]), acc[i][j], 0, 0, 0);
            }
          }
      }
    }
    if constexpr (NST == 2) {
      if (sl + 1 < nsl) {
        sstore((sl + 1) & 1);  // the other stage, last read before the previous barrier
        if (sl + 2 < nsl) gload((sl + 2) * kTileKBytes);
      }
      __syncthreads();
    }
  }
  // 32x32 accumulator layout: lane -> column l32, register v -> row 8*(v/4) + 4*half + v%4
  if constexpr (SP) {
    float* Ct = (float*)smem;
    __syncthreads();  // every wave is done reading the staged operands
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        const int col = wn * WN + j * 32 + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = wm * WM + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          Ct[rl * (BN + 1) + col] = acc[i][j][v];
        }
      }
    __syncthreads();
    if ((int)threadIdx.x < BM && sp_lo < sp_n) {
      float* zrow = C + (int64_t)(m0 + threadIdx.x) * ldc;
      const float* crow = Ct + threadIdx.x * (BN + 1);
      for (int j0 = sp_lo; j0 < sp_n; j0 += 8) {
        int tk[8];  // eight token loads in flight (clamped, unconditional)
#pragma unroll
        for (int u = 0; u < 8; ++u) tk[u] = tab.tok[sp_base + min(j0 + u, sp_n - 1)];
        bool done = false;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int jj = j0 + u;
          if (jj >= sp_n || tk[u] >= n0 + BN) {
            done = true;
          } else if (!done) {
            zrow[jj] = crow[tk[u] - n0];
          }
        }
        if (done) break;
      }
    }
    return;
  }
  if (!compact) {
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        const int col = n0 + wn * WN + j * 32 + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * WM + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          if (row < M && col < N) C[(int64_t)row * ldc + col] = acc[i][j][v];
        }
      }
    return;
  }
  if ((int)threadIdx.x < BM) {
#pragma unroll
    for (int k = 0; k < TW; ++k) {
      tword[threadIdx.x * TW + k] = make_int2((int)pdw[k].bits, pdw[k].rank);
    }
  }
  __syncthreads();
  // Each output: one LDS read (word and rank), a bit test, a popcount and a
  // 32-bit offset from the lane's first row (rows of the tile differ by a
  // constant times ldc; the compact rows have ldc = V <= 65536, so the
  // offsets stay below 2^31).
  // With zms, each row also gets the legal (max, sum of exp) of each 32-column
  // bitmap word: a 32x32 block's 16 rows per lane half are reduced over the
  // half's 32 lanes (four halving exchanges within 16-lane rows, then one
  // across them), after which lanes i and i + 16 of the half hold the pair of
  // row rev(i).
  const int ldc32 = (int)ldc;
  const uint32_t below = (1u << l32) - 1u;
  float* cw = C + (int64_t)(m0 + wm * WM + 4 * half) * ldc;
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int kw = (wn * WN + j * 32) >> 5;  // the block's 32 columns are one bitmap word
      float pm[16], ps[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ro = i * 32 + 8 * (v >> 2) + (v & 3);  // row within the lane's rows
        const int2 wr = tword[(wm * WM + 4 * half + ro) * TW + kw];
        const uint32_t x = (uint32_t)wr.x;
        const bool legal = (x >> l32) & 1u;
        if (legal) cw[ro * ldc32 + wr.y + (int)__popc(x & below)] = acc[i][j][v];
        pm[v] = legal ? acc[i][j][v] : -INFINITY;
        ps[v] = legal ? 1.f : 0.f;
      }
      if (zms) {  // uniform
        ms_halve<16, 16, 1>(pm, ps, l32);
        ms_join(pm[0], ps[0], xor_lane<16>(pm[0]), xor_lane<16>(ps[0]));
        const int v = ((l32 & 1) << 3) | ((l32 & 2) << 1) | ((l32 & 4) >> 1) | ((l32 & 8) >> 3);
        const int row = m0 + wm * WM + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        const int wd = (n0 >> 5) + kw;
        if (l32 < 16 && row < M && wd < tab.words)
          zms[(int64_t)row * tab.words + wd] = make_float2(pm[0], ps[0]);
      }
    }
}

// ---------------------------------------------------------------- k_gemm_small (MFMA 16x16)

// Full projection for few beams (the first step has one beam per request):
// 32x32 output tiles per block, one 16x16 MFMA tile per wave, operands
// streamed from global memory with 16-byte loads (the four 16-lane groups of
// a wave cover 64 contiguous bytes of each row).  The k order inside a 64-byte
// chunk is permuted identically for both operands.  Few blocks run, so each
// tile is split over two wave groups by halves of the hidden size (summed
// through LDS) and a wave keeps 8 chunks of loads in flight; the compact
// epilogue's row lookups are issued before the product.
constexpr int kSmallThreads = 512;

template <int DT, bool NX>
__global__ __launch_bounds__(kSmallThreads) void k_gemm_small(const void* __restrict__ A,
                                                              const void* __restrict__ Bm,
                                                              float* __restrict__ C, int32_t M,
                                                              int32_t N, int32_t D, int64_t ldc,
                                                              int32_t compact, DevTable tab,
                                                              const int32_t* __restrict__ row_in,
                                                              float2* __restrict__ zms) {
  __shared__ uint32_t tbits[32];
  __shared__ float2 wms[2][32];  // zms: each column half's (max, sum of exp) per tile row
  __shared__ int trank[32];
  __shared__ f32x4 part[4][64];
  constexpr int ES = (DT == ZGR_F32) ? 4 : 2;
  constexpr int U = 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tw = wave & 3, ks = wave >> 2;  // tile quarter, k half
  const int nbn = (N + 31) / 32;
  const int tm = blockIdx.x / nbn, tn = blockIdx.x - tm * nbn;
  const int l16 = lane & 15, g = lane >> 4;
  const int m = tm * 32 + (tw >> 1) * 16 + l16;
  const int n = tn * 32 + (tw & 1) * 16 + l16;
  const int64_t rowbytes = (int64_t)D * ES;
  const int nch = (int)(rowbytes / 64);
  const int c0 = ks * (nch / 2), c1 = ks ? nch : nch / 2;
  DWord pdw{0u, 0};
  if (compact && threadIdx.x < 32) {
    const int gm = tm * 32 + threadIdx.x;
    const int r = gm < M ? row_in[gm] : -1;
    if (r >= 0 && r < tab.rows && tn < tab.words) pdw = dense_word<NX>(tab, r, tn);
  }
  const char* ap = (const char*)A + (int64_t)min(m, M - 1) * rowbytes + g * 16;
  const char* bp = (const char*)Bm + (int64_t)min(n, N - 1) * rowbytes + g * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c = c0; c < c1; c += U) {
    uint4 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c + u < c1) {
        a[u] = *(const uint4*)(ap + (int64_t)(c + u) * 64);
        b[u] = *(const uint4*)(bp + (int64_t)(c + u) * 64);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c + u >= c1) break;
      if constexpr (DT == ZGR_F32) {
        const f32x4 av = __builtin_bit_cast(f32x4, a[u]);
        const f32x4 bv = __builtin_bit_cast(f32x4, b[u]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc, 0, 0, 0);
      } else if constexpr (DT == ZGR_BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u]),
                                                      __builtin_bit_cast(bf16x8, b[u]), acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[u]),
                                                     __builtin_bit_cast(f16x8, b[u]), acc, 0, 0, 0);
      }
    }
  }
  // the second k half hands its partial tile to the first
  if (ks) part[tw][lane] = acc;
  if (compact && threadIdx.x < 32) {
    tbits[threadIdx.x] = pdw.bits;
    trank[threadIdx.x] = pdw.rank;
  }
  __syncthreads();
  if (!ks) {
    const f32x4 o = part[tw][lane];
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] += o[v];
  }
  // 16x16 accumulator layout: lane -> column l16, register v -> row 4*g + v
  if (zms) {  // uniform: a dense table's compact epilogue
    // each tile row's legal (max, sum of exp) over the block's 32 columns
    // (one bitmap word): a wave's 4 rows per lane group are reduced over the
    // group's 16 lanes (halving over lane offsets 1 and 2, then offsets 4 and
    // 8, all within a 16-lane row), lanes 0-3 of the group hold row rev(l16),
    // and the two column halves are joined through LDS in a fixed order
    if (!ks) {
      const int bitq = (tw & 1) * 16 + l16;
      float pm[4], ps[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool legal = (tbits[(tw >> 1) * 16 + 4 * g + v] >> bitq) & 1u;
        pm[v] = legal ? acc[v] : -INFINITY;
        ps[v] = legal ? 1.f : 0.f;
      }
      ms_halve<4, 4, 1>(pm, ps, l16);
      ms_join(pm[0], ps[0], xor_lane<4>(pm[0]), xor_lane<4>(ps[0]));
      ms_join(pm[0], ps[0], xor_lane<8>(pm[0]), xor_lane<8>(ps[0]));
      const int v = ((l16 & 1) << 1) | ((l16 & 2) >> 1);
      if (l16 < 4) wms[tw & 1][(tw >> 1) * 16 + 4 * g + v] = make_float2(pm[0], ps[0]);
    }
    __syncthreads();
    if (threadIdx.x < 32) {
      const int row = tm * 32 + threadIdx.x;
      float m = wms[0][threadIdx.x].x, sm = wms[0][threadIdx.x].y;
      ms_join(m, sm, wms[1][threadIdx.x].x, wms[1][threadIdx.x].y);
      if (row < M && tn < tab.words) zms[(int64_t)row * tab.words + tn] = make_float2(m, sm);
    }
  }
  if (ks) return;
  if (!compact) {
    if (n < N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = tm * 32 + (tw >> 1) * 16 + 4 * g + v;
        if (row < M) C[(int64_t)row * ldc + n] = acc[v];
      }
    }
    return;
  }
  // dense table: legal columns only, at their legal rank (the block's 32
  // columns are one bitmap word)
  const int bit = (tw & 1) * 16 + l16;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rl = (tw >> 1) * 16 + 4 * g + v;
    const uint32_t x = tbits[rl];
    if ((x >> bit) & 1u)
      C[(int64_t)(tm * 32 + rl) * ldc + trank[rl] + __popc(x & ((1u << bit) - 1u))] = acc[v];
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
  const bool live = cum[src] != -INFINITY;
  item_out[i] = live ? row[src] : -1;
  if (score_out) score_out[i] = cum[src];
  if (sid_out)
    for (int l = 0; l < L; ++l) sid_out[(int64_t)i * L + l] = live ? prefix[(int64_t)src * L + l] : -1;
}

// Item id of each final beam's SID, found by walking the step tables from the
// root (sparse rows: binary search among the row's sorted tokens, the entry's
// position is the next row; dense rows: the bitmap bit, rank directory and
// popcount).  -1 when the SID is not in the catalog (possible only for codes
// produced without the filter) or the beam is empty.
struct TableSet {
  DevTable t[kMaxL];
};

__global__ void k_lookup_items(TableSet ts, int32_t L, const int32_t* __restrict__ prefix,
                               const float* __restrict__ cum, int32_t n, int32_t* __restrict__ item) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int64_t r = 0;
  if (cum[i] == -INFINITY) r = -1;
  for (int l = 0; l < L && r >= 0; ++l) {
    const DevTable& tb = ts.t[l];
    const int v = prefix[(int64_t)i * L + l];
    if (v < 0 || v >= tb.V || r >= tb.rows) {
      r = -1;
      break;
    }
    const int lo0 = tb.row_ptr[r], hi0 = tb.row_ptr[r + 1];
    if (tb.fmt == ZGR_FMT_SPARSE) {
      int lo = lo0, hi = hi0;  // first entry with token >= v
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int)tb.tok[mid] < v)
          lo = mid + 1;
        else
          hi = mid;
      }
      r = (lo < hi0 && (int)tb.tok[lo] == v) ? lo : -1;
    } else {
      const DWord dw = tb.next ? dense_word<true>(tb, r, v >> 5) : dense_word<false>(tb, r, v >> 5);
      const uint32_t x = dw.bits;
      r = ((x >> (v & 31)) & 1u) ? lo0 + dw.rank + __popc(x & ((1u << (v & 31)) - 1u)) : -1;
    }
  }
  item[i] = (int32_t)r;
}

// Log-sum-exp over all V scores of every live beam (the score-first
// normaliser): one wave per beam row, online max / sum of exp per lane, then
// a butterfly combine.
__global__ __launch_bounds__(256) void k_row_lse(const float* __restrict__ z, int64_t ldz, int32_t V,
                                                 int32_t M, const int32_t* __restrict__ row_in,
                                                 float* __restrict__ lse) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= M) return;  // wave-uniform
  if (row_in[b] < 0) {
    if (lane == 0) lse[b] = -INFINITY;
    return;
  }
  const float* zr = z + (int64_t)b * ldz;
  float m = -INFINITY, sum = 0.f;
  auto acc = [&](float v) {
    if (v > m) {
      sum = sum * __expf(m - v) + 1.f;
      m = v;
    } else {
      sum += __expf(v - m);
    }
  };
  if ((V & 3) == 0 && (ldz & 3) == 0) {
    const float4* z4 = (const float4*)zr;
    for (int i = lane; i < (V >> 2); i += 64) {
      const float4 q = z4[i];
      acc(q.x);
      acc(q.y);
      acc(q.z);
      acc(q.w);
    }
  } else {
    for (int i = lane; i < V; i += 64) acc(zr[i]);
  }
  xor_down<32>([&](auto o) {
    constexpr int X = decltype(o)::value;
    lse_combine(m, sum, xor_lane<X>(m), xor_lane<X>(sum));
  });
  if (lane == 0) lse[b] = m + __logf(sum);
}

// Tokens per dense selective tile: the tile's weight rows take at most
// kSelTileBytes (one XCD's L2).  Smaller tiles keep the rows in L2 but add
// (tile, beam) pairs, each with its own barrier, bitmap decode and hidden
// vector load; at d = 1024 fp32 a quarter-L2 tile measured 17% slower and a
// sixteenth 2.3x slower.
constexpr int64_t kSelTileBytes = 1 << 22;

int32_t dense_tile_tokens(int32_t d, int32_t dtype) {
  const int64_t row = (int64_t)d * (dtype == ZGR_F32 ? 4 : 2);
  int tt = kDenseTile;
  while (tt > 64 && tt * row > kSelTileBytes) tt >>= 1;
  return tt;
}

// Resident blocks per CU of a kernel (registers and LDS decide), so that a
// persistent grid is exactly one wave of blocks: a block that has to wait for
// another to finish would start its equal share of the work only then.
template <typename Kernel>
int resident_blocks_per_cu(Kernel kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = 1;
  }
  return n;
}

// At most this many selective-projection blocks per CU: more resident blocks
// gather more weight rows at once than an XCD's L2 keeps (1e8-item step 2,
// d = 1024 f32: 1109 us at 5 blocks per CU, 1181 us at 6).
constexpr int kSelMaxBlocksPerCu = 5;

// At most this many sparse-projection blocks per CU (the occupancy query
// decides below that).
constexpr int kSparseMaxBlocksPerCu = 8;

// The staged comparison on a dense step where its shape applies (true when
// it launched).
template <int DT, int D>
bool launch_staged(const StepArgs& a, hipStream_t s) {
  using SS = StagedShape<DT, D>;
  if constexpr (!SS::OK) {
    return false;
  } else {
    if (a.tab.fmt == ZGR_FMT_SPARSE) return false;
    if (a.tab.next)
      hipLaunchKernelGGL((k_score_staged<DT, D, true>), dim3(a.n_cu), dim3(kStageThreads), 0, s, a.M,
                         a.tab, a.row_in, a.hidden, a.W, a.z, a.ldz);
    else
      hipLaunchKernelGGL((k_score_staged<DT, D, false>), dim3(a.n_cu), dim3(kStageThreads), 0, s, a.M,
                         a.tab, a.row_in, a.hidden, a.W, a.z, a.ldz);
    return true;
  }
}

template <int DT, int D>
hipError_t launch_sel_typed(const StepArgs& a, hipStream_t s) {
  const int32_t tt = dense_tile_tokens(D, DT);
  if (a.tab.fmt == ZGR_FMT_SPARSE) {
    static const int per_cu =
        std::min(kSparseMaxBlocksPerCu, resident_blocks_per_cu(k_score_sparse<DT, D>, kThreads));
    // a sliced table needs a grid that is a multiple of kSlices
    int grid = a.n_cu * per_cu;
    if (a.tab.sdir) grid = std::max(kSlices, grid - grid % kSlices);
    hipLaunchKernelGGL((k_score_sparse<DT, D>), dim3(grid), dim3(kThreads), 0, s, a.ctot, a.umeta,
                       a.chunk_cap, a.M, a.tab, a.hidden, a.W, a.z, a.ldz);
  } else if (a.tab.next) {
    static const int per_cu =
        std::min(kSelMaxBlocksPerCu, resident_blocks_per_cu(k_score_selective<DT, D, true>, kThreads));
    hipLaunchKernelGGL((k_score_selective<DT, D, true>), dim3(a.n_cu * per_cu), dim3(kThreads), 0, s,
                       a.unit_start, a.M, a.tab, a.row_in, a.hidden, a.W, a.z, a.ldz, tt);
  } else {
    static const int per_cu =
        std::min(kSelMaxBlocksPerCu, resident_blocks_per_cu(k_score_selective<DT, D, false>, kThreads));
    hipLaunchKernelGGL((k_score_selective<DT, D, false>), dim3(a.n_cu * per_cu), dim3(kThreads), 0, s,
                       a.unit_start, a.M, a.tab, a.row_in, a.hidden, a.W, a.z, a.ldz, tt);
  }
  return hipGetLastError();
}

template <int DT, int D, bool STAGED>
hipError_t launch_sel_or_staged(const StepArgs& a, hipStream_t s) {
  if (STAGED && launch_staged<DT, D>(a, s)) return hipGetLastError();
  return launch_sel_typed<DT, D>(a, s);
}

template <int DT, bool STAGED = false>
hipError_t launch_sel_d(const StepArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_sel_or_staged<DT, 64, STAGED>(a, s);
    case 128: return launch_sel_or_staged<DT, 128, STAGED>(a, s);
    case 256: return launch_sel_or_staged<DT, 256, STAGED>(a, s);
    case 512: return launch_sel_or_staged<DT, 512, STAGED>(a, s);
    case 768: return launch_sel_or_staged<DT, 768, STAGED>(a, s);
    case 1024: return launch_sel_or_staged<DT, 1024, STAGED>(a, s);
    case 2048: return launch_sel_or_staged<DT, 2048, STAGED>(a, s);
    case 4096: return launch_sel_or_staged<DT, 4096, STAGED>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, bool NX>
hipError_t launch_proj_typed(const StepArgs& a, hipStream_t s) {
  const int V = a.tab.V;
  const bool dense = a.tab.fmt == ZGR_FMT_DENSE || a.tab.fmt == ZGR_FMT_DENSE_NEXT;
  const GemmVariant g = gemm_variant(a.M, V, dense, a.plain_z, a.n_cu);
  const int compact = g.epilogue;  // ZGR_EPI_PLAIN / DENSE / SLOT = 0 / 1 / 2
#define ZGR_GEMM(BM_, BN_, SP_)                                                                    \
  hipLaunchKernelGGL((k_gemm_nt<DT, BM_, BN_, NX, SP_>), dim3(GemmOrder(a.M, V, BM_, BN_).blocks()), \
                     dim3(gemm_threads(DT, BM_)), 0, s,                                                          \
                     a.hidden, a.W, a.z, a.M, V, a.d, a.ldz, compact, a.tab, a.row_in,                     \
                     compact == ZGR_EPI_DENSE ? a.zms : nullptr)
  if (g.kernel == ZGR_GEMM_TILED && g.tile_m == 128) {
    if (compact == ZGR_EPI_SLOT)
      ZGR_GEMM(128, 128, true);
    else
      ZGR_GEMM(128, 128, false);
  } else if (g.kernel == ZGR_GEMM_TILED) {
    if (compact == ZGR_EPI_SLOT)
      ZGR_GEMM(64, 64, true);
    else
      ZGR_GEMM(64, 64, false);
  } else {
    hipLaunchKernelGGL((k_gemm_small<DT, NX>), dim3(((a.M + 31) / 32) * ((V + 31) / 32)), dim3(kSmallThreads), 0, s,
                       a.hidden, a.W, a.z, a.M, V, a.d, a.ldz, compact, a.tab, a.row_in,
                       compact == ZGR_EPI_DENSE ? a.zms : nullptr);
  }
#undef ZGR_GEMM
  return hipGetLastError();
}

}  // namespace

GemmVariant gemm_variant(int32_t M, int32_t V, bool dense, bool plain, int32_t n_cu) {
  auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((V + bn - 1) / bn); };
  GemmVariant g{};
  // the largest tile that still gives every compute unit two blocks (or one);
  // few beams (the first step) take the 16x16-MFMA kernel
  if (tiles(128, 128) >= 2 * (int64_t)n_cu) {
    g.kernel = ZGR_GEMM_TILED;
    g.tile_m = g.tile_n = 128;
  } else if (tiles(64, 64) >= n_cu) {
    g.kernel = ZGR_GEMM_TILED;
    g.tile_m = g.tile_n = 64;
  } else {
    g.kernel = ZGR_GEMM_SMALL;
    g.tile_m = g.tile_n = 32;
  }
  // filter-first: dense rows keep their legal columns by legal rank; sparse
  // rows by slot when the tiled kernels run (the few-beam kernel writes
  // token-indexed rows there); the comparison modes keep every column
  if (plain)
    g.epilogue = ZGR_EPI_PLAIN;
  else if (dense)
    g.epilogue = ZGR_EPI_DENSE;
  else
    g.epilogue = g.kernel == ZGR_GEMM_TILED ? ZGR_EPI_SLOT : ZGR_EPI_PLAIN;
  return g;
}

bool full_projection_slot_layout(const StepArgs& a) {
  const bool dense = a.tab.fmt == ZGR_FMT_DENSE || a.tab.fmt == ZGR_FMT_DENSE_NEXT;
  return gemm_variant(a.M, a.tab.V, dense, a.plain_z, a.n_cu).epilogue == ZGR_EPI_SLOT;
}

bool supported_hidden_size(int d) {
  return d == 64 || d == 128 || d == 256 || d == 512 || d == 768 || d == 1024 || d == 2048 ||
         d == 4096;
}

hipError_t launch_units(const StepArgs& a, hipStream_t s) {
  const int nq = (a.M + 1023) / 1024;
  if (a.tab.sdir && a.tab.fmt == ZGR_FMT_SPARSE)
    hipLaunchKernelGGL(k_units<true>, dim3(nq * kSlices), dim3(1024), 0, s, a.row_in, a.M, a.tab,
                       a.ctot, a.umeta, a.chunk_cap, a.err);
  else
    hipLaunchKernelGGL(k_units<false>, dim3(nq), dim3(1024), 0, s, a.row_in, a.M, a.tab, a.ctot,
                       a.umeta, a.chunk_cap, a.err);
  return hipGetLastError();
}

hipError_t launch_selective_score(const StepArgs& a, hipStream_t s) {
  switch (a.dtype) {
    case ZGR_F32: return launch_sel_d<ZGR_F32>(a, s);
    case ZGR_BF16: return launch_sel_d<ZGR_BF16>(a, s);
    case ZGR_F16: return launch_sel_d<ZGR_F16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_staged_score(const StepArgs& a, hipStream_t s) {
  switch (a.dtype) {
    case ZGR_F32: return launch_sel_d<ZGR_F32, true>(a, s);
    case ZGR_BF16: return launch_sel_d<ZGR_BF16, true>(a, s);
    case ZGR_F16: return launch_sel_d<ZGR_F16, true>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_full_projection(const StepArgs& a, hipStream_t s) {
  const bool nx = a.tab.next != nullptr && !a.plain_z;  // only the compact epilogue reads the table
  switch (a.dtype) {
    case ZGR_F32: return nx ? launch_proj_typed<ZGR_F32, true>(a, s) : launch_proj_typed<ZGR_F32, false>(a, s);
    case ZGR_BF16: return nx ? launch_proj_typed<ZGR_BF16, true>(a, s) : launch_proj_typed<ZGR_BF16, false>(a, s);
    case ZGR_F16: return nx ? launch_proj_typed<ZGR_F16, true>(a, s) : launch_proj_typed<ZGR_F16, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

#define ZGR_STEP_ARGS                                                                            \
  a.tab, a.t, a.L, a.k_in, a.K, a.row_in, a.cum_in, a.hidden, a.W, a.z, a.ldz, a.parts,            \
      a.part_keys, a.part_cnt, a.part_ms, a.parent_out, a.token_out, a.row_out, a.cum_out, a.prefix_in,       \
      a.prefix_out, a.slot_dbg, a.lse_ext, (int32_t)a.z_token, a.zms, a.err

template <int DT, int D>
hipError_t launch_scored_step(const StepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_request_step<kZScore, DT, D, false>), dim3(a.B * a.parts), dim3(kSelThreads), 0, s,
                     ZGR_STEP_ARGS);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_scored_step_d(const StepArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_scored_step<DT, 64>(a, s);
    case 128: return launch_scored_step<DT, 128>(a, s);
    case 256: return launch_scored_step<DT, 256>(a, s);
    case 512: return launch_scored_step<DT, 512>(a, s);
    case 768: return launch_scored_step<DT, 768>(a, s);
    case 1024: return launch_scored_step<DT, 1024>(a, s);
    case 2048: return launch_scored_step<DT, 2048>(a, s);
    case 4096: return launch_scored_step<DT, 4096>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_request_step(const StepArgs& a, int zmode, hipStream_t s) {
  const dim3 grid(a.B * a.parts);
  hipError_t e = hipSuccess;
  if (zmode == kZScore) {
    switch (a.dtype) {
      case ZGR_F32: e = launch_scored_step_d<ZGR_F32>(a, s); break;
      case ZGR_BF16: e = launch_scored_step_d<ZGR_BF16>(a, s); break;
      case ZGR_F16: e = launch_scored_step_d<ZGR_F16>(a, s); break;
      default: return hipErrorInvalidValue;
    }
  } else if (zmode == kZToken) {
    if (a.tab.next)
      hipLaunchKernelGGL((k_request_step<kZToken, ZGR_F32, 64, true>), grid, dim3(kSelThreads), 0, s,
                         ZGR_STEP_ARGS);
    else
      hipLaunchKernelGGL((k_request_step<kZToken, ZGR_F32, 64, false>), grid, dim3(kSelThreads), 0, s,
                         ZGR_STEP_ARGS);
    e = hipGetLastError();
  } else if (zmode == kZPrune) {
    if (a.tab.next)
      hipLaunchKernelGGL((k_request_step<kZPrune, ZGR_F32, 64, true>), grid, dim3(kSelThreads), 0, s,
                         ZGR_STEP_ARGS);
    else
      hipLaunchKernelGGL((k_request_step<kZPrune, ZGR_F32, 64, false>), grid, dim3(kSelThreads), 0, s,
                         ZGR_STEP_ARGS);
    e = hipGetLastError();
  } else if (a.big_parts) {
    if (a.tab.next)
      hipLaunchKernelGGL((k_request_step<kZSlotBig, ZGR_F32, 64, true>), grid, dim3(kSelThreads), 0, s,
                         ZGR_STEP_ARGS);
    else
      hipLaunchKernelGGL((k_request_step<kZSlotBig, ZGR_F32, 64, false>), grid, dim3(kSelThreads), 0,
                         s, ZGR_STEP_ARGS);
    e = hipGetLastError();
  } else {
    if (a.tab.next)
      hipLaunchKernelGGL((k_request_step<kZSlot, ZGR_F32, 64, true>), grid, dim3(kSelThreads), 0, s,
                         ZGR_STEP_ARGS);
    else
      hipLaunchKernelGGL((k_request_step<kZSlot, ZGR_F32, 64, false>), grid, dim3(kSelThreads), 0, s,
                         ZGR_STEP_ARGS);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_request_merge(const StepArgs& a, hipStream_t s) {
  if (a.tab.next)
    hipLaunchKernelGGL((k_request_step<kZParts, ZGR_F32, 64, true>), dim3(a.B), dim3(kSelThreads), 0, s,
                       ZGR_STEP_ARGS);
  else
    hipLaunchKernelGGL((k_request_step<kZParts, ZGR_F32, 64, false>), dim3(a.B), dim3(kSelThreads), 0, s,
                       ZGR_STEP_ARGS);
  return hipGetLastError();
}
#undef ZGR_STEP_ARGS

hipError_t launch_naive_count(const StepArgs& a, int32_t* start, hipStream_t s) {
  hipLaunchKernelGGL(k_naive_scan, dim3(1), dim3(1024), 0, s, a.row_in, a.M, a.tab, start, a.err);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_naive_dot_typed(const StepArgs& a, const void* tmp, const int32_t* lbeam,
                                  const int32_t* start, int64_t n, hipStream_t s) {
  using Sh = SelShape<DT, D>;
  const int64_t want = (n + Sh::NG - 1) / Sh::NG;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)a.n_cu * 16));
  hipLaunchKernelGGL((k_naive_dot<DT, D>), dim3(grid), dim3(kThreads), 0, s, tmp, a.hidden, lbeam, start,
                     n, a.z, a.ldz);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_naive_dot_d(const StepArgs& a, const void* tmp, const int32_t* lbeam,
                              const int32_t* start, int64_t n, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_naive_dot_typed<DT, 64>(a, tmp, lbeam, start, n, s);
    case 128: return launch_naive_dot_typed<DT, 128>(a, tmp, lbeam, start, n, s);
    case 256: return launch_naive_dot_typed<DT, 256>(a, tmp, lbeam, start, n, s);
    case 512: return launch_naive_dot_typed<DT, 512>(a, tmp, lbeam, start, n, s);
    case 768: return launch_naive_dot_typed<DT, 768>(a, tmp, lbeam, start, n, s);
    case 1024: return launch_naive_dot_typed<DT, 1024>(a, tmp, lbeam, start, n, s);
    case 2048: return launch_naive_dot_typed<DT, 2048>(a, tmp, lbeam, start, n, s);
    case 4096: return launch_naive_dot_typed<DT, 4096>(a, tmp, lbeam, start, n, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_naive_score(const StepArgs& a, const int32_t* start, int64_t n, int32_t* lbeam,
                              int32_t* ltok, void* tmp, hipStream_t s) {
  hipLaunchKernelGGL(k_naive_compact, dim3((a.M + 3) / 4), dim3(256), 0, s, a.row_in, a.M, a.tab, start,
                     lbeam, ltok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n == 0) return e;
  const int es = a.dtype == ZGR_F32 ? 4 : 2;
  const int row_vec = a.d * es / 16;
  const int64_t vecs = n * row_vec;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((vecs + 255) / 256, (int64_t)a.n_cu * 16));
  hipLaunchKernelGGL(k_naive_gather, dim3(grid), dim3(256), 0, s, (const uint4*)a.W, row_vec, ltok, n,
                     (uint4*)tmp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.dtype) {
    case ZGR_F32: return launch_naive_dot_d<ZGR_F32>(a, tmp, lbeam, start, n, s);
    case ZGR_BF16: return launch_naive_dot_d<ZGR_BF16>(a, tmp, lbeam, start, n, s);
    case ZGR_F16: return launch_naive_dot_d<ZGR_F16>(a, tmp, lbeam, start, n, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_row_lse(const StepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_row_lse, dim3((a.M + 3) / 4), dim3(256), 0, s, a.z, a.ldz, a.tab.V, a.M, a.row_in,
                     a.lse_ext);
  return hipGetLastError();
}

hipError_t launch_lookup_items(const DevTable* tabs, int32_t L, const int32_t* prefix, const float* cum,
                               int32_t n, int32_t* item, hipStream_t s) {
  TableSet ts{};
  for (int l = 0; l < L; ++l) ts.t[l] = tabs[l];
  hipLaunchKernelGGL(k_lookup_items, dim3((n + 255) / 256), dim3(256), 0, s, ts, L, prefix, cum, n, item);
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
