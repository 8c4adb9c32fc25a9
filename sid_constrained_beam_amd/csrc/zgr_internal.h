// Internal structures shared by the host index builder, the engine and the
// kernel launchers.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/zgr.h"

namespace zgr {

constexpr int kMaxL = 8;
// Internal table format: one row in which every codebook token is legal (the
// unconstrained mode); laid out like a dense row.
constexpr int32_t kFmtAll = 4;
// Codebook slices of the slice directory: one per XCD of the MI355X.
constexpr int kSlices = 8;

// One step's table on the host.
struct HostTable {
  int32_t fmt = ZGR_FMT_SPARSE;
  int64_t rows = 0;
  int64_t nnz = 0;
  int32_t stride = 0;     // slots per beam
  int32_t max_legal = 0;  // largest row length
  std::vector<int32_t> row_ptr;  // [rows + 1]
  std::vector<uint16_t> tok;     // [nnz]
  std::vector<uint32_t> bits;    // dense: [rows][words]
  std::vector<uint16_t> rank;    // dense: [rows][words] set bits of the row before each word
  std::vector<int32_t> next;     // next-row matrix encoding: [rows][V], -1 = not legal
  std::vector<uint16_t> sdir;    // sparse, optional: [rows][kSlices] slice directory
};

// One step's table in HBM (plain pointers, passed to kernels by value).
struct DevTable {
  int32_t fmt;
  int32_t stride;
  int32_t words;  // ceil(V / 32)
  int32_t V;
  int64_t rows;
  const int32_t* row_ptr;
  const uint16_t* tok;   // sparse only
  const uint32_t* bits;  // dense only
  const uint16_t* rank;  // dense only: [rows][words] set bits of the row before each word
  const int32_t* next;   // next-row matrix encoding only: [rows][V], -1 = not legal
  const uint16_t* sdir;  // sparse, optional: [rows][kSlices] legal tokens below each slice's end
};

}  // namespace zgr

struct zgr_index {
  int32_t L = 0, V = 0, bits = 0;
  int64_t N = 0;
  zgr::HostTable host[zgr::kMaxL];
  zgr::DevTable dev[zgr::kMaxL];
  bool on_device = false;
  int device = -1;
  std::vector<void*> allocations;
  uint64_t generation = 0;
  zgr_build_times times{};  // phases of the last build and upload
};

namespace zgr {

// Registry of live indexes: a plan checks that the index it was made for
// (pointer and generation) has not been freed.
void index_register(const zgr_index* idx, uint64_t generation);
void index_unregister(const zgr_index* idx);
bool index_alive(const zgr_index* idx, uint64_t generation);

// thread-local error detail
int32_t fail(int32_t status, const std::string& msg);
int32_t hip_fail(hipError_t e, const char* what);

// ---- kernel launchers (zgr_kernels.hip) --------------------------------------------------
struct StepArgs {
  DevTable tab;
  int32_t t, L;
  int32_t B, K, k_in, M;  // M = B * k_in beams in
  int32_t d, dtype;
  const void* hidden;     // [M][d]
  const void* W;          // [V][d]
  const int32_t* row_in;
  const float* cum_in;
  int32_t* parent_out;
  int32_t* token_out;
  int32_t* row_out;
  float* cum_out;
  float* slot_dbg;
  const int32_t* prefix_in;  // decode only: [M][L]
  int32_t* prefix_out;       // decode only: [B*K][L]
  // scratch
  float* z;             // score buffer
  int64_t ldz;          // its row stride
  int32_t* unit_start;  // [M + 1] candidate prefix over the beams (naive baseline)
  int32_t* ctot;        // sparse projection: [slices][chunks] units of each 1,024-beam chunk
  int4* umeta;          // sparse projection: [slices][chunks][chunk_cap] unit places
                        // (beam, first entry, first slot, size)
  int64_t chunk_cap;    // unit places one chunk of one slice can hold
  float* lse;           // [M] per-beam log-sum-exp over legal tokens
  float* lse_ext;       // [M] or null: normaliser given to the request kernel (score-first)
  float2* zms;          // [M][words] or null: the full projection's legal (max, sum of exp)
                        // per 32-token word of a dense row, read by the pruned request kernel
  bool plain_z;         // full projection writes token-indexed rows even on dense steps
  bool z_token;         // the request kernel reads token-indexed score rows (zmode 0)
  int32_t parts;        // blocks per request in the request kernel (1 = no merge)
  bool big_parts;       // slot-indexed parts with the merge-sized key array (one block per CU)
  uint64_t* part_keys;  // [B * parts][K] best keys of each part
  int32_t* part_cnt;    // [B * parts]
  float2* part_ms;      // [B * parts] single-beam parts: (max, sum of exp) of their range
  int32_t* err;         // device error flag
  int32_t n_cu;
};

hipError_t launch_units(const StepArgs& a, hipStream_t s);
hipError_t launch_selective_score(const StepArgs& a, hipStream_t s);
// Dense steps: the LDS-staged comparison kernel where its shape applies, else
// the selective projection.
hipError_t launch_staged_score(const StepArgs& a, hipStream_t s);
hipError_t launch_full_projection(const StepArgs& a, hipStream_t s);
// Which full-projection kernel, tile and epilogue a step shape gets (host
// logic only; the launcher and zgr_full_projection_variant share it).
struct GemmVariant {
  int32_t kernel;    // ZGR_GEMM_*
  int32_t tile_m, tile_n;
  int32_t epilogue;  // ZGR_EPI_*
};
GemmVariant gemm_variant(int32_t M, int32_t V, bool dense, bool plain, int32_t n_cu);
// true when the full projection of this step writes sparse rows by slot
// (legal columns only, ldz = stride) rather than token-indexed rows (ldz = V)
bool full_projection_slot_layout(const StepArgs& a);
// zmode: 0 = z token-indexed, 1 = z slot-indexed, 2 = score inside the request kernel,
// 5 = dense rank-indexed rows pruned by the full projection's word partials (a.zms).
// With a.parts > 1 each request's candidates are split over a.parts blocks, then merged.
constexpr int kMaxParts = 64;
constexpr int kKeyCapHost = 5120;     // candidates of a request part whose keys fit the request kernel's LDS
constexpr int kMergeCapHost = 14336;  // part keys (parts x K) the merge holds in LDS
// word partials one thread of a pruned request joins: its beam's words split
// over min(64, 1024 / k_in rounded up to a power of two) threads
constexpr int kPruneWordsHost = 8;
hipError_t launch_request_step(const StepArgs& a, int zmode, hipStream_t s);
// after launch_request_step with a.parts > 1: the per-request merge of the parts
hipError_t launch_request_merge(const StepArgs& a, hipStream_t s);
// naive compaction baseline: legal counts scanned over all beams into start[0..M]
hipError_t launch_naive_count(const StepArgs& a, int32_t* start, hipStream_t s);
// then (n = start[M], read on the host) the compact list, the temporary matrix
// [n][d] and the row dots scattered into z by legal rank
hipError_t launch_naive_score(const StepArgs& a, const int32_t* start, int64_t n, int32_t* lbeam,
                              int32_t* ltok, void* tmp, hipStream_t s);
// score-first: log-sum-exp over all V token-indexed scores of each live beam into a.lse_ext
hipError_t launch_row_lse(const StepArgs& a, hipStream_t s);
// item id of each final SID by a walk of the L tables (-1 if not in the catalog)
hipError_t launch_lookup_items(const DevTable* tabs, int32_t L, const int32_t* prefix, const float* cum,
                               int32_t n, int32_t* item, hipStream_t s);
hipError_t launch_decode_init(int32_t* row, float* cum, int32_t B, int32_t K, hipStream_t s);
hipError_t launch_decode_final(const int32_t* row, const float* cum, const int32_t* prefix,
                               int32_t B, int32_t K, int32_t L, int32_t top_k, int64_t* item_out,
                               int32_t* sid_out, float* score_out, hipStream_t s);

// Tile of tokens handled by one work unit on dense steps, and of candidates on sparse steps.
constexpr int kDenseTile = 1024;
constexpr int kSparseTile = 64;
// Beam chunks (1,024 beams each) a sparse projection can take: M <= 1024 times this.
constexpr int kMaxUnitChunksHost = 2048;
// Units a beam can have in one slice of a sparse table: its run there holds
// at most S_t tokens, and with a slice directory at most ceil(V / kSlices).
inline int64_t slice_units_per_beam(int32_t stride, int32_t V, bool sliced) {
  const int64_t run = sliced ? std::min<int64_t>(stride, (V + kSlices - 1) / kSlices) : stride;
  return std::max<int64_t>(1, (run + kSparseTile - 1) / kSparseTile);
}

}  // namespace zgr
