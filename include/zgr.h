/*
 * zgr — filter-first constrained beam search over semantic IDs on MI355X.
 *
 * C ABI of the library.  The operations follow the ZeroGR description
 * ("ZeroGR: Filtering-First Constrained Decoding for Generative
 * Recommendation", paper-daily page):
 *   - "overall pipeline": an offline filter index, an online per-step engine
 *     and a rebuild on every catalog/model update; each step takes every
 *     beam's hidden vector, reads its legal tokens from the index, scores
 *     them, applies log-softmax over the legal tokens only, adds the result
 *     to the beam's cumulative log-prob and picks the next beams.
 *   - "why slice the index per step": one table per step; a row is a prefix
 *     of length t-1 and records its legal next tokens and their rows in the
 *     next table; dense tables for steps with many legal tokens (columns in
 *     full-projection order), sparse tables for late steps where an entry's
 *     position is its next row and the last step stores no item ids.
 *   - "why fewer scores is not faster": fixed padded candidate slots per beam
 *     (the per-step maximum legal count; a dense step uses the whole
 *     codebook), empty slots at minus infinity, weight rows read in place;
 *     per step, full or selective projection is chosen by timing both on
 *     warm-up traffic before serving and then frozen.
 *
 * Conventions
 *   - Every call returns a status (ZGR_OK = 0); no error crosses the ABI any
 *     other way.  zgr_last_error() gives a detail string for the calling
 *     thread's last failure.
 *   - Argument checks run before any HIP call, so bad arguments are reported
 *     without touching the device.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are HBM
 *     allocations of the current HIP device (for example torch CUDA tensors).
 *     The caller owns every pointer it passes and keeps it alive for the
 *     call (for asynchronous calls, until the stream has passed the work).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Step work is enqueued asynchronously on it.
 *   - The library owns zgr_index and zgr_plan objects and their HBM; only
 *     zgr_index_free / zgr_plan_free release them.  An index is immutable
 *     after upload and may be read by several plans; a plan owns scratch
 *     buffers and must be used from one stream at a time.
 *   - Tokens are int32 in [0, V); rows are int32 (-1 = dead beam); scores are
 *     float32 (-inf = no candidate).
 */
#ifndef ZGR_H
#define ZGR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------------------- */
#define ZGR_OK 0
#define ZGR_E_ARG 1          /* null pointer, out-of-range scalar argument */
#define ZGR_E_DUP_SID 2      /* two catalog rows share one SID */
#define ZGR_E_TOKEN_RANGE 3  /* a catalog token outside [0, V) */
#define ZGR_E_SHAPE 4        /* unsupported size combination (d, K, L*bits, ...) */
#define ZGR_E_NOMEM 5        /* host or device allocation failed */
#define ZGR_E_HIP 6          /* a HIP runtime call failed */
#define ZGR_E_STATE 7        /* object used out of order, or a stale plan */
#define ZGR_E_CALLBACK 8     /* the hidden-vector callback returned non-zero */
#define ZGR_E_DEVICE 9       /* a kernel saw an invalid beam row (reported at sync) */

/* ---- enums ----------------------------------------------------------------------------- */
#define ZGR_F32 0   /* float32 weights and hidden vectors */
#define ZGR_BF16 1  /* bfloat16 storage, float32 accumulation and log-softmax */
#define ZGR_F16 2   /* IEEE half storage, float32 accumulation and log-softmax */

#define ZGR_FMT_AUTO 0    /* smaller of the two encodings */
#define ZGR_FMT_DENSE 1   /* bitmap per row over the codebook, slot = token */
#define ZGR_FMT_SPARSE 2  /* sorted legal tokens per row, slot = position */
#define ZGR_FMT_DENSE_NEXT 3 /* dense rows stored as an int32 next-row matrix [rows][V]
                                (-1 = not legal) instead of the bitmap: the same results and
                                slots as DENSE at 32 times its bytes; never picked by AUTO,
                                kept to measure the two encodings against each other */

#define ZGR_PROJ_AUTO 0       /* decided by warm-up timing (or a cost model without warm-up) */
#define ZGR_PROJ_FULL 1       /* MFMA projection over the whole codebook, then legal columns */
#define ZGR_PROJ_SELECTIVE 2  /* score only the legal tokens, weight rows read in place */
#define ZGR_PROJ_NAIVE 3      /* baseline, never picked by the planner: the legal tokens scored
                                 through a compact candidate list (sized on the host from a
                                 device count, so the step synchronises its stream) and a
                                 temporary [candidates x d] matrix of copied weight rows */
#define ZGR_PROJ_STAGED 4     /* comparison, never picked by the planner: on dense steps the
                                 weight rows of a codebook tile are staged in LDS once and
                                 scored from there for every beam of a block (beams' hidden
                                 vectors held in registers); f32 with d >= 256 and bf16 with
                                 d >= 512 only, other dense steps and every sparse step run
                                 the selective projection */

typedef struct zgr_index zgr_index;
typedef struct zgr_plan zgr_plan;

/* Static description of one step's table. */
typedef struct {
  int64_t rows;    /* R_t: distinct prefixes of length t-1 */
  int64_t nnz;     /* legal (row, token) pairs = rows of table t+1 (N at t = L) */
  int32_t fmt;     /* ZGR_FMT_DENSE, ZGR_FMT_SPARSE or ZGR_FMT_DENSE_NEXT */
  int32_t stride;  /* S_t: slots per beam (max legal count of a row; V when dense) */
  int64_t bytes;   /* device bytes of this table */
  int32_t max_legal;  /* largest legal count of any row */
  int32_t slice_dir;  /* 1 if the (sparse) table holds a slice directory, else 0 */
} zgr_step_stats;

/* Text of a status code (static storage). */
const char* zgr_status_str(int32_t status);

/* Copy the calling thread's last error detail into buf (NUL-terminated,
 * truncated to n bytes).  Returns the status of that failure. */
int32_t zgr_last_error(char* buf, size_t n);

/* ---- index ---------------------------------------------------------------------------- */

/*
 * Build the per-step filter index of a catalog on the host (no HIP call).
 *   sids  host int32 [N][L], row i = SID of catalog row i, tokens in [0, V).
 *   fmt   host int32 [L] per-step ZGR_FMT_* or NULL (all AUTO).
 *   rank_of_input  host int64 [N] or NULL: receives the item id of each
 *         catalog row.  An item id is the lexicographic rank of the SID among
 *         all catalog SIDs, i.e. its position in the last table (the last
 *         step stores no ids: the position is the id).
 * Rows of table t are the distinct length-(t-1) prefixes in lexicographic
 * order; a legal (row, token) entry's next row is its lexicographic rank among
 * distinct length-t prefixes.  1 <= L <= 8, 2 <= V <= 65536, N < 2^31,
 * ceil(log2 V) * L <= 64.
 * Errors: ZGR_E_ARG, ZGR_E_TOKEN_RANGE, ZGR_E_DUP_SID, ZGR_E_SHAPE, ZGR_E_NOMEM.
 */
int32_t zgr_index_build_host(const int32_t* sids, int64_t N, int32_t L, int32_t V,
                             const int32_t* fmt, int64_t* rank_of_input, zgr_index** out);

/* Copy a host-built index to HBM of the current device (synchronous on
 * return).  Errors: ZGR_E_ARG, ZGR_E_STATE (already on device), ZGR_E_NOMEM,
 * ZGR_E_HIP. */
int32_t zgr_index_to_device(zgr_index* idx, void* stream);

/* zgr_index_build_host followed by zgr_index_to_device. */
int32_t zgr_index_upload(const int32_t* sids, int64_t N, int32_t L, int32_t V, const int32_t* fmt,
                         void* stream, zgr_index** out, int64_t* rank_of_input);

/* ---- index rebuild pipeline ---------------------------------------------------------
 * The index is rebuilt whenever the catalog or the model's codebook changes
 * (ZeroGR description, "overall pipeline": the index is built offline and
 * rebuilt on every update), so its build and upload bound the update window.
 * The host build sorts the packed SIDs and lays the tables out in two passes
 * over chunks of the sorted keys (count, prefix-sum of the chunk counts, fill)
 * on host_threads threads; the result does not depend on the thread count.
 * The upload copies through two pinned staging buffers in turn, so host
 * copies into one overlap the DMA of the other. */
#define ZGR_UPLOAD_STAGED 0 /* double-buffered pinned staging (default) */
#define ZGR_UPLOAD_DIRECT 1 /* one hipMemcpyAsync per array from the pageable host tables */

/* Slice directory of a sparse table: per row, uint16 [8], entry x < 7 the
 * number of the row's legal tokens below (x + 1) * ceil(V / 8) (entry 7 is
 * 0).  With it, the selective projection lets the compute units of one XCD
 * (one L2 cache) score only the candidates whose tokens fall in one eighth
 * of the codebook, so each L2 holds one eighth of the weight rows.  Our
 * addition to the per-step layout; AUTO builds it for sparse tables with
 * V >= 1024 whose rows hold 32 or more legal tokens on average (16 bytes per
 * row, at most a quarter of the table's token bytes). */
#define ZGR_SLICES_AUTO 0
#define ZGR_SLICES_ALWAYS 1 /* every sparse table */
#define ZGR_SLICES_NEVER 2

typedef struct {
  int32_t host_threads;  /* 0 = hardware threads (at most 16) for large catalogs; else 1..64 */
  int32_t upload;        /* ZGR_UPLOAD_STAGED or ZGR_UPLOAD_DIRECT */
  int64_t staging_bytes; /* bytes per staging buffer; 0 = 64 MiB (clamped to [4 KiB, upload size]) */
  int32_t slices;        /* ZGR_SLICES_* (build only) */
  int32_t reserved;      /* 0 */
} zgr_build_opts;

/* Wall-clock milliseconds of each phase of the last build / upload. */
typedef struct {
  double keys_ms;    /* pack SIDs into keys, token range check */
  double sort_ms;    /* radix sort of the keys (skipped for a catalog already in SID order) */
  double layout_ms;  /* duplicate check, count, offsets, fill of row_ptr / tok, item ids */
  double encode_ms;  /* per table: largest row, format, bitmap and rank directory */
  double build_ms;   /* whole host build */
  double alloc_ms;   /* hipMalloc of the device tables */
  double upload_ms;  /* host to HBM copies, synchronised */
  int64_t device_bytes; /* bytes uploaded */
  int32_t threads;      /* host threads the build used */
  int32_t upload;       /* ZGR_UPLOAD_* used */
} zgr_build_times;

/* zgr_index_build_host with options (NULL = defaults); times (nullable)
 * receives the build phases.  Errors: as zgr_index_build_host, and ZGR_E_ARG
 * for a negative host_threads or an unknown slices value. */
int32_t zgr_index_build_host_ex(const int32_t* sids, int64_t N, int32_t L, int32_t V,
                                const int32_t* fmt, int64_t* rank_of_input,
                                const zgr_build_opts* opts, zgr_build_times* times,
                                zgr_index** out);

/* zgr_index_to_device with options (NULL = defaults: staged, 64 MiB buffers);
 * times (nullable) receives the build and upload phases.  Pinned staging
 * buffers are allocated for the call and freed before it returns.
 * Errors: as zgr_index_to_device, and ZGR_E_ARG for an unknown upload mode or
 * negative sizes; on failure no device memory stays allocated. */
int32_t zgr_index_to_device_ex(zgr_index* idx, void* stream, const zgr_build_opts* opts,
                               zgr_build_times* times);

/* zgr_index_build_host_ex followed by zgr_index_to_device_ex. */
int32_t zgr_index_upload_ex(const int32_t* sids, int64_t N, int32_t L, int32_t V,
                            const int32_t* fmt, void* stream, const zgr_build_opts* opts,
                            zgr_build_times* times, zgr_index** out, int64_t* rank_of_input);

/* Phases of the index's build and upload.  Errors: ZGR_E_ARG. */
int32_t zgr_index_times(const zgr_index* idx, zgr_build_times* out);

/* Device copies of table t (valid while idx lives; NULL where the table's
 * format has no such array): row_ptr int32 [rows+1], tok uint16 [nnz]
 * (sparse), bits uint32 [rows][ceil(V/32)] and rank uint16 [rows][ceil(V/32)]
 * (dense; set bits of the row before each word), next int32 [rows][V]
 * (DENSE_NEXT).  Errors: ZGR_E_ARG, ZGR_E_STATE (not uploaded). */
int32_t zgr_index_device_table(const zgr_index* idx, int32_t t, const void** row_ptr,
                               const void** tok, const void** bits, const void** rank,
                               const void** next);

/* Per-step statistics, t in 1..L.  Errors: ZGR_E_ARG. */
int32_t zgr_index_stats(const zgr_index* idx, int32_t t, zgr_step_stats* out);

/* Host copies of table t (valid while idx lives): row_ptr int32 [rows+1]
 * (CSR offsets; also the dense table's base), tok uint16 [nnz] sorted per
 * row, bits uint32 [rows][ceil(V/32)] (NULL for sparse tables).  Any output
 * pointer may be NULL.  Errors: ZGR_E_ARG. */
int32_t zgr_index_host_table(const zgr_index* idx, int32_t t, const int32_t** row_ptr,
                             const uint16_t** tok, const uint32_t** bits);

/* Host copy of table t's slice directory (uint16 [rows][8], see
 * ZGR_SLICES_AUTO), or NULL in *sdir when the table has none.
 * Errors: ZGR_E_ARG. */
int32_t zgr_index_host_slices(const zgr_index* idx, int32_t t, const uint16_t** sdir);

/* Index shape: L, V, N (any output may be NULL). */
int32_t zgr_index_shape(const zgr_index* idx, int32_t* L, int32_t* V, int64_t* N);

void zgr_index_free(zgr_index* idx);

/* ---- plan ----------------------------------------------------------------------------- */

/*
 * Hidden-vector source (the model; its time is not part of a step).  Called
 * once per decode step with the B*k_in beams in flight: prefix_dev is device
 * int32 [B*k_in][prefix_ld] holding each beam's t-1 tokens so far (beam
 * b = request * k_in + rank), hidden_dev is device [B*k_in][d] of the plan's
 * dtype to be filled.  Work must be enqueued on `stream` (or completed before
 * returning).  Non-zero return aborts the decode with ZGR_E_CALLBACK.
 */
typedef int32_t (*zgr_hidden_fn)(void* user, int32_t t, int32_t B, int32_t k_in,
                                 const int32_t* prefix_dev, int32_t prefix_ld, void* hidden_dev,
                                 void* stream);

/*
 * Create a plan for batches of B requests, beam width K, hidden size d and
 * the given weights, and freeze each step's projection ("why fewer scores is
 * not faster": timed on warm-up traffic before serving, kept until the next
 * update).
 *   W_dev   L device pointers, W_t row-major [V][d] of dtype (kept, not copied;
 *           must outlive the plan).
 *   force   host int32 [L] of ZGR_PROJ_* or NULL (all AUTO).
 *   n_warmup  warm-up decodes; in each, every AUTO step runs both projections
 *           twice, interleaved, and the second run of each is timed with HIP
 *           events (so the device is not waiting on host launches and both
 *           see warm caches); the one with the lower median over the decodes
 *           wins (an exact tie picks selective).  With n_warmup = 0 or no callback,
 *           AUTO steps use a bandwidth/MFMA cost model instead.
 *   hidden_fn, user  source of warm-up hidden vectors (may be NULL if no timing).
 * Limits: d % 64 == 0, d <= 4096; 1 <= K <= 1024; B >= 1; B*K < 2^31.
 * Errors: ZGR_E_ARG, ZGR_E_SHAPE, ZGR_E_STATE (index not on device), ZGR_E_NOMEM,
 * ZGR_E_HIP, ZGR_E_CALLBACK.
 */
int32_t zgr_plan_warmup(const zgr_index* idx, const void* const* W_dev, int32_t dtype, int32_t d,
                        int32_t B, int32_t K, zgr_hidden_fn hidden_fn, void* user,
                        int32_t n_warmup, const int32_t* force, void* stream, zgr_plan** out);

/* The frozen choice of step t and the warm-up medians in microseconds
 * (negative when that option was not timed).  Errors: ZGR_E_ARG. */
int32_t zgr_plan_choice(const zgr_plan* plan, int32_t t, int32_t* proj, float* us_full,
                        float* us_sel);

/* Re-freeze step t's projection (ZGR_PROJ_FULL, ZGR_PROJ_SELECTIVE or one of
 * the comparisons ZGR_PROJ_NAIVE and ZGR_PROJ_STAGED), e.g. to resume a plan
 * exported by zgr_plan_choice without a new warm-up. */
int32_t zgr_plan_set_choice(zgr_plan* plan, int32_t t, int32_t proj);

/*
 * Decoding mode of a plan (default ZGR_MODE_FILTER_FIRST), applied by every
 * later zgr_step / zgr_decode.  The other two are the comparisons of the
 * ZeroGR description:
 *   ZGR_MODE_SCORE_FIRST  ("does filter-first change results"): every codebook
 *       token is scored (full projection at every step, whatever the frozen
 *       choice), the log-softmax denominator covers all V tokens, and only
 *       then are the candidates restricted to the legal tokens.  Inputs and
 *       outputs as in filter-first; cum_out and slot_dbg carry
 *       log-probabilities normalised over the whole codebook.
 *   ZGR_MODE_UNCONSTRAINED ("is it really better"): full projection,
 *       log-softmax over all V tokens, and every token is a candidate of every
 *       live beam; the index is not read during the steps, so a code need not
 *       be a catalog item.  row_in >= 0 marks a live beam (its value is not
 *       used), row_out is 0 for every chosen candidate (-1 = none), and
 *       slot_dbg has V slots per beam (slot = token).  zgr_decode returns the
 *       item id of each final code that is a catalog SID and -1 for the
 *       others (sid_out still holds the code).
 * Errors: ZGR_E_ARG.
 */
#define ZGR_MODE_FILTER_FIRST 0
#define ZGR_MODE_SCORE_FIRST 1
#define ZGR_MODE_UNCONSTRAINED 2
int32_t zgr_plan_set_mode(zgr_plan* plan, int32_t mode);
int32_t zgr_plan_mode(const zgr_plan* plan, int32_t* mode);

void zgr_plan_free(zgr_plan* plan);

/*
 * One decode step t (1..L) for the plan's B requests, asynchronous on stream.
 *   hidden_dev  device [B*k_in][d] (plan dtype): beam b = request*k_in + rank.
 *   row_in      device int32 [B*k_in]: the beam's row in table t (-1 = dead).
 *   cum_in      device float [B*k_in]: cumulative log-prob (ignored when dead).
 *   k_in        beams per request coming in (1 at t = 1, usually K after).
 * Outputs, device, [B*K], per request sorted best first:
 *   parent_out  int32: input beam index b of the chosen candidate (-1 = none)
 *   token_out   int32: the chosen token (-1 = none)
 *   row_out     int32: its row in table t+1; at t = L the item id (-1 = none)
 *   cum_out     float: cum_in[parent] + log-softmax of the token over the
 *               parent's legal tokens (-inf = none)
 *   slot_dbg    NULL or device float [B*k_in][S_t]: every slot's log-prob,
 *               -inf for empty slots and dead beams (S_t from zgr_index_stats).
 * Ranking: cum_out descending, then parent ascending, then token ascending.
 * Fewer than K candidates in a request: the tail is filled with "none".
 * An out-of-range row sets a device flag reported by zgr_plan_status.
 * Errors (before any work is enqueued): ZGR_E_ARG, ZGR_E_SHAPE, ZGR_E_HIP.
 */
int32_t zgr_step(zgr_plan* plan, int32_t t, const void* hidden_dev, const int32_t* row_in,
                 const float* cum_in, int32_t k_in, int32_t* parent_out, int32_t* token_out,
                 int32_t* row_out, float* cum_out, float* slot_dbg, void* stream);

/*
 * Full decode of the plan's B requests: L steps, each preceded by one
 * hidden_fn call, starting from one empty-prefix beam per request with
 * cumulative log-prob 0.  Outputs (device), per request best first:
 *   item_out  int64 [B][top_k] item ids (-1 = none)
 *   sid_out   int32 [B][top_k][L] or NULL
 *   score_out float [B][top_k] or NULL
 * 1 <= top_k <= K.  Synchronises the stream before returning and reports
 * device-side flags.  Errors: ZGR_E_ARG, ZGR_E_CALLBACK, ZGR_E_HIP, ZGR_E_DEVICE.
 */
int32_t zgr_decode(zgr_plan* plan, zgr_hidden_fn hidden_fn, void* user, int32_t top_k,
                   int64_t* item_out, int32_t* sid_out, float* score_out, void* stream);

/*
 * zgr_step without allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It runs the kernels of zgr_step for one step t of a
 * batch of B requests (beam width K, hidden size d, weights W_t of dtype) with
 * the given projection (ZGR_PROJ_FULL or ZGR_PROJ_SELECTIVE; there is no plan,
 * so no warm-up choice), filter-first, and keeps the step's scratch (score
 * buffer, unit scan, request parts' keys and partials, device flag) in one
 * file-scope device array of at most 64 MiB that each GPU holds for the life
 * of the process; it calls no allocator.
 *   idx        an index on the current device; W_t device [V][d] of dtype
 *   hidden_dev, row_in, cum_in, k_in, parent_out .. cum_out, slot_dbg: as in
 *              zgr_step (device buffers, caller-owned)
 *   err_out    device int32 or NULL: receives 1 when a beam row was outside
 *              the step's table (such beams count as dead), else 0
 * Every call on a GPU shares that GPU's scratch array, which keeps the last
 * call's contents: calls that overlap on one GPU (two streams, two host
 * threads) race and must be serialised by the caller.
 * Errors (before any work is enqueued): ZGR_E_ARG, ZGR_E_STATE (index not on
 * this device), ZGR_E_SHAPE (unsupported size, or a step whose scratch
 * exceeds the array: about B*k_in*max(S_t, V)*4 bytes for the scores plus
 * B*64*K*8 for the part keys), ZGR_E_HIP.
 */
int32_t zgr_step_noalloc(const zgr_index* idx, const void* W_t, int32_t dtype, int32_t d, int32_t B,
                         int32_t K, int32_t t, int32_t proj, const void* hidden_dev,
                         const int32_t* row_in, const float* cum_in, int32_t k_in,
                         int32_t* parent_out, int32_t* token_out, int32_t* row_out, float* cum_out,
                         float* slot_dbg, int32_t* err_out, void* stream);

/* Synchronise stream and report (then clear) the plan's device-side error
 * flag: ZGR_OK or ZGR_E_DEVICE; ZGR_E_HIP if the sync fails. */
int32_t zgr_plan_status(zgr_plan* plan, void* stream);

/* ---- full-projection kernel choice ------------------------------------------------------
 * Which MFMA kernel the full projection of a step runs ("why fewer scores is
 * not faster": dense steps compute every score and keep the legal columns).
 * Host logic only (no HIP call), shared with the launcher, so tests and
 * reports can list the kernels a workload runs.
 *   M      beams in the step (B * k_in), V the codebook size
 *   dtype  ZGR_F32 / ZGR_BF16 / ZGR_F16 (the tile choice does not depend on
 *          it; it is checked and kept for future per-type rules)
 *   fmt    the step table's ZGR_FMT_DENSE, ZGR_FMT_SPARSE or ZGR_FMT_DENSE_NEXT
 *   mode   ZGR_MODE_* of the plan; n_cu the device's compute units
 * Outputs (any may be NULL): kernel ZGR_GEMM_SMALL (16x16 MFMA over 32x32
 * tiles, for few beams) or ZGR_GEMM_TILED (32x32 MFMA, tile_m x tile_n block
 * tiles); epilogue ZGR_EPI_PLAIN (every column, token-indexed rows),
 * ZGR_EPI_DENSE (legal columns at their legal rank) or ZGR_EPI_SLOT (sparse
 * rows: legal columns at their slot).
 * Errors: ZGR_E_ARG (non-positive sizes, unknown dtype, fmt or mode). */
#define ZGR_GEMM_SMALL 0
#define ZGR_GEMM_TILED 1
#define ZGR_EPI_PLAIN 0
#define ZGR_EPI_DENSE 1
#define ZGR_EPI_SLOT 2
int32_t zgr_full_projection_variant(int32_t M, int32_t V, int32_t dtype, int32_t fmt, int32_t mode,
                                    int32_t n_cu, int32_t* kernel, int32_t* tile_m, int32_t* tile_n,
                                    int32_t* epilogue);

/* How the request kernel (normalise, select, advance) ran at step t in the
 * plan's last zgr_step or zgr_decode.  *kind: ZGR_REQ_TOKEN (scores in
 * token-indexed rows), ZGR_REQ_SLOT (scores at their slot or legal rank),
 * ZGR_REQ_SCORED (light sparse step: the request kernel gathers and scores
 * its candidates itself) or ZGR_REQ_PRUNED (dense step after the full
 * projection, whose epilogue left every beam's legal (max, sum of exp) per
 * 32-token word: the request normalises from those partials and reads only
 * the scores of the K words whose best candidates rank highest, which hold
 * its whole top K -- ZeroGR page, "why fewer scores is not faster": filter,
 * score and select share one pass over the slots).  *parts: blocks per
 * request (above 1 a merging dispatch follows).  Host state only; either
 * output may be NULL.  Errors: ZGR_E_ARG (null plan, t outside [1, L]),
 * ZGR_E_STATE (step t has not run on this plan). */
#define ZGR_REQ_TOKEN 0
#define ZGR_REQ_SLOT 1
#define ZGR_REQ_SCORED 2
#define ZGR_REQ_PRUNED 5
int32_t zgr_plan_request_path(const zgr_plan* plan, int32_t t, int32_t* kind, int32_t* parts);

/* ---- per-kernel timing ------------------------------------------------------------------ */

/* Kernel classes of a step, for zgr_plan_profile_read. */
#define ZGR_KERNEL_UNITS 0      /* per-beam legal counts and work-unit scan (selective) */
#define ZGR_KERNEL_SELECTIVE 1  /* selective projection: weight rows gathered in place */
#define ZGR_KERNEL_GEMM 2       /* full projection on MFMA */
#define ZGR_KERNEL_REQUEST 3    /* per request: legal-only log-softmax, cumulative add, top-K,
                                   next rows, prefixes (and, on light sparse steps, the
                                   selective projection itself); a request split over several
                                   blocks adds a second, merging dispatch */
#define ZGR_KERNEL_NORM 4       /* log-sum-exp over the whole codebook (score-first mode) */
#define ZGR_KERNEL_COUNT 5

/* Per-kernel timing: repeat > 0 turns it on, 0 off; counters are reset.
 * While on, every kernel launch of zgr_step / zgr_decode is issued `repeat`
 * times back to back between two HIP events on the launch stream and the
 * bracket's duration divided by `repeat` is recorded (the step kernels are
 * idempotent, so results are unchanged; repeat > 1 amortises the events'
 * own cost for short kernels).  Do not capture such launches into graphs.
 * Errors: ZGR_E_ARG (repeat outside [0, 1000]), ZGR_E_HIP. */
int32_t zgr_plan_profile(zgr_plan* plan, int32_t repeat);

/* Synchronise on the recorded events and return, for kernel class `kernel`
 * at step t, the number of timed launches and their summed duration (ms).
 * Errors: ZGR_E_ARG, ZGR_E_HIP. */
int32_t zgr_plan_profile_read(zgr_plan* plan, int32_t kernel, int32_t t, int64_t* launches,
                              double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* ZGR_H */
