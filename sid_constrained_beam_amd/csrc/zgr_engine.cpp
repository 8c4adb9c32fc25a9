// Step engine, decode loop, warm-up planner and error reporting.
//
// ZeroGR description, "why fewer scores is not faster": before a model
// version takes traffic, every step's projection options are timed on
// warm-up requests, the fastest is kept and frozen until the next update;
// there is no per-request decision, so the choice follows the GPU, the
// precision and the batch size.  Here a plan is made for one (index, weights,
// dtype, d, B, K) and owns the HBM scratch of a step; zgr_step enqueues one
// step on a stream without any host round trip.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "zgr_internal.h"

namespace zgr {

bool supported_hidden_size(int d);

namespace {
thread_local std::string g_err;
thread_local int32_t g_err_status = ZGR_OK;
}  // namespace

int32_t fail(int32_t status, const std::string& msg) {
  g_err = msg;
  g_err_status = status;
  return status;
}

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(ZGR_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace zgr

struct zgr_plan {
  const zgr_index* idx = nullptr;
  uint64_t idx_generation = 0;
  int device = -1;
  int32_t L = 0, V = 0, d = 0, B = 0, K = 0, dtype = 0;
  std::vector<const void*> W;
  int32_t choice[zgr::kMaxL] = {0};
  int32_t mode = ZGR_MODE_FILTER_FIRST;
  zgr::DevTable all_tab{};  // one row, every token legal (unconstrained mode)
  // naive compaction baseline: compact list and temporary matrix, grown on demand
  int32_t* naive_beam = nullptr;
  int32_t* naive_tok = nullptr;
  void* naive_tmp = nullptr;
  int64_t naive_cap = 0;
  float us_full[zgr::kMaxL], us_sel[zgr::kMaxL];
  int32_t req_kind[zgr::kMaxL] = {0}, req_parts[zgr::kMaxL] = {0};  // last run of each step
  int n_cu = 256;
  // HBM scratch
  std::vector<void*> allocations;
  float* z = nullptr;
  int64_t z_elems = 0;
  int32_t* unit_start = nullptr;
  int32_t* ctot = nullptr;
  int4* umeta = nullptr;
  int64_t chunk_cap = 0;
  float* lse = nullptr;
  float2* zms = nullptr;  // dense full projections: legal (max, sum of exp) per 32-token word
  uint64_t* part_keys = nullptr;
  int32_t* part_cnt = nullptr;
  float2* part_ms = nullptr;
  int32_t* err = nullptr;
  int32_t* err_host = nullptr;  // pinned copy of the flag, read after one stream sync
  // decode state: double-buffered beams and prefixes, hidden vectors, outputs
  void* hidden = nullptr;
  int32_t *row[2] = {nullptr, nullptr}, *prefix[2] = {nullptr, nullptr};
  float* cum[2] = {nullptr, nullptr};
  int32_t *parent = nullptr, *token = nullptr;
  // optional per-kernel timing: HIP events recorded around each launch on its stream
  struct ProfRec {
    hipEvent_t a, b;
    int kernel, t, repeat;
  };
  int profiling = 0;  // launches per timed bracket (0 = timing off)
  std::vector<ProfRec> pending;
  std::vector<hipEvent_t> pool;
  double prof_ms[ZGR_KERNEL_COUNT][zgr::kMaxL] = {};
  int64_t prof_n[ZGR_KERNEL_COUNT][zgr::kMaxL] = {};
};

namespace {

using namespace zgr;

int64_t elem_size(int32_t dtype) { return dtype == ZGR_F32 ? 4 : 2; }

int32_t beams_in(const zgr_plan* p, int32_t t) { return t == 1 ? 1 : p->K; }

int32_t plan_alloc(zgr_plan* p, void** dst, size_t bytes) {
  hipError_t e = hipMalloc(dst, std::max<size_t>(bytes, 256));
  if (e != hipSuccess) {
    *dst = nullptr;
    (void)hipGetLastError();
    return fail(ZGR_E_NOMEM, "zgr_plan: hipMalloc of " + std::to_string(bytes) + " bytes");
  }
  p->allocations.push_back(*dst);
  return ZGR_OK;
}

// Cost model used for AUTO steps when nothing was timed: the selective path
// moves one weight row per legal candidate (HBM bound), the full path does a
// dense [M x d] x [d x V] product (MFMA bound) and writes M x V scores.
int32_t model_choice(const zgr_plan* p, int32_t t) {
  const HostTable& h = p->idx->host[t - 1];
  const double M = (double)p->B * beams_in(p, t);
  const double mean_n = (double)h.nnz / (double)std::max<int64_t>(1, h.rows);
  const double es = (double)elem_size(p->dtype);
  const double sel_bytes = M * std::min((double)p->V, mean_n) * p->d * es;
  const double sel_s = sel_bytes / 4.0e12;
  const double peak = (p->dtype == ZGR_F32) ? 157.3e12 : 2.5e15;
  const double full_s = 2.0 * M * p->V * p->d / (0.5 * peak) + M * p->V * 8.0 / 4.0e12;
  return full_s < sel_s ? ZGR_PROJ_FULL : ZGR_PROJ_SELECTIVE;
}

int32_t check_args_step(const zgr_plan* p, int32_t t, const void* hidden, const int32_t* row_in,
                        const float* cum_in, int32_t k_in, const int32_t* parent_out,
                        const int32_t* token_out, const int32_t* row_out, const float* cum_out) {
  if (!p) return fail(ZGR_E_ARG, "zgr_step: null plan");
  if (t < 1 || t > p->L) return fail(ZGR_E_ARG, "zgr_step: t out of range");
  if (!hidden || !row_in || !cum_in || !parent_out || !token_out || !row_out || !cum_out)
    return fail(ZGR_E_ARG, "zgr_step: null buffer");
  if (k_in < 1 || k_in > p->K) return fail(ZGR_E_ARG, "zgr_step: k_in must be in [1, K]");
  if (!index_alive(p->idx, p->idx_generation))
    return fail(ZGR_E_STATE, "zgr_step: plan is stale (its index was freed)");
  return ZGR_OK;
}

StepArgs make_args(zgr_plan* p, int32_t t, const void* hidden, const int32_t* row_in,
                   const float* cum_in, int32_t k_in, int32_t* parent_out, int32_t* token_out,
                   int32_t* row_out, float* cum_out, float* slot_dbg, const int32_t* prefix_in,
                   int32_t* prefix_out) {
  StepArgs a{};
  a.tab = p->idx->dev[t - 1];
  a.t = t;
  a.L = p->L;
  a.B = p->B;
  a.K = p->K;
  a.k_in = k_in;
  a.M = p->B * k_in;
  a.d = p->d;
  a.dtype = p->dtype;
  a.hidden = hidden;
  a.W = p->W[t - 1];
  a.row_in = row_in;
  a.cum_in = cum_in;
  a.parent_out = parent_out;
  a.token_out = token_out;
  a.row_out = row_out;
  a.cum_out = cum_out;
  a.slot_dbg = slot_dbg;
  a.prefix_in = prefix_in;
  a.prefix_out = prefix_out;
  a.z = p->z;
  a.unit_start = p->unit_start;
  a.ctot = p->ctot;
  a.umeta = p->umeta;
  a.chunk_cap = p->chunk_cap;
  a.lse = p->lse;
  a.parts = 1;
  a.part_keys = p->part_keys;
  a.part_cnt = p->part_cnt;
  a.part_ms = p->part_ms;
  a.err = p->err;
  a.n_cu = p->n_cu;
  return a;
}

hipEvent_t prof_event(zgr_plan* p) {
  if (!p->pool.empty()) {
    hipEvent_t e = p->pool.back();
    p->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch through fn; when timing is on, the launch is issued `profiling`
// times back to back between two events (every kernel of a step is
// idempotent: it only reads its inputs and overwrites its outputs).
template <class F>
hipError_t prof_launch(zgr_plan* p, int kernel, int t, hipStream_t s, F&& fn) {
  if (p->profiling <= 0) return fn();
  hipEvent_t a = prof_event(p), b = prof_event(p);
  if (!a || !b) return fn();
  (void)hipEventRecord(a, s);
  hipError_t e = hipSuccess;
  for (int i = 0; i < p->profiling && e == hipSuccess; ++i) e = fn();
  (void)hipEventRecord(b, s);
  p->pending.push_back({a, b, kernel, t, p->profiling});
  return e;
}

int32_t prof_flush(zgr_plan* p) {
  for (auto& r : p->pending) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize (profiling)");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      p->prof_ms[r.kernel][r.t - 1] += ms / r.repeat;
      p->prof_n[r.kernel][r.t - 1] += 1;
    }
    p->pool.push_back(r.a);
    p->pool.push_back(r.b);
  }
  p->pending.clear();
  return ZGR_OK;
}

// A selective sparse step is "light" when one block per request can gather
// its candidates' weight rows itself: then the step is a single launch.
bool light_sparse_step(const zgr_plan* p, const StepArgs& a) {
  const HostTable& h = p->idx->host[a.t - 1];
  if (h.fmt != ZGR_FMT_SPARSE) return false;
  const double mean_n = (double)h.nnz / (double)std::max<int64_t>(1, h.rows);
  const double bytes = (double)a.k_in * std::min<double>(mean_n, h.stride) * p->d * elem_size(p->dtype);
  return bytes <= (double)(1 << 20);
}

// Blocks per request for the request kernel.  A request with many candidates
// is split over several blocks, each taking an equal share of its flat
// candidate list (a beam may span blocks), then merged; a request of at most
// kSmallRequest candidates (estimated from the table's mean row) stays whole,
// since below that a split does not pay for the merge launch.  A part aims at
// kPartCandidates candidates, with no more parts than one round of blocks at
// two per compute unit takes, but always enough parts that a part's keys fit
// the LDS key array (a part whose keys do not fit recomputes them from the
// scores in each pass, which costs more than more parts: measured on the
// dense-early catalog's second step); the parts' best K keys must fit the
// merge's LDS.  When those parts would take more than four rounds of blocks
// at two per compute unit, slot-indexed steps use big parts instead (the
// merge-sized key array, one block per compute unit): each part's fixed cost
// (the request's rows, the log-sum-exp reads of its beams) then repeats far
// less often.
constexpr double kSmallRequest = 6144.0;
constexpr double kPartCandidates = 2048.0;
constexpr double kPartMaxCandidates = 0.9 * kKeyCapHost;
constexpr double kPruneGain = 2.0;  // pruning needs this many candidates per kept-word bound
constexpr double kBigPartMaxCandidates = 0.9 * kMergeCapHost;
int32_t request_parts(const zgr_plan* p, const StepArgs& a, bool* big) {
  *big = false;
  const HostTable& h = p->idx->host[a.t - 1];
  double mean_n = (double)h.nnz / (double)std::max<int64_t>(1, h.rows);
  if (a.tab.fmt == kFmtAll) mean_n = p->V;
  const double est_c = a.k_in * std::min<double>(mean_n, a.tab.stride);
  if (est_c <= kSmallRequest) return 1;
  const int merge_cap = kMergeCapHost / std::max(1, a.K);
  const int p_occ = std::max(1, 2 * p->n_cu / std::max(1, a.B));
  int P = std::min((int)std::ceil(est_c / kPartCandidates), p_occ);
  P = std::max(P, (int)std::ceil(est_c / kPartMaxCandidates));
  if (!a.z_token && (double)a.B * P > 4.0 * 2 * p->n_cu) {
    const int Pb = (int)std::ceil(est_c / kBigPartMaxCandidates);
    if (Pb <= std::min(kMaxParts, merge_cap)) {
      *big = true;
      return std::max(2, Pb);
    }
  }
  P = std::min({P, kMaxParts, merge_cap});
  return std::max(1, P);
}

// A dense step under the tiled full projection can prune its requests: the
// epilogue leaves each (beam, 32-token word) its legal (max, sum of exp), and
// the request kernel reads only the scores of the K words whose best
// candidates rank highest (at most 32 K candidates per request).  It pays when
// the request holds several times that many candidates (estimated from the
// table's mean row); each thread of the request kernel joins at most
// kPruneWordsHost of its beam's words.
double prune_bound(const StepArgs& a) {
  return 32.0 * (double)std::min<int64_t>(a.K, (int64_t)a.k_in * a.tab.words);
}
bool prune_step(const zgr_plan* p, const StepArgs& a) {
  if (!p->zms || a.plain_z) return false;
  if (a.tab.fmt != ZGR_FMT_DENSE && a.tab.fmt != ZGR_FMT_DENSE_NEXT) return false;
  // a single-beam request split over blocks ranks its keys by the score alone
  // (the merge forms the cumulative scores), which the pruned path does not
  if (a.k_in == 1 && prune_bound(a) > kMergeCapHost) return false;
  int kp2 = 1;
  while (kp2 < a.k_in) kp2 <<= 1;
  const int G = std::max(1, std::min(64, 1024 / kp2));
  if ((a.tab.words + G - 1) / G > kPruneWordsHost) return false;
  const HostTable& h = p->idx->host[a.t - 1];
  const double mean_n = (double)h.nnz / (double)std::max<int64_t>(1, h.rows);
  return a.k_in * std::min<double>(mean_n, a.tab.stride) >= kPruneGain * prune_bound(a);
}

// Blocks per pruned request: the fewest whose shares of the kept words'
// candidates fit the merge-sized LDS key array (one block for K <= 448).
int32_t prune_parts(const StepArgs& a) {
  return std::max(1, (int)std::ceil(prune_bound(a) / kMergeCapHost));
}

// Enqueue one step with the given projection.
int32_t run_step(zgr_plan* p, StepArgs a, int32_t proj, hipStream_t s) {
  const bool dense = a.tab.fmt == ZGR_FMT_DENSE || a.tab.fmt == ZGR_FMT_DENSE_NEXT;
  const int t = a.t;
  hipError_t e;
  int zmode;
  if (p->mode != ZGR_MODE_FILTER_FIRST) {
    // score-first and unconstrained: every token is scored (token-indexed
    // rows); score-first normalises over the whole codebook and then keeps the
    // legal tokens, unconstrained keeps every token (the all-legal row, whose
    // legal rank is the token)
    const bool unc = p->mode == ZGR_MODE_UNCONSTRAINED;
    if (unc) a.tab = p->all_tab;
    a.ldz = p->V;
    a.plain_z = true;
    e = prof_launch(p, ZGR_KERNEL_GEMM, t, s, [&] { return launch_full_projection(a, s); });
    if (e != hipSuccess) return hip_fail(e, "full projection launch");
    if (!unc) {
      a.lse_ext = p->lse;
      e = prof_launch(p, ZGR_KERNEL_NORM, t, s, [&] { return launch_row_lse(a, s); });
      if (e != hipSuccess) return hip_fail(e, "codebook log-sum-exp launch");
    }
    zmode = unc ? 1 : 0;
    a.z_token = zmode == 0;
    a.parts = request_parts(p, a, &a.big_parts);
    p->req_kind[t - 1] = zmode;
    p->req_parts[t - 1] = a.parts;
    e = prof_launch(p, ZGR_KERNEL_REQUEST, t, s, [&] { return launch_request_step(a, zmode, s); });
    if (e != hipSuccess) return hip_fail(e, "request step launch");
    if (a.parts > 1) {
      e = prof_launch(p, ZGR_KERNEL_REQUEST, t, s, [&] { return launch_request_merge(a, s); });
      if (e != hipSuccess) return hip_fail(e, "request merge launch");
    }
    return ZGR_OK;
  }
  // z layout: by legal rank on dense steps and on selective sparse steps,
  // token-indexed after a full projection of a sparse step
  if (proj == ZGR_PROJ_NAIVE) {
    a.ldz = a.tab.stride;
    if ((int64_t)a.M * a.tab.stride >= (int64_t)INT32_MAX)
      return fail(ZGR_E_SHAPE, "naive projection: candidate list would exceed 2^31 entries");
    int32_t* start = a.unit_start;  // [M + 1]
    e = prof_launch(p, ZGR_KERNEL_UNITS, t, s, [&] { return launch_naive_count(a, start, s); });
    if (e != hipSuccess) return hip_fail(e, "naive count launch");
    // the list and the temporary matrix are sized from the device count
    int32_t n = 0;
    e = hipMemcpyAsync(&n, start + a.M, 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "naive list size read-back");
    if (n > p->naive_cap) {
      for (void* x : {(void*)p->naive_beam, (void*)p->naive_tok, p->naive_tmp})
        if (x) (void)hipFree(x);
      p->naive_beam = p->naive_tok = nullptr;
      p->naive_tmp = nullptr;
      p->naive_cap = 0;
      e = hipMalloc((void**)&p->naive_beam, (size_t)n * 4);
      if (e == hipSuccess) e = hipMalloc((void**)&p->naive_tok, (size_t)n * 4);
      if (e == hipSuccess) e = hipMalloc(&p->naive_tmp, (size_t)n * p->d * elem_size(p->dtype));
      if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(ZGR_E_NOMEM, "naive projection: temporary matrix of " + std::to_string(n) + " rows");
      }
      p->naive_cap = n;
    }
    e = prof_launch(p, ZGR_KERNEL_SELECTIVE, t, s, [&] {
      return launch_naive_score(a, start, n, p->naive_beam, p->naive_tok, p->naive_tmp, s);
    });
    if (e != hipSuccess) return hip_fail(e, "naive score launch");
    zmode = 1;
  } else if (proj == ZGR_PROJ_FULL) {
    // dense rows and tiled sparse steps: legal columns only, by legal rank /
    // slot; the few-beam kernel on a sparse step writes token-indexed rows
    const bool slot = dense || full_projection_slot_layout(a);
    a.ldz = (slot && !dense) ? a.tab.stride : p->V;
    const bool prune = prune_step(p, a);
    a.zms = prune ? p->zms : nullptr;
    e = prof_launch(p, ZGR_KERNEL_GEMM, t, s, [&] { return launch_full_projection(a, s); });
    if (e != hipSuccess) return hip_fail(e, "full projection launch");
    zmode = prune ? 5 : (slot ? 1 : 0);
  } else if (!dense && light_sparse_step(p, a)) {
    a.ldz = a.tab.stride;
    zmode = 2;
  } else {
    a.ldz = a.tab.stride;
    if (!dense) {  // dense rows all have the same tiles: no unit scan needed
      if ((a.M + 1023) / 1024 > kMaxUnitChunksHost)
        return fail(ZGR_E_SHAPE, "selective projection of a sparse step: more than " +
                                     std::to_string(1024 * kMaxUnitChunksHost) + " beams");
      e = prof_launch(p, ZGR_KERNEL_UNITS, t, s, [&] { return launch_units(a, s); });
      if (e != hipSuccess) return hip_fail(e, "unit count launch");
    }
    const bool staged = proj == ZGR_PROJ_STAGED && dense;
    e = prof_launch(p, ZGR_KERNEL_SELECTIVE, t, s, [&] {
      return staged ? launch_staged_score(a, s) : launch_selective_score(a, s);
    });
    if (e != hipSuccess) return hip_fail(e, "selective score launch");
    zmode = 1;
  }
  a.z_token = zmode == 0;
  a.parts = zmode == 5 ? prune_parts(a) : request_parts(p, a, &a.big_parts);
  if (zmode != 1) a.big_parts = false;  // big parts are slot-indexed only
  p->req_kind[t - 1] = zmode;
  p->req_parts[t - 1] = a.parts;
  e = prof_launch(p, ZGR_KERNEL_REQUEST, t, s, [&] { return launch_request_step(a, zmode, s); });
  if (e != hipSuccess) return hip_fail(e, "request step launch");
  if (a.parts > 1) {
    e = prof_launch(p, ZGR_KERNEL_REQUEST, t, s, [&] { return launch_request_merge(a, s); });
    if (e != hipSuccess) return hip_fail(e, "request merge launch");
  }
  return ZGR_OK;
}

int32_t read_device_flag(zgr_plan* p, hipStream_t s) {
  // the flag follows the stream's work into pinned memory: one synchronisation
  hipError_t e = hipMemcpyAsync(p->err_host, p->err, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync error flag");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  const int32_t flag = *(volatile int32_t*)p->err_host;
  if (flag) {
    const int32_t zero = 0;
    e = hipMemcpy(p->err, &zero, sizeof(int32_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy error flag reset");
    return fail(ZGR_E_DEVICE, "a beam row was outside its step table (beam treated as dead)");
  }
  return ZGR_OK;
}

// One decode (all L steps).  When time_opts is set, every AUTO step is run
// with both projections twice, interleaved (full, selective, full,
// selective), and the second pair is timed with HIP events: by then the
// stream holds queued work, so neither timing includes the device waiting on
// the host to enqueue its launches, and each option finds the caches as the
// other one left them.  A step only reads its inputs and overwrites its
// outputs, so the last run's outputs carry the decode forward.
int32_t decode_impl(zgr_plan* p, zgr_hidden_fn fn, void* user, hipStream_t s, bool time_opts,
                    std::vector<float>* t_full, std::vector<float>* t_sel, int* final_buf) {
  hipError_t e = launch_decode_init(p->row[0], p->cum[0], p->B, p->K, s);
  if (e != hipSuccess) return hip_fail(e, "decode init launch");
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  if (time_opts)
    for (auto& x : ev) {
      e = hipEventCreate(&x);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
  int cur = 0;
  int32_t rc = ZGR_OK;
  for (int32_t t = 1; t <= p->L && rc == ZGR_OK; ++t) {
    const int32_t k_in = beams_in(p, t);
    if (fn(user, t, p->B, k_in, p->prefix[cur], p->L, p->hidden, (void*)s) != 0) {
      rc = fail(ZGR_E_CALLBACK, "hidden-vector callback returned non-zero at step " + std::to_string(t));
      break;
    }
    StepArgs a = make_args(p, t, p->hidden, p->row[cur], p->cum[cur], k_in, p->parent, p->token,
                           p->row[1 - cur], p->cum[1 - cur], nullptr, p->prefix[cur],
                           p->prefix[1 - cur]);
    if (time_opts && p->choice[t - 1] == ZGR_PROJ_AUTO) {
      float ms_full = 0.f, ms_sel = 0.f;
      rc = run_step(p, a, ZGR_PROJ_FULL, s);
      if (rc == ZGR_OK) rc = run_step(p, a, ZGR_PROJ_SELECTIVE, s);
      (void)hipEventRecord(ev[0], s);
      if (rc == ZGR_OK) rc = run_step(p, a, ZGR_PROJ_FULL, s);
      (void)hipEventRecord(ev[1], s);
      if (rc == ZGR_OK) rc = run_step(p, a, ZGR_PROJ_SELECTIVE, s);
      (void)hipEventRecord(ev[2], s);
      if (rc != ZGR_OK) break;
      e = hipEventSynchronize(ev[2]);
      if (e != hipSuccess) {
        rc = hip_fail(e, "hipEventSynchronize");
        break;
      }
      (void)hipEventElapsedTime(&ms_full, ev[0], ev[1]);
      (void)hipEventElapsedTime(&ms_sel, ev[1], ev[2]);
      t_full[t - 1].push_back(ms_full * 1000.f);
      t_sel[t - 1].push_back(ms_sel * 1000.f);
    } else {
      int32_t proj = p->choice[t - 1];
      if (proj == ZGR_PROJ_AUTO) proj = model_choice(p, t);
      rc = run_step(p, a, proj, s);
    }
    cur = 1 - cur;
  }
  if (time_opts)
    for (auto& x : ev)
      if (x) (void)hipEventDestroy(x);
  if (rc != ZGR_OK) {
    (void)hipStreamSynchronize(s);
    return rc;
  }
  *final_buf = cur;  // index of the buffers holding the final beams
  return ZGR_OK;
}

float median(std::vector<float> v) {
  if (v.empty()) return -1.f;
  std::sort(v.begin(), v.end());
  const size_t n = v.size();
  return (n & 1) ? v[n / 2] : 0.5f * (v[n / 2 - 1] + v[n / 2]);
}

}  // namespace

extern "C" {

const char* zgr_status_str(int32_t status) {
  switch (status) {
    case ZGR_OK: return "ok";
    case ZGR_E_ARG: return "invalid argument";
    case ZGR_E_DUP_SID: return "duplicate SID in catalog";
    case ZGR_E_TOKEN_RANGE: return "catalog token outside [0, V)";
    case ZGR_E_SHAPE: return "unsupported shape";
    case ZGR_E_NOMEM: return "out of memory";
    case ZGR_E_HIP: return "HIP runtime error";
    case ZGR_E_STATE: return "invalid state";
    case ZGR_E_CALLBACK: return "hidden-vector callback failed";
    case ZGR_E_DEVICE: return "device-side invalid input";
    default: return "unknown status";
  }
}

int32_t zgr_last_error(char* buf, size_t n) {
  if (buf && n > 0) {
    const size_t k = std::min(n - 1, zgr::g_err.size());
    std::memcpy(buf, zgr::g_err.data(), k);
    buf[k] = '\0';
  }
  return zgr::g_err_status;
}

int32_t zgr_plan_warmup(const zgr_index* idx, const void* const* W_dev, int32_t dtype, int32_t d,
                        int32_t B, int32_t K, zgr_hidden_fn hidden_fn, void* user,
                        int32_t n_warmup, const int32_t* force, void* stream, zgr_plan** out) {
  if (!idx || !W_dev || !out) return fail(ZGR_E_ARG, "zgr_plan_warmup: null argument");
  *out = nullptr;
  if (dtype < ZGR_F32 || dtype > ZGR_F16) return fail(ZGR_E_ARG, "zgr_plan_warmup: bad dtype");
  if (B < 1 || K < 1) return fail(ZGR_E_ARG, "zgr_plan_warmup: B and K must be >= 1");
  if (K > 1024) return fail(ZGR_E_SHAPE, "zgr_plan_warmup: K must be <= 1024");
  if ((int64_t)B * K >= INT32_MAX) return fail(ZGR_E_SHAPE, "zgr_plan_warmup: B*K must be < 2^31");
  if (d < 64 || d % 64 != 0 || !supported_hidden_size(d))
    return fail(ZGR_E_SHAPE, "zgr_plan_warmup: d must be one of 64,128,256,512,768,1024,2048,4096");
  if (n_warmup < 0) return fail(ZGR_E_ARG, "zgr_plan_warmup: n_warmup must be >= 0");
  for (int l = 0; l < idx->L; ++l) {
    if (!W_dev[l]) return fail(ZGR_E_ARG, "zgr_plan_warmup: null W_t");
    if (force && (force[l] < ZGR_PROJ_AUTO || force[l] > ZGR_PROJ_STAGED))
      return fail(ZGR_E_ARG, "zgr_plan_warmup: force[t] must be AUTO, FULL, SELECTIVE, NAIVE or STAGED");
    // the slot code beam_rank * S_t + slot must fit 32 bits
    if ((int64_t)K * std::max<int32_t>(1, idx->host[l].stride) >= (int64_t)UINT32_MAX)
      return fail(ZGR_E_SHAPE, "zgr_plan_warmup: K * slot stride too large");
  }
  if (!idx->on_device) return fail(ZGR_E_STATE, "zgr_plan_warmup: index is not on the device");
  hipStream_t s = (hipStream_t)stream;
  zgr_plan* p = new (std::nothrow) zgr_plan();
  if (!p) return fail(ZGR_E_NOMEM, "zgr_plan_warmup: host allocation");
  p->idx = idx;
  p->idx_generation = idx->generation;
  p->L = idx->L;
  p->V = idx->V;
  p->d = d;
  p->B = B;
  p->K = K;
  p->dtype = dtype;
  p->W.assign(W_dev, W_dev + idx->L);
  for (int l = 0; l < zgr::kMaxL; ++l) {
    p->choice[l] = (force && l < idx->L) ? force[l] : ZGR_PROJ_AUTO;
    p->us_full[l] = p->us_sel[l] = -1.f;
  }
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "hipGetDevice");
  }
  if (p->device != idx->device) {
    delete p;
    return fail(ZGR_E_STATE, "zgr_plan_warmup: index lives on another device");
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, p->device) == hipSuccess && prop.multiProcessorCount > 0)
    p->n_cu = prop.multiProcessorCount;
  // scratch sizes over all steps
  const int64_t MK = (int64_t)B * K;
  int64_t zmax = 0;
  // any step may be called with up to K beams per request
  for (int l = 0; l < idx->L; ++l)
    zmax = std::max(zmax, MK * (int64_t)std::max(idx->host[l].stride, idx->V));
  p->z_elems = zmax;
  int32_t rc = ZGR_OK;
  auto A = [&](void** dst, size_t bytes) {
    if (rc == ZGR_OK) rc = plan_alloc(p, dst, bytes);
  };
  A((void**)&p->z, (size_t)zmax * 4);
  // unit scans: one row per codebook slice when a sparse table is sliced
  A((void**)&p->unit_start, (size_t)(MK + 1) * 4);
  // sparse projection: unit totals and places per slice and 1,024-beam chunk
  const int64_t nq_max = (MK + 1023) / 1024;
  A((void**)&p->ctot, (size_t)kSlices * nq_max * 4);
  for (int l = 0; l < idx->L; ++l)
    if (idx->host[l].fmt == ZGR_FMT_SPARSE)
      p->chunk_cap = std::max<int64_t>(
          p->chunk_cap, 1024 * slice_units_per_beam(idx->host[l].stride, idx->V, idx->dev[l].sdir != nullptr));
  if (p->chunk_cap > 0) A((void**)&p->umeta, (size_t)kSlices * nq_max * p->chunk_cap * 16);
  A((void**)&p->lse, (size_t)MK * 4);
  bool any_dense = false;
  for (int l = 0; l < idx->L; ++l) any_dense = any_dense || idx->host[l].fmt != ZGR_FMT_SPARSE;
  if (any_dense) A((void**)&p->zms, (size_t)MK * ((idx->V + 31) / 32) * 8);
  A((void**)&p->part_keys, (size_t)B * kMaxParts * K * 8);
  A((void**)&p->part_cnt, (size_t)B * kMaxParts * 4);
  A((void**)&p->part_ms, (size_t)B * kMaxParts * 8);
  A((void**)&p->err, 4);
  A(&p->hidden, (size_t)MK * d * elem_size(dtype));
  for (int i = 0; i < 2; ++i) {
    A((void**)&p->row[i], (size_t)MK * 4);
    A((void**)&p->cum[i], (size_t)MK * 4);
    A((void**)&p->prefix[i], (size_t)MK * p->L * 4);
  }
  A((void**)&p->parent, (size_t)MK * 4);
  A((void**)&p->token, (size_t)MK * 4);
  // the all-legal row: row_ptr {0, V}, every bit set, rank directory 32 * word
  const int32_t words = (p->V + 31) / 32;
  void *all_rp = nullptr, *all_bits = nullptr, *all_rank = nullptr;
  A(&all_rp, 8);
  A(&all_bits, (size_t)words * 4);
  A(&all_rank, (size_t)words * 2);
  if (rc == ZGR_OK && hipHostMalloc((void**)&p->err_host, sizeof(int32_t), hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    p->err_host = nullptr;
    rc = fail(ZGR_E_NOMEM, "zgr_plan: pinned host flag");
  }
  if (rc != ZGR_OK) {
    zgr_plan_free(p);
    return rc;
  }
  {
    const int32_t rp_h[2] = {0, p->V};
    std::vector<uint32_t> bits_h(words, 0xFFFFFFFFu);
    if (p->V % 32) bits_h[words - 1] = (1u << (p->V % 32)) - 1u;
    std::vector<uint16_t> rank_h(words);
    for (int32_t w = 0; w < words; ++w) rank_h[w] = (uint16_t)(32 * w);
    e = hipMemcpy(all_rp, rp_h, 8, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(all_bits, bits_h.data(), (size_t)words * 4, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(all_rank, rank_h.data(), (size_t)words * 2, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      zgr_plan_free(p);
      return hip_fail(e, "all-legal row upload");
    }
    DevTable& at = p->all_tab;
    at.fmt = kFmtAll;
    at.stride = p->V;
    at.words = words;
    at.V = p->V;
    at.rows = 1;
    at.row_ptr = (const int32_t*)all_rp;
    at.tok = nullptr;
    at.bits = (const uint32_t*)all_bits;
    at.rank = (const uint16_t*)all_rank;
  }
  e = hipMemsetAsync(p->err, 0, 4, s);
  if (e == hipSuccess) e = hipMemsetAsync(p->prefix[0], 0xFF, (size_t)MK * p->L * 4, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    zgr_plan_free(p);
    return hip_fail(e, "plan scratch init");
  }
  bool any_auto = false;
  for (int l = 0; l < p->L; ++l) any_auto |= p->choice[l] == ZGR_PROJ_AUTO;
  if (any_auto && n_warmup > 0 && hidden_fn) {
    std::vector<float> tf[zgr::kMaxL], ts[zgr::kMaxL];
    for (int w = 0; w < n_warmup; ++w) {
      int fb = 0;
      const int32_t r = decode_impl(p, hidden_fn, user, s, true, tf, ts, &fb);
      if (r != ZGR_OK) {
        zgr_plan_free(p);
        return r;
      }
    }
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      zgr_plan_free(p);
      return hip_fail(e, "hipStreamSynchronize after warm-up");
    }
    for (int l = 0; l < p->L; ++l) {
      if (p->choice[l] != ZGR_PROJ_AUTO) continue;
      p->us_full[l] = median(tf[l]);
      p->us_sel[l] = median(ts[l]);
      p->choice[l] = (p->us_full[l] < p->us_sel[l]) ? ZGR_PROJ_FULL : ZGR_PROJ_SELECTIVE;
    }
    const int32_t st = read_device_flag(p, s);
    if (st != ZGR_OK) {
      zgr_plan_free(p);
      return st;
    }
  }
  for (int l = 0; l < p->L; ++l)
    if (p->choice[l] == ZGR_PROJ_AUTO) p->choice[l] = model_choice(p, l + 1);
  *out = p;
  return ZGR_OK;
}

int32_t zgr_plan_choice(const zgr_plan* p, int32_t t, int32_t* proj, float* us_full, float* us_sel) {
  if (!p) return fail(ZGR_E_ARG, "zgr_plan_choice: null plan");
  if (t < 1 || t > p->L) return fail(ZGR_E_ARG, "zgr_plan_choice: t out of range");
  if (proj) *proj = p->choice[t - 1];
  if (us_full) *us_full = p->us_full[t - 1];
  if (us_sel) *us_sel = p->us_sel[t - 1];
  return ZGR_OK;
}

int32_t zgr_plan_set_choice(zgr_plan* p, int32_t t, int32_t proj) {
  if (!p) return fail(ZGR_E_ARG, "zgr_plan_set_choice: null plan");
  if (t < 1 || t > p->L) return fail(ZGR_E_ARG, "zgr_plan_set_choice: t out of range");
  if (proj != ZGR_PROJ_FULL && proj != ZGR_PROJ_SELECTIVE && proj != ZGR_PROJ_NAIVE &&
      proj != ZGR_PROJ_STAGED)
    return fail(ZGR_E_ARG, "zgr_plan_set_choice: proj must be FULL, SELECTIVE, NAIVE or STAGED");
  p->choice[t - 1] = proj;
  return ZGR_OK;
}

int32_t zgr_plan_set_mode(zgr_plan* p, int32_t mode) {
  if (!p) return fail(ZGR_E_ARG, "zgr_plan_set_mode: null plan");
  if (mode < ZGR_MODE_FILTER_FIRST || mode > ZGR_MODE_UNCONSTRAINED)
    return fail(ZGR_E_ARG, "zgr_plan_set_mode: unknown mode");
  p->mode = mode;
  return ZGR_OK;
}

int32_t zgr_plan_mode(const zgr_plan* p, int32_t* mode) {
  if (!p || !mode) return fail(ZGR_E_ARG, "zgr_plan_mode: null argument");
  *mode = p->mode;
  return ZGR_OK;
}

int32_t zgr_plan_profile(zgr_plan* p, int32_t repeat) {
  if (!p) return fail(ZGR_E_ARG, "zgr_plan_profile: null plan");
  if (repeat < 0 || repeat > 1000) return fail(ZGR_E_ARG, "zgr_plan_profile: repeat must be in [0, 1000]");
  const int32_t rc = prof_flush(p);
  if (rc != ZGR_OK) return rc;
  p->profiling = repeat;
  std::memset(p->prof_ms, 0, sizeof(p->prof_ms));
  std::memset(p->prof_n, 0, sizeof(p->prof_n));
  return ZGR_OK;
}

int32_t zgr_plan_profile_read(zgr_plan* p, int32_t kernel, int32_t t, int64_t* launches,
                              double* total_ms) {
  if (!p) return fail(ZGR_E_ARG, "zgr_plan_profile_read: null plan");
  if (kernel < 0 || kernel >= ZGR_KERNEL_COUNT) return fail(ZGR_E_ARG, "zgr_plan_profile_read: bad kernel id");
  if (t < 1 || t > p->L) return fail(ZGR_E_ARG, "zgr_plan_profile_read: t out of range");
  const int32_t rc = prof_flush(p);
  if (rc != ZGR_OK) return rc;
  if (launches) *launches = p->prof_n[kernel][t - 1];
  if (total_ms) *total_ms = p->prof_ms[kernel][t - 1];
  return ZGR_OK;
}

void zgr_plan_free(zgr_plan* p) {
  if (!p) return;
  (void)prof_flush(p);
  if (p->err_host) (void)hipHostFree(p->err_host);
  for (hipEvent_t e : p->pool) (void)hipEventDestroy(e);
  p->pool.clear();
  for (void* x : {(void*)p->naive_beam, (void*)p->naive_tok, p->naive_tmp})
    if (x) p->allocations.push_back(x);
  if (!p->allocations.empty()) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (p->device >= 0 && cur != p->device) (void)hipSetDevice(p->device);
    (void)hipDeviceSynchronize();
    for (void* x : p->allocations) (void)hipFree(x);
    if (cur >= 0 && cur != p->device) (void)hipSetDevice(cur);
  }
  delete p;
}

int32_t zgr_step(zgr_plan* p, int32_t t, const void* hidden_dev, const int32_t* row_in,
                 const float* cum_in, int32_t k_in, int32_t* parent_out, int32_t* token_out,
                 int32_t* row_out, float* cum_out, float* slot_dbg, void* stream) {
  int32_t rc = check_args_step(p, t, hidden_dev, row_in, cum_in, k_in, parent_out, token_out,
                               row_out, cum_out);
  if (rc != ZGR_OK) return rc;
  StepArgs a = make_args(p, t, hidden_dev, row_in, cum_in, k_in, parent_out, token_out, row_out,
                         cum_out, slot_dbg, nullptr, nullptr);
  return run_step(p, a, p->choice[t - 1], (hipStream_t)stream);
}

int32_t zgr_decode(zgr_plan* p, zgr_hidden_fn hidden_fn, void* user, int32_t top_k,
                   int64_t* item_out, int32_t* sid_out, float* score_out, void* stream) {
  if (!p || !hidden_fn || !item_out) return fail(ZGR_E_ARG, "zgr_decode: null argument");
  if (top_k < 1 || top_k > p->K) return fail(ZGR_E_ARG, "zgr_decode: top_k must be in [1, K]");
  if (!index_alive(p->idx, p->idx_generation))
    return fail(ZGR_E_STATE, "zgr_decode: plan is stale (its index was freed)");
  hipStream_t s = (hipStream_t)stream;
  int cur = 0;
  const int32_t rc = decode_impl(p, hidden_fn, user, s, false, nullptr, nullptr, &cur);
  if (rc != ZGR_OK) return rc;
  hipError_t e = hipSuccess;
  if (p->mode == ZGR_MODE_UNCONSTRAINED) {
    // the codes were produced without the filter: look each one up
    e = launch_lookup_items(p->idx->dev, p->L, p->prefix[cur], p->cum[cur], p->B * p->K, p->row[cur], s);
    if (e != hipSuccess) return hip_fail(e, "item lookup launch");
  }
  e = launch_decode_final(p->row[cur], p->cum[cur], p->prefix[cur], p->B, p->K, p->L,
                                     top_k, item_out, sid_out, score_out, s);
  if (e != hipSuccess) return hip_fail(e, "decode final launch");
  return read_device_flag(p, s);
}

int32_t zgr_full_projection_variant(int32_t M, int32_t V, int32_t dtype, int32_t fmt, int32_t mode,
                                    int32_t n_cu, int32_t* kernel, int32_t* tile_m, int32_t* tile_n,
                                    int32_t* epilogue) {
  if (M < 1 || V < 1 || n_cu < 1) return fail(ZGR_E_ARG, "zgr_full_projection_variant: sizes must be >= 1");
  if (dtype < ZGR_F32 || dtype > ZGR_F16) return fail(ZGR_E_ARG, "zgr_full_projection_variant: bad dtype");
  if (fmt != ZGR_FMT_DENSE && fmt != ZGR_FMT_SPARSE && fmt != ZGR_FMT_DENSE_NEXT)
    return fail(ZGR_E_ARG, "zgr_full_projection_variant: bad fmt");
  if (mode < ZGR_MODE_FILTER_FIRST || mode > ZGR_MODE_UNCONSTRAINED)
    return fail(ZGR_E_ARG, "zgr_full_projection_variant: bad mode");
  const GemmVariant g = gemm_variant(M, V, fmt != ZGR_FMT_SPARSE, mode != ZGR_MODE_FILTER_FIRST, n_cu);
  if (kernel) *kernel = g.kernel;
  if (tile_m) *tile_m = g.tile_m;
  if (tile_n) *tile_n = g.tile_n;
  if (epilogue) *epilogue = g.epilogue;
  return ZGR_OK;
}

int32_t zgr_plan_request_path(const zgr_plan* p, int32_t t, int32_t* kind, int32_t* parts) {
  if (!p) return fail(ZGR_E_ARG, "zgr_plan_request_path: null plan");
  if (t < 1 || t > p->L) return fail(ZGR_E_ARG, "zgr_plan_request_path: t out of range");
  if (p->req_parts[t - 1] < 1) return fail(ZGR_E_STATE, "zgr_plan_request_path: step not run yet");
  if (kind) *kind = p->req_kind[t - 1];
  if (parts) *parts = p->req_parts[t - 1];
  return ZGR_OK;
}

int32_t zgr_plan_status(zgr_plan* p, void* stream) {
  if (!p) return fail(ZGR_E_ARG, "zgr_plan_status: null plan");
  return read_device_flag(p, (hipStream_t)stream);
}

}  // extern "C"

// ---- step without allocation --------------------------------------------------------------
//
// zgr_step_noalloc runs the kernels of zgr_step with the step's scratch (the
// score buffer, the unit scan, the request parts' keys and partials, the
// device flag) in one file-scope device array instead of a plan's HBM.  Each
// device holds its own copy of the array for the life of the process; host
// code reaches a device's copy only through the address hipGetSymbolAddress
// gives for it, taken once per device with that device current.

constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;  // 64 MiB per device
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kNoAllocMaxDevices = 64;
struct NoAllocDevice {
  unsigned char* ptr = nullptr;  // the device's copy of scratch
  int n_cu = 0;
  bool ready = false;
};
std::mutex g_noalloc_mu;
NoAllocDevice g_noalloc[kNoAllocMaxDevices];

// The flag is cleared by a kernel, not a memset, so a captured graph replays it.
__global__ void k_noalloc_flag_clear(int32_t* flag) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *flag = 0;
}
__global__ void k_noalloc_flag_copy(const int32_t* flag, int32_t* out) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *out = *flag;
}

int32_t noalloc_device(NoAllocDevice** out, int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kNoAllocMaxDevices)
    return fail(ZGR_E_STATE, "zgr_step_noalloc: device id beyond the supported range");
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  NoAllocDevice& d = g_noalloc[dev];
  if (!d.ready) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    }
    int n_cu = 0;
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    d.ptr = (unsigned char*)ptr;
    d.n_cu = n_cu > 0 ? n_cu : 256;
    d.ready = true;
  }
  *out = &d;
  *dev_out = dev;
  return ZGR_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" int32_t zgr_step_noalloc(const zgr_index* idx, const void* W_t, int32_t dtype, int32_t d,
                                    int32_t B, int32_t K, int32_t t, int32_t proj,
                                    const void* hidden_dev, const int32_t* row_in, const float* cum_in,
                                    int32_t k_in, int32_t* parent_out, int32_t* token_out,
                                    int32_t* row_out, float* cum_out, float* slot_dbg,
                                    int32_t* err_out, void* stream) {
  using namespace zgr;
  if (!idx || !W_t || !hidden_dev || !row_in || !cum_in || !parent_out || !token_out || !row_out ||
      !cum_out)
    return fail(ZGR_E_ARG, "zgr_step_noalloc: null argument");
  if (dtype < ZGR_F32 || dtype > ZGR_F16) return fail(ZGR_E_ARG, "zgr_step_noalloc: bad dtype");
  if (B < 1 || K < 1) return fail(ZGR_E_ARG, "zgr_step_noalloc: B and K must be >= 1");
  if (K > 1024) return fail(ZGR_E_SHAPE, "zgr_step_noalloc: K must be <= 1024");
  if (d < 64 || d % 64 != 0 || !supported_hidden_size(d))
    return fail(ZGR_E_SHAPE, "zgr_step_noalloc: d must be one of 64,128,256,512,768,1024,2048,4096");
  if (t < 1 || t > idx->L) return fail(ZGR_E_ARG, "zgr_step_noalloc: t out of range");
  if (k_in < 1 || k_in > K) return fail(ZGR_E_ARG, "zgr_step_noalloc: k_in must be in [1, K]");
  if (proj != ZGR_PROJ_FULL && proj != ZGR_PROJ_SELECTIVE)
    return fail(ZGR_E_ARG, "zgr_step_noalloc: proj must be ZGR_PROJ_FULL or ZGR_PROJ_SELECTIVE");
  if (!idx->on_device) return fail(ZGR_E_STATE, "zgr_step_noalloc: index is not on the device");
  const HostTable& h = idx->host[t - 1];
  if ((int64_t)K * std::max<int32_t>(1, h.stride) >= (int64_t)UINT32_MAX)
    return fail(ZGR_E_SHAPE, "zgr_step_noalloc: K * slot stride too large");
  const int64_t M = (int64_t)B * k_in;
  if ((int64_t)B * K >= INT32_MAX) return fail(ZGR_E_SHAPE, "zgr_step_noalloc: B*K must be < 2^31");
  // the step's scratch, carved from the array at 256-byte boundaries
  const int64_t ldz_max = std::max<int64_t>(h.stride, idx->V);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + std::max<size_t>(bytes, 4));
    return at;
  };
  const size_t o_err = take(4);
  const size_t o_pcnt = take((size_t)B * kMaxParts * 4);
  const size_t o_pms = take((size_t)B * kMaxParts * 8);
  const size_t o_pkeys = take((size_t)B * kMaxParts * K * 8);
  const int64_t nsl = (h.fmt == ZGR_FMT_SPARSE && !h.sdir.empty()) ? kSlices : 1;
  const size_t o_units = take((size_t)(M + 1) * 4);
  const int64_t nq = (M + 1023) / 1024;
  const size_t o_ctot = take((size_t)(nsl * nq) * 4);
  const int64_t chunk_cap =
      h.fmt == ZGR_FMT_SPARSE ? 1024 * slice_units_per_beam(h.stride, idx->V, !h.sdir.empty()) : 0;
  const size_t o_umeta = take((size_t)(nsl * nq * chunk_cap) * 16);
  const size_t o_lse = take((size_t)M * 4);
  const size_t o_z = take((size_t)M * ldz_max * 4);
  if (off > kNoAllocScratchBytes)
    return fail(ZGR_E_SHAPE, "zgr_step_noalloc: the step needs " + std::to_string(off) +
                                 " bytes of scratch; the static maximum is " +
                                 std::to_string(kNoAllocScratchBytes) + " bytes (use zgr_step with a plan)");
  NoAllocDevice* dv = nullptr;
  int dev = -1;
  int32_t rc = noalloc_device(&dv, &dev);
  if (rc != ZGR_OK) return rc;
  if (dev != idx->device) return fail(ZGR_E_STATE, "zgr_step_noalloc: index lives on another device");
  unsigned char* base = dv->ptr;
  // the fields of a plan that a step reads (no device memory of its own)
  zgr_plan p;
  p.idx = idx;
  p.L = idx->L;
  p.V = idx->V;
  p.d = d;
  p.B = B;
  p.K = K;
  p.dtype = dtype;
  p.n_cu = dv->n_cu;
  StepArgs a{};
  a.tab = idx->dev[t - 1];
  a.t = t;
  a.L = idx->L;
  a.B = B;
  a.K = K;
  a.k_in = k_in;
  a.M = (int32_t)M;
  a.d = d;
  a.dtype = dtype;
  a.hidden = hidden_dev;
  a.W = W_t;
  a.row_in = row_in;
  a.cum_in = cum_in;
  a.parent_out = parent_out;
  a.token_out = token_out;
  a.row_out = row_out;
  a.cum_out = cum_out;
  a.slot_dbg = slot_dbg;
  a.z = (float*)(base + o_z);
  a.unit_start = (int32_t*)(base + o_units);
  a.ctot = (int32_t*)(base + o_ctot);
  a.umeta = (int4*)(base + o_umeta);
  a.chunk_cap = chunk_cap;
  a.lse = (float*)(base + o_lse);
  a.parts = 1;
  a.part_keys = (uint64_t*)(base + o_pkeys);
  a.part_cnt = (int32_t*)(base + o_pcnt);
  a.part_ms = (float2*)(base + o_pms);
  a.err = (int32_t*)(base + o_err);
  a.n_cu = dv->n_cu;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(k_noalloc_flag_clear, dim3(1), dim3(64), 0, s, a.err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "flag clear launch");
  rc = run_step(&p, a, proj, s);
  if (rc != ZGR_OK) return rc;
  if (err_out) {
    hipLaunchKernelGGL(k_noalloc_flag_copy, dim3(1), dim3(64), 0, s, a.err, err_out);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "flag copy launch");
  }
  return ZGR_OK;
}
