// spec_verify.hip -- host side of the C ABI declared in include/spec_verify.h:
// argument checks, workspace layout, and the two launches of one verify step
// on the caller's HIP stream.  The device code is in spec_verify_kernels.hpp
// (sampled verification, with draft logits or point-mass drafts) and
// greedy_kernels.hpp (greedy verification).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "spec_verify.h"
#include "spec_verify_adapt.h"
#include "spec_verify_kernels.hpp"
#include "greedy_kernels.hpp"
#include "tree_kernels.hpp"
#include "adaptive_k.hpp"
#include "read_probe.hpp"

static_assert(sv::kMaxTreeNodes == SPEC_VERIFY_MAX_TREE_NODES, "tree node limit");
static_assert(sv::kMaxChildren == SPEC_VERIFY_MAX_TREE_CHILDREN, "tree child limit");

// The workspace of spec_verify_run_static: a file-scope device array, one
// copy per device the library runs on, held until the process ends.  In
// host code its name is only a stand-in for the symbol, never a device
// address: the address comes from hipGetSymbolAddress, resolved once per
// device by spec_verify_create (resolve_scratch below), and only that
// address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[SPEC_VERIFY_STATIC_WORKSPACE_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return SPEC_VERIFY_EHIP;
}

// Workspace sections, in bytes from the workspace base.
struct Layout {
  size_t partials = 0;   // Partial[(max_seqs + 2 * max_draft_rows) * tasks_per_row]
  size_t tiles = 0;      // double[max_seqs * num_tiles * kTileTerms]
  size_t counters = 0;   // uint32[max_seqs], cleared by the row pass of each call
  size_t total = 0;
};

}  // namespace

struct spec_verify_ctx {
  int device;
  void* scratch;           // device address of `scratch` on this device
  int64_t vocab;
  int dtype;
  int32_t max_seqs;
  int64_t max_draft_rows;
  uint32_t flags;
  int cu_count;
  int64_t tasks_per_row;   // wave tasks of 4096 logits per row
  int64_t num_tiles;       // 2048-logit residual tiles per row
  Layout layout;
};

namespace {

Layout make_layout(int32_t max_seqs, int64_t max_draft_rows, int64_t tasks_per_row,
                   int64_t num_tiles) {
  Layout L;
  // row statistics cover every target row (R_t = B + R_d) and every draft
  // row (R_d)
  const int64_t rows = (int64_t)max_seqs + 2 * max_draft_rows;
  size_t off = 0;
  L.partials = off;
  off = align_up(off + (size_t)rows * (size_t)tasks_per_row * sizeof(sv::Partial));
  L.tiles = off;
  off = align_up(off + (size_t)max_seqs * (size_t)num_tiles * sv::kTileTerms * sizeof(double));
  L.counters = off;
  off = align_up(off + (size_t)max_seqs * sizeof(uint32_t));
  L.total = off < kAlign ? kAlign : off;
  return L;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];   // per device: the address of `scratch`, once resolved

// The device address of `scratch` on `device`, resolved on the first call
// for that device with the device made current (the caller's current device
// is restored).
hipError_t resolve_scratch(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  if (!g_scratch[device]) {
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return e;
    if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (prev != device) {
      const hipError_t r = hipSetDevice(prev);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    g_scratch[device] = ptr;
  }
  *out = g_scratch[device];
  return hipSuccess;
}

// log2(e)/T split into a float rounded down and a positive float remainder.
sv::ExpConsts exp_consts(float temperature) {
  sv::ExpConsts c;
  const double log2e = 1.4426950408889634074;
  c.T = (double)temperature;
  c.c64 = log2e / c.T;
  float hi = (float)c.c64;
  if ((double)hi > c.c64) hi = std::nextafter(hi, 0.0f);
  double lo = c.c64 - (double)hi;
  if (!(lo > 0.0)) {
    hi = std::nextafter(hi, 0.0f);
    lo = c.c64 - (double)hi;
  }
  c.c_hi = hi;
  c.c_lo = (float)lo;
  return c;
}

int combine_lanes(int64_t tasks_per_row) {
  int L = 1;
  while (L < tasks_per_row && L < 64) L <<= 1;
  return L;
}

enum class Mode { kSampled, kPointDrafts, kGreedy };

// Launch `kernel`; with timing events, the pair (ev[2k], ev[2k+1]) is the
// dispatch's own start / stop event (no separate event packets on the
// stream, so the recorded interval is the kernel's execution).
template <typename F, typename... Args>
hipError_t launch(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                  hipEvent_t const* ev, int k, Args... args) {
  if (ev)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, ev[2 * k], ev[2 * k + 1], 0,
                          args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
  return hipGetLastError();
}

template <int DT, bool VEC, bool CHECK, int MODE>
hipError_t launch_sampled(const spec_verify_ctx* ctx, const spec_verify_args* a,
                          const Layout& layout, hipStream_t stream) {
  using namespace sv;
  const int64_t B = a->num_seqs;
  const int64_t R_d = a->total_draft_rows;
  const int64_t R_t = R_d + B;
  // point-mass drafts have no draft rows to scan
  const int64_t rows = MODE == kDraftLogits ? R_t + R_d : R_t;
  const void* draft = MODE == kDraftLogits ? a->draft_logits : nullptr;
  const ExpConsts ec = exp_consts(a->temperature);
  char* ws = static_cast<char*>(a->workspace);
  Partial* partials = reinterpret_cast<Partial*>(ws + layout.partials);
  double* tiles = reinterpret_cast<double*>(ws + layout.tiles);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws + layout.counters);
  hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(a->timing_events);
  hipError_t e;

  // kernel 1: one pass over all target (and draft) rows
  const int64_t grid1 = ceil_div(rows * ctx->tasks_per_row, kStatsWaves);
  e = launch(row_stats_kernel<DT, VEC, CHECK>, dim3((unsigned)grid1), dim3(kStatsThreads), 0,
             stream, ev, 0, a->target_logits, draft, R_t, rows, a->ld, ctx->vocab,
             ctx->tasks_per_row, ec, partials, counters, (int64_t)B, a->status);
  if (e != hipSuccess) return e;

  // kernel 2: G workgroups per sequence, about one per compute unit in all,
  // sharing a residual's second pass over its rows, with at least two tiles
  // each (at B = 1-4 and V = 128256, 32 workgroups of two tiles finish
  // ~1 us sooner than 63 of one).  Point-mass drafts never make that pass
  // (their draws use the row pass's task sums): one each.
  int64_t G = ctx->cu_count / B;
  if (G > (ctx->num_tiles + 1) / 2) G = (ctx->num_tiles + 1) / 2;
  if (G < 1 || MODE == kDraftPoint) G = 1;
  const size_t lds = (size_t)ctx->num_tiles * kTileTerms * sizeof(double);
  return launch(finish_kernel<DT, VEC, CHECK, MODE>, dim3((unsigned)(B * G)), dim3(kThreads), lds,
                stream, ev, 1, a->target_logits, draft, a->ld, ctx->vocab, R_t, R_d,
                a->cu_draft, a->draft_tokens, a->uniforms, ec, (const Partial*)partials,
                ctx->tasks_per_row, combine_lanes(ctx->tasks_per_row), ctx->num_tiles, (int)G,
                tiles, counters, a->out_tokens, a->out_num_accepted, a->out_p_draft,
                a->out_q_draft, a->out_residual_sum, a->status);
}

template <int DT, bool VEC, bool CHECK>
hipError_t launch_greedy(const spec_verify_ctx* ctx, const spec_verify_args* a,
                         const Layout& layout, hipStream_t stream) {
  using namespace sv;
  const int64_t B = a->num_seqs;
  const int64_t R_d = a->total_draft_rows;
  const int64_t R_t = R_d + B;
  // the argmax partials reuse the row-statistics section of the workspace
  ArgPartial* partials =
      reinterpret_cast<ArgPartial*>(static_cast<char*>(a->workspace) + layout.partials);
  hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(a->timing_events);
  hipError_t e;
  const int64_t grid1 = ceil_div(R_t * ctx->tasks_per_row, kStatsWaves);
  e = launch(argmax_kernel<DT, VEC, CHECK>, dim3((unsigned)grid1), dim3(kStatsThreads), 0, stream,
             ev, 0, a->target_logits, R_t, a->ld, ctx->vocab, ctx->tasks_per_row, partials,
             a->status);
  if (e != hipSuccess) return e;
  return launch(greedy_finish_kernel<CHECK>, dim3((unsigned)B), dim3(kGreedyThreads), 0, stream,
                ev, 1, ctx->vocab, R_t, R_d, a->cu_draft, a->draft_tokens,
                (const ArgPartial*)partials, ctx->tasks_per_row,
                combine_lanes(ctx->tasks_per_row), a->out_tokens, a->out_num_accepted, a->status);
}

template <int DT, bool VEC, bool CHECK>
hipError_t launch_mode(const spec_verify_ctx* ctx, const spec_verify_args* a, const Layout& L,
                       hipStream_t s, Mode mode) {
  switch (mode) {
    case Mode::kSampled: return launch_sampled<DT, VEC, CHECK, sv::kDraftLogits>(ctx, a, L, s);
    case Mode::kPointDrafts: return launch_sampled<DT, VEC, CHECK, sv::kDraftPoint>(ctx, a, L, s);
    default: return launch_greedy<DT, VEC, CHECK>(ctx, a, L, s);
  }
}

template <int DT>
hipError_t dispatch_vec(const spec_verify_ctx* ctx, const spec_verify_args* a, const Layout& L,
                        hipStream_t s, bool vec, bool check, Mode mode) {
  if (vec) return check ? launch_mode<DT, true, true>(ctx, a, L, s, mode)
                        : launch_mode<DT, true, false>(ctx, a, L, s, mode);
  return check ? launch_mode<DT, false, true>(ctx, a, L, s, mode)
               : launch_mode<DT, false, false>(ctx, a, L, s, mode);
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// A launch's total thread count must stay below 2^32: the row pass runs one
// wave per 4096-logit task of `rows` rows, the finishing kernels at most
// cu_count / B (>= 1) workgroups of kThreads per sequence.
bool grids_fit(const spec_verify_ctx* ctx, int64_t rows, int64_t B) {
  const int64_t limit = (int64_t)1 << 32;
  if (rows > limit / 64 / ctx->tasks_per_row) return false;
  int64_t G = B > 0 ? ctx->cu_count / B : 1;
  if (G < 1) G = 1;
  return B <= limit / sv::kThreads / G;
}

// Host-side argument checks shared by the entry points, then the launches.
// Fields a mode does not use are not checked.  With use_scratch the
// workspace is the library's `scratch` array (args->workspace and
// workspace_bytes are ignored), laid out for this call's B and R_d.
int run_mode(const spec_verify_ctx* ctx, const spec_verify_args* a, void* hip_stream,
             Mode mode, bool use_scratch = false) {
  if (!ctx || !a) return SPEC_VERIFY_EINVAL;
  const bool sampled = mode != Mode::kGreedy;
  const bool draft_rows = mode == Mode::kSampled;
  const int64_t B = a->num_seqs;
  const int64_t R_d = a->total_draft_rows;
  if (B < 0 || R_d < 0) return SPEC_VERIFY_EINVAL;
  if (sampled && (!(a->temperature > 0.0f) || !std::isfinite(a->temperature)))
    return SPEC_VERIFY_EINVAL;
  if (a->ld < ctx->vocab) return SPEC_VERIFY_EINVAL;
  if (B > ctx->max_seqs || R_d > ctx->max_draft_rows) return SPEC_VERIFY_ECAPACITY;
  if (!grids_fit(ctx, 2 * R_d + B, B)) return SPEC_VERIFY_ECAPACITY;
  Layout layout = ctx->layout;
  void* workspace = a->workspace;
  size_t workspace_bytes = a->workspace_bytes;
  if (use_scratch) {
    layout = make_layout((int32_t)B, R_d, ctx->tasks_per_row, ctx->num_tiles);
    if (layout.total > SPEC_VERIFY_STATIC_WORKSPACE_BYTES) return SPEC_VERIFY_ECAPACITY;
    workspace = ctx->scratch;
    workspace_bytes = SPEC_VERIFY_STATIC_WORKSPACE_BYTES;
  }
  if (B == 0) return SPEC_VERIFY_OK;
  const size_t esize = ctx->dtype == SPEC_VERIFY_BF16 ? 2 : 4;
  if (!a->cu_draft || !a->target_logits || !a->out_tokens || !a->out_num_accepted ||
      !workspace)
    return SPEC_VERIFY_EINVAL;
  if (sampled && !a->uniforms) return SPEC_VERIFY_EINVAL;
  if (R_d > 0 && !a->draft_tokens) return SPEC_VERIFY_EINVAL;
  if (draft_rows && R_d > 0 && !a->draft_logits) return SPEC_VERIFY_EINVAL;
  const void* draft = draft_rows ? a->draft_logits : nullptr;
  if (!aligned(a->target_logits, esize) || (draft && !aligned(draft, esize)) ||
      !aligned(a->cu_draft, 4) || (sampled && !aligned(a->uniforms, 4)) ||
      !aligned(a->out_tokens, 4) || !aligned(a->out_num_accepted, 4) ||
      !aligned(workspace, kAlign))
    return SPEC_VERIFY_EINVAL;
  if (workspace_bytes < layout.total) return SPEC_VERIFY_ECAPACITY;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e);
  if (cur != ctx->device) return SPEC_VERIFY_EINVAL;

  spec_verify_args args = *a;
  args.workspace = workspace;
  args.workspace_bytes = workspace_bytes;
  const bool vec = aligned(a->target_logits, 16) && (R_d == 0 || !draft || aligned(draft, 16)) &&
                   ((size_t)a->ld * esize) % 16 == 0;
  const bool check = (ctx->flags & SPEC_VERIFY_FLAG_CHECK) != 0;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  e = ctx->dtype == SPEC_VERIFY_BF16 ? dispatch_vec<1>(ctx, &args, layout, s, vec, check, mode)
                                     : dispatch_vec<0>(ctx, &args, layout, s, vec, check, mode);
  if (e != hipSuccess) return hip_fail(e);
  return SPEC_VERIFY_OK;
}

// ---- tree verification

template <int DT, bool VEC, bool CHECK>
hipError_t launch_tree(const spec_verify_ctx* ctx, const spec_verify_tree_args* a,
                       hipStream_t stream, bool greedy) {
  using namespace sv;
  const int64_t B = a->num_seqs;
  const int64_t R = a->total_nodes;
  char* ws = static_cast<char*>(a->workspace);
  hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(a->timing_events);
  const int64_t grid1 = ceil_div(R * ctx->tasks_per_row, kStatsWaves);
  const int L = combine_lanes(ctx->tasks_per_row);
  hipError_t e;
  if (greedy) {
    ArgPartial* partials = reinterpret_cast<ArgPartial*>(ws + ctx->layout.partials);
    e = launch(argmax_kernel<DT, VEC, CHECK>, dim3((unsigned)grid1), dim3(kStatsThreads), 0,
               stream, ev, 0, a->target_logits, R, a->ld, ctx->vocab, ctx->tasks_per_row,
               partials, a->status);
    if (e != hipSuccess) return e;
    return launch(tree_greedy_kernel, dim3((unsigned)B), dim3(kGreedyThreads), 0, stream, ev, 1,
                  ctx->vocab, R, a->cu_nodes, a->parent, a->tokens, (const ArgPartial*)partials,
                  ctx->tasks_per_row, L, a->out_tokens, a->out_path, a->out_num_accepted,
                  a->status);
  }
  Partial* partials = reinterpret_cast<Partial*>(ws + ctx->layout.partials);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws + ctx->layout.counters);
  const ExpConsts ec = exp_consts(a->temperature);
  e = launch(row_stats_kernel<DT, VEC, CHECK>, dim3((unsigned)grid1), dim3(kStatsThreads), 0,
             stream, ev, 0, a->target_logits, (const void*)nullptr, R, R, a->ld, ctx->vocab,
             ctx->tasks_per_row, ec, partials, counters, (int64_t)0, a->status);
  if (e != hipSuccess) return e;
  const size_t lds =
      (size_t)(tree_slot_rows(ctx->tasks_per_row) + 1) * (size_t)ctx->tasks_per_row * sizeof(double);
  return launch(tree_point_kernel<DT, VEC>, dim3((unsigned)B), dim3(kThreads), lds, stream, ev, 1,
                a->target_logits, a->ld, ctx->vocab, R, a->cu_nodes, a->parent, a->tokens,
                a->uniforms, ec, (const Partial*)partials, ctx->tasks_per_row, L,
                a->out_tokens, a->out_path, a->out_num_accepted, a->status);
}

template <int DT>
hipError_t dispatch_tree(const spec_verify_ctx* ctx, const spec_verify_tree_args* a,
                         hipStream_t s, bool vec, bool check, bool greedy) {
  if (vec) return check ? launch_tree<DT, true, true>(ctx, a, s, greedy)
                        : launch_tree<DT, true, false>(ctx, a, s, greedy);
  return check ? launch_tree<DT, false, true>(ctx, a, s, greedy)
               : launch_tree<DT, false, false>(ctx, a, s, greedy);
}

int run_tree(const spec_verify_ctx* ctx, const spec_verify_tree_args* a, void* hip_stream,
             bool greedy) {
  if (!ctx || !a) return SPEC_VERIFY_EINVAL;
  const int64_t B = a->num_seqs;
  const int64_t R = a->total_nodes;
  if (B < 0 || R < 0) return SPEC_VERIFY_EINVAL;
  if (!greedy && (!(a->temperature > 0.0f) || !std::isfinite(a->temperature)))
    return SPEC_VERIFY_EINVAL;
  if (a->ld < ctx->vocab) return SPEC_VERIFY_EINVAL;
  if (B > ctx->max_seqs || R > (int64_t)ctx->max_seqs + 2 * ctx->max_draft_rows)
    return SPEC_VERIFY_ECAPACITY;
  if (!grids_fit(ctx, R, B)) return SPEC_VERIFY_ECAPACITY;
  if (B == 0) return SPEC_VERIFY_OK;
  if (R < B) return SPEC_VERIFY_EINVAL;   // every tree has a root
  const size_t esize = ctx->dtype == SPEC_VERIFY_BF16 ? 2 : 4;
  if (!a->cu_nodes || !a->parent || !a->tokens || !a->target_logits || !a->out_tokens ||
      !a->out_path || !a->out_num_accepted || !a->workspace)
    return SPEC_VERIFY_EINVAL;
  if (!greedy && !a->uniforms) return SPEC_VERIFY_EINVAL;
  if (!aligned(a->target_logits, esize) || !aligned(a->cu_nodes, 4) || !aligned(a->parent, 4) ||
      !aligned(a->tokens, 4) || (!greedy && !aligned(a->uniforms, 4)) ||
      !aligned(a->out_tokens, 4) || !aligned(a->out_path, 4) ||
      !aligned(a->out_num_accepted, 4) || !aligned(a->workspace, kAlign))
    return SPEC_VERIFY_EINVAL;
  if (a->workspace_bytes < ctx->layout.total) return SPEC_VERIFY_ECAPACITY;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e);
  if (cur != ctx->device) return SPEC_VERIFY_EINVAL;
  const bool vec = aligned(a->target_logits, 16) && ((size_t)a->ld * esize) % 16 == 0;
  const bool check = (ctx->flags & SPEC_VERIFY_FLAG_CHECK) != 0;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  e = ctx->dtype == SPEC_VERIFY_BF16 ? dispatch_tree<1>(ctx, a, s, vec, check, greedy)
                                     : dispatch_tree<0>(ctx, a, s, vec, check, greedy);
  if (e != hipSuccess) return hip_fail(e);
  return SPEC_VERIFY_OK;
}

}  // namespace

extern "C" {

int spec_verify_tree_run_greedy(const spec_verify_ctx* ctx, const spec_verify_tree_args* a,
                                void* hip_stream) {
  return run_tree(ctx, a, hip_stream, true);
}

int spec_verify_tree_run_point(const spec_verify_ctx* ctx, const spec_verify_tree_args* a,
                               void* hip_stream) {
  return run_tree(ctx, a, hip_stream, false);
}

int spec_verify_create(spec_verify_ctx** out, int device, int64_t vocab, int dtype,
                       int32_t max_seqs, int64_t max_draft_rows, uint32_t flags,
                       size_t* workspace_bytes) {
  if (!out) return SPEC_VERIFY_EINVAL;
  *out = nullptr;
  if (dtype != SPEC_VERIFY_F32 && dtype != SPEC_VERIFY_BF16) return SPEC_VERIFY_EUNSUPPORTED;
  if (vocab <= 0 || vocab > sv::kMaxVocab) return SPEC_VERIFY_EUNSUPPORTED;
  if (max_seqs < 0 || max_draft_rows < 0 || device < 0) return SPEC_VERIFY_EINVAL;
  if ((flags & ~SPEC_VERIFY_FLAG_CHECK) != 0) return SPEC_VERIFY_EINVAL;
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess) return hip_fail(e);
  if (device >= count) return SPEC_VERIFY_EINVAL;
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_fail(e);
  void* scratch_ptr = nullptr;
  e = resolve_scratch(device, &scratch_ptr);
  if (e != hipSuccess) return hip_fail(e);
  spec_verify_ctx* c = new (std::nothrow) spec_verify_ctx();
  if (!c) return SPEC_VERIFY_EINVAL;
  c->device = device;
  c->scratch = scratch_ptr;
  c->vocab = vocab;
  c->dtype = dtype;
  c->max_seqs = max_seqs;
  c->max_draft_rows = max_draft_rows;
  c->flags = flags;
  c->cu_count = cus > 0 ? cus : 1;
  c->tasks_per_row = ceil_div(vocab, sv::kWaveTaskElems);
  c->num_tiles = ceil_div(vocab, sv::kTileElems);
  c->layout = make_layout(max_seqs, max_draft_rows, c->tasks_per_row, c->num_tiles);
  if (workspace_bytes) *workspace_bytes = c->layout.total;
  *out = c;
  return SPEC_VERIFY_OK;
}

int spec_verify_query_workspace(int64_t vocab, int32_t max_seqs, int64_t max_draft_rows,
                                size_t* workspace_bytes) {
  if (!workspace_bytes || max_seqs < 0 || max_draft_rows < 0) return SPEC_VERIFY_EINVAL;
  if (vocab <= 0 || vocab > sv::kMaxVocab) return SPEC_VERIFY_EUNSUPPORTED;
  *workspace_bytes =
      make_layout(max_seqs, max_draft_rows, ceil_div(vocab, sv::kWaveTaskElems),
                  ceil_div(vocab, sv::kTileElems))
          .total;
  return SPEC_VERIFY_OK;
}

size_t spec_verify_workspace_size(const spec_verify_ctx* ctx) {
  return ctx ? ctx->layout.total : 0;
}

int spec_verify_num_kernels(const spec_verify_ctx* ctx) { return ctx ? 2 : 0; }

int spec_verify_run(const spec_verify_ctx* ctx, const spec_verify_args* a, void* hip_stream) {
  return run_mode(ctx, a, hip_stream, Mode::kSampled);
}

int spec_verify_run_static(const spec_verify_ctx* ctx, const spec_verify_args* a,
                           void* hip_stream) {
  return run_mode(ctx, a, hip_stream, Mode::kSampled, true);
}

int spec_verify_run_point_drafts(const spec_verify_ctx* ctx, const spec_verify_args* a,
                                 void* hip_stream) {
  return run_mode(ctx, a, hip_stream, Mode::kPointDrafts);
}

int spec_verify_run_greedy(const spec_verify_ctx* ctx, const spec_verify_args* a,
                           void* hip_stream) {
  return run_mode(ctx, a, hip_stream, Mode::kGreedy);
}

int spec_verify_destroy(spec_verify_ctx* ctx) {
  delete ctx;
  return SPEC_VERIFY_OK;
}

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SPEC_VERIFY_OK: return "ok";
    case SPEC_VERIFY_EINVAL: return "invalid argument";
    case SPEC_VERIFY_EUNSUPPORTED: return "unsupported dtype or vocabulary size";
    case SPEC_VERIFY_ECAPACITY: return "capacity exceeded (batch, draft rows or workspace)";
    case SPEC_VERIFY_EHIP: return "HIP runtime error (see spec_verify_last_hip_error)";
    default: return "unknown status";
  }
}

int spec_verify_last_hip_error(void) { return g_last_hip_error; }

int spec_verify_read_probe(const void* src, size_t bytes, int nontemporal, uint32_t* sink,
                           void* hip_stream, void* start_event, void* stop_event) {
  if (!src || !sink || bytes == 0 || bytes % sv::kProbeWaveBytes != 0 || !aligned(src, 16) ||
      !aligned(sink, 4) || (!start_event) != (!stop_event))
    return SPEC_VERIFY_EINVAL;
  const int64_t waves = (int64_t)(bytes / sv::kProbeWaveBytes);
  const int64_t grid = ceil_div(waves, sv::kProbeThreads / 64);
  if (grid > 0x7fffffffLL) return SPEC_VERIFY_ECAPACITY;
  hipEvent_t ev[2] = {static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const sv::u32x4* p = static_cast<const sv::u32x4*>(src);
  const hipError_t e =
      nontemporal ? launch(sv::read_probe_kernel<true>, dim3((unsigned)grid), dim3(sv::kProbeThreads),
                           0, s, start_event ? ev : nullptr, 0, p, waves, sink)
                  : launch(sv::read_probe_kernel<false>, dim3((unsigned)grid),
                           dim3(sv::kProbeThreads), 0, s, start_event ? ev : nullptr, 0, p, waves,
                           sink);
  return e == hipSuccess ? SPEC_VERIFY_OK : hip_fail(e);
}

// ------------------------------------------------------------------ adaptive draft length

}  // extern "C"

namespace {

bool adapt_params_ok(const spec_verify_adapt_params* p) {
  return p && p->k_min >= 0 && p->k_max >= p->k_min && p->k_init >= p->k_min &&
         p->k_init <= p->k_max && p->window >= 1 && p->window <= SPEC_VERIFY_ADAPT_MAX_WINDOW &&
         p->min_history >= 1 && p->min_history <= p->window && p->reserved == 0 &&
         std::isfinite(p->up) && std::isfinite(p->down) && p->down <= p->up;
}

sv::AdaptParams adapt_params(const spec_verify_adapt_params* p) {
  sv::AdaptParams q;
  q.k_min = p->k_min;
  q.k_max = p->k_max;
  q.k_init = p->k_init;
  q.window = p->window;
  q.min_history = p->min_history;
  q.up = p->up;
  q.down = p->down;
  return q;
}

// Common checks; on success *on_device says where the pointers live.
int adapt_check(const spec_verify_adapt_params* p, int64_t num_slots, const void* state,
                size_t state_bytes, int device) {
  if (!adapt_params_ok(p) || num_slots < 0 || !state) return SPEC_VERIFY_EINVAL;
  if (reinterpret_cast<uintptr_t>(state) % 256 != 0) return SPEC_VERIFY_EINVAL;
  if (state_bytes < sv::adapt_layout(num_slots, p->window).total) return SPEC_VERIFY_ECAPACITY;
  if (device < SPEC_VERIFY_ADAPT_HOST) return SPEC_VERIFY_EINVAL;
  if (device >= 0) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e);
    if (cur != device) return SPEC_VERIFY_EINVAL;
  }
  return SPEC_VERIFY_OK;
}

}  // namespace

extern "C" {

int spec_verify_adapt_preset(int which, spec_verify_adapt_params* out) {
  if (!out) return SPEC_VERIFY_EINVAL;
  spec_verify_adapt_params p;
  std::memset(&p, 0, sizeof(p));
  if (which == SPEC_VERIFY_ADAPT_PRESET_WINDOW50) {
    const double target = 0.6;
    p.k_min = 2;
    p.k_max = 8;
    p.k_init = 2;
    p.window = 50;
    p.min_history = 10;
    p.up = target + 0.1;
    p.down = target - 0.1;
  } else if (which == SPEC_VERIFY_ADAPT_PRESET_LAST10) {
    p.k_min = 1;
    p.k_max = 8;
    p.k_init = 4;
    p.window = 10;
    p.min_history = 10;
    p.up = 0.8;
    p.down = 0.5;
  } else {
    return SPEC_VERIFY_EINVAL;
  }
  *out = p;
  return SPEC_VERIFY_OK;
}

int spec_verify_adapt_state_bytes(const spec_verify_adapt_params* params, int64_t num_slots,
                                  size_t* bytes) {
  if (!adapt_params_ok(params) || num_slots < 0 || !bytes) return SPEC_VERIFY_EINVAL;
  *bytes = sv::adapt_layout(num_slots, params->window).total;
  return SPEC_VERIFY_OK;
}

int spec_verify_adapt_reset(const spec_verify_adapt_params* params, int64_t num_slots,
                            void* state, size_t state_bytes, int64_t count,
                            const int32_t* slots, int device, void* hip_stream) {
  int rc = adapt_check(params, num_slots, state, state_bytes, device);
  if (rc != SPEC_VERIFY_OK) return rc;
  if (!slots) count = num_slots;
  if (count < 0) return SPEC_VERIFY_EINVAL;
  if (count == 0) return SPEC_VERIFY_OK;
  const sv::AdaptParams p = adapt_params(params);
  const sv::AdaptState st = sv::adapt_state(state, num_slots, params->window);
  if (device == SPEC_VERIFY_ADAPT_HOST) {
    for (int64_t i = 0; i < count; ++i) {
      const int64_t s = slots ? (int64_t)slots[i] : i;
      if (s >= 0 && s < num_slots) sv::adapt_reset_slot(p, st, s);
    }
    return SPEC_VERIFY_OK;
  }
  const int64_t grid = ceil_div(count, sv::kAdaptThreads);
  hipLaunchKernelGGL(sv::adapt_reset_kernel, dim3((unsigned)grid), dim3(sv::kAdaptThreads), 0,
                     static_cast<hipStream_t>(hip_stream), p, st, count, slots);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SPEC_VERIFY_OK : hip_fail(e);
}

int spec_verify_adapt_update(const spec_verify_adapt_params* params, int64_t num_slots,
                             void* state, size_t state_bytes, int32_t num_seqs,
                             const int32_t* slots, const int32_t* cu_draft,
                             const int32_t* num_accepted, int32_t* next_k, int32_t* next_cu,
                             uint64_t* stats, uint32_t* status, int device, void* hip_stream) {
  int rc = adapt_check(params, num_slots, state, state_bytes, device);
  if (rc != SPEC_VERIFY_OK) return rc;
  if (num_seqs < 0) return SPEC_VERIFY_EINVAL;
  if (!slots && num_seqs > num_slots) return SPEC_VERIFY_EINVAL;
  if (num_seqs == 0) {
    if (next_cu && device == SPEC_VERIFY_ADAPT_HOST) next_cu[0] = 0;
    if (next_cu && device >= 0) {
      // one int32 zero, written by a kernel so the call stays capturable
      hipLaunchKernelGGL(sv::adapt_update_kernel, dim3(1), dim3(sv::kAdaptThreads), 0,
                         static_cast<hipStream_t>(hip_stream), adapt_params(params),
                         sv::adapt_state(state, num_slots, params->window), (int64_t)0,
                         slots, cu_draft, num_accepted, next_k, next_cu,
                         (unsigned long long*)nullptr, status);
      hipError_t e = hipGetLastError();
      return e == hipSuccess ? SPEC_VERIFY_OK : hip_fail(e);
    }
    return SPEC_VERIFY_OK;
  }
  if (!cu_draft || !num_accepted || !next_k) return SPEC_VERIFY_EINVAL;
  const sv::AdaptParams p = adapt_params(params);
  const sv::AdaptState st = sv::adapt_state(state, num_slots, params->window);
  if (device == SPEC_VERIFY_ADAPT_HOST) {
    int64_t run = 0;
    uint64_t v = 0, a = 0, d = 0;
    uint32_t bad = 0;
    for (int64_t b = 0; b < num_seqs; ++b) {
      const sv::AdaptOne r = sv::adapt_one(p, st, b, slots, cu_draft, num_accepted);
      next_k[b] = r.k;
      bad |= r.bad;
      if (next_cu) next_cu[b] = (int32_t)run;
      run += r.k;
      if (r.valid) {
        v += 1;
        a += (uint64_t)num_accepted[b];
        d += (uint64_t)(cu_draft[b + 1] - cu_draft[b]);
      }
    }
    if (next_cu) next_cu[num_seqs] = (int32_t)run;
    if (stats) {
      stats[0] += v;
      stats[1] += a;
      stats[2] += d;
      stats[3] += a + v;
    }
    if (status) *status |= bad;
    return SPEC_VERIFY_OK;
  }
  hipLaunchKernelGGL(sv::adapt_update_kernel, dim3(1), dim3(sv::kAdaptThreads), 0,
                     static_cast<hipStream_t>(hip_stream), p, st, (int64_t)num_seqs, slots,
                     cu_draft, num_accepted, next_k, next_cu,
                     reinterpret_cast<unsigned long long*>(stats), status);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SPEC_VERIFY_OK : hip_fail(e);
}

}  // extern "C"
