// greedy_kernels.hpp -- gfx950 device code of greedy verification (the
// temperature -> 0 limit of the verify step), included once, by
// spec_verify.hip after spec_verify_kernels.hpp.
//
// Page cited: [B] the blog.hotdry.top post on speculative decoding and
// dynamic batching, item 流程编排: the candidates are compared with the
// target's choices in order; at the first mismatch the matching prefix is
// kept and decoding restarts from the mismatched position.  Under greedy
// decoding the target's choice at a position is the argmax of its logits;
// equal maxima go to the lowest token id.  The token emitted at the first
// mismatch is the target's argmax there, and when every draft matches the
// bonus is the argmax of the sequence's last target row.
//
// Two kernels, ordered by the stream:
//   argmax_kernel: the only HBM pass, over the target rows alone.  The same
//     wave tasks as the row-statistics pass (4096 consecutive logits of one
//     row, 8 groups of 8 per lane, 16-byte non-temporal loads); each task
//     writes its maximum and the lowest index holding it.
//   greedy_finish_kernel: one 256-thread workgroup per sequence combines
//     the task results of each target row, compares the drafts with the row
//     argmaxes in windows of 64 positions (one wave ballot each) and writes
//     the accepted prefix, the argmax at the first mismatch (or the bonus)
//     and -1 after it.
#pragma once

namespace sv {

constexpr int kGreedyThreads = 256;
constexpr int kGreedyWaves = kGreedyThreads / 64;

struct ArgPartial {     // one wave task of one target row
  float v;              // the task's maximum (-inf when every logit is -inf)
  int32_t k;            // lowest logit index holding it
};
static_assert(sizeof(ArgPartial) == 8, "stored as one 8-byte vector");

// (v, k) beats (bv, bk): larger value, or equal value and lower index.
// NaN never beats anything.
__device__ __forceinline__ bool arg_better(float v, int64_t k, float bv, int64_t bk) {
  return v > bv || (v == bv && k < bk);
}

// Butterfly over groups of `width` consecutive lanes (a power of two <= 64,
// wave-uniform), in the same lane steps as group_reduce: every lane of a
// group ends with the group's best (v, k).  The order is strict on the
// values that occur (no NaN ever becomes a candidate), so both lanes of a
// pair pick the same winner.
__device__ __forceinline__ void group_argmax(float& v, int64_t& k, int width) {
  using LF = LaneBits<float>;
  using LK = LaneBits<int64_t>;
  auto step = [&](float ov, int64_t ok) {
    if (arg_better(ov, ok, v, k)) {
      v = ov;
      k = ok;
    }
  };
  if (width > 1) step(LF::dpp<kDppQuadXor1>(v), LK::dpp<kDppQuadXor1>(k));
  if (width > 2) step(LF::dpp<kDppQuadXor2>(v), LK::dpp<kDppQuadXor2>(k));
  if (width > 4) step(LF::dpp<kDppHalfMirror>(v), LK::dpp<kDppHalfMirror>(k));
  if (width > 8) step(LF::dpp<kDppMirror>(v), LK::dpp<kDppMirror>(k));
  if (width > 16) {
    float av, bv;
    int64_t ak, bk;
    LF::swap16(v, av, bv);
    LK::swap16(k, ak, bk);
    v = av;
    k = ak;
    step(bv, bk);
  }
  if (width > 32) {
    float av, bv;
    int64_t ak, bk;
    LF::swap32(v, av, bv);
    LK::swap32(k, ak, bk);
    v = av;
    k = ak;
    step(bv, bk);
  }
}

__device__ __forceinline__ void wave_argmax(float& v, int64_t& k) { group_argmax(v, k, 64); }

// Wave task t covers target row t / tasks_per_row, logits
// [(t % tasks_per_row) * 4096, +4096); partial index = t.
template <int DT, bool VEC, bool CHECK>
__global__ __launch_bounds__(kStatsThreads) void argmax_kernel(
    const void* __restrict__ target, int64_t target_rows, int64_t ld, int64_t V,
    int64_t tasks_per_row, ArgPartial* __restrict__ partials, uint32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * kStatsWaves + (threadIdx.x >> 6);
  if (task >= target_rows * tasks_per_row) return;
  const int64_t row = task / tasks_per_row;
  const int64_t chunk = task - row * tasks_per_row;
  GroupRaw<DT> raw[kTaskGroupsPerLane];
  load_task<DT, VEC>(row_ptr<DT>(target, row, ld), chunk, V, lane, raw);
  // this lane's groups are g0 + j*64 + lane, visited in ascending index
  // order, so a strict '>' keeps the lowest index among the lane's maxima.
  // Logits past V read as -inf and never win against the lane's first
  // index, which is below V whenever any of its logits is.
  const int64_t g0 = chunk * (kWaveTaskElems / kGroup);
  float bv = -INFINITY;
  int64_t bk = (g0 + lane) * kGroup;
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < kTaskGroupsPerLane; ++j) {
    float v[kGroup];
    unpack<DT>(raw[j], v);
    const int64_t e0 = (g0 + j * 64 + lane) * kGroup;
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      if (v[k] > bv) {
        bv = v[k];
        bk = e0 + k;
      }
      if (CHECK && !(v[k] < INFINITY) && !(v[k] == -INFINITY)) bad |= SPEC_VERIFY_DEV_BAD_LOGIT;
    }
  }
  wave_argmax(bv, bk);
  if (CHECK) bad = wave_or(bad);
  if (lane == 0) {
    // non-temporal, as the row-statistics partials
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 pv = {__float_as_uint(bv), (uint32_t)(int32_t)bk};
    __builtin_nontemporal_store(pv, reinterpret_cast<u32x2*>(partials + task));
    if (CHECK) status_or(status, bad);
  }
}

// Argmax of target row `row` from its task partials, L lanes per row
// (L a power of two; lanes loop when a row has more than L partials).
__device__ __forceinline__ int64_t combine_argmax(const ArgPartial* __restrict__ part,
                                                  int64_t tpr, int L, int64_t row, bool active,
                                                  int lane) {
  const int sub = lane & (L - 1);
  float bv = -INFINITY;
  int64_t bk = INT64_MAX;
  if (active)
    for (int64_t i = sub; i < tpr; i += L) {
      const ArgPartial p = part[row * tpr + i];
      if (arg_better(p.v, p.k, bv, bk)) {
        bv = p.v;
        bk = p.k;
      }
    }
  group_argmax(bv, bk, L);
  return bk;
}

struct GreedyShared {
  int32_t amax[64];     // argmaxes of the current window's target rows
  int n;
  int skip;
};

template <bool CHECK>
__global__ __launch_bounds__(kGreedyThreads) void greedy_finish_kernel(
    int64_t V, int64_t target_rows, int64_t draft_rows, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ tokens, const ArgPartial* __restrict__ part, int64_t tpr,
    int combine_lanes, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_num_accepted,
    uint32_t* __restrict__ status) {
  __shared__ GreedyShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t b = blockIdx.x;
  const int64_t c0 = cu[b], c1 = cu[b + 1];
  const int64_t gamma = c1 - c0;
  const int64_t trow0 = c0 + b, drow0 = c0;
  if (!(c0 >= 0 && gamma >= 0 && c1 <= draft_rows && trow0 + gamma < target_rows)) {
    if (tid == 0) {
      out_num_accepted[b] = 0;
      status_or(status, SPEC_VERIFY_DEV_BAD_OFFSETS);
    }
    if (c0 >= 0 && gamma >= 0 && trow0 + gamma < target_rows)
      for (int64_t i = tid; i <= gamma; i += kGreedyThreads) out_tokens[trow0 + i] = -1;
    return;
  }
  if (tid == 0) {
    sh.n = (int)gamma;
    sh.skip = 0;
  }
  __syncthreads();
  const int L = combine_lanes;
  const int rows_per_wave = 64 / L;
  int64_t lo = 0;
  int64_t n = gamma;
  for (;; lo += 64) {
    const int64_t hi_t = lo + 64 < gamma + 1 ? lo + 64 : gamma + 1;
    const int64_t hi_d = lo + 64 < gamma ? lo + 64 : gamma;
    const int64_t i_me = lo + lane;
    int32_t x = -1;
    if (wave == 0 && i_me < hi_d) x = tokens[drow0 + i_me];
    const int64_t nt = hi_t - lo;
    for (int64_t r0 = (int64_t)wave * rows_per_wave; r0 < nt;
         r0 += (int64_t)kGreedyWaves * rows_per_wave) {
      const int64_t r = r0 + lane / L;
      const bool active = (lane / L) < rows_per_wave && r < nt;
      const int64_t k = combine_argmax(part, tpr, L, trow0 + lo + r, active, lane);
      if (active && (lane & (L - 1)) == 0) sh.amax[r] = (int32_t)k;
    }
    __syncthreads();
    if (wave == 0) {
      const bool valid = i_me < hi_d;
      const bool badtok = valid && (x < 0 || x >= V);
      // accept while the draft equals the target's argmax
      const bool reject = valid && x != sh.amax[lane];
      const uint64_t mask = __ballot(reject);
      const uint64_t btok = __ballot(badtok);
      if (lane == 0) {
        if (btok) sh.skip = 1;
        else if (mask) sh.n = (int)(lo + __builtin_ctzll(mask));
      }
    }
    __syncthreads();
    n = sh.n;
    if (sh.skip || n < gamma || lo + 64 > gamma) break;
    __syncthreads();   // the next window overwrites sh.amax
  }
  if (sh.skip) {
    for (int64_t i = tid; i <= gamma; i += kGreedyThreads) out_tokens[trow0 + i] = -1;
    if (tid == 0) {
      out_num_accepted[b] = 0;
      status_or(status, SPEC_VERIFY_DEV_BAD_TOKEN);
    }
    return;
  }
  for (int64_t i = tid; i <= gamma; i += kGreedyThreads) {
    int32_t v;
    if (i < n) v = tokens[drow0 + i];
    else if (i == n) v = sh.amax[n - lo];
    else v = -1;
    out_tokens[trow0 + i] = v;
  }
  if (tid == 0) out_num_accepted[b] = (int32_t)n;
}

}  // namespace sv
