// adaptive_k.hpp -- the adaptive draft-length controller and the acceptance
// statistics, for a bank of request slots (included once, by spec_verify.hip).
//
// Pages cited (by title and section):
//   [D] "大模型推理加速新范式：推测解码（Speculative Decoding）原理剖析与
//       vLLM生产级实现", section 4.3: the draft length follows a sliding
//       window of per-step acceptance ratios; it grows by one when their mean
//       is above a band around a target and shrinks by one below it, within
//       [k_min, k_max]; nothing changes before the window holds a minimum
//       number of ratios.  Section 4.2: the accept rate as the core metric.
//   [B] the blog.hotdry.top post on speculative decoding and dynamic
//       batching, 延迟权衡与自适应策略 and 工程落地参数清单: the same kind of
//       rule over the last 10 rounds with thresholds 80% / 50%.
//
// One controller per request slot.  State, structure of arrays over S slots
// (slot-major, so a wave's lanes read consecutive words for consecutive
// slots):
//   int32  k[S]        current draft length
//   int32  len[S]      ratios held (<= window)
//   int32  head[S]     ring position of the next ratio
//   double hist[W][S]  the last W ratios, hist[j * S + s]
// A step's ratio is alpha = accepted / max(drafted, 1) in double; the mean is
// the sequential double sum of the held ratios, oldest first, divided by
// their count.  The same function updates a slot on the host and on the GPU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify_kernels.hpp"   // the wave-level steps

namespace sv {

struct AdaptLayout {
  size_t k, len, head, hist, total;
};

__host__ __device__ inline size_t adapt_align(size_t x) { return (x + 255) / 256 * 256; }

__host__ __device__ inline AdaptLayout adapt_layout(int64_t slots, int64_t window) {
  AdaptLayout L;
  L.k = 0;
  L.len = adapt_align(L.k + (size_t)slots * 4);
  L.head = adapt_align(L.len + (size_t)slots * 4);
  L.hist = adapt_align(L.head + (size_t)slots * 4);
  L.total = adapt_align(L.hist + (size_t)slots * (size_t)window * 8);
  return L;
}

struct AdaptParams {
  int32_t k_min, k_max, k_init, window, min_history;
  double up, down;
};

struct AdaptState {
  int32_t* k;
  int32_t* len;
  int32_t* head;
  double* hist;
  int64_t S;
};

__host__ __device__ inline AdaptState adapt_state(void* base, int64_t slots, int64_t window) {
  const AdaptLayout L = adapt_layout(slots, window);
  char* p = static_cast<char*>(base);
  AdaptState st;
  st.k = reinterpret_cast<int32_t*>(p + L.k);
  st.len = reinterpret_cast<int32_t*>(p + L.len);
  st.head = reinterpret_cast<int32_t*>(p + L.head);
  st.hist = reinterpret_cast<double*>(p + L.hist);
  st.S = slots;
  return st;
}

__host__ __device__ inline void adapt_reset_slot(const AdaptParams& p, const AdaptState& st,
                                                 int64_t s) {
  st.k[s] = p.k_init;
  st.len[s] = 0;
  st.head[s] = 0;
}

// One step of slot s ([D] 4.3): append the ratio, then move k by one towards
// the band once enough ratios are held.  Returns the new draft length.
__host__ __device__ inline int32_t adapt_step(const AdaptParams& p, const AdaptState& st,
                                              int64_t s, int32_t accepted, int32_t drafted) {
  const int64_t S = st.S;
  const int32_t W = p.window;
  const double alpha = (double)accepted / (double)(drafted > 1 ? drafted : 1);
  int32_t head = st.head[s];
  int32_t len = st.len[s];
  if (head < 0 || head >= W || len < 0 || len > W) {
    // never-reset or corrupted slot: start an empty history rather than
    // index outside it
    head = 0;
    len = 0;
  }
  st.hist[(int64_t)head * S + s] = alpha;
  head = head + 1 == W ? 0 : head + 1;
  len = len < W ? len + 1 : W;
  st.head[s] = head;
  st.len[s] = len;
  int32_t k = st.k[s];
  if (len >= p.min_history) {
    // held ratios, oldest first: ring positions [j0, W) then [0, head) when
    // the history wraps, else [j0, head).  The loads of a group of 8 are
    // issued together; the additions stay in order.
    const int32_t j0 = head - len < 0 ? head - len + W : head - len;
    const int32_t end0 = j0 + len <= W ? j0 + len : W;
    double total = 0.0;
    auto add_range = [&](int32_t a, int32_t e) {
      int32_t j = a;
      for (; j + 8 <= e; j += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = st.hist[(int64_t)(j + u) * S + s];
#pragma unroll
        for (int u = 0; u < 8; ++u) total += v[u];
      }
      for (; j < e; ++j) total += st.hist[(int64_t)j * S + s];
    };
    add_range(j0, end0);
    if (j0 + len > W) add_range(0, j0 + len - W);
    const double avg = total / (double)len;
    if (avg > p.up) k = k + 1 < p.k_max ? k + 1 : p.k_max;
    else if (avg < p.down) k = k - 1 > p.k_min ? k - 1 : p.k_min;
    st.k[s] = k;
  }
  return k;
}

// Per-sequence step with its checks: the slot must exist and
// 0 <= accepted <= drafted.  An invalid sequence leaves every controller
// unchanged, reports the slot's current length (k_init for a bad slot) and
// sets a status bit; it is not counted in the statistics.
struct AdaptOne {
  int32_t k;
  uint32_t bad;
  int32_t valid;
};

__host__ __device__ inline AdaptOne adapt_one(const AdaptParams& p, const AdaptState& st,
                                              int64_t b, const int32_t* slots,
                                              const int32_t* cu, const int32_t* accepted) {
  AdaptOne r;
  r.bad = 0;
  r.valid = 0;
  const int64_t s = slots ? (int64_t)slots[b] : b;
  if (s < 0 || s >= st.S) {
    r.k = p.k_init;
    r.bad = 1u;   // SPEC_VERIFY_ADAPT_BAD_SLOT
    return r;
  }
  const int32_t drafted = cu[b + 1] - cu[b];
  const int32_t acc = accepted[b];
  if (drafted < 0 || acc < 0 || acc > drafted) {
    r.k = st.k[s];
    r.bad = 2u;   // SPEC_VERIFY_ADAPT_BAD_COUNTS
    return r;
  }
  r.k = adapt_step(p, st, s, acc, drafted);
  r.valid = 1;
  return r;
}

constexpr int kAdaptThreads = 1024;
constexpr int kAdaptWaves = kAdaptThreads / 64;

__global__ __launch_bounds__(kAdaptThreads) void adapt_reset_kernel(AdaptParams p, AdaptState st,
                                                                    int64_t count,
                                                                    const int32_t* slots) {
  const int64_t i = (int64_t)blockIdx.x * kAdaptThreads + threadIdx.x;
  if (i >= count) return;
  const int64_t s = slots ? (int64_t)slots[i] : i;
  if (s >= 0 && s < st.S) adapt_reset_slot(p, st, s);
}

// One workgroup walks the batch in chunks of 1024 sequences: each thread
// steps one sequence's controller, then the workgroup writes the exclusive
// prefix of the new lengths (the next step's packed offsets) and adds the
// step's totals to the statistics.  Slots must be distinct within a batch.
__global__ __launch_bounds__(kAdaptThreads) void adapt_update_kernel(
    AdaptParams p, AdaptState st, int64_t B, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ accepted,
    int32_t* __restrict__ next_k, int32_t* __restrict__ next_cu,
    unsigned long long* __restrict__ stats, uint32_t* __restrict__ status) {
  __shared__ int64_t wave_k[kAdaptWaves];
  __shared__ unsigned long long wave_stat[3][kAdaptWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int64_t carry = 0;
  unsigned long long tot_seq = 0, tot_acc = 0, tot_draft = 0;
  uint32_t bad = 0;
  for (int64_t base = 0; base < B; base += kAdaptThreads) {
    const int64_t b = base + tid;
    int64_t k = 0;
    unsigned long long v = 0, a = 0, d = 0;
    if (b < B) {
      const AdaptOne r = adapt_one(p, st, b, slots, cu, accepted);
      k = r.k;
      bad |= r.bad;
      next_k[b] = r.k;
      if (r.valid) {
        v = 1;
        a = (unsigned long long)accepted[b];
        d = (unsigned long long)(cu[b + 1] - cu[b]);
      }
    }
    // inclusive wave scan of k, then wave totals through LDS
    const int64_t incl = sv::wave_scan(k);
    v = sv::group_reduce(v, 64, sv::OpAdd());
    a = sv::group_reduce(a, 64, sv::OpAdd());
    d = sv::group_reduce(d, 64, sv::OpAdd());
    if (lane == 63) wave_k[wave] = incl;
    if (lane == 0) {
      wave_stat[0][wave] = v;
      wave_stat[1][wave] = a;
      wave_stat[2][wave] = d;
    }
    __syncthreads();
    int64_t before = carry;
    for (int w = 0; w < wave; ++w) before += wave_k[w];
    if (next_cu && b < B) next_cu[b] = (int32_t)(before + incl - k);
    int64_t chunk = 0;
    for (int w = 0; w < kAdaptWaves; ++w) chunk += wave_k[w];
    if (tid == 0)
      for (int w = 0; w < kAdaptWaves; ++w) {
        tot_seq += wave_stat[0][w];
        tot_acc += wave_stat[1][w];
        tot_draft += wave_stat[2][w];
      }
    carry += chunk;
    __syncthreads();   // wave_k / wave_stat are reused by the next chunk
  }
  // any thread's bad bits reach the status word
  bad = sv::wave_or(bad);
  if (lane == 0 && bad && status) atomicOr(status, bad);
  if (tid == 0) {
    if (next_cu) next_cu[B] = (int32_t)carry;
    if (stats) {
      stats[0] += tot_seq;
      stats[1] += tot_acc;
      stats[2] += tot_draft;
      stats[3] += tot_acc + tot_seq;   // emitted: accepted + 1 per sequence
    }
  }
}

}  // namespace sv
