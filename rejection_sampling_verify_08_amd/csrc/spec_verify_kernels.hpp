// spec_verify_kernels.hpp -- gfx950 device code of the batched
// speculative-decoding verify step (included once, by spec_verify.hip).
//
// Pages cited (by title and section):
//   [A] "推测解码与连续批处理深度实战：突破自回归生成的双重瓶颈", section 1.2.
//   [D] "大模型推理加速新范式：推测解码（Speculative Decoding）原理剖析与
//       vLLM生产级实现", sections 2.1 and 2.2.
//   [B] the blog.hotdry.top post on speculative decoding and dynamic
//       batching, items 流程编排 and 硬件并行.
//
// Two kernels per call:
//
//   row_stats_kernel  (the HBM-bound pass, ~90% of the bytes): every target
//     and draft row is read once.  Work is cut into wave tasks of 4096
//     consecutive elements of one row; each lane owns 8 groups of 8
//     consecutive elements (16-byte loads for bf16), the wave's 64 lanes
//     cover 64 consecutive groups per load instruction.  A wave computes the
//     exact maximum m of its raw logits and s = sum 2^(y_k), with
//     y_k = fma(l, c_lo, fma(l, c_hi, A)), A = -m * c_hi rounded, and
//     c_hi + c_lo = log2(e)/T.  y_k equals (l_k - m) * log2(e)/T + K up to
//     one rounding of |y_k|, where K = (A + m c_hi) + m c_lo is a per-wave
//     constant known exactly in double; the combine removes it.  Sums of 8
//     terms are fp32, everything above is fp64 in a fixed order.  Each wave
//     writes one partial {m, s}.
//
//   accept_draw_kernel  (the accept test, the stop at the first rejection,
//     and the resample / bonus draw): G workgroups per sequence.  Each
//     combines the sequence's row partials into exact row maxima M and
//     normalisers s in double, evaluates r_i = p_i(x_i) / q_i(x_i) in double
//     and finds n_b as the lowest lane of a wave ballot of !(u_i < r_i)
//     ([A] 1.2 step 3, [D] 2.1).  It then re-reads its share of the final
//     draw row(s) -- the rejected target/draft pair, or the bonus target row
//     -- and writes one double per 2048-element tile of
//     w_k = max(0, p_k - q_k) (or p_k), in a common scale.  The last
//     workgroup of the sequence to finish (integer arrival counter; no float
//     atomics anywhere) scans the tile sums, finds the tile holding
//     t = u * S, re-scans that tile and writes the token.
//
// Determinism: every floating-point reduction has a fixed order; the same
// device function produces w_k in the tile pass and in the re-scan, and the
// code is compiled with contraction off and explicit fmaf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;                    // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kGroup = 8;                        // elements per lane group
constexpr int kStatsGroupsPerLane = 8;           // groups per lane per wave task
constexpr int64_t kWaveTaskElems = 64LL * kGroup * kStatsGroupsPerLane;  // 4096
constexpr int64_t kTileElems = (int64_t)kThreads * kGroup;              // 2048
constexpr int kTileBatch = 64;                   // tiles per LDS flush

struct Partial {        // one wave task of one row
  float m;              // exact maximum of the raw logits (or -inf)
  float pad;
  double s;             // sum of 2^(y_k), y_k as in the header comment
};

struct ExpConsts {
  float c_hi;           // log2(e)/T rounded down to float
  float c_lo;           // float(log2(e)/T - c_hi), > 0
  double c64;           // log2(e)/T in double
  double T;             // temperature in double
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xffff0000u); }

__device__ __forceinline__ float fmax_nan_ignoring(float a, float b) {
  return __builtin_fmaxf(a, b);
}

// y = fma(l, c_lo, fma(l, c_hi, A)); 2^y.  -inf logits give exactly 0
// (c_lo > 0, and A is finite).
__device__ __forceinline__ float exp_term(float l, float A, const ExpConsts& c) {
  float y = __builtin_fmaf(l, c.c_hi, A);
  y = __builtin_fmaf(l, c.c_lo, y);
  return __builtin_amdgcn_exp2f(y);
}

// A = -m * c_hi rounded to float (0 for an all -inf range).
__device__ __forceinline__ float shift_of(float m, const ExpConsts& c) {
  return (m == -INFINITY) ? 0.0f : __fmul_rn(-m, c.c_hi);
}

// K = (A + m c_hi) + m c_lo, the per-range constant the computed exponents
// carry; the first bracket is exact in double.
__device__ __forceinline__ double offset_of(float m, float A, const ExpConsts& c) {
  return ((double)A + (double)m * (double)c.c_hi) + (double)m * (double)c.c_lo;
}

template <typename T>
__device__ __forceinline__ T wave_xor_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax_nan_ignoring(v, __shfl_xor(v, o));
  return v;
}

// Inclusive Hillis-Steele scan over the 64 lanes, fixed order.
__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    double t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ void status_or(uint32_t* status, uint32_t bits) {
  if (status && bits) atomicOr(status, bits);
}

// Load group `g` (elements 8g..8g+7) of a row.  Elements at or beyond V read
// as -inf.  VEC: the row base is 16-byte aligned, full groups use 16-byte
// loads; the ragged last group and the scalar path read element by element.
template <int DT, bool VEC>
__device__ __forceinline__ void load_group(const void* row, int64_t g, int64_t V,
                                           float v[kGroup]) {
  const int64_t e0 = g * kGroup;
  if (DT == 1) {
    const uint16_t* r = static_cast<const uint16_t*>(row);
    if (VEC && e0 + kGroup <= V) {
      uint4 q = *reinterpret_cast<const uint4*>(r + e0);
      v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
      v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
      v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
      v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    } else {
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        v[j] = (e0 + j < V) ? __uint_as_float((uint32_t)r[e0 + j] << 16) : -INFINITY;
    }
  } else {
    const float* r = static_cast<const float*>(row);
    if (VEC && e0 + kGroup <= V) {
      float4 a = *reinterpret_cast<const float4*>(r + e0);
      float4 b = *reinterpret_cast<const float4*>(r + e0 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < kGroup; ++j) v[j] = (e0 + j < V) ? r[e0 + j] : -INFINITY;
    }
  }
}

template <int DT>
__device__ __forceinline__ float load_logit(const void* row, int64_t k) {
  if (DT == 1) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(row)[k] << 16);
  return static_cast<const float*>(row)[k];
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const void* base, int64_t row, int64_t ld) {
  return static_cast<const char*>(base) + row * ld * (DT == 1 ? 2 : 4);
}

// ---------------------------------------------------------------- kernel 1

// Raw 16-byte blocks of one wave task, kept in registers between the max pass
// and the exponent pass.
template <int DT>
struct GroupRaw;
template <>
struct GroupRaw<1> { uint4 q; };
template <>
struct GroupRaw<0> { float4 a, b; };

template <int DT, bool VEC>
__device__ __forceinline__ void load_raw(const void* row, int64_t g, int64_t V,
                                         GroupRaw<DT>& out) {
  const int64_t e0 = g * kGroup;
  if (VEC && e0 + kGroup <= V) {
    if constexpr (DT == 1) {
      out.q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + e0);
    } else {
      out.a = *reinterpret_cast<const float4*>(static_cast<const float*>(row) + e0);
      out.b = *reinterpret_cast<const float4*>(static_cast<const float*>(row) + e0 + 4);
    }
  } else {
    float v[kGroup];
    load_group<DT, false>(row, g, V, v);
    if constexpr (DT == 1) {
      // re-encode: every value came from a bf16 (or is -inf), so the top 16
      // bits hold it exactly.
      uint32_t h[kGroup];
#pragma unroll
      for (int j = 0; j < kGroup; ++j) h[j] = __float_as_uint(v[j]) >> 16;
      out.q.x = h[0] | (h[1] << 16);
      out.q.y = h[2] | (h[3] << 16);
      out.q.z = h[4] | (h[5] << 16);
      out.q.w = h[6] | (h[7] << 16);
    } else {
      out.a = make_float4(v[0], v[1], v[2], v[3]);
      out.b = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

template <int DT>
__device__ __forceinline__ void unpack(const GroupRaw<DT>& r, float v[kGroup]) {
  if constexpr (DT == 1) {
    v[0] = bf16_lo(r.q.x); v[1] = bf16_hi(r.q.x);
    v[2] = bf16_lo(r.q.y); v[3] = bf16_hi(r.q.y);
    v[4] = bf16_lo(r.q.z); v[5] = bf16_hi(r.q.z);
    v[6] = bf16_lo(r.q.w); v[7] = bf16_hi(r.q.w);
  } else {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
}

// One pass over every target and draft row ([A] 1.2 step 2: the target
// scores all gamma+1 positions; the draft rows give q).  Wave task t covers
// row t / tasks_per_row, elements [(t % tasks_per_row) * 4096, +4096).
template <int DT, bool VEC, bool CHECK>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(
    const void* __restrict__ target, const void* __restrict__ draft,
    int64_t target_rows, int64_t total_rows, int64_t ld, int64_t V,
    int64_t tasks_per_row, ExpConsts ec, Partial* __restrict__ partials,
    uint32_t* __restrict__ counters, int32_t num_seqs,
    uint32_t* __restrict__ status) {
  // Clear the per-sequence arrival counters of the accept/draw kernel that
  // follows on the same stream.
  {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < num_seqs) counters[i] = 0u;
  }
  const int lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (task >= total_rows * tasks_per_row) return;
  const int64_t row = task / tasks_per_row;
  const int64_t chunk = task - row * tasks_per_row;
  const void* rp = row < target_rows ? row_ptr<DT>(target, row, ld)
                                     : row_ptr<DT>(draft, row - target_rows, ld);
  const int64_t g0 = chunk * (kWaveTaskElems / kGroup);

  GroupRaw<DT> raw[kStatsGroupsPerLane];
#pragma unroll
  for (int j = 0; j < kStatsGroupsPerLane; ++j)
    load_raw<DT, VEC>(rp, g0 + j * 64 + lane, V, raw[j]);

  // exact maximum of the raw logits (NaN inputs are ignored by fmax)
  float m = -INFINITY;
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < kStatsGroupsPerLane; ++j) {
    float v[kGroup];
    unpack<DT>(raw[j], v);
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      m = fmax_nan_ignoring(m, v[k]);
      if (CHECK && !(v[k] < INFINITY) && !(v[k] == -INFINITY)) bad |= 8u;
    }
  }
  m = wave_max(m);
  const float A = shift_of(m, ec);

  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < kStatsGroupsPerLane; ++j) {
    float v[kGroup];
    unpack<DT>(raw[j], v);
    float e[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) e[k] = exp_term(v[k], A, ec);
    const float s8 = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    acc += (double)s8;
  }
  acc = wave_xor_sum(acc);
  if (CHECK) bad = wave_or(bad);
  if (lane == 0) {
    Partial p;
    p.m = m;
    p.pad = 0.0f;
    p.s = acc;
    partials[task] = p;
    if (CHECK) status_or(status, bad);
  }
}

// ---------------------------------------------------------------- kernel 2

struct RowNorm {
  float M;       // exact row maximum of the raw logits
  double s;      // sum_k 2^((l_k - M) log2(e)/T), in double
};

// Combine the wave partials of one row (run by one whole wave).
__device__ __forceinline__ RowNorm combine_row(const Partial* __restrict__ part,
                                               int64_t nparts, const ExpConsts& ec,
                                               int lane) {
  float M = -INFINITY;
  for (int64_t i = lane; i < nparts; i += 64) M = fmax_nan_ignoring(M, part[i].m);
  M = wave_max(M);
  double s = 0.0;
  for (int64_t i = lane; i < nparts; i += 64) {
    const Partial p = part[i];
    if (p.m == -INFINITY) continue;
    const double K = offset_of(p.m, shift_of(p.m, ec), ec);
    s += p.s * exp2(((double)p.m - (double)M) * ec.c64 - K);
  }
  s = wave_xor_sum(s);
  RowNorm r;
  r.M = M;
  r.s = s;
  return r;
}

// Final-draw weights of one group, in a common positive scale:
//   residual: w = max(0, e_p - rho * e_q) = max(0, p - q) * s_p * 2^Kp
//   bonus   : w = e_p                      = p * s_p * 2^Kp
struct DrawConsts {
  float Ap, Aq;          // per-row shifts
  float rho_hi, rho_lo;  // rho = (s_p / s_q) 2^(Kp - Kq), split
  int residual;          // 1: residual of (p, q); 0: bonus from p
};

template <int DT, bool VEC>
__device__ __forceinline__ void group_weights(const void* prow, const void* qrow,
                                              int64_t g, int64_t V,
                                              const DrawConsts& dc,
                                              const ExpConsts& ec, float w[kGroup]) {
  float lp[kGroup];
  load_group<DT, VEC>(prow, g, V, lp);
  if (dc.residual) {
    float lq[kGroup];
    load_group<DT, VEC>(qrow, g, V, lq);
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const float ep = exp_term(lp[k], dc.Ap, ec);
      const float eq = exp_term(lq[k], dc.Aq, ec);
      float d = __builtin_fmaf(-eq, dc.rho_hi, ep);
      d = __builtin_fmaf(-eq, dc.rho_lo, d);
      w[k] = d > 0.0f ? d : 0.0f;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kGroup; ++k) w[k] = exp_term(lp[k], dc.Ap, ec);
  }
}

__device__ __forceinline__ float seq_sum8(const float w[kGroup]) {
  float c = w[0];
#pragma unroll
  for (int k = 1; k < kGroup; ++k) c += w[k];
  return c;
}

struct SeqShared {
  float M[2][64];        // row maxima of the current 64-row window (0 target, 1 draft)
  double s[2][64];
  double tile_part[kWaves][kTileBatch];
  double wave_tot[kWaves];
  double scan_out[3];    // total S, t = u S, exclusive prefix of the found tile
  int64_t found_tile;
  int64_t cand[kWaves];
  int64_t lastpos[kWaves];
  int n;                 // accepted count
  int last;              // this workgroup finishes the sequence
  int skip;              // the sequence is invalid and skipped
  int final_row_valid;
  RowNorm fp, fq;        // normalisers of the final-draw rows
};

// Combine the normalisers of target row trow0 + i (which = 0) or draft row
// drow0 + i (which = 1) for i in [lo, hi) into sh.M/s[which][i - lo].
__device__ __forceinline__ void combine_rows(SeqShared& sh, const Partial* partials,
                                             int64_t tasks_per_row, int64_t row_base,
                                             int which, int64_t lo, int64_t hi,
                                             const ExpConsts& ec, int wave, int lane) {
  for (int64_t i = lo + wave; i < hi; i += kWaves) {
    const RowNorm r = combine_row(partials + (row_base + i) * tasks_per_row,
                                  tasks_per_row, ec, lane);
    if (lane == 0) {
      sh.M[which][i - lo] = r.M;
      sh.s[which][i - lo] = r.s;
    }
  }
}

template <int DT, bool VEC, bool CHECK>
__global__ __launch_bounds__(kThreads) void accept_draw_kernel(
    const void* __restrict__ target, const void* __restrict__ draft, int64_t ld,
    int64_t V, int64_t target_rows, int64_t draft_rows,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ tokens,
    const float* __restrict__ uniforms, ExpConsts ec,
    const Partial* __restrict__ partials, int64_t tasks_per_row,
    double* __restrict__ tile_sums, uint32_t* __restrict__ counters,
    int64_t num_tiles, int wgs_per_seq, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_num_accepted, float* __restrict__ out_p,
    float* __restrict__ out_q, float* __restrict__ out_residual,
    uint32_t* __restrict__ status) {
  __shared__ SeqShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t b = (int64_t)blockIdx.x / wgs_per_seq;
  const int gidx = (int)((int64_t)blockIdx.x - b * wgs_per_seq);

  // ---- sequence geometry, guarded so bad offsets never index out of bounds
  const int64_t c0 = cu[b], c1 = cu[b + 1];
  const int64_t gamma = c1 - c0;
  const int64_t trow0 = c0 + b, drow0 = c0;
  if (tid == 0) {
    sh.skip = (c0 < 0 || gamma < 0 || c1 > draft_rows || trow0 + gamma >= target_rows) ? 1 : 0;
    sh.n = (int)gamma;
  }
  __syncthreads();
  if (sh.skip) {
    if (gidx == 0) {
      if (tid == 0) {
        out_num_accepted[b] = 0;
        if (out_residual) out_residual[b] = 0.0f;
        status_or(status, SPEC_VERIFY_DEV_BAD_OFFSETS);
      }
      if (c0 >= 0 && gamma >= 0 && trow0 + gamma < target_rows)
        for (int64_t i = tid; i <= gamma; i += kThreads) out_tokens[trow0 + i] = -1;
    }
    return;
  }

  // ---- accept tests in windows of 64 positions; stop at the first rejection
  uint32_t bad = 0;
  int64_t n = gamma;
  for (int64_t lo = 0; lo < gamma; lo += 64) {
    const int64_t hi = lo + 64 < gamma ? lo + 64 : gamma;
    combine_rows(sh, partials, tasks_per_row, trow0, 0, lo, hi, ec, wave, lane);
    combine_rows(sh, partials, tasks_per_row, target_rows + drow0, 1, lo, hi, ec, wave, lane);
    __syncthreads();
    if (wave == 0) {
      const int64_t i = lo + lane;
      bool reject = false;
      if (i < hi) {
        const int32_t x = tokens[drow0 + i];
        double r = 0.0;
        if (x < 0 || x >= V) {
          bad |= SPEC_VERIFY_DEV_BAD_TOKEN;
        } else {
          const double lp = load_logit<DT>(row_ptr<DT>(target, trow0 + i, ld), x);
          const double lq = load_logit<DT>(row_ptr<DT>(draft, drow0 + i, ld), x);
          const double Mp = sh.M[0][lane], Mq = sh.M[1][lane];
          const double sp = sh.s[0][lane], sq = sh.s[1][lane];
          const double pp = exp((lp - Mp) / ec.T) / sp;   // p_i(x_i)
          const double qq = exp((lq - Mq) / ec.T) / sq;   // q_i(x_i)
          r = exp(((lp - Mp) - (lq - Mq)) / ec.T) * (sq / sp);
          if (gidx == 0) {
            if (out_p) out_p[drow0 + i] = (float)pp;
            if (out_q) out_q[drow0 + i] = (float)qq;
          }
          if (CHECK) {
            if (!(qq > 0.0)) bad |= SPEC_VERIFY_DEV_ZERO_Q;
            if (Mp == -INFINITY || Mq == -INFINITY) bad |= SPEC_VERIFY_DEV_EMPTY_ROW;
          }
        }
        const float u = uniforms[trow0 + i];
        if (CHECK && !(u >= 0.0f && u < 1.0f)) bad |= SPEC_VERIFY_DEV_BAD_UNIFORM;
        // accept iff u < r ([A] 1.2 step 3 with the strict reading)
        reject = !((double)u < r);
      }
      const uint64_t mask = __ballot(reject);
      const uint64_t badtok = __ballot((bad & SPEC_VERIFY_DEV_BAD_TOKEN) != 0);
      if (lane == 0) {
        if (badtok) sh.skip = 2;
        else if (mask && n == gamma) sh.n = (int)(lo + __builtin_ctzll(mask));
      }
    }
    __syncthreads();
    if (sh.skip) break;
    n = sh.n;
    if (n < gamma) break;          // the first rejection ends the test ([D] 2.1)
  }
  if (sh.skip) {  // a draft token outside [0, V): skip the sequence
    if (gidx == 0) {
      for (int64_t i = tid; i <= gamma; i += kThreads) out_tokens[trow0 + i] = -1;
      if (tid == 0) {
        out_num_accepted[b] = 0;
        if (out_residual) out_residual[b] = 0.0f;
      }
    }
    bad = wave_or(bad);
    if (gidx == 0 && tid == 0) status_or(status, bad | SPEC_VERIFY_DEV_BAD_TOKEN);
    return;
  }
  n = sh.n;

  // ---- emit the accepted prefix ([B] 流程编排: keep the drafts before the
  // first mismatch); the slot n is written by the finishing workgroup.
  if (gidx == 0) {
    for (int64_t i = tid; i <= gamma; i += kThreads) {
      if (i < n) out_tokens[trow0 + i] = tokens[drow0 + i];
      else if (i > n) out_tokens[trow0 + i] = -1;
    }
    if (tid == 0) out_num_accepted[b] = (int32_t)n;
    // p/q outputs of positions past the stop point were not produced above
    // (the loop breaks at the first rejecting window); fill them here.
    if (out_p || out_q) {
      const int64_t done = ((n / 64) + 1) * 64;
      for (int64_t i = done + wave; i < gamma; i += kWaves) {
        const int32_t x = tokens[drow0 + i];
        if (x < 0 || x >= V) continue;
        const RowNorm rp = combine_row(partials + (trow0 + i) * tasks_per_row,
                                       tasks_per_row, ec, lane);
        const RowNorm rq = combine_row(partials + (target_rows + drow0 + i) * tasks_per_row,
                                       tasks_per_row, ec, lane);
        if (lane == 0) {
          const double lp = load_logit<DT>(row_ptr<DT>(target, trow0 + i, ld), x);
          const double lq = load_logit<DT>(row_ptr<DT>(draft, drow0 + i, ld), x);
          if (out_p) out_p[drow0 + i] = (float)(exp((lp - (double)rp.M) / ec.T) / rp.s);
          if (out_q) out_q[drow0 + i] = (float)(exp((lq - (double)rq.M) / ec.T) / rq.s);
        }
      }
    }
  }

  // ---- normalisers of the final-draw rows
  const int residual = n < gamma ? 1 : 0;
  const void* prow = row_ptr<DT>(target, trow0 + n, ld);
  const void* qrow = residual ? row_ptr<DT>(draft, drow0 + n, ld) : prow;
  if (wave == 0) {
    const RowNorm r = combine_row(partials + (trow0 + n) * tasks_per_row, tasks_per_row, ec, lane);
    if (lane == 0) sh.fp = r;
  } else if (wave == 1 && residual) {
    const RowNorm r = combine_row(partials + (target_rows + drow0 + n) * tasks_per_row,
                                  tasks_per_row, ec, lane);
    if (lane == 0) sh.fq = r;
  }
  __syncthreads();
  DrawConsts dc;
  dc.residual = residual;
  dc.Ap = shift_of(sh.fp.M, ec);
  const double Kp = offset_of(sh.fp.M, dc.Ap, ec);
  if (residual) {
    dc.Aq = shift_of(sh.fq.M, ec);
    const double Kq = offset_of(sh.fq.M, dc.Aq, ec);
    const double rho = (sh.fp.s / sh.fq.s) * exp2(Kp - Kq);
    dc.rho_hi = (float)rho;
    dc.rho_lo = (float)(rho - (double)dc.rho_hi);
  } else {
    dc.Aq = 0.0f;
    dc.rho_hi = 0.0f;
    dc.rho_lo = 0.0f;
  }

  // ---- tile sums of this workgroup's share of the vocabulary
  const int64_t per = (num_tiles + wgs_per_seq - 1) / wgs_per_seq;
  const int64_t t_lo = (int64_t)gidx * per;
  const int64_t t_hi = t_lo + per < num_tiles ? t_lo + per : num_tiles;
  double* ts = tile_sums + b * num_tiles;
  for (int64_t tb = t_lo; tb < t_hi; tb += kTileBatch) {
    const int64_t te = tb + kTileBatch < t_hi ? tb + kTileBatch : t_hi;
    for (int64_t t = tb; t < te; ++t) {
      float w[kGroup];
      group_weights<DT, VEC>(prow, qrow, t * kThreads + tid, V, dc, ec, w);
      double part = wave_xor_sum((double)seq_sum8(w));
      if (lane == 0) sh.tile_part[wave][t - tb] = part;
    }
    __syncthreads();
    for (int64_t t = tb + tid; t < te; t += kThreads) {
      const int j = (int)(t - tb);
      ts[t] = ((sh.tile_part[0][j] + sh.tile_part[1][j]) + sh.tile_part[2][j]) +
              sh.tile_part[3][j];
    }
    __syncthreads();
  }

  // ---- arrival: the last workgroup of the sequence finishes the draw
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&counters[b], 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
    sh.last = (old == (uint32_t)(wgs_per_seq - 1)) ? 1 : 0;
  }
  __syncthreads();
  bad = wave_or(bad);
  if (!sh.last) {
    if (CHECK && gidx == 0 && tid == 0) status_or(status, bad);
    return;
  }
  __threadfence();

  const float u = uniforms[trow0 + gamma];
  double S = 0.0, t_target = 0.0, P_excl = 0.0;
  int64_t tau = -1;
  for (int attempt = 0; attempt < 2; ++attempt) {
    // scan the tile sums in order (wave 0), find the tile holding t = u * S
    if (wave == 0) {
      double total = 0.0;
      for (int64_t c = 0; c < num_tiles; c += 64) {
        const double v = (c + lane < num_tiles) ? ts[c + lane] : 0.0;
        total += __shfl(wave_incl_scan(v, lane), 63);
      }
      const double t = (double)u * total;
      double base = 0.0;
      int64_t found = -1;
      double found_excl = 0.0;
      for (int64_t c = 0; c < num_tiles && found < 0; c += 64) {
        const double v = (c + lane < num_tiles) ? ts[c + lane] : 0.0;
        const double incl = base + wave_incl_scan(v, lane);
        const uint64_t hit = __ballot(c + lane < num_tiles && incl > t);
        const double prev = __shfl_up(incl, 1);
        if (hit) {
          const int l = __builtin_ctzll(hit);
          found = c + l;
          found_excl = __shfl(lane == 0 ? base : prev, l);
        }
        base = __shfl(incl, 63);
      }
      if (lane == 0) {
        sh.found_tile = found;
        sh.scan_out[0] = total;
        sh.scan_out[1] = t;
        sh.scan_out[2] = found_excl;
      }
    }
    __syncthreads();
    S = sh.scan_out[0];
    t_target = sh.scan_out[1];
    P_excl = sh.scan_out[2];
    tau = sh.found_tile;
    __syncthreads();
    if (S > 0.0 || attempt == 1) break;
    // Empty residual (only possible for invalid input or extreme rounding):
    // fall back to the target row at this position, done by this workgroup.
    bad |= SPEC_VERIFY_DEV_EMPTY_RESIDUAL;
    dc.residual = 0;
    for (int64_t tb = 0; tb < num_tiles; tb += kTileBatch) {
      const int64_t te = tb + kTileBatch < num_tiles ? tb + kTileBatch : num_tiles;
      for (int64_t t = tb; t < te; ++t) {
        float w[kGroup];
        group_weights<DT, VEC>(prow, qrow, t * kThreads + tid, V, dc, ec, w);
        double part = wave_xor_sum((double)seq_sum8(w));
        if (lane == 0) sh.tile_part[wave][t - tb] = part;
      }
      __syncthreads();
      for (int64_t t = tb + tid; t < te; t += kThreads) {
        const int j = (int)(t - tb);
        ts[t] = ((sh.tile_part[0][j] + sh.tile_part[1][j]) + sh.tile_part[2][j]) +
                sh.tile_part[3][j];
      }
      __syncthreads();
    }
  }

  // ---- re-scan tile tau: block exclusive scan of the per-thread group sums
  int64_t token = -1;
  if (tau >= 0) {
    float w[kGroup];
    const int64_t g = tau * kThreads + tid;
    group_weights<DT, VEC>(prow, qrow, g, V, dc, ec, w);
    const double incl = wave_incl_scan((double)seq_sum8(w), lane);
    const double below = __shfl_up(incl, 1);
    if (lane == 63) sh.wave_tot[wave] = incl;
    __syncthreads();
    double wbase = 0.0;
    for (int i = 0; i < wave; ++i) wbase += sh.wave_tot[i];
    const double excl = wbase + (lane == 0 ? 0.0 : below);
    // first element with C_k > t inside this thread's group
    int64_t cand = INT64_MAX;
    float c = 0.0f;
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      c += w[k];
      if (cand == INT64_MAX && w[k] > 0.0f && P_excl + (excl + (double)c) > t_target)
        cand = g * kGroup + k;
    }
    int64_t last_pos = -1;
#pragma unroll
    for (int k = 0; k < kGroup; ++k)
      if (w[k] > 0.0f) last_pos = g * kGroup + k;
    // block min of cand, block max of last_pos
    for (int o = 32; o > 0; o >>= 1) {
      const int64_t oc = __shfl_xor(cand, o);
      const int64_t ol = __shfl_xor(last_pos, o);
      cand = oc < cand ? oc : cand;
      last_pos = ol > last_pos ? ol : last_pos;
    }
    if (lane == 0) {
      sh.cand[wave] = cand;
      sh.lastpos[wave] = last_pos;
    }
    __syncthreads();
    if (tid == 0) {
      int64_t best = INT64_MAX, lastp = -1;
      for (int i = 0; i < kWaves; ++i) {
        best = sh.cand[i] < best ? sh.cand[i] : best;
        lastp = sh.lastpos[i] > lastp ? sh.lastpos[i] : lastp;
      }
      token = best != INT64_MAX ? best : lastp;
    }
  }
  if (tid == 0) {
    out_tokens[trow0 + n] = (int32_t)token;
    if (out_residual)
      out_residual[b] = residual && !(bad & SPEC_VERIFY_DEV_EMPTY_RESIDUAL)
                            ? (float)(S * exp2(-Kp) / sh.fp.s)
                            : 0.0f;
    counters[b] = 0u;
  }
  if (tid == 0) status_or(status, bad);
}

}  // namespace sv
