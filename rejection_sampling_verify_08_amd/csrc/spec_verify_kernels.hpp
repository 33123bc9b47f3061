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
// Two kernels per call, ordered by the stream.  Within the finishing kernel
// the workgroups of one sequence exchange tile sums through agent-scope
// atomic stores and loads and one arrival counter; nothing ever waits.
//
//   row_stats_kernel (the HBM-bound pass, ~90% of the bytes): every target
//     and draft row is read once ([A] 1.2 step 2: all gamma+1 positions are
//     scored in one pass).  Work is cut into wave tasks of 4096 consecutive
//     logits of one row; a lane owns 8 groups of 8 consecutive logits and the
//     wave's 64 lanes cover 64 consecutive groups per 16-byte load
//     instruction.  Loads are non-temporal (the data is consumed once).  A
//     wave computes the exact maximum m of its raw logits and
//       s = sum_k 2^(y_k),  y_k = fma(l_k, c_lo, fma(l_k, c_hi, A)),
//     with A = -m * c_hi rounded to float and c_hi + c_lo = log2(e) / T.
//     y_k = (l_k - m) log2(e)/T + K up to one rounding of |y_k|, where
//     K = (A + m c_hi) + m c_lo is a per-task constant known exactly in
//     double that later steps divide out.  Sums of 8 terms are fp32,
//     everything above is fp64 in a fixed order (fp32 logits: every term in
//     double, y_k unrounded).  Each wave task writes one partial {m, s} with
//     a non-temporal store.
//
//   finish_kernel (G 512-thread workgroups per sequence): each combines
//     the partials into exact row maxima M and normalisers s in double,
//     evaluates r_i = p_i(x_i) / q_i(x_i) in double, and takes n_b as the
//     lowest lane of a wave ballot of !(u_i < r_i) ([A] 1.2 step 3, [D] 2.1:
//     the first rejection ends the test).  A residual w_k = max(0, p_k - q_k)
//     needs both rows again: the G workgroups share one more read of the
//     rejected target/draft pair, formed without cancellation (residual_term),
//     with four sums per 2048-logit tile, kept in double (residual_tiles; the
//     tiles of a workgroup handed to its waves through an LDS counter), and
//     the last workgroup to arrive (an integer counter cleared by the row
//     pass) moves the sums to the exact normaliser ratio and scans them for
//     the tile holding t = u * S.  A bonus draw (w_k = p_k) and a point-mass
//     residual (p with x removed) need no
//     second pass: the row pass's task sums, moved into the draw's scale,
//     locate the 4096-logit task holding t (the task holding x is summed
//     again without it).  Either way the workgroup's 512 threads then search
//     the one interval in parallel (one group of 8 logits each) and write
//     the token: the smallest k with C_k > t.

// Determinism: every floating-point reduction has a fixed order; the same
// device function produces w_k in the tile pass and in the re-scan, and the
// code is compiled with contraction off and explicit fmaf.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kGroup = 8;                        // logits per lane group
constexpr int kStatsThreads = 256;               // row statistics: 4 wave64
constexpr int kStatsWaves = kStatsThreads / 64;
constexpr int kThreads = 512;                    // finishing workgroup: 8 wave64
constexpr int kWaves = kThreads / 64;
constexpr int kTaskGroupsPerLane = 8;            // groups per lane per wave task
constexpr int64_t kWaveTaskElems = 64LL * kGroup * kTaskGroupsPerLane;  // 4096
constexpr int kTileGroupsPerLane = 4;            // a tile: one wave, 4 groups per lane
constexpr int64_t kTileGroups = 64LL * kTileGroupsPerLane;              // 256
constexpr int64_t kTileElems = kTileGroups * kGroup;                    // 2048
constexpr int64_t kMaxTiles = 1024;              // LDS tile sums: V <= 2^21
constexpr int64_t kMaxVocab = kMaxTiles * kTileElems;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Partial {        // one wave task of one row
  float m;              // exact maximum of the raw logits (or -inf)
  float pad;
  double s;             // sum of 2^(y_k), y_k as in the header comment
};
static_assert(sizeof(Partial) == 16 && offsetof(Partial, s) == 8, "stored as one 16-byte vector");

struct ExpConsts {
  float c_hi;           // log2(e)/T rounded down to float
  float c_lo;           // float(log2(e)/T - c_hi), > 0
  double c64;           // log2(e)/T in double
  double T;             // temperature in double
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xffff0000u); }

// maximum that ignores NaN operands
__device__ __forceinline__ float fmax_nan_ignoring(float a, float b) {
  return __builtin_fmaxf(a, b);
}

// y = fma(l, c_lo, fma(l, c_hi, A)); 2^y.  -inf logits give exactly 0
// (c_lo > 0 and A is finite).
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

// ---- cross-lane steps without the LDS crossbar.  A butterfly over 64 lanes
// runs in rising distance: lanes 1 and 2 apart through quad permutations,
// then 4 and 8 through the half-row and row mirrors (after the first two
// steps a quad holds one value in all four lanes, so the mirror partner
// holds what the xor partner holds), then 16 and 32 through the permlane
// swaps (each gives every lane the even and the odd half, in that order).
// Each step combines the same two operands in every lane, so all lanes end
// with bitwise equal results.

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  // lanes whose source is outside the row, or whose row is masked, get 0
  if constexpr (ROW_MASK == 0xF) {
    // every lane is written (bound_ctrl: an out-of-row source reads as 0),
    // so no old value has to be set up first
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
  } else {
    // lanes of masked rows are not written and keep the old value, 0
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
  }
}

constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within 16
constexpr int kDppRowShr = 0x110;     // + n: lane i <- i - n within a row of 16
constexpr int kDppBcast15 = 0x142;    // lane 15 of a row -> the next row
constexpr int kDppBcast31 = 0x143;    // lane 31 -> rows 2 and 3
constexpr int kDppWaveShr1 = 0x138;   // lane i <- i - 1 across the wave (lane 0 gets 0)

template <typename T>
struct LaneBits;
template <>
struct LaneBits<float> {
  template <int CTRL, int RM = 0xF>
  __device__ static float dpp(float v) { return __uint_as_float(dpp_u32<CTRL, RM>(__float_as_uint(v))); }
  __device__ static void swap16(float v, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
  __device__ static void swap32(float v, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
  __device__ static float read(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
  }
};
template <>
struct LaneBits<uint32_t> {
  template <int CTRL, int RM = 0xF>
  __device__ static uint32_t dpp(uint32_t v) { return dpp_u32<CTRL, RM>(v); }
  __device__ static void swap16(uint32_t v, uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  }
  __device__ static void swap32(uint32_t v, uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  }
  __device__ static uint32_t read(uint32_t v, int l) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
  }
};
// 64-bit values move as two 32-bit halves
template <typename T64>
struct LaneBits64 {
  __device__ static uint64_t bits(T64 v) { return __builtin_bit_cast(uint64_t, v); }
  __device__ static T64 val(uint32_t lo, uint32_t hi) {
    return __builtin_bit_cast(T64, ((uint64_t)hi << 32) | lo);
  }
  template <int CTRL, int RM = 0xF>
  __device__ static T64 dpp(T64 v) {
    const uint64_t b = bits(v);
    return val(dpp_u32<CTRL, RM>((uint32_t)b), dpp_u32<CTRL, RM>((uint32_t)(b >> 32)));
  }
  __device__ static void swap16(T64 v, T64& a, T64& b) {
    const uint64_t x = bits(v);
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
    a = val(lo[0], hi[0]);
    b = val(lo[1], hi[1]);
  }
  __device__ static void swap32(T64 v, T64& a, T64& b) {
    const uint64_t x = bits(v);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
    a = val(lo[0], hi[0]);
    b = val(lo[1], hi[1]);
  }
  __device__ static T64 read(T64 v, int l) {
    const uint64_t b = bits(v);
    return val((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l),
               (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l));
  }
};
template <>
struct LaneBits<double> : LaneBits64<double> {};
template <>
struct LaneBits<int64_t> : LaneBits64<int64_t> {};
template <>
struct LaneBits<unsigned long long> : LaneBits64<unsigned long long> {};

// Butterfly over groups of `width` consecutive lanes (a power of two <= 64,
// wave-uniform): every lane of a group gets op over the group.
template <typename T, typename Op>
__device__ __forceinline__ T group_reduce(T v, int width, Op op) {
  using LB = LaneBits<T>;
  if (width > 1) v = op(v, LB::template dpp<kDppQuadXor1>(v));
  if (width > 2) v = op(v, LB::template dpp<kDppQuadXor2>(v));
  if (width > 4) v = op(v, LB::template dpp<kDppHalfMirror>(v));
  if (width > 8) v = op(v, LB::template dpp<kDppMirror>(v));
  if (width > 16) {
    T a, b;
    LB::swap16(v, a, b);
    v = op(a, b);
  }
  if (width > 32) {
    T a, b;
    LB::swap32(v, a, b);
    v = op(a, b);
  }
  return v;
}

struct OpAdd {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a + b; }
};
struct OpOr {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; }
};
struct OpMax {   // maximum that ignores NaN operands
  __device__ float operator()(float a, float b) const { return fmax_nan_ignoring(a, b); }
};
struct OpMaxI32 {   // signed maximum of 32-bit values carried as uint32_t
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return (int32_t)a > (int32_t)b ? a : b;
  }
};

template <typename T>
__device__ __forceinline__ T wave_xor_sum(T v) {
  return group_reduce(v, 64, OpAdd());
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  return group_reduce(v, 64, OpOr());
}

__device__ __forceinline__ float wave_max(float v) {
  return group_reduce(v, 64, OpMax());
}

// Value of lane l (wave-uniform l) in every lane.
template <typename T>
__device__ __forceinline__ T lane_value(T v, int l) {
  return LaneBits<T>::read(v, l);
}

// Inclusive scan over the 64 lanes, fixed order: Hillis-Steele within each
// row of 16 lanes, then each row's total is carried into the rows after it
// (row 0 into row 1 and row 2 into row 3, then rows 0-1 into rows 2-3).
template <typename T>
__device__ __forceinline__ T wave_scan(T v) {
  using LB = LaneBits<T>;
  v += LB::template dpp<kDppRowShr + 1>(v);
  v += LB::template dpp<kDppRowShr + 2>(v);
  v += LB::template dpp<kDppRowShr + 4>(v);
  v += LB::template dpp<kDppRowShr + 8>(v);
  v += LB::template dpp<kDppBcast15, 0xA>(v);
  v += LB::template dpp<kDppBcast31, 0xC>(v);
  return v;
}

__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
  (void)lane;
  return wave_scan(v);
}

__device__ __forceinline__ void status_or(uint32_t* status, uint32_t bits) {
  if (status && bits) atomicOr(status, bits);
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const void* base, int64_t row, int64_t ld) {
  return static_cast<const char*>(base) + row * ld * (DT == 1 ? 2 : 4);
}

template <int DT>
__device__ __forceinline__ float load_logit(const void* row, int64_t k) {
  if (DT == 1) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(row)[k] << 16);
  return static_cast<const float*>(row)[k];
}

// One group of 8 logits as raw 16-byte blocks (bf16: one block, f32: two).
template <int DT>
struct GroupRaw;
template <>
struct GroupRaw<1> { u32x4 q; };
template <>
struct GroupRaw<0> { f32x4 a, b; };

// Full group at element e0 of a 16-byte aligned row: non-temporal 16-byte
// loads.
template <int DT>
__device__ __forceinline__ void load_full_nt(const void* row, int64_t e0, GroupRaw<DT>& out) {
  if constexpr (DT == 1) {
    out.q = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(row) + e0));
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + e0);
    out.a = __builtin_nontemporal_load(p);
    out.b = __builtin_nontemporal_load(p + 1);
  }
}

// Group g (logits 8g..8g+7) of a row; logits at or beyond V read as -inf.
// VEC: full groups of a 16-byte aligned row use 16-byte loads; the ragged
// last group and unaligned rows are read element by element.
template <int DT, bool VEC>
__device__ __forceinline__ void load_group(const void* row, int64_t g, int64_t V,
                                           GroupRaw<DT>& out) {
  const int64_t e0 = g * kGroup;
  if (VEC && e0 + kGroup <= V) {
    load_full_nt<DT>(row, e0, out);
    return;
  }
  if constexpr (DT == 1) {
    const uint16_t* r = static_cast<const uint16_t*>(row);
    uint32_t h[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) h[j] = (e0 + j < V) ? (uint32_t)r[e0 + j] : 0xFF80u;
    out.q = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                  h[6] | (h[7] << 16)};
  } else {
    const float* r = static_cast<const float*>(row);
    float v[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) v[j] = (e0 + j < V) ? r[e0 + j] : -INFINITY;
    out.a = f32x4{v[0], v[1], v[2], v[3]};
    out.b = f32x4{v[4], v[5], v[6], v[7]};
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

// ---------------------------------------------------------------- row statistics

// The wave task's 8 groups (lane-strided by 64 groups) of one row.
template <int DT, bool VEC>
__device__ __forceinline__ void load_task(const void* rp, int64_t chunk, int64_t V, int lane,
                                          GroupRaw<DT> raw[kTaskGroupsPerLane]) {
  const int64_t g0 = chunk * (kWaveTaskElems / kGroup);
  if (VEC && (chunk + 1) * kWaveTaskElems <= V) {
    // the whole task is inside the row: no per-group bounds checks
#pragma unroll
    for (int j = 0; j < kTaskGroupsPerLane; ++j)
      load_full_nt<DT>(rp, (g0 + j * 64 + lane) * kGroup, raw[j]);
  } else {
#pragma unroll
    for (int j = 0; j < kTaskGroupsPerLane; ++j)
      load_group<DT, VEC>(rp, g0 + j * 64 + lane, V, raw[j]);
  }
}

// One residual tile (2048 logits) of a row for one wave: lane l gets groups
// l, l+64, l+128, l+192 of the tile (each 16-byte load instruction covers
// 1 KB of contiguous logits); past V: all -inf.
template <int DT, bool VEC>
__device__ __forceinline__ void load_tile(const void* row, int64_t t, int64_t V, int lane,
                                          GroupRaw<DT> raw[kTileGroupsPerLane]) {
  const int64_t g0 = t * kTileGroups;
  if (VEC && (t + 1) * kTileElems <= V) {
    // the whole tile is inside the row: no per-group bounds checks
#pragma unroll
    for (int j = 0; j < kTileGroupsPerLane; ++j)
      load_full_nt<DT>(row, (g0 + j * 64 + lane) * kGroup, raw[j]);
  } else {
#pragma unroll
    for (int j = 0; j < kTileGroupsPerLane; ++j)
      load_group<DT, VEC>(row, g0 + j * 64 + lane, V, raw[j]);
  }
}

// 2^y in double for y below ~1000, y = -inf, NaN or below -1100 giving 0:
// y = n + f with n = rint(y) and |f| <= 1/2; 2^f from the degree-8
// polynomial that interpolates it at the Chebyshev nodes of [-1/2, 1/2]
// (coefficients computed in 40-digit arithmetic; relative error of the
// polynomial below 1.1e-12 on the interval), scaled by 2^n.  The
// coefficients sit in constant memory so that they load once into scalar
// registers; there is no branch.
__constant__ double kExp2Poly[9] = {   // highest degree first
    1.3255224878668817e-06, 1.5310079402249296e-05, 0.00015403455852453838,
    0.0013333450568000645,  0.009618129159402558,   0.05550410941205933,
    0.2402265069581299,     0.6931471805459335,     1.0};
__device__ __forceinline__ double exp2_accurate(double y) {
  // fmax drops a NaN; 2^-1100 underflows to 0
  const double yc = __builtin_fmax(y, -1100.0);
  const double n = __builtin_rint(yc);
  const double f = yc - n;
  double e = kExp2Poly[0];
#pragma unroll
  for (int i = 1; i < 9; ++i) e = __builtin_fma(e, f, kExp2Poly[i]);
  return __builtin_ldexp(e, (int)n);
}

// Exact maximum m and s = sum 2^(y_k) of one wave task (all lanes get both).
// fp32 logits take every term in double: y_k = l_k c_hi + A + l_k c_lo
// without rounding and 2^(y_k) to ~1e-12.  The ratio of two rows'
// normalisers enters the residual draw, and when the draft row is within a
// few thousandths of the target row the residual is a small difference of
// two near-equal distributions: float terms (one rounding of y_k, ~3e-8 per
// exponential) left its sum up to ~2.4e-5 off.  bf16 logits keep the float
// terms (their residual tolerance is 2e-3).
template <int DT, bool CHECK, bool RAGGED>
__device__ __forceinline__ void task_stats(const GroupRaw<DT> raw[kTaskGroupsPerLane],
                                           const ExpConsts& ec, int64_t valid, float& m_out,
                                           double& s_out, uint32_t& bad) {
  // RAGGED: the task ends past the row (its last task, or a row shorter
  // than one task), with `valid` logits inside it.  Load j covers task
  // logits [512 j, 512 j + 512); past the row they are -inf, which leaves
  // the maximum and the sum unchanged, so such loads are skipped.
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kTaskGroupsPerLane; ++j) {
    if (RAGGED && j * 64 * kGroup >= valid) break;
    float v[kGroup];
    unpack<DT>(raw[j], v);
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      m = fmax_nan_ignoring(m, v[k]);   // NaN inputs are ignored by fmax
      if (CHECK && !(v[k] < INFINITY) && !(v[k] == -INFINITY)) bad |= SPEC_VERIFY_DEV_BAD_LOGIT;
    }
  }
  m = wave_max(m);
  const float A = shift_of(m, ec);
  double acc = 0.0;
  if constexpr (DT == 0) {
    const double chd = ec.c_hi, cld = ec.c_lo, Ad = A;
#pragma unroll
    for (int j = 0; j < kTaskGroupsPerLane; ++j) {
      if (RAGGED && j * 64 * kGroup >= valid) break;
      float v[kGroup];
      unpack<DT>(raw[j], v);
      double e[kGroup];
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        const double l = v[k];
        e[k] = exp2_accurate(__builtin_fma(l, cld, __builtin_fma(l, chd, Ad)));
      }
      acc += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    }
  } else {
#pragma unroll
    for (int j = 0; j < kTaskGroupsPerLane; ++j) {
      if (RAGGED && j * 64 * kGroup >= valid) break;
      float v[kGroup];
      unpack<DT>(raw[j], v);
      float e[kGroup];
#pragma unroll
      for (int k = 0; k < kGroup; ++k) e[k] = exp_term(v[k], A, ec);
      const float s8 = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      acc += (double)s8;
    }
  }
  m_out = m;
  s_out = wave_xor_sum(acc);
}

// One pass over every target and draft row ([A] 1.2 step 2: the target
// scores all gamma+1 positions; the draft rows give q).  Wave task t covers
// row t / tasks_per_row, logits [(t % tasks_per_row) * 4096, +4096); rows
// [0, target_rows) are target rows, the rest draft rows.  A row's partials
// are contiguous: partial index = row * tasks_per_row + chunk.
template <int DT, bool VEC, bool CHECK>
__global__ __launch_bounds__(kStatsThreads) void row_stats_kernel(
    const void* __restrict__ target, const void* __restrict__ draft,
    int64_t target_rows, int64_t total_rows, int64_t ld, int64_t V,
    int64_t tasks_per_row, ExpConsts ec, Partial* __restrict__ partials,
    uint32_t* __restrict__ counters, int64_t num_seqs, uint32_t* __restrict__ status) {
  // Clear the per-sequence arrival counters of the finishing kernel that
  // follows on the same stream (the grid has more than num_seqs / 256
  // workgroups).
  {
    const int64_t i = (int64_t)blockIdx.x * kStatsThreads + threadIdx.x;
    if (i < num_seqs) counters[i] = 0u;
  }
  const int lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * kStatsWaves + (threadIdx.x >> 6);
  if (task >= total_rows * tasks_per_row) return;
  const int64_t row = task / tasks_per_row;
  const int64_t chunk = task - row * tasks_per_row;
  const void* rp = row < target_rows ? row_ptr<DT>(target, row, ld)
                                     : row_ptr<DT>(draft, row - target_rows, ld);
  GroupRaw<DT> raw[kTaskGroupsPerLane];
  load_task<DT, VEC>(rp, chunk, V, lane, raw);
  float m;
  double s;
  uint32_t bad = 0;
  const int64_t valid = V - chunk * kWaveTaskElems;
  if (valid >= kWaveTaskElems) task_stats<DT, CHECK, false>(raw, ec, valid, m, s, bad);
  else task_stats<DT, CHECK, true>(raw, ec, valid, m, s, bad);
  if (CHECK) bad = wave_or(bad);
  if (lane == 0) {
    // a non-temporal 16-byte store: the partial goes out now instead of
    // sitting dirty in this XCD's L2 until the end-of-kernel write-back
    // (measured: the row pass ends ~1.5 us sooner)
    const uint64_t sb = __builtin_bit_cast(uint64_t, s);
    const u32x4 pv = {__float_as_uint(m), 0u, (uint32_t)sb, (uint32_t)(sb >> 32)};
    __builtin_nontemporal_store(pv, reinterpret_cast<u32x4*>(partials + task));
    if (CHECK) status_or(status, bad);
  }
}

// ---------------------------------------------------------------- combine

struct RowNorm {
  float M;       // exact row maximum of the raw logits
  double s;      // sum_k 2^((l_k - M) log2(e)/T), in double
};

// One partial per lane: lane slot `sub` of row `row` (an empty partial when
// inactive or past the row's partials).
__device__ __forceinline__ Partial load_partial(const Partial* __restrict__ part, int64_t tpr,
                                                int64_t row, int sub, bool active) {
  Partial p;
  p.m = -INFINITY;
  p.pad = 0.0f;
  p.s = 0.0;
  if (active && sub < tpr) p = part[row * tpr + sub];
  return p;
}

// Row maximum and normaliser from one partial per lane, L lanes per row.
__device__ __forceinline__ RowNorm reduce_partials(const Partial& p, int L, const ExpConsts& ec) {
  const float M = group_reduce(p.m, L, OpMax());
  double s = 0.0;
  if (p.m != -INFINITY) {
    const double K = offset_of(p.m, shift_of(p.m, ec), ec);
    s = p.s * exp2(((double)p.m - (double)M) * ec.c64 - K);
  }
  s = group_reduce(s, L, OpAdd());
  RowNorm r;
  r.M = M;
  r.s = s;
  return r;
}

// Combine rows r0, r0 + 1, ... of a sequence's partial table, `L` lanes per
// row (L a power of two >= the partials per row, or 64 with a loop when a
// row has more), so one wave combines 64 / L rows at once.
__device__ __forceinline__ RowNorm combine_rows_packed(const Partial* __restrict__ part,
                                                       int64_t tpr, int L, int64_t row,
                                                       bool active, const ExpConsts& ec,
                                                       int lane) {
  const int sub = lane & (L - 1);
  float M = -INFINITY;
  double s = 0.0;
  if (tpr <= L) {
    // one partial per lane: a single load feeds both reductions
    const bool have = active && sub < tpr;
    Partial p;
    p.m = -INFINITY;
    p.s = 0.0;
    if (have) p = part[row * tpr + sub];
    M = group_reduce(p.m, L, OpMax());
    if (have && p.m != -INFINITY) {
      const double K = offset_of(p.m, shift_of(p.m, ec), ec);
      s = p.s * exp2(((double)p.m - (double)M) * ec.c64 - K);
    }
  } else {
    if (active)
      for (int64_t i = sub; i < tpr; i += L) M = fmax_nan_ignoring(M, part[row * tpr + i].m);
    M = group_reduce(M, L, OpMax());
    if (active) {
      for (int64_t i = sub; i < tpr; i += L) {
        const Partial p = part[row * tpr + i];
        if (p.m == -INFINITY) continue;
        const double K = offset_of(p.m, shift_of(p.m, ec), ec);
        s += p.s * exp2(((double)p.m - (double)M) * ec.c64 - K);
      }
    }
  }
  s = group_reduce(s, L, OpAdd());
  RowNorm r;
  r.M = M;
  r.s = s;
  return r;
}

// Final-draw weights of one group, in a common positive scale (the target
// row's terms e_p = 2^((l_p - M_p) c + K_p), i.e. p * s_p * 2^Kp):
//   residual : w = max(0, p - q) * s_p * 2^Kp
//   point    : w = e_p, except 0 at token x = max(0, p - delta_x) * s_p * 2^Kp
//   bonus    : w = e_p                      = p * s_p * 2^Kp
constexpr int kDrawBonus = 0;
constexpr int kDrawResidual = 1;   // draft distribution given by draft logits
constexpr int kDrawPoint = 2;      // draft distribution is the point mass at x

struct DrawConsts {
  float Ap;              // target row shift
  float Aq;              // residual: draft row shift
  float dK;              // residual: K_p - K_q, moves draft terms into the target's scale
  float dM;              // residual: M_p - M_q (the two rows' maxima)
  float g;               // residual: 1 - s_p / s_q (the normaliser ratio, see below)
  int residual;          // kDrawBonus, kDrawResidual or kDrawPoint
  int64_t x;             // kDrawPoint: the rejected draft token
};

// The residual max(0, p - q) without cancellation.  With each row centred on
// its own maximum, d0_k = ((l_p - l_q) - (M_p - M_q)) c is the log2 ratio of
// the two rows' centred terms (exactly 0 where the rows agree up to the
// shift), and q_k / p_k = 2^(-d0_k) s_p / s_q.  Then
//   p_k - q_k = p_k (m0_k + g (1 - m0_k)),  m0_k = 1 - 2^(-d0_k),  g = 1 - s_p / s_q,
// linear in g.  The element's terms, in the weights' scale:
//   r0 = e_p - e_q       (sums to s_p' - s_q', the C-free row difference)
//   qs = e_q             (q_k in the same scale; dw/dg)
//   w  = max(0, r0 + g qs)
// with e_q the draft term moved into the target's scale.  Below |d0| = 1/2
// r0 = e_p m0 from a polynomial in d0 (relative precision near 0); above it
// both terms are exponentials and their difference keeps at least 29% of its
// larger term.  qs is the draft exponential in both ranges (e_p - r0 below
// 1/2 would equal it up to rounding): it enters w only through g qs, and the
// exact ratio below needs its sum only to the row sums' precision.  -inf
// logits need no special case: d0 is then
// infinite or NaN (the exponential branch) and the exponentials are 0.
constexpr float kSeriesLimit = 0.5f;
// (1 - 2^-x) / x on |x| <= 1/2: the degree-5 polynomial that interpolates it
// at the 6 Chebyshev nodes of [-1/2, 1/2] (coefficients computed in 40-digit
// arithmetic, highest degree first; relative error of the polynomial below
// 1.3e-8 on the interval, of its fp32 Horner evaluation below 7.1e-8)
constexpr int kOmTerms = 6;
__constant__ float kOmExp2[kOmTerms] = {
    -1.5453163359779865e-04f, 1.3390863314270973e-03f, -9.618083015084267e-03f,
    5.5503569543361664e-02f, -2.4022650718688965e-01f, 6.931471824645996e-01f};

struct ResidualTerm {
  float w, wu, r0, qs;   // w = max(0, wu): wu is the weight before the clip
};

__device__ __forceinline__ ResidualTerm residual_term(float lp, float lq, const DrawConsts& dc,
                                                      const ExpConsts& ec) {
  const float ep = exp_term(lp, dc.Ap, ec);
  float yq = __builtin_fmaf(lq, ec.c_hi, dc.Aq);
  yq = __builtin_fmaf(lq, ec.c_lo, yq) + dc.dK;
  const float qx = __builtin_amdgcn_exp2f(yq);
  // c_hi alone: c_lo / c_hi < 2^-23 is a relative change of d0 below fp32
  // rounding
  const float d0 = ((lp - lq) - dc.dM) * ec.c_hi;
  float ps = kOmExp2[0];
#pragma unroll
  for (int i = 1; i < kOmTerms; ++i) ps = __builtin_fmaf(ps, d0, kOmExp2[i]);
  const bool small = __builtin_fabsf(d0) < kSeriesLimit;
  ResidualTerm r;
  r.r0 = small ? ep * (ps * d0) : ep - qx;
  r.qs = qx;
  r.wu = __builtin_fmaf(dc.g, r.qs, r.r0);
  r.w = __builtin_fmaxf(r.wu, 0.0f);     // a NaN (0 - 0 * inf) gives 0
  return r;
}

// rp/rq hold group g of the p and q rows (rq unused unless kDrawResidual);
// e0 = 8 g is the group's first logit index.
template <int DT>
__device__ __forceinline__ void weights_of(const GroupRaw<DT>& rp, const GroupRaw<DT>& rq,
                                           int64_t e0, const DrawConsts& dc,
                                           const ExpConsts& ec, float w[kGroup]) {
  float lp[kGroup];
  unpack<DT>(rp, lp);
  if (dc.residual == kDrawPoint) {
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const float ep = exp_term(lp[k], dc.Ap, ec);
      w[k] = (e0 + k == dc.x) ? 0.0f : ep;
    }
  } else if (dc.residual == kDrawResidual) {
    float lq[kGroup];
    unpack<DT>(rq, lq);
#pragma unroll
    for (int k = 0; k < kGroup; ++k) w[k] = residual_term(lp[k], lq[k], dc, ec).w;
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
  float M[2][64];        // row maxima of the current 64-position window
  double s[2][64];       // (0: target rows, 1: draft rows)
  int32_t x[64];         // draft tokens of the current window
  int n;                 // accepted count
  int skip;              // nonzero: a bad draft token, the sequence is skipped
  uint32_t bad;
  int tile_next;         // residual tiles handed out past each wave's first
};

// ---------------------------------------------------------------- the draw

struct DrawShared {
  double wave_tot[kWaves];   // block scan: per-wave group-sum totals
  int32_t cand[kWaves];      // block search: per-wave first hit (or -1)
  int32_t last_pos[kWaves];  // block search: per-wave last positive weight
  double red[kWaves];        // block reduction
  double total, tt, p_excl;  // the draw's total, u * total, mass before tau
  int64_t tau;               // the tile / task holding tt
  double dg;                 // residual: the first-order move g* - g
  float g_star;              // residual: the exact normaliser ratio
  int linear_ok;             // residual: the move is certified
  int empty;                 // the residual summed to 0
  int last_wg;               // this workgroup arrived last
};

// Sum of v[0..n) in a fixed order (64-lane chunks, inclusive scans), one wave.
__device__ __forceinline__ double wave_total(const double* v, int64_t n, int lane) {
  double total = 0.0;
  for (int64_t c = 0; c < n; c += 64) {
    const double x = (c + lane < n) ? v[c + lane] : 0.0;
    total += lane_value(wave_incl_scan(x, lane), 63);
  }
  return total;
}

// One wave: the first c with (sum of v[0..c]) > tt; writes ds.tau and
// ds.p_excl (the sum before it).  tt < total is assumed; rounding can leave
// no hit, then tau is the last c with v[c] > 0.
__device__ __forceinline__ void find_interval(const double* v, int64_t n, double tt, int lane,
                                              DrawShared& ds) {
  double base = 0.0, p_excl = 0.0;
  int64_t tau = -1;
  for (int64_t c = 0; c < n && tau < 0; c += 64) {
    const double x = (c + lane < n) ? v[c + lane] : 0.0;
    const double incl = base + wave_incl_scan(x, lane);
    const uint64_t hit = __ballot(c + lane < n && incl > tt);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      tau = c + l;
      p_excl = l == 0 ? base : lane_value(incl, l - 1);
    }
    base = lane_value(incl, 63);
  }
  if (tau < 0) {
    // t at or past the rounded total: the last interval with mass
    int64_t lastc = -1;
    double before = 0.0, run = 0.0;
    for (int64_t c = 0; c < n; ++c) {
      if (v[c] > 0.0) {
        lastc = c;
        before = run;
      }
      run += v[c];
    }
    tau = lastc;
    p_excl = before;
  }
  if (lane == 0) {
    ds.tau = tau;
    ds.p_excl = p_excl;
  }
}

// Block-wide search inside one interval of consecutive groups: thread t of
// the workgroup holds group gi (active threads form a prefix in ascending
// group order).  The running sum of the weights, starting at p_excl,
// crosses tt at the returned logit index: the smallest k with C_k > tt (a
// zero-weight logit is never returned).  If rounding leaves tt past the
// interval's last weight, the last positive-weight logit is returned.  All
// threads of the workgroup must call it; the result is valid in every
// thread.  This core takes the weights each thread already holds (zeros for
// an inactive thread); block_search below computes them first.
__device__ __forceinline__ int64_t block_search_weights(const float w[kGroup], int64_t gi,
                                                        double tt, double p_excl,
                                                        DrawShared& ds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const double gs = (double)seq_sum8(w);
  const double incl = wave_incl_scan(gs, lane);
  const double below = LaneBits<double>::dpp<kDppWaveShr1>(incl);   // lane - 1's, 0 in lane 0
  if (lane == 63) ds.wave_tot[wave] = incl;
  __syncthreads();
  double base = p_excl;
  for (int v = 0; v < wave; ++v) base += ds.wave_tot[v];
  const double excl = lane == 0 ? 0.0 : below;
  // logit indices fit 32 bits (V <= kMaxVocab)
  int k_hit = -1;
  int32_t last_pos = -1;
  float c = 0.0f;
#pragma unroll
  for (int k = 0; k < kGroup; ++k) {
    c += w[k];
    if (k_hit < 0 && w[k] > 0.0f && base + (excl + (double)c) > tt) k_hit = k;
    if (w[k] > 0.0f) last_pos = (int32_t)(gi * kGroup + k);
  }
  const uint64_t hit = __ballot(k_hit >= 0);
  int32_t cand = -1;
  if (hit) {
    const int l = __builtin_ctzll(hit);
    cand = (int32_t)((gi - lane + l) * kGroup) + (int32_t)lane_value((uint32_t)k_hit, l);
  }
  last_pos = (int32_t)group_reduce((uint32_t)last_pos, 64, OpMaxI32());
  if (lane == 0) {
    ds.cand[wave] = cand;
    ds.last_pos[wave] = last_pos;
  }
  __syncthreads();
  // the first wave with a hit (lanes 0..kWaves-1 read one wave's result
  // each), else the last positive weight of the interval
  const int32_t cv = lane < kWaves ? ds.cand[lane] : -1;
  const uint64_t hits = __ballot(cv >= 0);
  if (hits) return (int32_t)lane_value((uint32_t)cv, __builtin_ctzll(hits));
  const int32_t lv = lane < kWaves ? ds.last_pos[lane] : -1;
  return (int32_t)lane_value(group_reduce((uint32_t)lv, kWaves, OpMaxI32()), 0);
}

template <int DT>
__device__ __forceinline__ int64_t block_search(const GroupRaw<DT>& rp, const GroupRaw<DT>& rq,
                                                int64_t gi, bool active, const DrawConsts& dd,
                                                const ExpConsts& ec, double tt, double p_excl,
                                                DrawShared& ds) {
  float w[kGroup];
  if (active) {
    weights_of<DT>(rp, rq, gi * kGroup, dd, ec, w);
  } else {
#pragma unroll
    for (int k = 0; k < kGroup; ++k) w[k] = 0.0f;
  }
  return block_search_weights(w, gi, tt, p_excl, ds);
}

// Block-wide sum of one double per thread in a fixed order.
__device__ __forceinline__ double block_sum(double v, DrawShared& ds) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const double ws = lane_value(wave_incl_scan(v, lane), 63);
  if (lane == 0) ds.red[wave] = ws;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kWaves; ++i) t += ds.red[i];
  return t;
}

// Draw from weights that need no second pass over the rows: the bonus
// (w = e_p) and the point-mass residual (w = e_p with x removed).  The
// interval sums are the row pass's task sums (4096 logits each) moved into
// the draw's scale: a task with maximum m summed 2^(l c + A_m), and the draw
// uses 2^(l c + Ap), so its sum is s_task 2^(Ap - A_m).  The task holding x
// is summed again here without x (never by subtraction, which would cancel
// when x dominates it).  One task (512 groups, one per thread of the first
// 512) is then searched.  `part` points at the row's task partials; task_sum has room for
// tpr doubles.  Returns the token; `total` receives the weights' sum.
template <int DT, bool VEC>
__device__ __forceinline__ int64_t draw_from_task_sums(
    const Partial* __restrict__ part, int64_t tpr, const void* prow, int64_t V,
    DrawConsts dc, const ExpConsts& ec, float u_final, double* task_sum, DrawShared& ds,
    uint32_t& fbad, double& total) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int64_t kTaskGroups = kWaveTaskElems / kGroup;   // 512
  static_assert(kTaskGroups <= kThreads, "one group per thread in a task");
  const bool point = dc.residual == kDrawPoint;
  const int64_t xtask = point ? dc.x / kWaveTaskElems : -1;
  const bool active = tid < kTaskGroups;
  // A task whose groups are needed whatever the sums say (the x-task, or
  // the only task of a row of at most 4096 logits) is loaded first, so that
  // its loads and the partials' are in flight together.
  const int64_t early = point ? xtask : (tpr == 1 ? 0 : -1);
  GroupRaw<DT> rp;
  int64_t gi = early * kTaskGroups + tid;
  if (early >= 0 && active) load_group<DT, VEC>(prow, gi, V, rp);
  // A row of at most 64 tasks: wave 0 holds every task sum (lane c: task c)
  // and does the x-task's substitution, the total and the scan for t in
  // registers, with one workgroup barrier (the scans keep wave_total's and
  // find_interval's order).  Longer rows go through LDS.
  const bool one_wave = tpr <= 64;
  auto task_term = [&](const Partial& pc) {
    return (pc.m == -INFINITY) ? 0.0 : pc.s * exp2((double)dc.Ap - (double)shift_of(pc.m, ec));
  };
  Partial pl;
  if (one_wave && wave == 0 && lane < tpr) pl = part[lane];
  if (!one_wave)
    for (int64_t c = tid; c < tpr; c += kThreads) task_sum[c] = task_term(part[c]);
  double xsum = 0.0;
  if (point) {
    double gsum = 0.0;
    if (active) {
      float w[kGroup];
      weights_of<DT>(rp, rp, gi * kGroup, dc, ec, w);
      gsum = (double)seq_sum8(w);
    }
    xsum = block_sum(gsum, ds);                   // has a barrier
  }
  if (one_wave) {
    if (wave == 0) {
      double ts = lane < tpr ? task_term(pl) : 0.0;
      const double ts_bonus = ts;
      if (point && lane == xtask) ts = xsum;
      double incl = wave_incl_scan(ts, lane);
      double tot = lane_value(incl, 63);
      const bool empty = point && !(tot > 0.0);
      if (empty) {   // draw from p: the x-task's own sum again
        ts = ts_bonus;
        incl = wave_incl_scan(ts, lane);
        tot = lane_value(incl, 63);
      }
      if (lane < tpr) task_sum[lane] = ts;
      const double tt = (double)u_final * tot;
      const uint64_t hit = __ballot(lane < tpr && incl > tt);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        const double p_excl = l == 0 ? 0.0 : lane_value(incl, l - 1);
        if (lane == 0) {
          ds.tau = l;
          ds.p_excl = p_excl;
        }
      } else {
        find_interval(task_sum, tpr, tt, lane, ds);   // t past the rounded total, or no mass
      }
      if (lane == 0) {
        ds.total = tot;
        ds.empty = empty ? 1 : 0;
        ds.tt = tt;
      }
    }
    __syncthreads();
    if (ds.empty) {
      // empty residual (invalid input or extreme rounding): draw from p
      fbad |= SPEC_VERIFY_DEV_EMPTY_RESIDUAL;
      dc.residual = kDrawBonus;
    }
  } else {
    __syncthreads();
    double xtask_bonus = 0.0;
    if (point && tid == 0) {
      xtask_bonus = task_sum[xtask];
      task_sum[xtask] = xsum;
    }
    __syncthreads();
    if (wave == 0) {
      const double tot = wave_total(task_sum, tpr, lane);
      if (lane == 0) {
        ds.total = tot;
        ds.empty = point && !(tot > 0.0);
      }
    }
    __syncthreads();
    if (ds.empty) {
      // empty residual (invalid input or extreme rounding): draw from p
      fbad |= SPEC_VERIFY_DEV_EMPTY_RESIDUAL;
      dc.residual = kDrawBonus;
      if (tid == 0) task_sum[xtask] = xtask_bonus;
      __syncthreads();
      if (wave == 0) {
        const double tot = wave_total(task_sum, tpr, lane);
        if (lane == 0) ds.total = tot;
      }
      __syncthreads();
    }
    if (wave == 0) {
      const double tt = (double)u_final * ds.total;
      find_interval(task_sum, tpr, tt, lane, ds);
      if (lane == 0) ds.tt = tt;
    }
    __syncthreads();
  }
  total = ds.total;
  const int64_t tau = ds.tau;
  if (tau < 0) return -1;                      // no mass at all (invalid row)
  if (tau != early) {
    gi = tau * kTaskGroups + tid;
    if (active) load_group<DT, VEC>(prow, gi, V, rp);
  }
  const double tt = ds.tt, p_excl = ds.p_excl;
  __syncthreads();                             // ds.wave_tot etc. are reused
  return block_search<DT>(rp, rp, gi, active, dc, ec, tt, p_excl, ds);
}

// ---------------------------------------------------------------- residual tiles

constexpr int kTileTerms = 4;                 // W, Q, R0, B per tile
constexpr double kBand = 0x1p-20;             // |g* - g| / max(1, |g|) the first-order move covers
constexpr double kCorrectionTol = 0x1p-24;    // error bound allowed, relative to W
constexpr double kResidualFloor = 0x1p-60;    // residual mass the fp32 terms resolve

// The residual tile pass over tiles [t_lo, t_hi) of one row pair, by the
// calling workgroup: wave w takes tile t_lo + w first, then the next
// unclaimed tile from the LDS counter *next (cleared by the caller).  Waves
// progress at different rates (two share a SIMD), and a static round-robin
// left the last wave of a workgroup ~4.6 us behind its first.  A tile is
// 2048 logits: 256 consecutive groups, lane l holding groups l, l+64, l+128,
// l+192 (each 16-byte load instruction covers 1 KB of contiguous logits).
// For every tile, emit(t, v) is called by all lanes of the wave with the
// tile's sums v = {W, Q, R0, B} (double, equal in every lane); a tile's sums
// do not depend on the wave that computes them.  W and R0 cross the lanes in
// double (the draw and the exact ratio need them to the elements'
// precision); Q (the slope of the first-order move, ~1e-7 of W at most) and
// B (an error bound) in float.
// The four per-lane sums of one tile from its raw groups (see residual_tiles).
template <int DT>
__device__ __forceinline__ void tile_terms(const GroupRaw<DT> cp[kTileGroupsPerLane],
                                           const GroupRaw<DT> cq[kTileGroupsPerLane],
                                           const DrawConsts& dc, const ExpConsts& ec, float band,
                                           float& sw, float& sq, float& sr, float& sb) {
  // every sum starts from its first term, not from 0 + term (an addition
  // the compiler must keep, for the sign of a zero term)
#pragma unroll
  for (int j = 0; j < kTileGroupsPerLane; ++j) {
    float lp[kGroup], lq[kGroup];
    unpack<DT>(cp[j], lp);
    unpack<DT>(cq[j], lq);
    float gw, gq, gr, gb;
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const ResidualTerm r = residual_term(lp[k], lq[k], dc, ec);
      const float q = r.wu > 0.0f ? r.qs : 0.0f;
      // how far inside the band the element lies: the most its weight
      // can leave the first-order move for any |g* - g| <= band
      const float bk = __builtin_fmaxf(__builtin_fmaf(band, r.qs, -__builtin_fabsf(r.wu)), 0.0f);
      if (k == 0) {
        gw = r.w; gr = r.r0; gq = q; gb = bk;
      } else {
        gw += r.w; gr += r.r0; gq += q; gb += bk;
      }
    }
    if (j == 0) {
      sw = gw; sq = gq; sr = gr; sb = gb;
    } else {
      sw += gw; sq += gq; sr += gr; sb += gb;
    }
  }
}

template <int DT, bool VEC, typename Emit>
__device__ __forceinline__ void residual_tiles(const void* prow, const void* qrow, int64_t V,
                                               int64_t t_lo, int64_t t_hi, const DrawConsts& dc,
                                               const ExpConsts& ec, int* next, Emit emit) {
  const int lane = threadIdx.x & 63;
  // t is wave-uniform and kept in scalar registers, so that the test for a
  // whole tile below is a branch of the wave, not of its lanes
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the band scales with g: g's own rounding error is relative
  const float band = (float)kBand * __builtin_fmaxf(1.0f, __builtin_fabsf(dc.g));
  for (int64_t t = t_lo + wave; t < t_hi;) {
    GroupRaw<DT> cp[kTileGroupsPerLane], cq[kTileGroupsPerLane];
    float sw, sq, sr, sb;
    if (VEC && (t + 1) * kTileElems <= V) {
      // a whole tile: the two rows' loads alternate group by group, and the
      // arithmetic of a group waits only for that group's two loads (a
      // shared path with the ragged loads below waits for all eight)
      const int64_t g0 = t * kTileGroups + lane;
#pragma unroll
      for (int j = 0; j < kTileGroupsPerLane; ++j) {
        load_full_nt<DT>(prow, (g0 + j * 64) * kGroup, cp[j]);
        load_full_nt<DT>(qrow, (g0 + j * 64) * kGroup, cq[j]);
      }
      tile_terms<DT>(cp, cq, dc, ec, band, sw, sq, sr, sb);
      // keeps the compiler from merging this copy of the arithmetic with the
      // ragged path's below, which would bring back the wait for all loads
      __builtin_amdgcn_sched_barrier(0);
    } else {
      load_tile<DT, VEC>(prow, t, V, lane, cp);
      load_tile<DT, VEC>(qrow, t, V, lane, cq);
      tile_terms<DT>(cp, cq, dc, ec, band, sw, sq, sr, sb);
    }
    double v[kTileTerms];
    v[0] = wave_xor_sum((double)sw);
    v[1] = (double)wave_xor_sum(sq);
    v[2] = wave_xor_sum((double)sr);
    v[3] = (double)wave_xor_sum(sb);
    emit(t, v);
    int claimed = 0;
    if (lane == 0) claimed = atomicAdd(next, 1);
    t = t_lo + kWaves + (int64_t)__builtin_amdgcn_readfirstlane(claimed);
  }
}

// ---------------------------------------------------------------- finishing

// Draft-distribution modes of the finishing kernel.
//   kDraftLogits: q_i = softmax(draft logits / T) ([A] 1.2, [D] 2.2).
//   kDraftPoint : the draft proposes tokens without a distribution (n-gram /
//                 prompt-lookup drafting, [A] 1.4 and 3.3, [D] 4.1), so
//                 q_i is the point mass at x_i: the test is u < p(x), and
//                 a rejection draws from max(0, p - delta_x), i.e. p with
//                 x removed.  No draft row is read.
constexpr int kDraftLogits = 0;
constexpr int kDraftPoint = 1;

// G workgroups per sequence (blockIdx = b * G + g).  The row partials come
// from row_stats_kernel, which ran before on the same stream: target row r
// owns partials [r * tpr, +tpr), draft row d owns
// [(target_rows + d) * tpr, +tpr) (kDraftLogits only).
template <int DT, bool VEC, bool CHECK, int MODE>
__global__ __launch_bounds__(kThreads) void finish_kernel(
    const void* __restrict__ target, const void* __restrict__ draft, int64_t ld, int64_t V,
    int64_t target_rows, int64_t draft_rows, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, ExpConsts ec,
    const Partial* __restrict__ part, int64_t tpr, int combine_lanes, int64_t num_tiles,
    int G, double* __restrict__ tile_sums, uint32_t* __restrict__ counters,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_num_accepted,
    float* __restrict__ out_p, float* __restrict__ out_q, float* __restrict__ out_residual,
    uint32_t* __restrict__ status) {
  __shared__ SeqShared sh;
  extern __shared__ double tile_sum[];   // [kTileTerms * num_tiles]: tile sums, task sums
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t b = (int64_t)blockIdx.x / G;
  const int g = (int)((int64_t)blockIdx.x - b * G);

  // ---- sequence geometry, guarded so bad offsets never index out of bounds
  const int64_t c0 = cu[b], c1 = cu[b + 1];
  const int64_t gamma = c1 - c0;
  const int64_t trow0 = c0 + b, drow0 = c0;
  if (!(c0 >= 0 && gamma >= 0 && c1 <= draft_rows && trow0 + gamma < target_rows)) {
    if (g == 0) {
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
  const float u_final = uniforms[trow0 + gamma];   // issued early, used at the end
  // global partial-table rows of this sequence's target row j and draft row j
  const int64_t prow_t0 = trow0, prow_d0 = target_rows + drow0;
  if (tid == 0) {
    sh.bad = 0;
    sh.n = (int)gamma;
    sh.skip = 0;
    sh.tile_next = 0;
  }
  __syncthreads();

  // ================= the last workgroup of the sequence finishes it

  // ---- accept tests in windows of 64 positions; stop at the first
  // rejection ([D] 2.1).  The window holding n also holds the normalisers
  // of the final-draw rows (target rows run to gamma, one past the drafts).
  const int L = combine_lanes;
  const int rows_per_wave = 64 / L;
  int64_t lo = 0;
  int64_t n = gamma;
  for (;; lo += 64) {
    const int64_t hi_t = lo + 64 < gamma + 1 ? lo + 64 : gamma + 1;
    const int64_t hi_d = lo + 64 < gamma ? lo + 64 : gamma;   // draft positions
    // wave 0 gathers the logits at the draft tokens first; their latency
    // overlaps the combine below
    int32_t x = -1;
    float lpx = 0.0f, lqx = 0.0f, u = 0.0f;
    const int64_t i_me = lo + lane;
    if (wave == 0 && i_me < hi_d) {
      x = tokens[drow0 + i_me];
      u = uniforms[trow0 + i_me];
      if (x >= 0 && x < V) {
        lpx = load_logit<DT>(row_ptr<DT>(target, trow0 + i_me, ld), x);
        if (MODE == kDraftLogits) lqx = load_logit<DT>(row_ptr<DT>(draft, drow0 + i_me, ld), x);
      }
    }
    // combine: rows of this window, rows_per_wave at a time per wave
    const int64_t nt = hi_t - lo, nd = MODE == kDraftLogits ? hi_d - lo : 0;
    auto store_row = [&](int64_t r, bool active, const RowNorm& rn) {
      if (active && (lane & (L - 1)) == 0) {
        const bool is_t = r < nt;
        const int64_t i = is_t ? r : r - nt;
        sh.M[is_t ? 0 : 1][i] = rn.M;
        sh.s[is_t ? 0 : 1][i] = rn.s;
      }
    };
    auto table_row = [&](int64_t r) -> int64_t {
      return r < nt ? prow_t0 + lo + r : prow_d0 + lo + (r - nt);
    };
    // waves 1..7 combine (wave 0's loads wait on the draft tokens, so it
    // would join the combine late)
    const int cwave = wave - 1;
    const int64_t stride = (int64_t)(kWaves - 1) * rows_per_wave;
    if (wave == 0) {
      // the tokens, uniforms and logits above
    } else if (tpr <= L) {
      // one partial per lane; two passes' loads are issued before either
      // is reduced (with 32 lanes per row one iteration covers 28 rows,
      // gamma up to 13)
      for (int64_t r0 = (int64_t)cwave * rows_per_wave; r0 < nt + nd; r0 += 2 * stride) {
        const int64_t ra = r0 + lane / L, rb = ra + stride;
        const bool act_a = (lane / L) < rows_per_wave && ra < nt + nd;
        const bool act_b = (lane / L) < rows_per_wave && rb < nt + nd;
        const Partial pa = load_partial(part, tpr, act_a ? table_row(ra) : 0, lane & (L - 1), act_a);
        const Partial pb = load_partial(part, tpr, act_b ? table_row(rb) : 0, lane & (L - 1), act_b);
        store_row(ra, act_a, reduce_partials(pa, L, ec));
        store_row(rb, act_b, reduce_partials(pb, L, ec));
      }
    } else {
      for (int64_t r0 = (int64_t)cwave * rows_per_wave; r0 < nt + nd; r0 += stride) {
        const int64_t r = r0 + lane / L;
        const bool active = (lane / L) < rows_per_wave && r < nt + nd;
        store_row(r, active, combine_rows_packed(part, tpr, L, active ? table_row(r) : 0,
                                                 active, ec, lane));
      }
    }
    __syncthreads();
    if (wave == 0) {
      bool reject = false, badtok = false;
      uint32_t wbad = 0;
      float p_out = 0.0f, q_out = 0.0f;
      if (i_me < hi_d) {
        double r = 0.0;
        if (x < 0 || x >= V) {
          badtok = true;
        } else if (MODE == kDraftPoint) {
          const double Mp = sh.M[0][lane], sp = sh.s[0][lane];
          // r = p_i(x) / 1
          r = exp(((double)lpx - Mp) / ec.T) / sp;
          p_out = (float)r;
          q_out = 1.0f;
          if (CHECK && Mp == -INFINITY) wbad |= SPEC_VERIFY_DEV_EMPTY_ROW;
        } else {
          const double Mp = sh.M[0][lane], Mq = sh.M[1][lane];
          const double sp = sh.s[0][lane], sq = sh.s[1][lane];
          // p_i(x) = exp((l_x - M)/T) / s with s = sum_k exp((l_k - M)/T)
          const double pp = exp(((double)lpx - Mp) / ec.T) / sp;
          const double qq = exp(((double)lqx - Mq) / ec.T) / sq;
          r = exp((((double)lpx - Mp) - ((double)lqx - Mq)) / ec.T) * (sq / sp);
          p_out = (float)pp;
          q_out = (float)qq;
          if (CHECK) {
            if (!(qq > 0.0)) wbad |= SPEC_VERIFY_DEV_ZERO_Q;
            if (Mp == -INFINITY || Mq == -INFINITY) wbad |= SPEC_VERIFY_DEV_EMPTY_ROW;
          }
        }
        if (CHECK && !(u >= 0.0f && u < 1.0f)) wbad |= SPEC_VERIFY_DEV_BAD_UNIFORM;
        // accept iff u < r ([A] 1.2 step 3 with the strict reading)
        reject = !((double)u < r);
      }
      const uint64_t mask = __ballot(reject);
      const uint64_t btok = __ballot(badtok);
      // p and q go out after the test: loads and stores share one counter,
      // so a store issued before u's first use makes the wave wait for the
      // store's round trip there (the scheduling barrier keeps the compiler
      // from moving the stores above the ballots)
      __builtin_amdgcn_sched_barrier(0);
      if (g == 0 && i_me < hi_d && !badtok) {
        if (out_p) out_p[drow0 + i_me] = p_out;
        if (out_q) out_q[drow0 + i_me] = q_out;
      }
      wbad = wave_or(wbad);
      sh.x[lane] = x;
      if (lane == 0) {
        sh.bad |= wbad;
        if (btok) sh.skip = 1;
        else if (mask) sh.n = (int)(lo + __builtin_ctzll(mask));
      }
    }
    __syncthreads();
    n = sh.n;
    if (sh.skip || n < gamma || lo + 64 > gamma) break;
    __syncthreads();   // the next window overwrites sh.M / sh.s
  }
  if (sh.skip) {       // a draft token outside [0, V): the sequence is skipped
    if (g == 0) {
      for (int64_t i = tid; i <= gamma; i += kThreads) out_tokens[trow0 + i] = -1;
      if (tid == 0) {
        out_num_accepted[b] = 0;
        if (out_residual) out_residual[b] = 0.0f;
        status_or(status, sh.bad | SPEC_VERIFY_DEV_BAD_TOKEN);
      }
    }
    return;
  }

  // ---- emit the accepted prefix ([B] 流程编排: keep the drafts before the
  // first mismatch); slot n is written by the draw below.  n lies in the
  // last window [lo, lo + 64), whose drafts are in LDS; drafts of earlier
  // windows (gamma > 64 only) are read again.  Two loops, so that neither
  // reads through a pointer that may be LDS or global memory (a generic
  // load would make the stores wait for every store issued before them).
  if (g == 0) {
    for (int64_t i = tid; i < lo; i += kThreads) out_tokens[trow0 + i] = tokens[drow0 + i];
    for (int64_t i = lo + tid; i <= gamma; i += kThreads) {
      if (i < n) out_tokens[trow0 + i] = sh.x[i - lo];
      else if (i > n) out_tokens[trow0 + i] = -1;
    }
    if (tid == 0) out_num_accepted[b] = (int32_t)n;
  }
  // p/q at positions beyond the window that stopped the test
  if (g == 0 && (out_p || out_q)) {
    for (int64_t i = lo + 64 + wave; i < gamma; i += kWaves) {
      const int32_t xi = tokens[drow0 + i];
      if (xi < 0 || xi >= V) continue;
      const RowNorm rp = combine_rows_packed(part, tpr, 64, prow_t0 + i, true, ec, lane);
      if (lane == 0) {
        const double lp = load_logit<DT>(row_ptr<DT>(target, trow0 + i, ld), xi);
        if (out_p) out_p[drow0 + i] = (float)(exp((lp - (double)rp.M) / ec.T) / rp.s);
      }
      if (MODE == kDraftPoint) {
        if (lane == 0 && out_q) out_q[drow0 + i] = 1.0f;
        continue;
      }
      const RowNorm rq = combine_rows_packed(part, tpr, 64, prow_d0 + i, true, ec, lane);
      if (lane == 0) {
        const double lq = load_logit<DT>(row_ptr<DT>(draft, drow0 + i, ld), xi);
        if (out_q) out_q[drow0 + i] = (float)(exp((lq - (double)rq.M) / ec.T) / rq.s);
      }
    }
  }

  // ---- final draw ([A] 1.2 step 3, [D] 2.2), in the common scale s_p 2^Kp:
  // the residual at n, or the bonus from the last target row.
  const int residual = n < gamma ? 1 : 0;
  // Only a residual against draft logits needs a second pass over its rows;
  // bonus draws and point-mass residuals draw from the row-pass task sums.
  const bool tile_pass = MODE == kDraftLogits && residual;
  const void* prow = row_ptr<DT>(target, trow0 + n, ld);
  const void* qrow = tile_pass ? row_ptr<DT>(draft, drow0 + n, ld) : prow;
  const float Mp = sh.M[0][n - lo];
  const double sp = sh.s[0][n - lo];
  DrawConsts dc;
  dc.residual = !residual ? kDrawBonus : (MODE == kDraftPoint ? kDrawPoint : kDrawResidual);
  dc.x = (MODE == kDraftPoint && residual) ? (int64_t)sh.x[n - lo] : -1;
  dc.Ap = shift_of(Mp, ec);
  const double Kp = offset_of(Mp, dc.Ap, ec);
  const double unit = sp * exp2(Kp);   // the weights' scale: sum of e_p
  dc.Aq = 0.0f;
  dc.dK = 0.0f;
  dc.dM = 0.0f;
  dc.g = 0.0f;
  if (tile_pass) {
    const float Mq = sh.M[1][n - lo];
    const double sq = sh.s[1][n - lo];
    dc.Aq = shift_of(Mq, ec);
    dc.dK = (float)(Kp - offset_of(Mq, dc.Aq, ec));
    dc.dM = Mp - Mq;
    dc.g = (float)((sq - sp) / sq);    // 1 - s_p / s_q from the row pass
  }
  __shared__ DrawShared ds;
  uint32_t fbad = sh.bad;
  double total = 0.0;
  int64_t token = -1;

  if (!tile_pass) {
    if (g != 0) return;                  // one workgroup draws from the task sums
    token = draw_from_task_sums<DT, VEC>(part + (prow_t0 + n) * tpr, tpr, prow, V, dc, ec,
                                         u_final, tile_sum, ds, fbad, total);
  } else {
    // ---- the residual's tile pass.  Tile sums of this workgroup's share:
    // per tile the weights W (with the row pass's g), the draft terms Q over
    // the support (dW/dg), the C-free difference R0 and the band bound
    // B = sum max(0, band qs - |wu|) (band = 2^-20 max(1, |g|)).  Sums of a
    // lane's 32 elements are fp32.  Tile arrays, in LDS:
    // W at tile_sum[0, nt), Q at [nt, 2 nt), R0 at [2 nt, 3 nt), B at
    // [3 nt, 4 nt).
    const int64_t nt = num_tiles;
    const int64_t per = (nt + G - 1) / G;
    const int64_t t_lo = (int64_t)g * per;
    const int64_t t_hi = t_lo + per < nt ? t_lo + per : nt;
    double* ts_seq = tile_sums + b * nt * kTileTerms;
    residual_tiles<DT, VEC>(prow, qrow, V, t_lo, t_hi, dc, ec, &sh.tile_next,
                            [&](int64_t t, const double v[kTileTerms]) {
      // lane k < 4 stores term k (selected, not indexed: v stays in registers)
      const double vk = lane == 0 ? v[0] : lane == 1 ? v[1] : lane == 2 ? v[2] : v[3];
      if (lane < kTileTerms) {
        if (G == 1) tile_sum[lane * nt + t] = vk;
        else __hip_atomic_store(&ts_seq[t * kTileTerms + lane], vk, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
      }
    });
    // ---- arrival: with G > 1 the tile sums cross workgroups.  They were
    // written with agent-scope atomic stores, which on gfx950 write through
    // the XCD's L2 to the device-coherent level; each wave waits for their
    // acknowledgement (s_waitcnt) before the barrier, then one thread counts
    // the workgroup in with a relaxed agent-scope atomic add, which is
    // issued only after every store of the workgroup is acknowledged.  The
    // last of the G workgroups sees the count G - 1 and only then issues
    // agent-scope atomic loads, which read the device-coherent level rather
    // than its own L2.  This relies on that gfx950 behaviour (stores
    // acknowledged at the coherent level before the count, loads issued
    // after the count returns) instead of an agent-scope release / acquire
    // pair, whose L2 write-back and invalidate made the kernel several
    // times slower with hundreds of workgroups.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (G > 1) {
      if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&counters[b], 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        ds.last_wg = (old == (uint32_t)(G - 1)) ? 1 : 0;
      }
      __syncthreads();
      if (!ds.last_wg) return;
      // the last workgroup copies the tile sums into its LDS (a row of at
      // most 64 tiles: wave 0 loads them into registers below)
      if (nt > 64) {
        for (int64_t i = tid; i < nt * kTileTerms; i += kThreads) {
          const int64_t t = i / kTileTerms, k = i - t * kTileTerms;
          tile_sum[k * nt + t] =
              __hip_atomic_load(&ts_seq[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
      }
    }
    // ---- the exact normaliser ratio.  R0 = s_p' - s_q' (both in the
    // weights' scale) comes from per-element differences, so it is exact to
    // the rounding of those differences, while the row pass's s_p / s_q is
    // exact only to its sums' rounding (~1e-8): g* = 1 - s_p' / s_q' =
    // -R0 / (s_p' - R0).  W is linear in g for a fixed support, so the tile
    // sums move by dg Q (dg = g* - g).  An element that changes side is off
    // by |dg| qs - |wu| at most; max(0, x qs - |wu|) is convex in x and 0 at
    // x = 0, so for |dg| <= band the total error is at most (|dg| / band) B.
    // The four totals are scans in a fixed order (wave_total's).  Then,
    // with the move certified, the moved tile sums are scanned for the tile
    // holding t = u * S; an empty residual (invalid input or extreme
    // rounding) falls back to a draw from p_n through the task sums.
    const double band = kBand * __builtin_fmax(1.0, __builtin_fabs((double)dc.g));
    // from the four totals: g*, the move dg and whether it is certified,
    // also left in ds (lane 0) for the other waves
    auto certify = [&](double W, double Q, double R0, double B, double& dg) -> bool {
      const float g_star = (float)(-R0 / (unit - R0));
      dg = (double)g_star - (double)dc.g;
      const double w_star = W + dg * Q;
      const bool ok = w_star > 0.0 && __builtin_fabs(dg) <= band &&
                      2.0 * (__builtin_fabs(dg) / band) * B <= kCorrectionTol * w_star;
      if (lane == 0) {
        ds.g_star = g_star;
        ds.dg = dg;
        ds.linear_ok = ok ? 1 : 0;
      }
      return ok;
    };
    bool scanned = false;
    if (nt <= 64) {
      // One wave holds every tile (lane t: tile t) and does the totals, the
      // move and the scan in registers, without a workgroup barrier.
      if (wave == 0) {
        double v[kTileTerms] = {0.0, 0.0, 0.0, 0.0};
        if (lane < nt) {
#pragma unroll
          for (int k = 0; k < kTileTerms; ++k)
            v[k] = G > 1 ? __hip_atomic_load(&ts_seq[lane * kTileTerms + k], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)
                         : tile_sum[k * nt + lane];
        }
        double tot[kTileTerms];
#pragma unroll
        for (int k = 0; k < kTileTerms; ++k) tot[k] = lane_value(wave_incl_scan(v[k], lane), 63);
        double dg;
        if (certify(tot[0], tot[1], tot[2], tot[3], dg)) {
          double c = v[0] + dg * v[1];
          c = c > 0.0 ? c : 0.0;
          if (lane < nt) tile_sum[lane] = c;
          const double incl = wave_incl_scan(c, lane);
          const double sum = lane_value(incl, 63);
          double tt = 0.0;
          if (sum > 0.0) {
            tt = (double)u_final * sum;
            const uint64_t hit = __ballot(lane < nt && incl > tt);
            if (hit) {
              const int l = __builtin_ctzll(hit);
              const double p_excl = l == 0 ? 0.0 : lane_value(incl, l - 1);
              if (lane == 0) {
                ds.tau = l;
                ds.p_excl = p_excl;
              }
            } else {
              find_interval(tile_sum, nt, tt, lane, ds);   // t past the rounded total
            }
          }
          if (lane == 0) {
            ds.total = sum;
            ds.tt = tt;
          }
        }
      }
      __syncthreads();
      scanned = ds.linear_ok != 0;
    } else {
      if (wave < kTileTerms) {
        const double tot = wave_total(tile_sum + wave * nt, nt, lane);
        if (lane == 0) ds.red[wave] = tot;
      }
      __syncthreads();
      if (wave == 0) {
        double dg;
        certify(ds.red[0], ds.red[1], ds.red[2], ds.red[3], dg);
      }
      __syncthreads();
      if (ds.linear_ok) {
        const double dg = ds.dg;
        for (int64_t t = tid; t < nt; t += kThreads) {
          const double c = tile_sum[t] + dg * tile_sum[nt + t];
          tile_sum[t] = c > 0.0 ? c : 0.0;
        }
      }
    }
    dc.g = ds.g_star;                  // the search below uses g*
    if (!scanned) {
      if (!ds.linear_ok) {
        // the support moves with g: this workgroup passes over both rows
        // again with g* (rare: rows that agree to the row pass's rounding)
        if (tid == 0) sh.tile_next = 0;
        __syncthreads();
        residual_tiles<DT, VEC>(prow, qrow, V, 0, nt, dc, ec, &sh.tile_next,
                                [&](int64_t t, const double v[kTileTerms]) {
          if (lane == 0) tile_sum[t] = v[0];
        });
      }
      __syncthreads();
      if (wave == 0) {
        double tt = 0.0;
        total = wave_total(tile_sum, nt, lane);
        if (total > 0.0) {
          tt = (double)u_final * total;
          find_interval(tile_sum, nt, tt, lane, ds);
        }
        if (lane == 0) {
          ds.total = total;
          ds.tt = tt;
        }
      }
      __syncthreads();
    }
    total = ds.total;
    if (!(total > 0.0)) {
      fbad |= SPEC_VERIFY_DEV_EMPTY_RESIDUAL;
      DrawConsts dd = dc;
      dd.residual = kDrawBonus;
      __syncthreads();   // ds is reused
      double ptotal = 0.0;
      token = draw_from_task_sums<DT, VEC>(part + (prow_t0 + n) * tpr, tpr, prow, V, dd, ec,
                                           u_final, tile_sum, ds, fbad, ptotal);
    } else {
      // below 2^-60 of the unit mass, underflowed fp32 terms (< 2^-126 each)
      // could be a measurable share of the residual
      if (total < kResidualFloor * unit) fbad |= SPEC_VERIFY_DEV_RESIDUAL_UNRESOLVED;
      // ---- re-scan tile tau: thread t < 256 holds group tau*256 + t
      const int64_t tau = ds.tau;
      GroupRaw<DT> rp, rq;
      const bool active = tid < kTileGroups;
      const int64_t gi = tau * kTileGroups + tid;
      if (active) {
        load_group<DT, VEC>(prow, gi, V, rp);
        load_group<DT, VEC>(qrow, gi, V, rq);
      }
      token = block_search<DT>(rp, rq, gi, active, dc, ec, ds.tt, ds.p_excl, ds);
    }
  }
  if (tid == 0) {
    out_tokens[trow0 + n] = (int32_t)token;
    if (out_residual)
      out_residual[b] = (residual && !(fbad & SPEC_VERIFY_DEV_EMPTY_RESIDUAL))
                            ? (float)(total / unit)
                            : 0.0f;
    status_or(status, fbad);
  }
}

}  // namespace sv
