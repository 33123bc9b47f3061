// tree_kernels.hpp -- gfx950 device code of tree verification (included
// once, by spec_verify.hip, after spec_verify_kernels.hpp and
// greedy_kernels.hpp).
//
// Pages cited (by title and section):
//   [D] "大模型推理加速新范式：推测解码（Speculative Decoding）原理剖析与
//       vLLM生产级实现", section 3.2 (Tree Attention): the drafter proposes
//       its top candidates at each position, forming a tree, and the target
//       scores every node in one pass.  The page gives no acceptance rule.
//   [B] the blog.hotdry.top post on speculative decoding and dynamic
//       batching, item 流程编排: compare with the target's choice, keep the
//       matching prefix.
//   [A] "推测解码与连续批处理深度实战：突破自回归生成的双重瓶颈", section 1.2
//       step 3: accept with min(1, p/q), resample from clip(p - q, 0).
//
// Readings (the same as the oracle's): greedy trees move to the lowest-index
// child whose token is the current node's argmax and emit that argmax where
// none matches.  Point-mass candidates (top-k proposals without a
// distribution): the children of the current node are tried in index order;
// child c is accepted with probability p'(x_c), p' being the node's p with
// the tokens of already rejected siblings removed and renormalised (a token
// already rejected has p' = 0); when every child is rejected, or at a node
// without children, the final token is drawn from p'.
//
// Layout: sequence b owns nodes g = cu[b] + n, n < N_b; node 0 is the root;
// parent[g] is a local index below n; target row g scores the token after
// node n; uniforms[g] is node n's test and the root's slot the final draw.
//
// Both kernels run after a row pass over the R node rows (argmax_kernel or
// row_stats_kernel) and use one workgroup per sequence: the tree's nodes go
// to LDS, every row's statistic is combined at once, then one wave walks the
// tree from the root.  The point kernel needs, at a node whose children are
// tested, the exact mass of the node's row without its children's tokens:
// the row pass's task sums moved into one scale, and the tasks that hold a
// child token summed again without those tokens (never by subtraction).
// Every sibling after the first, and the final draw, use those sums.  Small
// trees gather them for every internal node in one round of loads before the
// walk; larger trees gather the current node at each level.
#pragma once

namespace sv {

constexpr int kMaxTreeNodes = 1024;
constexpr int kMaxChildren = 64;

struct TreeNodes {
  int32_t par[kMaxTreeNodes];
  int32_t tok[kMaxTreeNodes];
  int32_t nkids[kMaxTreeNodes];
  int32_t path[kMaxTreeNodes];
  int bad;
  int depth;
};

// Load sequence b's nodes into LDS and check them: 0 <= parent < n and
// 0 <= token < V for every non-root node, at most kMaxChildren children per
// node.  tn.bad != 0 afterwards marks a malformed tree.
template <int NT>
__device__ __forceinline__ void load_tree(const int32_t* __restrict__ parent,
                                          const int32_t* __restrict__ tokens, int64_t g0,
                                          int64_t N, int64_t V, TreeNodes& tn) {
  const int tid = threadIdx.x;
  for (int64_t n = tid; n < N; n += NT) tn.nkids[n] = 0;
  if (tid == 0) tn.bad = 0;
  __syncthreads();
  for (int64_t n = tid; n < N; n += NT) {
    const int32_t p = n == 0 ? -1 : parent[g0 + n];
    const int32_t t = n == 0 ? 0 : tokens[g0 + n];
    const bool ok = n == 0 || (p >= 0 && p < n && t >= 0 && t < V);
    tn.par[n] = ok ? p : -1;
    tn.tok[n] = ok ? t : 0;
    if (!ok) tn.bad = 1;
    else if (n > 0) atomicAdd(&tn.nkids[p], 1);
  }
  __syncthreads();
  for (int64_t n = tid; n < N; n += NT)
    if (tn.nkids[n] > kMaxChildren) tn.bad = 1;
  __syncthreads();
}

// Outputs of sequence b from the walk held in LDS: slot n < depth holds the
// n-th accepted node's token and index, slot depth the final token, later
// slots -1.  Every slot is written once.
template <int NT>
__device__ __forceinline__ void write_tree_outputs(const TreeNodes& tn, int64_t g0, int64_t N,
                                                   int32_t final_tok, int32_t* out_tokens,
                                                   int32_t* out_path) {
  const int depth = tn.depth;
  for (int64_t n = threadIdx.x; n < N; n += NT) {
    out_tokens[g0 + n] = n < depth ? tn.tok[tn.path[n]] : (n == depth ? final_tok : -1);
    out_path[g0 + n] = n < depth ? tn.path[n] : -1;
  }
}

// A malformed or out-of-range sequence: -1 outputs (when its slots are in
// range), 0 accepted, a status bit.
template <int NT>
__device__ __forceinline__ void reject_tree(int64_t b, int64_t g0, int64_t N, bool slots_ok,
                                            uint32_t bit, int32_t* out_tokens,
                                            int32_t* out_path, int32_t* out_num_accepted,
                                            uint32_t* status) {
  if (slots_ok)
    for (int64_t n = threadIdx.x; n < N; n += NT) {
      out_tokens[g0 + n] = -1;
      out_path[g0 + n] = -1;
    }
  if (threadIdx.x == 0) {
    out_num_accepted[b] = 0;
    status_or(status, bit);
  }
}

// ---------------------------------------------------------------- greedy

struct TreeGreedyShared {
  TreeNodes tn;
  int32_t amax[kMaxTreeNodes];
};

__global__ __launch_bounds__(kGreedyThreads) void tree_greedy_kernel(
    int64_t V, int64_t R, const int32_t* __restrict__ cu, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ tokens, const ArgPartial* __restrict__ part, int64_t tpr,
    int combine_lanes, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_path,
    int32_t* __restrict__ out_num_accepted, uint32_t* __restrict__ status) {
  __shared__ TreeGreedyShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t b = blockIdx.x;
  const int64_t g0 = cu[b], g1 = cu[b + 1];
  const int64_t N = g1 - g0;
  const bool slots_ok = g0 >= 0 && N >= 1 && g1 <= R;
  if (!slots_ok || N > kMaxTreeNodes) {
    reject_tree<kGreedyThreads>(b, g0, N, slots_ok,
                                slots_ok ? SPEC_VERIFY_DEV_BAD_TREE : SPEC_VERIFY_DEV_BAD_OFFSETS,
                                out_tokens, out_path, out_num_accepted, status);
    return;
  }
  load_tree<kGreedyThreads>(parent, tokens, g0, N, V, sh.tn);
  if (sh.tn.bad) {
    reject_tree<kGreedyThreads>(b, g0, N, true, SPEC_VERIFY_DEV_BAD_TREE, out_tokens, out_path,
                                out_num_accepted, status);
    return;
  }
  // the argmax of every node's row
  const int L = combine_lanes;
  const int rows_per_wave = 64 / L;
  for (int64_t r0 = (int64_t)wave * rows_per_wave; r0 < N;
       r0 += (int64_t)kGreedyWaves * rows_per_wave) {
    const int64_t r = r0 + lane / L;
    const bool active = (lane / L) < rows_per_wave && r < N;
    const int64_t k = combine_argmax(part, tpr, L, active ? g0 + r : 0, active, lane);
    if (active && (lane & (L - 1)) == 0) sh.amax[r] = (int32_t)k;
  }
  __syncthreads();
  // one wave walks: the lowest-index child holding the argmax, or stop
  __shared__ int32_t final_tok;
  if (wave == 0) {
    int64_t cur = 0;
    int depth = 0;
    for (;;) {
      const int32_t a = sh.amax[cur];
      int64_t next = -1;
      for (int64_t base = cur + 1; base < N && next < 0; base += 64) {
        const int64_t n = base + lane;
        const bool hit = n < N && sh.tn.par[n] == cur && sh.tn.tok[n] == a;
        const uint64_t m = __ballot(hit);
        if (m) next = base + __builtin_ctzll(m);
      }
      if (next < 0) {
        if (lane == 0) final_tok = a;
        break;
      }
      if (lane == 0) sh.tn.path[depth] = (int32_t)next;
      ++depth;
      cur = next;
    }
    if (lane == 0) sh.tn.depth = depth;
  }
  __syncthreads();
  write_tree_outputs<kGreedyThreads>(sh.tn, g0, N, final_tok, out_tokens, out_path);
  if (tid == 0) out_num_accepted[b] = sh.tn.depth;
}

// ---------------------------------------------------------------- point-mass candidates

// Gathered data of up to kSlots internal nodes ("slots"): each node's
// children (in index order), their distinct tokens in order of first
// occurrence with the tokens' weights in the node's draw scale, the distinct
// tasks holding those tokens with the tasks' exact sums without the tokens,
// the node's task sums, and the node's mass without its children's tokens.
// A slot's children, tokens and tasks share one range [k0, k0 + nk) of the
// flat arrays (a node has at least as many children as distinct tokens or
// tasks).  Small trees gather every internal node in one round of loads;
// larger trees gather the current node at each level of the walk.
constexpr int kSlots = 8;            // = kWaves: one wave per slot
constexpr int64_t kPrefetchNodes = 64;
constexpr int64_t kPrefetchTasksPerRow = 64;
constexpr int kPairsPerRound = 1;    // child-token tasks in flight per wave
static_assert(kSlots == kWaves, "one wave gathers one slot");

// Slots whose task sums the dynamic LDS holds for rows of tpr tasks.
__host__ __device__ inline int64_t tree_slot_rows(int64_t tpr) {
  return tpr <= kPrefetchTasksPerRow ? kSlots : 1;
}

struct TreePointShared {
  TreeNodes tn;
  float M[kMaxTreeNodes];        // row maxima
  double s[kMaxTreeNodes];       // row normalisers (exact scale)
  float lx[kMaxTreeNodes];       // logit of node n's token in its parent's row
  float u[kMaxTreeNodes];        // node n's uniform (root: the final draw)
  int32_t kids[kMaxChildren];    // children, slot by slot
  int32_t kid_jx[kMaxChildren];  // distinct-token index (in the slot) of each child's token
  int32_t kid_dup[kMaxChildren]; // the child's token appeared at an earlier child
  int32_t xs[kMaxChildren];      // distinct child tokens
  float wx[kMaxChildren];        // their weights in the node's scale
  int32_t xtask[kMaxChildren];   // distinct tasks holding them
  double xsum[kMaxChildren];     // exact sums of those tasks without the tokens
  int32_t pair[kMaxChildren];    // flat indices of the (slot, task) pairs to load
  int32_t slot_node[kSlots], slot_k0[kSlots], slot_nk[kSlots], slot_nx[kSlots], slot_nt[kSlots];
  float slot_Ap[kSlots];
  double slot_rest[kSlots];      // the node's mass without its children's tokens
  int nslots, npairs;
  int prefetch;                  // a small tree: every internal node gathered up front
  int next;                      // accepted child, or -1
  int empty;                     // the final weights summed to 0
};

// Weights of one group of row `prow` in the scale 2^(l c + Ap), zero at the
// listed tokens.
template <int DT>
__device__ __forceinline__ void group_weights_without(const GroupRaw<DT>& r, int64_t gi,
                                                      float Ap, const ExpConsts& ec,
                                                      const int32_t* excl, int nexcl,
                                                      float w[kGroup]) {
  float v[kGroup];
  unpack<DT>(r, v);
#pragma unroll
  for (int k = 0; k < kGroup; ++k) w[k] = exp_term(v[k], Ap, ec);
  // one (wave-uniform) read per listed token; only the thread whose group
  // holds it clears that weight
  const int64_t base = gi * kGroup;
  for (int i = 0; i < nexcl; ++i) {
    const int64_t d = (int64_t)excl[i] - base;
    if (d >= 0 && d < kGroup) {
#pragma unroll
      for (int k = 0; k < kGroup; ++k)
        if (k == d) w[k] = 0.0f;
    }
  }
}

// Task sum of a row-pass partial moved into the draw scale 2^(l c + Ap).
__device__ __forceinline__ double task_sum_in(const Partial& pc, float Ap, const ExpConsts& ec) {
  return pc.m == -INFINITY ? 0.0 : pc.s * exp2((double)Ap - (double)shift_of(pc.m, ec));
}

// Gather slots [0, sh.nslots) (slot_node, slot_k0 and slot_nk set): every
// wave w < nslots lists slot w's children, tokens and tasks; then all waves
// load the (slot, task) pairs, kPairsPerRound per wave per round, each task
// as one row-pass wave task (lane l holds groups l, l + 64, ..., l + 448),
// and the slots' task partials; then wave w sums slot w's mass without its
// children's tokens.  slot_ts holds kSlots * tpr doubles.  All threads call.
template <int DT, bool VEC>
__device__ __forceinline__ void gather_slots(TreePointShared& sh, double* slot_ts,
                                             const void* target, int64_t ld, int64_t V,
                                             int64_t g0, int64_t N, const ExpConsts& ec,
                                             const Partial* __restrict__ part, int64_t tpr) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ns = sh.nslots;
  if (wave < ns) {
    const int64_t node = sh.slot_node[wave];
    const int k0 = sh.slot_k0[wave];
    const float Ap = shift_of(sh.M[node], ec);
    int cnt = 0;
    for (int64_t base = node + 1; base < N; base += 64) {
      const int64_t n = base + lane;
      const bool hit = n < N && sh.tn.par[n] == node;
      const uint64_t m = __ballot(hit);
      if (hit) sh.kids[k0 + cnt + __builtin_popcountll(m & ((1ull << lane) - 1))] = (int32_t)n;
      cnt += __builtin_popcountll(m);
    }
    // distinct tokens and tasks in order of first occurrence (one child per
    // lane: a node has at most kMaxChildren = 64 children)
    const bool act = lane < cnt;
    const int32_t c = act ? sh.kids[k0 + lane] : 0;
    const int32_t x = act ? sh.tn.tok[c] : -1;
    const int32_t t = act ? (int32_t)(x / kWaveTaskElems) : -1;
    bool first_x = act, first_t = act;
    int first_lane = lane;
    for (int j = cnt - 1; j >= 0; --j) {
      const int32_t xj = (int32_t)lane_value((uint32_t)x, j);
      if (j < lane && xj == x) {
        first_x = false;
        first_lane = j;
      }
      if (j < lane && xj / (int32_t)kWaveTaskElems == t) first_t = false;
    }
    const uint64_t fx = __ballot(first_x), ft = __ballot(first_t);
    const uint64_t below = (1ull << lane) - 1;
    if (first_x) {
      const int jx = __builtin_popcountll(fx & below);
      sh.xs[k0 + jx] = x;
      sh.wx[k0 + jx] = exp_term(sh.lx[c], Ap, ec);
    }
    if (first_t) sh.xtask[k0 + __builtin_popcountll(ft & below)] = t;
    if (act) {
      sh.kid_jx[k0 + lane] = __builtin_popcountll(fx & ((1ull << first_lane) - 1));
      sh.kid_dup[k0 + lane] = first_x ? 0 : 1;
    }
    if (lane == 0) {
      sh.slot_nk[wave] = cnt;
      sh.slot_nx[wave] = __builtin_popcountll(fx);
      sh.slot_nt[wave] = __builtin_popcountll(ft);
      sh.slot_Ap[wave] = Ap;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // the (slot, task) pairs: flat index k0 + j for j < nt of each slot
    int np = 0;
    for (int sl = 0; sl < ns; ++sl) {
      const int nt = sh.slot_nt[sl], k0 = sh.slot_k0[sl];
      if (lane < nt) sh.pair[np + lane] = k0 + lane;
      np += nt;
    }
    if (lane == 0) sh.npairs = np;
  }
  __syncthreads();
  const int np = sh.npairs;
  // one round of loads: the slots' task partials (at most one per thread:
  // ns * tpr <= kThreads) and the first kPairsPerRound tasks of every wave
  // are issued before any of them is used
  static_assert(kSlots * kPrefetchTasksPerRow <= kThreads, "one slot partial per thread");
  const bool have_part = tid < (int64_t)ns * tpr;
  const int my_slot = have_part ? (int)(tid / tpr) : 0;
  Partial my_part = {-INFINITY, 0.0f, 0.0};
  if (have_part) my_part = part[(g0 + sh.slot_node[my_slot]) * tpr + (tid - my_slot * tpr)];
  for (int r0 = wave * kPairsPerRound; r0 < np; r0 += kWaves * kPairsPerRound) {
    GroupRaw<DT> raw[kPairsPerRound][kTaskGroupsPerLane];
    int slot_of[kPairsPerRound];
#pragma unroll
    for (int q = 0; q < kPairsPerRound; ++q) {
      slot_of[q] = -1;
      if (r0 + q < np) {
        const int f = sh.pair[r0 + q];
        int sl = 0;
        while (sl + 1 < ns && sh.slot_k0[sl + 1] <= f) ++sl;
        slot_of[q] = sl;
        const void* prow = row_ptr<DT>(target, g0 + sh.slot_node[sl], ld);
        load_task<DT, VEC>(prow, (int64_t)sh.xtask[f], V, lane, raw[q]);
      }
    }
    if (r0 == wave * kPairsPerRound && have_part)
      slot_ts[tid] = task_sum_in(my_part, sh.slot_Ap[my_slot], ec);
#pragma unroll
    for (int q = 0; q < kPairsPerRound; ++q) {
      if (slot_of[q] < 0) continue;
      const int sl = slot_of[q];
      const int f = sh.pair[r0 + q];
      const int k0 = sh.slot_k0[sl];
      const int64_t g_task = (int64_t)sh.xtask[f] * (kWaveTaskElems / kGroup);
      // bit 8 j + k: logit k of this lane's group j is a child token (the
      // owning lane of each token sets it)
      uint64_t excl = 0;
      const int nx = sh.slot_nx[sl];
      for (int i = 0; i < nx; ++i) {
        const int32_t x = sh.xs[k0 + i];
        const int64_t g = (int64_t)(x / kGroup) - g_task;
        if (g >= 0 && g < 64 * kTaskGroupsPerLane && (int)(g & 63) == lane)
          excl |= 1ull << ((g >> 6) * kGroup + (x % kGroup));
      }
      const float Ap = sh.slot_Ap[sl];
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < kTaskGroupsPerLane; ++j) {
        float v[kGroup], w[kGroup];
        unpack<DT>(raw[q][j], v);
#pragma unroll
        for (int k = 0; k < kGroup; ++k)
          w[k] = ((excl >> (j * kGroup + k)) & 1) ? 0.0f : exp_term(v[k], Ap, ec);
        acc += (double)seq_sum8(w);
      }
      acc = wave_xor_sum(acc);
      if (lane == 0) sh.xsum[f] = acc;
    }
  }
  if (wave * kPairsPerRound >= np && have_part)   // no task loads in this wave
    slot_ts[tid] = task_sum_in(my_part, sh.slot_Ap[my_slot], ec);
  __syncthreads();
  if (wave < ns) {
    // the mass without the children's tokens, in a fixed order
    const int k0 = sh.slot_k0[wave], nt = sh.slot_nt[wave];
    const double* ts = slot_ts + (int64_t)wave * tpr;
    double total = 0.0;
    for (int64_t c0 = 0; c0 < tpr; c0 += 64) {
      const int64_t c = c0 + lane;
      double v = c < tpr ? ts[c] : 0.0;
      for (int j = 0; j < nt; ++j)
        if (sh.xtask[k0 + j] == c) v = sh.xsum[k0 + j];
      total += lane_value(wave_incl_scan(v, lane), 63);
    }
    if (lane == 0) sh.slot_rest[wave] = total;
  }
  __syncthreads();
}

// Wave-level tests of the children of `node` (gathered in `slot`), in index
// order.  Lane i tests child i as if children 0..i-1 were rejected: the first
// child sees p' = p ([A] 1.2 step 3 with q the point mass at the candidate);
// a later one sees p without the tokens already rejected -- the slot's
// distinct tokens 0..d-1 -- p'(x_i) = w(x_i) / (mass without every child
// token + w_d + ... + w_{nx-1}), summed in that order; a token seen before
// has p' = 0.  The lowest accepting lane is the child the sequential tests
// take: lane 0 appends it to the path; every lane returns it, or -1.
__device__ __forceinline__ int64_t test_children(TreePointShared& sh, int slot, int64_t node,
                                                 const ExpConsts& ec, int lane) {
  const int k0 = sh.slot_k0[slot], nk = sh.slot_nk[slot], nx = sh.slot_nx[slot];
  bool accept = false;
  if (lane < nk) {
    const int32_t c = sh.kids[k0 + lane];
    const int jx = sh.kid_jx[k0 + lane];
    double r;
    if (lane == 0) {
      r = exp(((double)sh.lx[c] - (double)sh.M[node]) / ec.T) / sh.s[node];
    } else if (sh.kid_dup[k0 + lane]) {
      r = 0.0;
    } else {
      double rest = sh.slot_rest[slot];
      for (int j = jx; j < nx; ++j) rest += (double)sh.wx[k0 + j];
      r = rest > 0.0 ? (double)sh.wx[k0 + jx] / rest : 0.0;
    }
    accept = (double)sh.u[c] < r;
  }
  const uint64_t acc = __ballot(accept);
  if (!acc) return -1;
  const int64_t next = sh.kids[k0 + __builtin_ctzll(acc)];
  if (lane == 0) sh.tn.path[sh.tn.depth++] = (int32_t)next;
  return next;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void tree_point_kernel(
    const void* __restrict__ target, int64_t ld, int64_t V, int64_t R,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, ExpConsts ec,
    const Partial* __restrict__ part, int64_t tpr, int combine_lanes,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_path,
    int32_t* __restrict__ out_num_accepted, uint32_t* __restrict__ status) {
  __shared__ TreePointShared sh;
  __shared__ DrawShared ds;
  // dynamic LDS: the slots' task sums (kSlots slots when the row has at most
  // kPrefetchTasksPerRow tasks, else one), then the draw sums
  extern __shared__ double lds_dyn[];
  double* slot_ts = lds_dyn;
  double* draw_sum = lds_dyn + tree_slot_rows(tpr) * tpr;
  constexpr int64_t kTaskGroups = kWaveTaskElems / kGroup;   // 512 = one group per thread
  static_assert(kTaskGroups == kThreads, "a task is one group per thread");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t b = blockIdx.x;
  const int64_t g0 = cu[b], g1 = cu[b + 1];
  const int64_t N = g1 - g0;
  const bool slots_ok = g0 >= 0 && N >= 1 && g1 <= R;
  if (!slots_ok || N > kMaxTreeNodes) {
    reject_tree<kThreads>(b, g0, N, slots_ok,
                          slots_ok ? SPEC_VERIFY_DEV_BAD_TREE : SPEC_VERIFY_DEV_BAD_OFFSETS,
                          out_tokens, out_path, out_num_accepted, status);
    return;
  }
  for (int64_t n = tid; n < N; n += kThreads) sh.u[n] = uniforms[g0 + n];
  load_tree<kThreads>(parent, tokens, g0, N, V, sh.tn);
  if (sh.tn.bad) {
    reject_tree<kThreads>(b, g0, N, true, SPEC_VERIFY_DEV_BAD_TREE, out_tokens, out_path,
                          out_num_accepted, status);
    return;
  }
  // ---- every node's row normaliser and its token's logit in the parent's
  // row; the loads of two row passes and of the logits are issued before any
  // is reduced
  {
    const int L = combine_lanes;
    const int rows_per_wave = 64 / L;
    const int64_t stride = (int64_t)kWaves * rows_per_wave;
    float lxv[2];
    for (int64_t n0 = 0; n0 < N; n0 += 2 * kThreads) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t n = n0 + h * kThreads + tid;
        lxv[h] = (n >= 1 && n < N)
                     ? load_logit<DT>(row_ptr<DT>(target, g0 + sh.tn.par[n], ld), sh.tn.tok[n])
                     : 0.0f;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t n = n0 + h * kThreads + tid;
        if (n < N) sh.lx[n] = lxv[h];
      }
    }
    auto store = [&](int64_t r, bool active, const RowNorm& rn) {
      if (active && (lane & (L - 1)) == 0) {
        sh.M[r] = rn.M;
        sh.s[r] = rn.s;
      }
    };
    if (tpr <= L) {
      for (int64_t r0 = (int64_t)wave * rows_per_wave; r0 < N; r0 += 2 * stride) {
        const int64_t ra = r0 + lane / L, rb = ra + stride;
        const bool act_a = (lane / L) < rows_per_wave && ra < N;
        const bool act_b = (lane / L) < rows_per_wave && rb < N;
        const Partial pa = load_partial(part, tpr, act_a ? g0 + ra : 0, lane & (L - 1), act_a);
        const Partial pb = load_partial(part, tpr, act_b ? g0 + rb : 0, lane & (L - 1), act_b);
        store(ra, act_a, reduce_partials(pa, L, ec));
        store(rb, act_b, reduce_partials(pb, L, ec));
      }
    } else {
      for (int64_t r0 = (int64_t)wave * rows_per_wave; r0 < N; r0 += stride) {
        const int64_t r = r0 + lane / L;
        const bool active = (lane / L) < rows_per_wave && r < N;
        store(r, active, combine_rows_packed(part, tpr, L, active ? g0 + r : 0, active, ec, lane));
      }
    }
  }
  // ---- small trees (at most kPrefetchNodes nodes and kSlots internal nodes,
  // rows of at most kPrefetchTasksPerRow tasks): every internal node is
  // gathered now, in one round of loads, and wave 0 walks without loads.
  // Larger trees gather the current node at each level of the walk.
  if (wave == 0) {
    int ns = 0, k0 = 0;
    bool fits = N <= kPrefetchNodes && tpr <= kPrefetchTasksPerRow;
    for (int64_t base = 0; fits && base < N; base += 64) {
      const int64_t n = base + lane;
      const int nk = n < N ? sh.tn.nkids[n] : 0;
      const uint64_t m = __ballot(nk > 0);
      if (ns + __builtin_popcountll(m) > kSlots) {
        fits = false;
        break;
      }
      // flat ranges in node order
      const int before = (int)wave_scan((uint32_t)nk);
      if (nk > 0) {
        const int sl = ns + __builtin_popcountll(m & ((1ull << lane) - 1));
        sh.slot_node[sl] = (int32_t)n;
        sh.slot_k0[sl] = k0 + before - nk;
      }
      ns += __builtin_popcountll(m);
      k0 += (int)lane_value((uint32_t)before, 63);
    }
    if (lane == 0) {
      sh.prefetch = fits ? 1 : 0;
      sh.nslots = fits ? ns : 0;
      sh.tn.depth = 0;
    }
  }
  __syncthreads();

  // ---- the walk from the root
  int64_t cur = 0;
  int slot = -1;
  if (sh.prefetch) {
    if (sh.nslots > 0) gather_slots<DT, VEC>(sh, slot_ts, target, ld, V, g0, N, ec, part, tpr);
    if (wave == 0) {
      int64_t c = 0;
      int sl = -1;
      for (;;) {
        sl = -1;
        for (int k = 0; k < sh.nslots; ++k)
          if (sh.slot_node[k] == c) sl = k;
        if (sl < 0) break;
        const int64_t nxt = test_children(sh, sl, c, ec, lane);
        if (nxt < 0) break;
        c = nxt;
      }
      if (lane == 0) {
        sh.next = (int32_t)c;   // the node of the final draw
        sh.empty = sl;          // its slot (-1: no children)
      }
    }
    __syncthreads();
    cur = sh.next;
    slot = sh.empty;
    __syncthreads();            // sh.next and sh.empty are reused below
  } else {
    for (;;) {
      if (sh.tn.nkids[cur] == 0) {
        slot = -1;              // a node without children: the final draw from p
        break;
      }
      __syncthreads();          // the previous level's slot is read no more
      if (tid == 0) {
        sh.nslots = 1;
        sh.slot_node[0] = (int32_t)cur;
        sh.slot_k0[0] = 0;
      }
      __syncthreads();
      gather_slots<DT, VEC>(sh, slot_ts, target, ld, V, g0, N, ec, part, tpr);
      slot = 0;
      if (wave == 0) {
        const int64_t nxt = test_children(sh, 0, cur, ec, lane);
        if (lane == 0) sh.next = (int32_t)nxt;
      }
      __syncthreads();
      const int64_t nxt = sh.next;
      if (nxt < 0) break;       // every child rejected: the final draw at cur
      cur = nxt;
    }
  }

  // ---- final draw at `cur`: from p without its children's tokens (every
  // child was rejected), or from p at a node without children
  const void* prow = row_ptr<DT>(target, g0 + cur, ld);
  const float Ap = shift_of(sh.M[cur], ec);
  uint32_t fbad = 0;
  if (slot < 0) {
    // p at a node without children: its task sums
    for (int64_t c = tid; c < tpr; c += kThreads)
      draw_sum[c] = task_sum_in(part[(g0 + cur) * tpr + c], Ap, ec);
    __syncthreads();
  }
  const int k0 = slot >= 0 ? sh.slot_k0[slot] : 0;
  const int nt = slot >= 0 ? sh.slot_nt[slot] : 0;
  const int nx = slot >= 0 ? sh.slot_nx[slot] : 0;
  if (wave == 0) {
    const double* ts = slot >= 0 ? slot_ts + (int64_t)slot * tpr : draw_sum;
    if (slot >= 0) {
      for (int64_t c = lane; c < tpr; c += 64) {
        double v = ts[c];
        for (int j = 0; j < nt; ++j)
          if (sh.xtask[k0 + j] == c) v = sh.xsum[k0 + j];
        draw_sum[c] = v;
      }
    }
    const double* sums = draw_sum;
    double total = wave_total(sums, tpr, lane);
    int empty = 0;
    if (!(total > 0.0)) {
      // empty residual (invalid input or extreme rounding): draw from p
      empty = 1;
      sums = ts;
      total = wave_total(sums, tpr, lane);
    }
    const double tt = (double)sh.u[0] * total;
    find_interval(sums, tpr, tt, lane, ds);
    if (lane == 0) {
      ds.tt = tt;
      sh.empty = empty;
    }
  }
  __syncthreads();
  const bool exclude = slot >= 0 && !sh.empty;
  if (sh.empty) fbad |= SPEC_VERIFY_DEV_EMPTY_RESIDUAL;
  const int64_t tau = ds.tau;
  int64_t token = -1;
  if (tau >= 0) {
    GroupRaw<DT> r;
    const int64_t gi = tau * kTaskGroups + tid;
    load_group<DT, VEC>(prow, gi, V, r);
    float w[kGroup];
    group_weights_without<DT>(r, gi, Ap, ec, sh.xs + k0, exclude ? nx : 0, w);
    const double tt = ds.tt, p_excl = ds.p_excl;
    __syncthreads();   // ds is reused by the search
    token = block_search_weights(w, gi, tt, p_excl, ds);
  }
  write_tree_outputs<kThreads>(sh.tn, g0, N, (int32_t)token, out_tokens, out_path);
  if (tid == 0) {
    out_num_accepted[b] = sh.tn.depth;
    status_or(status, fbad);
  }
}

}  // namespace sv
