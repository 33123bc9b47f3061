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
// tree from the root.  The point kernel computes, when a node's first child
// is rejected, the exact mass of the node's row without its children's
// tokens: the row pass's task sums moved into one scale, and the tasks that
// hold a child token summed again without those tokens (never by
// subtraction).  Every later sibling's renormalised probability, and the
// final draw, use those sums.
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

struct TreePointShared {
  TreeNodes tn;
  float M[kMaxTreeNodes];        // row maxima
  double s[kMaxTreeNodes];       // row normalisers (exact scale)
  float lx[kMaxTreeNodes];       // logit of node n's token in its parent's row
  float u[kMaxTreeNodes];        // node n's uniform (root: the final draw)
  int32_t kids[kMaxChildren];    // children of the current node, in index order
  int32_t xs[kMaxChildren];      // their distinct tokens
  float wx[kMaxChildren];        // w of each distinct token in the node's scale
  int32_t xtask[kMaxChildren];   // distinct tasks holding those tokens
  double xsum[kMaxChildren];     // exact sums of those tasks without the tokens
  int nkids, nx, ntask;
  int next;                      // accepted child, or -1
  int have_x;                    // xsum / xs hold the current node's values
  double rest_x;                 // mass of the row without the children's tokens
};

// One block pass over task `task` of row `prow` (thread t < 512 holds group
// task * 512 + t): weights 2^(l c + Ap), zero at the listed tokens.
template <int DT, bool VEC>
__device__ __forceinline__ void task_weights_without(const void* prow, int64_t task, int64_t V,
                                                     float Ap, const ExpConsts& ec,
                                                     const int32_t* excl, int nexcl,
                                                     float w[kGroup], int64_t& gi, bool& active) {
  constexpr int64_t kTaskGroups = kWaveTaskElems / kGroup;
  active = threadIdx.x < kTaskGroups;
  gi = task * kTaskGroups + threadIdx.x;
#pragma unroll
  for (int k = 0; k < kGroup; ++k) w[k] = 0.0f;
  if (!active) return;
  GroupRaw<DT> r;
  load_group<DT, VEC>(prow, gi, V, r);
  float v[kGroup];
  unpack<DT>(r, v);
#pragma unroll
  for (int k = 0; k < kGroup; ++k) {
    const int64_t e = gi * kGroup + k;
    bool out = false;
    for (int i = 0; i < nexcl; ++i) out = out || (excl[i] == e);
    w[k] = out ? 0.0f : exp_term(v[k], Ap, ec);
  }
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
  extern __shared__ double lds_dyn[];   // [2 * tpr]: converted task sums, draw sums
  double* task_sum = lds_dyn;
  double* draw_sum = lds_dyn + tpr;
  constexpr int64_t kTaskGroups = kWaveTaskElems / kGroup;
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
  load_tree<kThreads>(parent, tokens, g0, N, V, sh.tn);
  if (sh.tn.bad) {
    reject_tree<kThreads>(b, g0, N, true, SPEC_VERIFY_DEV_BAD_TREE, out_tokens, out_path,
                          out_num_accepted, status);
    return;
  }
  // every node's row normaliser, its token's logit in the parent's row, its
  // uniform
  {
    const int L = combine_lanes;
    const int rows_per_wave = 64 / L;
    for (int64_t n = tid; n < N; n += kThreads) {
      sh.u[n] = uniforms[g0 + n];
      sh.lx[n] = n == 0 ? 0.0f
                        : load_logit<DT>(row_ptr<DT>(target, g0 + sh.tn.par[n], ld), sh.tn.tok[n]);
    }
    for (int64_t r0 = (int64_t)wave * rows_per_wave; r0 < N;
         r0 += (int64_t)kWaves * rows_per_wave) {
      const int64_t r = r0 + lane / L;
      const bool active = (lane / L) < rows_per_wave && r < N;
      const RowNorm rn = tpr <= L
          ? reduce_partials(load_partial(part, tpr, active ? g0 + r : 0, lane & (L - 1), active),
                            L, ec)
          : combine_rows_packed(part, tpr, L, active ? g0 + r : 0, active, ec, lane);
      if (active && (lane & (L - 1)) == 0) {
        sh.M[r] = rn.M;
        sh.s[r] = rn.s;
      }
    }
  }
  if (tid == 0) sh.tn.depth = 0;
  __syncthreads();

  uint32_t fbad = 0;
  int64_t cur = 0;
  for (;;) {
    const void* prow = row_ptr<DT>(target, g0 + cur, ld);
    const float Ap = shift_of(sh.M[cur], ec);
    // ---- the current node's children in index order, and its task sums
    // moved into the draw's scale 2^(l c + Ap)
    if (wave == 0) {
      int cnt = 0;
      for (int64_t base = cur + 1; base < N; base += 64) {
        const int64_t n = base + lane;
        const bool hit = n < N && sh.tn.par[n] == cur;
        const uint64_t m = __ballot(hit);
        if (hit) sh.kids[cnt + __builtin_popcountll(m & ((1ull << lane) - 1))] = (int32_t)n;
        cnt += __builtin_popcountll(m);
      }
      if (lane == 0) {
        sh.nkids = cnt;
        sh.next = -1;
        sh.have_x = 0;
      }
    }
    const Partial* prt = part + (g0 + cur) * tpr;
    for (int64_t c = tid; c < tpr; c += kThreads) {
      const Partial pc = prt[c];
      task_sum[c] = pc.m == -INFINITY ? 0.0 : pc.s * exp2((double)Ap - (double)shift_of(pc.m, ec));
    }
    __syncthreads();
    const int nk = sh.nkids;
    // ---- the first child: nothing removed yet, p' = p ([A] 1.2 step 3 with
    // q the point mass at the candidate)
    if (tid == 0 && nk > 0) {
      const int32_t c = sh.kids[0];
      const double r = exp(((double)sh.lx[c] - (double)sh.M[cur]) / ec.T) / sh.s[cur];
      if ((double)sh.u[c] < r) sh.next = c;
    }
    __syncthreads();
    // ---- the children's tokens, their weights and the exact mass without
    // them (needed by every later sibling and by the final draw)
    if (sh.next < 0 && nk > 0) {
      if (tid == 0) {
        int nx = 0, nt = 0;
        for (int i = 0; i < nk; ++i) {
          const int32_t c = sh.kids[i];
          const int32_t x = sh.tn.tok[c];
          bool seen = false;
          for (int j = 0; j < nx; ++j) seen = seen || sh.xs[j] == x;
          if (seen) continue;
          sh.xs[nx] = x;
          sh.wx[nx] = exp_term(sh.lx[c], Ap, ec);
          ++nx;
          const int32_t t = (int32_t)(x / kWaveTaskElems);
          bool tseen = false;
          for (int j = 0; j < nt; ++j) tseen = tseen || sh.xtask[j] == t;
          if (!tseen) sh.xtask[nt++] = t;
        }
        sh.nx = nx;
        sh.ntask = nt;
      }
      __syncthreads();
      for (int j = 0; j < sh.ntask; ++j) {
        float w[kGroup];
        int64_t gi;
        bool active;
        task_weights_without<DT, VEC>(prow, sh.xtask[j], V, Ap, ec, sh.xs, sh.nx, w, gi, active);
        const double ts = block_sum((double)seq_sum8(w), ds);
        if (tid == 0) sh.xsum[j] = ts;
        __syncthreads();   // ds.red is reused
      }
      if (wave == 0) {
        // draw sums: task sums, with the children's tasks summed without them
        for (int64_t c = lane; c < tpr; c += 64) {
          double v = task_sum[c];
          for (int j = 0; j < sh.ntask; ++j)
            if (sh.xtask[j] == c) v = sh.xsum[j];
          draw_sum[c] = v;
        }
        const double rest = wave_total(draw_sum, tpr, lane);
        if (lane == 0) {
          sh.rest_x = rest;
          sh.have_x = 1;
        }
      }
      __syncthreads();
      // ---- later siblings: p'(x) = w(x) / (mass without the children's
      // tokens + the children's tokens not yet rejected)
      if (tid == 0) {
        uint64_t removed = 0;   // bit j: xs[j] rejected
        for (int i = 0; i < nk; ++i) {
          const int32_t c = sh.kids[i];
          const int32_t x = sh.tn.tok[c];
          int jx = 0;
          while (sh.xs[jx] != x) ++jx;
          if (i > 0) {
            double r = 0.0;
            if (!((removed >> jx) & 1)) {
              double rest = sh.rest_x;
              for (int j = 0; j < sh.nx; ++j)
                if (!((removed >> j) & 1)) rest += (double)sh.wx[j];
              r = rest > 0.0 ? (double)sh.wx[jx] / rest : 0.0;
            }
            if ((double)sh.u[c] < r) {
              sh.next = c;
              break;
            }
          }
          removed |= 1ull << jx;
        }
      }
      __syncthreads();
    }
    if (sh.next >= 0) {
      if (tid == 0) sh.tn.path[sh.tn.depth++] = sh.next;
      cur = sh.next;
      __syncthreads();
      continue;
    }
    break;
  }

  // ---- final draw at `cur`: from p without its children's tokens (every
  // child was rejected), or from p at a node without children
  const int nk = sh.nkids;
  const void* prow = row_ptr<DT>(target, g0 + cur, ld);
  const float Ap = shift_of(sh.M[cur], ec);
  const double* sums = nk > 0 ? draw_sum : task_sum;
  if (wave == 0) {
    double total = wave_total(sums, tpr, lane);
    if (!(total > 0.0)) {
      // empty residual (invalid input or extreme rounding): draw from p
      if (lane == 0) ds.empty = 1;
      sums = task_sum;
      total = wave_total(sums, tpr, lane);
    } else if (lane == 0) {
      ds.empty = 0;
    }
    const double tt = (double)sh.u[0] * total;
    find_interval(sums, tpr, tt, lane, ds);
    if (lane == 0) ds.tt = tt;
  }
  __syncthreads();
  const bool exclude = nk > 0 && !ds.empty;
  if (ds.empty) fbad |= SPEC_VERIFY_DEV_EMPTY_RESIDUAL;
  const int64_t tau = ds.tau;
  int64_t token = -1;
  if (tau >= 0) {
    float w[kGroup];
    int64_t gi;
    bool active;
    task_weights_without<DT, VEC>(prow, tau, V, Ap, ec, sh.xs, exclude ? sh.nx : 0, w, gi,
                                  active);
    const double tt = ds.tt, p_excl = ds.p_excl;
    __syncthreads();   // ds is reused by the search
    token = block_search_weights(w, gi, tt, p_excl, ds);
  }
  write_tree_outputs<kThreads>(sh.tn, g0, N, (int32_t)token, out_tokens, out_path);
  if (tid == 0) {
    out_num_accepted[b] = sh.tn.depth;
    status_or(status, fbad);
  }
  (void)kTaskGroups;
}

}  // namespace sv
