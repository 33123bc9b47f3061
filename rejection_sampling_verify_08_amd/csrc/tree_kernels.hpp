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
constexpr int kXBatch = 4;        // child-token tasks loaded per round

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
  double red[kWaves][kXBatch];   // per-wave partial sums of a batch of tasks
  int nkids, nx, ntask;
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
  if (tid == 0) sh.tn.depth = 0;
  __syncthreads();

  // The groups of the last batch of child-token tasks stay in registers: the
  // final search reuses them when it lands in one of those tasks.
  GroupRaw<DT> xraw[kXBatch];
  int32_t xraw_task[kXBatch];
#pragma unroll
  for (int j = 0; j < kXBatch; ++j) xraw_task[j] = -1;
  uint32_t fbad = 0;
  int64_t cur = 0;
  for (;;) {
    const void* prow = row_ptr<DT>(target, g0 + cur, ld);
    const float Ap = shift_of(sh.M[cur], ec);
    // ---- the current node's children in index order, their distinct tokens
    // and the tasks holding them (wave 0)
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
        int nx = 0, nt = 0;
        for (int i = 0; i < cnt; ++i) {
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
        sh.nkids = cnt;
        sh.nx = nx;
        sh.ntask = nt;
        sh.next = -1;
      }
    }
    __syncthreads();
    const int nk = sh.nkids, nx = sh.nx, ntask = sh.ntask;
    // ---- one round of loads: the row's task partials and the groups of the
    // tasks holding child tokens; then the task sums in the draw's scale
    // 2^(l c + Ap) and those tasks summed without the child tokens
    const Partial* prt = part + (g0 + cur) * tpr;
    for (int64_t j0 = 0; j0 < (ntask > 0 ? ntask : 1); j0 += kXBatch) {
      const int nb = ntask - (int)j0 < kXBatch ? ntask - (int)j0 : kXBatch;
#pragma unroll
      for (int j = 0; j < kXBatch; ++j) {
        xraw_task[j] = j < nb ? sh.xtask[j0 + j] : -1;
        if (j < nb) load_group<DT, VEC>(prow, (int64_t)xraw_task[j] * kTaskGroups + tid, V, xraw[j]);
      }
      if (j0 == 0)
        for (int64_t c = tid; c < tpr; c += kThreads) {
          const Partial pc = prt[c];
          task_sum[c] = pc.m == -INFINITY ? 0.0
                                          : pc.s * exp2((double)Ap - (double)shift_of(pc.m, ec));
        }
#pragma unroll
      for (int j = 0; j < kXBatch; ++j) {
        double gs = 0.0;
        if (j < nb) {
          float w[kGroup];
          group_weights_without<DT>(xraw[j], (int64_t)xraw_task[j] * kTaskGroups + tid, Ap, ec,
                                    sh.xs, nx, w);
          gs = (double)seq_sum8(w);
        }
        gs = __shfl(wave_incl_scan(gs, lane), 63);
        if (lane == 0) sh.red[wave][j] = gs;
      }
      __syncthreads();
      if (tid < nb) {
        double t = 0.0;
        for (int v = 0; v < kWaves; ++v) t += sh.red[v][tid];
        sh.xsum[j0 + tid] = t;
      }
      __syncthreads();
    }
    // ---- wave 0: the mass without the children's tokens, then the tests
    // in index order.  The first child sees p' = p ([A] 1.2 step 3 with q
    // the point mass at the candidate); each later one p without the tokens
    // already rejected: p'(x) = w(x) / (mass without every child token + the
    // child tokens not yet rejected).
    if (wave == 0 && nk > 0) {
      for (int64_t c = lane; c < tpr; c += 64) {
        double v = task_sum[c];
        for (int j = 0; j < ntask; ++j)
          if (sh.xtask[j] == c) v = sh.xsum[j];
        draw_sum[c] = v;
      }
      const double rest_x = wave_total(draw_sum, tpr, lane);
      if (lane == 0) {
        uint64_t removed = 0;   // bit j: xs[j] rejected
        for (int i = 0; i < nk; ++i) {
          const int32_t c = sh.kids[i];
          const int32_t x = sh.tn.tok[c];
          int jx = 0;
          while (sh.xs[jx] != x) ++jx;
          double r;
          if (i == 0) {
            r = exp(((double)sh.lx[c] - (double)sh.M[cur]) / ec.T) / sh.s[cur];
          } else if ((removed >> jx) & 1) {
            r = 0.0;
          } else {
            double rest = rest_x;
            for (int j = 0; j < nx; ++j)
              if (!((removed >> j) & 1)) rest += (double)sh.wx[j];
            r = rest > 0.0 ? (double)sh.wx[jx] / rest : 0.0;
          }
          if ((double)sh.u[c] < r) {
            sh.next = c;
            break;
          }
          removed |= 1ull << jx;
        }
      }
    }
    __syncthreads();
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
  if (wave == 0) {
    const double* sums = nk > 0 ? draw_sum : task_sum;
    double total = wave_total(sums, tpr, lane);
    int empty = 0;
    if (!(total > 0.0)) {
      // empty residual (invalid input or extreme rounding): draw from p
      empty = 1;
      sums = task_sum;
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
  const bool exclude = nk > 0 && !sh.empty;
  if (sh.empty) fbad |= SPEC_VERIFY_DEV_EMPTY_RESIDUAL;
  const int64_t tau = ds.tau;
  int64_t token = -1;
  if (tau >= 0) {
    GroupRaw<DT> r;
    bool have = false;
#pragma unroll
    for (int j = 0; j < kXBatch; ++j)
      if (xraw_task[j] == tau) {
        r = xraw[j];
        have = true;
      }
    const int64_t gi = tau * kTaskGroups + tid;
    if (!have) load_group<DT, VEC>(prow, gi, V, r);
    float w[kGroup];
    group_weights_without<DT>(r, gi, Ap, ec, sh.xs, exclude ? sh.nx : 0, w);
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
