// Draft-tree verification: the statistics pass over every node of each row's
// tree and the tree walk with its residual passes.  Included by
// spec_verify.hip inside its anonymous namespace; it uses that file's
// helpers (tiles, reductions, published words, segment_search).
//
// Source: [RheoSampling] section 4 (RheoVerification).  A node's children are
// candidate tokens drawn from the drafter's distribution q~ at the node; they
// are tested in increasing node index, the first with min(1, p/q~) at its
// token.  An
// accepted child is descended into; after a rejection the target is replaced
// by the residual norm(max(0, r - q~)) and the next child is tested against
// it.  Every residual is r_j = max(0, p - c_j q) / W_j with c_0 = 0, W_0 = 1,
// c_{j+1} = c_j + W_j and W_j = sum_x max(0, p - c_j q): a rejection costs
// one pass over the node's target and draft logits to get the next W.  When
// every child is rejected the final token is drawn from the last residual;
// at a leaf it is the bonus token drawn from the leaf's target.  Greedy rows
// (T <= 0) descend into the first child equal to the node's target argmax.
//
// Kernels.  tree_stats_kernel: one work-group per (row, node, chunk), for
// the node's target and, if the node has children, its draft (partial slots
// 0..N-1 the targets, N..2N-1 the drafts); it writes the chunk partials, the
// logits of each child's token at its parent (target and draft), and for a
// leaf the 32 sub-block sums of its target.  tree_finish_kernel: one work-group per
// (row, chunk) walks the row's tree; the residual passes are shared out among
// the row's work-groups chunk by chunk (see the kernel).

constexpr int MAX_NODES = SV_MAX_NODES;

struct TreeArgs {
  const void* tgt;           // [B, N, V]
  const void* dft;           // [B, N, V]
  const int32_t* tok;        // [B, N]
  const int32_t* par;        // [B, N]
  const float* uni;          // [B, N]
  const float* temp;         // [B]
  int32_t* out;              // [B, N]
  int32_t* onodes;           // [B, N]
  int32_t* nacc;             // [B]
  uint32_t* part;            // [B, 2N, C, 4] chunk partials {max | argmax value, sum, argmax id, 0}
  uint32_t* subK;            // [B, N, C, NSUB] target sub-block sums (vs chunk max): leaves', every node's when sparse
  uint32_t* subR;            // [B, N, C, NSUB] published residual sub-block sums, one set per pass
  unsigned* claim;           // [B] residual-pass tickets handed out
  unsigned* leave;           // [B] work-groups of the row that have finished
  float* gath;               // [B, N, 2] l_t, l_q of each node's token at its parent
  float* probes;             // [B, N, 3] (p(d), q(d), r(d)) of each tested node, NaN elsewhere; or null
  float* mass;               // [B] total weight of the final draw's distribution; or null
  // Sparse drafts (topk > 0): chunk candidate lists, then per node the kept
  // set (ascending id) and {max kept logit, Z_q, -, kept count}.
  void* cand;                // [B, N, C, cstride]
  int* ccnt;                 // [B, N, C, 2] list lengths and bound keys
  float4* qstat;             // [B, N]
  uint2* kept;               // [B, N, topk]
  int B, N, V, C, CS, topk;
  int cstride, ckeep;        // candidate entries per chunk; logits a chunk lists at least
};

template <typename ET>
__device__ __forceinline__ const ET* tree_row(const TreeArgs& a, bool draft, int b, int v) {
  return static_cast<const ET*>(draft ? a.dft : a.tgt) + ((size_t)b * a.N + v) * (size_t)a.V;
}
__device__ __forceinline__ uint32_t* tree_part(const TreeArgs& a, int b, int slot, int c) {
  return a.part + (((size_t)b * 2 * a.N + slot) * (size_t)a.C + c) * 4;
}


// ============================================================================
// Statistics of one slot's chunk, from its tile r (target slot: slot = node;
// draft slot: slot = N + node).  kids: the node's children mask.
// ============================================================================
template <typename ET, bool ALIGNED>
__device__ __forceinline__ void tree_slot_stats(const TreeArgs& a, int b, int node, bool is_draft, int c, int lo,
                                                int len, const u32x4 (&r)[NV_TILE], float T, bool greedy,
                                                unsigned long long kids, float* shf, int* shi, float* shsub) {
  constexpr int VEC = Tr<ET>::VEC;
  const int N = a.N, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const ET* row = tree_row<ET>(a, is_draft, b, node);
  if (is_draft && a.topk > 0) {
    // A truncated draft: the chunk's candidates for the node's top k.
    const size_t chunk = ((size_t)b * N + node) * a.C + c;
    topk_chunk<ET>(r, lo, len, a.topk, a.ckeep, a.cstride,
                   reinterpret_cast<typename Cand<ET>::T*>(a.cand) + chunk * a.cstride, a.ccnt + 2 * chunk, shf);
    return;
  }
  uint32_t* dst = tree_part(a, b, is_draft ? N + node : node, c);
  if (greedy) {
    float bv = Tr<ET>::at(r[0], 0);
    int bi = lo + t * VEC;
#pragma unroll
    for (int j = 0; j < NV_TILE; ++j)
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float x = Tr<ET>::at(r[j], k);
        if (x > bv) { bv = x; bi = lo + (j * WG + t) * VEC + k; }
      }
    block_argmax(bv, bi, shf, shi);
    if (t == 0) *reinterpret_cast<u32x4*>(dst) = u32x4{__float_as_uint(bv), 0u, (uint32_t)bi, 0u};
    return;
  }
  const float m = block_max(tile_max<ET, NV_TILE>(r), shf);
  const float s = LOG2E / T;
  const float msr = m == NEG_INF ? 0.f : mul_rn(m, s);
  float zj[NV_TILE];
#pragma unroll
  for (int j = 0; j < NV_TILE; ++j) {
    float e0 = exp2_fast(fmaf(Tr<ET>::at(r[j], 0), s, -msr));
    float e1 = exp2_fast(fmaf(Tr<ET>::at(r[j], 1), s, -msr));
#pragma unroll
    for (int k = 2; k < VEC; k += 2) {
      e0 += exp2_fast(fmaf(Tr<ET>::at(r[j], k), s, -msr));
      e1 += exp2_fast(fmaf(Tr<ET>::at(r[j], k + 1), s, -msr));
    }
    zj[j] = e0 + e1;
  }
  float zl = zj[0];
#pragma unroll
  for (int j = 1; j < NV_TILE; ++j) zl += zj[j];
  const float z = block_sum(zl, shf);
  if (!is_draft && (kids == 0 || a.topk > 0)) {
    // A leaf: sub-block sums of its target for a bonus draw there; with a
    // truncated draft every node's, for its residuals' mass.
#pragma unroll
    for (int j = 0; j < NV_TILE; ++j) {
      const float v = wave_sum(zj[j]);
      if (lane == 0) shsub[j * NWAVE + wave] = v;
    }
    __syncthreads();
    if (t < NSUB) a.subK[(((size_t)b * N + node) * a.C + c) * NSUB + t] = __float_as_uint(shsub[t]);
  }
  // Each child's token logit, recorded by the chunk that holds it.
  if (t < N && (kids >> t & 1ull)) {
    const int d = a.tok[(size_t)b * N + t];
    if (d >= lo && d < lo + len) a.gath[((size_t)b * N + t) * 2 + (is_draft ? 1 : 0)] = Tr<ET>::load1(row + d);
  }
  if (t == 0) *reinterpret_cast<u32x4*>(dst) = u32x4{__float_as_uint(m), __float_as_uint(z), 0u, 0u};
}

// ============================================================================
// Statistics of one (row, node, chunk): the node's target and, for a node
// with children in a sampling row, its draft (the distribution the children
// were drawn from).  The target's tile, the temperature and the parents are
// loaded at once; the draft's loads are issued as soon as the children mask
// is known and overlap the target's statistics.  Leaves and greedy rows read
// no draft.  Four waves per SIMD; three for bf16 rows that are not 16-byte
// aligned (odd V), whose element-wise loads need one register more than
// four waves allow.
// ============================================================================
template <typename ET, bool ALIGNED>
__global__ __launch_bounds__(WG) __attribute__((
    amdgpu_waves_per_eu(ALIGNED || sizeof(ET) == 4 ? STATS_WAVES : 3, ALIGNED || sizeof(ET) == 4 ? STATS_WAVES : 3)))
void tree_stats_kernel(TreeArgs a) {
  const int N = a.N;
  const int c = blockIdx.x % a.C;
  const int rest = blockIdx.x / a.C;
  const int node = rest % N;
  const int b = rest / N;
  const int t = threadIdx.x, lane = t & 63;
  __shared__ float shf[NWAVE];
  __shared__ int shi[NWAVE];
  __shared__ float shsub[NSUB];
  const int lo = c * a.CS;
  const int len = min(a.CS, a.V - lo);
  u32x4 rt[NV_TILE], rq[NV_TILE];
  load_tile<ET, ALIGNED, NV_TILE>(tree_row<ET>(a, false, b, node), lo, len, rt);
  // Every wave forms the node's children mask itself.
  const float T = a.temp[b];
  const int p = (lane > 0 && lane < N) ? a.par[(size_t)b * N + lane] : -1;
  const unsigned long long kids = __ballot(lane > node && lane < N && p == node);
  if (a.probes && node == 0 && c == 0)
    for (int i = t; i < 3 * N; i += WG) a.probes[(size_t)b * 3 * N + i] = __builtin_nanf("");
  const bool greedy = !is_sampling_temperature(T);
  const bool with_draft = !greedy && kids != 0;  // uniform
  if (with_draft) load_tile<ET, ALIGNED, NV_TILE>(tree_row<ET>(a, true, b, node), lo, len, rq);
  tree_slot_stats<ET, ALIGNED>(a, b, node, false, c, lo, len, rt, T, greedy, kids, shf, shi, shsub);
  if (!with_draft) return;
  __syncthreads();  // the shared scratch is reused
  tree_slot_stats<ET, ALIGNED>(a, b, node, true, c, lo, len, rq, T, greedy, kids, shf, shi, shsub);
}

// ============================================================================
// Sparse drafts: the exact top-k selection of each node with children (the
// merge of spec_verify's sparse path, one work-group per (row, node)), then
// each child's token logit in the kept set (-inf when not kept), for the
// node's q~ at the child's token.
// ============================================================================
template <typename ET>
__global__ __launch_bounds__(WG) void tree_merge_kernel(TreeArgs ta, Args ma) {
  const int N = ta.N;
  const int node = blockIdx.x % N, b = blockIdx.x / N;
  const int t = threadIdx.x;
  __shared__ int s_has;
  if (!is_sampling_temperature(ta.temp[b])) return;
  int p = -1;
  if (t > node && t < N) p = ta.par[(size_t)b * N + t];
  if (t == 0) s_has = 0;
  __syncthreads();
  if (p == node) s_has = 1;
  __syncthreads();
  if (!s_has) return;
  const int kk = merge_body<ET>(ma, b, node, -1);
  __syncthreads();  // the kept list is written
  if (p == node) {
    const int d = ta.tok[(size_t)b * N + t];
    const uint2* kept = ta.kept + ((size_t)b * N + node) * ta.topk;
    int lo = 0, hi = kk;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int)kept[mid].x < d) lo = mid + 1; else hi = mid;
    }
    ta.gath[((size_t)b * N + t) * 2 + 1] =
        (lo < kk && (int)kept[lo].x == d) ? __uint_as_float(kept[lo].y) : NEG_INF;
  }
}

// ============================================================================
// The walk, on the row's merged statistics in LDS.
// ============================================================================
struct TreeRow {
  float M[2 * MAX_NODES];    // target (0..N-1) and draft (N..2N-1) max, or argmax value (greedy)
  float Z[2 * MAX_NODES];
  unsigned long long kids[MAX_NODES];  // bit x: node x is a child of the node
  int idx[MAX_NODES];        // target argmax (greedy)
  int tok[MAX_NODES];
  float u[MAX_NODES];
  float gt[MAX_NODES], gq[MAX_NODES];
  int path[MAX_NODES];
  float s;
  int greedy;
  // walk result
  int nk[MAX_NODES];         // sparse draft: kept count of each node with children
  int status;                // W_PASS, W_LEAF, W_RESID, W_GREEDY, W_FALLBACK
  int v, j, n, x;
  float c, W;
};
enum { W_PASS = 0, W_LEAF = 1, W_RESID = 2, W_GREEDY = 3, W_FALLBACK = 4 };

// Merges the chunk statistics of every node (and of the draft of every node
// with children) into tr.M / tr.Z / tr.idx: one group of G lanes per slot,
// lane g of the group holding chunks g, g + G, ... (G = 64 when C > 32), so
// that the results equal the wave reductions of the linear verifier bit for
// bit.
template <int G>
__device__ __forceinline__ void tree_merge(TreeRow& tr, const uint32_t* pw, int N, int C, bool greedy, bool sparse,
                                           float s) {
  constexpr int PER = 64 / G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gl = lane % G;
  const int nslots = greedy ? N : 2 * N;
  for (int base = wave * PER; base < nslots; base += NWAVE * PER) {
    const int slot = base + lane / G;
    const int node = slot < N ? slot : slot - N;
    const bool need = slot < nslots && (slot < N || (!sparse && tr.kids[node] != 0ull));
    auto word = [&](int cc, int w) { return __uint_as_float(pw[((size_t)slot * C + cc) * 4 + w]); };
    if (greedy) {
      float bv = NEG_INF;
      int bi = INT_MAX;
      if (need)
        for (int cc = gl; cc < C; cc += G) argmax_merge(bv, bi, word(cc, 0), __float_as_int(word(cc, 2)));
      group_argmax<G>(bv, bi);
      if (need && gl == G - 1) {
        tr.M[slot] = bv;
        tr.Z[slot] = 0.f;
        tr.idx[node] = bi;
      }
    } else {
      float m = NEG_INF;
      if (need)
        for (int cc = gl; cc < C; cc += G) m = fmaxf(m, word(cc, 0));
      m = group_last<G>(group_max<G>(m));
      const float MS = mul_rn(m, s);
      float z = 0.f;
      if (need)
        for (int cc = gl; cc < C; cc += G) {
          const float mc = word(cc, 0), zc = word(cc, 1);
          if (mc != NEG_INF) z += zc * exp2_fast(mul_rn(mc, s) - MS);
        }
      z = group_sum<G>(z);
      if (need && gl == G - 1) {
        tr.M[slot] = m;
        tr.Z[slot] = z;
      }
    }
  }
}

// Continues the walk at node v, testing the children after child `after`
// against the residual (c, W).  Thread 0 only.  With `probe` (the row's
// [N, 3] diagnostics) each tested node's p(d), q(d), r(d) are recorded.
__device__ __forceinline__ void tree_walk(TreeRow& tr, int N, int V, int v, int after, float c, float W, float* probe) {
  const float s = tr.s;
  int n = tr.n;
  for (;;) {
    const unsigned long long kids = tr.kids[v];
    if (tr.greedy) {
      int nxt = -1;
      for (unsigned long long m = kids; m; m &= m - 1) {
        const int x = (int)__builtin_ctzll(m);
        if (tr.tok[x] == tr.idx[v]) { nxt = x; break; }
      }
      if (nxt < 0) { tr.status = W_GREEDY; tr.v = v; tr.x = tr.idx[v]; break; }
      tr.path[n++] = nxt;
      v = nxt;
      continue;
    }
    if (kids == 0) { tr.status = W_LEAF; tr.v = v; break; }
    const float MSt = mul_rn(tr.M[v], s), MSq = mul_rn(tr.M[N + v], s);
    int acc = -1, rej = -1;
    // The next child after `after` (children are tested in node order).
    const unsigned long long rest = after >= 63 ? 0ull : kids & ~((2ull << after) - 1ull);
    if (rest) {
      const int x = (int)__builtin_ctzll(rest);
      const int d = tr.tok[x];
      float pd = 0.f, qd = 0.f;
      if (d >= 0 && d < V) {
        pd = exp2_fast(fmaf(tr.gt[x], s, -MSt)) / tr.Z[v];
        qd = exp2_fast(fmaf(tr.gq[x], s, -MSq)) / tr.Z[N + v];
      }
      const float rd = fmaxf(0.f, pd - c * qd) / W;
      if (probe) {
        probe[x * 3 + 0] = pd;
        probe[x * 3 + 1] = qd;
        probe[x * 3 + 2] = rd;
      }
      if (tr.u[x] * qd < rd) acc = x;
      else rej = x;  // a rejection needs the next residual's mass first
    }
    if (acc >= 0) {
      tr.path[n++] = acc;
      v = acc;
      after = 0;
      c = 0.f;
      W = 1.f;
      continue;
    }
    if (rej >= 0) { tr.status = W_PASS; tr.v = v; tr.j = rej; tr.c = c + W; break; }
    // every child has been tested and rejected: draw from the residual (c, W)
    tr.status = W_RESID;
    tr.v = v;
    tr.c = c;
    tr.W = W;
    break;
  }
  tr.n = n;
}

// ============================================================================
// Final draw (wave 0).  Residual: weights max(0, p_v - c q_v) with the
// sub-block sums in `csub` (LDS); leaf: p_v with the leaf's sub-block sums
// rescaled from the chunk max; fallback: p_v with chunk masses from the
// partials and a walk over the whole chunk.  The walk of the levels follows
// final_draw.  Returns the token in every lane of wave 0; also the total S
// (the residual's W when `want_total`).
// ============================================================================
template <typename ET, bool ALIGNED>
__device__ __forceinline__ int tree_draw(const TreeArgs& a, const TreeRow& tr, const uint32_t* pw, const float* csub,
                                         int b, int v, int mode, float cscale, float uK, float* S_out,
                                         const int* kid = nullptr, const float* kq = nullptr, int nkept = 0) {
  constexpr int VEC = Tr<ET>::VEC;
  const int N = a.N, C = a.C, l = threadIdx.x & 63;
  const float s = tr.s;
  const float MSt = mul_rn(tr.M[v], s), rZt = 1.f / tr.Z[v];
  auto pword = [&](int slot, int c, int w) { return __uint_as_float(pw[((size_t)slot * C + c) * 4 + w]); };
  const uint32_t* gleaf = a.subK + ((size_t)b * N + v) * C * NSUB;
  auto bonus_scale = [&](int c) {
    const float mc = pword(v, c, 0);
    return mc == NEG_INF ? 0.f : exp2_fast(mul_rn(mc, s) - MSt) * rZt;
  };
  auto sub_weight = [&](int c, int q, float sc) {
    return mode == W_LEAF ? __uint_as_float(gleaf[c * NSUB + q]) * sc : csub[c * NSUB + q];
  };
  auto chunk_mass = [&](int c) {
    if (mode == W_FALLBACK) {
      const float mc = pword(v, c, 0), zc = pword(v, c, 1);
      return mc == NEG_INF ? 0.f : zc * exp2_fast(mul_rn(mc, s) - MSt) * rZt;
    }
    const float sc = mode == W_LEAF ? bonus_scale(c) : 1.f;
    float w[NSUB];
#pragma unroll
    for (int q = 0; q < NSUB; ++q) w[q] = sub_weight(c, q, sc);
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < NSUB; ++q) m += w[q];
    return m;
  };
  auto group = [&](int base, float& m, float& in, float& ex) {
    const int c = base + l;
    m = c < C ? chunk_mass(c) : 0.f;
    in = wave_incl_scan(m);
    ex = __shfl_up(in, 1, 64);
    if (l == 0) ex = 0.f;
  };
  float m0, in0, ex0;
  group(0, m0, in0, ex0);
  float S = lane63(in0);
  for (int base = 64; base < C; base += 64) {
    float m, in, ex;
    group(base, m, in, ex);
    S += lane63(in);
  }
  *S_out = S;
  if (uK < 0.f) return -1;  // total only
  const float tv = uK * S;
  int cs = -1, last = -1;
  float exc_cs = 0.f, carry = 0.f;
  for (int base = 0; base < C; base += 64) {
    float m = m0, in = in0, ex = ex0;
    if (base > 0) group(base, m, in, ex);
    const int c = base + l;
    const unsigned long long hit = __ballot(c < C && carry + in > tv);
    if (hit) {
      const int q = (int)__builtin_ctzll(hit);
      cs = base + q;
      exc_cs = carry + __shfl(ex, q, 64);
      break;
    }
    const unsigned long long pos = __ballot(c < C && m > 0.f);
    if (pos) last = base + 63 - (int)__builtin_clzll(pos);
    carry += lane63(in);
  }
  if (cs < 0) {
    cs = last >= 0 ? last : 0;
    exc_cs = -__builtin_inff();
  }
  const float t1 = tv - exc_cs;
  const int lo = cs * a.CS;
  const int len = min(a.CS, a.V - lo);
  const ET* trow = tree_row<ET>(a, false, b, v);
  const ET* drow = (mode == W_RESID && !kid) ? tree_row<ET>(a, true, b, v) : nullptr;
  const float MSq = mode == W_RESID ? mul_rn(tr.M[N + v], s) : 0.f;
  const float rZq = mode == W_RESID ? cscale / tr.Z[N + v] : 0.f;
  if (mode == W_FALLBACK) {
    float cy = 0.f;
    int lastp = -1, x = -1;
    for (int seg = 0; seg < len && x < 0; seg += 64 * VEC) {
      const SegResult r = segment_search<ET, ALIGNED>(trow, nullptr, nullptr, nullptr, 0, lo + seg,
                                                      min(64 * VEC, len - seg), t1 - cy, s, MSt, rZt, 0.f, 0.f);
      if (r.found >= 0) x = r.found;
      if (r.last_pos >= 0) lastp = r.last_pos;
      cy += r.total;
    }
    return x >= 0 ? x : (lastp >= 0 ? lastp : lo);
  }
  const float sc = mode == W_LEAF ? bonus_scale(cs) : 1.f;
  float ws[NSUB];
#pragma unroll
  for (int q = 0; q < NSUB; ++q) ws[q] = sub_weight(cs, q, sc);
  float pre = 0.f;
#pragma unroll
  for (int q = 0; q < NSUB; ++q)
    if (q <= l) pre += ws[q];
  const float wl = l < NSUB ? sub_weight(cs, l, sc) : 0.f;
  const unsigned long long hit = __ballot(l < NSUB && pre > t1);
  int q;
  float tl;
  if (hit) {
    q = (int)__builtin_ctzll(hit);
    const float pex = __shfl(pre, q > 0 ? q - 1 : 0, 64);
    tl = q > 0 ? t1 - pex : t1;
  } else {
    const unsigned long long pos = __ballot(l < NSUB && wl > 0.f);
    q = pos ? 63 - (int)__builtin_clzll(pos) : 0;
    tl = __builtin_inff();
  }
  const int jj = q / NWAVE, w = q % NWAVE;
  const int start = lo + (jj * WG + w * 64) * VEC;
  const int slen = max(0, min(64 * VEC, lo + len - start));
  if (slen <= 0) return lo;
  const SegResult r = segment_search<ET, ALIGNED>(trow, drow, mode == W_RESID ? kid : nullptr, kq, nkept, start,
                                                  slen, tl, s, MSt, rZt, MSq, rZq);
  return r.found >= 0 ? r.found : (r.last_pos >= 0 ? r.last_pos : start);
}

// Sub-block sums of max(0, p_v - c q_v) over one chunk (all threads); the 32
// sums go to dst[0..NSUB).
template <typename ET, bool ALIGNED>
__device__ __forceinline__ void tree_chunk_residual(const TreeArgs& a, const TreeRow& tr, int b, int v, float cscale,
                                                    int chunk, float* dst) {
  constexpr int VEC = Tr<ET>::VEC;
  const int N = a.N, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float s = tr.s;
  const float MSt = mul_rn(tr.M[v], s), rZt = 1.f / tr.Z[v];
  const float MSq = mul_rn(tr.M[N + v], s), rZq = cscale / tr.Z[N + v];
  const int lo = chunk * a.CS;
  const int len = min(a.CS, a.V - lo);
  u32x4 rt[NV_TILE], rq[NV_TILE];
  load_tile<ET, ALIGNED, NV_TILE, false>(tree_row<ET>(a, false, b, v), lo, len, rt);
  load_tile<ET, ALIGNED, NV_TILE, false>(tree_row<ET>(a, true, b, v), lo, len, rq);
#pragma unroll
  for (int j = 0; j < NV_TILE; ++j) {
    float w0 = 0.f, w1 = 0.f;
#pragma unroll
    for (int k = 0; k < VEC; k += 2) {
      const float p0 = exp2_fast(fmaf(Tr<ET>::at(rt[j], k), s, -MSt)) * rZt;
      const float q0 = exp2_fast(fmaf(Tr<ET>::at(rq[j], k), s, -MSq)) * rZq;
      const float p1 = exp2_fast(fmaf(Tr<ET>::at(rt[j], k + 1), s, -MSt)) * rZt;
      const float q1 = exp2_fast(fmaf(Tr<ET>::at(rq[j], k + 1), s, -MSq)) * rZq;
      w0 += fmaxf(0.f, p0 - q0);
      w1 += fmaxf(0.f, p1 - q1);
    }
    const float sum = wave_sum(w0 + w1);
    if (lane == 0) dst[j * NWAVE + wave] = sum;
  }
  __syncthreads();
}

// ============================================================================
// The tree walk: one work-group per (row, chunk), one launch.
//
// Every work-group of a row merges the row's statistics and walks the tree
// up to the first rejection.  The residual passes that follow are split into
// tickets, pass = ticket / C and chunk = ticket % C, handed out by an atomic
// counter to the row's work-groups in the order they ask.  A work-group
// computes the chunk of a ticket of the current pass and publishes its 32
// sums; holding a ticket of a later pass, it waits for the current pass's
// sums, which it may do because every chunk of that pass has been handed out
// to a running work-group, and continues the walk with them.  All of a row's
// work-groups thus walk the same way.  The holder of the first ticket past
// the last pass draws the final token; the last work-group of the row to
// finish clears the row's tickets and published sums for the next call.
// ============================================================================
template <typename ET, bool ALIGNED>
__global__ __launch_bounds__(WG) void tree_finish_kernel(TreeArgs a) {
  // Dynamic LDS: [2N * C * 4] partial words, [C * NSUB] residual sums, then
  // for a sparse draft [topk] kept ids, [topk] c q~ values, [topk]
  // corrections, [topk] kept logits and [topk] target probabilities at them.
  extern __shared__ __align__(16) uint32_t tcache[];
  __shared__ TreeRow tr;
  __shared__ float shsub[NSUB];
  __shared__ unsigned s_ticket;
  __shared__ float s_W;
  const int N = a.N, C = a.C;
  const int c = blockIdx.x % C, b = blockIdx.x / C;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t* pw = tcache;
  float* csub = reinterpret_cast<float*>(tcache + (size_t)2 * N * C * 4);
  int* kid = reinterpret_cast<int*>(csub + (size_t)C * NSUB);
  float* kq = reinterpret_cast<float*>(kid + a.topk);
  float* kcorr = kq + a.topk;
  float* kl = kcorr + a.topk;
  float* kp = kl + a.topk;
  float* probe = (c == 0 && a.probes) ? a.probes + (size_t)b * 3 * N : nullptr;
  // The row's partials and scalars in one round of loads.
  const u32x4* src = reinterpret_cast<const u32x4*>(tree_part(a, b, 0, 0));
  for (int i = t; i < 2 * N * C; i += WG) reinterpret_cast<u32x4*>(pw)[i] = src[i];
  int p = -1;
  if (t < N) {
    const size_t i = (size_t)b * N + t;
    tr.tok[t] = t == 0 ? -1 : a.tok[i];
    tr.u[t] = a.uni[i];
    tr.gt[t] = a.gath[i * 2];
    tr.gq[t] = a.gath[i * 2 + 1];
    if (t > 0) p = a.par[i];
  }
  if (t < MAX_NODES) tr.kids[t] = 0ull;
  const float T = a.temp[b];
  const bool greedy = !is_sampling_temperature(T);
  __syncthreads();
  // Children masks: node t sets its bit in its parent's mask.
  if (p >= 0 && p < t) atomicOr(&tr.kids[p], 1ull << t);
  __syncthreads();
  // Merge each node's chunk statistics (draft slots only where they exist).
  const float s = greedy ? 0.f : LOG2E / T;
  const bool sparse = a.topk > 0 && !greedy;
  if (C <= 16) tree_merge<16>(tr, pw, N, C, greedy, sparse, s);
  else if (C <= 32) tree_merge<32>(tr, pw, N, C, greedy, sparse, s);
  else tree_merge<64>(tr, pw, N, C, greedy, sparse, s);
  if (sparse && t < N && tr.kids[t] != 0ull) {
    // The truncated draft's statistics come from the merge kernel.
    const float4 q = a.qstat[(size_t)b * N + t];
    tr.M[N + t] = q.x;
    tr.Z[N + t] = q.y;
    tr.nk[t] = (int)q.w;
  }
  __syncthreads();
  if (t == 0) {
    tr.s = s;
    tr.greedy = greedy ? 1 : 0;
    tr.n = 0;
    tree_walk(tr, N, a.V, 0, 0, 0.f, 1.f, probe);
  }
  __syncthreads();
  auto emit = [&](int x, float S) {  // wave 0
    int32_t* out = a.out + (size_t)b * N;
    int32_t* on = a.onodes + (size_t)b * N;
    for (int i = lane; i < N; i += 64) {
      out[i] = i < tr.n ? tr.tok[tr.path[i]] : (i == tr.n ? x : -1);
      on[i] = i < tr.n ? tr.path[i] : -1;
    }
    if (lane == 0) {
      a.nacc[b] = tr.n;
      if (a.mass) a.mass[b] = S;
    }
  };
  if (tr.status != W_PASS) {
    // Finished without a residual pass: the chunk-0 work-group emits.
    if (c != 0 || wave != 0) return;
    float S = 0.f;
    const int x = tr.status == W_GREEDY
                      ? tr.x
                      : tree_draw<ET, ALIGNED>(a, tr, pw, csub, b, tr.v, tr.status, 0.f, tr.u[0], &S);
    emit(x, S);
    return;
  }
  // Residual passes.
  uint32_t* subR_row = a.subR + (size_t)b * N * C * NSUB;
  constexpr unsigned NONE = 0xFFFFFFFFu;
  int pass = 0;            // passes applied to the walk so far
  unsigned ticket = NONE;  // held ticket
  bool ok = true;
  if (sparse) {
    // A truncated draft: a pass needs no logits but the target's at the
    // kept ids (sparse_residual), so the chunk-0 work-group makes every pass
    // and the draw alone; the others only leave.
    if (c == 0) {
      int nk = 0, kv = -1;  // the node whose kept list and target probabilities are in LDS
      for (;;) {
        const int v = tr.v;
        const float MSt = mul_rn(tr.M[v], s), rZt = 1.f / tr.Z[v];
        if (v != kv) {
          // Node v's kept ids and logits, and the target's probabilities
          // there: the same for every pass at the node.
          nk = tr.nk[v];
          const uint2* kept = a.kept + ((size_t)b * N + v) * a.topk;
          const ET* trow = tree_row<ET>(a, false, b, v);
          for (int j = t; j < nk; j += WG) {
            const uint2 e = kept[j];
            kid[j] = (int)e.x;
            kl[j] = __uint_as_float(e.y);
            kp[j] = exp2_fast(fmaf(Tr<ET>::load1(trow + e.x), s, -MSt)) * rZt;
          }
          kv = v;
        }
        // This pass's c q~ at the kept ids.
        const float MSq = mul_rn(tr.M[N + v], s), rZq = tr.c / tr.Z[N + v];
        for (int j = t; j < nk; j += WG) kq[j] = exp2_fast(fmaf(kl[j], s, -MSq)) * rZq;
        __syncthreads();
        const uint32_t* gsub = a.subK + ((size_t)b * N + v) * C * NSUB;
        sparse_residual<ET>(
            a.V, C, a.CS, s, MSt, rZt, kid, kq, nk, kcorr, [&](int j) { return kp[j]; },
            [&](int cc, int u) { return __uint_as_float(gsub[cc * NSUB + u]); },
            [&](int cc) { return __uint_as_float(pw[((size_t)v * C + cc) * 4]); },
            [&](int i, float r) { csub[i] = r; });
        if (wave == 0) {
          float S;
          tree_draw<ET, ALIGNED>(a, tr, pw, csub, b, v, W_RESID, tr.c, -1.f, &S);
          if (lane == 0) s_W = S;
        }
        __syncthreads();
        if (t == 0) {
          if (s_W == 0.f)  // only through rounding: draw from the node's target
            tr.status = W_FALLBACK;
          else
            tree_walk(tr, N, a.V, tr.v, tr.j, tr.c, s_W, probe);
        }
        __syncthreads();
        if (tr.status != W_PASS) break;
      }
      // A residual draw uses the last pass's sums and kept list (its node
      // and scale are the walk's).
      if (wave == 0) {
        float S;
        const bool resid = tr.status == W_RESID;
        const int x = tree_draw<ET, ALIGNED>(a, tr, pw, csub, b, tr.v, tr.status, tr.c, tr.u[0], &S,
                                             resid ? kid : nullptr, kq, resid ? nk : 0);
        emit(x, S);
      }
    }
  }
  for (; !sparse;) {
    if (ticket == NONE) {
      if (t == 0) s_ticket = __hip_atomic_fetch_add(a.claim + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      ticket = s_ticket;
    }
    const int tp = (int)(ticket / (unsigned)C);
    if (tp == pass) {
      // A chunk of the current pass: its sums of max(0, p_v - c q_v).
      const int tc = (int)(ticket % (unsigned)C);
      tree_chunk_residual<ET, ALIGNED>(a, tr, b, tr.v, tr.c, tc, shsub);
      if (t < NSUB) pub_f32(subR_row + ((size_t)pass * C + tc) * NSUB + t, shsub[t]);
      ticket = NONE;
      continue;
    }
    // Every chunk of the current pass has been handed out: collect its sums.
    ok = wait_words(subR_row + (size_t)pass * C * NSUB, C * NSUB, reinterpret_cast<uint32_t*>(csub), nullptr, 0,
                    nullptr, wall_clock64() + WAIT_TICKS);
    if (!ok) break;
    if (wave == 0) {
      float S;
      tree_draw<ET, ALIGNED>(a, tr, pw, csub, b, tr.v, W_RESID, tr.c, -1.f, &S);
      if (lane == 0) s_W = S;
    }
    __syncthreads();
    if (t == 0) {
      if (s_W == 0.f)  // only through rounding: draw from the node's target
        tr.status = W_FALLBACK;
      else
        tree_walk(tr, N, a.V, tr.v, tr.j, tr.c, s_W, probe);
    }
    __syncthreads();
    ++pass;
    if (tr.status != W_PASS) break;
  }
  if (!ok) {
    // Reached only if a wait ran past its deadline: num_accepted = -1 marks it.
    for (int i = t; i < N; i += WG) {
      a.out[(size_t)b * N + i] = -1;
      a.onodes[(size_t)b * N + i] = -1;
    }
    if (t == 0) a.nacc[b] = -1;
  } else if (!sparse && ticket == (unsigned)pass * (unsigned)C) {
    if (wave == 0) {
      float S;
      const int x = tree_draw<ET, ALIGNED>(a, tr, pw, csub, b, tr.v, tr.status, tr.c, tr.u[0], &S);
      emit(x, S);
    }
  }
  // The last work-group of the row to finish clears its tickets and sums.
  __syncthreads();
  if (t == 0)
    s_ticket = __hip_atomic_fetch_add(a.leave + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)C - 1u;
  __syncthreads();
  if (!s_ticket) return;
  const int used = ok ? pass : N;
  for (int i = t; i < used * C * NSUB; i += WG) clear_word(subR_row + i);
  if (t == 0) {
    __hip_atomic_store(a.claim + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.leave + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
