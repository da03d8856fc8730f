// Early-exit verification: positions are verified one after the other and a
// row stops reading logits at its first rejection.  Included by
// spec_verify.hip inside its anonymous namespace, after finish_kernel; it
// uses that file's statistics arithmetic, published words, wait and draw.
//
// Sources: [nalar], subsection "Penolakan memendekkan pekerjaan speculative
// yang berguna" (after the first rejection no later draft is committed) and
// subsection "KV cache harus mengikuti token yang di-commit"; the decisions,
// the residual and the draws are those of spec_verify ([RheoSampling]
// section 4).  The result equals spec_verify's bit for bit: every sum is
// formed in the same order.
//
// The walk: one launch, one work-group per (row, chunk), numbered
// chunk-major.  A row's work is cut into stages: stage i <= n computes the chunk statistics
// of position i (target, and the draft of a sampling row); after a rejection
// at n one more stage computes the residual sums of position n.  Each stage
// is cut into tickets, one per chunk and slot, numbered consecutively across
// the stages and handed out by an agent-scope counter to the row's
// work-groups in the order they ask.  A work-group holding a ticket of the
// current stage computes that chunk and publishes it; holding a ticket of a
// later stage, it waits for the current stage's words -- every ticket of
// which has been handed out to a running work-group -- and takes the row's
// next decision with them.  So a stage is computed only once the decision
// before it has accepted, and no work-group waits for one that may not have
// started.  The holder of the first ticket past the last stage draws the
// final token; the last work-group of the row to finish clears the row's
// published words and counters for the next call.
//
// A truncated draft's exact selection does not depend on any decision, and
// made inside the walk it sat on every stage's critical path.  Such calls
// therefore run two launches first: the statistics kernel's body over
// position 0's target and every draft slot (candidate lists), then the merge
// kernel (every position's selection).  The walk then starts at its first
// decision, and each later stage holds the target's chunks only.

// Truncated drafts, the first of the call's three launches: one work-group
// per (row, slot, chunk) over position 0's target (slot 0) and the K draft
// slots (slots 1..K), with the statistics kernel's body: plain partial words
// for position 0, candidate lists for the drafts of sampling rows.
template <typename ET, bool ALIGNED, int WAVES>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(WAVES, WAVES))) void ee_first_kernel(Args a) {
  const int rest = blockIdx.x / a.C;
  const int j = rest % (a.K + 1);
  stats_body<ET, ALIGNED>(a, rest / (a.K + 1), j == 0 ? 0 : a.K + j, blockIdx.x % a.C);
}

// Statistics of one chunk of one slot (target position `pos`, or the draft
// of position `pos` when `draft`), published as the words spec_verify's
// statistics kernel writes; the bonus position also publishes its 32
// sub-block sums.
template <typename ET, bool ALIGNED>
__device__ __forceinline__ void ee_stats_chunk(const Args& a, int b, int pos, int c, bool greedy, bool draft,
                                               float s, float* shf, int* shi, float* shsub) {
  constexpr int VEC = Tr<ET>::VEC;
  const int K = a.K, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int lo = c * a.CS;
  const int len = min(a.CS, a.V - lo);
  const ET* row = draft ? draft_row<ET>(a, b, pos) : target_row<ET>(a, b, pos);
  u32x4 r[NV_TILE];
  load_tile<ET, ALIGNED, NV_TILE>(row, lo, len, r);
  const int d = pos < K ? a.tok[(size_t)b * K + pos] : -1;
  uint32_t* dst = part_words(a, b, draft ? K + 1 + pos : pos, c);
  if (greedy) {
    // The thread's argmax, lowest id among equal maxima: its max, then the
    // first of its logits (in id order) equal to it -- the value and id the
    // statistics kernel finds, with fewer live registers.
    const float mx = tile_max<ET, NV_TILE>(r);
    float bv = mx;
    int bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < NV_TILE; ++j)
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float x = Tr<ET>::at(r[j], k);
        if (bi == INT_MAX && x == mx) { bv = x; bi = lo + (j * WG + t) * VEC + k; }
      }
    if (bi == INT_MAX) bi = lo + t * VEC;  // a NaN maximum: the first logit, as an unspecified result
    block_argmax(bv, bi, shf, shi);
    if (t < 4) pub_u32(dst + t, t == 0 ? __float_as_uint(bv) : (t == 2 ? (uint32_t)bi : 0u));
    return;
  }
  // The sums in the statistics kernel's order.
  const float m = block_max(tile_max<ET, NV_TILE>(r), shf);
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
  if (!draft && (pos == K || a.topk > 0)) {
    // The 32 sub-block sums of the bonus position for the draw, and with a
    // truncated draft of every target position (its residual's mass).
#pragma unroll
    for (int j = 0; j < NV_TILE; ++j) {
      const float v = wave_sum(zj[j]);
      if (lane == 0) shsub[j * NWAVE + wave] = v;
    }
    __syncthreads();
    if (t < NSUB) pub_f32(uniform_ptr(sub_words(a, b, pos, c)) + t, shsub[t]);
  }
  if (t < 4) {
    uint32_t w = 0u;
    if (t == 0) w = __float_as_uint(m);
    if (t == 1) w = __float_as_uint(z);
    if (t == 3 && d >= lo && d < lo + len) w = __float_as_uint(Tr<ET>::load1(row + d));
    pub_u32(dst + t, w);
  }
}

// Sums of max(0, p_n - q_n) over the 32 sub-blocks of one chunk, published.
// Half a tile of each row at a time (sub-block (j, wave) is vector row j of
// the wave, so its sum is formed as in finish_kernel).
template <typename ET, bool ALIGNED>
__device__ __forceinline__ void ee_residual_chunk(const Args& a, int b, int n, int c, float s, float MSt, float rZt,
                                                  float MSq, float rZq, float* shsub) {
  constexpr int VEC = Tr<ET>::VEC;
  constexpr int H = NV_TILE / 2;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int lo = c * a.CS;
  const int len = min(a.CS, a.V - lo);
  const ET* trow = target_row<ET>(a, b, n);
  const ET* drow = draft_row<ET>(a, b, n);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 rt[H], rq[H];
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int e = ((h * H + j) * WG + t) * VEC;
      rt[j] = load_vec<ET, ALIGNED>(trow, lo + e, len - e);
      rq[j] = load_vec<ET, ALIGNED>(drow, lo + e, len - e);
    }
#pragma unroll
    for (int j = 0; j < H; ++j) {
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
      const float v = wave_sum(w0 + w1);
      if (lane == 0) shsub[(h * H + j) * NWAVE + wave] = v;
    }
  }
  __syncthreads();
  if (t < NSUB) pub_f32(uniform_ptr(a.subR + ((size_t)b * a.C + c) * NSUB) + t, shsub[t]);
}

// Merge of one slot's decoded chunk words (LDS) by one wave, in the order of
// decide_row.
__device__ __forceinline__ void ee_merge_slot(const Args& a, RowShared& rs, const uint32_t* pw, int slot,
                                              bool greedy, float s) {
  const int C = a.C, lane = threadIdx.x & 63;
  auto word = [&](int c, int w) { return __uint_as_float(pw[((size_t)slot * C + c) * 4 + w]); };
  if (greedy) {
    float bv = NEG_INF;
    int bi = INT_MAX;
    for (int c = lane; c < C; c += 64) argmax_merge(bv, bi, word(c, 0), __float_as_int(word(c, 2)));
    wave_argmax(bv, bi);
    if (lane == 0) { rs.M[slot] = bv; rs.Z[slot] = 0.f; rs.idx[slot] = bi; }
  } else {
    float m = NEG_INF;
    for (int c = lane; c < C; c += 64) m = fmaxf(m, word(c, 0));
    m = wave_max(m);
    const float MS = mul_rn(m, s);
    float z = 0.f;
    for (int c = lane; c < C; c += 64) {
      const float mc = word(c, 0), zc = word(c, 1);
      if (mc != NEG_INF) z += zc * exp2_fast(mul_rn(mc, s) - MS);
    }
    z = wave_sum(z);
    if (lane == 0) { rs.M[slot] = m; rs.Z[slot] = z; rs.idx[slot] = 0; }
  }
}

// SPARSE: the instantiation for truncated drafts, whose position-0
// statistics (plain words) and selections (qstat, kept) were written by the
// two launches before it.  Four waves per SIMD, two for truncated drafts
// over rows that are not 16-byte aligned (their element-wise loads need more
// registers; at four they would spill).  Stages go by ticket, so nothing
// here depends on how many work-groups are resident.
template <typename ET, bool ALIGNED, bool SPARSE>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(SPARSE && !ALIGNED ? 2 : 4))) void
early_exit_kernel(Args a) {
  // Dynamic LDS: [(2K+1) * C * 4] decoded words, [C * NSUB] sums, then for a
  // sparse draft [topk] kept ids, q~ values and corrections.
  extern __shared__ __align__(16) uint32_t ee_cache[];
  __shared__ RowShared rs;
  __shared__ float shf[NWAVE];
  __shared__ int shi[NWAVE];
  __shared__ float shsub[NSUB];
  __shared__ unsigned s_ticket;
  __shared__ int s_acc;
  const int K = a.K, C = a.C, S = 2 * K + 1;
  // Chunk-major numbering: the first work-groups to start are a few per row
  // for every row; later ones join their rows as slots free up (a row still
  // running by then gets the help, one already done is walked through).
  const int b = blockIdx.x % a.B, c = blockIdx.x / a.B;
  const int t = threadIdx.x, wave = t >> 6;
  uint32_t* pw = ee_cache;
  uint32_t* sub = ee_cache + (size_t)S * C * 4;
  int* kid = reinterpret_cast<int*>(sub + (size_t)C * NSUB);
  float* kq = reinterpret_cast<float*>(kid + a.topk);
  float* kcorr = kq + a.topk;
  // Sparse draft: every position's {max kept logit, Z_q, q~(d), kept count},
  // loaded once; the kept list is read by the drawer only.
  __shared__ float4 s_qst[SV_MAX_K];
  const float T = a.temp[b];
  const bool greedy = !is_sampling_temperature(T);
  const bool sparse = SPARSE && !greedy;
  const float s = greedy ? 0.f : LOG2E / T;
  if (t < K) rs.tok[t] = a.tok[(size_t)b * K + t];
  if (SPARSE && sparse && t < K) s_qst[t] = a.qstat[(size_t)b * K + t];
  if (t == 0) {
    rs.uK = a.uni[(size_t)b * (K + 1) + K];
    rs.greedy = greedy;
    rs.s = s;
  }
  if (a.probs && c == 0)
    for (int i = t; i < 2 * K; i += WG) a.probs[(size_t)b * 2 * K + i] = __builtin_nanf("");
  __syncthreads();
  constexpr unsigned NONE = 0xFFFFFFFFu;
  enum { STATS, RESID, DONE };
  int phase = STATS;       // what the current stage computes
  int pos = 0;             // position of the current stage
  unsigned base = 0;       // first ticket of the current stage
  unsigned ticket = NONE;  // held ticket
  bool ok = true;
  // A truncated draft's later stages hold the target only, and every
  // sampling row needs position i + 1's statistics once it accepts at i.
  // A work-group holding a ticket of the next stage computes that chunk
  // before it collects the current stage (one stage ahead at most), so the
  // next stage's loads overlap the current decision.  `ahead`: the held
  // ticket's chunk is computed; `went_ahead`: this work-group published a
  // chunk that may never be collected.
  bool ahead = false, went_ahead = false;
  // Tickets of the current stage: one per chunk and slot (a sampling
  // position below K has a target and a draft slot; with a truncated draft
  // position 0 is computed already and later positions hold the target only).
  auto stage_size = [&]() -> unsigned {
    if (SPARSE && phase == STATS && pos == 0) return 0u;
    return (phase == STATS && !SPARSE && !greedy && pos < K) ? 2u * C : (unsigned)C;
  };
  unsigned size = stage_size();
  for (;;) {
    if (ticket == NONE) {
      if (t == 0) s_ticket = __hip_atomic_fetch_add(a.claim + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      ticket = s_ticket;
    }
    if (ticket - base < size) {
      const int k = (int)(ticket - base);
      if (phase == STATS) {
        ee_stats_chunk<ET, ALIGNED>(a, b, pos, k % C, greedy, !SPARSE && k >= C, s, shf, shi, shsub);
      } else {
        const float MSt = mul_rn(rs.M[pos], s), rZt = 1.f / rs.Z[pos];
        const float MSq = mul_rn(rs.M[K + 1 + pos], s), rZq = 1.f / rs.Z[K + 1 + pos];
        ee_residual_chunk<ET, ALIGNED>(a, b, pos, k, s, MSt, rZt, MSq, rZq, shsub);
      }
      __syncthreads();  // the chunk's shared scratch is reused by the next one
      ticket = NONE;
      continue;
    }
    if (SPARSE && sparse && phase == STATS && !ahead && pos < K && ticket - base - size < (unsigned)C) {
      // A ticket of the next stage (position pos + 1, target only): its
      // chunk is the same whatever the current decision.
      ee_stats_chunk<ET, ALIGNED>(a, b, pos + 1, (int)(ticket - base - size), false, false, s, shf, shi, shsub);
      __syncthreads();
      ahead = went_ahead = true;
    }
    // Every chunk of the current stage has been handed out: collect it.
    if (phase == STATS) {
      const bool draft = !greedy && pos < K && !sparse;
      // The position's sub-block sums: the bonus position's for its draw,
      // and with a truncated draft every position's (its residual's mass).
      const bool sums = !greedy && (pos == K || sparse);
      if (SPARSE && pos == 0) {
        // Written by the statistics launch before this one: plain words.
        for (int i = t; i < C * 4; i += WG) pw[i] = part_words(a, b, 0, 0)[i];
        if (sums)
          for (int i = t; i < C * NSUB; i += WG) sub[i] = sub_words(a, b, 0, 0)[i];
      } else {
        ok = wait_words(part_words(a, b, pos, 0), C * 4, pw + (size_t)pos * C * 4,
                        draft ? part_words(a, b, K + 1 + pos, 0) : (sums ? sub_words(a, b, pos, 0) : nullptr),
                        draft ? C * 4 : (sums ? C * NSUB : 0),
                        draft ? pw + (size_t)(K + 1 + pos) * C * 4 : (sums ? sub : nullptr),
                        wall_clock64() + WAIT_TICKS);
      }
      if (!ok) break;
      if constexpr (SPARSE) if (sparse && pos < K && t == 0) {
        // The position's selection statistics, made by the merge kernel.
        rs.M[K + 1 + pos] = s_qst[pos].x;
        rs.Z[K + 1 + pos] = s_qst[pos].y;
      }
      if (wave == 0) ee_merge_slot(a, rs, pw, pos, greedy, s);
      if (wave == 1 && draft) ee_merge_slot(a, rs, pw, K + 1 + pos, greedy, s);
      __syncthreads();
      if (t == 0) {
        bool acc = false;
        if (pos < K) {
          // The acceptance test of decide_row at position pos.
          const int d = rs.tok[pos];
          if (greedy) {
            acc = d == rs.idx[pos];
          } else {
            float p = 0.f, q = 0.f;
            if (d >= 0 && d < a.V) {
              const int cd = d / a.CS;
              const float lt = __uint_as_float(pw[((size_t)pos * C + cd) * 4 + 3]);
              p = exp2_fast(fmaf(lt, s, -mul_rn(rs.M[pos], s))) / rs.Z[pos];
              if (sparse) {
                q = s_qst[pos].z;  // q~(d) of the truncated draft
              } else {
                const float lq = __uint_as_float(pw[((size_t)(K + 1 + pos) * C + cd) * 4 + 3]);
                q = exp2_fast(fmaf(lq, s, -mul_rn(rs.M[K + 1 + pos], s))) / rs.Z[K + 1 + pos];
              }
            }
            const float u = a.uni[(size_t)b * (K + 1) + pos];
            acc = u * q < p;
            if (a.probs && c == 0) {
              a.probs[((size_t)b * K + pos) * 2 + 0] = p;
              a.probs[((size_t)b * K + pos) * 2 + 1] = q;
            }
          }
        }
        s_acc = acc;
      }
      __syncthreads();
      base += size;
      if (s_acc) {
        ++pos;
      } else {
        // A truncated draft's residual is formed by the drawer (no pass).
        phase = (greedy || pos == K || sparse) ? DONE : RESID;
      }
    } else {
      ok = wait_words(a.subR + (size_t)b * C * NSUB, C * NSUB, sub, nullptr, 0, nullptr,
                      wall_clock64() + WAIT_TICKS);
      if (!ok) break;
      base += size;
      phase = DONE;
    }
    if (phase == DONE) break;
    size = stage_size();
    if (ahead) {
      // The held ticket is in the new current stage and already computed.
      ahead = false;
      ticket = NONE;
    }
  }
  if (!ok) {
    write_failed_row(a, b);
  } else if (ticket == base) {
    // The holder of the first ticket past the last stage draws and emits.
    const int n = pos;
    if (greedy) {
      int32_t* out = a.out + (size_t)b * (K + 1);
      for (int i = t; i <= K; i += WG) out[i] = i < n ? rs.tok[i] : (i == n ? rs.idx[n] : -1);
      if (t == 0) {
        a.nacc[b] = n;
        if (a.mass) a.mass[b] = 0.f;
      }
    } else {
      const float MSt = mul_rn(rs.M[n], s), rZt = 1.f / rs.Z[n];
      const float MSq = n < K ? mul_rn(rs.M[K + 1 + n], s) : 0.f;
      const float rZq = n < K ? 1.f / rs.Z[K + 1 + n] : 0.f;
      const RowView<true> view{pw, sub, true};
      if constexpr (SPARSE) {
        const int nkept = sparse && n < K ? (int)s_qst[n].w : 0;
        if (sparse && n < K) {
          // Position n's kept list (ids and q~ values), then the residual's
          // sub-block sums from its sums (in `sub`) and the list, in place.
          const uint2* kept = a.kept + ((size_t)b * K + n) * a.topk;
          for (int j = t; j < nkept; j += WG) {
            const uint2 e = kept[j];
            kid[j] = (int)e.x;
            kq[j] = exp2_fast(fmaf(__uint_as_float(e.y), s, -MSq)) * rZq;
          }
          __syncthreads();
          float* R = reinterpret_cast<float*>(sub);
          const ET* trow = target_row<ET>(a, b, n);
          sparse_residual<ET>(
              a.V, C, a.CS, s, MSt, rZt, kid, kq, nkept, kcorr,
              [&](int j) { return exp2_fast(fmaf(Tr<ET>::load1(trow + kid[j]), s, -MSt)) * rZt; },
              [&](int cc, int u) { return R[cc * NSUB + u]; },
              [&](int cc) { return __uint_as_float(pw[((size_t)n * C + cc) * 4]); },
              [&](int i, float r) { R[i] = r; });
        }
        final_draw<ET, ALIGNED, true>(a, b, n, s, MSt, rZt, MSq, rZq, rs, view, sparse ? kid : nullptr, kq, nkept);
      } else {
        final_draw<ET, ALIGNED, true>(a, b, n, s, MSt, rZt, MSq, rZq, rs, view, nullptr, nullptr, 0);
      }
    }
  }
  // The last work-group of the row to finish clears its published words.
  // A chunk computed ahead may be one nobody collects: its stores complete
  // before this work-group counts itself, so the clear comes after them.
  if (went_ahead) wait_vmem();
  __syncthreads();
  if (t == 0)
    s_ticket = __hip_atomic_fetch_add(a.leave + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)C - 1u;
  __syncthreads();
  if (!s_ticket) return;
  // Positions whose words may have been published (with a truncated
  // draft, one past the last decision: a chunk computed ahead).
  const int last = ok ? (SPARSE && sparse ? min(pos + 1, K) : pos) : K;
  for (int i = t; i < (last + 1) * C * 4; i += WG) clear_word(part_words(a, b, 0, 0) + i);
  if (!greedy || !ok)
    for (int i = t; i < min(last + 1, K) * C * 4; i += WG) clear_word(part_words(a, b, K + 1, 0) + i);
  if (SPARSE && (!ok || !greedy)) {
    // Every position reached published its sums (position 0's are plain).
    for (int i = t; i < (last + 1) * C * NSUB; i += WG) clear_word(sub_words(a, b, 0, 0) + i);
  } else if (!ok || (!greedy && pos == K)) {
    for (int i = t; i < C * NSUB; i += WG) clear_word(sub_words(a, b, K, 0) + i);
  }
  if (!ok || (!greedy && pos < K))
    for (int i = t; i < C * NSUB; i += WG) clear_word(a.subR + (size_t)b * C * NSUB + i);
  if (t == 0) {
    __hip_atomic_store(a.claim + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.leave + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
