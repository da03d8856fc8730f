// Batched speculative-sampling verifier: HIP kernels for gfx950 and the C ABI.
//
// Sources (cited by page title and section):
//   [RheoSampling] "RheoSampling 2026: Mengatasi Dilema One-Hot pada
//     Stochastic Dynamic-Tree Speculative Decoding, ..." (newsaint.id):
//     section 3 (top-128 draft truncation), section 4 (acceptance with
//     min(1, p/q~), residual norm(max(0, p - q~))), section 7 (temperature at
//     the verification gate; truncation inside the GPU kernel).
//   [nalar] "Speculative decoding: memverifikasi token draft sebelum
//     diterima" (nalar.dev): batched verification of all draft positions from
//     one target pass, greedy vs sampling semantics, first-rejection cut.
//
// Two launches per call, both on the caller's stream:
//
//   A. stats_kernel, one work-group per (row, position, vocabulary chunk).
//      Streams its chunk of target or draft logits once from HBM (16-byte
//      loads into a register tile) and writes the chunk max and the sum of
//      exp2((l - max) * log2(e)/T) -- or, for greedy rows, the chunk argmax.
//      The chunk holding a position's draft token records that token's
//      logit; the bonus position also writes 32 sub-block sums for the final
//      draw.  No work-group waits for or talks to another.
//   B. finish_kernel, one work-group per (row, chunk).  Each work-group
//      merges its row's partials and runs the first-rejection scan.  Greedy
//      rows and rows that accepted every draft are completed by the row's
//      work-group 0.  For a rejected row every work-group re-reads target and
//      draft logits of the rejected position in its chunk and publishes 32
//      sub-block sums of max(0, p_n - q_n); the last work-group of the row to
//      finish (atomic counter) draws the correction token.
//
// The final draw is an inverse CDF over a three-level hierarchy: chunk
// masses (block scan), the 32 sub-block sums of the selected chunk, and a
// block prefix sum over the 512 (bf16) or 256 (fp32) ids of the selected
// sub-block.
//
// Numerical conventions.  With s = log2(e)/T and MS = fl(M*s) for a max M,
// every exponential is exp2(fma(l, s, -MS)); sums computed against a chunk
// max m are rescaled by exp2(fl(m*s) - fl(M*s)), so the rounding of the
// reference products cancels between numerator and denominator.  All
// reductions combine partial results in a fixed order (no float atomics), so
// outputs are bitwise reproducible.
//
// Cross-work-group hand-off inside B: a work-group publishes its 32 sums
// with write-through agent-scope atomic stores, waits for them to complete,
// then increments its row's counter; the work-group that observes the final
// count reads the others' sums with agent-scope atomic loads and resets the
// counter to zero for the next call.  Nothing ever waits on another
// work-group.

#include <climits>
#include <cstddef>
#include <cstdint>

#include "spec_verify.h"
#include "sv_device.h"

using namespace sv;

namespace {

constexpr int NV_TILE = 8;                 // 16-byte vectors per thread per chunk
constexpr int NSUB = NV_TILE * NWAVE;      // sub-blocks per chunk (one wave x one vector row)
constexpr int MAX_C = 2048;                // vocabulary chunks per position
constexpr int MAX_SLOTS = 2 * SV_MAX_K + 1;

struct Args {
  const void* tgt;           // [B, K+1, V]
  const void* dft;           // [B, K, V]
  const int32_t* tok;        // [B, K]
  const float* uni;          // [B, K+1]
  const float* temp;         // [B]
  int32_t* out;              // [B, K+1]
  int32_t* nacc;             // [B]
  float* probs;              // [B, K, 2] or null
  float* mass;               // [B] or null
  float4* part;              // [B, 2K+1, C] {max | argmax value, sum, argmax id bits, 0}
  float* ldv;                // [B, 2K+1] logit of the position's draft token
  float* subK;               // [B, C, NSUB] bonus-position sub-block sums (vs chunk max)
  float* subR;               // [B, C, NSUB] residual sub-block sums
  unsigned* cnt;             // [B] zero between calls
  int B, K, V, C, CS, topk;
};

__device__ __forceinline__ size_t part_index(const Args& a, int b, int slot, int c) {
  return ((size_t)b * (2 * a.K + 1) + slot) * (size_t)a.C + c;
}
template <typename ET>
__device__ __forceinline__ const ET* target_row(const Args& a, int b, int i) {
  return static_cast<const ET*>(a.tgt) + ((size_t)b * (a.K + 1) + i) * (size_t)a.V;
}
template <typename ET>
__device__ __forceinline__ const ET* draft_row(const Args& a, int b, int i) {
  return static_cast<const ET*>(a.dft) + ((size_t)b * a.K + i) * (size_t)a.V;
}
__device__ __forceinline__ float mul_rn(float x, float y) { return __fmul_rn(x, y); }
// Rows with T > 0 (including +inf) sample; T <= 0, -0 and NaN are greedy.
__device__ __forceinline__ bool is_sampling_temperature(float T) {
  return __float_as_uint(T) - 1u < 0x7F800000u;
}

// One 16-byte vector at element offset pos of a row, -inf past `rem` elements.
template <typename ET, bool ALIGNED>
__device__ __forceinline__ u32x4 load_vec(const ET* __restrict__ row, int pos, int rem) {
  constexpr int VEC = Tr<ET>::VEC;
  if (ALIGNED && rem >= VEC) return *reinterpret_cast<const u32x4*>(row + pos);
  const uint32_t f = Tr<ET>::NEG_INF_WORD;
  u32x4 v = {f, f, f, f};
#pragma unroll
  for (int k = 0; k < VEC; ++k)
    if (k < rem) Tr<ET>::set(v, k, row + pos + k);
  return v;
}

// Largest logit of a register tile (bf16: both halves of each word widened
// exactly, as in the exponential pass, which reuses them).
template <typename ET, int NV>
__device__ __forceinline__ float tile_max(const u32x4 (&r)[NV]);

template <>
__device__ __forceinline__ float tile_max<uint16_t, NV_TILE>(const u32x4 (&r)[NV_TILE]) {
  float m0 = NEG_INF, m1 = NEG_INF, m2 = NEG_INF, m3 = NEG_INF;
#pragma unroll
  for (int j = 0; j < NV_TILE; ++j) {
    m0 = max3_raw(m0, Tr<uint16_t>::at(r[j], 0), Tr<uint16_t>::at(r[j], 1));
    m1 = max3_raw(m1, Tr<uint16_t>::at(r[j], 2), Tr<uint16_t>::at(r[j], 3));
    m2 = max3_raw(m2, Tr<uint16_t>::at(r[j], 4), Tr<uint16_t>::at(r[j], 5));
    m3 = max3_raw(m3, Tr<uint16_t>::at(r[j], 6), Tr<uint16_t>::at(r[j], 7));
  }
  return max3_raw(max3_raw(m0, m1, m2), m3, m3);
}

template <>
__device__ __forceinline__ float tile_max<float, NV_TILE>(const u32x4 (&r)[NV_TILE]) {
  float m0 = NEG_INF, m1 = NEG_INF;
#pragma unroll
  for (int j = 0; j < NV_TILE; ++j) {
    m0 = max3_raw(m0, __uint_as_float(r[j].x), __uint_as_float(r[j].y));
    m1 = max3_raw(m1, __uint_as_float(r[j].z), __uint_as_float(r[j].w));
  }
  return max3_raw(m0, m1, m1);
}

// ============================================================================
// Kernel A: per-chunk statistics.
// ============================================================================
template <typename ET, bool ALIGNED>
__global__ __launch_bounds__(WG) void stats_kernel(Args a) {
  constexpr int VEC = Tr<ET>::VEC;
  const int S = 2 * a.K + 1;
  const int c = blockIdx.x % a.C;
  const int rest = blockIdx.x / a.C;
  const int slot = rest % S;
  const int b = rest / S;
  const float T = a.temp[b];
  const bool greedy = !is_sampling_temperature(T);
  const bool is_draft = slot > a.K;
  // Greedy rows never read the draft.
  if (is_draft && greedy) return;
  const int pos = is_draft ? slot - a.K - 1 : slot;
  const ET* row = is_draft ? draft_row<ET>(a, b, pos) : target_row<ET>(a, b, pos);
  const int lo = c * a.CS;
  const int len = min(a.CS, a.V - lo);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

  u32x4 r[NV_TILE];
  load_tile<ET, ALIGNED, NV_TILE>(row, lo, len, r);

  __shared__ float shf[NWAVE];
  __shared__ int shi[NWAVE];
  __shared__ float shsub[NSUB];
  float4* dst = a.part + part_index(a, b, slot, c);

  if (greedy) {
    // Argmax of raw logits, lowest id among equal maxima.  A thread visits its
    // elements in increasing id order, so a strict '>' keeps the first; its
    // real elements precede the -inf padding.
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
    if (t == 0) *dst = make_float4(bv, 0.f, __int_as_float(bi), 0.f);
    return;
  }

  const float m = block_max(tile_max<ET, NV_TILE>(r), shf);
  const float s = LOG2E / T;
  const float ms = mul_rn(m, s);
  // A chunk of -inf only would give exp2(nan): use the reference 0 then
  // (every term is exp2(-inf) = 0).
  const float msr = m == NEG_INF ? 0.f : ms;
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
  if (slot == a.K) {
    // Sub-block sums of the bonus position: sub-block (j, wave) holds the
    // 64 * VEC consecutive ids of vector row j owned by that wave.
#pragma unroll
    for (int j = 0; j < NV_TILE; ++j) {
      const float v = wave_sum(zj[j]);
      if (lane == 0) shsub[j * NWAVE + wave] = v;
    }
    __syncthreads();
    if (t < NSUB) a.subK[((size_t)b * a.C + c) * NSUB + t] = shsub[t];
  }
  if (t == 0) {
    *dst = make_float4(m, z, 0.f, 0.f);
    if (pos < a.K) {
      const int d = a.tok[(size_t)b * a.K + pos];
      if (d >= lo && d < lo + len) a.ldv[(size_t)b * S + slot] = Tr<ET>::load1(row + d);
    }
  }
}

// ============================================================================
// Row decision from the statistics partials (kernel B, every work-group).
// ============================================================================
struct RowShared {
  float M[MAX_SLOTS];    // position max (sampling) or argmax value (greedy)
  float Z[MAX_SLOTS];    // sum of exp2(fma(l, s, -fl(M*s)))
  int idx[MAX_SLOTS];    // argmax id (greedy)
  float p[SV_MAX_K];     // p_i(d_i)
  float q[SV_MAX_K];     // q_i(d_i)
  int tok[SV_MAX_K];
  float red_f[NWAVE];
  int n;                 // accepted drafts
  int greedy;
  float s;               // log2(e)/T
};

__device__ void decide_row(const Args& a, int b, RowShared& rs) {
  const int K = a.K, C = a.C, S = 2 * K + 1, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float T = a.temp[b];
  const bool greedy = !is_sampling_temperature(T);
  const float s = greedy ? 0.f : LOG2E / T;
  // Per-position inputs, issued before the merge so that their latency
  // overlaps it.
  int d = -1;
  float u = 0.f, lt = 0.f, lq = 0.f;
  if (t < K) {
    d = a.tok[(size_t)b * K + t];
    u = a.uni[(size_t)b * (K + 1) + t];
    lt = a.ldv[(size_t)b * S + t];
    lq = a.ldv[(size_t)b * S + K + 1 + t];
  }
  const int nmerge = (greedy || a.topk > 0) ? K + 1 : 2 * K + 1;
  for (int slot = wave; slot < nmerge; slot += NWAVE) {
    const float4* p = a.part + part_index(a, b, slot, 0);
    if (greedy) {
      float bv = NEG_INF;
      int bi = INT_MAX;
      for (int c = lane; c < C; c += 64) {
        const float4 v = p[c];
        argmax_merge(bv, bi, v.x, __float_as_int(v.z));
      }
      wave_argmax(bv, bi);
      if (lane == 0) { rs.M[slot] = bv; rs.Z[slot] = 0.f; rs.idx[slot] = bi; }
    } else {
      float m = NEG_INF;
      for (int c = lane; c < C; c += 64) m = fmaxf(m, p[c].x);
      m = wave_max(m);
      const float MS = mul_rn(m, s);
      float z = 0.f;
      for (int c = lane; c < C; c += 64) {
        const float4 pc = p[c];
        if (pc.x != NEG_INF) z += pc.y * exp2_fast(mul_rn(pc.x, s) - MS);
      }
      z = wave_sum(z);
      if (lane == 0) { rs.M[slot] = m; rs.Z[slot] = z; rs.idx[slot] = 0; }
    }
  }
  __syncthreads();
  if (wave == 0) {
    // Acceptance test of every position at once ([RheoSampling] section 4
    // step 1: u*q < p; [nalar] greedy rule: draft equals the argmax), then
    // the first rejection by ballot (K <= 64 positions fit one wave).
    bool acc = true;
    if (t < K) {
      float p = 0.f, q = 0.f;
      if (!greedy && d >= 0 && d < a.V) {
        p = exp2_fast(fmaf(lt, s, -mul_rn(rs.M[t], s))) / rs.Z[t];
        q = exp2_fast(fmaf(lq, s, -mul_rn(rs.M[K + 1 + t], s))) / rs.Z[K + 1 + t];
      }
      rs.p[t] = p;
      rs.q[t] = q;
      rs.tok[t] = d;
      acc = greedy ? (d == rs.idx[t]) : (u * q < p);
    }
    const unsigned long long rej = __ballot(!acc);
    if (t == 0) {
      rs.n = rej ? (int)__builtin_ctzll(rej) : K;
      rs.greedy = greedy;
      rs.s = s;
    }
  }
  __syncthreads();
}

// ============================================================================
// Inverse-CDF search inside an id range [start, start + len) of one row.
// Weights: p(x) = exp2(fma(l_t, s, -MSt)) * rZt, or max(0, p(x) - q(x)) when
// a draft row is given.  Returns the smallest id whose cumulative weight
// (from start) exceeds tl; if none does (only through rounding), the last id
// with positive weight, else start.  Segments of WG * VEC ids are scanned in
// order with a block prefix sum.
// ============================================================================
template <typename ET, bool ALIGNED>
__device__ int range_search(const ET* __restrict__ trow, const ET* __restrict__ drow, int start, int len,
                            float tl, float s, float MSt, float rZt, float MSq, float rZq, float* red) {
  constexpr int VEC = Tr<ET>::VEC;
  __shared__ int sh_first, sh_last;
  const int t = threadIdx.x;
  if (t == 0) { sh_first = INT_MAX; sh_last = -1; }
  __syncthreads();
  float carry = 0.f;
  int last_pos = -1;
  for (int seg = 0; seg < len; seg += WG * VEC) {
    const int e = seg + t * VEC;
    const u32x4 vt = load_vec<ET, ALIGNED>(trow, start + e, len - e);
    u32x4 vq = vt;
    if (drow) vq = load_vec<ET, ALIGNED>(drow, start + e, len - e);
    float w[VEC];
    float local = 0.f;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      const float p = exp2_fast(fmaf(Tr<ET>::at(vt, k), s, -MSt)) * rZt;
      float wk = p;
      if (drow) wk = fmaxf(0.f, p - exp2_fast(fmaf(Tr<ET>::at(vq, k), s, -MSq)) * rZq);
      w[k] = wk;
      local += wk;
    }
    float excl, total;
    block_scan(local, red, excl, total);
    float cum = carry + excl;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      const bool in = e + k < len;
      cum += w[k];
      if (in && w[k] > 0.f) last_pos = start + e + k;
      if (in && cum > tl) { atomicMin(&sh_first, start + e + k); break; }
    }
    __syncthreads();
    if (sh_first != INT_MAX) break;
    carry += total;
  }
  if (last_pos >= 0) atomicMax(&sh_last, last_pos);
  __syncthreads();
  const int x = sh_first != INT_MAX ? sh_first : (sh_last >= 0 ? sh_last : start);
  __syncthreads();
  return x;
}

// ============================================================================
// Final draw for a sampling row ([RheoSampling] section 4 step 3): from the
// residual sub-block sums (n < K) or the bonus position's sub-block sums
// (n == K).  Writes out_tokens / num_accepted / mass.
// ============================================================================
template <typename ET, bool ALIGNED>
__device__ void final_draw(const Args& a, int b, int n, float s, float MSt, float rZt, float MSq,
                           float rZq, float* red) {
  constexpr int VEC = Tr<ET>::VEC;
  __shared__ int sh_i, sh_last;
  __shared__ float sh_tl;
  const int K = a.K, C = a.C, t = threadIdx.x;
  const bool reject = n < K;
  // mode 0: residual sub-block sums; 1: bonus sub-block sums (rescaled from
  // the chunk max); 2: target chunk masses from the statistics partials
  // (fallback for a zero residual, reachable only through rounding).
  int mode = reject ? 0 : 1;
  auto bonus_scale = [&](int c) {
    const float mc = pub_load(&a.part[part_index(a, b, K, c)].x);
    return mc == NEG_INF ? 0.f : exp2_fast(mul_rn(mc, s) - MSt) * rZt;
  };
  // Mass of chunk c: the ordered sum of its sub-block sums.
  auto chunk_mass = [&](int c) {
    if (c >= C) return 0.f;
    if (mode == 2) {
      const float4 v = pub_load4(&a.part[part_index(a, b, n, c)]);
      return v.x == NEG_INF ? 0.f : v.y * exp2_fast(mul_rn(v.x, s) - MSt) * rZt;
    }
    const float* sub = (mode == 0 ? a.subR : a.subK) + ((size_t)b * C + c) * NSUB;
    const float sc = mode == 0 ? 1.f : bonus_scale(c);
    float acc = 0.f;
    for (int q = 0; q < NSUB; ++q) acc += mode == 0 ? pub_load(sub + q) : pub_load(sub + q) * sc;
    return acc;
  };
  // Pass 1: total mass S (tiles of WG chunks, block scans in a fixed order).
  auto total_mass = [&]() {
    float carry = 0.f;
    for (int base = 0; base < C; base += WG) {
      float ex, tot;
      block_scan(chunk_mass(base + t), red, ex, tot);
      carry += tot;
    }
    return carry;
  };
  float S = total_mass();
  if (reject && S == 0.f) {
    mode = 2;
    S = total_mass();
  }
  const float tv = a.uni[(size_t)b * (K + 1) + K] * S;
  // Pass 2: the first chunk whose inclusive prefix exceeds t (same sums).
  if (t == 0) { sh_i = INT_MAX; sh_last = 0; }
  __syncthreads();
  float carry = 0.f;
  for (int base = 0; base < C; base += WG) {
    const int c = base + t;
    const float v = chunk_mass(c);
    float ex, tot;
    const float in = block_scan(v, red, ex, tot);
    if (c < C && v > 0.f) atomicMax(&sh_last, c);
    if (c < C && carry + in > tv) atomicMin(&sh_i, c);
    __syncthreads();
    const int hit = sh_i;
    if (hit != INT_MAX) {
      if (c == hit) sh_tl = tv - (carry + ex);
      break;
    }
    carry += tot;
  }
  __syncthreads();
  int cs = sh_i;
  float t1 = sh_tl;
  if (cs == INT_MAX) {   // t reached the total only through rounding
    cs = sh_last;
    t1 = __builtin_inff();
  }
  __syncthreads();
  const int lo = cs * a.CS;
  const int len = min(a.CS, a.V - lo);
  const ET* trow = target_row<ET>(a, b, n);
  const ET* drow = mode == 0 ? draft_row<ET>(a, b, n) : nullptr;
  int start = lo, slen = len;
  float tl = t1;
  if (mode != 2) {
    // Sub-block of the selected chunk, by a sequential scan of its sums
    // (the same sequence of additions that gave the chunk mass).
    if (t == 0) {
      const float* sub = (mode == 0 ? a.subR : a.subK) + ((size_t)b * C + cs) * NSUB;
      const float sc = mode == 0 ? 1.f : bonus_scale(cs);
      float cum = 0.f;
      int qs = -1, qlast = 0;
      float tq = __builtin_inff();
      for (int q = 0; q < NSUB; ++q) {
        const float v = mode == 0 ? pub_load(sub + q) : pub_load(sub + q) * sc;
        if (v > 0.f) qlast = q;
        if (qs < 0 && cum + v > t1) { qs = q; tq = t1 - cum; }
        cum += v;
      }
      if (qs < 0) qs = qlast;
      sh_i = qs;
      sh_tl = tq;
    }
    __syncthreads();
    const int q = sh_i;
    tl = sh_tl;
    const int j = q / NWAVE, w = q % NWAVE;
    start = lo + (j * WG + w * 64) * VEC;
    slen = max(0, min(64 * VEC, lo + len - start));
    __syncthreads();
  }
  int x = lo;
  if (slen > 0) x = range_search<ET, ALIGNED>(trow, drow, start, slen, tl, s, MSt, rZt, MSq, rZq, red);
  int32_t* out = a.out + (size_t)b * (K + 1);
  for (int i = t; i <= K; i += WG) out[i] = i < n ? a.tok[(size_t)b * K + i] : (i == n ? x : -1);
  if (t == 0) {
    a.nacc[b] = n;
    if (a.mass) a.mass[b] = S;
  }
}

// ============================================================================
// Kernel B: row decision, completion of greedy and bonus rows, residual
// sub-block sums of rejected rows and their correction draw.
// ============================================================================
template <typename ET, bool ALIGNED>
__global__ __launch_bounds__(WG) void finish_kernel(Args a) {
  constexpr int VEC = Tr<ET>::VEC;
  const int c = blockIdx.x % a.C;
  const int b = blockIdx.x / a.C;
  const int K = a.K, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  __shared__ RowShared rs;
  __shared__ float shsub[NSUB];
  __shared__ int sh_flag;
  decide_row(a, b, rs);
  const int n = rs.n;
  if (c == 0 && a.probs && t < K) {
    a.probs[((size_t)b * K + t) * 2 + 0] = rs.greedy ? 0.f : rs.p[t];
    a.probs[((size_t)b * K + t) * 2 + 1] = rs.greedy ? 0.f : rs.q[t];
  }
  if (rs.greedy) {
    if (c != 0) return;
    // The target's argmax replaces the first mismatch or fills the bonus slot.
    int32_t* out = a.out + (size_t)b * (K + 1);
    for (int i = t; i <= K; i += WG) out[i] = i < n ? rs.tok[i] : (i == n ? rs.idx[n] : -1);
    if (t == 0) {
      a.nacc[b] = n;
      if (a.mass) a.mass[b] = 0.f;
    }
    return;
  }
  const float s = rs.s;
  const float MSt = mul_rn(rs.M[n], s), rZt = 1.f / rs.Z[n];
  if (n == K) {
    if (c == 0) final_draw<ET, ALIGNED>(a, b, n, s, MSt, rZt, 0.f, 0.f, rs.red_f);
    return;
  }
  // Rejected at position n: residual max(0, p_n - q_n) over this chunk.
  const float MSq = mul_rn(rs.M[K + 1 + n], s), rZq = 1.f / rs.Z[K + 1 + n];
  const int lo = c * a.CS;
  const int len = min(a.CS, a.V - lo);
  u32x4 rt[NV_TILE], rq[NV_TILE];
  load_tile<ET, ALIGNED, NV_TILE>(target_row<ET>(a, b, n), lo, len, rt);
  load_tile<ET, ALIGNED, NV_TILE>(draft_row<ET>(a, b, n), lo, len, rq);
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
    const float v = wave_sum(w0 + w1);
    if (lane == 0) shsub[j * NWAVE + wave] = v;
  }
  __syncthreads();
  if (t < NSUB) pub_store(a.subR + ((size_t)b * a.C + c) * NSUB + t, shsub[t]);
  if (t < 64) wait_vmem();
  __syncthreads();
  if (t == 0)
    sh_flag = __hip_atomic_fetch_add(a.cnt + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)a.C - 1u;
  __syncthreads();
  if (sh_flag) {
    final_draw<ET, ALIGNED>(a, b, n, s, MSt, rZt, MSq, rZq, rs.red_f);
    if (t == 0) a.cnt[b] = 0;
  }
}

// ============================================================================
// Host side.
// ============================================================================
struct Plan {
  int C = 0, CS = 0;
  size_t off_cnt = 0, off_part = 0, off_ldv = 0, off_subK = 0, off_subR = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int make_plan(int B, int K, int V, int topk, int dtype, Plan& pl) {
  if (B < 1 || K < 0 || V < 1 || topk < 0 || (dtype != SV_BF16 && dtype != SV_F32)) return SV_ERR_ARG;
  if (K > SV_MAX_K) return SV_ERR_UNSUPPORTED;
  if (topk > 0 && topk < V) return SV_ERR_UNSUPPORTED;  // sparse drafts: not built yet
  const long vec = dtype == SV_BF16 ? 8 : 4;
  const long tile = (long)WG * NV_TILE * vec;
  long C = (V + tile - 1) / tile;
  if (C > MAX_C) return SV_ERR_UNSUPPORTED;
  long CS = ((V + C - 1) / C + vec - 1) / vec * vec;
  C = (V + CS - 1) / CS;
  const long long grid = (long long)B * (2 * K + 1) * C;
  if (grid > INT_MAX) return SV_ERR_UNSUPPORTED;
  pl.C = (int)C;
  pl.CS = (int)CS;
  const size_t S = 2 * (size_t)K + 1;
  size_t off = 0;
  pl.off_cnt = off;   // per-row counters: zero before the first call, zero after every call
  off = align256(off + sizeof(unsigned) * (size_t)B);
  pl.off_part = off;
  off = align256(off + sizeof(float4) * (size_t)B * S * C);
  pl.off_ldv = off;
  off = align256(off + sizeof(float) * (size_t)B * S);
  pl.off_subK = off;
  off = align256(off + sizeof(float) * (size_t)B * C * NSUB);
  pl.off_subR = off;
  off = align256(off + sizeof(float) * (size_t)B * C * NSUB);
  pl.total = off;
  return SV_OK;
}

template <typename ET, bool AL>
int launch_typed(const Args& a, const Plan& pl, hipStream_t st, hipEvent_t* ev) {
  const dim3 blk(WG);
  const int S = 2 * a.K + 1;
  if (ev && hipEventRecord(ev[0], st) != hipSuccess) return SV_ERR_HIP;
  hipLaunchKernelGGL((stats_kernel<ET, AL>), dim3(a.B * S * pl.C), blk, 0, st, a);
  if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
  if (ev && hipEventRecord(ev[1], st) != hipSuccess) return SV_ERR_HIP;
  if (ev && hipEventRecord(ev[2], st) != hipSuccess) return SV_ERR_HIP;
  hipLaunchKernelGGL((finish_kernel<ET, AL>), dim3(a.B * pl.C), blk, 0, st, a);
  if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
  if (ev && hipEventRecord(ev[3], st) != hipSuccess) return SV_ERR_HIP;
  if (ev && hipEventRecord(ev[4], st) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

int run(const void* tgt, const void* dft, const int32_t* tok, const float* uni, const float* temp,
        int B, int K, int V, int topk, int dtype, int32_t* out, int32_t* nacc, void* ws,
        size_t* ws_bytes, hipStream_t st, float* probs, float* mass, hipEvent_t* ev, int nev) {
  if (!ws_bytes) return SV_ERR_ARG;
  if (topk >= V) topk = 0;
  Plan pl;
  const int rc = make_plan(B, K, V, topk, dtype, pl);
  if (rc != SV_OK) return rc;
  if (!ws) {
    *ws_bytes = pl.total;
    return SV_OK;
  }
  if (*ws_bytes < pl.total) return SV_ERR_WORKSPACE;
  if (!tgt || !uni || !temp || !out || !nacc) return SV_ERR_ARG;
  if (K > 0 && (!dft || !tok)) return SV_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return SV_ERR_ARG;
  if (nev != 0 && (nev != 5 || !ev)) return SV_ERR_ARG;
  Args a;
  a.tgt = tgt; a.dft = dft; a.tok = tok; a.uni = uni; a.temp = temp;
  a.out = out; a.nacc = nacc; a.probs = probs; a.mass = mass;
  char* base = static_cast<char*>(ws);
  a.cnt = reinterpret_cast<unsigned*>(base + pl.off_cnt);
  a.part = reinterpret_cast<float4*>(base + pl.off_part);
  a.ldv = reinterpret_cast<float*>(base + pl.off_ldv);
  a.subK = reinterpret_cast<float*>(base + pl.off_subK);
  a.subR = reinterpret_cast<float*>(base + pl.off_subR);
  a.B = B; a.K = K; a.V = V; a.C = pl.C; a.CS = pl.CS; a.topk = topk;
  const size_t esz = dtype == SV_BF16 ? 2 : 4;
  const bool aligned = (reinterpret_cast<uintptr_t>(tgt) % 16 == 0) &&
                       (K == 0 || reinterpret_cast<uintptr_t>(dft) % 16 == 0) &&
                       ((size_t)V * esz) % 16 == 0;
  (void)hipGetLastError();  // start from a clean error state
  hipEvent_t* e = nev ? ev : nullptr;
  if (dtype == SV_BF16)
    return aligned ? launch_typed<uint16_t, true>(a, pl, st, e) : launch_typed<uint16_t, false>(a, pl, st, e);
  return aligned ? launch_typed<float, true>(a, pl, st, e) : launch_typed<float, false>(a, pl, st, e);
}

}  // namespace

extern "C" {

int spec_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                const float* uniforms, const float* temperature, int B, int K, int V, int topk_draft,
                int dtype, int32_t* out_tokens, int32_t* num_accepted, void* workspace,
                size_t* workspace_bytes, hipStream_t stream) {
  return run(target_logits, draft_logits, draft_tokens, uniforms, temperature, B, K, V, topk_draft,
             dtype, out_tokens, num_accepted, workspace, workspace_bytes, stream, nullptr, nullptr,
             nullptr, 0);
}

int spec_verify_probe(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                      const float* uniforms, const float* temperature, int B, int K, int V,
                      int topk_draft, int dtype, int32_t* out_tokens, int32_t* num_accepted,
                      void* workspace, size_t* workspace_bytes, hipStream_t stream, float* probs_out,
                      float* mass_out) {
  return run(target_logits, draft_logits, draft_tokens, uniforms, temperature, B, K, V, topk_draft,
             dtype, out_tokens, num_accepted, workspace, workspace_bytes, stream, probs_out, mass_out,
             nullptr, 0);
}

int spec_verify_timed(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                      const float* uniforms, const float* temperature, int B, int K, int V,
                      int topk_draft, int dtype, int32_t* out_tokens, int32_t* num_accepted,
                      void* workspace, size_t* workspace_bytes, hipStream_t stream, hipEvent_t* events,
                      int n_events) {
  return run(target_logits, draft_logits, draft_tokens, uniforms, temperature, B, K, V, topk_draft,
             dtype, out_tokens, num_accepted, workspace, workspace_bytes, stream, nullptr, nullptr,
             events, n_events);
}

int spec_verify_plan(int B, int K, int V, int topk_draft, int dtype, int* chunks, int* chunk_len) {
  if (!chunks || !chunk_len) return SV_ERR_ARG;
  if (topk_draft >= V) topk_draft = 0;
  Plan pl;
  const int rc = make_plan(B, K, V, topk_draft, dtype, pl);
  if (rc != SV_OK) return rc;
  *chunks = pl.C;
  *chunk_len = pl.CS;
  return SV_OK;
}

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_ARG: return "invalid argument";
    case SV_ERR_WORKSPACE: return "workspace too small";
    case SV_ERR_UNSUPPORTED: return "unsupported shape or top-k";
    case SV_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
