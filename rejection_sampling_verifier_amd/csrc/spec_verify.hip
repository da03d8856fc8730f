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
// Two launches per call (three with a truncated draft), all on the caller's
// stream; no work-group ever waits for another one that may not have
// started.
//
//   A. stats_kernel, one work-group per (row, position, vocabulary chunk).
//      Streams its chunk of target or draft logits once from HBM (16-byte
//      loads into a register tile) and writes the chunk max and the sum of
//      exp2((l - max) * log2(e)/T) -- or, for greedy rows, the chunk argmax.
//      The chunk holding a position's draft token records that token's
//      logit; the bonus position also writes 32 sub-block sums for the final
//      draw (with a truncated draft every target position does).  A
//      truncated draft's chunks write candidate lists instead of sums, and
//      merge_kernel (one work-group per (row, position)) selects exactly.
//   B. finish_kernel, up to C work-groups per row.  Each loads its row's
//      partials into LDS in one round of loads, merges them and runs the
//      first-rejection scan.  Greedy rows and rows that accepted every draft
//      are completed by the row's work-group 0.  For a row rejected with a
//      dense draft, the row's first G work-groups re-read target and draft
//      logits of the rejected position, chunk j, j + G, ... each, and
//      publish 32 sub-block sums of max(0, p_n - q_n) per chunk; the last of
//      them to arrive (atomic counter) draws the correction token.  With a
//      truncated draft the row's single work-group forms those sums from the
//      statistics pass's sub-block sums and the kept list, reading no logits
//      but the target's at the kept ids, and draws.
//
// The final draw is an inverse CDF over a three-level hierarchy: chunk
// masses (a wave scan), the 32 sub-block sums of the selected chunk, and a
// wave prefix sum over the 512 (bf16) or 256 (fp32) ids of the selected
// sub-block.
//
// Numerical conventions.  With s = log2(e)/T and MS = fl(M*s) for a max M,
// every exponential is exp2(fma(l, s, -MS)); sums computed against a chunk
// max m are rescaled by exp2(fl(m*s) - fl(M*s)), so the rounding of the
// reference products cancels between numerator and denominator.  All
// reductions combine partial results in a fixed order (no float atomics), so
// outputs are bitwise reproducible.
//
// Hand-off inside B: residual sums are published as complemented words with
// write-through agent-scope atomic stores (a zero word means "not written"),
// so a producer never waits; the last work-group of the row, which knows its
// peers have issued their stores, polls them and clears them after use.

#include <algorithm>
#include <climits>
#include <cstddef>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include <hip/hip_ext.h>

#include "spec_verify.h"
#include "sv_device.h"

using namespace sv;

namespace {

#ifndef SV_NV_TILE
#define SV_NV_TILE 8
#endif
// Waves per SIMD of the statistics kernels (a cap: more in flight measured
// slower), for dense drafts and for truncated ones, whose draft work-groups
// hold their slots longer (candidate filter and list stores).  The tree's
// statistics kernel keeps STATS_WAVES: at five it spills.  Early exit's first
// launch over a truncated draft (position 0's target, then draft slots only:
// eight of every nine work-groups run the candidate filter) is fastest at
// six.
constexpr int STATS_WAVES = 4;
constexpr int STATS_WAVES_TOPK = 5;
constexpr int EE_FIRST_WAVES = 6;
constexpr int NV_TILE = SV_NV_TILE;        // 16-byte vectors per thread per chunk
constexpr int NSUB = NV_TILE * NWAVE;      // sub-blocks per chunk (one wave x one vector row)
constexpr int MAX_C = 2048;                // vocabulary chunks per position
constexpr int MAX_SLOTS = 2 * SV_MAX_K + 1;
constexpr int MAX_CACHE_WORDS = 8192;       // dynamic LDS for a row's published words (32 KiB)
constexpr int TOPK_FAST_MAX = 512;         // sparse drafts: fast chunk selection for k <= 512
constexpr int WCAP = 256;                  // candidate list length per wave of a chunk
// Longest wait for another work-group's results: 100 ms of the 100 MHz
// constant clock.  Every wait ends well before that in a correct launch; the
// bound only guarantees termination.
constexpr uint64_t WAIT_TICKS = 10000000ull;

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
  uint32_t* part;            // [B, 2K+1, C, 4] published {max | argmax value, sum, argmax id, l(d)}
  uint32_t* subK;            // [B, NT, C, NSUB] target sub-block sums (vs chunk max), see sub_words
  uint32_t* subR;            // [B, C, NSUB] published residual sub-block sums
  unsigned* cnt;             // [B] finishing work-groups that have arrived
  void* cand;                // [B, K, C, cstride] chunk candidate lists of sparse drafts (Cand<ET>::T)
  int* ccnt;                 // [B, K, C, 2] their lengths and the order keys of their bounds (0: none)
  float4* qstat;             // [B, K] sparse draft: {max kept logit, Z_q, q(d_i), kept count}
  uint2* kept;               // [B, K, topk] sparse draft: kept (id, logit bits), ascending id
  int B, K, V, C, CS, topk;
  int cstride;               // sparse drafts: candidate entries per chunk
  int ckeep;                 // sparse drafts: logits a chunk lists at least
  // Relaxed (lossy) acceptance: 0 = the lossless rule.  With max_rank > 0 the
  // statistics kernel also counts, per target chunk, the logits above l(d_i).
  int relaxed, max_rank;
  float alpha, min_prob;
  float* kl;                 // [B, K] KL(p_i || q_i) out (spec_verify_kl: paired statistics), or null
  unsigned* claim;           // [B] early exit: stage tickets handed out
  unsigned* leave;           // [B] early exit: work-groups of the row that have finished
  int GA;                    // statistics work-groups per row: (2K+1) * C
  int resident;              // finishing work-groups the device holds at once (0: unknown)
  int cache;                 // 1: finishing work-groups keep the row's words in dynamic LDS
};

// ---- published words -------------------------------------------------------
// A value another work-group reads is published as the bitwise complement of
// its bits with a write-through agent-scope atomic store; a word of zero --
// the state of the workspace between calls -- therefore means "not written
// yet", and a reader polls with agent-scope atomic loads until every word it
// needs is non-zero.  Each word is validated on its own, so no ordering
// between words is needed and producers never wait.  The last work-group of
// a row clears the row's words for the next call.
__device__ __forceinline__ void pub_u32(uint32_t* p, uint32_t bits) {
  bits = bits == 0xFFFFFFFFu ? 0x7FC00000u : bits;  // a NaN pattern whose complement is 0
  __hip_atomic_store(p, ~bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void pub_f32(uint32_t* p, float v) { pub_u32(p, __float_as_uint(v)); }
// A uniform pointer taken into scalar registers where it is used: a store to
// uniform_ptr(base) + lane is then addressed as a scalar base plus a 32-bit
// lane offset, instead of the compiler keeping base's lane-dependent part as
// a 64-bit address live across a loop.
__device__ __forceinline__ uint32_t* uniform_ptr(uint32_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<uint32_t*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t peek(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t got_u32(const uint32_t* p) { return ~peek(p); }
__device__ __forceinline__ float got_f32(const uint32_t* p) { return __uint_as_float(~peek(p)); }
__device__ __forceinline__ void clear_word(uint32_t* p) {
  __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Candidate lists: written once by the statistics pass and read once by the
// merge kernel, a later launch (streaming stores, plain loads).
__device__ __forceinline__ void cand_st(uint64_t* p, uint64_t v) { __builtin_nontemporal_store(v, p); }

// Sub-block sums of a target position (vs the chunk max), [B, NT, C, NSUB]:
// with a truncated draft every target position's (NT = K + 1), else the
// bonus position's only (NT = 1).
__device__ __forceinline__ uint32_t* sub_words(const Args& a, int b, int slot, int c) {
  const int nt = a.topk > 0 ? a.K + 1 : 1;
  const int sl = a.topk > 0 ? slot : 0;
  return a.subK + (((size_t)b * nt + sl) * a.C + c) * NSUB;
}
__device__ __forceinline__ uint32_t* part_words(const Args& a, int b, int slot, int c) {
  return a.part + (((size_t)b * (2 * a.K + 1) + slot) * (size_t)a.C + c) * 4;
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
// Sparse draft truncation ([RheoSampling] section 3).  The global top k of a
// draft position takes about k / C logits from each of its C chunks, so a
// chunk lists only its best logits down to a bound: every logit at or above
// the bound, at least `keep` of them (keep = min(k, ceil(1.5k/C) + 8)).  With
// the list goes the bound's order key, or 0 when the list holds the chunk's
// whole top k (keep = k, the bound is -inf, or the exact path ran).  The
// merge kernel selects the k-th largest of the union and checks that it is
// at or above every chunk's bound: then every logit of the global top k is
// listed.  Otherwise it selects again with the logits of the chunks whose
// bound is higher read from the draft row itself.
// ============================================================================
// Chunk candidate as written by the statistics kernel: the composite of the
// logit and its vocabulary id.
template <typename ET>
struct Cand {
  using T = uint64_t;
};
template <typename ET>
__device__ __forceinline__ uint64_t cand_composite(typename Cand<ET>::T c, int /*chunk_lo*/) {
  return c;
}
// A passing logit staged in LDS by the statistics kernel: its bits and its
// offset in the chunk, packed as cheaply as possible; turned into a
// composite when the list is written out.  bf16: the widened value's low 16
// bits are zero and chunk offsets are below 2^16, so both fit 32 bits.
template <typename ET>
struct Staged;
template <>
struct Staged<uint16_t> {
  using T = uint32_t;
  static __device__ __forceinline__ T pack(float x, int off) { return __float_as_uint(x) | (uint32_t)off; }
  static __device__ __forceinline__ uint64_t composite_at(T v, int lo) {
    return composite(__uint_as_float(v & 0xFFFF0000u), lo + (int)(v & 0xFFFFu));
  }
};
template <>
struct Staged<float> {
  using T = uint64_t;
  static __device__ __forceinline__ T pack(float x, int off) {
    return ((uint64_t)__float_as_uint(x) << 32) | (uint32_t)off;
  }
  static __device__ __forceinline__ uint64_t composite_at(T v, int lo) {
    return composite(__uint_as_float((uint32_t)(v >> 32)), lo + (int)(uint32_t)v);
  }
};

// Exact selection by a 32-step binary search on order keys: the largest key
// tau with at least kk logits >= tau is the kk-th largest; logits above tau
// are all kept, ties at tau are kept in increasing id order.  The kk kept
// composites are written to dst[0..kk).
template <typename ET>
__device__ void topk_chunk_exact(const u32x4 (&r)[NV_TILE], int lo, int len, int kk, uint64_t* dst,
                                 float* red) {
  constexpr int VEC = Tr<ET>::VEC;
  const int t = threadIdx.x;
  auto count_keys = [&](uint32_t thr, bool strict) {
    int n = 0;
#pragma unroll 1
    for (int j = 0; j < NV_TILE; ++j)
      for (int e = 0; e < VEC; ++e) {
        const uint32_t key = order_key(Tr<ET>::at(r[j], e));
        const bool valid = (j * WG + t) * VEC + e < len;
        n += valid && (strict ? key > thr : key >= thr);
      }
    return (int)block_sum((float)n, red);  // exact: counts are below 2^24
  };
  // The largest key tau with at least kk logits at or above it: the kk-th
  // largest key.  A bf16 logit's key has the low 16 bits all zero (positive)
  // or all one (negative), so only the upper 16 bits are searched.
  constexpr int LOW = Tr<ET>::VEC == 8 ? 16 : 0;
  uint32_t tau = 0;
  for (int bit = 31; bit >= LOW; --bit) {
    const uint32_t cand = tau | (1u << bit);
    if (count_keys(cand, false) >= kk) tau = cand;
  }
  if (LOW) tau |= (tau & 0x80000000u) ? 0u : 0xFFFFu;
  // Logits above tau, then the first ties, each in id order (places by
  // block scans, so that the lists -- and every sum over them -- do not
  // depend on timing).
  float carry = 0.f;
#pragma unroll 1
  for (int j = 0; j < NV_TILE; ++j) {
    int mine = 0;
    for (int e = 0; e < VEC; ++e)
      mine += (j * WG + t) * VEC + e < len && order_key(Tr<ET>::at(r[j], e)) > tau;
    float ex, tot;
    block_scan((float)mine, red, ex, tot);
    int at = (int)(carry + ex);
    for (int e = 0; e < VEC; ++e) {
      const float x = Tr<ET>::at(r[j], e);
      const int off = (j * WG + t) * VEC + e;
      if (off < len && order_key(x) > tau) cand_st(dst + at++, composite(x, lo + off));
    }
    carry += tot;
  }
  const int above = (int)carry;
  const int need = kk - above;
  carry = 0.f;
#pragma unroll 1
  for (int j = 0; j < NV_TILE; ++j) {
    int mine = 0;
    for (int e = 0; e < VEC; ++e)
      mine += (j * WG + t) * VEC + e < len && order_key(Tr<ET>::at(r[j], e)) == tau;
    float ex, tot;
    block_scan((float)mine, red, ex, tot);
    int rank = (int)(carry + ex);
    for (int e = 0; e < VEC; ++e) {
      const float x = Tr<ET>::at(r[j], e);
      const int off = (j * WG + t) * VEC + e;
      if (off < len && order_key(x) == tau) {
        if (rank < need) cand_st(dst + above + rank, composite(x, lo + off));
        ++rank;
      }
    }
    carry += tot;
  }
  __syncthreads();
}

// Chunk candidates, written to the chunk's candidate area (cap entries) as
// one list of composites; cnt[0] gets its length and cnt[1] the order key of
// the bound above which it is complete (0: it holds the chunk's top k).
// Fast path (k <= 512): in each wave, a lower bound of the ceil(keep/4)-th
// largest of its 512 vector maxima (VEC logits each) is found by a ballot
// binary search on the upper 16 bits of their order keys; each of those
// vectors holds a distinct logit at or above it, so the smallest of the four
// bounds is a lower bound of the chunk's keep-th largest logit: at least
// keep logits pass it.
// Each wave lists the logits that pass (at most WCAP): the vectors whose
// maximum passes (a few percent) are compacted into LDS in vector order,
// then each lane tests the logits of one of them, so the per-logit work is
// spent on those vectors only; a wave with more than VCAP such vectors marks
// its logits one by one instead.  The four waves' lists are written back to
// back by the whole block, one contiguous run per chunk (four short runs
// apart in memory cost the statistics pass about 10 us on a 256-row,
// 8-draft batch).  The list is unsorted; the merge kernel selects exactly.
// Exact path (k > 512, a wave's list over WCAP or the chunk's over cap): the
// chunk's exact top min(k, len).
constexpr int VCAP = 128;  // passing vectors a wave compacts

// The 32-bit word of a vector that holds element e (e < VEC), selected
// without dynamic register indexing.
template <typename ET>
__device__ __forceinline__ float vec_elem(const u32x4& v, int e) {
  constexpr int VEC = Tr<ET>::VEC;
  const int wi = e / (VEC / 4);
  uint32_t word = v[0];
  word = wi == 1 ? v[1] : word;
  word = wi == 2 ? v[2] : word;
  word = wi == 3 ? v[3] : word;
  if constexpr (VEC == 8)
    return __uint_as_float((e & 1) ? (word & 0xFFFF0000u) : (word << 16));
  else
    return __uint_as_float(word);
}

template <typename ET>
__device__ __forceinline__ float vec_max(const u32x4& v) {
  if constexpr (Tr<ET>::VEC == 8)
    return max3_raw(max3_raw(Tr<ET>::at(v, 0), Tr<ET>::at(v, 1), Tr<ET>::at(v, 2)),
                    max3_raw(Tr<ET>::at(v, 3), Tr<ET>::at(v, 4), Tr<ET>::at(v, 5)),
                    max3_raw(Tr<ET>::at(v, 6), Tr<ET>::at(v, 7), Tr<ET>::at(v, 7)));
  else
    return max3_raw(max3_raw(Tr<ET>::at(v, 0), Tr<ET>::at(v, 1), Tr<ET>::at(v, 2)), Tr<ET>::at(v, 3),
                    Tr<ET>::at(v, 3));
}

template <typename ET>
__device__ void topk_chunk(const u32x4 (&r)[NV_TILE], int lo, int len, int k, int keep, int cap,
                           typename Cand<ET>::T* dst, int* cnt, float* red) {
  constexpr int VEC = Tr<ET>::VEC;
  constexpr int NE = NV_TILE * VEC;  // logits per thread: 64 (bf16) or 32 (fp32)
  using CT = typename Cand<ET>::T;
  using ST = typename Staged<ET>::T;
  // Fast path: each wave's list of passing logits, staged as (bits, offset).
  __shared__ uint64_t sbuf[NWAVE * WCAP];
  __shared__ u32x4 vbuf[NWAVE * VCAP];      // the wave's passing vectors
  __shared__ uint16_t voff[NWAVE * VCAP];   // and their offsets in the chunk
  __shared__ uint32_t wkey[NWAVE];
  __shared__ int s_wn[NWAVE];
  __shared__ int s_over;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int kk = min(k, len);
  bool done = false;
  if (k <= TOPK_FAST_MAX) {
    float vm[NV_TILE];  // the thread's vector maxima (padding reads as -inf)
    uint32_t vk[NV_TILE];  // and the upper 16 bits of their order keys
#pragma unroll
    for (int j = 0; j < NV_TILE; ++j) {
      vm[j] = vec_max<ET>(r[j]);
      vk[j] = order_key(vm[j]) >> 16;
    }
    const int m = (keep + NWAVE - 1) / NWAVE;  // at most 128 of the wave's 512 vectors
    uint32_t pre = 0;
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t cand = pre | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < NV_TILE; ++j) cnt += __popcll(__ballot(vk[j] >= cand));
      if (cnt >= m) pre = cand;
    }
    if (lane == 0) wkey[wave] = pre << 16;
    if (t == 0) s_over = 0;
    __syncthreads();
    // A negative prefix reads back as the lowest value of its bucket; the
    // bucket of -inf reads back as a NaN pattern, which must become -inf.
    float bound = key_value(min(min(wkey[0], wkey[1]), min(wkey[2], wkey[3])));
    if (bound != bound) bound = NEG_INF;
    // The wave's list is staged as (bits, offset).  Positions wrap inside the
    // wave's staging area: a list that overflows it is discarded below, so
    // its clobbered entries are never read.
    ST* wl_stage = reinterpret_cast<ST*>(sbuf) + wave * WCAP;
    // Vectors whose maximum passes, compacted in the wave's area (only for a
    // finite bound: with a bound of -inf every logit passes).  List order:
    // vector j, then thread, then logit.
    int nv = 0;  // wave-uniform
    if (bound > NEG_INF) {
#pragma unroll
      for (int j = 0; j < NV_TILE; ++j) {
        const bool p = vm[j] >= bound;
        const uint64_t bal = __ballot(p);
        if (bal) {
          const int idx = nv + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          if (p && idx < VCAP) {
            vbuf[wave * VCAP + idx] = r[j];
            voff[wave * VCAP + idx] = (uint16_t)((j * WG + t) * VEC);
          }
          nv += __popcll(bal);
        }
      }
    }
    int n;
    if (bound > NEG_INF && nv <= VCAP) {
      __builtin_amdgcn_wave_barrier();  // the compacted vectors are read by other lanes
      int pos0 = 0;
      for (int q0 = 0; q0 < nv; q0 += 64) {
        const int q = q0 + lane;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        int off = 0;
        uint32_t m8 = 0u;  // logit e of the vector at bit VEC-1-e
        if (q < nv) {
          v = vbuf[wave * VCAP + q];
          off = voff[wave * VCAP + q];
#pragma unroll
          for (int e = 0; e < VEC; ++e) m8 = m8 + m8 + (Tr<ET>::at(v, e) >= bound ? 1u : 0u);
        }
        const int c = __popc(m8);
        const float incl = wave_incl_scan((float)c);  // exact: at most 512
        int pos = pos0 + (int)incl - c;
        while (m8) {
          const int bp = 31 - __builtin_clz(m8);
          m8 &= ~(1u << bp);
          const int e = VEC - 1 - bp;
          wl_stage[pos & (WCAP - 1)] = Staged<ET>::pack(vec_elem<ET>(v, e), off + e);
          ++pos;
        }
        pos0 += (int)lane63(incl);
      }
      n = pos0;
    } else {
      // Each thread marks its passing logits in bit masks, logit i of the
      // thread at bit 31 - (i % 32) of mask i / 32; padding past the chunk
      // reads as -inf, so it can pass only a bound of -inf, the one case that
      // needs the range check.  List order: thread, then logit.
      uint32_t mask[NE / 32];
      auto mark = [&](auto check) {
#pragma unroll
        for (int h = 0; h < NE / 32; ++h) mask[h] = 0u;
#pragma unroll
        for (int j = 0; j < NV_TILE; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const int i = j * VEC + e;
            bool pass = Tr<ET>::at(r[j], e) >= bound;
            if (decltype(check)::value) pass = pass && (j * WG + t) * VEC + e < len;
            mask[i / 32] = mask[i / 32] + mask[i / 32] + (pass ? 1u : 0u);
          }
      };
      if (bound > NEG_INF)
        mark(std::false_type{});
      else
        mark(std::true_type{});
      int cnt = 0;
#pragma unroll
      for (int h = 0; h < NE / 32; ++h) cnt += __popc(mask[h]);
      const float incl = wave_incl_scan((float)cnt);  // exact: at most 4096
      n = (int)lane63(incl);
      int pos = (int)incl - cnt;
#pragma unroll
      for (int j = 0; j < NV_TILE; ++j) {
        // Vector j's logits e = 0..VEC-1 sit at bits VEC-1-e of mj.
        constexpr unsigned VMASK = (1u << VEC) - 1u;
        uint32_t mj = (mask[(j * VEC) / 32] >> (32 - VEC - (j * VEC) % 32)) & VMASK;
        while (mj) {
          const int bp = 31 - __builtin_clz(mj);
          mj &= ~(1u << bp);
          const int e = VEC - 1 - bp;
          wl_stage[pos & (WCAP - 1)] = Staged<ET>::pack(vec_elem<ET>(r[j], e), (j * WG + t) * VEC + e);
          ++pos;
        }
      }
    }
    if (lane == 0) {
      s_wn[wave] = n;
      if (n > WCAP) s_over = 1;
    }
    __syncthreads();
    const int o1 = s_wn[0], o2 = o1 + s_wn[1], o3 = o2 + s_wn[2], tot = o3 + s_wn[3];
    done = s_over == 0 && tot <= cap;
    if (done) {
      // The chunk's list: the waves' lists back to back, written by the
      // whole block (the merge kernel reads it once: streaming stores).
      for (int q = t; q < tot; q += WG) {
        const int w = (q >= o1) + (q >= o2) + (q >= o3);
        const int from = w == 0 ? 0 : (w == 1 ? o1 : (w == 2 ? o2 : o3));
        const ST* ws = reinterpret_cast<const ST*>(sbuf) + w * WCAP;
        cand_st(dst + q, Staged<ET>::composite_at(ws[q - from], lo));
      }
      if (t == 0) {
        // The list holds every logit at or above the bound: all of the
        // chunk's top k unless fewer than k were asked for.
        cnt[0] = tot;
        cnt[1] = keep < kk && bound > NEG_INF ? (int)order_key(bound) : 0;
      }
    }
  }
  if (!done) {
    __syncthreads();  // the fast path's staging is no longer read
    topk_chunk_exact<ET>(r, lo, len, kk, dst, red);
    if (t == 0) {
      cnt[0] = kk;
      cnt[1] = 0;
    }
  }
}

// ============================================================================
// Kernel A: statistics of one (row, position, chunk).
// ============================================================================
template <typename ET, bool ALIGNED>
__device__ __forceinline__ void stats_body(const Args& a, int b, int slot, int c) {
  constexpr int VEC = Tr<ET>::VEC;
  const int S = 2 * a.K + 1;
  const bool is_draft = slot > a.K;
  const int pos = is_draft ? slot - a.K - 1 : slot;
  const ET* row = is_draft ? draft_row<ET>(a, b, pos) : target_row<ET>(a, b, pos);
  const int lo = c * a.CS;
  const int len = min(a.CS, a.V - lo);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

  // A target slot issues its loads before it needs the temperature; a draft
  // slot first checks it, since greedy rows never read the draft.
  u32x4 r[NV_TILE];
  float T;
  // Relaxed rule with a rank guard: a target position counts its logits
  // above the draft token's logit (a token outside [0, V) counts nothing).
  const bool count_rank = a.relaxed && a.max_rank > 0 && !is_draft && pos < a.K;
  float lref = __builtin_inff();
  if (!is_draft) {
    load_tile<ET, ALIGNED, NV_TILE>(row, lo, len, r);
    T = a.temp[b];
    if (count_rank) {
      const int d = a.tok[(size_t)b * a.K + pos];
      if (d >= 0 && d < a.V) lref = Tr<ET>::load1(row + d);
    }
  } else {
    T = a.temp[b];
    if (!is_sampling_temperature(T)) return;
    load_tile<ET, ALIGNED, NV_TILE>(row, lo, len, r);
  }
  const bool greedy = !is_sampling_temperature(T);

  __shared__ float shf[NWAVE];
  __shared__ int shi[NWAVE];
  __shared__ float shsub[NSUB];
  uint32_t* dst = part_words(a, b, slot, c);

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
    if (t == 0) *reinterpret_cast<u32x4*>(dst) = u32x4{__float_as_uint(bv), 0u, (uint32_t)bi, 0u};
    return;
  }

  if (is_draft && a.topk > 0) {
    const size_t chunk = ((size_t)b * a.K + pos) * a.C + c;
    topk_chunk<ET>(r, lo, len, a.topk, a.ckeep, a.cstride,
                   reinterpret_cast<typename Cand<ET>::T*>(a.cand) + chunk * a.cstride, a.ccnt + 2 * chunk, shf);
    return;
  }
  const float m = block_max(tile_max<ET, NV_TILE>(r), shf);
  const float s = LOG2E / T;
  // A chunk of -inf only would give exp2(nan): use the reference 0 then
  // (every term is exp2(-inf) = 0).
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
  float z;
  uint32_t above = 0u;
  if (count_rank) {
    // The count of logits above l(d) shares the sum's block reduction.
    __shared__ float shn[NWAVE];
    int na = 0;
#pragma unroll
    for (int j = 0; j < NV_TILE; ++j)
#pragma unroll
      for (int k = 0; k < VEC; ++k) na += Tr<ET>::at(r[j], k) > lref;  // padding reads as -inf
    const float zw = wave_sum(zl), nw = wave_sum((float)na);  // exact: counts are below 2^24
    if (lane == 0) {
      shf[wave] = zw;
      shn[wave] = nw;
    }
    __syncthreads();
    z = shf[0];
    float nt = shn[0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) {
      z += shf[w];
      nt += shn[w];
    }
    __syncthreads();
    above = (uint32_t)nt;
  } else {
    z = block_sum(zl, shf);
  }
  if (slot == a.K || (a.topk > 0 && !is_draft)) {
    // Sub-block sums of the bonus position, and with a truncated draft of
    // every target position (its residual's mass outside the kept ids):
    // sub-block (j, wave) holds the 64 * VEC consecutive ids of vector row
    // j owned by that wave.
#pragma unroll
    for (int j = 0; j < NV_TILE; ++j) {
      const float v = wave_sum(zj[j]);
      if (lane == 0) shsub[j * NWAVE + wave] = v;
    }
    __syncthreads();
    if (t < NSUB) sub_words(a, b, slot, c)[t] = __float_as_uint(shsub[t]);
  }
  if (t == 0) {
    uint32_t ld = 0u;
    if (pos < a.K) {
      // The chunk holding this position's draft token records its logit.
      const int d = a.tok[(size_t)b * a.K + pos];
      if (d >= lo && d < lo + len) ld = __float_as_uint(Tr<ET>::load1(row + d));
    }
    *reinterpret_cast<u32x4*>(dst) = u32x4{__float_as_uint(m), __float_as_uint(z), above, ld};
  }
  (void)S;
}

template <typename ET, bool ALIGNED, int WAVES>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(WAVES, WAVES))) void stats_kernel(Args a) {
  const int S = 2 * a.K + 1;
  const int rest = blockIdx.x / a.C;
  stats_body<ET, ALIGNED>(a, rest / S, rest % S, blockIdx.x % a.C);
}

// ============================================================================
// Kernel A' (spec_verify_kl): the statistics pass with the draft position
// paired to its target position.  The work-group of target position i < K of
// a sampling row holds both chunks (target and draft) and writes both
// partials; the draft slot's third word carries
//   A_c = sum over the chunk of exp2(fma(l_t, s, -fl(m_t,c * s))) * (l_t - l_q),
// from which the finishing kernel forms KL(p_i || q_i).  The grid covers the
// K+1 target slots only; the bonus slot and greedy rows run the usual
// statistics (greedy rows never read the draft).
// ============================================================================
template <typename ET, bool ALIGNED>
__global__ __launch_bounds__(WG) void paired_kernel(Args a) {
  constexpr int VEC = Tr<ET>::VEC;
  const int c = blockIdx.x % a.C;
  const int rest = blockIdx.x / a.C;
  const int slot = rest % (a.K + 1);
  const int b = rest / (a.K + 1);
  const float T = a.temp[b];
  if (slot == a.K || !is_sampling_temperature(T)) {
    stats_body<ET, ALIGNED>(a, b, slot, c);
    return;
  }
  const int pos = slot;
  const int lo = c * a.CS;
  const int len = min(a.CS, a.V - lo);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const ET* trow = target_row<ET>(a, b, pos);
  const ET* drow = draft_row<ET>(a, b, pos);
  u32x4 rt[NV_TILE], rq[NV_TILE];
  load_tile<ET, ALIGNED, NV_TILE>(trow, lo, len, rt);
  load_tile<ET, ALIGNED, NV_TILE>(drow, lo, len, rq);
  __shared__ float sh[3 * NWAVE];
  float mt = wave_max(tile_max<ET, NV_TILE>(rt)), mq = wave_max(tile_max<ET, NV_TILE>(rq));
  if (lane == 0) {
    sh[wave] = mt;
    sh[NWAVE + wave] = mq;
  }
  __syncthreads();
  mt = sh[0];
  mq = sh[NWAVE];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) {
    mt = fmaxf(mt, sh[w]);
    mq = fmaxf(mq, sh[NWAVE + w]);
  }
  __syncthreads();
  const float s = LOG2E / T;
  const float mst = mt == NEG_INF ? 0.f : mul_rn(mt, s);
  const float msq = mq == NEG_INF ? 0.f : mul_rn(mq, s);
  // Sums in the same order as the unpaired pass (pairs of elements per
  // vector, vectors in order, then the block).
  float zt = 0.f, zq = 0.f, ac = 0.f;
#pragma unroll
  for (int j = 0; j < NV_TILE; ++j) {
    float t0 = 0.f, t1 = 0.f, q0 = 0.f, q1 = 0.f;
#pragma unroll
    for (int k = 0; k < VEC; k += 2) {
      const float la = Tr<ET>::at(rt[j], k), lb = Tr<ET>::at(rt[j], k + 1);
      const float ea = exp2_fast(fmaf(la, s, -mst)), eb = exp2_fast(fmaf(lb, s, -mst));
      t0 += ea;
      t1 += eb;
      q0 += exp2_fast(fmaf(Tr<ET>::at(rq[j], k), s, -msq));
      q1 += exp2_fast(fmaf(Tr<ET>::at(rq[j], k + 1), s, -msq));
      // A token the target cannot produce adds nothing (also when both are -inf).
      if (ea > 0.f) ac += ea * (la - Tr<ET>::at(rq[j], k));
      if (eb > 0.f) ac += eb * (lb - Tr<ET>::at(rq[j], k + 1));
    }
    zt = j ? zt + (t0 + t1) : t0 + t1;
    zq = j ? zq + (q0 + q1) : q0 + q1;
  }
  zt = wave_sum(zt);
  zq = wave_sum(zq);
  ac = wave_sum(ac);
  if (lane == 0) {
    sh[wave] = zt;
    sh[NWAVE + wave] = zq;
    sh[2 * NWAVE + wave] = ac;
  }
  __syncthreads();
  if (t == 0) {
    float Zt = sh[0], Zq = sh[NWAVE], A = sh[2 * NWAVE];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) {
      Zt += sh[w];
      Zq += sh[NWAVE + w];
      A += sh[2 * NWAVE + w];
    }
    uint32_t ldt = 0u, ldq = 0u;
    const int d = a.tok[(size_t)b * a.K + pos];
    if (d >= lo && d < lo + len) {
      ldt = __float_as_uint(Tr<ET>::load1(trow + d));
      ldq = __float_as_uint(Tr<ET>::load1(drow + d));
    }
    *reinterpret_cast<u32x4*>(part_words(a, b, pos, c)) = u32x4{__float_as_uint(mt), __float_as_uint(Zt), 0u, ldt};
    *reinterpret_cast<u32x4*>(part_words(a, b, a.K + 1 + pos, c)) =
        u32x4{__float_as_uint(mq), __float_as_uint(Zq), __float_as_uint(A), ldq};
  }
}

// ============================================================================
// Row decision from the published statistics.
// ============================================================================
// Where a finishing work-group reads a row's words: copies in LDS when they
// fit, else global memory.  Partials and bonus sub-block sums were written by
// the statistics kernel (plain words); residual sub-block sums are published
// by this kernel's work-groups (complemented words, see pub_u32).
// A row's published words, read from their LDS copy (CACHED) or from the
// workspace.  Keeping CACHED a compile-time choice lets every access to the
// copy compile to an LDS instruction.
template <bool CACHED>
struct RowView {
  const uint32_t* pw;    // CACHED: [(2K+1) * C * 4] partial words in LDS
  const uint32_t* sub;   // CACHED: [C * NSUB] sub-block sums in LDS (plain)
  bool sub_loaded;       // whether `sub` holds the sums (else they are read from the workspace)
};
template <bool CACHED>
__device__ __forceinline__ float view_part(const Args& a, const RowView<CACHED>& v, int b, int slot, int c, int w) {
  if constexpr (CACHED) return __uint_as_float(v.pw[((size_t)slot * a.C + c) * 4 + w]);
  else return __uint_as_float(part_words(a, b, slot, c)[w]);
}
template <bool CACHED>
__device__ __forceinline__ float view_sub(const RowView<CACHED>& v, const uint32_t* gsub, bool published, int c,
                                          int q) {
  if (CACHED && v.sub_loaded) return __uint_as_float(v.sub[c * NSUB + q]);
  const uint32_t* p = gsub + (size_t)c * NSUB + q;
  return __uint_as_float(published ? got_u32(p) : *p);
}

// Block-wide wait until the words p0[0..n0) and p1[0..n1) are published.
// Decoded values are left in d0 / d1 (LDS) when those are given.  Returns
// false (uniformly) if the deadline passed first.
__device__ __forceinline__ bool wait_words(const uint32_t* p0, int n0, uint32_t* d0, const uint32_t* p1, int n1,
                                           uint32_t* d1, uint64_t deadline) {
  for (;;) {
    bool ok = true;
    for (int i = threadIdx.x; i < n0; i += WG) {
      const uint32_t w = peek(p0 + i);
      ok &= w != 0u;
      if (d0) d0[i] = ~w;
    }
    for (int i = threadIdx.x; i < n1; i += WG) {
      const uint32_t w = peek(p1 + i);
      ok &= w != 0u;
      if (d1) d1[i] = ~w;
    }
    if (__syncthreads_and(ok)) return true;
    if (__syncthreads_or(wall_clock64() > deadline)) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

struct RowShared {
  float M[MAX_SLOTS];    // position max (sampling) or argmax value (greedy)
  float Z[MAX_SLOTS];    // sum of exp2(fma(l, s, -fl(M*s)))
  int idx[MAX_SLOTS];    // argmax id (greedy)
  float p[SV_MAX_K];     // p_i(d_i)
  float q[SV_MAX_K];     // q_i(d_i)
  int tok[SV_MAX_K];
  float red_f[NWAVE];
  float uK;              // u_K: drives the final draw
  int n;                 // accepted drafts
  int greedy;
  float s;               // log2(e)/T
};

// Per-row scalars, loaded by each thread t <= K at the start of a kernel so
// that their latency overlaps the loads of the row's partials.
struct RowIn {
  float T;    // temperature of the row
  int d;      // d_t (t < K)
  float u;    // u_t (t <= K)
  float qd;   // sparse draft: q~_t(d_t) (t < K)
};
__device__ __forceinline__ RowIn load_row_in(const Args& a, int b) {
  const int K = a.K, t = threadIdx.x;
  // Loaded per lane, without branches, so that nothing waits for these
  // loads before their first use (lanes past K read a valid entry and drop it).
  int bv = b;
  asm volatile("" : "+v"(bv));
  RowIn in{a.temp[bv], -1, 0.f, 0.f};
  in.u = a.uni[(size_t)b * (K + 1) + min(t, K)];
  if (K > 0) {
    const size_t i = (size_t)b * K + min(t, K - 1);
    in.d = a.tok[i];
    if (a.topk > 0) in.qd = a.qstat[i].z;
  }
  if (t > K) in.u = 0.f;
  if (t >= K) {
    in.d = -1;
    in.qd = 0.f;
  }
  return in;
}

// Merge of slots 0..nmerge of a row's chunk statistics: the row's max and
// sum against it (the argmax for greedy rows) per slot, into rs.  One group of
// G lanes per slot, lane g of the group holding chunks g, g + G, ... (G is
// the smallest of 16, 32, 64 that holds C, else 64), so every result equals
// the wave-wide merge of the slot's chunks bit for bit: the same operations
// per lane, and the reduction steps that stay inside the group.
template <int G, bool CACHED>
__device__ __forceinline__ void merge_slots(const Args& a, int b, RowShared& rs, const RowView<CACHED>& v,
                                            int nmerge, bool greedy, float s) {
  constexpr int PER = 64 / G;
  const int C = a.C, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, gl = lane % G;
  for (int base = wave * PER; base < nmerge; base += NWAVE * PER) {
    const int slot = base + lane / G;
    const bool need = slot < nmerge;
    if (greedy) {
      float bv = NEG_INF;
      int bi = INT_MAX;
      if (need)
        for (int c = gl; c < C; c += G)
          argmax_merge(bv, bi, view_part(a, v, b, slot, c, 0), __float_as_int(view_part(a, v, b, slot, c, 2)));
      group_argmax<G>(bv, bi);
      if (need && gl == G - 1) {
        rs.M[slot] = bv;
        rs.Z[slot] = 0.f;
        rs.idx[slot] = bi;
      }
    } else {
      float m = NEG_INF;
      if (need)
        for (int c = gl; c < C; c += G) m = fmaxf(m, view_part(a, v, b, slot, c, 0));
      m = group_last<G>(group_max<G>(m));
      const float MS = mul_rn(m, s);
      float z = 0.f;
      if (need)
        for (int c = gl; c < C; c += G) {
          const float mc = view_part(a, v, b, slot, c, 0), zc = view_part(a, v, b, slot, c, 1);
          if (mc != NEG_INF) z += zc * exp2_fast(mul_rn(mc, s) - MS);
        }
      z = group_sum<G>(z);
      if (need && gl == G - 1) {
        rs.M[slot] = m;
        rs.Z[slot] = z;
        rs.idx[slot] = 0;
      }
    }
  }
}

template <bool CACHED>
__device__ __forceinline__ void decide_row(const Args& a, int b, RowShared& rs, const RowView<CACHED>& v,
                                           const RowIn& in) {
  const int K = a.K, C = a.C, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float T = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(in.T)));
  const bool greedy = !is_sampling_temperature(T);
  const float s = greedy ? 0.f : LOG2E / T;
  const int d = in.d;
  const float u = in.u;
  if (t == K) rs.uK = u;
  const int nmerge = (greedy || a.topk > 0) ? K + 1 : 2 * K + 1;
  // Groups of G lanes (the smallest of 16, 32, 64 that holds C) merge one
  // slot each, so a wave merges 64 / G slots at once.
  if (C <= 16) merge_slots<16>(a, b, rs, v, nmerge, greedy, s);
  else if (C <= 32) merge_slots<32>(a, b, rs, v, nmerge, greedy, s);
  else merge_slots<64>(a, b, rs, v, nmerge, greedy, s);
  __syncthreads();
  if (wave == 0) {
    // Acceptance test of every position at once ([RheoSampling] section 4
    // step 1: u*q < p; [nalar] greedy rule: draft equals the argmax), then
    // the first rejection by ballot (K <= 64 positions fit one wave).
    bool acc = true;
    if (t < K) {
      float p = 0.f, q = 0.f;
      if (!greedy && d >= 0 && d < a.V) {
        const int cd = d / a.CS;
        const float lt = view_part(a, v, b, t, cd, 3);
        p = exp2_fast(fmaf(lt, s, -mul_rn(rs.M[t], s))) / rs.Z[t];
        if (a.topk > 0) {
          q = in.qd;  // q~(d_t) of the truncated draft
        } else {
          const float lq = view_part(a, v, b, K + 1 + t, cd, 3);
          q = exp2_fast(fmaf(lq, s, -mul_rn(rs.M[K + 1 + t], s))) / rs.Z[K + 1 + t];
        }
      }
      rs.p[t] = p;
      rs.q[t] = q;
      rs.tok[t] = d;
      if (greedy) {
        acc = d == rs.idx[t];
      } else if (!a.relaxed) {
        acc = u * q < p;
      } else {
        // Relaxed rule ([Acceptance Is Not Speed] sections 1, 6, 7): a
        // support guard on the rank and probability of d, the strict branch
        // q <= p, else acceptance against gamma = min(p + sqrt(2 a p (1-p)), 1).
        bool ok = d >= 0 && d < a.V;
        if (ok && a.max_rank > 0) {
          uint32_t above = 0u;
          for (int c = 0; c < C; ++c) above += __float_as_uint(view_part(a, v, b, t, c, 2));
          ok = above + 1u <= (uint32_t)a.max_rank;
        }
        if (ok && a.min_prob > 0.f) ok = p >= a.min_prob;
        if (!ok) {
          acc = false;
        } else if (p > 0.f && q <= p) {
          acc = true;
        } else {
          const float g = fminf(p + __fsqrt_rn(2.f * a.alpha * p * (1.f - p)), 1.f);
          acc = u * q < g;
        }
      }
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
// Inverse-CDF search inside one segment [start, start + len) of a row,
// len <= 64 * VEC, by one wave: lane l holds the ids start + l*VEC .. + VEC-1.
// Weights: p(x) = exp2(fma(l_t, s, -MSt)) * rZt; with a draft row
// max(0, p(x) - q(x)); with a kept list (sparse draft: ids ascending in kid,
// q~ values in kq) max(0, p(x) - q~(x)).  The prefix is a wave scan in id
// order.  Result, the same in every lane: the smallest id whose prefix
// exceeds tl (-1 if none), the last id of positive weight (-1 if none) and
// the segment's total weight.
// ============================================================================
struct SegResult {
  int found;
  int last_pos;
  float total;
};

template <typename ET, bool ALIGNED>
__device__ __forceinline__ SegResult segment_search(const ET* __restrict__ trow, const ET* __restrict__ drow,
                                                    const int* kid, const float* kq, int nkept, int start,
                                                    int len, float tl, float s, float MSt, float rZt, float MSq,
                                                    float rZq) {
  constexpr int VEC = Tr<ET>::VEC;
  const int l = threadIdx.x & 63, e = l * VEC;
  const u32x4 vt = load_vec<ET, ALIGNED>(trow, start + e, len - e);
  const u32x4 vq = drow ? load_vec<ET, ALIGNED>(drow, start + e, len - e) : vt;
  int j = 0;  // first kept entry with id >= start + e
  if (kid) {
    int lo = 0, hi = nkept;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (kid[mid] < start + e) lo = mid + 1; else hi = mid;
    }
    j = lo;
  }
  float w[VEC];
  float local = 0.f;
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    const float p = exp2_fast(fmaf(Tr<ET>::at(vt, k), s, -MSt)) * rZt;
    float wk = p;
    if (drow) {
      wk = fmaxf(0.f, p - exp2_fast(fmaf(Tr<ET>::at(vq, k), s, -MSq)) * rZq);
    } else if (kid) {
      float qk = 0.f;
      if (j < nkept && kid[j] == start + e + k) qk = kq[j++];
      wk = fmaxf(0.f, p - qk);
    }
    w[k] = e + k < len ? wk : 0.f;
    local += w[k];
  }
  float inc = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float u = __shfl_up(inc, o, 64);
    if (l >= o) inc += u;
  }
  float cum = __shfl_up(inc, 1, 64);
  if (l == 0) cum = 0.f;
  int found = -1, last_pos = -1;
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    cum += w[k];
    if (w[k] > 0.f) last_pos = start + e + k;
    if (found < 0 && e + k < len && cum > tl) found = start + e + k;
  }
  SegResult r;
  const unsigned long long hit = __ballot(found >= 0);
  r.found = hit ? __shfl(found, (int)__builtin_ctzll(hit), 64) : -1;
  const unsigned long long pos = __ballot(last_pos >= 0);
  r.last_pos = pos ? __shfl(last_pos, 63 - (int)__builtin_clzll(pos), 64) : -1;
  r.total = __shfl(inc, 63, 64);
  return r;
}

// ============================================================================
// Residual of a truncated draft ([RheoSampling] sections 3 and 4): the
// sub-block sums of max(0, p - q~) over a position, by the calling
// work-group (all threads), with no pass over the logits.  q~ is zero
// outside its kept ids, so the sum over sub-block (c, u) is
//   R(c, u) = max(0, P(c, u) - sum over its kept ids x, in list order, of min(p(x), kq[x])),
// where P(c, u) = sub(c, u) * exp2(fl(m_c s) - MSt) * rZt is the target's
// mass over the sub-block, from the statistics pass's sum of
// exp2(fma(l, s, -fl(m_c s))) there and the chunk max m_c.  Only the target
// at the kept ids is needed: pk(j) = p(kid[j]) = exp2(fma(l, s, -MSt)) * rZt
// (read from the logits, or kept from an earlier pass).  kid / kq: the kept
// ids (ascending) and their q~ values (or c q~ for a tree's later residual),
// in LDS; corr: LDS scratch of nkept floats.  sub(c, u) and chunk_max(c) read
// the position's statistics; out(i, R) stores R(c, u) at i = c * NSUB + u.  Sub-block u of
// chunk c holds the ids c * CS + [u, u + 1) * 64 * VEC below the chunk's end
// min((c + 1) * CS, V).
// ============================================================================
template <typename ET, typename PkF, typename SubF, typename MaxF, typename OutF>
__device__ __forceinline__ void sparse_residual(int V, int C, int CS, float s, float MSt, float rZt, const int* kid,
                                                const float* kq, int nkept, float* corr, PkF&& pk, SubF&& sub,
                                                MaxF&& chunk_max, OutF&& out) {
  constexpr int VEC = Tr<ET>::VEC;
  for (int j = threadIdx.x; j < nkept; j += WG) corr[j] = fminf(pk(j), kq[j]);
  __syncthreads();
  auto lower = [&](int x) {
    int l0 = 0, h0 = nkept;
    while (l0 < h0) {
      const int mid = (l0 + h0) >> 1;
      if (kid[mid] < x) l0 = mid + 1; else h0 = mid;
    }
    return l0;
  };
  for (int i = threadIdx.x; i < C * NSUB; i += WG) {
    const int c = i / NSUB, u = i % NSUB;
    const int end = min((c + 1) * CS, V);
    const int x0 = min(c * CS + u * 64 * VEC, end);
    const int j0 = lower(x0), j1 = lower(min(x0 + 64 * VEC, end));
    float cs = 0.f;
    for (int j = j0; j < j1; ++j) cs += corr[j];
    const float mc = chunk_max(c);
    const float sc = mc == NEG_INF ? 0.f : exp2_fast(mul_rn(mc, s) - MSt) * rZt;
    out(i, fmaxf(0.f, sub(c, u) * sc - cs));
  }
  __syncthreads();
}

// ============================================================================
// Final draw for a sampling row ([RheoSampling] section 4 step 3), by wave 0
// of the calling work-group alone (no block barriers).  The weights are the
// residual max(0, p_n - q_n) after a rejection at n < K, or the bonus
// position's p_K; their CDF is walked in three levels:
//   1. chunk masses: lane c sums chunk c's 32 sub-block sums in order
//      (residual sums published by the finishing work-groups, or bonus sums
//      from the statistics kernel rescaled from the chunk max); a wave scan
//      over the chunks gives S and the chunk c* whose inclusive prefix first
//      exceeds t = u_K * S;
//   2. in c*, lane q forms the prefix of sub-blocks 0..q in the same order
//      (so the prefix of the last sub-block is the chunk mass bit for bit);
//      the first sub-block whose prefix exceeds the remainder is selected;
//   3. a wave prefix sum over its 64 * VEC ids picks the token.
// A zero residual (reachable only through rounding) falls back to p_n with
// chunk masses from the partials and a walk over the whole chunk.  Writes
// out_tokens, num_accepted and mass.  A sparse draft's kept list must be in
// kid / kq (LDS, ascending id) before the call.
// ============================================================================
template <typename ET, bool ALIGNED, bool CACHED>
__device__ __forceinline__ void final_draw(const Args& a, int b, int n, float s, float MSt, float rZt, float MSq,
                                           float rZq, const RowShared& rs, const RowView<CACHED>& v,
                                           const int* kid, const float* kq, int nkept) {
  constexpr int VEC = Tr<ET>::VEC;
  static_assert(NSUB == 32, "a chunk has 32 sub-blocks");
  const int K = a.K, C = a.C, l = threadIdx.x;
  if (l >= 64) return;
  const bool reject = n < K;
  const uint32_t* gsub = reject ? a.subR + (size_t)b * C * NSUB : sub_words(a, b, K, 0);
  auto bonus_scale = [&](int c) {
    const float mc = view_part(a, v, b, K, c, 0);
    return mc == NEG_INF ? 0.f : exp2_fast(mul_rn(mc, s) - MSt) * rZt;
  };
  // Sub-block weight q of chunk c; sc is the chunk's bonus scale.
  auto sub_weight = [&](int c, int q, float sc) {
    return reject ? view_sub(v, gsub, true, c, q) : view_sub(v, gsub, false, c, q) * sc;
  };
  auto chunk_mass = [&](int c) {
    const float sc = reject ? 1.f : bonus_scale(c);
    float w[NSUB];
#pragma unroll
    for (int q = 0; q < NSUB; ++q) w[q] = sub_weight(c, q, sc);
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < NSUB; ++q) m += w[q];
    return m;
  };
  auto p_mass = [&](int c) {  // fallback: mass of p_n in chunk c from the partials
    const float mc = view_part(a, v, b, n, c, 0), zc = view_part(a, v, b, n, c, 1);
    return mc == NEG_INF ? 0.f : zc * exp2_fast(mul_rn(mc, s) - MSt) * rZt;
  };
  // Chunk masses in groups of 64 chunks (lane l holds chunk base + l) and
  // their wave scan (DPP); the exclusive prefix is the previous lane's.
  auto group = [&](bool use_p, int base, float& m, float& in, float& ex) {
    const int c = base + l;
    m = c < C ? (use_p ? p_mass(c) : chunk_mass(c)) : 0.f;
    in = wave_incl_scan(m);
    ex = __shfl_up(in, 1, 64);
    if (l == 0) ex = 0.f;
  };
  // Pass 1: the total S.  The first group's values are kept for pass 2.
  bool fallback = false;
  float m0, in0, ex0;
  auto total = [&](bool use_p) {
    group(use_p, 0, m0, in0, ex0);
    float carry = lane63(in0);
    for (int base = 64; base < C; base += 64) {
      float m, in, ex;
      group(use_p, base, m, in, ex);
      carry += lane63(in);
    }
    return carry;
  };
  float S = total(false);
  if (reject && S == 0.f) {
    fallback = true;
    S = total(true);
  }
  const float tv = rs.uK * S;
  // Pass 2: the first chunk whose inclusive prefix exceeds tv.
  int cs = -1, last = -1;
  float exc_cs = 0.f, carry = 0.f;
  for (int base = 0; base < C; base += 64) {
    float m = m0, in = in0, ex = ex0;
    if (base > 0) group(fallback, base, m, in, ex);
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
  if (cs < 0) {  // t reached the total only through rounding: last chunk of positive mass
    cs = last >= 0 ? last : 0;
    exc_cs = -__builtin_inff();
  }
  const float t1 = tv - exc_cs;  // +inf when t reached the total through rounding
  const int lo = cs * a.CS;
  const int len = min(a.CS, a.V - lo);
  const ET* trow = target_row<ET>(a, b, n);
  const bool sparse = reject && !fallback && a.topk > 0;
  const ET* drow = (reject && !fallback && !sparse) ? draft_row<ET>(a, b, n) : nullptr;
  int x = lo;
  if (fallback) {
    // Walk the whole chunk in segments of 64 * VEC ids.
    float carry = 0.f;
    int last = -1;
    x = -1;
    for (int seg = 0; seg < len && x < 0; seg += 64 * VEC) {
      const SegResult r = segment_search<ET, ALIGNED>(trow, nullptr, nullptr, nullptr, 0, lo + seg,
                                                      min(64 * VEC, len - seg), t1 - carry, s, MSt, rZt, 0.f,
                                                      0.f);
      if (r.found >= 0) x = r.found;
      if (r.last_pos >= 0) last = r.last_pos;
      carry += r.total;
    }
    if (x < 0) x = last >= 0 ? last : lo;
  } else {
    // Sub-block of the chunk: lane q < 32 holds the prefix through q.
    const float sc = reject ? 1.f : bonus_scale(cs);
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
    const int j = q / NWAVE, w = q % NWAVE;
    const int start = lo + (j * WG + w * 64) * VEC;
    const int slen = max(0, min(64 * VEC, lo + len - start));
    if (slen > 0) {
      const SegResult r = segment_search<ET, ALIGNED>(trow, drow, sparse ? kid : nullptr, kq, nkept, start, slen,
                                                      tl, s, MSt, rZt, MSq, rZq);
      x = r.found >= 0 ? r.found : (r.last_pos >= 0 ? r.last_pos : start);
    }
  }
  int32_t* out = a.out + (size_t)b * (K + 1);
  for (int i = l; i <= K; i += 64) out[i] = i < n ? rs.tok[i] : (i == n ? x : -1);
  if (l == 0) {
    a.nacc[b] = n;
    if (a.mass) a.mass[b] = S;
  }
}

// ============================================================================
// Kernel M (sparse drafts only): one work-group per (row, draft position) of
// a sampling row.  Selects the kk = min(k, V) best of the chunk candidates
// (ties to the lower id), which define the truncated draft distribution q~
// used at verification; writes the kept (id, logit) list in increasing id
// order, the max kept logit, Z_q = sum over kept of exp2(fma(l, s, -fl(max*s)))
// (summed in id order) and q~(d_i).
//
// The kk-th largest composite is found by a radix select with 10-bit
// windows over the bits in which the candidates differ.  Composites are
// distinct, so exactly kk candidates are at or above it.  The candidates are
// held in registers (one per list and lane) when the lists are few enough,
// and read from their lists in global memory at every pass otherwise.
// ============================================================================
constexpr int MERGE_REG = 12;     // lists per wave whose first 64 entries are held in registers
constexpr int MERGE_OVF = 480;    // list entries past the 64th, gathered into LDS (sized so that
                                  // eight merge work-groups fit a CU's LDS)

// Candidates of one (row, position) held by the work-group: register r of
// wave w holds entries [64 w, 64 w + 64) of chunk r's list (lane l holding
// entry 64 w + l); entries past the 256th of a list are in an LDS overflow
// buffer as composites.
template <typename ET>
struct RegCands {
  typename Cand<ET>::T v[MERGE_REG];
  uint32_t valid;          // bit r: v[r] is an entry
  int CS;
  const uint64_t* ovf;
  int novf;
  template <typename F>
  __device__ __forceinline__ void each(F&& f) const {
#pragma unroll
    for (int r = 0; r < MERGE_REG; ++r)
      if (valid >> r & 1u) f(cand_composite<ET>(v[r], r * CS));
    for (int j = threadIdx.x; j < novf; j += WG) f(ovf[j]);
  }
};
// Candidates read from their lists in global memory (wave w reads the lists
// of chunks w, w + NWAVE, ...).
template <typename ET>
struct ListCands {
  const typename Cand<ET>::T* g;
  const int* gcnt;
  int C, CS, stride;
  template <typename F>
  __device__ __forceinline__ void each(F&& f) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int L = wave; L < C; L += NWAVE) {
      const int n = *(gcnt + 2 * L);
      for (int j = lane; j < n; j += 64) f(cand_composite<ET>(*(g + (size_t)L * stride + j), L * CS));
    }
  }
};
// The fallback's candidates: the lists of the chunks whose bound key is at
// or below `key`, and the logits of the other chunks read from the draft row
// (those whose key is at least `key`; no other can reach the top k).
template <typename ET>
struct MixedCands {
  const typename Cand<ET>::T* g;
  const int* gcnt;
  const ET* row;
  int C, CS, V, stride;
  uint32_t key;
  template <typename F>
  __device__ __forceinline__ void each(F&& f) const {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    for (int L = wave; L < C; L += NWAVE) {
      if ((uint32_t)*(gcnt + 2 * L + 1) > key) continue;
      const int n = *(gcnt + 2 * L);
      for (int j = lane; j < n; j += 64) f(cand_composite<ET>(*(g + (size_t)L * stride + j), L * CS));
    }
    for (int L = 0; L < C; ++L) {
      if ((uint32_t)*(gcnt + 2 * L + 1) <= key) continue;
      const int lo = L * CS, hi = min(lo + CS, V);
      for (int x = lo + t; x < hi; x += WG) {
        const float v = Tr<ET>::load1(row + x);
        if (order_key(v) >= key) f(composite(v, x));
      }
    }
  }
};

// Threshold composite: exactly kk candidates are >= it.  A radix select over
// the bits in which the candidates differ: the highest undecided differing
// bit starts a 10-bit window, the window's digits of the candidates that
// match the prefix decided so far are counted in an LDS histogram, and the
// digit at which the count of larger candidates reaches kk is appended to
// the prefix.  Bits equal in every candidate are taken as they are.  It stops
// once every candidate with the chosen digit is needed (usually after the
// first window; ties in value continue into the id bits).  Also returns the
// largest candidate value (the largest kept logit) in *vmax.
constexpr int RADIX_BITS = 10;  // wider windows need fewer passes, but clearing and
                                // scanning their bins costs more LDS traffic per pass
constexpr int RADIX_BINS = 1 << RADIX_BITS;  // 1024 bins, 4 per thread

template <typename Src>
__device__ uint64_t select_threshold(const Src& src, int kk, uint32_t* sh32, float* red, int* ired,
                                     uint32_t* hist, float* vmax) {
  __shared__ int s_digit, s_above, s_count;
  constexpr int PER = RADIX_BINS / WG;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t and_lo = ~0u, and_hi = ~0u, or_lo = 0u, or_hi = 0u;
  float best = NEG_INF;
  src.each([&](uint64_t v) {
    and_lo &= (uint32_t)v;
    and_hi &= (uint32_t)(v >> 32);
    or_lo |= (uint32_t)v;
    or_hi |= (uint32_t)(v >> 32);
    best = fmaxf(best, composite_value(v));
  });
  and_lo = wave_and(and_lo);
  and_hi = wave_and(and_hi);
  or_lo = wave_or(or_lo);
  or_hi = wave_or(or_hi);
  best = wave_max(best);
  if (lane == 0) {
    sh32[wave] = and_lo;
    sh32[NWAVE + wave] = and_hi;
    sh32[2 * NWAVE + wave] = or_lo;
    sh32[3 * NWAVE + wave] = or_hi;
    red[wave] = best;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) hist[t * PER + i] = 0u;
  __syncthreads();
  uint64_t all_and = ~0ull, any_or = 0ull;
  float mx = NEG_INF;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    all_and &= ((uint64_t)sh32[NWAVE + w] << 32) | sh32[w];
    any_or |= ((uint64_t)sh32[3 * NWAVE + w] << 32) | sh32[2 * NWAVE + w];
    mx = fmaxf(mx, red[w]);
  }
  // Uniform: taken into a scalar register here, so that the compiler does
  // not keep the four partial maxima live (and spilled) through the windows.
  *vmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mx)));
  uint64_t var = all_and ^ any_or;  // bits that differ between candidates
  uint64_t tau = all_and;           // constant bits; variable bits start at 0
  int need = kk;
  while (var) {
    const int hb = 63 - __builtin_clzll(var);
    const int lo = max(hb - (RADIX_BITS - 1), 0);
    const uint64_t hi_mask = hb == 63 ? 0ull : ~((2ull << hb) - 1);  // bits above the window: all decided
    const uint32_t dmask = (uint32_t)((2ull << (hb - lo)) - 1);
    const uint64_t pre = tau & hi_mask;
    src.each([&](uint64_t v) {
      if ((v & hi_mask) == pre) atomicAdd(&hist[(uint32_t)(v >> lo) & dmask], 1u);
    });
    __syncthreads();
    // Thread t holds the bins of group 255 - t, so the exclusive scan counts
    // the candidates in higher bins.
    const int g = WG - 1 - t;
    uint32_t h[PER];
    int local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      h[i] = hist[g * PER + i];
      local += (int)h[i];
    }
    int tot;
    int above = block_count_scan(local, ired, tot);
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (above < need && need <= above + (int)h[i]) {
        s_digit = g * PER + i;
        s_above = above;
        s_count = (int)h[i];
      }
      above += (int)h[i];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) hist[g * PER + i] = 0u;  // ready for the next window
    __syncthreads();
    need -= s_above;
    tau |= (uint64_t)s_digit << lo;
    var &= ~((uint64_t)dmask << lo);
    // No barrier before the next window: s_* are rewritten only after its
    // first barrier, which every thread reaches after reading them here.
    if (s_count == need) break;
  }
  return tau;
}

// Kept set from the threshold: the kept composites go to sel[] (in
// arbitrary order) and each thread sums exp2(fma(l, s, -ms)) over the kept
// candidates it holds, in its own fixed order.  The logit of draft token d,
// if kept, goes to *ld_bits.
template <typename Src>
__device__ __forceinline__ float take_kept(const Src& src, uint64_t thr, int d, float s, float ms, uint64_t* sel,
                                           int* n_sel, uint32_t* ld_bits) {
  float z = 0.f;
  src.each([&](uint64_t v) {
    if (v >= thr) {
      const int at = atomicAdd(n_sel, 1);
      if (at < SV_MAX_TOPK) sel[at] = v;
      const float l = composite_value(v);
      z += exp2_fast(fmaf(l, s, -ms));
      if (composite_id(v) == d) *ld_bits = __float_as_uint(l);
    }
  });
  return z;
}

// Whether every chunk's list reaches down to the union's kk-th largest
// composite thr: each chunk's bound key (0 for a list holding the chunk's
// top k) is at most thr's value key.  Uniform over the block; the vote goes
// through vote[NWAVE] (LDS), which every thread has read when it returns:
// the caller must pass a barrier before writing vote again (the merge next
// writes it inside a selection, after that selection's first barrier).
__device__ __forceinline__ bool lists_hold_top(const int* gcnt, int C, uint64_t thr, int* vote) {
  const uint32_t key = (uint32_t)(thr >> 32);
  bool ok = true;
  for (int c = threadIdx.x; c < C; c += WG) ok &= (uint32_t)*(gcnt + 2 * c + 1) <= key;
  const bool wave_ok = __ballot(!ok) == 0ull;
  if ((threadIdx.x & 63) == 0) vote[threadIdx.x >> 6] = wave_ok;
  __syncthreads();
  bool all = true;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) all &= vote[w] != 0;
  return all;
}

// The merge of slot (row b, position i): `d` is the token whose q~ is
// recorded (-1 for none).  Writes {max kept logit, Z_q, q~(d), kk} to qstat
// and the kept ids and logits in ascending id order to kept; returns kk,
// the number of kept ids.
template <typename ET>
__device__ __forceinline__ int merge_body(const Args& a, int b, int i, int d) {
  __shared__ __align__(16) uint64_t sel[SV_MAX_TOPK + 2];  // kept composites (+ a zero pad entry)
  __shared__ uint64_t ovf[MERGE_OVF];
  __shared__ uint32_t hist[RADIX_BINS > SV_MAX_TOPK ? RADIX_BINS : SV_MAX_TOPK];  // radix histogram, then the
                                                                             // ranks of the kept entries
  int* rank = reinterpret_cast<int*>(hist);
  __shared__ uint32_t sh32[4 * NWAVE];
  __shared__ float red[NWAVE];
  __shared__ int ired[NWAVE];
  __shared__ int s_n, s_novf;
  __shared__ int s_wext[NWAVE];
  __shared__ uint32_t s_ld;
  const float T = a.temp[b];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int C = a.C, kk = min(a.topk, a.V);
  const size_t slot = (size_t)b * a.K + i;
  using CT = typename Cand<ET>::T;
  const CT* g = reinterpret_cast<const CT*>(a.cand) + slot * C * a.cstride;  // chunk r's list at r * cstride
  const int* gcnt = a.ccnt + slot * C * 2;  // chunk r: {length, bound key}
  const float s = LOG2E / T;
  if (t == 0) {
    s_n = 0;
    s_novf = 0;
    s_ld = 0xFFFFFFFFu;
  }
  uint64_t thr;
  float m, z = 0.f;
  bool held;
  if (C <= MERGE_REG) {
    // The list lengths (lane r holds chunk r's) and a window of 64 entries
    // of each list (wave w: entries [64 w, 64 w + 64), read whole: a list
    // area holds at least NWAVE * 64 entries).  Wave 0's windows come in the
    // lengths' round of loads; the other waves load theirs only where a list
    // reaches them (lists are usually shorter than 64).
    constexpr int HELD = NWAVE * 64;  // entries of a list held in registers
    RegCands<ET> rc;
    rc.CS = a.CS;
    const int my_cnt = lane < C ? *(gcnt + 2 * lane) : 0;
    if (wave == 0) {
#pragma unroll
      for (int r = 0; r < MERGE_REG; ++r) rc.v[r] = r < C ? *(g + (size_t)r * a.cstride + lane) : CT(0);
    } else {
#pragma unroll
      for (int r = 0; r < MERGE_REG; ++r) {
        const int n = r < C ? __builtin_amdgcn_readlane(my_cnt, r) : 0;
        rc.v[r] = wave * 64 < n ? *(g + (size_t)r * a.cstride + wave * 64 + lane) : CT(0);
      }
    }
    __syncthreads();  // s_n / s_novf / rank initialised
    // Entries past the first HELD of a list go to the overflow buffer: wave
    // w takes those of chunks w, w + NWAVE, ... (rare).
    rc.valid = 0u;
    int extra = 0;
#pragma unroll
    for (int r = 0; r < MERGE_REG; ++r) {
      const int n = r < C ? __builtin_amdgcn_readlane(my_cnt, r) : 0;
      if (wave * 64 + lane < n) rc.valid |= 1u << r;
      if (r % NWAVE == wave) extra += max(0, n - HELD);
    }
    // Each wave's overflow entries go to a fixed place in the buffer (waves
    // in order), so that the order of the candidates -- and with it every
    // sum over them -- does not depend on timing.
    if (lane == 0) s_wext[wave] = extra;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      if (w < wave) base += s_wext[w];
      total += s_wext[w];
    }
    if (t == 0) s_novf = total;
    if (extra > 0) {  // wave-uniform
      int o = base;
      for (int r = __builtin_amdgcn_readfirstlane(wave); r < C; r += NWAVE) {
        const int n = __builtin_amdgcn_readlane(my_cnt, r);
        for (int j = HELD + lane; j < n; j += 64)
          if (o + j - HELD < MERGE_OVF)
            ovf[o + j - HELD] = cand_composite<ET>(*(g + (size_t)r * a.cstride + j), r * a.CS);
        o += max(0, n - HELD);
      }
    }
    __syncthreads();
    rc.ovf = ovf;
    rc.novf = s_novf;
    if (rc.novf <= MERGE_OVF) {
      thr = select_threshold(rc, kk, sh32, red, ired, hist, &m);
      held = lists_hold_top(gcnt, C, thr, ired);
      if (held) z = take_kept(rc, thr, d, s, mul_rn(m, s), sel, &s_n, &s_ld);
    } else {
      const ListCands<ET> lc{g, gcnt, C, a.CS, a.cstride};
      thr = select_threshold(lc, kk, sh32, red, ired, hist, &m);
      held = lists_hold_top(gcnt, C, thr, ired);
      if (held) z = take_kept(lc, thr, d, s, mul_rn(m, s), sel, &s_n, &s_ld);
    }
  } else {
    __syncthreads();
    const ListCands<ET> lc{g, gcnt, C, a.CS, a.cstride};
    thr = select_threshold(lc, kk, sh32, red, ired, hist, &m);
    held = lists_hold_top(gcnt, C, thr, ired);
    if (held) z = take_kept(lc, thr, d, s, mul_rn(m, s), sel, &s_n, &s_ld);
  }
  if (!held) {
    // A chunk's list stops above the k-th largest of the union, so some of
    // its unlisted logits may belong to the top k: select again, with those
    // chunks' logits read from the draft row.  Only logits whose key is at
    // least the union's k-th largest can (it is a lower bound of the
    // global one).  The largest logit is always listed, so m stands.
    const MixedCands<ET> mc{g, gcnt, draft_row<ET>(a, b, i), C, a.CS, a.V, a.cstride, (uint32_t)(thr >> 32)};
    float m2;
    thr = select_threshold(mc, kk, sh32, red, ired, hist, &m2);
    z = take_kept(mc, thr, d, s, mul_rn(m, s), sel, &s_n, &s_ld);
  }
  const float Z = block_sum(z, red);  // also orders sel[] and s_ld before their reads
  const float ms = mul_rn(m, s);
  // Rank of each kept composite in id order (~id is larger for lower ids):
  // work items (entry j, block of 64 others) add their counts to rank[j].
  // Entries are read two at a time (16-byte LDS reads); sel[kk] (no kept
  // entry is written there) is zeroed first so that an odd kk reads a zero
  // (never larger) in its last pair.
  for (int j = t; j < kk; j += WG) rank[j] = 0;
  if (t == 0) sel[kk] = 0ull;  // kk < SV_MAX_TOPK + 1 entries: see the declaration
  __syncthreads();
  const int nblk = (kk + 63) / 64;
  const uint4* s4 = reinterpret_cast<const uint4*>(sel);
  for (int w = t; w < kk * nblk; w += WG) {
    const int j = w % kk, p0 = (w / kk) * 32, p1 = min(p0 + 32, (kk + 1) / 2);
    const uint32_t nid = (uint32_t)sel[j];
    int c = 0;
#pragma unroll 8
    for (int q = p0; q < p1; ++q) {
      const uint4 e = s4[q];
      c += (e.x > nid) + (e.z > nid);
    }
    atomicAdd(&rank[j], c);
  }
  __syncthreads();
  for (int j = t; j < kk; j += WG) {
    const uint64_t v = sel[j];
    a.kept[slot * a.topk + rank[j]] = make_uint2((uint32_t)composite_id(v), __float_as_uint(composite_value(v)));
  }
  if (t == 0) {
    const uint32_t lb = s_ld;
    const float qd = lb != 0xFFFFFFFFu ? exp2_fast(fmaf(__uint_as_float(lb), s, -ms)) / Z : 0.f;
    a.qstat[slot] = make_float4(m, Z, qd, (float)kk);
  }
  (void)lane;
  return kk;
}

// Eight waves per SIMD (64 VGPRs, no spills): the 2048 work-groups of a
// 256-row, 8-draft batch are resident at once.
template <typename ET>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(8, 8))) void merge_kernel(Args a) {
  const int i = blockIdx.x % a.K, b = blockIdx.x / a.K;
  if (!is_sampling_temperature(a.temp[b])) return;
  merge_body<ET>(a, b, i, a.tok[(size_t)b * a.K + i]);
}

// Finishing work-groups that take part per row, G <= C: each takes m chunks,
// with m the smallest count for which the sampling rows' work-groups are
// all resident at once (greedy rows need one work-group each, briefly).
constexpr int FINISH_COUNT_MAX = 4096;  // rows whose temperatures a work-group counts
__host__ __device__ __forceinline__ int finish_groups(int nsamp, int C, int resident) {
  if (resident <= 0 || nsamp <= 0) return C;
  const long long q = ((long long)nsamp * C + resident - 1) / resident;
  const long long m = q > 1 ? q : 1;
  return (int)((C + m - 1) / m);
}

// ============================================================================
// Kernel B: finishing work-group j of row b.  Decides the row from the
// statistics partials, then: greedy rows and rows that accepted every draft
// are completed by the row's work-group 0; for a rejected row each
// work-group publishes the 32 sub-block sums of max(0, p_n - q_n) over its
// chunks j, j + G, j + 2G, ..., and the last of the row's G work-groups to
// arrive (atomic counter) draws the correction token and clears the row's
// published words.  G is chosen from the number of sampling rows so that the
// working grid is about what the chip holds at once: every work-group
// decides once and then streams, and no late generation of work-groups
// drains after the others.
//
// Numbering.  Work-group x < B is work-group 0 of row x (every row has one).
// Work-group x >= B is work-group 1 + (x - B) / ns of the ((x - B) % ns)-th
// sampling row in row order (ns sampling rows), so the working work-groups
// come first in dispatch order and greedy rows take no slot beyond their
// first; those past the working set leave at once.  Each work-group first
// loads the row it would serve if every row sampled, which is its row
// whenever that is so, and loads its own row again otherwise.
// ============================================================================
__device__ __forceinline__ void write_failed_row(const Args& a, int b) {
  // Reached only if a wait ran past its deadline: num_accepted = -1 marks it.
  for (int i = threadIdx.x; i <= a.K; i += WG) a.out[(size_t)b * (a.K + 1) + i] = -1;
  if (threadIdx.x == 0) a.nacc[b] = -1;
}

template <typename ET, bool ALIGNED, bool CACHED>
__global__ __launch_bounds__(WG) void finish_kernel(Args a) {
  constexpr int VEC = Tr<ET>::VEC;
  extern __shared__ uint32_t row_cache[];
  __shared__ RowShared rs;
  __shared__ float shsub[NSUB];
  __shared__ int sh_last;
  __shared__ int sh_ns[NWAVE];
  __shared__ int sh_row;
  const int x = blockIdx.x, B = a.B;
  int b = x < B ? x : (x - B) % B;  // the row if every row samples
  // Waves issue at high priority while they decide and draw (a dependent
  // chain), and at the lowest while they stream the residual, so that the
  // streaming waves sharing a SIMD do not slow the decisions.
  __builtin_amdgcn_s_setprio(3);
  const int K = a.K, C = a.C, S = 2 * K + 1, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // Sparse draft: the row's kept list at the rejected position (ids and q~
  // values, for the residual and the final draw) and the corrections
  // min(p, q~) of the ids in this chunk.
  __shared__ float kq[SV_MAX_TOPK];
  __shared__ float kcorr[SV_MAX_TOPK];
  __shared__ int kid[SV_MAX_TOPK];
  uint32_t* cache_pw = CACHED ? row_cache : nullptr;
  uint32_t* cache_sub = CACHED ? cache_pw + (size_t)S * C * 4 : nullptr;
  RowIn in = load_row_in(a, b);
  // All partials of the row in one round of loads (also the draft-token
  // logits, which the decision reads at a token-dependent chunk).
  auto cache_partials = [&]() {
    if (CACHED) {
      const u32x4* src = reinterpret_cast<const u32x4*>(part_words(a, b, 0, 0));
      for (int i = t; i < S * C; i += WG) reinterpret_cast<u32x4*>(cache_pw)[i] = src[i];
    }
  };
  // The sampling rows of the batch, counted in the same round of loads:
  // thread t flags rows [t R, t R + R), so a scan of the counts ranks the
  // sampling rows in row order.
  const bool counted = B <= FINISH_COUNT_MAX;
  const int R = (B + WG - 1) / WG;  // at most 16 when counted
  uint32_t flags = 0u;
  if (counted)
    for (int i = 0; i < R; ++i) {
      const int r = t * R + i;
      if (r < B && is_sampling_temperature(a.temp[r])) flags |= 1u << i;
    }
  cache_partials();
  int total;
  const int mine = __popc(flags);
  const int before = block_count_scan(mine, sh_ns, total);  // exact: counts below 2^24
  const int ns = counted ? total : B;
  // A truncated draft's residual needs no pass over the logits: one
  // work-group per row.
  const int G = a.topk > 0 ? 1 : finish_groups(ns, C, a.resident);
  int j0 = 0;
  if (x >= B) {
    // Work-groups past the working set have nothing to do.
    const int y = x - B;
    if (ns == 0 || 1 + y / ns >= G) return;
    j0 = 1 + y / ns;
    if (ns < B) {
      // Serve the (y % ns)-th sampling row: its thread finds it.
      const int k = y % ns - before;
      if (k >= 0 && k < mine) {
        uint32_t f = flags;
        for (int i = 0; i < k; ++i) f &= f - 1u;
        sh_row = t * R + __builtin_ctz(f);
      }
      __syncthreads();
      if (sh_row != b) {
        b = sh_row;
        in = load_row_in(a, b);
        cache_partials();
        __syncthreads();
      }
    }
  }
  // A greedy row's work-groups past the first have nothing to do (reached
  // only when the rows were not counted).
  if (j0 != 0 && !is_sampling_temperature(in.T)) return;
  RowView<CACHED> view{cache_pw, cache_sub, false};
  decide_row(a, b, rs, view, in);
  const int n = rs.n;
  if (j0 == 0 && a.kl && t < K) {
    // KL(p_t || q_t) = E_p[l_t - l_q] / T - ln2 (fl(M_t s) - fl(M_q s)) - ln Z_t + ln Z_q,
    // with E_p[l_t - l_q] = sum_c A_c exp2(fl(m_c s) - fl(M_t s)) / Z_t; the
    // combination is done in double.
    float kl = __builtin_nanf("");
    if (!rs.greedy) {
      const float s = rs.s;
      const float MSt = mul_rn(rs.M[t], s), MSq = mul_rn(rs.M[K + 1 + t], s);
      double sa = 0.0;
      for (int cc = 0; cc < C; ++cc) {
        const float mc = view_part(a, view, b, t, cc, 0);
        if (mc != NEG_INF)
          sa += (double)view_part(a, view, b, K + 1 + t, cc, 2) * (double)exp2_fast(mul_rn(mc, s) - MSt);
      }
      const double ln2 = 0.69314718055994530942;
      const double Zt = rs.Z[t], Zq = rs.Z[K + 1 + t];
      kl = (float)(sa / Zt * ((double)s * ln2) - ln2 * ((double)MSt - (double)MSq) - log(Zt) + log(Zq));
    }
    a.kl[(size_t)b * K + t] = kl;
  }
  if (j0 == 0 && a.probs && t < K) {
    a.probs[((size_t)b * K + t) * 2 + 0] = rs.greedy ? 0.f : rs.p[t];
    a.probs[((size_t)b * K + t) * 2 + 1] = rs.greedy ? 0.f : rs.q[t];
  }
  if (rs.greedy) {
    if (j0 != 0) return;
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
    if (j0 == 0) final_draw<ET, ALIGNED, CACHED>(a, b, n, s, MSt, rZt, 0.f, 0.f, rs, view, nullptr, nullptr, 0);
    return;
  }
  uint32_t* subR_row = a.subR + (size_t)b * C * NSUB;
  if (a.topk > 0) {
    // Rejected at position n with a truncated draft: the row's single
    // work-group forms the residual's sub-block sums from the statistics
    // pass's sums and the kept list (no pass over the logits) and draws.
    const uint2* kept = a.kept + ((size_t)b * K + n) * a.topk;
    const float4 qs = a.qstat[(size_t)b * K + n];
    const float MSq = mul_rn(qs.x, s), rZq = 1.f / qs.y;
    const int nkept = (int)qs.w;
    // The kept list and the position's sub-block sums in one round of loads.
    float* R = reinterpret_cast<float*>(cache_sub);
    for (int j = t; j < nkept; j += WG) {
      const uint2 e = kept[j];
      kid[j] = (int)e.x;
      kq[j] = exp2_fast(fmaf(__uint_as_float(e.y), s, -MSq)) * rZq;
    }
    if (CACHED)
      for (int i = t; i < C * NSUB; i += WG) R[i] = __uint_as_float(sub_words(a, b, n, 0)[i]);
    __syncthreads();
    const ET* trow = target_row<ET>(a, b, n);
    sparse_residual<ET>(
        a.V, C, a.CS, s, MSt, rZt, kid, kq, nkept, kcorr,
        [&](int j) { return exp2_fast(fmaf(Tr<ET>::load1(trow + kid[j]), s, -MSt)) * rZt; },
        [&](int c, int u) { return CACHED ? R[c * NSUB + u] : __uint_as_float(sub_words(a, b, n, c)[u]); },
        [&](int c) { return view_part(a, view, b, n, c, 0); },
        [&](int i, float r) {
          if (CACHED) R[i] = r;
          else pub_f32(subR_row + i, r);
        });
    bool ok = true;
    if (!CACHED)  // this work-group's own published sums, read back as published words
      ok = wait_words(subR_row, C * NSUB, nullptr, nullptr, 0, nullptr, wall_clock64() + WAIT_TICKS);
    view.sub_loaded = CACHED;
    if (ok) final_draw<ET, ALIGNED, CACHED>(a, b, n, s, MSt, rZt, MSq, rZq, rs, view, kid, kq, nkept);
    else write_failed_row(a, b);
    if (!CACHED) {
      __syncthreads();
      for (int i = t; i < C * NSUB; i += WG) clear_word(subR_row + i);
    }
    return;
  }
  // Rejected at position n: residual max(0, p_n - q_n) over the
  // work-group's chunks, each published as 32 sub-block sums.
  const float MSq = mul_rn(rs.M[K + 1 + n], s), rZq = 1.f / rs.Z[K + 1 + n];
  __builtin_amdgcn_s_setprio(0);
  for (int c = j0; c < C; c += G) {
    const int lo = c * a.CS;
    const int len = min(a.CS, a.V - lo);
    u32x4 rt[NV_TILE], rq[NV_TILE];
    load_tile<ET, ALIGNED, NV_TILE>(target_row<ET>(a, b, n), lo, len, rt);
    load_tile<ET, ALIGNED, NV_TILE>(draft_row<ET>(a, b, n), lo, len, rq);
#pragma unroll
    for (int jv = 0; jv < NV_TILE; ++jv) {
      float w0 = 0.f, w1 = 0.f;
#pragma unroll
      for (int k = 0; k < VEC; k += 2) {
        const float p0 = exp2_fast(fmaf(Tr<ET>::at(rt[jv], k), s, -MSt)) * rZt;
        const float q0 = exp2_fast(fmaf(Tr<ET>::at(rq[jv], k), s, -MSq)) * rZq;
        const float p1 = exp2_fast(fmaf(Tr<ET>::at(rt[jv], k + 1), s, -MSt)) * rZt;
        const float q1 = exp2_fast(fmaf(Tr<ET>::at(rq[jv], k + 1), s, -MSq)) * rZq;
        w0 += fmaxf(0.f, p0 - q0);
        w1 += fmaxf(0.f, p1 - q1);
      }
      const float v = wave_sum(w0 + w1);
      if (lane == 0) shsub[jv * NWAVE + wave] = v;
    }
    __syncthreads();
    if (t < NSUB) pub_f32(subR_row + (size_t)c * NSUB + t, shsub[t]);
    __syncthreads();  // shsub is reused by the next chunk
  }
  __builtin_amdgcn_s_setprio(3);
  // Count this work-group.  Its sums need no ordering with the count: the
  // last work-group polls them until they are published (each of its peers
  // has already issued its stores, so the wait ends).
  if (t == 0)
    sh_last = __hip_atomic_fetch_add(a.cnt + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)G - 1u;
  __syncthreads();
  if (!sh_last) return;
  const bool ok = wait_words(subR_row, C * NSUB, cache_sub, nullptr, 0, nullptr, wall_clock64() + WAIT_TICKS);
  view.sub_loaded = CACHED;
  final_draw<ET, ALIGNED, CACHED>(a, b, n, s, MSt, rZt, MSq, rZq, rs, view, nullptr, nullptr, 0);
  // With the sums in LDS the other waves clear the published words while
  // wave 0 draws; otherwise the draw reads them, so the clear waits.
  if (!CACHED || !ok) __syncthreads();
  if (!ok) write_failed_row(a, b);
  // Clear the row's published sums and counter for the next call.
  for (int i = t; i < C * NSUB; i += WG) clear_word(subR_row + i);
  if (t == 0) __hip_atomic_store(a.cnt + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

#include "early_exit.h"

// ============================================================================
// Host side.
// ============================================================================
struct Plan {
  int C = 0, CS = 0;
  int ckeep = 0, cstride = 0;  // sparse drafts: see cand_layout
  size_t off_cnt = 0, off_part = 0, off_subK = 0, off_subR = 0, off_cand = 0, off_ccnt = 0, off_qstat = 0, off_kept = 0,
         total = 0;
  size_t zero_bytes = 0;    // leading bytes holding every region that must be zero before a call
  size_t merge_lds = 0;
  bool cache = false;       // finishing work-groups copy the row's words to LDS
  size_t lds_bytes = 0;     // dynamic LDS of the finishing work-groups
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Vocabulary chunks: as few as hold the row with one register tile per
// thread, then equal lengths (a multiple of the vector width), the last one
// possibly shorter.
bool vocab_split(int V, int dtype, int& C, int& CS) {
  const long vec = dtype == SV_BF16 ? 8 : 4;
  const long tile = (long)WG * NV_TILE * vec;
  long c = (V + tile - 1) / tile;
  if (c > MAX_C) return false;
  const long cs = ((V + c - 1) / c + vec - 1) / vec * vec;
  C = (int)((V + cs - 1) / cs);
  CS = (int)cs;
  return true;
}

// Sparse drafts: the logits each chunk lists at least, one and a half times
// a chunk's share of the top k plus 8 (a chunk holding more of the top k
// than its list is read again by the merge kernel), and the entries of a chunk's
// candidate area: room for three times that (a fast-path list over it takes
// the exact path), for the exact path's min(k, len) and for the merge
// kernel's fixed windows of NWAVE * 64 entries.
void cand_layout(int topk, int V, int C, int& keep, int& stride) {
  const int kk = std::min(topk, V);
  keep = std::min(kk, (3 * kk + 2 * C - 1) / (2 * C) + 8);
  const int st = std::max(std::max(NWAVE * 64, kk), 3 * keep);
  stride = (st + 63) / 64 * 64;
}

int make_plan(int B, int K, int V, int topk, int dtype, Plan& pl) {
  if (B < 1 || K < 0 || V < 1 || topk < 0 || (dtype != SV_BF16 && dtype != SV_F32)) return SV_ERR_ARG;
  if (K > SV_MAX_K) return SV_ERR_UNSUPPORTED;
  if (topk > SV_MAX_TOPK) return SV_ERR_UNSUPPORTED;
  int C, CS;
  if (!vocab_split(V, dtype, C, CS)) return SV_ERR_UNSUPPORTED;
  const long long grid = (long long)B * (2 * K + 1) * C;
  if (grid > INT_MAX) return SV_ERR_UNSUPPORTED;
  pl.C = C;
  pl.CS = CS;
  const size_t S = 2 * (size_t)K + 1;
  // Every region is zero between calls (see spec_verify.h).
  size_t off = 0;
  pl.off_cnt = off;
  off = align256(off + sizeof(unsigned) * (size_t)B);
  pl.off_part = off;
  off = align256(off + 4 * sizeof(uint32_t) * (size_t)B * S * C);
  pl.off_subK = off;  // target sub-block sums: every position's with a truncated draft, else the bonus's
  off = align256(off + sizeof(uint32_t) * (size_t)B * (topk > 0 ? K + 1 : 1) * C * NSUB);
  pl.off_subR = off;
  off = align256(off + sizeof(uint32_t) * (size_t)B * C * NSUB);
  if (topk > 0) {
    const size_t slots = (size_t)B * K;
    cand_layout(topk, V, C, pl.ckeep, pl.cstride);
    pl.off_cand = off;
    off = align256(off + sizeof(uint64_t) * slots * C * pl.cstride);
    pl.off_ccnt = off;
    off = align256(off + 2 * sizeof(int) * slots * C);
    pl.off_qstat = off;
    off = align256(off + sizeof(float4) * slots);
    pl.off_kept = off;
    off = align256(off + sizeof(uint2) * slots * topk);
    pl.merge_lds = 0;
  }
  pl.total = off;
  pl.zero_bytes = topk > 0 ? pl.off_cand : off;  // the candidate area is written before it is read
  // Dynamic LDS of the finishing work-groups: the row's partials and
  // sub-block sums when they fit.
  const size_t words = S * C * 4 + (size_t)C * NSUB;
  pl.cache = words <= (size_t)MAX_CACHE_WORDS;
  pl.lds_bytes = (pl.cache ? words : 0) * sizeof(uint32_t);
  return SV_OK;
}

// Launches a kernel; with a start/stop event pair (timed calls) the events
// take the dispatch's own start and end timestamps.
template <typename F>
int launch(F kernel, int grid, size_t lds, hipStream_t st, hipEvent_t* ev2, const Args& a) {
  if (ev2)
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(WG), (uint32_t)lds, st, ev2[0], ev2[1], 0, a);
  else
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(WG), lds, st, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

// Work-groups of `kernel` (WG threads, `lds` bytes of dynamic LDS) that the
// current device holds at once, or 0 if unknown; remembered per device,
// kernel and LDS size.
int resident_groups(const void* kernel, size_t lds) {
  struct Entry {
    int dev;
    const void* kernel;
    size_t lds;
    int groups;
  };
  constexpr int N = 64;
  static Entry seen[N];
  static int used = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (seen[i].dev == dev && seen[i].kernel == kernel && seen[i].lds == lds) return seen[i].groups;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, WG, lds) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int groups = cus * per_cu;
  if (used < N) seen[used++] = Entry{dev, kernel, lds, groups};
  return groups;
}

// Finishing grid: B work-groups (one per row) plus the largest number that
// serve sampling rows past their first, over every count of sampling rows
// the batch may hold (the kernel counts them).  Remembered per shape.
int finish_grid(int B, int C, int resident, int topk) {
  if (topk > 0) return B;  // one work-group per row
  if (B > FINISH_COUNT_MAX) return B * finish_groups(B, C, resident);  // rows not counted: all sample
  struct Entry {
    int B, C, resident, grid;
  };
  constexpr int N = 64;
  static Entry seen[N];
  static int used = 0, next = 0;
  static std::mutex mu;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (seen[i].B == B && seen[i].C == C && seen[i].resident == resident) return seen[i].grid;
  long long w = B;
  for (int ns = 1; ns <= B; ++ns) w = std::max(w, B + (long long)(finish_groups(ns, C, resident) - 1) * ns);
  const int grid = (int)w;
  seen[next] = Entry{B, C, resident, grid};
  next = (next + 1) % N;
  used = std::min(used + 1, N);
  return grid;
}

template <typename ET, bool AL>
int launch_typed(const Args& a, size_t lds, size_t merge_lds, hipStream_t st, hipEvent_t* ev) {
  int rc = a.kl ? launch(paired_kernel<ET, AL>, a.B * (a.K + 1) * a.C, 0, st, ev, a)
                : launch(a.topk > 0 ? stats_kernel<ET, AL, STATS_WAVES_TOPK> : stats_kernel<ET, AL, STATS_WAVES>,
                         a.B * a.GA, 0, st, ev, a);
  if (rc != SV_OK) return rc;
  if (a.topk > 0 && a.K > 0) {
    rc = launch(merge_kernel<ET>, a.B * a.K, merge_lds, st, ev ? ev + 2 : nullptr, a);
    if (rc != SV_OK) return rc;
  } else if (ev) {
    if (hipEventRecord(ev[2], st) != hipSuccess || hipEventRecord(ev[3], st) != hipSuccess) return SV_ERR_HIP;
  }
  void (*const fk)(Args) = a.cache ? finish_kernel<ET, AL, true> : finish_kernel<ET, AL, false>;
  Args af = a;
  af.resident = resident_groups(reinterpret_cast<const void*>(fk), lds);
  return launch(fk, finish_grid(a.B, a.C, af.resident, a.topk), lds, st, ev ? ev + 4 : nullptr, af);
}

struct RelaxedRule {
  float alpha;
  int max_rank;
  float min_prob;
};

int run(const void* tgt, const void* dft, const int32_t* tok, const float* uni, const float* temp,
        int B, int K, int V, int topk, int dtype, int32_t* out, int32_t* nacc, void* ws,
        size_t* ws_bytes, hipStream_t st, float* probs, float* mass, hipEvent_t* ev, int nev,
        const RelaxedRule* rule = nullptr, float* kl = nullptr) {
  if (!ws_bytes) return SV_ERR_ARG;
  if (rule && !(rule->alpha >= 0.f && rule->alpha <= 1e30f && rule->min_prob >= 0.f &&
                rule->min_prob <= 1.f && rule->max_rank >= 0))
    return SV_ERR_ARG;
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
  if (nev != 0 && (nev != 6 || !ev)) return SV_ERR_ARG;
  Args a;
  a.tgt = tgt; a.dft = dft; a.tok = tok; a.uni = uni; a.temp = temp;
  a.out = out; a.nacc = nacc; a.probs = probs; a.mass = mass;
  char* base = static_cast<char*>(ws);
  a.cnt = reinterpret_cast<unsigned*>(base + pl.off_cnt);
  a.part = reinterpret_cast<uint32_t*>(base + pl.off_part);
  a.subK = reinterpret_cast<uint32_t*>(base + pl.off_subK);
  a.subR = reinterpret_cast<uint32_t*>(base + pl.off_subR);
  a.B = B; a.K = K; a.V = V; a.C = pl.C; a.CS = pl.CS; a.topk = topk;
  a.ckeep = pl.ckeep; a.cstride = pl.cstride;
  a.GA = (2 * K + 1) * pl.C;
  a.resident = 0;
  a.cache = pl.cache ? 1 : 0;
  a.kl = kl;
  a.relaxed = rule ? 1 : 0;
  a.alpha = rule ? rule->alpha : 0.f;
  a.max_rank = rule ? rule->max_rank : 0;
  a.min_prob = rule ? rule->min_prob : 0.f;
  a.cand = topk > 0 ? static_cast<void*>(base + pl.off_cand) : nullptr;
  a.ccnt = topk > 0 ? reinterpret_cast<int*>(base + pl.off_ccnt) : nullptr;
  a.qstat = topk > 0 ? reinterpret_cast<float4*>(base + pl.off_qstat) : nullptr;
  a.kept = topk > 0 ? reinterpret_cast<uint2*>(base + pl.off_kept) : nullptr;
  const size_t esz = dtype == SV_BF16 ? 2 : 4;
  const bool aligned = (reinterpret_cast<uintptr_t>(tgt) % 16 == 0) &&
                       (K == 0 || reinterpret_cast<uintptr_t>(dft) % 16 == 0) &&
                       ((size_t)V * esz) % 16 == 0;
  (void)hipGetLastError();  // start from a clean error state
  hipEvent_t* e = nev ? ev : nullptr;
  if (dtype == SV_BF16)
    return aligned ? launch_typed<uint16_t, true>(a, pl.lds_bytes, pl.merge_lds, st, e)
                   : launch_typed<uint16_t, false>(a, pl.lds_bytes, pl.merge_lds, st, e);
  return aligned ? launch_typed<float, true>(a, pl.lds_bytes, pl.merge_lds, st, e)
                 : launch_typed<float, false>(a, pl.lds_bytes, pl.merge_lds, st, e);
}

// ---- early exit ---------------------------------------------------------------
constexpr int EE_MAX_LDS_WORDS = 14336;  // the early-exit kernel's dynamic LDS (56 KiB)

struct EEPlan {
  int C = 0, CS = 0;
  int ckeep = 0, cstride = 0;
  size_t off_cnt = 0, off_part = 0, off_subK = 0, off_subR = 0, total = 0;
  size_t off_cand = 0, off_ccnt = 0, off_qstat = 0, off_kept = 0;
  size_t lds_bytes = 0;
};

int make_ee_plan(int B, int K, int V, int dtype, int topk, EEPlan& pl) {
  if (B < 1 || K < 0 || V < 1 || (dtype != SV_BF16 && dtype != SV_F32)) return SV_ERR_ARG;
  if (K > SV_MAX_K || topk > SV_MAX_TOPK) return SV_ERR_UNSUPPORTED;
  int C, CS;
  if (!vocab_split(V, dtype, C, CS)) return SV_ERR_UNSUPPORTED;
  if ((long long)B * (K + 1) * C > INT_MAX) return SV_ERR_UNSUPPORTED;
  const size_t S = 2 * (size_t)K + 1;
  const size_t words = S * C * 4 + (size_t)C * NSUB + 3 * (size_t)topk;
  if (words > (size_t)EE_MAX_LDS_WORDS) return SV_ERR_UNSUPPORTED;
  pl.C = C;
  pl.CS = CS;
  // The counters, partial words and sums are zero between calls: the kernel
  // publishes into them and clears what it used.  The candidate lists and
  // selections of a truncated draft are plain, written before they are read.
  size_t off = 0;
  pl.off_cnt = off;  // claim [B], then leave [B]
  off = align256(off + 2 * sizeof(unsigned) * (size_t)B);
  pl.off_part = off;
  off = align256(off + 4 * sizeof(uint32_t) * (size_t)B * S * C);
  pl.off_subK = off;  // target sub-block sums: every position's with a truncated draft, else the bonus's
  off = align256(off + sizeof(uint32_t) * (size_t)B * (topk > 0 ? K + 1 : 1) * C * NSUB);
  pl.off_subR = off;
  off = align256(off + sizeof(uint32_t) * (size_t)B * C * NSUB);
  if (topk > 0) {
    const size_t slots = (size_t)B * K;
    cand_layout(topk, V, C, pl.ckeep, pl.cstride);
    pl.off_cand = off;
    off = align256(off + sizeof(uint64_t) * slots * C * pl.cstride);
    pl.off_ccnt = off;
    off = align256(off + 2 * sizeof(int) * slots * C);
    pl.off_qstat = off;
    off = align256(off + sizeof(float4) * slots);
    pl.off_kept = off;
    off = align256(off + sizeof(uint2) * slots * topk);
  }
  pl.total = off;
  pl.lds_bytes = words * sizeof(uint32_t);
  return SV_OK;
}

// A truncated draft: position 0's statistics and the drafts' candidate
// lists, the selections, then the walk.  A dense draft: the walk alone.
template <typename ET, bool AL>
int launch_early_exit(const Args& a, size_t lds, hipStream_t st) {
  if (a.topk > 0) {
    int rc = launch(ee_first_kernel<ET, AL, EE_FIRST_WAVES>, a.B * (a.K + 1) * a.C, 0, st, nullptr, a);
    if (rc == SV_OK) rc = launch(merge_kernel<ET>, a.B * a.K, 0, st, nullptr, a);
    if (rc != SV_OK) return rc;
    return launch(early_exit_kernel<ET, AL, true>, a.B * a.C, lds, st, nullptr, a);
  }
  return launch(early_exit_kernel<ET, AL, false>, a.B * a.C, lds, st, nullptr, a);
}

int run_early_exit(const void* tgt, const void* dft, const int32_t* tok, const float* uni, const float* temp,
                   int B, int K, int V, int topk, int dtype, int32_t* out, int32_t* nacc, void* ws,
                   size_t* ws_bytes, hipStream_t st, float* probs, float* mass) {
  if (!ws_bytes || topk < 0) return SV_ERR_ARG;
  if (topk >= V || K == 0) topk = 0;  // no draft to truncate
  EEPlan pl;
  const int rc = make_ee_plan(B, K, V, dtype, topk, pl);
  if (rc != SV_OK) return rc;
  if (!ws) {
    *ws_bytes = pl.total;
    return SV_OK;
  }
  if (*ws_bytes < pl.total) return SV_ERR_WORKSPACE;
  if (!tgt || !uni || !temp || !out || !nacc) return SV_ERR_ARG;
  if (K > 0 && (!dft || !tok)) return SV_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return SV_ERR_ARG;
  Args a{};
  a.tgt = tgt; a.dft = dft; a.tok = tok; a.uni = uni; a.temp = temp;
  a.out = out; a.nacc = nacc; a.probs = probs; a.mass = mass;
  char* base = static_cast<char*>(ws);
  a.claim = reinterpret_cast<unsigned*>(base + pl.off_cnt);
  a.leave = a.claim + B;
  a.part = reinterpret_cast<uint32_t*>(base + pl.off_part);
  a.subK = reinterpret_cast<uint32_t*>(base + pl.off_subK);
  a.subR = reinterpret_cast<uint32_t*>(base + pl.off_subR);
  a.cand = topk > 0 ? static_cast<void*>(base + pl.off_cand) : nullptr;
  a.ccnt = topk > 0 ? reinterpret_cast<int*>(base + pl.off_ccnt) : nullptr;
  a.qstat = topk > 0 ? reinterpret_cast<float4*>(base + pl.off_qstat) : nullptr;
  a.kept = topk > 0 ? reinterpret_cast<uint2*>(base + pl.off_kept) : nullptr;
  a.B = B; a.K = K; a.V = V; a.C = pl.C; a.CS = pl.CS; a.topk = topk;
  a.ckeep = pl.ckeep; a.cstride = pl.cstride;
  const size_t esz = dtype == SV_BF16 ? 2 : 4;
  const bool aligned = (reinterpret_cast<uintptr_t>(tgt) % 16 == 0) &&
                       (K == 0 || reinterpret_cast<uintptr_t>(dft) % 16 == 0) && ((size_t)V * esz) % 16 == 0;
  (void)hipGetLastError();
  if (dtype == SV_BF16)
    return aligned ? launch_early_exit<uint16_t, true>(a, pl.lds_bytes, st)
                   : launch_early_exit<uint16_t, false>(a, pl.lds_bytes, st);
  return aligned ? launch_early_exit<float, true>(a, pl.lds_bytes, st)
                 : launch_early_exit<float, false>(a, pl.lds_bytes, st);
}

// ---- draft trees ------------------------------------------------------------
#include "tree_kernels.h"

constexpr int TREE_MAX_LDS_WORDS = 14336;  // the walking kernel's dynamic LDS (56 KiB)

struct TreePlan {
  int C = 0, CS = 0;
  int ckeep = 0, cstride = 0;
  size_t off_cnt = 0, off_part = 0, off_subK = 0, off_subR = 0, off_gath = 0, total = 0;
  size_t off_cand = 0, off_ccnt = 0, off_qstat = 0, off_kept = 0;
  size_t lds_bytes = 0;
};

int make_tree_plan(int B, int N, int V, int dtype, int topk, TreePlan& pl) {
  if (B < 1 || N < 1 || V < 1 || (dtype != SV_BF16 && dtype != SV_F32)) return SV_ERR_ARG;
  if (N > SV_MAX_NODES || topk > SV_MAX_TOPK) return SV_ERR_UNSUPPORTED;
  int C, CS;
  if (!vocab_split(V, dtype, C, CS)) return SV_ERR_UNSUPPORTED;
  if ((long long)B * 2 * N * C > INT_MAX) return SV_ERR_UNSUPPORTED;
  const size_t words = (size_t)2 * N * C * 4 + (size_t)C * NSUB + 5 * (size_t)topk;
  if (words > (size_t)TREE_MAX_LDS_WORDS) return SV_ERR_UNSUPPORTED;
  pl.C = C;
  pl.CS = CS;
  // The counters and subR are zero between calls; the other regions are
  // written before they are read.
  size_t off = 0;
  pl.off_cnt = off;  // claim [B], then leave [B]
  off = align256(off + 2 * sizeof(unsigned) * (size_t)B);
  pl.off_part = off;
  off = align256(off + 4 * sizeof(uint32_t) * (size_t)B * 2 * N * C);
  pl.off_subK = off;
  off = align256(off + sizeof(uint32_t) * (size_t)B * N * C * NSUB);
  pl.off_subR = off;
  off = align256(off + sizeof(uint32_t) * (size_t)B * N * C * NSUB);
  pl.off_gath = off;
  off = align256(off + 2 * sizeof(float) * (size_t)B * N);
  if (topk > 0) {
    const size_t nodes = (size_t)B * N;
    cand_layout(topk, V, C, pl.ckeep, pl.cstride);
    pl.off_cand = off;
    off = align256(off + sizeof(uint64_t) * nodes * C * pl.cstride);
    pl.off_ccnt = off;
    off = align256(off + 2 * sizeof(int) * nodes * C);
    pl.off_qstat = off;
    off = align256(off + sizeof(float4) * nodes);
    pl.off_kept = off;
    off = align256(off + sizeof(uint2) * nodes * topk);
  }
  pl.total = off;
  pl.lds_bytes = words * sizeof(uint32_t);
  return SV_OK;
}

template <typename F>
int launch_tree_kernel(F kernel, int grid, size_t lds, hipStream_t st, hipEvent_t start, hipEvent_t stop,
                       const TreeArgs& a) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(WG), (uint32_t)lds, st, start, stop, 0, a);
  else
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(WG), lds, st, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

template <typename ET, bool AL>
int launch_tree(const TreeArgs& a, size_t lds, hipStream_t st, hipEvent_t* ev) {
  int rc = launch_tree_kernel(tree_stats_kernel<ET, AL>, a.B * a.N * a.C, 0, st, ev ? ev[0] : nullptr,
                              ev ? ev[1] : nullptr, a);
  if (rc != SV_OK) return rc;
  if (a.topk > 0) {
    // The exact top-k of each node's draft, through the merge of the sparse
    // linear path (positions read as nodes).
    Args m{};
    m.temp = a.temp;
    m.dft = a.dft;  // node v's draft row is row (b, v) of [B, N, V]: the fallback reads it
    m.cand = a.cand; m.ccnt = a.ccnt; m.qstat = a.qstat; m.kept = a.kept;
    m.B = a.B; m.K = a.N; m.V = a.V; m.C = a.C; m.CS = a.CS; m.topk = a.topk;
    m.ckeep = a.ckeep; m.cstride = a.cstride;
    hipLaunchKernelGGL(tree_merge_kernel<ET>, dim3(a.B * a.N), dim3(WG), 0, st, a, m);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
  }
  return launch_tree_kernel(tree_finish_kernel<ET, AL>, a.B * a.C, lds, st, ev ? ev[2] : nullptr,
                            ev ? ev[3] : nullptr, a);
}

int run_tree(const void* tgt, const void* dft, const int32_t* tok, const int32_t* par, const float* uni,
             const float* temp, int B, int N, int V, int topk, int dtype, int32_t* out, int32_t* onodes,
             int32_t* nacc, void* ws, size_t* ws_bytes, hipStream_t st, float* probs, float* mass,
             hipEvent_t* ev, int nev) {
  if (!ws_bytes || topk < 0) return SV_ERR_ARG;
  if (topk >= V) topk = 0;
  TreePlan pl;
  const int rc = make_tree_plan(B, N, V, dtype, topk, pl);
  if (rc != SV_OK) return rc;
  if (!ws) {
    *ws_bytes = pl.total;
    return SV_OK;
  }
  if (*ws_bytes < pl.total) return SV_ERR_WORKSPACE;
  if (!tgt || !uni || !temp || !out || !onodes || !nacc) return SV_ERR_ARG;
  if (N > 1 && (!dft || !tok || !par)) return SV_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return SV_ERR_ARG;
  if (nev != 0 && (nev != 4 || !ev)) return SV_ERR_ARG;
  TreeArgs a;
  a.tgt = tgt; a.dft = dft; a.tok = tok; a.par = par; a.uni = uni; a.temp = temp;
  a.out = out; a.onodes = onodes; a.nacc = nacc; a.probes = probs; a.mass = mass;
  char* base = static_cast<char*>(ws);
  a.claim = reinterpret_cast<unsigned*>(base + pl.off_cnt);
  a.leave = a.claim + B;
  a.part = reinterpret_cast<uint32_t*>(base + pl.off_part);
  a.subK = reinterpret_cast<uint32_t*>(base + pl.off_subK);
  a.subR = reinterpret_cast<uint32_t*>(base + pl.off_subR);
  a.gath = reinterpret_cast<float*>(base + pl.off_gath);
  a.cand = topk > 0 ? static_cast<void*>(base + pl.off_cand) : nullptr;
  a.ccnt = topk > 0 ? reinterpret_cast<int*>(base + pl.off_ccnt) : nullptr;
  a.qstat = topk > 0 ? reinterpret_cast<float4*>(base + pl.off_qstat) : nullptr;
  a.kept = topk > 0 ? reinterpret_cast<uint2*>(base + pl.off_kept) : nullptr;
  a.B = B; a.N = N; a.V = V; a.C = pl.C; a.CS = pl.CS; a.topk = topk;
  a.ckeep = pl.ckeep; a.cstride = pl.cstride;
  const size_t esz = dtype == SV_BF16 ? 2 : 4;
  const bool aligned = (reinterpret_cast<uintptr_t>(tgt) % 16 == 0) &&
                       (N == 1 || reinterpret_cast<uintptr_t>(dft) % 16 == 0) && ((size_t)V * esz) % 16 == 0;
  (void)hipGetLastError();
  hipEvent_t* e = nev ? ev : nullptr;
  if (dtype == SV_BF16)
    return aligned ? launch_tree<uint16_t, true>(a, pl.lds_bytes, st, e)
                   : launch_tree<uint16_t, false>(a, pl.lds_bytes, st, e);
  return aligned ? launch_tree<float, true>(a, pl.lds_bytes, st, e)
                 : launch_tree<float, false>(a, pl.lds_bytes, st, e);
}

// Zeroes n 16-byte words (the no-allocation entry point's scratch, before a
// call): an ordinary kernel, so a call stays capturable in a HIP graph.
__global__ __launch_bounds__(WG) void zero_fill_kernel(u32x4* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * WG + threadIdx.x; i < n; i += (size_t)gridDim.x * WG)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

// ---- static scratch of spec_verify_noalloc ----------------------------------
// One copy per GPU, zero at module load, held until the process ends.  In
// host code `scratch` names a host-side stand-in, not the device array: its
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[SV_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::once_flag g_scratch_once[SCRATCH_MAX_DEVICES];
void* g_scratch_ptr[SCRATCH_MAX_DEVICES];

// The scratch's device address on the current device (nullptr on failure).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) p = nullptr;
    g_scratch_ptr[dev] = p;
  });
  return g_scratch_ptr[dev];
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

int spec_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                        const float* uniforms, const float* temperature, int B, int K, int V, int topk_draft,
                        int dtype, int32_t* out_tokens, int32_t* num_accepted, hipStream_t stream) {
  Plan pl;
  const int rc = make_plan(B, K, V, topk_draft >= V ? 0 : topk_draft, dtype, pl);
  if (rc != SV_OK) return rc;
  if (pl.total > (size_t)SV_SCRATCH_BYTES) return SV_ERR_SCRATCH;
  if (!target_logits || !uniforms || !temperature || !out_tokens || !num_accepted) return SV_ERR_ARG;
  if (K > 0 && (!draft_logits || !draft_tokens)) return SV_ERR_ARG;
  void* ws = scratch_address();
  if (!ws) return SV_ERR_HIP;
  // The regions that must start at zero: the previous call may have had
  // another shape, whose layout left other words there.
  (void)hipGetLastError();
  const size_t n16 = pl.zero_bytes / 16;
  if (n16 > 0) {
    const int grid = (int)std::min<size_t>(1024, (n16 + WG - 1) / WG);
    hipLaunchKernelGGL(zero_fill_kernel, dim3(grid), dim3(WG), 0, stream, static_cast<u32x4*>(ws), n16);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
  }
  size_t ws_bytes = SV_SCRATCH_BYTES;
  return run(target_logits, draft_logits, draft_tokens, uniforms, temperature, B, K, V, topk_draft, dtype,
             out_tokens, num_accepted, ws, &ws_bytes, stream, nullptr, nullptr, nullptr, 0);
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

int spec_verify_relaxed(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                        const float* uniforms, const float* temperature, int B, int K, int V,
                        int topk_draft, int dtype, float alpha, int max_rank, float min_prob,
                        int32_t* out_tokens, int32_t* num_accepted, void* workspace,
                        size_t* workspace_bytes, hipStream_t stream, float* probs_out, float* mass_out) {
  const RelaxedRule rule{alpha, max_rank, min_prob};
  return run(target_logits, draft_logits, draft_tokens, uniforms, temperature, B, K, V, topk_draft,
             dtype, out_tokens, num_accepted, workspace, workspace_bytes, stream, probs_out, mass_out,
             nullptr, 0, &rule);
}

int spec_verify_kl(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                   const float* uniforms, const float* temperature, int B, int K, int V, int topk_draft,
                   int dtype, int32_t* out_tokens, int32_t* num_accepted, void* workspace,
                   size_t* workspace_bytes, hipStream_t stream, float* kl_out) {
  if (topk_draft > 0 && topk_draft < V) return SV_ERR_UNSUPPORTED;
  if (workspace && K > 0 && !kl_out) return SV_ERR_ARG;
  return run(target_logits, draft_logits, draft_tokens, uniforms, temperature, B, K, V, topk_draft,
             dtype, out_tokens, num_accepted, workspace, workspace_bytes, stream, nullptr, nullptr,
             nullptr, 0, nullptr, K > 0 ? kl_out : nullptr);
}

int spec_verify_early_exit(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                           const float* uniforms, const float* temperature, int B, int K, int V, int topk_draft,
                           int dtype, int32_t* out_tokens, int32_t* num_accepted, void* workspace,
                           size_t* workspace_bytes, hipStream_t stream, float* probs_out, float* mass_out) {
  return run_early_exit(target_logits, draft_logits, draft_tokens, uniforms, temperature, B, K, V, topk_draft,
                        dtype, out_tokens, num_accepted, workspace, workspace_bytes, stream, probs_out, mass_out);
}

int spec_verify_tree(const void* target_logits, const void* draft_logits, const int32_t* node_tokens,
                     const int32_t* parents, const float* uniforms, const float* temperature, int B, int N,
                     int V, int topk_draft, int dtype, int32_t* out_tokens, int32_t* out_nodes,
                     int32_t* num_accepted, void* workspace, size_t* workspace_bytes, hipStream_t stream,
                     float* probs_out, float* mass_out) {
  return run_tree(target_logits, draft_logits, node_tokens, parents, uniforms, temperature, B, N, V, topk_draft,
                  dtype, out_tokens, out_nodes, num_accepted, workspace, workspace_bytes, stream, probs_out,
                  mass_out, nullptr, 0);
}

int spec_verify_tree_timed(const void* target_logits, const void* draft_logits, const int32_t* node_tokens,
                           const int32_t* parents, const float* uniforms, const float* temperature, int B,
                           int N, int V, int topk_draft, int dtype, int32_t* out_tokens, int32_t* out_nodes,
                           int32_t* num_accepted, void* workspace, size_t* workspace_bytes,
                           hipStream_t stream, hipEvent_t* events, int n_events) {
  if (workspace && n_events != 4) return SV_ERR_ARG;
  return run_tree(target_logits, draft_logits, node_tokens, parents, uniforms, temperature, B, N, V, topk_draft,
                  dtype, out_tokens, out_nodes, num_accepted, workspace, workspace_bytes, stream, nullptr,
                  nullptr, events, n_events);
}

int spec_verify_launches(int B, int K, int V, int topk_draft, int dtype) {
  if (topk_draft >= V) topk_draft = 0;
  Plan pl;
  const int rc = make_plan(B, K, V, topk_draft, dtype, pl);
  if (rc != SV_OK) return -rc;
  return topk_draft > 0 && K > 0 ? 3 : 2;
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
    case SV_ERR_SCRATCH: return "shape needs more than the static scratch of spec_verify_noalloc (SV_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
