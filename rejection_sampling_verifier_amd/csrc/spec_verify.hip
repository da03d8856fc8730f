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
// Pipeline per call (all on the caller's stream, no host synchronisation):
//   1. stats     one work-group per (row, position, vocabulary chunk): streams
//                the chunk of target or draft logits once, writes the chunk
//                max and sum of exp2((l - max) * log2(e)/T), or for greedy
//                rows the chunk argmax; the chunk holding the draft token also
//                records that token's logit.
//   3. residual  one work-group per (row, chunk), only rows rejected with a
//                dense draft: recomputes the row's decision from the partials
//                and sums max(0, p_n - q_n) over its chunk.
//   4. sample    one work-group per row: decision, chunk selection by an
//                exclusive scan of chunk masses, block prefix sum inside the
//                selected chunk, inverse-CDF pick, output.
// Stage 2 (top-k merge) is reserved for sparse drafts.
//
// Numerical conventions.  With s = log2(e)/T and MS = fl(M*s) for a max M,
// every exponential is exp2(fma(l, s, -MS)); chunk sums computed against a
// chunk max m are rescaled by exp2(fl(m*s) - fl(M*s)), so the rounding of the
// reference products cancels between numerator and denominator.  Reductions
// combine partial results in a fixed order (no float atomics): outputs are
// bitwise reproducible.

#include <climits>
#include <cstddef>
#include <cstdint>

#include "spec_verify.h"
#include "sv_device.h"

using namespace sv;

namespace {

constexpr int NV_TILE = 8;        // 16-byte vectors per thread per chunk
constexpr int MAX_C = 2048;       // vocabulary chunks per position
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
  float4* part;              // [B, 2K+1, C] {max | argmax value, sum, argmax id, l(d)}
  float* sums;               // [B, C] residual mass per chunk
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

// ============================================================================
// Stage 1: per-chunk statistics.
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
  const bool greedy = !(T > 0.f);
  const bool is_draft = slot > a.K;
  // Greedy rows never read the draft; sparse drafts are handled by stage 2.
  if (is_draft && (greedy || a.topk > 0)) return;
  const int pos = is_draft ? slot - a.K - 1 : slot;
  const ET* row = is_draft ? draft_row<ET>(a, b, pos) : target_row<ET>(a, b, pos);
  const int lo = c * a.CS;
  const int len = min(a.CS, a.V - lo);
  const int t = threadIdx.x;

  u32x4 r[NV_TILE];
  load_tile<ET, ALIGNED, NV_TILE>(row, lo, len, r);

  __shared__ float shf[NWAVE];
  __shared__ int shi[NWAVE];
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

  float m0 = NEG_INF, m1 = NEG_INF;
#pragma unroll
  for (int j = 0; j < NV_TILE; ++j)
#pragma unroll
    for (int k = 0; k < VEC; k += 2) {
      m0 = fmaxf(m0, Tr<ET>::at(r[j], k));
      m1 = fmaxf(m1, Tr<ET>::at(r[j], k + 1));
    }
  const float m = block_max(fmaxf(m0, m1), shf);
  const float s = LOG2E / T;
  const float ms = mul_rn(m, s);
  float z0 = 0.f, z1 = 0.f, z2 = 0.f, z3 = 0.f;
  if (m != NEG_INF) {
#pragma unroll
    for (int j = 0; j < NV_TILE; ++j)
#pragma unroll
      for (int k = 0; k < VEC; k += 4) {
        z0 += exp2_fast(fmaf(Tr<ET>::at(r[j], k + 0), s, -ms));
        z1 += exp2_fast(fmaf(Tr<ET>::at(r[j], k + 1), s, -ms));
        z2 += exp2_fast(fmaf(Tr<ET>::at(r[j], k + 2), s, -ms));
        z3 += exp2_fast(fmaf(Tr<ET>::at(r[j], k + 3), s, -ms));
      }
  }
  const float z = block_sum((z0 + z1) + (z2 + z3), shf);
  if (t == 0) {
    float ld = 0.f;
    if (pos < a.K) {
      const int d = a.tok[(size_t)b * a.K + pos];
      if (d >= lo && d < lo + len) ld = Tr<ET>::load1(row + d);
    }
    *dst = make_float4(m, z, 0.f, ld);
  }
}

// ============================================================================
// Row decision, shared by stages 3 and 4 (every work-group of a row computes
// the identical result from the same partials).
// ============================================================================
struct RowShared {
  float M[MAX_SLOTS];    // position max (sampling) or argmax value (greedy)
  float Z[MAX_SLOTS];    // sum of exp2(fma(l, s, -fl(M*s)))
  int idx[MAX_SLOTS];    // argmax id (greedy)
  float p[SV_MAX_K];     // p_i(d_i)
  float q[SV_MAX_K];     // q_i(d_i)
  int tok[SV_MAX_K];
  float red_f[NWAVE];
  int red_i[NWAVE];
  int n;                 // accepted drafts
  int greedy;
  float s;               // log2(e)/T
};

template <typename ET>
__device__ void decide_row(const Args& a, int b, RowShared& rs) {
  const int K = a.K, C = a.C, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float T = a.temp[b];
  const bool greedy = !(T > 0.f);
  const float s = greedy ? 0.f : LOG2E / T;
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
        const float4 v = p[c];
        if (v.x != NEG_INF) z += v.y * exp2_fast(mul_rn(v.x, s) - MS);
      }
      z = wave_sum(z);
      if (lane == 0) { rs.M[slot] = m; rs.Z[slot] = z; rs.idx[slot] = 0; }
    }
  }
  __syncthreads();
  if (t < K) {
    const int i = t;
    const int d = a.tok[(size_t)b * K + i];
    float p = 0.f, q = 0.f;
    if (!greedy && d >= 0 && d < a.V) {
      const int cd = d / a.CS;
      const float lt = a.part[part_index(a, b, i, cd)].w;
      p = exp2_fast(fmaf(lt, s, -mul_rn(rs.M[i], s))) / rs.Z[i];
      const float lq = a.part[part_index(a, b, K + 1 + i, cd)].w;
      q = exp2_fast(fmaf(lq, s, -mul_rn(rs.M[K + 1 + i], s))) / rs.Z[K + 1 + i];
    }
    rs.p[i] = p;
    rs.q[i] = q;
    rs.tok[i] = d;
  }
  __syncthreads();
  if (t == 0) {
    // First rejection ([RheoSampling] section 4 step 1; [nalar] greedy rule).
    int n = K;
    for (int i = 0; i < K; ++i) {
      const bool acc = greedy ? (rs.tok[i] == rs.idx[i])
                              : (a.uni[(size_t)b * (K + 1) + i] * rs.q[i] < rs.p[i]);
      if (!acc) { n = i; break; }
    }
    rs.n = n;
    rs.greedy = greedy;
    rs.s = s;
  }
  __syncthreads();
}

// ============================================================================
// Stage 3: residual mass per chunk for rows rejected with a dense draft.
// ============================================================================
template <typename ET, bool ALIGNED>
__global__ __launch_bounds__(WG) void residual_kernel(Args a) {
  constexpr int VEC = Tr<ET>::VEC;
  const int c = blockIdx.x % a.C;
  const int b = blockIdx.x / a.C;
  __shared__ RowShared rs;
  decide_row<ET>(a, b, rs);
  const int K = a.K, n = rs.n;
  if (rs.greedy || n == K || a.topk > 0) return;
  const float s = rs.s;
  const float MSt = mul_rn(rs.M[n], s), rZt = 1.f / rs.Z[n];
  const float MSq = mul_rn(rs.M[K + 1 + n], s), rZq = 1.f / rs.Z[K + 1 + n];
  const int lo = c * a.CS;
  const int len = min(a.CS, a.V - lo);
  u32x4 rt[NV_TILE], rq[NV_TILE];
  load_tile<ET, ALIGNED, NV_TILE>(target_row<ET>(a, b, n), lo, len, rt);
  load_tile<ET, ALIGNED, NV_TILE>(draft_row<ET>(a, b, n), lo, len, rq);
  float w0 = 0.f, w1 = 0.f;
#pragma unroll
  for (int j = 0; j < NV_TILE; ++j)
#pragma unroll
    for (int k = 0; k < VEC; k += 2) {
      const float p0 = exp2_fast(fmaf(Tr<ET>::at(rt[j], k), s, -MSt)) * rZt;
      const float q0 = exp2_fast(fmaf(Tr<ET>::at(rq[j], k), s, -MSq)) * rZq;
      const float p1 = exp2_fast(fmaf(Tr<ET>::at(rt[j], k + 1), s, -MSt)) * rZt;
      const float q1 = exp2_fast(fmaf(Tr<ET>::at(rq[j], k + 1), s, -MSq)) * rZq;
      w0 += fmaxf(0.f, p0 - q0);
      w1 += fmaxf(0.f, p1 - q1);
    }
  const float w = block_sum(w0 + w1, rs.red_f);
  if (threadIdx.x == 0) a.sums[(size_t)b * a.C + c] = w;
}

// ============================================================================
// Stage 4: final draw and output, one work-group per row.
// ============================================================================
template <typename ET, bool ALIGNED>
__global__ __launch_bounds__(WG) void sample_kernel(Args a) {
  constexpr int VEC = Tr<ET>::VEC;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  __shared__ RowShared rs;
  __shared__ float csum[MAX_C];
  __shared__ int sh_chunk, sh_mode, sh_first, sh_last;
  __shared__ float sh_S, sh_tloc;
  decide_row<ET>(a, b, rs);
  const int K = a.K, C = a.C, n = rs.n;
  int32_t* out = a.out + (size_t)b * (K + 1);

  if (a.probs && t < K) {
    a.probs[((size_t)b * K + t) * 2 + 0] = rs.greedy ? 0.f : rs.p[t];
    a.probs[((size_t)b * K + t) * 2 + 1] = rs.greedy ? 0.f : rs.q[t];
  }
  if (rs.greedy) {
    // The target's argmax replaces the first mismatch or fills the bonus slot.
    for (int i = t; i <= K; i += WG) out[i] = i < n ? rs.tok[i] : (i == n ? rs.idx[n] : -1);
    if (t == 0) {
      a.nacc[b] = n;
      if (a.mass) a.mass[b] = 0.f;
    }
    return;
  }

  const float s = rs.s;
  const bool reject = n < K;
  const float MSt = mul_rn(rs.M[n], s), rZt = 1.f / rs.Z[n];
  // Chunk masses of the target row n from the statistics partials.
  auto target_chunk_mass = [&](int c) {
    const float4 v = a.part[part_index(a, b, n, c)];
    return v.x == NEG_INF ? 0.f : v.y * exp2_fast(mul_rn(v.x, s) - MSt) * rZt;
  };
  for (int c = t; c < C; c += WG) csum[c] = reject ? a.sums[(size_t)b * C + c] : target_chunk_mass(c);
  __syncthreads();
  if (t == 0) {
    float S = 0.f;
    for (int c = 0; c < C; ++c) { S += csum[c]; csum[c] = S; }
    sh_mode = reject ? 0 : 1;     // 0: residual max(0, p_n - q_n); 1: p_n
    sh_S = S;
  }
  __syncthreads();
  if (reject && sh_S == 0.f) {
    // A zero residual (reachable only through rounding) falls back to p_n.
    for (int c = t; c < C; c += WG) csum[c] = target_chunk_mass(c);
    __syncthreads();
    if (t == 0) {
      float S = 0.f;
      for (int c = 0; c < C; ++c) { S += csum[c]; csum[c] = S; }
      sh_mode = 1;
      sh_S = S;
    }
    __syncthreads();
  }
  if (t == 0) {
    const float S = sh_S;
    const float tv = a.uni[(size_t)b * (K + 1) + K] * S;
    int cs = -1;
    for (int c = 0; c < C; ++c)
      if (csum[c] > tv) { cs = c; break; }
    float tl;
    if (cs >= 0) {
      tl = tv - (cs ? csum[cs - 1] : 0.f);
    } else {
      // t reached the total only through rounding: take the last positive
      // weight, i.e. the last chunk with mass and its last positive id.
      cs = 0;
      for (int c = C - 1; c >= 0; --c)
        if (csum[c] > (c ? csum[c - 1] : 0.f)) { cs = c; break; }
      tl = __builtin_inff();
    }
    sh_chunk = cs;
    sh_tloc = tl;
    sh_first = INT_MAX;
    sh_last = -1;
  }
  __syncthreads();

  const int cs = sh_chunk, mode = sh_mode;
  const float tl = sh_tloc;
  const int lo = cs * a.CS;
  const int len = min(a.CS, a.V - lo);
  u32x4 rt[NV_TILE], rq[NV_TILE];
  load_tile<ET, ALIGNED, NV_TILE>(target_row<ET>(a, b, n), lo, len, rt);
  float MSq = 0.f, rZq = 0.f;
  if (mode == 0) {
    load_tile<ET, ALIGNED, NV_TILE>(draft_row<ET>(a, b, n), lo, len, rq);
    MSq = mul_rn(rs.M[K + 1 + n], s);
    rZq = 1.f / rs.Z[K + 1 + n];
  }
  float carry = 0.f;
  int last_pos = -1;
#pragma unroll
  for (int j = 0; j < NV_TILE; ++j) {
    float w[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      const float p = exp2_fast(fmaf(Tr<ET>::at(rt[j], k), s, -MSt)) * rZt;
      float wk = p;
      if (mode == 0) {
        const float q = exp2_fast(fmaf(Tr<ET>::at(rq[j], k), s, -MSq)) * rZq;
        wk = fmaxf(0.f, p - q);
      }
      w[k] = wk;
    }
    float local = 0.f;
#pragma unroll
    for (int k = 0; k < VEC; ++k) local += w[k];
    float excl, total;
    block_scan(local, rs.red_f, excl, total);
    float cum = carry + excl;
    const int base = lo + (j * WG + t) * VEC;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      cum += w[k];
      if (w[k] > 0.f && base + k < lo + len) last_pos = base + k;
      if (cum > tl && base + k < lo + len) { atomicMin(&sh_first, base + k); break; }
    }
    __syncthreads();
    if (sh_first != INT_MAX) break;
    carry += total;
  }
  if (last_pos >= 0) atomicMax(&sh_last, last_pos);
  __syncthreads();
  if (t == 0) {
    int x = sh_first;
    if (x == INT_MAX) x = sh_last >= 0 ? sh_last : lo;
    sh_first = x;
  }
  __syncthreads();
  const int x = sh_first;
  for (int i = t; i <= K; i += WG) out[i] = i < n ? rs.tok[i] : (i == n ? x : -1);
  if (t == 0) {
    a.nacc[b] = n;
    if (a.mass) a.mass[b] = sh_S;
  }
}

// ============================================================================
// Host side.
// ============================================================================
struct Plan {
  int C = 0, CS = 0;
  size_t off_part = 0, off_sums = 0, total = 0;
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
  size_t off = 0;
  pl.off_part = off;
  off = align256(off + sizeof(float4) * (size_t)B * (2 * K + 1) * C);
  pl.off_sums = off;
  off = align256(off + sizeof(float) * (size_t)B * C);
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
  if (a.K > 0) {
    hipLaunchKernelGGL((residual_kernel<ET, AL>), dim3(a.B * pl.C), blk, 0, st, a);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
  }
  if (ev && hipEventRecord(ev[3], st) != hipSuccess) return SV_ERR_HIP;
  hipLaunchKernelGGL((sample_kernel<ET, AL>), dim3(a.B), blk, 0, st, a);
  if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
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
  a.part = reinterpret_cast<float4*>(base + pl.off_part);
  a.sums = reinterpret_cast<float*>(base + pl.off_sums);
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
