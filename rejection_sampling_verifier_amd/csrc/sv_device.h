// Device helpers for the speculative-sampling verifier kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>

namespace sv {

constexpr int WG = 256;            // threads per work-group: 4 wave64
constexpr int NWAVE = WG / 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_inff();

// Native 16-byte vector (a clang ext_vector_type, so the load builtins accept it).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- cross-work-group publication ------------------------------------------
// Values that another work-group of the same launch reads are written with
// agent-scope relaxed atomic stores (write-through, coherent across XCDs) and
// read with agent-scope atomic loads.  A work-group that publishes waits for
// its stores to complete (vmcnt(0)) before its counter increment, which
// orders them without writing back the whole L2 as a general release fence
// would.
__device__ __forceinline__ void pub_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float pub_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void pub_store4(float4* p, float4 v) {
  float* f = reinterpret_cast<float*>(p);
  pub_store(f + 0, v.x); pub_store(f + 1, v.y); pub_store(f + 2, v.z); pub_store(f + 3, v.w);
}
__device__ __forceinline__ float4 pub_load4(const float4* p) {
  const float* f = reinterpret_cast<const float*>(p);
  return make_float4(pub_load(f + 0), pub_load(f + 1), pub_load(f + 2), pub_load(f + 3));
}
// Wait until every vector memory operation of this wave has completed.
__device__ __forceinline__ void wait_vmem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt unconstrained
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- element storage traits ------------------------------------------------
// Logits arrive as bf16 (raw 16-bit patterns) or float32; a 16-byte vector
// holds 8 or 4 of them.  bf16 widens to float32 exactly by a 16-bit shift.
template <typename ET> struct Tr;

template <> struct Tr<uint16_t> {
  static constexpr int VEC = 8;
  static constexpr uint32_t NEG_INF_WORD = 0xFF80FF80u;  // two bf16 -inf
  __device__ __forceinline__ static float at(const u32x4& v, int k) {
    const uint32_t w = v[k >> 1];
    return (k & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  }
  __device__ __forceinline__ static float load1(const uint16_t* p) {
    return __uint_as_float(uint32_t(*p) << 16);
  }
  __device__ __forceinline__ static void set(u32x4& v, int k, const uint16_t* p) {
    const uint32_t h = *p;
    const uint32_t w = v[k >> 1];
    v[k >> 1] = (k & 1) ? ((w & 0x0000FFFFu) | (h << 16)) : ((w & 0xFFFF0000u) | h);
  }
};

template <> struct Tr<float> {
  static constexpr int VEC = 4;
  static constexpr uint32_t NEG_INF_WORD = 0xFF800000u;
  __device__ __forceinline__ static float at(const u32x4& v, int k) { return __uint_as_float(v[k]); }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void set(u32x4& v, int k, const float* p) { v[k] = __float_as_uint(*p); }
};

// ---- register tile ----------------------------------------------------------
// A work-group holds up to WG * NV * VEC consecutive logits of one
// (row, position) in registers.  Thread t owns vector j at element offset
// (j * WG + t) * VEC of the chunk, so each load instruction of the wave covers
// 64 consecutive 16-byte vectors (1 KiB).  Elements past the chunk end read
// as -inf.  ALIGNED requires row + lo to be 16-byte aligned.  Logits read
// once use nontemporal loads (NT); rows read again soon (a tree node's
// residual passes) keep the cache.
template <typename ET, bool ALIGNED, int NV, bool NT = true>
__device__ __forceinline__ void load_tile(const ET* __restrict__ row, int lo, int len, u32x4 (&r)[NV]) {
  constexpr int VEC = Tr<ET>::VEC;
  const int t = threadIdx.x;
  const uint32_t f = Tr<ET>::NEG_INF_WORD;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = (j * WG + t) * VEC;
    if (ALIGNED) {
      // Aligned rows hold a multiple of VEC logits and chunks start on VEC
      // boundaries, so a vector is either wholly inside the chunk or past it.
      if (e < len) {
        const u32x4* src = reinterpret_cast<const u32x4*>(row + lo + e);
        r[j] = NT ? __builtin_nontemporal_load(src) : *src;
      }
      else r[j] = u32x4{f, f, f, f};
    } else {
      u32x4 v = {f, f, f, f};
#pragma unroll
      for (int k = 0; k < VEC; ++k)
        if (e + k < len) Tr<ET>::set(v, k, row + lo + e + k);
      r[j] = v;
    }
  }
}

// ---- wave64 / block reductions ----------------------------------------------
// DPP all-reduce: quad swaps, half-row and row mirrors, then the row
// broadcasts of lane 15 and lane 31; lane 63 ends with the result.  The
// combination order is fixed, so float sums are reproducible.
namespace dpp {
constexpr int QUAD_1032 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int QUAD_2301 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int ROW_HALF_MIRROR = 0x141;
constexpr int ROW_MIRROR = 0x140;
constexpr int ROW_BCAST15 = 0x142;
constexpr int ROW_BCAST31 = 0x143;
constexpr int ROW_SHR1 = 0x111;
constexpr int ROW_SHR2 = 0x112;
constexpr int ROW_SHR4 = 0x114;
constexpr int ROW_SHR8 = 0x118;
}  // namespace dpp

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float identity, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), CTRL,
                                                    ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int identity, int v) {
  return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ float lane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<dpp::QUAD_1032>(NEG_INF, v));
  v = fmaxf(v, dpp_f<dpp::QUAD_2301>(NEG_INF, v));
  v = fmaxf(v, dpp_f<dpp::ROW_HALF_MIRROR>(NEG_INF, v));
  v = fmaxf(v, dpp_f<dpp::ROW_MIRROR>(NEG_INF, v));
  v = fmaxf(v, dpp_f<dpp::ROW_BCAST15, 0xA>(NEG_INF, v));
  v = fmaxf(v, dpp_f<dpp::ROW_BCAST31, 0xC>(NEG_INF, v));
  return lane63(v);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<dpp::QUAD_1032>(0.f, v);
  v += dpp_f<dpp::QUAD_2301>(0.f, v);
  v += dpp_f<dpp::ROW_HALF_MIRROR>(0.f, v);
  v += dpp_f<dpp::ROW_MIRROR>(0.f, v);
  v += dpp_f<dpp::ROW_BCAST15, 0xA>(0.f, v);
  v += dpp_f<dpp::ROW_BCAST31, 0xC>(0.f, v);
  return lane63(v);
}
// Inclusive scan over the 64 lanes in lane order: shifts by 1, 2, 4, 8 inside
// each row of 16 lanes, then lane 15 of a row is added to the next row and
// lane 31 to the upper half.  Exact for integer-valued floats below 2^24.
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += dpp_f<dpp::ROW_SHR1>(0.f, v);
  v += dpp_f<dpp::ROW_SHR2>(0.f, v);
  v += dpp_f<dpp::ROW_SHR4>(0.f, v);
  v += dpp_f<dpp::ROW_SHR8>(0.f, v);
  v += dpp_f<dpp::ROW_BCAST15, 0xA>(0.f, v);
  v += dpp_f<dpp::ROW_BCAST31, 0xC>(0.f, v);
  return v;
}
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  v &= (uint32_t)dpp_i<dpp::QUAD_1032>(-1, (int)v);
  v &= (uint32_t)dpp_i<dpp::QUAD_2301>(-1, (int)v);
  v &= (uint32_t)dpp_i<dpp::ROW_HALF_MIRROR>(-1, (int)v);
  v &= (uint32_t)dpp_i<dpp::ROW_MIRROR>(-1, (int)v);
  v &= (uint32_t)dpp_i<dpp::ROW_BCAST15, 0xA>(-1, (int)v);
  v &= (uint32_t)dpp_i<dpp::ROW_BCAST31, 0xC>(-1, (int)v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= (uint32_t)dpp_i<dpp::QUAD_1032>(0, (int)v);
  v |= (uint32_t)dpp_i<dpp::QUAD_2301>(0, (int)v);
  v |= (uint32_t)dpp_i<dpp::ROW_HALF_MIRROR>(0, (int)v);
  v |= (uint32_t)dpp_i<dpp::ROW_MIRROR>(0, (int)v);
  v |= (uint32_t)dpp_i<dpp::ROW_BCAST15, 0xA>(0, (int)v);
  v |= (uint32_t)dpp_i<dpp::ROW_BCAST31, 0xC>(0, (int)v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// (value, index) argmax: larger value wins, equal values go to the lower index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float v2 = dpp_f<CTRL, ROW_MASK>(NEG_INF, v);
  const int i2 = dpp_i<CTRL, ROW_MASK>(INT_MAX, i);
  argmax_merge(v, i, v2, i2);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<dpp::QUAD_1032>(v, i);
  argmax_step<dpp::QUAD_2301>(v, i);
  argmax_step<dpp::ROW_HALF_MIRROR>(v, i);
  argmax_step<dpp::ROW_MIRROR>(v, i);
  argmax_step<dpp::ROW_BCAST15, 0xA>(v, i);
  argmax_step<dpp::ROW_BCAST31, 0xC>(v, i);
  v = lane63(v);
  i = __builtin_amdgcn_readlane(i, 63);
}

// Reductions over groups of G = 16, 32 or 64 lanes of a wave, G a compile-time
// constant.  They take the steps of wave_sum / wave_max / wave_argmax that
// stay inside the group, so a group whose lanes past the data hold the
// identity gives bit for bit what those reductions give over the wave.  The
// group's result is in its last lane.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<dpp::QUAD_1032>(0.f, v);
  v += dpp_f<dpp::QUAD_2301>(0.f, v);
  v += dpp_f<dpp::ROW_HALF_MIRROR>(0.f, v);
  v += dpp_f<dpp::ROW_MIRROR>(0.f, v);
  if (G >= 32) v += dpp_f<dpp::ROW_BCAST15, 0xA>(0.f, v);
  if (G >= 64) v += dpp_f<dpp::ROW_BCAST31, 0xC>(0.f, v);
  return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_f<dpp::QUAD_1032>(NEG_INF, v));
  v = fmaxf(v, dpp_f<dpp::QUAD_2301>(NEG_INF, v));
  v = fmaxf(v, dpp_f<dpp::ROW_HALF_MIRROR>(NEG_INF, v));
  v = fmaxf(v, dpp_f<dpp::ROW_MIRROR>(NEG_INF, v));
  if (G >= 32) v = fmaxf(v, dpp_f<dpp::ROW_BCAST15, 0xA>(NEG_INF, v));
  if (G >= 64) v = fmaxf(v, dpp_f<dpp::ROW_BCAST31, 0xC>(NEG_INF, v));
  return v;
}
template <int G>
__device__ __forceinline__ void group_argmax(float& v, int& i) {
  argmax_step<dpp::QUAD_1032>(v, i);
  argmax_step<dpp::QUAD_2301>(v, i);
  argmax_step<dpp::ROW_HALF_MIRROR>(v, i);
  argmax_step<dpp::ROW_MIRROR>(v, i);
  if (G >= 32) argmax_step<dpp::ROW_BCAST15, 0xA>(v, i);
  if (G >= 64) argmax_step<dpp::ROW_BCAST31, 0xC>(v, i);
}
// Broadcast of the group's last lane to the whole group.
template <int G>
__device__ __forceinline__ float group_last(float v) {
  const int lane = threadIdx.x & 63;
  return __shfl(v, (lane & ~(G - 1)) + G - 1, 64);
}

// max(a, b, c) issued directly.  The compiler's fmaxf first quiets possible
// signaling NaNs in operands it cannot prove canonical (such as logits
// widened from loaded bits); here only a NaN logit could be one, and a NaN
// logit has no defined result.  Callers must not pass bit patterns that are
// NaN for other reasons (e.g. a packed pair of bf16 values).
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Block reductions combine the four wave results in a fixed order, so every
// result is bitwise reproducible.  `sh` needs NWAVE floats (ints).
__device__ __forceinline__ float block_max(float v, float* sh) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) r = fmaxf(r, sh[w]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) r += sh[w];
  __syncthreads();
  return r;
}
__device__ __forceinline__ void block_argmax(float& v, int& i, float* shv, int* shi) {
  wave_argmax(v, i);
  if ((threadIdx.x & 63) == 0) { shv[threadIdx.x >> 6] = v; shi[threadIdx.x >> 6] = i; }
  __syncthreads();
  v = shv[0]; i = shi[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) argmax_merge(v, i, shv[w], shi[w]);
  __syncthreads();
}
// Scan over the block in thread order: returns the inclusive prefix, sets the
// exclusive prefix (computed from the same partial sums) and the block total.
__device__ __forceinline__ float block_scan(float v, float* sh, float& excl, float& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float u = __shfl_up(inc, o, 64);
    if (lane >= o) inc += u;
  }
  float prev = __shfl_up(inc, 1, 64);
  if (lane == 0) prev = 0.f;
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  float base = 0.f, tot = 0.f;
#pragma unroll
  for (int k = 0; k < NWAVE; ++k) {
    if (k < w) base += sh[k];
    tot += sh[k];
  }
  __syncthreads();
  total = tot;
  excl = base + prev;
  return base + inc;
}

// Scan of integer counts over the block in thread order (DPP inside waves,
// one barrier pair across them): returns the exclusive prefix, sets the total.
// `sh` needs NWAVE ints.
__device__ __forceinline__ int block_count_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = (int)wave_incl_scan((float)v);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < NWAVE; ++k) {
    if (k < w) base += sh[k];
    tot += sh[k];
  }
  __syncthreads();
  total = tot;
  return base + inc - v;
}

}  // namespace sv

namespace sv {

// ---- ordering keys for the sparse-draft (top-k) selection -------------------
// order_key maps a float to an unsigned key with the same order (-0 and +0
// map to the same key, as they compare equal).  A candidate is the 64-bit
// composite (order_key(value) << 32) | ~id: larger composites are better,
// i.e. a larger value, or an equal value at a lower id.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ uint64_t composite(float v, int id) {
  return ((uint64_t)order_key(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ int composite_id(uint64_t c) { return (int)(0xFFFFFFFFu - (uint32_t)c); }
__device__ __forceinline__ float composite_value(uint64_t c) { return key_value((uint32_t)(c >> 32)); }

// Bitonic sort of n (a power of two) LDS entries into descending order, by
// the whole block.
template <typename T>
__device__ void bitonic_sort_desc(T* x, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += WG) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const T u = x[lo], v = x[hi];
        if ((u < v) == desc) { x[lo] = v; x[hi] = u; }
      }
      __syncthreads();
    }
  }
}

}  // namespace sv
