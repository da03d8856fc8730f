// Device helpers for the speculative-sampling verifier kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int WG = 256;            // threads per work-group: 4 wave64
constexpr int NWAVE = WG / 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_inff();

// Native 16-byte vector (a clang ext_vector_type, so the load builtins accept it).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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
// as -inf.  ALIGNED requires row + lo to be 16-byte aligned.
template <typename ET, bool ALIGNED, int NV>
__device__ __forceinline__ void load_tile(const ET* __restrict__ row, int lo, int len, u32x4 (&r)[NV]) {
  constexpr int VEC = Tr<ET>::VEC;
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = (j * WG + t) * VEC;
    if (ALIGNED && e + VEC <= len) {
      r[j] = *reinterpret_cast<const u32x4*>(row + lo + e);
    } else {
      const uint32_t f = Tr<ET>::NEG_INF_WORD;
      u32x4 v = {f, f, f, f};
#pragma unroll
      for (int k = 0; k < VEC; ++k)
        if (e + k < len) Tr<ET>::set(v, k, row + lo + e + k);
      r[j] = v;
    }
  }
}

// ---- wave64 / block reductions ----------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// (value, index) argmax: larger value wins, equal values go to the lower index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(v, o, 64);
    const int i2 = __shfl_xor(i, o, 64);
    argmax_merge(v, i, v2, i2);
  }
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

}  // namespace sv
