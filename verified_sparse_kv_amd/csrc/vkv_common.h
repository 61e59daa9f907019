// Device helpers shared by the VerKV kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vkv {

constexpr int kHeadDim = 128;   // head dimension handled by every kernel
constexpr int kBlock = 256;     // threads per workgroup (4 waves of 64)
constexpr int kWave = 64;

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
// Eight bf16 values held in one 16-byte vector -> eight floats.
__device__ __forceinline__ void unpack8(const uint4 u, float f[8]) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
  f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

// ---------------------------------------------------------------- shuffles
template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, kWave);
}

// Lane exchange within rows of 16 lanes by DPP (no LDS): CTRL is a DPP
// control (quad_perm, row_half_mirror, row_mirror).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W lanes (W in {1, 2, 4, 8, 16}); every lane of
// the group receives the same total: pairs, then pairs of pairs (quad
// permutes), then the two quads of each half-row (half mirror), then the
// two halves of the row (mirror) -- each step adds two equal partial sums
// in either order, so all lanes agree bit for bit.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16, "group");
  if constexpr (W >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (W >= 16) v += dpp_f<0x140>(v); // row_mirror
  return v;
}

// Block-wide reductions with a fixed combination order (deterministic).
// `scratch` must hold kBlock/kWave entries of T.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    T o = shfl_xor(v, m);
    v = o > v ? o : v;
  }
  return v;
}
template <typename T>
__device__ __forceinline__ T block_sum(T v, T *scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) scratch[w] = v;
  __syncthreads();
  T s = scratch[0];
#pragma unroll
  for (int i = 1; i < kBlock / kWave; ++i) s += scratch[i];
  return s;
}
template <typename T>
__device__ __forceinline__ T block_max(T v, T *scratch) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) scratch[w] = v;
  __syncthreads();
  T s = scratch[0];
#pragma unroll
  for (int i = 1; i < kBlock / kWave; ++i) s = scratch[i] > s ? scratch[i] : s;
  return s;
}

// Exclusive prefix sum over the block (thread order); returns the total
// through *total. `scratch` holds kBlock/kWave + 1 entries.
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T *scratch, T *total) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  T incl = v;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    T o = __shfl_up(incl, m, kWave);
    if (l >= m) incl += o;
  }
  __syncthreads();
  if (l == kWave - 1) scratch[w] = incl;
  __syncthreads();
  T base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kBlock / kWave; ++i) {
    if (i < w) base += scratch[i];
    tot += scratch[i];
  }
  *total = tot;
  return base + incl - v;
}

// ---------------------------------------------------------------- Philox
// Philox4x32-10 (Salmon et al., SC'11): 10 rounds of the 4x32 bijection with
// multipliers M0, M1 and Weyl key increments W0, W1. Returns the first of
// the four output words, which is the only one the sampler uses.
__device__ __forceinline__ uint32_t philox4x32_10_x0(uint32_t c0, uint32_t c1,
                                                     uint32_t c2, uint32_t c3,
                                                     uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(M0, c0), lo0 = M0 * c0;
    const uint32_t hi1 = __umulhi(M1, c2), lo1 = M1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += W0; k1 += W1;
  }
  return c0;
}

}  // namespace vkv
