// The pages' 2-bit key sketch ("Verify Before You Fetch", Appendix A.1,
// and section 5.1, "2-bit sketch implementation"), built from prefill keys.
//
// Per slice (one layer or request, one KV head):
//  sk_energy  partial sums of k_c^2 per channel over blocks of tokens
//             (float64, fixed order inside a block);
//  sk_pick    pair energies E_j = sum k_j^2 + sum k_{j+64}^2 from the
//             partials in block order, the 16 largest pairs (ties: lower j),
//             and the 32 kept channels in increasing index;
//  sk_quant   per 128-token group: each kept channel's minimum and maximum,
//             zero = fp16(min), scale = fp16((max - min) / 3) (saturated at
//             the largest finite fp16), and every token's 2-bit codes
//             clamp(rint((k - zero) / scale), 0, 3), packed two bits per
//             kept channel into one 64-bit word.
// The three kernels read the keys twice (energies, then quantisation); the
// build runs once per prefill.

#include "vkv_common.h"
#include "vkv_internal.h"

namespace vkv {

constexpr int kSkEnergyTok = 4096;  // tokens per energy workgroup

namespace {

constexpr int kSkPairs = 16;
constexpr int kSkChan = 2 * kSkPairs;
constexpr int kSkGroup = 128;
constexpr int kSkRowWords = kHeadDim / 2 + 1;  // LDS row: 64 words + 1 pad

__global__ __launch_bounds__(kBlock) void sk_energy(const vkv_sketch2_args a,
                                                    double *part) {
  const int blk = blockIdx.x, sl = blockIdx.y;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int t0 = blk * kSkEnergyTok, t1 = min(t0 + kSkEnergyTok, a.n_tokens);
  const uint16_t *k = a.k + (size_t)sl * a.slice_stride;
  // lane l holds channels 2l and 2l + 1; eight rows in flight per wave
  double e0 = 0.0, e1 = 0.0;
  constexpr int U = 8;
  for (int t = t0 + wave * U; t < t1; t += kBlock / kWave * U) {
    uint32_t w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tt = min(t + u, t1 - 1);
      w[u] = reinterpret_cast<const uint32_t *>(k + (size_t)tt * a.key_stride)[lane];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u >= t1) continue;
      const double x0 = (double)bf16_lo(w[u]), x1 = (double)bf16_hi(w[u]);
      e0 += x0 * x0;
      e1 += x1 * x1;
    }
  }
  __shared__ double s_e[kBlock / kWave][kHeadDim];
  s_e[wave][2 * lane] = e0;
  s_e[wave][2 * lane + 1] = e1;
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w) s += s_e[w][threadIdx.x];
    part[((size_t)sl * gridDim.x + blk) * kHeadDim + threadIdx.x] = s;
  }
}

__global__ __launch_bounds__(kWave) void sk_pick(const vkv_sketch2_args a,
                                                 const double *part, int nblk) {
  const int sl = blockIdx.x, j = threadIdx.x;  // lane j: pair (j, j + 64)
  double ea = 0.0, eb = 0.0;
  for (int b = 0; b < nblk; ++b) {
    const double *pp = part + ((size_t)sl * nblk + b) * kHeadDim;
    ea += pp[j];
    eb += pp[j + kHeadDim / 2];
  }
  const double e = ea + eb;
  // rank: pairs with more energy, or as much at a lower index
  int rank = 0;
  for (int o = 0; o < kWave; ++o) {
    const double eo = __shfl(e, o, kWave);
    rank += (eo > e || (eo == e && o < j)) ? 1 : 0;
  }
  const bool kept = rank < kSkPairs;
  const unsigned long long m = __ballot(kept);
  if (kept) {
    const int slot = __popcll(m & ((1ull << j) - 1ull));
    a.chan[(size_t)sl * kSkChan + slot] = j;
    a.chan[(size_t)sl * kSkChan + kSkPairs + slot] = j + kHeadDim / 2;
  }
}

__device__ __forceinline__ float fp16_sat(float x) {
  x = fminf(fmaxf(x, -65504.0f), 65504.0f);
  return (float)(_Float16)x;
}

// One workgroup of 128 threads per 128-token group.
__global__ __launch_bounds__(kSkGroup) void sk_quant(const vkv_sketch2_args a) {
  const int grp = blockIdx.x, sl = blockIdx.y;
  const int t = threadIdx.x;
  const int t0 = grp * kSkGroup, m = min(kSkGroup, a.n_tokens - t0);
  __shared__ uint32_t s_row[kSkGroup][kSkRowWords];
  __shared__ int s_ch[kSkChan];
  __shared__ float s_mn[4][kSkChan], s_mx[4][kSkChan];
  __shared__ float s_z[kSkChan], s_s[kSkChan];
  if (t < kSkChan) s_ch[t] = a.chan[(size_t)sl * kSkChan + t];
  // the group's key rows into LDS (16-byte pieces, coalesced per row)
  const uint16_t *k = a.k + (size_t)sl * a.slice_stride;
  for (int i = t; i < kSkGroup * 16; i += kSkGroup) {
    const int row = i / 16, piece = i % 16;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < m)
      v = reinterpret_cast<const uint4 *>(k + (size_t)(t0 + row) * a.key_stride)[piece];
    s_row[row][4 * piece] = v.x;
    s_row[row][4 * piece + 1] = v.y;
    s_row[row][4 * piece + 2] = v.z;
    s_row[row][4 * piece + 3] = v.w;
  }
  __syncthreads();
  auto val = [&](int row, int ch) {
    const uint32_t w = s_row[row][ch >> 1];
    return (ch & 1) ? bf16_hi(w) : bf16_lo(w);
  };
  // channel c = t % 32 over rows t / 32, t / 32 + 4, ...: min and max
  {
    const int c = t % kSkChan, q = t / kSkChan;
    const int ch = s_ch[c];
    float mn = INFINITY, mx = -INFINITY;
    for (int row = q; row < m; row += 4) {
      const float v = val(row, ch);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    s_mn[q][c] = mn;
    s_mx[q][c] = mx;
  }
  __syncthreads();
  if (t < kSkChan) {
    const float mn = fminf(fminf(s_mn[0][t], s_mn[1][t]), fminf(s_mn[2][t], s_mn[3][t]));
    const float mx = fmaxf(fmaxf(s_mx[0][t], s_mx[1][t]), fmaxf(s_mx[2][t], s_mx[3][t]));
    const float z = fp16_sat(mn);
    const float s = fp16_sat((mx - mn) / 3.0f);
    s_z[t] = z;
    s_s[t] = s;
    const int os = a.out_stride > 0 ? a.out_stride : a.n_tokens;
    const size_t zs = ((size_t)sl * ((os + kSkGroup - 1) / kSkGroup) + grp) * 2 * kSkChan;
    a.zs[zs + t] = __builtin_bit_cast(uint16_t, (_Float16)z);
    a.zs[zs + kSkChan + t] = __builtin_bit_cast(uint16_t, (_Float16)s);
  }
  __syncthreads();
  if (t < m) {
    unsigned long long word = 0ull;
#pragma unroll 8
    for (int c = 0; c < kSkChan; ++c) {
      const float s = s_s[c];
      const float x = (val(t, s_ch[c]) - s_z[c]) / s;
      const float cf = s > 0.0f ? fminf(fmaxf(rintf(x), 0.0f), 3.0f) : 0.0f;
      word |= (unsigned long long)(uint32_t)cf << (2 * c);
    }
    a.codes[(size_t)sl * (a.out_stride > 0 ? a.out_stride : a.n_tokens) + t0 + t] = word;
  }
}

}  // namespace

Sketch2Layout sketch2_layout(const vkv_sketch2_args &a) {
  Sketch2Layout L{};
  L.nblk = (a.n_tokens + kSkEnergyTok - 1) / kSkEnergyTok;
  Carve c;
  L.part = c.take<double>((size_t)a.n_slices * L.nblk * kHeadDim);
  L.total = (c.off + 255) & ~size_t(255);
  return L;
}

hipError_t launch_sketch2(const vkv_sketch2_args &a, const Sketch2Layout &L,
                          hipStream_t s) {
  double *part = at<double>(a.workspace, L.part);
  hipLaunchKernelGGL(sk_energy, dim3((unsigned)L.nblk, (unsigned)a.n_slices),
                     dim3(kBlock), 0, s, a, part);
  hipLaunchKernelGGL(sk_pick, dim3((unsigned)a.n_slices), dim3(kWave), 0, s, a,
                     (const double *)part, L.nblk);
  const int ng = (a.n_tokens + kSkGroup - 1) / kSkGroup;
  hipLaunchKernelGGL(sk_quant, dim3((unsigned)ng, (unsigned)a.n_slices),
                     dim3(kSkGroup), 0, s, a);
  return hipGetLastError();
}

}  // namespace vkv
