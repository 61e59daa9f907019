// Decode-time maintenance ("Verify Before You Fetch", section 3 and
// Appendix A.3.1): each generated token joins H of every (request, KV head)
// -- its K/V row written to the host cache and appended to the resident
// rows, its position to the resident list, r = 1 -- with its sketch rows.

#include "vkv_common.h"
#include "vkv_internal.h"

namespace vkv {
namespace {

// One workgroup of 128 threads (one per dimension) per (request, KV head).
__global__ __launch_bounds__(kHeadDim) void mk_append(const vkv_append_args a,
                                                      uint16_t *host_kv) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int bg = b * a.n_kv_heads + g, t = threadIdx.x;
  const size_t ns = (size_t)a.ctx_stride;
  __shared__ float s_k[kHeadDim];
  __shared__ int s_cnt, s_ok;
  const uint16_t kt = a.k_new[(size_t)bg * kHeadDim + t];
  const uint16_t vt = a.v_new[(size_t)bg * kHeadDim + t];
  s_k[t] = __uint_as_float((uint32_t)kt << 16);
  uint16_t *hrow = host_kv + ((size_t)bg * ns + a.pos) * 2 * kHeadDim;
  hrow[t] = kt;
  hrow[kHeadDim + t] = vt;
  if (t == 0) {
    const int cnt = a.resident_count[bg];
    int bits = 0;
    if (cnt < 0 || cnt >= a.cap) bits |= VKV_STATUS_RESIDENT_OVERFLOW;
    else if (cnt > 0 && a.resident_idx[(size_t)bg * a.cap + cnt - 1] >= a.pos)
      bits |= VKV_STATUS_BAD_RESIDENT;
    s_cnt = cnt;
    s_ok = bits == 0;
    if (bits) atomicOr(a.status, (uint32_t)bits);
    a.r[(size_t)bg * ns + a.pos] = 1.0f;
  }
  __syncthreads();
  if (s_ok) {
    uint16_t *rrow = a.resident_kv + ((size_t)bg * a.cap + s_cnt) * 2 * kHeadDim;
    rrow[t] = kt;
    rrow[kHeadDim + t] = vt;
  }
  // the projected sketch row: fp32 sums over increasing dimension (no
  // fused multiply-add), rounded to bf16 (nearest even)
  if (a.sketch && t < a.sketch_dim) {
    const float *P = a.proj + (size_t)g * kHeadDim * a.sketch_dim;
    float acc = 0.0f;
    for (int e = 0; e < kHeadDim; ++e) {
      const float prod = P[(size_t)e * a.sketch_dim + t] * s_k[e];
      acc = acc + prod;
    }
    const uint32_t u = __float_as_uint(acc);
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    a.sketch[((size_t)bg * ns + a.pos) * a.sketch_dim + t] = (uint16_t)rounded;
  }
  // the 2-bit sketch: code word 0; a group that starts here gets zero
  // points and scales 0
  if (a.sk2_codes) {
    if (t == 0) a.sk2_codes[(size_t)bg * ns + a.pos] = 0ull;
    if (a.pos % 128 == 0 && t < 64) {
      const size_t ng = (ns + 127) / 128;
      a.sk2_zs[((size_t)bg * ng + a.pos / 128) * 64 + t] = 0u;
    }
  }
  __syncthreads();
  if (t == 0 && s_ok) {
    a.resident_idx[(size_t)bg * a.cap + s_cnt] = a.pos;
    a.resident_count[bg] = s_cnt + 1;
  }
}

}  // namespace

hipError_t launch_append(const vkv_append_args &a, uint16_t *host_kv_dev,
                         hipStream_t s) {
  hipLaunchKernelGGL(mk_append, dim3((unsigned)a.n_kv_heads, (unsigned)a.batch),
                     dim3(kHeadDim), 0, s, a, host_kv_dev);
  return hipGetLastError();
}

}  // namespace vkv
