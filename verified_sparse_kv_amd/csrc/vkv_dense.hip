// Exact decode attention over a whole cache (eq. 1 of "Verify Before You
// Fetch", section 3): the Dense baselines of its section 5, kept here to
// restate that comparison on this hardware. Dense (resident) reads the cache
// from device memory; Dense (offload) reads all of it from pinned host memory
// at every step, by GPU loads over the host link (zero-copy), with nothing
// staged in device memory.
//
//   dd_part   grid (parts, KV heads, requests): each workgroup streams its
//             share of one KV head's rows, 16 lanes per row (each lane 16
//             bytes of the K row and the same 16 bytes of the V row, so the
//             logit's 16-lane sum reaches every lane that needs it), four
//             rows per lane group in flight, and keeps for each of the KV
//             head's query heads a running softmax (shift, sum of weights,
//             weighted sum of V); the sixteen lane groups merge in LDS into
//             the workgroup's partial.
//   dd_merge  grid (query heads, requests): the log-sum-exp merge of the
//             partials into o and log D, in a fixed order (float64 sums).

#include <math.h>

#include "vkv_common.h"
#include "vkv_internal.h"

namespace vkv {
namespace {

constexpr float kDenseScale = 0.08838834764831845f;  // 1/sqrt(128)

struct DenseParams {
  const uint16_t *q;
  const uint16_t *kv;   // [B][G][n][2][d], device or host-mapped
  float *out, *log_d;
  float *pm, *pd, *po;  // partials [row][P], [row][P], [row][P][d]
  int B, Hq, G, n, P;
};

// Rows per lane group with loads in flight (fewer with eight query heads,
// whose per-head registers double).
template <int GRP>
constexpr int dense_batch() { return GRP >= 8 ? 2 : 4; }
constexpr int kDenseLanes = 16;                   // lanes per row
constexpr int kDenseGroups = kBlock / kDenseLanes;  // rows at a time

template <int GRP>
__global__ __launch_bounds__(kBlock) void dd_part(DenseParams p) {
  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  // a lane group of 16 lanes takes one row at a time: lane u holds
  // dimensions 8u .. 8u + 7 of its K row and of its V row
  const int lg = threadIdx.x / kDenseLanes;
  const int unit = threadIdx.x % kDenseLanes;
  const int dim0 = unit * 8;
  const int lo = (int)(((long long)p.n * part) / p.P);
  const int hi = (int)(((long long)p.n * (part + 1)) / p.P);
  // the query heads' values at this lane's 8 dimensions, pre-scaled
  float qv[GRP][8];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const uint4 u = *reinterpret_cast<const uint4 *>(
        p.q + ((size_t)b * p.Hq + g * GRP + h) * kHeadDim + dim0);
    float f[8];
    unpack8(u, f);
#pragma unroll
    for (int k = 0; k < 8; ++k) qv[h][k] = f[k] * kDenseScale;
  }
  const uint4 *rows = reinterpret_cast<const uint4 *>(
      p.kv + ((size_t)b * p.G + g) * (size_t)p.n * 2 * kHeadDim);
  float m[GRP], d[GRP], o[GRP][8];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    m[h] = -INFINITY;
    d[h] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[h][k] = 0.0f;
  }
  constexpr int NB = dense_batch<GRP>();
  constexpr int STEP = kDenseGroups * NB;
  uint4 ck[NB], cv[NB];
  auto load = [&](int base, uint4 (&dk)[NB], uint4 (&dv)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = base + j * kDenseGroups + lg;
      const bool in = i < hi;
      dk[j] = in ? rows[(size_t)i * 32 + unit] : make_uint4(0u, 0u, 0u, 0u);
      dv[j] = in ? rows[(size_t)i * 32 + 16 + unit] : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  if (lo < hi) load(lo, ck, cv);
  for (int base = lo; base < hi; base += STEP) {
    uint4 nk[NB], nv[NB];
    if (base + STEP < hi) load(base + STEP, nk, nv);  // next batch in flight
    float lgt[GRP][NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      float f[8];
      unpack8(ck[j], f);
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        float sdot = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) sdot += qv[h][k] * f[k];
        lgt[h][j] = group_sum<kDenseLanes>(sdot);  // the row's logit, all 16 lanes
      }
    }
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      float mx = m[h];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (base + j * kDenseGroups + lg < hi) mx = fmaxf(mx, lgt[h][j]);
      // (a lane group with no row yet keeps m = -inf: scale 1, not NaN)
      const float sc = mx == -INFINITY ? 1.0f : expf(m[h] - mx);
      float ds = 0.0f;
      float acc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = o[h][k] * sc;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (!(base + j * kDenseGroups + lg < hi)) continue;
        const float wgt = expf(lgt[h][j] - mx);
        ds += wgt;
        float f[8];
        unpack8(cv[j], f);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += wgt * f[k];
      }
      m[h] = mx;
      d[h] = d[h] * sc + ds;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[h][k] = acc[k];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      ck[j] = nk[j];
      cv[j] = nv[j];
    }
  }
  // merge the lane groups (fixed order) into the workgroup's partial
  __shared__ float s_m[kDenseGroups][GRP], s_d[kDenseGroups][GRP];
  __shared__ float s_o[kDenseGroups][GRP][kHeadDim];
  if (unit == 0) {
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      s_m[lg][h] = m[h];
      s_d[lg][h] = d[h];
    }
  }
#pragma unroll
  for (int h = 0; h < GRP; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) s_o[lg][h][dim0 + k] = o[h][k];
  __syncthreads();
  for (int t = threadIdx.x; t < GRP * kHeadDim; t += kBlock) {
    const int h = t / kHeadDim, k = t % kHeadDim;
    float mx = -INFINITY;
    for (int j = 0; j < kDenseGroups; ++j)
      if (s_d[j][h] > 0.0f) mx = fmaxf(mx, s_m[j][h]);
    float dd = 0.0f, oo = 0.0f;
    for (int j = 0; j < kDenseGroups; ++j) {
      if (!(s_d[j][h] > 0.0f)) continue;  // a lane group that saw no row
      const float f = expf(s_m[j][h] - mx);
      dd += s_d[j][h] * f;
      oo += s_o[j][h][k] * f;
    }
    const size_t row = (size_t)b * p.Hq + g * GRP + h;
    p.po[(row * p.P + part) * kHeadDim + k] = oo;
    if (k == 0) {
      p.pm[row * p.P + part] = mx;
      p.pd[row * p.P + part] = dd;
    }
  }
}

__global__ __launch_bounds__(kHeadDim) void dd_merge(DenseParams p) {
  const int h = blockIdx.x, b = blockIdx.y, k = threadIdx.x;
  const size_t row = (size_t)b * p.Hq + h;
  const float *pm = p.pm + row * p.P;
  const float *pd = p.pd + row * p.P;
  // the partials' shifts and sums in LDS (P <= 64), one load per thread
  __shared__ float s_m[64], s_d[64], s_f[64];
  __shared__ float s_mx;
  if (k < p.P) {
    s_m[k] = pm[k];
    s_d[k] = pd[k];
  }
  __syncthreads();
  if (k == 0) {
    float mx = -INFINITY;
    for (int j = 0; j < p.P; ++j)
      if (s_d[j] > 0.0f) mx = fmaxf(mx, s_m[j]);
    s_mx = mx;
  }
  __syncthreads();
  const float mx = s_mx;
  if (k < p.P) s_f[k] = s_d[k] > 0.0f ? expf(s_m[k] - mx) : 0.0f;
  __syncthreads();
  // fixed order over the partials; their weighted V sums are independent
  // loads, all in flight at once
  double dd = 0.0, oo = 0.0;
  for (int j = 0; j < p.P; ++j) {
    const double f = (double)s_f[j];
    dd += (double)s_d[j] * f;
    oo += (double)p.po[(row * p.P + j) * kHeadDim + k] * f;
  }
  p.out[row * kHeadDim + k] = (float)(oo / dd);
  if (k == 0) p.log_d[row] = (float)(log(dd) + (double)mx);
}

}  // namespace

DenseLayout dense_layout(const vkv_dense_args &a) {
  DenseLayout L{};
  const long long groups = (long long)a.batch * a.n_kv_heads;
  // about 1024 workgroups (enough host loads in flight for the link), at
  // least 256 rows each, at most 64 parts per KV head
  long long P = (1024 + groups - 1) / groups;
  P = std::min<long long>(P, 64);  // (the merge holds 64 partials in LDS)
  P = std::min<long long>(P, (a.n_tokens + 255) / 256);
  L.parts = (int)std::max<long long>(P, 1);
  const size_t rows = (size_t)a.batch * a.n_q_heads;
  Carve c;
  L.pm = c.take<float>(rows * L.parts);
  L.pd = c.take<float>(rows * L.parts);
  L.po = c.take<float>(rows * L.parts * (size_t)kHeadDim);
  L.total = (c.off + 255) & ~size_t(255);
  return L;
}

hipError_t launch_dense(const vkv_dense_args &a, const DenseLayout &L,
                        const uint16_t *kv_dev, hipStream_t s) {
  DenseParams p{};
  p.q = a.q;
  p.kv = kv_dev;
  p.out = a.out;
  p.log_d = a.log_d;
  p.pm = at<float>(a.workspace, L.pm);
  p.pd = at<float>(a.workspace, L.pd);
  p.po = at<float>(a.workspace, L.po);
  p.B = a.batch;
  p.Hq = a.n_q_heads;
  p.G = a.n_kv_heads;
  p.n = a.n_tokens;
  p.P = L.parts;
  const dim3 grid((unsigned)p.P, (unsigned)p.G, (unsigned)p.B);
  switch (a.n_q_heads / a.n_kv_heads) {
    case 1: dd_part<1><<<grid, dim3(kBlock), 0, s>>>(p); break;
    case 2: dd_part<2><<<grid, dim3(kBlock), 0, s>>>(p); break;
    case 4: dd_part<4><<<grid, dim3(kBlock), 0, s>>>(p); break;
    case 8: dd_part<8><<<grid, dim3(kBlock), 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  dd_merge<<<dim3((unsigned)p.Hq, (unsigned)p.B), dim3(kHeadDim), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace vkv
