// KVFetch decode step on gfx950 ("Verify Before You Fetch", Algorithm 2,
// section 4.2; Definition 2, Lemma 1, eqs. 5-10, Theorem 2).
//
// A "group" is one (request b, KV head g) with its GRP = Hq/G query heads
// ("rows"). Token passes split the n positions into chunks of `chunk` tokens,
// one workgroup per (chunk, g, b); every row-level decision is taken by the
// last workgroup of the group to finish a pass ("last block done"), so a
// launch never waits on another workgroup.
//
//  dk_scan      sketch logits s_i = <P_g^T q, sk_i>/sqrt(d) for every token and
//               the GRP heads at once (one sketch row serves all of them).
//  dk_resident  exact logits l_j = <q, k_j>/sqrt(d) on the resident rows,
//               residency bitmap, common shift m = max(max_R l, max_L s).
//  dk_beta x4   Definition 2 fixed point beta = sum_L w~(1 - lambda(beta)):
//               h(beta) is piecewise linear with breakpoints w~(1-r) and
//               w~(1-r)/r; four radix levels over the fp32 bit patterns of the
//               breakpoints (8+8+8+7 bits) bracket the root between adjacent
//               floats, where h is linear and the root is solved exactly.
//               Level 0 also forms D~ = sum_H w + sum_L w~.
//  dk_cert      lambda_i, beta(L), V(L), top-2 of b_i -> eps^(L) (eq. 7).
//  dk_select x3 radix select driven by the stopping rule (eq. 10): keys are
//               (gain bits, inverted position) so descending key order is
//               L_g; per-bin counts and fixed-point sums of beta_i and v_i let
//               the last block find the bin where eps^(L_g[k:]) first drops
//               below eps without sorting L. Small bins are collected.
//  dk_finish    sorts the collected bin in LDS and walks it to the exact k*.
//  dk_mark      fetch set of the KV head = union over its heads of
//               {key >= threshold} minus the resident rows (bitmap + counts).
//  dk_gather    ascending fetch list; rows copied from pinned host memory by
//               GPU loads (zero-copy) into device staging.
//  dk_attn      weights w on H u F_h, lambda w / r on S \ F_h, exact logits of
//               fetched rows, partial softmax sums merged by log-sum-exp.
//
// All per-token recomputations (weights, lambda, certificate terms, gains)
// go through the same inline functions and the library is built with
// floating-point contraction off, so every pass sees identical values.

#include <algorithm>

#include "vkv_common.h"
#include "vkv_internal.h"

namespace vkv {
namespace {

constexpr int kCand = 2048;      // candidates the finisher sorts in LDS
constexpr int kBetaEdges = 257;  // difference arrays per radix level
constexpr int kSelBins = 256;
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)

enum { MODE_HIST = 0, MODE_COLLECT = 1, MODE_COLLECTED = 2, MODE_DONE = 3 };

struct RowState {
  float m;                // common shift of the planning and resident logits
  int32_t bdone;          // beta* known
  uint32_t bpre;          // bit pattern of the beta bracket's lower edge
  int32_t fetch;          // eps^(L) >= eps
  double dnorm;           // D~ * exp(-m)
  double beta;            // beta*
  double betaL, VL;       // beta(L), V(L) (float64 sums of fp32 terms)
  double s_full;          // sqrt((a b)^2 + 2 V l)
  double eps0;            // eps^(L)
  float b1, b2;           // largest and second largest b_i (with multiplicity)
  int32_t amax;           // position of the unique argmax of b_i, else -1
  int32_t eb, ev;         // fixed-point exponents for beta_i and v_i
  int32_t mode;           // selection state (MODE_*)
  int32_t level;          // next radix digit (MODE_HIST)
  int32_t shift;          // tokens match when (key >> shift) == pre
  uint32_t bin_cnt;       // tokens in the crossing bin
  uint32_t ncand;         // candidates collected
  uint32_t cntA;          // tokens fetched above the current bracket
  uint32_t bB;            // max b_i (float bits) below the current bracket
  int32_t kstar;
  unsigned long long pre;
  unsigned long long bL_fx, VL_fx;   // fixed-point totals over L
  unsigned long long betaA, VA;      // fixed-point sums fetched above
  unsigned long long T;              // member iff (key >> T_shift) >= T
  int32_t T_shift;
  float eps1;             // eps^(L') after fetching
};

struct GroupState {
  uint32_t arrive[8];
};

struct CertPart {
  double beta, var;
  float b1, b2;
  int32_t p1, pad;
};

struct SelBin {
  uint32_t cnt, bmax;
  unsigned long long bsum, vsum;
};

struct Cand {
  unsigned long long key, bfx, vfx;
  uint32_t rb, pad;
};

struct AttnPart {
  float m, d;
  float o[kHeadDim];
  float pad[2];
};

enum { ARR_RES = 0, ARR_BETA = 1, ARR_CERT = 2, ARR_SEL = 3, ARR_ATTN = 4 };

struct DParams {
  const uint16_t *q, *rkv, *sketch, *host_kv;
  const int32_t *ridx, *rcount;
  const float *proj, *r;
  float *out, *d_hat, *log_shift, *eps_hat0, *eps_hat;
  int32_t *k_star, *fidx, *fcount;
  unsigned long long *host_bytes;
  double *row_stats;
  uint32_t *status;
  float *shat, *ell;
  uint32_t *resbits, *fbits;
  float *pmax;
  uint32_t *hpart;
  RowState *rows;
  GroupState *groups;
  double *bbins;
  double2 *dpart;
  CertPart *cpart;
  SelBin *sbins;
  Cand *cand;
  uint32_t *fcnt;
  AttnPart *apart;
  uint16_t *staging;
  int B, Hq, G, n, cap, fetch_cap, nch, ncr, ncf, nwords, chunk;
  float eps;
  double l_delta, a_delta;
  int est, weights;
};

// ------------------------------------------------------------ shared math
struct Terms {
  float wt, lam, bi, vi, rb;
};

// Planning weight w~ = exp(s - m), lambda (Definition 2) and the three
// certificate terms of Lemma 1 for one token of L.
__device__ __forceinline__ Terms token_terms(float s, float r, float m,
                                             float beta, int est) {
  Terms t;
  t.wt = expf(s - m);
  float lam = 1.0f;
  if (est == VKV_EST_CLIP && t.wt > 0.0f) {
    const float x = beta * r / (t.wt * (1.0f - r));
    lam = fminf(1.0f, fmaxf(r, x));
  }
  t.lam = lam;
  t.bi = t.wt * (1.0f - lam);
  const float lw = lam * t.wt;
  t.vi = lw * lw * (1.0f - r) / r;
  t.rb = lw * fmaxf(r, 1.0f - r) / r;
  return t;
}

// eq. 7 in float64.
__device__ __forceinline__ double eps_of(double beta, double var, double b,
                                         double dn, double a, double l) {
  const double ab = a * b;
  return (beta + ab + sqrt(ab * ab + 2.0 * var * l)) / dn;
}

// Gain g_i * D~ (eq. 9, cancellation-free form), rounded to float for the key.
__device__ __forceinline__ float token_gain(const Terms &t, int pos,
                                            const RowState &rs, double a,
                                            double l) {
  const double b1 = rs.b1;
  const double bp = (pos == rs.amax) ? (double)rs.b2 : b1;
  const double vi = t.vi;
  const double vp = fmax(rs.VL - vi, 0.0);
  const double sp = sqrt(a * a * bp * bp + 2.0 * vp * l);
  const double num = a * a * (b1 - bp) * (b1 + bp) + 2.0 * vi * l;
  const double den = rs.s_full + sp;
  const double frac = den > 0.0 ? num / den : 0.0;
  return (float)((double)t.bi + a * (b1 - bp) + frac);
}

// Descending key order = gain descending, then position ascending.
__device__ __forceinline__ unsigned long long make_key(float gain, int pos) {
  return ((unsigned long long)__float_as_uint(gain) << 24) |
         (unsigned long long)(0xFFFFFFu - (uint32_t)pos);
}

__device__ __forceinline__ unsigned long long to_fx(float x, int e) {
  return (unsigned long long)__double2ull_rn(ldexp((double)x, e));
}

__device__ __forceinline__ bool is_member(unsigned long long key,
                                          const RowState &rs) {
  return (key >> rs.T_shift) >= rs.T;
}

__device__ __forceinline__ int sel_off(int d) { return d < 6 ? 47 - 8 * d : 0; }
__device__ __forceinline__ int sel_width(int d) { return d < 6 ? 8 : 7; }

__device__ __forceinline__ int row_of(const DParams &p, int b, int g, int h,
                                      int grp) {
  return b * p.Hq + g * grp + h;
}

// Rows [lo, hi) of `total` handled by part `idx` of `parts` (even split).
__device__ __forceinline__ void split_range(int total, int parts, int idx,
                                            int &lo, int &hi) {
  lo = (int)(((long long)total * idx) / parts);
  hi = (int)(((long long)total * (idx + 1)) / parts);
}

// Inclusive prefix sum over the lanes of a wave (lane order).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v, int lane) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const T o = __shfl_up(v, m, kWave);
    if (lane >= m) v += o;
  }
  return v;
}

// Inclusive prefix maximum over the lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t v, int lane) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const uint32_t o = __shfl_up(v, m, kWave);
    if (lane >= m) v = max(v, o);
  }
  return v;
}

// ------------------------------------------------------------ dk_scan
template <int GRP, int SD>
__global__ __launch_bounds__(kBlock) void dk_scan(DParams p) {
  constexpr int LPT = SD / 8;           // lanes per token (16 bytes each)
  constexpr int TPI = kBlock / LPT;     // tokens per block iteration
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.G + g;
  const int lane = threadIdx.x % kWave;
  __shared__ float s_qp[GRP][SD];
  __shared__ float s_red[kBlock / kWave];
  __shared__ uint32_t s_ured[kBlock / kWave];

  // step-start initialisation of this group's state (no other block of
  // this launch touches it)
  if (c == 0) {
    if (threadIdx.x < 8) p.groups[bg].arrive[threadIdx.x] = 0u;
    for (int h = 0; h < GRP; ++h) {
      const int row = row_of(p, b, g, h, GRP);
      double *bb = p.bbins + (size_t)row * 3 * kBetaEdges;
      for (int i = threadIdx.x; i < 3 * kBetaEdges; i += kBlock) bb[i] = 0.0;
      SelBin *sb = p.sbins + (size_t)row * kSelBins;
      for (int i = threadIdx.x; i < kSelBins; i += kBlock)
        sb[i] = SelBin{0u, 0u, 0ull, 0ull};
      if (threadIdx.x == 0) {
        RowState z{};
        z.amax = -1;
        z.T = ~0ull;
        z.mode = MODE_DONE;
        p.rows[row] = z;
      }
    }
    if (bg == 0 && threadIdx.x == 0) {
      *p.status = 0u;
      *p.host_bytes = 0ull;
    }
  }
  // clear this chunk's bitmap words
  {
    const int w0 = c * p.chunk / 32, nw = p.chunk / 32;
    for (int w = threadIdx.x; w < nw; w += kBlock) {
      if (w0 + w < p.nwords) {
        p.resbits[(size_t)bg * p.nwords + w0 + w] = 0u;
        p.fbits[(size_t)bg * p.nwords + w0 + w] = 0u;
      }
    }
  }
  // projected, pre-scaled queries: stage q and P_g in LDS, then one output
  // per thread
  {
    __shared__ float s_proj[kHeadDim * SD];
    __shared__ float s_q[GRP][kHeadDim];
    const float4 *P4 =
        reinterpret_cast<const float4 *>(p.proj + (size_t)g * kHeadDim * SD);
    for (int i = threadIdx.x; i < kHeadDim * SD / 4; i += kBlock)
      reinterpret_cast<float4 *>(s_proj)[i] = P4[i];
    for (int i = threadIdx.x; i < GRP * kHeadDim; i += kBlock) {
      const int h = i / kHeadDim, e = i % kHeadDim;
      s_q[h][e] = __uint_as_float(
          (uint32_t)p.q[(size_t)row_of(p, b, g, h, GRP) * kHeadDim + e] << 16);
    }
    __syncthreads();
    if (threadIdx.x < GRP * SD) {
      const int h = threadIdx.x / SD, j = threadIdx.x % SD;
      float acc = 0.0f;
      for (int e = 0; e < kHeadDim; ++e)
        acc = __builtin_fmaf(s_proj[e * SD + j], s_q[h][e], acc);
      s_qp[h][j] = acc * kInvSqrtD;
    }
    __syncthreads();
  }
  const int u = lane % LPT;
  float qv[GRP][8];
#pragma unroll
  for (int h = 0; h < GRP; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) qv[h][k] = s_qp[h][u * 8 + k];

  float mx[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) mx[h] = -INFINITY;
  uint32_t n_h = 0;
  bool bad = false;
  const uint16_t *sk = p.sketch + (size_t)bg * p.n * SD;
  const float *rr = p.r + (size_t)bg * p.n;
  const int base = c * p.chunk;
  const int lim = min(base + p.chunk, p.n);
  constexpr int UNR = 4;  // sketch rows in flight per lane
  for (int i0 = base; i0 < lim; i0 += TPI * UNR) {
    uint4 raw[UNR];
    float rv[UNR];
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int i = i0 + k * TPI + threadIdx.x / LPT;
      if (i < lim) {
        raw[k] = *reinterpret_cast<const uint4 *>(sk + (size_t)i * SD + u * 8);
        rv[k] = rr[i];
      }
    }
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int i = i0 + k * TPI + threadIdx.x / LPT;
      if (i >= lim) continue;
      float f[8];
      unpack8(raw[k], f);
      float dot[GRP];
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(qv[h][e], f[e], acc);
        dot[h] = group_sum<LPT>(acc);
      }
      const float ri = rv[k];
      if (!(ri > 0.0f && ri <= 1.0f)) bad = true;
      const bool in_l = ri < 1.0f;
      if (u == 0 && !in_l) ++n_h;
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        if (h % LPT == u)
          p.shat[(size_t)row_of(p, b, g, h, GRP) * p.n + i] = dot[h];
        if (in_l) mx[h] = fmaxf(mx[h], dot[h]);
      }
    }
  }
  if (bad) atomicOr(p.status, VKV_STATUS_BAD_R);
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const float v = block_max<float>(mx[h], s_red);
    if (threadIdx.x == 0)
      p.pmax[(size_t)row_of(p, b, g, h, GRP) * (p.nch + p.ncr) + c] = v;
  }
  const uint32_t th = block_sum<uint32_t>(n_h, s_ured);
  if (threadIdx.x == 0) p.hpart[(size_t)bg * (p.nch + p.ncr) + c] = th;
}

// Same outputs with exact keys read from the host cache (perfect sketch).
template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_scan_exact(DParams p) {
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.G + g;
  const int lane = threadIdx.x % kWave;
  __shared__ float s_red[kBlock / kWave];
  __shared__ uint32_t s_ured[kBlock / kWave];
  if (c == 0) {
    if (threadIdx.x < 8) p.groups[bg].arrive[threadIdx.x] = 0u;
    for (int h = 0; h < GRP; ++h) {
      const int row = row_of(p, b, g, h, GRP);
      double *bb = p.bbins + (size_t)row * 3 * kBetaEdges;
      for (int i = threadIdx.x; i < 3 * kBetaEdges; i += kBlock) bb[i] = 0.0;
      SelBin *sb = p.sbins + (size_t)row * kSelBins;
      for (int i = threadIdx.x; i < kSelBins; i += kBlock)
        sb[i] = SelBin{0u, 0u, 0ull, 0ull};
      if (threadIdx.x == 0) {
        RowState z{};
        z.amax = -1;
        z.T = ~0ull;
        z.mode = MODE_DONE;
        p.rows[row] = z;
      }
    }
    if (bg == 0 && threadIdx.x == 0) {
      *p.status = 0u;
      *p.host_bytes = 0ull;
    }
  }
  {
    const int w0 = c * p.chunk / 32, nw = p.chunk / 32;
    for (int w = threadIdx.x; w < nw; w += kBlock) {
      if (w0 + w < p.nwords) {
        p.resbits[(size_t)bg * p.nwords + w0 + w] = 0u;
        p.fbits[(size_t)bg * p.nwords + w0 + w] = 0u;
      }
    }
  }
  const int u = lane % 16;
  float qv[GRP][8];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(
        p.q + (size_t)row_of(p, b, g, h, GRP) * kHeadDim + u * 8);
    unpack8(raw, qv[h]);
  }
  float mx[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) mx[h] = -INFINITY;
  uint32_t n_h = 0;
  bool bad = false;
  const float *rr = p.r + (size_t)bg * p.n;
  const int base = c * p.chunk;
  const int lim = min(base + p.chunk, p.n);
  for (int i0 = base; i0 < lim; i0 += kBlock / 16) {
    const int i = i0 + threadIdx.x / 16;
    if (i < lim) {
      const float ri = rr[i];
      if (!(ri > 0.0f && ri <= 1.0f)) bad = true;
      const bool in_l = ri < 1.0f;
      if (u == 0 && !in_l) ++n_h;
      float dot[GRP];
      if (in_l) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(
            p.host_kv + ((size_t)bg * p.n + i) * 2 * kHeadDim + u * 8);
        float f[8];
        unpack8(raw, f);
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) acc = __builtin_fmaf(qv[h][k], f[k], acc);
          dot[h] = group_sum<16>(acc) * kInvSqrtD;
          mx[h] = fmaxf(mx[h], dot[h]);
        }
      } else {
#pragma unroll
        for (int h = 0; h < GRP; ++h) dot[h] = 0.0f;
      }
#pragma unroll
      for (int h = 0; h < GRP; ++h)
        if (u == h) p.shat[(size_t)row_of(p, b, g, h, GRP) * p.n + i] = dot[h];
    }
  }
  if (bad) atomicOr(p.status, VKV_STATUS_BAD_R);
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const float v = block_max<float>(mx[h], s_red);
    if (threadIdx.x == 0)
      p.pmax[(size_t)row_of(p, b, g, h, GRP) * (p.nch + p.ncr) + c] = v;
  }
  const uint32_t th = block_sum<uint32_t>(n_h, s_ured);
  if (threadIdx.x == 0) p.hpart[(size_t)bg * (p.nch + p.ncr) + c] = th;
}

// ------------------------------------------------------------ dk_resident
// The group's resident rows are split evenly over gridDim.x workgroups.
template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_resident(DParams p) {
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.G + g;
  const int lane = threadIdx.x % kWave;
  const int u = lane % 16;
  __shared__ float s_red[kBlock / kWave];
  __shared__ uint32_t s_ured[kBlock / kWave];
  float qv[GRP][8];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(
        p.q + (size_t)row_of(p, b, g, h, GRP) * kHeadDim + u * 8);
    unpack8(raw, qv[h]);
  }
  int cnt = p.rcount[bg];
  bool bad = cnt < 0 || cnt > p.cap;
  cnt = max(0, min(cnt, p.cap));
  const int32_t *ridx = p.ridx + (size_t)bg * p.cap;
  const float *rr = p.r + (size_t)bg * p.n;
  float mx[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) mx[h] = -INFINITY;
  uint32_t n_h = 0;
  int lo, hi;
  split_range(cnt, gridDim.x, c, lo, hi);
  for (int j0 = lo; j0 < hi; j0 += kBlock / 16) {
    const int j = j0 + threadIdx.x / 16;
    if (j < hi) {
      const int pos = ridx[j];
      const bool ok = pos >= 0 && pos < p.n && (j == 0 || ridx[j - 1] < pos);
      const uint4 raw = *reinterpret_cast<const uint4 *>(
          p.rkv + ((size_t)bg * p.cap + j) * 2 * kHeadDim + u * 8);
      float f[8];
      unpack8(raw, f);
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc = __builtin_fmaf(qv[h][k], f[k], acc);
        const float dot = group_sum<16>(acc) * kInvSqrtD;
        if (u == h) p.ell[(size_t)row_of(p, b, g, h, GRP) * p.cap + j] = dot;
        mx[h] = fmaxf(mx[h], dot);
      }
      if (u == 0) {
        if (ok) {
          atomicOr(p.resbits + (size_t)bg * p.nwords + pos / 32,
                   1u << (pos % 32));
          if (rr[pos] >= 1.0f) ++n_h;
        } else {
          bad = true;
        }
      }
    }
  }
  if (bad) atomicOr(p.status, VKV_STATUS_BAD_RESIDENT);
  const int np = p.nch + p.ncr;
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const float v = block_max<float>(mx[h], s_red);
    if (threadIdx.x == 0)
      p.pmax[(size_t)row_of(p, b, g, h, GRP) * np + p.nch + c] = v;
  }
  const uint32_t th = block_sum<uint32_t>(n_h, s_ured);
  if (threadIdx.x == 0) p.hpart[(size_t)bg * np + p.nch + c] = th;
  if (!last_block_arrive(&p.groups[bg].arrive[ARR_RES], gridDim.x)) return;
  // shift per row (one wave per head); every token with r == 1 must be resident
  const int wave = threadIdx.x / kWave;
  for (int h = wave; h < GRP; h += kBlock / kWave) {
    const int row = row_of(p, b, g, h, GRP);
    float m = -INFINITY;
    for (int i = lane; i < np; i += kWave) m = fmaxf(m, p.pmax[(size_t)row * np + i]);
    m = wave_max(m);
    if (lane == 0) p.rows[row].m = m;
  }
  if (wave == 0) {
    uint32_t all_h = 0, res_h = 0;
    for (int i = lane; i < p.nch; i += kWave) all_h += p.hpart[(size_t)bg * np + i];
    for (int i = lane; i < p.ncr; i += kWave) res_h += p.hpart[(size_t)bg * np + p.nch + i];
    all_h = wave_sum(all_h);
    res_h = wave_sum(res_h);
    if (lane == 0 && all_h != res_h) atomicOr(p.status, VKV_STATUS_BAD_RESIDENT);
  }
}

// ------------------------------------------------------------ dk_beta
// Radix level `lev` of the beta* search (digit widths 8, 8, 8, 7 over the
// float bit pattern; level 0 digits are the exponent field).
template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_beta(DParams p, int lev) {
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.G + g;
  const int shift = lev == 0 ? 23 : (lev == 1 ? 15 : (lev == 2 ? 7 : 0));
  const int nb = lev == 3 ? 128 : 256;
  __shared__ double s_bins[GRP][3][kBetaEdges];
  __shared__ double s_dred[kBlock / kWave];
  __shared__ float s_m[GRP];
  __shared__ uint32_t s_pa[GRP];
  __shared__ int s_active[GRP];
  if (threadIdx.x < GRP) {
    const RowState &rs = p.rows[row_of(p, b, g, threadIdx.x, GRP)];
    s_m[threadIdx.x] = rs.m;
    s_pa[threadIdx.x] = rs.bpre;
    s_active[threadIdx.x] = (p.est == VKV_EST_CLIP) && !rs.bdone;
  }
  __syncthreads();
  bool any = lev == 0;
  for (int h = 0; h < GRP; ++h) any |= s_active[h] != 0;
  if (!any) return;
  for (int i = threadIdx.x; i < GRP * 3 * kBetaEdges; i += kBlock)
    (&s_bins[0][0][0])[i] = 0.0;
  __syncthreads();
  double baseC[GRP], baseW[GRP], baseR[GRP], sumL[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) baseC[h] = baseW[h] = baseR[h] = sumL[h] = 0.0;
  const float *rr = p.r + (size_t)bg * p.n;
  const int base = c * p.chunk;
  const int lim = min(base + p.chunk, p.n);
  for (int i = base + threadIdx.x; i < lim; i += kBlock) {
    const float ri = rr[i];
    if (!(ri < 1.0f)) continue;
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const int row = row_of(p, b, g, h, GRP);
      const float wt = expf(p.shat[(size_t)row * p.n + i] - s_m[h]);
      if (lev == 0) sumL[h] += (double)wt;
      if (!s_active[h] || !(wt > 0.0f)) continue;
      const float lo = wt * (1.0f - ri);
      const float hi = lo / ri;
      const float rho = ri / (1.0f - ri);
      const uint32_t pa = s_pa[h];
      const uint32_t pb = pa + ((uint32_t)nb << shift);
      const uint32_t lb = __float_as_uint(lo), hb = __float_as_uint(hi);
      const int pl = lb < pa ? -1 : (lb >= pb ? nb : (int)((lb - pa) >> shift));
      const int ph = hb < pa ? -1 : (hb >= pb ? nb : (int)((hb - pa) >> shift));
      // constant lo_i on edges [0, pl]
      if (pl >= 0) {
        baseC[h] += (double)lo;
        if (pl < nb) unsafeAtomicAdd(&s_bins[h][0][pl + 1], -(double)lo);
      }
      // linear w~ - e rho on edges [pl + 1, ph]
      if (pl + 1 <= ph) {
        if (pl + 1 == 0) {
          baseW[h] += (double)wt;
          baseR[h] += (double)rho;
        } else {
          unsafeAtomicAdd(&s_bins[h][1][pl + 1], (double)wt);
          unsafeAtomicAdd(&s_bins[h][2][pl + 1], (double)rho);
        }
        if (ph < nb) {
          unsafeAtomicAdd(&s_bins[h][1][ph + 1], -(double)wt);
          unsafeAtomicAdd(&s_bins[h][2][ph + 1], -(double)rho);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const double bc = block_sum<double>(baseC[h], s_dred);
    const double bw = block_sum<double>(baseW[h], s_dred);
    const double br = block_sum<double>(baseR[h], s_dred);
    if (threadIdx.x == 0) {
      s_bins[h][0][0] += bc;
      s_bins[h][1][0] += bw;
      s_bins[h][2][0] += br;
    }
  }
  // level 0: per-chunk parts of D~ (L from the sketch, H from resident rows)
  if (lev == 0) {
    const int cnt = max(0, min(p.rcount[bg], p.cap));
    const int32_t *ridx = p.ridx + (size_t)bg * p.cap;
    int jlo, jhi;
    split_range(cnt, gridDim.x, c, jlo, jhi);
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const int row = row_of(p, b, g, h, GRP);
      double sh = 0.0;
      for (int j = jlo + threadIdx.x; j < jhi; j += kBlock) {
        const int pos = ridx[j];
        if (pos >= 0 && pos < p.n && rr[pos] >= 1.0f)
          sh += (double)expf(p.ell[(size_t)row * p.cap + j] - s_m[h]);
      }
      const double tsh = block_sum<double>(sh, s_dred);
      const double tsl = block_sum<double>(sumL[h], s_dred);
      if (threadIdx.x == 0) p.dpart[(size_t)row * p.nch + c] = make_double2(tsl, tsh);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < GRP * 3 * kBetaEdges; i += kBlock) {
    const double v = (&s_bins[0][0][0])[i];
    if (v != 0.0) {
      const int h = i / (3 * kBetaEdges), rest = i % (3 * kBetaEdges);
      unsafeAtomicAdd(p.bbins + (size_t)row_of(p, b, g, h, GRP) * 3 * kBetaEdges +
                          rest,
                      v);
    }
  }
  if (!last_block_arrive(&p.groups[bg].arrive[ARR_BETA], gridDim.x)) return;
  // ---- last block: one wave per head scans the edges of the bracket.
  // h(e_j) = C(j) + W(j) - e_j (1 + R(j)) with C, W, R the prefix sums of the
  // difference arrays; h decreases, so the root lies after the last edge
  // with h > 0.
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  constexpr int PER = 5;  // 64 lanes x 5 >= 257 edges
  for (int h = wave; h < GRP; h += kBlock / kWave) {
    const int row = row_of(p, b, g, h, GRP);
    RowState &rs = p.rows[row];
    double *gb = p.bbins + (size_t)row * 3 * kBetaEdges;
    if (lev == 0) {
      double dl = 0.0, dh = 0.0;
      for (int i = lane; i < p.nch; i += kWave) {
        const double2 v = p.dpart[(size_t)row * p.nch + i];
        dl += v.x;
        dh += v.y;
      }
      dl = wave_sum(dl);
      dh = wave_sum(dh);
      if (lane == 0) {
        rs.dnorm = dh + dl;
        if (p.est != VKV_EST_CLIP) {
          rs.bdone = 1;
          rs.beta = 0.0;
        }
      }
    }
    if (s_active[h]) {
      const uint32_t pa = s_pa[h];
      const int nedge = lev == 0 ? 255 : nb + 1;  // level 0 stops before +inf
      double C[PER], W[PER], R[PER];
      double tc = 0.0, tw = 0.0, tr = 0.0;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int j = lane * PER + k;
        const bool in = j < nedge;
        tc += in ? gb[j] : 0.0;
        tw += in ? gb[kBetaEdges + j] : 0.0;
        tr += in ? gb[2 * kBetaEdges + j] : 0.0;
        C[k] = tc;
        W[k] = tw;
        R[k] = tr;
      }
      const double oc = wave_incl_scan(tc, lane) - tc;
      const double ow = wave_incl_scan(tw, lane) - tw;
      const double orr = wave_incl_scan(tr, lane) - tr;
      double Hv[PER];
      int best = -1;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int j = lane * PER + k;
        const double e = (double)__uint_as_float(pa + ((uint32_t)j << shift));
        Hv[k] = (oc + C[k]) + (ow + W[k]) - e * (1.0 + (orr + R[k]));
        if (j < nedge && j < nb && Hv[k] > 0.0) best = j;
      }
      int root = best;
      for (int m = 32; m >= 1; m >>= 1) root = max(root, __shfl_xor(root, m, kWave));
      // values at the root edge and the next one
      double h0 = 0.0, h1 = 0.0;
      const int r0 = max(root, 0), r1 = r0 + 1;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        if (lane * PER + k == r0) h0 = Hv[k];
        if (lane * PER + k == r1) h1 = Hv[k];
      }
      h0 = __shfl(h0, r0 / PER, kWave);
      h1 = __shfl(h1, min(r1 / PER, kWave - 1), kWave);
      if (lane == 0) {
        if (root < 0 && lev == 0) {  // no weight in L
          rs.beta = 0.0;
          rs.bdone = 1;
        } else {
          const uint32_t pj = pa + ((uint32_t)r0 << shift);
          if (lev < 3) {
            rs.bpre = pj;
          } else {
            const double e0 = (double)__uint_as_float(pj);
            const double e1 = (double)__uint_as_float(pj + 1u);
            const double d = h0 - h1;
            double bt = d > 0.0 ? e0 + h0 * (e1 - e0) / d : e0;
            bt = fmin(fmax(bt, e0), e1);
            rs.beta = bt;
            rs.bdone = 1;
          }
        }
      }
    }
    for (int i = lane; i < 3 * kBetaEdges; i += kWave) gb[i] = 0.0;
  }
}

// ------------------------------------------------------------ dk_cert
__device__ __forceinline__ void top2_merge(float &x1, int &p1, float &x2,
                                           float y1, int q1, float y2) {
  if (y1 > x1 || (y1 == x1 && q1 < p1)) {
    x2 = fmaxf(x1, y2);
    x1 = y1;
    p1 = q1;
  } else {
    x2 = fmaxf(x2, y1);
  }
}

template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_cert(DParams p) {
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.G + g;
  __shared__ double s_dred[kBlock / kWave];
  __shared__ float s_w1[kBlock / kWave], s_w2[kBlock / kWave];
  __shared__ int s_wp[kBlock / kWave];
  __shared__ float s_m[GRP], s_beta[GRP];
  if (threadIdx.x < GRP) {
    const RowState &rs = p.rows[row_of(p, b, g, threadIdx.x, GRP)];
    s_m[threadIdx.x] = rs.m;
    s_beta[threadIdx.x] = (float)rs.beta;
  }
  __syncthreads();
  double sb[GRP], sv[GRP];
  float x1[GRP], x2[GRP];
  int p1[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    sb[h] = sv[h] = 0.0;
    x1[h] = x2[h] = 0.0f;
    p1[h] = 0x7fffffff;
  }
  const float *rr = p.r + (size_t)bg * p.n;
  const int base = c * p.chunk;
  const int lim = min(base + p.chunk, p.n);
  for (int i = base + threadIdx.x; i < lim; i += kBlock) {
    const float ri = rr[i];
    if (!(ri < 1.0f)) continue;
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const int row = row_of(p, b, g, h, GRP);
      const Terms t =
          token_terms(p.shat[(size_t)row * p.n + i], ri, s_m[h], s_beta[h], p.est);
      sb[h] += (double)t.bi;
      sv[h] += (double)t.vi;
      top2_merge(x1[h], p1[h], x2[h], t.rb, i, 0.0f);
    }
  }
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const double tb = block_sum<double>(sb[h], s_dred);
    const double tv = block_sum<double>(sv[h], s_dred);
    float a1 = x1[h], a2 = x2[h];
    int q1 = p1[h];
    for (int m = 32; m >= 1; m >>= 1) {
      const float o1 = shfl_xor(a1, m), o2 = shfl_xor(a2, m);
      const int oq = shfl_xor(q1, m);
      top2_merge(a1, q1, a2, o1, oq, o2);
    }
    __syncthreads();
    if (lane == 0) {
      s_w1[wave] = a1;
      s_w2[wave] = a2;
      s_wp[wave] = q1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float y1 = s_w1[0], y2 = s_w2[0];
      int yq = s_wp[0];
      for (int w = 1; w < kBlock / kWave; ++w) top2_merge(y1, yq, y2, s_w1[w], s_wp[w], s_w2[w]);
      CertPart cp;
      cp.beta = tb;
      cp.var = tv;
      cp.b1 = y1;
      cp.b2 = y2;
      cp.p1 = yq;
      cp.pad = 0;
      p.cpart[(size_t)row_of(p, b, g, h, GRP) * p.nch + c] = cp;
    }
  }
  if (!last_block_arrive(&p.groups[bg].arrive[ARR_CERT], gridDim.x)) return;
  for (int h = wave; h < GRP; h += kBlock / kWave) {
    const int row = row_of(p, b, g, h, GRP);
    RowState &rs = p.rows[row];
    double tb = 0.0, tv = 0.0;
    float y1 = 0.0f, y2 = 0.0f;
    int yq = 0x7fffffff;
    for (int i = lane; i < p.nch; i += kWave) {
      const CertPart cp = p.cpart[(size_t)row * p.nch + i];
      tb += cp.beta;
      tv += cp.var;
      top2_merge(y1, yq, y2, cp.b1, cp.p1, cp.b2);
    }
    tb = wave_sum(tb);
    tv = wave_sum(tv);
    for (int m = 32; m >= 1; m >>= 1) {
      const float o1 = shfl_xor(y1, m), o2 = shfl_xor(y2, m);
      const int oq = shfl_xor(yq, m);
      top2_merge(y1, yq, y2, o1, oq, o2);
    }
    if (lane != 0) continue;
    const double a = p.a_delta, l = p.l_delta;
    rs.betaL = tb;
    rs.VL = tv;
    rs.b1 = y1;
    rs.b2 = y2;
    rs.amax = (y2 < y1) ? yq : -1;
    rs.s_full = sqrt(a * a * (double)y1 * (double)y1 + 2.0 * tv * l);
    const double e0 = ((double)tb + a * (double)y1 + rs.s_full) / rs.dnorm;
    rs.eps0 = e0;
    if (e0 < (double)p.eps) {
      rs.fetch = 0;
      rs.kstar = 0;
      rs.eps1 = (float)e0;
      rs.mode = MODE_DONE;
      rs.T = ~0ull;
      rs.T_shift = 0;
    } else {
      rs.fetch = 1;
      int eb = 0, ev = 0;
      if (tb > 0.0) { (void)frexp(tb, &eb); eb = 61 - eb; } else { eb = 0; }
      if (tv > 0.0) { (void)frexp(tv, &ev); ev = 61 - ev; } else { ev = 0; }
      rs.eb = eb;
      rs.ev = ev;
      rs.mode = MODE_HIST;
      rs.level = 0;
      rs.shift = 55;
      rs.pre = 0ull;
      rs.cntA = 0u;
      rs.betaA = 0ull;
      rs.VA = 0ull;
      rs.bB = 0u;
      rs.bL_fx = 0ull;
      rs.VL_fx = 0ull;
      rs.ncand = 0u;
      rs.T = ~0ull;
      rs.T_shift = 0;
    }
  }
}

// ------------------------------------------------------------ selection
// Resolve one radix level for one row with a single wave. `bins` holds the
// 2^width bins of digit `d`; updates the row state.
__device__ void sel_resolve(RowState &rs, const SelBin *bins, int d,
                            const DParams &p, int lane) {
  const int w = sel_width(d), off = sel_off(d);
  const int nbins = 1 << w;
  const int per = nbins / kWave;  // 4 or 2
  const double a = p.a_delta, l = p.l_delta;
  const double sb = ldexp(1.0, -rs.eb), sv = ldexp(1.0, -rs.ev);
  // lane-local bins x = lane * per + k
  uint32_t cnt[4];
  unsigned long long bs[4], vs[4];
  uint32_t bm[4];
  uint32_t lc = 0, lmax = 0;
  unsigned long long lb = 0, lv = 0;
  for (int k = 0; k < per; ++k) {
    const SelBin sbn = bins[lane * per + k];
    cnt[k] = sbn.cnt;
    bs[k] = sbn.bsum;
    vs[k] = sbn.vsum;
    bm[k] = sbn.bmax;
    lc += cnt[k];
    lb += bs[k];
    lv += vs[k];
    lmax = max(lmax, bm[k]);
  }
  // sums over the lanes above (higher bins) and max over the lanes below
  const uint32_t ic = wave_incl_scan<uint32_t>(lc, lane);
  const unsigned long long ib = wave_incl_scan<unsigned long long>(lb, lane);
  const unsigned long long iv = wave_incl_scan<unsigned long long>(lv, lane);
  const uint32_t ac = __shfl(ic, kWave - 1, kWave) - ic;
  const unsigned long long ab = __shfl(ib, kWave - 1, kWave) - ib;
  const unsigned long long av = __shfl(iv, kWave - 1, kWave) - iv;
  uint32_t bmax_below = __shfl_up(wave_incl_max(lmax, lane), 1, kWave);
  if (lane == 0) bmax_below = 0u;
  // evaluate eps^(tail_x) for each local bin, top to bottom
  int best = -1;
  {
    uint32_t c_ge = ac;
    unsigned long long b_ge = ab, v_ge = av;
    for (int k = per - 1; k >= 0; --k) {
      c_ge += cnt[k];
      b_ge += bs[k];
      v_ge += vs[k];
      uint32_t bt = max(rs.bB, bmax_below);
      for (int k2 = 0; k2 < k; ++k2) bt = max(bt, bm[k2]);
      const double tb = (double)(rs.bL_fx - rs.betaA - b_ge) * sb;
      const double tv = (double)(rs.VL_fx - rs.VA - v_ge) * sv;
      const double e = eps_of(tb, tv, (double)__uint_as_float(bt), rs.dnorm, a, l);
      if (e < (double)p.eps && best < 0) best = lane * per + k;
    }
  }
  int top = best;
  for (int m = 32; m >= 1; m >>= 1) top = max(top, __shfl_xor(top, m, kWave));
  if (top < 0) top = 0;  // unreachable: the bracket bottom always certifies
  if (lane == top / per) {
    const int k = top % per;
    uint32_t c_gt = ac;
    unsigned long long b_gt = ab, v_gt = av;
    for (int k2 = per - 1; k2 > k; --k2) {
      c_gt += cnt[k2];
      b_gt += bs[k2];
      v_gt += vs[k2];
    }
    uint32_t bt = max(rs.bB, bmax_below);
    for (int k2 = 0; k2 < k; ++k2) bt = max(bt, bm[k2]);
    const uint32_t cb = cnt[k];
    const unsigned long long pre2 = (rs.pre << w) | (unsigned long long)top;
    const unsigned long long fa_b = rs.betaA + b_gt + bs[k];
    const unsigned long long fa_v = rs.VA + v_gt + vs[k];
    const double e_through = eps_of((double)(rs.bL_fx - fa_b) * sb,
                                    (double)(rs.VL_fx - fa_v) * sv,
                                    (double)__uint_as_float(bt), rs.dnorm, a, l);
    if (cb == 0u) {
      rs.kstar = (int)(rs.cntA + c_gt);
      rs.T = pre2 + 1ull;
      rs.T_shift = off;
      rs.eps1 = (float)e_through;
      rs.mode = MODE_DONE;
    } else if (cb == 1u || d == 6) {
      rs.kstar = (int)(rs.cntA + c_gt + cb);
      rs.T = pre2;
      rs.T_shift = off;
      rs.eps1 = (float)e_through;
      rs.mode = MODE_DONE;
    } else {
      rs.cntA += c_gt;
      rs.betaA += b_gt;
      rs.VA += v_gt;
      rs.bB = bt;
      rs.pre = pre2;
      rs.shift = off;
      rs.bin_cnt = cb;
      if (cb <= (uint32_t)kCand) {
        rs.mode = MODE_COLLECT;
        rs.ncand = 0u;
      } else {
        rs.mode = MODE_HIST;
        rs.level = d + 1;
      }
    }
  }
}

template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_select(DParams p) {
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.G + g;
  __shared__ SelBin s_bins[GRP][kSelBins];
  __shared__ RowState s_rs[GRP];
  __shared__ unsigned long long s_ured[kBlock / kWave];
  if (threadIdx.x < GRP) s_rs[threadIdx.x] = p.rows[row_of(p, b, g, threadIdx.x, GRP)];
  __syncthreads();
  bool any = false;
  for (int h = 0; h < GRP; ++h)
    any |= s_rs[h].fetch && (s_rs[h].mode == MODE_HIST || s_rs[h].mode == MODE_COLLECT);
  if (!any) return;
  for (int i = threadIdx.x; i < GRP * kSelBins; i += kBlock)
    (&s_bins[0][0])[i] = SelBin{0u, 0u, 0ull, 0ull};
  __syncthreads();
  const double a = p.a_delta, l = p.l_delta;
  unsigned long long tb[GRP], tv[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) tb[h] = tv[h] = 0ull;
  const float *rr = p.r + (size_t)bg * p.n;
  const int base = c * p.chunk;
  const int lim = min(base + p.chunk, p.n);
  for (int i = base + threadIdx.x; i < lim; i += kBlock) {
    const float ri = rr[i];
    if (!(ri < 1.0f)) continue;
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const RowState &rs = s_rs[h];
      if (!rs.fetch) continue;
      const int mode = rs.mode;
      if (mode != MODE_HIST && mode != MODE_COLLECT) continue;
      const int row = row_of(p, b, g, h, GRP);
      const Terms t = token_terms(p.shat[(size_t)row * p.n + i], ri, rs.m,
                                  (float)rs.beta, p.est);
      const unsigned long long bfx = to_fx(t.bi, rs.eb);
      const unsigned long long vfx = to_fx(t.vi, rs.ev);
      if (mode == MODE_HIST && rs.level == 0) {
        tb[h] += bfx;
        tv[h] += vfx;
      }
      const unsigned long long key = make_key(token_gain(t, i, rs, a, l), i);
      if ((key >> rs.shift) != rs.pre) continue;
      if (mode == MODE_HIST) {
        const int d = rs.level;
        const int dig = (int)((key >> sel_off(d)) & ((1ull << sel_width(d)) - 1));
        SelBin &sb = s_bins[h][dig];
        atomicAdd(&sb.cnt, 1u);
        atomicAdd(&sb.bsum, bfx);
        atomicAdd(&sb.vsum, vfx);
        atomicMax(&sb.bmax, __float_as_uint(t.rb));
      } else {
        const uint32_t slot = atomicAdd(&p.rows[row].ncand, 1u);
        if (slot < (uint32_t)kCand) {
          Cand cd;
          cd.key = key;
          cd.bfx = bfx;
          cd.vfx = vfx;
          cd.rb = __float_as_uint(t.rb);
          cd.pad = 0u;
          p.cand[(size_t)row * kCand + slot] = cd;
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const RowState &rs = s_rs[h];
    if (!(rs.fetch && rs.mode == MODE_HIST)) continue;
    const int row = row_of(p, b, g, h, GRP);
    if (rs.level == 0) {
      const unsigned long long xb = block_sum<unsigned long long>(tb[h], s_ured);
      const unsigned long long xv = block_sum<unsigned long long>(tv[h], s_ured);
      if (threadIdx.x == 0) {
        atomicAdd(&p.rows[row].bL_fx, xb);
        atomicAdd(&p.rows[row].VL_fx, xv);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < GRP * kSelBins; i += kBlock) {
    const int h = i / kSelBins, x = i % kSelBins;
    const RowState &rs = s_rs[h];
    if (!(rs.fetch && rs.mode == MODE_HIST)) continue;
    const SelBin &sb = s_bins[h][x];
    if (sb.cnt == 0u) continue;
    SelBin *gbn = p.sbins + (size_t)row_of(p, b, g, h, GRP) * kSelBins + x;
    atomicAdd(&gbn->cnt, sb.cnt);
    atomicAdd(&gbn->bsum, sb.bsum);
    atomicAdd(&gbn->vsum, sb.vsum);
    atomicMax(&gbn->bmax, sb.bmax);
  }
  if (!last_block_arrive(&p.groups[bg].arrive[ARR_SEL], gridDim.x)) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  for (int h = wave; h < GRP; h += kBlock / kWave) {
    const int row = row_of(p, b, g, h, GRP);
    RowState &rs = p.rows[row];
    if (!rs.fetch) continue;
    if (rs.mode == MODE_COLLECT) {
      if (lane == 0) rs.mode = MODE_COLLECTED;
      continue;
    }
    if (rs.mode != MODE_HIST) continue;
    SelBin *gbn = p.sbins + (size_t)row * kSelBins;
    sel_resolve(rs, gbn, rs.level, p, lane);
    for (int x = lane; x < kSelBins; x += kWave) gbn[x] = SelBin{0u, 0u, 0ull, 0ull};
  }
}

// One workgroup per row: finish the selection (fallback radix levels over the
// whole row if a bin stayed large, then sort the collected bin and walk it).
template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_finish(DParams p) {
  const int h = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.G + g;
  const int row = row_of(p, b, g, h, GRP);
  RowState &grs = p.rows[row];
  __shared__ RowState s_rs;
  __shared__ SelBin s_bins[kSelBins];
  __shared__ unsigned long long s_key[kCand];
  __shared__ uint32_t s_idx[kCand];
  __shared__ uint32_t s_cnt;
  __shared__ unsigned long long s_scan[kBlock / kWave + 1];
  __shared__ uint32_t s_uscan[kBlock / kWave + 1];
  __shared__ int s_best;
  if (threadIdx.x == 0) s_rs = grs;
  __syncthreads();
  if (!s_rs.fetch || s_rs.mode == MODE_DONE) return;
  const double a = p.a_delta, l = p.l_delta;
  const float *rr = p.r + (size_t)bg * p.n;
  const float *sh = p.shat + (size_t)row * p.n;
  // fallback: remaining radix levels over the whole row
  while (s_rs.mode == MODE_HIST) {
    for (int x = threadIdx.x; x < kSelBins; x += kBlock) s_bins[x] = SelBin{0u, 0u, 0ull, 0ull};
    __syncthreads();
    const int d = s_rs.level;
    for (int i = threadIdx.x; i < p.n; i += kBlock) {
      const float ri = rr[i];
      if (!(ri < 1.0f)) continue;
      const Terms t = token_terms(sh[i], ri, s_rs.m, (float)s_rs.beta, p.est);
      const unsigned long long key = make_key(token_gain(t, i, s_rs, a, l), i);
      if ((key >> s_rs.shift) != s_rs.pre) continue;
      const int dig = (int)((key >> sel_off(d)) & ((1ull << sel_width(d)) - 1));
      atomicAdd(&s_bins[dig].cnt, 1u);
      atomicAdd(&s_bins[dig].bsum, to_fx(t.bi, s_rs.eb));
      atomicAdd(&s_bins[dig].vsum, to_fx(t.vi, s_rs.ev));
      atomicMax(&s_bins[dig].bmax, __float_as_uint(t.rb));
    }
    __syncthreads();
    if (threadIdx.x < kWave) sel_resolve(s_rs, s_bins, d, p, threadIdx.x);
    __syncthreads();
  }
  if (s_rs.mode == MODE_DONE) {
    if (threadIdx.x == 0) grs = s_rs;
    return;
  }
  // the crossing bin's tokens: collected by dk_select, or here
  if (s_rs.mode == MODE_COLLECT) {
    if (threadIdx.x == 0) s_cnt = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < p.n; i += kBlock) {
      const float ri = rr[i];
      if (!(ri < 1.0f)) continue;
      const Terms t = token_terms(sh[i], ri, s_rs.m, (float)s_rs.beta, p.est);
      const unsigned long long key = make_key(token_gain(t, i, s_rs, a, l), i);
      if ((key >> s_rs.shift) != s_rs.pre) continue;
      const uint32_t slot = atomicAdd(&s_cnt, 1u);
      if (slot < (uint32_t)kCand) {
        Cand cd;
        cd.key = key;
        cd.bfx = to_fx(t.bi, s_rs.eb);
        cd.vfx = to_fx(t.vi, s_rs.ev);
        cd.rb = __float_as_uint(t.rb);
        cd.pad = 0u;
        p.cand[(size_t)row * kCand + slot] = cd;
      }
    }
    __syncthreads();
  } else {
    if (threadIdx.x == 0) s_cnt = s_rs.ncand;
    __syncthreads();
  }
  const uint32_t nc = min(s_cnt, (uint32_t)kCand);
  const Cand *cand = p.cand + (size_t)row * kCand;
  // bitonic sort (descending key) of the candidates
  uint32_t np2 = 1;
  while (np2 < nc) np2 <<= 1;
  for (uint32_t i = threadIdx.x; i < np2; i += kBlock) {
    s_key[i] = i < nc ? cand[i].key : 0ull;
    s_idx[i] = i;
  }
  __syncthreads();
  for (uint32_t k = 2; k <= np2; k <<= 1) {
    for (uint32_t j = k >> 1; j > 0; j >>= 1) {
      for (uint32_t i = threadIdx.x; i < np2; i += kBlock) {
        const uint32_t ixj = i ^ j;
        if (ixj > i) {
          const bool desc = (i & k) == 0;
          const unsigned long long ki = s_key[i], kj = s_key[ixj];
          if (desc ? (ki < kj) : (ki > kj)) {
            s_key[i] = kj;
            s_key[ixj] = ki;
            const uint32_t t = s_idx[i];
            s_idx[i] = s_idx[ixj];
            s_idx[ixj] = t;
          }
        }
      }
      __syncthreads();
    }
  }
  // walk: fetching the first k+1 sorted candidates (k = 0..nc-1)
  const uint32_t per = (nc + kBlock - 1) / kBlock;
  const uint32_t lo = threadIdx.x * per, hi = min(lo + per, nc);
  unsigned long long mb = 0, mv = 0;
  uint32_t mmax_after = 0;
  for (uint32_t k = lo; k < hi; ++k) {
    const Cand &cd = cand[s_idx[k]];
    mb += cd.bfx;
    mv += cd.vfx;
  }
  unsigned long long tot_b, tot_v;
  const unsigned long long pb = block_exclusive_scan<unsigned long long>(mb, s_scan, &tot_b);
  const unsigned long long pv = block_exclusive_scan<unsigned long long>(mv, s_scan, &tot_v);
  // suffix max of b over candidates after position k: reverse scan of maxima
  uint32_t my_max = 0;
  for (uint32_t k = lo; k < hi; ++k) my_max = max(my_max, cand[s_idx[k]].rb);
  // max over threads with higher index
  __shared__ uint32_t s_tmax[kBlock];
  s_tmax[threadIdx.x] = my_max;
  __syncthreads();
  uint32_t after = 0;
  for (int t2 = threadIdx.x + 1; t2 < kBlock; ++t2) after = max(after, s_tmax[t2]);
  int best = 0x7fffffff;
  double best_e = 0.0;
  {
    // walk local range backwards to know the suffix max, then forwards
    uint32_t sufmax[1];
    (void)sufmax;
    unsigned long long cb = pb, cv = pv;
    for (uint32_t k = lo; k < hi; ++k) {
      const Cand &cd = cand[s_idx[k]];
      cb += cd.bfx;
      cv += cd.vfx;
      uint32_t bt = max(s_rs.bB, after);
      for (uint32_t k2 = k + 1; k2 < hi; ++k2) bt = max(bt, cand[s_idx[k2]].rb);
      const double tb = (double)(s_rs.bL_fx - s_rs.betaA - cb) * ldexp(1.0, -s_rs.eb);
      const double tv = (double)(s_rs.VL_fx - s_rs.VA - cv) * ldexp(1.0, -s_rs.ev);
      const double e = eps_of(tb, tv, (double)__uint_as_float(bt), s_rs.dnorm, a, l);
      if (e < (double)p.eps) {
        best = (int)k;
        best_e = e;
        break;
      }
    }
  }
  (void)mmax_after;
  __shared__ int s_bt[kBlock / kWave];
  const int bmin = -block_max<int>(-best, s_bt);
  if (threadIdx.x == 0) s_best = bmin;
  __syncthreads();
  if (best == s_best && best != 0x7fffffff) {
    RowState rs = s_rs;
    rs.kstar = (int)(rs.cntA + (uint32_t)best + 1u);
    rs.T = s_key[best];
    rs.T_shift = 0;
    rs.eps1 = (float)best_e;
    rs.mode = MODE_DONE;
    grs = rs;
  } else if (threadIdx.x == 0 && s_best == 0x7fffffff) {
    // unreachable: fetching the whole bin always certifies
    RowState rs = s_rs;
    rs.kstar = (int)(rs.cntA + nc);
    rs.T = nc ? s_key[nc - 1] : (rs.pre << rs.shift);
    rs.T_shift = 0;
    rs.eps1 = 0.0f;
    rs.mode = MODE_DONE;
    grs = rs;
  }
}

// ------------------------------------------------------------ fetch
template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_mark(DParams p) {
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.G + g;
  __shared__ RowState s_rs[GRP];
  __shared__ uint32_t s_red[kBlock / kWave];
  if (threadIdx.x < GRP) s_rs[threadIdx.x] = p.rows[row_of(p, b, g, threadIdx.x, GRP)];
  __syncthreads();
  bool any = false;
  for (int h = 0; h < GRP; ++h) any |= s_rs[h].fetch && s_rs[h].kstar > 0;
  const double a = p.a_delta, l = p.l_delta;
  const float *rr = p.r + (size_t)bg * p.n;
  const uint32_t *rb = p.resbits + (size_t)bg * p.nwords;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int base = c * p.chunk;
  uint32_t count = 0;
  if (any) {
    for (int k = 0; k < p.chunk / kBlock; ++k) {
      const int i = base + k * kBlock + threadIdx.x;
      bool f = false;
      if (i < p.n) {
        const float ri = rr[i];
        if (ri < 1.0f && !((rb[i / 32] >> (i % 32)) & 1u)) {
#pragma unroll
          for (int h = 0; h < GRP; ++h) {
            const RowState &rs = s_rs[h];
            if (!rs.fetch || rs.kstar == 0 || f) continue;
            const int row = row_of(p, b, g, h, GRP);
            const Terms t = token_terms(p.shat[(size_t)row * p.n + i], ri, rs.m,
                                        (float)rs.beta, p.est);
            f = is_member(make_key(token_gain(t, i, rs, a, l), i), rs);
          }
        }
      }
      count += f ? 1u : 0u;
      const unsigned long long m = __ballot(f);
      const int w0 = (base + k * kBlock + wave * kWave) / 32;
      if (lane == 0 && w0 < p.nwords) p.fbits[(size_t)bg * p.nwords + w0] = (uint32_t)m;
      if (lane == 32 && w0 + 1 < p.nwords)
        p.fbits[(size_t)bg * p.nwords + w0 + 1] = (uint32_t)(m >> 32);
    }
  }
  const uint32_t tot = block_sum<uint32_t>(count, s_red);
  if (threadIdx.x == 0) p.fcnt[(size_t)bg * p.nch + c] = tot;
}

template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_gather(DParams p) {
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.G + g;
  __shared__ int s_pos[4096];
  __shared__ uint32_t s_red[kBlock / kWave + 1];
  uint32_t before = 0;
  for (int i = threadIdx.x; i < c; i += kBlock) before += p.fcnt[(size_t)bg * p.nch + i];
  const uint32_t offset = block_sum<uint32_t>(before, s_red);
  const int wpc = p.chunk / 32;
  const int w0 = c * wpc;
  uint32_t total = 0;
  // chunk sizes are at most 4096 tokens (128 words)
  uint32_t word = 0;
  if ((int)threadIdx.x < wpc && w0 + (int)threadIdx.x < p.nwords)
    word = p.fbits[(size_t)bg * p.nwords + w0 + threadIdx.x];
  const uint32_t at0 = block_exclusive_scan<uint32_t>((uint32_t)__popc(word), s_red, &total);
  {
    uint32_t w = word, o = at0;
    while (w) {
      const int bit = __ffs(w) - 1;
      s_pos[o++] = (w0 + (int)threadIdx.x) * 32 + bit;
      w &= w - 1;
    }
  }
  __syncthreads();
  int32_t *fidx = p.fidx + (size_t)bg * p.fetch_cap;
  for (uint32_t k = threadIdx.x; k < total; k += kBlock) {
    const uint32_t slot = offset + k;
    if (slot < (uint32_t)p.fetch_cap) fidx[slot] = s_pos[k];
  }
  // copy host rows (K then V, 512 bytes) into staging, 16 bytes per lane;
  // four rows' worth of loads are issued before their stores
  const uint16_t *src_base = p.host_kv + (size_t)bg * p.n * 2 * kHeadDim;
  uint16_t *dst_base = p.staging + (size_t)bg * p.fetch_cap * 2 * kHeadDim;
  const uint32_t units = total * 32u;
  const uint32_t lim = min(units, ((uint32_t)p.fetch_cap > offset
                                       ? ((uint32_t)p.fetch_cap - offset) * 32u
                                       : 0u));
  auto src_of = [&](uint32_t u) {
    return reinterpret_cast<const uint4 *>(
        src_base + (size_t)s_pos[u >> 5] * 2 * kHeadDim + (u & 31u) * 8);
  };
  auto dst_of = [&](uint32_t u) {
    return reinterpret_cast<uint4 *>(
        dst_base + (size_t)(offset + (u >> 5)) * 2 * kHeadDim + (u & 31u) * 8);
  };
  uint32_t u = threadIdx.x;
  // four 16-byte host loads in flight per lane before their stores
  for (; u + 3 * kBlock < lim; u += 4 * kBlock) {
    const uint4 v0 = *src_of(u), v1 = *src_of(u + kBlock),
                v2 = *src_of(u + 2 * kBlock), v3 = *src_of(u + 3 * kBlock);
    *dst_of(u) = v0;
    *dst_of(u + kBlock) = v1;
    *dst_of(u + 2 * kBlock) = v2;
    *dst_of(u + 3 * kBlock) = v3;
  }
  for (; u < lim; u += kBlock) *dst_of(u) = *src_of(u);
  if (c == p.nch - 1 && threadIdx.x == 0) {
    const uint32_t all = offset + total;
    p.fcount[bg] = (int32_t)all;
    if (all > (uint32_t)p.fetch_cap) atomicOr(p.status, VKV_STATUS_FETCH_OVERFLOW);
    const uint32_t moved = min(all, (uint32_t)p.fetch_cap);
    atomicAdd(p.host_bytes, (unsigned long long)moved * 2ull * kHeadDim * 2ull);
  }
}

// ------------------------------------------------------------ attention
constexpr int kMaxFetchRowsPerBlock = 512;

// Coefficient of one resident row for one head: w on H and on F_h, and
// lambda w / r on S \ F_h.
template <int GRP>
__device__ __forceinline__ float resident_alpha(const DParams &p,
                                                const RowState &rs, int row,
                                                int pos, float ri, float ell,
                                                double a, double l) {
  const float w = expf(ell - rs.m);
  if (ri >= 1.0f) return w;
  const Terms t = token_terms(p.shat[(size_t)row * p.n + pos], ri, rs.m,
                              (float)rs.beta, p.est);
  if (rs.fetch && rs.kstar > 0 &&
      is_member(make_key(token_gain(t, pos, rs, a, l), pos), rs))
    return w;
  return t.lam * w / ri;
}

// gridDim.x = ncr resident-row blocks followed by ncf fetched-row blocks;
// each writes a partial (shift, sum of weights, weighted sum of V) per head.
template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_attn(DParams p) {
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.G + g;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int u = lane % 16;             // 8 dims per lane
  const int slot = threadIdx.x / 16;   // row slot within an iteration
  __shared__ RowState s_rs[GRP];
  __shared__ float s_lg[GRP][kMaxFetchRowsPerBlock];
  __shared__ float s_o[kBlock / kWave][GRP][kHeadDim];
  __shared__ float s_d[kBlock / kWave][GRP];
  __shared__ float s_red[kBlock / kWave];
  __shared__ float s_scale[kBlock / kWave][512];  // ncr + ncf <= 512
  if (threadIdx.x < GRP) s_rs[threadIdx.x] = p.rows[row_of(p, b, g, threadIdx.x, GRP)];
  __syncthreads();
  const double a = p.a_delta, l = p.l_delta;
  const float *rr = p.r + (size_t)bg * p.n;
  float acc[GRP][8], dsum[GRP], mloc[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    dsum[h] = 0.0f;
    mloc[h] = s_rs[h].m;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[h][k] = 0.0f;
  }
  if (x < p.ncr) {
    const int cnt = max(0, min(p.rcount[bg], p.cap));
    int lo, hi;
    split_range(cnt, p.ncr, x, lo, hi);
    const int32_t *ridx = p.ridx + (size_t)bg * p.cap;
    for (int j0 = lo; j0 < hi; j0 += kBlock / 16) {
      const int j = j0 + slot;
      if (j >= hi) continue;
      const int pos = ridx[j];
      if (pos < 0 || pos >= p.n) continue;
      const float ri = rr[pos];
      const uint4 raw = *reinterpret_cast<const uint4 *>(
          p.rkv + ((size_t)bg * p.cap + j) * 2 * kHeadDim + kHeadDim + u * 8);
      float vv[8];
      unpack8(raw, vv);
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        const int row = row_of(p, b, g, h, GRP);
        const float alpha = resident_alpha<GRP>(
            p, s_rs[h], row, pos, ri, p.ell[(size_t)row * p.cap + j], a, l);
        dsum[h] += alpha;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[h][k] = __builtin_fmaf(alpha, vv[k], acc[h][k]);
      }
    }
  } else {
    const int fc = max(0, min(p.fcount[bg], p.fetch_cap));
    int lo, hi;
    split_range(fc, p.ncf, x - p.ncr, lo, hi);
    const int32_t *fidx = p.fidx + (size_t)bg * p.fetch_cap;
    const uint16_t *st = p.staging + (size_t)bg * p.fetch_cap * 2 * kHeadDim;
    if (lo < hi) {
      float qv[GRP][8];
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(
            p.q + (size_t)row_of(p, b, g, h, GRP) * kHeadDim + u * 8);
        unpack8(raw, qv[h]);
      }
      // sub-blocks of at most kMaxFetchRowsPerBlock rows; the running shift
      // only grows, and earlier sums are rescaled when it does
      for (int sub = lo; sub < hi; sub += kMaxFetchRowsPerBlock) {
        const int shi = min(sub + kMaxFetchRowsPerBlock, hi);
        float mb[GRP];
#pragma unroll
        for (int h = 0; h < GRP; ++h) mb[h] = -INFINITY;
        // pass 1: exact logits of the fetched rows that belong to F_h
        for (int j0 = sub; j0 < shi; j0 += kBlock / 16) {
          const int j = j0 + slot;
          if (j >= shi) continue;
          const int pos = fidx[j];
          const float ri = rr[pos];
          const uint4 raw =
              *reinterpret_cast<const uint4 *>(st + (size_t)j * 2 * kHeadDim + u * 8);
          float kk[8];
          unpack8(raw, kk);
#pragma unroll
          for (int h = 0; h < GRP; ++h) {
            float accd = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) accd = __builtin_fmaf(qv[h][k], kk[k], accd);
            const float lg = group_sum<16>(accd) * kInvSqrtD;
            const RowState &rs = s_rs[h];
            bool member = false;
            if (rs.fetch && rs.kstar > 0) {
              const int row = row_of(p, b, g, h, GRP);
              const Terms t = token_terms(p.shat[(size_t)row * p.n + pos], ri, rs.m,
                                          (float)rs.beta, p.est);
              member = is_member(make_key(token_gain(t, pos, rs, a, l), pos), rs);
            }
            const float v = member ? lg : -INFINITY;
            if (u == 0) s_lg[h][j - sub] = v;
            mb[h] = fmaxf(mb[h], v);
          }
        }
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
          const float m2 = fmaxf(mloc[h], block_max<float>(mb[h], s_red));
          if (m2 > mloc[h]) {
            const float sc = expf(mloc[h] - m2);
            dsum[h] *= sc;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[h][k] *= sc;
            mloc[h] = m2;
          }
        }
        __syncthreads();
        // pass 2: weights and values
        for (int j0 = sub; j0 < shi; j0 += kBlock / 16) {
          const int j = j0 + slot;
          if (j >= shi) continue;
          const uint4 raw = *reinterpret_cast<const uint4 *>(
              st + (size_t)j * 2 * kHeadDim + kHeadDim + u * 8);
          float vv[8];
          unpack8(raw, vv);
#pragma unroll
          for (int h = 0; h < GRP; ++h) {
            const float lg = s_lg[h][j - sub];
            const float alpha = lg == -INFINITY ? 0.0f : expf(lg - mloc[h]);
            dsum[h] += alpha;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[h][k] = __builtin_fmaf(alpha, vv[k], acc[h][k]);
          }
        }
        __syncthreads();
      }
    }
  }
  // reduce the four 16-lane row slots of each wave, then the waves
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float v = acc[h][k];
      v += shfl_xor(v, 16);
      v += shfl_xor(v, 32);
      acc[h][k] = v;
    }
    float d = dsum[h];
    d += shfl_xor(d, 16);
    d += shfl_xor(d, 32);
    dsum[h] = d;
  }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
#pragma unroll
      for (int k = 0; k < 8; ++k) s_o[wave][h][u * 8 + k] = acc[h][k];
      if (lane == 0) s_d[wave][h] = dsum[h];
    }
  }
  __syncthreads();
  const int np = p.ncr + p.ncf;
  for (int i = threadIdx.x; i < GRP * kHeadDim; i += kBlock) {
    const int h = i / kHeadDim, e = i % kHeadDim;
    float o = 0.0f;
    for (int w = 0; w < kBlock / kWave; ++w) o += s_o[w][h][e];
    p.apart[(size_t)row_of(p, b, g, h, GRP) * np + x].o[e] = o;
  }
  if (threadIdx.x < GRP) {
    const int h = threadIdx.x;
    float d = 0.0f;
    for (int w = 0; w < kBlock / kWave; ++w) d += s_d[w][h];
    AttnPart *ap = p.apart + (size_t)row_of(p, b, g, h, GRP) * np + x;
    ap->d = d;
    ap->m = mloc[h];
  }
  if (!last_block_arrive(&p.groups[bg].arrive[ARR_ATTN], gridDim.x)) return;
  // ---- merge the partial softmax sums by log-sum-exp (one wave per head)
  for (int h = wave; h < GRP; h += kBlock / kWave) {
    const int row = row_of(p, b, g, h, GRP);
    const AttnPart *ap = p.apart + (size_t)row * np;
    float M = -INFINITY;
    for (int i = lane; i < np; i += kWave)
      if (ap[i].d > 0.0f) M = fmaxf(M, ap[i].m);
    M = wave_max(M);
    float D = 0.0f;
    for (int i = lane; i < np; i += kWave) {
      const float sc = ap[i].d > 0.0f ? expf(ap[i].m - M) : 0.0f;
      s_scale[wave][i] = sc;
      D += ap[i].d * sc;
    }
    D = wave_sum(D);
    for (int e = lane; e < kHeadDim; e += kWave) {
      float o = 0.0f;
      for (int i = 0; i < np; ++i) {
        const float sc = s_scale[wave][i];
        if (sc != 0.0f) o += ap[i].o[e] * sc;
      }
      p.out[(size_t)row * kHeadDim + e] = o / D;
    }
    if (lane == 0) {
      const RowState &rs = p.rows[row];
      p.d_hat[row] = D;
      p.log_shift[row] = M;
      p.eps_hat0[row] = (float)rs.eps0;
      p.eps_hat[row] = rs.fetch ? rs.eps1 : (float)rs.eps0;
      p.k_star[row] = rs.fetch ? rs.kstar : 0;
      if (p.row_stats) {
        double *sr = p.row_stats + (size_t)row * 8;
        sr[0] = rs.m;
        sr[1] = rs.dnorm;
        sr[2] = rs.beta;
        sr[3] = rs.betaL;
        sr[4] = rs.VL;
        sr[5] = rs.b1;
        sr[6] = rs.eps0;
        sr[7] = rs.fetch ? rs.eps1 : rs.eps0;
      }
    }
  }
}

// Records the timing event after kernel `k` when the caller asked for it.
struct PhaseMark {
  void **ev;
  hipStream_t s;
  void operator()(int k) const {
    if (ev) (void)hipEventRecord(static_cast<hipEvent_t>(ev[k]), s);
  }
};

template <int GRP>
hipError_t run(const DParams &p, hipStream_t s, int sd, void **events) {
  const dim3 blk(kBlock);
  const dim3 gch((unsigned)p.nch, (unsigned)p.G, (unsigned)p.B);
  const dim3 gres((unsigned)p.ncr, (unsigned)p.G, (unsigned)p.B);
  const PhaseMark mark{events, s};
  int k = 0;
  mark(k++);
  if (p.weights == VKV_W_PERFECT)
    dk_scan_exact<GRP><<<gch, blk, 0, s>>>(p);
  else if (sd == 32)
    dk_scan<GRP, 32><<<gch, blk, 0, s>>>(p);
  else
    dk_scan<GRP, 16><<<gch, blk, 0, s>>>(p);
  mark(k++);
  dk_resident<GRP><<<gres, blk, 0, s>>>(p);
  mark(k++);
  for (int lev = 0; lev < 4; ++lev) {
    dk_beta<GRP><<<gch, blk, 0, s>>>(p, lev);
    mark(k++);
  }
  dk_cert<GRP><<<gch, blk, 0, s>>>(p);
  mark(k++);
  for (int pass = 0; pass < 3; ++pass) {
    dk_select<GRP><<<gch, blk, 0, s>>>(p);
    mark(k++);
  }
  dk_finish<GRP><<<dim3((unsigned)GRP, (unsigned)p.G, (unsigned)p.B), blk, 0, s>>>(p);
  mark(k++);
  dk_mark<GRP><<<gch, blk, 0, s>>>(p);
  mark(k++);
  dk_gather<GRP><<<gch, blk, 0, s>>>(p);
  mark(k++);
  dk_attn<GRP><<<dim3((unsigned)(p.ncr + p.ncf), (unsigned)p.G, (unsigned)p.B), blk, 0, s>>>(p);
  mark(k++);
  return hipGetLastError();
}

const char *const kPhaseNames[] = {
    "scan", "resident", "beta0", "beta1", "beta2", "beta3", "cert",
    "select0", "select1", "select2", "finish", "mark", "gather", "attn"};

}  // namespace

int decode_phase_count() {
  return (int)(sizeof(kPhaseNames) / sizeof(kPhaseNames[0]));
}

const char *decode_phase_name(int i) {
  return (i >= 0 && i < decode_phase_count()) ? kPhaseNames[i] : nullptr;
}

DecodeLayout decode_layout(const vkv_decode_args &a) {
  DecodeLayout L{};
  L.grp = a.n_q_heads / a.n_kv_heads;
  L.chunk = 512;
  L.nch = (a.n_tokens + L.chunk - 1) / L.chunk;
  // workgroups per group for the resident rows and for the fetched rows:
  // about 2048 workgroups per launch in total, at least 64 rows each
  const long long groups_ll = (long long)a.batch * a.n_kv_heads;
  const int target = (int)((2048 + groups_ll - 1) / groups_ll);
  const int rmax = a.cap < a.n_tokens ? a.cap : a.n_tokens;
  // (each at most 256, so the merge sees at most 512 partial sums)
  L.ncr = std::max(1, std::min(std::min(target, 256), (rmax + 63) / 64));
  L.ncf = std::max(1, std::min(std::min(target / 2, 256), (a.fetch_cap + 63) / 64));
  L.nwords = (a.n_tokens + 31) / 32;
  const size_t B = (size_t)a.batch, Hq = (size_t)a.n_q_heads,
               G = (size_t)a.n_kv_heads, n = (size_t)a.n_tokens;
  const size_t rows = B * Hq, groups = B * G;
  Carve c;
  L.rows = c.take<RowState>(rows);
  L.groups = c.take<GroupState>(groups);
  L.shat = c.take<float>(rows * n);
  L.ell = c.take<float>(rows * (size_t)a.cap);
  L.resbits = c.take<uint32_t>(groups * L.nwords);
  L.fbits = c.take<uint32_t>(groups * L.nwords);
  L.pmax = c.take<float>(rows * (L.nch + L.ncr));
  L.hpart = c.take<uint32_t>(groups * (L.nch + L.ncr));  // H counts per chunk
  L.bbins = c.take<double>(rows * 3 * kBetaEdges);
  L.cpart = c.take<CertPart>(rows * L.nch);
  L.dpart = c.take<double2>(rows * L.nch);
  L.sbins = c.take<SelBin>(rows * kSelBins);
  L.cand = c.take<Cand>(rows * kCand);
  L.fcnt = c.take<uint32_t>(groups * L.nch);
  L.apart = c.take<AttnPart>(rows * (L.ncr + L.ncf));
  L.staging = c.take<uint16_t>(groups * (size_t)a.fetch_cap * 2 * kHeadDim);
  L.total = (c.off + 255) & ~size_t(255);
  return L;
}

hipError_t launch_decode(const vkv_decode_args &a, const DecodeLayout &L,
                         const uint16_t *host_kv_dev, hipStream_t s) {
  DParams p{};
  p.q = a.q;
  p.rkv = a.resident_kv;
  p.sketch = a.sketch;
  p.host_kv = host_kv_dev;
  p.ridx = a.resident_idx;
  p.rcount = a.resident_count;
  p.proj = a.proj;
  p.r = a.r;
  p.out = a.out;
  p.d_hat = a.d_hat;
  p.log_shift = a.log_shift;
  p.eps_hat0 = a.eps_hat0;
  p.eps_hat = a.eps_hat;
  p.k_star = a.k_star;
  p.fidx = a.fetch_idx;
  p.fcount = a.fetch_count;
  p.host_bytes = reinterpret_cast<unsigned long long *>(a.host_bytes);
  p.row_stats = a.row_stats;
  p.status = a.status;
  void *w = a.workspace;
  p.rows = at<RowState>(w, L.rows);
  p.groups = at<GroupState>(w, L.groups);
  p.shat = at<float>(w, L.shat);
  p.ell = at<float>(w, L.ell);
  p.resbits = at<uint32_t>(w, L.resbits);
  p.fbits = at<uint32_t>(w, L.fbits);
  p.pmax = at<float>(w, L.pmax);
  p.hpart = at<uint32_t>(w, L.hpart);
  p.bbins = at<double>(w, L.bbins);
  p.cpart = at<CertPart>(w, L.cpart);
  p.dpart = at<double2>(w, L.dpart);
  p.sbins = at<SelBin>(w, L.sbins);
  p.cand = at<Cand>(w, L.cand);
  p.fcnt = at<uint32_t>(w, L.fcnt);
  p.apart = at<AttnPart>(w, L.apart);
  p.staging = at<uint16_t>(w, L.staging);
  p.B = a.batch;
  p.Hq = a.n_q_heads;
  p.G = a.n_kv_heads;
  p.n = a.n_tokens;
  p.cap = a.cap;
  p.fetch_cap = a.fetch_cap;
  p.nch = L.nch;
  p.ncr = L.ncr;
  p.ncf = L.ncf;
  p.nwords = L.nwords;
  p.chunk = L.chunk;
  p.eps = a.eps;
  p.l_delta = log(2.0 / (double)a.delta);
  p.a_delta = p.l_delta / 3.0;
  p.est = a.estimator;
  p.weights = a.weights;
  switch (L.grp) {
    case 1: return run<1>(p, s, a.sketch_dim, a.phase_events);
    case 2: return run<2>(p, s, a.sketch_dim, a.phase_events);
    case 4: return run<4>(p, s, a.sketch_dim, a.phase_events);
    case 8: return run<8>(p, s, a.sketch_dim, a.phase_events);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vkv
