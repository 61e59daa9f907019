// PoissonComp on gfx950 ("Verify Before You Fetch", Algorithm 1 and
// section 4.1, eq. 3).
//
// One slice = one (layer, KV head) of n tokens. Scores are read on the 2^-32
// grid (tq in [1, 2^32]). The water level c is the root of
//     f(c) = sum_{free i} min(1, c tq_i) = B_U        (B_U = budget - |F|).
// With e = 1/c this is g(e) = sum min(tq_i, e) - B_U e = 0, where g is concave
// with g(1) > 0, so F(e) := [g(e) >= 0] is true up to the root and false
// after it. Three radix passes over 11-bit digits of the 33-bit scores, each
// with exact per-bin counts and u64 sums, find e* = max{integer e : F(e)}
// exactly; the saturation count j* and c = (B_U - j*)/T follow in integers.
// Then r_i = float(double(num * tq_i) / double(den)) (one correctly rounded
// divide, one conversion), H = forced u {num * tq_i >= den}, and the sample is
// Z_i = [u_i < r_i] with u_i from Philox4x32-10 keyed by the seed, counter
// (token, head, layer, 0). Finally the resident rows H u S are listed in
// ascending position and their K/V rows are gathered (K then V per row).
//
// Every launch is HBM-streaming: 4 bytes of tau per token per radix pass,
// 4 bytes of r written, and 512 bytes moved per resident row.

#include "vkv_common.h"
#include "vkv_internal.h"

namespace vkv {
namespace {

struct CParams {
  const float *tau;
  const uint16_t *k, *v;
  float *r;
  int32_t *ridx;
  int32_t *rcount;
  uint16_t *rkv;
  double *wl;
  uint32_t *status;
  CompressSlice *slices;
  uint32_t *hcnt;
  unsigned long long *hsum;
  uint32_t *ccnt;
  uint32_t *bits;
  int n, n_heads, n_sink, n_local, cap, layer0, ncc, nwords;
  int64_t ns, kvs;  // positions per slice in tau, r, k, v; elements per token in k, v
  int64_t b_free;
  uint32_t seed_lo, seed_hi;
};

// floor(tau * 2^32) clamped to [1, 2^32]; the scaling is exact in fp32.
__device__ __forceinline__ uint64_t tau_q(float t) {
  const float s = t * 4294967296.0f;
  if (!(s >= 1.0f)) return 1ull;
  if (s >= 4294967296.0f) return 4294967296ull;
  return (uint64_t)s;
}

__device__ __forceinline__ bool is_forced(const CParams &p, int i) {
  return i < p.n_sink || i >= p.n - p.n_local;
}

__global__ __launch_bounds__(kBlock) void ck_zero(uint32_t *buf, size_t words,
                                                  uint32_t *status) {
  for (size_t i = blockIdx.x * (size_t)kBlock + threadIdx.x; i < words;
       i += (size_t)gridDim.x * kBlock)
    buf[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0 && status) *status = 0u;
}

// One radix level: histogram of the 11-bit digit at `shift` among free tokens
// whose higher digits match the slice's bracket, added to the slice's global
// histogram (ck_pick then picks the bin holding e* and narrows the bracket).
__global__ __launch_bounds__(kBlock) void ck_hist(CParams p, int level) {
  const int slice = blockIdx.y, chunk = blockIdx.x;
  CompressSlice *st = p.slices + slice;
  if (st->done) return;
  __shared__ uint32_t s_cnt[kCompBins];
  __shared__ unsigned long long s_sum[kCompBins];
  for (int b = threadIdx.x; b < kCompBins; b += kBlock) {
    s_cnt[b] = 0u;
    s_sum[b] = 0ull;
  }
  __syncthreads();
  const int shift = level == 0 ? 22 : (level == 1 ? 11 : 0);
  const int hshift = shift + 11;
  const uint64_t lo = st->lo;
  const uint64_t pref = lo >> hshift;
  const float *tau = p.tau + (size_t)slice * p.ns;
  const int base = chunk * kCompChunk;
  // the thread's scores first, all in flight together (indices past the
  // slice read its last score, which is not used)
  constexpr int PT = kCompChunk / kBlock;
  float tv[PT];
#pragma unroll
  for (int k = 0; k < PT; ++k)
    tv[k] = tau[min(base + k * kBlock + (int)threadIdx.x, p.n - 1)];
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    const int i = base + k * kBlock + threadIdx.x;
    if (i >= p.n || is_forced(p, i)) continue;
    const uint64_t v = tau_q(tv[k]);
    if (level > 0 && (v >> hshift) != pref) continue;
    const int d = (int)((v >> shift) & (kCompBins - 1));
    atomicAdd(&s_cnt[d], 1u);
    atomicAdd(&s_sum[d], (unsigned long long)v);
  }
  __syncthreads();
  uint32_t *gc = p.hcnt + (size_t)slice * kCompBins;
  unsigned long long *gs = p.hsum + (size_t)slice * kCompBins;
  for (int b = threadIdx.x; b < kCompBins; b += kBlock) {
    if (s_cnt[b]) {
      atomicAdd(gc + b, s_cnt[b]);
      atomicAdd(gs + b, s_sum[b]);
    }
  }
}

// One workgroup per slice, after each histogram level: locate the bin that
// holds e* from the slice's global histogram (complete once the level's
// launch has ended), narrow the bracket or settle c, and zero the histogram
// for the next level. (A separate launch instead of a last-arriving
// workgroup: no workgroup of the histogram launch needs a device-scope
// fence.)
__global__ __launch_bounds__(kBlock) void ck_pick(CParams p, int level) {
  const int slice = blockIdx.x;
  CompressSlice *st = p.slices + slice;
  if (st->done) return;
  __shared__ unsigned long long s_red[kBlock / kWave + 1];
  __shared__ int s_best;
  const int shift = level == 0 ? 22 : (level == 1 ? 11 : 0);
  const uint64_t lo = st->lo;
  uint32_t *gc = p.hcnt + (size_t)slice * kCompBins;
  unsigned long long *gs = p.hsum + (size_t)slice * kCompBins;
  constexpr int PER = kCompBins / kBlock;  // 8 bins per thread
  uint64_t c[PER], s[PER];
  uint64_t my_c = 0, my_s = 0;
  for (int j = 0; j < PER; ++j) {
    const int b = threadIdx.x * PER + j;
    c[j] = gc[b];
    s[j] = gs[b];
    my_c += c[j];
    my_s += s[j];
  }
  unsigned long long tot_c, tot_s;
  const uint64_t c_before = block_exclusive_scan<unsigned long long>(
      my_c, s_red, &tot_c);
  const uint64_t s_before = block_exclusive_scan<unsigned long long>(
      my_s, s_red, &tot_s);
  const uint64_t bu = (uint64_t)p.b_free;
  if (level == 0 && bu >= tot_c) {
    // every free token saturates: c = +inf, L is empty
    if (threadIdx.x == 0) {
      st->n_free = (uint32_t)tot_c;
      st->all_sat = 1;
      st->done = 1;
      st->num = 1;
      st->den = 0;
      if (p.wl) p.wl[slice] = __longlong_as_double(0x7ff0000000000000ll);
    }
  } else {
    const uint64_t s_below = st->s_below;
    const uint64_t c_above = st->c_above;
    int best = -1;
    uint64_t cb = c_before, sb = s_before;
    for (int j = 0; j < PER; ++j) {
      const int b = threadIdx.x * PER + j;
      const uint64_t e = lo + ((uint64_t)b << shift);
      const uint64_t s_lt = s_below + sb;
      const uint64_t c_ge = c_above + (tot_c - cb);
      if (s_lt + c_ge * e >= bu * e) best = b;
      cb += c[j];
      sb += s[j];
    }
    const int top = block_max<int>(best, reinterpret_cast<int *>(s_red));
    if (threadIdx.x == 0) s_best = top;
    __syncthreads();
    const int jb = s_best;
    if (threadIdx.x == jb / PER) {
      uint64_t cb2 = c_before, sb2 = s_before;
      for (int j = 0; j < jb % PER; ++j) {
        cb2 += c[j];
        sb2 += s[j];
      }
      const uint64_t m = c[jb % PER];
      const uint64_t e = lo + ((uint64_t)jb << shift);
      const uint64_t s_lt = s_below + sb2;          // scores below e
      const uint64_t c_ge = c_above + (tot_c - cb2);  // scores at or above e
      if (level == 0) st->n_free = (uint32_t)tot_c;
      if (level < 2) {
        st->lo = e;
        st->s_below = s_lt;
        st->c_above = (uint32_t)(c_ge - m);
      } else {
        // e is now a single score value: decide whether the tokens equal to
        // it saturate (they do exactly when f(1/e) == B_U).
        const bool strict = s_lt + c_ge * e > bu * e;
        const uint64_t j_star = strict ? c_ge - m : c_ge;
        const uint64_t T = strict ? s_lt + m * e : s_lt;
        st->num = bu - j_star;
        st->den = T;
        st->done = 1;
        if (p.wl)
          p.wl[slice] = (double)(bu - j_star) * 4294967296.0 / (double)T;
      }
    }
  }
  // leave the global histogram zeroed for the next level
  for (int b = threadIdx.x; b < kCompBins; b += kBlock) {
    gc[b] = 0u;
    gs[b] = 0ull;
  }
}

// r_i, H/L and the Poisson sample; one residency bit per token.
__global__ __launch_bounds__(kBlock) void ck_rate(CParams p) {
  const int slice = blockIdx.y, chunk = blockIdx.x;
  const uint32_t layer = (uint32_t)(p.layer0 + slice / p.n_heads);
  const uint32_t head = (uint32_t)(slice % p.n_heads);
  const CompressSlice *st = p.slices + slice;
  const uint64_t num = st->num, den = st->den;
  const bool all_sat = st->all_sat != 0;
  const double dden = (double)den;
  const float *tau = p.tau + (size_t)slice * p.ns;
  float *rr = p.r + (size_t)slice * p.ns;
  uint32_t *bits = p.bits + (size_t)slice * p.nwords;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int base = chunk * kCompChunk;
  // the thread's scores first, all in flight together (indices past the
  // slice read its last score, which is not used)
  constexpr int PT = kCompChunk / kBlock;
  float tv[PT];
#pragma unroll
  for (int k = 0; k < PT; ++k)
    tv[k] = tau[min(base + k * kBlock + (int)threadIdx.x, p.n - 1)];
  uint32_t count = 0;
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    const int i = base + k * kBlock + threadIdx.x;
    bool res = false;
    if (i < p.n) {
      float ri = 1.0f;
      if (is_forced(p, i) || all_sat) {
        res = true;
      } else {
        const uint64_t prod = num * tau_q(tv[k]);
        if (prod >= den) {
          res = true;
        } else {
          const float qv = (float)((double)prod / dden);
          ri = fminf(qv, 0.99999994039535522461f);  // 1 - 2^-24
          const uint32_t x0 = philox4x32_10_x0((uint32_t)i, head, layer, 0u,
                                               p.seed_lo, p.seed_hi);
          const float u = (float)(x0 >> 8) * 5.9604644775390625e-08f;
          res = u < ri;
        }
      }
      rr[i] = ri;
    }
    count += res ? 1u : 0u;
    const unsigned long long m = __ballot(res);
    const int w0 = (base + k * kBlock + wave * kWave) / 32;
    if (lane == 0 && w0 < p.nwords) bits[w0] = (uint32_t)m;
    if (lane == 32 && w0 + 1 < p.nwords) bits[w0 + 1] = (uint32_t)(m >> 32);
  }
  __shared__ uint32_t s_red[kBlock / kWave];
  const uint32_t tot = block_sum<uint32_t>(count, s_red);
  if (threadIdx.x == 0) p.ccnt[(size_t)slice * p.ncc + chunk] = tot;
}

// Ascending list of resident positions and the K/V row gather.
__global__ __launch_bounds__(kBlock) void ck_compact(CParams p) {
  const int slice = blockIdx.y, chunk = blockIdx.x;
  constexpr int WPC = kCompChunk / 32;  // 128 bitmap words per chunk
  __shared__ int s_pos[kCompChunk];
  __shared__ uint32_t s_red[kBlock / kWave + 1];
  // rows of earlier chunks
  uint32_t before = 0;
  for (int c = threadIdx.x; c < chunk; c += kBlock)
    before += p.ccnt[(size_t)slice * p.ncc + c];
  const uint32_t offset = block_sum<uint32_t>(before, s_red);
  const int w0 = chunk * WPC;
  uint32_t word = 0;
  if (threadIdx.x < WPC && w0 + threadIdx.x < p.nwords)
    word = p.bits[(size_t)slice * p.nwords + w0 + threadIdx.x];
  uint32_t cnt;
  const uint32_t at0 =
      block_exclusive_scan<uint32_t>((uint32_t)__popc(word), s_red, &cnt);
  {
    uint32_t w = word, o = at0;
    while (w) {
      const int b = __ffs(w) - 1;
      s_pos[o++] = (w0 + (int)threadIdx.x) * 32 + b;
      w &= w - 1;
    }
  }
  __syncthreads();
  int32_t *ridx = p.ridx + (size_t)slice * p.cap;
  for (uint32_t k = threadIdx.x; k < cnt; k += kBlock) {
    const uint32_t slot = offset + k;
    if (slot < (uint32_t)p.cap) ridx[slot] = s_pos[k];
  }
  if (p.rkv) {
    for (uint32_t u = threadIdx.x; u < cnt * 32u; u += kBlock) {
      const uint32_t row = u >> 5, part = u & 31u;
      const uint32_t slot = offset + row;
      if (slot >= (uint32_t)p.cap) continue;
      const size_t pos = (size_t)s_pos[row];
      const uint16_t *src = (part < 16 ? p.k : p.v) +
                            ((size_t)slice * p.ns + pos) * p.kvs +
                            (part & 15u) * 8;
      uint16_t *dst = p.rkv + ((size_t)slice * p.cap + slot) * (2 * kHeadDim) +
                      part * 8;
      *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    }
  }
  if (chunk == p.ncc - 1 && threadIdx.x == 0) {
    const uint32_t total = offset + cnt;
    p.rcount[slice] = (int32_t)total;
    if (total > (uint32_t)p.cap) atomicOr(p.status, VKV_STATUS_RESIDENT_OVERFLOW);
  }
}

}  // namespace

CompressLayout compress_layout(const vkv_compress_args &a) {
  CompressLayout L{};
  L.n_slices = a.n_layers * a.n_kv_heads;
  L.ncc = (a.n_tokens + kCompChunk - 1) / kCompChunk;
  L.nwords = (a.n_tokens + 31) / 32;
  Carve c;
  L.slices = c.take<CompressSlice>((size_t)L.n_slices);
  L.hcnt = c.take<uint32_t>((size_t)L.n_slices * kCompBins);
  L.hsum = c.take<unsigned long long>((size_t)L.n_slices * kCompBins);
  L.ccnt = c.take<uint32_t>((size_t)L.n_slices * L.ncc);
  L.bits = c.take<uint32_t>((size_t)L.n_slices * L.nwords);
  L.total = (c.off + 255) & ~size_t(255);
  return L;
}

hipError_t launch_compress(const vkv_compress_args &a, const CompressLayout &L,
                           int64_t b_free, int32_t n_forced, hipStream_t s) {
  (void)n_forced;
  CParams p{};
  p.tau = a.tau;
  p.k = a.k;
  p.v = a.v;
  p.r = a.r;
  p.ridx = a.resident_idx;
  p.rcount = a.resident_count;
  p.rkv = a.resident_kv;
  p.wl = a.water_level;
  p.status = a.status;
  p.slices = at<CompressSlice>(a.workspace, L.slices);
  p.hcnt = at<uint32_t>(a.workspace, L.hcnt);
  p.hsum = at<unsigned long long>(a.workspace, L.hsum);
  p.ccnt = at<uint32_t>(a.workspace, L.ccnt);
  p.bits = at<uint32_t>(a.workspace, L.bits);
  p.n = a.n_tokens;
  p.ns = a.ctx_stride > 0 ? a.ctx_stride : a.n_tokens;
  p.kvs = a.kv_stride > 0 ? a.kv_stride : kHeadDim;
  p.n_heads = a.n_kv_heads;
  p.n_sink = a.n_sink;
  p.n_local = a.n_local;
  p.cap = a.cap;
  p.layer0 = a.layer0;
  p.ncc = L.ncc;
  p.nwords = L.nwords;
  p.b_free = b_free;
  p.seed_lo = (uint32_t)(a.seed & 0xffffffffull);
  p.seed_hi = (uint32_t)(a.seed >> 32);

  // zero the slice states and the histograms (contiguous at the front)
  const size_t zero_words = L.ccnt / 4;
  ck_zero<<<dim3((unsigned)((zero_words + 4 * kBlock - 1) / (4 * kBlock) + 1)),
            dim3(kBlock), 0, s>>>(static_cast<uint32_t *>(a.workspace),
                                  zero_words, a.status);
  const dim3 grid((unsigned)L.ncc, (unsigned)L.n_slices);
  for (int level = 0; level < 3; ++level) {
    ck_hist<<<grid, dim3(kBlock), 0, s>>>(p, level);
    ck_pick<<<dim3((unsigned)L.n_slices), dim3(kBlock), 0, s>>>(p, level);
  }
  ck_rate<<<grid, dim3(kBlock), 0, s>>>(p);
  ck_compact<<<grid, dim3(kBlock), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace vkv
