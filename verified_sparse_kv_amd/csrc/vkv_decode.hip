// KVFetch decode step on gfx950 ("Verify Before You Fetch", Algorithm 2,
// section 4.2; Definition 2, Lemma 1, eqs. 5-10, Theorem 2).
//
// A "group" is one (request b, KV head g) with its GRP = Hq/G query heads
// ("rows"). Kernels, in launch order:
//
//  dk_front     one launch of two kinds of workgroups. Scan workgroups: the
//               sketch logits s_i = <P_g^T q, sk_i>/sqrt(d) of every token for
//               the GRP heads at once (one sketch row serves all of them), and
//               per chunk the pass-0 sums of the beta* iteration against the
//               chunk's running shift. Resident workgroups: the exact logits
//               l_j = <q, k_j>/sqrt(d) on the resident rows, and per part the
//               shift and sum_H exp(l).
//  dk_rbeta x2  common shift m = max(max_R l, max_L s), D~ = sum_H w + sum_L
//               w~, then the Definition 2 fixed point beta* by bracketed
//               Newton passes on a convex piecewise-linear function, settled
//               from the band of undecided tokens (one launch per pass).
//  dk_rbin      binary shrinkage only (Appendix A.2): the tokens set to
//               lambda = r, one workgroup per row.
//  dk_rcert     lambda_i, beta(L), V(L) and the top two b_i per chunk
//               (Lemma 1, eq. 7).
//  dk_rcand     eps^(L) and, for a row that must fetch, the gain keys (eq. 9)
//               and each workgroup's local top candidates.
//  dk_rwalk     per row: the stopping rule (eq. 10) over the candidates by a
//               radix select, F_h into the row's and the KV head's bitmaps.
//  dk_fetch     the attention over the resident rows, and in the same launch
//               the gather of F_h minus S from pinned host memory by GPU
//               loads (zero-copy) with the attention over those rows.
//  dk_attn      merge of the partial softmax sums by log-sum-exp.
//
// With read-ahead (prefetch_rows), a second stream forks once the pass-0
// records exist and runs beside the planning launches: sp_hist (a sampled
// histogram of a planning score per KV head), sp_sel (the tokens above its
// threshold take slots of a device area) and sp_move (their rows copied
// from pinned host memory); dk_fetch waits for it and reads a fetched row
// from that area when it was read ahead.
//
// Passes over a row's tokens run as many workgroups per row; every
// workgroup combines the partial records of the previous launch itself, so
// no workgroup waits for another.
//
// All per-token recomputations (weights, lambda, certificate terms, gains)
// go through the same inline functions and the library is built with
// floating-point contraction off, so every pass sees identical values.

#include <algorithm>
#include <mutex>

#include <hip/hip_ext.h>

#include "vkv_common.h"
#include "vkv_internal.h"

namespace vkv {
namespace {

constexpr int kChunk = 512;      // tokens per workgroup in token passes
constexpr int kMaxTokens = 1 << 17;  // context length the decode kernels take
constexpr int kRowChunk = 2048;  // tokens per workgroup in row passes
constexpr int kRowTok = kRowChunk / kBlock;
constexpr int kCand = 2048;      // candidates per round of the streaming selection
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)
constexpr int kSelDigit = 11;    // radix digit of the selections' keys
constexpr int kSelBinsP = 1 << kSelDigit;
constexpr int kBinCap = 256;     // keys per round of the binary shrinkage
constexpr int kSpecBins = 1024;  // read-ahead score histogram: bin = -32 score
static_assert(kBinCap <= 4 * kWave, "one wave sorts a round");

struct RowState {
  float m;                // common shift of the planning and resident logits
  int32_t fetch;          // eps^(L) >= eps
  double dnorm;           // D~ * exp(-m)
  double beta;            // beta*
  double betaL, VL;       // beta(L), V(L) (float64 sums of fp32 terms)
  double s_full;          // sqrt((a b)^2 + 2 V l)
  float s_full_f;         // the same in fp32 (the gain formula's s)
  float ab1sq;            // ((a a) b1) b1 in fp32: the gain's (a b')^2 when b' = b1
  double eps0;            // eps^(L)
  float b1, b2;           // largest and second largest b_i (with multiplicity)
  int32_t amax;           // position of the unique argmax of b_i, else -1
  int32_t eb, ev;         // fixed-point exponents for beta_i and v_i
  double capb, capv;      // caps of beta_i and v_i in the fixed-point sums
  int32_t kstar;
  unsigned long long T;   // F_h = {i in L : key_i >= T}
  unsigned long long bkey;  // binary shrinkage: lambda = r for keys >= bkey
  float eps1;             // eps^(L') after fetching
  int32_t path;           // how k* was decided (VKV_PATH_*)
};


// State of a row's beta* iteration between launches.
struct BetaState {
  double lo, hi;        // bracket of the root
  double prev_cnt;      // |A| whose Newton step gave lo (-1: none)
  double beta;          // beta* once done
  double dnorm;         // D~ * exp(-m)
  int32_t done, pad;
};

// Binary shrinkage of a row (Appendix A.2): the tokens whose binary key is
// at least `key` have lambda = r; `beta` is their bias sum w~ (1 - r).
struct BinState {
  unsigned long long key;  // ~0: no token moved
  double beta;
};

// Certificate terms of one chunk of a row.
struct CertPart {
  double tb, tv;        // sums of beta_i and v_i
  float x1, x2;         // largest and second largest b_i
  int32_t p1, pad;      // position of x1 (smallest on ties)
};



struct DParams {
  const uint16_t *q, *rkv, *sketch, *host_kv;
  // 2-bit sketch (Appendix A.1): codes [B][G][n], zero points and scales
  // [B][G][ceil(n/128)][2][32], kept channels [B][G][32]; the shortlist
  // size and output; the scan's shortlist keys [B][G][n]
  const unsigned long long *sk2_codes;
  const uint16_t *sk2_zs;
  const int32_t *sk2_chan;
  int n_short;
  int32_t *shortlist;
  uint32_t *skey;
  const int32_t *ridx, *rcount;
  const float *proj, *r;
  float *out, *d_hat, *log_shift, *eps_hat0, *eps_hat;
  int32_t *k_star, *fidx, *fcount;
  unsigned long long *host_bytes;
  double *row_stats;
  int32_t *row_path;
  uint32_t *status;
  float *shat, *ell;
  uint32_t *fbits;
  uint32_t *hbits;   // [row][nwords] F_h of each row
  uint32_t *fstat;   // [B][G][nch + nrr] input-check bits of the front launch
  float *pmax;       // [row][nch + nrr] shift of each scan chunk / resident part
  double *p0part;    // [row][nch + nrr][4] pass-0 sums of each scan chunk
  double *hres;      // [row][nrr] sum over H of exp(l - shift) per part
  uint32_t *hpart;
  RowState *rows;
  int nsub, rsub;    // kRowChunk sub-chunks per row, and per row workgroup
  int nsel;          // candidate workgroups per row
  int nbeta;         // Newton launches of the beta* iteration (2 to 4)
  int ns;            // positions per (request, KV head) in r, the sketches
                     // and host_kv (>= n)
  // rows staged by the previous step and by this one (NULL: none)
  const int32_t *smap_prev;
  const uint16_t *stage_prev;
  int32_t *smap_next;
  uint16_t *stage_next;
  double *bpart;     // [2][row][nrc][kBetaRec] beta pass records
  float2 *band;      // [2][row][nrc][kBandChunk] (w~, rho) of band tokens
  BetaState *bstate; // [2][row]
  double *rbeta;     // [row][2] beta*, D~
  BinState *binst;   // [row] binary shrinkage: last moved key, its bias
  // binary shrinkage's first round, gathered by the beta launches: the
  // row's histogram of the top key digit, then per row workgroup its keys at
  // or above the round's bound (count, keys, biases)
  uint32_t *bhist;   // [row][kSelBinsP]
  uint32_t *bcnt;    // [row][nrc]
  unsigned long long *bkeys;  // [row][nrc][kBinCap]
  float *bav;        // [row][nrc][kBinCap]
  CertPart *cpart;   // [row][nrc]
  // candidate workgroups: [row][kSelWG] counts, local bounds, max b_i of
  // the keys not written, fixed-point totals; candidates [row][kCandMax]
  uint32_t *ccount;
  unsigned long long *clo;
  uint32_t *rpart;
  unsigned long long *tpart;
  unsigned long long *candk;
  float *candw, *candq;  // w~ and r of each candidate
  double *dpart;         // [row][kSelWG][2] float64 sums below the bound
  // read-ahead: per group a sampled score histogram and a slot counter, the
  // bitmaps of S and of the rows read ahead with each word's first slot;
  // the rows [group][spec_m]
  uint32_t *sp_hist;
  uint32_t *sp_cnt;
  uint32_t *sp_res, *sp_bits, *sp_base;
  int32_t *sp_list;  // [group][spec_m] positions to read, in slot order
  uint16_t *spec_kv;
  int spec_m;        // rows per group read ahead (0: none)
  int spec_cpw;      // kChunk chunks per selection workgroup
  float2 *apart;     // [row][ncr + ncf] (shift, sum of weights)
  float *aparto;     // [row][d][npad] weighted sums of V, part index fastest
  int B, Hq, G, n, cap, fetch_cap, nch, nrr, ncr, ncf, npad, nwords, chunk, nrc;
  float eps;
  double l_delta, a_delta;
  int est, weights;
};

// ------------------------------------------------------------ shared math
struct Terms {
  float wt, lam, bi, vi, rb, qr;  // qr = (1 - r) / r
};

// Descending key order = value descending, then position ascending (the
// gain order of eq. 10 and the binary-shrinkage order of Appendix A.2).
__device__ __forceinline__ unsigned long long make_key(float v, int pos) {
  return ((unsigned long long)__float_as_uint(v) << 24) |
         (unsigned long long)(0xFFFFFFu - (uint32_t)pos);
}
__device__ __forceinline__ int key_pos(unsigned long long key) {
  return (int)(0xFFFFFFu - (uint32_t)(key & 0xFFFFFFull));
}
// Binary-shrinkage key of a token of L: kappa = w~ (1 - r) / r (qr =
// (1 - r) / r), clamped to >= 0 so that malformed r cannot leave the key
// range.
__device__ __forceinline__ unsigned long long bin_key(float wt, float qr, int pos) {
  return make_key(fmaxf(wt * qr, 0.0f), pos);
}

// How lambda is formed: the clipped fixed point at beta (Definition 2), the
// binary rule of Appendix A.2 (lambda = r for the tokens whose binary key
// is at least bkey, 1 for the rest), or 1 (the unbiased estimator).
struct LamRule {
  float beta;
  int est;
  unsigned long long bkey;
};
__device__ __forceinline__ LamRule lam_rule(float beta, int est,
                                            unsigned long long bkey) {
  LamRule q;
  q.beta = beta;
  q.est = est;
  q.bkey = bkey;
  return q;
}

// (1 - r) / r with the hardware reciprocal (within 2 ulp): the same
// expression in every pass that forms it, so all passes agree bit for bit.
__device__ __forceinline__ float qr_of(float r) {
  return (1.0f - r) * __builtin_amdgcn_rcpf(r);
}

// lambda and the three certificate terms of Lemma 1 for the token of L at
// `pos` with planning weight wt. Divisions and the square root of the gain
// use the hardware reciprocal and square root (~1 ulp each): the terms only
// order tokens and feed float64 sums checked to 1e-4, and every pass uses
// these same functions.
__device__ __forceinline__ Terms token_terms_w(float wt, float r,
                                               const LamRule &lr, int pos) {
  Terms t;
  t.wt = wt;
  t.qr = qr_of(r);
  float lam = 1.0f;
  if (lr.est == VKV_EST_CLIP) {  // (uniform; the rest selects, no branches)
    const float x = lr.beta * r * __builtin_amdgcn_rcpf(wt * (1.0f - r));
    lam = wt > 0.0f ? fminf(1.0f, fmaxf(r, x)) : 1.0f;
  } else if (lr.est == VKV_EST_BINARY) {
    lam = bin_key(wt, t.qr, pos) >= lr.bkey ? r : 1.0f;
  }
  t.lam = lam;
  t.bi = wt * (1.0f - lam);
  const float lw = lam * wt;
  t.vi = lw * lw * t.qr;
  t.rb = lw * fmaxf(r, 1.0f - r) * __builtin_amdgcn_rcpf(r);
  return t;
}

// beta_i and v_i in float64 for the sums that give eps^(L') itself: v_i is
// squared in float64, so that the terms of tiny weights (a rest after the
// dominant tokens are fetched) do not underflow.
__device__ __forceinline__ void direct_terms(const Terms &t, double &bd,
                                             double &vd) {
  bd = (double)t.bi;
  const double lw = (double)t.lam * (double)t.wt;
  vd = lw * lw * (double)t.qr;
}

// The same from the planning logit s and the shift m (w~ = exp(s - m)).
__device__ __forceinline__ Terms token_terms(float s, float r, float m,
                                             const LamRule &lr, int pos) {
  return token_terms_w(expf(s - m), r, lr, pos);
}

// eq. 7 in float64.
__device__ __forceinline__ double eps_of(double beta, double var, double b,
                                         double dn, double a, double l) {
  const double ab = a * b;
  return (beta + ab + sqrt(ab * ab + 2.0 * var * l)) / dn;
}

// Gain g_i * D~ (eq. 9, cancellation-free form). With b' the largest b after
// removing token i (b itself unless i is the unique argmax),
//   s  = sqrt((a b)^2 + 2 V l),  s' = sqrt((a b')^2 + 2 (V - v_i) l),
//   g_i D~ = beta_i + a (b - b') + [a^2 (b - b')(b + b') + 2 v_i l] / (s + s').
// V - v_i is formed in float64 (it cancels when one token dominates V); the
// rest is fp32, which only perturbs the order of gains equal to ~1e-7.
__device__ __forceinline__ float token_gain(const Terms &t, int pos,
                                            const RowState &rs, float a,
                                            float l) {
  const float b1 = rs.b1;
  const float vp = (float)fmax(rs.VL - (double)t.vi, 0.0);
  if (pos != rs.amax) {
    // b' = b: the terms in b - b' are exact zeros, so the same value as the
    // general form below with (a b)^2 taken from the row
    const float sp = __builtin_amdgcn_sqrtf(rs.ab1sq + 2.0f * vp * l);
    const float den = rs.s_full_f + sp;
    const float frac = den > 0.0f ? (2.0f * t.vi * l) * __builtin_amdgcn_rcpf(den) : 0.0f;
    return t.bi + frac;
  }
  const float bp = rs.b2;
  const float sp = __builtin_amdgcn_sqrtf(a * a * bp * bp + 2.0f * vp * l);
  const float num = a * a * (b1 - bp) * (b1 + bp) + 2.0f * t.vi * l;
  const float den = rs.s_full_f + sp;
  const float frac = den > 0.0f ? num * __builtin_amdgcn_rcpf(den) : 0.0f;
  return t.bi + a * (b1 - bp) + frac;
}

// A term of the selection's fixed-point sums: min(x, cap) 2^e, truncated to
// an integer. The caps are c = 2 eps D~ for beta_i and c^2 / (2 l) for v_i
// (compared in fp32): a rest holding a term at its cap has eps^ >= 2 eps (to
// within the cap's fp32 rounding) whether the term is capped or not, so
// capping never changes a stopping decision, while a rest that can stop
// holds only exact terms. The scale follows eps D~ (cap 2^e < 2^40), not the
// largest term, so rests near the stopping point keep ~40 bits however heavy
// the fetched tokens are; with at most 2^17 tokens no sum overflows. The
// term is formed in float64, where x 2^e is exact and below 2^40, so a sum
// of at most 2^13 terms (one candidate workgroup's share) is still an exact
// integer in float64; other sums take it as a 64-bit integer. Every pass
// forms the terms with this one function, so all passes agree bit for bit.
__device__ __forceinline__ double fx_term(float x, double cap, int e) {
  const float cf = (float)cap;
  // (the product is exact in float64 and below 2^40; NaN takes the cap)
  return trunc(ldexp((double)(x < cf ? x : cf), e));
}
__device__ __forceinline__ unsigned long long sat_fx(float x, double cap,
                                                     int e) {
  return (unsigned long long)fx_term(x, cap, e);
}

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

// ------------------------------------------------------------ reductions
constexpr int kPlanThreads = 1024;  // row-level workgroups
constexpr int kPlanWaves = kPlanThreads / kWave;

// rho = r / (1 - r); the same expression in every pass.
__device__ __forceinline__ float plan_rho(float r) {
  return r * __builtin_amdgcn_rcpf(1.0f - r);
}

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

// Block-wide combination of NV values per thread for THREADS threads, in a
// fixed order (the same inputs give the same bits in every workgroup), and
// every thread gets the results. Within a wave the values move by DPP row
// operations (no LDS): quad exchanges and row rotations leave each 16-lane
// row's total in all of its lanes, and the four row totals are read from
// lanes 0, 16, 32 and 48 and folded in that order; across waves through LDS.
template <typename T>
struct OpSum {
  __device__ static T f(T a, T b) { return a + b; }
};
template <typename T>
struct OpMax {
  __device__ static T f(T a, T b) { return a > b ? a : b; }
};
template <typename T>
struct OpMin {
  __device__ static T f(T a, T b) { return a < b ? a : b; }
};

// DPP move of a 32- or 64-bit value (64-bit values move as two halves).
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_mov(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "dpp");
  if constexpr (sizeof(T) == 4) {
    int x;
    __builtin_memcpy(&x, &v, 4);
    x = __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
    T r;
    __builtin_memcpy(&r, &x, 4);
    return r;
  } else {
    int x[2];
    __builtin_memcpy(x, &v, 8);
    x[0] = __builtin_amdgcn_update_dpp(x[0], x[0], CTRL, 0xF, 0xF, false);
    x[1] = __builtin_amdgcn_update_dpp(x[1], x[1], CTRL, 0xF, 0xF, false);
    T r;
    __builtin_memcpy(&r, x, 8);
    return r;
  }
}
template <typename T>
__device__ __forceinline__ T lane_read(T v, int lane) {
  if constexpr (sizeof(T) == 4) {
    int x;
    __builtin_memcpy(&x, &v, 4);
    x = __builtin_amdgcn_readlane(x, lane);
    T r;
    __builtin_memcpy(&r, &x, 4);
    return r;
  } else {
    int x[2];
    __builtin_memcpy(x, &v, 8);
    x[0] = __builtin_amdgcn_readlane(x[0], lane);
    x[1] = __builtin_amdgcn_readlane(x[1], lane);
    T r;
    __builtin_memcpy(&r, x, 8);
    return r;
  }
}
// The wave's total, the same in every lane (all 64 lanes must be active).
template <typename T, typename OP>
__device__ __forceinline__ T wave_fold(T v) {
  constexpr int kXor1 = 0xB1, kXor2 = 0x4E;    // quad_perm [1,0,3,2], [2,3,0,1]
  constexpr int kRor4 = 0x124, kRor8 = 0x128;  // row_ror:4, row_ror:8
  v = OP::f(v, dpp_mov<kXor1>(v));
  v = OP::f(v, dpp_mov<kXor2>(v));
  v = OP::f(v, dpp_mov<kRor4>(v));
  v = OP::f(v, dpp_mov<kRor8>(v));
  return OP::f(OP::f(lane_read(v, 0), lane_read(v, 16)),
               OP::f(lane_read(v, 32), lane_read(v, 48)));
}
template <typename T, int NV, int THREADS, typename OP>
__device__ __forceinline__ void blk_combine(T (&v)[NV]) {
  constexpr int W = THREADS / kWave;
  __shared__ T buf[W * NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] = wave_fold<T, OP>(v[k]);
  __syncthreads();  // an earlier call may still be reading buf
  if (threadIdx.x % kWave == 0) {
#pragma unroll
    for (int k = 0; k < NV; ++k) buf[(threadIdx.x / kWave) * NV + k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    T acc = buf[k];
#pragma unroll
    for (int w = 1; w < W; ++w) acc = OP::f(acc, buf[w * NV + k]);
    v[k] = acc;
  }
}
template <typename T, int NV, int THREADS>
__device__ __forceinline__ void blk_reduce(T (&v)[NV]) {
  blk_combine<T, NV, THREADS, OpSum<T>>(v);
}
template <typename T, int NV>
__device__ __forceinline__ void plan_reduce(T (&v)[NV]) {
  blk_combine<T, NV, kPlanThreads, OpSum<T>>(v);
}
template <typename T, int THREADS>
__device__ __forceinline__ T blk_max(T x) {
  T v[1] = {x};
  blk_combine<T, 1, THREADS, OpMax<T>>(v);
  return v[0];
}
template <typename T>
__device__ __forceinline__ T plan_max(T x) {
  return blk_max<T, kPlanThreads>(x);
}
// Two sums and two maxima of 64-bit integers over a plan workgroup in one
// LDS round: each folded per wave, the waves combined in wave order; every
// thread gets the results.
__device__ __forceinline__ void plan_sum2_max2(unsigned long long (&v)[4]) {
  using U = unsigned long long;
  __shared__ U buf[kPlanWaves][4];
  v[0] = wave_fold<U, OpSum<U>>(v[0]);
  v[1] = wave_fold<U, OpSum<U>>(v[1]);
  v[2] = wave_fold<U, OpMax<U>>(v[2]);
  v[3] = wave_fold<U, OpMax<U>>(v[3]);
  __syncthreads();  // an earlier call may still be reading buf
  if (threadIdx.x % kWave == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) buf[threadIdx.x / kWave][k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = buf[0][k];
#pragma unroll
  for (int w = 1; w < kPlanWaves; ++w) {
    v[0] = OpSum<U>::f(v[0], buf[w][0]);
    v[1] = OpSum<U>::f(v[1], buf[w][1]);
    v[2] = OpMax<U>::f(v[2], buf[w][2]);
    v[3] = OpMax<U>::f(v[3], buf[w][3]);
  }
}

// Block-wide top two of (value, position) pairs as top2_merge keeps them
// (the merge does not depend on order), through LDS.
template <int THREADS>
__device__ __forceinline__ void blk_top2(float &x1, int &p1, float &x2) {
  __shared__ float b1[THREADS + 17], b2[THREADS + 17];
  __shared__ int bp[THREADS + 17];
  __syncthreads();
  b1[threadIdx.x] = x1;
  b2[threadIdx.x] = x2;
  bp[threadIdx.x] = p1;
  __syncthreads();
  if (threadIdx.x < 16) {
    float y1 = b1[threadIdx.x], y2 = b2[threadIdx.x];
    int yq = bp[threadIdx.x];
    for (int i = 1; i < THREADS / 16; ++i) {
      const int t = i * 16 + threadIdx.x;
      top2_merge(y1, yq, y2, b1[t], bp[t], b2[t]);
    }
    b1[THREADS + threadIdx.x] = y1;
    b2[THREADS + threadIdx.x] = y2;
    bp[THREADS + threadIdx.x] = yq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float y1 = b1[THREADS], y2 = b2[THREADS];
    int yq = bp[THREADS];
    for (int j = 1; j < 16; ++j)
      top2_merge(y1, yq, y2, b1[THREADS + j], bp[THREADS + j], b2[THREADS + j]);
    b1[THREADS + 16] = y1;
    b2[THREADS + 16] = y2;
    bp[THREADS + 16] = yq;
  }
  __syncthreads();
  x1 = b1[THREADS + 16];
  x2 = b2[THREADS + 16];
  p1 = bp[THREADS + 16];
}

// ------------------------------------------------------------ dk_scan
// End of a scan chunk: the per-head maxima over L of the chunk's logits
// (sd[h][t], r in sr[t], cnt tokens, staged in LDS), then pass 0 of the
// beta* iteration with the chunk's own shift mL: sum_L w~, sum rho over w~ >
// 0, their count, and max w~ (1 - r). The planning rescales them to the
// common shift.
// Pass-0 sums of one query head over a thread's tokens of L, with a running
// shift: w~ = exp(s - m) against the largest logit seen so far, the sums
// rescaled when it grows. A token counts in sum rho and |A(0)| when its w~
// is nonzero against that shift, a superset of the tokens nonzero against
// any larger shift, so the Newton step from 0 stays below the root.
struct P0Acc {
  float m, sw, sr, cnt, lb;  // shift, sum w~, sum rho, |A(0)|, max w~ (1 - r)
};
__device__ __forceinline__ void p0_init(P0Acc &a) {
  a.m = -INFINITY;
  a.sw = a.sr = a.cnt = a.lb = 0.0f;
}
// Raises the shift to mx (>= a.m) first, then adds the token (s, r).
__device__ __forceinline__ void p0_shift(P0Acc &a, float mx) {
  if (mx > a.m) {
    const float f = expf(a.m - mx);  // 0 while a.m is -inf
    a.sw *= f;
    a.lb *= f;
    a.m = mx;
  }
}
__device__ __forceinline__ void p0_add(P0Acc &a, float s, float r) {
  const float wt = expf(s - a.m);
  a.sw += wt;
  if (wt > 0.0f) {
    a.sr += plan_rho(r);
    a.cnt += 1.0f;
    a.lb = fmaxf(a.lb, wt * (1.0f - r));
  }
}

// The workgroup's pass-0 record of each query head (chunk c): the chunk's
// shift (the largest logit of L) and the sums rescaled to it, combined in a
// fixed order; and the chunk's count of tokens with r == 1.
template <int GRP>
__device__ __forceinline__ void p0_finish(const DParams &p, int b, int g,
                                          int c, P0Acc (&acc)[GRP],
                                          uint32_t n_h) {
  const int np = p.nch + p.nrr;
  const int bg = b * p.G + g;
  constexpr int W = kBlock / kWave;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  // two LDS rounds: the shifts (and the H count), then the sums rescaled to
  // them; each value folded per wave, the waves combined in wave order
  __shared__ float s_mx[W][GRP];
  __shared__ uint32_t s_nh[W];
  __shared__ double s_v[W][4 * GRP];
  float mx[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) mx[h] = wave_fold<float, OpMax<float>>(acc[h].m);
  const uint32_t nhw = wave_fold<uint32_t, OpSum<uint32_t>>(n_h);
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GRP; ++h) s_mx[wave][h] = mx[h];
    s_nh[wave] = nhw;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    float m = s_mx[0][h];
#pragma unroll
    for (int w = 1; w < W; ++w) m = OpMax<float>::f(m, s_mx[w][h]);
    mx[h] = m;
  }
  // (a wave's 64 partial sums folded in fp32, its count as an integer; the
  // waves combined in float64)
  double v[4 * GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const P0Acc &a = acc[h];
    const float f = expf(a.m - mx[h]);  // 0 for a thread without L
    v[4 * h] = (double)wave_fold<float, OpSum<float>>(a.sw * f);
    v[4 * h + 1] = (double)wave_fold<float, OpSum<float>>(a.sr);
    v[4 * h + 2] = (double)wave_fold<uint32_t, OpSum<uint32_t>>((uint32_t)a.cnt);
    v[4 * h + 3] = (double)wave_fold<float, OpMax<float>>(a.lb * f);
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < 4 * GRP; ++k) s_v[wave][k] = v[k];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      double t[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) t[k] = s_v[0][4 * h + k];
#pragma unroll
      for (int w = 1; w < W; ++w) {
#pragma unroll
        for (int k = 0; k < 3; ++k) t[k] = OpSum<double>::f(t[k], s_v[w][4 * h + k]);
        t[3] = OpMax<double>::f(t[3], s_v[w][4 * h + 3]);
      }
      const int row = row_of(p, b, g, h, GRP);
      p.pmax[(size_t)row * np + c] = mx[h];
      double *rec = p.p0part + ((size_t)row * np + c) * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) rec[k] = t[k];
    }
    uint32_t nh = s_nh[0];
#pragma unroll
    for (int w = 1; w < W; ++w) nh += s_nh[w];
    p.hpart[(size_t)bg * np + c] = nh;
  }
}

// Binary shrinkage: scan chunk c of group (b, g) clears its share of the
// group's rows' key-digit histograms (added to by the first beta launch).
template <int GRP>
__device__ __forceinline__ void clear_bin_hist(const DParams &p, int c, int b,
                                               int g) {
  if (p.est != VKV_EST_BINARY) return;
  const int total = GRP * kSelBinsP;
  int lo, hi;
  split_range(total, p.nch, c, lo, hi);
  uint32_t *h0 = p.bhist + (size_t)row_of(p, b, g, 0, GRP) * kSelBinsP;
  for (int t = lo + (int)threadIdx.x; t < hi; t += kBlock) h0[t] = 0u;
}

// Step-start work of scan chunk c of group (b, g): the group's row states
// (chunk 0; no other block of the launch touches them), the status word and
// host byte count (chunk 0 of group 0), and this chunk's share of the
// bitmaps and histograms the later launches fill.
template <int GRP>
__device__ __forceinline__ void scan_setup(const DParams &p, int c, int g,
                                           int b) {
  const int bg = b * p.G + g;
  if (c == 0) {
    for (int h = 0; h < GRP; ++h) {
      const int row = row_of(p, b, g, h, GRP);
      if (threadIdx.x == 0) {
        RowState z{};
        z.amax = -1;
        z.T = ~0ull;
        p.rows[row] = z;
      }
    }
    if (bg == 0 && threadIdx.x == 0) {
      *p.status = 0u;
      *p.host_bytes = 0ull;
    }
  }
  clear_bin_hist<GRP>(p, c, b, g);
  if (p.spec_m > 0) {  // the read-ahead's histogram and slot counter
    int lo, hi;
    split_range(kSpecBins, p.nch, c, lo, hi);
    for (int t = lo + (int)threadIdx.x; t < hi; t += kBlock)
      p.sp_hist[(size_t)bg * kSpecBins + t] = 0u;
    if (c == 0 && threadIdx.x == 0) p.sp_cnt[bg] = 0u;
  }
  if (p.smap_next) {  // this step's staging map starts empty
    const int i1 = min((c + 1) * p.chunk, p.n);
    for (int i = c * p.chunk + (int)threadIdx.x; i < i1; i += kBlock)
      p.smap_next[(size_t)bg * p.ns + i] = -1;
  }
  const int w0 = c * p.chunk / 32, nw = p.chunk / 32;
  for (int w = threadIdx.x; w < nw; w += kBlock) {
    if (w0 + w < p.nwords) {
      p.fbits[(size_t)bg * p.nwords + w0 + w] = 0u;
      if (p.spec_m > 0) p.sp_res[(size_t)bg * p.nwords + w0 + w] = 0u;
      for (int h = 0; h < GRP; ++h)
        p.hbits[(size_t)row_of(p, b, g, h, GRP) * p.nwords + w0 + w] = 0u;
    }
  }
}

template <int GRP, int SD, int UNR>
__device__ __forceinline__ void scan_body(const DParams &p, int c, int g,
                                          int b) {
  // 16 sketch dimensions (32 bytes) per lane: two lanes per token at
  // s = 32, one at s = 16 (fewer cross-lane sums and selects per token than
  // narrower lanes; the FMAs are the same)
  constexpr int DPL = 16;
  constexpr int LPT = SD / DPL;         // lanes per token
  constexpr int TPI = kBlock / LPT;     // tokens per block iteration
  const int bg = b * p.G + g;
  const int lane = threadIdx.x % kWave;
  __shared__ float s_qp[GRP][SD];
  // the chunk's sketch rows and r first, all in flight while q is projected
  const int u = lane % LPT;
  const uint16_t *sk = p.sketch + (size_t)bg * p.ns * SD;
  const float *rr = p.r + (size_t)bg * p.ns;
  const int base = c * p.chunk;
  const int lim = min(base + p.chunk, p.n);
  // sub-batches of SUB tokens, UNR per thread (LPT lanes per token); the
  // next sub-batch is loaded while one is used. Large launches take one
  // token per lane (the registers of a second would cost the launch's
  // resident workgroups a wave per SIMD); a launch of 512-token chunks
  // loads its whole chunk at once (one round trip instead of four)
  constexpr int SUB = UNR * TPI;
  static_assert(kChunk % SUB == 0, "chunk");
  uint4 raw[UNR][2], nraw[UNR][2];
  float rv[UNR], nrv[UNR];
  auto load_sub = [&](int sb, uint4 (&ra)[UNR][2], float (&ro)[UNR]) {
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int i = sb + k * TPI + (int)threadIdx.x / LPT;
      if (i < lim) {
        const uint4 *src = reinterpret_cast<const uint4 *>(sk + (size_t)i * SD + u * DPL);
        ra[k][0] = src[0];
        ra[k][1] = src[1];
        ro[k] = rr[i];
      } else {
        ro[k] = 1.0f;
      }
    }
  };
  load_sub(base, raw, rv);
  scan_setup<GRP>(p, c, g, b);
  // projected, pre-scaled queries: stage q and P_g in LDS, then one output
  // per thread (loaded after the chunk's rows: measured at batch 1, loading
  // them first made the launch 2.5 us longer)
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
  float qv[GRP][DPL];
#pragma unroll
  for (int h = 0; h < GRP; ++h)
#pragma unroll
    for (int k = 0; k < DPL; ++k) qv[h][k] = s_qp[h][u * DPL + k];

  // lane u of a token keeps the heads u, u + LPT, ... (NH of them)
  constexpr int NH = (GRP + LPT - 1) / LPT;
  P0Acc acc[NH];
#pragma unroll
  for (int k = 0; k < NH; ++k) p0_init(acc[k]);
  uint32_t n_h = 0;
  bool bad = false;
  for (int sb = base; sb < lim; sb += SUB) {
    // (a sub-batch that covers the chunk has no next one: no second buffer)
    if (SUB < kChunk && sb + SUB < lim) load_sub(sb + SUB, nraw, nrv);
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int i = sb + k * TPI + (int)threadIdx.x / LPT;
      float f[DPL];
      unpack8(raw[k][0], f);
      unpack8(raw[k][1], f + 8);
      float dot[GRP];
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) a = __builtin_fmaf(qv[h][e], f[e], a);
        dot[h] = group_sum<LPT>(a);
      }
      if (i >= lim) continue;
      const float ri = rv[k];
      if (!(ri > 0.0f && ri <= 1.0f)) bad = true;
      const bool in_l = ri < 1.0f;
      if (u == 0 && !in_l) ++n_h;
#pragma unroll
      for (int kk = 0; kk < NH; ++kk) {
        // this lane's head h = u + LPT kk and its logit
        float val = dot[kk * LPT];
#pragma unroll
        for (int j = 1; j < LPT; ++j)
          if (kk * LPT + j < GRP && u == j) val = dot[kk * LPT + j];
        const int h = u + LPT * kk;
        if (h >= GRP) continue;
        // (non-temporal: the later passes read it from other compute units)
        __builtin_nontemporal_store(val, &p.shat[(size_t)row_of(p, b, g, h, GRP) * p.n + i]);
        if (in_l) {
          p0_shift(acc[kk], val);
          p0_add(acc[kk], val, ri);
        }
      }
    }
    if constexpr (SUB < kChunk) {
#pragma unroll
      for (int k = 0; k < UNR; ++k) {
        raw[k][0] = nraw[k][0];
        raw[k][1] = nraw[k][1];
        rv[k] = nrv[k];
      }
    }
  }
  // each head's accumulator, from the lanes that keep it
  P0Acc hacc[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    p0_init(hacc[h]);
    if (h % LPT == u) hacc[h] = acc[h / LPT];
  }
  const int np = p.nch + p.nrr;
  {
    const int any = __syncthreads_or((int)bad);
    if (threadIdx.x == 0) p.fstat[(size_t)bg * np + c] = any ? VKV_STATUS_BAD_R : 0u;
  }
  p0_finish<GRP>(p, b, g, c, hacc, n_h);
}

// Same outputs with exact keys read from the host cache (perfect sketch).
template <int GRP>
__device__ __forceinline__ void scan_exact_body(const DParams &p, int c,
                                                int g, int b) {
  const int bg = b * p.G + g;
  const int lane = threadIdx.x % kWave;
  scan_setup<GRP>(p, c, g, b);
  const int u = lane % 16;
  float qv[GRP][8];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(
        p.q + (size_t)row_of(p, b, g, h, GRP) * kHeadDim + u * 8);
    unpack8(raw, qv[h]);
  }
  P0Acc acc[GRP];  // lane h keeps head h
#pragma unroll
  for (int h = 0; h < GRP; ++h) p0_init(acc[h]);
  uint32_t n_h = 0;
  bool bad = false;
  const float *rr = p.r + (size_t)bg * p.ns;
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
            p.host_kv + ((size_t)bg * p.ns + i) * 2 * kHeadDim + u * 8);
        float f[8];
        unpack8(raw, f);
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
          float dp = 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) dp = __builtin_fmaf(qv[h][k], f[k], dp);
          dot[h] = group_sum<16>(dp) * kInvSqrtD;
          if (u == h) {
            p0_shift(acc[h], dot[h]);
            p0_add(acc[h], dot[h], ri);
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < GRP; ++h) dot[h] = 0.0f;
      }
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        if (u == h) p.shat[(size_t)row_of(p, b, g, h, GRP) * p.n + i] = dot[h];
      }
    }
  }
  {
    const int any = __syncthreads_or((int)bad);
    if (threadIdx.x == 0)
      p.fstat[(size_t)bg * (p.nch + p.nrr) + c] = any ? VKV_STATUS_BAD_R : 0u;
  }
  p0_finish<GRP>(p, b, g, c, acc, n_h);
}

// ------------------------------------------------------------ dk_resident
// The group's resident rows are split evenly over gridDim.x workgroups.
// Exact logits of the resident rows by matrix cores: per wave, tiles of 16
// rows times the group's query heads (padded to 16 columns) with
// v_mfma_f32_16x16x16_bf16 over eight 16-dimension slices of d. The inputs
// are the bf16 K rows and q as stored, and products of bf16 values are exact
// in fp32, so the logits match a vector dot product up to the order of the
// fp32 additions. The k index of the product is permuted so that each lane
// reads 64 contiguous bytes of its row: lane (g, i) of a wave (g = lane / 16,
// i = lane % 16) loads dimensions 32 g .. 32 g + 31 of row i of the tile, and
// slice c takes dimensions 32 g + 4 c .. 32 g + 4 c + 3 from each lane group;
// q is read with the same permutation. Lane (g, j) then holds the logits of
// rows 4 g .. 4 g + 3 of the tile for query head j.
typedef short vkv_short4 __attribute__((ext_vector_type(4)));
typedef float vkv_float4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ vkv_short4 mfma_slice(const uint4 (&w)[4], int c) {
  // bf16 elements 4c .. 4c + 3 of the lane's 32 (words 2c and 2c + 1)
  const uint32_t *x = reinterpret_cast<const uint32_t *>(w);
  const uint32_t lo = x[2 * c], hi = x[2 * c + 1];
  vkv_short4 r;
  r[0] = (short)(lo & 0xFFFFu);
  r[1] = (short)(lo >> 16);
  r[2] = (short)(hi & 0xFFFFu);
  r[3] = (short)(hi >> 16);
  return r;
}

template <int GRP>
__device__ __forceinline__ void resident_body(const DParams &p, int c, int g,
                                              int b) {
  static_assert(GRP <= 16, "heads per MFMA tile");
  const int bg = b * p.G + g;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int lg = lane / 16, li = lane % 16;  // lane group, row / head index
  __shared__ uint32_t s_ured[kBlock / kWave];
  // B operand: q of head li (zero for the padding columns), permuted slices
  vkv_short4 bq[8];
  {
    uint4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = make_uint4(0u, 0u, 0u, 0u);
    if (li < GRP) {
      const uint4 *src = reinterpret_cast<const uint4 *>(
          p.q + (size_t)row_of(p, b, g, li, GRP) * kHeadDim + 32 * lg);
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = src[k];
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) bq[cc] = mfma_slice(w, cc);
  }
  int cnt = p.rcount[bg];
  bool bad = cnt < 0 || cnt > p.cap;
  cnt = max(0, min(cnt, p.cap));
  const int32_t *ridx = p.ridx + (size_t)bg * p.cap;
  const float *rr = p.r + (size_t)bg * p.ns;
  const int hl = li < GRP ? li : 0;  // this lane's head (lanes li >= GRP idle)
  float mx = -INFINITY, hm = -INFINITY;  // this lane's head: max, H shift
  double hsum = 0.0;
  uint32_t n_h = 0;
  int lo, hi;
  split_range(cnt, p.nrr, c, lo, hi);
  constexpr int WV = kBlock / kWave;
  // Loads are branch-free (indices past the range read its last row; the
  // results for them are never used), so that the loop waits only for what
  // it uses: the K tile one tile ahead, the resident positions two tiles
  // ahead and their r one tile ahead.
  auto load_tile = [&](int t0, uint4 (&w)[4]) {
    const int j = min(t0 + li, hi - 1);
    const uint4 *src = reinterpret_cast<const uint4 *>(
        p.rkv + ((size_t)bg * p.cap + j) * 2 * kHeadDim + 32 * lg);
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = src[k];
  };
  // positions of rows t0 + 4 lg - 1 .. t0 + 4 lg + 3 (the row before first)
  auto load_idx = [&](int t0, int (&pi)[5]) {
#pragma unroll
    for (int u = 0; u < 5; ++u)
      pi[u] = ridx[min(max(t0 + 4 * lg + u - 1, 0), hi - 1)];
  };
  auto load_r = [&](const int (&pi)[5], float (&rk)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) rk[t] = rr[min(max(pi[t + 1], 0), p.n - 1)];
  };
  uint4 cur[4], nxt[4];
  int ia[5], ib[5], ic[5];
  float ra[4], rb[4];
  int t0 = lo + 16 * wave;
  if (t0 < hi) {
    load_tile(t0, cur);
    load_idx(t0, ia);
    load_idx(t0 + 16 * WV, ib);
    load_r(ia, ra);
  }
  for (; t0 < hi; t0 += 16 * WV) {
    load_tile(t0 + 16 * WV, nxt);  // next tile in flight
    load_r(ib, rb);
    load_idx(t0 + 32 * WV, ic);
    // the rows this lane post-processes: 4 lg .. 4 lg + 3 of the tile
    int pos[4];
    bool okr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = t0 + 4 * lg + t;
      pos[t] = ia[t + 1];
      okr[t] = li < GRP && j < hi && pos[t] >= 0 && pos[t] < p.n &&
               (j == 0 || ia[t] < pos[t]);
    }
    vkv_float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mfma_slice(cur, cc), bq[cc],
                                                     acc, 0, 0, 0);
    if (li < GRP) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = t0 + 4 * lg + t;
        if (j >= hi) continue;
        const float dot = acc[t] * kInvSqrtD;
        p.ell[(size_t)row_of(p, b, g, hl, GRP) * p.cap + j] = dot;
        mx = fmaxf(mx, dot);
        const bool in_h = okr[t] && ra[t] >= 1.0f;
        if (in_h) {  // sum over H of exp(l), with a running shift
          if (dot > hm) {
            hsum = hsum * (double)expf(hm - dot) + 1.0;
            hm = dot;
          } else {
            hsum += (double)expf(dot - hm);
          }
        }
        if (li == 0) {
          if (okr[t]) {
            if (in_h) ++n_h;
          } else {
            bad = true;
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) cur[k] = nxt[k];
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      ia[u] = ib[u];
      ib[u] = ic[u];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) ra[t] = rb[t];
  }
  const int np = p.nch + p.nrr;
  {
    const int any = __syncthreads_or((int)bad);
    if (threadIdx.x == 0)
      p.fstat[(size_t)bg * np + p.nch + c] = any ? VKV_STATUS_BAD_RESIDENT : 0u;
  }
  float mxv[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) mxv[h] = (li < GRP && h == hl) ? mx : -INFINITY;
  blk_combine<float, GRP, kBlock, OpMax<float>>(mxv);
  double hsv[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h)
    hsv[h] = (li < GRP && h == hl && hsum > 0.0) ? hsum * (double)expf(hm - mxv[h]) : 0.0;
  blk_reduce<double, GRP, kBlock>(hsv);
  if (threadIdx.x == 0) {
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const int row = row_of(p, b, g, h, GRP);
      p.pmax[(size_t)row * np + p.nch + c] = mxv[h];
      p.hres[(size_t)row * p.nrr + c] = hsv[h];
    }
  }
  const uint32_t th = block_sum<uint32_t>(n_h, s_ured);
  if (threadIdx.x == 0) p.hpart[(size_t)bg * np + p.nch + c] = th;
}

// ------------------------------------------------------------ front launch
// Sketch scan (blockIdx.x < nch) and resident logits (the rest) in one
// launch: they read disjoint inputs and write disjoint outputs.
template <int GRP, int SD, int UNR>
__global__ __launch_bounds__(kBlock) void dk_front(DParams p) {
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (x < p.nch)
    scan_body<GRP, SD, UNR>(p, x, g, b);
  else
    resident_body<GRP>(p, x - p.nch, g, b);
}
template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_front_exact(DParams p) {
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (x < p.nch)
    scan_exact_body<GRP>(p, x, g, b);
  else
    resident_body<GRP>(p, x - p.nch, g, b);
}

// ------------------------------------------------------------ 2-bit sketch
// The pages' deployed sketch ("Verify Before You Fetch", Appendix A.1 and
// section 5.1): 2-bit codes of 32 kept key channels per token, an fp16 zero
// point z and scale s per kept channel and 128-token group. With the query
// entries q_c of the kept channels (scaled by 1/sqrt(d)), the sketch logit
// of token i is A + sum_c code_ic u_c, where A = sum_c q_c z_c and
// u_c = q_c s_c are per group and head. The plan then uses exact logits on
// S and on the shortlist (the n_short tokens of L outside S with the
// largest sketch logit over the group's heads, whose keys are read from
// host memory) and these sketch logits on the rest of L.
constexpr int kSk2Chan = 32;
constexpr int kSk2Group = 128;
constexpr int kSk2Sub = 1024;              // tokens per scan sub-batch
constexpr int kSk2Tok = kSk2Sub / kBlock;  // tokens per thread and sub-batch
constexpr int kShortMax = 1024;            // largest shortlist
constexpr int kShortKPT = 32;              // shortlist keys per thread and tile
constexpr int kShortTile = kShortKPT * kPlanThreads;  // positions per tile
constexpr int kShortSWG = 4;  // workgroups per KV head writing the logits of S

// fp32 -> an unsigned key in the same order (0 is never produced for a
// finite value, so it marks tokens that are not eligible).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Scan workgroup of the 2-bit sketch: the sketch logits of chunk c for the
// group's heads into shat, and each token's shortlist key (the largest of
// them as order_key, 0 for r == 1).
template <int GRP>
__device__ __forceinline__ void scan2_body(const DParams &p, int c, int g,
                                           int b) {
  const int bg = b * p.G + g;
  const int base = c * p.chunk, lim = min(base + p.chunk, p.n);
  const int ngrp = (p.ns + kSk2Group - 1) / kSk2Group;
  __shared__ float s_q[GRP][kSk2Chan];
  __shared__ float s_u[kSk2Sub / kSk2Group][kSk2Chan][GRP];
  __shared__ float s_a[kSk2Sub / kSk2Group][GRP];
  const unsigned long long *codes = p.sk2_codes + (size_t)bg * p.ns;
  const float *rr = p.r + (size_t)bg * p.ns;
  unsigned long long wv[kSk2Tok];
  float rv[kSk2Tok];
  auto load = [&](int sb, unsigned long long (&w)[kSk2Tok], float (&r)[kSk2Tok]) {
#pragma unroll
    for (int k = 0; k < kSk2Tok; ++k) {
      const int i = sb + k * kBlock + (int)threadIdx.x;
      const bool ok = i < lim;
      w[k] = ok ? codes[i] : 0ull;
      r[k] = ok ? rr[i] : 1.0f;
    }
  };
  load(base, wv, rv);  // first sub-batch in flight
  scan_setup<GRP>(p, c, g, b);
  if (threadIdx.x < GRP * kSk2Chan) {
    const int h = threadIdx.x / kSk2Chan, cc = threadIdx.x % kSk2Chan;
    // (a channel outside 0..127 is read as the nearest one)
    const int ch = min(max(p.sk2_chan[(size_t)bg * kSk2Chan + cc], 0), kHeadDim - 1);
    s_q[h][cc] = __uint_as_float(
                     (uint32_t)p.q[(size_t)row_of(p, b, g, h, GRP) * kHeadDim + ch] << 16) *
                 kInvSqrtD;
  }
  bool bad = false;
  for (int sb = base; sb < lim; sb += kSk2Sub) {
    __syncthreads();  // s_q written; the previous sub-batch done with s_u
    const int ng = (min(sb + kSk2Sub, lim) - sb + kSk2Group - 1) / kSk2Group;
    const uint16_t *zs = p.sk2_zs + ((size_t)bg * ngrp + sb / kSk2Group) * 2 * kSk2Chan;
    for (int e = threadIdx.x; e < ng * kSk2Chan * GRP; e += kBlock) {
      const int gi = e / (kSk2Chan * GRP), cc = (e / GRP) % kSk2Chan, h = e % GRP;
      s_u[gi][cc][h] = s_q[h][cc] * half_to_float(zs[gi * 2 * kSk2Chan + kSk2Chan + cc]);
    }
    for (int e = threadIdx.x; e < ng * GRP; e += kBlock) {
      const int gi = e / GRP, h = e % GRP;
      float a = 0.0f;
      for (int cc = 0; cc < kSk2Chan; ++cc)
        a = __builtin_fmaf(s_q[h][cc], half_to_float(zs[gi * 2 * kSk2Chan + cc]), a);
      s_a[gi][h] = a;
    }
    __syncthreads();
    unsigned long long nw[kSk2Tok];
    float nr[kSk2Tok];
    if (sb + kSk2Sub < lim) load(sb + kSk2Sub, nw, nr);  // next in flight
#pragma unroll
    for (int k = 0; k < kSk2Tok; ++k) {
      const int i = sb + k * kBlock + (int)threadIdx.x;
      if (i >= lim) continue;
      const int gi = (k * kBlock + (int)threadIdx.x) / kSk2Group;
      float acc[GRP];
#pragma unroll
      for (int h = 0; h < GRP; ++h) acc[h] = s_a[gi][h];
      const uint32_t lo = (uint32_t)wv[k], hi = (uint32_t)(wv[k] >> 32);
#pragma unroll
      for (int cc = 0; cc < kSk2Chan; ++cc) {
        const uint32_t w = cc < 16 ? lo : hi;
        const float cf = (float)((w >> (2 * (cc & 15))) & 3u);
#pragma unroll
        for (int h = 0; h < GRP; ++h) acc[h] = __builtin_fmaf(cf, s_u[gi][cc][h], acc[h]);
      }
      const float ri = rv[k];
      if (!(ri > 0.0f && ri <= 1.0f)) bad = true;
      float mx = -INFINITY;
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        __builtin_nontemporal_store(acc[h], &p.shat[(size_t)row_of(p, b, g, h, GRP) * p.n + i]);
        mx = fmaxf(mx, acc[h]);
      }
      p.skey[(size_t)bg * p.n + i] = ri < 1.0f ? order_key(mx) : 0u;
    }
#pragma unroll
    for (int k = 0; k < kSk2Tok; ++k) {
      wv[k] = nw[k];
      rv[k] = nr[k];
    }
  }
  const int np = p.nch + p.nrr;
  const int any = __syncthreads_or((int)bad);
  if (threadIdx.x == 0) p.fstat[(size_t)bg * np + c] = any ? VKV_STATUS_BAD_R : 0u;
}

template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_front2(DParams p) {
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (x < p.nch)
    scan2_body<GRP>(p, x, g, b);
  else
    resident_body<GRP>(p, x - p.nch, g, b);
}

// Exclusive prefix sum over the 1024 threads of a row-level workgroup
// (thread order); the total through *total.
__device__ __forceinline__ uint32_t plan_excl_scan(uint32_t v, uint32_t *s_w,
                                                   uint32_t *total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_scan<uint32_t>(v, lane);
  __syncthreads();
  if (lane == kWave - 1) s_w[wave] = incl;
  __syncthreads();
  uint32_t before = 0u, tot = 0u;
  for (int w = 0; w < kPlanWaves; ++w) {
    before += w < wave ? s_w[w] : 0u;
    tot += s_w[w];
  }
  *total = tot;
  return before + incl - v;
}

// Shortlist of one (request, KV head), one 1024-thread workgroup: the
// n_short eligible tokens (L outside S) with the largest keys, equal keys by
// position, found by an 11/11/10-bit radix select over the scan's keys;
// their key rows read from host memory and scored exactly for the group's
// heads, those logits written over the sketch logits. kShortSWG more
// workgroups per KV head write the resident logits over the sketch logits
// of S (disjoint positions).
template <int GRP>
__global__ __launch_bounds__(kPlanThreads) void dk_short(DParams p) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int bg = b * p.G + g, n = p.n, tid = threadIdx.x;
  if (blockIdx.z > 0) {
    // the exact logits of S over the plan's logits: share blockIdx.z - 1 of
    // the resident rows, beside the select (its scattered stores would
    // otherwise follow it on the same compute unit)
    const int cnt = max(0, min(p.rcount[bg], p.cap));
    int j0, j1;
    split_range(cnt, kShortSWG, (int)blockIdx.z - 1, j0, j1);
    const int32_t *ridx = p.ridx + (size_t)bg * p.cap;
    const float *rr = p.r + (size_t)bg * p.ns;
    for (int j = j0 + tid; j < j1; j += kPlanThreads) {
      const int pos = ridx[j];
      if (pos < 0 || pos >= n || !(rr[pos] < 1.0f)) continue;
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        const int row = row_of(p, b, g, h, GRP);
        p.shat[(size_t)row * n + pos] = p.ell[(size_t)row * p.cap + j];
      }
    }
    return;
  }
  const int lane = tid % kWave;
  constexpr int kWords = kMaxTokens / 32;
  __shared__ uint32_t s_res[kWords];  // resident positions
  __shared__ uint32_t s_sel[kWords];  // chosen positions
  __shared__ uint32_t s_eq[kWords];   // positions with key == T (ties only)
  __shared__ uint32_t s_hist[kSelBinsP];
  __shared__ int s_list[kShortMax];
  __shared__ float s_q[GRP][kHeadDim];
  __shared__ uint32_t s_w[kPlanWaves];
  __shared__ uint32_t s_pick[3];
  const int nw = (n + 31) / 32;
  for (int w = tid; w < nw; w += kPlanThreads) {
    s_res[w] = 0u;
    s_sel[w] = 0u;
    s_eq[w] = 0u;
  }
  for (int e = tid; e < GRP * kHeadDim; e += kPlanThreads) {
    const int h = e / kHeadDim, k = e % kHeadDim;
    s_q[h][k] = __uint_as_float(
        (uint32_t)p.q[(size_t)row_of(p, b, g, h, GRP) * kHeadDim + k] << 16);
  }
  __syncthreads();
  const int cnt = max(0, min(p.rcount[bg], p.cap));
  const int32_t *ridx = p.ridx + (size_t)bg * p.cap;
  for (int j = tid; j < cnt; j += kPlanThreads) {
    const int pos = ridx[j];
    if (pos >= 0 && pos < n) atomicOr(&s_res[pos >> 5], 1u << (pos & 31));
  }
  __syncthreads();
  // the keys in tiles of kShortKPT per thread (position tile * kShortTile +
  // k * 1024 + tid), all loads of a tile in flight together; resident
  // positions read as 0 (not eligible). One tile (n <= 32K) stays in
  // registers for every pass.
  const uint32_t *keys = p.skey + (size_t)bg * n;
  const int ntiles = (n + kShortTile - 1) / kShortTile;
  uint32_t kr[kShortKPT];
  auto load_tile = [&](int tile, uint32_t (&kk)[kShortKPT]) {
#pragma unroll
    for (int k = 0; k < kShortKPT; ++k) {
      const int i = tile * kShortTile + k * kPlanThreads + tid;
      kk[k] = i < n ? keys[i] : 0u;
    }
#pragma unroll
    for (int k = 0; k < kShortKPT; ++k) {
      const int i = tile * kShortTile + k * kPlanThreads + tid;
      if (i < n && ((s_res[i >> 5] >> (i & 31)) & 1u)) kk[k] = 0u;
    }
  };
  load_tile(0, kr);
  // fn(position, key) for every position < n
  auto for_keys = [&](auto fn) {
    for (int tile = 0; tile < ntiles; ++tile) {
      uint32_t kt[kShortKPT];
      if (ntiles == 1) {
#pragma unroll
        for (int k = 0; k < kShortKPT; ++k) kt[k] = kr[k];
      } else {
        load_tile(tile, kt);
      }
#pragma unroll
      for (int k = 0; k < kShortKPT; ++k) {
        const int i = tile * kShortTile + k * kPlanThreads + tid;
        if (i < n) fn(i, kt[k]);
      }
    }
  };
  // radix select: the chosen tokens are those with key > T and the first
  // `need` (by position) of the `neq` tokens with key == T
  uint32_t prefix = 0u, mask = 0u, T = 0xFFFFFFFFu, neq = 0u;
  int need = p.n_short;
  if (need > 0) {
    bool all = false;
    for (int lvl = 0; lvl < 3; ++lvl) {
      // key bits [21, 32), then [10, 21), then [0, 10)
      const int sh = lvl == 0 ? 21 : (lvl == 1 ? 10 : 0);
      const int nb = lvl == 2 ? 1 << 10 : 1 << 11;
      for (int e = tid; e < kSelBinsP; e += kPlanThreads) s_hist[e] = 0u;
      __syncthreads();
      for_keys([&](int, uint32_t k) {
        if (k != 0u && (k & mask) == prefix) atomicAdd(&s_hist[(k >> sh) & (nb - 1)], 1u);
      });
      __syncthreads();
      if (tid < kWave) {
        // lane l owns bins [l * per, (l + 1) * per)
        const int per = nb / kWave;
        uint32_t own = 0u;
        for (int e = 0; e < per; ++e) own += s_hist[lane * per + e];
        // inclusive suffix sums over the lanes (keys in this lane's bins and
        // those of higher lanes), by shuffles from above
        uint32_t suf = own;
        for (int o = 1; o < kWave; o <<= 1) {
          const uint32_t v = __shfl_down(suf, o, kWave);
          if (lane + o < kWave) suf += v;
        }
        const uint32_t above = suf - own;
        const uint32_t total = __shfl(suf, 0, kWave);
        if (lvl == 0 && total <= (uint32_t)need) {
          if (lane == 0) {
            s_pick[0] = 0xFFFFFFFFu;  // every eligible token
            s_pick[1] = 0u;
            s_pick[2] = 0u;
          }
        } else if (above < (uint32_t)need && (uint32_t)need <= suf) {
          uint32_t acc = above;
          int bin = lane * per;
          for (int e = per - 1; e >= 0; --e) {
            const uint32_t h = s_hist[lane * per + e];
            if (acc + h >= (uint32_t)need) {
              bin = lane * per + e;
              break;
            }
            acc += h;
          }
          s_pick[0] = (uint32_t)bin;
          s_pick[1] = acc;                  // keys above the bin
          s_pick[2] = s_hist[bin];          // keys in it
        }
      }
      __syncthreads();
      const uint32_t bin = s_pick[0], acc = s_pick[1], inbin = s_pick[2];
      __syncthreads();
      if (bin == 0xFFFFFFFFu) {
        all = true;
        break;
      }
      prefix |= bin << sh;
      mask |= (uint32_t)(nb - 1) << sh;
      need -= (int)acc;
      neq = inbin;  // after the last level: the keys equal to T
    }
    if (all) {
      T = 0u;
      need = 0;
    } else {
      T = prefix;
    }
  }
  // mark the chosen positions; equal keys go to s_eq only when they do not
  // all fit (then by position below)
  const bool ties = need > 0 && neq > (uint32_t)need;
  for_keys([&](int i, uint32_t k) {
    if (k > T || (k == T && k != 0u && need > 0 && !ties))
      atomicOr(&s_sel[i >> 5], 1u << (i & 31));
    else if (ties && k == T)
      atomicOr(&s_eq[i >> 5], 1u << (i & 31));
  });
  __syncthreads();
  // thread t owns words [t * wpt, (t + 1) * wpt): positions in order
  const int wpt = (nw + kPlanThreads - 1) / kPlanThreads;
  const int w0 = min(nw, tid * wpt), w1 = min(nw, w0 + wpt);
  uint32_t tot;
  if (ties) {  // (uniform)
    uint32_t mine = 0u;
    for (int w = w0; w < w1; ++w) mine += (uint32_t)__popc(s_eq[w]);
    uint32_t rank = plan_excl_scan(mine, s_w, &tot);
    for (int w = w0; w < w1; ++w) {
      uint32_t x = s_eq[w], take = 0u;
      while (x) {
        const uint32_t bit = x & (0u - x);
        if (rank++ < (uint32_t)need) take |= bit;
        x &= x - 1u;
      }
      s_sel[w] |= take;  // (this thread's words only)
    }
    __syncthreads();
  }
  uint32_t mine = 0u;
  for (int w = w0; w < w1; ++w) mine += (uint32_t)__popc(s_sel[w]);
  uint32_t ns;
  uint32_t slot = plan_excl_scan(mine, s_w, &ns);
  for (int w = w0; w < w1; ++w) {
    uint32_t x = s_sel[w];
    while (x) {
      const int bit = __ffs(x) - 1;
      if (slot < (uint32_t)kShortMax) s_list[slot] = w * 32 + bit;
      ++slot;
      x &= x - 1u;
    }
  }
  __syncthreads();
  ns = min(ns, (uint32_t)kShortMax);
  if (p.shortlist)
    for (int j = tid; j < p.n_short; j += kPlanThreads)
      p.shortlist[(size_t)bg * p.n_short + j] = j < (int)ns ? s_list[j] : -1;
  if (tid == 0 && ns > 0)
    atomicAdd(p.host_bytes, (unsigned long long)ns * kHeadDim * 2ull);
  // exact logits of the shortlist: 8 threads per token, 16 dimensions each
  const uint16_t *hk = p.host_kv;
  for (int j0 = 0; j0 < (int)ns; j0 += kPlanThreads / 8) {
    const int j = j0 + tid / 8, part = tid % 8;
    const bool ok = j < (int)ns;
    const int pos = ok ? s_list[j] : 0;
    float kf[16];
    {
      uint4 w0 = make_uint4(0u, 0u, 0u, 0u), w1 = w0;
      if (ok) {
        const uint4 *src = reinterpret_cast<const uint4 *>(
            hk + ((size_t)bg * p.ns + pos) * 2 * kHeadDim + part * 16);
        w0 = src[0];
        w1 = src[1];
      }
      unpack8(w0, kf);
      unpack8(w1, kf + 8);
    }
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) a = __builtin_fmaf(s_q[h][part * 16 + e], kf[e], a);
      a = group_sum<8>(a);
      if (ok && part == 0) p.shat[(size_t)row_of(p, b, g, h, GRP) * n + pos] = a * kInvSqrtD;
    }
  }
}

// Pass-0 sums of the beta* iteration for the 2-bit sketch, per scan chunk,
// from the planning logits once S and the shortlist hold exact logits: the
// records the scan itself writes in the other modes.
template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_p0(DParams p) {
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * p.G + g;
  const int base = c * p.chunk, lim = min(base + p.chunk, p.n);
  const float *rr = p.r + (size_t)bg * p.ns;
  P0Acc acc[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) p0_init(acc[h]);
  uint32_t n_h = 0u;
  constexpr int U = 4;
  for (int i0 = base + (int)threadIdx.x; i0 < lim; i0 += kBlock * U) {
    float rv[U], sv[U][GRP];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kBlock;
      const bool ok = i < lim;
      rv[u] = ok ? rr[i] : 1.0f;
#pragma unroll
      for (int h = 0; h < GRP; ++h)
        sv[u][h] = ok ? p.shat[(size_t)row_of(p, b, g, h, GRP) * p.n + i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u * kBlock >= lim) continue;
      if (!(rv[u] < 1.0f)) {
        ++n_h;
        continue;
      }
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        p0_shift(acc[h], sv[u][h]);
        p0_add(acc[h], sv[u][h], rv[u]);
      }
    }
  }
  p0_finish<GRP>(p, b, g, c, acc, n_h);
}

// ------------------------------------------------------------ planning
// The plan of Algorithm 2 for every (request, query head) ("row"):
//   D~ -> beta* -> certificate (Lemma 1, eq. 7) -> k* (eq. 10) -> F_h.
// Data-parallel passes over a row's tokens run as launches of kBlock-thread
// workgroups, one per chunk of kRowChunk tokens of a row; each writes a
// partial record, and every workgroup of the next launch combines the
// records of its row itself (in one fixed order, so all of them get
// bit-identical results). No workgroup ever waits for another.
//
// beta*: at the root, beta* >= max_i w~_i (1 - r_i) (below that the heaviest
// token alone would give more than beta), so every token is at or above its
// lower clip and the Definition 2 fixed point is also the unique root of
//     h(beta) = sum_i max(0, w~_i - beta rho_i) - beta,  rho_i = r_i/(1-r_i),
// a convex, decreasing, piecewise-linear function. Pass 0 gives the sums at
// beta = 0 and the lower bound above; each later pass evaluates, at
// kBetaPts points of the bracket [lo, hi], the sums of w~ and rho over the
// active set A(beta) = {w~_i > beta rho_i} and its size. The Newton step
// from a point with h >= 0, beta' = sum_A w~ / (1 + sum_A rho), never
// overshoots the root (convexity); it is the root itself when no breakpoint
// lies between the point and the next evaluated point (equal active counts)
// or when the next pass finds the same active set at beta'. Since h' <= -1,
// beta + h(beta) bounds the root from above. A row still open after the
// last Newton launch finishes in the certificate launch, where each of its
// workgroups iterates over the whole row (rare; same arithmetic).
//
// Selection: keys (gain bits, inverted position) order L as L_g
// (descending). Each of nsel workgroups per row takes a block-cyclic share of the row's tokens and writes its keys at or
// above a local bound lo_s (at most kCandMax / nsel of them, the top
// quarter first) with their w~ and r; the terms of Lemma 1 are recomputed
// from those. One workgroup per row then runs the stopping rule on the
// union to the exact k* and threshold T; that is the answer whenever T >=
// max_s lo_s (every key >= T was written). Otherwise, or when fetching every
// candidate cannot certify the row, it runs the streaming selection below
// instead. The stopping decisions use fixed-point integer sums of capped
// terms (sat_fx), so a rest's sum is the total minus the fetched part
// exactly; the reported eps^(L') is formed from float64 sums over the rest
// itself, which keep their relative accuracy however small the rest is.
constexpr int kSelUnroll = 4;       // streamed tokens per thread in flight
constexpr int kBetaPts = 4;         // points of h per Newton pass
constexpr int kBetaRec = 3 * kBetaPts + 1;  // + the band count
constexpr int kBetaLaunchMax = 4;   // Newton passes (pass 0 is in the scan):
                                    // p.nbeta of them, 2 to 4
constexpr int kBandChunk = 1024;    // band tokens a chunk may store
constexpr int kBandMax = 2048;      // band tokens a row may be settled from
constexpr int kBandWave = 512;      // ... by one wave; the whole workgroup above
constexpr int kMaxChunks = kMaxTokens / kRowChunk;
constexpr int kBetaPassMax = 96;    // never reached: the bracket shrinks >= 2x
constexpr int kCandMax = 8192;      // candidates held by the walk
constexpr int kSelLevels = 5;       // five 11-bit digits cover the 55-bit key
constexpr unsigned long long kKeyEnd = 1ull << 55;  // above every key
__device__ __forceinline__ int sel_off(int d) { return 44 - kSelDigit * d; }

// LDS of the streaming selection: the count histogram, then the collected
// candidates.
union SelLds {
  uint32_t hist[kSelBinsP];
  struct {
    unsigned long long key[kCand];
    unsigned long long bfx[kCand];
    unsigned long long vfx[kCand];
    uint32_t rb[kCand];
  } cand;
};

// Selection (eq. 10) and marking of F_h minus S for one row by one
// 1024-thread workgroup that streams the row itself, with no limit on how
// many tokens are fetched. It is the fallback of the candidate walk, taken
// when the collected candidates cannot certify the row; `rs` (LDS) holds the
// row's certificate and receives k*, T and eps^(L').
// The parameters the streaming selection reads, passed by value: a
// reference to the kernel's parameter block would make the caller copy all
// of it to scratch memory.
struct SelArgs {
  const float *r, *shat;
  const uint32_t *resbits;  // the KV head's resident bitmap (in LDS)
  uint32_t *fbits, *hbits;
  double a_delta, l_delta;
  float eps;
  int n, ns, nwords, est;  // (ns: positions per KV head in r)
};

__device__ __forceinline__ void select_row(const SelArgs p, int row,
                                                     int bg, RowState &rs,
                                                     SelLds &lds) {
  const int n = p.n;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  __shared__ unsigned long long s_u[kPlanWaves * 4 + 4];
  __shared__ uint32_t s_m[kPlanWaves];
  __shared__ uint32_t s_cnt;
  __shared__ unsigned long long s_lo;  // the resolved lower key bound
  __shared__ int s_more;               // another count level is needed
  __shared__ int s_j[kPlanWaves];
  const float *rr = p.r + (size_t)bg * p.ns;
  const float *sh = p.shat + (size_t)row * n;
  const float m = rs.m;
  const LamRule lr = lam_rule((float)rs.beta, p.est, rs.bkey);
  const float af = (float)p.a_delta, lf = (float)p.l_delta;
  const double a = p.a_delta, l = p.l_delta;
  const int eb = rs.eb, ev = rs.ev;
  const double capb = rs.capb, capv = rs.capv;
  const double sbs = ldexp(1.0, -eb), svs = ldexp(1.0, -ev);
  const uint32_t *rbits = p.resbits;
  uint32_t *fb = p.fbits + (size_t)bg * p.nwords;
  uint32_t *hb = p.hbits + (size_t)row * p.nwords;

  // One pass over L with every lane active: g(i, valid, key, terms).
  auto stream = [&](auto &&g) {
    for (int base = 0; base < n; base += kSelUnroll * kPlanThreads) {
      float r8[kSelUnroll], s8[kSelUnroll];
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) {
        const int i = base + u * kPlanThreads + (int)threadIdx.x;
        r8[u] = i < n ? rr[i] : 1.0f;
        s8[u] = i < n ? sh[i] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) {
        const int i = base + u * kPlanThreads + (int)threadIdx.x;
        const bool valid = r8[u] < 1.0f;
        Terms t{};
        unsigned long long key = 0ull;
        if (valid) {
          t = token_terms_w(expf(s8[u] - m), r8[u], lr, i);
          key = make_key(token_gain(t, i, rs, af, lf), i);
        }
        g(i, valid, key, t);
      }
    }
  };

  // totals over L (first count pass), and what has been fetched so far
  unsigned long long tot_b = 0ull, tot_v = 0ull;
  unsigned long long fet_b = 0ull, fet_v = 0ull;
  uint32_t fet_c = 0u;
  unsigned long long hi_key = kKeyEnd;
  bool first = true;
  // every round fetches at least one more token, so |L| + 1 rounds suffice
  for (int round = 0; round <= n; ++round) {
    // ---- count levels: lo with |[lo, hi_key)| <= kCand, as large as useful
    unsigned long long pre = 0ull;
    uint32_t base_cnt = 0u;
    for (int d = 0; d < kSelLevels; ++d) {
      const int off = sel_off(d);
      for (int i = threadIdx.x; i < kSelBinsP; i += kPlanThreads) lds.hist[i] = 0u;
      __syncthreads();
      unsigned long long lb_ = 0ull, lv_ = 0ull;
      stream([&](int, bool valid, unsigned long long key, const Terms &t) {
        if (!valid) return;
        if (first && d == 0) {
          lb_ += sat_fx(t.bi, capb, eb);
          lv_ += sat_fx(t.vi, capv, ev);
        }
        if (key >= hi_key || (key >> (off + kSelDigit)) != pre) return;
        atomicAdd(&lds.hist[(int)((key >> off) & (kSelBinsP - 1))], 1u);
      });
      if (first && d == 0) {
        unsigned long long tv2[2] = {lb_, lv_};
        plan_reduce<unsigned long long, 2>(tv2);
        tot_b = tv2[0];
        tot_v = tv2[1];
      }
      __syncthreads();
      if (wave == 0) {
        // lane owns bins [lane * 32, lane * 32 + 32); c_ge(j) = keys in bins >= j
        constexpr int PER = kSelBinsP / kWave;
        uint32_t lc = 0u;
        for (int k = 0; k < PER; ++k) lc += lds.hist[lane * PER + k];
        const uint32_t incl = wave_incl_scan<uint32_t>(lc, lane);
        const uint32_t above = __shfl(incl, kWave - 1, kWave) - incl;
        const uint32_t budget = (uint32_t)kCand - base_cnt;
        int j0 = kSelBinsP;  // smallest bin whose suffix fits
        uint32_t c = above;
        if (c <= budget) {
          for (int k = PER - 1; k >= 0; --k) {
            const uint32_t c2 = c + lds.hist[lane * PER + k];
            if (c2 > budget) break;
            c = c2;
            j0 = lane * PER + k;
          }
        }
        int jm = j0;
        for (int s2 = 32; s2 >= 1; s2 >>= 1) jm = min(jm, __shfl_xor(jm, s2, kWave));
        // keys in bins >= jm
        uint32_t take = 0u;
        if (jm < kSelBinsP && lane == jm / PER) {
          take = above;
          for (int k = PER - 1; k >= jm % PER; --k) take += lds.hist[lane * PER + k];
        }
        take = wave_sum(take) + base_cnt;
        if (lane == 0) {
          const unsigned long long bin_lo =
              ((pre << kSelDigit) | (unsigned long long)min(jm, kSelBinsP - 1)) << off;
          const unsigned long long top = (pre + 1ull) << (off + kSelDigit);
          if (jm == 0) {
            s_lo = pre << (off + kSelDigit);
            s_more = 0;
          } else if (d == kSelLevels - 1 || take >= (uint32_t)kCand / 2) {
            s_lo = jm == kSelBinsP ? top : bin_lo;
            s_more = 0;
          } else {
            // refine the bin just below: it alone would overflow the budget
            s_lo = (pre << kSelDigit) | (unsigned long long)(jm - 1);
            s_j[0] = (int)take;
            s_more = 1;
          }
        }
      }
      __syncthreads();
      if (!s_more) break;
      pre = s_lo;
      base_cnt = (uint32_t)s_j[0];
      __syncthreads();
    }
    first = false;
    const unsigned long long lo_key = s_lo;

    // ---- collect [lo_key, hi_key); max of b_i below lo_key
    if (threadIdx.x == 0) s_cnt = 0u;
    __syncthreads();
    uint32_t below_max = 0u;
    unsigned long long cb_ = 0ull, cv_ = 0ull;
    stream([&](int, bool valid, unsigned long long key, const Terms &t) {
      const bool sel = valid && key >= lo_key && key < hi_key;
      if (valid && key < lo_key) below_max = max(below_max, __float_as_uint(t.rb));
      const unsigned long long msk = __ballot(sel);
      if (msk == 0ull) return;
      const int leader = __ffsll((long long)msk) - 1;
      uint32_t slot0 = 0u;
      if (lane == leader) slot0 = atomicAdd(&s_cnt, (uint32_t)__popcll(msk));
      slot0 = __shfl(slot0, leader, kWave);
      if (sel) {
        const uint32_t slot =
            slot0 + (uint32_t)__popcll(msk & ((1ull << lane) - 1ull));
        const unsigned long long bx = sat_fx(t.bi, capb, eb),
                                 vx = sat_fx(t.vi, capv, ev);
        cb_ += bx;
        cv_ += vx;
        if (slot < (uint32_t)kCand) {
          lds.cand.key[slot] = key;
          lds.cand.bfx[slot] = bx;
          lds.cand.vfx[slot] = vx;
          lds.cand.rb[slot] = __float_as_uint(t.rb);
        }
      }
    });
    unsigned long long cs[2] = {cb_, cv_};
    plan_reduce<unsigned long long, 2>(cs);
    below_max = plan_max<uint32_t>(below_max);
    const int nc = (int)min(s_cnt, (uint32_t)kCand);
    const double e_below =
        eps_of((double)(tot_b - fet_b - cs[0]) * sbs,
               (double)(tot_v - fet_v - cs[1]) * svs,
               (double)__uint_as_float(below_max), rs.dnorm, a, l);
    if (!(e_below < (double)p.eps) && lo_key > 0ull) {
      // not enough: every candidate is fetched, the region moves below
      for (int c = threadIdx.x; c < nc; c += kPlanThreads) {
        const int pos = (int)(0xFFFFFFu - (uint32_t)(lds.cand.key[c] & 0xFFFFFFull));
        atomicOr(hb + pos / 32, 1u << (pos % 32));
        if (!((rbits[pos / 32] >> (pos % 32)) & 1u)) atomicOr(fb + pos / 32, 1u << (pos % 32));
      }
      fet_c += (uint32_t)nc;
      fet_b += cs[0];
      fet_v += cs[1];
      hi_key = lo_key;
      __syncthreads();
      continue;
    }

    // ---- rank sort of the candidates by key, descending (keys are unique)
    constexpr int PT = kCand / kPlanThreads;
    unsigned long long mk[PT], mb[PT], mv[PT];
    uint32_t mr[PT];
    int rank[PT];
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int c = threadIdx.x + q * kPlanThreads;
      rank[q] = -1;
      if (c < nc) {
        mk[q] = lds.cand.key[c];
        mb[q] = lds.cand.bfx[c];
        mv[q] = lds.cand.vfx[c];
        mr[q] = lds.cand.rb[c];
        int rk = 0;
        for (int o = 0; o < nc; ++o) rk += lds.cand.key[o] > mk[q] ? 1 : 0;
        rank[q] = rk;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      if (rank[q] >= 0) {
        lds.cand.key[rank[q]] = mk[q];
        lds.cand.bfx[rank[q]] = mb[q];
        lds.cand.vfx[rank[q]] = mv[q];
        lds.cand.rb[rank[q]] = mr[q];
      }
    }
    __syncthreads();

    // ---- walk: fetching sorted candidates 0..k (k = 0..nc-1); each thread
    // owns PT consecutive positions
    const int k0 = threadIdx.x * PT;
    unsigned long long lb2 = 0ull, lv2 = 0ull;
    uint32_t lmax = 0u;
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      if (k0 + q < nc) {
        lb2 += lds.cand.bfx[k0 + q];
        lv2 += lds.cand.vfx[k0 + q];
        lmax = max(lmax, lds.cand.rb[k0 + q]);
      }
    }
    // exclusive prefix sums over threads, max of b_i over later threads
    const unsigned long long ib = wave_incl_scan<unsigned long long>(lb2, lane);
    const unsigned long long iv = wave_incl_scan<unsigned long long>(lv2, lane);
    uint32_t rmax = lmax;  // suffix max over this lane and the lanes above
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t v = __shfl_down(rmax, o, kWave);
      if (lane + o < kWave) rmax = max(rmax, v);
    }
    uint32_t after = __shfl_down(rmax, 1, kWave);
    if (lane == kWave - 1) after = 0u;
    __syncthreads();
    if (lane == kWave - 1) {
      s_u[2 * wave] = ib;
      s_u[2 * wave + 1] = iv;
    }
    if (lane == 0) s_m[wave] = rmax;
    __syncthreads();
    unsigned long long base_b = 0ull, base_v = 0ull;
    for (int w = 0; w < kPlanWaves; ++w) {
      if (w < wave) {
        base_b += s_u[2 * w];
        base_v += s_u[2 * w + 1];
      }
      if (w > wave) after = max(after, s_m[w]);
    }
    after = max(after, below_max);
    unsigned long long cb = base_b + ib - lb2, cvv = base_v + iv - lv2;
    int best = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int k = k0 + q;
      if (k >= nc || best != 0x7fffffff) continue;
      cb += lds.cand.bfx[k];
      cvv += lds.cand.vfx[k];
      uint32_t bt = after;
      for (int q2 = q + 1; q2 < PT; ++q2)
        if (k0 + q2 < nc) bt = max(bt, lds.cand.rb[k0 + q2]);
      const double e = eps_of((double)(tot_b - fet_b - cb) * sbs,
                              (double)(tot_v - fet_v - cvv) * svs,
                              (double)__uint_as_float(bt), rs.dnorm, a, l);
      if (e < (double)p.eps) {
        best = k;
      }
    }
    int first_k = best;
    first_k = -plan_max<int>(-first_k);
    // (fetching every candidate certifies, so first_k < nc; the guard keeps
    // the state sane if rounding ever said otherwise)
    const int kk = first_k < nc ? first_k : nc - 1;
    if (best == first_k && best != 0x7fffffff) {
      rs.kstar = (int)(fet_c + (uint32_t)best + 1u);
      rs.T = lds.cand.key[best];
    }
    __syncthreads();
    if (threadIdx.x == 0 && first_k >= nc) {
      rs.kstar = (int)(fet_c + (uint32_t)nc);
      rs.T = nc > 0 ? lds.cand.key[nc - 1] : (hi_key == kKeyEnd ? ~0ull : hi_key);
    }
    // mark the fetched candidates
    for (int c = threadIdx.x; c <= kk; c += kPlanThreads) {
      const int pos = (int)(0xFFFFFFu - (uint32_t)(lds.cand.key[c] & 0xFFFFFFull));
      atomicOr(hb + pos / 32, 1u << (pos % 32));
      if (!((rbits[pos / 32] >> (pos % 32)) & 1u)) atomicOr(fb + pos / 32, 1u << (pos % 32));
    }
    __syncthreads();
    break;
  }
  // eps^(L') from float64 sums over the rest (every token below T), added
  // directly rather than as the total minus the fetched part
  const unsigned long long T = rs.T;
  double dr[2] = {0.0, 0.0};
  uint32_t bm = 0u;
  stream([&](int, bool valid, unsigned long long key, const Terms &t) {
    if (!valid || key >= T) return;
    double bd, vd;
    direct_terms(t, bd, vd);
    dr[0] += bd;
    dr[1] += vd;
    bm = max(bm, __float_as_uint(t.rb));
  });
  plan_reduce<double, 2>(dr);
  bm = plan_max<uint32_t>(bm);
  if (threadIdx.x == 0)
    rs.eps1 = (float)eps_of(dr[0], dr[1], (double)__uint_as_float(bm), rs.dnorm,
                            a, l);
  __syncthreads();
}

// ------------------------------------------------------------ row passes
// This thread's tokens of chunk c of a row: r and the planning logit s (r = 1
// past n). Token u is c * kRowChunk + u * kBlock + tid. The kernels issue
// these loads first and their other loads right after, so that they wait
// for memory once.
__device__ __forceinline__ void row_load(const DParams &p, int row, int bg,
                                         int c, float (&r8)[kRowTok],
                                         float (&s8)[kRowTok]) {
  const float *rr = p.r + (size_t)bg * p.ns;
  const float *sh = p.shat + (size_t)row * p.n;
#pragma unroll
  for (int u = 0; u < kRowTok; ++u) {
    const int i = c * kRowChunk + u * kBlock + (int)threadIdx.x;
    r8[u] = i < p.n ? rr[i] : 1.0f;
    s8[u] = i < p.n ? sh[i] : 0.0f;
  }
}
// w~ = exp(s - m) on L, 0 elsewhere.
__device__ __forceinline__ void row_weights(float m, const float (&r8)[kRowTok],
                                            const float (&s8)[kRowTok],
                                            float (&w8)[kRowTok]) {
#pragma unroll
  for (int u = 0; u < kRowTok; ++u) w8[u] = r8[u] < 1.0f ? expf(s8[u] - m) : 0.0f;
}
__device__ __forceinline__ int row_pos(int c, int u) {
  return c * kRowChunk + u * kBlock + (int)threadIdx.x;
}

// Points of h evaluated by a Newton pass: lo and three points geometrically
// closer to it than to hi (Newton usually lands just below the root).
__device__ __forceinline__ void beta_points(const BetaState &st,
                                            double (&pts)[kBetaPts]) {
  const double span = st.hi - st.lo;
  pts[0] = st.lo;
  pts[1] = st.lo + span * 0x1p-6;
  pts[2] = st.lo + span * 0x1p-3;
  pts[3] = st.lo + span * 0.5;
}

// State after pass 0 from its totals {sum_L w~, sum rho over w~ > 0, |A(0)|,
// max w~(1 - r), sum_H w}.
__device__ __forceinline__ BetaState beta_init(const double (&v)[kBetaRec],
                                               int est) {
  BetaState st{};
  st.dnorm = v[0] + v[4];
  if (est != VKV_EST_CLIP || !(v[2] > 0.0)) {
    st.done = 1;
    return st;
  }
  // (w~(1 - r) was rounded once in fp32: step below it to stay a bound)
  const double lb = v[3] * (1.0 - 0x1p-22);
  const double nx = v[0] / (1.0 + v[1]);
  st.lo = fmax(nx, lb);
  st.hi = v[0];
  st.prev_cnt = st.lo == nx ? v[2] : -1.0;  // |A| whose Newton step gave lo
  st.beta = st.lo;
  if (!(st.hi > st.lo)) st.done = 1;
  return st;
}

// One bracketed Newton step from the sums v at the points of `st` (per
// point: sum w~, sum rho, |A|).
__device__ __forceinline__ BetaState beta_advance(BetaState st,
                                                  const double (&v)[kBetaRec]) {
  double pts[kBetaPts];
  beta_points(st, pts);
  if (v[2] == st.prev_cnt) {  // the set that produced lo is active at lo
    st.beta = st.lo;
    st.done = 1;
    return st;
  }
  int jl = -1;
#pragma unroll
  for (int j = 0; j < kBetaPts; ++j)
    if (v[3 * j] - pts[j] * (1.0 + v[3 * j + 1]) >= 0.0) jl = j;
  if (jl < 0) {  // h(lo) < 0 only by rounding: the step from lo is the root
    st.beta = v[0] / (1.0 + v[1]);
    st.done = 1;
    return st;
  }
  // the point jl and the next one, selected by unrolled compares (an index
  // computed at run time would put the arrays in scratch memory)
  double sw = 0.0, sr = 0.0, c = 0.0, pl = 0.0, pn = 0.0, cn = 0.0;
  bool next = false;
#pragma unroll
  for (int j = 0; j < kBetaPts; ++j) {
    if (j == jl) {
      sw = v[3 * j];
      sr = v[3 * j + 1];
      c = v[3 * j + 2];
      pl = pts[j];
    }
    if (j == jl + 1) {
      cn = v[3 * j + 2];
      pn = pts[j];
      next = true;
    }
  }
  const double nb = sw / (1.0 + sr);
  if (next && cn == c) {  // h linear up to there
    st.beta = nb;
    st.done = 1;
    return st;
  }
  double nhi = fmin(st.hi, pl + (sw - pl * (1.0 + sr)));
  if (next) nhi = fmin(nhi, pn);
  st.lo = fmax(nb, pl);
  st.hi = nhi;
  st.prev_cnt = c;
  st.beta = st.lo;
  if (!(st.hi > st.lo)) st.done = 1;
  return st;
}

// Adds token (w~, r)'s terms at the points to v.
__device__ __forceinline__ void beta_accumulate(const double (&pts)[kBetaPts],
                                                float wt, float ri,
                                                double (&v)[kBetaRec]) {
  if (!(wt > 0.0f)) return;
  const double w = (double)wt, rh = (double)plan_rho(ri);
#pragma unroll
  for (int j = 0; j < kBetaPts; ++j) {
    if (w - pts[j] * rh > 0.0) {
      v[3 * j] += w;
      v[3 * j + 1] += rh;
      v[3 * j + 2] += 1.0;
    }
  }
}

// The per-chunk band counts of the records last loaded (LDS).
__device__ __forceinline__ int *band_counts() {
  __shared__ int s_cnt[kMaxChunks];
  return s_cnt;
}
// Wave-level totals: every wave folds its lanes' shares by DPP on its own.
// With shares taken by lane (records lane, lane + 64, ... in order) every
// wave, and every workgroup of the row, gets the same bits without a
// workgroup barrier.
template <bool LB>
__device__ __forceinline__ void beta_rec_fold(double (&v)[kBetaRec]) {
  // (pass 0's records fill slots 0-4 only; the rest stay 0)
  constexpr int N = LB ? 5 : kBetaRec;
#pragma unroll
  for (int k = 0; k < N; ++k)
    v[k] = (LB && k == 3) ? wave_fold<double, OpMax<double>>(v[k])
                          : wave_fold<double, OpSum<double>>(v[k]);
}
// A row's S <= 64 chunk records combined by every wave (see beta_rec_fold);
// the first wave also keeps the per-chunk band counts in LDS.
__device__ __forceinline__ void beta_rec_wave(const double *rec, int S,
                                              double (&v)[kBetaRec]) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int k = 0; k < kBetaRec; ++k) v[k] = 0.0;
  for (int t = lane; t < S; t += kWave) {
#pragma unroll
    for (int k = 0; k < kBetaRec; ++k) v[k] += rec[(size_t)t * kBetaRec + k];
    if (threadIdx.x < kWave)
      band_counts()[t] = (int)rec[(size_t)t * kBetaRec + kBetaRec - 1];
  }
  beta_rec_fold<false>(v);
}

// The row's common shift m = max(max_R l, max_L s) and the pass-0 sums
// rescaled to it, as this lane's share (beta_rec_fold totals them): slots
// 0-2 sum_L w~, sum rho over
// w~ > 0 and their count, slot 3 max w~ (1 - r) (combined by maximum), slot
// 4 sum_H w. Workgroup 0 of the row stores m; with `check`, it also checks
// that every token with r == 1 of the KV head is resident.
__device__ __forceinline__ float row_pass0(const DParams &p, int row, int bg,
                                           int c, bool check,
                                           double (&v)[kBetaRec]) {
  const int np = p.nch + p.nrr;
  const int lane = threadIdx.x % kWave;
  // (every wave on its own: lane-strided shares folded by DPP; the first
  // kPre shares of each lane, records included, loaded before any is used)
  constexpr int kPre = 2;
  float pmv[kPre];
  double rc[kPre][4];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int t = lane + k * kWave;
    pmv[k] = t < np ? p.pmax[(size_t)row * np + t] : -INFINITY;
    const double *rec = p.p0part + ((size_t)row * np + t) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) rc[k][e] = t < p.nch ? rec[e] : 0.0;
  }
  float pm = -INFINITY;
#pragma unroll
  for (int k = 0; k < kPre; ++k) pm = fmaxf(pm, pmv[k]);
  for (int t = lane + kPre * kWave; t < np; t += kWave)
    pm = fmaxf(pm, p.pmax[(size_t)row * np + t]);
  const float m = wave_fold<float, OpMax<float>>(pm);
#pragma unroll
  for (int k = 0; k < kBetaRec; ++k) v[k] = 0.0;
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    if (!(lane + k * kWave < p.nch) || !(rc[k][0] > 0.0)) continue;
    const double f = exp((double)pmv[k] - (double)m);
    v[0] += rc[k][0] * f;
    v[1] += rc[k][1];
    v[2] += rc[k][2];
    v[3] = fmax(v[3], rc[k][3] * f);
  }
  for (int t = lane + kPre * kWave; t < p.nch; t += kWave) {
    const double *rec = p.p0part + ((size_t)row * np + t) * 4;
    if (!(rec[0] > 0.0)) continue;
    const double f = exp((double)p.pmax[(size_t)row * np + t] - (double)m);
    v[0] += rec[0] * f;
    v[1] += rec[1];
    v[2] += rec[2];
    v[3] = fmax(v[3], rec[3] * f);
  }
  for (int t = lane; t < p.nrr; t += kWave) {
    const double hs = p.hres[(size_t)row * p.nrr + t];
    if (hs > 0.0) v[4] += hs * exp((double)p.pmax[(size_t)row * np + p.nch + t] - (double)m);
  }
  if (c == 0) {
    if (threadIdx.x == 0) p.rows[row].m = m;
    if (check && threadIdx.x < kWave) {
      // the front launch's input checks (its workgroups cannot touch the
      // status word, which that launch clears), and the H counts: tokens
      // with r == 1, all of them and the resident ones; by the first wave
      // alone (lane-strided shares folded by DPP, no workgroup barrier)
      uint32_t hc0 = 0u, hc1 = 0u, fr = 0u, fh = 0u;
      for (int t = lane; t < np; t += kWave) {
        const uint32_t hv = p.hpart[(size_t)bg * np + t];
        const uint32_t fv = p.fstat[(size_t)bg * np + t];
        if (t < p.nch) hc0 += hv;
        else hc1 += hv;
        fr = OpMax<uint32_t>::f(fr, (fv & VKV_STATUS_BAD_R) ? 1u : 0u);
        fh = OpMax<uint32_t>::f(fh, (fv & VKV_STATUS_BAD_RESIDENT) ? 1u : 0u);
      }
      hc0 = wave_fold<uint32_t, OpSum<uint32_t>>(hc0);
      hc1 = wave_fold<uint32_t, OpSum<uint32_t>>(hc1);
      fr = wave_fold<uint32_t, OpMax<uint32_t>>(fr);
      fh = wave_fold<uint32_t, OpMax<uint32_t>>(fh);
      uint32_t bits = 0u;
      if (fr) bits |= VKV_STATUS_BAD_R;
      if (fh || hc0 != hc1) bits |= VKV_STATUS_BAD_RESIDENT;
      if (threadIdx.x == 0 && bits) atomicOr(p.status, bits);
    }
  }
  return m;
}

// The band of a bracket [lo, hi]: the tokens active at lo and not at hi,
// the only ones whose share of h can change inside it. Each pass stores its
// workgroup's band (when it fits) in a fixed order and counts it in the
// record.
__device__ __forceinline__ bool in_band(const BetaState &st, float wt, float ri) {
  if (!(wt > 0.0f)) return false;
  const double w = (double)wt, rh = (double)plan_rho(ri);
  return w - st.lo * rh > 0.0 && !(w - st.hi * rh > 0.0);
}
// The state after a pass whose combined records are v: one bracketed Newton
// step; then, when the pass's band was small enough to keep, the iteration
// goes on over the band alone in LDS (the tokens outside it have the same
// status at every point of the new, narrower bracket: their sums are those
// at lo minus the band's), to the root. Every workgroup of the row gets the
// same state (same data, same order).
__device__ __forceinline__ BetaState beta_settle(const DParams &p, BetaState st,
                                                 const double (&v)[kBetaRec],
                                                 int row, int parity) {
  __shared__ float s_bw[kBandMax], s_br[kBandMax];
  __shared__ int s_bo[kMaxChunks + 1];
  __shared__ int s_bok;
  st = beta_advance(st, v);
  if (st.done || !(v[kBetaRec - 1] <= (double)kBandMax)) return st;
  const size_t rows = (size_t)p.B * p.Hq;
  const float2 *band = p.band + ((size_t)parity * rows + row) * p.nrc * kBandChunk;
  if (threadIdx.x < kWave) {  // one wave: nrc <= 64 chunk counts
    const int t = threadIdx.x;
    const int k = t < p.nrc ? band_counts()[t] : 0;
    const int incl = wave_incl_scan<int>(k, t);
    // a chunk over its capacity stored nothing
    const int bad = wave_max<int>(k > kBandChunk ? 1 : 0);
    if (t < p.nrc) s_bo[t] = incl - k;
    if (t == kWave - 1) {
      s_bo[p.nrc] = incl;
      s_bok = !bad;
    }
  }
  __syncthreads();
  if (!s_bok) return st;
  const int nb = s_bo[p.nrc];
  for (int k = threadIdx.x; k < nb; k += kBlock) {
    int lo = 0, hi = p.nrc;  // the chunk holding entry k
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (s_bo[mid] <= k) lo = mid; else hi = mid;
    }
    const float2 e = band[(size_t)lo * kBandChunk + (k - s_bo[lo])];
    s_bw[k] = e.x;
    s_br[k] = e.y;
  }
  __syncthreads();
  if (nb > kBandWave) {
    // a large band: the Newton steps by the whole workgroup, per-thread sums
    // over a share of the band folded per wave and combined across the
    // waves in wave order (every thread gets the same sums and takes the
    // same steps)
    double bs[3] = {0.0, 0.0, 0.0};  // the band's sums of w~ and rho, its size
    for (int k = threadIdx.x; k < nb; k += kBlock) {
      bs[0] += (double)s_bw[k];
      bs[1] += (double)s_br[k];
      bs[2] += 1.0;
    }
    blk_reduce<double, 3, kBlock>(bs);
    // the tokens active at every point of the bracket (v: the sums at lo)
    const double aw = v[0] - bs[0], ar = v[1] - bs[1], ac = v[2] - bs[2];
    for (int it = 0; it < kBetaPassMax && !st.done; ++it) {
      double pts[kBetaPts], t[3 * kBetaPts], u[kBetaRec];
      beta_points(st, pts);
#pragma unroll
      for (int k = 0; k < 3 * kBetaPts; ++k) t[k] = 0.0;
      for (int k = threadIdx.x; k < nb; k += kBlock) {
        const double w = (double)s_bw[k], rh = (double)s_br[k];
#pragma unroll
        for (int j = 0; j < kBetaPts; ++j) {
          if (w - pts[j] * rh > 0.0) {
            t[3 * j] += w;
            t[3 * j + 1] += rh;
            t[3 * j + 2] += 1.0;
          }
        }
      }
      blk_reduce<double, 3 * kBetaPts, kBlock>(t);
#pragma unroll
      for (int j = 0; j < kBetaPts; ++j) {
        u[3 * j] = t[3 * j] + aw;
        u[3 * j + 1] = t[3 * j + 1] + ar;
        u[3 * j + 2] = t[3 * j + 2] + ac;
      }
      u[kBetaRec - 1] = 0.0;
      st = beta_advance(st, u);
    }
    return st;
  }
  // a small band: the Newton steps by the first wave alone (its sums fold
  // by DPP: no workgroup barrier per step); the result goes to the other
  // waves through LDS
  __shared__ BetaState s_st;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    double bs[3] = {0.0, 0.0, 0.0};  // the band's sums of w~ and rho, its size
    for (int k = lane; k < nb; k += kWave) {
      bs[0] += (double)s_bw[k];
      bs[1] += (double)s_br[k];
      bs[2] += 1.0;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) bs[k] = wave_fold<double, OpSum<double>>(bs[k]);
    // the tokens active at every point of the bracket (v: the sums at lo)
    const double aw = v[0] - bs[0], ar = v[1] - bs[1], ac = v[2] - bs[2];
    for (int it = 0; it < kBetaPassMax && !st.done; ++it) {
      double pts[kBetaPts], u[kBetaRec];
      beta_points(st, pts);
#pragma unroll
      for (int k = 0; k < kBetaRec; ++k) u[k] = 0.0;
      for (int k = lane; k < nb; k += kWave) {
        const double w = (double)s_bw[k], rh = (double)s_br[k];
#pragma unroll
        for (int j = 0; j < kBetaPts; ++j) {
          if (w - pts[j] * rh > 0.0) {
            u[3 * j] += w;
            u[3 * j + 1] += rh;
            u[3 * j + 2] += 1.0;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 3 * kBetaPts; ++k) u[k] = wave_fold<double, OpSum<double>>(u[k]);
#pragma unroll
      for (int j = 0; j < kBetaPts; ++j) {
        u[3 * j] += aw;
        u[3 * j + 1] += ar;
        u[3 * j + 2] += ac;
      }
      st = beta_advance(st, u);
    }
    if (lane == 0) s_st = st;
  }
  __syncthreads();
  return s_st;
}

// ------------------------------------------------------------ binary shrinkage,
// first round (in the beta launches, which binary shrinkage leaves idle)
// The first round's lower key bound from a row's top-digit histogram (LDS),
// by the calling wave: the smallest bin j0 whose keys, with those of the
// bins above it, fit in kBinCap. It is usable (ok) unless a finer digit
// would be taken, i.e. j0 > 0 with fewer than kBinCap / 4 keys above it --
// the same decision as the first digit of the streaming rounds below.
__device__ __forceinline__ void bin_bound(const uint32_t *hist, int lane,
                                          unsigned long long &lo, int &ok) {
  constexpr int per = kSelBinsP / kWave;
  uint32_t tot = 0u;
  for (int k = 0; k < per; ++k) tot += hist[lane * per + k];
  const uint32_t incl = wave_incl_scan<uint32_t>(tot, lane);
  uint32_t cum = __shfl(incl, kWave - 1, kWave) - incl;  // bins above
  int jf = kSelBinsP;
  for (int k = per - 1; k >= 0; --k) {
    cum += hist[lane * per + k];
    if (cum > (uint32_t)kBinCap) break;
    jf = lane * per + k;
  }
  const int j0 = -wave_max<int>(-jf);
  uint32_t part = 0u;
  for (int k = 0; k < per; ++k)
    if (lane * per + k >= j0) part += hist[lane * per + k];
  const uint32_t cnt = wave_sum<uint32_t>(part);
  ok = (j0 > 0 && cnt < (uint32_t)(kBinCap / 4)) ? 0 : 1;
  lo = (unsigned long long)j0 << sel_off(0);
}

// The histogram buffer both beta launches use (LDS).
__device__ __forceinline__ uint32_t *bin_lds_hist() {
  __shared__ uint32_t s_h[kSelBinsP];
  return s_h;
}

// First beta launch: this workgroup's tokens of L counted by the top digit
// of their binary key, added to the row's histogram (integer atomics: the
// same counts in any order).
__device__ __forceinline__ void bin_hist_pass(const DParams &p, int row, int bg,
                                              int cc0, int cc1, float m,
                                              float (&r8)[kRowTok],
                                              float (&s8)[kRowTok]) {
  uint32_t *s_h = bin_lds_hist();
  for (int k = threadIdx.x; k < kSelBinsP; k += kBlock) s_h[k] = 0u;
  __syncthreads();
  for (int cc = cc0; cc < cc1; ++cc) {
    float nr[kRowTok], ns[kRowTok];
    if (cc + 1 < cc1) row_load(p, row, bg, cc + 1, nr, ns);  // next in flight
#pragma unroll
    for (int u = 0; u < kRowTok; ++u) {
      if (!(r8[u] < 1.0f)) continue;
      const float wt = expf(s8[u] - m);
      const float qr = qr_of(r8[u]);
      atomicAdd(&s_h[(int)(bin_key(wt, qr, row_pos(cc, u)) >> sel_off(0))], 1u);
    }
#pragma unroll
    for (int u = 0; u < kRowTok; ++u) {
      r8[u] = nr[u];
      s8[u] = ns[u];
    }
  }
  __syncthreads();
  uint32_t *gh = p.bhist + (size_t)row * kSelBinsP;
  for (int k = threadIdx.x; k < kSelBinsP; k += kBlock)
    if (s_h[k]) atomicAdd(&gh[k], s_h[k]);
}

// Second beta launch: the first round's bound from the row's histogram and,
// when it is usable, this workgroup's keys at or above it (with their
// biases) in its own segment; a count of 0 otherwise.
__device__ __forceinline__ void bin_collect_pass(const DParams &p, int row,
                                                 int bg, int c, int cc0,
                                                 int cc1, float m,
                                                 float (&r8)[kRowTok],
                                                 float (&s8)[kRowTok]) {
  uint32_t *s_h = bin_lds_hist();
  __shared__ unsigned long long s_lo;
  __shared__ int s_ok;
  __shared__ uint32_t s_n;
  const int lane = threadIdx.x % kWave;
  for (int k = threadIdx.x; k < kSelBinsP; k += kBlock)
    s_h[k] = p.bhist[(size_t)row * kSelBinsP + k];
  if (threadIdx.x == 0) s_n = 0u;
  __syncthreads();
  if (threadIdx.x < kWave) {
    unsigned long long l0;
    int ok;
    bin_bound(s_h, lane, l0, ok);
    if (lane == 0) {
      s_lo = l0;
      s_ok = ok;
    }
  }
  __syncthreads();
  const size_t seg = (size_t)row * p.nrc + c;
  if (!s_ok) {
    if (threadIdx.x == 0) p.bcnt[seg] = 0u;
    return;
  }
  const unsigned long long lo = s_lo;
  for (int cc = cc0; cc < cc1; ++cc) {
    float nr[kRowTok], ns[kRowTok];
    if (cc + 1 < cc1) row_load(p, row, bg, cc + 1, nr, ns);  // next in flight
#pragma unroll
    for (int u = 0; u < kRowTok; ++u) {
      bool take = false;
      unsigned long long key = 0ull;
      float a = 0.0f;
      if (r8[u] < 1.0f) {
        const float wt = expf(s8[u] - m);
        const float qr = qr_of(r8[u]);
        key = bin_key(wt, qr, row_pos(cc, u));
        a = wt * (1.0f - r8[u]);
        take = key >= lo;
      }
      // one LDS atomic per wave: the wave's takers get consecutive slots
      const unsigned long long bal = __ballot(take);
      if (bal == 0ull) continue;
      const int leader = __ffsll((long long)bal) - 1;
      uint32_t base = 0u;
      if (lane == leader) base = atomicAdd(&s_n, (uint32_t)__popcll(bal));
      base = __shfl(base, leader, kWave);
      if (take) {
        const uint32_t slot = base + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
        if (slot < (uint32_t)kBinCap) {
          p.bkeys[seg * kBinCap + slot] = key;
          p.bav[seg * kBinCap + slot] = a;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRowTok; ++u) {
      r8[u] = nr[u];
      s8[u] = ns[u];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) p.bcnt[seg] = min(s_n, (uint32_t)kBinCap);
}

// Newton pass `pass` (>= 1) of the beta* iteration; pass 1 starts from the
// pass-0 sums that the scan and resident-logit kernels left per chunk and
// part. Grid (chunks, Hq, B).
template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_rbeta(DParams p, int pass) {
  const int c = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int row = b * p.Hq + hq, bg = b * p.G + hq / GRP;
  const size_t rows = (size_t)p.B * p.Hq;
  const int q = (pass - 1) & 1;
  if (pass >= 3 && p.bstate[(size_t)q * rows + row].done) {
    // settled by an earlier pass: carry the state forward, read nothing else
    if (c == 0 && threadIdx.x == 0)
      p.bstate[(size_t)(pass & 1) * rows + row] = p.bstate[(size_t)q * rows + row];
    return;
  }
  // sub-chunks [cc0, cc1) of kRowChunk tokens; the first in flight now
  const int cc0 = c * p.rsub, cc1 = min(cc0 + p.rsub, p.nsub);
  float w8[kRowTok], r8[kRowTok], s8[kRowTok];
  row_load(p, row, bg, cc0, r8, s8);
  // the previous pass: this thread's share of the records, and the state
  double rv[kBetaRec];
  BetaState st{};
  float m;
  if (pass == 1) {
    m = row_pass0(p, row, bg, c, hq % GRP == 0, rv);
    beta_rec_fold<true>(rv);
    st = beta_init(rv, p.est);
  } else {
    m = p.rows[row].m;
    st = p.bstate[(size_t)q * rows + row];
    if (!st.done)
      beta_rec_wave(p.bpart + ((size_t)q * rows + row) * p.nrc * kBetaRec, p.nrc, rv);
  }
  double v[kBetaRec];
#pragma unroll
  for (int k = 0; k < kBetaRec; ++k) v[k] = 0.0;
  double *out = p.bpart + (((size_t)(pass & 1) * rows + row) * p.nrc + c) * kBetaRec;
  if (pass >= 2 && !st.done) st = beta_settle(p, st, rv, row, q);
  if (c == 0 && threadIdx.x == 0) p.bstate[(size_t)(pass & 1) * rows + row] = st;
  if (p.est == VKV_EST_BINARY) {  // (st.done: no beta* to find)
    if (pass == 1) bin_hist_pass(p, row, bg, cc0, cc1, m, r8, s8);
    else if (pass == 2) bin_collect_pass(p, row, bg, c, cc0, cc1, m, r8, s8);
    return;
  }
  if (st.done) return;
  double pts[kBetaPts];
  beta_points(st, pts);
  // the band: which of this thread's tokens are in it (bit 8 j + u for
  // sub-chunk cc0 + j), stored once all are seen, in (thread, token) order
  static_assert(kRowTok * 8 <= 64, "band mask");
  unsigned long long bmask = 0ull;
  for (int cc = cc0; cc < cc1; ++cc) {
    float nr[kRowTok], ns[kRowTok];
    if (cc + 1 < cc1) row_load(p, row, bg, cc + 1, nr, ns);  // next in flight
    row_weights(m, r8, s8, w8);
#pragma unroll
    for (int u = 0; u < kRowTok; ++u) {
      beta_accumulate(pts, w8[u], r8[u], v);
      if (in_band(st, w8[u], r8[u])) bmask |= 1ull << ((cc - cc0) * kRowTok + u);
    }
#pragma unroll
    for (int u = 0; u < kRowTok; ++u) {
      r8[u] = nr[u];
      s8[u] = ns[u];
    }
  }
  uint32_t nband;
  {
    __shared__ uint32_t s_bs[kBlock / kWave + 1];
    uint32_t k = block_exclusive_scan<uint32_t>((uint32_t)__popcll(bmask), s_bs, &nband);
    if (nband <= (uint32_t)kBandChunk) {
      float2 *bdst = p.band + (((size_t)(pass & 1) * rows + row) * p.nrc + c) * kBandChunk;
      const float *rr = p.r + (size_t)bg * p.ns;
      const float *sh = p.shat + (size_t)row * p.n;
      while (bmask) {
        const int bit = __ffsll((long long)bmask) - 1;
        bmask &= bmask - 1ull;
        const int i = row_pos(cc0 + bit / kRowTok, bit % kRowTok);
        const float ri = rr[i];
        bdst[k++] = make_float2(expf(sh[i] - m), plan_rho(ri));
      }
    }
  }
  blk_reduce<double, kBetaRec, kBlock>(v);
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < kBetaRec - 1; ++k) out[k] = v[k];
    out[kBetaRec - 1] = (double)nband;
  }
}

// ------------------------------------------------------------ binary shrinkage
// Appendix A.2: lambda_i in {1, r_i}. The tokens of L are visited by binary
// key (kappa = w~ (1 - r) / r descending, then position ascending) and
// moved to lambda = r while kappa exceeds twice the bias w~ (1 - r) of the
// tokens moved before them. Kappa falls and the bias grows along the order,
// so the first token that fails ends the moves, and only the top of the
// order matters (tens of tokens move in the workloads measured). One
// 1024-thread workgroup per row takes the keys in rounds of at most kBinCap,
// largest first: count histograms of 11-bit key digits give the round's
// lower key bound (a second digit only while the round would hold fewer
// than kBinCap / 4 keys), the round's keys and biases are gathered into
// LDS (slots by wave, in wave order of arrival; the sort fixes the order)
// and sorted, and float64 prefix sums of the biases in that order, in a
// fixed tree order, find the first token that stops the moves. A round that
// moves all of its tokens passes its bias total on to the next. The result
// is the key of the last token moved (~0 for none) and the moved tokens'
// bias; every later pass recomputes lambda from it.

template <int GRP>
__global__ __launch_bounds__(kPlanThreads) void dk_rbin(DParams p) {
  const int hq = blockIdx.x, b = blockIdx.y;
  const int row = b * p.Hq + hq, bg = b * p.G + hq / GRP;
  const int n = p.n;
  const float *rr = p.r + (size_t)bg * p.ns;
  const float *sh = p.shat + (size_t)row * n;
  const float m = p.rows[row].m;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  __shared__ uint32_t s_hist[kSelBinsP];
  __shared__ unsigned long long s_key[kBinCap];
  __shared__ float s_a[kBinCap];
  __shared__ double s_wsum[kPlanWaves];
  __shared__ unsigned long long s_pre, s_lo;
  __shared__ uint32_t s_room, s_cnt;
  __shared__ int s_more, s_stop;
  __shared__ double s_excl;

  // f(binary key, bias w~ (1 - r)) for this thread's tokens of L
  auto stream = [&](auto &&f) {
    constexpr int U = 8;
    for (int base = 0; base < n; base += U * kPlanThreads) {
      float ru[U], su[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * kPlanThreads + (int)threadIdx.x;
        ru[u] = i < n ? rr[i] : 1.0f;
        su[u] = i < n ? sh[i] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!(ru[u] < 1.0f)) continue;
        const float wt = expf(su[u] - m);
        const float qr = qr_of(ru[u]);
        f(bin_key(wt, qr, base + u * kPlanThreads + (int)threadIdx.x),
          wt * (1.0f - ru[u]));
      }
    }
  };

  unsigned long long hi = kKeyEnd;  // the keys at or above hi are decided
  unsigned long long last = ~0ull;  // key of the last token moved
  double beta = 0.0;                // bias of the tokens moved
  // the first round as the beta launches gathered it: its bound from the
  // row's top-digit histogram (the same decision they took) and their keys
  bool pre;
  {
    for (int k = threadIdx.x; k < kSelBinsP; k += kPlanThreads)
      s_hist[k] = p.bhist[(size_t)row * kSelBinsP + k];
    __syncthreads();
    if (wave == 0) {
      unsigned long long l0;
      int ok;
      bin_bound(s_hist, lane, l0, ok);
      if (lane == 0) {
        s_lo = l0;
        s_more = ok;
      }
    }
    __syncthreads();
    pre = s_more != 0;
  }
  for (;;) {
    unsigned long long lo = 0ull;
    if (pre) {
      __shared__ uint32_t s_off[kMaxChunks + 1];
      lo = s_lo;
      if (wave == 0) {  // nrc <= 64 segment counts, one per lane
        const uint32_t k = lane < p.nrc ? p.bcnt[(size_t)row * p.nrc + lane] : 0u;
        const uint32_t incl = wave_incl_scan<uint32_t>(k, lane);
        if (lane < p.nrc) s_off[lane] = incl - k;
        if (lane == kWave - 1) {
          s_off[p.nrc] = incl;
          s_cnt = incl;
        }
      }
      __syncthreads();
      const int tot = (int)min(s_off[p.nrc], (uint32_t)kBinCap);
      for (int e = threadIdx.x; e < tot; e += kPlanThreads) {
        int a0 = 0, a1 = p.nrc;  // the segment holding entry e
        while (a1 - a0 > 1) {
          const int mid = (a0 + a1) / 2;
          if ((int)s_off[mid] <= e) a0 = mid; else a1 = mid;
        }
        const size_t at = ((size_t)row * p.nrc + a0) * kBinCap + (e - (int)s_off[a0]);
        s_key[e] = p.bkeys[at];
        s_a[e] = p.bav[at];
      }
      __syncthreads();
    } else {
    // ---- the round's lower key bound, digit by digit from the top
    if (threadIdx.x == 0) {
      s_pre = 0ull;
      s_room = (uint32_t)kBinCap;
    }
    for (int d = 0; d < kSelLevels; ++d) {
      const int off = sel_off(d);
      for (int k = threadIdx.x; k < kSelBinsP; k += kPlanThreads) s_hist[k] = 0u;
      __syncthreads();
      const unsigned long long pre = s_pre;
      stream([&](unsigned long long key, float) {
        if (key < hi && (key >> (off + kSelDigit)) == pre)
          atomicAdd(&s_hist[(int)((key >> off) & (kSelBinsP - 1))], 1u);
      });
      __syncthreads();
      if (wave == 0) {
        // j0 = the smallest bin j whose keys and those of the bins above it
        // fit in the room left; cnt = their number
        constexpr int per = kSelBinsP / kWave;
        const uint32_t room = s_room;
        uint32_t tot = 0u;
        for (int k = 0; k < per; ++k) tot += s_hist[lane * per + k];
        const uint32_t incl = wave_incl_scan<uint32_t>(tot, lane);
        uint32_t cum = __shfl(incl, kWave - 1, kWave) - incl;  // bins above
        int jf = kSelBinsP;
        for (int k = per - 1; k >= 0; --k) {
          cum += s_hist[lane * per + k];
          if (cum > room) break;
          jf = lane * per + k;
        }
        const int j0 = -wave_max<int>(-jf);
        uint32_t part = 0u;
        for (int k = 0; k < per; ++k)
          if (lane * per + k >= j0) part += s_hist[lane * per + k];
        const uint32_t cnt = wave_sum<uint32_t>(part);
        if (lane == 0) {
          const bool more = j0 > 0 && cnt < (uint32_t)(kBinCap / 4) &&
                            d + 1 < kSelLevels;
          if (more) {
            s_pre = (pre << kSelDigit) | (unsigned long long)(j0 - 1);
            s_room = room - cnt;
          } else {
            s_lo = ((pre << kSelDigit) | (unsigned long long)j0) << off;
          }
          s_more = more ? 1 : 0;
        }
      }
      __syncthreads();
      if (!s_more) {
        lo = s_lo;
        break;
      }
    }
    // ---- gather the round's keys [lo, hi) and sort them, descending
    if (threadIdx.x == 0) s_cnt = 0u;
    __syncthreads();
    stream([&](unsigned long long key, float a) {
      const bool take = key >= lo && key < hi;
      // one LDS atomic per wave: the wave's takers get consecutive slots
      const unsigned long long bal = __ballot(take);
      if (bal == 0ull) return;
      const int leader = __ffsll((long long)bal) - 1;
      uint32_t base = 0u;
      if (lane == leader) base = atomicAdd(&s_cnt, (uint32_t)__popcll(bal));
      base = __shfl(base, leader, kWave);
      if (take) {
        const uint32_t slot =
            base + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
        if (slot < (uint32_t)kBinCap) {
          s_key[slot] = key;
          s_a[slot] = a;
        }
      }
    });
    __syncthreads();
    }
    pre = false;
    const int cnt = (int)min(s_cnt, (uint32_t)kBinCap);
    int np2 = 1;
    while (np2 < cnt) np2 <<= 1;
    for (int k = cnt + (int)threadIdx.x; k < np2; k += kPlanThreads) {
      s_key[k] = 0ull;  // below every key of L
      s_a[k] = 0.0f;
    }
    __syncthreads();
    // bitonic sort by the first wave alone (at most 256 entries: two
    // compare-exchanges per lane and step), its LDS accesses ordered by a
    // wavefront fence between steps instead of workgroup barriers
    if (wave == 0) {
      for (int k = 2; k <= np2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
          for (int t = lane; t < np2 / 2; t += kWave) {
            const int i = 2 * t - (t & (j - 1)), ix = i + j;
            const unsigned long long x = s_key[i], y = s_key[ix];
            if (((i & k) == 0) ? (x < y) : (x > y)) {
              s_key[i] = y;
              s_key[ix] = x;
              const float ta = s_a[i];
              s_a[i] = s_a[ix];
              s_a[ix] = ta;
            }
          }
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
    __syncthreads();
    // ---- prefix sums of the bias in key order (two entries per thread)
    const int e0 = 2 * (int)threadIdx.x;
    const double a0 = e0 < cnt ? (double)s_a[e0] : 0.0;
    const double a1 = e0 + 1 < cnt ? (double)s_a[e0 + 1] : 0.0;
    const double winc = wave_incl_scan<double>(a0 + a1, lane);
    if (lane == kWave - 1) s_wsum[wave] = winc;
    if (threadIdx.x == 0) s_excl = 0.0;
    __syncthreads();
    double ex = winc - (a0 + a1);
    double total = 0.0;
    for (int w = 0; w < kPlanWaves; ++w) {
      if (w < wave) ex += s_wsum[w];
      total += s_wsum[w];
    }
    // the first entry that does not move: kappa <= 2 (beta + bias before it)
    int kf = cnt;
    for (int u = 1; u >= 0; --u) {
      const int e = e0 + u;
      if (e >= cnt) continue;
      const double kap = (double)__uint_as_float((uint32_t)(s_key[e] >> 24));
      const double before = beta + (u ? ex + a0 : ex);
      if (!(kap > 2.0 * before)) kf = e;
    }
    int kv[1] = {kf};
    blk_combine<int, 1, kPlanThreads, OpMin<int>>(kv);
    kf = kv[0];
    if (kf < cnt) {
      // the bias of the entries before kf
      if (e0 == kf) s_excl = ex;
      if (e0 + 1 == kf) s_excl = ex + a0;
      __syncthreads();
      if (kf > 0) last = s_key[kf - 1];
      beta += s_excl;
      break;
    }
    if (cnt > 0) last = s_key[cnt - 1];
    beta += total;
    if (lo == 0ull) break;  // every token of L moved
    hi = lo;
    __syncthreads();  // LDS reuse by the next round
  }
  if (threadIdx.x == 0) {
    BinState bs;
    bs.key = last;
    bs.beta = beta;
    p.binst[row] = bs;
  }
}

// Certificate terms (Lemma 1) at beta*. Settles beta* from the last Newton
// pass first; a row still open iterates here over all of its tokens.
template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_rcert(DParams p) {
  const int c = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int row = b * p.Hq + hq, bg = b * p.G + hq / GRP;
  const size_t rows = (size_t)p.B * p.Hq;
  const int cc0 = c * p.rsub, cc1 = min(cc0 + p.rsub, p.nsub);
  float w8[kRowTok], r8[kRowTok], s8[kRowTok];
  row_load(p, row, bg, cc0, r8, s8);
  const float m = p.rows[row].m;
  const int q = p.nbeta & 1;
  BetaState st = p.bstate[(size_t)q * rows + row];
  if (!st.done) {  // (uniform: the same state in every workgroup)
    double rv[kBetaRec];
    beta_rec_wave(p.bpart + ((size_t)q * rows + row) * p.nrc * kBetaRec, p.nrc, rv);
    st = beta_settle(p, st, rv, row, q);
  }
  if (!st.done) {
    // rare (a band too large to keep): more Newton passes, each over the
    // whole row by this workgroup
    for (int it = 0; it < kBetaPassMax && !st.done; ++it) {
      double pts[kBetaPts], v[kBetaRec];
      beta_points(st, pts);
#pragma unroll
      for (int k = 0; k < kBetaRec; ++k) v[k] = 0.0;
      for (int cc = 0; cc < p.nsub; ++cc) {
        float fr[kRowTok], fs[kRowTok], fw[kRowTok];
        row_load(p, row, bg, cc, fr, fs);
        row_weights(m, fr, fs, fw);
#pragma unroll
        for (int u = 0; u < kRowTok; ++u) beta_accumulate(pts, fw[u], fr[u], v);
      }
      blk_reduce<double, kBetaRec, kBlock>(v);
      st = beta_advance(st, v);
    }
    if (!st.done) st.beta = st.lo;
  }
  // (binary shrinkage: beta is the bias of the moved tokens)
  const bool bin = p.est == VKV_EST_BINARY;
  const double beta = bin ? p.binst[row].beta : st.beta;
  const LamRule lr = lam_rule((float)beta, p.est, bin ? p.binst[row].key : ~0ull);
  if (c == 0 && threadIdx.x == 0) {
    p.rbeta[2 * row] = beta;
    p.rbeta[2 * row + 1] = st.dnorm;
  }
  double cv[2] = {0.0, 0.0};
  float x1 = 0.0f, x2 = 0.0f;
  int p1 = 0x7fffffff;
  for (int cc = cc0; cc < cc1; ++cc) {
    float nr[kRowTok], ns[kRowTok];
    if (cc + 1 < cc1) row_load(p, row, bg, cc + 1, nr, ns);  // next in flight
    row_weights(m, r8, s8, w8);
#pragma unroll
    for (int u = 0; u < kRowTok; ++u) {
      if (!(r8[u] < 1.0f)) continue;
      const Terms t = token_terms_w(w8[u], r8[u], lr, row_pos(cc, u));
      cv[0] += (double)t.bi;
      cv[1] += (double)t.vi;
      top2_merge(x1, p1, x2, t.rb, row_pos(cc, u), 0.0f);
    }
#pragma unroll
    for (int u = 0; u < kRowTok; ++u) {
      r8[u] = nr[u];
      s8[u] = ns[u];
    }
  }
  blk_reduce<double, 2, kBlock>(cv);
  blk_top2<kBlock>(x1, p1, x2);
  if (threadIdx.x == 0) {
    CertPart cp;
    cp.tb = cv[0];
    cp.tv = cv[1];
    cp.x1 = x1;
    cp.x2 = x2;
    cp.p1 = p1;
    cp.pad = 0;
    p.cpart[(size_t)row * p.nrc + c] = cp;
  }
}

// This thread's share of a row's certificate records.
struct CertShare {
  double cv[2];
  float x1, x2;
  int p1;
};
__device__ __forceinline__ CertShare cert_rec_load(const DParams &p, int row) {
  CertShare z;
  z.cv[0] = z.cv[1] = 0.0;
  z.x1 = z.x2 = 0.0f;
  z.p1 = 0x7fffffff;
  for (int t = threadIdx.x % kWave; t < p.nrc; t += kWave) {
    const CertPart cp = p.cpart[(size_t)row * p.nrc + t];
    z.cv[0] += cp.tb;
    z.cv[1] += cp.tv;
    top2_merge(z.x1, z.p1, z.x2, cp.x1, cp.p1, cp.x2);
  }
  return z;
}

// The certificate of a row from its chunk records (this thread's share in
// `sh`): every workgroup of the row computes the same RowState.
__device__ __forceinline__ void row_certificate(const DParams &p, CertShare sh,
                                                float m, double beta,
                                                double dnorm,
                                                unsigned long long bkey,
                                                RowState &rs) {
  // (every wave folds the lane-strided shares on its own: sums by DPP, the
  // top two by a butterfly of exact merges, the same in every lane)
  double cv[2] = {wave_fold<double, OpSum<double>>(sh.cv[0]),
                  wave_fold<double, OpSum<double>>(sh.cv[1])};
  float x1 = sh.x1, x2 = sh.x2;
  int p1 = sh.p1;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const float y1 = __shfl_xor(x1, o, kWave), y2 = __shfl_xor(x2, o, kWave);
    const int q1 = __shfl_xor(p1, o, kWave);
    top2_merge(x1, p1, x2, y1, q1, y2);
  }
  if (threadIdx.x == 0) {
    const float y1 = x1, y2 = x2;
    const int yq = p1;
    const double a = p.a_delta, l = p.l_delta;
    const double tb = cv[0], tv = cv[1];
    RowState z{};
    z.m = m;
    z.dnorm = dnorm;
    z.beta = beta;
    z.bkey = bkey;
    z.betaL = tb;
    z.VL = tv;
    z.b1 = y1;
    z.b2 = y2;
    z.amax = (y2 < y1) ? yq : -1;
    z.s_full = sqrt(a * a * (double)y1 * (double)y1 + 2.0 * tv * l);
    const float af = (float)a, lf = (float)l;
    z.s_full_f = __builtin_amdgcn_sqrtf(af * af * y1 * y1 + 2.0f * (float)tv * lf);
    z.ab1sq = af * af * y1 * y1;
    const double e0 = (tb + a * (double)y1 + z.s_full) / dnorm;
    z.eps0 = e0;
    z.eps1 = (float)e0;
    z.kstar = 0;
    z.T = ~0ull;
    z.fetch = e0 < (double)p.eps ? 0 : 1;
    z.capb = 2.0 * (double)p.eps * dnorm;
    z.capv = z.capb * z.capb / (2.0 * l);
    int eb = 0, ev = 0;
    (void)frexp(z.capb, &eb);
    (void)frexp(z.capv, &ev);
    z.eb = 40 - eb;
    z.ev = 40 - ev;
    rs = z;
  }
  __syncthreads();
}

// Candidate workgroups per row and the candidates each may write. Their
// tokens are split block-cyclically (blocks of kSelBlk positions), so that a
// run of high-gain positions is spread over all of them.
constexpr int kSelWG = 16;           // at most; p.nsel per row at run time
// Per workgroup of a row's p.nsel: kCandMax / nsel candidates, the top
// quarter of them tried first.
__device__ __forceinline__ int cand_cap(const DParams &p) { return kCandMax / p.nsel; }
constexpr int kSelBlk = 64;
constexpr int kSelIt = 8;  // tokens per thread whose keys stay in registers

// Certificate of the row (workgroup 0 stores it), then for a row that
// fetches: this workgroup's keys, their count histogram over the top 11 key
// bits and the fixed-point totals of beta_i and v_i; its local bound lo_s,
// the smallest bin edge with at most kCandMax / nsel of its keys at or
// above it; and
// those keys, written with their fixed-point beta_i, v_i and b_i. Keys below
// lo_s are not written; their largest b_i is.
template <int GRP, bool KEEP>
__global__ __launch_bounds__(kBlock) void dk_rcand(DParams p) {
  const int s = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int row = b * p.Hq + hq, bg = b * p.G + hq / GRP;
  const int nsel = p.nsel, capw = cand_cap(p);
  __shared__ RowState rs;
  __shared__ uint32_t s_hist[kSelBinsP];
  __shared__ int s_j0, s_j1;
  __shared__ uint32_t s_c0;
  const float *rr = p.r + (size_t)bg * p.ns;
  const float *sh = p.shat + (size_t)row * p.n;
  const int n = p.n;
  // token of iteration it for this thread
  auto pos_of = [&](int it) {
    return ((it * (kBlock / kSelBlk) + (int)threadIdx.x / kSelBlk) * nsel + s) * kSelBlk +
           (int)threadIdx.x % kSelBlk;
  };
  const int nblk = (n + kSelBlk - 1) / kSelBlk;
  const int iters = ((nblk + nsel - 1) / nsel + kBlock / kSelBlk - 1) / (kBlock / kSelBlk);
  // loads first: the first kSelIt tokens, the certificate records
  float r8[kSelIt], s8[kSelIt];
#pragma unroll
  for (int it = 0; it < kSelIt; ++it) {
    const int i = pos_of(it);
    r8[it] = (it < iters && i < n) ? rr[i] : 1.0f;
    s8[it] = (it < iters && i < n) ? sh[i] : 0.0f;
  }
  const float m = p.rows[row].m;
  const CertShare cs = cert_rec_load(p, row);
  const double beta = p.rbeta[2 * row], dnorm = p.rbeta[2 * row + 1];
  for (int i = threadIdx.x; i < kSelBinsP; i += kBlock) s_hist[i] = 0u;
  row_certificate(p, cs, m, beta, dnorm,
                  p.est == VKV_EST_BINARY ? p.binst[row].key : ~0ull, rs);
  if (s == 0 && threadIdx.x == 0) p.rows[row] = rs;
  if (!rs.fetch) return;
  const LamRule lr = lam_rule((float)rs.beta, p.est, rs.bkey);
  const float af = (float)p.a_delta, lf = (float)p.l_delta;
  const int eb = rs.eb, ev = rs.ev;
  const double capb = rs.capb, capv = rs.capv;
  auto key_of = [&](int i, float ri, float si, Terms &t) {
    t = token_terms_w(expf(si - m), ri, lr, i);
    return make_key(token_gain(t, i, rs, af, lf), i);
  };
  // ---- keys: histogram and totals (the register tokens keep their terms)
  // (KEEP: a launch small enough to fit at the lower occupancy the extra
  // registers cost)
  // (s8 holds each register token's w~ from here on)
  unsigned long long key8[kSelIt];
  float bi8[KEEP ? kSelIt : 1], lw8[KEEP ? kSelIt : 1], rb8[KEEP ? kSelIt : 1];
  double tx[2] = {0.0, 0.0};  // exact integers (fx_term)
#pragma unroll
  for (int it = 0; it < kSelIt; ++it) {
    key8[it] = 0ull;
    if (!(r8[it] < 1.0f)) continue;
    Terms t;
    key8[it] = key_of(pos_of(it), r8[it], s8[it], t);
    s8[it] = t.wt;
    if constexpr (KEEP) {
      bi8[it] = t.bi;
      lw8[it] = t.lam * t.wt;
      rb8[it] = t.rb;
    }
    atomicAdd(&s_hist[(int)(key8[it] >> sel_off(0))], 1u);
    tx[0] += fx_term(t.bi, capb, eb);
    tx[1] += fx_term(t.vi, capv, ev);
  }
  // long rows: the rest in batches of kSelIt tokens (recomputed below)
  auto load_batch = [&](int it0, float (&rb)[kSelIt], float (&sb)[kSelIt]) {
#pragma unroll
    for (int k = 0; k < kSelIt; ++k) {
      const int i = pos_of(it0 + k);
      const bool ok = it0 + k < iters && i < n;
      rb[k] = ok ? rr[i] : 1.0f;
      sb[k] = ok ? sh[i] : 0.0f;
    }
  };
  for (int it0 = kSelIt; it0 < iters; it0 += kSelIt) {
    float rb[kSelIt], sb[kSelIt];
    load_batch(it0, rb, sb);
#pragma unroll
    for (int k = 0; k < kSelIt; ++k) {
      if (!(rb[k] < 1.0f)) continue;
      Terms t;
      const unsigned long long key = key_of(pos_of(it0 + k), rb[k], sb[k], t);
      atomicAdd(&s_hist[(int)(key >> sel_off(0))], 1u);
      tx[0] += fx_term(t.bi, capb, eb);
      tx[1] += fx_term(t.vi, capv, ev);
    }
  }
  // (tx: exact integers below 2^53, summed with the others at the end)
  __syncthreads();  // the histogram is complete
  // ---- local bounds: thread t owns bins [8 t, 8 t + 8). Tier 0 is the
  // smallest bin edge with at most capw / 4 keys at or above it, tier 1 the
  // same for capw; c0 = keys at or above the tier-0 edge.
  __shared__ uint32_t s_scan[kBlock / kWave + 1];
  {
    constexpr int PB = kSelBinsP / kBlock;
    uint32_t hc[PB], own = 0u;
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      hc[k] = s_hist[threadIdx.x * PB + k];
      own += hc[k];
    }
    uint32_t all;
    const uint32_t excl = block_exclusive_scan<uint32_t>(own, s_scan, &all);
    uint32_t c = all - excl - own;  // keys in the bins of later threads
    int jb[2] = {kSelBinsP, kSelBinsP};
    uint32_t cj0 = 0u;
#pragma unroll
    for (int k = PB - 1; k >= 0; --k) {
      c += hc[k];
      if (c <= (uint32_t)(capw / 4)) {
        jb[0] = (int)threadIdx.x * PB + k;
        cj0 = c;
      }
      if (c <= (uint32_t)capw) jb[1] = (int)threadIdx.x * PB + k;
    }
    const int my0 = jb[0];
    blk_combine<int, 2, kBlock, OpMin<int>>(jb);
    if (threadIdx.x == 0) {
      s_j0 = jb[0];
      s_j1 = jb[1];
      if (jb[0] == kSelBinsP) s_c0 = 0u;
    }
    if (my0 == jb[0] && my0 < kSelBinsP) s_c0 = cj0;  // the owner of that bin
  }
  __syncthreads();
  const unsigned long long lo0 =
      s_j0 < kSelBinsP ? ((unsigned long long)s_j0 << sel_off(0)) : kKeyEnd;
  const unsigned long long lo =
      s_j1 < kSelBinsP ? ((unsigned long long)s_j1 << sel_off(0)) : kKeyEnd;
  const uint32_t c0 = s_c0;
  // ---- the keys at or above lo (with w~ and r), tier 0 first, each tier in
  // token order (slots from a block scan); for the keys below lo and for
  // those of tier 1 alone, the max of b_i and the float64 sums of beta_i
  // and v_i
  const size_t seg = (size_t)row * kCandMax + (size_t)s * capw;
  uint32_t below = 0u, below1 = 0u;
  double dsum[4] = {0.0, 0.0, 0.0, 0.0};
  uint32_t o0 = 0u, o1 = 0u;  // slots taken by earlier batches, per tier
  // (wb: each token's w~)
  // (the batch's results are returned, not written through captures: the
  // captured counters and maxima were otherwise kept in scratch memory)
  struct EmitRes {
    uint32_t t0, t1, bl, bl1;
    double d[4];
  };
  auto emit_batch = [&](const unsigned long long (&kb)[kSelIt],
                        const float (&rb)[kSelIt], const float (&wb)[kSelIt],
                        const float *kbi, const float *klw, const float *krb,
                        uint32_t o0, uint32_t o1) {
    EmitRes e{0u, 0u, 0u, 0u, {0.0, 0.0, 0.0, 0.0}};
    uint32_t n0 = 0u, n1 = 0u;
#pragma unroll
    for (int k = 0; k < kSelIt; ++k) {
      if (!(rb[k] < 1.0f)) continue;
      if (kb[k] >= lo0) ++n0;
      else if (kb[k] >= lo) ++n1;
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<uint32_t>(n0 | (n1 << 16), s_scan, &tot);
    uint32_t a0 = o0 + (ex & 0xFFFFu), a1 = c0 + o1 + (ex >> 16);
#pragma unroll
    for (int k = 0; k < kSelIt; ++k) {
      if (!(rb[k] < 1.0f)) continue;
      uint32_t slot;
      if (kb[k] >= lo0) {
        slot = a0++;
      } else {
        // the token's float64 terms (v_i squared in float64) and b_i
        double bd, vd;
        float tb;
        if (kbi) {
          bd = (double)kbi[k];
          vd = (double)klw[k] * (double)klw[k] * (double)qr_of(rb[k]);
          tb = krb[k];
        } else {
          const Terms t = token_terms_w(wb[k], rb[k], lr, key_pos(kb[k]));
          direct_terms(t, bd, vd);
          tb = t.rb;
        }
        if (kb[k] >= lo) {
          e.d[2] += bd;
          e.d[3] += vd;
          e.bl1 = OpMax<uint32_t>::f(e.bl1, __float_as_uint(tb));
          slot = a1++;
        } else {
          e.d[0] += bd;
          e.d[1] += vd;
          e.bl = OpMax<uint32_t>::f(e.bl, __float_as_uint(tb));
          continue;
        }
      }
      if (slot < (uint32_t)capw) {
        p.candk[seg + slot] = kb[k];
        p.candw[seg + slot] = wb[k];
        p.candq[seg + slot] = rb[k];
      }
    }
    e.t0 = tot & 0xFFFFu;
    e.t1 = tot >> 16;
    return e;
  };
  auto take = [&](const EmitRes &e) {
    o0 += e.t0;
    o1 += e.t1;
    below = OpMax<uint32_t>::f(below, e.bl);
    below1 = OpMax<uint32_t>::f(below1, e.bl1);
#pragma unroll
    for (int k = 0; k < 4; ++k) dsum[k] += e.d[k];
  };
  if constexpr (KEEP)
    take(emit_batch(key8, r8, s8, bi8, lw8, rb8, o0, o1));
  else
    take(emit_batch(key8, r8, s8, nullptr, nullptr, nullptr, o0, o1));
  for (int it0 = kSelIt; it0 < iters; it0 += kSelIt) {
    float rb[kSelIt], sb[kSelIt];
    unsigned long long kb[kSelIt];
    load_batch(it0, rb, sb);
#pragma unroll
    for (int k = 0; k < kSelIt; ++k) {
      kb[k] = 0ull;
      if (!(rb[k] < 1.0f)) continue;
      Terms t;
      kb[k] = key_of(pos_of(it0 + k), rb[k], sb[k], t);
      sb[k] = t.wt;
    }
    take(emit_batch(kb, rb, sb, nullptr, nullptr, nullptr, o0, o1));
  }
  // the workgroup's totals in one LDS round (thread 0 writes them): each
  // value folded per wave, the waves combined in wave order
  {
    constexpr int W = kBlock / kWave;
    __shared__ double s_fd[W][6];
    __shared__ uint32_t s_fb[W][2];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    double fd[6] = {tx[0], tx[1], dsum[0], dsum[1], dsum[2], dsum[3]};
#pragma unroll
    for (int k = 0; k < 6; ++k) fd[k] = wave_fold<double, OpSum<double>>(fd[k]);
    const uint32_t b0 = wave_fold<uint32_t, OpMax<uint32_t>>(below);
    const uint32_t b1 = wave_fold<uint32_t, OpMax<uint32_t>>(below1);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < 6; ++k) s_fd[wave][k] = fd[k];
      s_fb[wave][0] = b0;
      s_fb[wave][1] = b1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        fd[k] = s_fd[0][k];
#pragma unroll
        for (int w = 1; w < W; ++w) fd[k] = OpSum<double>::f(fd[k], s_fd[w][k]);
      }
      below = s_fb[0][0];
      below1 = s_fb[0][1];
#pragma unroll
      for (int w = 1; w < W; ++w) {
        below = OpMax<uint32_t>::f(below, s_fb[w][0]);
        below1 = OpMax<uint32_t>::f(below1, s_fb[w][1]);
      }
      tx[0] = fd[0];
      tx[1] = fd[1];
#pragma unroll
      for (int k = 0; k < 4; ++k) dsum[k] = fd[2 + k];
    }
  }
  if (threadIdx.x == 0) {
    // per tier: candidates, bound, and over the tokens not written in that
    // tier the max of b_i and the float64 sums
    const size_t at = (size_t)row * kSelWG + s;
    p.ccount[2 * at] = min(o0, c0);
    p.ccount[2 * at + 1] = min(c0 + o1, (uint32_t)capw);
    p.clo[2 * at] = lo0;
    p.clo[2 * at + 1] = lo;
    p.rpart[2 * at] = max(below, below1);
    p.rpart[2 * at + 1] = below;
    p.dpart[4 * at] = dsum[0] + dsum[2];
    p.dpart[4 * at + 1] = dsum[1] + dsum[3];
    p.dpart[4 * at + 2] = dsum[0];
    p.dpart[4 * at + 3] = dsum[1];
    p.tpart[2 * at] = (unsigned long long)tx[0];
    p.tpart[2 * at + 1] = (unsigned long long)tx[1];
  }
}

// Candidate select: per-bin counts, fixed-point sums of beta_i and v_i and
// the max of b_i over eight key bits at a time.
constexpr int kWalkBins = 256;
struct WalkBin {
  uint32_t cnt, bmax;
  unsigned long long bsum, vsum;
};

union WalkLds {
  struct {
    unsigned long long key[kCandMax];
    float w[kCandMax];  // w~ and r: every term is recomputed from them
    float r[kCandMax];
    WalkBin bin[kWalkBins];
  } c;
  SelLds sel;
};

// State of the candidate select between its levels.
struct WalkState {
  unsigned long long pre;     // key bits above the current digit
  unsigned long long ab, av;  // fixed-point sums fetched above the bracket
  unsigned long long T;       // F_h = keys >= T, once done
  uint32_t ac;                // candidates fetched above the bracket
  uint32_t bmax;              // max b_i certainly left in the rest
  int32_t off, w;             // current digit: key bits [off, off + w)
  int32_t done, kstar;
};

// One 1024-thread workgroup per fetching row: the stopping rule (eq. 10)
// over the collected candidates by a radix select. Each level bins the
// candidates inside the current bracket by eight key bits; with the fetched
// part F(j) = (fetched above) + (bins >= j), eps^ of L \ F(j) falls as j
// falls, and the highest bin j* with eps^ < eps holds the last token of
// F_h: if it holds one candidate that is k*, otherwise j* becomes the
// bracket of the next level. F_h minus S then goes into the KV head's fetch
// bitmap. When the candidates cannot certify the row it runs the streaming
// selection instead.
template <int GRP>
__global__ __launch_bounds__(kPlanThreads) void dk_rwalk(DParams p) {
  const int hq = blockIdx.x, b = blockIdx.y;
  const int row = b * p.Hq + hq, bg = b * p.G + hq / GRP;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  __shared__ WalkLds lds;
  __shared__ RowState rs;
  __shared__ WalkState ws;
  __shared__ uint32_t s_wc[kSelWG], s_off[kSelWG];
  __shared__ unsigned long long s_tot[2], s_lomax;
  __shared__ uint32_t s_below;
  __shared__ double s_dsum[2];
  __shared__ int s_nc;
  // the row and the candidate workgroups' summaries of both tiers
  const size_t cb0 = (size_t)row * kCandMax;
  if (threadIdx.x == 0) rs = p.rows[row];
  __shared__ uint32_t s_pc[2][kSelWG], s_pb[2][kSelWG];
  __shared__ unsigned long long s_plo[2][kSelWG], s_pt[2][kSelWG];
  __shared__ double s_pd[4][kSelWG];
  // the KV head's resident positions as a bitmap (for F_h minus S), built
  // while the candidates are loaded
  __shared__ uint32_t s_res[kMaxTokens / 32];
  for (int i = threadIdx.x; i < p.nwords; i += kPlanThreads) s_res[i] = 0u;
  const int nsel = p.nsel, capw = cand_cap(p);
  if (threadIdx.x < nsel) {
    const int j = threadIdx.x;
    const size_t at = (size_t)row * kSelWG + j;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s_pc[t][j] = p.ccount[2 * at + t];
      s_plo[t][j] = p.clo[2 * at + t];
      s_pb[t][j] = p.rpart[2 * at + t];
      s_pt[t][j] = p.tpart[2 * at + t];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) s_pd[k][j] = p.dpart[4 * at + k];
  }
  __syncthreads();
  if (!rs.fetch) return;
  {
    const int cnt = max(0, min(p.rcount[bg], p.cap));
    const int32_t *ridx = p.ridx + (size_t)bg * p.cap;
    for (int j = threadIdx.x; j < cnt; j += kPlanThreads) {
      const int pos = ridx[j];
      if (pos >= 0 && pos < p.n) atomicOr(&s_res[pos / 32], 1u << (pos % 32));
    }
  }
  const double a = p.a_delta, l = p.l_delta;
  const int eb = rs.eb, ev = rs.ev;
  const double capb = rs.capb, capv = rs.capv;
  const double sbs = ldexp(1.0, -eb), svs = ldexp(1.0, -ev);
  const LamRule lr = lam_rule((float)rs.beta, p.est, rs.bkey);
  // Tier 0 holds each workgroup's top capw / 4 keys, tier 1 all capw; the
  // larger set is only walked when the smaller one cannot decide the row.
#pragma unroll 1
  for (int tier = 0; tier < 2; ++tier) {
    const int cap = tier == 0 ? capw / 4 : capw;
    if (wave == 0) {
      const bool on = lane < nsel;
      const int j = on ? lane : 0;
      const uint32_t c = on ? s_pc[tier][j] : 0u;
      const uint32_t incl = wave_incl_scan<uint32_t>(c, lane);
      if (on) {
        s_wc[lane] = c;
        s_off[lane] = incl - c;
      }
      const unsigned long long tb = wave_sum(on ? s_pt[0][j] : 0ull),
                               tv = wave_sum(on ? s_pt[1][j] : 0ull);
      const double db = wave_sum(on ? s_pd[2 * tier][j] : 0.0),
                   dv = wave_sum(on ? s_pd[2 * tier + 1][j] : 0.0);
      const uint32_t bl = wave_max(on ? s_pb[tier][j] : 0u);
      const unsigned long long lm = wave_max(on ? s_plo[tier][j] : 0ull);
      if (lane == kWave - 1) s_nc = (int)incl;
      if (lane == 0) {
        s_tot[0] = tb;
        s_tot[1] = tv;
        s_below = bl;
        s_lomax = lm;
        s_dsum[0] = db;
        s_dsum[1] = dv;
      }
    }
    __syncthreads();
    const int nc = s_nc;
    const unsigned long long tot_b = s_tot[0], tot_v = s_tot[1];
    const uint32_t below = s_below;
    // the tier's candidates into LDS (loads first), their fixed-point sums
    unsigned long long cs[2] = {0ull, 0ull};
    unsigned long long kmin = ~0ull, kmax = 0ull;
    for (int q0 = 0; q0 < nsel * cap; q0 += kPlanThreads * 2) {
      unsigned long long ck[2];
      float cw[2], cq[2];
      int dst[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = q0 + u * kPlanThreads + (int)threadIdx.x;
        const int sw = idx / cap, slot = idx % cap;
        dst[u] = -1;
        if (idx < nsel * cap && slot < (int)s_wc[sw]) {
          const size_t at = cb0 + (size_t)sw * capw + slot;
          ck[u] = p.candk[at];
          cw[u] = p.candw[at];
          cq[u] = p.candq[at];
          dst[u] = (int)s_off[sw] + slot;
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (dst[u] < 0) continue;
        lds.c.key[dst[u]] = ck[u];
        lds.c.w[dst[u]] = cw[u];
        lds.c.r[dst[u]] = cq[u];
        const Terms t = token_terms_w(cw[u], cq[u], lr, key_pos(ck[u]));
        cs[0] += sat_fx(t.bi, capb, eb);
        cs[1] += sat_fx(t.vi, capv, ev);
        kmin = min(kmin, ck[u]);
        kmax = max(kmax, ck[u]);
      }
    }
    {  // the candidates' sums and key range in one LDS round
      unsigned long long red[4] = {cs[0], cs[1], kmax, ~kmin};
      plan_sum2_max2(red);
      cs[0] = red[0];
      cs[1] = red[1];
      kmax = red[2];
      kmin = ~red[3];
    }
    // fetching every candidate leaves exactly the tokens not written
    const double e_below =
        eps_of((double)(tot_b - cs[0]) * sbs, (double)(tot_v - cs[1]) * svs,
               (double)__uint_as_float(below), rs.dnorm, a, l);
    if (!(e_below < (double)p.eps) || nc == 0) {
      __syncthreads();
      continue;
    }
    if (threadIdx.x == 0) {
      // the first digit starts where the candidates' keys start to differ
      const int span = kmax == kmin ? 0 : 64 - __clzll((long long)(kmax ^ kmin));
      WalkState z{};
      z.off = max(0, span - 8);
      z.w = max(1, span - z.off);
      z.pre = kmax >> (z.off + z.w);
      z.bmax = below;
      ws = z;
    }
    __syncthreads();
    for (int level = 0; level < 10; ++level) {  // at most 7 eight-bit digits
      if (threadIdx.x < kWalkBins) lds.c.bin[threadIdx.x] = WalkBin{0u, 0u, 0ull, 0ull};
      __syncthreads();
      const int off = ws.off, w = ws.w;
      const unsigned long long pre = ws.pre;
      for (int k = threadIdx.x; k < nc; k += kPlanThreads) {
        const unsigned long long key = lds.c.key[k];
        if ((key >> (off + w)) != pre) continue;
        WalkBin &x = lds.c.bin[(int)((key >> off) & ((1ull << w) - 1ull))];
        const Terms t = token_terms_w(lds.c.w[k], lds.c.r[k], lr, key_pos(key));
        atomicAdd(&x.cnt, 1u);
        atomicAdd(&x.bsum, sat_fx(t.bi, capb, eb));
        atomicAdd(&x.vsum, sat_fx(t.vi, capv, ev));
        atomicMax(&x.bmax, __float_as_uint(t.rb));
      }
      __syncthreads();
      if (wave == 0) {
        // lane owns bins 4 lane .. 4 lane + 3
        constexpr int PER = kWalkBins / kWave;
        uint32_t lc = 0u, lmx = 0u;
        unsigned long long lb = 0ull, lv = 0ull;
  #pragma unroll
        for (int q = 0; q < PER; ++q) {
          const WalkBin &x = lds.c.bin[lane * PER + q];
          lc += x.cnt;
          lb += x.bsum;
          lv += x.vsum;
          lmx = max(lmx, x.bmax);
        }
        // sums over the lanes above, max over the lanes below
        uint32_t sc = lc;
        unsigned long long sb = lb, sv = lv;
        for (int o = 1; o < kWave; o <<= 1) {
          const uint32_t xc = __shfl_down(sc, o, kWave);
          const unsigned long long xb = __shfl_down(sb, o, kWave), xv = __shfl_down(sv, o, kWave);
          if (lane + o < kWave) {
            sc += xc;
            sb += xb;
            sv += xv;
          }
        }
        sc -= lc;
        sb -= lb;
        sv -= lv;
        uint32_t pm = lmx;
        for (int o = 1; o < kWave; o <<= 1) {
          const uint32_t x = __shfl_up(pm, o, kWave);
          if (lane >= o) pm = max(pm, x);
        }
        uint32_t mlow = __shfl_up(pm, 1, kWave);
        if (lane == 0) mlow = 0u;
        mlow = max(mlow, ws.bmax);
        // the lane's highest bin whose fetched-through eps^ is below eps
        int best = -1;
        {
          unsigned long long fb = ws.ab + sb, fv = ws.av + sv;
          for (int q = PER - 1; q >= 0 && best < 0; --q) {
            const WalkBin &x = lds.c.bin[lane * PER + q];
            fb += x.bsum;
            fv += x.vsum;
            uint32_t mb = mlow;
            for (int q2 = 0; q2 < q; ++q2) mb = max(mb, lds.c.bin[lane * PER + q2].bmax);
            const double e = eps_of((double)(tot_b - fb) * sbs,
                                    (double)(tot_v - fv) * svs,
                                    (double)__uint_as_float(mb), rs.dnorm, a, l);
            if (x.cnt > 0u && e < (double)p.eps) best = lane * PER + q;
          }
        }
        int top = best;
        for (int o = 32; o >= 1; o >>= 1) top = max(top, __shfl_xor(top, o, kWave));
        if (top < 0) top = 0;  // unreachable: fetching every candidate certifies
        if (lane == top / PER) {
          const int q = top % PER;
          uint32_t c = sc;
          unsigned long long fb = ws.ab + sb, fv = ws.av + sv;
          for (int q2 = PER - 1; q2 > q; --q2) {
            const WalkBin &x = lds.c.bin[lane * PER + q2];
            c += x.cnt;
            fb += x.bsum;
            fv += x.vsum;
          }
          uint32_t mb = mlow;
          for (int q2 = 0; q2 < q; ++q2) mb = max(mb, lds.c.bin[lane * PER + q2].bmax);
          const WalkBin &x = lds.c.bin[top];
          if (x.cnt <= 1u || off == 0) {
            ws.kstar = (int)(ws.ac + c + x.cnt);
            ws.pre = (pre << w) | (unsigned long long)top;  // the last key's digits
            ws.done = 1;
          } else {
            ws.ac += c;
            ws.ab = fb;
            ws.av = fv;
            ws.bmax = mb;
            ws.pre = (pre << w) | (unsigned long long)top;
            const int noff = max(0, off - 8);
            ws.w = off - noff;
            ws.off = noff;
          }
        }
      }
      __syncthreads();
      if (ws.done) break;
    }
    // the last fetched key: the one candidate whose bits above `off` are pre
    {
      const int off = ws.off;
      const unsigned long long pre = ws.pre;
      for (int k = threadIdx.x; k < nc; k += kPlanThreads)
        if ((lds.c.key[k] >> off) == pre) ws.T = lds.c.key[k];
    }
    __syncthreads();
    const unsigned long long T = ws.T;
    // a candidate workgroup may hold keys in [T, its bound) that it did not
    // write: then this tier cannot decide the row
    if (T < s_lomax) {
      __syncthreads();
      continue;
    }
    // mark F_h; eps^(L') from float64 sums over the rest (the candidates
    // below T and the tokens not written), added directly rather than as the
    // total minus the fetched part
    const uint32_t *rbits = s_res;
    uint32_t *fbm = p.fbits + (size_t)bg * p.nwords;
    uint32_t *hb = p.hbits + (size_t)row * p.nwords;
    double dr[2] = {0.0, 0.0};
    uint32_t bm = 0u;
    for (int k = threadIdx.x; k < nc; k += kPlanThreads) {
      const unsigned long long key = lds.c.key[k];
      if (key < T) {
        const Terms t = token_terms_w(lds.c.w[k], lds.c.r[k], lr, key_pos(key));
        double bd, vd;
        direct_terms(t, bd, vd);
        dr[0] += bd;
        dr[1] += vd;
        bm = max(bm, __float_as_uint(t.rb));
        continue;
      }
      const int pos = (int)(0xFFFFFFu - (uint32_t)(key & 0xFFFFFFull));
      atomicOr(hb + pos / 32, 1u << (pos % 32));
      if (!((rbits[pos / 32] >> (pos % 32)) & 1u)) atomicOr(fbm + pos / 32, 1u << (pos % 32));
    }
    {  // the rest's float64 sums and its max b_i in one LDS round, for
       // thread 0: each folded per wave, the waves combined in wave order
      __shared__ double s_dr[kPlanWaves][2];
      __shared__ uint32_t s_bm[kPlanWaves];
      const double d0 = wave_fold<double, OpSum<double>>(dr[0]);
      const double d1 = wave_fold<double, OpSum<double>>(dr[1]);
      const uint32_t m0 = wave_fold<uint32_t, OpMax<uint32_t>>(max(bm, below));
      if (lane == 0) {
        s_dr[wave][0] = d0;
        s_dr[wave][1] = d1;
        s_bm[wave] = m0;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        dr[0] = s_dr[0][0];
        dr[1] = s_dr[0][1];
        bm = s_bm[0];
        for (int w = 1; w < kPlanWaves; ++w) {
          dr[0] = OpSum<double>::f(dr[0], s_dr[w][0]);
          dr[1] = OpSum<double>::f(dr[1], s_dr[w][1]);
          bm = OpMax<uint32_t>::f(bm, s_bm[w]);
        }
      }
    }
    if (threadIdx.x == 0) {
      rs.kstar = ws.kstar;
      rs.T = T;
      rs.eps1 = (float)eps_of(dr[0] + s_dsum[0], dr[1] + s_dsum[1],
                              (double)__uint_as_float(bm), rs.dnorm, a, l);
      rs.path = tier == 0 ? VKV_PATH_TOP_CANDIDATES : VKV_PATH_ALL_CANDIDATES;
      p.rows[row] = rs;
    }
    return;
  }
  // neither tier decides the row: the streaming selection
  __syncthreads();
  const SelArgs sa{p.r, p.shat, s_res, p.fbits, p.hbits, p.a_delta,
                   p.l_delta, p.eps, p.n, p.ns, p.nwords, p.est};
  select_row(sa, row, bg, rs, lds.sel);
  __syncthreads();
  if (threadIdx.x == 0) {
    rs.path = VKV_PATH_STREAMING;
    p.rows[row] = rs;
  }
}

// ------------------------------------------------------------ fetch
// Workgroups per KV head that read fetched rows: enough host loads in flight
// for the link, few enough that most compute units stay free for the
// attention over the resident rows running in the same launch (host loads
// queued in a compute unit delay every other load issued there).
constexpr int kGatherWG = 8;        // gather workgroups per KV head
constexpr int kGatherWGSmall = 24;  // ... when the launch has <= 8 KV heads
// Rows per half-wave with loads in flight (a batch in use and the next in
// flight). Measured at 1, 2, 4 and 8: two gave the shortest steps at batch
// 1, 4 and 16 (the launch keeps enough rows in flight for the host link,
// and the host loads queued in a compute unit delay less the loads of a
// resident part sharing it).
constexpr int kGatherBatch = 2;

// Gather and attention over the fetched rows by workgroup j of a KV head:
// rows [j R / ncf, (j + 1) R / ncf) of the KV head's ascending
// fetch list (R rows in all), so every workgroup reads the same number of
// rows wherever they lie. It lists its positions (up to kGatherSeg at a
// time) with, per position, which of the KV head's query heads fetch it,
// writes its part of the fetch list, and reads the rows from pinned host
// memory by GPU loads (zero-copy), 32 lanes (16-byte units, K then V) per
// row, the next batch of rows always in flight while one is used. The K
// lanes form the exact logits of the row for the query heads; for each head
// that fetches the row (F_h) the half-wave folds exp(logit) and the V row
// into a running softmax (shift, sum of weights, weighted sum of V). The
// half-waves are merged at the end into the workgroup's partial, index
// ncr + j.
// The 16-byte unit `unit` of a listed row: from the previous step's staging
// (sl >= 0) or this step's read-ahead (sl <= -2) when either holds it, else
// from host memory (sl == -1).
__device__ __forceinline__ const uint4 *gather_row(int sl, int pos,
                                                   const uint16_t *stg,
                                                   const uint16_t *host,
                                                   const uint16_t *spec,
                                                   int unit) {
  const uint16_t *base = sl >= 0 ? stg + (size_t)sl * 2 * kHeadDim
                       : sl == -1 ? host + (size_t)pos * 2 * kHeadDim
                                  : spec + (size_t)(-2 - sl) * 2 * kHeadDim;
  return reinterpret_cast<const uint4 *>(base + unit * 8);
}
constexpr int kGatherSeg = 4096;   // listed positions held at a time
constexpr int kGatherWPT = 16;     // bitmap words per thread: n <= 2^17
template <int GRP>
__device__ __forceinline__ void gather_attend(const DParams &p, int j, int g,
                                              int b) {
  const int bg = b * p.G + g;
  const int hw = threadIdx.x / 32;          // half-wave: one row at a time
  const int unit = threadIdx.x % 32;        // 16-byte unit of the row
  const bool is_v = unit >= 16;
  const int dim0 = (unit & 15) * 8;
  constexpr int HW = kBlock / 32;
  constexpr int STEP = HW * kGatherBatch;   // rows per batch of the workgroup
  __shared__ int s_pos[kGatherSeg];
  __shared__ int s_src[kGatherSeg];  // index in stage_prev; -1: host; -2 - k: row k read ahead
  __shared__ uint8_t s_msk[kGatherSeg];
  __shared__ uint32_t s_red[kBlock / kWave + 1];
  __shared__ float s_m[HW][GRP], s_d[HW][GRP];
  __shared__ float s_o[HW][GRP][kHeadDim];
  // this thread's bitmap words [w0, w0 + wpt) and their counts
  const int wpt = (p.nwords + kBlock - 1) / kBlock;  // <= kGatherWPT (host check)
  const int w0 = (int)threadIdx.x * wpt;
  const uint32_t *fb = p.fbits + (size_t)bg * p.nwords;
  uint32_t words[kGatherWPT];
  uint32_t mine = 0;
#pragma unroll
  for (int k = 0; k < kGatherWPT; ++k) {
    words[k] = (k < wpt && w0 + k < p.nwords) ? fb[w0 + k] : 0u;
    mine += (uint32_t)__popc(words[k]);
  }
  float qv[GRP][8];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(
        p.q + (size_t)row_of(p, b, g, h, GRP) * kHeadDim + dim0);
    unpack8(raw, qv[h]);
  }
  uint32_t total = 0;
  const uint32_t before = block_exclusive_scan<uint32_t>(mine, s_red, &total);
  // this workgroup's share of the list, within fetch_cap (rows past it are
  // neither listed nor read; the status says so)
  int lo_i, hi_i;
  split_range((int)total, p.ncf, j, lo_i, hi_i);
  const uint32_t lo = (uint32_t)lo_i;
  const uint32_t hi = min((uint32_t)hi_i, (uint32_t)p.fetch_cap);
  float mrun[GRP], dsum[GRP], acc[GRP][8];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    mrun[h] = -INFINITY;
    dsum[h] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[h][k] = 0.0f;
  }
  const uint16_t *src_base = p.host_kv + (size_t)bg * p.ns * 2 * kHeadDim;
  const uint16_t *stg_base =
      p.stage_prev ? p.stage_prev + (size_t)bg * p.fetch_cap * 2 * kHeadDim : nullptr;
  const uint16_t *spec_base =
      p.spec_m > 0 ? p.spec_kv + (size_t)bg * p.spec_m * 2 * kHeadDim : nullptr;
  int32_t *fidx = p.fidx + (size_t)bg * p.fetch_cap;

  uint32_t n_host = 0u;  // rows this thread listed that come from host memory
  for (uint32_t seg = lo; seg < hi; seg += kGatherSeg) {
    const uint32_t seg_hi = min(hi, seg + (uint32_t)kGatherSeg);
    // ---- list the positions with list index in [seg, seg_hi): each
    // thread the set bits of its own words, with no loads; then, one list
    // entry per thread at a time, which query heads fetch it and whether
    // the previous step staged it (all those loads issued together, not one
    // dependent round trip per listed position)
    {
      uint32_t gi = before;
#pragma unroll
      for (int k = 0; k < kGatherWPT; ++k) {
        uint32_t x = words[k];
        const uint32_t cnt = (uint32_t)__popc(x);
        if (gi + cnt > seg && gi < seg_hi) {
          while (x) {
            const int bit = __ffs(x) - 1;
            if (gi >= seg && gi < seg_hi) s_pos[gi - seg] = (w0 + k) * 32 + bit;
            ++gi;
            x &= x - 1;
          }
        } else {
          gi += cnt;
        }
      }
    }
    __syncthreads();
    const uint32_t nrow = seg_hi - seg;
    for (uint32_t k = threadIdx.x; k < nrow; k += kBlock) {
      const int pos = s_pos[k];
      const int wi = pos / 32, bit = pos % 32;
      uint32_t msk = 0u;
#pragma unroll
      for (int h = 0; h < GRP; ++h)
        msk |= ((p.hbits[(size_t)row_of(p, b, g, h, GRP) * p.nwords + wi] >> bit) & 1u) << h;
      int sl = -1;
      if (p.smap_prev) {
        sl = p.smap_prev[(size_t)bg * p.ns + pos];
        if (sl < 0 || sl >= p.fetch_cap) sl = -1;
      }
      if (p.spec_m > 0) {  // read ahead this step: slot -2 - sl of spec_kv
        const uint32_t wb = p.sp_bits[(size_t)bg * p.nwords + wi];
        const uint32_t w0s = p.sp_base[(size_t)bg * p.nwords + wi];
        if (sl < 0 && ((wb >> bit) & 1u))
          sl = -2 - (int)(w0s + (uint32_t)__popc(wb & ((1u << bit) - 1u)));
      }
      n_host += sl == -1 ? 1u : 0u;
      s_src[k] = sl;
      s_msk[k] = (uint8_t)msk;
    }
    __syncthreads();
    for (uint32_t k = threadIdx.x; k < nrow; k += kBlock) {
      fidx[seg + k] = s_pos[k];
      if (p.smap_next) p.smap_next[(size_t)bg * p.ns + s_pos[k]] = (int32_t)(seg + k);
    }
    uint16_t *stg_next =
        p.stage_next ? p.stage_next + (size_t)bg * p.fetch_cap * 2 * kHeadDim : nullptr;
    // ---- rows: batch r0 in use while batch r0 + STEP is in flight
    uint4 cur[kGatherBatch], nxt[kGatherBatch];
#pragma unroll
    for (int it = 0; it < kGatherBatch; ++it) {
      const uint32_t rk = it * HW + hw;
      if (rk < nrow) cur[it] = *gather_row(s_src[rk], s_pos[rk], stg_base, src_base, spec_base, unit);
    }
    for (uint32_t r0 = 0; r0 < nrow; r0 += STEP) {
#pragma unroll
      for (int it = 0; it < kGatherBatch; ++it) {
        const uint32_t rk = r0 + STEP + it * HW + hw;
        if (rk < nrow) nxt[it] = *gather_row(s_src[rk], s_pos[rk], stg_base, src_base, spec_base, unit);
      }
#pragma unroll
      for (int it = 0; it < kGatherBatch; ++it) {
        const uint32_t rk = r0 + it * HW + hw;
        if (rk >= nrow) continue;  // (uniform over the half-wave)
        if (stg_next)  // this step's staging: the row at its list index
          reinterpret_cast<uint4 *>(stg_next + (size_t)(seg + rk) * 2 * kHeadDim)[unit] = cur[it];
        float x[8];
        unpack8(cur[it], x);
        const uint32_t msk = s_msk[rk];
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
          float dp = 0.0f;
          if (!is_v) {
#pragma unroll
            for (int k = 0; k < 8; ++k) dp = __builtin_fmaf(qv[h][k], x[k], dp);
          }
          dp = group_sum<16>(dp);
          // the V lanes take the logit from the K lanes of their row
          const float lg = __shfl(dp, (int)(threadIdx.x % kWave) & ~16, kWave) * kInvSqrtD;
          if (!((msk >> h) & 1u)) continue;
          const float mn = fmaxf(mrun[h], lg);
          const float sc = expf(mrun[h] - mn);
          const float wgt = expf(lg - mn);
          dsum[h] = dsum[h] * sc + wgt;
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[h][k] = __builtin_fmaf(wgt, x[k], acc[h][k] * sc);
          mrun[h] = mn;
        }
      }
#pragma unroll
      for (int it = 0; it < kGatherBatch; ++it) cur[it] = nxt[it];
    }
    __syncthreads();  // s_pos and s_msk are rewritten by the next segment
  }
  // merge the half-waves' running sums into the workgroup's partial
  if (unit == 16) {
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      s_m[hw][h] = mrun[h];
      s_d[hw][h] = dsum[h];
    }
  }
  if (is_v) {
#pragma unroll
    for (int h = 0; h < GRP; ++h)
#pragma unroll
      for (int k = 0; k < 8; ++k) s_o[hw][h][dim0 + k] = acc[h][k];
  }
  __syncthreads();
  const int x = p.ncr + j, np = p.ncr + p.ncf;
  for (int i = threadIdx.x; i < GRP * kHeadDim; i += kBlock) {
    const int h = i / kHeadDim, e = i % kHeadDim;
    float mx = -INFINITY;
    for (int s = 0; s < HW; ++s) mx = fmaxf(mx, s_d[s][h] > 0.0f ? s_m[s][h] : -INFINITY);
    float o = 0.0f, d = 0.0f;
    for (int s = 0; s < HW; ++s) {
      if (!(s_d[s][h] > 0.0f)) continue;
      const float sc = expf(s_m[s][h] - mx);
      o += s_o[s][h][e] * sc;
      d += s_d[s][h] * sc;
    }
    const int row = row_of(p, b, g, h, GRP);
    p.aparto[((size_t)row * kHeadDim + e) * p.npad + x] = o;
    if (e == 0) p.apart[(size_t)row * np + x] = make_float2(mx, d);
  }
  // bytes read from host memory: the rows not found in the staging
  const uint32_t moved = block_sum<uint32_t>(n_host, s_red);
  if (threadIdx.x == 0 && moved > 0u)
    atomicAdd(p.host_bytes, (unsigned long long)moved * 2ull * kHeadDim * 2ull);
  if (j == p.ncf - 1 && threadIdx.x == 0) {
    p.fcount[bg] = (int32_t)total;
    if (total > (uint32_t)p.fetch_cap) atomicOr(p.status, VKV_STATUS_FETCH_OVERFLOW);
  }
}

// ------------------------------------------------------------ read-ahead
// Speculative host reads while the planning passes run (a second stream,
// joined before the gather). A query head fetches a prefix of its gain
// order (eqs. 9-10), and a token's gain grows with its share w~_i / D~ of
// the plug-in denominator and with 1 - r_i (the bias and variance terms of
// Lemma 1 vanish as r_i -> 1). So the tokens of L outside S with the largest
//   score_i = max_h (s_hi - m_h - log D~_L,h) + log(1 - r_i),
// up to spec_m per KV head, are copied from host memory into a device area
// before the decision; the gather takes a listed row from there when it
// finds it. A row is the same bytes wherever it is read from, so no output
// depends on the read-ahead; a row read ahead but not fetched costs only
// host-link time that the planning leaves idle.
constexpr float kSpecBinScale = 32.0f;  // (bin 1023 takes every score < -32)
constexpr int kSpecRun = 64;            // tokens sampled per kChunk tokens
constexpr int kSpecUnroll = 8;          // samples per thread in flight
// Rows in flight for the copy: 32 workgroups x 8 half-waves x 2 rows, about
// 256 KB, what the host link needs to stay busy. More (64 x 8 x 8) flooded
// the memory path and held up the planning launches' HBM loads on every
// compute unit (c2 step 0.196 against 0.163 ms).
constexpr int kSpecMoveUnroll = 2;      // rows per half-wave in flight
constexpr int kSpecMovers = 32;         // copying workgroups (compute units)
// dynamic LDS each copying workgroup asks for: with its own few bytes it
// leaves less of a compute unit's 160 KB free than the smallest planning
// workgroup needs (8.4 KB), so no planning workgroup fits beside it
constexpr int kSpecMoveLds = 156 * 1024;

__device__ __forceinline__ int spec_bin(float sc) {
  const float x = fminf(fmaxf(-sc * kSpecBinScale, 0.0f), (float)(kSpecBins - 1));
  return (int)x;
}

// kSpecUnroll samples of a thread (sample k is token (k / kSpecRun) kChunk
// + k % kSpecRun): position (-1: none), r and the group's plan logits.
template <int GRP, int U>
__device__ __forceinline__ void spec_samples(const DParams &p, int b, int g,
                                             int s0, int nsamp,
                                             int (&ii)[U],
                                             float (&rv)[U],
                                             float (&sv)[U][GRP]) {
  const float *rr = p.r + (size_t)(b * p.G + g) * p.ns;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int sidx = s0 + u * kBlock + (int)threadIdx.x;
    const int i = (sidx / kSpecRun) * kChunk + sidx % kSpecRun;
    ii[u] = sidx < nsamp && i < p.n ? i : -1;
    rv[u] = ii[u] >= 0 ? rr[i] : 1.0f;
#pragma unroll
    for (int h = 0; h < GRP; ++h)
      sv[u][h] = ii[u] >= 0 ? p.shat[(size_t)row_of(p, b, g, h, GRP) * p.n + i] : 0.0f;
  }
}

// m_h + log D~_L,h of the group's query heads into s_c (LDS), from the scan
// chunks' pass-0 records (one wave per head; +inf for a head without
// weight on L). Ends with a workgroup barrier.
constexpr int kSpecRecPerLane = kMaxTokens / kChunk / kWave;
template <int GRP>
__device__ __forceinline__ void spec_norms(const DParams &p, int b, int g,
                                           float *s_c) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  constexpr int W = kBlock / kWave;
  const int np = p.nch + p.nrr;
  for (int h = wave; h < GRP; h += W) {
    const int row = row_of(p, b, g, h, GRP);
    float pm[kSpecRecPerLane], pw[kSpecRecPerLane];
#pragma unroll
    for (int k = 0; k < kSpecRecPerLane; ++k) {
      const int t = lane + k * kWave;
      pm[k] = t < p.nch ? p.pmax[(size_t)row * np + t] : -INFINITY;
      pw[k] = t < p.nch ? (float)p.p0part[((size_t)row * np + t) * 4] : 0.0f;
    }
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kSpecRecPerLane; ++k) m = fmaxf(m, pm[k]);
    m = wave_fold<float, OpMax<float>>(m);
    float sw = 0.0f;
#pragma unroll
    for (int k = 0; k < kSpecRecPerLane; ++k)
      if (pw[k] > 0.0f) sw += pw[k] * __expf(pm[k] - m);
    sw = wave_fold<float, OpSum<float>>(sw);
    if (lane == 0) s_c[h] = sw > 0.0f ? m + __logf(sw) : INFINITY;
  }
  __syncthreads();
}

// Per kSpecHistSamples samples of a KV head (sample k is token (k /
// kSpecRun) kChunk + k % kSpecRun: the first kSpecRun tokens of every
// kChunk): their scores into the group's histogram (cleared by the front
// launch), and this workgroup's share of the resident list into the group's
// bitmap of S (cleared likewise). The samples are loaded before anything
// else; the histogram counts the tokens of L, S included.
constexpr int kSpecHistUnroll = 2;
constexpr int kSpecHistSamples = kBlock * kSpecHistUnroll;
constexpr int kSpecResUnroll = 8;
template <int GRP>
__global__ __launch_bounds__(kBlock) void sp_hist(DParams p) {
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z, bg = b * p.G + g;
  __shared__ float s_c[GRP];
  __shared__ uint32_t s_hist[kSpecBins];
  const int nsamp = (p.n + kChunk - 1) / kChunk * kSpecRun;
  int ii[kSpecHistUnroll];
  float rv[kSpecHistUnroll], sv[kSpecHistUnroll][GRP];
  spec_samples<GRP, kSpecHistUnroll>(p, b, g, j * kSpecHistSamples, nsamp, ii, rv, sv);
  const int cnt = min(p.rcount[bg], p.cap);
  int k0, k1;
  split_range(max(cnt, 0), (int)gridDim.x, j, k0, k1);
  const int32_t *ri = p.ridx + (size_t)bg * p.cap;
  // each thread a run of kSpecResUnroll consecutive entries of the
  // (ascending) resident list: the bits of a run that share a bitmap word
  // go out in one atomic
  int rp[kSpecResUnroll];
  const int kr = k0 + (int)threadIdx.x * kSpecResUnroll;
#pragma unroll
  for (int u = 0; u < kSpecResUnroll; ++u) rp[u] = kr + u < k1 ? ri[kr + u] : -1;
  for (int i = threadIdx.x; i < kSpecBins; i += kBlock) s_hist[i] = 0u;
  spec_norms<GRP>(p, b, g, s_c);
  uint32_t *res = p.sp_res + (size_t)bg * p.nwords;
  auto or_run = [res](const int (&pos)[kSpecResUnroll], int n) {
    int word = -1;
    uint32_t bits = 0u;
#pragma unroll
    for (int u = 0; u < kSpecResUnroll; ++u) {
      const int q = pos[u];
      if (q < 0 || q >= n) continue;
      if (q / 32 != word) {
        if (word >= 0) atomicOr(&res[word], bits);
        word = q / 32;
        bits = 0u;
      }
      bits |= 1u << (q % 32);
    }
    if (word >= 0) atomicOr(&res[word], bits);
  };
  or_run(rp, p.n);
  for (int kb = k0 + kBlock * kSpecResUnroll; kb < k1; kb += kBlock * kSpecResUnroll) {
    const int kt = kb + (int)threadIdx.x * kSpecResUnroll;
#pragma unroll
    for (int u = 0; u < kSpecResUnroll; ++u) rp[u] = kt + u < k1 ? ri[kt + u] : -1;
    or_run(rp, p.n);
  }
  float c[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) c[h] = s_c[h];
#pragma unroll
  for (int u = 0; u < kSpecHistUnroll; ++u) {
    if (ii[u] < 0 || !(rv[u] < 1.0f)) continue;
    float sc = -INFINITY;
#pragma unroll
    for (int h = 0; h < GRP; ++h) sc = fmaxf(sc, sv[u][h] - c[h]);
    sc += __logf(1.0f - rv[u]);
    if (sc == sc) atomicAdd(&s_hist[spec_bin(sc)], 1u);
  }
  __syncthreads();
  uint32_t *gh = p.sp_hist + (size_t)bg * kSpecBins;
  for (int i = threadIdx.x; i < kSpecBins; i += kBlock)
    if (s_hist[i] != 0u) atomicAdd(&gh[i], s_hist[i]);
}

// The score bin at and above which about spec_m tokens of the group lie:
// the last bin (best first) whose cumulative sampled count stays within the
// sample's share of spec_m (at least bin 0). Every workgroup of the group
// forms it from the same histogram, so all agree.
__device__ __forceinline__ int spec_threshold(const DParams &p, int bg,
                                              uint32_t *s_scan, int *s_best) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  constexpr int W = kBlock / kWave;
  constexpr int BPT = kSpecBins / kBlock;
  const uint32_t tgt = (uint32_t)(((long long)p.spec_m * kSpecRun) / kChunk);
  const uint32_t *gh = p.sp_hist + (size_t)bg * kSpecBins;
  uint32_t loc[BPT], mine = 0u;
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    loc[k] = gh[threadIdx.x * BPT + k];
    mine += loc[k];
  }
  uint32_t tot;
  uint32_t run = block_exclusive_scan<uint32_t>(mine, s_scan, &tot);
  int best = -1;
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    run += loc[k];
    if (run <= tgt) best = (int)threadIdx.x * BPT + k;
  }
  best = wave_fold<int, OpMax<int>>(best);
  if (lane == 0) s_best[wave] = best;
  __syncthreads();
  int bb = s_best[0];
#pragma unroll
  for (int w = 1; w < W; ++w) bb = max(bb, s_best[w]);
  return max(bb, 0);
}

// The r, S-bitmap word and plan logits of this thread's tokens of the
// kChunk tokens from t0 (token t0 + k kBlock + thread).
template <int GRP>
__device__ __forceinline__ void spec_chunk(const DParams &p, int b, int g, int t0,
                                           float (&rv)[kChunk / kBlock],
                                           uint32_t (&rw)[kChunk / kBlock],
                                           float (&sv)[kChunk / kBlock][GRP]) {
  const int bg = b * p.G + g;
  const float *rr = p.r + (size_t)bg * p.ns;
  const uint32_t *res = p.sp_res + (size_t)bg * p.nwords;
#pragma unroll
  for (int k = 0; k < kChunk / kBlock; ++k) {
    const int i = t0 + k * kBlock + (int)threadIdx.x;
    const bool in = i < p.n;
    rv[k] = in ? rr[i] : 1.0f;
    rw[k] = in ? res[i / 32] : 0u;
#pragma unroll
    for (int h = 0; h < GRP; ++h)
      sv[k][h] = in ? p.shat[(size_t)row_of(p, b, g, h, GRP) * p.n + i] : 0.0f;
  }
}

// Per spec_cpw consecutive kChunk-token chunks of a KV head (one at batch 1,
// up to kSpecSelMax when the launch would otherwise hold far more
// workgroups than run at once): the tokens of L outside S (and not staged
// by the previous step) whose score bin is within the threshold take slots
// of the KV head's area in position order (one slot counter per KV head,
// one atomic add per workgroup; tokens past spec_m are dropped); their bits
// and each word's first slot are written for the gather, and their
// positions into the KV head's list of rows to read. The next chunk's
// tokens load while one is scored.
constexpr int kSpecSelMax = 8;
template <int GRP>
__global__ __launch_bounds__(kBlock) void sp_sel(DParams p) {
  const int g = blockIdx.y, b = blockIdx.z, bg = b * p.G + g;
  constexpr int NW = kChunk / 32;
  constexpr int TPT = kChunk / kBlock;
  static_assert(TPT * kBlock == kChunk && kBlock == 4 * kWave, "token layout");
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int nw = p.nwords;
  const int nchunk = (p.n + kChunk - 1) / kChunk;
  const int c0 = (int)blockIdx.x * p.spec_cpw;
  const int nc = min(p.spec_cpw, nchunk - c0);  // >= 1 (grid)
  __shared__ uint32_t s_bits[kSpecSelMax * NW], s_keep[kSpecSelMax * NW];
  __shared__ uint32_t s_before[kSpecSelMax * NW];
  __shared__ int s_list[kSpecSelMax * kChunk];
  __shared__ uint32_t s_base;
  __shared__ float s_c[GRP];
  __shared__ uint32_t s_scan[kBlock / kWave + 1];
  __shared__ int s_best[kBlock / kWave];
  float rv[TPT], sv[TPT][GRP], nrv[TPT], nsv[TPT][GRP];
  uint32_t rw[TPT], nrw[TPT];
  spec_chunk<GRP>(p, b, g, c0 * kChunk, rv, rw, sv);
  spec_norms<GRP>(p, b, g, s_c);
  const int thr = spec_threshold(p, bg, s_scan, s_best);
  float cc[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) cc[h] = s_c[h];
  for (int q = 0; q < nc; ++q) {
    const int t0 = (c0 + q) * kChunk;
    if (q + 1 < nc) spec_chunk<GRP>(p, b, g, t0 + kChunk, nrv, nrw, nsv);
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int i = t0 + k * kBlock + (int)threadIdx.x;
      bool sel = false;
      if (i < p.n && rv[k] < 1.0f && !((rw[k] >> (i % 32)) & 1u)) {
        float sc = -INFINITY;
#pragma unroll
        for (int h = 0; h < GRP; ++h) sc = fmaxf(sc, sv[k][h] - cc[h]);
        sc += __logf(1.0f - rv[k]);
        sel = sc == sc && spec_bin(sc) <= thr;
      }
      if (sel && p.smap_prev) {
        const int sl = p.smap_prev[(size_t)bg * p.ns + i];
        sel = !(sl >= 0 && sl < p.fetch_cap);
      }
      const unsigned long long m = __ballot(sel);
      if (lane == 0) {
        s_bits[q * NW + k * (kBlock / 32) + 2 * wave] = (uint32_t)m;
        s_bits[q * NW + k * (kBlock / 32) + 2 * wave + 1] = (uint32_t)(m >> 32);
      }
    }
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      rv[k] = nrv[k];
      rw[k] = nrw[k];
#pragma unroll
      for (int h = 0; h < GRP; ++h) sv[k][h] = nsv[k][h];
    }
  }
  __syncthreads();
  // the words in (chunk, word) order: one per thread, an exclusive prefix of
  // their counts, one slot claim for all of them
  const int nwt = nc * NW;
  static_assert(kSpecSelMax * NW <= kBlock, "one word per thread");
  const uint32_t pc = (int)threadIdx.x < nwt ? (uint32_t)__popc(s_bits[threadIdx.x]) : 0u;
  uint32_t tot;
  uint32_t before = block_exclusive_scan<uint32_t>(pc, s_scan, &tot);
  if (threadIdx.x == 0) s_base = tot > 0u ? atomicAdd(&p.sp_cnt[bg], tot) : 0u;
  __syncthreads();
  const uint32_t base = s_base;
  const uint32_t room = base >= (uint32_t)p.spec_m ? 0u : (uint32_t)p.spec_m - base;
  if ((int)threadIdx.x < nwt) {
    uint32_t bits = s_bits[threadIdx.x];
    // (the rows past the KV head's area: the highest positions go first)
    while (bits != 0u && before + (uint32_t)__popc(bits) > room)
      bits &= ~(1u << (31 - __clz(bits)));
    if (before > room) before = room;
    s_before[threadIdx.x] = before;
    s_keep[threadIdx.x] = bits;
    const int gw = c0 * NW + (int)threadIdx.x;
    if (gw < nw) {
      p.sp_bits[(size_t)bg * nw + gw] = bits;
      p.sp_base[(size_t)bg * nw + gw] = base + before;
    }
  }
  __syncthreads();
  for (int q = 0; q < nc; ++q) {
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int o = q * kChunk + k * kBlock + (int)threadIdx.x, w = o / 32, bit = o % 32;
      const uint32_t wb = s_keep[w];
      if ((wb >> bit) & 1u)
        s_list[s_before[w] + (uint32_t)__popc(wb & ((1u << bit) - 1u))] = c0 * kChunk + o;
    }
  }
  const uint32_t kept = s_before[nwt - 1] + (uint32_t)__popc(s_keep[nwt - 1]);
  __syncthreads();
  int32_t *list = p.sp_list + (size_t)bg * p.spec_m + base;
  for (uint32_t k = threadIdx.x; k < kept; k += kBlock) list[k] = s_list[k];
}

// The rows of every KV head's list, from host memory into the read-ahead
// area, by kSpecMovers workgroups that each hold a whole compute unit (they
// ask for all of its LDS, so no planning workgroup shares a unit with their
// host loads in flight): 32 lanes per row, kSpecMoveUnroll rows per
// half-wave in flight, the rows of all KV heads in one grid-strided loop.
__global__ __launch_bounds__(kBlock) void sp_move(DParams p) {
  const int hw = threadIdx.x / 32, unit = threadIdx.x % 32;
  constexpr int HW = kBlock / 32;
  __shared__ uint32_t s_red[kBlock / kWave];
  const long long total = (long long)p.B * p.G * p.spec_m;
  const long long stride = (long long)gridDim.x * HW;
  uint32_t moved = 0u;
  for (long long t0 = (long long)blockIdx.x * HW + hw; t0 < total;
       t0 += stride * kSpecMoveUnroll) {
    int pos[kSpecMoveUnroll];
    int bgs[kSpecMoveUnroll];
#pragma unroll
    for (int u = 0; u < kSpecMoveUnroll; ++u) {
      const long long t = t0 + u * stride;
      const int bg = (int)(t / p.spec_m), k = (int)(t % p.spec_m);
      const bool ok = t < total && k < (int)min(p.sp_cnt[t < total ? bg : 0], (uint32_t)p.spec_m);
      pos[u] = ok ? p.sp_list[t] : -1;
      bgs[u] = bg;
    }
    uint4 v[kSpecMoveUnroll];
#pragma unroll
    for (int u = 0; u < kSpecMoveUnroll; ++u) {
      v[u] = make_uint4(0u, 0u, 0u, 0u);
      if (pos[u] >= 0)
        v[u] = reinterpret_cast<const uint4 *>(
            p.host_kv + ((size_t)bgs[u] * p.ns + pos[u]) * 2 * kHeadDim)[unit];
    }
#pragma unroll
    for (int u = 0; u < kSpecMoveUnroll; ++u) {
      if (pos[u] < 0) continue;
      const long long t = t0 + u * stride;
      reinterpret_cast<uint4 *>(p.spec_kv + (size_t)t * 2 * kHeadDim)[unit] = v[u];
      moved += unit == 0 ? 1u : 0u;
    }
  }
  moved = block_sum<uint32_t>(moved, s_red);
  if (threadIdx.x == 0 && moved > 0u)
    atomicAdd(p.host_bytes, (unsigned long long)moved * 2ull * kHeadDim * 2ull);
}

// ------------------------------------------------------------ attention
// Partial x < ncr of a KV head's attention: a share of the resident rows,
// written as (shift, sum of weights, weighted sum of V) per head. Rows go in
// batches of kResBatch: first every row's coefficient per head, once (one
// thread per row, the loads of its rows issued together), into LDS; then
// the V rows, 16 lanes per row and kResUnroll rows per lane in flight. (A
// loop that took position, r and the coefficient inside each row's V step
// waited on three dependent loads per row, and behind host reads when the
// compute unit also ran a gather.)
constexpr int kResBatch = 512;
constexpr int kResUnroll = 4;
template <int GRP>
__device__ __forceinline__ void attn_part(const DParams &p, int x, int g,
                                          int b) {
  const int bg = b * p.G + g;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int u = lane % 16;             // 8 dims per lane
  const int slot = threadIdx.x / 16;   // row slot within an iteration
  constexpr int kSlots = kBlock / 16;
  __shared__ RowState s_rs[GRP];
  __shared__ float s_o[kBlock / kWave][GRP][kHeadDim];
  __shared__ float s_d[kBlock / kWave][GRP];
  __shared__ float s_al[kResBatch][GRP];  // coefficients; -1: row skipped
  if (threadIdx.x < GRP) s_rs[threadIdx.x] = p.rows[row_of(p, b, g, threadIdx.x, GRP)];
  __syncthreads();
  const float *rr = p.r + (size_t)bg * p.ns;
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
    constexpr int RPT = kResBatch / kBlock;  // rows per thread in a batch
    for (int c0 = lo; c0 < hi; c0 += kResBatch) {
      const int c1 = min(c0 + kResBatch, hi);
      // the coefficients (w on H and on F_h, lambda w / r on S minus F_h):
      // positions, then r, F_h bits, logits and planning logits of all of
      // this thread's rows, then the arithmetic
      int pos[RPT];
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int j = c0 + k * kBlock + (int)threadIdx.x;
        pos[k] = j < c1 ? ridx[j] : -1;
      }
      float ri[RPT], el[RPT][GRP], sv[RPT][GRP];
      uint32_t fw[RPT][GRP];
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int j = c0 + k * kBlock + (int)threadIdx.x;
        const bool ok = pos[k] >= 0 && pos[k] < p.n;
        const int ps = ok ? pos[k] : 0;
        ri[k] = ok ? rr[ps] : 1.0f;
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
          const int row = row_of(p, b, g, h, GRP);
          el[k][h] = ok ? p.ell[(size_t)row * p.cap + j] : 0.0f;
          fw[k][h] = ok ? p.hbits[(size_t)row * p.nwords + ps / 32] : 0u;
          sv[k][h] = ok ? p.shat[(size_t)row * p.n + ps] : 0.0f;
        }
      }
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int jj = k * kBlock + (int)threadIdx.x;
        if (c0 + jj >= c1) continue;
        const bool ok = pos[k] >= 0 && pos[k] < p.n;
#pragma unroll
        for (int h = 0; h < GRP; ++h) {
          float al = -1.0f;
          if (ok) {
            const RowState &rs = s_rs[h];
            const float w = expf(el[k][h] - rs.m);
            if (ri[k] >= 1.0f || ((fw[k][h] >> (pos[k] % 32)) & 1u)) {
              al = w;
            } else {
              const Terms t = token_terms(sv[k][h], ri[k], rs.m,
                                          lam_rule((float)rs.beta, p.est, rs.bkey), pos[k]);
              al = t.lam * w / ri[k];
            }
            dsum[h] += al;
          }
          s_al[jj][h] = al;
        }
      }
      __syncthreads();
      // the V rows: 16 lanes per row, kResUnroll rows per lane in flight
      const int nb = c1 - c0;
      for (int q0 = 0; q0 < nb; q0 += kSlots * kResUnroll) {
        uint4 raw[kResUnroll];
#pragma unroll
        for (int k = 0; k < kResUnroll; ++k) {
          const int jj = q0 + k * kSlots + slot;
          raw[k] = jj < nb ? *reinterpret_cast<const uint4 *>(
                                 p.rkv + ((size_t)bg * p.cap + c0 + jj) * 2 * kHeadDim +
                                 kHeadDim + u * 8)
                           : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < kResUnroll; ++k) {
          const int jj = q0 + k * kSlots + slot;
          if (jj >= nb || s_al[jj][0] < 0.0f) continue;
          float vv[8];
          unpack8(raw[k], vv);
#pragma unroll
          for (int h = 0; h < GRP; ++h) {
            const float alpha = s_al[jj][h];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(alpha, vv[e], acc[h][e]);
          }
        }
      }
      __syncthreads();  // s_al is rewritten by the next batch
    }
  }
  // reduce the four 16-lane row slots of each wave, then the waves (the
  // weight sums were formed one thread per row: over all 64 lanes)
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float v = acc[h][k];
      v += shfl_xor(v, 16);
      v += shfl_xor(v, 32);
      acc[h][k] = v;
    }
    dsum[h] = wave_sum(dsum[h]);
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
    p.aparto[((size_t)row_of(p, b, g, h, GRP) * kHeadDim + e) * p.npad + x] = o;
  }
  if (threadIdx.x < GRP) {
    const int h = threadIdx.x;
    float d = 0.0f;
    for (int w = 0; w < kBlock / kWave; ++w) d += s_d[w][h];
    p.apart[(size_t)row_of(p, b, g, h, GRP) * np + x] = make_float2(mloc[h], d);
  }
}

// Merge of one row's partial softmax sums by log-sum-exp. Each thread takes
// one output dimension and half of the partials; a dimension's partials are
// consecutive and read as 16-byte vectors, all loads issued first. Partial
// slots past ncr + ncf (padding) are never read into the sum.
__device__ __forceinline__ void attn_merge_row(const DParams &p, int row) {
  const int np = p.ncr + p.ncf;  // at most 56 (32 resident, <= 24 fetched)
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  __shared__ float s_sc[64];
  __shared__ float s_half[kHeadDim];
  __shared__ float s_md[2];
  const int e = threadIdx.x % kHeadDim, half = threadIdx.x / kHeadDim;
  const int nq = p.npad / 4, per = (nq + 1) / 2, q0 = half * per;
  const float4 *src = reinterpret_cast<const float4 *>(
      p.aparto + ((size_t)row * kHeadDim + e) * p.npad);
  float4 v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    v[k] = (k < per && q0 + k < nq) ? src[q0 + k] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const float2 md = (int)threadIdx.x < np ? p.apart[(size_t)row * np + threadIdx.x]
                                          : make_float2(0.0f, 0.0f);
  if (wave == 0) {
    const float M = wave_max(md.y > 0.0f ? md.x : -INFINITY);
    const float sc = md.y > 0.0f ? expf(md.x - M) : 0.0f;
    const float D = wave_sum(md.y * sc);
    s_sc[lane] = sc;
    if (lane == 0) {
      s_md[0] = M;
      s_md[1] = D;
    }
  }
  __syncthreads();
  float o = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (!(k < per && q0 + k < nq)) continue;
    const float *sp = &s_sc[(q0 + k) * 4];
    o += sp[0] != 0.0f ? v[k].x * sp[0] : 0.0f;
    o += sp[1] != 0.0f ? v[k].y * sp[1] : 0.0f;
    o += sp[2] != 0.0f ? v[k].z * sp[2] : 0.0f;
    o += sp[3] != 0.0f ? v[k].w * sp[3] : 0.0f;
  }
  if (half == 1) s_half[e] = o;
  __syncthreads();
  const float M = s_md[0], D = s_md[1];
  if (half == 0) p.out[(size_t)row * kHeadDim + e] = (o + s_half[e]) / D;
  if (threadIdx.x == 0) {
    const RowState &rs = p.rows[row];
    p.d_hat[row] = D;
    p.log_shift[row] = M;
    p.eps_hat0[row] = (float)rs.eps0;
    p.eps_hat[row] = rs.fetch ? rs.eps1 : (float)rs.eps0;
    p.k_star[row] = rs.fetch ? rs.kstar : 0;
    if (p.row_path) p.row_path[row] = rs.fetch ? rs.path : VKV_PATH_NO_FETCH;
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

// The gather (bound by the host link) and the attention over the resident
// rows, which does not depend on it, in one launch: blocks x < ncr take a
// share of the resident rows, the others a share of the fetch bitmap.
// One launch of both kinds of workgroups, every resident part first in
// dispatch order: gather workgroups hold their compute-unit slots for the
// whole transfer, so a resident part queued behind them would start only
// once a gather has ended (at batch 16 the launch holds three times the
// workgroups that fit at once).
template <int GRP>
__global__ __launch_bounds__(kBlock) void dk_fetch(DParams p) {
  const int x = (int)blockIdx.x, nres = p.ncr * p.G * p.B;
  if (x < nres) {
    const int gb = x / p.ncr;
    attn_part<GRP>(p, x % p.ncr, gb % p.G, gb / p.G);
  } else {
    const int y = x - nres, gb = y / p.ncf;
    gather_attend<GRP>(p, y % p.ncf, gb % p.G, gb / p.G);
  }
}

// The merge of each row's partials. Grid (Hq, B).
__global__ __launch_bounds__(kBlock) void dk_attn(DParams p) {
  attn_merge_row(p, (int)blockIdx.y * p.Hq + (int)blockIdx.x);
}

// The caller's timing events: entry k is recorded before the kernel of
// phase k and entry k + 1 after it. When only the two entries of one phase
// are given, its kernel's own dispatch records them (the span of that
// kernel alone, with no marker packets around it).
struct PhaseMark {
  void **ev;
  hipStream_t s;
  int solo;  // the phase whose two entries alone are given, else -1
  PhaseMark(void **e, hipStream_t st, int n) : ev(e), s(st), solo(-1) {
    if (!ev) return;
    int first = -1, count = 0;
    for (int i = 0; i <= n; ++i)
      if (ev[i]) {
        if (first < 0) first = i;
        ++count;
      }
    if (count == 2 && first < n && ev[first + 1]) solo = first;
  }
  void operator()(int k) const {
    const bool own = solo >= 0 && (k == solo || k == solo + 1);
    if (ev && ev[k] && !own)
      (void)hipEventRecord(static_cast<hipEvent_t>(ev[k]), s);
  }
  // a phase with no kernel in this mode: its events as markers
  void empty(int k) const {
    if (k == solo) {
      (void)hipEventRecord(static_cast<hipEvent_t>(ev[k]), s);
      (void)hipEventRecord(static_cast<hipEvent_t>(ev[k + 1]), s);
    }
  }
  // a launch whose completion also records `done` (when given): through the
  // dispatch itself, or with the phase timed alone, a record after it
  template <typename... A>
  void launch_then(int k, hipEvent_t done, void (*f)(A...), dim3 g, dim3 b,
                   A... args) const {
    if (done == nullptr || k == solo) {
      launch(k, f, g, b, args...);
      if (done) (void)hipEventRecord(done, s);
    } else {
      hipExtLaunchKernelGGL(f, g, b, 0, s, nullptr, done, 0u, args...);
    }
  }
  template <typename... A>
  void launch(int k, void (*f)(A...), dim3 g, dim3 b, A... args) const {
    if (k == solo)
      hipExtLaunchKernelGGL(f, g, b, 0, s, static_cast<hipEvent_t>(ev[k]),
                            static_cast<hipEvent_t>(ev[k + 1]), 0u, args...);
    else
      hipLaunchKernelGGL(f, g, b, 0, s, args...);
  }
};

// The second stream of a step that reads ahead and its two events, one set
// per device, made on the first such step on that device (default
// priority; non-blocking, so it waits on nothing but its events). The fork
// event is recorded by the completion of the launch that finishes the
// pass-0 records (no packet of its own on the caller's stream).
struct SpecStream {
  std::mutex mu;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kSpecDevices = 64;
std::mutex g_spec_mu;
SpecStream g_spec[kSpecDevices];

hipError_t spec_stream(SpecStream **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kSpecDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_spec_mu);
  SpecStream &x = g_spec[dev];
  if (x.side == nullptr) {
    int lds = 0;
    e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    if (lds < kSpecMoveLds + 1024) return hipErrorNotSupported;
    hipStream_t sd = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    e = hipStreamCreateWithFlags(&sd, hipStreamNonBlocking);
    // (both order work of this device only: no system-scope fence, whose
    // cache write-back and invalidation would delay the launches after the
    // fork by some microseconds; measured 0.170 against 0.174 ms a step at
    // 1 x 32 x 32K)
    const unsigned flags = hipEventDisableTiming | hipEventDisableSystemFence;
    if (e == hipSuccess) e = hipEventCreateWithFlags(&f, flags);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j, flags);
    if (e != hipSuccess) {
      if (j) (void)hipEventDestroy(j);
      if (f) (void)hipEventDestroy(f);
      if (sd) (void)hipStreamDestroy(sd);
      return e;
    }
    x.fork = f;
    x.join = j;
    x.side = sd;
  }
  *out = &x;
  return hipSuccess;
}

template <int GRP>
hipError_t run(const DParams &p, hipStream_t s, int sd, void **events,
               const SpecStream *sx) {
  const dim3 blk(kBlock);
  const dim3 gfront((unsigned)(p.nch + p.nrr), (unsigned)p.G, (unsigned)p.B);
  constexpr int kPhases = 13;  // the entries of kPhaseNames
  const PhaseMark mark(events, s, kPhases);
  const bool sk2 = p.weights == VKV_W_SKETCH2;
  // the read-ahead forks once the pass-0 records are written: after the
  // front launch, or with the 2-bit sketch after the pass-0 launch
  hipEvent_t fork_front = sx && !sk2 ? sx->fork : nullptr;
  hipEvent_t fork_p0 = sx && sk2 ? sx->fork : nullptr;
  int k = 0;
  mark(k);
  if (p.weights == VKV_W_PERFECT)
    mark.launch_then(k, fork_front, dk_front_exact<GRP>, gfront, blk, p);
  else if (sk2)
    mark.launch(k, dk_front2<GRP>, gfront, blk, p);
  else if (sd == 32)
    mark.launch_then(k, fork_front,
                     p.chunk == kChunk ? dk_front<GRP, 32, kChunk / kBlock * 2>
                                       : dk_front<GRP, 32, 1>,
                     gfront, blk, p);
  else
    mark.launch_then(k, fork_front,
                     p.chunk == kChunk ? dk_front<GRP, 16, kChunk / kBlock>
                                       : dk_front<GRP, 16, 1>,
                     gfront, blk, p);
  mark(++k);
  // 2-bit sketch: the shortlist with its exact logits, then pass 0
  if (sk2)
    mark.launch(k, dk_short<GRP>, dim3((unsigned)p.G, (unsigned)p.B, 1u + kShortSWG),
                dim3(kPlanThreads), p);
  else
    mark.empty(k);
  mark(++k);
  if (sk2)
    mark.launch_then(k, fork_p0, dk_p0<GRP>,
                     dim3((unsigned)p.nch, (unsigned)p.G, (unsigned)p.B), blk, p);
  else
    mark.empty(k);
  mark(++k);
  // the read-ahead on the second stream, beside the planning launches; the
  // gather waits for it
  if (sx) {
    hipError_t e = hipStreamWaitEvent(sx->side, sx->fork, 0);
    if (e != hipSuccess) return e;
    const int nsamp = (p.n + kChunk - 1) / kChunk * kSpecRun;
    hipLaunchKernelGGL(sp_hist<GRP>,
                       dim3((unsigned)((nsamp + kSpecHistSamples - 1) / kSpecHistSamples),
                            (unsigned)p.G, (unsigned)p.B),
                       blk, 0, sx->side, p);
    const int nchunk = (p.n + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(sp_sel<GRP>,
                       dim3((unsigned)((nchunk + p.spec_cpw - 1) / p.spec_cpw),
                            (unsigned)p.G, (unsigned)p.B),
                       blk, 0, sx->side, p);
    hipLaunchKernelGGL(sp_move, dim3((unsigned)kSpecMovers), blk,
                       (size_t)kSpecMoveLds, sx->side, p);
    e = hipEventRecord(sx->join, sx->side);
    if (e != hipSuccess) return e;
  }
  const PhaseMark &pmark = mark;
  const dim3 grow((unsigned)p.nrc, (unsigned)p.Hq, (unsigned)p.B);
  const dim3 gone((unsigned)p.Hq, (unsigned)p.B);
  for (int j = 1; j <= kBetaLaunchMax; ++j) {
    if (j <= p.nbeta)
      pmark.launch(k, dk_rbeta<GRP>, grow, blk, p, j);
    else
      pmark.empty(k);
    pmark(++k);
  }
  if (p.est == VKV_EST_BINARY)
    pmark.launch(k, dk_rbin<GRP>, gone, dim3(kPlanThreads), p);
  else
    pmark.empty(k);
  pmark(++k);
  pmark.launch(k, dk_rcert<GRP>, grow, blk, p);
  pmark(++k);
  {
    // the register-heavy variant only while its grid fits in one round at
    // three waves per SIMD (768 workgroups)
    const dim3 gc((unsigned)p.nsel, (unsigned)p.Hq, (unsigned)p.B);
    if ((long long)p.nsel * p.Hq * p.B <= 768)
      pmark.launch(k, dk_rcand<GRP, true>, gc, blk, p);
    else
      pmark.launch(k, dk_rcand<GRP, false>, gc, blk, p);
  }
  pmark(++k);
  pmark.launch(k, dk_rwalk<GRP>, gone, dim3(kPlanThreads), p);
  pmark(++k);
  if (sx) {
    const hipError_t e = hipStreamWaitEvent(s, sx->join, 0);
    if (e != hipSuccess) return e;
  }
  mark.launch(k, dk_fetch<GRP>,
              dim3((unsigned)((p.ncr + p.ncf) * p.G * p.B)), blk, p);
  mark(++k);
  mark.launch(k, dk_attn, dim3((unsigned)p.Hq, (unsigned)p.B), blk, p);
  mark(++k);
  return hipGetLastError();
}

const char *const kPhaseNames[] = {
    "scan", "shortlist", "pass0", "beta1", "beta2", "beta3", "beta4", "shrink",
    "cert", "cand", "walk", "fetch", "attn"};
static_assert(sizeof(kPhaseNames) / sizeof(kPhaseNames[0]) == 13,
              "one name per phase of run()");

}  // namespace

int decode_phase_count() {
  return (int)(sizeof(kPhaseNames) / sizeof(kPhaseNames[0]));
}

const char *decode_phase_name(int i) {
  return (i >= 0 && i < decode_phase_count()) ? kPhaseNames[i] : nullptr;
}

// Rows per (request, KV head) read ahead: the caller's count, or with -1
// the library's choice: about as many rows as the host link moves while the
// planning launches run, which grow less than linearly with the query
// heads times the context; 6144 * (B Hq n / 2^20)^0.6 rows in all, shared
// by the B G KV heads, within [64, n / 8] each. (Measured with 64 copying
// workgroups: the best of 512-896 rows per KV head at 1 x 32 x 32K, of
// 160-512 at 16 x 32 x 32K and of 768-2048 at 4 x 32 x 128K; the rule
// gives 768, 253 and 1013.)
// With the 2-bit sketch, the exact shortlist already holds the heaviest
// tokens and a small batch fetches a few hundred rows per KV head: the
// fixed cost of the second stream (about 12 us: the fork after the pass-0
// launch, the join before the gather, the compute units held) is then more
// than the read-ahead saves (measured at 1 x 32 x 32K: 0.199 ms with 64 rows
// read ahead against 0.187 ms without; at 16 x 32 x 32K 2.49 against 2.62),
// so there the library's choice is none below B Hq n = 2^23.
int spec_rows(const vkv_decode_args &a) {
  if (a.prefetch_rows >= 0) return std::min(a.prefetch_rows, a.n_tokens);
  const double work = (double)a.batch * a.n_q_heads * a.n_tokens / 1048576.0;
  if (a.weights == VKV_W_SKETCH2 && work < 8.0) return 0;
  const double total = 6144.0 * pow(work, 0.6);
  const double per = total / ((double)a.batch * a.n_kv_heads);
  const int hi = std::max(1, a.n_tokens / 8);
  return std::min(hi, std::max(std::min(64, hi), (int)per));
}

DecodeLayout decode_layout(const vkv_decode_args &a) {
  DecodeLayout L{};
  L.grp = a.n_q_heads / a.n_kv_heads;
  // tokens per scan workgroup: kChunk, or up to 16x more while the launch
  // keeps about 512 workgroups (large batches), so that each workgroup's
  // fixed costs (the projected query, the reductions) cover more tokens
  {
    const long long groups = (long long)a.batch * a.n_kv_heads;
    int mult = 1;
    while (mult < 16 &&
           groups * ((a.n_tokens + 2 * mult * kChunk - 1) / (2 * mult * kChunk)) >= 512)
      mult *= 2;
    L.chunk = kChunk * mult;
  }
  L.nch = (a.n_tokens + L.chunk - 1) / L.chunk;
  // workgroups per group for the resident rows and for the fetched rows:
  // about 512 resident-row workgroups per launch in total, at least 64 rows
  // each
  const long long groups_ll = (long long)a.batch * a.n_kv_heads;
  const int target = (int)((512 + groups_ll - 1) / groups_ll);
  const int rmax = a.cap < a.n_tokens ? a.cap : a.n_tokens;
  // (each at most 32, so the merge sees at most 64 partial sums)
  // (and with the gather workgroups of the same launch, at most one
  // workgroup per compute unit where the batch allows)
  // gather workgroups per KV head: more when the batch is small, so that
  // the KV head with the most rows to fetch keeps enough rows in flight
  // at the end (measured at 8 KV heads with two rows per half-wave in
  // flight: 24 per KV head 1% faster steps than 12 or 32)
  // Beyond one workgroup per compute unit, the launch keeps its workgroups
  // within what runs at once (two per compute unit at the kernel's register
  // and LDS use): gather workgroups hold their slots for the whole
  // transfer, so any workgroup past that count starts only when a gather
  // ends (measured at batch 16: resident parts then ended 190 us after the
  // gathers).
  const long long per_head = std::max<long long>(2, 512 / std::max<long long>(1, groups_ll));
  const int ncf = (int)std::min<long long>(groups_ll <= 8 ? kGatherWGSmall : kGatherWG,
                                           per_head - 1);
  const int fit = (int)(256 / std::max<long long>(1, groups_ll)) - ncf;
  const int room = fit >= 1 ? fit : (int)std::max<long long>(1, per_head - ncf);
  L.ncr = std::max(1, std::min(std::min(std::min(target, 32), room),
                               (rmax + 63) / 64));
  // resident parts of the front launch (the resident logits beside the
  // scan): about 512 per launch, at most 32 per KV head and at least 64
  // rows each, and up to one workgroup per compute unit beside 12 (at most
  // 8 KV heads) or 8 other workgroups per KV head where the batch allows
  // (the front launch's workgroups all run at once at its register use)
  {
    const int other = groups_ll <= 8 ? 12 : 8;
    const int fit_f = (int)(256 / std::max<long long>(1, groups_ll)) - other;
    L.nrr = std::max(1, std::min(std::min(std::min(target, 32), std::max(fit_f, 8)),
                                 (rmax + 63) / 64));
  }
  L.ncf = ncf;
  L.npad = (L.ncr + L.ncf + 3) / 4 * 4;
  L.nwords = (a.n_tokens + 31) / 32;
  // row passes: kRowChunk-token sub-chunks, several per workgroup while a
  // launch keeps about 1024 workgroups (large batches)
  L.nsub = (a.n_tokens + kRowChunk - 1) / kRowChunk;
  {
    const long long rows_ll = (long long)a.batch * a.n_q_heads;
    int rs = 1;
    while (rs < 8 && rows_ll * ((L.nsub + 2 * rs - 1) / (2 * rs)) >= 1024) rs *= 2;
    L.rsub = rs;
  }
  L.nrc = (L.nsub + L.rsub - 1) / L.rsub;
  // candidate workgroups per row (fewer, with more tokens each, measured
  // slower at every batch size: the gain arithmetic per token dominates)
  L.nsel = kSelWG;
  const size_t B = (size_t)a.batch, Hq = (size_t)a.n_q_heads,
               G = (size_t)a.n_kv_heads, n = (size_t)a.n_tokens;
  const size_t rows = B * Hq, groups = B * G;
  Carve c;
  L.rows = c.take<RowState>(rows);
  L.shat = c.take<float>(rows * n);
  L.ell = c.take<float>(rows * (size_t)a.cap);
  L.fstat = c.take<uint32_t>(groups * (L.nch + L.nrr));
  L.fbits = c.take<uint32_t>(groups * L.nwords);
  L.hbits = c.take<uint32_t>(rows * L.nwords);
  L.pmax = c.take<float>(rows * (L.nch + L.nrr));
  L.p0part = c.take<double>(rows * (L.nch + L.nrr) * 4);
  L.hres = c.take<double>(rows * L.nrr);
  L.hpart = c.take<uint32_t>(groups * (L.nch + L.nrr));  // H counts per chunk
  L.bpart = c.take<double>(2 * rows * L.nrc * (size_t)kBetaRec);
  L.band = c.take<float2>(2 * rows * L.nrc * (size_t)kBandChunk);
  L.bstate = c.take<BetaState>(2 * rows);
  L.rbeta = c.take<double>(2 * rows);
  L.binst = c.take<BinState>(rows);
  L.bhist = c.take<uint32_t>(rows * (size_t)kSelBinsP);
  L.bcnt = c.take<uint32_t>(rows * (size_t)L.nrc);
  L.bkeys = c.take<unsigned long long>(rows * (size_t)L.nrc * kBinCap);
  L.bav = c.take<float>(rows * (size_t)L.nrc * kBinCap);
  L.cpart = c.take<CertPart>(rows * L.nrc);
  L.ccount = c.take<uint32_t>(rows * kSelWG * 2);
  L.clo = c.take<unsigned long long>(rows * kSelWG * 2);
  L.tpart = c.take<unsigned long long>(rows * kSelWG * 2);
  L.candk = c.take<unsigned long long>(rows * (size_t)kCandMax);
  L.candw = c.take<float>(rows * (size_t)kCandMax);
  L.candq = c.take<float>(rows * (size_t)kCandMax);
  L.dpart = c.take<double>(rows * (size_t)kSelWG * 4);
  L.rpart = c.take<uint32_t>(rows * kSelWG * 2);
  L.apart = c.take<float2>(rows * (L.ncr + L.ncf));
  L.aparto = c.take<float>(rows * kHeadDim * (size_t)L.npad);
  L.skey = c.take<uint32_t>(groups * n);  // (2-bit sketch only)
  L.spec_m = spec_rows(a);
  if (L.spec_m > 0) {
    L.sp_hist = c.take<uint32_t>(groups * (size_t)kSpecBins);
    L.sp_cnt = c.take<uint32_t>(groups);
    L.sp_res = c.take<uint32_t>(groups * L.nwords);
    L.sp_bits = c.take<uint32_t>(groups * L.nwords);
    L.sp_base = c.take<uint32_t>(groups * L.nwords);
    L.sp_list = c.take<int32_t>(groups * (size_t)L.spec_m);
    L.spec_kv = c.take<uint16_t>(groups * (size_t)L.spec_m * 2 * kHeadDim);
  }
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
  p.row_path = a.row_path;
  p.status = a.status;
  p.sk2_codes = reinterpret_cast<const unsigned long long *>(a.sk2_codes);
  p.sk2_zs = a.sk2_zs;
  p.sk2_chan = a.sk2_chan;
  p.n_short = a.n_short;
  p.shortlist = a.shortlist;
  void *w = a.workspace;
  p.rows = at<RowState>(w, L.rows);
  p.shat = at<float>(w, L.shat);
  p.ell = at<float>(w, L.ell);
  p.fstat = at<uint32_t>(w, L.fstat);
  p.fbits = at<uint32_t>(w, L.fbits);
  p.hbits = at<uint32_t>(w, L.hbits);
  p.pmax = at<float>(w, L.pmax);
  p.p0part = at<double>(w, L.p0part);
  p.hres = at<double>(w, L.hres);
  p.hpart = at<uint32_t>(w, L.hpart);
  p.bpart = at<double>(w, L.bpart);
  p.band = at<float2>(w, L.band);
  p.bstate = at<BetaState>(w, L.bstate);
  p.rbeta = at<double>(w, L.rbeta);
  p.binst = at<BinState>(w, L.binst);
  p.bhist = at<uint32_t>(w, L.bhist);
  p.bcnt = at<uint32_t>(w, L.bcnt);
  p.bkeys = at<unsigned long long>(w, L.bkeys);
  p.bav = at<float>(w, L.bav);
  p.cpart = at<CertPart>(w, L.cpart);
  p.ccount = at<uint32_t>(w, L.ccount);
  p.clo = at<unsigned long long>(w, L.clo);
  p.tpart = at<unsigned long long>(w, L.tpart);
  p.candk = at<unsigned long long>(w, L.candk);
  p.candw = at<float>(w, L.candw);
  p.candq = at<float>(w, L.candq);
  p.dpart = at<double>(w, L.dpart);
  p.rpart = at<uint32_t>(w, L.rpart);
  p.nrc = L.nrc;
  p.nsub = L.nsub;
  p.rsub = L.rsub;
  p.nsel = L.nsel;
  p.apart = at<float2>(w, L.apart);
  p.aparto = at<float>(w, L.aparto);
  p.skey = at<uint32_t>(w, L.skey);
  p.npad = L.npad;
  p.spec_m = L.spec_m;
  {
    // selection workgroups: one chunk each while a launch holds about 512,
    // more chunks per workgroup (at most kSpecSelMax) at large batches
    const long long nchunk = (a.n_tokens + kChunk - 1) / kChunk;
    const long long wgs = (long long)a.batch * a.n_kv_heads * nchunk;
    p.spec_cpw = (int)std::max<long long>(1, std::min<long long>(kSpecSelMax, wgs / 512));
  }
  if (L.spec_m > 0) {
    p.sp_hist = at<uint32_t>(w, L.sp_hist);
    p.sp_cnt = at<uint32_t>(w, L.sp_cnt);
    p.sp_res = at<uint32_t>(w, L.sp_res);
    p.sp_bits = at<uint32_t>(w, L.sp_bits);
    p.sp_base = at<uint32_t>(w, L.sp_base);
    p.sp_list = at<int32_t>(w, L.sp_list);
    p.spec_kv = at<uint16_t>(w, L.spec_kv);
  }
  p.B = a.batch;
  p.Hq = a.n_q_heads;
  p.G = a.n_kv_heads;
  p.n = a.n_tokens;
  p.ns = a.ctx_stride > 0 ? a.ctx_stride : a.n_tokens;
  p.smap_prev = a.stage_map_prev;
  p.stage_prev = a.stage_prev;
  p.smap_next = a.stage_map_next;
  p.stage_next = a.stage_next;
  p.cap = a.cap;
  p.fetch_cap = a.fetch_cap;
  p.nch = L.nch;
  p.nrr = L.nrr;
  p.ncr = L.ncr;
  p.ncf = L.ncf;
  p.nwords = L.nwords;
  p.chunk = L.chunk;
  p.eps = a.eps;
  p.l_delta = log(2.0 / (double)a.delta);
  p.a_delta = p.l_delta / 3.0;
  p.est = a.estimator;
  p.weights = a.weights;
  // planning weights that are exact on the sample (and the shortlist) put
  // far more tokens near the root after one Newton launch than the
  // projected sketch's do (hundreds to tens of thousands against tens), so
  // those modes take a third launch before the band settle
  // (and contexts above 32K tokens one more again)
  p.nbeta = (a.weights == VKV_W_SKETCH ? 2 : 3) + (a.n_tokens > 32768 ? 1 : 0);
  SpecStream *sx = nullptr;
  std::unique_lock<std::mutex> lock;
  if (p.spec_m > 0) {
    const hipError_t e = spec_stream(&sx);
    if (e != hipSuccess) return e;
    // (the fork, the read-ahead launches and the join of one step are
    // enqueued together: the device's second stream and events are shared)
    lock = std::unique_lock<std::mutex>(sx->mu);
  }
  switch (L.grp) {
    case 1: return run<1>(p, s, a.sketch_dim, a.phase_events, sx);
    case 2: return run<2>(p, s, a.sketch_dim, a.phase_events, sx);
    case 4: return run<4>(p, s, a.sketch_dim, a.phase_events, sx);
    case 8: return run<8>(p, s, a.sketch_dim, a.phase_events, sx);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vkv
