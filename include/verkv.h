/*
 * verkv.h -- C ABI of the VerKV hot path on AMD Instinct MI355X (gfx950).
 *
 * Two operations from "Verify Before You Fetch: Reliable KV Cache
 * Compression for LLM Inference" (Jha, Kumar, Chowdhury, Agrawal, Desai):
 *
 *   vkv_compress     PoissonComp, Algorithm 1 and section 4.1 (eq. 3): water-fill
 *                    the inclusion probabilities r_i = min(1, c tau_i) so that
 *                    they sum to the budget, split H (r = 1) from L (r < 1),
 *                    draw the Poisson sample S (independent Bernoulli(r_i))
 *                    and compact the resident rows H u S.
 *   vkv_decode_step  KVFetch, Algorithm 2 and section 4.2: sketch weights, the
 *                    bounded-shrinkage estimator (Definition 2, eq. 5), the
 *                    Bernstein certificate (Lemma 1, eq. 7), and when it fails
 *                    the gains (eq. 9), the fetch count k* (eq. 10, Theorem 2),
 *                    the gather of the chosen rows from pinned host memory and
 *                    the corrected attention output (section 3, eq. 1).
 *
 * Conventions shared by every entry point:
 *   - Every pointer is owned by the caller. "dev" marks device memory, "host"
 *     marks pinned host memory (hipHostMalloc) that the GPU reads directly.
 *     The library never allocates, frees or keeps a pointer after a call.
 *   - bfloat16 values are passed as uint16_t bit patterns.
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = default stream) and
 *     the outputs are valid once the stream has been synchronised.
 *   - Argument checks run on the host before anything is launched and return
 *     VKV_EINVAL (or VKV_ENOTPINNED for host_kv); nothing is enqueued then.
 *   - Conditions only the GPU can see (a resident count above `cap`, a fetch
 *     union above `fetch_cap`, malformed r or resident lists) are ORed into the
 *     caller's device status word; vkv_check_status() reads and maps it.
 *   - vkv_last_error() returns a thread-local message for the last failure.
 *   - The workspace needs no initialisation; its size comes from the matching
 *     *_workspace_bytes() call for the same arguments.
 */
#ifndef VERKV_H
#define VERKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VKV_OK = 0,
  VKV_EINVAL = 1,       /* bad shape, pointer, range or workspace size       */
  VKV_ENOTPINNED = 2,   /* host_kv is not device-accessible pinned memory    */
  VKV_EOVERFLOW = 3,    /* a device-side capacity (cap, fetch_cap) overflowed */
  VKV_EHIP = 4,         /* a HIP runtime call failed                         */
  VKV_EUNSUPPORTED = 5, /* valid but unsupported configuration               */
  VKV_EDATA = 6         /* malformed inputs seen on the device               */
} vkv_status;

/* Device status word bits (ORed by the kernels of one call). */
#define VKV_STATUS_RESIDENT_OVERFLOW 0x1u /* compress: |H u S| > cap          */
#define VKV_STATUS_FETCH_OVERFLOW 0x2u    /* decode: union > fetch_cap        */
#define VKV_STATUS_BAD_R 0x4u             /* decode: r outside (0, 1]         */
#define VKV_STATUS_BAD_RESIDENT 0x8u      /* decode: resident list malformed, */
                                          /* or a token with r = 1 missing   */

/* How the fetch count k* of a row was decided (row_path output): no fetch
 * (eps^(L) < eps), from the top-tier gain candidates, from all gain
 * candidates, or by the streaming selection over every token of L (taken
 * when the candidates cannot decide the row, e.g. k* above 8192). */
enum {
  VKV_PATH_NO_FETCH = 0,
  VKV_PATH_TOP_CANDIDATES = 1,
  VKV_PATH_ALL_CANDIDATES = 2,
  VKV_PATH_STREAMING = 3
};

/* Estimators for the L part: clipped shrinkage (Definition 2, eq. 5), the
 * unbiased lambda = 1 estimator (the PoissonComp-only baseline), or binary
 * shrinkage (Appendix A.2, Figure 2): lambda_i in {1, r_i}, with the tokens
 * of L taken by w~ (1 - r) / r descending (ties: position ascending) and set
 * to lambda = r while that value exceeds twice the bias w~ (1 - r) of the
 * tokens set before them. */
enum { VKV_EST_CLIP = 0, VKV_EST_UNBIASED = 1, VKV_EST_BINARY = 2 };
/* Planning weights on L: from the projected key sketch (sketch, proj); the
 * exact weights (the "perfect sketch" of section 4.2; reads every key of L
 * from host memory, so it is a slow test mode); or the pages' deployed
 * sketch ("Verify Before You Fetch", Appendix A.1 and section 5.1): 2-bit
 * keys over 16 RoPE channel pairs (vkv_sketch2_build) and an exact
 * shortlist of the n_short non-resident tokens with the largest sketch
 * logit over the KV head's query heads, whose keys are read from host
 * memory; the plan then uses exact weights on S and the shortlist and the
 * sketch's weights on the rest of L. */
enum { VKV_W_SKETCH = 0, VKV_W_PERFECT = 1, VKV_W_SKETCH2 = 2 };

/*
 * PoissonComp over n_layers x n_kv_heads independent slices of n_tokens.
 *
 * tau      dev [n_layers][n_kv_heads][ctx_stride] f32. Importance scores in [0,1]
 *          (section 4.1 maps other ranges through a softmax first; that is the
 *          caller's job). They are read on a 2^-32 grid and floored at one
 *          step, so every token gets r > 0; values outside [0,1] are clamped.
 * k, v     [n_layers][n_kv_heads][n_tokens][head_dim] bf16 prefill keys and
 *          values, in device memory or pinned host memory (hipHostMalloc);
 *          may be NULL when resident_kv is NULL. Token t of slice i at
 *          k + (i * ctx_stride + t) * kv_stride elements (so the interleaved
 *          K/V rows of a decode cache, k = host_kv and v = host_kv + d with
 *          kv_stride 2 d, compress again as they are).
 * ctx_stride  positions per slice in tau, r and k/v (0: n_tokens; else
 *          >= n_tokens). kv_stride  elements per token in k and v (0:
 *          head_dim; else >= head_dim and a multiple of 8).
 * budget   expected number of GPU-resident rows per slice (eta * n rounded);
 *          it includes the forced sink/local tokens and must exceed their
 *          count (unless every token is forced).
 * n_sink, n_local  the first n_sink and last n_local tokens go to H.
 * seed     Philox4x32-10 key; the draw for (layer0 + l, head, token) is
 *          counter (token, head, layer0 + l, 0) so any slice can be redrawn
 *          alone.
 * cap      resident-row capacity per slice (>= 1).
 * Outputs (dev): r [n_layers][n_kv_heads][ctx_stride] f32 (exactly 1.0 on H,
 * below 1 on L); resident_idx [n_layers][n_kv_heads][cap] i32 ascending
 * positions of H u S; resident_count [n_layers][n_kv_heads] i32 (the true
 * count even when it exceeds cap; then only cap rows are written and the
 * status word gets VKV_STATUS_RESIDENT_OVERFLOW); resident_kv (may be NULL)
 * [n_layers][n_kv_heads][cap][2][head_dim] bf16, each row K then V;
 * water_level (may be NULL) [n_layers][n_kv_heads] f64, c in units of tau
 * (+inf when every token is in H).
 * status   dev u32 [1], cleared at the start of the call.
 * Supported: head_dim = 128, 1 <= n_tokens <= 2^21 and budget <= 2^21, so that
 * every integer product of the water-level solve stays below 2^53.
 */
typedef struct {
  int32_t n_layers, n_kv_heads, n_tokens, head_dim;
  int32_t layer0;
  int32_t ctx_stride;
  int64_t kv_stride;
  const float *tau;
  const uint16_t *k;
  const uint16_t *v;
  int64_t budget;
  int32_t n_sink, n_local;
  uint64_t seed;
  int32_t cap;
  float *r;
  int32_t *resident_idx;
  int32_t *resident_count;
  uint16_t *resident_kv;
  double *water_level;
  uint32_t *status;
  void *workspace;
  size_t workspace_bytes;
} vkv_compress_args;

/*
 * One KVFetch decode step for one layer: every request and every query head.
 *
 * Shapes: B = batch, Hq query heads over G KV heads (Hq/G in {1,2,4,8}),
 * head_dim d = 128, n tokens (1 <= n <= 2^17; larger n returns
 * VKV_EUNSUPPORTED), sketch_dim s in {16, 32}.
 * ctx_stride   positions allocated per (request, KV head) in r, sketch,
 *              sk2_codes, sk2_zs (ceil(ctx_stride / 128) groups) and
 *              host_kv: 0 means n; otherwise n <= ctx_stride <= 2^24, so a
 *              context can grow in place (vkv_append_token) between steps.
 * q            dev [B][Hq][d] bf16.
 * resident_kv  dev [B][G][cap][2][d] bf16 (rows of H u S, K then V), with
 * resident_idx dev [B][G][cap] i32 ascending positions and
 * resident_count dev [B][G] i32 (as written by vkv_compress).
 * sketch       dev [B][G][n][s] bf16 projected keys sk_i = P_g^T k_i.
 * proj         dev [G][d][s] f32 projection P_g (q is projected inside).
 * r            dev [B][G][n] f32 inclusion probabilities, H <=> r == 1.
 * host_kv      host [B][G][n][2][d] bf16 full cache in pinned memory
 *              (hipHostMalloc); rows chosen for fetching are read from it.
 * sk2_codes, sk2_zs, sk2_chan  the 2-bit sketch of every (request, KV
 *              head), as vkv_sketch2_build writes it (VKV_W_SKETCH2 only;
 *              otherwise ignored and may be NULL).
 * n_short      shortlist size per (request, KV head), 0..1024 (the pages
 *              use 128); VKV_W_SKETCH2 only.
 * Reuse of rows staged in earlier steps ("Verify Before You Fetch",
 * Appendix A.3.2, fetching: a device map keyed by (request, KV head,
 * position) lets the fetch reuse rows staged before). All four may be NULL
 * (no staging); the caller alternates two maps and two staging areas:
 * stage_map_prev dev [B][G][ctx_stride] i32, read only: for each position,
 *              its row's index in stage_prev, or -1 (as the previous step
 *              left it in its stage_map_next; a map of -1 to start).
 * stage_prev   dev [B][G][fetch_cap][2][d] bf16, read only: rows staged by
 *              the previous step. A fetched row found there is read from
 *              it instead of from host_kv (and not counted in host_bytes).
 * stage_map_next, stage_next  the same for this step, written: every row
 *              fetched this step is staged at its index in fetch_idx, and
 *              the map holds that index (-1 elsewhere). Both pairs must be
 *              given together; prev and next must not alias.
 *              Staging assumes the positions and rows of the cache did not
 *              change since the previous step (appending keeps them; a new
 *              compression or a new request starts again from a map of -1).
 * eps, delta   tolerance (eps > 0, 0 < delta < 1) of the (eps, delta)
 *              guarantee on the attention denominator.
 * estimator    VKV_EST_CLIP, VKV_EST_UNBIASED or VKV_EST_BINARY; weights
 *              VKV_W_SKETCH or VKV_W_PERFECT.
 * fetch_cap    most rows read from host_kv per (request, KV head) (1..n); rows
 *              of a larger union are neither listed nor read, and the status
 *              word gets VKV_STATUS_FETCH_OVERFLOW.
 * Outputs (dev): out [B][Hq][d] f32 attention output; d_hat and log_shift
 * [B][Hq] f32 with D^ = d_hat * exp(log_shift); eps_hat0 / eps_hat [B][Hq] f32,
 * the certificate before fetching and after (on L'); k_star [B][Hq] i32;
 * fetch_idx [B][G][fetch_cap] i32 ascending positions fetched for the KV head
 * (the union over its query heads, minus S); fetch_count [B][G] i32 (true
 * count, see VKV_STATUS_FETCH_OVERFLOW); host_bytes u64 [1] bytes read from
 * host_kv this step; row_stats (may be NULL) [B][Hq][8] f64 =
 * {m, D~ (scaled by exp(-m)), beta*, beta(L), V(L), b(L), eps^(L), eps^(L')}
 * (with VKV_EST_BINARY, beta* is the bias of the tokens set to lambda = r);
 * row_path (may be NULL) [B][Hq] i32, how k* was decided (VKV_PATH_*);
 * shortlist (may be NULL; VKV_W_SKETCH2 only) [B][G][n_short] i32, the
 * shortlisted positions ascending, -1 after the last (fewer when fewer
 * tokens are eligible). With VKV_W_SKETCH2, host_bytes also counts the
 * 2 d bytes of each shortlisted key.
 * prefetch_rows  read-ahead: up to this many rows per (request, KV head)
 *          are copied from host_kv into the workspace on a second stream
 *          (one per device, owned by the library) while the planning
 *          kernels run, chosen by their planning weight before k* is known;
 *          the gather takes a fetched row from there when it was read ahead.
 *          No output except host_bytes depends on it (host_bytes counts
 *          the rows read ahead too, fetched or not). 0: none; -1: the
 *          library's choice for the shapes; otherwise 1..n_tokens. The
 *          workspace grows by prefetch_rows * 2 d * 2 bytes per (request,
 *          KV head). Steps on one device that read ahead share its second
 *          stream and are ordered on it in call order. Code under HIP graph
 *          capture passes 0 (or calls vkv_decode_step_noalloc, which reads
 *          nothing ahead): the second stream is the library's, not the
 *          caller's.
 * status   dev u32 [1], cleared at the start of the call.
 * phase_events  optional timing hook: NULL, or vkv_decode_phase_count() + 1
 *          hipEvent_t handles (created by the caller); event 0 is recorded on
 *          `stream` before the first kernel and event i + 1 after kernel i.
 *          NULL entries are skipped, so a caller can time one kernel without
 *          putting a record between every pair of kernels. When exactly the
 *          two entries i and i + 1 are non-NULL, kernel i's own dispatch
 *          records them (hipExtLaunchKernel): the span of that kernel alone,
 *          as a kernel trace reports it. Phase 3 has no kernel unless the
 *          estimator is VKV_EST_BINARY; its events are then plain records.
 */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim, n_tokens, sketch_dim, cap;
  int32_t ctx_stride;
  const uint16_t *q;
  const uint16_t *resident_kv;
  const int32_t *resident_idx;
  const int32_t *resident_count;
  const uint16_t *sketch;
  const float *proj;
  const float *r;
  const uint16_t *host_kv;
  const uint64_t *sk2_codes;
  const uint16_t *sk2_zs;
  const int32_t *sk2_chan;
  int32_t n_short;
  const int32_t *stage_map_prev;
  const uint16_t *stage_prev;
  int32_t *stage_map_next;
  uint16_t *stage_next;
  float eps, delta;
  int32_t estimator, weights, fetch_cap;
  float *out;
  float *d_hat;
  float *log_shift;
  float *eps_hat0;
  float *eps_hat;
  int32_t *k_star;
  int32_t *fetch_idx;
  int32_t *fetch_count;
  uint64_t *host_bytes;
  double *row_stats;
  int32_t *row_path;
  int32_t *shortlist;
  uint32_t *status;
  void **phase_events;
  void *workspace;
  size_t workspace_bytes;
  int32_t prefetch_rows;
} vkv_decode_args;

/*
 * Exact decode attention over the whole cache, eq. 1 (section 3): the Dense
 * baselines of section 5. Dense (resident) passes a cache in device memory;
 * Dense (offload) passes it in pinned host memory (hipHostMalloc), and every
 * row is then read over the host link at every call (no device staging).
 *
 * Shapes: B = batch, Hq query heads over G KV heads (Hq/G in {1,2,4,8}),
 * d = 128, 1 <= n <= 2^24 tokens.
 * q       dev [B][Hq][d] bf16.
 * kv      [B][G][n][2][d] bf16 (K row then V row per token), device memory or
 *         pinned host memory.
 * Outputs (dev): out [B][Hq][d] f32, o = sum_i w_i v_i / sum_i w_i with
 * w_i = exp(<q, k_i>/sqrt(d)); log_d [B][Hq] f32, the natural log of
 * sum_i w_i.
 * Pageable host memory returns VKV_ENOTPINNED; bad shapes VKV_EINVAL.
 */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim, n_tokens;
  const uint16_t *q;
  const uint16_t *kv;
  float *out;
  float *log_d;
  void *workspace;
  size_t workspace_bytes;
} vkv_dense_args;

/*
 * The pages' 2-bit key sketch ("Verify Before You Fetch", Appendix A.1 and
 * section 5.1), built from the prefill keys of n_slices independent slices
 * (layers x KV heads, or requests x KV heads) of n_tokens each.
 *
 * Per slice: the 16 RoPE channel pairs (j, j + d/2) with the largest key
 * energy, the sum over tokens of k_j^2 + k_{j+d/2}^2 (ties: lower j), give
 * the 32 kept channels, listed in increasing channel index in chan. Each
 * kept channel is quantised per group of 128 tokens (the last group may be
 * shorter) between the group's minimum and maximum: zero z = fp16(min),
 * scale s = fp16(fp32(max - min) / 3), both saturated at +-65504, and code
 * clamp(rint(fp32(fp32(k - z) / s)), 0, 3) (0 when s == 0). The dequantised
 * key is z + code * s. Bits 2c and 2c + 1 of a token's 64-bit code word
 * hold the code of kept channel c. Stored size: 8 bytes per token and
 * 128 bytes per group, 1.76% of the bf16 K/V cache.
 *
 * k         bf16 keys in device memory or device-accessible pinned host
 *           memory; token t of slice i at k + i * slice_stride +
 *           t * key_stride (elements; key_stride >= head_dim, so K rows
 *           interleaved with V rows can be passed as they are).
 * out_stride  positions per slice in codes and zs (0: n_tokens; else >=
 *           n_tokens), so a capacity layout can be filled.
 * codes     out dev [n_slices][out_stride] u64.
 * zs        out dev [n_slices][ceil(out_stride / 128)][2][32] fp16 bits: the
 *           group's 32 zero points, then its 32 scales (groups past the
 *           context are left as they are).
 * chan      out dev [n_slices][32] i32.
 * Supported: head_dim = 128, 1 <= n_tokens <= 2^24, n_slices <= 65535.
 * The pair choice sums squares in float64; pairs whose energies agree to
 * rounding may be chosen either way.
 */
typedef struct {
  int32_t n_slices, n_tokens, head_dim, out_stride;
  int64_t key_stride, slice_stride;
  const uint16_t *k;
  uint64_t *codes;
  uint16_t *zs;
  int32_t *chan;
  void *workspace;
  size_t workspace_bytes;
} vkv_sketch2_args;

/*
 * Decode-time maintenance: one generated token joins every (request, KV
 * head) at position pos ("Verify Before You Fetch", section 3: sinks and
 * the local window stay resident; Appendix A.3.1: the per-(layer, head)
 * list of resident positions is extended as tokens are generated and new
 * tokens are written after the packed region). The token goes to H: its
 * K/V row is written to host_kv at pos and appended to resident_kv at
 * resident_count, pos is appended to resident_idx, resident_count grows by
 * one and r[pos] = 1. When given, its projected sketch row is written
 * (sketch = bf16(P_g^T k), round to nearest even, P_g^T k summed in fp32
 * over increasing dimension) and its 2-bit code word is 0, with a group
 * that starts at pos getting zero points and scales 0 (the sketch of a
 * token of H is never used while it stays in H; a new compression
 * rebuilds it). The next decode step then takes n_tokens = pos + 1.
 *
 * k_new, v_new  dev [B][G][d] bf16 rows of the new token.
 * host_kv     host [B][G][ctx_stride][2][d] bf16, pinned (hipHostMalloc).
 * resident_kv dev [B][G][cap][2][d]; resident_idx dev [B][G][cap];
 *             resident_count dev [B][G] (updated in place).
 * r           dev [B][G][ctx_stride] f32.
 * sketch, proj  dev [B][G][ctx_stride][s] bf16 and [G][d][s] f32, or both
 *             NULL; sk2_codes dev [B][G][ctx_stride] u64 and sk2_zs dev
 *             [B][G][ceil(ctx_stride/128)][2][32], or both NULL.
 * status      dev u32 [1]: VKV_STATUS_RESIDENT_OVERFLOW when a list is at
 *             cap (that list is left as it is), VKV_STATUS_BAD_RESIDENT
 *             when pos does not exceed the list's last position.
 * Requires 0 <= pos < ctx_stride <= 2^24; not cleared: bits accumulate
 * until the caller clears the word.
 */
typedef struct {
  int32_t batch, n_kv_heads, head_dim, pos, cap, ctx_stride, sketch_dim;
  const uint16_t *k_new;
  const uint16_t *v_new;
  uint16_t *host_kv;
  uint16_t *resident_kv;
  int32_t *resident_idx;
  int32_t *resident_count;
  float *r;
  uint16_t *sketch;
  const float *proj;
  uint64_t *sk2_codes;
  uint16_t *sk2_zs;
  uint32_t *status;
} vkv_append_args;

/* Enqueue one token's append (see vkv_append_args). */
vkv_status vkv_append_token(const vkv_append_args *a, void *stream);

/* Workspace sizes in bytes for these arguments (0 if the shapes are invalid). */
size_t vkv_compress_workspace_bytes(const vkv_compress_args *a);
size_t vkv_decode_workspace_bytes(const vkv_decode_args *a);
size_t vkv_dense_workspace_bytes(const vkv_dense_args *a);
size_t vkv_sketch2_workspace_bytes(const vkv_sketch2_args *a);

/* Enqueue the 2-bit sketch build (see vkv_sketch2_args). */
vkv_status vkv_sketch2_build(const vkv_sketch2_args *a, void *stream);

/* Enqueue one PoissonComp pass (see vkv_compress_args). */
vkv_status vkv_compress(const vkv_compress_args *a, void *stream);

/* Rows per (request, KV head) that a decode step with these arguments
 * reads ahead (prefetch_rows resolved: -1 gives the library's choice for
 * the shapes); -1 when the shapes are invalid. */
int32_t vkv_decode_prefetch_rows(const vkv_decode_args *a);

/* Enqueue one KVFetch decode step (see vkv_decode_args). */
vkv_status vkv_decode_step(const vkv_decode_args *a, void *stream);

/* Size of the library's own decode workspace (128 MiB per GPU), used by
 * vkv_decode_step_noalloc. */
#define VKV_NOALLOC_WORKSPACE_BYTES (128u << 20)

/* vkv_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same step and outputs, with the workspace taken from a
 * buffer the library holds on each GPU (VKV_NOALLOC_WORKSPACE_BYTES,
 * placed when the library's code is loaded on that GPU and held until the
 * process ends). a->workspace must be NULL and a->workspace_bytes 0; the
 * caller still passes every input and output. Shapes whose workspace
 * (vkv_decode_workspace_bytes) exceeds the buffer return VKV_EUNSUPPORTED
 * (for example: batch 1 fits up to 128K tokens at 32 query heads over 8
 * KV heads; batch 16 at 32K does not). The call allocates nothing and
 * needs the buffer cleared by nobody: the kernels initialise what they
 * read. Every call on one GPU shares that GPU's buffer, which keeps the
 * last call's contents: calls that overlap on one GPU (other streams,
 * other threads) race, and the caller must order them. It reads no rows
 * ahead: prefetch_rows is taken as 0. */
vkv_status vkv_decode_step_noalloc(const vkv_decode_args *a, void *stream);

/* Enqueue one exact decode attention over the whole cache (see
 * vkv_dense_args). */
vkv_status vkv_dense_attention(const vkv_dense_args *a, void *stream);

/* Synchronise `stream`, read the device status word and map it to a status:
 * VKV_OK, VKV_EOVERFLOW (capacity bits) or VKV_EDATA (data bits). The word
 * itself is returned through *bits when bits != NULL. */
vkv_status vkv_check_status(const uint32_t *status, void *stream,
                            uint32_t *bits);

/* Thread-local text describing the last non-OK status of this thread. */
const char *vkv_last_error(void);

/* Kernels one decode step launches, in order, and their names (for the
 * phase_events timing hook); NULL for an index out of range. */
int32_t vkv_decode_phase_count(void);
const char *vkv_decode_phase_name(int32_t i);

/* Library version as major*10000 + minor*100 + patch. */
int32_t vkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VERKV_H */
