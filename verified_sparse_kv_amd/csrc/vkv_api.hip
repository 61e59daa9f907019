// C ABI of the VerKV hot path: argument validation, workspace sizing, the
// pinned-memory check and dispatch to the kernels. See include/verkv.h.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "vkv_common.h"
#include "vkv_internal.h"

namespace {

thread_local char g_err[512] = "";

vkv_status fail(vkv_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

vkv_status hip_fail(hipError_t e, const char *what) {
  return fail(VKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define REQUIRE(cond, ...)                          \
  do {                                              \
    if (!(cond)) return fail(VKV_EINVAL, __VA_ARGS__); \
  } while (0)

// Forced tokens: the first n_sink and the last n_local (they may overlap).
int64_t forced_count(int64_t n, int64_t n_sink, int64_t n_local) {
  if (n_sink + n_local >= n) return n;
  return n_sink + n_local;
}

vkv_status check_compress_shapes(const vkv_compress_args *a) {
  REQUIRE(a != nullptr, "compress: args is NULL");
  REQUIRE(a->n_layers >= 1 && a->n_kv_heads >= 1,
          "compress: n_layers and n_kv_heads must be >= 1");
  REQUIRE((int64_t)a->n_layers * a->n_kv_heads <= 65535,
          "compress: n_layers * n_kv_heads must be <= 65535");
  REQUIRE(a->n_tokens >= 1 && a->n_tokens <= (1 << 21),
          "compress: n_tokens must be in [1, 2^21]");
  REQUIRE(a->head_dim == vkv::kHeadDim, "compress: head_dim must be 128");
  REQUIRE(a->layer0 >= 0, "compress: layer0 must be >= 0");
  REQUIRE(a->n_sink >= 0 && a->n_local >= 0,
          "compress: n_sink and n_local must be >= 0");
  REQUIRE(a->cap >= 1, "compress: cap must be >= 1");
  REQUIRE(a->ctx_stride == 0 || (a->ctx_stride >= a->n_tokens && a->ctx_stride <= (1 << 24)),
          "compress: ctx_stride must be 0 or in [n_tokens, 2^24]");
  REQUIRE(a->kv_stride == 0 || (a->kv_stride >= a->head_dim && a->kv_stride % 8 == 0),
          "compress: kv_stride must be 0 or >= head_dim and a multiple of 8");
  return VKV_OK;
}

vkv_status check_dense_shapes(const vkv_dense_args *a) {
  REQUIRE(a != nullptr, "dense: args is NULL");
  REQUIRE(a->batch >= 1 && a->batch <= 65535, "dense: batch must be in [1, 65535]");
  REQUIRE(a->n_kv_heads >= 1 && a->n_kv_heads <= 65535,
          "dense: n_kv_heads must be in [1, 65535]");
  REQUIRE(a->n_q_heads >= a->n_kv_heads && a->n_q_heads % a->n_kv_heads == 0,
          "dense: n_q_heads must be a multiple of n_kv_heads");
  const int grp = a->n_q_heads / a->n_kv_heads;
  REQUIRE(grp == 1 || grp == 2 || grp == 4 || grp == 8,
          "dense: n_q_heads / n_kv_heads must be 1, 2, 4 or 8");
  REQUIRE((int64_t)a->batch * a->n_q_heads <= 65535,
          "dense: batch * n_q_heads must be <= 65535");
  REQUIRE(a->head_dim == vkv::kHeadDim, "dense: head_dim must be 128");
  REQUIRE(a->n_tokens >= 1 && a->n_tokens <= (1 << 24),
          "dense: n_tokens must be in [1, 2^24]");
  return VKV_OK;
}

vkv_status check_decode_shapes(const vkv_decode_args *a) {
  REQUIRE(a != nullptr, "decode: args is NULL");
  REQUIRE(a->batch >= 1 && a->batch <= 65535, "decode: batch must be in [1, 65535]");
  REQUIRE(a->n_kv_heads >= 1 && a->n_kv_heads <= 65535,
          "decode: n_kv_heads must be in [1, 65535]");
  REQUIRE(a->n_q_heads >= a->n_kv_heads && a->n_q_heads % a->n_kv_heads == 0,
          "decode: n_q_heads must be a multiple of n_kv_heads");
  const int grp = a->n_q_heads / a->n_kv_heads;
  if (!(grp == 1 || grp == 2 || grp == 4 || grp == 8))
    return fail(VKV_EUNSUPPORTED, "decode: n_q_heads / n_kv_heads = %d (supported: 1, 2, 4, 8)", grp);
  REQUIRE(a->head_dim == vkv::kHeadDim, "decode: head_dim must be 128");
  REQUIRE(a->n_tokens >= 1 && a->n_tokens < (1 << 24),
          "decode: n_tokens must be in [1, 2^24)");
  if (a->n_tokens > (1 << 17))
    return fail(VKV_EUNSUPPORTED, "decode: n_tokens %d (supported: up to 2^17)", a->n_tokens);
  if (a->weights == VKV_W_SKETCH && !(a->sketch_dim == 16 || a->sketch_dim == 32))
    return fail(VKV_EUNSUPPORTED, "decode: sketch_dim %d (supported: 16, 32)", a->sketch_dim);
  REQUIRE(a->cap >= 1, "decode: cap must be >= 1");
  REQUIRE(a->prefetch_rows >= -1 && a->prefetch_rows <= a->n_tokens,
          "decode: prefetch_rows must be -1, 0 or in [1, n_tokens]");
  REQUIRE(a->fetch_cap >= 1 && a->fetch_cap <= a->n_tokens,
          "decode: fetch_cap must be in [1, n_tokens]");
  REQUIRE(a->ctx_stride == 0 || (a->ctx_stride >= a->n_tokens && a->ctx_stride <= (1 << 24)),
          "decode: ctx_stride must be 0 or in [n_tokens, 2^24]");
  return VKV_OK;
}

// The workspace of vkv_decode_step_noalloc: one library-owned device buffer
// per GPU (the loader places it when the code object is loaded on that GPU;
// it is held until the process ends). In host code `scratch` names a
// host-side stand-in, not the device buffer: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[VKV_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call
// on that device, with the device current).
vkv_status scratch_for_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(VKV_EUNSUPPORTED, "decode_noalloc: device %d (supported: 0..%d)",
                dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "decode_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return VKV_OK;
}

// Argument checks of a decode step that need no workspace and no GPU.
vkv_status check_decode_args(const vkv_decode_args *a) {
  vkv_status st = check_decode_shapes(a);
  if (st != VKV_OK) return st;
  REQUIRE(a->eps > 0.0f && isfinite(a->eps), "decode: eps must be > 0");
  REQUIRE(a->delta > 0.0f && a->delta < 1.0f, "decode: delta must be in (0, 1)");
  REQUIRE(a->estimator == VKV_EST_CLIP || a->estimator == VKV_EST_UNBIASED ||
              a->estimator == VKV_EST_BINARY,
          "decode: unknown estimator %d", a->estimator);
  REQUIRE(a->weights == VKV_W_SKETCH || a->weights == VKV_W_PERFECT ||
              a->weights == VKV_W_SKETCH2,
          "decode: unknown weights mode %d", a->weights);
  REQUIRE(a->q && a->resident_kv && a->resident_idx && a->resident_count && a->r &&
              a->host_kv,
          "decode: q, resident_kv, resident_idx, resident_count, r and host_kv are required");
  REQUIRE(a->weights != VKV_W_SKETCH || (a->sketch && a->proj),
          "decode: sketch and proj are required in sketch mode");
  REQUIRE(a->weights != VKV_W_SKETCH2 || (a->sk2_codes && a->sk2_zs && a->sk2_chan),
          "decode: sk2_codes, sk2_zs and sk2_chan are required with the 2-bit sketch");
  REQUIRE(a->weights != VKV_W_SKETCH2 || (a->n_short >= 0 && a->n_short <= 1024),
          "decode: n_short must be in [0, 1024]");
  REQUIRE(a->out && a->d_hat && a->log_shift && a->eps_hat0 && a->eps_hat &&
              a->k_star && a->fetch_idx && a->fetch_count && a->host_bytes && a->status,
          "decode: every output pointer except row_stats and row_path is required");
  REQUIRE((a->stage_map_prev == nullptr) == (a->stage_prev == nullptr) &&
              (a->stage_map_next == nullptr) == (a->stage_next == nullptr),
          "decode: stage_map_prev/stage_prev and stage_map_next/stage_next are given in pairs");
  REQUIRE(a->stage_prev == nullptr ||
              (a->stage_prev != a->stage_next && a->stage_map_prev != a->stage_map_next),
          "decode: the previous and next staging must not alias");
  return VKV_OK;
}

// A device-readable address for p: device memory as it is, pinned host
// memory (hipHostMalloc) through its device view. Anything else fails.
bool device_view(const void *p, const void **dev) {
  hipPointerAttribute_t attr;
  const hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (attr.type == hipMemoryTypeDevice) {
    *dev = p;
    return true;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer && attr.hostPointer) {
    *dev = static_cast<const char *>(attr.devicePointer) +
           (static_cast<const char *>(p) - static_cast<const char *>(attr.hostPointer));
    return true;
  }
  return false;
}

vkv_status check_sketch2_args(const vkv_sketch2_args *a) {
  REQUIRE(a != nullptr, "sketch2: args is NULL");
  REQUIRE(a->n_slices >= 1 && a->n_slices <= 65535, "sketch2: n_slices must be in [1, 65535]");
  REQUIRE(a->n_tokens >= 1 && a->n_tokens <= (1 << 24), "sketch2: n_tokens must be in [1, 2^24]");
  REQUIRE(a->head_dim == vkv::kHeadDim, "sketch2: head_dim must be 128");
  REQUIRE(a->key_stride >= a->head_dim && a->key_stride % 8 == 0,
          "sketch2: key_stride must be >= head_dim and a multiple of 8");
  REQUIRE(a->slice_stride >= 0 && a->slice_stride % 8 == 0,
          "sketch2: slice_stride must be >= 0 and a multiple of 8");
  REQUIRE(a->out_stride == 0 || (a->out_stride >= a->n_tokens && a->out_stride <= (1 << 24)),
          "sketch2: out_stride must be 0 or in [n_tokens, 2^24]");
  return VKV_OK;
}

vkv_status check_append_args(const vkv_append_args *a) {
  REQUIRE(a != nullptr, "append: args is NULL");
  REQUIRE(a->batch >= 1 && a->batch <= 65535 && a->n_kv_heads >= 1 &&
              a->n_kv_heads <= 65535,
          "append: batch and n_kv_heads must be in [1, 65535]");
  REQUIRE(a->head_dim == vkv::kHeadDim, "append: head_dim must be 128");
  REQUIRE(a->ctx_stride >= 1 && a->ctx_stride <= (1 << 24),
          "append: ctx_stride must be in [1, 2^24]");
  REQUIRE(a->pos >= 0 && a->pos < a->ctx_stride, "append: pos must be in [0, ctx_stride)");
  REQUIRE(a->cap >= 1, "append: cap must be >= 1");
  REQUIRE(a->k_new && a->v_new && a->host_kv && a->resident_kv && a->resident_idx &&
              a->resident_count && a->r && a->status,
          "append: k_new, v_new, host_kv, resident_kv, resident_idx, "
          "resident_count, r and status are required");
  REQUIRE((a->sketch == nullptr) == (a->proj == nullptr),
          "append: sketch and proj are given together");
  REQUIRE(a->sketch == nullptr || a->sketch_dim == 16 || a->sketch_dim == 32,
          "append: sketch_dim must be 16 or 32 with a sketch");
  REQUIRE((a->sk2_codes == nullptr) == (a->sk2_zs == nullptr),
          "append: sk2_codes and sk2_zs are given together");
  return VKV_OK;
}

// The pinned-memory check and the launch, with the workspace `ws`.
vkv_status decode_launch(const vkv_decode_args *a, const vkv::DecodeLayout &L,
                         void *ws, void *stream) {
  // host_kv must be pinned host memory the GPU can read
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, a->host_kv);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr) {
    (void)hipGetLastError();
    return fail(VKV_ENOTPINNED,
                "decode: host_kv is not device-accessible pinned host memory (%s)",
                e != hipSuccess ? hipGetErrorString(e) : "wrong memory type");
  }
  const uint16_t *hkv = static_cast<const uint16_t *>(attr.devicePointer);
  vkv_decode_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = L.total;
  e = vkv::launch_decode(b, L, hkv, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return VKV_OK;
}

}  // namespace

extern "C" {

const char *vkv_last_error(void) { return g_err; }

int32_t vkv_version(void) { return 100; }

int32_t vkv_decode_phase_count(void) { return vkv::decode_phase_count(); }

const char *vkv_decode_phase_name(int32_t i) { return vkv::decode_phase_name(i); }

size_t vkv_compress_workspace_bytes(const vkv_compress_args *a) {
  if (check_compress_shapes(a) != VKV_OK) return 0;
  return vkv::compress_layout(*a).total;
}

size_t vkv_decode_workspace_bytes(const vkv_decode_args *a) {
  if (check_decode_shapes(a) != VKV_OK) return 0;
  return vkv::decode_layout(*a).total;
}

int32_t vkv_decode_prefetch_rows(const vkv_decode_args *a) {
  if (check_decode_shapes(a) != VKV_OK) return -1;
  return vkv::decode_layout(*a).spec_m;
}

size_t vkv_sketch2_workspace_bytes(const vkv_sketch2_args *a) {
  if (check_sketch2_args(a) != VKV_OK) return 0;
  return vkv::sketch2_layout(*a).total;
}

vkv_status vkv_sketch2_build(const vkv_sketch2_args *a, void *stream) {
  vkv_status st = check_sketch2_args(a);
  if (st != VKV_OK) return st;
  REQUIRE(a->k && a->codes && a->zs && a->chan, "sketch2: k, codes, zs and chan are required");
  REQUIRE(((uintptr_t)a->k & 15u) == 0, "sketch2: k must be 16-byte aligned");
  const vkv::Sketch2Layout L = vkv::sketch2_layout(*a);
  REQUIRE(a->workspace != nullptr && a->workspace_bytes >= L.total,
          "sketch2: workspace of %zu bytes needed", L.total);
  vkv_sketch2_args b = *a;
  const void *kd = nullptr;
  if (!device_view(a->k, &kd))
    return fail(VKV_ENOTPINNED, "sketch2: k is neither device memory nor pinned host memory");
  b.k = static_cast<const uint16_t *>(kd);
  const hipError_t e = vkv::launch_sketch2(b, L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sketch2 launch");
  return VKV_OK;
}

size_t vkv_dense_workspace_bytes(const vkv_dense_args *a) {
  if (check_dense_shapes(a) != VKV_OK) return 0;
  return vkv::dense_layout(*a).total;
}

vkv_status vkv_compress(const vkv_compress_args *a, void *stream) {
  vkv_status st = check_compress_shapes(a);
  if (st != VKV_OK) return st;
  REQUIRE(a->tau && a->r && a->resident_idx && a->resident_count && a->status,
          "compress: tau, r, resident_idx, resident_count and status are required");
  REQUIRE(a->resident_kv == nullptr || (a->k && a->v),
          "compress: k and v are required when resident_kv is given");
  const int64_t n = a->n_tokens;
  const int64_t nf = forced_count(n, a->n_sink, a->n_local);
  const int64_t b_free = a->budget - nf;
  REQUIRE(b_free >= 0, "compress: budget %lld is smaller than the %lld forced tokens",
          (long long)a->budget, (long long)nf);
  REQUIRE(nf == n || b_free >= 1,
          "compress: budget must exceed the forced tokens so that every token gets r > 0");
  REQUIRE(a->budget <= (1 << 21), "compress: budget must be <= 2^21");
  const vkv::CompressLayout L = vkv::compress_layout(*a);
  REQUIRE(a->workspace != nullptr && a->workspace_bytes >= L.total,
          "compress: workspace of %zu bytes needed", L.total);
  vkv_compress_args b = *a;
  if (a->resident_kv) {  // k and v: device memory or pinned host memory
    const void *kd = nullptr, *vd = nullptr;
    if (!device_view(a->k, &kd) || !device_view(a->v, &vd))
      return fail(VKV_ENOTPINNED,
                  "compress: k and v must be device memory or pinned host memory");
    b.k = static_cast<const uint16_t *>(kd);
    b.v = static_cast<const uint16_t *>(vd);
  }
  const hipError_t e = vkv::launch_compress(b, L, b_free, (int32_t)nf,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "compress launch");
  return VKV_OK;
}

vkv_status vkv_decode_step(const vkv_decode_args *a, void *stream) {
  vkv_status st = check_decode_args(a);
  if (st != VKV_OK) return st;
  const vkv::DecodeLayout L = vkv::decode_layout(*a);
  REQUIRE(a->workspace != nullptr && a->workspace_bytes >= L.total,
          "decode: workspace of %zu bytes needed", L.total);
  return decode_launch(a, L, a->workspace, stream);
}

vkv_status vkv_decode_step_noalloc(const vkv_decode_args *a, void *stream) {
  vkv_status st = check_decode_args(a);
  if (st != VKV_OK) return st;
  REQUIRE(a->workspace == nullptr && a->workspace_bytes == 0,
          "decode_noalloc: workspace must be NULL with workspace_bytes 0 (the "
          "library's own buffer is used)");
  vkv_decode_args b = *a;
  b.prefetch_rows = 0;  // (no read-ahead: its stream is made on first use)
  a = &b;
  const vkv::DecodeLayout L = vkv::decode_layout(*a);
  if (L.total > (size_t)VKV_NOALLOC_WORKSPACE_BYTES)
    return fail(VKV_EUNSUPPORTED,
                "decode_noalloc: these shapes need a workspace of %zu bytes, "
                "above the library's buffer of %zu bytes (use vkv_decode_step "
                "with a caller workspace)",
                L.total, (size_t)VKV_NOALLOC_WORKSPACE_BYTES);
  void *ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != VKV_OK) return st;
  return decode_launch(a, L, ws, stream);
}

vkv_status vkv_append_token(const vkv_append_args *a, void *stream) {
  vkv_status st = check_append_args(a);
  if (st != VKV_OK) return st;
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, a->host_kv);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr) {
    (void)hipGetLastError();
    return fail(VKV_ENOTPINNED, "append: host_kv is not device-accessible pinned host memory");
  }
  e = vkv::launch_append(*a, static_cast<uint16_t *>(attr.devicePointer),
                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return VKV_OK;
}

vkv_status vkv_dense_attention(const vkv_dense_args *a, void *stream) {
  vkv_status st = check_dense_shapes(a);
  if (st != VKV_OK) return st;
  REQUIRE(a->q && a->kv && a->out && a->log_d, "dense: q, kv, out and log_d are required");
  const vkv::DenseLayout L = vkv::dense_layout(*a);
  REQUIRE(a->workspace != nullptr && a->workspace_bytes >= L.total,
          "dense: workspace of %zu bytes needed", L.total);
  // device memory as it is; host memory only when pinned and mapped
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, a->kv);
  const uint16_t *kv = nullptr;
  if (e == hipSuccess && attr.type == hipMemoryTypeDevice) {
    kv = a->kv;
  } else if (e == hipSuccess && attr.type == hipMemoryTypeHost && attr.devicePointer) {
    kv = static_cast<const uint16_t *>(attr.devicePointer);
  } else {
    (void)hipGetLastError();
    return fail(VKV_ENOTPINNED,
                "dense: kv is neither device memory nor device-accessible pinned host memory (%s)",
                e != hipSuccess ? hipGetErrorString(e) : "wrong memory type");
  }
  e = vkv::launch_dense(*a, L, kv, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dense launch");
  return VKV_OK;
}

vkv_status vkv_check_status(const uint32_t *status, void *stream, uint32_t *bits) {
  REQUIRE(status != nullptr, "check_status: status is NULL");
  uint32_t h = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&h, status, sizeof(h), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "check_status copy");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "check_status sync");
  if (bits) *bits = h;
  if (h & (VKV_STATUS_BAD_R | VKV_STATUS_BAD_RESIDENT))
    return fail(VKV_EDATA, "device status 0x%x: malformed r or resident list", h);
  if (h & (VKV_STATUS_RESIDENT_OVERFLOW | VKV_STATUS_FETCH_OVERFLOW))
    return fail(VKV_EOVERFLOW, "device status 0x%x: capacity exceeded", h);
  return VKV_OK;
}

}  // extern "C"
