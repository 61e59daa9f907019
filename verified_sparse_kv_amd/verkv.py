"""Thin Python binding of libverkv.so (include/verkv.h).

Argument marshalling only: every step of compression and decoding runs in
the HIP library. PyTorch supplies device memory, pinned host memory and the
current stream. Importing this module loads the library and raises if it is
missing or does not export the ABI; there is no fallback.

The functions named like the C entry points (``vkv_compress``,
``vkv_decode_step``, ``vkv_*_workspace_bytes``, ``vkv_check_status``,
``vkv_last_error``) take the ctypes argument structs directly; ``compress``
and ``decode_step`` allocate outputs and workspace as torch tensors.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libverkv.so")

VKV_OK, VKV_EINVAL, VKV_ENOTPINNED, VKV_EOVERFLOW, VKV_EHIP, \
    VKV_EUNSUPPORTED, VKV_EDATA = range(7)
STATUS_NAMES = {0: "VKV_OK", 1: "VKV_EINVAL", 2: "VKV_ENOTPINNED",
                3: "VKV_EOVERFLOW", 4: "VKV_EHIP", 5: "VKV_EUNSUPPORTED",
                6: "VKV_EDATA"}
STATUS_RESIDENT_OVERFLOW = 0x1
STATUS_FETCH_OVERFLOW = 0x2
STATUS_BAD_R = 0x4
STATUS_BAD_RESIDENT = 0x8
EST_CLIP, EST_UNBIASED, EST_BINARY = 0, 1, 2
PATH_NO_FETCH, PATH_TOP_CANDIDATES, PATH_ALL_CANDIDATES, PATH_STREAMING = \
    0, 1, 2, 3
W_SKETCH, W_PERFECT, W_SKETCH2 = 0, 1, 2
SK2_CHANNELS, SK2_GROUP = 32, 128

EXPORTS = ("vkv_compress_workspace_bytes", "vkv_decode_workspace_bytes",
           "vkv_compress", "vkv_decode_step", "vkv_check_status",
           "vkv_last_error", "vkv_version", "vkv_decode_phase_count",
           "vkv_decode_phase_name", "vkv_dense_workspace_bytes",
           "vkv_dense_attention", "vkv_decode_step_noalloc",
           "vkv_sketch2_workspace_bytes", "vkv_sketch2_build",
           "vkv_append_token", "vkv_decode_prefetch_rows")
NOALLOC_WORKSPACE_BYTES = 128 << 20

_p = ctypes.c_void_p
_i32 = ctypes.c_int32


class CompressArgs(ctypes.Structure):
    _fields_ = [("n_layers", _i32), ("n_kv_heads", _i32), ("n_tokens", _i32),
                ("head_dim", _i32), ("layer0", _i32), ("ctx_stride", _i32),
                ("kv_stride", ctypes.c_int64),
                ("tau", _p), ("k", _p), ("v", _p),
                ("budget", ctypes.c_int64), ("n_sink", _i32), ("n_local", _i32),
                ("seed", ctypes.c_uint64), ("cap", _i32),
                ("r", _p), ("resident_idx", _p), ("resident_count", _p),
                ("resident_kv", _p), ("water_level", _p), ("status", _p),
                ("workspace", _p), ("workspace_bytes", ctypes.c_size_t)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("batch", _i32), ("n_q_heads", _i32), ("n_kv_heads", _i32),
                ("head_dim", _i32), ("n_tokens", _i32), ("sketch_dim", _i32),
                ("cap", _i32), ("ctx_stride", _i32),
                ("q", _p), ("resident_kv", _p), ("resident_idx", _p),
                ("resident_count", _p), ("sketch", _p), ("proj", _p), ("r", _p),
                ("host_kv", _p),
                ("sk2_codes", _p), ("sk2_zs", _p), ("sk2_chan", _p),
                ("n_short", _i32),
                ("stage_map_prev", _p), ("stage_prev", _p),
                ("stage_map_next", _p), ("stage_next", _p),
                ("eps", ctypes.c_float), ("delta", ctypes.c_float),
                ("estimator", _i32), ("weights", _i32), ("fetch_cap", _i32),
                ("out", _p), ("d_hat", _p), ("log_shift", _p), ("eps_hat0", _p),
                ("eps_hat", _p), ("k_star", _p), ("fetch_idx", _p),
                ("fetch_count", _p), ("host_bytes", _p), ("row_stats", _p),
                ("row_path", _p), ("shortlist", _p), ("status", _p),
                ("phase_events", _p),
                ("workspace", _p),
                ("workspace_bytes", ctypes.c_size_t),
                ("prefetch_rows", _i32)]


class DenseArgs(ctypes.Structure):
    _fields_ = [("batch", _i32), ("n_q_heads", _i32), ("n_kv_heads", _i32),
                ("head_dim", _i32), ("n_tokens", _i32),
                ("q", _p), ("kv", _p), ("out", _p), ("log_d", _p),
                ("workspace", _p), ("workspace_bytes", ctypes.c_size_t)]


class Sketch2Args(ctypes.Structure):
    _fields_ = [("n_slices", _i32), ("n_tokens", _i32), ("head_dim", _i32),
                ("out_stride", _i32),
                ("key_stride", ctypes.c_int64), ("slice_stride", ctypes.c_int64),
                ("k", _p), ("codes", _p), ("zs", _p), ("chan", _p),
                ("workspace", _p), ("workspace_bytes", ctypes.c_size_t)]


class AppendArgs(ctypes.Structure):
    _fields_ = [("batch", _i32), ("n_kv_heads", _i32), ("head_dim", _i32),
                ("pos", _i32), ("cap", _i32), ("ctx_stride", _i32),
                ("sketch_dim", _i32),
                ("k_new", _p), ("v_new", _p), ("host_kv", _p),
                ("resident_kv", _p), ("resident_idx", _p),
                ("resident_count", _p), ("r", _p), ("sketch", _p),
                ("proj", _p), ("sk2_codes", _p), ("sk2_zs", _p),
                ("status", _p)]


class VerKVError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m verified_sparse_kv_amd.build` (there is no fallback)")
    # torch first when it is installed: its bundled HIP runtime then
    # satisfies the library's dependency (same soname), so the process holds
    # one HIP runtime; loading the library first would map the system
    # runtime beside torch's, and pointers of one are unknown to the other
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    for name in EXPORTS:
        if not hasattr(lib, name):
            raise ImportError(f"{LIB_PATH} does not export {name}")
    lib.vkv_compress_workspace_bytes.argtypes = [ctypes.POINTER(CompressArgs)]
    lib.vkv_compress_workspace_bytes.restype = ctypes.c_size_t
    lib.vkv_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeArgs)]
    lib.vkv_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.vkv_compress.argtypes = [ctypes.POINTER(CompressArgs), _p]
    lib.vkv_compress.restype = ctypes.c_int
    lib.vkv_decode_prefetch_rows.argtypes = [ctypes.POINTER(DecodeArgs)]
    lib.vkv_decode_prefetch_rows.restype = ctypes.c_int32
    lib.vkv_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _p]
    lib.vkv_decode_step.restype = ctypes.c_int
    lib.vkv_decode_step_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), _p]
    lib.vkv_decode_step_noalloc.restype = ctypes.c_int
    lib.vkv_check_status.argtypes = [_p, _p, ctypes.POINTER(ctypes.c_uint32)]
    lib.vkv_check_status.restype = ctypes.c_int
    lib.vkv_last_error.argtypes = []
    lib.vkv_last_error.restype = ctypes.c_char_p
    lib.vkv_version.argtypes = []
    lib.vkv_version.restype = ctypes.c_int32
    lib.vkv_decode_phase_count.argtypes = []
    lib.vkv_decode_phase_count.restype = ctypes.c_int32
    lib.vkv_decode_phase_name.argtypes = [ctypes.c_int32]
    lib.vkv_decode_phase_name.restype = ctypes.c_char_p
    lib.vkv_dense_workspace_bytes.argtypes = [ctypes.POINTER(DenseArgs)]
    lib.vkv_dense_workspace_bytes.restype = ctypes.c_size_t
    lib.vkv_dense_attention.argtypes = [ctypes.POINTER(DenseArgs), _p]
    lib.vkv_dense_attention.restype = ctypes.c_int
    lib.vkv_sketch2_workspace_bytes.argtypes = [ctypes.POINTER(Sketch2Args)]
    lib.vkv_sketch2_workspace_bytes.restype = ctypes.c_size_t
    lib.vkv_sketch2_build.argtypes = [ctypes.POINTER(Sketch2Args), _p]
    lib.vkv_sketch2_build.restype = ctypes.c_int
    lib.vkv_append_token.argtypes = [ctypes.POINTER(AppendArgs), _p]
    lib.vkv_append_token.restype = ctypes.c_int
    return lib


LIB = _load()


# ------------------------------------------------------------ C-named calls
def vkv_compress_workspace_bytes(args):
    return int(LIB.vkv_compress_workspace_bytes(ctypes.byref(args)))


def vkv_decode_workspace_bytes(args):
    return int(LIB.vkv_decode_workspace_bytes(ctypes.byref(args)))


def vkv_decode_prefetch_rows(args):
    return int(LIB.vkv_decode_prefetch_rows(ctypes.byref(args)))


def vkv_compress(args, stream=None):
    return int(LIB.vkv_compress(ctypes.byref(args), stream))


def vkv_decode_step(args, stream=None):
    return int(LIB.vkv_decode_step(ctypes.byref(args), stream))


def vkv_decode_step_noalloc(args, stream=None):
    return int(LIB.vkv_decode_step_noalloc(ctypes.byref(args), stream))


def vkv_dense_workspace_bytes(args):
    return int(LIB.vkv_dense_workspace_bytes(ctypes.byref(args)))


def vkv_dense_attention(args, stream=None):
    return int(LIB.vkv_dense_attention(ctypes.byref(args), stream))


def vkv_sketch2_workspace_bytes(args):
    return int(LIB.vkv_sketch2_workspace_bytes(ctypes.byref(args)))


def vkv_sketch2_build(args, stream=None):
    return int(LIB.vkv_sketch2_build(ctypes.byref(args), stream))


def vkv_append_token(args, stream=None):
    return int(LIB.vkv_append_token(ctypes.byref(args), stream))


def vkv_check_status(status_ptr, stream=None):
    bits = ctypes.c_uint32(0)
    rc = int(LIB.vkv_check_status(status_ptr, stream, ctypes.byref(bits)))
    return rc, int(bits.value)


def vkv_last_error():
    return LIB.vkv_last_error().decode()


def vkv_version():
    return int(LIB.vkv_version())


def vkv_decode_phase_count():
    return int(LIB.vkv_decode_phase_count())


def vkv_decode_phase_name(i):
    v = LIB.vkv_decode_phase_name(int(i))
    return None if v is None else v.decode()


def decode_phase_names():
    return [vkv_decode_phase_name(i) for i in range(vkv_decode_phase_count())]


def _check(rc):
    if rc != VKV_OK:
        raise VerKVError(rc, vkv_last_error())


# ------------------------------------------------------------ torch helpers
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, shape, name, device=True):
    torch = _torch()
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not device and (t.is_cuda or not t.is_pinned()):
        raise ValueError(f"{name}: must be pinned host memory")
    return torch


def compress(tau, k, v, budget, n_sink, n_local, seed, cap, layer0=0,
             with_kv=True, stream=None, workspace=None):
    """PoissonComp. tau [Lyr][G][n] f32, k/v [Lyr][G][n][d] int16 (bf16
    bits) on the device. Returns a dict of device tensors."""
    torch = _torch()
    Ly, G, n = tau.shape
    _need(tau, torch.float32, (Ly, G, n), "tau")
    d = 128
    if with_kv:
        _need(k, torch.int16, (Ly, G, n, d), "k")
        _need(v, torch.int16, (Ly, G, n, d), "v")
    dev = tau.device
    out = dict(
        r=torch.empty((Ly, G, n), dtype=torch.float32, device=dev),
        resident_idx=torch.empty((Ly, G, cap), dtype=torch.int32, device=dev),
        resident_count=torch.empty((Ly, G), dtype=torch.int32, device=dev),
        resident_kv=(torch.empty((Ly, G, cap, 2, d), dtype=torch.int16,
                                 device=dev) if with_kv else None),
        water_level=torch.empty((Ly, G), dtype=torch.float64, device=dev),
        status=torch.zeros((1,), dtype=torch.int32, device=dev))
    a = CompressArgs(n_layers=Ly, n_kv_heads=G, n_tokens=n, head_dim=d,
                     layer0=layer0, tau=_ptr(tau),
                     k=_ptr(k) if with_kv else None,
                     v=_ptr(v) if with_kv else None, budget=int(budget),
                     n_sink=n_sink, n_local=n_local,
                     seed=int(seed) & 0xFFFFFFFFFFFFFFFF, cap=cap,
                     r=_ptr(out["r"]), resident_idx=_ptr(out["resident_idx"]),
                     resident_count=_ptr(out["resident_count"]),
                     resident_kv=_ptr(out["resident_kv"]),
                     water_level=_ptr(out["water_level"]),
                     status=_ptr(out["status"]))
    nbytes = vkv_compress_workspace_bytes(a)
    if nbytes == 0:
        _check(vkv_compress(a, _stream(stream)))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = nbytes
    _check(vkv_compress(a, _stream(stream)))
    out["workspace"] = workspace
    out["_args"] = a
    return out


def sketch2_build(k, key_stride=None, stream=None, n=None, out=None):
    """The 2-bit key sketch of every slice of ``k`` (bf16 bits, int16,
    shaped [..., ns, key_stride] with the key in the first 128 elements of
    each token's row; leading dimensions are the slices; device memory or
    pinned host memory). The first ``n`` (default ns) tokens are sketched.
    Returns (or fills ``out``) dict(codes [..., ns] int64,
    zs [..., ceil(ns/128), 2, 32] int16, chan [..., 32] int32)."""
    torch = _torch()
    if k.dtype != torch.int16 or not k.is_contiguous() or \
            not (k.is_cuda or k.is_pinned()):
        raise ValueError("k: contiguous int16 tensor in device or pinned memory expected")
    lead = tuple(k.shape[:-2])
    ns, stride = k.shape[-2], k.shape[-1]
    n = ns if n is None else n
    slices = 1
    for x in lead:
        slices *= x
    ng = (ns + SK2_GROUP - 1) // SK2_GROUP
    dev = torch.device("cuda")
    if out is None:
        out = dict(codes=torch.empty(lead + (ns,), dtype=torch.int64, device=dev),
                   zs=torch.empty(lead + (ng, 2, SK2_CHANNELS), dtype=torch.int16,
                                  device=dev),
                   chan=torch.empty(lead + (SK2_CHANNELS,), dtype=torch.int32,
                                    device=dev))
    a = Sketch2Args(n_slices=slices, n_tokens=n, head_dim=128, out_stride=ns,
                    key_stride=stride if key_stride is None else key_stride,
                    slice_stride=ns * stride, k=_ptr(k),
                    codes=_ptr(out["codes"]), zs=_ptr(out["zs"]),
                    chan=_ptr(out["chan"]))
    nbytes = vkv_sketch2_workspace_bytes(a)
    if nbytes == 0:
        _check(vkv_sketch2_build(a, _stream(stream)))
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = _ptr(ws), nbytes
    _check(vkv_sketch2_build(a, _stream(stream)))
    out["_ws"] = ws
    return out


def append_token(k_new, v_new, pos, host_kv, resident_kv, resident_idx,
                 resident_count, r, status, sketch=None, proj=None,
                 sketch2=None, stream=None):
    """One generated token joins H of every (request, KV head) at ``pos``
    (see vkv_append_args). k_new/v_new [B][G][d] int16 on the device;
    host_kv [B][G][ns][2][d] pinned; the resident arrays, r [B][G][ns],
    the sketches and status on the device, all updated in place."""
    B, G, ns = host_kv.shape[0], host_kv.shape[1], host_kv.shape[2]
    cap = resident_idx.shape[-1]
    a = AppendArgs(batch=B, n_kv_heads=G, head_dim=128, pos=int(pos), cap=cap,
                   ctx_stride=ns,
                   sketch_dim=0 if sketch is None else sketch.shape[-1],
                   k_new=_ptr(k_new), v_new=_ptr(v_new), host_kv=_ptr(host_kv),
                   resident_kv=_ptr(resident_kv), resident_idx=_ptr(resident_idx),
                   resident_count=_ptr(resident_count), r=_ptr(r),
                   sketch=_ptr(sketch), proj=_ptr(proj),
                   sk2_codes=None if sketch2 is None else _ptr(sketch2["codes"]),
                   sk2_zs=None if sketch2 is None else _ptr(sketch2["zs"]),
                   status=_ptr(status))
    _check(vkv_append_token(a, _stream(stream)))


def recompress(tau, host_kv, n, budget, n_sink, n_local, seed, out, layer0=0,
               stream=None, workspace=None):
    """PoissonComp again over the first ``n`` tokens of a decode cache held
    in pinned host memory (host_kv [B][G][ns][2][d]), with fresh scores tau
    [B][G][ns] (first n read). Fills ``out`` (r [B][G][ns], resident_idx,
    resident_count, resident_kv, water_level, status: device tensors)."""
    torch = _torch()
    B, G, ns = host_kv.shape[0], host_kv.shape[1], host_kv.shape[2]
    cap = out["resident_idx"].shape[-1]
    base = host_kv.data_ptr()
    a = CompressArgs(n_layers=B, n_kv_heads=G, n_tokens=n, head_dim=128,
                     layer0=layer0, ctx_stride=ns, kv_stride=256,
                     tau=_ptr(tau), k=ctypes.c_void_p(base),
                     v=ctypes.c_void_p(base + 256), budget=int(budget),
                     n_sink=n_sink, n_local=n_local,
                     seed=int(seed) & 0xFFFFFFFFFFFFFFFF, cap=cap,
                     r=_ptr(out["r"]), resident_idx=_ptr(out["resident_idx"]),
                     resident_count=_ptr(out["resident_count"]),
                     resident_kv=_ptr(out["resident_kv"]),
                     water_level=_ptr(out["water_level"]),
                     status=_ptr(out["status"]))
    nbytes = vkv_compress_workspace_bytes(a)
    if nbytes == 0:
        _check(vkv_compress(a, _stream(stream)))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=out["r"].device)
    a.workspace, a.workspace_bytes = _ptr(workspace), nbytes
    _check(vkv_compress(a, _stream(stream)))
    return workspace


class DecodeStep:
    """Reusable decode-step launcher: outputs and workspace are allocated once
    for a shape, so repeated steps only marshal pointers and launch."""

    def __init__(self, B, Hq, G, n, s, cap, fetch_cap, device, d=128,
                 n_short=128, ctx_stride=None, prefetch_rows=0):
        torch = _torch()
        self.shape = (B, Hq, G, n, s, cap, fetch_cap)
        self.n_short = n_short
        self.ns = n if ctx_stride is None else ctx_stride
        self.out = dict(
            out=torch.empty((B, Hq, d), dtype=torch.float32, device=device),
            d_hat=torch.empty((B, Hq), dtype=torch.float32, device=device),
            log_shift=torch.empty((B, Hq), dtype=torch.float32, device=device),
            eps_hat0=torch.empty((B, Hq), dtype=torch.float32, device=device),
            eps_hat=torch.empty((B, Hq), dtype=torch.float32, device=device),
            k_star=torch.empty((B, Hq), dtype=torch.int32, device=device),
            fetch_idx=torch.empty((B, G, fetch_cap), dtype=torch.int32,
                                  device=device),
            fetch_count=torch.empty((B, G), dtype=torch.int32, device=device),
            host_bytes=torch.zeros((1,), dtype=torch.int64, device=device),
            row_stats=torch.empty((B, Hq, 8), dtype=torch.float64,
                                  device=device),
            row_path=torch.empty((B, Hq), dtype=torch.int32, device=device),
            shortlist=torch.empty((B, G, max(n_short, 1)), dtype=torch.int32,
                                  device=device),
            status=torch.zeros((1,), dtype=torch.int32, device=device))
        self.args = DecodeArgs(batch=B, n_q_heads=Hq, n_kv_heads=G, head_dim=d,
                               n_tokens=n, sketch_dim=s, cap=cap,
                               ctx_stride=self.ns, fetch_cap=fetch_cap,
                               n_short=n_short, prefetch_rows=prefetch_rows)
        for key in ("out", "d_hat", "log_shift", "eps_hat0", "eps_hat", "k_star",
                    "fetch_idx", "fetch_count", "host_bytes", "row_stats",
                    "row_path", "shortlist", "status"):
            setattr(self.args, key, _ptr(self.out[key]))
        nbytes = vkv_decode_workspace_bytes(self.args)
        if nbytes == 0:
            raise VerKVError(VKV_EINVAL, vkv_last_error())
        self.workspace = torch.empty((nbytes,), dtype=torch.uint8, device=device)
        self.args.workspace = _ptr(self.workspace)
        self.args.workspace_bytes = nbytes

    def bind(self, q, resident_kv, resident_idx, resident_count, sketch, proj, r,
             host_kv, eps, delta, estimator=EST_CLIP, weights=W_SKETCH,
             sketch2=None):
        """``sketch2``: with W_SKETCH2, the dict sketch2_build returns for
        keys shaped [B][G][n][...] (codes, zs, chan)."""
        torch = _torch()
        B, Hq, G, n, s, cap, _ = self.shape
        ns = self.ns
        d = 128
        _need(q, torch.int16, (B, Hq, d), "q")
        _need(resident_kv, torch.int16, (B, G, cap, 2, d), "resident_kv")
        _need(resident_idx, torch.int32, (B, G, cap), "resident_idx")
        _need(resident_count, torch.int32, (B, G), "resident_count")
        _need(r, torch.float32, (B, G, ns), "r")
        _need(host_kv, torch.int16, (B, G, ns, 2, d), "host_kv", device=False)
        if weights == W_SKETCH:
            _need(sketch, torch.int16, (B, G, ns, s), "sketch")
            _need(proj, torch.float32, (G, d, s), "proj")
        a = self.args
        if weights == W_SKETCH2:
            ng = (ns + SK2_GROUP - 1) // SK2_GROUP
            _need(sketch2["codes"], torch.int64, (B, G, ns), "sketch2 codes")
            _need(sketch2["zs"], torch.int16, (B, G, ng, 2, SK2_CHANNELS), "sketch2 zs")
            _need(sketch2["chan"], torch.int32, (B, G, SK2_CHANNELS), "sketch2 chan")
            a.sk2_codes = _ptr(sketch2["codes"])
            a.sk2_zs = _ptr(sketch2["zs"])
            a.sk2_chan = _ptr(sketch2["chan"])
        else:
            a.sk2_codes = a.sk2_zs = a.sk2_chan = None
        a.q, a.resident_kv = _ptr(q), _ptr(resident_kv)
        a.resident_idx, a.resident_count = _ptr(resident_idx), _ptr(resident_count)
        a.sketch, a.proj, a.r = _ptr(sketch), _ptr(proj), _ptr(r)
        a.host_kv = _ptr(host_kv)
        a.eps, a.delta = float(eps), float(delta)
        a.estimator, a.weights = int(estimator), int(weights)
        self._keep = (q, resident_kv, resident_idx, resident_count, sketch, proj,
                      r, host_kv, sketch2)
        return self

    def set_tokens(self, n):
        """The context length of the next launch (<= the capacity)."""
        B, Hq, G, _, s, cap, fetch_cap = self.shape
        if not 1 <= n <= self.ns or fetch_cap > n:
            raise ValueError(f"n_tokens {n} outside [fetch_cap, {self.ns}]")
        self.shape = (B, Hq, G, n, s, cap, fetch_cap)
        self.args.n_tokens = n
        nbytes = vkv_decode_workspace_bytes(self.args)
        if nbytes > self.workspace.numel():
            torch = _torch()
            self.workspace = torch.empty((nbytes,), dtype=torch.uint8,
                                         device=self.workspace.device)
            self.args.workspace = _ptr(self.workspace)
        self.args.workspace_bytes = self.workspace.numel()

    def set_staging(self, prev=None, nxt=None):
        """Rows staged by the previous step (prev = (map, rows)) and this
        step's staging (nxt = (map, rows)): maps [B][G][ns] int32, rows
        [B][G][fetch_cap][2][d] int16, device tensors; None for none."""
        a = self.args
        a.stage_map_prev = None if prev is None else _ptr(prev[0])
        a.stage_prev = None if prev is None else _ptr(prev[1])
        a.stage_map_next = None if nxt is None else _ptr(nxt[0])
        a.stage_next = None if nxt is None else _ptr(nxt[1])
        self._stage = (prev, nxt)

    def set_phase_events(self, events):
        """Attach phase_count()+1 torch.cuda.Event objects (or None); None
        entries of the list are skipped by the library."""
        if events is None:
            self._ev = None
            self.args.phase_events = None
            return
        self._ev = (ctypes.c_void_p * len(events))(
            *[None if e is None else e.cuda_event for e in events])
        self.args.phase_events = ctypes.cast(self._ev, ctypes.c_void_p)

    def launch(self, stream=None):
        _check(vkv_decode_step(self.args, _stream(stream)))
        return self.out

    def check_status(self, stream=None):
        rc, bits = vkv_check_status(_ptr(self.out["status"]), _stream(stream))
        return rc, bits


def decode_step(q, resident_kv, resident_idx, resident_count, sketch, proj, r,
                host_kv, eps, delta, fetch_cap=None, estimator=EST_CLIP,
                weights=W_SKETCH, stream=None, sketch2=None, n_short=128):
    """One KVFetch decode step (allocates outputs and workspace)."""
    B, Hq, _ = q.shape
    _, G, cap = resident_idx.shape
    n = r.shape[-1]
    s = sketch.shape[-1] if sketch is not None else 32
    step = DecodeStep(B, Hq, G, n, s, cap, fetch_cap or n, q.device,
                      n_short=n_short)
    step.bind(q, resident_kv, resident_idx, resident_count, sketch, proj, r,
              host_kv, eps, delta, estimator, weights, sketch2)
    return step.launch(stream)


class DenseAttention:
    """Reusable launcher of the exact whole-cache attention (the Dense
    baselines): `kv` [B][G][n][2][d] int16 (bf16 bits) either on the device
    (Dense resident) or in pinned host memory (Dense offload)."""

    def __init__(self, B, Hq, G, n, device, d=128):
        torch = _torch()
        self.shape = (B, Hq, G, n)
        self.out = dict(
            out=torch.empty((B, Hq, d), dtype=torch.float32, device=device),
            log_d=torch.empty((B, Hq), dtype=torch.float32, device=device))
        self.args = DenseArgs(batch=B, n_q_heads=Hq, n_kv_heads=G, head_dim=d,
                              n_tokens=n, out=_ptr(self.out["out"]),
                              log_d=_ptr(self.out["log_d"]))
        nbytes = vkv_dense_workspace_bytes(self.args)
        if nbytes == 0:
            raise VerKVError(VKV_EINVAL, vkv_last_error())
        self.workspace = torch.empty((nbytes,), dtype=torch.uint8, device=device)
        self.args.workspace = _ptr(self.workspace)
        self.args.workspace_bytes = nbytes

    def bind(self, q, kv):
        torch = _torch()
        B, Hq, G, n = self.shape
        _need(q, torch.int16, (B, Hq, 128), "q")
        _need(kv, torch.int16, (B, G, n, 2, 128), "kv", device=kv.is_cuda)
        self.args.q, self.args.kv = _ptr(q), _ptr(kv)
        self._keep = (q, kv)
        return self

    def launch(self, stream=None):
        _check(vkv_dense_attention(self.args, _stream(stream)))
        return self.out
