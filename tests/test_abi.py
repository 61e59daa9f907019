"""The C ABI on the CPU: the library loads, exports every function that
include/verkv.h declares, the ctypes structs match the C layout, and host-side
validation rejects bad arguments before anything is launched."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "verkv.h")

vk = pytest.importorskip("verified_sparse_kv_amd.verkv")


def header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(vkv_\w+)\s*\(", src,
                                 re.MULTILINE)))


def test_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(vk.EXPORTS), names
    lib = ctypes.CDLL(vk.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", vk.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    for name in names:
        assert re.search(rf"\bT {name}$", out, re.MULTILINE), name


def _c_layout(struct, fields):
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "verkv.h"',
            "int main(void) {", f'  printf("%zu\\n", sizeof({struct}));']
    for f in fields:
        prog.append(f'  printf("%zu\\n", offsetof({struct}, {f}));')
    prog.append("  return 0; }")
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "p.c")
        exe = os.path.join(td, "p")
        open(c, "w").write("\n".join(prog))
        subprocess.run(["gcc", "-I", os.path.dirname(HEADER), c, "-o", exe],
                       check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True,
                                               text=True).stdout.split()]
    return vals[0], vals[1:]


@pytest.mark.parametrize("cls,cname", [(vk.CompressArgs, "vkv_compress_args"),
                                       (vk.DecodeArgs, "vkv_decode_args"),
                                       (vk.DenseArgs, "vkv_dense_args"),
                                       (vk.Sketch2Args, "vkv_sketch2_args"),
                                       (vk.AppendArgs, "vkv_append_args")])
def test_struct_layout_matches_c(cls, cname):
    fields = [f for f, _ in cls._fields_]
    size, offs = _c_layout(cname, fields)
    assert ctypes.sizeof(cls) == size
    for f, o in zip(fields, offs):
        assert getattr(cls, f).offset == o, f


def _compress_args(**kw):
    a = vk.CompressArgs(n_layers=2, n_kv_heads=3, n_tokens=5000, head_dim=128,
                        layer0=0, budget=600, n_sink=4, n_local=32, seed=1,
                        cap=1000)
    fake = ctypes.c_void_p(0x1000)
    for f in ("tau", "r", "resident_idx", "resident_count", "status"):
        setattr(a, f, fake)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _decode_args(**kw):
    a = vk.DecodeArgs(batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128,
                      n_tokens=4096, sketch_dim=32, cap=600, eps=0.1, delta=0.05,
                      estimator=0, weights=0, fetch_cap=4096)
    fake = ctypes.c_void_p(0x1000)
    for f in ("q", "resident_kv", "resident_idx", "resident_count", "sketch",
              "proj", "r", "host_kv", "out", "d_hat", "log_shift", "eps_hat0",
              "eps_hat", "k_star", "fetch_idx", "fetch_count", "host_bytes",
              "status"):
        setattr(a, f, fake)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_workspace_sizes():
    a = _compress_args()
    w1 = vk.vkv_compress_workspace_bytes(a)
    assert w1 > 0 and w1 % 256 == 0
    w2 = vk.vkv_compress_workspace_bytes(_compress_args(n_tokens=50000))
    assert w2 > w1
    assert vk.vkv_compress_workspace_bytes(_compress_args(head_dim=64)) == 0
    d = _decode_args()
    dw = vk.vkv_decode_workspace_bytes(d)
    assert dw > 0
    assert vk.vkv_decode_workspace_bytes(_decode_args(n_tokens=1024, fetch_cap=1024)) < dw
    assert vk.vkv_decode_workspace_bytes(_decode_args(cap=300)) < dw
    assert vk.vkv_decode_workspace_bytes(_decode_args(n_q_heads=20)) == 0
    # the read-ahead area: prefetch_rows rows of 2 d bf16 per KV head
    pf = vk.vkv_decode_workspace_bytes(_decode_args(prefetch_rows=1000))
    assert pf >= dw + 2 * 8 * 1000 * 512
    assert vk.vkv_decode_workspace_bytes(_decode_args(prefetch_rows=-1)) > dw
    assert vk.vkv_decode_prefetch_rows(_decode_args(prefetch_rows=1000)) == 1000
    assert vk.vkv_decode_prefetch_rows(_decode_args(prefetch_rows=0)) == 0
    # the library's choice: 6144 (B Hq n / 2^20)^0.6 rows over the B G KV heads
    assert vk.vkv_decode_prefetch_rows(_decode_args(
        batch=1, n_tokens=32768, fetch_cap=32768, prefetch_rows=-1)) == 768
    assert vk.vkv_decode_prefetch_rows(_decode_args(
        batch=16, n_tokens=32768, fetch_cap=32768, prefetch_rows=-1)) == 253
    assert vk.vkv_decode_prefetch_rows(_decode_args(
        batch=4, n_tokens=131072, fetch_cap=131072, prefetch_rows=-1)) == 1013
    assert vk.vkv_decode_prefetch_rows(_decode_args(n_q_heads=20)) == -1
    # with the 2-bit sketch, none below 2^23 query-head tokens
    assert vk.vkv_decode_prefetch_rows(_decode_args(
        batch=1, n_tokens=32768, fetch_cap=32768, weights=2, prefetch_rows=-1)) == 0
    assert vk.vkv_decode_prefetch_rows(_decode_args(
        batch=16, n_tokens=32768, fetch_cap=32768, weights=2, prefetch_rows=-1)) == 253
    # the shapes named in the configs fit easily in 288 GB
    big = _decode_args(batch=16, n_tokens=32768, cap=4600, fetch_cap=32768)
    assert vk.vkv_decode_workspace_bytes(big) < 8 * 2 ** 30


@pytest.mark.parametrize("kw,code,frag", [
    (dict(n_layers=0), vk.VKV_EINVAL, "n_layers"),
    (dict(head_dim=64), vk.VKV_EINVAL, "head_dim"),
    (dict(n_tokens=(1 << 21) + 1), vk.VKV_EINVAL, "n_tokens"),
    (dict(budget=30), vk.VKV_EINVAL, "smaller than"),
    (dict(budget=36), vk.VKV_EINVAL, "exceed"),
    (dict(cap=0), vk.VKV_EINVAL, "cap"),
    (dict(tau=None), vk.VKV_EINVAL, "required"),
    (dict(resident_kv=ctypes.c_void_p(0x1000)), vk.VKV_EINVAL, "k and v"),
    (dict(workspace=None), vk.VKV_EINVAL, "workspace"),
    (dict(ctx_stride=4999), vk.VKV_EINVAL, "ctx_stride"),
    (dict(kv_stride=100), vk.VKV_EINVAL, "kv_stride"),
    (dict(kv_stride=132), vk.VKV_EINVAL, "kv_stride"),
])
def test_compress_validation(kw, code, frag):
    a = _compress_args(**kw)
    if "workspace" not in kw:
        a.workspace = ctypes.c_void_p(0x1000)
        a.workspace_bytes = 1
    assert vk.vkv_compress(a, None) == code
    msg = vk.vkv_last_error()
    assert frag in msg, msg


@pytest.mark.parametrize("kw,code,frag", [
    (dict(eps=0.0), vk.VKV_EINVAL, "eps"),
    (dict(eps=float("inf")), vk.VKV_EINVAL, "eps"),
    (dict(delta=1.0), vk.VKV_EINVAL, "delta"),
    (dict(delta=0.0), vk.VKV_EINVAL, "delta"),
    (dict(n_q_heads=20), vk.VKV_EINVAL, "multiple"),
    (dict(n_q_heads=24), vk.VKV_EUNSUPPORTED, "= 3"),
    (dict(n_q_heads=48, n_kv_heads=4), vk.VKV_EUNSUPPORTED, "12"),
    (dict(sketch_dim=24), vk.VKV_EUNSUPPORTED, "sketch_dim"),
    (dict(fetch_cap=0), vk.VKV_EINVAL, "fetch_cap"),
    (dict(fetch_cap=5000), vk.VKV_EINVAL, "fetch_cap"),
    (dict(n_tokens=1 << 24), vk.VKV_EINVAL, "n_tokens"),
    (dict(n_tokens=(1 << 17) + 1, fetch_cap=1 << 17), vk.VKV_EUNSUPPORTED, "2^17"),
    (dict(estimator=7), vk.VKV_EINVAL, "estimator"),
    (dict(weights=3), vk.VKV_EINVAL, "weights"),
    (dict(sketch=None), vk.VKV_EINVAL, "sketch"),
    (dict(k_star=None), vk.VKV_EINVAL, "output"),
    (dict(host_kv=None), vk.VKV_EINVAL, "required"),
    (dict(weights=2), vk.VKV_EINVAL, "sk2_codes"),
    (dict(ctx_stride=4095), vk.VKV_EINVAL, "ctx_stride"),
    (dict(prefetch_rows=-2), vk.VKV_EINVAL, "prefetch_rows"),
    (dict(prefetch_rows=4097), vk.VKV_EINVAL, "prefetch_rows"),
    (dict(stage_map_prev=ctypes.c_void_p(0x1000)), vk.VKV_EINVAL, "pairs"),
    (dict(stage_map_next=ctypes.c_void_p(0x1000)), vk.VKV_EINVAL, "pairs"),
    (dict(stage_map_prev=ctypes.c_void_p(0x1000), stage_prev=ctypes.c_void_p(0x2000),
          stage_map_next=ctypes.c_void_p(0x1000), stage_next=ctypes.c_void_p(0x3000)),
     vk.VKV_EINVAL, "alias"),
    (dict(weights=2, sk2_codes=ctypes.c_void_p(0x1000), sk2_zs=ctypes.c_void_p(0x1000),
          sk2_chan=ctypes.c_void_p(0x1000), n_short=1025), vk.VKV_EINVAL, "n_short"),
    (dict(weights=2, sk2_codes=ctypes.c_void_p(0x1000), sk2_zs=ctypes.c_void_p(0x1000),
          sk2_chan=ctypes.c_void_p(0x1000), n_short=-1), vk.VKV_EINVAL, "n_short"),
    # the projected sketch is neither needed nor checked with the 2-bit one:
    # validation passes and the pinned-memory check of host_kv is next
    (dict(weights=2, sketch=None, proj=None, sketch_dim=0,
          sk2_codes=ctypes.c_void_p(0x1000), sk2_zs=ctypes.c_void_p(0x1000),
          sk2_chan=ctypes.c_void_p(0x1000), n_short=128), vk.VKV_ENOTPINNED, "host_kv"),
])
def test_decode_validation(kw, code, frag):
    a = _decode_args(**kw)
    a.workspace = ctypes.c_void_p(0x1000)
    a.workspace_bytes = 1 << 40
    assert vk.vkv_decode_step(a, None) == code
    msg = vk.vkv_last_error()
    assert frag in msg, msg


def test_decode_workspace_too_small():
    a = _decode_args()
    a.workspace = ctypes.c_void_p(0x1000)
    a.workspace_bytes = 16
    assert vk.vkv_decode_step(a, None) == vk.VKV_EINVAL
    assert "workspace" in vk.vkv_last_error()


def test_version():
    assert vk.vkv_version() >= 100


def test_phase_names():
    names = vk.decode_phase_names()
    assert len(names) == vk.vkv_decode_phase_count() >= 5
    assert names[0] == "scan" and names[-1] == "attn"
    assert vk.vkv_decode_phase_name(len(names)) is None
    assert vk.vkv_decode_phase_name(-1) is None


def _dense_args(**kw):
    a = vk.DenseArgs(batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     n_tokens=4096)
    fake = ctypes.c_void_p(0x1000)
    for f in ("q", "kv", "out", "log_d"):
        setattr(a, f, fake)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_dense_workspace_sizes():
    w = vk.vkv_dense_workspace_bytes(_dense_args())
    assert w > 0 and w % 256 == 0
    assert vk.vkv_dense_workspace_bytes(_dense_args(n_q_heads=20)) == 0
    assert vk.vkv_dense_workspace_bytes(_dense_args(n_tokens=1)) > 0


@pytest.mark.parametrize("kw,frag", [
    (dict(n_q_heads=20), "multiple"),
    (dict(n_q_heads=24), "1, 2, 4 or 8"),
    (dict(head_dim=64), "head_dim"),
    (dict(n_tokens=0), "n_tokens"),
    (dict(n_tokens=(1 << 24) + 1), "n_tokens"),
    (dict(kv=None), "required"),
    (dict(log_d=None), "required"),
    (dict(workspace=None), "workspace"),
])
def test_dense_validation(kw, frag):
    a = _dense_args(**kw)
    if "workspace" not in kw:
        a.workspace = ctypes.c_void_p(0x1000)
        a.workspace_bytes = 1 << 40
    assert vk.vkv_dense_attention(a, None) == vk.VKV_EINVAL
    msg = vk.vkv_last_error()
    assert frag in msg, msg


def test_one_hip_runtime_in_process():
    """The binding loads torch (when installed) before the library, so the
    process maps a single HIP runtime: the library's pointers and torch's
    must belong to the same one."""
    pytest.importorskip("torch")
    maps = open("/proc/self/maps").read().splitlines()
    hip = {l.split()[-1] for l in maps if "libamdhip64" in l}
    assert len(hip) == 1, hip


def test_noalloc_validation_before_any_launch():
    """The no-allocation decode entry point checks its arguments on the host:
    a caller workspace is refused, and shapes whose workspace exceeds the
    library's buffer return VKV_EUNSUPPORTED, both before touching a GPU."""
    a = _decode_args(batch=16, n_tokens=32768, cap=4700, fetch_cap=32768)
    assert vk.vkv_decode_workspace_bytes(a) > vk.NOALLOC_WORKSPACE_BYTES
    assert vk.vkv_decode_step_noalloc(a, None) == vk.VKV_EUNSUPPORTED
    assert "buffer" in vk.vkv_last_error()
    a = _decode_args()
    a.workspace, a.workspace_bytes = ctypes.c_void_p(0x1000), 1 << 20
    assert vk.vkv_decode_step_noalloc(a, None) == vk.VKV_EINVAL
    assert "NULL" in vk.vkv_last_error()


def _sketch2_args(**kw):
    a = vk.Sketch2Args(n_slices=4, n_tokens=1000, head_dim=128, key_stride=256,
                       slice_stride=256000)
    fake = ctypes.c_void_p(0x1000)
    for f in ("k", "codes", "zs", "chan"):
        setattr(a, f, fake)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_sketch2_workspace_sizes():
    w = vk.vkv_sketch2_workspace_bytes(_sketch2_args())
    assert w > 0 and w % 256 == 0
    assert vk.vkv_sketch2_workspace_bytes(_sketch2_args(n_tokens=100000)) > w
    assert vk.vkv_sketch2_workspace_bytes(_sketch2_args(head_dim=64)) == 0
    assert vk.vkv_sketch2_workspace_bytes(_sketch2_args(key_stride=100)) == 0


@pytest.mark.parametrize("kw,frag", [
    (dict(n_slices=0), "n_slices"),
    (dict(n_tokens=0), "n_tokens"),
    (dict(n_tokens=(1 << 24) + 1), "n_tokens"),
    (dict(head_dim=96), "head_dim"),
    (dict(key_stride=64), "key_stride"),
    (dict(key_stride=260), "key_stride"),
    (dict(slice_stride=4), "slice_stride"),
    (dict(codes=None), "required"),
    (dict(k=ctypes.c_void_p(0x1008)), "aligned"),
    (dict(workspace=None), "workspace"),
])
def test_sketch2_validation(kw, frag):
    a = _sketch2_args(**kw)
    if "workspace" not in kw:
        a.workspace = ctypes.c_void_p(0x1000)
        a.workspace_bytes = 1
    assert vk.vkv_sketch2_build(a, None) == vk.VKV_EINVAL
    msg = vk.vkv_last_error()
    assert frag in msg, msg


def _append_args(**kw):
    a = vk.AppendArgs(batch=2, n_kv_heads=8, head_dim=128, pos=100, cap=64,
                      ctx_stride=200, sketch_dim=0)
    fake = ctypes.c_void_p(0x1000)
    for f in ("k_new", "v_new", "host_kv", "resident_kv", "resident_idx",
              "resident_count", "r", "status"):
        setattr(a, f, fake)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,frag", [
    (dict(batch=0), "batch"),
    (dict(head_dim=64), "head_dim"),
    (dict(ctx_stride=0), "ctx_stride"),
    (dict(pos=200), "pos"),
    (dict(pos=-1), "pos"),
    (dict(cap=0), "cap"),
    (dict(r=None), "required"),
    (dict(sketch=ctypes.c_void_p(0x1000)), "together"),
    (dict(sketch=ctypes.c_void_p(0x1000), proj=ctypes.c_void_p(0x1000),
          sketch_dim=24), "sketch_dim"),
    (dict(sk2_codes=ctypes.c_void_p(0x1000)), "together"),
])
def test_append_validation(kw, frag):
    a = _append_args(**kw)
    assert vk.vkv_append_token(a, None) == vk.VKV_EINVAL
    msg = vk.vkv_last_error()
    assert frag in msg, msg


def test_append_needs_pinned_host_cache():
    """Valid arguments with a host_kv that is not pinned memory: refused
    before any launch."""
    import numpy as np
    buf = np.zeros(16, dtype=np.uint16)
    a = _append_args(host_kv=ctypes.c_void_p(buf.ctypes.data))
    assert vk.vkv_append_token(a, None) == vk.VKV_ENOTPINNED
