"""The C ABI of libfa2.so on the CPU: exports, work decomposition and every error path.

Nothing here launches a kernel.  Invalid arguments are rejected before any HIP
call; the HIP-error path is exercised only where no GPU is visible.
"""
from __future__ import annotations

import ctypes
import json
import os
import re
import subprocess

import pytest
import torch

from exact_attention_62_amd import fa2 as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(F.library_path()),
                                reason="libfa2.so not built (python -m exact_attention_62_amd.build)")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails before a launch


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared_functions() == ["fa2_bwd", "fa2_bwd_block_map", "fa2_bwd_cross",
                                     "fa2_bwd_workspace_size", "fa2_fwd",
                                     "fa2_fwd_cross", "fa2_fwd_partial", "fa2_fwd_splitkv",
                                     "fa2_fwd_splitkv_noalloc", "fa2_last_error", "fa2_launch_shape", "fa2_merge",
                                     "fa2_num_splits", "fa2_schedule_blocks",
                                     "fa2_schedule_map", "fa2_splitkv_workspace_size",
                                     "fa2_strerror"]


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", F.library_path()], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa2_\w+)", out))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(F.load_library(), name)


def _fwd(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, L=FAKE + 0x400000,
         B=1, H=1, N=16, d=64, causal=0, scale=0.125, dtype=F.FA2_BF16):
    lib = F.load_library()
    return lib.fa2_fwd(q, k, v, o, L, B, H, N, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,needle", [
    (dict(q=None), "Q is NULL"),
    (dict(L=None), "L is NULL"),
    (dict(v=FAKE + 8), "V="),
    (dict(L=FAKE + 0x400002), "4-byte aligned"),
    (dict(B=-1), "sizes must be >= 0"),
    (dict(N=-5), "sizes must be >= 0"),
    (dict(causal=2), "causal=2"),
    (dict(scale=float("nan")), "finite"),
    (dict(scale=float("inf")), "finite"),
    (dict(o=FAKE), "overlaps"),
    (dict(L=FAKE + 0x300000 + 64), "overlaps"),
    (dict(N=(1 << 31) // 256 + 1), "maximum"),
    (dict(B=1 << 20, H=1 << 12), "exceeds"),
])
def test_invalid_arguments_are_rejected_before_any_hip_call(kw, needle):
    assert _fwd(**kw) == F.FA2_EINVAL
    assert needle in F.fa2_last_error()


@pytest.mark.parametrize("kw", [dict(d=48), dict(d=16), dict(d=512), dict(d=0), dict(dtype=7)])
def test_unsupported_requests(kw):
    assert _fwd(**kw) == F.FA2_ENOTSUP
    assert F.fa2_last_error()


def test_empty_problem_is_a_no_op():
    for kw in (dict(B=0), dict(H=0), dict(N=0)):
        assert _fwd(q=None, k=None, v=None, o=None, L=None, **kw) == F.FA2_OK
        assert F.fa2_last_error() == ""


def test_strerror_covers_every_status():
    assert F.fa2_strerror(0) == "success"
    for s in (F.FA2_EINVAL, F.FA2_ENOTSUP, F.FA2_EHIP):
        assert F.fa2_strerror(s) not in ("", "unknown status")
    assert F.fa2_strerror(42) == "unknown status"


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a visible GPU")
@pytest.mark.parametrize("kw", [dict(), dict(dtype=F.FA2_FP16), dict(dtype=F.FA2_FP32),
                                dict(d=32), dict(d=96)])
def test_valid_call_without_a_device_reports_the_hip_error(kw):
    assert _fwd(**kw) == F.FA2_EHIP
    assert "hip" in F.fa2_last_error().lower()


# ---- query and key lengths that differ -------------------------------------------------
def _cross(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, L=FAKE + 0x400000,
           B=1, H=1, Nq=16, Nk=40, d=64, causal=1, scale=0.125, dtype=F.FA2_BF16):
    lib = F.load_library()
    return lib.fa2_fwd_cross(q, k, v, o, L, B, H, Nq, Nk, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(Nq=-1), F.FA2_EINVAL, "sizes must be >= 0"),
    (dict(Nk=-2), F.FA2_EINVAL, "sizes must be >= 0"),
    (dict(Nk=(1 << 31) // 256 + 1), F.FA2_EINVAL, "maximum"),
    (dict(k=None), F.FA2_EINVAL, "K is NULL"),
    # K and V hold 40 rows of 128 bytes: O placed 1 KB after K's start overlaps K
    (dict(o=FAKE + 0x100000 + 1024), F.FA2_EINVAL, "O overlaps K"),
    (dict(d=80), F.FA2_ENOTSUP, "d=80"),
])
def test_cross_invalid_arguments_before_any_hip_call(kw, status, needle):
    assert _cross(**kw) == status
    assert needle in F.fa2_last_error()


def test_cross_empty_query_side_is_a_no_op():
    assert _cross(q=None, k=None, v=None, o=None, L=None, Nq=0) == F.FA2_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a visible GPU")
def test_cross_without_keys_does_not_need_k_or_v():
    # Nk == 0 passes the argument checks with K = V = NULL (they are not read); the call then
    # needs the device.
    assert _cross(k=None, v=None, Nk=0) == F.FA2_EHIP
    assert "K is NULL" not in F.fa2_last_error()


def test_grid_matches_the_pages_worked_example():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "grid_example.json")))
    kBlockM, _, _ = F.fa2_launch_shape(1, 1, 1, 128)
    N = g["num_m_block"] * kBlockM
    km, nmb, blocks = F.fa2_launch_shape(g["batch_size"], g["num_heads"], N, 128)
    assert (km, nmb, blocks) == (kBlockM, g["num_m_block"], g["blocks"])
    # A ragged length rounds the row blocks up.
    assert F.fa2_launch_shape(1, 2, N - 1, 128)[1:] == (4, 8)
    assert F.fa2_launch_shape(1, 2, N + 1, 128)[1:] == (5, 10)


def test_grid_of_the_named_workloads():
    # (kBlockM, query blocks, items) for the five workloads (bf16): 128 query
    # rows per workgroup (four wavefronts of 32), 256 for d = 128 (eight).
    assert F.fa2_launch_shape(2, 4, 1024, 64) == (128, 8, 64)
    assert F.fa2_launch_shape(16, 16, 2048, 128) == (256, 8, 2048)
    assert F.fa2_launch_shape(1, 16, 16384, 128) == (256, 64, 1024)
    assert F.fa2_launch_shape(2, 16, 8191, 256) == (128, 64, 2048)
    # d = 128 takes 256-row blocks only on grids of at least 256 such items.
    assert F.fa2_launch_shape(1, 16, 4096, 128) == (256, 16, 256)
    assert F.fa2_launch_shape(1, 16, 3840, 128) == (128, 30, 480)
    assert F.fa2_launch_shape(1, 64, 1000, 128) == (256, 4, 256)
    assert F.fa2_launch_shape(64, 1, 1000, 64) == (128, 8, 512)
    assert F.fa2_launch_shape(1, 1, 128, 64, torch.float32) == (4, 32, 32)


def test_launch_shape_rejects_what_fwd_rejects():
    with pytest.raises(F.FA2Error) as e:
        F.fa2_launch_shape(1, 1, 16, 100)
    assert e.value.status == F.FA2_ENOTSUP
    with pytest.raises(F.FA2Error) as e:
        F.fa2_launch_shape(-1, 1, 16, 64)
    assert e.value.status == F.FA2_EINVAL


def test_binding_rejects_cpu_tensors():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        F.fa2_fwd(q, q.clone(), q.clone(), q.clone(), torch.zeros(1, 1, 8))
    with pytest.raises(ValueError, match="shape"):
        F.fa2_fwd(q, q[:, :, :4].clone(), q.clone(), q.clone(), torch.zeros(1, 1, 8))
    with pytest.raises(ValueError, match="lse"):
        F.fa2_fwd(q, q.clone(), q.clone(), q.clone(), torch.zeros(1, 1, 8, dtype=torch.float64))


def test_last_error_is_thread_local():
    import threading
    assert _fwd(causal=5) == F.FA2_EINVAL
    seen = {}

    def other():
        seen["msg"] = F.fa2_last_error()
        _fwd(d=48)

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "causal=5" in F.fa2_last_error()


# ---- split-KV entry points ---------------------------------------------------------------
def _split(ws=FAKE + 0x500000, ws_bytes=1 << 24, num_splits=2, dtype=F.FA2_BF16, **kw):
    args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000,
                L=FAKE + 0x400000, B=1, H=1, Nq=16, Nk=16, d=64, causal=0, scale=0.125)
    args.update(kw)
    lib = F.load_library()
    return lib.fa2_fwd_splitkv(args["q"], args["k"], args["v"], args["o"], args["L"], args["B"],
                               args["H"], args["Nq"], args["Nk"], args["d"], args["causal"],
                               args["scale"], dtype, num_splits, ws, ws_bytes, None)


def test_workspace_size_formula():
    # num_splits * B*H*Nq * (d + 1) float32 values: O_s and L_s of every split
    assert F.fa2_splitkv_workspace_size(2, 4, 1024, 1024, 64, 8) == 8 * 2 * 4 * 1024 * 65 * 4
    assert F.fa2_splitkv_workspace_size(1, 1, 1, 1, 256, 1) == 257 * 4
    assert F.fa2_splitkv_workspace_size(0, 4, 1024, 1024, 64, 3) == 0
    assert F.fa2_splitkv_workspace_size(1, 2, 5, 4096, 128, 3) == 3 * 2 * 5 * 129 * 4
    assert F.fa2_splitkv_workspace_size(1, 1, 8, 8, 96, 2) == 2 * 8 * 97 * 4


@pytest.mark.parametrize("s", [0, -1, 129])
def test_workspace_size_rejects_split_counts(s):
    with pytest.raises(F.FA2Error) as e:
        F.fa2_splitkv_workspace_size(1, 1, 64, 64, 64, s)
    assert e.value.status == F.FA2_EINVAL and "num_splits" in str(e.value)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=F.FA2_FP32), F.FA2_ENOTSUP, "FA2_BF16 and FA2_FP16 only"),
    (dict(d=48), F.FA2_ENOTSUP, "d=48"),
    (dict(Nk=-1), F.FA2_EINVAL, "sizes must be >= 0"),
    (dict(num_splits=-1), F.FA2_EINVAL, "num_splits=-1"),
    (dict(num_splits=200), F.FA2_EINVAL, "num_splits=200"),
    (dict(ws=None), F.FA2_EINVAL, "workspace is NULL"),
    (dict(ws=FAKE + 0x500004), F.FA2_EINVAL, "workspace="),
    (dict(ws_bytes=100), F.FA2_EINVAL, "smaller than"),
    (dict(ws=FAKE + 0x300000 + 512), F.FA2_EINVAL, "overlaps"),
    (dict(o=FAKE + 0x500000 + 64), F.FA2_EINVAL, "overlaps"),
    (dict(causal=3), F.FA2_EINVAL, "causal=3"),
])
def test_splitkv_invalid_arguments_before_any_hip_call(kw, status, needle):
    assert _split(**kw) == status
    assert needle in F.fa2_last_error()


def _split_noalloc(num_splits=2, dtype=F.FA2_BF16, **kw):
    args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000,
                L=FAKE + 0x400000, B=1, H=1, Nq=16, Nk=16, d=64, causal=0, scale=0.125)
    args.update(kw)
    return F.load_library().fa2_fwd_splitkv_noalloc(
        args["q"], args["k"], args["v"], args["o"], args["L"], args["B"], args["H"], args["Nq"],
        args["Nk"], args["d"], args["causal"], args["scale"], dtype, num_splits, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=F.FA2_FP32), F.FA2_ENOTSUP, "FA2_BF16 and FA2_FP16 only"),
    (dict(num_splits=-1), F.FA2_EINVAL, "num_splits=-1"),
    (dict(num_splits=129), F.FA2_EINVAL, "num_splits=129"),
    (dict(q=None), F.FA2_EINVAL, "Q is NULL"),
    (dict(o=FAKE), F.FA2_EINVAL, "overlaps"),
    # 8 * 64 * 1024 * 129 * 4 bytes of partial results: over the 32 MiB scratch
    (dict(B=4, H=16, Nq=1024, Nk=1024, d=128, num_splits=8), F.FA2_EINVAL, "library scratch"),
])
def test_splitkv_noalloc_invalid_arguments_before_any_hip_call(kw, status, needle):
    assert _split_noalloc(**kw) == status
    assert needle in F.fa2_last_error()


def test_splitkv_noalloc_limit_is_inclusive():
    # 2 splits * 64527 rows * 65 * 4 bytes fit the 32 MiB scratch: the size check passes
    # and the call fails later, on the fake pointers (or on the missing device).
    nq = (32 << 20) // (4 * 65 * 2)
    step = 0x1000000
    st = _split_noalloc(q=FAKE, k=FAKE + step, v=FAKE + 2 * step, o=FAKE + 3 * step,
                        L=FAKE + 4 * step, Nq=nq, Nk=64, num_splits=2)
    assert st != F.FA2_OK and "library scratch" not in F.fa2_last_error()
    st = _split_noalloc(q=FAKE, k=FAKE + step, v=FAKE + 2 * step, o=FAKE + 3 * step,
                        L=FAKE + 4 * step, Nq=nq + 1, Nk=64, num_splits=2)
    assert st == F.FA2_EINVAL and "library scratch" in F.fa2_last_error()


def test_splitkv_noalloc_scratch_size_constant():
    text = open(HEADER).read()
    assert "#define FA2_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in text


def test_splitkv_empty_problem_is_a_no_op():
    assert _split(q=None, k=None, v=None, o=None, L=None, ws=None, ws_bytes=0, B=0) == F.FA2_OK
    assert _split(q=None, k=None, v=None, o=None, L=None, ws=None, ws_bytes=0, Nq=0) == F.FA2_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a visible GPU")
def test_num_splits_without_a_device_reports_the_hip_error():
    out = ctypes.c_int(0)
    assert F.load_library().fa2_num_splits(1, 1, 1024, 1024, 64, ctypes.byref(out)) == F.FA2_EHIP
    assert _split(num_splits=0) == F.FA2_EHIP  # the rule needs the device's CU count


# ---- backward entry points ---------------------------------------------------------------
def _bwd(dtype=F.FA2_BF16, ws_bytes=1 << 16, **kw):
    base = FAKE
    a = dict(q=base, k=base + 0x100000, v=base + 0x200000, o=base + 0x300000, do=base + 0x400000,
             L=base + 0x500000, dq=base + 0x600000, dk=base + 0x700000, dv=base + 0x800000,
             ws=base + 0x900000, B=1, H=1, N=16, d=64, causal=0, scale=0.125)
    a.update(kw)
    return F.load_library().fa2_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["L"], a["dq"],
                                    a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["causal"],
                                    a["scale"], dtype, a["ws"], ws_bytes, None)


def test_bwd_workspace_size_formula():
    # two float32 arrays (D and L*log2 e), each head's rows padded to a multiple of 32
    assert F.fa2_bwd_workspace_size(2, 4, 1024, 64) == 2 * 4 * 1024 * 8
    assert F.fa2_bwd_workspace_size(2, 4, 1000, 64) == 2 * 4 * 1024 * 8
    assert F.fa2_bwd_workspace_size(1, 3, 33, 128) == 3 * 64 * 8
    assert F.fa2_bwd_workspace_size(1, 1, 0, 128) == 0
    # every forward head dimension has a backward; others are refused
    for d in (32, 64, 96, 128, 256):
        assert F.fa2_bwd_workspace_size(1, 1, 16, d) == 32 * 8
    with pytest.raises(F.FA2Error) as e:
        F.fa2_bwd_workspace_size(1, 1, 16, 80)
    assert e.value.status == F.FA2_ENOTSUP


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=F.FA2_FP32), F.FA2_ENOTSUP, "FA2_BF16 and FA2_FP16 only"),
    (dict(d=80), F.FA2_ENOTSUP, "d=80"),
    (dict(d=48), F.FA2_ENOTSUP, "d=48"),
    (dict(do=None), F.FA2_EINVAL, "dO is NULL"),
    (dict(ws=None), F.FA2_EINVAL, "workspace is NULL"),
    (dict(dk=FAKE + 0x700008), F.FA2_EINVAL, "dK="),
    (dict(ws_bytes=8), F.FA2_EINVAL, "smaller than"),
    (dict(dq=FAKE + 64), F.FA2_EINVAL, "dQ overlaps Q"),
    (dict(dv=FAKE + 0x600000 + 128), F.FA2_EINVAL, "overlaps"),
    (dict(causal=7), F.FA2_EINVAL, "causal=7"),
    (dict(scale=float("nan")), F.FA2_EINVAL, "finite"),
])
def test_bwd_invalid_arguments_before_any_hip_call(kw, status, needle):
    assert _bwd(**kw) == status
    assert needle in F.fa2_last_error()


def test_bwd_empty_problem_is_a_no_op():
    nulls = dict(q=None, k=None, v=None, o=None, do=None, L=None, dq=None, dk=None, dv=None,
                 ws=None)
    assert _bwd(N=0, **nulls) == F.FA2_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a visible GPU")
def test_bwd_without_a_device_reports_the_hip_error():
    assert _bwd() == F.FA2_EHIP


# ---- partial results and their merge -----------------------------------------------------
def _partial(dtype=F.FA2_BF16, **kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, L=FAKE + 0x400000,
             B=1, H=1, Nq=16, Nk=64, d=64, causal=0, scale=0.125)
    a.update(kw)
    return F.load_library().fa2_fwd_partial(a["q"], a["k"], a["v"], a["o"], a["L"], a["B"], a["H"],
                                            a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"],
                                            dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=F.FA2_FP32), F.FA2_ENOTSUP, "FA2_BF16 and FA2_FP16 only"),
    (dict(o=None), F.FA2_EINVAL, "O is NULL"),
    # O_part is float32: 16 rows x 64 dims x 4 bytes = 4 KB, so L placed 2 KB in overlaps it
    (dict(L=FAKE + 0x300000 + 2048), F.FA2_EINVAL, "O overlaps L"),
    (dict(Nk=-1), F.FA2_EINVAL, "sizes must be >= 0"),
    (dict(d=40), F.FA2_ENOTSUP, "d=40"),
])
def test_partial_invalid_arguments_before_any_hip_call(kw, status, needle):
    assert _partial(**kw) == status
    assert needle in F.fa2_last_error()


def _merge(dtype=F.FA2_BF16, **kw):
    a = dict(op=FAKE, lp=FAKE + 0x400000, o=FAKE + 0x500000, L=FAKE + 0x600000, S=3, rows=64, d=64)
    a.update(kw)
    return F.load_library().fa2_merge(a["op"], a["lp"], a["S"], a["o"], a["L"], a["rows"], a["d"],
                                      dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(S=0), F.FA2_EINVAL, "num_parts=0"),
    (dict(S=129), F.FA2_EINVAL, "num_parts=129"),
    (dict(rows=-1), F.FA2_EINVAL, "rows=-1"),
    (dict(d=100), F.FA2_ENOTSUP, "d=100"),
    (dict(dtype=9), F.FA2_ENOTSUP, "dtype 9"),
    (dict(op=None), F.FA2_EINVAL, "O_parts is NULL"),
    (dict(lp=FAKE + 0x400002), F.FA2_EINVAL, "4-byte aligned"),
    (dict(o=FAKE + 0x100), F.FA2_EINVAL, "O overlaps O_parts"),
])
def test_merge_invalid_arguments_before_any_hip_call(kw, status, needle):
    assert _merge(**kw) == status
    assert needle in F.fa2_last_error()


def test_merge_of_no_rows_is_a_no_op():
    assert _merge(op=None, lp=None, o=None, L=None, rows=0) == F.FA2_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a visible GPU")
def test_partial_and_merge_without_a_device_report_the_hip_error():
    assert _partial() == F.FA2_EHIP
    assert _merge() == F.FA2_EHIP


def _bwd_cross(dtype=F.FA2_BF16, ws_bytes=1 << 16, **kw):
    base = FAKE
    a = dict(q=base, k=base + 0x100000, v=base + 0x200000, o=base + 0x300000, do=base + 0x400000,
             L=base + 0x500000, dq=base + 0x600000, dk=base + 0x700000, dv=base + 0x800000,
             ws=base + 0x900000, B=1, H=1, Nq=16, Nk=48, d=64, causal=1, scale=0.125)
    a.update(kw)
    return F.load_library().fa2_bwd_cross(
        a["q"], a["k"], a["v"], a["o"], a["do"], a["L"], a["dq"], a["dk"], a["dv"], a["B"], a["H"],
        a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"], dtype, a["ws"], ws_bytes, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(Nk=-1), F.FA2_EINVAL, "sizes must be >= 0"),
    (dict(dk=None), F.FA2_EINVAL, "dK is NULL"),
    # dK holds 48 rows of 128 bytes: dV placed 4 KB after its start overlaps it
    (dict(dv=FAKE + 0x700000 + 4096), F.FA2_EINVAL, "overlaps"),
    (dict(d=80), F.FA2_ENOTSUP, "d=80"),
])
def test_bwd_cross_invalid_arguments_before_any_hip_call(kw, status, needle):
    assert _bwd_cross(**kw) == status
    assert needle in F.fa2_last_error()


def test_bwd_cross_empty_problem_is_a_no_op():
    nulls = dict(q=None, k=None, v=None, o=None, do=None, L=None, dq=None, dk=None, dv=None,
                 ws=None)
    assert _bwd_cross(Nq=0, Nk=0, **nulls) == F.FA2_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a visible GPU")
def test_bwd_cross_zero_size_sides_need_no_pointers():
    # No queries: Q, O, dO, L, dQ and the workspace are empty and may be NULL (dK = dV = 0 is
    # still written, so the call then needs the device); likewise K, V, dK, dV without keys.
    assert _bwd_cross(q=None, o=None, do=None, L=None, dq=None, ws=None, ws_bytes=0, Nq=0) == F.FA2_EHIP
    assert _bwd_cross(k=None, v=None, dk=None, dv=None, Nk=0) == F.FA2_EHIP


def test_enums_span_every_int32_value():
    """fa2_dtype_t and fa2_status_t carry a 0x7fffffff member, so any 32-bit code a caller
    passes is a valid value of the type (no undefined behaviour before the dtype check)."""
    text = open(HEADER).read()
    assert "FA2_DTYPE_INVALID = -1" in text and "FA2_DTYPE_MAX_ENUM = 0x7fffffff" in text
    assert "FA2_STATUS_MAX_ENUM = 0x7fffffff" in text
    for code in (3, 7, -1, -(1 << 31), 0x7fffffff):
        assert _fwd(dtype=code) == F.FA2_ENOTSUP
