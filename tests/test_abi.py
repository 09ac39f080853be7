"""C-ABI checks that need no GPU: libfa.so loads, exports every function that
include/fa.h declares, and rejects invalid arguments with the documented status
before touching the device.  No call here reaches a kernel launch: every call
carries at least one invalid argument."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_tiled_attention_27_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

A = 0x10000   # 16-byte-aligned fake address (never dereferenced: validation fails first)
MIS = A + 4   # misaligned fake address


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def exported(lib_path):
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True,
                         text=True, check=True).stdout
    return set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))


def test_debug_build_exports_both_headers():
    """libfa_debug.so (the event-counter build) exports every fa.h function
    plus fa_debug.h's; the product library libfa.so has no counter entry."""
    debug_lib = os.path.join(os.path.dirname(fa.LIB_PATH), "libfa_debug.so")
    dbg_names = declared_functions(os.path.join(ROOT, "include", "fa_debug.h"))
    assert dbg_names == ["fa_debug_atomic_tiles", "fa_debug_counters"]
    syms = exported(debug_lib)
    for n in declared_functions() + dbg_names:
        assert n in syms, n
    for n in dbg_names:
        assert n not in exported(fa.LIB_PATH), n


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert names == ["fa_bwd", "fa_bwd_alibi", "fa_bwd_noalloc", "fa_bwd_window",
                     "fa_bwd_workspace_bytes", "fa_fwd", "fa_fwd_alibi", "fa_fwd_splitkv",
                     "fa_fwd_splitkv_workspace_bytes", "fa_fwd_window", "fa_status_string"]
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(ctypes.CDLL(fa.LIB_PATH), n)


def test_status_strings():
    for code, name in fa.STATUS.items():
        assert fa.fa_status_string(code).startswith(name)
    assert "unknown" in fa.fa_status_string(99)


def fwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, B=1, Hq=2, Hkv=2, N=128, d=64, scale=0.125,
                causal=0, stream=0)
    args.update(kw)
    return fa.fa_fwd(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2), (dict(N=0), 2), (dict(N=-5), 2),
    (dict(Hq=3, Hkv=2), 2), (dict(scale=0.0), 2), (dict(scale=-1.0), 2),
    (dict(scale=float("inf")), 2), (dict(scale=float("nan")), 2),
    (dict(d=32), 3), (dict(d=96), 3), (dict(d=256), 3),
    # one head's bf16 rows must stay below 2 GiB
    (dict(N=1 << 23, d=128), 2), (dict(N=1 << 24, d=64), 2),
    (dict(q=MIS), 4), (dict(k=MIS), 4), (dict(v=MIS), 4), (dict(o=MIS), 4), (dict(lse=MIS), 4),
])
def test_fwd_rejects(kw, status):
    assert fwd(**kw) == status


@pytest.mark.parametrize("window", [0, -1, -(1 << 31)])
def test_window_rejects_non_positive(window):
    args = dict(q=A, k=A, v=A, o=A, lse=A, B=1, Hq=2, Hkv=2, N=128, d=64, scale=0.125,
                window=window, stream=0)
    assert fa.fa_fwd_window(**args) == 2
    bargs = dict(q=A, k=A, v=A, o=A, lse=A, dout=A, dq=A, dk=A, dv=A, B=1, Hq=2, Hkv=2, N=128,
                 d=64, scale=0.125, window=window, deterministic=1, workspace=A,
                 workspace_bytes=1 << 20, stream=0)
    assert fa.fa_bwd_window(**bargs) == 2


def test_window_validates_like_fa_fwd():
    args = dict(q=A, k=A, v=A, o=A, lse=A, B=1, Hq=2, Hkv=2, N=128, d=64, scale=0.125,
                window=16, stream=0)
    assert fa.fa_fwd_window(**dict(args, q=None)) == 1
    assert fa.fa_fwd_window(**dict(args, d=80)) == 3
    assert fa.fa_fwd_window(**dict(args, o=MIS)) == 4
    bargs = dict(q=A, k=A, v=A, o=A, lse=A, dout=A, dq=A, dk=A, dv=A, B=1, Hq=2, Hkv=2, N=128,
                 d=64, scale=0.125, window=16, deterministic=0, workspace=A,
                 workspace_bytes=1 << 20, stream=0)
    assert fa.fa_bwd_window(**dict(bargs, dk=None)) == 1
    assert fa.fa_bwd_window(**dict(bargs, workspace_bytes=16)) == 5
    assert fa.fa_bwd_window(**dict(bargs, dv=MIS)) == 4


def fwd_split(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, B=1, Hq=2, Hkv=2, N=128, d=64, scale=0.125,
                causal=0, num_splits=4, workspace=A, workspace_bytes=1 << 30, stream=0)
    args.update(kw)
    return fa.fa_fwd_splitkv(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(Hq=3, Hkv=2), 2), (dict(scale=0.0), 2), (dict(N=1 << 23, d=128), 2),
    (dict(num_splits=0), 2), (dict(num_splits=-1), 2), (dict(num_splits=fa.MAX_SPLITS + 1), 2),
    # more workgroups than a 32-bit grid holds
    (dict(B=1 << 14, Hq=1 << 10, Hkv=1, N=4096, num_splits=fa.MAX_SPLITS), 2),
    (dict(d=96), 3),
    (dict(q=MIS), 4), (dict(lse=MIS), 4), (dict(workspace=MIS), 4),
    (dict(workspace=None), 5), (dict(workspace_bytes=0), 5), (dict(workspace_bytes=4096), 5),
])
def test_fwd_splitkv_rejects(kw, status):
    assert fwd_split(**kw) == status


def test_splitkv_workspace_bytes():
    # partial O [S][B*Hq][N][d] and partial LSE [S][B*Hq][N], fp32, each to 256 B
    rows = 4 * 2 * 2 * 1000
    assert fa.fa_fwd_splitkv_workspace_bytes(2, 2, 1, 1000, 128, 4) == \
        (rows * 128 * 4 + 255) // 256 * 256 + (rows * 4 + 255) // 256 * 256
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 3, 64, 2) == 2 * 2 * 3 * 64 * 4 + 256
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 128, 64, 1) == 0   # one pass, no partials
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 128, 64, 0) == 0
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 128, 64, fa.MAX_SPLITS + 1) == 0
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 128, 48, 2) == 0
    need = fa.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 128, 64, 4)
    assert fwd_split(workspace_bytes=need - 1) == 5
    assert fwd_split(workspace_bytes=need, o=MIS) == 4
    # one split needs no workspace: the remaining checks still run
    assert fwd_split(num_splits=1, workspace=None, workspace_bytes=0, v=MIS) == 4


def bwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, dout=A, dq=A, dk=A, dv=A, B=1, Hq=2, Hkv=2, N=128,
                d=64, scale=0.125, causal=1, deterministic=0, workspace=A,
                workspace_bytes=1 << 20, stream=0)
    args.update(kw)
    return fa.fa_bwd(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(lse=None), 1), (dict(dout=None), 1), (dict(dq=None), 1), (dict(dk=None), 1),
    (dict(dv=None), 1),
    (dict(B=0), 2), (dict(Hq=4, Hkv=3), 2), (dict(N=0), 2), (dict(scale=0.0), 2),
    (dict(N=1 << 23, d=128, workspace_bytes=1 << 40), 2),
    (dict(d=80), 3),
    (dict(dq=MIS), 4), (dict(dout=MIS), 4), (dict(lse=MIS), 4),
    (dict(workspace=None), 5), (dict(workspace_bytes=0), 5), (dict(workspace_bytes=1024), 5),
    (dict(workspace=MIS), 4),
])
def test_bwd_rejects(kw, status):
    assert bwd(**kw) == status


def r256(x):
    return (x + 255) // 256 * 256


def atomic_pair_bytes(B, Hq, Hkv, N, d):
    """The paired atomic mode's pairing block and hand-over ring, as fa.h lays them out."""
    P = (-(-N // 128) + 1) // 2
    words = 64 + 22 * B * Hkv * P
    return r256(4 * words) + 4 * 4 * B * Hkv * P * 64 * d


def test_workspace_bytes():
    rows = 2 * 16 * 8192
    per = r256(rows * 4)
    for det in (0, 1):
        assert fa.fa_bwd_workspace_bytes(2, 16, 16, 8192, 128, det) == 2 * per
    assert fa.fa_bwd_workspace_bytes(2, 16, 16, 8192, 128, 3) == \
        2 * per + atomic_pair_bytes(2, 16, 16, 8192, 128)
    # rows are padded to a multiple of 64 per head: N = 3 -> 64 rows per head
    assert fa.fa_bwd_workspace_bytes(1, 2, 2, 3, 64, 0) == 2 * 512
    assert fa.fa_bwd_workspace_bytes(1, 2, 2, 3, 64, 3) == 2 * 512 + atomic_pair_bytes(1, 2, 2, 3, 64)
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 65, 64, 1) == 2 * 512
    # grouped heads: pairing words and ring per kv head
    assert fa.fa_bwd_workspace_bytes(1, 32, 8, 32768, 128, 3) == \
        2 * r256(32 * 32768 * 4) + atomic_pair_bytes(1, 32, 8, 32768, 128)
    assert fa.fa_bwd_workspace_bytes(1, 2, 2, 3, 64, 4) == 0
    assert fa.fa_bwd_workspace_bytes(0, 2, 2, 3, 64, 0) == 0
    assert fa.fa_bwd_workspace_bytes(1, 2, 2, 3, 48, 0) == 0
    # exactly the required size passes validation far enough to reach the other checks
    need = fa.fa_bwd_workspace_bytes(1, 2, 2, 128, 64, 0)
    assert bwd(workspace_bytes=need - 1) == 5
    assert bwd(workspace_bytes=need, dv=MIS) == 4


def test_library_has_no_oracle_dependency():
    """The product library links nothing from oracle/ and names no oracle symbol."""
    out = subprocess.run(["nm", "-D", fa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert "oracle" not in out
    ldd = subprocess.run(["ldd", fa.LIB_PATH], capture_output=True, text=True).stdout
    assert "liboracle" not in ldd


def test_single_hip_runtime_in_process():
    """Importing the package (even before torch) maps exactly one HIP runtime,
    so the library's launches and torch's allocations/streams share it."""
    code = ("import re, exact_tiled_attention_27_amd, torch\n"
            "m = open('/proc/self/maps').read()\n"
            "print(len(set(re.findall(r'\\S*libamdhip64\\S*', m))))\n")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT,
                         check=True).stdout.strip()
    assert out == "1"


@pytest.mark.parametrize("mode", [-1, 4, 1 << 20])
def test_bwd_rejects_unknown_dq_mode(mode):
    assert fa.fa_bwd_workspace_bytes(1, 2, 2, 128, 64, mode) == 0
    assert bwd(deterministic=mode) == 2
    bargs = dict(q=A, k=A, v=A, o=A, lse=A, dout=A, dq=A, dk=A, dv=A, B=1, Hq=2, Hkv=2, N=128,
                 d=64, scale=0.125, window=16, deterministic=mode, workspace=A,
                 workspace_bytes=1 << 20, stream=0)
    assert fa.fa_bwd_window(**bargs) == 2


def test_bwd_ordered_workspace_bytes():
    # D and LSE2 ([B*Hq][N'] fp32 each, N' = N rounded up to 64, each to 256 B),
    # then 64 + 4 * B*Hq*N'/64 int32 counters, to 256 B
    for B, Hq, Hkv, N, d in ((1, 2, 2, 128, 64), (2, 4, 2, 1000, 128), (1, 1, 1, 1, 64)):
        npad = (N + 63) // 64 * 64
        rows = (B * Hq * npad * 4 + 255) // 256 * 256
        sync = ((64 + 4 * B * Hq * npad // 64) * 4 + 255) // 256 * 256
        assert fa.fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, fa.BWD_SEPARATE) == 2 * rows
        assert fa.fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, fa.BWD_ATOMIC) == 2 * rows
        assert fa.fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, fa.BWD_ATOMIC_PAIRED) == \
            2 * rows + atomic_pair_bytes(B, Hq, Hkv, N, d)
        assert fa.fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, fa.BWD_ORDERED) == 2 * rows + sync
    for mode in (fa.BWD_ORDERED, fa.BWD_ATOMIC_PAIRED):
        need = fa.fa_bwd_workspace_bytes(1, 2, 2, 128, 64, mode)
        assert bwd(deterministic=mode, workspace_bytes=need - 1) == 5
        assert bwd(deterministic=mode, workspace_bytes=need, dq=MIS) == 4


def test_alibi_validates():
    """The bias entry points need their slopes (FA_ERR_NULL; 4-byte alignment)
    and otherwise check like fa_fwd / fa_bwd."""
    args = dict(q=A, k=A, v=A, o=A, lse=A, slopes=A, B=1, Hq=2, Hkv=2, N=128, d=64,
                scale=0.125, causal=1, stream=0)
    assert fa.fa_fwd_alibi(**dict(args, slopes=None)) == 1
    assert fa.fa_fwd_alibi(**dict(args, slopes=A + 2)) == 4
    assert fa.fa_fwd_alibi(**dict(args, q=None)) == 1
    assert fa.fa_fwd_alibi(**dict(args, Hq=3)) == 2
    assert fa.fa_fwd_alibi(**dict(args, d=96)) == 3
    assert fa.fa_fwd_alibi(**dict(args, o=MIS)) == 4
    bargs = dict(q=A, k=A, v=A, o=A, lse=A, dout=A, dq=A, dk=A, dv=A, slopes=A, B=1, Hq=2,
                 Hkv=2, N=128, d=64, scale=0.125, causal=0, deterministic=1, workspace=A,
                 workspace_bytes=1 << 20, stream=0)
    assert fa.fa_bwd_alibi(**dict(bargs, slopes=None)) == 1
    assert fa.fa_bwd_alibi(**dict(bargs, slopes=A + 1)) == 4
    assert fa.fa_bwd_alibi(**dict(bargs, dk=None)) == 1
    assert fa.fa_bwd_alibi(**dict(bargs, deterministic=4)) == 2
    assert fa.fa_bwd_alibi(**dict(bargs, workspace_bytes=16)) == 5
    assert fa.fa_bwd_alibi(**dict(bargs, dv=MIS)) == 4


def test_noalloc_checks_arguments_before_the_device():
    """fa_bwd_noalloc refuses bad arguments, and a workspace beyond
    FA_NOALLOC_MAX_WORKSPACE, before any HIP call (fake aligned addresses)."""
    base = dict(q=A, k=A, v=A, o=A, lse=A, dout=A, dq=A, dk=A, dv=A, B=1, Hq=64, Hkv=64,
                N=131072, d=128, scale=0.1, causal=1, deterministic=1)
    need = fa.fa_bwd_workspace_bytes(1, 64, 64, 131072, 128, 1)
    assert need > fa.NOALLOC_MAX_WORKSPACE
    assert fa.fa_bwd_noalloc(**base) == 5
    assert fa.fa_bwd_noalloc(**{**base, "dq": None}) == 1
    assert fa.fa_bwd_noalloc(**{**base, "dk": MIS}) == 4
    assert fa.fa_bwd_noalloc(**{**base, "deterministic": 4}) == 2
    assert fa.fa_bwd_noalloc(**{**base, "d": 96}) == 3
    # The paired mode's hand-over ring counts against the limit: B1 Hq8 Hkv8
    # N8192 d128 fits in the other modes but not in the paired one.
    small = {**base, "Hq": 8, "Hkv": 8, "N": 8192}
    assert fa.fa_bwd_workspace_bytes(1, 8, 8, 8192, 128, 0) <= fa.NOALLOC_MAX_WORKSPACE
    assert fa.fa_bwd_workspace_bytes(1, 8, 8, 8192, 128, 3) > fa.NOALLOC_MAX_WORKSPACE
    assert fa.fa_bwd_noalloc(**{**small, "deterministic": 3}) == 5
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    assert "#define FA_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)" in src
    assert fa.NOALLOC_MAX_WORKSPACE == 32 << 20
