"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function that
include/*.h declares, and rejects invalid arguments with the documented status before touching
the GPU (invalid calls return before the first HIP call, so dummy pointers are never used)."""
import ctypes
import glob
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import exact_io_aware_flash_amd as fa
    if not os.path.exists(fa.LIB_PATH):
        from exact_io_aware_flash_amd import build
        build.build()
    return fa.lib()


def declared_functions():
    names = []
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(flash_attn_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("flash_attn_fwd", "flash_attn_bwd", "flash_attn_fwd_f32", "flash_attn_bwd_f32",
              "flash_attn_bwd_workspace_bytes", "flash_attn_status_string", "flash_attn_bwd_preprocess",
              "flash_attn_bwd_dkdv", "flash_attn_bwd_dq", "flash_attn_fwd_splitkv",
              "flash_attn_fwd_splitkv_workspace_bytes", "flash_attn_merge", "flash_attn_fwd_mxfp8",
              "flash_attn_mxfp8_quantize_rows", "flash_attn_mxfp8_quantize_vt", "flash_attn_mxfp8_vt_cols"):
        assert n in names, n


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in include/ but not exported"


def test_status_strings(L):
    import exact_io_aware_flash_amd as fa
    for code in range(0, 11):
        s = fa.status_string(code)
        assert s and s != "unknown status", code
    assert fa.status_string(12345) == "unknown status"


def test_workspace_bytes(L):
    import exact_io_aware_flash_amd as fa
    a256 = lambda x: (x + 255) // 256 * 256
    for B, H, N, d in ((1, 1, 1, 64), (2, 3, 100, 128), (1, 32, 16384, 128), (4, 16, 8192, 64)):
        assert fa.workspace_bytes(B, H, N, d) == a256(B * H * N * 4), (B, H, N, d)
    assert fa.workspace_bytes(0, 1, 1, 64) == 0
    assert fa.workspace_bytes(1, 1, 1, 96) == 0


# fake, 16-byte aligned, non-overlapping device addresses: never dereferenced by invalid calls
BIG = 1 << 36


def ptrs(n, start=1 << 40):
    return [ctypes.c_void_p(start + i * BIG) for i in range(n)]


def fwd_call(L, q, k, v, o, lse, B=1, H=1, N=128, d=64, scale=0.125, causal=0, mask=None, f32=False):
    fn = L.flash_attn_fwd_f32 if f32 else L.flash_attn_fwd
    return fn(q, k, v, o, lse, B, H, N, d, scale, causal, mask, None)


@pytest.mark.parametrize("f32", [False, True])
def test_fwd_argument_errors(L, f32):
    import exact_io_aware_flash_amd as fa
    q, k, v, o, lse = ptrs(5)
    assert fwd_call(L, None, k, v, o, lse, f32=f32) == fa.FA_ERR_NULL
    assert fwd_call(L, q, k, v, o, None, f32=f32) == fa.FA_ERR_NULL
    assert fwd_call(L, q, k, v, o, lse, N=0, f32=f32) == fa.FA_ERR_SHAPE
    assert fwd_call(L, q, k, v, o, lse, B=0, f32=f32) == fa.FA_ERR_SHAPE
    assert fwd_call(L, q, k, v, o, lse, H=-1, f32=f32) == fa.FA_ERR_SHAPE
    for d in (0, 32, 96, 256):
        assert fwd_call(L, q, k, v, o, lse, d=d, f32=f32) == fa.FA_ERR_HEADDIM
    for s in (0.0, -0.0, float("inf"), -float("inf"), float("nan")):
        assert fwd_call(L, q, k, v, o, lse, scale=s, f32=f32) == fa.FA_ERR_SCALE
    assert fwd_call(L, q, k, v, o, lse, causal=2, f32=f32) == fa.FA_ERR_FLAG
    mis = ctypes.c_void_p(q.value + 8)
    assert fwd_call(L, mis, k, v, o, lse, f32=f32) == fa.FA_ERR_ALIGN
    # any finite nonzero scale passes validation, negative ones included: these calls get as far
    # as the alignment check (so nothing is launched on the fake pointers)
    for s in (-0.5, -1e-30, -3e38, 1e-30):
        assert fwd_call(L, mis, k, v, o, lse, scale=s, f32=f32) == fa.FA_ERR_ALIGN
    # outputs aliasing inputs or each other
    assert fwd_call(L, q, k, v, q, lse, f32=f32) == fa.FA_ERR_ALIAS
    assert fwd_call(L, q, k, v, o, ctypes.c_void_p(o.value + 64), f32=f32) == fa.FA_ERR_ALIAS


@pytest.mark.parametrize("f32", [False, True])
def test_fwd_size_limits(L, f32):
    """Shapes beyond the documented limits are refused before any HIP call: B*H above 2^30, one
    head's float32 slice beyond a 31-bit byte range, more than 2^31 - 1 query tiles, and (fp32
    kernels, which put B*H on grid.y) B*H above 65535.  Every case here fails validation, so the
    fake pointers are never used."""
    import exact_io_aware_flash_amd as fa
    q, k, v, o, lse = ptrs(5)
    assert fwd_call(L, q, k, v, o, lse, B=1 << 16, H=1 << 15, N=1, f32=f32) == fa.FA_ERR_SHAPE
    assert fwd_call(L, q, k, v, o, lse, N=1 << 22, d=128, f32=f32) == fa.FA_ERR_SHAPE
    assert fwd_call(L, q, k, v, o, lse, B=1 << 15, H=1 << 15, N=256, f32=f32) == fa.FA_ERR_SHAPE
    # B*H = 2^30 with N = 2^30: the per-head size check runs before any product that could
    # leave 64 bits
    assert fwd_call(L, q, k, v, o, lse, B=1 << 15, H=1 << 15, N=1 << 30, d=128, f32=f32) == fa.FA_ERR_SHAPE
    assert fwd_call(L, q, k, v, o, lse, B=1 << 15, H=1 << 15, N=(1 << 31) - 1, d=128, f32=f32) == fa.FA_ERR_SHAPE
    if f32:
        assert fwd_call(L, q, k, v, o, lse, B=65536, H=1, N=1, f32=True) == fa.FA_ERR_SHAPE


def test_fwd_mask_limit(L):
    import exact_io_aware_flash_amd as fa
    q, k, v, o, lse, m = ptrs(6)
    N = (2048 + 1) * 128
    assert fwd_call(L, q, k, v, o, lse, N=N, mask=m) == fa.FA_ERR_SHAPE


def bwd_call(L, p, ws, ws_bytes, B=1, H=1, N=128, d=64, scale=0.125, causal=0, mask=None, f32=False):
    fn = L.flash_attn_bwd_f32 if f32 else L.flash_attn_bwd
    return fn(*p, ws, ws_bytes, B, H, N, d, scale, causal, mask, None)


@pytest.mark.parametrize("f32", [False, True])
def test_bwd_argument_errors(L, f32):
    import exact_io_aware_flash_amd as fa
    p = ptrs(9)
    ws = ptrs(1, start=1 << 45)[0]
    need = fa.workspace_bytes(1, 1, 128, 64)
    assert bwd_call(L, p, ctypes.c_void_p(ws.value + 8), need, f32=f32) == fa.FA_ERR_ALIGN
    assert bwd_call(L, p, None, need, f32=f32) == fa.FA_ERR_WORKSPACE
    assert bwd_call(L, p, ws, need - 1, f32=f32) == fa.FA_ERR_WORKSPACE
    for i in range(9):
        pp = list(p)
        pp[i] = None
        assert bwd_call(L, pp, ws, need, f32=f32) == fa.FA_ERR_NULL, i
    assert bwd_call(L, p, ws, need, d=80, f32=f32) == fa.FA_ERR_HEADDIM
    assert bwd_call(L, p, ws, need, scale=0.0, f32=f32) == fa.FA_ERR_SCALE
    assert bwd_call(L, p, ws, need, scale=float("-inf"), f32=f32) == fa.FA_ERR_SCALE
    assert bwd_call(L, p, ws, need, causal=-1, f32=f32) == fa.FA_ERR_FLAG
    pp = list(p)
    pp[6] = pp[0]  # dq == q
    assert bwd_call(L, pp, ws, need, f32=f32) == fa.FA_ERR_ALIAS
    # a negative scale and a workspace aligned to 16 bytes (not 256) pass validation: the call
    # gets as far as the alias check
    assert bwd_call(L, pp, ws, need, scale=-1.0, f32=f32) == fa.FA_ERR_ALIAS
    assert bwd_call(L, pp, ctypes.c_void_p(ws.value + 16), need, f32=f32) == fa.FA_ERR_ALIAS
    pp = list(p)
    pp[7] = pp[8]  # dk == dv
    assert bwd_call(L, pp, ws, need, f32=f32) == fa.FA_ERR_ALIAS
    assert bwd_call(L, p, p[1], need, f32=f32) == fa.FA_ERR_ALIAS  # workspace over k
    mis = ctypes.c_void_p(ws.value + 4)
    assert bwd_call(L, p, mis, need, f32=f32) == fa.FA_ERR_ALIGN


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    import exact_io_aware_flash_amd as fa
    monkeypatch.delenv("FLASH_ATTN_LIB", raising=False)
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        fa.lib()


def test_stage_argument_errors(L):
    import exact_io_aware_flash_amd as fa
    q, k, v, do, lse, ws, dk, dv, o = ptrs(9)
    dims = (1, 1, 128, 64)
    need = fa.workspace_bytes(*dims)
    assert L.flash_attn_bwd_preprocess(None, o, do, ws, need, *dims, None) == fa.FA_ERR_NULL
    assert L.flash_attn_bwd_preprocess(q, o, do, ws, need, 1, 1, 128, 32, None) == fa.FA_ERR_HEADDIM
    assert L.flash_attn_bwd_preprocess(q, o, do, ws, need - 1, *dims, None) == fa.FA_ERR_WORKSPACE
    assert L.flash_attn_bwd_preprocess(q, o, do, ctypes.c_void_p(ws.value + 8), need, *dims,
                                       None) == fa.FA_ERR_ALIGN
    assert L.flash_attn_bwd_preprocess(q, o, do, ctypes.c_void_p(o.value + 256), need, *dims,
                                       None) == fa.FA_ERR_ALIAS
    args = [q, k, v, do, lse, ws, need, dk, dv]
    for i in (0, 1, 2, 3, 4, 5, 7, 8):
        a = list(args)
        a[i] = None
        assert L.flash_attn_bwd_dkdv(*a, *dims, 0.125, 0, None, None) == fa.FA_ERR_NULL, i
    assert L.flash_attn_bwd_dkdv(*args[:6], need - 1, *args[7:], *dims, 0.125, 0, None, None) == fa.FA_ERR_WORKSPACE
    assert L.flash_attn_bwd_dkdv(*args, 1, 1, 0, 64, 0.125, 0, None, None) == fa.FA_ERR_SHAPE
    assert L.flash_attn_bwd_dkdv(*args, *dims, 0.0, 0, None, None) == fa.FA_ERR_SCALE
    a = list(args)
    a[8] = a[7]
    assert L.flash_attn_bwd_dkdv(*a, *dims, 0.125, 0, None, None) == fa.FA_ERR_ALIAS
    assert L.flash_attn_bwd_dkdv(*a, *dims, -0.125, 0, None, None) == fa.FA_ERR_ALIAS
    a = list(args)
    a[7] = a[4]  # dk over lse
    assert L.flash_attn_bwd_dkdv(*a, *dims, 0.125, 0, None, None) == fa.FA_ERR_ALIAS
    a = list(args)
    a[7] = a[5]  # dk over the workspace
    assert L.flash_attn_bwd_dkdv(*a, *dims, 0.125, 0, None, None) == fa.FA_ERR_ALIAS
    qargs = [q, k, v, do, lse, ws, need, dk]
    assert L.flash_attn_bwd_dq(*qargs, *dims, 0.125, 3, None, None) == fa.FA_ERR_FLAG
    a = list(qargs)
    a[7] = ctypes.c_void_p(dk.value + 2)
    assert L.flash_attn_bwd_dq(*a, *dims, 0.125, 0, None, None) == fa.FA_ERR_ALIGN
    a = list(qargs)
    a[7] = a[0]
    assert L.flash_attn_bwd_dq(*a, *dims, 0.125, 0, None, None) == fa.FA_ERR_ALIAS


def test_splitkv_workspace_bytes(L):
    import exact_io_aware_flash_amd as fa
    a256 = lambda x: (x + 255) // 256 * 256
    for B, H, N, d, S in ((1, 1, 1, 64, 1), (2, 3, 100, 128, 3), (1, 32, 16384, 128, 4), (1, 1, 300, 64, 64)):
        want = a256(S * B * H * N * d * 4) + a256(S * B * H * N * 4)
        assert fa.splitkv_workspace_bytes(B, H, N, d, S) == want, (B, H, N, d, S)
    assert fa.splitkv_workspace_bytes(1, 1, 128, 64, 0) == 0
    assert fa.splitkv_workspace_bytes(1, 1, 128, 64, fa.MAX_SPLITS + 1) == 0
    assert fa.splitkv_workspace_bytes(1, 1, 128, 96, 2) == 0


def test_splitkv_argument_errors(L):
    import exact_io_aware_flash_amd as fa
    q, k, v, o, lse, m = ptrs(6)
    ws = ptrs(1, start=1 << 45)[0]
    need = fa.splitkv_workspace_bytes(1, 1, 128, 64, 2)

    def call(q=q, o=o, lse=lse, ws=ws, wsb=need, N=128, d=64, scale=0.125, causal=0, mask=None, splits=2):
        return L.flash_attn_fwd_splitkv(q, k, v, o, lse, 1, 1, N, d, scale, causal, mask, splits, ws, wsb, None)

    assert call(q=None) == fa.FA_ERR_NULL
    assert call(d=96) == fa.FA_ERR_HEADDIM
    assert call(scale=float("nan")) == fa.FA_ERR_SCALE
    assert call(causal=5) == fa.FA_ERR_FLAG
    assert call(splits=0) == fa.FA_ERR_SPLITS
    assert call(splits=fa.MAX_SPLITS + 1) == fa.FA_ERR_SPLITS
    assert call(ws=None) == fa.FA_ERR_WORKSPACE
    assert call(wsb=need - 1) == fa.FA_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(ws.value + 8)) == fa.FA_ERR_ALIGN
    # a 16-byte aligned workspace and a negative scale pass validation (stopped by the alias check)
    assert call(ws=ctypes.c_void_p(k.value + 16)) == fa.FA_ERR_ALIAS
    assert call(scale=-0.125, o=q) == fa.FA_ERR_ALIAS
    assert call(ws=k) == fa.FA_ERR_ALIAS  # workspace over an input
    assert call(ws=ctypes.c_void_p(o.value + 256)) == fa.FA_ERR_ALIAS  # workspace over the output
    assert call(o=q) == fa.FA_ERR_ALIAS


def test_merge_argument_errors(L):
    import exact_io_aware_flash_amd as fa
    op, lp, o, lse = ptrs(4)

    def call(op=op, lp=lp, parts=2, rows=100, d=64, o=o, lse=lse):
        return L.flash_attn_merge(op, lp, parts, rows, d, o, lse, None)

    assert call(op=None) == fa.FA_ERR_NULL
    assert call(lse=None) == fa.FA_ERR_NULL
    assert call(parts=0) == fa.FA_ERR_SPLITS
    assert call(parts=fa.MAX_SPLITS + 1) == fa.FA_ERR_SPLITS
    assert call(rows=0) == fa.FA_ERR_SHAPE
    assert call(d=32) == fa.FA_ERR_HEADDIM
    assert call(o=ctypes.c_void_p(o.value + 8)) == fa.FA_ERR_ALIGN
    assert call(o=ctypes.c_void_p(op.value + 1024)) == fa.FA_ERR_ALIAS
    assert call(lse=ctypes.c_void_p(o.value + 64)) == fa.FA_ERR_ALIAS


def test_mxfp8_vt_cols(L):
    import exact_io_aware_flash_amd as fa
    assert [fa.mxfp8_vt_cols(n) for n in (0, 1, 63, 64, 65, 128, 16384, 16385)] == [0, 64, 64, 64, 128, 128, 16384,
                                                                                   16448]


def test_mxfp8_argument_errors(L):
    import exact_io_aware_flash_amd as fa
    q8, qs, k8, ks, vt, vs, o, lse = ptrs(8)

    def fwd8(*args, B=1, H=1, N=128, d=64, scale=0.125, causal=0, mask=None):
        a = list(args) if args else [q8, qs, k8, ks, vt, vs, o, lse]
        return L.flash_attn_fwd_mxfp8(*a, B, H, N, d, scale, causal, mask, None)

    base = [q8, qs, k8, ks, vt, vs, o, lse]
    for i in range(8):
        a = list(base)
        a[i] = None
        assert fwd8(*a) == fa.FA_ERR_NULL, i
    assert fwd8(N=0) == fa.FA_ERR_SHAPE
    assert fwd8(d=96) == fa.FA_ERR_HEADDIM
    assert fwd8(scale=0.0) == fa.FA_ERR_SCALE
    assert fwd8(scale=float("nan")) == fa.FA_ERR_SCALE
    assert fwd8(causal=2) == fa.FA_ERR_FLAG
    a = list(base)
    a[2] = ctypes.c_void_p((1 << 40) + 2 * BIG + 8)
    assert fwd8(*a) == fa.FA_ERR_ALIGN
    assert fwd8(*a, scale=-0.125) == fa.FA_ERR_ALIGN  # a negative scale passes validation
    a = list(base)
    a[6] = a[4]  # output over V's codes
    assert fwd8(*a) == fa.FA_ERR_ALIAS
    x, c, sc = ptrs(3)
    for fn in (L.flash_attn_mxfp8_quantize_rows, L.flash_attn_mxfp8_quantize_vt):
        assert fn(None, c, sc, 1, 1, 128, 64, None) == fa.FA_ERR_NULL
        assert fn(x, c, sc, 1, 1, 128, 48, None) == fa.FA_ERR_HEADDIM
        assert fn(x, c, sc, 1, 0, 128, 64, None) == fa.FA_ERR_SHAPE
        assert fn(x, x, sc, 1, 1, 128, 64, None) == fa.FA_ERR_ALIAS
        assert fn(x, ctypes.c_void_p((1 << 40) + BIG + 4), sc, 1, 1, 128, 64, None) == fa.FA_ERR_ALIGN


def test_noalloc_argument_errors(L):
    """flash_attn_bwd_noalloc refuses shapes beyond its fixed scratch (B * H * N rows) and every
    other invalid argument before any HIP call, like flash_attn_bwd."""
    import exact_io_aware_flash_amd as fa
    p = ptrs(9)

    def call(pp=p, B=1, H=1, N=128, d=64, scale=0.125, causal=0):
        return L.flash_attn_bwd_noalloc(*pp, B, H, N, d, scale, causal, None, None)

    assert fa.NOALLOC_MAX_ROWS == 1 << 22
    assert call(B=1, H=1025, N=4096) == fa.FA_ERR_SCRATCH
    assert call(B=2, H=1, N=(1 << 21) + 1) == fa.FA_ERR_SCRATCH
    assert call(B=1 << 15, H=1 << 15, N=1 << 30, d=128) == fa.FA_ERR_SHAPE
    for i in range(9):
        pp = list(p)
        pp[i] = None
        assert call(pp) == fa.FA_ERR_NULL, i
    assert call(d=96) == fa.FA_ERR_HEADDIM
    assert call(scale=0.0) == fa.FA_ERR_SCALE
    assert call(causal=3) == fa.FA_ERR_FLAG
    pp = list(p)
    pp[0] = ctypes.c_void_p(pp[0].value + 8)
    assert call(pp) == fa.FA_ERR_ALIGN
    pp = list(p)
    pp[6] = pp[1]  # dq == k
    assert call(pp) == fa.FA_ERR_ALIAS
    # the largest accepted size and a negative scale pass the size and scale checks
    assert call(pp, B=1, H=1024, N=4096, scale=-0.125) == fa.FA_ERR_ALIAS
    assert "FA_NOALLOC_MAX_ROWS" in fa.status_string(fa.FA_ERR_SCRATCH)


def test_pingpong_argument_errors(L):
    """flash_attn_fwd_pingpong: flash_attn_fwd's checks, then d = 128 without a block mask only."""
    import exact_io_aware_flash_amd as fa
    q, k, v, o, lse, m = ptrs(6)

    def call(d=128, mask=None, scale=0.125, o=o):
        return L.flash_attn_fwd_pingpong(q, k, v, o, lse, 1, 1, 256, d, scale, 0, mask, None)

    assert call(d=64) == fa.FA_ERR_UNSUPPORTED
    assert call(mask=m) == fa.FA_ERR_UNSUPPORTED
    assert call(d=96) == fa.FA_ERR_HEADDIM
    assert call(scale=0.0) == fa.FA_ERR_SCALE
    assert call(o=q) == fa.FA_ERR_ALIAS


def test_validation_under_host_sanitizers():
    """The argument checks of the C ABI, every case of this file, run against the build whose host
    code carries AddressSanitizer and UndefinedBehaviorSanitizer (overflowing products, bad shifts,
    out-of-bounds reads in the validators abort the run with a report)."""
    import subprocess

    from exact_io_aware_flash_amd import build as B
    lib = B.variant_path("asan")
    rt = B.sanitizer_runtime()
    if not os.path.exists(lib) or rt is None:
        pytest.skip("sanitized build or sanitizer runtime missing (built by exact_io_aware_flash_amd.build)")
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the asan build is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", FLASH_ATTN_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.abspath(__file__), "-q", "-p", "no:cacheprovider",
                        "-k", "not sanitizers"], capture_output=True, text=True, env=env, timeout=600,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
