"""Host-side checks of the C ABI: symbols, no device allocation, argument
validation before any device work. CPU only (no GPU is touched: every call
below fails validation and returns before any HIP call)."""

import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flash_attn.h")

import online_softmax_flash_amd as fa  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(fa.lib_path()), reason="libflashattn.so not built")

FAKE = 0x10000  # non-null, 16-byte aligned; never dereferenced (validation fails first)
OK_SHAPE = (2, 8, 2, 100, 128)
STATUS = {"FA_OK": 0, "FA_ERR_NULL": 1, "FA_ERR_SHAPE": 2, "FA_ERR_UNSUPPORTED": 3, "FA_ERR_ALIGN": 4,
          "FA_ERR_SCALE": 5, "FA_ERR_HIP": 6, "FA_ERR_WORKSPACE": 7, "FA_ERR_SCRATCH": 8}


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(flash_attn_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 6, names
    lib = fa.load_library()
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
    out = subprocess.run(["nm", "-D", "--defined-only", fa.lib_path()], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), f"{n} not a defined text symbol"


def test_no_device_allocation_imports():
    out = subprocess.run(["nm", "-D", "--undefined-only", fa.lib_path()], capture_output=True, text=True).stdout
    bad = [l for l in out.splitlines() if re.search(r"hip(Ext)?(Malloc|Free|MallocAsync|HostMalloc|MallocManaged)", l)]
    assert not bad, bad


def test_status_strings():
    for name, code in STATUS.items():
        assert fa.flash_attn_status_str(code) == name
    assert fa.flash_attn_status_str(99) == "FA_UNKNOWN"


def _fwd(fn="flash_attn_fwd", ptrs=(FAKE,) * 5, shape=OK_SHAPE, scale=0.1, causal=0):
    lib = fa.load_library()
    p = [ctypes.c_void_p(x) if x else None for x in ptrs]
    return getattr(lib, fn)(*p, *shape, ctypes.c_float(scale), causal, None)


def _bwd(fn="flash_attn_bwd", ptrs=(FAKE,) * 10, shape=OK_SHAPE, scale=0.1, causal=0, ws_bytes=1 << 40):
    lib = fa.load_library()
    p = [ctypes.c_void_p(x) if x else None for x in ptrs]
    return getattr(lib, fn)(*p, ctypes.c_size_t(ws_bytes), *shape, ctypes.c_float(scale), causal, None)


@pytest.mark.parametrize("fn", ["flash_attn_fwd", "flash_attn_fwd_f32"])
def test_forward_validation(fn):
    for i in range(5):
        ptrs = [FAKE] * 5
        ptrs[i] = 0
        assert _fwd(fn, ptrs) == STATUS["FA_ERR_NULL"]
        ptrs[i] = FAKE + 8
        assert _fwd(fn, ptrs) == STATUS["FA_ERR_ALIGN"]
    for shape in [(0, 8, 2, 100, 128), (2, 0, 2, 100, 128), (2, 8, 0, 100, 128), (2, 8, 2, 0, 128),
                  (2, 8, 3, 100, 128), (-1, 8, 2, 100, 128), (1, 1, 1, 2 ** 30, 256)]:
        assert _fwd(fn, shape=shape) == STATUS["FA_ERR_SHAPE"], shape
    for d in (0, 32, 96, 100, 512):
        assert _fwd(fn, shape=(2, 8, 2, 100, d)) == STATUS["FA_ERR_UNSUPPORTED"], d
    assert _fwd(fn, causal=2) == STATUS["FA_ERR_UNSUPPORTED"]
    for s in (math.nan, math.inf, -math.inf, -0.5):
        assert _fwd(fn, scale=s) == STATUS["FA_ERR_SCALE"], s


@pytest.mark.parametrize("fn", ["flash_attn_bwd", "flash_attn_bwd_f32"])
def test_backward_validation(fn):
    for i in range(9):
        ptrs = [FAKE] * 10
        ptrs[i] = 0
        assert _bwd(fn, ptrs) == STATUS["FA_ERR_NULL"]
        ptrs[i] = FAKE + 4
        assert _bwd(fn, ptrs) == STATUS["FA_ERR_ALIGN"]
    ptrs = [FAKE] * 10
    ptrs[9] = 0
    assert _bwd(fn, ptrs) == STATUS["FA_ERR_WORKSPACE"]
    ptrs[9] = FAKE + 2
    assert _bwd(fn, ptrs) == STATUS["FA_ERR_ALIGN"]
    # A workspace shorter than flash_attn_bwd_workspace_bytes is refused before any device work.
    need = fa.flash_attn_bwd_workspace_bytes(*OK_SHAPE)
    assert need > 0
    assert _bwd(fn, ws_bytes=need - 1) == STATUS["FA_ERR_WORKSPACE"]
    assert _bwd(fn, ws_bytes=0) == STATUS["FA_ERR_WORKSPACE"]
    assert _bwd(fn, shape=(2, 8, 3, 100, 128)) == STATUS["FA_ERR_SHAPE"]
    assert _bwd(fn, shape=(2, 8, 2, 100, 48)) == STATUS["FA_ERR_UNSUPPORTED"]
    assert _bwd(fn, scale=math.nan) == STATUS["FA_ERR_SCALE"]


def test_workspace_bytes_linear_in_n():
    ws = fa.flash_attn_bwd_workspace_bytes
    # Per query row: D and lse * log2(e) (fp32 each), the second from a
    # 256-byte boundary.
    def up(n):
        return (n + 255) // 256 * 256
    R = 2 * 16 * 4096
    assert ws(2, 16, 16, 4096, 128) == 2 * 4 * R
    assert ws(1, 1, 1, 1, 64) == 2 * 256
    assert ws(1, 2, 1, 1000, 64) == 2 * up(4 * 2000)
    kws = fa.flash_attn_bwd_kv_workspace_bytes
    assert kws(2 * 16 * 4096, 128) == ws(2, 16, 16, 4096, 128)
    assert kws(0, 128) == 0 and kws(10, 96) == 0
    assert ws(2, 16, 16, 8192, 128) == 2 * ws(2, 16, 16, 4096, 128)
    assert ws(0, 1, 1, 1, 64) == 0
    assert ws(1, 3, 2, 1, 64) == 0
    assert ws(1, 1, 1, 1, 100) == 0


def _kv(ptrs=(FAKE,) * 5, shape=(2, 8, 2, 3, 100, 128), scale=0.1, causal=1, splits=1, ws=None, ws_bytes=0):
    lib = fa.load_library()
    p = [ctypes.c_void_p(x) if x else None for x in ptrs]
    w = ctypes.c_void_p(ws) if ws else None
    return lib.flash_attn_fwd_kv(*p, *shape, ctypes.c_float(scale), causal, splits, w, ctypes.c_size_t(ws_bytes),
                                 None)


def _varlen(cu=(FAKE, FAKE), shape=(2, 8, 2, 50, 60, 30, 40, 128), splits=1):
    lib = fa.load_library()
    p = [ctypes.c_void_p(FAKE)] * 5
    c = [ctypes.c_void_p(x) if x else None for x in cu]
    return lib.flash_attn_fwd_varlen(*p, *c, *shape, ctypes.c_float(0.1), 1, splits, None, ctypes.c_size_t(0), None)


def test_kv_rejects_bad_arguments():
    assert _kv(ptrs=(FAKE, 0, FAKE, FAKE, FAKE)) == STATUS["FA_ERR_NULL"]
    assert _kv(ptrs=(FAKE, FAKE, FAKE + 4, FAKE, FAKE)) == STATUS["FA_ERR_ALIGN"]
    assert _kv(shape=(2, 8, 3, 3, 100, 128)) == STATUS["FA_ERR_SHAPE"]
    assert _kv(shape=(2, 8, 2, 0, 100, 128)) == STATUS["FA_ERR_SHAPE"]
    assert _kv(shape=(2, 8, 2, 3, 0, 128)) == STATUS["FA_ERR_SHAPE"]
    assert _kv(shape=(2, 8, 2, 3, 100, 96)) == STATUS["FA_ERR_UNSUPPORTED"]
    assert _kv(causal=2) == STATUS["FA_ERR_UNSUPPORTED"]
    assert _kv(scale=math.inf) == STATUS["FA_ERR_SCALE"]
    assert _kv(splits=-1) == STATUS["FA_ERR_SHAPE"]
    assert _kv(splits=257) == STATUS["FA_ERR_SHAPE"]
    # More workgroups than a 65536 x 65535 grid holds (65536 sequences x 1024
    # K/V heads x 256 splits).
    assert _kv(shape=(1 << 16, 1024, 1024, 1, 64, 128), splits=256) == STATUS["FA_ERR_SHAPE"]
    # Split keys need the partials' workspace, of at least the stated size, aligned.
    rows = 2 * 8 * 3
    need = fa.flash_attn_fwd_kv_workspace_bytes(rows, 128, 4)
    assert _kv(splits=4) == STATUS["FA_ERR_WORKSPACE"]
    assert _kv(splits=4, ws=FAKE, ws_bytes=need - 1) == STATUS["FA_ERR_WORKSPACE"]
    assert _kv(splits=4, ws=FAKE + 8, ws_bytes=need) == STATUS["FA_ERR_ALIGN"]


def test_varlen_rejects_bad_arguments():
    assert _varlen(cu=(0, FAKE)) == STATUS["FA_ERR_NULL"]
    assert _varlen(cu=(FAKE, 0)) == STATUS["FA_ERR_NULL"]
    assert _varlen(shape=(0, 8, 2, 50, 60, 30, 40, 128)) == STATUS["FA_ERR_SHAPE"]
    assert _varlen(shape=(2, 8, 2, 50, 60, 0, 40, 128)) == STATUS["FA_ERR_SHAPE"]
    assert _varlen(shape=(2, 8, 2, 50, 60, 30, 40, 80)) == STATUS["FA_ERR_UNSUPPORTED"]


def test_kv_workspace_and_split_choice():
    ws = fa.flash_attn_fwd_kv_workspace_bytes
    assert ws(10, 128, 1) == 0
    assert ws(10, 128, 3) == ((3 * 10 * 128 * 4 + 255) // 256) * 256 + ((3 * 10 * 4 + 255) // 256) * 256
    assert ws(0, 128, 3) == 0 and ws(10, 100, 3) == 0 and ws(10, 128, 0) == 0 and ws(10, 128, 257) == 0
    ns = fa.flash_attn_fwd_kv_num_splits
    # A decode step of 8 sequences x 8 K/V heads is 64 workgroups: split the keys.
    s = ns(8, 32, 8, 1, 32768, 128)
    assert 2 <= s <= 256 and s <= 32768 // 256
    # A long prefill fills the chip without splitting; short key ranges are never split.
    assert ns(1, 32, 32, 8192, 8192, 128) == 1
    assert ns(1, 8, 8, 1, 300, 128) == 1
    # 256 four-wave workgroups: half the chip's slots at d = 128 (split), all
    # of them at d = 256, where one fills a compute unit's LDS (no split).
    assert ns(1, 16, 16, 2048, 8192, 128) >= 2
    assert ns(1, 16, 16, 2048, 8192, 256) == 1
    assert ns(1, 8, 3, 1, 300, 128) == 0


def test_naive_rejects_bad_arguments_and_sizes_workspace():
    lib = fa.load_library()
    p = [ctypes.c_void_p(FAKE)] * 5

    def call(shape=(1, 4, 2, 100, 128), causal=1, ws=FAKE, nbytes=None):
        n = fa.flash_attn_naive_workspace_bytes(shape[0], shape[1], shape[3]) if nbytes is None else nbytes
        w = ctypes.c_void_p(ws) if ws else None
        return lib.flash_attn_naive_fwd(*p, *shape, ctypes.c_float(0.1), causal, w, ctypes.c_size_t(n), None)

    assert call(shape=(1, 4, 3, 100, 128)) == STATUS["FA_ERR_SHAPE"]
    assert call(shape=(1, 4, 2, 100, 32)) == STATUS["FA_ERR_UNSUPPORTED"]
    assert call(ws=0) == STATUS["FA_ERR_WORKSPACE"]
    assert call(nbytes=1000) == STATUS["FA_ERR_WORKSPACE"]
    assert call(ws=FAKE + 4) == STATUS["FA_ERR_ALIGN"]
    # quadratic in N: N*N fp32 scores plus N*N bf16 weights per head
    assert fa.flash_attn_naive_workspace_bytes(2, 16, 4096) == 2 * 16 * 4096 * 4096 * 6
    assert fa.flash_attn_naive_workspace_bytes(0, 16, 4096) == 0


def test_noalloc_refuses_partials_beyond_its_scratch():
    """flash_attn_fwd_kv_noalloc checks its arguments like flash_attn_fwd_kv and
    refuses, before any device work, an explicit split count whose partials
    exceed the static scratch (FLASH_ATTN_SCRATCH_BYTES = 32 MiB)."""
    lib = fa.load_library()
    p = [ctypes.c_void_p(FAKE)] * 5

    def call(shape, splits, ptrs=p, causal=1):
        return lib.flash_attn_fwd_kv_noalloc(*ptrs, *shape, ctypes.c_float(0.1), causal, splits, None)

    big = (64, 64, 8, 64, 4096, 256)  # 262144 rows x 256 fp32 per split
    assert fa.flash_attn_fwd_kv_workspace_bytes(64 * 64 * 64, 256, 8) > 32 << 20
    assert call(big, 8) == STATUS["FA_ERR_SCRATCH"]
    assert call((2, 8, 2, 3, 100, 128), 1, ptrs=[ctypes.c_void_p(FAKE)] * 4 + [None]) == STATUS["FA_ERR_NULL"]
    assert call((2, 8, 3, 3, 100, 128), 2) == STATUS["FA_ERR_SHAPE"]
    assert call((2, 8, 2, 3, 100, 96), 2) == STATUS["FA_ERR_UNSUPPORTED"]
    assert call((2, 8, 2, 3, 100, 128), 300) == STATUS["FA_ERR_SHAPE"]
    src = open(HEADER).read()
    assert re.search(r"#define FLASH_ATTN_SCRATCH_BYTES \(32u << 20\)", src)


def _bwdkv(ptrs=(FAKE,) * 10, shape=(2, 8, 2, 3, 100, 128), scale=0.1, causal=1, ws_bytes=1 << 40):
    lib = fa.load_library()
    p = [ctypes.c_void_p(x) if x else None for x in ptrs]
    return lib.flash_attn_bwd_kv(*p, ctypes.c_size_t(ws_bytes), *shape, ctypes.c_float(scale), causal, None)


def test_bwd_kv_and_varlen_reject_bad_arguments():
    for i in range(10):
        ptrs = [FAKE] * 10
        ptrs[i] = 0
        assert _bwdkv(ptrs) == (STATUS["FA_ERR_WORKSPACE"] if i == 9 else STATUS["FA_ERR_NULL"])
        ptrs[i] = FAKE + 8
        assert _bwdkv(ptrs) == STATUS["FA_ERR_ALIGN"]
    assert _bwdkv(shape=(2, 8, 3, 3, 100, 128)) == STATUS["FA_ERR_SHAPE"]
    assert _bwdkv(shape=(2, 8, 2, 0, 100, 128)) == STATUS["FA_ERR_SHAPE"]
    assert _bwdkv(shape=(2, 8, 2, 3, 0, 128)) == STATUS["FA_ERR_SHAPE"]
    assert _bwdkv(shape=(2, 8, 2, 3, 100, 32)) == STATUS["FA_ERR_UNSUPPORTED"]
    assert _bwdkv(causal=2) == STATUS["FA_ERR_UNSUPPORTED"]
    assert _bwdkv(scale=math.nan) == STATUS["FA_ERR_SCALE"]
    need = fa.flash_attn_bwd_kv_workspace_bytes(2 * 8 * 3, 128)
    assert need > 0
    assert _bwdkv(ws_bytes=need - 1) == STATUS["FA_ERR_WORKSPACE"]
    lib = fa.load_library()
    p = [ctypes.c_void_p(FAKE)] * 9

    def varlen(cu=(FAKE, FAKE), shape=(2, 8, 2, 50, 60, 30, 40, 128), ws_bytes=1 << 40):
        c = [ctypes.c_void_p(x) if x else None for x in cu]
        return lib.flash_attn_bwd_varlen(*p, *c, ctypes.c_void_p(FAKE), ctypes.c_size_t(ws_bytes), *shape,
                                         ctypes.c_float(0.1), 1, None)

    assert varlen(cu=(0, FAKE)) == STATUS["FA_ERR_NULL"]
    assert varlen(cu=(FAKE, 0)) == STATUS["FA_ERR_NULL"]
    assert varlen(shape=(0, 8, 2, 50, 60, 30, 40, 128)) == STATUS["FA_ERR_SHAPE"]
    assert varlen(shape=(2, 8, 2, 50, 60, 0, 40, 128)) == STATUS["FA_ERR_SHAPE"]
    assert varlen(shape=(2, 8, 2, 50, 60, 30, 40, 80)) == STATUS["FA_ERR_UNSUPPORTED"]
    assert varlen(ws_bytes=fa.flash_attn_bwd_kv_workspace_bytes(8 * 50, 128) - 1) == STATUS["FA_ERR_WORKSPACE"]
