"""Host-side parts of the weight pager, no GPU needed.

- The extent allocator (csrc/pw_arena.h) is compiled with g++ into a
  randomized unit test against a byte occupancy map.
- The pager's C-ABI bookkeeping (create, set_block, request, info, destroy)
  checks its arguments and keeps its state on the host: with placeholder
  device addresses that are never dereferenced, none of these calls reaches
  the GPU.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

from any_precision_bitplane_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_extent_allocator(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "arena_test")
    subprocess.run([gxx, "-O1", "-std=c++17", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "any_precision_bitplane_amd", "csrc"),
                    os.path.join(ROOT, "tests", "cpp", "arena_test.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libpagedweight.so is not built (python -m any_precision_bitplane_amd.build)")
    return B.load()


# placeholder device addresses: aligned, never dereferenced by host-only calls
FAKE_ARENA = 0x7F0000000000
FAKE_TABLE = 0x7F0000100000
FAKE_Q = 0x7F0000200000
FAKE_LUT = 0x7F0000300000


def _create(lib, rows, cols, arena=FAKE_ARENA, nbytes=1 << 20, table=FAKE_TABLE, q=FAKE_Q):
    n = len(rows)
    out = ctypes.c_void_p(0)
    st = lib.pw_pager_create(n, (ctypes.c_int32 * n)(*rows), (ctypes.c_int32 * n)(*cols), arena, nbytes, table,
                             q, ctypes.byref(out))
    return st, out.value


def test_create_rejects_bad_arguments(lib):
    assert _create(lib, [64], [32], arena=None)[0] == B.PW_ERR_INVALID_ARG
    assert _create(lib, [64], [32], table=None)[0] == B.PW_ERR_INVALID_ARG
    assert _create(lib, [64], [32], q=None)[0] == B.PW_ERR_INVALID_ARG
    assert _create(lib, [64], [48])[0] == B.PW_ERR_UNSUPPORTED_SHAPE     # K % 32
    assert _create(lib, [0], [32])[0] == B.PW_ERR_INVALID_ARG
    assert _create(lib, [1 << 16], [1 << 16])[0] == B.PW_ERR_UNSUPPORTED_SHAPE   # > 2^31 weights
    assert _create(lib, [64], [32], arena=FAKE_ARENA + 16)[0] == B.PW_ERR_ALIGNMENT
    assert lib.pw_pager_create(1, None, None, FAKE_ARENA, 1 << 20, FAKE_TABLE, FAKE_Q, None) == B.PW_ERR_INVALID_ARG


def test_bookkeeping_before_any_commit(lib):
    st, p = _create(lib, [1024, 256], [256, 512])
    assert st == B.PW_OK and p
    host = ctypes.create_string_buffer(8 * 1024 * 256 // 8 + 64)
    host_ptr = (ctypes.addressof(host) + 15) // 16 * 16
    # a request needs the block's storage registered first
    assert lib.pw_pager_request(p, 0, 5) == B.PW_ERR_INVALID_ARG
    assert lib.pw_pager_set_block(p, 0, host_ptr, FAKE_LUT) == B.PW_OK
    assert lib.pw_pager_set_block(p, 0, host_ptr, FAKE_LUT + 2) == B.PW_ERR_ALIGNMENT
    assert lib.pw_pager_set_block(p, 2, host_ptr, FAKE_LUT) == B.PW_ERR_INVALID_ARG
    assert lib.pw_pager_request(p, 0, 2) == B.PW_ERR_BITWIDTH
    assert lib.pw_pager_request(p, 0, 9) == B.PW_ERR_BITWIDTH
    assert lib.pw_pager_request(p, 0, 5) == B.PW_OK
    info = B.PwPageInfo()
    assert lib.pw_pager_info(p, 0, ctypes.byref(info)) == B.PW_OK
    assert (info.desired, info.committed, info.resident, info.pending, info.state) == (5, 0, 0, 0, B.PW_PAGE_CPU)
    assert info.arena_offset == 2 ** 64 - 1
    assert lib.pw_pager_info(p, 1, ctypes.byref(info)) == B.PW_OK
    assert info.desired == 0 and info.state == B.PW_PAGE_CPU
    assert lib.pw_pager_info(p, 2, ctypes.byref(info)) == B.PW_ERR_INVALID_ARG
    assert lib.pw_pager_arena_used(p) == 0
    assert lib.pw_pager_destroy(p) == B.PW_OK
    assert lib.pw_pager_destroy(None) == B.PW_OK


def test_status_string_of_the_pager_error(lib):
    assert B.pw_status_str(B.PW_ERR_OUT_OF_MEMORY) == "arena has no free range large enough"
