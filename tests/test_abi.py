"""The C ABI without a GPU: the library loads, exports every entry point the header
declares, and its host-side checks return the documented status codes.  No call here
touches a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moba.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moba_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def moba():
    import block_sparse_long_pool_amd as m
    return m


def test_header_declares_the_path(moba):
    names = declared_functions()
    for n in ["moba_check_args", "moba_workspace_bytes", "moba_forward", "moba_strerror",
              "moba_pool_centroids", "moba_gate_topk", "moba_build_index",
              "moba_history_partials", "moba_current_merge"]:
        assert n in names


def test_every_declared_symbol_is_exported(moba):
    lib = ctypes.CDLL(moba.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_check_args_codes(moba):
    ok = moba.check_args(1, 131072, 32, 8, 128, 4096, 12, 0.088)
    assert ok == 0
    E_ARG, E_UNS = -1, -2
    assert moba.check_args(0, 128, 1, 1, 64, 16, 1, 1.0) == E_ARG
    assert moba.check_args(1, 128, 3, 2, 64, 16, 1, 1.0) == E_ARG          # hq % hkv
    assert moba.check_args(1, 128, 1, 1, 64, 16, 0, 1.0) == E_ARG          # topk
    assert moba.check_args(1, 128, 1, 1, 64, 16, 1, float("nan")) == E_ARG
    assert moba.check_args(1, 128, 1, 1, 64, 16, 1, float("inf")) == E_ARG
    assert moba.check_args(1, 128, 1, 1, 96, 16, 1, 1.0) == E_UNS          # head_dim
    assert moba.check_args(1, 128, 1, 1, 64, 24, 1, 1.0) == E_UNS          # block % 16
    assert moba.check_args(1, 130, 1, 1, 64, 16, 1, 1.0) == ok             # partial last block
    assert moba.check_args(1, 16 * 8192, 1, 1, 64, 16, 2, 1.0) == ok       # 8192 blocks
    assert moba.check_args(1, 16 * 8193, 1, 1, 64, 16, 2, 1.0) == E_UNS    # > 8192 blocks
    # topk >= the number of blocks: dense causal attention, any topk and block count
    assert moba.check_args(1, 16 * 8193, 1, 1, 64, 16, 8193, 1.0) == ok
    assert moba.check_args(1, 4096, 4, 2, 128, 128, 40, 1.0) == ok         # topk 40 > 32 blocks
    # the backward takes a partial last block as well
    assert moba.backward_workspace_bytes(1, 130, 1, 1, 64, 16, 2)[0] > 0
    assert moba.backward_workspace_bytes(1, 128, 1, 1, 64, 16, 2)[0] > 0
    assert moba.backward_varlen_workspace_bytes(2, 300, 200, 4, 2, 64, 16, 3)[0] > 0
    assert moba.backward_varlen_workspace_bytes(2, 300, 400, 4, 2, 64, 16, 3) == (0, 0)
    assert moba.check_args(1, 2048, 1, 1, 64, 16, 65, 1.0) == 0            # 64 history slots
    assert moba.check_args(1, 2048, 1, 1, 64, 16, 66, 1.0) == E_UNS        # 65 history slots
    assert moba.check_args(1, 2048, 1, 1, 64, 16, 128, 1.0) == 0           # topk = nb: dense
    assert moba.check_args(1, 128, 1, 1, 64, 16, 34, 1.0) == 0             # topk > nb
    assert moba.check_args(1, 128, 1, 1, 64, 16, 2, -1.0) == E_UNS         # scale <= 0
    assert moba.check_args(1, 1 << 27, 1, 1, 64, 1 << 20, 2, 1.0) == E_UNS  # T*G too big
    # 33 .. 64 history slots take 6 slot bits: rows t*G + h%G must fit 26 bits
    assert moba.check_args(1, (1 << 26) // 4, 4, 1, 64, 4096, 40, 1.0) == E_UNS
    assert moba.check_args(1, (1 << 26) // 4 - 16, 4, 1, 64, 4096, 40, 1.0) == 0


def test_workspace_sizes(moba):
    full, mn = moba.workspace_bytes(1, 131072, 32, 8, 128, 4096, 12)
    assert 0 < mn < full
    # history partials dominate: [Hq, T, topk - 1, d] bf16 for all heads
    assert full > 32 * 131072 * 11 * 128 * 2
    assert mn < full / 4
    assert moba.workspace_bytes(1, 130, 1, 1, 64, 16, 2)[0] > 0    # partial last block
    assert moba.workspace_bytes(1, 130, 1, 1, 96, 16, 2) == (0, 0)    # head_dim 96
    # topk >= the number of blocks runs as dense causal attention and uses no workspace
    assert moba.workspace_bytes(1, 131072, 32, 8, 128, 4096, 32) == (256, 256)
    assert moba.workspace_bytes(1, 131072, 32, 8, 128, 4096, 31)[0] > 256
    # the backward of that case needs D = rowsum(dO * out), Hq * T floats, and a few
    # aligned words of an empty index
    full, mn = moba.backward_workspace_bytes(1, 1000, 4, 2, 64, 128, 8)
    assert full == mn and 4 * 1000 * 4 <= full <= 4 * 1000 * 4 + 8 * 256


def test_index_entry_count_closed_form(moba):
    # B * Hq * sum_c min(c, k-1): 4096 * 32 * (0+1+...+10 + 21*11) = 37,486,592
    assert moba.index_entries(1, 131072, 32, 8, 4096, 12, 8) == 37_486_592
    assert moba.index_entries(1, 131072, 32, 8, 4096, 12, 1) == 37_486_592 // 8
    assert moba.index_entries(1, 131072, 32, 8, 4096, 12, 9) == -1
    # the index packs at most 64 history slots
    assert moba.index_entries(1, 16 * 65, 1, 1, 16, 65, 1) > 0
    assert moba.index_entries(1, 16 * 66, 1, 1, 16, 66, 1) == -1


def test_strerror(moba):
    assert moba.strerror(0) == "success"
    assert "workspace" in moba.strerror(-3)
    assert moba.strerror(12345) == "unknown status"


def test_forward_rejects_bad_args_before_any_launch(moba):
    lib = moba.lib
    # null pointers with a valid shape: rejected on the host
    st = lib.moba_forward(None, None, None, 1, 128, 1, 1, 64, 16, 2, 0.125, None, None,
                          None, None, 0, None)
    assert st == -1
    # unsupported shape is reported before pointers are looked at
    st = lib.moba_forward(None, None, None, 1, 128, 1, 1, 96, 16, 2, 0.125, None, None,
                          None, None, 0, None)
    assert st == -2
    # packed sequences: the same shape rules, then the pointers (cu_seqlens first)
    vargs = (None, None, None, None, 2, 300, 200, 1, 1, 64, 16, 2, 0.125, None, None, None,
             None, 0, None)
    assert lib.moba_forward_varlen(*vargs) == -1
    assert lib.moba_forward_varlen(None, None, None, None, 2, 300, 200, 1, 1, 96, 16, 2,
                                   0.125, None, None, None, None, 0, None) == -1
    assert lib.moba_varlen_workspace_bytes(2, 300, 200, 1, 1, 96, 16, 2, None) == 0
    assert lib.moba_varlen_workspace_bytes(2, 300, 400, 1, 1, 64, 16, 2, None) == 0
    assert lib.moba_varlen_workspace_bytes(2, 300, 200, 1, 1, 64, 16, 2, None) > 0
    # dense causal attention: any seqlen (130 is not a multiple of 16), pointers checked
    # on the host
    assert lib.moba_dense_forward(None, None, None, 1, 130, 1, 1, 64, 0.125, None, None,
                                  None) == -1
    assert lib.moba_dense_forward(None, None, None, 1, 130, 1, 1, 96, 0.125, None, None,
                                  None) == -2
    assert lib.moba_dense_forward(None, None, None, 1, 128, 1, 1, 64, 0.125, None, None,
                                  None) == -1
    # the timed variant needs MOBA_NUM_STAGES + 1 non-null event handles
    args = (None, None, None, 1, 128, 1, 1, 64, 16, 2, 0.125, None, None, None, None, 0, None)
    assert lib.moba_forward_timed(*args, None) == -1
    ev = (ctypes.c_void_p * (len(moba.STAGES) + 1))(*([1] * len(moba.STAGES) + [None]))
    assert lib.moba_forward_timed(*args, ev) == -1


def test_history_and_merge_stages_reject_bad_args_before_any_launch(moba):
    lib = moba.lib
    shape = (1, 4096, 8, 2, 128, 256, 4, 0.088)
    one = ctypes.c_void_p(1)        # non-null, never dereferenced: every call below fails
    ws_needed = lib.moba_stage_workspace_bytes(1, 4096, 8, 2, 128, 256, 4)
    assert ws_needed > 0

    def hist(kv_begin=0, kv_count=2, topk=4, ptr=one, ws=ws_needed, d=128):
        b, T, hq, hkv, _, B, _, sc = shape
        return lib.moba_history_partials(ptr, ptr, ptr, b, T, hq, hkv, d, B, topk, sc,
                                         kv_begin, kv_count, ptr, ptr, 0, ptr, ptr, ptr, ws,
                                         None)
    assert hist(ptr=None) == -1                   # null pointers
    assert hist(kv_begin=1, kv_count=2) == -1     # kv range past hkv
    assert hist(kv_count=0) == -1
    assert hist(topk=1) == -2                     # no history slots
    assert hist(d=96) == -2                       # unsupported head dim, before pointers
    assert hist(ws=ws_needed // 1000) == -3       # workspace too small
    b, T, hq, hkv, d, B, k, sc = shape
    m = lib.moba_current_merge
    assert m(None, None, None, b, T, hq, hkv, d, B, k, sc, 0, 2, None, None, None, None,
             None) == -1
    # topk > 1 needs the parts
    assert m(one, one, one, b, T, hq, hkv, d, B, k, sc, 0, 2, None, None, one, one,
             None) == -1
    assert m(one, one, one, b, T, hq, hkv, d, B, k, sc, 2, 1, one, one, one, one, None) == -1
    assert m(one, one, one, b, T, hq, hkv, 96, B, k, sc, 0, 2, one, one, one, one,
             None) == -2


def test_decode_args_and_workspace(moba):
    lib = moba.lib
    ws = moba.decode_workspace_bytes(1, 1, 131072, 32, 8, 128)
    # fp32 partials of 4 rows per kv-head and split, and their lse: small next to the
    # 537 MB the cache holds
    assert 0 < ws < 64 << 20
    assert moba.decode_workspace_bytes(1, 8, 1000, 4, 1, 64) > 0        # G * n = 32
    assert moba.decode_workspace_bytes(1, 9, 1000, 4, 1, 64) > 0        # two row tiles
    assert moba.decode_workspace_bytes(1, 257, 1000, 4, 1, 64) == 0     # G * n = 1028
    assert moba.decode_workspace_bytes(1, 5, 4, 1, 1, 64) == 0          # n > kv_len
    assert moba.decode_workspace_bytes(1, 1, 100, 6, 4, 64) == 0        # hq % hkv
    assert moba.decode_workspace_bytes(1, 1, 100, 4, 1, 96) == 0        # head_dim 96
    # shape rules first, then the pointers, all on the host
    assert lib.moba_decode(None, None, None, 1, 1, 100, 4, 1, 96, 0.125, None, None, None,
                           0, None) == -2
    assert lib.moba_decode(None, None, None, 1, 1, 100, 4, 1, 64, 0.125, None, None, None,
                           0, None) == -1
    assert lib.moba_decode(None, None, None, 1, 2, 1, 4, 1, 64, 0.125, None, None, None,
                           0, None) == -1


_ASAN_DRIVER = r"""
import ctypes, sys
lib = ctypes.CDLL(sys.argv[1])
i, f, vp, sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
lib.moba_check_args.argtypes = [i] * 7 + [f]
lib.moba_workspace_bytes.restype = sz
lib.moba_workspace_bytes.argtypes = [i] * 7 + [ctypes.POINTER(sz)]
lib.moba_backward_workspace_bytes.restype = sz
lib.moba_backward_workspace_bytes.argtypes = [i] * 7 + [ctypes.POINTER(sz)]
lib.moba_varlen_workspace_bytes.restype = sz
lib.moba_varlen_workspace_bytes.argtypes = [i] * 8 + [ctypes.POINTER(sz)]
lib.moba_backward_varlen_workspace_bytes.restype = sz
lib.moba_backward_varlen_workspace_bytes.argtypes = [i] * 8 + [ctypes.POINTER(sz)]
lib.moba_decode_workspace_bytes.restype = sz
lib.moba_decode_workspace_bytes.argtypes = [i] * 6
lib.moba_stage_workspace_bytes.restype = sz
lib.moba_stage_workspace_bytes.argtypes = [i] * 7
lib.moba_index_entries.restype = ctypes.c_int64
lib.moba_index_entries.argtypes = [i] * 7
lib.moba_strerror.restype = ctypes.c_char_p
lib.moba_forward.argtypes = [vp] * 3 + [i] * 7 + [f] + [vp] * 4 + [sz, vp]
lib.moba_forward_noalloc.argtypes = [vp] * 3 + [i] * 7 + [f] + [vp] * 4
lib.moba_dense_forward.argtypes = [vp] * 3 + [i] * 5 + [f] + [vp] * 3
mn = sz(0)
shapes = [(1, 131072, 32, 8, 128, 4096, 12), (2, 1000, 4, 2, 64, 128, 4), (1, 48005, 2, 1, 64, 16, 8),
          (1, 4096, 4, 2, 128, 128, 40), (1, 777, 8, 2, 128, 16, 200), (3, 1, 4, 2, 128, 16, 3),
          (1, 65536, 32, 8, 128, 128, 16), (1, 16 * 8193, 1, 1, 64, 16, 2), (1, 128, 3, 2, 64, 16, 1),
          (0, 128, 1, 1, 64, 16, 1), (1, 1 << 27, 1, 1, 64, 1 << 20, 2), (1, 4480, 2, 1, 64, 64, 65)]
n = 0
for s in shapes:
    lib.moba_check_args(*s, 0.125)
    lib.moba_workspace_bytes(*s, ctypes.byref(mn))
    lib.moba_backward_workspace_bytes(*s, ctypes.byref(mn))
    lib.moba_stage_workspace_bytes(*s)
    b, T, hq, hkv, d, B, k = s
    lib.moba_varlen_workspace_bytes(max(b, 1), max(b, 1) * T, T, hq, hkv, d, B, k, ctypes.byref(mn))
    lib.moba_backward_varlen_workspace_bytes(max(b, 1), max(b, 1) * T, T, hq, hkv, d, B, k,
                                             ctypes.byref(mn))
    lib.moba_index_entries(b, T, hq, hkv, B, k, hkv)
    lib.moba_decode_workspace_bytes(b, 1, T, hq, hkv, d)
    # every pointer NULL: rejected on the host before any device work
    assert lib.moba_forward(None, None, None, *s, 0.125, None, None, None, None, 0, None) < 0
    assert lib.moba_forward_noalloc(None, None, None, *s, 0.125, None, None, None, None) < 0
    assert lib.moba_dense_forward(None, None, None, b, T, hq, hkv, d, 0.125, None, None, None) < 0
    n += 1
for st in range(-6, 2):
    assert lib.moba_strerror(st)
print("asan driver ok", n)
"""


def test_host_code_under_address_sanitizer(tmp_path):
    """The host code (argument checks, workspace layouts, the entry points' early
    rejections) built with AddressSanitizer and driven over edge shapes in a process
    that preloads the ASan runtime: any out-of-bounds access or use after free on the
    host aborts it."""
    import importlib.util
    import subprocess
    import sys
    spec = importlib.util.spec_from_file_location(
        "_moba_build", os.path.join(ROOT, "block_sparse_long_pool_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    try:
        rt = b.asan_runtime()
    except RuntimeError:
        pytest.skip("no clang ASan runtime in this image")
    lib = b.build_host_asan(str(tmp_path / "asan"))
    drv = tmp_path / "drive.py"
    drv.write_text(_ASAN_DRIVER)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, str(drv), lib], capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0 and "asan driver ok" in r.stdout, r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr
