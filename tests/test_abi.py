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
              "moba_pool_centroids", "moba_gate_topk", "moba_build_index"]:
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
    assert moba.check_args(1, 16 * 2049, 1, 1, 64, 16, 1, 1.0) == E_UNS    # > 2048 blocks
    # the backward takes a partial last block as well
    assert moba.backward_workspace_bytes(1, 130, 1, 1, 64, 16, 2)[0] > 0
    assert moba.backward_workspace_bytes(1, 128, 1, 1, 64, 16, 2)[0] > 0
    assert moba.backward_varlen_workspace_bytes(2, 300, 200, 4, 2, 64, 16, 3)[0] > 0
    assert moba.backward_varlen_workspace_bytes(2, 300, 400, 4, 2, 64, 16, 3) == (0, 0)
    assert moba.check_args(1, 128, 1, 1, 64, 16, 34, 1.0) == E_UNS         # topk > 33
    assert moba.check_args(1, 128, 1, 1, 64, 16, 33, 1.0) == 0
    assert moba.check_args(1, 128, 1, 1, 64, 16, 2, -1.0) == E_UNS         # scale <= 0
    assert moba.check_args(1, 1 << 27, 1, 1, 64, 1 << 20, 2, 1.0) == E_UNS  # T*G too big


def test_workspace_sizes(moba):
    full, mn = moba.workspace_bytes(1, 131072, 32, 8, 128, 4096, 12)
    assert 0 < mn < full
    # history partials dominate: [Hq, T, topk - 1, d] bf16 for all heads
    assert full > 32 * 131072 * 11 * 128 * 2
    assert mn < full / 4
    assert moba.workspace_bytes(1, 130, 1, 1, 64, 16, 2)[0] > 0    # partial last block
    assert moba.workspace_bytes(1, 130, 1, 1, 96, 16, 2) == (0, 0)    # head_dim 96


def test_index_entry_count_closed_form(moba):
    # B * Hq * sum_c min(c, k-1): 4096 * 32 * (0+1+...+10 + 21*11) = 37,486,592
    assert moba.index_entries(1, 131072, 32, 8, 4096, 12, 8) == 37_486_592
    assert moba.index_entries(1, 131072, 32, 8, 4096, 12, 1) == 37_486_592 // 8
    assert moba.index_entries(1, 131072, 32, 8, 4096, 12, 9) == -1


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
    # dense causal attention: seqlen a multiple of 16, pointers checked on the host
    assert lib.moba_dense_forward(None, None, None, 1, 130, 1, 1, 64, 0.125, None, None,
                                  None) == -2
    assert lib.moba_dense_forward(None, None, None, 1, 128, 1, 1, 64, 0.125, None, None,
                                  None) == -1
    # the timed variant needs MOBA_NUM_STAGES + 1 non-null event handles
    args = (None, None, None, 1, 128, 1, 1, 64, 16, 2, 0.125, None, None, None, None, 0, None)
    assert lib.moba_forward_timed(*args, None) == -1
    ev = (ctypes.c_void_p * (len(moba.STAGES) + 1))(*([1] * len(moba.STAGES) + [None]))
    assert lib.moba_forward_timed(*args, ev) == -1


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
