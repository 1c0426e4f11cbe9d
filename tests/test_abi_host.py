"""Host-only checks of the C ABI: the library loads, exports every function
include/csa.h declares, and rejects bad arguments on the host (before any
GPU call) with the documented codes.  No compute call is made."""
import ctypes

import pytest

from compressed_sparse_attention_c4a_amd import binding as K

CSA_ERR_NULL, CSA_ERR_SHAPE, CSA_ERR_DTYPE, CSA_ERR_ALIGN, CSA_ERR_WORKSPACE = -1, -2, -3, -5, -6


@pytest.fixture(scope="module")
def lib():
    return K.load()


def test_exports_every_declared_function(lib):
    names = K.declared_functions()
    assert {"csa_compress", "csa_index_topk", "csa_sparse_attn", "hca_attn"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libcsa.so does not export {n}"


def test_version_and_error_strings(lib):
    assert lib.csa_version() >= 1
    assert lib.csa_error_string(0) == b"ok"
    assert lib.csa_error_string(CSA_ERR_WORKSPACE).startswith(b"workspace")


P = ctypes.c_void_p(4096)       # a non-null, aligned host stand-in: never dereferenced on these paths
MIS = ctypes.c_void_p(4096 + 4)


def _compress(lib, kv=P, sc=P, gamma=P, cache=P, pos0=P, B=2, L=8, d=512, rope=64, ratio=4, overlap=1, N=16,
              eps=1e-6, dtype=1):
    return lib.csa_compress(kv, sc, gamma, cache, pos0, B, L, d, rope, ratio, overlap, N, eps, 10000.0, dtype, None)


def test_compress_validation(lib):
    assert _compress(lib, kv=None) == CSA_ERR_NULL
    assert b"kv_state" in lib.csa_last_error()
    assert _compress(lib, cache=MIS) == CSA_ERR_ALIGN
    assert _compress(lib, dtype=7) == CSA_ERR_DTYPE
    assert _compress(lib, d=513) == CSA_ERR_SHAPE
    assert _compress(lib, rope=66, d=64) == CSA_ERR_SHAPE
    assert _compress(lib, ratio=0) == CSA_ERR_SHAPE
    assert _compress(lib, overlap=2) == CSA_ERR_SHAPE
    assert _compress(lib, B=0) == CSA_ERR_SHAPE


def test_index_and_topk_validation(lib):
    a = (P, P, P, P, P)
    assert lib.csa_index_scores(None, P, P, P, P, 1, 1, 64, 128, 100, 4, 0, 1, None) == CSA_ERR_NULL
    assert lib.csa_index_scores(*a, 1, 1, 64, 128, 100, 4, 8, 1, None) == CSA_ERR_SHAPE      # unknown flag
    assert lib.csa_topk(P, P, P, None, None, 0, 1, 1, 100, 0, 4, None) == CSA_ERR_SHAPE       # k = 0
    assert lib.csa_topk(P, P, P, None, None, 0, 1, 1, 100, 5000, 4, None) == CSA_ERR_SHAPE    # k > 4096
    # a row longer than 32 keys per thread is cut into chunks: their kept lists need workspace
    assert lib.csa_topk_workspace_size(8, 1, 32768, 1024) == 0
    nws = lib.csa_topk_workspace_size(8, 1, 262144, 1024)
    assert nws >= 2 * 8 * 16 * 1024 * 8      # 16 chunks of 16384 entries; two buffers of values + indices
    assert lib.csa_topk(P, P, P, None, None, 0, 8, 1, 262144, 1024, 4, None) == CSA_ERR_WORKSPACE
    assert lib.csa_topk(P, P, P, None, P, nws - 1, 8, 1, 262144, 1024, 4, None) == CSA_ERR_WORKSPACE
    need = lib.csa_index_topk_workspace_size(2, 1, 100, 16)
    assert need >= 2 * 100 * 4
    assert lib.csa_index_topk(P, P, P, P, P, None, P, need - 1, 2, 1, 64, 128, 100, 16, 4, 0, 1,
                              None) == CSA_ERR_WORKSPACE
    assert lib.csa_index_topk(P, P, P, P, P, None, None, need, 2, 1, 64, 128, 100, 16, 4, 0, 1,
                              None) == CSA_ERR_WORKSPACE


def _cit(lib, kv=P, idx_cache=P, pos0=P, topk=P, ws=P, ws_bytes=1 << 30, d=512, di=128, L=8, k=16, ratio=4):
    """csa_compress_index_topk with valid-looking host arguments (no launch
    happens: every case below fails validation first)."""
    return lib.csa_compress_index_topk(kv, P, P, P, d, 64, 1, P, P, P, idx_cache, 64, pos0, L, P, P, P, topk, None,
                                       ws, ws_bytes, 2, 1, 64, di, 100, k, ratio, 0, 1e-6, 10000.0, 1, None)


def test_compress_index_topk_validation(lib):
    assert _cit(lib, kv=None) == CSA_ERR_NULL
    assert _cit(lib, idx_cache=None) == CSA_ERR_NULL
    assert _cit(lib, pos0=None) == CSA_ERR_NULL
    assert _cit(lib, topk=None) == CSA_ERR_NULL
    assert _cit(lib, kv=MIS) == CSA_ERR_ALIGN
    assert _cit(lib, d=513) == CSA_ERR_SHAPE
    assert _cit(lib, L=0) == CSA_ERR_SHAPE
    assert _cit(lib, k=0) == CSA_ERR_SHAPE
    need = lib.csa_index_topk_workspace_size(2, 1, 100, 16)
    assert _cit(lib, ws_bytes=need - 1) == CSA_ERR_WORKSPACE
    assert _cit(lib, ws=None) == CSA_ERR_WORKSPACE


def _attn(lib, q=P, cmp=P, idx=P, win=P, wp=None, sink=P, qp=P, out=P, lse=None, B=1, S=1, H=128, D=512, rope=64,
          N=100, k=16, W=128, window=128, dtype=1):
    return lib.csa_sparse_attn(q, cmp, idx, win, wp, sink, qp, out, lse, None, 0, B, S, H, D, rope, N, k, W, window,
                               0.04, 10000.0, dtype, None)


def test_attention_validation(lib):
    assert _attn(lib, q=None) == CSA_ERR_NULL
    assert _attn(lib, idx=None) == CSA_ERR_NULL
    assert _attn(lib, out=MIS) == CSA_ERR_ALIGN
    assert _attn(lib, D=514) == CSA_ERR_SHAPE
    assert _attn(lib, rope=65) == CSA_ERR_SHAPE
    assert _attn(lib, window=129) == CSA_ERR_SHAPE            # ring window larger than the ring
    assert _attn(lib, dtype=2) == CSA_ERR_DTYPE
    assert lib.hca_attn(P, P, P, None, P, P, P, None, None, 0, 1, 1, 128, 512, 64, 100, 0, 128, 128, 0.04, 10000.0,
                        1, None) == CSA_ERR_SHAPE               # ratio 0


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4)
    with pytest.raises(ValueError):
        K._ptr(x, None, "x")
