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


def test_attention_plan(lib):
    """Head grouping and splits come from the cost model; read back through the
    workspace size (one 33024-byte partial per workgroup when the list is
    split, none otherwise)."""
    part = 4 * 8 * 2 * 64 * 4 * 2 + 64 * 4

    def ws(B, H, n_cand):
        return lib.csa_attn_workspace_size(B, 1, H, 512, n_cand)

    assert ws(32, 128, 1152) == 256 * part   # CSA decode, 32K: 32 heads, 2 splits (16 heads: no split)
    assert ws(64, 128, 1152) == 0            # HCA decode, 128K: 32 heads, no split
    assert ws(32, 128, 384) == 0             # HCA decode, 32K: 16 heads, no split (32 heads: 2 splits)
    assert ws(32, 128, 128) == 0             # window-only layer: 16 heads, no split
    assert ws(8192, 128, 1152) == 0          # prefill chunk
    assert ws(5, 128, 224) == 80 * part      # 5 queries: 16 heads (8 groups) x 2 splits
    assert ws(16, 128, 1152) == 256 * part   # 16 queries: 32 heads x 4 splits


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
    assert _attn(lib, dtype=5) == CSA_ERR_DTYPE
    assert lib.hca_attn(P, P, P, None, P, P, P, None, None, 0, 1, 1, 128, 512, 64, 100, 0, 128, 128, 0.04, 10000.0,
                        1, None) == CSA_ERR_SHAPE               # ratio 0


def test_swa_validation(lib):
    def swa(q=P, win=P, sink=P, qp=P, out=P, B=2, H=128, D=512, rope=64, W=128, window=128, dtype=1, ws=None, nws=0):
        return lib.swa_attn(q, win, None, sink, qp, out, None, ws, nws, B, 1, H, D, rope, W, window, 0.04, 10000.0,
                            dtype, None)
    assert swa(win=None) == CSA_ERR_NULL
    assert swa(q=MIS) == CSA_ERR_ALIGN
    assert swa(window=129) == CSA_ERR_SHAPE
    assert swa(dtype=3) == CSA_ERR_DTYPE
    assert swa(B=8, H=16, W=1024, window=1024) == CSA_ERR_WORKSPACE   # 8 items over 16 tiles: split partials


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4)
    with pytest.raises(ValueError):
        K._ptr(x, None, "x")


def test_q_proj_validation(lib):
    """Argument checks of csa_q_proj, all rejected before any launch."""
    def qp(x=P, wa=P, g=P, wb=P, pos=P, qr=P, q=P, B=32, S=1, dm=7168, qrk=1536, H=128, D=512, rope=64, ws=P,
           nws=1 << 30):
        return lib.csa_q_proj(x, wa, g, wb, pos, qr, q, ws, nws, B, S, dm, qrk, H, D, rope, 1e-6, 10000.0, None)
    assert qp(wb=None) == CSA_ERR_NULL
    assert qp(qr=MIS) == CSA_ERR_ALIGN
    assert qp(qrk=700) == CSA_ERR_SHAPE
    assert qp(qrk=4096) == CSA_ERR_SHAPE
    assert qp(dm=7000) == CSA_ERR_SHAPE
    assert qp(D=500) == CSA_ERR_SHAPE
    assert qp(rope=65) == CSA_ERR_SHAPE
    assert qp(B=0) == CSA_ERR_SHAPE
    need = lib.csa_q_proj_workspace_size(32, 7168, 1536, 128, 512)
    assert need >= 32 * 128 * 512 * 4
    assert qp(ws=None) == CSA_ERR_WORKSPACE
    assert qp(nws=need - 1) == CSA_ERR_WORKSPACE


def test_o_proj_validation(lib):
    def op(o=P, wa=P, wb=P, r=P, y=P, M=32, H=128, D=512, G=16, orank=1024, dm=7168, ws=P, nws=1 << 30):
        return lib.csa_o_proj(o, wa, wb, r, y, ws, nws, M, H, D, G, orank, dm, None)
    assert op(y=None) == CSA_ERR_NULL
    assert op(wa=MIS) == CSA_ERR_ALIGN
    assert op(G=3) == CSA_ERR_SHAPE          # does not divide H
    assert op(orank=1000) == CSA_ERR_SHAPE
    assert op(dm=7100) == CSA_ERR_SHAPE
    assert op(M=0) == CSA_ERR_SHAPE
    need = lib.csa_o_proj_workspace_size(32, 128, 512, 16, 1024, 7168)
    assert need >= 16 * 32 * 1024 * 4
    assert op(nws=need - 1) == CSA_ERR_WORKSPACE


def test_pack_weights_validation(lib):
    assert lib.csa_pack_weights(None, P, 1, 64, 512, None) == CSA_ERR_NULL
    assert lib.csa_pack_weights(P, MIS, 1, 64, 512, None) == CSA_ERR_ALIGN
    assert lib.csa_pack_weights(P, P, 1, 96, 512, None) == CSA_ERR_SHAPE       # N % 64
    assert lib.csa_pack_weights(P, P, 1, 64, 768, None) == CSA_ERR_SHAPE       # K % 512
    assert lib.csa_pack_weights(P, ctypes.c_void_p(4096 + 1024), 1, 64, 512, None) == CSA_ERR_SHAPE   # overlap


def test_fp8_rows_validation(lib):
    assert lib.csa_quantize_rows(None, P, 4, 512, 64, None) == CSA_ERR_NULL
    assert lib.csa_quantize_rows(P, MIS, 4, 512, 64, None) == CSA_ERR_ALIGN
    assert lib.csa_quantize_rows(P, ctypes.c_void_p(1 << 20), 4, 256, 64, None) == CSA_ERR_SHAPE   # D != 512
    assert lib.csa_quantize_rows(P, ctypes.c_void_p(1 << 20), 4, 512, 32, None) == CSA_ERR_SHAPE   # rope != 64
    assert lib.csa_dequantize_rows(P, ctypes.c_void_p(4096 + 640), 4, 512, 64, None) == CSA_ERR_SHAPE  # overlap
    assert lib.csa_quantize_rows(P, ctypes.c_void_p(1 << 20), -1, 512, 64, None) == CSA_ERR_SHAPE


def test_fp8_attention_shapes(lib):
    CSA_ERR_UNSUPPORTED = -4
    assert _attn(lib, dtype=2, H=48 + 8) == CSA_ERR_UNSUPPORTED        # H % 16 != 0
    assert _attn(lib, dtype=2, rope=32) == CSA_ERR_UNSUPPORTED
    assert _attn(lib, dtype=2, D=256, rope=64) == CSA_ERR_UNSUPPORTED
    assert _attn(lib, dtype=2, k=4096) == CSA_ERR_UNSUPPORTED
    assert _attn(lib, dtype=3) == CSA_ERR_DTYPE


def test_compressor_grid_covers_every_complete_group():
    """The compressor launches ceil(L / ratio) candidate groups per sequence
    (x = 0 .. ceil(L / ratio) - 1 after floor(p0 / ratio)): brute force over
    buffer starts (negative ones too), lengths and ratios finds no complete
    group beyond that."""
    for ratio in (1, 3, 4, 7, 128):
        for L in range(1, 3 * ratio + 5):
            gx = (L + ratio - 1) // ratio
            for p0 in range(-2 * ratio - 3, 3 * ratio + 3):
                g0 = p0 // ratio
                for g in range(g0 - 1, g0 + gx + 3):
                    complete = g * ratio >= p0 and g * ratio + ratio - 1 <= p0 + L - 1
                    if complete:
                        assert 0 <= g - g0 < gx, (ratio, L, p0, g)
