"""GPU parity of the FP8 KV row format against the oracle, bit for bit:
csa_dequantize_rows on rows holding every E4M3 code under many block
exponents, and csa_quantize_rows on bf16 rows whose blocks span zero,
subnormal-range, tie and boundary values."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_c4a_amd import binding as K
from compressed_sparse_attention_c4a_amd import workloads as W

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def test_dequantize_every_code_and_exponent(orc):
    rng = np.random.default_rng(21)
    R = 64
    rows = np.zeros((R, 640), dtype=np.uint8)
    rows[:, :448] = np.tile(np.arange(256, dtype=np.uint8), 112)[: R * 448].reshape(R, 448)
    rng.shuffle(rows[:, :448], axis=1)
    rows[:, 448:576] = W.bf16_bits(rng.standard_normal((R, 64)).astype(np.float32)).view(np.uint8).reshape(R, 128)
    rows[:, 576:583] = rng.integers(-40, 41, size=(R, 7)).astype(np.int8).view(np.uint8)
    print(f"[fp8] dequantize {R} rows", flush=True)
    got = _bits(K.csa_dequantize_rows(torch.from_numpy(rows).cuda()))
    ref = orc.dequantize_rows_fp8(rows)
    nan = np.isnan(ref)
    got_f = (got.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(np.isnan(got_f), nan)
    assert np.array_equal(got[~nan], orc.round_bf16(ref[~nan]))
    # every value is exact: the oracle's fp64 value is a bf16 value
    assert np.array_equal((got[~nan].astype(np.uint32) << 16).view(np.float32).astype(np.float64), ref[~nan])


def test_dequantize_all_codes_at_every_exponent(orc):
    """Each exponent k in [-120, 120] with every code in every block (4 rows
    per k), against the oracle's exact values: the extremes give bf16
    subnormals (2^-129) and 448 * 2^120."""
    ks = np.arange(-120, 121)
    codes = np.concatenate([np.arange(256, dtype=np.uint8)] * 7)          # 1792 = 4 rows x 448
    rows = np.zeros((len(ks) * 4, 640), dtype=np.uint8)
    rows[:, :448] = np.tile(codes.reshape(4, 448), (len(ks), 1))
    rows[:, 576:583] = np.repeat(ks, 4)[:, None].astype(np.int8).view(np.uint8)
    got = _bits(K.csa_dequantize_rows(torch.from_numpy(rows).cuda()))
    ref = orc.dequantize_rows_fp8(rows)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan((got.astype(np.uint32) << 16).view(np.float32)), nan)
    assert np.array_equal(got[~nan], orc.round_bf16(ref[~nan]))


def _hard_rows(rng, R):
    x = rng.standard_normal((R, 512)).astype(np.float32)
    scale = np.exp2(rng.integers(-30, 20, size=(R, 8))).astype(np.float32)
    x *= np.repeat(scale, 64, axis=1)
    x[0, :64] = 0.0                                             # all-zero block
    x[1, :64] = 1e-30                                           # tiny block
    x[2, 64:128] = 0.0
    x[2, 64] = 448.0 * 2.0 ** 3                                 # maximum exactly on a boundary
    x[3, :64] = rng.choice([-1.0, 1.0], 64) * np.float32(1.0)
    x[3, 1:9] = np.array([1.0625, 1.1875, 1.3125, 1.4375, 1.5625, 1.6875, 1.8125, 1.9375], np.float32) / 256
    x[4, :64] = np.float32(2.0 ** -20) * rng.standard_normal(64).astype(np.float32)
    x[4, 0] = 1.0                                               # wide block: most values in the subnormal range
    return W.bf16_bits(x)


def test_quantize_matches_oracle_bit_for_bit(orc):
    rng = np.random.default_rng(22)
    R = 1000
    bits = _hard_rows(rng, R)
    print(f"[fp8] quantize {R} rows", flush=True)
    dev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    got = K.csa_quantize_rows(dev).cpu().numpy()
    ref = orc.quantize_rows_fp8(orc.widen(bits))
    assert np.array_equal(got, ref)
    back = _bits(K.csa_dequantize_rows(K.csa_quantize_rows(dev)))
    assert np.array_equal(back, orc.round_bf16(orc.dequantize_rows_fp8(ref)))


def test_quantize_empty_and_odd_counts(orc):
    rng = np.random.default_rng(23)
    for R in (0, 1, 5):
        bits = W.bf16_bits(rng.standard_normal((R, 512)).astype(np.float32))
        dev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16).reshape(R, 512)
        got = K.csa_quantize_rows(dev).cpu().numpy()
        assert got.shape == (R, 640)
        if R:
            assert np.array_equal(got, orc.quantize_rows_fp8(orc.widen(bits)))


# ---------------------------------------------------------------- attention on FP8 rows
from test_gpu_attention import VARIANTS, _dev, _inputs, _seed  # noqa: E402
from parity import TOL, assert_close, to_np  # noqa: E402


def _attn(x, cmp, win, dense, window, H, B, S):
    out = torch.empty((B, S, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, S, H), dtype=torch.float32, device="cuda")
    if dense:
        K.hca_attn(_dev(x["q"]), cmp, win, _dev(x["win_pos0"]), _dev(x["sink"]), _dev(x["q_pos"]), out, lse,
                   ratio=4, rope_dim=64, window=window)
    else:
        K.csa_sparse_attn(_dev(x["q"]), cmp, _dev(x["topk"]), win, _dev(x["win_pos0"]), _dev(x["sink"]),
                          _dev(x["q_pos"]), out, lse, rope_dim=64, window=window)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("name", sorted(VARIANTS))
@pytest.mark.parametrize("dense", [False, True])
def test_attention_on_fp8_rows(orc, name, dense):
    """The FP8-row kernel equals the bf16 kernel on the dequantised rows bit for
    bit (it stages exactly those values), and the oracle reading FP8 rows."""
    B, S, H, N_cap, W_cap, k, q_pos, linear, window = VARIANTS[name]
    x = _inputs(_seed(name) + 7, B, S, H, N_cap, W_cap, k, q_pos, linear)
    print(f"[fp8] attention {name} dense={dense}", flush=True)
    cmp8, win8 = K.csa_quantize_rows(_dev(x["cmp"])), K.csa_quantize_rows(_dev(x["win"]))
    cmp8_h, win8_h = cmp8.cpu().numpy(), win8.cpu().numpy()
    assert np.array_equal(cmp8_h, orc.quantize_rows_fp8(orc.widen(x["cmp"])))
    assert np.array_equal(win8_h, orc.quantize_rows_fp8(orc.widen(x["win"])))
    out8, lse8 = _attn(x, cmp8, win8, dense, window, H, B, S)
    outd, lsed = _attn(x, K.csa_dequantize_rows(cmp8), K.csa_dequantize_rows(win8), dense, window, H, B, S)
    assert torch.equal(out8, outd) and torch.equal(lse8, lsed)
    ref, rlse, _ = orc.attn(x["q"], cmp8_h, win8_h, x["sink"], x["q_pos"], topk_idx=None if dense else x["topk"],
                            ratio=4, win_pos0=x["win_pos0"], window=window, rope_dim=64)
    assert_close(to_np(out8), ref, TOL["bf16"], f"fp8 {name} dense={dense}: output")
    assert_close(lse8.cpu().numpy(), rlse, 1e-3, f"fp8 {name} dense={dense}: lse")


def test_swa_on_fp8_rows(orc):
    B, H, W_cap, window = 3, 128, 256, 256
    x = _inputs(31, B, 1, H, 1, W_cap, 1, [5000, 40, 0])
    win8 = K.csa_quantize_rows(_dev(x["win"]))
    out = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 1, H), dtype=torch.float32, device="cuda")
    K.swa_attn(_dev(x["q"]), win8, None, _dev(x["sink"]), _dev(x["q_pos"]), out, lse, rope_dim=64, window=window)
    torch.cuda.synchronize()
    none = np.zeros((B, 0, 640), dtype=np.uint8)
    ref, rlse, _ = orc.attn(x["q"], none, win8.cpu().numpy(), x["sink"], x["q_pos"],
                            topk_idx=np.zeros((B, 1, 0), dtype=np.int32), ratio=1, window=window, rope_dim=64)
    assert_close(to_np(out), ref, TOL["bf16"], "fp8 swa: output")
    assert_close(lse.cpu().numpy(), rlse, 1e-3, "fp8 swa: lse")


# ---------------------------------------------------------------- whole path with FP8 caches
from compressed_sparse_attention_c4a_amd import path as P  # noqa: E402
from parity import check_topk_sets  # noqa: E402
from test_gpu_parity import CASES  # noqa: E402

FP8_CASES = ["csa_decode_ragged_bf16", "csa_decode_short_ctx_bf16", "csa_prefill_small_bf16", "hca_decode_small_bf16"]


def _fp8_copies(inp, orc):
    """Device and host copies of a workload with the main cache and the window
    rows in FP8: quantised by the library and by the oracle, bit-identical."""
    dev = P.to_device(inp)
    dev["cmp_cache"] = K.csa_quantize_rows(dev["cmp_cache"])
    dev["win_kv"] = K.csa_quantize_rows(dev["win_kv"])
    host = dict(inp)
    host["cmp_cache"] = orc.quantize_rows_fp8(orc.widen(inp["cmp_cache"]))
    host["win_kv"] = orc.quantize_rows_fp8(orc.widen(inp["win_kv"]))
    assert np.array_equal(dev["cmp_cache"].cpu().numpy(), host["cmp_cache"])
    assert np.array_equal(dev["win_kv"].cpu().numpy(), host["win_kv"])
    return dev, host


def _compare_fp8_entries(gpu_rows, orc_rows, orc_vals, what):
    """Fresh FP8 entries: the kernels decide on their float32 values and the
    oracle on the float32 rounding of its fp64 values, so a code may differ
    where the two straddle a rounding boundary; almost every byte must agree,
    the RoPE dims within one bf16 step and every value within two E4M3 steps
    of the oracle's value."""
    g, o = np.asarray(gpu_rows), np.asarray(orc_rows)
    assert g.shape == o.shape and g.shape[-1] == 640
    same = np.mean(g[..., :583] == o[..., :583])
    print(f"[fp8] {what}: {g.shape[0]} entries, {100 * same:.3f}% of code/exponent bytes identical", flush=True)
    assert same >= 0.999, f"{what}: only {same:.4%} of the bytes agree"
    assert np.all(g[..., 583:] == 0)
    from oracle import oracle as orc
    gd, od = orc.dequantize_rows_fp8(g), orc.dequantize_rows_fp8(o)
    k = o[..., 576:583].view(np.int8).astype(np.int64)
    a = np.abs(np.asarray(orc_vals)[..., :448]).reshape(-1, 7, 64) / np.ldexp(1.0, k.reshape(-1, 7))[..., None]
    _, E = np.frexp(np.maximum(a, 2.0 ** -6))
    step = np.ldexp(1.0, k.reshape(-1, 7))[..., None] * np.ldexp(1.0, E - 4)
    assert np.all(np.abs(gd[..., :448].reshape(-1, 7, 64) - np.asarray(orc_vals)[..., :448].reshape(-1, 7, 64))
                  <= 2 * step + 1e-30)
    assert np.max(np.abs(gd[..., 448:] - od[..., 448:]) / np.maximum(np.abs(od[..., 448:]), 1e-30)) <= 2.0 ** -7


@pytest.mark.parametrize("name", FP8_CASES)
def test_path_with_fp8_caches(orc, name):
    inp = CASES[name]
    sh = inp["shape"]
    print(f"[fp8] path {name}", flush=True)
    dev, host = _fp8_copies(inp, orc)
    ref = orc.pipeline(host)
    step = P.Step(dev)
    out = step.run(dev)
    torch.cuda.synchronize()
    gcache = dev["cmp_cache"].cpu().numpy()
    wr = ref["written"]
    if wr.any():
        _compare_fp8_entries(gcache[wr], ref["cmp_cache"][wr], ref["cmp_vals"][wr], f"{name}: compressed rows")
    assert np.array_equal(gcache[~wr], host["cmp_cache"][~wr])        # untouched rows stay as they were
    topk = None
    if sh.indexer:
        topk = step.topk_idx.cpu().numpy()
        check_topk_sets(topk, ref["topk_idx"], ref["scores"], ref["nvis"], sh.k)
    # the oracle's attention over the GPU's own FP8 cache and selection
    o2, l2, _ = orc.attn(inp["q"], gcache, host["win_kv"], inp["sink"], inp["q_pos"], topk_idx=topk,
                         ratio=sh.ratio, win_pos0=inp.get("win_pos0"), window=sh.window, rope_dim=sh.rope)
    assert_close(to_np(out), o2, TOL["bf16"], f"fp8 {name}: output")


def test_fused_decode_with_fp8_cache_equals_separate_calls(orc):
    inp = CASES["csa_decode_ragged_bf16"]
    sh = inp["shape"]
    res = []
    for fused in (False, True):
        d, _ = _fp8_copies(inp, orc)
        idx = torch.empty((sh.B, sh.S, sh.k), dtype=torch.int32, device="cuda")
        ws = torch.empty(K.csa_index_topk_workspace_size(sh.B, sh.S, sh.N_cap, sh.k), dtype=torch.uint8,
                         device="cuda")
        if fused:
            K.csa_compress_index_topk(d["kv_state"], d["score_state"], d["gamma"], d["cmp_cache"], d["idx_kv_state"],
                                      d["idx_score_state"], d["idx_gamma"], d["idx_cache"], d["state_pos0"],
                                      d["q_idx"], d["w"], d["q_pos"], idx, ratio=sh.ratio, overlap=sh.overlap,
                                      rope_dim=sh.rope, idx_rope_dim=sh.idx_rope, workspace=ws)
        else:
            K.csa_compress_kv_index(d["kv_state"], d["score_state"], d["gamma"], d["cmp_cache"], d["idx_kv_state"],
                                    d["idx_score_state"], d["idx_gamma"], d["idx_cache"], d["state_pos0"],
                                    ratio=sh.ratio, overlap=sh.overlap, rope_dim=sh.rope, idx_rope_dim=sh.idx_rope)
            K.csa_index_topk(d["q_idx"], d["w"], d["idx_cache"], d["q_pos"], idx, ratio=sh.ratio, workspace=ws)
        torch.cuda.synchronize()
        res.append((d["cmp_cache"].cpu().numpy(), d["idx_cache"].cpu().view(torch.int16).numpy(), idx.cpu().numpy()))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["csa_decode_32k", "hca_decode_128k"])
def test_full_size_decode_with_fp8_caches(orc, name):
    """The bench's FP8 workloads (the same Step and launch shapes): fresh
    entries, the index sets, and every output against the oracle on the
    GPU's own FP8 cache and selection."""
    sh = getattr(W, name)()
    inp = W.generate(sh)
    print(f"[fp8] full size {name}", flush=True)
    dev, host = _fp8_copies(inp, orc)
    step = P.Step(dev)
    out = step.run(dev)
    torch.cuda.synchronize()
    ref = orc.pipeline(host)
    wr = ref["written"]
    assert wr.any()
    gcache = dev["cmp_cache"].cpu().numpy()
    _compare_fp8_entries(gcache[wr], ref["cmp_cache"][wr], ref["cmp_vals"][wr], f"{name}: compressed rows")
    topk = None
    if sh.indexer:
        topk = step.topk_idx.cpu().numpy()
        check_topk_sets(topk, ref["topk_idx"], ref["scores"], ref["nvis"], sh.k)
    o2, l2, _ = orc.attn(inp["q"], gcache, host["win_kv"], inp["sink"], inp["q_pos"], topk_idx=topk,
                         ratio=sh.ratio, window=sh.window, rope_dim=sh.rope)
    assert_close(to_np(out), o2, TOL["bf16"], f"fp8 {name}: output")
    assert_close(step.lse.cpu().numpy(), l2, 1e-3, f"fp8 {name}: lse")
