"""CPU pins of the oracle's projections (low-rank Q, grouped O-proj).

"DeepSeek-V4-Pro 架构：一个 token 的旅程", sections "低秩 Q：两次矩阵乘法接起来" and
"输出投影也分组，并且降低中间维度".  Each pin is a closed form, an invariant or a
special case that reduces to a library routine; none retypes the oracle.
"""
import numpy as np
import scipy.linalg

from oracle import oracle as orc


def _perm(n, seed):
    p = np.random.default_rng(seed).permutation(n)
    P = np.zeros((n, n))
    P[np.arange(n), p] = 1.0
    return P, p


def test_q_proj_closed_form_permutation():
    """wq_a = I, gamma = 1, wq_b a permutation, eps = 0, position 0: qr is x
    over its RMS and every head of q is the sign pattern of its permuted
    inputs, whatever per-head magnitude x gave it.  A wrong norm axis, a
    transposed weight or a head-major/dim-major mix-up changes the result."""
    H, D = 4, 8
    n = H * D
    rng = np.random.default_rng(1)
    P, p = _perm(n, 2)
    # magnitudes chosen per *output* head, so the head norm has work to do
    c = np.array([0.5, 2.0, 1.0, 3.0])
    signs = rng.choice([-1.0, 1.0], size=(3, n))
    y_target = signs * np.repeat(c, D)[None, :]        # what P x should be, head by head
    x = np.empty_like(y_target)
    x[:, p] = y_target                                  # (P x)[i] = x[p[i]] = y_target[i]
    q, qr = orc.q_proj(x, np.eye(n), np.ones(n), P, np.zeros(3, dtype=np.int64), H=H, D=D, rope_dim=0, eps=0.0)
    rms = np.sqrt(np.mean(x * x, axis=1, keepdims=True))
    np.testing.assert_allclose(qr, x / rms, rtol=1e-14, atol=0)
    np.testing.assert_allclose(q.reshape(3, n), signs, rtol=1e-14, atol=0)


def test_q_proj_gain_and_scale():
    """The qr gain acts per qr channel (doubling gamma_q is absorbed by the
    head norm, a gain on one channel is not) and q does not depend on the
    scale of x; the RMS of qr over gamma_q is 1 per row."""
    rng = np.random.default_rng(3)
    M, dm, qrk, H, D = 5, 24, 16, 2, 8
    x = rng.standard_normal((M, dm))
    wa = rng.standard_normal((qrk, dm))
    wb = rng.standard_normal((H * D, qrk))
    g = 1.0 + 0.5 * rng.random(qrk)
    pos = np.array([7], dtype=np.int64)
    q1, qr1 = orc.q_proj(x, wa, g, wb, pos, H=H, D=D, rope_dim=4, S=M, eps=0.0)
    q2, _ = orc.q_proj(3.0 * x, wa, 2.0 * g, wb, pos, H=H, D=D, rope_dim=4, S=M, eps=0.0)
    np.testing.assert_allclose(q1, q2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.sqrt(np.mean((qr1 / g) ** 2, axis=1)), 1.0, rtol=1e-13)
    g3 = g.copy()
    g3[0] *= 4.0
    q3, _ = orc.q_proj(x, wa, g3, wb, pos, H=H, D=D, rope_dim=4, S=M, eps=0.0)
    assert np.max(np.abs(q3 - q1)) > 1e-3
    # every head has unit RMS (RoPE only rotates pairs)
    np.testing.assert_allclose(np.sqrt(np.mean(q1 * q1, axis=-1)), 1.0, rtol=1e-13)


def test_q_proj_rope_positions():
    """RoPE touches only the last rope_dim dims, keeps each pair's length, and
    is relative: for equal pre-RoPE heads at positions t1 and t2 the dot
    product of the tails equals that of the tail at t1 - t2 with the tail at
    0.  Row m of a batch with S tokens sits at pos[m // S] + m % S."""
    rng = np.random.default_rng(4)
    dm, qrk, H, D, R = 12, 10, 3, 16, 8
    x1 = rng.standard_normal((1, dm))
    wa, wb, g = rng.standard_normal((qrk, dm)), rng.standard_normal((H * D, qrk)), np.ones(qrk)
    x = np.repeat(x1, 6, axis=0)                       # B=2 sequences of S=3 equal rows
    pos = np.array([5, 100], dtype=np.int64)            # rows at 5,6,7,100,101,102
    q, _ = orc.q_proj(x, wa, g, wb, pos, H=H, D=D, rope_dim=R, S=3)
    q0, _ = orc.q_proj(x1, wa, g, wb, np.array([0]), H=H, D=D, rope_dim=R)
    np.testing.assert_allclose(q[:, :, :D - R], np.broadcast_to(q0[:, :, :D - R], q[:, :, :D - R].shape),
                               rtol=0, atol=1e-14)
    t = np.array([5, 6, 7, 100, 101, 102])
    tail0 = q0[0, :, D - R:]
    pl = lambda a: np.hypot(a[..., 0::2], a[..., 1::2])
    np.testing.assert_allclose(pl(q[:, :, D - R:]), np.broadcast_to(pl(tail0), (6, H, R // 2)), rtol=1e-13)
    for i, j in [(0, 4), (2, 3), (1, 0), (5, 2)]:
        d, _ = orc.q_proj(x1, wa, g, wb, np.array([t[i] - t[j]]), H=H, D=D, rope_dim=R)
        lhs = np.sum(q[i, :, D - R:] * q[j, :, D - R:], axis=-1)
        rhs = np.sum(d[0, :, D - R:] * tail0, axis=-1)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    # position 0 leaves the tail as the head norm left it: unit RMS over the
    # whole head with the tail unrotated, i.e. equal to rope_dim=0 output
    qn, _ = orc.q_proj(x1, wa, g, wb, np.array([0]), H=H, D=D, rope_dim=0)
    np.testing.assert_allclose(q0, qn, rtol=0, atol=1e-15)


def test_o_proj_block_diagonal():
    """The grouped first stage equals one product with the block-diagonal
    matrix of the groups' weights (scipy's block_diag), heads taken in order,
    8 per group here."""
    rng = np.random.default_rng(5)
    M, H, D, G, orank, dm = 3, 16, 4, 2, 5, 7
    o = rng.standard_normal((M, H, D))
    wa = rng.standard_normal((G, orank, H * D // G))
    wb = rng.standard_normal((dm, G * orank))
    y, r = orc.o_proj(o, wa, wb, groups=G)
    bd = scipy.linalg.block_diag(*[wa[g] for g in range(G)])      # [G*orank, H*D]
    r_ref = o.reshape(M, H * D) @ bd.T
    np.testing.assert_allclose(r.reshape(M, -1), r_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y, r_ref @ wb.T, rtol=1e-12, atol=1e-12)


def test_o_proj_group_membership():
    """Output of head h reaches only group h // (H / groups)."""
    rng = np.random.default_rng(6)
    M, H, D, G, orank, dm = 1, 16, 4, 4, 3, 5
    wa = rng.standard_normal((G, orank, H * D // G))
    wb = np.eye(dm, G * orank)
    for h in (0, 3, 4, 9, 15):
        o = np.zeros((M, H, D))
        o[0, h] = rng.standard_normal(D)
        _, r = orc.o_proj(o, wa, wb, groups=G)
        nz = np.flatnonzero(np.any(r[0] != 0, axis=-1))
        assert list(nz) == [h // (H // G)]


def test_proj_bf16_store_bound():
    """Holding qr (or r) in bf16 moves it by at most half a bf16 ulp, 2^-9
    relative, and the outputs by no more than that error propagates."""
    rng = np.random.default_rng(7)
    M, dm, qrk, H, D = 4, 32, 24, 4, 16
    x = rng.standard_normal((M, dm))
    wa = rng.standard_normal((qrk, dm)) / np.sqrt(dm)
    wb = rng.standard_normal((H * D, qrk)) / np.sqrt(qrk)
    qa, qra = orc.q_proj(x, wa, np.ones(qrk), wb, np.zeros(M, dtype=np.int64), H=H, D=D, rope_dim=8)
    qb, qrb = orc.q_proj(x, wa, np.ones(qrk), wb, np.zeros(M, dtype=np.int64), H=H, D=D, rope_dim=8, store="bf16")
    assert np.all(np.abs(qrb - qra) <= np.abs(qra) * 2.0 ** -8 + 1e-300)
    assert np.any(qrb != qra)
    # |dq| <= |wb| |dqr| before the head norm; the norm is 1-Lipschitz-ish at unit scale
    assert np.max(np.abs(qb - qa)) < 50 * 2.0 ** -9
    o = rng.standard_normal((M, 8, 4))
    woa = rng.standard_normal((2, 6, 16))
    wob = rng.standard_normal((5, 12))
    ya, ra = orc.o_proj(o, woa, wob, groups=2)
    yb, rb = orc.o_proj(o, woa, wob, groups=2, store="bf16")
    assert np.all(np.abs(rb - ra) <= np.abs(ra) * 2.0 ** -8)
    assert np.any(rb != ra)
    np.testing.assert_allclose(yb, rb.reshape(M, -1) @ wob.T, rtol=1e-13)
