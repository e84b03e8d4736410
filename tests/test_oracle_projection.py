"""Pins of the projection oracle (low-rank query path, grouped output
projection) against facts the pages print and against independent
formulations (no GPU).  Source: "DeepSeek-V4-Flash 架构：一个 token 的旅程",
sections "低秩 Q：两次矩阵乘法接起来" and "输出投影也分组，并且降低中间维度"."""
import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import projection as P

Mi = 1 << 20
# the Flash model's widths as the two sections state them
D_MODEL, Q_RANK, HEADS, HEAD_DIM, GROUPS, O_RANK = 4096, 1024, 64, 512, 8, 1024


def test_parameter_counts_printed_on_the_page():
    """"两块权重共有 4096x1024 + 1024x32768 = 36 Mi 个参数。直接投影需要 128 Mi"
    and "每组包含 8 个头。第一段共 32 Mi 参数，第二段 32 Mi，共 64 Mi。...
    直接映射回 d 需要 128 Mi": the widths used here give exactly these counts."""
    wq_a, wq_b = (Q_RANK, D_MODEL), (HEADS * HEAD_DIM, Q_RANK)
    assert wq_a[0] * wq_a[1] + wq_b[0] * wq_b[1] == 36 * Mi
    assert D_MODEL * HEADS * HEAD_DIM == 128 * Mi               # a direct query projection
    heads_per_group = HEADS // GROUPS
    assert heads_per_group == 8
    wo_a = (GROUPS, O_RANK, HEADS * HEAD_DIM // GROUPS)
    wo_b = (D_MODEL, GROUPS * O_RANK)
    assert wo_a[2] == 4096                                       # o.reshape(B, S, groups, 4096)
    assert np.prod(wo_a) == 32 * Mi and np.prod(wo_b) == 32 * Mi
    assert HEADS * HEAD_DIM * D_MODEL == 128 * Mi                # all heads straight back to d


def test_out_proj_accepts_the_flash_shapes():
    """The oracle's operand layouts are the ones the counts above describe."""
    o = np.zeros((1, 1, HEADS, HEAD_DIM))
    wo_a = np.zeros((GROUPS, O_RANK, HEADS * HEAD_DIM // GROUPS))
    wo_b = np.zeros((D_MODEL, GROUPS * O_RANK))
    assert P.out_proj(o, wo_a, wo_b, GROUPS).shape == (1, 1, D_MODEL)
    x = np.zeros((2, D_MODEL))
    q = P.q_path(x + 1.0, np.ones((Q_RANK, D_MODEL)) / D_MODEL, np.ones(Q_RANK),
                 np.zeros((HEADS * HEAD_DIM, Q_RANK)), HEADS, HEAD_DIM, np.array([0, 5]), 64)
    assert q.shape == (2, HEADS, HEAD_DIM)


def _small_out_case(seed, H=16, D=8, G=4, R=32, d=7):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((3, H, D))
    wo_a = rng.standard_normal((G, R, H * D // G))
    wo_b = rng.standard_normal((d, G * R))
    return o, wo_a, wo_b, G


def test_grouped_projection_is_a_block_diagonal_matmul():
    """einsum("bsgd,grd->bsgr") over groups of consecutive heads equals one
    dense product with the block-diagonal matrix diag(wo_a[0], .., wo_a[G-1])
    applied to the flattened head outputs (scipy's block_diag, numpy matmul)."""
    o, wo_a, wo_b, G = _small_out_case(1)
    dense = scipy.linalg.block_diag(*wo_a)                       # (G*R, H*D)
    flat = o.reshape(o.shape[0], -1)
    r_dense = flat @ dense.T
    assert np.allclose(P.grouped_down(o, wo_a, G).reshape(o.shape[0], -1), r_dense, rtol=0, atol=1e-12)
    assert np.allclose(P.out_proj(o, wo_a, wo_b, G), r_dense @ wo_b.T, rtol=0, atol=1e-11)


def test_each_group_reads_only_its_own_heads():
    """"每组包含 8 个头": changing head h moves only the result of group
    h // (H/G); every other group's r is unchanged bit for bit."""
    o, wo_a, _, G = _small_out_case(2)
    H = o.shape[1]
    base = P.grouped_down(o, wo_a, G)
    for h in (0, 5, H - 1):
        o2 = o.copy()
        o2[1, h] += 1.0
        r = P.grouped_down(o2, wo_a, G)
        g = h // (H // G)
        for gg in range(G):
            same = np.array_equal(r[1, gg], base[1, gg])
            assert same == (gg != g), (h, gg)
        assert np.array_equal(r[0], base[0]) and np.array_equal(r[2], base[2])


def _small_q_case(seed, d=12, r=6, H=3, hd=8, rope=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((4, d))
    wq_a = rng.standard_normal((r, d)) / np.sqrt(d)
    gamma = 1 + 0.3 * rng.standard_normal(r)
    wq_b = rng.standard_normal((H * hd, r)) / np.sqrt(r)
    pos = np.array([0, 1, 7, 1000])
    return x, wq_a, gamma, wq_b, H, hd, pos, rope


def test_q_path_matches_torch_rms_norm_and_complex_rotation():
    """The whole query path through independent library routines in float64:
    torch's rms_norm for both normalisations (the latent with its gain, each
    head without one), torch matmuls, and RoPE as multiplication of the
    trailing channel pairs by e^{i pos theta} (torch complex numbers)."""
    x, wq_a, gamma, wq_b, H, hd, pos, rope = _small_q_case(3)
    eps = 1e-6
    tx = torch.from_numpy(x)
    qr = torch.nn.functional.rms_norm(tx @ torch.from_numpy(wq_a).T, (wq_a.shape[0],),
                                      weight=torch.from_numpy(gamma), eps=eps)
    q = (qr @ torch.from_numpy(wq_b).T).reshape(len(x), H, hd)
    q = torch.nn.functional.rms_norm(q, (hd,), eps=eps)
    theta = 10000.0 ** (-torch.arange(rope // 2, dtype=torch.float64) * 2 / rope)
    ang = torch.from_numpy(pos).double()[:, None, None] * theta
    tail = torch.view_as_complex(q[..., hd - rope:].reshape(len(x), H, rope // 2, 2).contiguous())
    tail = tail * torch.polar(torch.ones_like(ang), ang)
    want = torch.cat([q[..., :hd - rope], torch.view_as_real(tail).reshape(len(x), H, rope)], dim=-1)
    got = P.q_path(x, wq_a, gamma, wq_b, H, hd, pos, rope, eps=eps)
    assert np.allclose(got, want.numpy(), rtol=0, atol=1e-12)


def test_q_heads_have_unit_rms_and_rope_spares_the_leading_dims():
    """Every head is divided by its own RMS (closed form ms/(ms+eps) for the
    mean square, kept by the rotation), and the rotation touches the last
    rope_dim dims only: with pos = 0 nothing turns, and at any pos the
    leading dims equal the pos-0 values."""
    x, wq_a, gamma, wq_b, H, hd, pos, rope = _small_q_case(4)
    eps = 1e-3
    q = P.q_path(x, wq_a, gamma, wq_b, H, hd, pos, rope, eps=eps)
    q0 = P.q_path(x, wq_a, gamma, wq_b, H, hd, np.zeros_like(pos), rope, eps=eps)
    ms_rot = np.mean(q * q, axis=-1)
    assert np.allclose(ms_rot, np.mean(q0 * q0, axis=-1), rtol=0, atol=1e-12)
    pre = (P.csa.rms_norm(x @ wq_a.T, gamma, eps) @ wq_b.T).reshape(len(x), H, hd)
    ms = np.mean(pre * pre, axis=-1)
    assert np.allclose(ms_rot, ms / (ms + eps), rtol=1e-12, atol=0)
    assert np.array_equal(q[..., :hd - rope], q0[..., :hd - rope])
    assert not np.allclose(q[1:, :, hd - rope:], q0[1:, :, hd - rope:])


def test_low_rank_query_is_a_two_step_product():
    """With a unit gain and the identity as the second factor the path is
    the per-head normalisation of the RMS-normalised down-projection; a
    rank-1 input (every row of x a multiple of one vector) gives the same
    head directions for every token at position 0 (scale invariance of the
    two normalisations)."""
    rng = np.random.default_rng(5)
    d, r, H, hd = 10, 8, 2, 4
    v = rng.standard_normal(d)
    x = np.stack([v, 3.0 * v, 0.5 * v])
    wq_a = rng.standard_normal((r, d))
    q = P.q_path(x, wq_a, np.ones(r), np.eye(r), H, hd, np.zeros(3, int), 2, eps=0.0)
    assert np.allclose(q[1], q[0], atol=1e-12) and np.allclose(q[2], q[0], atol=1e-12)
    y = x[0] @ wq_a.T
    y = y / np.sqrt(np.mean(y * y))
    heads = y.reshape(H, hd)
    heads = heads / np.sqrt(np.mean(heads * heads, axis=-1, keepdims=True))
    assert np.allclose(q[0], heads, atol=1e-12)
