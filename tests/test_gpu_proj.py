"""GPU parity of the projections on either side of the attention against the
float64 oracle ("DeepSeek-V4-Flash 架构：一个 token 的旅程", sections
"低秩 Q：两次矩阵乘法接起来" and "输出投影也分组，并且降低中间维度"), at the Flash
widths (d_model 4096, q_rank 1024, 64 heads of 512, 8 groups, o_rank 1024)
and at small widths with ragged token counts.

Tolerances: the queries are stored as bf16 (the attention reads them so):
each value within one bf16 ulp of the oracle's or within 1e-3 of its head's
largest value; the output projection (fp32) within 1e-3 normwise per token.
The products accumulate in fp32 from exact bf16 weights and inputs; fp32
intermediates enter the next product as a bf16 head plus remainder, so the
fp32 error sits near 1e-5, far inside these bounds."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import assert_bf16_matches, assert_normwise, dev, dev_bf16, host, progress

pytestmark = pytest.mark.gpu
f64 = synth.bf16_to_f64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_06_amd as csa
    csa.lib()


@pytest.fixture(autouse=True)
def _name(request):
    progress(request.node.nodeid)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def flash():
    return synth.proj_weights(90)


def _small_weights(seed, d, r, H, D, G, R):
    rng = np.random.default_rng(seed)
    w = lambda shape, fan: synth.bf16_bits((rng.standard_normal(shape) / np.sqrt(fan)).astype(np.float32))
    return dict(wq_a=w((r, d), d), gamma_q=(1 + 0.1 * rng.standard_normal(r)).astype(np.float32),
                wq_b=w((H * D, r), r), wo_a=w((G, R, H * D // G), H * D // G), wo_b=w((d, G * R), G * R))


def _check_q(x, wts, H, D, rope, pos, eps=1e-6):
    import compressed_sparse_attention_06_amd as csa
    M = x.shape[0]
    q = torch.empty((M, H, D), dtype=torch.bfloat16, device="cuda")
    csa.csa_q_proj(dev_bf16(x), dev_bf16(wts["wq_a"]), dev(wts["gamma_q"]), dev_bf16(wts["wq_b"]),
                   dev(pos.astype(np.int32)), q, rope_dim=rope, eps=eps)
    want = oracle.projection.q_path(f64(x), f64(wts["wq_a"]), wts["gamma_q"], f64(wts["wq_b"]), H, D, pos, rope,
                                    eps=eps)
    got = host(q)
    assert_bf16_matches(got.reshape(-1, D), want.reshape(-1, D), what="queries")
    return got


@pytest.mark.parametrize("M", [8, 1, 37])
def test_q_proj_flash_widths(flash, M):
    """Decode-sized token counts (one, eight, and a ragged 37 over three
    token tiles) at the Flash widths; positions up to 1M."""
    dims = synth.FLASH_PROJ
    x = synth.hidden_states(91, M, dims.d_model)
    pos = np.random.default_rng(M).integers(0, 1 << 20, M)
    pos[0] = 0
    _check_q(x, flash, 64, 512, 64, pos)


@pytest.mark.parametrize("M,d,r,H,D,rope", [(5, 256, 128, 2, 64, 16), (70, 128, 384, 3, 32, 8)])
def test_q_proj_small_widths(M, d, r, H, D, rope):
    wts = _small_weights(M, d, r, H, D, 1, 16)
    x = synth.bf16_bits(np.random.default_rng(M + 1).standard_normal((M, d)).astype(np.float32))
    _check_q(x, wts, H, D, rope, np.arange(M) * 7 + 3)


def _check_out(o_bits, o_dtype, wts, G, y_dtype=torch.float32):
    import compressed_sparse_attention_06_amd as csa
    M, H, D = o_bits.shape
    d = wts["wo_b"].shape[0]
    o = dev_bf16(o_bits) if o_dtype == "bf16" else dev(synth.bf16_to_f32(o_bits))
    y = torch.empty((M, d), dtype=y_dtype, device="cuda")
    csa.csa_out_proj(o, dev_bf16(wts["wo_a"]), dev_bf16(wts["wo_b"]), y)
    want = oracle.projection.out_proj(f64(o_bits), f64(wts["wo_a"]), f64(wts["wo_b"]), G)
    if y_dtype == torch.float32:
        assert_normwise(host(y), want, what="output projection")
    else:
        assert_bf16_matches(host(y), want, what="output projection (bf16)")


@pytest.mark.parametrize("M,o_dtype,y_dtype", [(8, "bf16", torch.float32), (4, "f32", torch.float32),
                                               (37, "bf16", torch.bfloat16)])
def test_out_proj_flash_widths(flash, M, o_dtype, y_dtype):
    """The attention output of M tokens (unit-RMS heads) through the grouped
    down-projection (8 groups of 8 heads) and the up-projection to 4096."""
    o = synth.bf16_bits(synth.unit_rms(np.random.default_rng(M + 50), (M, 64, 512)))
    _check_out(o, o_dtype, flash, 8, y_dtype)


def test_out_proj_small_widths():
    wts = _small_weights(3, 256, 128, 4, 64, 2, 64)
    o = synth.bf16_bits(synth.unit_rms(np.random.default_rng(4), (19, 4, 64)))
    _check_out(o, "bf16", wts, 2)


def test_projection_groups_see_only_their_heads(flash):
    """Zeroing the heads of one group changes the output exactly as the
    oracle's grouped product says (group g = heads 8g .. 8g+7)."""
    o = synth.bf16_bits(synth.unit_rms(np.random.default_rng(77), (3, 64, 512)))
    o[:, 16:24] = 0
    _check_out(o, "bf16", flash, 8)
