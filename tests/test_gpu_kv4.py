"""GPU parity of the quantised compressed-KV cache (FP4 E2M1 latent, FP8 E4M3
RoPE tail, one power-of-two scale per 32 channels; "Lab tổng hợp
DeepSeek-V4.1-Flash", section "3 Giải pháp") against the float64 oracle.

* csa_kv4_quantize of exact (bf16 / fp32) rows: bit-exact bytes -- the
  scaled values are exact in both precisions, so every rounding decision is
  the same.
* The compressor writing quantised entries: its fp32 entry differs from the
  oracle's float64 entry in the last bits, so codes may differ where the
  oracle's scaled value sits within 1e-5 relative of a rounding boundary (and
  a scale where the block maximum sits that close to a power of two); every
  other byte is equal.
* Attention over a quantised cache built by the oracle's quantiser: within
  max-abs 2e-2 / mean-abs 2e-3 of the oracle over the rows the bytes stand
  for (the device dequantises exactly to bf16), on the split, one-split and
  one-workgroup-per-query paths and the vector path.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import quant as Q
from tests.conftest import read_golden
from tests.gpu_util import assert_attn, dev, dev_bf16, host, progress

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


def _special_rows(rng, n, D):
    """Unit-RMS rows plus rows that hit the format's corners: an all-zero
    block, exact E2M1 midpoints, block maxima of exactly 6 * 2^k and 448 * 2^k,
    values that round to zero with either sign, large and tiny scales."""
    x = synth.unit_rms(rng, (n, D)).astype(np.float32)
    x[0, :32] = 0.0
    x[1, :16] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 2) * np.r_[np.ones(8), -np.ones(8)]
    x[2, :32] *= 0.0
    x[2, :32] += 6.0 * 2.0 ** -3
    x[3, D - 32:] = 448.0 * 2.0 ** -7
    x[4, 32:64] = np.r_[1e-4, -1e-4, 3.0, np.zeros(29)]
    x[5] *= 1000.0
    x[6] *= 1e-3
    return x


@pytest.mark.parametrize("D,rope,dtype", [(512, 64, "bf16"), (512, 64, "f32"), (96, 32, "f32"), (1024, 64, "bf16")])
def test_kv4_quantize_bit_exact(D, rope, dtype):
    import compressed_sparse_attention_06_amd as csa
    rng = np.random.default_rng(D + rope)
    x = _special_rows(rng, 37, D)
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        xin, x64 = dev_bf16(bits), f64(bits)
    else:
        xin, x64 = dev(x), x.astype(np.float64)
    rb = csa.csa_kv4_row_bytes(D, rope)
    assert rb == Q.row_bytes(D, rope)
    out = torch.full((37, rb), 0xAB, dtype=torch.uint8, device="cuda")
    csa.csa_kv4_quantize(xin, out, rope_dim=rope)
    got = out.cpu().numpy()
    for r in range(37):
        want = Q.quantize_row(x64[r], rope)
        assert np.array_equal(got[r], want), f"row {r}: bytes {np.nonzero(got[r] != want)[0][:8]}"


def test_kv4_hand_worked_row_on_the_gpu():
    """The hand-worked row of tests/golden/quant_row.txt, quantised on the GPU."""
    import compressed_sparse_attention_06_amd as csa
    g = read_golden("quant_row.txt")
    v = np.array([float(t) for t in g["values"]], dtype=np.float32)
    want = np.array([int(t, 16) for t in g["bytes"]], dtype=np.uint8)
    out = torch.empty((1, int(g["row_bytes"][0])), dtype=torch.uint8, device="cuda")
    csa.csa_kv4_quantize(dev(v[None]), out, rope_dim=int(g["rope_dim"][0]))
    assert np.array_equal(out.cpu().numpy()[0], want)


def _band_equal(got_row, want_entry, rope, what, rel=1e-5):
    """Bytes equal to the oracle's quantisation of its entry, except codes
    whose scaled oracle value lies within `rel` of a rounding boundary and
    scales whose block maximum lies within `rel` of a power of two."""
    D = want_entry.shape[-1]
    want = Q.quantize_row(want_entry, rope)
    if np.array_equal(got_row, want):
        return 0
    g_deq = Q.dequantize_row(got_row, D, rope)
    w_deq = Q.dequantize_row(want, D, rope)
    lat = D - rope
    for b0 in range(0, D, 32):
        blk = want_entry[b0:b0 + 32]
        fmax = 6.0 if b0 < lat else 448.0
        x = Q.block_scale_exp(blk, fmax)
        a = np.max(np.abs(blk))
        near_pow2 = abs(a / 2.0 ** x / fmax - 1) < rel or abs(a / 2.0 ** (x - 1) / fmax - 1) < rel
        diff = np.nonzero(g_deq[b0:b0 + 32] != w_deq[b0:b0 + 32])[0]
        if diff.size == 0:
            continue
        if near_pow2:
            continue
        vals = Q.e2m1_decode(np.arange(8)) if b0 < lat else np.unique(np.abs(Q._E4M3_VALUES))
        mids = (vals[1:] + vals[:-1]) / 2
        for i in diff:
            y = abs(blk[i]) / 2.0 ** x
            assert np.min(np.abs(mids - y)) <= rel * max(y, 1.0), \
                f"{what}: channel {b0 + i} code differs away from a rounding boundary"
    return 1


@pytest.mark.parametrize("mode", ["ring_csa", "ring_hca_split", "span_prefill"])
def test_compress_writes_kv4_entries(mode):
    import compressed_sparse_attention_06_amd as csa
    D, rope = 512, 64
    rng = np.random.default_rng(5)
    gamma = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    rb = csa.csa_kv4_row_bytes(D, rope)
    if mode == "span_prefill":
        B, T, r, ov, n = 1, 4 * 600, 4, 1, 600
        kv = synth.bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32))
        gate = synth.bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32))
        out = torch.zeros((B, n, rb), dtype=torch.uint8, device="cuda")
        csa.csa_compress(dev_bf16(kv), dev_bf16(gate), dev(gamma), out, ratio=r, overlap=ov, rope_dim=rope,
                         n_entries=n)
        got = out.cpu().numpy()
        wants = oracle.compress(f64(kv[0]), f64(gate[0]), gamma, r, ov, rope, n_entries=n)
        cases = [(0, e, wants[e]) for e in range(n)]
    else:
        r, ov = (4, 1) if mode == "ring_csa" else (128, 0)
        B, T = 6, (1 + ov) * r
        kv = synth.bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32))
        gate = synth.bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32))
        pos = np.array([(3 + b) * r - 1 for b in range(B)], np.int32)
        cap = 12
        out = torch.zeros((B, cap, rb), dtype=torch.uint8, device="cuda")
        csa.csa_compress(dev_bf16(kv), dev_bf16(gate), dev(gamma), out, ratio=r, overlap=ov, rope_dim=rope,
                         pos=dev(pos))
        got = out.cpu().numpy()
        cases = []
        for b in range(B):
            p = int(pos[b])
            e = p // r
            full_kv = np.zeros((p + 1, D)); full_g = np.zeros((p + 1, D))
            for t in range(p + 1 - T, p + 1):
                full_kv[t] = f64(kv[b, t % T]); full_g[t] = f64(gate[b, t % T])
            cases.append((b, e, oracle.compress_entry(e, full_kv, full_g, full_kv, full_g, gamma, r, ov, rope,
                                                      10000.0, 1e-6)))
    differing = sum(_band_equal(got[b, e], w, rope, f"{mode} b={b} e={e}") for b, e, w in cases)
    assert differing <= max(2, len(cases) // 20)


def _kv4_cache(seed, B, Ncap, D, rope):
    """A quantised cache built by the oracle's quantiser from unit-RMS rows;
    returns (device bytes, the float64 rows the bytes stand for)."""
    rows = synth.unit_rms(np.random.default_rng(seed), (B, Ncap, D)).astype(np.float64)
    rb = Q.row_bytes(D, rope)
    byts = np.zeros((B, Ncap, rb), dtype=np.uint8)
    deq = np.zeros((B, Ncap, D))
    for b in range(B):
        for e in range(Ncap):
            byts[b, e] = Q.quantize_row(rows[b, e], rope)
            deq[b, e] = Q.dequantize_row(byts[b, e], D, rope)
    return torch.from_numpy(byts).cuda(), deq


def _bf16_case(seed, B, S, H, D, Wcap):
    q = synth.bf16_bits(synth.unit_rms(np.random.default_rng(seed), (B, S, H, D)))
    win = synth.bf16_bits(synth.unit_rms(np.random.default_rng(seed + 1), (B, Wcap, D)))
    sink = np.random.default_rng(seed + 2).standard_normal(H).astype(np.float32)
    return q, win, sink


@pytest.mark.parametrize("path", ["csa_split", "hca_split", "csa_one_split", "csa_many", "vector"])
def test_attention_over_kv4_cache(path):
    import compressed_sparse_attention_06_amd as csa
    H, D, rope = (4, 96, 32) if path == "vector" else (64, 512, 64)
    Ncap, window, k = (48, 8, 8) if path == "vector" else (700, 128, 512)
    if path in ("csa_split", "hca_split", "vector"):
        B, S, Wcap = 2, 1, (16 if path == "vector" else 128)
        pos = np.array([[4 * Ncap + 3], [97]], np.int32) if path != "hca_split" else \
            np.array([[16 * Ncap + 5], [16 * 300 - 1]], np.int32)
    else:
        B, S = 1, (300 if path == "csa_one_split" else 600)
        Wcap = 4 * Ncap + S + 8
        pos = (np.arange(S) + 4 * Ncap - 200).astype(np.int32)[None]
    hca = path == "hca_split"
    r = 16 if hca else 4
    cache, deq = _kv4_cache(11, B, Ncap, D, rope)
    q, win, sink = _bf16_case(12, B, S, H, D, Wcap)
    sel = np.full((B, S, k), -1, np.int32)
    for b in range(B):
        for s_ in range(S):
            nv = min(oracle.visible(int(pos[b, s_]), r), Ncap)
            sel[b, s_] = synth.random_selection(13, nv, k, b=b, t=s_)
    scale = 1 / math.sqrt(D)
    out = torch.empty((B, S, H, D), dtype=torch.float32, device="cuda")
    if hca:
        csa.hca_attn(dev_bf16(q), cache, dev_bf16(win), dev(pos), dev(sink), out, ratio=r, window=window,
                     scale=scale, rope_dim=rope)
    else:
        csa.csa_sparse_attn(dev_bf16(q), cache, dev(sel), dev_bf16(win), dev(pos), dev(sink), out, window=window,
                            scale=scale, rope_dim=rope)
    got = host(out)
    checked = range(S) if S <= 8 else list(range(0, S, 37)) + [S - 1]
    for b in range(B):
        for s_ in checked:
            p = int(pos[b, s_])
            wr = np.stack([f64(win[b, pp % Wcap]) for pp in oracle.window_positions(p, window)])
            if hca:
                nv = min(oracle.visible(p, r), Ncap)
                want = oracle.hca_attn(f64(q[b, s_]), deq[b], nv, wr, sink, scale, p, rope)
            else:
                want = oracle.sparse_attn(f64(q[b, s_]), deq[b], sel[b, s_], wr, sink, scale, p, rope)
            assert_attn(got[b, s_], want, what=f"{path} b={b} s={s_}")
