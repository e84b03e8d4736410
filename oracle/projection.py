"""Float64 CPU oracle of the projections on either side of the attention:
the low-rank query path and the grouped output projection.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it, and it imports nothing from the product path.

Source: "DeepSeek-V4-Flash 架构：一个 token 的旅程" (hs-black.github.io/posts/
deepseek-v4-flash/):

* section "低秩 Q：两次矩阵乘法接起来": the hidden state goes through a
  down-projection to a 1024-wide latent, an RMSNorm, an up-projection to
  64 heads of 512, a per-head RMS normalisation (no gain) and RoPE on the
  last 64 dims of every head at the token position.  The two weights hold
  4096x1024 + 1024x32768 = 36 Mi parameters.
* section "输出投影也分组，并且降低中间维度": after the inverse rotation the
  64 head outputs are cut into 8 groups of 8 heads (4096 wide each); every
  group has its own 1024x4096 down-projection (32 Mi parameters in all), the
  eight 1024-wide results are concatenated and one 4096x8192 matrix maps them
  to the model width (32 Mi).

Readings (the pages are silent): the latent's RMSNorm carries a learned gain
(the pseudo-code calls a normalisation layer, as the compressor's RMSNorm);
eps is 1e-6 for both norms and sits inside the square root; heads are
numbered so that group g holds heads 8g .. 8g+7 (the reshape of the head
axis in the pseudo-code); RoPE follows the same convention as the rest of
the path (interleaved pairs of the trailing slice, angle pos * base^(-2i/n)).
"""
from __future__ import annotations

import numpy as np

from . import csa


def q_path(x, wq_a, gamma_q, wq_b, heads, head_dim, pos, rope_dim, rope_base=10000.0, eps=1e-6):
    """Query heads of the tokens x, ready for the attention.

    ["低秩 Q：两次矩阵乘法接起来"]: ``qr = rms_norm(x @ wq_a.T)``, ``q = qr @
    wq_b.T`` viewed as ``heads`` heads of ``head_dim``, every head divided by
    its own root mean square, then RoPE on the last ``rope_dim`` dims of
    every head at the token's position.

    x: (..., d); wq_a: (r, d); gamma_q: (r,); wq_b: (heads*head_dim, r);
    pos: integer array of shape x.shape[:-1] (or a scalar).
    Returns (..., heads, head_dim).
    """
    x = np.asarray(x, dtype=np.float64)
    qr = csa.rms_norm(x @ np.asarray(wq_a, dtype=np.float64).T, gamma_q, eps)
    q = (qr @ np.asarray(wq_b, dtype=np.float64).T).reshape(*x.shape[:-1], heads, head_dim)
    q = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + eps)
    p = np.broadcast_to(np.asarray(pos)[..., None], q.shape[:-1])
    return csa.rope(q, p, rope_dim, rope_base)


def grouped_down(o, wo_a, groups):
    """First stage of the output projection: one down-projection per group.

    ["输出投影也分组，并且降低中间维度"]: ``o`` (..., H, D) -- the attention
    output after the inverse rotation -- is viewed as ``groups`` groups of
    H*D/groups values (heads h*groups/H .. in order), and
    ``r[..., g, :] = wo_a[g] @ o_group_g``, i.e. einsum("bsgd,grd->bsgr").

    wo_a: (groups, R, H*D/groups).  Returns (..., groups, R).
    """
    o = np.asarray(o, dtype=np.float64)
    lead = o.shape[:-2]
    og = o.reshape(*lead, groups, -1)
    return np.einsum("...gd,grd->...gr", og, np.asarray(wo_a, dtype=np.float64))


def out_proj(o, wo_a, wo_b, groups):
    """Whole output projection: grouped down-projection, then the shared
    up-projection of the concatenated group results.

    ["输出投影也分组，并且降低中间维度"]: ``y = r.flatten(-2) @ wo_b.T``.
    o: (..., H, D); wo_a: (groups, R, H*D/groups); wo_b: (d, groups*R).
    Returns (..., d).
    """
    r = grouped_down(o, wo_a, groups)
    return r.reshape(*r.shape[:-2], -1) @ np.asarray(wo_b, dtype=np.float64).T
