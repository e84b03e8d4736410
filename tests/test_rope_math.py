"""The kernels' RoPE angle (csrc/rope_math.h), compiled for the host with g++
and checked against 80-bit extended precision on the CPU.

The angle of pair i at position p is p * base^(-2i/rope_dim), reduced into
[-pi, pi] ("DeepSeek-V4-Flash 架构：一个 token 的旅程", section "压缩是逐通道的
learned pooling": the trailing channels carry the position)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from compressed_sparse_attention_06_amd import build as B

SRC = r'''
#include <cstdio>
#include <cstdlib>
#include "rope_math.h"
int main(int argc, char** argv) {
  double x;
  long long p;
  int i, rd;
  double l2b;
  char kind;
  while (std::scanf(" %c", &kind) == 1) {
    if (kind == 'e') {
      std::scanf("%lf", &x);
      std::printf("%.17g\n", csa::exp2_taylor(x));
    } else {
      std::scanf("%lld %d %d %lf", &p, &i, &rd, &l2b);
      std::printf("%.17g\n", csa::rope_angle(p, i, rd, l2b));
    }
  }
  return 0;
}
'''


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("rope")
    (d / "t.cpp").write_text(SRC)
    exe = d / "t"
    res = subprocess.run(["g++", "-O2", "-ffp-contract=off", "-I", B.CSRC, str(d / "t.cpp"), "-o", str(exe)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def _run(exe, lines):
    out = subprocess.run([str(exe)], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
    return np.array([float(v) for v in out.stdout.split()])


def test_exp2_taylor_accuracy(prog):
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.uniform(-40, 40, 400), np.arange(-30, 31) + 0.5, [0.0, -1e-300, 1e-12, -0.4999999]])
    got = _run(prog, [f"e {float(x)!r}" for x in xs])
    ref = np.exp2(xs.astype(np.longdouble))
    rel = np.abs((got.astype(np.longdouble) - ref) / ref)
    assert float(rel.max()) < 4e-16, float(rel.max())
    # exact powers of two stay exact
    ints = np.arange(-20, 21).astype(float)
    assert np.array_equal(_run(prog, [f"e {float(x)!r}" for x in ints]), np.exp2(ints))


def test_rope_angle_reduction(prog):
    rng = np.random.default_rng(6)
    base = 10000.0
    l2b = float(np.log2(np.longdouble(base)))
    rows = []
    for p in [0, 1, 7, 127, 4096, 65535, 524287, 1048575, 1048576 + 4096]:
        for i in [0, 1, 5, 16, 31]:
            rows.append((p, i, 64))
    for _ in range(200):
        rows.append((int(rng.integers(0, 1 << 21)), int(rng.integers(0, 64)), 128))
    got = _run(prog, [f"r {p} {i} {rd} {l2b!r}" for p, i, rd in rows])
    two_pi = 2 * np.pi if not hasattr(np, "longdouble") else np.longdouble("6.28318530717958647692528676655900577")
    for (p, i, rd), a in zip(rows, got):
        theta = np.exp2(np.longdouble(-2.0) * i / rd * np.log2(np.longdouble(base)))
        x = np.longdouble(p) * theta
        ref = x - np.rint(x / two_pi) * two_pi
        assert -np.pi - 1e-9 <= a <= np.pi + 1e-9
        # same point on the circle within 1e-9 rad (positions up to 2^21)
        d = float(np.remainder(np.longdouble(a) - ref + two_pi / 2, two_pi) - two_pi / 2)
        assert abs(d) < 1e-9, (p, i, rd, a, float(ref))
