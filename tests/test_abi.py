"""The C ABI library (no GPU): it builds and loads, exports every symbol that
include/csa.h declares, and rejects invalid arguments on the host before any
HIP call.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

INVALID, UNSUPPORTED, WORKSPACE = -1, -2, -4
P = ctypes.c_void_p(0x10000)  # a non-null address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:csa|hca)_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import compressed_sparse_attention_06_amd as pkg
    if not os.path.exists(pkg.LIB_PATH):
        from compressed_sparse_attention_06_amd import build
        build.build()
    return pkg.lib()


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("csa_compress", "csa_index_score", "csa_topk", "csa_sparse_attn", "hca_attn"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from compressed_sparse_attention_06_amd._lib import SIGNATURES
    names = declared_functions()
    assert set(names) == set(SIGNATURES), "binding table and header disagree"
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.csa_status_string(0) == b"ok"
    assert lib.csa_status_string(-1) == b"invalid argument"
    assert lib.csa_status_string(-4) == b"workspace too small"
    assert lib.csa_status_string(7) == b"unknown status"
    assert lib.csa_version() >= 10000


def _compress(lib, **kw):
    a = dict(kv=P, gate=P, kv_prev=None, gate_prev=None, in_dtype=1, gamma=P, B=1, T=16, in_bstride=16 * 512,
             D=512, ratio=4, overlap=1, rope_dim=64, rope_base=10000.0, eps=1e-6, tok0=0, e0=0, n_entries=4,
             pos=None, out=P, out_dtype=0, out_bstride=4 * 512, out_cap=4, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.csa_compress(*a.values())


@pytest.mark.parametrize("bad", [
    dict(kv=None), dict(gate=None), dict(gamma=None), dict(out=None), dict(in_dtype=2), dict(out_dtype=-1),
    dict(ratio=0), dict(overlap=2), dict(rope_dim=63), dict(rope_dim=514), dict(eps=-1.0), dict(rope_base=0.0),
    dict(T=0), dict(B=-1), dict(in_bstride=100), dict(out_cap=3), dict(n_entries=5),
    dict(tok0=1),                                  # entry 0 needs token 0
    dict(e0=1, n_entries=3, tok0=1, T=15),         # entry 1 with overlap needs token 0
    dict(pos=P, T=7),                              # ring smaller than (1+overlap)*ratio
])
def test_compress_rejects(lib, bad):
    assert _compress(lib, **bad) == INVALID


def test_compress_workspace(lib):
    # short candidate lists, or many entries: one workgroup per entry, no workspace
    assert lib.csa_compress_workspace_size(8, 512, 4, 1) == 0
    assert lib.csa_compress_workspace_size(257, 512, 128, 0) == 0
    assert lib.csa_compress_workspace_size(4, 100, 128, 0) == 0      # one-wave path
    # 128 candidates of 4 entries: a fixed block of 256 arrival counters (the
    # same offset for every call shape), then 8 slices of (max, sum, weighted
    # sum) per channel and entry
    need = lib.csa_compress_workspace_size(4, 512, 128, 0)
    assert need == 1024 + 4 * 8 * 3 * 512 * 4
    assert lib.csa_compress_workspace_size(2, 128, 32, 1) == 1024 + 2 * 4 * 3 * 128 * 4
    assert lib.csa_compress_workspace_size(1, 512, 1024, 0) == 1024 + 1 * 16 * 3 * 512 * 4  # at most 16 slices
    assert lib.csa_compress_workspace_size(256, 512, 128, 0) == 1024 + 256 * 8 * 3 * 512 * 4
    long = dict(ratio=128, overlap=0, T=512, in_bstride=512 * 512)
    assert _compress(lib, **long) == WORKSPACE
    assert _compress(lib, **long, ws=P, ws_bytes=need - 1) == WORKSPACE
    assert _compress(lib, **long, ws=ctypes.c_void_p(0x10008), ws_bytes=need) == INVALID
    assert _compress(lib, **long, ws=P, ws_bytes=need, B=-1) == INVALID


def test_compress_job_layout_matches_header(tmp_path):
    """The binding's CompressJob has the size and field offsets of csa_compress_job."""
    import shutil
    import subprocess
    from compressed_sparse_attention_06_amd import build as B
    from compressed_sparse_attention_06_amd._lib import CompressJob
    if shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    fields = [f for f, _ in CompressJob._fields_]
    src = "#include <cstdio>\n#include <cstddef>\n#include \"csa.h\"\nint main() {\n"
    src += '  printf("%zu\\n", sizeof(csa_compress_job));\n'
    src += "".join(f'  printf("%zu\\n", offsetof(csa_compress_job, {f}));\n' for f in fields) + "  return 0;\n}\n"
    (tmp_path / "l.cpp").write_text(src)
    res = subprocess.run([B.HIPCC, "-I", os.path.join(B.ROOT, "include"), str(tmp_path / "l.cpp"), "-o",
                          str(tmp_path / "l")], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    got = [int(v) for v in subprocess.run([str(tmp_path / "l")], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(CompressJob)
    assert got[1:] == [getattr(CompressJob, f).offset for f in fields]


def test_compress_jobs_validation(lib):
    from compressed_sparse_attention_06_amd._lib import CompressJob
    good = dict(kv=P, gate=P, kv_prev=None, gate_prev=None, in_dtype=1, gamma=P, B=1, T=16, in_bstride=16 * 512,
                D=512, ratio=4, overlap=1, rope_dim=64, rope_base=10000.0, eps=1e-6, tok0=0, e0=0, n_entries=4,
                pos=None, out=P, out_dtype=0, out_bstride=4 * 512, out_cap=4, ws=None, ws_bytes=0)
    arr = (CompressJob * 3)(CompressJob(**good), CompressJob(**dict(good, ratio=0)), CompressJob(**good))
    assert lib.csa_compress_jobs(arr, 0, None) == 0                     # nothing to do
    assert lib.csa_compress_jobs(arr, -1, None) == INVALID
    assert lib.csa_compress_jobs(arr, 17, None) == INVALID              # above CSA_MAX_COMPRESS_JOBS
    assert lib.csa_compress_jobs(None, 2, None) == INVALID
    assert lib.csa_compress_jobs(arr, 3, None) == INVALID                # job 1 is invalid: nothing launches
    long = dict(good, ratio=128, overlap=0, T=512, in_bstride=512 * 512)
    arr2 = (CompressJob * 2)(CompressJob(**good), CompressJob(**long))
    assert lib.csa_compress_jobs(arr2, 2, None) == WORKSPACE             # the split job lacks its workspace


def test_compress_rejects_huge_rows(lib):
    assert _compress(lib, D=8200, rope_dim=64, in_bstride=16 * 8200, out_bstride=4 * 8200) == UNSUPPORTED


def _index(lib, **kw):
    a = dict(q=P, w=P, cache=P, dtype=1, pos=P, B=2, S=1, H=64, D=128, Ncap=1000, ratio=4, scores=P, stream=None)
    a.update(kw)
    return lib.csa_index_score(*a.values())


@pytest.mark.parametrize("bad", [dict(q=None), dict(w=None), dict(cache=None), dict(pos=None), dict(scores=None),
                                 dict(dtype=3), dict(H=0), dict(D=0), dict(Ncap=-1), dict(ratio=0), dict(B=-2)])
def test_index_score_rejects(lib, bad):
    assert _index(lib, **bad) == INVALID


def test_index_score_unsupported(lib):
    assert _index(lib, dtype=0, H=200, D=128) == UNSUPPORTED        # vector path limit
    assert _index(lib, Ncap=65535 * 256 + 1) == UNSUPPORTED


def test_topk_validation_and_workspace(lib):
    assert lib.csa_topk(None, None, 1, 10, 4, P, None, 0, None) == INVALID
    assert lib.csa_topk(P, None, 1, 10, 0, P, None, 0, None) == INVALID
    assert lib.csa_topk(P, None, 1, 10, 4097, P, None, 0, None) == INVALID
    # rows of at most one 16384-position tile: a single pass, no workspace
    assert lib.csa_topk_workspace_size(8192, 2048, 512) == 0
    assert lib.csa_topk_workspace_size(8, 16384, 512) == 0
    # longer rows: each 8192-position chunk keeps 512 candidates (two buffers of key + index)
    need = lib.csa_topk_workspace_size(32, 262144, 512)
    assert need == 2 * 32 * (262144 // 8192 * 512) * 8
    assert lib.csa_topk(P, None, 32, 262144, 512, P, P, need - 1, None) == WORKSPACE
    assert lib.csa_topk(P, None, 32, 262144, 512, P, None, need, None) == WORKSPACE


def test_topk_noalloc_validation(lib):
    """The no-allocation top-k validates like csa_topk and rejects calls whose
    chunk candidates exceed its 16 MiB static scratch (checked before any HIP
    call)."""
    from compressed_sparse_attention_06_amd import CSA_TOPK_NOALLOC_SCRATCH_BYTES
    assert CSA_TOPK_NOALLOC_SCRATCH_BYTES == 16 << 20
    assert lib.csa_topk_noalloc(None, None, 1, 10, 4, P, None) == INVALID
    assert lib.csa_topk_noalloc(P, None, 1, 10, 0, P, None) == INVALID
    assert lib.csa_topk_noalloc(P, None, 1, 10, 4097, P, None) == INVALID
    assert lib.csa_topk_noalloc(P, None, 1, 10, 4, None, None) == INVALID
    # 32 rows of 262,144 at k = 1024 need exactly the scratch; 64 such rows need twice it
    assert lib.csa_topk_workspace_size(32, 262144, 1024) == 16 << 20
    assert lib.csa_topk_noalloc(P, None, 64, 262144, 1024, P, None) == WORKSPACE
    assert lib.csa_topk_noalloc(P, None, 33, 262144, 1024, P, None) == WORKSPACE


def _attn(lib, **kw):
    a = dict(q=P, cmp=P, Ncap=1000, idx=P, k=512, win=P, Wcap=128, window=128, pos=P, sink=P, dtype=1, scale=0.04,
             rope_dim=64, rope_base=10000.0, B=8, S=1, H=64, D=512, out=P, out_dtype=0, ws=P, ws_bytes=1 << 40,
             stream=None)
    a.update(kw)
    return lib.csa_sparse_attn(*a.values())


@pytest.mark.parametrize("bad", [dict(q=None), dict(cmp=None), dict(idx=None), dict(pos=None), dict(sink=None),
                                 dict(out=None), dict(win=None), dict(Wcap=64), dict(window=-1), dict(k=-1),
                                 dict(rope_dim=65), dict(rope_dim=600), dict(dtype=5), dict(H=0),
                                 dict(scale=float("inf"))])
def test_sparse_attn_rejects(lib, bad):
    assert _attn(lib, **bad) == INVALID


def test_attn_workspace_sizes(lib):
    ws = lib.csa_sparse_attn_workspace_size(8, 1, 64, 512, 512, 128)
    assert ws > 0 and ws % (8 * 64 * (512 * 2 + 16)) == 0  # whole (query, split) partials: fp16 O/l, fp32 records
    # many queries: one persistent pass, one recompute flag per query
    assert lib.csa_sparse_attn_workspace_size(1, 8192, 64, 512, 512, 128) == 8192 * 4
    assert lib.csa_sparse_attn_workspace_size(1, 300, 64, 512, 512, 128) == 0  # one split per query
    assert lib.hca_attn_workspace_size(2, 4096, 64, 512, 64, 128) == 2 * 4096 * 4
    assert _attn(lib, ws=None, ws_bytes=0) == WORKSPACE
    assert _attn(lib, ws_bytes=ws - 1) == WORKSPACE
    assert _attn(lib, dtype=0, D=2048, H=64, rope_dim=64) == UNSUPPORTED
    hws = lib.hca_attn_workspace_size(4, 1, 64, 512, 8192, 128)
    assert hws > 0
    assert lib.hca_attn(P, P, 8192, 0, P, 128, 128, P, P, 1, 0.04, 64, 1e4, 4, 1, 64, 512, P, 0, P, hws, None) == INVALID
    assert lib.hca_attn(P, P, 8192, 128, P, 128, 128, P, P, 1, 0.04, 64, 1e4, 4, 1, 64, 512, P, 0, P, hws - 1,
                        None) == WORKSPACE


MIS = ctypes.c_void_p(0x10008)  # 8-byte but not 16-byte aligned


def test_misaligned_fast_shapes_are_rejected(lib):
    """The header requires 16-byte aligned tensors; on the matrix-core and
    lane-kernel shapes a misaligned pointer is an invalid argument (no slower
    fallback)."""
    for key in ("kv", "gate", "out", "kv_prev", "gate_prev"):
        assert _compress(lib, **{key: MIS}) == INVALID, key
    assert _compress(lib, in_bstride=16 * 512 + 4) == INVALID        # sequence starts off 16 bytes
    assert _compress(lib, out_bstride=4 * 512 + 2) == INVALID        # fp32 output: 8,200-byte stride
    for key in ("q", "cache", "scores"):
        assert _index(lib, **{key: MIS}) == INVALID, key
    for key in ("q", "cmp", "win", "out"):
        assert _attn(lib, **{key: MIS}) == INVALID, key
    hws = lib.hca_attn_workspace_size(4, 1, 64, 512, 8192, 128)
    assert lib.hca_attn(MIS, P, 8192, 128, P, 128, 128, P, P, 1, 0.04, 64, 1e4, 4, 1, 64, 512, P, 0, P, hws,
                        None) == INVALID


def _qproj(lib, **kw):
    a = dict(x=P, wq_a=P, gamma=P, wq_b=P, pos=P, M=8, d=4096, r=1024, H=64, hd=512, rope=64, base=10000.0,
             eps=1e-6, q=P, ws=P, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.csa_q_proj(*a.values())


def test_q_proj_validation(lib):
    # the first product runs in 16 K chunks of 256 (partials summed by the latent's norm), the second in one
    assert lib.csa_q_proj_workspace_size(8, 4096, 1024, 64, 512) == (16 * 8 * 1024 + 8 * 1024 + 8 * 64 * 512) * 4
    for bad in (dict(x=None), dict(wq_a=None), dict(gamma=None), dict(wq_b=None), dict(q=None), dict(pos=None),
                dict(rope=63), dict(rope=514), dict(eps=-1.0), dict(base=0.0), dict(M=-1), dict(H=0),
                dict(x=MIS), dict(wq_b=MIS), dict(q=MIS)):
        assert _qproj(lib, **bad) == INVALID, bad
    assert _qproj(lib, d=4000) == UNSUPPORTED          # K of the first product not a multiple of 128
    assert _qproj(lib, r=1000) == UNSUPPORTED
    assert _qproj(lib, ws_bytes=100) == WORKSPACE
    assert _qproj(lib, ws=None, ws_bytes=0) == WORKSPACE
    assert _qproj(lib, M=0, ws=None, ws_bytes=0) == 0   # nothing to do, nothing launched


def _oproj(lib, **kw):
    a = dict(o=P, o_dtype=1, wo_a=P, wo_b=P, M=8, H=64, hd=512, G=8, R=1024, d=4096, y=P, y_dtype=0, ws=P,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.csa_out_proj(*a.values())


def test_out_proj_validation(lib):
    # grouped product in 4 K chunks of 1024, the up-projection in 8 (its partials reduced into y)
    assert lib.csa_out_proj_workspace_size(8, 64, 512, 8, 1024, 4096, 1) == (4 * 8 * 8192 + 8 * 8 * 4096) * 4
    for bad in (dict(o=None), dict(wo_a=None), dict(wo_b=None), dict(y=None), dict(o_dtype=3), dict(y_dtype=7),
                dict(G=7), dict(M=-1), dict(o=MIS), dict(wo_b=MIS), dict(y=MIS)):
        assert _oproj(lib, **bad) == INVALID, bad
    assert _oproj(lib, R=1000) == UNSUPPORTED            # o_rank not a multiple of 16
    assert _oproj(lib, H=64, hd=500, G=8) == UNSUPPORTED  # 4000-wide groups: not a multiple of 128
    assert _oproj(lib, G=8, R=8) == UNSUPPORTED          # o_rank 8: not a multiple of 16
    assert _oproj(lib, G=8, R=24) == UNSUPPORTED         # 8 x 24 = 192: K of the second product off 128
    assert _oproj(lib, ws_bytes=100) == WORKSPACE


def test_calls_with_no_work_accept_null_pointers(lib):
    """A call with no work checks its scalar arguments, then returns ok without
    any HIP call (so it runs here); its pointers may be NULL, as torch passes
    for empty tensors.  Bad scalars are still rejected."""
    from compressed_sparse_attention_06_amd._lib import CompressJob, PageTableC
    none = dict(kv=None, gate=None, gamma=None, out=None)
    assert _compress(lib, B=0, **none) == 0
    assert _compress(lib, n_entries=0, **none) == 0                       # span mode, no entry to build
    hca = dict(ratio=128, overlap=0, T=128, in_bstride=128 * 512)       # a split plan: no workspace needed either
    assert _compress(lib, B=0, pos=P, **hca, **none) == 0
    assert _compress(lib, B=0, n_entries=4, **hca, **none) == 0          # an empty ring batch: torch's pos is NULL
    assert _compress(lib, B=0, ratio=0, **none) == INVALID
    assert _compress(lib, B=0, D=0, **none) == INVALID
    nul = dict(q=None, w=None, cache=None, pos=None, scores=None)
    assert _index(lib, B=0, **nul) == 0
    assert _index(lib, S=0, **nul) == 0
    assert _index(lib, Ncap=0, **nul) == 0
    assert _index(lib, B=0, ratio=0, **nul) == INVALID
    assert lib.csa_topk(None, None, 0, 10, 4, None, None, 0, None) == 0
    assert lib.csa_topk(None, None, 0, 262144, 512, None, None, 0, None) == 0   # no workspace for no row
    assert lib.csa_topk(None, None, 0, 10, 0, None, None, 0, None) == INVALID
    assert lib.csa_topk(None, None, 2, 0, 4, None, None, 0, None) == INVALID    # rows to fill need idx
    assert lib.csa_topk_noalloc(None, None, 0, 10, 4, None, None) == 0
    anul = dict(q=None, cmp=None, idx=None, win=None, pos=None, sink=None, out=None, ws=None, ws_bytes=0)
    assert _attn(lib, B=0, **anul) == 0
    assert _attn(lib, S=0, **anul) == 0
    assert _attn(lib, B=0, H=0, **anul) == INVALID
    assert lib.hca_attn(None, None, 8192, 128, None, 128, 128, None, None, 1, 0.04, 64, 1e4, 0, 1, 64, 512, None,
                        0, None, 0, None) == 0
    assert lib.hca_attn(None, None, 8192, 0, None, 128, 128, None, None, 1, 0.04, 64, 1e4, 0, 1, 64, 512, None,
                        0, None, 0, None) == INVALID
    assert lib.csa_kv4_quantize(None, 1, 0, 512, 64, None, None) == 0
    assert lib.csa_kv4_quantize(None, 1, 0, 500, 64, None, None) == INVALID
    assert _qproj(lib, M=0, x=None, wq_a=None, gamma=None, wq_b=None, pos=None, q=None, ws=None, ws_bytes=0) == 0
    assert _oproj(lib, M=0, o=None, wo_a=None, wo_b=None, y=None, ws=None, ws_bytes=0) == 0
    assert _oproj(lib, M=0, o=None, wo_a=None, wo_b=None, y=None, ws=None, ws_bytes=0, o_dtype=3) == INVALID
    # paged calls: an empty batch reads no page table, which may be absent
    assert lib.csa_index_score_paged(None, None, None, 1, None, 0, 1, 64, 128, None, 4, None, None) == 0
    assert lib.csa_index_score_paged(None, None, None, 1, None, 2, 1, 64, 128, None, 4, None, None) == INVALID
    assert lib.csa_sparse_attn_paged(None, None, None, None, 512, None, 128, 128, None, None, 1, 0.04, 64, 1e4,
                                     0, 1, 64, 512, None, 0, None, 0, None) == 0
    assert lib.hca_attn_paged(None, None, None, 128, None, 128, 128, None, None, 1, 0.04, 64, 1e4, 0, 1, 64, 512,
                              None, 0, None, 0, None) == 0
    job = CompressJob(None, None, None, None, 1, None, 0, 16, 16 * 512, 512, 4, 1, 64, 1e4, 1e-6, 0, 0, 0, P, None,
                      1, 0, 0, None, 0)
    tab = PageTableC(None, 0, 0, 0)
    assert lib.csa_compress_paged(ctypes.byref(job), ctypes.byref(tab), 1, None) == 0
    job.B = 2
    assert lib.csa_compress_paged(ctypes.byref(job), ctypes.byref(tab), 1, None) == INVALID
