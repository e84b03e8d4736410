"""GPU parity of paged, variable-length compressed caches ("LLM Atlas:
DeepSeek" §19: serving depends on the sequence-length mix and the page
allocator).  The same rows laid out in a shuffled page pool must give
bit-identical results to the contiguous layout wherever both take the same
kernel (addresses change, arithmetic does not); the persistent-kernel sizes,
which the paged layout serves with one workgroup per query, are checked
against the oracle.  Unused pool pages hold large values, so a read through a
wrong table entry shows up."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
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


def _paginate(cache, rows_used, page_rows, seed, spare_pages=5):
    """A shuffled page pool holding cache[b, :rows_used[b]] and its table;
    pages not used by any sequence hold large values."""
    B, Ncap, W = cache.shape
    max_pages = Ncap // page_rows
    need = [(int(n) + page_rows - 1) // page_rows for n in rows_used]
    n_pool = sum(need) + spare_pages
    order = np.random.default_rng(seed).permutation(n_pool)
    table = np.full((B, max_pages), -1, np.int32)
    k = 0
    for b in range(B):
        for j in range(need[b]):
            table[b, j] = order[k]
            k += 1
    if cache.dtype == torch.uint8:
        pool = torch.full((n_pool * page_rows, W), 0x7E, dtype=torch.uint8, device="cuda")
    else:
        pool = torch.full((n_pool * page_rows, W), 1000.0, dtype=cache.dtype, device="cuda")
    for b in range(B):
        rows = min(need[b] * page_rows, Ncap)
        dst = (torch.from_numpy(table[b, :need[b]]).long()[:, None] * page_rows + torch.arange(page_rows)).view(-1)
        pool[dst[:rows].cuda()] = cache[b, :rows]
    return pool, dev(table), table


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("page_rows,long", [(256, False), (64, False), (128, True)])
def test_paged_index_scores_match_contiguous(page_rows, long):
    """Short caches take the streaming kernel, long ones (2M rows and more in
    all) the balanced persistent one, paged or not."""
    import compressed_sparse_attention_06_amd as csa
    B, Ncap = (4, 1 << 20) if long else (4, 4096)
    rng = np.random.default_rng(1)
    vis = np.array([Ncap, 1000, 300, 2049]) if not long else np.array([Ncap, 700_001, 17, 262_144])
    pos = dev((4 * vis - 1).astype(np.int32)[:, None])
    qi = dev_bf16(synth.bf16_bits(synth.unit_rms(rng, (B, 1, 64, 128))))
    w = dev((rng.standard_normal((B, 1, 64)) / 128 ** 0.5 / 8).astype(np.float32))
    if long:  # (512 MiB of rows: drawn on the device from a seeded generator)
        gen = torch.Generator(device="cuda").manual_seed(1)
        cache = torch.randn((B, Ncap, 128), generator=gen, device="cuda").to(torch.bfloat16)
    else:
        cache = dev_bf16(synth.bf16_bits(synth.unit_rms(rng, (B, Ncap, 128))))
    want = torch.empty((B, 1, Ncap), device="cuda")
    csa.csa_index_score(qi, w, cache, pos, want, ratio=4)
    pool, table, _ = _paginate(cache, vis, page_rows, 2)
    got = torch.full((B, 1, Ncap), 7.0, device="cuda")
    csa.csa_index_score_paged(qi, w, pool, pos, got, table, page_rows=page_rows, ratio=4)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    # and the oracle on the first and last visible rows of one sequence
    b = 1
    rows = np.r_[0:min(2048, vis[b]), max(vis[b] - 2048, 0):vis[b]]
    o = oracle.index_score(host(qi)[b, 0], host(w)[b, 0], host(cache[b, torch.from_numpy(rows).cuda()]), len(rows))
    g = got[b, 0].cpu().numpy()
    assert np.all(np.isneginf(g[vis[b]:]))
    assert np.max(np.abs(g[rows] - o)) <= 1e-3 * np.max(np.abs(o))


def _attn_inputs(seed, B, S, Ncap, kv4, window=128, Wcap=128):
    import compressed_sparse_attention_06_amd as csa
    rng = np.random.default_rng(seed)
    q = dev_bf16(synth.bf16_bits(synth.unit_rms(rng, (B, S, 64, 512))))
    win = dev_bf16(synth.bf16_bits(synth.unit_rms(rng, (B, Wcap, 512))))
    sink = dev(rng.standard_normal(64).astype(np.float32))
    rows = dev_bf16(synth.bf16_bits(synth.unit_rms(rng, (B, Ncap, 512))))
    if kv4:
        q4 = torch.empty((B, Ncap, csa.csa_kv4_row_bytes(512, 64)), dtype=torch.uint8, device="cuda")
        csa.csa_kv4_quantize(rows, q4, rope_dim=64)
        rows = q4
    return q, win, sink, rows


@pytest.mark.parametrize("kind,kv4", [("csa_split", False), ("hca_split", False), ("csa_one_split", False),
                                      ("csa_split", True), ("hca_split", True)])
def test_paged_attention_matches_contiguous(kind, kv4):
    import compressed_sparse_attention_06_amd as csa
    page_rows, Ncap = 256, 2048
    hca = kind.startswith("hca")
    r = 16 if hca else 4
    if kind == "csa_one_split":
        B, S = 1, 300
        Wcap = 4 * Ncap + S
        pos = (np.arange(S) + 4 * 1500).astype(np.int32)[None]
    else:
        B, S, Wcap = 3, 1, 128
        pos = (np.array([[2048], [700], [130]]) * r - 1).astype(np.int32)
    vis = np.minimum((pos.max(axis=1) + 1) // r, Ncap)
    q, win, sink, rows = _attn_inputs(3, B, S, Ncap, kv4, Wcap=Wcap)
    sel = np.full((B, S, 512), -1, np.int32)
    for b in range(B):
        for s_ in range(S):
            sel[b, s_] = synth.random_selection(4, min((int(pos[b, s_]) + 1) // r, Ncap), 512, b=b, t=s_)
    scale = 1 / math.sqrt(512)
    pool, table, _ = _paginate(rows, vis, page_rows, 5)
    want = torch.empty((B, S, 64, 512), device="cuda")
    got = torch.full((B, S, 64, 512), 7.0, device="cuda")
    if hca:
        csa.hca_attn(q, rows, win, dev(pos), sink, want, ratio=r, window=128, scale=scale, rope_dim=64)
        csa.hca_attn_paged(q, pool, table, win, dev(pos), sink, got, page_rows=page_rows, ratio=r, window=128,
                           scale=scale, rope_dim=64)
    else:
        csa.csa_sparse_attn(q, rows, dev(sel), win, dev(pos), sink, want, window=128, scale=scale, rope_dim=64)
        csa.csa_sparse_attn_paged(q, pool, table, dev(sel), win, dev(pos), sink, got, page_rows=page_rows,
                                  window=128, scale=scale, rope_dim=64)
    torch.cuda.synchronize()
    assert torch.equal(got, want), f"max diff {float((got - want).abs().max())}"


def test_paged_prefill_attention_against_the_oracle():
    """600 queries: the contiguous layout takes the persistent kernel, the
    paged one a workgroup per query; sampled queries against the oracle."""
    import compressed_sparse_attention_06_amd as csa
    page_rows, Ncap, B, S = 128, 2048, 1, 600
    Wcap = 8192
    pos = (np.arange(S) + 7000).astype(np.int32)[None]
    vis = np.array([Ncap])
    q, win, sink, rows = _attn_inputs(6, B, S, Ncap, False, Wcap=Wcap)
    sel = np.stack([synth.random_selection(7, min(oracle.visible(int(pos[0, s_]), 4), Ncap), 512, b=0, t=s_)
                    for s_ in range(S)])[None]
    pool, table, _ = _paginate(rows, vis, page_rows, 8)
    got = torch.empty((B, S, 64, 512), device="cuda")
    scale = 1 / math.sqrt(512)
    csa.csa_sparse_attn_paged(q, pool, table, dev(sel), win, dev(pos), sink, got, page_rows=page_rows, window=128,
                              scale=scale, rope_dim=64)
    torch.cuda.synchronize()
    g = host(got)
    qh, wh, rh, sk = host(q), host(win), host(rows), sink.cpu().numpy()
    for s_ in (0, 1, 299, 599):
        p = int(pos[0, s_])
        wr = np.stack([wh[0, pp % Wcap] for pp in oracle.window_positions(p, 128)])
        want = oracle.sparse_attn(qh[0, s_], rh[0], sel[0, s_], wr, sk, scale, p, 64)
        assert_attn(g[0, s_], want, what=f"query {s_}")


@pytest.mark.parametrize("kv4", [False, True])
def test_paged_compress_append_matches_contiguous(kv4):
    import compressed_sparse_attention_06_amd as csa
    B, D, r, page_rows, Ncap = 4, 512, 4, 64, 512
    rng = np.random.default_rng(9)
    kv = dev_bf16(synth.bf16_bits(rng.standard_normal((B, 2 * r, D)).astype(np.float32)))
    gate = dev_bf16(synth.bf16_bits(rng.standard_normal((B, 2 * r, D)).astype(np.float32)))
    gamma = dev((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    # entries 63 and 64 straddle a page boundary; one sequence emits nothing
    ent = np.array([63, 64, 300, 17])
    pos = (ent * r + r - 1).astype(np.int32)
    pos[3] += 1
    row_w = csa.csa_kv4_row_bytes(D, 64) if kv4 else D
    dt = torch.uint8 if kv4 else torch.bfloat16
    cont = torch.zeros((B, Ncap, row_w), dtype=dt, device="cuda")
    csa.csa_compress(kv, gate, gamma, cont, ratio=r, overlap=1, rope_dim=64, pos=dev(pos))
    pool, table, tab = _paginate(torch.zeros_like(cont), ent + 1, page_rows, 10)
    csa.csa_compress_paged(kv, gate, gamma, pool, table, page_rows=page_rows, ratio=r, overlap=1, rope_dim=64,
                           pos=dev(pos))
    torch.cuda.synchronize()
    for b in range(B):
        e = int(ent[b])
        row = int(tab[b, e // page_rows]) * page_rows + e % page_rows
        if b == 3:
            assert torch.equal(_bits(pool[row]), _bits(torch.zeros_like(pool[row])))   # no emission
        else:
            assert torch.equal(_bits(pool[row]), _bits(cont[b, e])), f"b={b}"


def test_paged_compress_hca_ring_matches_contiguous():
    """HCA's ratio-128 groups (the split compressor: partial pools merged by
    the last workgroup of each entry) appending into pages."""
    import compressed_sparse_attention_06_amd as csa
    B, D, r, page_rows, Ncap = 5, 512, 128, 64, 256
    rng = np.random.default_rng(12)
    kv = dev_bf16(synth.bf16_bits(rng.standard_normal((B, r, D)).astype(np.float32)))
    gate = dev_bf16(synth.bf16_bits(rng.standard_normal((B, r, D)).astype(np.float32)))
    gamma = dev((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    ent = np.array([0, 63, 64, 200, 255])
    pos = (ent * r + r - 1).astype(np.int32)
    cont = torch.zeros((B, Ncap, D), dtype=torch.bfloat16, device="cuda")
    csa.csa_compress(kv, gate, gamma, cont, ratio=r, overlap=0, rope_dim=64, pos=dev(pos))
    pool, table, tab = _paginate(torch.zeros_like(cont), ent + 1, page_rows, 13)
    csa.csa_compress_paged(kv, gate, gamma, pool, table, page_rows=page_rows, ratio=r, overlap=0, rope_dim=64,
                           pos=dev(pos))
    torch.cuda.synchronize()
    for b in range(B):
        e = int(ent[b])
        row = int(tab[b, e // page_rows]) * page_rows + e % page_rows
        assert torch.equal(_bits(pool[row]), _bits(cont[b, e])), f"b={b}"


@pytest.mark.parametrize("e0", [0, 37])
def test_paged_compress_span_matches_contiguous(e0):
    """A prefill span of 300 entries starting at entry e0 written into pages
    of 64 rows (crossing several page boundaries) equals the contiguous
    span, and no row outside it is written."""
    import compressed_sparse_attention_06_amd as csa
    B, D, r, page_rows, n = 1, 512, 4, 64, 300
    Ncap = 512
    rng = np.random.default_rng(14)
    tok0 = max(e0 - 1, 0) * r               # the chunk starts with the group before entry e0
    T = (e0 + n) * r - tok0
    kv = dev_bf16(synth.bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32)))
    gate = dev_bf16(synth.bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32)))
    gamma = dev((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    # the overlap role's own rows of the same tokens
    kvp = dev_bf16(synth.bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32)))
    gp = dev_bf16(synth.bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32)))
    cont = torch.zeros((B, Ncap, D), dtype=torch.bfloat16, device="cuda")
    csa.csa_compress(kv, gate, gamma, cont, ratio=r, overlap=1, rope_dim=64, tok0=tok0, e0=e0, n_entries=n,
                     kv_prev=kvp, gate_prev=gp)
    pool, table, tab = _paginate(torch.zeros_like(cont), [e0 + n], page_rows, 15)
    before = pool.clone()
    csa.csa_compress_paged(kv, gate, gamma, pool, table, page_rows=page_rows, ratio=r, overlap=1, rope_dim=64,
                           tok0=tok0, e0=e0, n_entries=n, kv_prev=kvp, gate_prev=gp)
    torch.cuda.synchronize()
    written = torch.zeros(pool.shape[0], dtype=torch.bool, device="cuda")
    for e in range(e0, e0 + n):
        row = int(tab[0, e // page_rows]) * page_rows + e % page_rows
        written[row] = True
        assert torch.equal(_bits(pool[row]), _bits(cont[0, e])), f"entry {e}"
    assert torch.equal(_bits(pool[~written]), _bits(before[~written]))


def test_paged_decode_steps_with_the_page_pool():
    """Sequences of different lengths grow through several decode steps, the
    page allocator adding a page whenever a sequence's next entry crosses into
    one; every step (append both caches, score, top-k, attention) matches the
    contiguous layout bit for bit."""
    import compressed_sparse_attention_06_amd as csa
    B, D, DI, r, page_rows, Ncap, k = 3, 512, 128, 4, 64, 512, 64
    rng = np.random.default_rng(11)
    ents = np.array([62, 127, 10])            # entries present before the first step
    pool_pages = 3 * (Ncap // page_rows)
    alloc = csa.PagePool(pool_pages)
    tab = np.full((B, Ncap // page_rows), -1, np.int32)
    for b in range(B):
        alloc.reserve(tab[b], page_rows, int(ents[b]))
    kv_pool = torch.full((pool_pages * page_rows, D), 1000.0, dtype=torch.bfloat16, device="cuda")
    ix_pool = torch.full((pool_pages * page_rows, DI), 1000.0, dtype=torch.bfloat16, device="cuda")
    kv_c = torch.zeros((B, Ncap, D), dtype=torch.bfloat16, device="cuda")
    ix_c = torch.zeros((B, Ncap, DI), dtype=torch.bfloat16, device="cuda")
    for b in range(B):                        # the same initial rows in both layouts
        rows = dev_bf16(synth.bf16_bits(synth.unit_rms(rng, (int(ents[b]), D))))
        irows = dev_bf16(synth.bf16_bits(synth.unit_rms(rng, (int(ents[b]), DI))))
        kv_c[b, :ents[b]] = rows
        ix_c[b, :ents[b]] = irows
        for e in range(int(ents[b])):
            pr = int(tab[b, e // page_rows]) * page_rows + e % page_rows
            kv_pool[pr] = rows[e]
            ix_pool[pr] = irows[e]
    gamma = dev((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    gamma_i = dev((1 + 0.1 * rng.standard_normal(DI)).astype(np.float32))
    sink = dev(rng.standard_normal(64).astype(np.float32))
    win = dev_bf16(synth.bf16_bits(synth.unit_rms(rng, (B, 128, D))))
    scale = 1 / math.sqrt(D)
    t = ents * r                               # next token of each sequence
    for step in range(12):
        progress(f"paged decode step {step}")
        # the page of the entry this token may complete must exist before the append
        for b in range(B):
            alloc.reserve(tab[b], page_rows, int(t[b] // r) + 1)
        table = dev(tab)
        pos = dev(t.astype(np.int32))
        n_vis = dev(((t + 1) // r).astype(np.int32))
        stg = [dev_bf16(synth.bf16_bits(rng.standard_normal((B, 2 * r, d)).astype(np.float32))) for d in (D, D, DI, DI)]
        qi = dev_bf16(synth.bf16_bits(synth.unit_rms(rng, (B, 1, 64, DI))))
        w = dev((rng.standard_normal((B, 1, 64)) / 128 ** 0.5 / 8).astype(np.float32))
        q = dev_bf16(synth.bf16_bits(synth.unit_rms(rng, (B, 1, 64, D))))
        outs = []
        for paged in (False, True):
            if paged:
                # both appends in one launch
                common = dict(pages=table, page_rows=page_rows, ratio=r, overlap=1, rope_dim=64, pos=pos)
                csa.csa_compress_paged_jobs([dict(kv=stg[0], gate=stg[1], gamma=gamma, pool=kv_pool, **common),
                                             dict(kv=stg[2], gate=stg[3], gamma=gamma_i, pool=ix_pool, **common)])
            else:
                csa.csa_compress(stg[0], stg[1], gamma, kv_c, ratio=r, overlap=1, rope_dim=64, pos=pos)
                csa.csa_compress(stg[2], stg[3], gamma_i, ix_c, ratio=r, overlap=1, rope_dim=64, pos=pos)
            sc = torch.empty((B, 1, Ncap), device="cuda")
            if paged:
                csa.csa_index_score_paged(qi, w, ix_pool, pos.view(B, 1), sc, table, page_rows=page_rows, ratio=r)
            else:
                csa.csa_index_score(qi, w, ix_c, pos.view(B, 1), sc, ratio=r)
            sel = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
            csa.csa_topk(sc.view(B, Ncap), n_vis, k, sel.view(B, k))
            o = torch.empty((B, 1, 64, D), device="cuda")
            if paged:
                csa.csa_sparse_attn_paged(q, kv_pool, table, sel, win, pos.view(B, 1), sink, o, page_rows=page_rows,
                                          window=128, scale=scale, rope_dim=64)
            else:
                csa.csa_sparse_attn(q, kv_c, sel, win, pos.view(B, 1), sink, o, window=128, scale=scale, rope_dim=64)
            outs.append((sc, sel, o))
        torch.cuda.synchronize()
        for a_, b_ in zip(outs[0], outs[1]):
            assert torch.equal(a_, b_), f"step {step}"
        t += 1
    # the pool hands out exactly the pages the sequences' lengths need
    need = sum((int(tt) // r + 1 + page_rows - 1) // page_rows for tt in t - 1)
    assert alloc.available() == pool_pages - need


def test_paged_pages_outside_the_pool_are_skipped():
    """Table entries that are not pages of the pool (-1, or past its end)
    are never read or written: an attended row on such a page is left out
    (the same result as the contiguous layout with that selection removed),
    an HCA query attends only the rows whose pages exist (the oracle over
    those rows), an append into such a page writes nothing, and the indexer
    still scores every row of the valid pages exactly."""
    import compressed_sparse_attention_06_amd as csa
    page_rows, Ncap, B = 256, 2048, 2
    q, win, sink, rows = _attn_inputs(21, B, 1, Ncap, False)
    pos = np.array([[2048 * 4 - 1], [1500 * 4 - 1]], np.int32)
    vis = np.array([2048, 1500])
    pool, table, tab = _paginate(rows, vis, page_rows, 22)
    bad = tab.copy()
    bad[0, 3] = -1                       # entries 768 .. 1023 of sequence 0
    bad[1, 1] = pool.shape[0] // page_rows + 5   # entries 256 .. 511 of sequence 1: past the pool
    bad_t = dev(bad)
    dropped = [lambda e: 768 <= e < 1024, lambda e: 256 <= e < 512]
    sel = np.stack([synth.random_selection(23, int(vis[b]), 512, b=b) for b in range(B)])[:, None]
    sel_c = sel.copy()
    for b in range(B):
        sel_c[b, 0] = [e if e >= 0 and not dropped[b](e) else -1 for e in sel[b, 0]]
    scale = 1 / math.sqrt(512)
    want = torch.empty((B, 1, 64, 512), device="cuda")
    got = torch.empty((B, 1, 64, 512), device="cuda")
    csa.csa_sparse_attn(q, rows, dev(sel_c), win, dev(pos), sink, want, window=128, scale=scale, rope_dim=64)
    csa.csa_sparse_attn_paged(q, pool, bad_t, dev(sel), win, dev(pos), sink, got, page_rows=page_rows, window=128,
                              scale=scale, rope_dim=64)
    torch.cuda.synchronize()
    assert torch.equal(got, want)

    # HCA (ratio 16): the rows of the missing pages are left out
    hpos = np.array([[2048 * 16 - 1], [1500 * 16 - 1]], np.int32)
    out = torch.empty((B, 1, 64, 512), device="cuda")
    csa.hca_attn_paged(q, pool, bad_t, win, dev(hpos), sink, out, page_rows=page_rows, ratio=16, window=128,
                       scale=scale, rope_dim=64)
    torch.cuda.synchronize()
    g, qh, rh, wh, sk = host(out), host(q), host(rows), host(win), sink.cpu().numpy()
    for b in range(B):
        p = int(hpos[b, 0])
        keep = np.array([e for e in range(int(vis[b])) if not dropped[b](e)])
        wr = np.stack([wh[b, pp % 128] for pp in oracle.window_positions(p, 128)])
        w_ = oracle.sparse_attn(qh[b, 0], rh[b], keep, wr, sk, scale, p, 64)
        assert_attn(g[b, 0], w_, what=f"hca b={b}")

    # an append whose page is missing writes nothing
    D, r = 512, 4
    rng = np.random.default_rng(24)
    kv = dev_bf16(synth.bf16_bits(rng.standard_normal((B, 2 * r, D)).astype(np.float32)))
    gate = dev_bf16(synth.bf16_bits(rng.standard_normal((B, 2 * r, D)).astype(np.float32)))
    gamma = dev(np.ones(D, np.float32))
    apos = dev(np.array([800 * r + r - 1, 300 * r + r - 1], np.int32))   # entries 800 (b=0), 300 (b=1)
    before = pool.clone()
    csa.csa_compress_paged(kv, gate, gamma, pool, bad_t, page_rows=page_rows, ratio=r, overlap=1, rope_dim=64,
                           pos=apos)
    torch.cuda.synchronize()
    assert torch.equal(_bits(pool), _bits(before))

    # the indexer: rows of valid pages scored exactly as in the contiguous layout
    rngi = np.random.default_rng(25)
    qi = dev_bf16(synth.bf16_bits(synth.unit_rms(rngi, (B, 1, 64, 128))))
    w = dev((rngi.standard_normal((B, 1, 64)) / 128 ** 0.5 / 8).astype(np.float32))
    icache = dev_bf16(synth.bf16_bits(synth.unit_rms(rngi, (B, Ncap, 128))))
    ipool, itable, itab = _paginate(icache, vis, page_rows, 26)
    ibad = itab.copy()
    ibad[0, 3] = -1
    ibad[1, 1] = ipool.shape[0] // page_rows + 5
    sw = torch.empty((B, 1, Ncap), device="cuda")
    sg = torch.empty((B, 1, Ncap), device="cuda")
    csa.csa_index_score(qi, w, icache, dev(pos), sw, ratio=4)
    csa.csa_index_score_paged(qi, w, ipool, dev(pos), sg, dev(ibad), page_rows=page_rows, ratio=4)
    torch.cuda.synchronize()
    for b in range(B):
        ok = np.array([not dropped[b](e) for e in range(Ncap)])
        assert torch.equal(sg[b, 0][torch.from_numpy(ok).cuda()], sw[b, 0][torch.from_numpy(ok).cuda()])
        assert torch.isfinite(sg[b, 0][torch.from_numpy(~ok).cuda()][: int(vis[b])]).all()


@pytest.mark.parametrize("kind,kv4,k", [("csa", True, 512), ("hca", False, 0), ("csa", False, 1024)])
def test_paged_many_queries_against_the_oracle(kind, kv4, k):
    """Prefill-sized calls on paged caches (one workgroup per query, the
    persistent kernel being for contiguous bf16 caches): a quantised pool, HCA
    over every visible row, and the Pro model's top-k 1024; sampled queries
    against the oracle on the rows the pool holds (dequantised for the
    quantised pool)."""
    import compressed_sparse_attention_06_amd as csa
    page_rows, Ncap, S = 128, 2048, 520
    hca = kind == "hca"
    r = 16 if hca else 4
    pos = (np.arange(S) + (r * Ncap - 300 if hca else 4 * 1800)).astype(np.int32)[None]
    Wcap = 4 * Ncap * (4 if hca else 1) + S + 8
    vis = np.array([min((int(pos[0, -1]) + 1) // r, Ncap)])
    q, win, sink, rows = _attn_inputs(31, 1, S, Ncap, False, Wcap=Wcap)
    rows64 = host(rows)[0]
    if kv4:
        rb = csa.csa_kv4_row_bytes(512, 64)
        q4 = torch.empty((1, Ncap, rb), dtype=torch.uint8, device="cuda")
        csa.csa_kv4_quantize(rows, q4, rope_dim=64)
        bytes_ = q4.cpu().numpy()[0]
        from oracle import quant as Q
        rows64 = np.stack([Q.dequantize_row(bytes_[e], 512, 64) for e in range(Ncap)])
        rows = q4
    pool, table, _ = _paginate(rows, vis, page_rows, 32)
    out = torch.empty((1, S, 64, 512), device="cuda")
    scale = 1 / math.sqrt(512)
    if hca:
        csa.hca_attn_paged(q, pool, table, win, dev(pos), sink, out, page_rows=page_rows, ratio=r, window=128,
                           scale=scale, rope_dim=64)
        sel = None
    else:
        sel = np.stack([synth.random_selection(33, min(oracle.visible(int(pos[0, s_]), r), Ncap), k, b=0, t=s_)
                        for s_ in range(S)])[None]
        csa.csa_sparse_attn_paged(q, pool, table, dev(sel), win, dev(pos), sink, out, page_rows=page_rows,
                                  window=128, scale=scale, rope_dim=64)
    torch.cuda.synchronize()
    g, qh, wh, sk = host(out), host(q), host(win), sink.cpu().numpy()
    for s_ in (0, 1, 257, S - 1):
        p = int(pos[0, s_])
        wr = np.stack([wh[0, pp % Wcap] for pp in oracle.window_positions(p, 128)])
        if hca:
            want = oracle.hca_attn(qh[0, s_], rows64, min(oracle.visible(p, r), Ncap), wr, sk, scale, p, 64)
        else:
            want = oracle.sparse_attn(qh[0, s_], rows64, sel[0, s_], wr, sk, scale, p, 64)
        assert_attn(g[0, s_], want, what=f"{kind} query {s_}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_vector_paths_match_contiguous(dtype):
    """Shapes off the matrix cores (4 heads of 96, a 2 x 16 indexer, 96-wide
    compressed rows) take the vector kernels, which translate rows through
    the table one entry at a time: bit-identical to the contiguous layout."""
    import compressed_sparse_attention_06_amd as csa
    B, Ncap, page_rows, D, H, DI, HI = 2, 256, 64, 96, 4, 16, 2
    rng = np.random.default_rng(41)

    def t(x):
        return dev_bf16(synth.bf16_bits(x)) if dtype == "bf16" else dev(x.astype(np.float32))

    vis = np.array([256, 150])
    pos = np.array([[4 * 256 - 1], [4 * 150 - 1]], np.int32)
    # indexer
    qi = t(synth.unit_rms(rng, (B, 1, HI, DI)))
    w = dev((rng.standard_normal((B, 1, HI)) / 4).astype(np.float32))
    icache = t(synth.unit_rms(rng, (B, Ncap, DI)))
    ipool, itable, _ = _paginate(icache, vis, page_rows, 42)
    sw = torch.empty((B, 1, Ncap), device="cuda")
    sg = torch.empty((B, 1, Ncap), device="cuda")
    csa.csa_index_score(qi, w, icache, dev(pos), sw, ratio=4)
    csa.csa_index_score_paged(qi, w, ipool, dev(pos), sg, itable, page_rows=page_rows, ratio=4)
    # attention, CSA and HCA
    q = t(synth.unit_rms(rng, (B, 1, H, D)))
    win = t(synth.unit_rms(rng, (B, 8, D)))
    sink = dev(rng.standard_normal(H).astype(np.float32))
    rows = t(synth.unit_rms(rng, (B, Ncap, D)))
    pool, table, _ = _paginate(rows, vis, page_rows, 43)
    sel = np.stack([synth.random_selection(44, int(vis[b]), 32, b=b) for b in range(B)])[:, None]
    scale = 1 / math.sqrt(D)
    outs = []
    for paged in (False, True):
        o1 = torch.empty((B, 1, H, D), device="cuda")
        o2 = torch.empty((B, 1, H, D), device="cuda")
        if paged:
            csa.csa_sparse_attn_paged(q, pool, table, dev(sel), win, dev(pos), sink, o1, page_rows=page_rows, window=8,
                                      scale=scale, rope_dim=32)
            csa.hca_attn_paged(q, pool, table, win, dev(pos), sink, o2, page_rows=page_rows, ratio=4, window=8,
                               scale=scale, rope_dim=32)
        else:
            csa.csa_sparse_attn(q, rows, dev(sel), win, dev(pos), sink, o1, window=8, scale=scale, rope_dim=32)
            csa.hca_attn(q, rows, win, dev(pos), sink, o2, ratio=4, window=8, scale=scale, rope_dim=32)
        outs.append((o1, o2))
    # compressor (a 96-wide row is not a multiple of 128: the one-wave path)
    kv = t(rng.standard_normal((B, 8, D)))
    gate = t(rng.standard_normal((B, 8, D)))
    gamma = dev((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    apos = dev(np.array([63 * 4 + 3, 64 * 4 + 3], np.int32))       # entries 63 and 64: two pages
    cont = torch.zeros((B, Ncap, D), dtype=rows.dtype, device="cuda")
    csa.csa_compress(kv, gate, gamma, cont, ratio=4, overlap=1, rope_dim=32, pos=apos)
    cpool, ctable, ctab = _paginate(torch.zeros_like(cont), np.array([64, 65]), page_rows, 45)
    csa.csa_compress_paged(kv, gate, gamma, cpool, ctable, page_rows=page_rows, ratio=4, overlap=1, rope_dim=32,
                           pos=apos)
    torch.cuda.synchronize()
    assert torch.equal(sg, sw)
    for a_, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a_, b_)
    for b, e in ((0, 63), (1, 64)):
        row = int(ctab[b, e // page_rows]) * page_rows + e % page_rows
        assert torch.equal(_bits(cpool[row]), _bits(cont[b, e]))
