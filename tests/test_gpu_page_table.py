"""GPU parity of the decodes over page tables (mla_decode_mxfp4_page_table,
mla_decode_fp8_page_table, mla_decode_bf16_page_table) against the fp64
page-table oracle, through the C ABI, and bit-identity with the row-list
decodes reading the same rows. Same bar as the contiguous decodes."""

import math
import sys

import numpy as np
import pytest
import torch

from mla_mxfp4_kv_amd import binding, synth
from oracle import dense_ref as dref
from oracle import mxfp4_ref as ref
from oracle import paging_ref as pref

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(576.0)
ATOL = 1e-2
RTOL = 1e-2
NORMWISE = 5e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    yield


def _qbits(q):
    return q.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _check(got, want, label):
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan_w), f"{label}: NaN pattern differs"
    g, w = got[~nan_w], want[~nan_w]
    err = np.abs(g - w)
    assert np.all(err <= ATOL + RTOL * np.abs(w)), f"{label}: max err {float(err.max()):.3e}"
    den = np.linalg.norm(w)
    if den > 0:
        nw = np.linalg.norm(g - w) / den
        assert nw <= NORMWISE, f"{label}: normwise {nw:.3e}"


def _table(lens, ps, seed, extra=2):
    """A page table for sequences of `lens` tokens: page offsets, valid rows
    of each last page, and the pool slot of every page (random, over
    `extra` times as many slots as pages)."""
    npages = [(n + ps - 1) // ps for n in lens]
    pi = np.concatenate([[0], np.cumsum(npages)]).astype(np.int64)
    last = [n - (p - 1) * ps if p else 0 for n, p in zip(lens, npages)]
    slots = max(1, extra * int(pi[-1]))
    pages = np.random.default_rng(seed).permutation(slots)[: int(pi[-1])].astype(np.int32)
    return pi, last, pages, slots


def _fill(pool, cache, indptr, pi, pages, ps, lens):
    """Copy each sequence's contiguous rows into its pages of the pool."""
    for b, n in enumerate(lens):
        lo = int(indptr[b])
        for j in range((n + ps - 1) // ps):
            used = min(ps, n - j * ps)
            r0 = int(pages[int(pi[b]) + j]) * ps
            pool[r0:r0 + used] = cache[lo + j * ps:lo + j * ps + used]


def _case(fmt, lens, ps, seed):
    pi, last, pages, slots = _table(lens, ps, seed)
    rows = slots * ps
    rng = np.random.default_rng(seed + 1)
    w = synth.Workload("p", len(lens), None, None, 1.0, False, seed)
    if fmt == "mxfp4":
        q, packed, scales, indptr, _ = synth.make_inputs(w, lengths=lens)
        pool = (torch.from_numpy(rng.integers(0, 256, (rows, 288), dtype=np.uint8)),
                torch.from_numpy(rng.integers(118, 136, (rows, 18), dtype=np.uint8)))
        _fill(pool[0], packed, indptr, pi, pages, ps, lens)
        _fill(pool[1], scales, indptr, pi, pages, ps, lens)
        scale = None
    else:
        q, cache, scale, indptr, _ = synth.make_dense_inputs(w, fmt, lengths=lens)
        if fmt == "fp8":
            p = torch.from_numpy(rng.integers(0, 0x7E, (rows, 576), dtype=np.uint8))
        else:
            p = torch.randn(rows, 576, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
        _fill(p, cache, indptr, pi, pages, ps, lens)
        pool = (p,)
    return q, pool, scale, indptr, pi, last, pages


def _oracle(fmt, q, pool, scale, pi, last, pages, ps, batches=None):
    qb = _qbits(q)
    if fmt == "mxfp4":
        return ref.mla_decode_ref_page_table(qb, pool[0].numpy(), pool[1].numpy(), pages, pi, last, ps, SM,
                                             batches=batches)
    if fmt == "fp8":
        return dref.mla_decode_ref_fp8_page_table(qb, pool[0].numpy(), float(scale[0]), pages, pi, last, ps,
                                                  SM, batches=batches)
    bits = pool[0].view(torch.int16).numpy().view(np.uint16)
    return dref.mla_decode_ref_bf16_page_table(qb, bits, pages, pi, last, ps, SM, batches=batches)


def _run(dec, fmt, q, pool, scale, pages, **kw):
    if fmt == "mxfp4":
        return dec.mxfp4(q, pool[0], pool[1], pages, sm_scale=SM, **kw)
    if fmt == "fp8":
        return dec.fp8(q, pool[0], scale, pages, sm_scale=SM, **kw)
    return dec.bf16(q, pool[0], pages, sm_scale=SM, **kw)


def _run_rows(fmt, indptr, q, pool, scale, rows, num_cus):
    dec = binding.MlaDecode(indptr, device="cuda", num_cus=num_cus)
    if fmt == "mxfp4":
        return dec.mxfp4_paged(q, pool[0], pool[1], rows, sm_scale=SM)
    if fmt == "fp8":
        return dec.fp8_paged(q, pool[0], scale, rows, sm_scale=SM)
    return dec.bf16_paged(q, pool[0], rows, sm_scale=SM)


# (lengths, page size, CUs the plan is spread over; 0 = the device's)
CASES = [
    ([1], 16, 0),
    ([31, 32, 33], 16, 0),
    ([127, 128, 129], 7, 3),
    ([0, 300, 0, 1000], 64, 0),
    ([5000], 16, 0),
    ([1, 1, 1, 1, 700], 1, 7),
    ([257, 4097, 33, 2000], 32, 0),
    ([100, 200], 100, 2),
]


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8", "bf16"])
@pytest.mark.parametrize("lens,ps,num_cus", CASES)
def test_page_table_matches_oracle(fmt, lens, ps, num_cus):
    """Element-wise against the page-table oracle, and bit for bit against
    the row-list decode of the same rows (the same kernels read the same
    bytes in the same order)."""
    _say(f"case page table {fmt} lens={lens} page_size={ps} num_cus={num_cus}")
    q, pool, scale, indptr, pi, last, pages = _case(fmt, lens, ps, seed=sum(lens) + ps)
    dec = binding.MlaDecodePageTable(pi.tolist(), last, ps, device="cuda", num_cus=num_cus)
    assert dec.kv_indptr.cpu().tolist() == indptr.tolist()
    qd = q.cuda()
    dpool = tuple(p.cuda() for p in pool)
    dscale = scale.cuda() if scale is not None else None
    out = _run(dec, fmt, qd, dpool, dscale, torch.from_numpy(pages).cuda())
    torch.cuda.synchronize()
    _check(out.float().cpu().numpy(), _oracle(fmt, q, pool, scale, pi, last, pages, ps), f"{fmt} {lens} ps={ps}")
    rows = np.concatenate(pref.page_table_rows(pages, pi, last, ps) + [np.zeros(0, np.int64)])
    rows = torch.from_numpy(rows.astype(np.int32)).cuda()
    same = _run_rows(fmt, indptr.tolist(), qd, dpool, dscale, rows, num_cus)
    torch.cuda.synchronize()
    assert torch.equal(out, same), f"{fmt} {lens} ps={ps}: page table and row list differ"


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8"])
def test_b256_kv8192_in_16_row_pages(fmt):
    """B=256, kv=8192 with every sequence in shuffled 16-row pages: bit
    identical to the row-list decode of the same rows, and every sequence
    against the oracle."""
    w = synth.WORKLOADS["b256_kv8192"]
    ps = 16
    _say(f"case page table b256_kv8192 {fmt}: generating")
    if fmt == "mxfp4":
        q, packed, scales, indptr, lens = synth.make_inputs(w, device="cuda")
        cache = (packed, scales)
        scale = None
    else:
        q, c, scale, indptr, lens = synth.make_dense_inputs(w, fmt, device="cuda")
        cache = (c,)
    t = int(indptr[-1])
    npages = t // ps
    assert t % ps == 0 and all(int(n) % ps == 0 for n in lens)
    g = torch.Generator(device="cpu").manual_seed(7)
    pages = torch.randperm(npages, generator=g).to(torch.int32).cuda()
    rows = (pages.long().repeat_interleave(ps) * ps + torch.arange(ps, device="cuda").repeat(npages))
    pool = tuple(torch.empty_like(x) for x in cache)
    for p, x in zip(pool, cache):
        p[rows] = x
    pi = [int(v) // ps for v in indptr]
    last = [ps if int(n) else 0 for n in lens]
    dec = binding.MlaDecodePageTable(pi, last, ps, device="cuda")
    _say(f"case page table b256_kv8192 {fmt}: decode")
    out = _run(dec, fmt, q, pool, scale, pages)
    same = _run_rows(fmt, indptr.tolist(), q, pool, scale, rows.to(torch.int32), 0)
    torch.cuda.synchronize()
    assert torch.equal(out, same)
    got = out.float().cpu().numpy()
    qb = _qbits(q)
    host = [x.cpu().numpy() for x in cache]
    for b in range(len(lens)):
        lo, hi = int(indptr[b]), int(indptr[b + 1])
        if fmt == "mxfp4":
            want = ref.mla_decode_ref_seq(qb[b], host[0][lo:hi], host[1][lo:hi], w.sm_scale)
        else:
            want = dref.mla_decode_ref_fp8_seq(qb[b], host[0][lo:hi], float(scale[0]), w.sm_scale)
        _check(got[b], want, f"b256 page table {fmt} b={b}")


def test_graph_replays_page_table_decode():
    """The page-table decode captured in a HIP graph (host plan, checks done
    before capture) replays to the eager result, with eager work between
    the replays."""
    _say("case page table graph replay")
    lens, ps = [300, 0, 1500, 77], 16
    q, pool, scale, indptr, pi, last, pages = _case("mxfp4", lens, ps, seed=41)
    dec = binding.MlaDecodePageTable(pi.tolist(), last, ps, device="cuda", num_cus=5)
    qd, dpool, dpages = q.cuda(), tuple(p.cuda() for p in pool), torch.from_numpy(pages).cuda()
    out = torch.empty(len(lens), 16, 512, dtype=torch.bfloat16, device="cuda")
    eager = _run(dec, "mxfp4", qd, dpool, None, dpages, out=out).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        _run(dec, "mxfp4", qd, dpool, None, dpages, out=out, stream=s, check=False)   # warm the stream
        s.synchronize()
        with torch.cuda.graph(graph, stream=s):
            _run(dec, "mxfp4", qd, dpool, None, dpages, out=out, stream=s, check=False)
    torch.cuda.synchronize()
    for k in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {k}"


def test_page_table_errors():
    _say("case page table errors")
    lens, ps = [40], 16
    q, pool, scale, indptr, pi, last, pages = _case("mxfp4", lens, ps, seed=3)
    dec = binding.MlaDecodePageTable(pi.tolist(), last, ps, device="cuda")
    qd, dpool, dpages = q.cuda(), tuple(p.cuda() for p in pool), torch.from_numpy(pages).cuda()
    with pytest.raises(ValueError):   # a page past the pool
        _run(dec, "mxfp4", qd, dpool, None, dpages + 1000)
    with pytest.raises(ValueError):   # fewer pages than the offsets say
        _run(dec, "mxfp4", qd, dpool, None, dpages[:1])
    out = torch.empty(1, 16, 512, dtype=torch.bfloat16, device="cuda")
    ptr = lambda t: binding.ctypes.c_void_p(t.data_ptr())
    L = binding.lib()
    args = (ptr(qd), ptr(dpool[0]), ptr(dpool[1]), ptr(dpages))
    tail = (ptr(dec.kv_indptr), ptr(out), SM, ptr(dec.plan.workspace), None)
    assert L.mla_decode_mxfp4_page_table(*args, ptr(dec.page_indptr), 0, *tail) == -1   # page size 0
    assert L.mla_decode_mxfp4_page_table(*args, None, ps, *tail) == -1                  # no page offsets
    assert L.mla_decode_mxfp4_page_table(*args[:3], None, ptr(dec.page_indptr), ps, *tail) == -1
    assert L.mla_decode_mxfp4_page_table(*args, ptr(dec.page_indptr), ps, *tail) == 0
    torch.cuda.synchronize()


def test_growing_page_table_replayed_in_a_graph():
    """A serving loop: the GPU-side plan and the page-table decode captured
    once in a HIP graph, then replayed while every sequence grows by one
    token per step (crossing page boundaries, new pages taken from a free
    list) and the tables are rewritten in place between replays. Each
    replay equals the eager decode of the same state through a host plan."""
    _say("case page table growing in a graph")
    ps, batch, steps = 16, 4, 6
    start = [15, 31, 1, 40]            # sequences 0 and 1 cross a page boundary on step 1
    max_tokens = sum(start) + batch * steps
    slots = 64
    rng = np.random.default_rng(11)
    pool_p = torch.from_numpy(rng.integers(0, 256, (slots * ps, 288), dtype=np.uint8)).cuda()
    # scales 2^-5..2^0 keep the scores of random codes moderate (larger ones
    # make softmax pick single tokens, where the tolerance is too tight)
    pool_s = torch.from_numpy(rng.integers(122, 128, (slots * ps, 18), dtype=np.uint8)).cuda()
    free = list(rng.permutation(slots))
    owned = [[] for _ in range(batch)]

    def tables(lens):
        for b, n in enumerate(lens):
            while len(owned[b]) * ps < n:
                owned[b].append(int(free.pop()))
        pi = np.concatenate([[0], np.cumsum([len(o) for o in owned])])
        last = [n - (len(o) - 1) * ps for n, o in zip(lens, owned)]
        pages = np.concatenate([np.array(o, dtype=np.int32) for o in owned])
        return pi, last, pages

    q = torch.randn(batch, 16, 576, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).cuda()
    max_pages = (max_tokens + batch * ps) // ps
    dev = binding.MlaDecodeDevicePlan(batch, max_tokens, device="cuda", num_cus=6)
    d_pages = torch.zeros(max_pages, dtype=torch.int32, device="cuda")
    d_pi = torch.zeros(batch + 1, dtype=torch.int32, device="cuda")
    d_tok = torch.zeros(batch + 1, dtype=torch.int32, device="cuda")
    out = torch.empty(batch, 16, 512, dtype=torch.bfloat16, device="cuda")

    def upload(lens):
        pi, last, pages = tables(lens)
        d_pages[: len(pages)].copy_(torch.from_numpy(pages))
        d_pi.copy_(torch.from_numpy(pi.astype(np.int32)))
        tok = binding.page_table_kv_indptr(pi.tolist(), last, ps)
        d_tok.copy_(torch.tensor(tok, dtype=torch.int32))
        torch.cuda.synchronize()
        return pi, last

    lens = list(start)
    upload(lens)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        dev.plan(d_tok, stream=s)
        dev.decode_page_table("mxfp4", q, pool_p, pool_s, d_pages, d_pi, ps, d_tok, out, sm_scale=SM, stream=s)
        s.synchronize()
        with torch.cuda.graph(graph, stream=s):
            dev.plan(d_tok, stream=s)
            dev.decode_page_table("mxfp4", q, pool_p, pool_s, d_pages, d_pi, ps, d_tok, out, sm_scale=SM,
                                  stream=s)
    torch.cuda.synchronize()
    for step in range(steps):
        lens = [n + 1 for n in lens]
        pi, last = upload(lens)
        out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        host = binding.MlaDecodePageTable(pi.tolist(), last, ps, device="cuda", num_cus=6)
        want = host.mxfp4(q, pool_p, pool_s, d_pages[: int(pi[-1])].contiguous(), sm_scale=SM)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"step {step}"
    # the last state against the oracle
    exp = ref.mla_decode_ref_page_table(_qbits(q), pool_p.cpu().numpy(), pool_s.cpu().numpy(),
                                        d_pages[: int(pi[-1])].cpu().numpy(), pi, last, ps, SM)
    _check(out.float().cpu().numpy(), exp, "growing page table, last step")


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8"])
def test_rows_at_the_top_of_the_largest_pool(fmt):
    """Row lists and page tables reading the last rows of the largest pool
    the 32-bit offsets allow (pool bytes just under 2^32) give the same bits
    as the contiguous decode of those rows."""
    row_bytes = 288 if fmt == "mxfp4" else 576
    ps = 16
    rows_max = (2 ** 32 - 1) // row_bytes // ps * ps          # whole pages, pool below 2^32 bytes
    assert rows_max * row_bytes < 2 ** 32
    lens = [70, 33]
    _say(f"case largest pool {fmt}: {rows_max} rows")
    w = synth.Workload("top", len(lens), None, None, 1.0, False, 9)
    if fmt == "mxfp4":
        q, packed, scales, indptr, _ = synth.make_inputs(w, lengths=lens)
        cache = (packed.cuda(), scales.cuda())
        scale = None
    else:
        q, c, scale, indptr, _ = synth.make_dense_inputs(w, fmt, lengths=lens)
        cache = (c.cuda(),)
        scale = scale.cuda()
    q = q.cuda()
    total = int(indptr[-1])
    # sequence b's pages are the last pages of the pool, in reverse order
    npages = [(n + ps - 1) // ps for n in lens]
    pi = np.concatenate([[0], np.cumsum(npages)])
    pages = np.arange(rows_max // ps - 1, rows_max // ps - 1 - int(pi[-1]), -1).astype(np.int32)
    last = [n - (p - 1) * ps for n, p in zip(lens, npages)]
    rows = np.concatenate(pref.page_table_rows(pages, pi, last, ps)).astype(np.int64)
    assert rows.min() >= 0 and rows.max() <= rows_max - 1 and rows.max() >= rows_max - ps
    pool = [torch.empty((rows_max,) + tuple(x.shape[1:]), dtype=x.dtype, device="cuda") for x in cache]
    ridx = torch.from_numpy(rows).cuda()
    for p, x in zip(pool, cache):
        p[ridx] = x
    plain = binding.MlaDecode(indptr.tolist(), device="cuda")
    if fmt == "mxfp4":
        want = plain(q, cache[0], cache[1], sm_scale=SM).clone()
        by_rows = plain.mxfp4_paged(q, pool[0], pool[1], ridx.to(torch.int32), sm_scale=SM).clone()
    else:
        want = plain.fp8(q, cache[0], scale, sm_scale=SM).clone()
        by_rows = plain.fp8_paged(q, pool[0], scale, ridx.to(torch.int32), sm_scale=SM).clone()
    dec = binding.MlaDecodePageTable(pi.tolist(), last, ps, device="cuda")
    by_pages = _run(dec, fmt, q, tuple(pool), scale, torch.from_numpy(pages).cuda())
    torch.cuda.synchronize()
    assert torch.equal(by_rows, want), "row list at the top of the pool"
    assert torch.equal(by_pages, want), "page table at the top of the pool"
    del pool
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8", "bf16"])
def test_random_page_tables_match_oracle(fmt):
    """Seeded random page sizes (1..80), lengths and CU counts, against the
    page-table oracle."""
    rng = np.random.default_rng({"mxfp4": 11, "fp8": 12, "bf16": 13}[fmt])
    for k in range(6):
        b = int(rng.integers(1, 6))
        lens = [int(rng.choice([0, 1, int(rng.integers(1, 200)), int(rng.integers(1, 2500))])) for _ in range(b)]
        ps = int(rng.choice([1, int(rng.integers(2, 17)), 16, 32, int(rng.integers(17, 81))]))
        cus = int(rng.choice([0, 1, 3, 9]))
        _say(f"case random page table {fmt} #{k} lens={lens} page_size={ps} num_cus={cus}")
        q, pool, scale, indptr, pi, last, pages = _case(fmt, lens, ps, seed=1000 + k)
        dec = binding.MlaDecodePageTable(pi.tolist(), last, ps, device="cuda", num_cus=cus)
        out = _run(dec, fmt, q.cuda(), tuple(p.cuda() for p in pool), scale.cuda() if scale is not None else None,
                   torch.from_numpy(pages).cuda())
        torch.cuda.synchronize()
        _check(out.float().cpu().numpy(), _oracle(fmt, q, pool, scale, pi, last, pages, ps),
               f"random page table {fmt} #{k}")
