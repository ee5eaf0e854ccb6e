"""GPU parity of the decodes over per-token row lists (mla_decode_mxfp4_paged,
mla_decode_fp8_paged, mla_decode_bf16_paged; page size 1) against the fp64
oracle, through the C ABI. Same bar as the contiguous decodes."""

import math
import sys

import numpy as np
import pytest
import torch

from mla_mxfp4_kv_amd import binding, synth
from oracle import dense_ref as dref
from oracle import mxfp4_ref as ref

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


def _case(lens, seed, extra=2.0):
    """Contiguous inputs plus a row pool `extra` times larger holding the
    same rows at random positions (the rest random bytes), and the indices."""
    w = synth.Workload("g", len(lens), None, None, 1.0, False, seed)
    q, packed, scales, indptr, _ = synth.make_inputs(w, lengths=lens)
    t = int(indptr[-1])
    rng = np.random.default_rng(seed)
    rows = max(1, int(extra * t))
    pos = torch.from_numpy(rng.permutation(rows)[:t].astype(np.int32))
    pool_p = torch.from_numpy(rng.integers(0, 256, (rows, 288), dtype=np.uint8))
    pool_s = torch.from_numpy(rng.integers(118, 136, (rows, 18), dtype=np.uint8))
    pool_p[pos.long()] = packed
    pool_s[pos.long()] = scales
    return q, packed, scales, indptr, pool_p, pool_s, pos


CASES = [
    ([1], 0),
    ([31, 32, 33], 0),
    ([127, 128, 129], 3),
    ([0, 300, 0, 1000], 0),
    ([5000], 0),
    ([1, 1, 1, 1, 700], 7),
    ([257, 4097, 33, 2000], 0),
]


@pytest.mark.parametrize("lens,num_cus", CASES)
def test_gather_matches_oracle(lens, num_cus):
    _say(f"case gather lens={lens} num_cus={num_cus}")
    q, packed, scales, indptr, pool_p, pool_s, pos = _case(lens, seed=sum(lens) + 5)
    dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=num_cus)
    out = dec.mxfp4_paged(q.cuda(), pool_p.cuda(), pool_s.cuda(), pos.cuda(), sm_scale=SM)
    torch.cuda.synchronize()
    want = ref.mla_decode_ref_gather(_qbits(q), pool_p.numpy(), pool_s.numpy(), pos.numpy(),
                                     indptr.numpy(), SM)
    _check(out.float().cpu().numpy(), want, f"gather {lens}")


def test_identity_rows_are_bit_identical_to_contiguous():
    """kv_indices = arange: the same values in the same order through the same
    plan, so the output equals the contiguous decode bit for bit."""
    _say("case gather identity")
    lens = [700, 33, 4100]
    w = synth.Workload("g", len(lens), None, None, 1.0, False, 17)
    q, packed, scales, indptr, _ = synth.make_inputs(w, lengths=lens)
    dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=9)
    qd, pd, sd = q.cuda(), packed.cuda(), scales.cuda()
    a = dec(qd, pd, sd, sm_scale=SM).clone()
    ident = torch.arange(int(indptr[-1]), dtype=torch.int32, device="cuda")
    b = dec.mxfp4_paged(qd, pd, sd, ident, sm_scale=SM)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_shared_rows_and_misaligned_scale_pool():
    """Two sequences reading the same rows (a shared prefix), with the scale
    pool starting 2 and 6 bytes past an aligned address."""
    _say("case gather shared rows, scale pool offsets")
    lens = [500, 300, 64]
    q, packed, scales, indptr, pool_p, pool_s, pos = _case(lens, seed=23)
    pos = pos.clone()
    pos[500:600] = pos[0:100]          # sequence 1 starts with sequence 0's first 100 rows
    want = ref.mla_decode_ref_gather(_qbits(q), pool_p.numpy(), pool_s.numpy(), pos.numpy(),
                                     indptr.numpy(), SM)
    dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=4)
    for shift in (2, 6):
        flat = torch.zeros(pool_s.numel() + 16, dtype=torch.uint8)
        flat[shift:shift + pool_s.numel()] = pool_s.reshape(-1)
        sd = flat.cuda()[shift:shift + pool_s.numel()].view(-1, 18)
        out = dec.mxfp4_paged(q.cuda(), pool_p.cuda(), sd, pos.cuda(), sm_scale=SM)
        torch.cuda.synchronize()
        _check(out.float().cpu().numpy(), want, f"shared rows, scale shift {shift}")


def test_gather_errors():
    _say("case gather errors")
    q, packed, scales, indptr, pool_p, pool_s, pos = _case([40], seed=29)
    dec = binding.MlaDecode(indptr.tolist(), device="cuda")
    qd, pd, sd, idx = q.cuda(), pool_p.cuda(), pool_s.cuda(), pos.cuda()
    with pytest.raises(ValueError):
        dec.mxfp4_paged(qd, pd, sd, idx + pool_p.shape[0], sm_scale=SM)   # rows outside the pool
    with pytest.raises(ValueError):
        dec.mxfp4_paged(qd, pd, sd, idx[:10], sm_scale=SM)                # too few indices
    out = torch.empty(1, 16, 512, dtype=torch.bfloat16, device="cuda")
    L = binding.lib()
    ptr = lambda t: binding.ctypes.c_void_p(t.data_ptr())
    st = L.mla_decode_mxfp4_paged(ptr(qd), ptr(pd), ptr(sd), None, ptr(dec.kv_indptr), ptr(out), SM,
                                  ptr(dec.workspace), None)
    assert st == -1
    flat = torch.zeros(sd.numel() + 16, dtype=torch.uint8, device="cuda")
    odd = flat[1:1 + sd.numel()]
    st = L.mla_decode_mxfp4_paged(ptr(qd), ptr(pd), ptr(odd), ptr(idx), ptr(dec.kv_indptr), ptr(out), SM,
                                  ptr(dec.workspace), None)
    assert st == -1


def test_gather_workload_b256_page_shuffled():
    """B=256, kv=8192 with its rows scattered over the pool in 16-row
    pages (a paged cache), every sequence against the oracle."""
    w = synth.WORKLOADS["b256_kv8192"]
    _say("case gather b256_kv8192: generating")
    q, packed, scales, indptr, lens = synth.make_inputs(w, device="cuda")
    t = int(indptr[-1])
    g = torch.Generator(device="cpu").manual_seed(99)
    perm = torch.randperm(t // 16, generator=g).to(torch.int32)
    idx = (perm.repeat_interleave(16) * 16 + torch.arange(16, dtype=torch.int32).repeat(t // 16)).cuda()
    pool_p = torch.empty_like(packed)
    pool_s = torch.empty_like(scales)
    pool_p[idx.long()] = packed
    pool_s[idx.long()] = scales
    dec = binding.MlaDecode(indptr.tolist(), device="cuda")
    _say("case gather b256_kv8192: decode")
    out = dec.mxfp4_paged(q, pool_p, pool_s, idx, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    qb = _qbits(q)
    ind = indptr.numpy()
    pk, sc = packed.cpu().numpy(), scales.cpu().numpy()
    for b in range(len(lens)):
        lo, hi = int(ind[b]), int(ind[b + 1])
        want = ref.mla_decode_ref_seq(qb[b], pk[lo:hi], sc[lo:hi], w.sm_scale)
        _check(got[b], want, f"b256 gather b={b}")


def _dense_case(fmt, lens, seed, extra=2.0):
    w = synth.Workload("g", len(lens), None, None, 1.0, False, seed)
    q, cache, scale, indptr, _ = synth.make_dense_inputs(w, fmt, lengths=lens)
    t = int(indptr[-1])
    rng = np.random.default_rng(seed)
    rows = max(1, int(extra * t))
    pos = torch.from_numpy(rng.permutation(rows)[:t].astype(np.int32))
    if fmt == "fp8":
        pool = torch.from_numpy(rng.integers(0, 0x7E, (rows, 576), dtype=np.uint8))
    else:
        pool = torch.randn(rows, 576, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    pool[pos.long()] = cache
    return q, cache, scale, indptr, pool, pos


def _dense_oracle(fmt, q, pool, scale, pos, indptr):
    qb = _qbits(q)
    rows = pool.numpy() if fmt == "fp8" else pool.view(torch.int16).numpy().view(np.uint16)
    out = np.zeros((len(indptr) - 1, 16, 512))
    for b in range(len(indptr) - 1):
        sel = pos.numpy()[int(indptr[b]):int(indptr[b + 1])]
        if fmt == "fp8":
            out[b] = dref.mla_decode_ref_fp8_seq(qb[b], rows[sel], float(scale[0]), SM)
        else:
            out[b] = dref.mla_decode_ref_bf16_seq(qb[b], rows[sel], SM)
    return out


def _dense_paged(dec, fmt, q, pool, scale, pos):
    if fmt == "fp8":
        return dec.fp8_paged(q.cuda(), pool.cuda(), scale.cuda(), pos.cuda(), sm_scale=SM)
    return dec.bf16_paged(q.cuda(), pool.cuda(), pos.cuda(), sm_scale=SM)


@pytest.mark.parametrize("fmt", ["fp8", "bf16"])
@pytest.mark.parametrize("lens,num_cus", CASES)
def test_dense_gather_matches_oracle(fmt, lens, num_cus):
    _say(f"case {fmt} gather lens={lens} num_cus={num_cus}")
    q, cache, scale, indptr, pool, pos = _dense_case(fmt, lens, seed=sum(lens) + 7)
    dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=num_cus)
    out = _dense_paged(dec, fmt, q, pool, scale, pos)
    torch.cuda.synchronize()
    _check(out.float().cpu().numpy(), _dense_oracle(fmt, q, pool, scale, pos, indptr.numpy()),
           f"{fmt} gather {lens}")


@pytest.mark.parametrize("fmt", ["fp8", "bf16"])
def test_dense_identity_rows_are_bit_identical(fmt):
    _say(f"case {fmt} gather identity")
    lens = [700, 33, 4100, 1]
    w = synth.Workload("g", len(lens), None, None, 1.0, False, 19)
    q, cache, scale, indptr, _ = synth.make_dense_inputs(w, fmt, lengths=lens)
    dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=9)
    ident = torch.arange(int(indptr[-1]), dtype=torch.int32)
    if fmt == "fp8":
        a = dec.fp8(q.cuda(), cache.cuda(), scale.cuda(), sm_scale=SM).clone()
    else:
        a = dec.bf16(q.cuda(), cache.cuda(), sm_scale=SM).clone()
    b = _dense_paged(dec, fmt, q, cache, scale, ident)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("fmt", ["fp8", "bf16"])
def test_dense_gather_workload_b256_page_shuffled(fmt):
    w = synth.WORKLOADS["b256_kv8192"]
    _say(f"case {fmt} gather b256_kv8192: generating")
    q, cache, scale, indptr, lens = synth.make_dense_inputs(w, fmt, device="cuda")
    t = int(indptr[-1])
    g = torch.Generator(device="cpu").manual_seed(98)
    perm = torch.randperm(t // 16, generator=g).to(torch.int32)
    idx = (perm.repeat_interleave(16) * 16 + torch.arange(16, dtype=torch.int32).repeat(t // 16)).cuda()
    pool = torch.empty_like(cache)
    pool[idx.long()] = cache
    dec = binding.MlaDecode(indptr.tolist(), device="cuda")
    _say(f"case {fmt} gather b256_kv8192: decode")
    out = dec.fp8_paged(q, pool, scale, idx, sm_scale=w.sm_scale) if fmt == "fp8" else \
        dec.bf16_paged(q, pool, idx, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    qb = _qbits(q)
    ind = indptr.numpy()
    for b in (0, 131, 255):
        lo, hi = int(ind[b]), int(ind[b + 1])
        if fmt == "fp8":
            want = dref.mla_decode_ref_fp8_seq(qb[b], cache[lo:hi].cpu().numpy(), float(scale[0]), w.sm_scale)
        else:
            want = dref.mla_decode_ref_bf16_seq(
                qb[b], cache[lo:hi].cpu().contiguous().view(torch.int16).numpy().view(np.uint16), w.sm_scale)
        _check(got[b], want, f"{fmt} b256 gather b={b}")
    assert np.all(np.isfinite(got))


def test_graph_replay_device_plan_with_row_lists():
    """GPU-side plan + the three row-list decodes recorded in one HIP graph;
    between replays both the offsets and the row indices change in place on
    the device (a serving step: tokens appended, pages remapped)."""
    steps = [[37, 1025, 0, 300], [38, 1026, 1, 301], [200, 64, 900, 5]]
    batch = 4
    max_total = max(sum(st) for st in steps)
    pool_rows = 3 * max_total
    rng = np.random.default_rng(61)
    qb = torch.randn(batch, 16, 576, generator=torch.Generator().manual_seed(62)).to(torch.bfloat16)
    pool_p = torch.from_numpy(rng.integers(0, 256, (pool_rows, 288), dtype=np.uint8))
    # scales 2^-5 .. 2^0 keep the decoded rows in the range of the synthetic
    # workloads (random bytes with larger scales make outputs that cancel
    # between values in the hundreds, below what a bf16 P can resolve)
    pool_s = torch.from_numpy(rng.integers(122, 128, (pool_rows, 18), dtype=np.uint8))
    pool_8 = torch.from_numpy(rng.integers(0, 0x7E, (pool_rows, 576), dtype=np.uint8))
    pool_16 = torch.randn(pool_rows, 576, generator=torch.Generator().manual_seed(63)).to(torch.bfloat16)
    scale8 = torch.tensor([0.0173], dtype=torch.float32)
    dev = [t.cuda() for t in (qb, pool_p, pool_s, pool_8, pool_16, scale8)]
    qd, pd, sd, p8, p16, s8 = dev
    dp = binding.MlaDecodeDevicePlan(batch, max_total, num_cus=6)
    kvi = torch.zeros(batch + 1, dtype=torch.int32, device="cuda")
    idx = torch.zeros(max_total, dtype=torch.int32, device="cuda")
    outs = [torch.empty(batch, 16, 512, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    stream = torch.cuda.Stream()

    def record():
        dp.plan(kvi, stream=stream)
        dp.decode_paged("mxfp4", qd, pd, sd, idx, kvi, outs[0], sm_scale=SM, stream=stream)
        dp.decode_paged("fp8", qd, p8, s8, idx, kvi, outs[1], sm_scale=SM, stream=stream)
        dp.decode_paged("bf16", qd, p16, None, idx, kvi, outs[2], sm_scale=SM, stream=stream)

    with torch.cuda.stream(stream):
        record()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        record()
    torch.cuda.synchronize()
    qbits = _qbits(qb)
    for k, lens in enumerate(steps):
        ind = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        rows = rng.choice(pool_rows, size=int(ind[-1]), replace=False).astype(np.int32)
        _say(f"replay step {k} lens={lens}")
        kvi.copy_(torch.from_numpy(ind.astype(np.int32)))
        idx.zero_()
        idx[: len(rows)].copy_(torch.from_numpy(rows))
        torch.cuda.synchronize()
        want_mx = ref.mla_decode_ref_gather(qbits, pool_p.numpy(), pool_s.numpy(), rows, ind, SM)
        want_8 = np.zeros_like(want_mx)
        want_16 = np.zeros_like(want_mx)
        b16 = pool_16.view(torch.int16).numpy().view(np.uint16)
        for b in range(batch):
            sel = rows[ind[b]:ind[b + 1]]
            want_8[b] = dref.mla_decode_ref_fp8_seq(qbits[b], pool_8.numpy()[sel], float(scale8[0]), SM)
            want_16[b] = dref.mla_decode_ref_bf16_seq(qbits[b], b16[sel], SM)
        for rep in range(2):
            for o in outs:
                o.fill_(7)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for name, o, want in (("mxfp4", outs[0], want_mx), ("fp8", outs[1], want_8), ("bf16", outs[2], want_16)):
                _check(o.float().cpu().numpy(), want, f"{name} step {k} replay {rep}")
