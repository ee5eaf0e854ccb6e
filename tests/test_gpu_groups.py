"""GPU parity of the decodes over shared contiguous rows
(mla_decode_mxfp4_starts, mla_decode_fp8_starts, mla_decode_bf16_starts):
several 16-head query entries per sequence -- q_seq_len > 1 and 128 heads
as 8 groups of 16 -- against the fp64 oracle, through the C ABI."""

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


def _inputs(fmt, lens, groups, seed):
    """A cache for `lens` and a query of groups x 16 heads per sequence."""
    w = synth.Workload("g", len(lens), None, None, 1.0, False, seed)
    if fmt == "mxfp4":
        _, packed, scales, indptr, _ = synth.make_inputs(w, lengths=lens)
        cache, scale = (packed, scales), None
    else:
        _, c, scale, indptr, _ = synth.make_dense_inputs(w, fmt, lengths=lens)
        cache = (c,)
    gq = torch.Generator().manual_seed(seed)
    q = (torch.randn(len(lens) * groups, 16, 576, generator=gq) * 0.5).to(torch.bfloat16)
    return q, cache, scale, indptr


def _oracle(fmt, q, cache, scale, indptr, groups, batches=None):
    qb = _qbits(q)
    if fmt == "mxfp4":
        return ref.mla_decode_ref_groups(qb, cache[0].numpy(), cache[1].numpy(), indptr.numpy(), groups, SM,
                                         batches=batches)
    if fmt == "fp8":
        return dref.mla_decode_ref_fp8_groups(qb, cache[0].numpy(), float(scale[0]), indptr.numpy(), groups, SM,
                                              batches=batches)
    bits = cache[0].view(torch.int16).numpy().view(np.uint16)
    return dref.mla_decode_ref_bf16_groups(qb, bits, indptr.numpy(), groups, SM, batches=batches)


def _run(dec, fmt, q, cache, scale, **kw):
    if fmt == "mxfp4":
        return dec.mxfp4(q, cache[0], cache[1], sm_scale=SM, **kw)
    if fmt == "fp8":
        return dec.fp8(q, cache[0], scale, sm_scale=SM, **kw)
    return dec.bf16(q, cache[0], sm_scale=SM, **kw)


CASES = [
    ([1, 300, 0, 700], 2, 0),      # q_seq_len = 2
    ([33, 129], 8, 5),             # 128 heads
    ([2000], 3, 0),                # q_seq_len = 3, one long sequence split over CUs
    ([64, 1, 257], 16, 0),         # 128 heads x q_seq_len 2
]


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8", "bf16"])
@pytest.mark.parametrize("lens,groups,num_cus", CASES)
def test_groups_match_oracle(fmt, lens, groups, num_cus):
    _say(f"case groups {fmt} lens={lens} groups={groups} num_cus={num_cus}")
    q, cache, scale, indptr = _inputs(fmt, lens, groups, seed=sum(lens) + groups)
    dec = binding.MlaDecodeGroups(indptr.tolist(), groups, device="cuda", num_cus=num_cus)
    out = _run(dec, fmt, q.cuda(), tuple(c.cuda() for c in cache),
               scale.cuda() if scale is not None else None)
    torch.cuda.synchronize()
    _check(out.float().cpu().numpy(), _oracle(fmt, q, cache, scale, indptr, groups), f"{fmt} {lens} g={groups}")


def test_128_heads_view_and_cache_offset():
    """q as [B, 128, 576] and out as [B, 128, 512] (the same memory as
    [8B, 16, ...]); the sequences sit after 100 unused rows of the cache."""
    _say("case groups 128-head view")
    lens = [300, 45, 1000]
    q, cache, _, indptr = _inputs("mxfp4", lens, 8, seed=12)
    shifted = [torch.cat([torch.zeros((100,) + tuple(c.shape[1:]), dtype=c.dtype), c]) for c in cache]
    ind = [int(v) + 100 for v in indptr]
    dec = binding.MlaDecodeGroups(ind, 8, device="cuda")
    q128 = q.reshape(len(lens), 128, 576).cuda()
    out = torch.empty(len(lens), 128, 512, dtype=torch.bfloat16, device="cuda")
    dec.mxfp4(q128, shifted[0].cuda(), shifted[1].cuda(), out=out, sm_scale=SM)
    torch.cuda.synchronize()
    want = _oracle("mxfp4", q, cache, None, indptr, 8).reshape(len(lens), 128, 512)
    _check(out.float().cpu().numpy(), want, "128-head view")


def test_b32_kv8192_128_heads():
    """B=32, kv=8192 with 128 heads (256 entries): every entry against the
    oracle."""
    w = synth.Workload("b32_kv8192", 32, 8192, None, 1.0, False, 5)
    _say("case groups b32_kv8192 h128: generating")
    _, packed, scales, indptr, _ = synth.make_inputs(w, device="cuda")
    q = (torch.randn(32 * 8, 16, 576, generator=torch.Generator().manual_seed(5)) * 0.5).to(torch.bfloat16)
    dec = binding.MlaDecodeGroups(indptr.tolist(), 8, device="cuda")
    _say("case groups b32_kv8192 h128: decode")
    out = dec.mxfp4(q.cuda(), packed, scales, sm_scale=SM)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    want = ref.mla_decode_ref_groups(_qbits(q), packed.cpu().numpy(), scales.cpu().numpy(), indptr.numpy(), 8, SM)
    for e in range(got.shape[0]):
        _check(got[e], want[e], f"b32 h128 entry {e}")


def test_groups_errors():
    _say("case groups errors")
    q, cache, _, indptr = _inputs("mxfp4", [40], 2, seed=3)
    dec = binding.MlaDecodeGroups(indptr.tolist(), 2, device="cuda")
    qd, pd, sd = q.cuda(), cache[0].cuda(), cache[1].cuda()
    with pytest.raises(ValueError):
        dec.mxfp4(qd, pd[:10].contiguous(), sd[:10].contiguous(), sm_scale=SM)   # cache shorter than kv_indptr
    with pytest.raises(ValueError):
        binding.MlaDecodeGroups(indptr.tolist(), 0)
    out = torch.empty(2, 16, 512, dtype=torch.bfloat16, device="cuda")
    ptr = lambda t: binding.ctypes.c_void_p(t.data_ptr())
    L = binding.lib()
    assert L.mla_decode_mxfp4_starts(ptr(qd), ptr(pd), ptr(sd), None, ptr(dec.kv_indptr), ptr(out), SM,
                                     ptr(dec.plan.workspace), None) == -1
    assert L.mla_decode_mxfp4_starts(ptr(qd), ptr(pd), ptr(sd), ptr(dec.kv_start), ptr(dec.kv_indptr), ptr(out),
                                     SM, ptr(dec.plan.workspace), None) == 0
    torch.cuda.synchronize()


def test_graph_replays_growing_query_groups():
    """128 heads over sequences that grow by one token per step: the GPU-side
    plan and the shared-row decode captured once in a HIP graph, replayed
    with the offsets rewritten in place; every replay equals the eager
    decode of the same state through a host plan."""
    _say("case groups graph replay")
    g, steps = 8, 4
    start = [100, 1, 257]
    total = sum(start) + len(start) * steps
    q, cache, _, _ = _inputs("mxfp4", [total], g * len(start), seed=21)   # one cache, q for 3 x 8 entries
    packed, scales = cache[0].cuda(), cache[1].cuda()
    q = q.reshape(len(start) * g, 16, 576).cuda()
    entries = len(start) * g
    dev = binding.MlaDecodeDevicePlan(entries, total * g, device="cuda", num_cus=6)
    d_start = torch.zeros(entries, dtype=torch.int32, device="cuda")
    d_ind = torch.zeros(entries + 1, dtype=torch.int32, device="cuda")
    out = torch.empty(entries, 16, 512, dtype=torch.bfloat16, device="cuda")

    def upload(lens):
        # sequence b's rows start where the previous one ends (room to grow)
        base = np.concatenate([[0], np.cumsum([n + steps for n in start])])[:-1]
        ent = [0]
        for n in lens:
            for _ in range(g):
                ent.append(ent[-1] + n)
        d_start.copy_(torch.tensor([int(base[e // g]) for e in range(entries)], dtype=torch.int32))
        d_ind.copy_(torch.tensor(ent, dtype=torch.int32))
        torch.cuda.synchronize()
        return base

    lens = list(start)
    upload(lens)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        dev.plan(d_ind, stream=s)
        dev.decode_starts("mxfp4", q, packed, scales, d_start, d_ind, out, sm_scale=SM, stream=s)
        s.synchronize()
        with torch.cuda.graph(graph, stream=s):
            dev.plan(d_ind, stream=s)
            dev.decode_starts("mxfp4", q, packed, scales, d_start, d_ind, out, sm_scale=SM, stream=s)
    torch.cuda.synchronize()
    for step in range(steps):
        lens = [n + 1 for n in lens]
        base = upload(lens)
        out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # the same state through a host plan over a contiguous copy of the rows
        rows = np.concatenate([np.arange(base[b], base[b] + n) for b, n in enumerate(lens)])
        idx = torch.from_numpy(rows).cuda()
        ind = np.concatenate([[0], np.cumsum(lens)]).tolist()
        host = binding.MlaDecodeGroups(ind, g, device="cuda", num_cus=6)
        want = host.mxfp4(q, packed[idx].contiguous(), scales[idx].contiguous(), sm_scale=SM)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"step {step}"
