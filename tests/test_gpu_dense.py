"""GPU parity of the fp8-KV and bf16-KV decodes against the fp64 CPU oracle
(through the C ABI), with the bar of the MXFP4 decode: per element
|gpu - ref| <= 1e-2 + 1e-2 * |ref|, and normwise ||gpu - ref|| / ||ref||
<= 5e-3."""

import math
import sys

import numpy as np
import pytest
import torch

from mla_mxfp4_kv_amd import binding, synth
from oracle import dense_ref as dref
from oracle import mxfp4_ref as mref

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(576.0)
ATOL = 1e-2
RTOL = 1e-2
NORMWISE = 5e-3
PAIRWISE = 2.0 ** -8
FORMATS = ["fp8", "bf16"]


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


def _bits(x):
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _check(got, want, label):
    assert got.shape == want.shape
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan_w), f"{label}: NaN pattern differs"
    g, w = got[~nan_w], want[~nan_w]
    err = np.abs(g - w)
    bound = ATOL + RTOL * np.abs(w)
    worst = float(np.max(err - bound)) if err.size else -1.0
    assert np.all(err <= bound), f"{label}: max excess {worst:.3e}"
    den = np.linalg.norm(w)
    if den > 0:
        nw = np.linalg.norm(g - w) / den
        assert nw <= NORMWISE, f"{label}: normwise {nw:.3e}"
        return nw
    return 0.0


def _inputs(fmt, lens, seed, q_std=1.0, token_scale=False):
    w = synth.Workload("small", len(lens), None, None, q_std, token_scale, seed)
    return synth.make_dense_inputs(w, fmt, lengths=lens)


def _run(fmt, q, cache, scale, indptr, num_cus=0, out=None):
    dec = binding.MlaDecode(indptr, device="cuda", num_cus=num_cus)
    if fmt == "fp8":
        out = dec.fp8(q.cuda(), cache.cuda(), scale.cuda(), out=out, sm_scale=SM)
    else:
        out = dec.bf16(q.cuda(), cache.cuda(), out=out, sm_scale=SM)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _oracle(fmt, q, cache, scale, indptr, batches=None):
    if fmt == "fp8":
        return dref.mla_decode_ref_fp8(_qbits(q), cache.cpu().numpy(), float(scale[0]), indptr, SM, batches)
    return dref.mla_decode_ref_bf16(_qbits(q), _bits(cache), indptr, SM, batches)


SMALL_CASES = [
    ([1], 0),
    ([2, 3], 0),
    ([15, 16, 17], 0),
    ([31, 32, 33], 0),
    ([127, 128, 129], 3),
    ([0, 300, 0, 1000], 0),
    ([5000], 0),
    ([1, 1, 1, 1, 700], 7),
    ([257, 4097, 33, 2000], 0),
]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("lens,num_cus", SMALL_CASES)
def test_small_cases_match_oracle(fmt, lens, num_cus):
    _say(f"case {fmt} lens={lens} num_cus={num_cus}")
    q, cache, scale, indptr, _ = _inputs(fmt, lens, seed=len(lens) + sum(lens))
    got = _run(fmt, q, cache, scale, indptr.tolist(), num_cus)
    _check(got, _oracle(fmt, q, cache, scale, indptr.numpy()), f"{fmt} lens={lens}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_one_token_is_exact(fmt):
    """kv_len = 1: p = 1, out = V (times the per-tensor scale) rounded to
    bf16, bit for bit."""
    _say(f"case {fmt} one token")
    q, cache, scale, indptr, _ = _inputs(fmt, [1, 1, 1], seed=9)
    got = _run(fmt, q, cache, scale, indptr.tolist())
    want = _oracle(fmt, q, cache, scale, indptr.numpy())
    want_bf16 = torch.from_numpy(want).to(torch.float32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got, want_bf16)


@pytest.mark.parametrize("fmt", FORMATS)
def test_token_scaled_and_wide_query(fmt):
    _say(f"case {fmt} token-scaled rows, q std 2")
    q, cache, scale, indptr, _ = _inputs(fmt, [900, 77, 2049], seed=21, q_std=2.0, token_scale=True)
    got = _run(fmt, q, cache, scale, indptr.tolist(), num_cus=5)
    _check(got, _oracle(fmt, q, cache, scale, indptr.numpy()), f"{fmt} tokscale")


@pytest.mark.parametrize("fmt", FORMATS)
def test_more_slots_than_workgroups(fmt):
    """A plan for 600 slots on a device with fewer CUs: each workgroup walks
    several slots."""
    _say(f"case {fmt} more slots than workgroups")
    q, cache, scale, indptr, _ = _inputs(fmt, [120000, 300, 40000, 5], seed=31)
    got = _run(fmt, q, cache, scale, indptr.tolist(), num_cus=600)
    _check(got, _oracle(fmt, q, cache, scale, indptr.numpy()), f"{fmt} 600 slots")


@pytest.mark.parametrize("fmt", FORMATS)
def test_split_invariance(fmt):
    """The same inputs planned on 1, 7, 64 and all CUs (different splits and
    reduce merges) agree to the bf16 output rounding."""
    _say(f"case {fmt} split invariance")
    q, cache, scale, indptr, _ = _inputs(fmt, [3000, 1, 700], seed=23)
    runs = [_run(fmt, q, cache, scale, indptr.tolist(), n) for n in (1, 7, 64, 0)]
    want = _oracle(fmt, q, cache, scale, indptr.numpy())
    for r in runs:
        _check(r, want, f"{fmt} split")
        nw = np.linalg.norm(r - runs[-1]) / np.linalg.norm(runs[-1])
        assert nw <= PAIRWISE, nw


@pytest.mark.parametrize("fmt", FORMATS)
def test_permutation_invariance(fmt):
    _say(f"case {fmt} permutation")
    q, cache, scale, indptr, _ = _inputs(fmt, [1500], seed=25)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(1500))
    a = _run(fmt, q, cache, scale, indptr.tolist())
    b = _run(fmt, q, cache[perm].contiguous(), scale, indptr.tolist())
    # each run is rounded to bf16 once at the end: at most one bf16 ulp apart
    nw = np.linalg.norm(a - b) / np.linalg.norm(a)
    assert nw <= PAIRWISE, nw
    want = _oracle(fmt, q, cache, scale, indptr.numpy())
    _check(a, want, f"{fmt} in order")
    _check(b, want, f"{fmt} permuted")


def test_fp8_and_bf16_agree_with_mxfp4_on_the_same_values():
    """Caches holding the same decoded MXFP4 values (exact in e4m3 for E8M0
    bytes 124..128 and in bf16 for any byte) give the MXFP4 decode's result
    within the bar, through all three kernels."""
    _say("case cross-format")
    lens = [333, 1024, 5]
    w = synth.Workload("x", len(lens), None, None, 1.0, False, 31)
    q, packed, scales, indptr, _ = synth.make_inputs(w, lengths=lens)
    scales = torch.clamp(scales, 124, 128)
    k = mref.dequant_mxfp4(packed.numpy(), scales.numpy())
    want = mref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    dec = binding.MlaDecode(indptr.tolist(), device="cuda")
    mx = dec(q.cuda(), packed.cuda(), scales.cuda(), sm_scale=SM)
    kv8 = torch.from_numpy(k).to(torch.float8_e4m3fn)
    assert np.array_equal(kv8.to(torch.float64).numpy(), k)
    f8 = dec.fp8(q.cuda(), kv8.view(torch.uint8).cuda(), torch.ones(1, device="cuda"), sm_scale=SM)
    b16 = dec.bf16(q.cuda(), torch.from_numpy(k).to(torch.bfloat16).cuda(), sm_scale=SM)
    torch.cuda.synchronize()
    for name, o in (("mxfp4", mx), ("fp8", f8), ("bf16", b16)):
        _check(o.float().cpu().numpy(), want, name)


def test_fp8_scale_is_read_on_the_device():
    """Changing the per-tensor scale in place changes the result like the
    oracle (the kernel reads it at run time)."""
    _say("case fp8 scale in place")
    q, cache, scale, indptr, _ = _inputs("fp8", [600, 40], seed=27)
    dec = binding.MlaDecode(indptr.tolist(), device="cuda")
    qd, cd, sd = q.cuda(), cache.cuda(), scale.cuda()
    for s in (float(scale[0]), 0.5 * float(scale[0]), 3.0 * float(scale[0])):
        sd.fill_(s)
        out = dec.fp8(qd, cd, sd, sm_scale=SM)
        torch.cuda.synchronize()
        want = dref.mla_decode_ref_fp8(_qbits(q), cache.numpy(), s, indptr.numpy(), SM)
        _check(out.float().cpu().numpy(), want, f"fp8 scale {s:.3e}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_empty_and_nan_query(fmt):
    """An empty sequence gets zeros; a NaN in one query element turns only
    that head's output into NaN."""
    _say(f"case {fmt} empty + NaN query")
    q, cache, scale, indptr, _ = _inputs(fmt, [0, 200, 65], seed=29)
    q[2, 5, 100] = float("nan")
    got = _run(fmt, q, cache, scale, indptr.tolist(), num_cus=2)
    assert np.all(got[0] == 0)
    assert np.all(np.isnan(got[2, 5]))
    mask = np.ones(got.shape, bool)
    mask[2, 5] = False
    assert np.all(np.isfinite(got[mask]))
    want = _oracle(fmt, q, cache, scale, indptr.numpy())
    _check(got[1], want[1], f"{fmt} seq 1")


def test_errors():
    _say("case dense error codes")
    q, cache, scale, indptr, _ = _inputs("fp8", [10], seed=33)
    qd, cd, sd = q.cuda(), cache.cuda(), scale.cuda()
    out = torch.empty(1, 16, 512, dtype=torch.bfloat16, device="cuda")
    ind_dev = indptr.cuda()
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    binding.plan(indptr.tolist(), ws)
    L = binding.lib()
    ptr = lambda t: binding.ctypes.c_void_p(t.data_ptr())
    # no per-tensor scale
    st = L.mla_decode_fp8(ptr(qd), ptr(cd), None, ptr(ind_dev), ptr(out), SM, ptr(ws), None)
    assert st == -1
    # non-finite softmax scale (any finite value, negative included, is valid)
    for bad in (float("inf"), float("-inf"), float("nan")):
        with pytest.raises(binding.MlaError) as e:
            binding.decode_fp8(qd, cd, sd, ind_dev, out, bad, ws)
        assert e.value.status == -1
    # cache rows not 16-byte aligned
    with pytest.raises(binding.MlaError) as e:
        binding.decode_bf16(qd, cd.view(-1)[1:], ind_dev, out, SM, ws)
    assert e.value.status == -1
    # workspace never planned
    with pytest.raises(binding.MlaError) as e:
        binding.decode_bf16(qd, cd, ind_dev, out, SM, ws[256:])
    assert e.value.status == -5
    # still works afterwards
    binding.decode_fp8(qd, cd, sd, ind_dev, out, SM, ws)
    torch.cuda.synchronize()
    want = dref.mla_decode_ref_fp8(_qbits(q), cache.numpy(), float(scale[0]), indptr.numpy(), SM)
    _check(out.float().cpu().numpy(), want, "after errors")


def _indptr(lens):
    out = [0]
    for n in lens:
        out.append(out[-1] + n)
    return out


def test_graph_replay_with_device_plan():
    """GPU-side plan + fp8 decode + bf16 decode recorded in one HIP graph;
    every replay follows the offsets in the device tensor at that moment and
    matches the oracle."""
    lens0 = [37, 1025, 0, 300, 2000]
    steps = [lens0, [n + 1 for n in lens0], [n + 200 for n in lens0], [0, 0, 0, 0, 1]]
    max_total = sum(steps[2])
    batch = len(lens0)
    q, c8, s8, _, _ = _inputs("fp8", [max_total], seed=35)
    _, c16, _, _, _ = _inputs("bf16", [max_total], seed=35)
    qb = torch.randn(batch, 16, 576, generator=torch.Generator().manual_seed(36)).to(torch.bfloat16)
    qd, c8d, s8d, c16d = qb.cuda(), c8.cuda(), s8.cuda(), c16.cuda()
    dp = binding.MlaDecodeDevicePlan(batch, max_total, num_cus=7)
    kvi = torch.tensor(_indptr(steps[0]), dtype=torch.int32, device="cuda")
    o8 = torch.empty(batch, 16, 512, dtype=torch.bfloat16, device="cuda")
    o16 = torch.empty_like(o8)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        dp.plan(kvi, stream=stream)
        dp.decode_fp8(qd, c8d, s8d, kvi, o8, sm_scale=SM, stream=stream)
        dp.decode_bf16(qd, c16d, kvi, o16, sm_scale=SM, stream=stream)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        dp.plan(kvi, stream=stream)
        dp.decode_fp8(qd, c8d, s8d, kvi, o8, sm_scale=SM, stream=stream)
        dp.decode_bf16(qd, c16d, kvi, o16, sm_scale=SM, stream=stream)
    torch.cuda.synchronize()
    qbits = _qbits(qb)
    for k, lens in enumerate(steps):
        _say(f"replay step {k} lens={lens}")
        kvi.copy_(torch.tensor(_indptr(lens), dtype=torch.int32))
        ind = np.array(_indptr(lens))
        want8 = dref.mla_decode_ref_fp8(qbits, c8.numpy(), float(s8[0]), ind, SM)
        want16 = dref.mla_decode_ref_bf16(qbits, _bits(c16), ind, SM)
        torch.cuda.synchronize()
        for rep in range(2):
            o8.fill_(7)
            o16.fill_(7)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            _check(o8.float().cpu().numpy(), want8, f"fp8 step {k} replay {rep}")
            _check(o16.float().cpu().numpy(), want16, f"bf16 step {k} replay {rep}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_zero_and_negative_sm_scale(fmt):
    """Any finite softmax scale, tail tiles included."""
    lens = [37, 300, 1025, 5]
    w = synth.Workload("s", len(lens), None, None, 1.0, False, 71)
    q, cache, scale, indptr, _ = synth.make_dense_inputs(w, fmt, lengths=lens)
    for sm in (0.0, -0.0, -SM, -2.5 * SM):
        _say(f"case {fmt} sm_scale={sm!r}")
        dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=3)
        if fmt == "fp8":
            out = dec.fp8(q.cuda(), cache.cuda(), scale.cuda(), sm_scale=sm)
            want = dref.mla_decode_ref_fp8(_qbits(q), cache.numpy(), float(scale[0]), indptr.numpy(),
                                           float(np.float32(sm)))
        else:
            out = dec.bf16(q.cuda(), cache.cuda(), sm_scale=sm)
            want = dref.mla_decode_ref_bf16(_qbits(q), _bits(cache), indptr.numpy(), float(np.float32(sm)))
        torch.cuda.synchronize()
        _check(out.float().cpu().numpy(), want, f"{fmt} sm_scale={sm!r}")


def _workload_check(fmt, name):
    """The workload at full size on the device's CU count, every element of
    every sequence against the dense oracle."""
    w = synth.WORKLOADS[name]
    _say(f"case {fmt} workload {name}: generating")
    q, cache, scale, indptr, lens = synth.make_dense_inputs(w, fmt, device="cuda")
    dec = binding.MlaDecode(indptr.tolist(), device="cuda")
    _say(f"case {fmt} workload {name}: decode T={indptr[-1].item()}")
    out = dec.fp8(q, cache, scale, sm_scale=w.sm_scale) if fmt == "fp8" else dec.bf16(q, cache, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    qb = _qbits(q)
    ind = indptr.numpy()
    host = cache.cpu().numpy() if fmt == "fp8" else _bits(cache)
    vs = float(scale[0]) if fmt == "fp8" else None
    worst = 0.0
    for b in range(len(lens)):
        lo, hi = int(ind[b]), int(ind[b + 1])
        if fmt == "fp8":
            want = dref.mla_decode_ref_fp8_seq(qb[b], host[lo:hi], vs, w.sm_scale)
        else:
            want = dref.mla_decode_ref_bf16_seq(qb[b], host[lo:hi], w.sm_scale)
        worst = max(worst, _check(got[b], want, f"{fmt} {name} b={b}"))
    _say(f"  {fmt} {name}: {len(lens)} sequences, worst normwise {worst:.2e}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workloads_every_sequence(fmt, name):
    _workload_check(fmt, name)
