"""The GPU-side planner (mla_plan_device) against the plain-Python planner
oracle, and decodes planned on the GPU against host-planned ones and the
fp64 oracle, including a HIP graph of plan + decode replayed while the
sequence offsets change on the device."""

import math
import sys

import numpy as np
import pytest
import torch

from mla_mxfp4_kv_amd import binding, synth
from oracle import mxfp4_ref as ref
from oracle import planner_ref as pref

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


def _indptr(lens, base=0):
    ind = [base]
    for n in lens:
        ind.append(ind[-1] + n)
    return ind


def _device_words(dp):
    """The plan words (header up to the partial arrays) of the workspace."""
    torch.cuda.synchronize()
    hdr = dp.workspace[:64].view(torch.int32).cpu().tolist()
    n = max(hdr[14] // 4, 16)     # the partial LSE array starts after the words
    w = dp.workspace[: 4 * n].view(torch.int32).cpu().tolist()
    return pref.decode_plan_words(w)


PLAN_CASES = [
    ([], 0, 4),
    ([0, 0, 0], 0, 4),
    ([1], 0, 1),
    ([700, 0, 8300, 1, 11000], 0, 5),
    ([65536], 0, 256),
    ([8192] * 64, 0, 256),
    ([3, 0, 5, 2, 0, 1] * 150, 0, 3),
    ([40, 0, 300, 129], 77, 3),
    ([256] * 10, 0, 10),
    ([255, 257, 1, 511, 513], 5, 7),
    ([2 ** 30, 2 ** 31 - 1 - 2 ** 30], 0, 1),     # the int32 token limit on one CU
    # item charges: short sequences on a weighted line, across the
    # 1024-sequence blocks of the planner's scans
    ([5, 0, 300, 17] * 400, 3, 7),
    ([3000, 200, 100, 700], 0, 2),
    (synth.seq_lengths(synth.WORKLOADS["b128_ragged"]), 0, 256),
    ([40000, 1, 2, 3] + [6000] * 60 + [5] * 30, 11, 256),
]


@pytest.mark.parametrize("lens,base,num_cus", PLAN_CASES)
def test_device_plan_words_match_oracle(lens, base, num_cus):
    _say(f"case plan lens[:6]={lens[:6]} n={len(lens)} base={base} num_cus={num_cus}")
    ind = _indptr(lens, base)
    batch = len(lens)
    total = ind[-1] - ind[0]
    want = pref.build_plan(ind, batch, num_cus)
    dp = binding.MlaDecodeDevicePlan(batch, min(total + 1000, 2 ** 31 - 1), num_cus=num_cus)
    dp.plan(torch.tensor(ind, dtype=torch.int32, device="cuda"))
    got = _device_words(dp)
    assert got["magic"] == pref.PlanConsts.MAGIC
    assert got["version"] == pref.PlanConsts.VERSION
    assert (got["batch"], got["base"], got["total"], got["num_cus"], got["chunk"]) == \
        (batch, want.base, want.total, num_cus, want.chunk)
    assert got["slot_indptr"] == want.slot_indptr
    assert got["items"] == [tuple(i) for i in want.items]
    assert got["num_partials"] == want.num_partials
    assert got["reduce"] == [tuple(r) for r in want.reduce]
    # the words are laid out for the bounds; the partial arrays fit the workspace
    assert got["off_o"] + 4 * 16 * 512 * got["num_partials"] <= dp.workspace.numel()


def _check(got, want, label):
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan_w), f"{label}: NaN pattern differs"
    g, w = got[~nan_w], want[~nan_w]
    err = np.abs(g - w)
    assert np.all(err <= ATOL + RTOL * np.abs(w)), f"{label}: max err {err.max():.3e}"
    den = np.linalg.norm(w)
    if den > 0:
        assert np.linalg.norm(g - w) / den <= NORMWISE, label


def _inputs(lens, seed):
    w = synth.Workload("devplan", len(lens), None, None, 1.0, False, seed)
    q, packed, scales, _, _ = synth.make_inputs(w, lengths=list(lens))
    return q, packed, scales


@pytest.mark.parametrize("lens,num_cus", [([700, 0, 8300, 1, 4000], 5), ([1, 2, 3, 0, 4096, 37], 3),
                                          ([5000], 16)])
def test_device_plan_decode_equals_host_plan(lens, num_cus):
    _say(f"case decode lens={lens} num_cus={num_cus}")
    q, packed, scales = _inputs(lens, seed=7 + len(lens))
    ind = _indptr(lens)
    qd, pd, sd = q.cuda(), packed.cuda(), scales.cuda()
    host = binding.MlaDecode(ind, device="cuda", num_cus=num_cus)
    want = host(qd, pd, sd, sm_scale=SM)
    dp = binding.MlaDecodeDevicePlan(len(lens), ind[-1], num_cus=num_cus)
    kvi = torch.tensor(ind, dtype=torch.int32, device="cuda")
    out = torch.empty_like(want)
    dp.plan(kvi)
    dp.decode(qd, pd, sd, kvi, out, sm_scale=SM)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))


def test_device_plan_graph_replays_as_lengths_change():
    """Plan + decode recorded once; each replay follows the offsets that sit
    in the device tensor at that moment (tokens appended between replays)."""
    lens0 = [37, 1025, 0, 300, 2000]
    steps = [lens0, [n + 1 for n in lens0], [n + 200 for n in lens0], [0, 0, 0, 0, 1]]
    max_total = sum(steps[2])
    batch = len(lens0)
    # one cache big enough for every step; each step's sequences are laid out
    # contiguously from row 0
    q, packed, scales = _inputs([max_total], seed=11)
    qb = torch.randn(batch, 16, 576, generator=torch.Generator().manual_seed(12)).to(torch.bfloat16)
    qd, pd, sd = qb.cuda(), packed.cuda(), scales.cuda()
    dp = binding.MlaDecodeDevicePlan(batch, max_total, num_cus=7)
    kvi = torch.tensor(_indptr(steps[0]), dtype=torch.int32, device="cuda")
    out = torch.empty(batch, 16, 512, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()
    # warm-up outside the graph (loads the library's kernels)
    with torch.cuda.stream(stream):
        dp.plan(kvi, stream=stream)
        dp.decode(qd, pd, sd, kvi, out, sm_scale=SM, stream=stream)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        dp.plan(kvi, stream=stream)
        dp.decode(qd, pd, sd, kvi, out, sm_scale=SM, stream=stream)
    torch.cuda.synchronize()
    for k, lens in enumerate(steps):
        _say(f"replay step {k} lens={lens}")
        kvi.copy_(torch.tensor(_indptr(lens), dtype=torch.int32))
        torch.cuda.synchronize()
        for rep in range(2):
            out.fill_(7)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = out.float().cpu().numpy()
            ind = np.array(_indptr(lens))
            want = ref.mla_decode_ref(qb.contiguous().view(torch.int16).numpy().view(np.uint16),
                                      packed.numpy(), scales.numpy(), ind, SM)
            _check(got, want, f"step {k} replay {rep}")


def test_device_plan_rejects_bad_offsets_on_the_gpu():
    """Decreasing offsets, or more tokens than the bound, give an empty plan:
    the decode then leaves the output untouched."""
    q, packed, scales = _inputs([600], seed=13)
    qd, pd, sd = q.repeat(3, 1, 1).cuda(), packed.cuda(), scales.cuda()
    dp = binding.MlaDecodeDevicePlan(3, 500, num_cus=4)
    out = torch.full((3, 16, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    for ind in ([0, 100, 50, 200], [0, 200, 400, 600], [-1, 10, 20, 30]):
        _say(f"case bad offsets {ind}")
        kvi = torch.tensor(ind, dtype=torch.int32, device="cuda")
        dp.plan(kvi)
        words = _device_words(dp)
        assert words["magic"] == 0 and words["num_slots"] == 0 and words["num_reduce"] == 0
        dp.decode(qd, pd, sd, kvi, out, sm_scale=SM)
        torch.cuda.synchronize()
        assert bool((out.float() == 3.0).all())


def test_device_plan_host_errors():
    lib = binding.lib()
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    kvi = torch.zeros(4, dtype=torch.int32, device="cuda")
    import ctypes
    st = lib.mla_plan_device(ctypes.c_void_p(kvi.data_ptr()), -1, 100, 4, ctypes.c_void_p(ws.data_ptr()),
                             ws.numel(), None)
    assert st == -1
    st = lib.mla_plan_device(None, 3, 100, 4, ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert st == -1
    st = lib.mla_plan_device(ctypes.c_void_p(kvi.data_ptr()), 3, 1 << 31, 4, ctypes.c_void_p(ws.data_ptr()),
                             ws.numel(), None)
    assert st == -1
    st = lib.mla_plan_device(ctypes.c_void_p(kvi.data_ptr()), 3, 1 << 20, 256,
                             ctypes.c_void_p(ws.data_ptr()), 1024, None)
    assert st == -2
