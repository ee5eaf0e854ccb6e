"""GPU parity of the HIP decode against the fp64 CPU oracle (through the C ABI).

Bar (per element, bf16 output): |gpu - ref| <= 1e-2 + 1e-2 * |ref|; also a
stricter normwise check ||gpu - ref|| / ||ref|| <= 5e-3, since the official
bar is loose for long contexts where outputs are ~1e-2.
"""

import math
import sys

import numpy as np
import pytest
import torch

from mla_mxfp4_kv_amd import binding, synth
from oracle import mxfp4_ref as ref

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(576.0)
ATOL = 1e-2
RTOL = 1e-2
NORMWISE = 5e-3
# Two runs that sum in different orders are each rounded to bf16 at the end;
# two roundings of nearly equal values differ by at most one bf16 ulp
# (2^-8 relative), so that is the bound for run-to-run comparisons.
PAIRWISE = 2.0 ** -8


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


def _run(q, packed, scales, indptr, num_cus=0):
    dec = binding.MlaDecode(indptr, device="cuda", num_cus=num_cus)
    out = dec(q.cuda(), packed.cuda(), scales.cuda(), sm_scale=SM)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


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


def _small(lens, seed, q_std=1.0, token_scale=False):
    w = synth.Workload("small", len(lens), None, None, q_std, token_scale, seed)
    return synth.make_inputs(w, lengths=lens)


SMALL_CASES = [
    ([1], 0),
    ([2, 3], 0),
    ([31, 32, 33], 0),
    ([127, 128, 129], 3),
    ([0, 300, 0, 1000], 0),
    ([5000], 0),
    ([1, 1, 1, 1, 700], 7),
    ([257, 4097, 33, 2000], 0),
]


@pytest.mark.parametrize("lens,num_cus", SMALL_CASES)
def test_small_cases_match_oracle(lens, num_cus):
    _say(f"case lens={lens} num_cus={num_cus}")
    q, packed, scales, indptr, _ = _small(lens, seed=len(lens) + sum(lens))
    got = _run(q, packed, scales, indptr.tolist(), num_cus)
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    _check(got, want, f"lens={lens}")


def test_cache_rows_before_the_first_sequence():
    """kv_indptr[0] > 0: the rows before it belong to no sequence and are
    never read as part of one (they hold NaN scales here)."""
    lens = [40, 0, 300, 129]
    _say(f"case lens={lens} base=77")
    q, packed, scales, indptr, _ = _small(lens, seed=41)
    base = 77
    packed = torch.cat([torch.full((base, 288), 0x77, dtype=torch.uint8), packed])
    scales = torch.cat([torch.full((base, 18), 255, dtype=torch.uint8), scales])
    indptr = indptr + base
    got = _run(q, packed, scales, indptr.tolist(), num_cus=3)
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    assert not np.isnan(want).any()
    _check(got, want, "base offset")


def test_many_tiny_sequences_per_slot():
    """Hundreds of 0..5-token sequences on 2 CUs: every slot walks a long
    item list, each item a tail tile (and empties in between)."""
    rng = np.random.default_rng(5)
    lens = [int(v) for v in rng.integers(0, 6, size=400)]
    _say(f"case 400 tiny sequences, {sum(lens)} tokens, num_cus=2")
    q, packed, scales, indptr, _ = _small(lens, seed=43)
    got = _run(q, packed, scales, indptr.tolist(), num_cus=2)
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    _check(got, want, "tiny sequences")


def test_token_scaled_and_wide_q():
    _say("case token-scaled KV, q std 2")
    q, packed, scales, indptr, _ = _small([900, 1500, 64], seed=11, q_std=2.0, token_scale=True)
    got = _run(q, packed, scales, indptr.tolist(), 5)
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    _check(got, want, "tokscale")


def test_one_token_is_exact():
    _say("case one-token exactness")
    q, packed, scales, indptr, _ = _small([1] * 9, seed=5, q_std=3.0, token_scale=True)
    got = _run(q, packed, scales, indptr.tolist())
    v = ref.dequant_mxfp4(packed.numpy(), scales.numpy())[:, :512]
    want = torch.from_numpy(np.repeat(v[:, None, :], 16, axis=1)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got, want)
    assert np.array_equal(want, np.repeat(v[:, None, :], 16, axis=1))  # V is bf16-exact


def test_empty_sequences_are_zero():
    _say("case empty sequences")
    q, packed, scales, indptr, _ = _small([0, 100, 0, 0, 40], seed=2)
    got = _run(q, packed, scales, indptr.tolist(), 3)
    for b in (0, 2, 3):
        assert np.all(got[b] == 0)
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    _check(got, want, "empty")


def test_all_empty_batch():
    _say("case all-empty batch")
    q, packed, scales, indptr, _ = _small([0, 0], seed=2)
    q = q.cuda()
    packed = torch.zeros(1, 288, dtype=torch.uint8, device="cuda")
    scales = torch.full((1, 18), 127, dtype=torch.uint8, device="cuda")
    dec = binding.MlaDecode([0, 0, 0], device="cuda")
    out = torch.full((2, 16, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    dec(q, packed, scales, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_nan_scale_poisons_only_its_sequence():
    _say("case E8M0 255")
    q, packed, scales, indptr, _ = _small([300, 200, 500], seed=4)
    scales[300 + 57, 3] = 255
    got = _run(q, packed, scales, indptr.tolist(), 4)
    assert np.all(np.isnan(got[1]))
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[2]))
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    _check(got, want, "nan")


def test_scale_rows_at_any_byte_offset():
    """kv_scale may start at any byte: the tile's E8M0 rows are fetched as the
    aligned 16-byte chunks that cover them, so the result must not change."""
    _say("case kv_scale byte offsets")
    lens = [37, 300, 1, 1025, 64, 0, 95]
    q, packed, scales, indptr, _ = _small(lens, seed=11)
    base = _run(q, packed, scales, indptr.tolist(), 5)
    for off in (1, 2, 7, 15):
        buf = torch.full((scales.numel() + 64,), 255, dtype=torch.uint8, device="cuda")
        view = buf[off:off + scales.numel()].view(scales.shape)
        view.copy_(scales.cuda())
        got = _run(q, packed, view, indptr.tolist(), 5)
        assert np.array_equal(got, base), f"kv_scale at byte offset {off}"


def test_query_dynamic_range():
    """Query blocks whose elements span many binades (and exact zeros): the
    latent product splits each bf16 q into two e4m3 terms on a per-block
    power-of-two scale."""
    _say("case query dynamic range")
    g = torch.Generator().manual_seed(21)
    lens = [40, 257, 1000]
    q, packed, scales, indptr, _ = _small(lens, seed=21)
    mag = torch.exp2(torch.randint(-20, 1, q.shape, generator=g).float())
    qw = q.float() * mag
    qw[torch.rand(q.shape, generator=g) < 0.05] = 0.0
    qw = qw.to(torch.bfloat16)
    got = _run(qw, packed, scales, indptr.tolist(), 0)
    want = ref.mla_decode_ref(_qbits(qw), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    _check(got, want, "q dynamic range")


def test_nan_query_poisons_only_its_head():
    _say("case NaN in q")
    lens = [100, 500]
    q, packed, scales, indptr, _ = _small(lens, seed=5)
    q = q.clone()
    q[1, 6, 300] = float("nan")
    got = _run(q, packed, scales, indptr.tolist(), 0)
    assert np.all(np.isnan(got[1, 6]))
    mask = np.ones(got.shape, dtype=bool)
    mask[1, 6] = False
    assert np.all(np.isfinite(got[mask]))
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    _check(got, want, "nan q")


def test_wide_scale_range():
    """E8M0 bytes spread over 116..138 per block: the K scales go straight into
    the scaled MFMA (QK) and through the converter (PV)."""
    _say("case wide E8M0 range")
    g = torch.Generator().manual_seed(33)
    lens = [64, 333, 1500]
    q, packed, scales, indptr, _ = _small(lens, seed=33)
    scales = torch.randint(116, 139, scales.shape, generator=g).to(torch.uint8)
    qs = (q.float() * 0.02).to(torch.bfloat16)
    got = _run(qs, packed, scales, indptr.tolist(), 0)
    want = ref.mla_decode_ref(_qbits(qs), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    # |V| reaches 6 * 2^11 here and scores span hundreds of units, so the bf16
    # rounding of P (relative 2^-9) allows absolute errors of order |V| * 2^-9
    # where tokens cancel: bound each head's error by its row's magnitude.
    assert np.array_equal(np.isnan(got), np.isnan(want)), "wide scales: NaN pattern differs"
    assert np.all(np.isfinite(got))
    for b in range(got.shape[0]):
        for h in range(16):
            g, w = got[b, h], want[b, h]
            scale = float(np.max(np.abs(w)))
            assert np.max(np.abs(g - w)) <= ATOL + RTOL * scale, f"wide scales b={b} h={h}"
            if scale > 0:
                assert np.linalg.norm(g - w) / np.linalg.norm(w) <= NORMWISE, f"wide scales b={b} h={h} normwise"


def test_hip_graph_capture_replays():
    """The decode enqueues kernels only (no allocation, sync or memset), so it
    can be captured in a HIP graph: each replay must reproduce the eager
    result bit for bit, also after the inputs change in place."""
    _say("case HIP graph capture")
    lens = [37, 1025, 0, 300, 2000]
    q, packed, scales, indptr, _ = _small(lens, seed=9)
    q, packed, scales = q.cuda(), packed.cuda(), scales.cuda()
    dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=7)   # splits -> reduce kernel too
    out = torch.empty(len(lens), 16, 512, dtype=torch.bfloat16, device="cuda")
    eager = dec(q, packed, scales, out=torch.empty_like(out), sm_scale=SM).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dec(q, packed, scales, out=out, sm_scale=SM)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dec(q, packed, scales, out=out, sm_scale=SM)
    for rep in range(3):
        out.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
    q.mul_(0.5)
    eager2 = dec(q, packed, scales, out=torch.empty_like(out), sm_scale=SM).clone()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager2)
    want = ref.mla_decode_ref(_qbits(q), packed.cpu().numpy(), scales.cpu().numpy(), indptr.numpy(), SM)
    _check(out.float().cpu().numpy(), want, "graph")


def test_permutation_invariance():
    _say("case permutation invariance")
    q, packed, scales, indptr, _ = _small([3000], seed=9)
    a = _run(q, packed, scales, indptr.tolist())
    perm = torch.randperm(3000, generator=torch.Generator().manual_seed(1))
    b = _run(q, packed[perm].contiguous(), scales[perm].contiguous(), indptr.tolist())
    assert np.linalg.norm(a - b) / np.linalg.norm(a) <= PAIRWISE
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    _check(b, want, "permuted")


def test_split_invariance():
    _say("case split invariance")
    q, packed, scales, indptr, _ = _small([9000, 300, 17000, 1], seed=8)
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    outs = []
    for cus in (1, 7, 64, 0):
        got = _run(q, packed, scales, indptr.tolist(), cus)
        _check(got, want, f"cus={cus}")
        outs.append(got)
    for o in outs[1:]:
        assert np.linalg.norm(o - outs[0]) / np.linalg.norm(outs[0]) <= PAIRWISE


def test_deterministic():
    _say("case determinism")
    q, packed, scales, indptr, _ = _small([4000, 123], seed=3)
    a = _run(q, packed, scales, indptr.tolist())
    b = _run(q, packed, scales, indptr.tolist())
    assert np.array_equal(a, b)


def test_device_plan_matches_host_planner():
    _say("case device plan words")
    ind = [0, 700, 700, 9000, 9001, 20000]
    dec = binding.MlaDecode(ind, device="cuda", num_cus=5)
    words, _ = binding.plan_host(ind, 5)
    dev_words = dec.workspace[: 4 * len(words)].view(torch.int32).cpu().tolist()
    assert dev_words == words


def test_error_codes():
    _say("case error codes")
    q, packed, scales, indptr, _ = _small([50], seed=1)
    q, packed, scales = q.cuda(), packed.cuda(), scales.cuda()
    out = torch.empty(1, 16, 512, dtype=torch.bfloat16, device="cuda")
    ind_dev = indptr.cuda()
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.MlaError) as e:
        binding.decode(q, packed, scales, ind_dev, out, SM, ws[256:])
    assert e.value.status == -5
    binding.plan(indptr.tolist(), ws)
    with pytest.raises(binding.MlaError) as e:
        binding.decode(q, packed, scales, ind_dev, out, float("nan"), ws)
    assert e.value.status == -1
    with pytest.raises(binding.MlaError) as e:
        binding.decode(q, packed, scales, ind_dev, out.view(-1)[1:], SM, ws)
    assert e.value.status == -1
    with pytest.raises(binding.MlaError) as e:
        binding.plan(indptr.tolist(), ws[:64])
    assert e.value.status == -2
    with pytest.raises(binding.MlaError) as e:
        binding.plan([0, 10, 5], ws)
    assert e.value.status == -1
    binding.decode(q, packed, scales, ind_dev, out, SM, ws)
    torch.cuda.synchronize()
    want = ref.mla_decode_ref(_qbits(q), packed.cpu().numpy(), scales.cpu().numpy(), indptr.numpy(), SM)
    _check(out.float().cpu().numpy(), want, "after errors")


def _sampled_workload_check(name, sample):
    w = synth.WORKLOADS[name]
    _say(f"case workload {name}: generating")
    q, packed, scales, indptr, lens = synth.make_inputs(w, device="cuda")
    dec = binding.MlaDecode(indptr.tolist(), device="cuda")
    _say(f"case workload {name}: decode T={indptr[-1].item()}")
    out = dec(q, packed, scales, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    qb = _qbits(q)
    ind = indptr.numpy()
    for b in sample(lens):
        lo, hi = int(ind[b]), int(ind[b + 1])
        want = ref.mla_decode_ref_seq(qb[b], packed[lo:hi].cpu().numpy(), scales[lo:hi].cpu().numpy(),
                                      w.sm_scale)
        nw = _check(got[b], want, f"{name} b={b}")
        _say(f"  {name} b={b} len={hi - lo} normwise={nw:.2e}")
    assert np.all(np.isfinite(got))


def test_workload_b4_kv1024():
    _sampled_workload_check("b4_kv1024", lambda lens: range(len(lens)))


def test_workload_b1_kv65536():
    _sampled_workload_check("b1_kv65536", lambda lens: [0])


def test_workload_b64_kv8192_tokscale():
    _sampled_workload_check("b64_kv8192_tokscale", lambda lens: [0, 17, 40, 63])


def test_workload_b256_kv8192():
    _sampled_workload_check("b256_kv8192", lambda lens: [0, 101, 200, 255])


def test_workload_b128_ragged():
    def pick(lens):
        order = np.argsort(lens)
        return sorted({int(order[0]), int(order[-1]), 5, 64, 127})
    _sampled_workload_check("b128_ragged", pick)


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        b = int(rng.integers(1, 7))
        lens = [int(rng.choice([0, 1, int(rng.integers(1, 300)), int(rng.integers(1, 3000)),
                                int(rng.choice([31, 32, 33, 127, 128, 129, 255, 256, 257]))])) for _ in range(b)]
        yield lens, int(rng.choice([0, 1, 3, 7, 16]))


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8", "bf16"])
def test_random_shapes_match_oracle(fmt):
    """Seeded random batches (empty, one-token, tile-edge and long
    sequences) on several CU counts, every element against the oracle."""
    from oracle import dense_ref as dref
    for k, (lens, cus) in enumerate(_random_shapes(8, {"mxfp4": 1, "fp8": 2, "bf16": 3}[fmt])):
        _say(f"case random {fmt} #{k} lens={lens} num_cus={cus}")
        w = synth.Workload("r", len(lens), None, None, 1.0, False, 100 + k)
        dec = None
        if fmt == "mxfp4":
            q, packed, scales, indptr, _ = synth.make_inputs(w, lengths=lens)
            dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=cus)
            out = dec(q.cuda(), packed.cuda(), scales.cuda(), sm_scale=SM)
            want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
        else:
            q, cache, scale, indptr, _ = synth.make_dense_inputs(w, fmt, lengths=lens)
            dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=cus)
            if fmt == "fp8":
                out = dec.fp8(q.cuda(), cache.cuda(), scale.cuda(), sm_scale=SM)
                want = dref.mla_decode_ref_fp8(_qbits(q), cache.numpy(), float(scale[0]), indptr.numpy(), SM)
            else:
                out = dec.bf16(q.cuda(), cache.cuda(), sm_scale=SM)
                bits = cache.view(torch.int16).numpy().view(np.uint16)
                want = dref.mla_decode_ref_bf16(_qbits(q), bits, indptr.numpy(), SM)
        torch.cuda.synchronize()
        _check(out.float().cpu().numpy(), want, f"random {fmt} #{k} {lens} cus={cus}")
