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


def _vmax(packed, scales, indptr):
    """max_t |V[t, d]| over each sequence's tokens: [B, 512] (the oracle's
    exact dequantisation)."""
    v = np.abs(ref.dequant_mxfp4(packed, scales)[:, :512])
    out = np.zeros((len(indptr) - 1, 512))
    for b in range(len(indptr) - 1):
        lo, hi = int(indptr[b]), int(indptr[b + 1])
        if hi > lo:
            out[b] = v[lo:hi].max(axis=0)
    return out


def test_wide_scale_range():
    """E8M0 bytes spread over 116..138 per block: the K scales go straight into
    the scaled MFMA (QK) and through the converter (PV).

    Here |V| reaches 6 * 2^11 while the outputs are much smaller (tokens
    cancel), so the bf16 rounding of P (relative 2^-9 per token, the pages'
    own precision for P) is no longer covered by 1e-2 + 1e-2 |ref|. Its
    effect on element d is at most 2^-9 * sum_t p_t |V[t,d] - out[d]| <=
    2^-8 * max_t |V[t,d]|, so every element is held to
    1e-2 + 1e-2 |ref| + 2^-8 max_t |V[t,d]|."""
    _say("case wide E8M0 range")
    g = torch.Generator().manual_seed(33)
    lens = [64, 333, 1500]
    q, packed, scales, indptr, _ = _small(lens, seed=33)
    scales = torch.randint(116, 139, scales.shape, generator=g).to(torch.uint8)
    qs = (q.float() * 0.02).to(torch.bfloat16)
    got = _run(qs, packed, scales, indptr.tolist(), 0)
    want = ref.mla_decode_ref(_qbits(qs), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    assert np.array_equal(np.isnan(got), np.isnan(want)), "wide scales: NaN pattern differs"
    assert np.all(np.isfinite(got))
    vmax = _vmax(packed.numpy(), scales.numpy(), indptr.numpy())[:, None, :]
    bound = ATOL + RTOL * np.abs(want) + 2.0 ** -8 * vmax
    err = np.abs(got - want)
    assert np.all(err <= bound), f"wide scales: max excess {float(np.max(err - bound)):.3e}"
    # the bound is not loose by orders of magnitude: the P rounding shows up
    assert float(np.max(err / (2.0 ** -8 * vmax + 1e-30))) > 1e-3


def test_zero_and_negative_sm_scale():
    """Any finite softmax scale: zero gives the plain mean of V (tail tiles
    included: the masked tokens must not turn into NaN), a negative scale
    favours the lowest scores."""
    lens = [37, 300, 1025, 5, 64]
    q, packed, scales, indptr, _ = _small(lens, seed=17)
    for sm in (0.0, -0.0, -SM, -3.0 * SM, 3.0 * SM):
        _say(f"case sm_scale={sm!r}")
        dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=3)
        out = dec(q.cuda(), packed.cuda(), scales.cuda(), sm_scale=sm)
        torch.cuda.synchronize()
        want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), float(np.float32(sm)))
        _check(out.float().cpu().numpy(), want, f"sm_scale={sm!r}")
    # zero scale: the plain mean of each sequence's V rows
    v = ref.dequant_mxfp4(packed.numpy(), scales.numpy())[:, :512]
    dec = binding.MlaDecode(indptr.tolist(), device="cuda")
    out = dec(q.cuda(), packed.cuda(), scales.cuda(), sm_scale=0.0)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    for b, (lo, hi) in enumerate(zip(indptr[:-1].tolist(), indptr[1:].tolist())):
        mean = v[lo:hi].mean(axis=0)
        assert np.all(np.abs(got[b] - mean[None, :]) <= ATOL + RTOL * np.abs(mean)[None, :]), f"mean b={b}"


def test_plan_release_and_cleared_header():
    """A released workspace is refused (MLA_ERR_NOT_PLANNED); a workspace
    whose plan header was cleared after planning leaves the output
    untouched (decode and reduce kernels both check the header)."""
    _say("case plan release / cleared header")
    lens = [300, 1000, 0, 45]
    q, packed, scales, indptr, _ = _small(lens, seed=6)
    q, packed, scales = q.cuda(), packed.cuda(), scales.cuda()
    ind_dev = indptr.cuda()
    nbytes = binding.workspace_bytes(len(lens), int(indptr[-1]), 5)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((len(lens), 16, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    binding.plan(indptr.tolist(), ws, num_cus=5)      # splits: decode + reduce kernels
    assert binding.plan_release(ws.data_ptr()) == 0
    with pytest.raises(binding.MlaError) as e:
        binding.decode(q, packed, scales, ind_dev, out, SM, ws)
    assert e.value.status == -5
    assert binding.plan_release(ws.data_ptr()) == -5
    binding.plan(indptr.tolist(), ws, num_cus=5)
    ws[:4].zero_()                                    # the magic word
    binding.decode(q, packed, scales, ind_dev, out, SM, ws)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    binding.plan(indptr.tolist(), ws, num_cus=5)
    ws[4:8].zero_()                                   # the version word
    binding.decode(q, packed, scales, ind_dev, out, SM, ws)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    binding.plan(indptr.tolist(), ws, num_cus=5)
    binding.decode(q, packed, scales, ind_dev, out, SM, ws)
    torch.cuda.synchronize()
    want = ref.mla_decode_ref(_qbits(q), packed.cpu().numpy(), scales.cpu().numpy(), indptr.numpy(), SM)
    _check(out.float().cpu().numpy(), want, "replanned")
    binding.plan_release(ws.data_ptr())


def test_entry_offsets_at_the_int32_limit():
    """Entry offsets that end at 2^31 - 1 (shared rows: the offsets only give
    lengths and order): lengths that are not multiples of 32, so the last
    tiles are partial right below the limit. Same plan relative to its
    base, so the output must equal the same decode at offset 0 bit for bit."""
    lens = [1000, 37, 513, 70]
    _say(f"case entry offsets ending at 2^31-1, lens={lens}")
    q, packed, scales, indptr, _ = _small(lens, seed=19)
    q, packed, scales = q.cuda(), packed.cuda(), scales.cuda()
    low = indptr.tolist()
    top = 2 ** 31 - 1
    high = [v + top - low[-1] for v in low]
    starts = torch.tensor(low[:-1], dtype=torch.int32, device="cuda")
    outs = []
    for ind in (low, high):
        for cus in (3, 0):
            dec = binding.MlaDecode(ind, device="cuda", num_cus=cus)
            out = torch.empty(len(lens), 16, 512, dtype=torch.bfloat16, device="cuda")
            binding.decode_starts("mxfp4", q, packed, scales, starts, dec.kv_indptr, out, SM, dec.workspace)
            torch.cuda.synchronize()
            outs.append(out.float().cpu().numpy())
    assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[1], outs[3])
    want = ref.mla_decode_ref(_qbits(q), packed.cpu().numpy(), scales.cpu().numpy(), indptr.numpy(), SM)
    for o in outs:
        _check(o, want, "offsets at the int32 limit")


def test_e8m0_edge_bytes():
    """E8M0 bytes 0 and 1 (2^-127, 2^-126: decoded elements below the bf16
    normal range) on random blocks match the oracle within the bar. Bytes
    253 and 254: a one-token sequence whose decoded row is finite in bf16
    returns it exactly; in longer sequences each output element is either
    within the bar or non-finite (the fp32 accumulation of P V can overflow
    there, where the exact result is finite), never silently wrong."""
    g = torch.Generator().manual_seed(23)
    lens = [300, 77, 1200]
    q, packed, scales, indptr, _ = _small(lens, seed=23)
    sc = scales.clone()
    pick = torch.rand(sc.shape, generator=g) < 0.15
    sc[pick] = torch.randint(0, 2, sc.shape, generator=g).to(torch.uint8)[pick]
    _say("case E8M0 bytes 0/1")
    got = _run(q, packed, sc, indptr.tolist(), 3)
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), sc.numpy(), indptr.numpy(), SM)
    _check(got, want, "bytes 0/1")

    _say("case E8M0 bytes 253/254, one token")
    n1 = 6
    packed1 = torch.randint(0, 256, (n1, 288), generator=g).to(torch.uint8)
    # codes of magnitude <= 1.5 (0..3 and 8..11) in blocks with the top bytes
    packed1 = packed1 & 0x33
    sc1 = torch.full((n1, 18), 127, dtype=torch.uint8)
    sc1[:, 0] = 254
    sc1[:, 5] = 253
    sc1[:, 17] = 254
    q1 = (torch.randn(n1, 16, 576, generator=g) * 0.01).to(torch.bfloat16)
    q1[:, :, 0:32] = 0            # keep the logits finite: one token needs no logit anyway
    q1[:, :, 160:192] = 0
    q1[:, :, 544:576] = 0
    ind1 = list(range(n1 + 1))
    got1 = _run(q1, packed1, sc1, ind1, 0)
    v = ref.dequant_mxfp4(packed1.numpy(), sc1.numpy())[:, :512]
    assert np.all(np.isfinite(v)) and np.max(np.abs(v)) > 1e37
    assert np.array_equal(got1, np.repeat(v[:, None, :], 16, axis=1)), "one token at bytes 253/254"

    _say("case E8M0 bytes 253/254, long sequences")
    sc2 = scales.clone()
    pick = torch.rand(sc2.shape, generator=g) < 0.02
    sc2[pick] = torch.randint(253, 255, sc2.shape, generator=g).to(torch.uint8)[pick]
    qz = (q.float() * 1e-3).to(torch.bfloat16)
    got2 = _run(qz, packed, sc2, indptr.tolist(), 3)
    want2 = ref.mla_decode_ref(_qbits(qz), packed.numpy(), sc2.numpy(), indptr.numpy(), SM)
    fin = np.isfinite(got2)
    err = np.abs(got2[fin] - want2[fin])
    assert np.all(err <= ATOL + RTOL * np.abs(want2[fin])), "bytes 253/254: a finite element is off"


def _two_token_logits(qrow, codes, kscales):
    """Logit probe: a two-token sequence whose second token is all zero codes
    (score 0, V = 0), so out[h, d] = w_h V1[d] with w_h = 1 / (1 + e^-z_h).
    Returns (z measured from the GPU output, z exact in fp64) per head."""
    codes = np.asarray(codes, dtype=np.uint8)
    row = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    packed = torch.from_numpy(np.stack([row, np.zeros(288, np.uint8)]))
    scales = torch.from_numpy(np.stack([np.asarray(kscales, np.uint8), np.full(18, 127, np.uint8)]))
    q = qrow.reshape(1, 16, 576)
    got = _run(q, packed, scales, [0, 2], 0)[0]
    k = ref.dequant_mxfp4(packed.numpy(), scales.numpy())[0]
    qf = _qbits(q).astype(np.uint32)
    qd = (qf << 16).view(np.float32).astype(np.float64).reshape(16, 576)
    z_exact = float(np.float32(SM)) * (qd @ k)
    d = int(np.argmax(np.abs(k[:512])))
    w = got[:, d] / k[d]
    return np.log(w / (1.0 - w)), z_exact, qd, k


def test_qk_error_bounds_of_the_scaled_mfma():
    """The latent half of QK runs on the MX-scaled MFMA with q split into
    e4m3 hi + lo parts (per 32-dim block). Two bounds are pinned:
    * accumulation: |z - z_exact| <= 1.2e-4 * sm * sum_j |q_j K_j| on rows
      whose terms cancel (sum |terms| * sm ~ 10^4, exact z = 0 or ~1);
    * the split: an element 2^-15 below its block's max is kept to within
      2^-20 * max |q_block| (here it carries the whole logit).
    z is read off a two-token softmax (resolution ~0.01)."""
    g = torch.Generator().manual_seed(31)
    res = 0.02
    # accumulation: pairs (2i, 2i+1) with equal q and K = +6, -6
    codes = np.tile(np.array([7, 15], dtype=np.uint8), 288)
    kscales = np.full(18, 133, dtype=np.uint8)          # 6 * 2^6 per element
    mag = torch.exp2(torch.randint(-6, 7, (16, 288), generator=g).float())
    sgn = torch.where(torch.rand(16, 288, generator=g) < 0.5, -1.0, 1.0)
    half = (mag * sgn).to(torch.bfloat16)
    qrow = torch.stack([half, half], dim=2).reshape(16, 576)
    # second row: one pair gets K = +6, +6 and q = 2^-5, for an exact logit of 1
    codes_off = codes.copy()
    codes_off[2 * 100 + 1] = 7
    for c, label in ((codes, "cancelling"), (codes_off, "offset")):
        q_use = qrow.clone()
        if label == "offset":
            q_use[:, 200] = q_use[:, 201] = torch.tensor(2.0 ** -5, dtype=torch.bfloat16)
        _say(f"case QK accumulation bound ({label})")
        z, z_exact, qd, k = _two_token_logits(q_use, c, kscales)
        terms = float(np.float32(SM)) * np.abs(qd * k[None, :]).sum(axis=1)
        assert np.all(terms > 5e3)
        assert np.all(np.abs(z_exact) < 3.0)
        bound = 1.2e-4 * terms + res
        assert np.all(np.abs(z - z_exact) <= bound), (label, np.abs(z - z_exact).max(), bound.min())
    # split: block 0 holds max 2^9 at dim 0 (K = 0 there) and a tiny element at dim 1
    _say("case QK split bound")
    codes = np.zeros(576, dtype=np.uint8)
    codes[1] = 7                                         # K[1] = 6 * 2^7
    kscales = np.full(18, 127, dtype=np.uint8)
    kscales[0] = 134
    tiny = torch.tensor([2.0 ** -6 * (1 + 2.0 ** -1 + 2.0 ** -7)], dtype=torch.bfloat16)
    qrow = torch.zeros(16, 576, dtype=torch.bfloat16)
    qrow[:, 0] = 2.0 ** 9
    qrow[:, 1] = tiny * torch.tensor([1.0 if h % 2 == 0 else -1.0 for h in range(16)]).to(torch.bfloat16)
    z, z_exact, qd, k = _two_token_logits(qrow, codes, kscales)
    assert np.all(np.abs(z_exact) > 0.5) and np.all(np.abs(z_exact) < 3.0)
    bound = 2.0 ** -20 * 2.0 ** 9 * abs(k[1]) * float(np.float32(SM)) + res
    assert np.all(np.abs(z - z_exact) <= bound), (np.abs(z - z_exact).max(), bound)


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


@pytest.mark.parametrize("lens,num_cus", [([120000, 300, 40000, 5], 600), ([160000, 300, 60000, 5], 300)])
def test_more_slots_than_workgroups(lens, num_cus):
    """Plans for more slots than the device has CUs (418 and 289): the grid
    stays at one workgroup per CU and each workgroup walks several slots
    (the first slot's item read with the header does not apply to the later
    ones). The 300-CU plan has item charges on (two short sequences)."""
    _say(f"case more slots than workgroups lens={lens} num_cus={num_cus}")
    q, packed, scales, indptr, _ = _small(lens, seed=31)
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    got = _run(q, packed, scales, indptr.tolist(), num_cus)
    _check(got, want, f"num_cus={num_cus}")


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


def _workload_check(name):
    """The workload at full size, in the benchmark's launch configuration
    (the device's CU count), every element of every sequence against the
    oracle."""
    w = synth.WORKLOADS[name]
    _say(f"case workload {name}: generating")
    q, packed, scales, indptr, lens = synth.make_inputs(w, device="cuda")
    dec = binding.MlaDecode(indptr.tolist(), device="cuda")
    _say(f"case workload {name}: decode T={indptr[-1].item()}")
    out = dec(q, packed, scales, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    qb = _qbits(q)
    ind = indptr.numpy()
    pk, sc = packed.cpu().numpy(), scales.cpu().numpy()
    worst = 0.0
    for b in range(len(lens)):
        lo, hi = int(ind[b]), int(ind[b + 1])
        want = ref.mla_decode_ref_seq(qb[b], pk[lo:hi], sc[lo:hi], w.sm_scale)
        worst = max(worst, _check(got[b], want, f"{name} b={b}"))
    _say(f"  {name}: {len(lens)} sequences, worst normwise {worst:.2e}")


def test_workload_b4_kv1024():
    _workload_check("b4_kv1024")


def test_workload_b1_kv65536():
    _workload_check("b1_kv65536")


def test_workload_b64_kv8192_tokscale():
    _workload_check("b64_kv8192_tokscale")


def test_workload_b256_kv8192():
    _workload_check("b256_kv8192")


def test_workload_b128_ragged():
    _workload_check("b128_ragged")


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
