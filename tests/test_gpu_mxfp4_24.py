"""GPU parity of the 24-scale MXFP4 decode (mla_decode_mxfp4_24) against the
fp64 oracle of that layout (oracle.mxfp4_24_ref), through the C ABI.

Bar (per element, bf16 output): |gpu - ref| <= 1e-2 + 1e-2 * |ref|, plus the
normwise gate ||gpu - ref|| / ||ref|| <= 5e-3."""

import math
import sys

import numpy as np
import pytest
import torch

from mla_mxfp4_kv_amd import binding, synth
from oracle import mxfp4_24_ref as r24
from oracle import mxfp4_ref as ref

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(576.0)
ATOL = 1e-2
RTOL = 1e-2
NORMWISE = 5e-3
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


def _check(got, want, label):
    assert got.shape == want.shape
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan_w), f"{label}: NaN pattern differs"
    g, w = got[~nan_w], want[~nan_w]
    err = np.abs(g - w)
    bound = ATOL + RTOL * np.abs(w)
    assert np.all(err <= bound), f"{label}: max excess {float(np.max(err - bound)) if err.size else 0:.3e}"
    den = np.linalg.norm(w)
    if den > 0:
        nw = np.linalg.norm(g - w) / den
        assert nw <= NORMWISE, f"{label}: normwise {nw:.3e}"
        return nw
    return 0.0


def _inputs(lens, seed, q_std=1.0, token_scale=False):
    w = synth.Workload("s24", len(lens), None, None, q_std, token_scale, seed)
    return synth.make_inputs(w, lengths=lens, block=24)


def _run(q, packed, scales, indptr, num_cus=0, sm=SM):
    dec = binding.MlaDecode(indptr, device="cuda", num_cus=num_cus)
    out = dec.mxfp4_24(q.cuda(), packed.cuda(), scales.cuda(), sm_scale=sm)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


CASES = [
    ([1], 0),
    ([2, 3], 0),
    ([31, 32, 33], 0),
    ([127, 128, 129], 3),
    ([0, 300, 0, 1000], 0),
    ([5000], 0),
    ([1, 1, 1, 1, 700], 7),
    ([257, 4097, 33, 2000], 0),
    ([9000, 300, 17000, 1], 5),
]


@pytest.mark.parametrize("lens,num_cus", CASES)
def test_small_cases_match_oracle(lens, num_cus):
    _say(f"case 24-scale lens={lens} num_cus={num_cus}")
    q, packed, scales, indptr, _ = _inputs(lens, seed=len(lens) + sum(lens))
    assert scales.shape[1] == 24
    got = _run(q, packed, scales, indptr.tolist(), num_cus)
    want = r24.mla_decode_ref_24(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    _check(got, want, f"lens={lens}")


def test_more_slots_than_workgroups():
    """A plan for 600 slots on a device with fewer CUs: each workgroup walks
    several slots."""
    _say("case 24-scale more slots than workgroups")
    q, packed, scales, indptr, _ = _inputs([120000, 300, 40000, 5], seed=31)
    got = _run(q, packed, scales, indptr.tolist(), num_cus=600)
    want = r24.mla_decode_ref_24(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    _check(got, want, "600 slots")


def test_one_token_is_exact():
    """One token: p = 1, so the output is that token's V (bf16-exact)."""
    _say("case 24-scale one-token exactness")
    q, packed, scales, indptr, _ = _inputs([1] * 9, seed=5, q_std=3.0, token_scale=True)
    got = _run(q, packed, scales, indptr.tolist())
    v = r24.dequant_mxfp4_24(packed.numpy(), scales.numpy())[:, :512]
    assert np.array_equal(got, np.repeat(v[:, None, :], 16, axis=1))


def test_split_and_permutation_invariance():
    _say("case 24-scale split / permutation invariance")
    lens = [9000, 300, 17000, 1]
    q, packed, scales, indptr, _ = _inputs(lens, seed=8)
    want = r24.mla_decode_ref_24(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    outs = []
    for cus in (1, 7, 64, 0):
        got = _run(q, packed, scales, indptr.tolist(), cus)
        _check(got, want, f"cus={cus}")
        outs.append(got)
    for o in outs[1:]:
        assert np.linalg.norm(o - outs[0]) / np.linalg.norm(outs[0]) <= PAIRWISE
    perm = torch.randperm(9000, generator=torch.Generator().manual_seed(2))
    pk, sc = packed.clone(), scales.clone()
    pk[:9000] = packed[:9000][perm]
    sc[:9000] = scales[:9000][perm]
    got = _run(q, pk, sc, indptr.tolist())
    assert np.linalg.norm(got[0] - outs[0][0]) / np.linalg.norm(outs[0][0]) <= PAIRWISE


def test_zero_and_negative_sm_scale():
    lens = [37, 300, 1025, 5]
    q, packed, scales, indptr, _ = _inputs(lens, seed=17)
    for sm in (0.0, -0.0, -SM, -3.0 * SM):
        _say(f"case 24-scale sm_scale={sm!r}")
        got = _run(q, packed, scales, indptr.tolist(), 3, sm=sm)
        want = r24.mla_decode_ref_24(_qbits(q), packed.numpy(), scales.numpy(), indptr.numpy(),
                                     float(np.float32(sm)))
        _check(got, want, f"sm={sm!r}")


def test_wide_scale_range_and_block_edges():
    """E8M0 bytes 100..160 drawn per block, so neighbouring 24-element blocks
    inside one 32-dim fragment differ widely. The bf16 rounding of P bounds
    the per-element error by 2^-8 max_t |V[t, d]| on top of the bar (tokens
    cancel where |V| is far above the output)."""
    _say("case 24-scale wide scale range")
    g = torch.Generator().manual_seed(41)
    lens = [64, 333, 1500]
    q, packed, _, indptr, _ = _inputs(lens, seed=41)
    scales = torch.randint(100, 161, (int(indptr[-1]), 24), generator=g).to(torch.uint8)
    qs = (q.float() * 2.0 ** -12).to(torch.bfloat16)
    got = _run(qs, packed, scales, indptr.tolist())
    want = r24.mla_decode_ref_24(_qbits(qs), packed.numpy(), scales.numpy(), indptr.numpy(), SM)
    v = np.abs(r24.dequant_mxfp4_24(packed.numpy(), scales.numpy())[:, :512])
    ind = indptr.numpy()
    vmax = np.stack([v[ind[b]:ind[b + 1]].max(axis=0) for b in range(len(lens))])[:, None, :]
    assert np.all(np.isfinite(got))
    bound = ATOL + RTOL * np.abs(want) + 2.0 ** -8 * vmax
    err = np.abs(got - want)
    assert np.all(err <= bound), f"max excess {float(np.max(err - bound)):.3e}"


@pytest.mark.parametrize("k", [0, 5, 21, 23])
def test_nan_scale_poisons_only_its_sequence(k):
    _say(f"case 24-scale NaN byte in block {k}")
    q, packed, scales, indptr, _ = _inputs([300, 200, 500], seed=4)
    scales = scales.clone()
    scales[300 + 57, k] = 255
    got = _run(q, packed, scales, indptr.tolist(), 4)
    assert np.all(np.isnan(got[1]))
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[2]))


def test_agrees_with_the_18_scale_decode_on_shared_values():
    """Scale bytes constant over 96-element spans (the common multiple of 24
    and 32) give the same values in both layouts: the two decodes agree with
    each other (normwise 2^-8) and both match the oracle.

    The bytes reach 2^-7..2^7, so |V| runs far above the outputs where the
    tokens cancel: as in test_wide_scale_range, the bf16 rounding of P (the
    pages' own precision for P) adds up to 2^-8 max_t |V[t, d]| per element
    on top of the bar. q is scaled by 2^-4 (exact), so that the scores' MX
    accumulation error (<= 1.2e-4 x sum |q_j K_j|, pinned below) stays far
    below that term while a wrong block's scale would still move the scores
    by orders of magnitude."""
    _say("case 24-scale vs 18-scale on the same values")
    lens = [700, 33, 2100]
    q, packed, _, indptr, _ = _inputs(lens, seed=23)
    q = (q.float() * 2.0 ** -4).to(torch.bfloat16)
    t = int(indptr[-1])
    g = torch.Generator().manual_seed(23)
    span = torch.randint(120, 135, (t, 6), generator=g).to(torch.uint8)
    s24 = span.repeat_interleave(4, dim=1).contiguous()   # 24 bytes per token, 4 per 96 dims
    s18 = span.repeat_interleave(3, dim=1).contiguous()   # 18 bytes per token, 3 per 96 dims
    assert np.array_equal(r24.dequant_mxfp4_24(packed.numpy(), s24.numpy()),
                          ref.dequant_mxfp4(packed.numpy(), s18.numpy()))
    got24 = _run(q, packed, s24, indptr.tolist())
    dec = binding.MlaDecode(indptr.tolist(), device="cuda")
    got18 = dec(q.cuda(), packed.cuda(), s18.cuda(), sm_scale=SM).float().cpu().numpy()
    want = ref.mla_decode_ref(_qbits(q), packed.numpy(), s18.numpy(), indptr.numpy(), SM)
    v = np.abs(ref.dequant_mxfp4(packed.numpy(), s18.numpy())[:, :512])
    ind = indptr.numpy()
    vmax = np.stack([v[ind[b]:ind[b + 1]].max(axis=0) for b in range(len(lens))])[:, None, :]
    bound = ATOL + RTOL * np.abs(want) + 2.0 ** -8 * vmax
    for got, label in ((got24, "24-scale"), (got18, "18-scale")):
        assert np.all(np.isfinite(got)), label
        err = np.abs(got - want)
        assert np.all(err <= bound), f"{label}: max excess {float(np.max(err - bound)):.3e}"
        assert np.linalg.norm(got - want) / np.linalg.norm(want) <= NORMWISE, label
    assert np.linalg.norm(got24 - got18) / np.linalg.norm(want) <= PAIRWISE


def test_scale_rows_at_an_8_byte_offset_and_errors():
    """kv_scale 8 bytes past a 16-byte boundary (the chunks covering a tile's
    scale rows then start mid-chunk) gives the same bits; a kv_scale that is
    not 8-byte aligned is refused."""
    _say("case 24-scale scale offsets / errors")
    lens = [37, 300, 1, 1025, 64, 0, 95]
    q, packed, scales, indptr, _ = _inputs(lens, seed=11)
    base = _run(q, packed, scales, indptr.tolist(), 5)
    buf = torch.full((scales.numel() + 64,), 255, dtype=torch.uint8, device="cuda")
    view = buf[8:8 + scales.numel()].view(scales.shape)
    view.copy_(scales.cuda())
    assert view.data_ptr() % 16 == 8
    got = _run(q, packed, view, indptr.tolist(), 5)
    assert np.array_equal(got, base)
    dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=5)
    out = torch.empty(len(lens), 16, 512, dtype=torch.bfloat16, device="cuda")
    odd = buf[4:4 + scales.numel()].view(scales.shape)
    with pytest.raises(binding.MlaError) as e:
        binding.decode_mxfp4_24(q.cuda(), packed.cuda(), odd, dec.kv_indptr, out, SM, dec.workspace)
    assert e.value.status == -1


def test_hip_graph_capture_replays():
    _say("case 24-scale graph replay")
    lens = [37, 1025, 0, 300, 2000]
    q, packed, scales, indptr, _ = _inputs(lens, seed=9)
    q, packed, scales = q.cuda(), packed.cuda(), scales.cuda()
    dec = binding.MlaDecode(indptr.tolist(), device="cuda", num_cus=7)
    out = torch.empty(len(lens), 16, 512, dtype=torch.bfloat16, device="cuda")
    eager = dec.mxfp4_24(q, packed, scales, out=torch.empty_like(out), sm_scale=SM).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dec.mxfp4_24(q, packed, scales, out=out, sm_scale=SM)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dec.mxfp4_24(q, packed, scales, out=out, sm_scale=SM)
    for rep in range(3):
        out.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workloads_every_sequence(name):
    """The five workloads at full size with their latent rows encoded in the
    24-scale layout, every element of every sequence against the oracle."""
    w = synth.WORKLOADS[name]
    _say(f"case 24-scale workload {name}: generating")
    q, packed, scales, indptr, lens = synth.make_inputs(w, device="cuda", block=24)
    dec = binding.MlaDecode(indptr.tolist(), device="cuda")
    _say(f"case 24-scale workload {name}: decode T={int(indptr[-1])}")
    got = dec.mxfp4_24(q, packed, scales, sm_scale=w.sm_scale).float().cpu().numpy()
    assert np.all(np.isfinite(got))
    qb = _qbits(q)
    ind = indptr.numpy()
    pk, sc = packed.cpu().numpy(), scales.cpu().numpy()
    worst = 0.0
    for b in range(len(lens)):
        lo, hi = int(ind[b]), int(ind[b + 1])
        want = r24.mla_decode_ref_24_seq(qb[b], pk[lo:hi], sc[lo:hi], w.sm_scale)
        worst = max(worst, _check(got[b], want, f"{name} b={b}"))
    _say(f"  24-scale {name}: {len(lens)} sequences, worst normwise {worst:.2e}")


def test_qk_accumulation_bound_of_the_padded_blocks():
    """The scores run on the MX-scaled MFMA with every 24-element block padded
    to a 32-element MX block. A two-token sequence whose second token has
    zero codes (score 0, V = 0) gives out[h, d] = w_h V1[d] with
    w_h = 1 / (1 + e^-z_h), so each head's logit z is read off the output.
    Rows whose terms cancel in pairs (K = +6, -6 at 2^6, equal q in a pair,
    exact z = 0) hold |z| <= 1.2e-4 * sm * sum_j |q_j K_j| + resolution, the
    bound the 18-scale decode pins for the same matrix core; a second row
    with one pair made equal (+6, +6) and q = 2^-5 there has exact z ~ 0.8."""
    g = torch.Generator().manual_seed(37)
    res = 0.02
    codes = np.tile(np.array([7, 15], dtype=np.uint8), 288)        # +6, -6, +6, ...
    kscales = np.full(24, 133, dtype=np.uint8)                    # 2^6
    mag = torch.exp2(torch.randint(-6, 7, (16, 288), generator=g).float())
    sgn = torch.where(torch.rand(16, 288, generator=g) < 0.5, -1.0, 1.0)
    half = (mag * sgn).to(torch.bfloat16)
    qrow = torch.stack([half, half], dim=2).reshape(16, 576)
    codes_off = codes.copy()
    codes_off[2 * 100 + 1] = 7
    for c, label in ((codes, "cancelling"), (codes_off, "offset")):
        _say(f"case 24-scale QK accumulation bound ({label})")
        q_use = qrow.clone()
        if label == "offset":
            q_use[:, 200] = q_use[:, 201] = torch.tensor(2.0 ** -5, dtype=torch.bfloat16)
        row = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)
        packed = torch.from_numpy(np.stack([row, np.zeros(288, np.uint8)]))
        scales = torch.from_numpy(np.stack([kscales, np.full(24, 127, np.uint8)]))
        got = _run(q_use.reshape(1, 16, 576), packed, scales, [0, 2])[0]
        k = r24.dequant_mxfp4_24(packed.numpy(), scales.numpy())[0]
        qd = (_qbits(q_use.reshape(1, 16, 576)).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        qd = qd.reshape(16, 576)
        z_exact = float(np.float32(SM)) * (qd @ k)
        d = int(np.argmax(np.abs(k[:512])))
        w = got[:, d] / k[d]
        z = np.log(w / (1.0 - w))
        terms = float(np.float32(SM)) * np.abs(qd * k[None, :]).sum(axis=1)
        assert np.all(terms > 5e3) and np.all(np.abs(z_exact) < 3.0)
        bound = 1.2e-4 * terms + res
        assert np.all(np.abs(z - z_exact) <= bound), (label, float(np.abs(z - z_exact).max()), float(bound.min()))
