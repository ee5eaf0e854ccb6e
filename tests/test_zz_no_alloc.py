"""The entry point that allocates nothing (mla_decode_mxfp4_noalloc), for
callers that cannot allocate device memory: its plan words and partials live
in the library's static device scratch. Checked through the C ABI against
mla_decode_mxfp4 on a planned workspace (same plan rule, so the same bits)
and against the oracle, on two calls in a row, the second smaller."""

import ctypes
import math
import sys

import numpy as np
import pytest
import torch

from mla_mxfp4_kv_amd import binding, synth
from oracle import mxfp4_ref as ref

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(576.0)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _fn():
    L = binding.lib()
    f = L.mla_decode_mxfp4_noalloc
    f.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]
    f.restype = ctypes.c_int
    return f


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _qbits(q):
    return q.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    yield


def test_noalloc_matches_the_workspace_entry_point():
    f = _fn()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for k, lens in enumerate(([37, 1025, 0, 300, 2000, 4097, 1], [5, 400])):
        _say(f"case noalloc call {k} lens={lens}")
        w = synth.Workload("na", len(lens), None, None, 1.0, False, 60 + k)
        q, packed, scales, indptr, _ = synth.make_inputs(w, lengths=lens)
        q, packed, scales = q.cuda(), packed.cuda(), scales.cuda()
        ind_dev = indptr.cuda()
        out = torch.full((len(lens), 16, 512), 9.0, dtype=torch.bfloat16, device="cuda")
        st = f(_p(q), _p(packed), _p(scales), _p(ind_dev), len(lens), _p(out), SM, stream)
        assert st == 0, binding.lib().mla_last_error()
        dec = binding.MlaDecode(indptr.tolist(), device="cuda")
        want_ws = dec(q, packed, scales, sm_scale=SM)
        torch.cuda.synchronize()
        assert torch.equal(out, want_ws), f"call {k}: differs from mla_decode_mxfp4"
        want = ref.mla_decode_ref(_qbits(q), packed.cpu().numpy(), scales.cpu().numpy(), indptr.numpy(), SM)
        got = out.float().cpu().numpy()
        err = np.abs(got - want)
        assert np.all(err <= 1e-2 + 1e-2 * np.abs(want)), f"call {k}: max err {float(err.max()):.3e}"
        assert np.all(got[[i for i, n in enumerate(lens) if n == 0]] == 0)


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    f = _fn()
    ind = torch.zeros(2, dtype=torch.int32, device="cuda")
    buf = torch.zeros(1024, dtype=torch.uint8, device="cuda")   # never read: the size check comes first
    st = f(_p(buf), _p(buf), _p(buf), _p(ind), 10 ** 7, _p(buf), SM, None)
    assert st == -2
    assert b"static scratch" in binding.lib().mla_last_error()
