"""C-ABI checks that need no GPU: exported symbols and the host planner."""

import ctypes
import os
import random
import re

import pytest

from mla_mxfp4_kv_amd import binding
from oracle.planner_ref import plan_words_ref, workspace_bound_ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "mla_mxfp4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    names = _header_functions()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
        assert isinstance(getattr(L, n), ctypes._CFuncPtr)


def test_status_strings():
    assert binding.status_string(0) == "MLA_OK"
    assert binding.status_string(-2) == "MLA_ERR_WORKSPACE"
    assert binding.status_string(-5) == "MLA_ERR_NOT_PLANNED"
    assert binding.status_string(7) == "MLA_ERR_UNKNOWN"


def _random_indptrs(n, seed):
    rng = random.Random(seed)
    for _ in range(n):
        b_n = rng.randint(0, 60)
        base = rng.choice([0, 0, rng.randint(0, 5000)])
        ind = [base]
        for _ in range(b_n):
            ind.append(ind[-1] + rng.choice([0, 1, 7, rng.randint(0, 400), rng.randint(0, 40000)]))
        yield ind, rng.choice([1, 2, 5, 7, 64, 255, 256, 304, 1024])


def test_host_plan_bit_exact_random():
    for ind, cus in _random_indptrs(400, 1):
        want, need = plan_words_ref(ind, len(ind) - 1, cus)
        got, got_need = binding.plan_host(ind, cus)
        assert got == want, (ind[:6], cus)
        assert got_need == need
        assert need <= binding.workspace_bytes(len(ind) - 1, ind[-1] - ind[0], cus)
        assert binding.workspace_bytes(len(ind) - 1, ind[-1] - ind[0], cus) == \
            workspace_bound_ref(len(ind) - 1, ind[-1] - ind[0], cus)


def test_host_plan_bit_exact_workloads():
    from mla_mxfp4_kv_amd import synth
    for w in synth.WORKLOADS.values():
        lens = synth.seq_lengths(w)
        ind = [0]
        for n in lens:
            ind.append(ind[-1] + n)
        for cus in (1, 7, 64, 256):
            assert binding.plan_host(ind, cus) == plan_words_ref(ind, len(lens), cus)


@pytest.mark.parametrize("ind,cus", [([0, 5, 3], 4), ([-1, 5], 4), ([0, 5], 0)])
def test_host_plan_rejects_bad_input(ind, cus):
    with pytest.raises(binding.MlaError) as e:
        binding.plan_host(ind, cus)
    assert e.value.status == -1


def test_host_plan_reports_small_buffer():
    L = binding.lib()
    arr = (ctypes.c_int32 * 3)(0, 500, 900)
    n, need = ctypes.c_size_t(0), ctypes.c_size_t(0)
    words = (ctypes.c_int32 * 4)()
    st = L.mla_plan_host(arr, 2, 2, words, 4, ctypes.byref(n), ctypes.byref(need))
    assert st == -2 and n.value > 4
    assert b"too small" in L.mla_last_error()


def test_workspace_bytes_rejects_bad_sizes():
    with pytest.raises(binding.MlaError):
        binding.workspace_bytes(-1, 10, 4)
    with pytest.raises(binding.MlaError):
        binding.workspace_bytes(1, -10, 4)
    # a layout whose partial outputs would start past the int32 byte offsets
    # of a plan (the GPU-side planner refuses the same layout); only the
    # start is an int32 word, so a large partial area itself is fine
    with pytest.raises(binding.MlaError):
        binding.workspace_bytes(2 ** 31 - 1, 2 ** 31 - 1, 256)
    assert binding.workspace_bytes(10 ** 6, 2 ** 31 - 1, 256) > 0
    assert binding.workspace_bytes(1, 2 ** 31 - 1, 2 ** 20) > 2 ** 31


def test_host_plan_at_the_int32_token_limit():
    """Offsets up to 2^31 - 1 (the largest int32 kv_indptr): the plan words
    still equal the planner oracle's, split over every CU count tried."""
    for ind in ([0, 2 ** 30, 2 ** 31 - 1], [5, 2 ** 31 - 1], [0, 1, 2 ** 31 - 2, 2 ** 31 - 1]):
        for cus in (1, 256):
            assert binding.plan_host(ind, cus) == plan_words_ref(ind, len(ind) - 1, cus)


def test_host_plan_matches_oracle_property():
    """Property test: any non-decreasing int32 offsets (bases and lengths up
    to the int32 limit, empty sequences, lengths near chunk edges) plan to
    the oracle's words on any CU count."""
    from hypothesis import given, settings, HealthCheck, strategies as st

    lens_st = st.lists(st.one_of(st.integers(0, 300), st.integers(0, 2 ** 20),
                                 st.sampled_from([127, 128, 129, 255, 256, 257, 8192])), min_size=0, max_size=40)

    @settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
    @given(lens=lens_st, base=st.one_of(st.just(0), st.integers(0, 2 ** 31 - 1)), cus=st.integers(1, 300))
    def check(lens, base, cus):
        ind = [base]
        for n in lens:
            ind.append(ind[-1] + n)
        if ind[-1] > 2 ** 31 - 1:
            return
        assert binding.plan_host(ind, cus) == plan_words_ref(ind, len(lens), cus)

    check()


def test_decode_on_an_unplanned_workspace_is_refused_without_a_device():
    """The plan registry is consulted before any HIP call: a workspace
    address that was never planned (or was released) gives
    MLA_ERR_NOT_PLANNED, for every decode entry point, with no GPU."""
    L = binding.lib()
    fake = ctypes.c_void_p(0x7F0000100000)
    p = [ctypes.c_void_p(0x7F0000200000 + 256 * i) for i in range(8)]
    calls = {
        "mla_decode_mxfp4": (p[0], p[1], p[2], p[3], p[4], ctypes.c_float(0.1), fake, None),
        "mla_decode_fp8": (p[0], p[1], p[2], p[3], p[4], ctypes.c_float(0.1), fake, None),
        "mla_decode_bf16": (p[0], p[1], p[3], p[4], ctypes.c_float(0.1), fake, None),
        "mla_decode_mxfp4_paged": (p[0], p[1], p[2], p[5], p[3], p[4], ctypes.c_float(0.1), fake, None),
        "mla_decode_mxfp4_starts": (p[0], p[1], p[2], p[5], p[3], p[4], ctypes.c_float(0.1), fake, None),
    }
    for name, args in calls.items():
        assert getattr(L, name)(*args) == -5, name
        assert b"not prepared" in L.mla_last_error()
    assert L.mla_plan_release(fake) == -5
    assert b"no plan" in L.mla_last_error()
