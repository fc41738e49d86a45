"""The debug build (libhca_debug.so, -DHCA_DEBUG) on the GPU: the same kernels
with index checks.  A clean call records nothing and gives the release build's
bytes; an unmapped page, a page id past the pool and a selected entry past the
sequence are skipped as the release build skips them, and each sets its bit
in hca_debug_status (1 page, 4 selected entry), with no fault.
"""

import contextlib
import os

import numpy as np
import pytest
import torch

import synth
from tests import helpers as H
from tests.test_gpu_parity import _attn_workload, _run_attn

pytestmark = pytest.mark.gpu

hca = pytest.importorskip("decode_attention_compressed_amd")

DEBUG_LIB = os.path.join(os.path.dirname(hca.__file__), "libhca_debug.so")
OK, INVALID = 0, 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(DEBUG_LIB):
        pytest.fail(f"{DEBUG_LIB} is missing: build it with `python -m decode_attention_compressed_amd.build --debug`")
    hca.lib()


@contextlib.contextmanager
def debug_library():
    """The binding's calls go to the debug build inside the block (both builds stay loaded)."""
    saved = hca._lib, hca.LIB_PATH
    hca._lib, hca.LIB_PATH = None, DEBUG_LIB
    try:
        assert hca.version().endswith(" debug")
        assert hca.debug_status() == (OK, 0)  # a clean start
        yield
    finally:
        hca._lib, hca.LIB_PATH = saved


def _c4a(d=512):
    kind = synth.LayerKind("c4a", 4, 64, "fp8", 128)
    return H.SeqData(_attn_workload("fp8", d, 16, 128, kind, 2), 0, [1000, 300])


def test_release_build_reports_unsupported():
    assert not hca.version().endswith(" debug")
    assert hca.debug_status() == (2, 0)  # HCA_ERR_UNSUPPORTED: the release build records nothing


def test_clean_call_records_nothing_and_matches_release():
    H.flush("debug build: clean attention call")
    sd = _c4a()
    sel = [np.arange(0, 250, 3), np.arange(0, 75, 2)]
    base = _run_attn(sd, sel, 128, fp8="both")
    with debug_library():
        got = _run_attn(sd, sel, 128, fp8="both")
        assert hca.debug_status() == (OK, 0)
    for a, b in zip(base, got):
        assert np.array_equal(a, b)


def test_selected_entry_past_the_sequence_sets_bit_4():
    H.flush("debug build: selected entry out of range")
    sd = _c4a()
    good = np.arange(0, 250, 5)
    sel = [np.concatenate([good, [-3, 250, 10 ** 6]]), np.arange(0, 75, 2)]
    base = _run_attn(sd, sel, 128, fp8="both")
    with debug_library():
        got = _run_attn(sd, sel, 128, fp8="both")
        st, bits = hca.debug_status()
    assert st == INVALID and bits == 4
    for a, b in zip(base, got):  # the same rows skipped as in the release build
        assert np.array_equal(a, b)


@pytest.mark.parametrize("bad", [-1, 10 ** 6])
def test_page_outside_the_pool_sets_bit_1(bad):
    H.flush(f"debug build: page id {bad}")
    sd = _c4a()
    table = sd.table.copy()
    table[0, 1] = bad  # entries 64 .. 127 of sequence 0
    sel = [np.arange(0, 250, 3), np.arange(0, 75, 2)]
    base = _run_attn(sd, sel, 128, fp8="both", table=table)
    with debug_library():
        got = _run_attn(sd, sel, 128, fp8="both", table=table)
        st, bits = hca.debug_status()
        assert hca.debug_status() == (OK, 0)  # read and cleared
    assert st == INVALID and bits == 1
    for a, b in zip(base, got):
        assert np.array_equal(a, b)
