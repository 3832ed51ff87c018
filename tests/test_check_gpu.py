"""MLA_CHECK=1: the device validation of seq_lens and of the used page-table entries that
runs before the decode. Valid inputs decode exactly as without the check; an out-of-range
length or used page id returns MLA_ERR_DEVICE_CHECK; entries past a sequence's last page are
not inspected (they may hold anything)."""
import os

import pytest
import torch

import workloads as W
from tests.gpu_helpers import gpu_decode, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    return need_gpu()


@pytest.fixture
def check_env():
    old = os.environ.get("MLA_CHECK")
    os.environ["MLA_CHECK"] = "1"
    yield
    if old is None:
        del os.environ["MLA_CHECK"]
    else:
        os.environ["MLA_CHECK"] = old


def _inp():
    return W.make_inputs(4, 128, 128, 512, 64, 128, [1, 65, 300, 128], 31)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu()


def test_valid_inputs_decode_as_without_check(M):
    d = to_dev(_inp())
    say("check: valid inputs")
    ref = gpu_decode(M, d)
    torch.cuda.synchronize()
    os.environ["MLA_CHECK"] = "1"
    try:
        got = gpu_decode(M, d)
    finally:
        del os.environ["MLA_CHECK"]
    torch.cuda.synchronize()
    assert torch.equal(_bits(got), _bits(ref))


@pytest.mark.parametrize("bad", ["page_high", "page_negative", "length_high", "length_negative"])
def test_out_of_range_inputs_are_reported(M, check_env, bad):
    inp = _inp()
    pt, sl = inp["page_table"].clone(), inp["seq_lens"].clone()
    if bad == "page_high":
        pt[2, 3] = inp["kv_pages"].shape[0]      # page 3 of a 300-token sequence is used
    elif bad == "page_negative":
        pt[1, 1] = -1                            # page 1 of a 65-token sequence is used
    elif bad == "length_high":
        sl[0] = pt.shape[1] * 64 + 1
    else:
        sl[3] = -5
    inp["page_table"], inp["seq_lens"] = pt, sl
    say("check:", bad)
    with pytest.raises(M.MlaError) as e:
        gpu_decode(M, to_dev(inp))
    assert M.STATUS[e.value.code] == "MLA_ERR_DEVICE_CHECK"


def test_unused_entries_are_not_inspected(M, check_env):
    inp = _inp()
    pt = inp["page_table"].clone()
    pt[0, 1:] = -7        # a 1-token sequence uses page 0 only
    pt[1, 2:] = 1 << 30   # a 65-token sequence uses pages 0 and 1
    inp["page_table"] = pt
    say("check: unused entries")
    out = gpu_decode(M, to_dev(inp))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
