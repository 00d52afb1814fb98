"""mla_verify_attention_noalloc (the entry point for callers that cannot
allocate: its split partials live in the library's static per-GPU scratch)
against mla_verify_attention with a caller workspace, through the C ABI: the
same kernels, so the results must agree bitwise, over consecutive calls that
shrink (each call must write every partial it reads back, whatever the
previous call left in the shared scratch)."""

import numpy as np
import pytest
import torch

import speculative_decoding_mla_amd as mv
from workloads import make_case
from workloads.gen import small_case
from tests.gpu_util import check_parity, device_case, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mv.load_library()


def _noalloc(case, dc, dev_err=None):
    b, t, h, _ = case.q.shape
    out = torch.full((b, t, h, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((b, t, h), 7.0, dtype=torch.float32, device="cuda")
    mv.verify_attention_noalloc(dc["q"], dc["kv"], dc["page_table"], dc["seq_lens"], dc["tree_parent"], out, lse,
                                dev_err, page_size=case.page_size, nsplit=case.nsplit, sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()


def test_noalloc_equals_workspace_call_on_shrinking_inputs():
    cases = [
        make_case("C3"),  # 65,536 keys, 256 rows, NSPLIT 128: 34 MB of partials
        make_case("C2"),  # 4,112 keys, 128 rows, NSPLIT 64, four column parts
        small_case(seed=801, batch=3, nodes=9, heads=8, contexts=[1000, 33, 2], page_size=4, nsplit=7),
    ]
    for case in cases:
        say(f"no-alloc vs workspace: {case.name} nsplit {case.nsplit}")
        dc = device_case(case)
        want_out, want_lse, err_ws = run_gpu(case, dc=dc)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        got_out, got_lse = _noalloc(case, dc, err)
        assert err_ws == 0 and int(err.item()) == 0
        assert np.array_equal(got_out, want_out), case.name
        assert np.array_equal(got_lse, want_lse), case.name
        check_parity(case, got_out, got_lse, label=f"no-alloc {case.name}")
        # and without an error word
        got_out2, got_lse2 = _noalloc(case, dc, None)
        assert np.array_equal(got_out2, want_out) and np.array_equal(got_lse2, want_lse)
        del dc
        torch.cuda.empty_cache()


def test_noalloc_reports_data_errors_to_the_callers_word():
    case = small_case(seed=802, batch=1, nodes=8, heads=8, contexts=[260], page_size=1, nsplit=4)
    pt = case.page_table.copy()
    pt[0, 77] = case.kv.shape[0] + 5  # past the pool: masked and flagged
    bad = case.with_(page_table=pt)
    dc = device_case(bad)
    want_out, want_lse, err_ws = run_gpu(bad, dc=dc)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got_out, got_lse = _noalloc(bad, dc, err)
    assert int(err.item()) & mv.DEVERR_SLOT_RANGE and err_ws & mv.DEVERR_SLOT_RANGE
    assert np.array_equal(got_out, want_out) and np.array_equal(got_lse, want_lse)


def test_noalloc_rejects_a_problem_past_the_scratch():
    case = small_case(seed=803, batch=1, nodes=4, heads=8, contexts=[100], page_size=1, nsplit=1)
    dc = device_case(case)
    b, t, h, _ = case.q.shape
    out = torch.empty((b, t, h, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, t, h), dtype=torch.float32, device="cuda")
    big_nsplit = 200_000  # 200,000 splits x 32 rows x 1 KiB > 64 MiB
    with pytest.raises(mv.MlaError) as ei:
        mv.verify_attention_noalloc(dc["q"], dc["kv"], dc["page_table"], dc["seq_lens"], dc["tree_parent"], out,
                                    lse, None, page_size=1, nsplit=big_nsplit, sm_scale=case.sm_scale)
    assert ei.value.status == -7
