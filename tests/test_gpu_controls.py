"""Planted controls on the GPU: each control build (the library compiled with one planted
mistake, -DWA_CONTROL=k) must fail the strict interval on the 12B decode or the 12B prompt
chunk, where the product library passes it on the same inputs.

After TensorFold pull request #1123, "Receipt", kernel-contract bullet (six controls, each red
at the strict gate): the window one key early (decode; p32 prompt), the merge without
exp(m_c - M), the merge rounding toward zero, rows ignoring an image's last key, and P rounded
to one bf16 under the p32 interval. The strict tier is fp32-tight: w = (e_P + 2**-16) S.
"""

import functools

import pytest

from oracle import check
from sliding_window_gqa_amd import api, build, workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# control -> (form, workload, what it plants)
CONTROLS = {
    1: ("decode", "window one key early"),
    2: ("prompt", "window one key early (p32 prompt)"),
    3: ("decode", "merge without exp(m_c - M)"),
    4: ("decode", "merge rounding toward zero"),
    5: ("prompt", "rows ignoring an image's last key"),
    6: ("prompt", "P as one bf16 under p32"),
}


@functools.lru_cache(maxsize=None)
def _inputs(form):
    """12B decode (64 rows, 3 streams) or 12B prompt chunk (p32, image rows 40..300), with
    the oracle's values."""
    if form == "decode":
        case = workloads.decode_12b()
        x, S, _ = gu.oracle_decode(case)
        return case, x, S, check.E_P_FP32
    case = workloads.prompt_12b()
    x, S, _ = gu.oracle_prompt(case)
    return case, x, S, check.E_P_P32


def _run(form, case):
    return gu.run_decode(case) if form == "decode" else gu.run_prompt(case)


@pytest.mark.parametrize("k", sorted(CONTROLS))
def test_control_build_goes_red(k):
    form, what = CONTROLS[k]
    case, x, S, e_p = _inputs(form)
    gu.log(f"control {k}: {what} on the {case.name}")
    good = check.report(_run(form, case), x, S, e_p)
    L = api.load_library(build.control_lib(k))
    with api.using(L):
        bad = check.report(_run(form, case), x, S, e_p)
    gu.log(f"  product: tierS_fail={good['tier_S_fail']} tierG_fail={good['tier_G_fail']}; "
           f"control: tierS_fail={bad['tier_S_fail']} tierG_fail={bad['tier_G_fail']} "
           f"of {bad['n']}")
    assert good["tier_S_fail"] == 0 and good["tier_G_fail"] == 0
    assert bad["tier_S_fail"] > 0, f"control {k} ({what}) stays green"
