"""Host-side build logic: the resource-report parser that rejects kernels using scratch."""
from weight_only_quantized_mpgemm_amd import build

REPORT = """\
k.hip:27:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]
k.hip:27:1: remark:     VGPRs: 27 [-Rpass-analysis=kernel-resource-usage]
k.hip:27:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:43:1: remark: Function Name: _Z3barPf [-Rpass-analysis=kernel-resource-usage]
k.hip:43:1: remark:     ScratchSize [bytes/lane]: 488 [-Rpass-analysis=kernel-resource-usage]
k.hip:60:1: remark: Function Name: _Z3bazPf [-Rpass-analysis=kernel-resource-usage]
k.hip:60:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_users_names_only_spilling_kernels():
    assert build.scratch_users(REPORT) == [("_Z3barPf", 488)]


def test_scratch_users_empty_report():
    assert build.scratch_users("") == []
