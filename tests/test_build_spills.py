"""The build's refusal of kernels that spill VGPRs: the parser of the
compiler's kernel-resource-usage remarks."""
from draft_token_verification_flattened_amd import build

REMARKS = """\
verify.hip:790:1: remark: Function Name: _ZN5specv13verify_decideILi0ELi1ELb0ELi1024EEEvNS_10VerifyArgsE [-Rpass-analysis=kernel-resource-usage]
verify.hip:790:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]
verify.hip:790:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
verify.hip:790:1: remark:     SGPRs Spill: 56 [-Rpass-analysis=kernel-resource-usage]
verify.hip:790:1: remark:     VGPRs Spill: 6 [-Rpass-analysis=kernel-resource-usage]
verify.hip:260:1: remark: Function Name: _ZN5specv13verify_streamILi0ELi1ELb1EEEvNS_10VerifyArgsE [-Rpass-analysis=kernel-resource-usage]
verify.hip:260:1: remark:     VGPRs: 101 [-Rpass-analysis=kernel-resource-usage]
verify.hip:260:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
verify.hip:260:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_spills_found_per_kernel():
    got = build.vgpr_spills(REMARKS)
    assert got == {"_ZN5specv13verify_decideILi0ELi1ELb0ELi1024EEEvNS_10VerifyArgsE": 6}


def test_sgpr_spills_and_clean_kernels_pass():
    # SGPR spills go to VGPR lanes (no scratch); a kernel without VGPR spills passes
    assert build.vgpr_spills(REMARKS.split("verify.hip:260")[0].replace("VGPRs Spill: 6", "VGPRs Spill: 0")) == {}
    assert build.vgpr_spills("") == {}
