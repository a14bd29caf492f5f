"""Host logic of the build: the scratch-memory guard reads hipcc's resource-usage remarks."""
from gqa_attention_rope_amd import build

REMARKS = """\
remark: decode.hip:10:0: Function Name: kernel_a [-Rpass-analysis=kernel-resource-usage]
remark: decode.hip:10:0:     VGPRs: 151 [-Rpass-analysis=kernel-resource-usage]
remark: decode.hip:10:0:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
remark: decode.hip:20:0: Function Name: kernel_b [-Rpass-analysis=kernel-resource-usage]
remark: decode.hip:20:0:     ScratchSize [bytes/lane]: 72 [-Rpass-analysis=kernel-resource-usage]
remark: prefill.hip:5:0: Function Name: kernel_c
remark: prefill.hip:5:0:     ScratchSize [bytes/lane]: 8
"""


def test_scratch_guard_names_only_kernels_with_scratch():
    assert build.kernels_using_scratch(REMARKS) == [("kernel_b", 72), ("kernel_c", 8)]


def test_scratch_guard_accepts_clean_builds():
    assert build.kernels_using_scratch("") == []
    clean = "\n".join(l for l in REMARKS.splitlines() if "72" not in l and ": 8" not in l)
    assert build.kernels_using_scratch(clean) == []
