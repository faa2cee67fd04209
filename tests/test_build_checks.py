"""Host-side checks of the build: the reading of the compiler's kernel resource report that keeps
scratch memory out of the latent comparator's kernels."""
from value_only_kv_amd import _build as B


def test_scratch_report_parsing():
    rep = "\n".join([
        "k.hip:1:1: remark: Function Name: kA [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:1:1: remark:     VGPRs: 398 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:1:1: remark: Function Name: kB [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:1:1: remark:     ScratchSize [bytes/lane]: 304 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert B.scratch_users(rep) == ["kB"]
    assert B.scratch_users("") == []


def test_latent_source_is_checked():
    assert "k_latent.hip" in B.NO_SCRATCH
    assert "-Rpass-analysis=kernel-resource-usage" in B.HIP_FILE_FLAGS["k_latent.hip"]
