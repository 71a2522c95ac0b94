"""Host-side checks of the build script (CPU only)."""
from structured_decay_sequence_amd import build


def test_scratch_users_reads_the_resource_remarks():
    remarks = (
        "x.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     VGPRs: 168 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 96 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n"
    )
    assert build.scratch_users(remarks) == [("kern_a", 96)]
    assert build.scratch_users("") == []


def test_scratch_free_sources_exist():
    names = {s.rsplit("/", 1)[-1] for s in build.sources()}
    assert set(build.SCRATCH_FREE) <= names
