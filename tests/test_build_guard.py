"""The build refuses kernels that use scratch memory (register spills)."""
from edge_aware_graph_amd import build as B

REMARKS = """\
k.hip:10:1: remark: Function Name: kernel_a [-Rpass-analysis=kernel-resource-usage]
k.hip:10:1: remark:     VGPRs: 64 [-Rpass-analysis=kernel-resource-usage]
k.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark: Function Name: kernel_b [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark:     ScratchSize [bytes/lane]: 52 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_users_found():
    assert B.scratch_users(REMARKS) == [("kernel_b", 52)]


def test_no_scratch_users():
    assert B.scratch_users(REMARKS.replace(": 52 ", ": 0 ")) == []


def test_built_library_defines_every_kernel_stub():
    """Every kernel the host code launches has its launch stub in the library
    (an undefined stub makes the library fail to load)."""
    import os
    import pytest
    if not os.path.exists(B.LIB):
        pytest.skip("library not built")
    assert B.missing_stubs(B.LIB) == []
