"""The package's smoke entry point (one small NVFP4 layer pass on cuda:0 against the oracle)
runs through the same marshalling a user's inputs take, including the oracle's transposed
factor arrays."""
import pytest

from tests.gpu_common import torch_mod

pytestmark = pytest.mark.gpu


def test_smoke_entry_point():
    if not torch_mod().cuda.is_available():
        pytest.skip("no GPU")
    import __graft_entry__
    __graft_entry__.smoke()
