"""The Python binding hands the library the caller's current HIP stream."""
import pytest
import torch

from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


def test_binding_passes_current_stream():
    """The raw handle the binding passes equals torch's current stream on the
    default stream and inside a side-stream context."""
    from gated_deltanet_gla_amd import ops
    t = torch.empty(1, device=DEV)
    assert ops._stream(t) == torch.cuda.current_stream(t.device).cuda_stream
    s = torch.cuda.Stream(device=t.device)
    with torch.cuda.stream(s):
        assert ops._stream(t) == s.cuda_stream
        assert ops._stream(t) != torch.cuda.default_stream(t.device).cuda_stream
    assert ops._stream(t) == torch.cuda.current_stream(t.device).cuda_stream
