"""The Python binding refuses host tensors and wrong dtypes before anything
reaches the library: there is no CPU path, so a call with host memory must
fail loudly instead of passing host pointers to the device code."""
import pytest
import torch

from gate_projection_top_amd import router as R


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


CALLS = {
    "router_fwd": lambda x, w: R.router_fwd(x, w, None, 8),
    "router_fwd_mxfp4": lambda x, w: R.router_fwd_mxfp4(x, w, u8(256, 4), None, 8),
    "router_fwd_mxfp8": lambda x, w: R.router_fwd_mxfp8(x, w, u8(256, 4), None, 8),
}
GATES = {"router_fwd": bf16(256, 128), "router_fwd_mxfp4": u8(256, 64), "router_fwd_mxfp8": u8(256, 128)}


@pytest.mark.parametrize("entry", sorted(CALLS))
def test_host_tensors_are_refused(entry):
    with pytest.raises(ValueError, match="GPU"):
        CALLS[entry](bf16(2, 128), GATES[entry])


@pytest.mark.parametrize("entry", sorted(CALLS))
def test_wrong_activation_dtype_is_refused(entry):
    with pytest.raises(TypeError, match="bfloat16"):
        CALLS[entry](torch.zeros((2, 128), dtype=torch.float32), GATES[entry])


@pytest.mark.parametrize("entry", sorted(CALLS))
def test_wrong_rank_is_refused(entry):
    with pytest.raises(ValueError, match="dims"):
        CALLS[entry](bf16(2, 128, 1), GATES[entry])


def test_topk_refuses_host_logits():
    with pytest.raises(ValueError, match="GPU"):
        R.router_topk_from_logits(torch.zeros((4, 256), dtype=torch.float32), None, 8)


def test_exports_match_the_header():
    # every name the binding exports is declared in include/router.h
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    header = open(os.path.join(root, "include", "router.h")).read()
    for name in R.EXPORTS:
        assert f" {name}(" in header, name
