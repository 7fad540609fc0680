"""GPU checks of the per-layer recompute mode (gradient checkpointing handled
per layer by the streamer, as in the docs' "Layer Streaming" configuration).

The forward keeps only each layer's input; the backward recomputes the layer
from it with the weights already in the slot. Same kernels on the same bytes,
so y, dx0, dA and dB must equal the saved-activation mode bitwise, streamed and
resident, and with the slots reused at both turnarounds. The recompute run is
also compared with the oracle itself, every layer teacher-forced: each layer's
output from its kept input, and its input gradient, dA and dB from the GPU's
upstream gradient (re-derived by 1-layer recompute-mode calls).
"""

import pytest
import torch

from gpu_util import ql, require_gpu
from stack_util import GpuStack, identical, teacher_forced

pytestmark = pytest.mark.gpu

L, M = 6, 160


@pytest.fixture(scope="module")
def pair():
    require_gpu()
    return GpuStack("smollm2_stack", L=L, M=M), GpuStack("smollm2_stack", L=L, M=M, recompute=1)


def same_outputs(a, b):
    def eq(x, y):
        return torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    if not eq(a["y"], b["y"]) or not eq(a["dx"], b["dx"]):
        return False
    return all(eq(la[p], lb[p]) for la, lb in zip(a["dA"], b["dA"]) for p in la) and \
        all(eq(la[p], lb[p]) for la, lb in zip(a["dB"], b["dB"]) for p in la)


def test_recompute_equals_saved_mode_bitwise(pair):
    full, rc = pair
    assert full.step(resident=False, reuse=True) == ql.QL_OK
    a = full.results()
    assert rc.step(resident=False, reuse=True) == ql.QL_OK
    b = rc.results()
    assert same_outputs(a, b)
    teacher_forced(rc, b, full_saved=False)
    # the recompute-mode forward keeps exactly the layer inputs of the full mode
    _, per_full = ql.stream_layer_stack_saved_layout(full.cfg, M)
    _, per_rc = ql.stream_layer_stack_saved_layout(rc.cfg, M)
    H = full.w["H"]
    for layer in range(L):
        h_full = a["saved"][layer * per_full: layer * per_full + M * H * 2]
        h_rc = b["saved"][layer * per_rc: layer * per_rc + M * H * 2]
        assert torch.equal(h_full, h_rc)


def test_recompute_streamed_equals_resident_and_reuses_slots(pair):
    _, rc = pair
    rc.fwd()
    for _ in range(2):
        assert rc.bwd(reuse=True) == ql.QL_OK
        assert rc.fwd(reuse=True) == ql.QL_OK
    assert rc.bwd(reuse=True) == ql.QL_OK
    streamed = rc.results()
    rc.step(resident=True)
    assert identical(streamed, rc.results())


def test_recompute_saves_only_layer_inputs(pair):
    full, rc = pair
    H = full.w["H"]
    per_in = (M * H * 2 + 255) // 256 * 256
    assert rc.saved.numel() == L * per_in
    assert full.saved.numel() > 5 * rc.saved.numel()
    offs, _ = ql.stream_layer_stack_saved_layout(rc.cfg, M)
    assert offs["h_in"] == 0 and all(v == -1 for k, v in offs.items() if k != "h_in")
