"""GPU parity of the adapter-off reference forward (stream_layer_stack_fwd_ref).

For preference losses the reference model is the streamed frozen base with the
adapters switched off (the aiany.app entry "Soup", section "How It Works"). The
call runs it in the same pass over the layers as the policy forward. Checked:
the policy outputs are bitwise those of stream_layer_stack_fwd; the reference
output matches the oracle stack with every LoRA factor zero (the definition of
"adapters off"); it equals the GPU's own adapted forward with B = 0 in value
(a zero LoRA term adds exact zeros); reference alone, fused, streamed and
resident runs agree bitwise; and the slots it leaves serve the backward.
"""

import numpy as np
import pytest
import torch

from gpu_util import DEV, close, f64, ql, require_gpu
from oracle import stack as ostack
from stack_util import GpuStack, identical

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def st():
    require_gpu()
    s = GpuStack("smollm2_stack", L=4, M=96)
    _, per = ql.stream_layer_stack_saved_layout(s.cfg, s.M)
    s.ref_scratch = torch.empty(per, dtype=torch.uint8, device=DEV)
    s.ref_y = torch.empty_like(s.y)
    return s


def run_ref(s, lora=True, resident=False, reuse=False, y=None, saved=None):
    cfg = s.cfg_mode(resident)
    store = s.store_dev if resident else s.store
    return ql.stream_layer_stack_fwd_ref(cfg, store, s.lora if lora else None, s.x, s.M,
                                         s.y if y is None else y, s.saved if saved is None else saved,
                                         s.ref_y, s.ref_scratch, None if resident else s.slots, s.ws,
                                         s.compute, s.copy, reuse_bwd_slots=reuse)


def test_policy_outputs_unchanged(st):
    assert st.fwd() == ql.QL_OK
    a = st.results()
    assert run_ref(st) == ql.QL_OK
    b = st.results()
    assert torch.equal(a["y"].view(torch.uint8), b["y"].view(torch.uint8))
    assert torch.equal(a["saved"], b["saved"])


@pytest.mark.parametrize("M", [5, 200])
def test_fused_rmsnorm_equals_standalone_bitwise(M):
    # The policy forward makes n1 = RMSNorm(h) inside its LoRA row launch; the
    # adapter-off reference forward has no row launch and runs the standalone
    # RMSNorm kernel. On layer 0 both normalise the same input x, so their n1
    # agree bitwise (the fused kernel sums in the standalone kernel's order),
    # also for a row count that leaves the last 16-row tile partial.
    require_gpu()
    s = GpuStack("smollm2_stack", L=1, M=M)
    _, per = ql.stream_layer_stack_saved_layout(s.cfg, s.M)
    s.ref_scratch = torch.empty(per, dtype=torch.uint8, device=DEV)
    s.ref_y = torch.empty_like(s.y)
    assert run_ref(s) == ql.QL_OK
    torch.cuda.synchronize()
    pol = s.saved_tensor(0, "n1")
    ref = s.saved_tensor(0, "n1", buf=s.ref_scratch)
    assert torch.equal(pol.view(torch.int16), ref.view(torch.int16))
    assert torch.count_nonzero(pol.float()) > 0


def test_reference_matches_oracle_with_adapters_off(st):
    assert run_ref(st) == ql.QL_OK
    torch.cuda.synchronize()
    layers = st.oracle_layers()
    for lay in layers:
        lay.lora = {p: (np.zeros_like(A), np.zeros_like(B)) for p, (A, B) in lay.lora.items()}
    h, _ = ostack.stack_fwd(layers, f64(st.x))
    close(f64(st.ref_y), h, what="ref_y")
    # and it differs from the adapted output (the adapters are not a no-op)
    assert not torch.equal(st.ref_y, st.y)


def test_reference_equals_zero_B_adapted_forward(st):
    assert run_ref(st) == ql.QL_OK
    ref = st.ref_y.clone()
    saved_lora = st.lora
    st.lora = [{p: (A, torch.zeros_like(B)) for p, (A, B) in d.items()} for d in saved_lora]
    try:
        assert st.fwd() == ql.QL_OK
        torch.cuda.synchronize()
        assert torch.equal(ref.float(), st.y.float())
    finally:
        st.lora = saved_lora


def test_reference_alone_fused_streamed_resident_agree(st):
    outs = []
    for lora, resident in ((True, False), (False, False), (True, True), (False, True)):
        assert run_ref(st, lora=lora, resident=resident) == ql.QL_OK
        torch.cuda.synchronize()
        outs.append(st.ref_y.clone())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.uint8), outs[0].view(torch.uint8))


def test_reference_alone_needs_no_policy_buffers(st):
    scratch_y = st.y.clone()
    assert ql.stream_layer_stack_fwd_ref(st.cfg, st.store, None, st.x, st.M, None, None, st.ref_y,
                                         st.ref_scratch, st.slots, st.ws, st.compute, st.copy) == ql.QL_OK
    torch.cuda.synchronize()
    assert torch.equal(st.y.view(torch.uint8), scratch_y.view(torch.uint8))


def test_training_step_with_reference_reuses_slots(st):
    # preference step: (policy + reference) forward, then the backward reusing
    # the slots; equal bitwise to the plain streamed step and the resident one
    assert run_ref(st) == ql.QL_OK
    assert st.bwd(reuse=True) == ql.QL_OK
    assert run_ref(st, reuse=True) == ql.QL_OK
    assert st.bwd(reuse=True) == ql.QL_OK
    a = st.results()
    st.step(resident=True)
    assert identical(a, st.results())


def test_reference_argument_errors(st):
    with pytest.raises(ql.QlError) as e:
        ql.stream_layer_stack_fwd_ref(st.cfg, st.store, None, st.x, st.M, None, None, st.ref_y,
                                      st.ref_scratch[:1024], st.slots, st.ws, st.compute, st.copy)
    assert e.value.status == ql.QL_ERR_WORKSPACE
    with pytest.raises(ql.QlError) as e:
        ql.stream_layer_stack_fwd_ref(st.cfg, st.store, None, st.x, st.M, None, None, None,
                                      st.ref_scratch, st.slots, st.ws, st.compute, st.copy)
    assert e.value.status == ql.QL_ERR_ARG
