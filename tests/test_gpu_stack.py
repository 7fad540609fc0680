"""GPU parity of the layer-streamed stack (stream_layer_stack_fwd / _bwd) through the C ABI.

The pages require a streamed run to be bit-identical to a resident one, forward
and backward stated separately; results are checked against the oracle from
the same seeded inputs.

Tolerance. One layer agrees element-wise within 2e-2 (relative, with an
rms-scaled floor). A deep stack of bf16 layers is ill-conditioned end to end:
at 30 layers the random-weight stand-in's backward amplifies |dx0| about 30x
over |dy|, and the bf16-faithful oracle itself lands about 24% (normwise) from
the float64-exact gradient. So every layer of a deep stack is checked
teacher-forced (tests/stack_util.py): the oracle layer runs on the GPU's own
input to that layer, and all of the layer's outputs (saved activations, output,
input gradient, dA, dB) are compared element-wise at 2e-2. Stacks of up to 8
layers are also held to 2e-2 normwise end to end; deeper, the end-to-end
normwise distance is printed as a report only.
"""

import numpy as np
import pytest
import torch

from gpu_util import DEV, close, close_norm, f64, ql, require_gpu
from oracle import stack as ostack
from stack_util import GpuStack, LayerChain, identical, teacher_forced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def smol():
    require_gpu()
    return GpuStack("smollm2_stack")


def _end_to_end_report(s, got, tag):
    """Normwise distance of y and dx0 from the bf16-faithful oracle run end to end (printed)."""
    layers = s.oracle_layers()
    h, saved = ostack.stack_fwd(layers, f64(s.x))
    dx0, _ = ostack.stack_bwd(layers, saved, f64(s.dy))
    ny = np.linalg.norm(f64(got["y"]) - h) / np.linalg.norm(h)
    nd = np.linalg.norm(f64(got["dx"]) - dx0) / np.linalg.norm(dx0)
    print(f"{tag}: end to end vs the faithful oracle, normwise: y {ny:.3g}, dx0 {nd:.3g}")
    return ny, nd


def test_smollm2_stack_matches_oracle(smol):
    # all 30 layers teacher-forced, every output of each layer element-wise
    st = smol.step(resident=False, reuse=True)
    assert st == ql.QL_OK
    got = smol.results()
    teacher_forced(smol, got)
    # end to end the bf16 roundings of 30 layers add up; measured 0.004 (y)
    # and 0.013 (dx0) normwise from the faithful oracle, held to 2e-2
    ny, nd = _end_to_end_report(smol, got, "smollm2 30 layers")
    assert ny <= 2e-2 and nd <= 2e-2


def test_smollm2_8_layers_normwise():
    require_gpu()
    s = GpuStack("smollm2_stack", L=8)
    assert s.step(resident=False, reuse=True) == ql.QL_OK
    got = s.results()
    layers = s.oracle_layers()
    x, dy = f64(s.x), f64(s.dy)
    h, saved = ostack.stack_fwd(layers, x)
    close_norm(f64(got["y"]), h, what="y")
    dx0, grads = ostack.stack_bwd(layers, saved, dy)
    close_norm(f64(got["dx"]), dx0, what="dx0")
    for li in range(8):
        for p in ("v", "o", "gate", "up", "down"):
            for j, nm in ((0, "dA"), (1, "dB")):
                close_norm(f64(got[nm][li][p]), grads[li][p][j], what=f"L{li}:{p}:{nm}")


def test_streamed_equals_resident_bitwise(smol):
    assert smol.step(resident=False, reuse=True) == ql.QL_OK
    streamed = smol.results()
    assert smol.step(resident=True) == ql.QL_OK
    resident = smol.results()
    assert identical(streamed, resident)


def test_forward_and_backward_bitwise_separately(smol):
    # forward: y and saved activations; backward: dx0 and gradients
    smol.fwd(resident=False)
    a = smol.results()
    smol.fwd(resident=True)
    b = smol.results()
    assert torch.equal(a["y"].view(torch.uint8), b["y"].view(torch.uint8))
    assert torch.equal(a["saved"], b["saved"])
    smol.bwd(resident=False, reuse=False)
    c = smol.results()
    smol.bwd(resident=True)
    d = smol.results()
    assert identical(c, d)


def test_repeated_runs_are_bitwise_identical(smol):
    runs = []
    for _ in range(3):
        smol.step(resident=False, reuse=True)
        runs.append(smol.results())
    assert identical(runs[0], runs[1]) and identical(runs[1], runs[2])


def test_slot_reuse_at_turnaround_matches_full_copies(smol):
    smol.fwd()
    smol.bwd(reuse=True)
    a = smol.results()
    smol.fwd()
    smol.bwd(reuse=False)
    b = smol.results()
    assert identical(a, b)


def test_training_loop_reuses_slots_both_ways(smol):
    # fwd, then (bwd, fwd) pairs that each skip the two copies the other left
    # in the slots; the last step must equal the resident step bitwise
    smol.fwd()
    for _ in range(2):
        smol.bwd(reuse=True)
        smol.fwd(reuse=True)
    smol.bwd(reuse=True)
    streamed = smol.results()
    smol.step(resident=True)
    assert identical(streamed, smol.results())


def test_two_stores_share_slots_without_sync(smol):
    # a second store (the layers in reverse order) through the same slots right
    # after the first, with no host synchronisation in between: the second
    # call's first copies must wait for the first call's compute
    other = ql.build_store(smol.cfg, smol.layer_stores()[::-1], pinned=True)
    other_dev = other.to(DEV)
    smol.fwd(store=smol.store_dev, resident=True)
    torch.cuda.synchronize()
    y_first_resident = smol.y.clone()
    smol.fwd(store=other_dev, resident=True)
    torch.cuda.synchronize()
    y_other_resident = smol.y.clone()
    smol.fwd()
    with torch.cuda.stream(smol.compute):
        y_first = smol.y.clone()
    smol.fwd(store=other)
    torch.cuda.synchronize()
    assert torch.equal(y_first.view(torch.uint8), y_first_resident.view(torch.uint8))
    assert torch.equal(smol.y.view(torch.uint8), y_other_resident.view(torch.uint8))


def test_pageable_store_warns_and_matches(smol):
    smol.step(resident=False, reuse=True)
    pinned = smol.results()
    n = smol.store.numel()
    raw = torch.empty(n + 256, dtype=torch.uint8)  # plain (pageable) host memory, 256-byte aligned view
    off = (-raw.data_ptr()) % 256
    pageable = raw[off: off + n]
    pageable.copy_(smol.store)
    assert not pageable.is_pinned()
    st1 = smol.fwd(store=pageable)
    st2 = smol.bwd(store=pageable, reuse=False)
    assert st1 == ql.QL_WARN_PAGEABLE_HOST and st2 == ql.QL_WARN_PAGEABLE_HOST
    assert identical(pinned, smol.results())


def test_accumulate_adds_the_step_gradients(smol):
    smol.step(resident=False, reuse=True)
    base = smol.results()
    smol.fwd()
    smol.bwd(reuse=True, accumulate=True)
    acc = smol.results()
    for li in range(smol.cfg.n_layers):
        for p in ql.PROJ:
            assert torch.equal(acc["dA"][li][p], base["dA"][li][p] + base["dA"][li][p])
            assert torch.equal(acc["dB"][li][p], base["dB"][li][p] + base["dB"][li][p])


class poisoned:
    """Slot poisoning on for the block (ql_debug_poison_slots)."""

    def __enter__(self):
        ql.ql_debug_poison_slots(1)

    def __exit__(self, *exc):
        ql.ql_debug_poison_slots(0)


def test_poisoned_slots_training_loop_equals_resident(smol):
    # every slot is filled with 0xFF before each copy into it: a kernel that
    # read a slot before its copy landed would produce NaN; the training loop
    # (both turnarounds reused, no host sync between calls) must still equal
    # the resident step bitwise
    with poisoned():
        assert smol.fwd() == ql.QL_OK
        for _ in range(2):
            assert smol.bwd(reuse=True) == ql.QL_OK
            assert smol.fwd(reuse=True) == ql.QL_OK
        assert smol.bwd(reuse=True) == ql.QL_OK
        streamed = smol.results()
    assert torch.isfinite(streamed["y"].float()).all() and torch.isfinite(streamed["dx"].float()).all()
    smol.step(resident=True)
    assert identical(streamed, smol.results())


def test_poisoning_refuses_capture_and_switches_off(smol):
    with poisoned():
        with pytest.raises(ql.QlError) as e:
            ql.stream_layer_stack_step_capture(smol.cfg, smol.store, smol.lora, smol.x, smol.dy, smol.M, smol.y,
                                               smol.saved, smol.dx, smol.dA, smol.dB, 0, 1, smol.slots, smol.ws,
                                               smol.compute, smol.copy)
        assert e.value.status == ql.QL_ERR_UNSUPPORTED
    with pytest.raises(ql.QlError) as e:
        ql.ql_debug_poison_slots(2)
    assert e.value.status == ql.QL_ERR_ARG


def test_qk_grads_zero_and_the_rest_nonzero_at_layer0(smol):
    smol.step()
    got = smol.results()
    for p in ("q", "k"):
        assert torch.count_nonzero(got["dA"][0][p]) == 0 and torch.count_nonzero(got["dB"][0][p]) == 0
    for p in ("v", "o", "gate", "up", "down"):
        assert torch.count_nonzero(got["dA"][0][p]) > 0 and torch.count_nonzero(got["dB"][0][p]) > 0


def test_slot_memory_is_two_layer_records(smol):
    offs, _, _ = ql.stream_layer_stack_layout(smol.cfg)
    assert smol.slots.numel() == 2 * offs[1]


@pytest.fixture(scope="module")
def smol8():
    require_gpu()
    return GpuStack("smollm2_stack", n_buffers=8)


@pytest.mark.parametrize("nb", [3, 5, 8])
def test_deeper_ring_training_loop_equals_resident(smol8, nb):
    # the pages expose 2..8 stream buffers; with n slots layer l uses slot
    # l % n, the prefetch runs n - 1 layers ahead and each turnaround reuses n
    # layers: fwd, then (bwd, fwd) pairs reusing the slots, must equal the
    # resident step bitwise
    # (the loop runs with the slots poisoned before every copy: a read ahead
    # of a copy in the deeper ring would show as NaN)
    smol8.set_buffers(nb)
    with poisoned():
        assert smol8.fwd() == ql.QL_OK
        for _ in range(2):
            assert smol8.bwd(reuse=True) == ql.QL_OK
            assert smol8.fwd(reuse=True) == ql.QL_OK
        assert smol8.bwd(reuse=True) == ql.QL_OK
        streamed = smol8.results()
    if nb == 8:  # the deepest ring against the oracle, every layer teacher-forced
        teacher_forced(smol8, streamed)
    smol8.step(resident=True)
    assert identical(streamed, smol8.results())
    # and without reuse (every call copies its first n layers itself)
    smol8.fwd()
    smol8.bwd(reuse=False)
    assert identical(streamed, smol8.results())


def test_deeper_ring_slot_memory(smol8):
    offs, _, _ = ql.stream_layer_stack_layout(smol8.cfg)
    for nb in (2, 5, 8):
        c = ql.StackCfg(**{**smol8.cfg.__dict__, "n_buffers": nb})
        assert ql.stream_layer_stack_workspace(c, smol8.M)[0] == nb * offs[1]
    # slot memory for fewer records than n_buffers is refused before anything runs
    smol8.set_buffers(8)
    with pytest.raises(ql.QlError) as e:
        ql.stream_layer_stack_fwd(smol8.cfg, smol8.store, smol8.lora, smol8.x, smol8.M, smol8.y, smol8.saved,
                                  smol8.slots[: 7 * offs[1]], smol8.ws, smol8.compute, smol8.copy)
    assert e.value.status == ql.QL_ERR_WORKSPACE


@pytest.mark.parametrize("L,nb", [(5, 8), (8, 8), (9, 4)])
def test_ring_longer_than_or_equal_to_stack(L, nb):
    # fewer layers than slots: every layer is copied once in the prologue
    require_gpu()
    s = GpuStack("smollm2_stack", L=L, M=64, n_buffers=nb)
    assert s.fwd() == ql.QL_OK
    assert s.bwd(reuse=True) == ql.QL_OK
    assert s.fwd(reuse=True) == ql.QL_OK
    assert s.bwd(reuse=True) == ql.QL_OK
    got = s.results()
    s.step(resident=True)
    assert identical(got, s.results())


@pytest.mark.parametrize("L,M", [(1, 77), (3, 1), (1, 700)])
def test_small_stacks_ragged_rows(L, M):
    # M = 700: the layer's adapter-gradient reductions split over rows
    require_gpu()
    s = GpuStack("smollm2_stack", L=L, M=M)
    assert s.step(resident=False, reuse=True) == ql.QL_OK
    got = s.results()
    assert s.step(resident=True) == ql.QL_OK
    assert identical(got, s.results())
    layers = s.oracle_layers()
    h, saved = ostack.stack_fwd(layers, f64(s.x))
    close(f64(got["y"]), h, what="y")
    dx0, grads = ostack.stack_bwd(layers, saved, f64(s.dy))
    close(f64(got["dx"]), dx0, what="dx0")
    for li in range(L):
        for p in ("v", "o", "gate", "up", "down"):
            close(f64(got["dA"][li][p]), grads[li][p][0], what=f"L{li}:{p}:dA")
            close(f64(got["dB"][li][p]), grads[li][p][1], what=f"L{li}:{p}:dB")


@pytest.mark.parametrize("r", [40, 64])
def test_ranks_above_the_fused_swiglu_backward(r):
    # r > 32 takes the separate SwiGLU backward and the two-problem row launch
    # for G of gate and up; r = 64 also splits q | k | v's LoRA down per projection
    require_gpu()
    s = GpuStack("smollm2_stack", L=1, M=77, r=r)
    assert s.step(resident=False, reuse=True) == ql.QL_OK
    got = s.results()
    assert s.step(resident=True) == ql.QL_OK
    assert identical(got, s.results())
    layers = s.oracle_layers()
    h, saved = ostack.stack_fwd(layers, f64(s.x))
    close(f64(got["y"]), h, what="y")
    dx0, grads = ostack.stack_bwd(layers, saved, f64(s.dy))
    close(f64(got["dx"]), dx0, what="dx0")
    for p in ("v", "o", "gate", "up", "down"):
        close(f64(got["dA"][0][p]), grads[0][p][0], what=f"{p}:dA")
        close(f64(got["dB"][0][p]), grads[0][p][1], what=f"{p}:dB")


def test_stack_argument_errors(smol):
    with pytest.raises(ql.QlError) as e:
        ql.stream_layer_stack_fwd(smol.cfg, smol.store, smol.lora, smol.x, smol.M, smol.y, smol.saved,
                                  smol.slots[:1024], smol.ws, smol.compute, smol.copy)
    assert e.value.status == ql.QL_ERR_WORKSPACE
    with pytest.raises(ql.QlError) as e:
        ql.stream_layer_stack_fwd(smol.cfg, smol.store, smol.lora, smol.x, smol.M, smol.y, smol.saved,
                                  smol.slots, smol.ws[:1024], smol.compute, smol.copy)
    assert e.value.status == ql.QL_ERR_WORKSPACE
    with pytest.raises(ql.QlError) as e:   # resident mode needs a device store
        ql.stream_layer_stack_fwd(smol.cfg_mode(True), smol.store, smol.lora, smol.x, smol.M, smol.y,
                                  smol.saved, None, smol.ws, smol.compute, smol.copy)
    assert e.value.status == ql.QL_ERR_ARG
    with pytest.raises(ql.QlError) as e:   # streamed mode needs a host store
        ql.stream_layer_stack_fwd(smol.cfg, smol.store_dev, smol.lora, smol.x, smol.M, smol.y, smol.saved,
                                  smol.slots, smol.ws, smol.compute, smol.copy)
    assert e.value.status == ql.QL_ERR_ARG


@pytest.fixture(scope="module")
def qwen():
    # 36 layers, hidden 2048, intermediate 11008, kv 256, r 16, M = 512: the
    # full Qwen2.5-3B-shaped stack, streamed, with the per-layer upstream
    # gradients of its backward re-derived by the 1-layer chain
    require_gpu()
    s = GpuStack("qwen3b_stack", gen_device=DEV)
    assert s.step(resident=False, reuse=True) == ql.QL_OK
    s.got = s.results()
    s.dh = LayerChain(s).upstream(s.got)
    return s


@pytest.mark.parametrize("group", range(4))
def test_qwen3b_stack_teacher_forced(qwen, group):
    # layers 9 g .. 9 g + 8 of 36, each teacher-forced, every output element-wise
    teacher_forced(qwen, qwen.got, layers=range(9 * group, 9 * group + 9), dh=qwen.dh)


def test_qwen3b_stack_streamed_equals_resident(qwen):
    assert qwen.step(resident=True) == ql.QL_OK
    assert identical(qwen.got, qwen.results())
    _end_to_end_report(qwen, qwen.got, "qwen3b 36 layers")


def test_queued_steps_of_a_large_record_stack_equal_resident():
    # Qwen2.5-3B widths, 4 layers: 43 MB records, so each streamed call first
    # waits on the host for the previous call of its direction to finish on
    # the GPU. Three training steps queued back to back (no synchronisation
    # between the calls, slots reused at every turnaround) end bitwise equal
    # to the resident step.
    require_gpu()
    s = GpuStack("qwen3b_stack", L=4, gen_device=DEV)
    offs, _, _ = ql.stream_layer_stack_layout(s.cfg)
    assert offs[1] >= 8 << 20
    with poisoned():   # slots filled with 0xFF before every copy
        assert s.fwd() == ql.QL_OK
        for _ in range(2):
            assert s.bwd(reuse=True) == ql.QL_OK
            assert s.fwd(reuse=True) == ql.QL_OK
        assert s.bwd(reuse=True) == ql.QL_OK
        streamed = s.results()
    assert s.step(resident=True) == ql.QL_OK
    assert identical(streamed, s.results())


@pytest.mark.parametrize("L,nb,recompute,dq", [(3, 2, 0, 0), (5, 3, 0, 0), (4, 2, 1, 0), (4, 2, 0, 1)])
def test_weight_group_handoffs_equal_resident(L, nb, recompute, dq):
    # Stacks of records of 8 MiB or more copy each pass's last layer one
    # weight group at a time (q|k|v, o, gate|up, down; the backward in
    # reverse), and that layer starts each GEMM once its group has landed.
    # With every group poisoned just before its copy, a GEMM that ran ahead of
    # its group would read NaN: forward, (backward, forward) pairs reusing the
    # slots, then a backward must equal the resident step bitwise. With 3
    # slots the ring is deeper; with recomputation the backward's last layer
    # first reruns its forward on the groups as they land; with
    # double-quantised scales each group's scales are expanded as it lands.
    require_gpu()
    s = GpuStack("qwen3b_stack", L=L, gen_device=DEV, n_buffers=nb, recompute=recompute, absmax_dq=dq)
    offs, _, _ = ql.stream_layer_stack_layout(s.cfg)
    assert offs[1] >= 8 << 20
    with poisoned():
        assert s.fwd() == ql.QL_OK
        for _ in range(2):
            assert s.bwd(reuse=True) == ql.QL_OK
            assert s.fwd(reuse=True) == ql.QL_OK
        assert s.bwd(reuse=True) == ql.QL_OK
        streamed = s.results()
    assert s.step(resident=True) == ql.QL_OK
    assert identical(streamed, s.results())


def test_llama8b_widths_at_bench_launch_config_teacher_forced():
    # The 8B layer shapes at M = 2048 (the benchmark's launch configuration:
    # the same kernels, tile geometry, split-K and batched adapter-gradient
    # launches as each layer of the 32-layer step), 2 layers, all 2048 rows:
    # every saved activation, both layer outputs, dx0 and dA, dB of v, o,
    # gate, up and down element-wise against the oracle.
    require_gpu()
    s = GpuStack("llama8b_stack", L=2, gen_device=DEV)
    assert s.step(resident=False, reuse=True) == ql.QL_OK
    got = s.results()
    teacher_forced(s, got)
    assert s.step(resident=True) == ql.QL_OK
    assert identical(got, s.results())


def test_llama8b_stack_full_streamed_equals_resident():
    # The benchmark workload itself: 32 layers, M = 2048, 3.93 GB pinned store.
    # A streamed step allocates nothing: device memory in use is the caller's
    # buffers, of which the frozen weights take the two slots (the pages'
    # bounded-memory claim, here measured around the step).
    require_gpu()
    s = GpuStack("llama8b_stack", gen_device=DEV)
    assert s.step(resident=False, reuse=True) == ql.QL_OK
    torch.cuda.synchronize()
    in_use = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    free0 = torch.cuda.mem_get_info()[0]
    assert s.step(resident=False, reuse=True) == ql.QL_OK
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert torch.cuda.max_memory_allocated() == in_use
    assert free0 - free1 <= 64 << 20, (free0, free1)
    offs, _, _ = ql.stream_layer_stack_layout(s.cfg)
    assert s.slots.numel() == 2 * offs[1]
    lora = sum(t.numel() * t.element_size() for d in s.lora for A, B in d.values() for t in (A, B))
    grads = sum(t.numel() * 4 for d in s.dA + s.dB for t in d.values())
    print(f"8B streamed step, device bytes: slots {s.slots.numel()} (2 records of {offs[1]}), saved "
          f"{s.saved.numel()}, ws {s.ws.numel()}, lora {lora}, grads {grads}; store on host {s.store.numel()}; "
          f"device free before/after the step {free0}/{free1}")
    a = s.results()
    assert torch.isfinite(a["y"].float()).all() and torch.isfinite(a["dx"].float()).all()
    assert s.step(resident=True) == ql.QL_OK
    assert identical(a, s.results())
