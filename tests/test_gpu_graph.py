"""GPU checks of the captured training step (stream_layer_stack_step_capture).

One step of the SmolLM2-shaped streamed stack (about 690 kernels, 57 copies)
is captured once and replayed; every replay, interleaved with eager steps and
host synchronisations, must equal the eager step bitwise. The first replay's
results are also compared with the oracle, every layer teacher-forced.
"""

import pytest
import torch

from gpu_util import ql, require_gpu
from stack_util import GpuStack, identical, teacher_forced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sm():
    require_gpu()
    s = GpuStack("smollm2_stack")
    s.fwd()
    s.bwd(reuse=True)          # the slots now hold layers 0 and 1
    assert s.fwd(reuse=True) == ql.QL_OK
    assert s.bwd(reuse=True) == ql.QL_OK
    s.eager = s.results()      # a steady-state step
    return s


def capture(s, turnaround, resident=False):
    cfg = s.cfg_mode(resident)
    store = s.store_dev if resident else s.store
    return ql.stream_layer_stack_step_capture(cfg, store, s.lora, s.x, s.dy, s.M, s.y, s.saved, s.dx, s.dA, s.dB,
                                              0, turnaround, None if resident else s.slots, s.ws, s.compute,
                                              s.copy)


def clobber(s):
    for t in (s.y, s.dx):
        t.fill_(7.0)
    for d in s.dA + s.dB:
        for t in d.values():
            t.fill_(-3.0)
    torch.cuda.synchronize()


def test_replays_with_turnaround_equal_the_eager_step(sm):
    g = capture(sm, 1)
    for rep in range(3):
        clobber(sm)
        g.launch(sm.compute)
        torch.cuda.synchronize()
        replay = sm.results()
        assert identical(replay, sm.eager), rep
        if rep == 0:
            teacher_forced(sm, replay)
        # eager work between replays (it also leaves the slots as a step does)
        assert sm.fwd(reuse=True) == ql.QL_OK
        assert sm.bwd(reuse=True) == ql.QL_OK
        torch.cuda.synchronize()
        assert identical(sm.results(), sm.eager), rep
    g.destroy()


def test_replays_without_turnaround_and_resident(sm):
    for resident in (False, True):
        g = capture(sm, 0, resident)
        for rep in range(2):
            clobber(sm)
            g.launch(sm.compute)
            torch.cuda.synchronize()
            assert identical(sm.results(), sm.eager), (resident, rep)
        g.destroy()
    # leave the slots as a streamed step does for the other tests
    sm.fwd()
    sm.bwd(reuse=True)


def test_capture_refusals(sm):
    n = sm.store.numel()
    raw = torch.empty(n + 256, dtype=torch.uint8)   # plain (pageable) host memory, 256-byte aligned view
    off = (-raw.data_ptr()) % 256
    pageable = raw[off: off + n]
    pageable.copy_(sm.store)
    with pytest.raises(ql.QlError) as e:
        ql.stream_layer_stack_step_capture(sm.cfg, pageable, sm.lora, sm.x, sm.dy, sm.M, sm.y, sm.saved, sm.dx,
                                           sm.dA, sm.dB, 0, 1, sm.slots, sm.ws, sm.compute, sm.copy)
    assert e.value.status == ql.QL_ERR_UNSUPPORTED
    ql.ql_profile_enable(1)
    try:
        with pytest.raises(ql.QlError) as e:
            capture(sm, 1)
        assert e.value.status == ql.QL_ERR_UNSUPPORTED
    finally:
        ql.ql_profile_enable(0)


def test_graph_info_counts_the_step(sm):
    # one replay: the device copy of x0 into the saved area and the 2 (L - 2)
    # layer copies of a step with both turnarounds reused are the copy nodes;
    # the kernels are the compute kernels
    g = capture(sm, 1)
    k, c, n = g.info()
    L = sm.cfg.n_layers
    assert c == 1 + 2 * (L - 2)
    assert 10 * L <= k <= 60 * L and n >= k + c
    g.destroy()


def test_weight_group_copies_replay_equal_eager():
    # 4 layers of Qwen2.5-3B widths (43 MB records): each pass's last copy goes
    # by weight group (four copies), the rest whole. The captured step holds
    # those copies and their group events; replays equal the eager step
    # bitwise.
    require_gpu()
    s = GpuStack("qwen3b_stack", L=4, gen_device="cuda:0")
    s.fwd()
    s.bwd(reuse=True)
    assert s.fwd(reuse=True) == ql.QL_OK
    assert s.bwd(reuse=True) == ql.QL_OK
    eager = s.results()
    g = capture(s, 1)
    for rep in range(2):
        clobber(s)
        g.launch(s.compute)
        torch.cuda.synchronize()
        assert identical(s.results(), eager), rep
    k, c, n = g.info()
    L = s.cfg.n_layers
    assert c == 1 + 2 * (L - 2) + 2 * 3
    g.destroy()
