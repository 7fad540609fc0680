"""The library called from two host threads at once, each on its own stream.

The launch geometry's per-device caches (compute-unit count, kernel
attributes) and the error strings are shared or thread-local state of the
library; two threads that run linears concurrently must get the same bits
as one thread running them in turn, and those bits must match the oracle.
"""

import threading

import numpy as np
import pytest
import torch

import synth
from oracle import linear as olin
from oracle import nf4 as onf4
from gpu_util import DEV, close, f64, ql, require_gpu

pytestmark = pytest.mark.gpu

# (M, K, N, r, alpha): ragged tails, a split reduction at M = 1100, and r not a multiple of 8
SHAPES = [(300, 1024, 400, 16, 32.0), (1100, 2048, 1024, 16, 32.0), (77, 320, 208, 5, 7.0)]


class Problem:
    def __init__(self, M, K, N, r, alpha, key):
        inp = synth.linear_inputs(M, K, N, r, key)
        self.M, self.K, self.N, self.r, self.alpha = M, K, N, r, alpha
        self.x, self.A, self.B, self.dy = (inp[k].contiguous() for k in ("x", "A", "B", "dy"))
        packed, absmax = onf4.quantize(inp["W"].numpy().reshape(-1))
        self.packed, self.absmax = torch.from_numpy(packed), torch.from_numpy(absmax)

    def run(self, stream):
        """fwd + bwd with every allocation, copy and call on `stream`."""
        M, K, N, r = self.M, self.K, self.N, self.r
        with torch.cuda.stream(stream):
            d = lambda t: t.to(DEV)
            W = ql.NF4Weight(d(self.packed), d(self.absmax), N, K)
            L = ql.Lora(d(self.A), d(self.B), r, self.alpha)
            fw, bw = ql.qlora_linear_workspace(M, N, K, r)
            ws = torch.empty(max(fw, bw, 1), dtype=torch.uint8, device=DEV)
            x, dy = d(self.x), d(self.dy)
            y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
            U = torch.empty(M, r, dtype=torch.bfloat16, device=DEV)
            dx = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
            dA = torch.zeros(r, K, dtype=torch.float32, device=DEV)
            dB = torch.zeros(N, r, dtype=torch.float32, device=DEV)
            ql.qlora_linear_fwd(x, M, W, L, y, U, ws, stream=stream)
            ql.qlora_linear_bwd(dy, x, U, M, W, L, dx, dA, dB, 0, ws, stream=stream)
            out = {k: v.cpu() for k, v in dict(y=y, U=U, dx=dx, dA=dA, dB=dB).items()}
        stream.synchronize()
        return out

    def oracle(self):
        p, a = self.packed.numpy(), self.absmax.numpy()
        x, A, B, dy = f64(self.x), f64(self.A), f64(self.B), f64(self.dy)
        y, U = olin.fwd(x, p, a, self.N, self.K, A, B, self.alpha)
        dX, dA, dB, _ = olin.bwd(dy, x, U, p, a, self.N, self.K, A, B, self.alpha)
        return dict(y=y, U=U, dx=dX, dA=dA, dB=dB)


def test_two_threads_equal_one_thread_and_the_oracle():
    require_gpu()
    probs = [Problem(*s, ("threads", i)) for i, s in enumerate(SHAPES)]
    main = torch.cuda.Stream(DEV)
    ref = [p.run(main) for p in probs]
    for i, (p, got) in enumerate(zip(probs, ref)):
        want = p.oracle()
        for k in ("U", "y", "dx", "dA", "dB"):
            close(f64(got[k]), want[k], what=f"shape {i}:{k}")

    # thread t runs every problem, starting at problem t, three rounds, on its own stream
    rounds = 3
    results = [[None] * (rounds * len(probs)) for _ in range(2)]
    errors = []
    barrier = threading.Barrier(2)

    def work(t):
        try:
            s = torch.cuda.Stream(DEV)
            barrier.wait()
            for j in range(rounds * len(probs)):
                i = (t + j) % len(probs)
                results[t][j] = (i, probs[i].run(s))
        except BaseException as e:  # noqa: BLE001 (reported below)
            errors.append(e)

    threads = [threading.Thread(target=work, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    for t in range(2):
        for j, (i, got) in enumerate(results[t]):
            for k, v in got.items():
                assert torch.equal(v, ref[i][k]), f"thread {t} call {j} (shape {i}) {k} differs from one thread"
