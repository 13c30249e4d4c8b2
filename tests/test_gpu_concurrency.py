"""Concurrent calls: several host threads drive cr_linear_nvfp4 at the same time, each on
its own stream with its own workspace and output, over different shapes and both layer
paths.  The library keeps no mutable state apart from two internal caches (device
architecture, occupancy per kernel shape), so every result must equal the serial one bit
for bit."""
import threading

import pytest
import torch

import rotated_bit_linear_amd as rbl
import synth
from helpers import dev, say

pytestmark = pytest.mark.gpu

SHAPES = [(16, 300, 1000, False), (300, 520, 768, True), (129, 1000, 5376, False), (3, 257, 20000, False)]


def _inputs(i, M, N, K, swiglu):
    w = synth.Workload(f"c{i}", M, N, K, synth.DT_BF16, (synth.DT_BF16,), 50 + i, swiglu=swiglu)
    x = synth.make_activation(w).to(dev())
    p = synth.make_weight_nvfp4(w)
    return (x, p.codes.to(dev()), p.sf.to(dev()), torch.tensor([p.g], dtype=torch.float32, device=dev()),
            K, swiglu)


def test_threads_on_separate_streams_match_serial():
    inputs = [_inputs(i, *s) for i, s in enumerate(SHAPES)]
    say("serial reference calls")
    ref = [rbl.linear_nvfp4(x, c, sf, g, K, swiglu=sw) for (x, c, sf, g, K, sw) in inputs]
    torch.cuda.synchronize()

    errors = []
    results = [[None] * 6 for _ in inputs]

    def worker(t):
        try:
            x, c, sf, g, K, sw = inputs[t]
            stream = torch.cuda.Stream()
            aux = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for r in range(6):
                    results[t][r] = rbl.linear_nvfp4(x, c, sf, g, K, swiglu=sw, aux_stream=aux if r % 2 else None)
            stream.synchronize()
        except Exception as e:                      # noqa: BLE001 - reported below
            errors.append((t, repr(e)))

    say(f"{len(inputs)} threads x 6 calls, separate streams")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(len(inputs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for t, outs in enumerate(results):
        for r, o in enumerate(outs):
            assert torch.equal(o, ref[t]), f"thread {t} call {r} differs from the serial result"
