"""Calls from several host threads, each on its own stream, at once: the
library keeps no state between calls beyond its per-device architecture
check, so every thread must get exactly the results one thread gets."""
from concurrent.futures import ThreadPoolExecutor

import pytest
import torch

import attn_inputs
import exact_attention_87_amd as ea

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, N, d, causal): every head dimension, a grouped-query split of
# the dK/dV stage (few kv heads, short sequence) and a ragged length
CASES = [(2, 8, 2, 700, 64, True), (1, 8, 8, 900, 128, False), (1, 4, 2, 300, 256, True),
         (1, 12, 2, 513, 128, True)]


def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def run(q, k, v, do, causal):
    o, lse = ea.fwd(q, k, v, causal=causal)
    dq, dk, dv = ea.bwd(q, k, v, o, lse, do, causal=causal)
    return o, lse, dq, dk, dv


def test_threads_on_separate_streams_get_the_single_thread_results():
    dev = gpu()
    inputs = []
    for i, (B, Hq, Hkv, N, d, causal) in enumerate(CASES):
        t = attn_inputs.make(B, Hq, Hkv, N, d, "bf16", seed=90 + i, with_dout=True)
        inputs.append((tuple(x.to(dev) for x in t), causal))
    ref = [run(*t, causal) for t, causal in inputs]
    torch.cuda.synchronize()

    def work(i):
        (q, k, v, do), causal = inputs[i]
        stream = torch.cuda.Stream(dev)  # default priority
        outs = []
        with torch.cuda.stream(stream):
            for _ in range(4):
                outs.append(run(q, k, v, do, causal))
        stream.synchronize()
        return outs

    with ThreadPoolExecutor(len(CASES)) as ex:
        results = list(ex.map(work, range(len(CASES))))
    torch.cuda.synchronize()
    for i, outs in enumerate(results):
        for rep in outs:
            for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), ref[i], rep):
                assert torch.equal(a, b), f"case {CASES[i]}: {name} differs from the single-thread run"
