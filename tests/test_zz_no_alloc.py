"""attn_bwd_noalloc (the backward with its workspace in the library's static
device scratch) against attn_bwd with a caller workspace, through the C ABI.

Both run the same kernels with the same launch plan, so the gradients must be
identical bit for bit.  Two calls in a row on one device share the scratch; the
second is smaller, so it runs over the first call's leftover contents.  One
shape splits the dK/dV stage over query heads (partial sums in the scratch
too).  The comparison is also checked against the fp64 oracle on one slice.
"""
import numpy as np
import pytest
import torch

import attn_inputs
import exact_attention_87_amd as ea

pytestmark = pytest.mark.gpu


def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def grads(fn_name, q, k, v, o, lse, do, causal, scale):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    code = ea.ATTN_BF16 if q.dtype == torch.bfloat16 else ea.ATTN_F16
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [t.data_ptr() for t in (q, k, v, o, lse, do, dq, dk, dv)]
    if fn_name == "noalloc":
        st = ea.attn_bwd_noalloc(*ptrs, B, Hq, Hkv, N, d, causal, scale, code, stream)
    else:
        nbytes = ea.attn_bwd_workspace_bytes(B, Hq, Hkv, N, d, code)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
        st = ea.attn_bwd(*ptrs, ws.data_ptr(), B, Hq, Hkv, N, d, causal, scale, code, stream)
        torch.cuda.synchronize()
        del ws
    assert st == ea.ATTN_OK, ea.attn_status_str(st)
    torch.cuda.synchronize()
    return dq, dk, dv


# (B, Hq, Hkv, N, d, causal, dtype): a larger call, then a smaller one over its
# leftovers; the third splits the dK/dV stage 4 ways (partials in the scratch).
SHAPES = [(2, 4, 2, 1000, 64, True, "bf16"), (1, 2, 1, 300, 128, False, "bf16"),
          (1, 8, 2, 512, 64, True, "fp16"), (1, 1, 1, 77, 256, True, "bf16")]


def test_noalloc_matches_attn_bwd_bitwise_on_consecutive_calls(oracle_mod):
    dev = gpu()
    for i, (B, Hq, Hkv, N, d, causal, dt) in enumerate(SHAPES):
        print(f"noalloc case {i}: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} {dt}",
              flush=True)
        q, k, v, do = attn_inputs.make(B, Hq, Hkv, N, d, dt, seed=40 + i, with_dout=True)
        qg, kg, vg, dog = (t.to(dev) for t in (q, k, v, do))
        scale = 1.0 / d ** 0.5
        o, lse = ea.fwd(qg, kg, vg, causal=causal, scale=scale)
        ref = grads("attn_bwd", qg, kg, vg, o, lse, dog, causal, scale)
        got = grads("noalloc", qg, kg, vg, o, lse, dog, causal, scale)
        again = grads("noalloc", qg, kg, vg, o, lse, dog, causal, scale)
        for name, a, b, c in zip(("dQ", "dK", "dV"), ref, got, again):
            assert torch.equal(a, b), f"case {i} {name}: noalloc differs from attn_bwd"
            assert torch.equal(b, c), f"case {i} {name}: noalloc not repeatable"
        # and the gradients are right: the oracle on the first kv group
        group = Hq // Hkv
        rdq, rdk, rdv = oracle_mod.bwd(q[:1, :group], k[:1, :1], v[:1, :1], do[:1, :group],
                                       causal=causal, scale=scale)
        for name, g, r in (("dQ", got[0][:1, :group], rdq), ("dK", got[1][:1, :1], rdk),
                           ("dV", got[2][:1, :1], rdv)):
            g = g.float().cpu().numpy()
            assert np.all(np.isfinite(g))
            assert np.abs(g - r).max() <= 5e-2 * np.abs(r).max(), f"case {i} {name}"


def test_noalloc_refuses_problems_beyond_the_scratch():
    dev = gpu()
    x = torch.zeros(16, dtype=torch.bfloat16, device=dev)
    # B=1 Hq=32 Hkv=8 N=2048 d=128 needs 64.5 MiB of workspace: refused before
    # any pointer is touched (sizes are validated first)
    p = x.data_ptr()
    st = ea.attn_bwd_noalloc(p, p, p, p, p, p, p, p, p, 1, 32, 8, 2048, 128, 1, 0.1,
                             ea.ATTN_BF16, None)
    assert st == ea.ATTN_ERR_UNSUPPORTED
