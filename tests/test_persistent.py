"""The persistent launch of the D = 128 bf16 kernel: with more work items than
compute units, one workgroup per CU walks a list of items and their key/value
tiles form one stream.

Shapes here have more items than the MI355X's 256 CUs, with ragged tails,
item counts that are not a multiple of the grid, every group size the kernel
packs (1, 2, 4, 8 query heads per item) and the three masks it serves.  Each
case compares every output element with the fp64 oracle, and the output with
attn_fwd_ex's (the same arithmetic, one workgroup per item) bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

attn = pytest.importorskip("transformer_attention_attn_amd")

CASES = [
    # (B, Hq, Hkv, S, mask, window)
    (3, 8, 2, 4100, "causal", 0),          # 390 items: a partial second round
    (1, 32, 8, 2113, "full", 0),           # 272 items
    (2, 16, 4, 3000, "causal_window", 700),
    (2, 16, 2, 2100, "causal", 0),         # eight heads per item (one wave per head)
    (1, 40, 40, 1800, "causal", 0),        # one head per item, 256 rows
    (9, 8, 4, 1000, "causal_window", 129),  # two heads per item
    (1, 8, 1, 8400, "full", 0),            # MQA
]


def items(B, Hq, Hkv, S):
    G = Hq // Hkv
    hp = 8 if G % 8 == 0 else 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    return B * Hkv * (G // hp) * -(-S // (256 // hp))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}-H{c[1]}x{c[2]}-S{c[3]}-{c[4]}")
def test_persistent_against_oracle(device, case):
    import torch

    B, Hq, Hkv, S, mask, window = case
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    assert items(B, Hq, Hkv, S) > cus, "the case must take the persistent launch"
    print(f"persistent case {case} items {items(B, Hq, Hkv, S)}", flush=True)
    inp = workloads.make_inputs(B, Hq, Hkv, S, 128, "bf16", seed=S + Hq)
    q, k, v = workloads.to_torch(inp, "bf16", device)
    o = attn.fwd(q, k, v, mask=mask, window=window)
    e = attn.fwd_ex(q, k, v, mask=mask, window=window)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), e.view(torch.int16))
    got = o.float().cpu().numpy().astype(np.float64)
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], mask, window)
    err = float(np.max(np.abs(got - ref)))
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= 2e-2, err


def test_persistent_repeatable(device):
    """Several launches of one persistent call (graph-free) agree bit for bit."""
    import torch

    inp = workloads.make_inputs(1, 32, 8, 4096, 128, "bf16", seed=77)
    q, k, v = workloads.to_torch(inp, "bf16", device)
    a = attn.fwd(q, k, v, mask="causal")
    for _ in range(3):
        b = attn.fwd(q, k, v, mask="causal")
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
