"""GPU properties of the HIP path that hold at any size (checked through the
C ABI): causality, window >= S equals causal, identical keys give the mean of
the visible values, grouped heads equal multi-head on repeated K/V, bitwise
reproducibility, no device allocation, and a non-default stream."""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


def _inputs(device, B, Hq, Hkv, S, D, dtype="bf16", seed=0):
    inp = workloads.make_inputs(B, Hq, Hkv, S, D, dtype, seed)
    return inp, workloads.to_torch(inp, dtype, device)


def test_causality_perturbation(device):
    """Rewriting K/V rows after position i0 leaves rows <= i0 bit-identical
    ("Transformer 架构及其变体", validation checklist, causality item)."""
    import torch
    import transformer_attention_attn_amd as attn

    S, i0 = 2048, 700
    _, (q, k, v) = _inputs(device, 1, 8, 2, S, 128, seed=1)
    for mask, w in (("causal", 0), ("causal_window", 300)):
        a = attn.fwd(q, k, v, mask=mask, window=w)
        k2, v2 = k.clone(), v.clone()
        k2[:, :, i0 + 1:] = torch.randn_like(k2[:, :, i0 + 1:].float()).to(k2.dtype)
        v2[:, :, i0 + 1:] = torch.randn_like(v2[:, :, i0 + 1:].float()).to(v2.dtype)
        b = attn.fwd(q, k2, v2, mask=mask, window=w)
        torch.cuda.synchronize()
        assert torch.equal(a[:, :, :i0 + 1], b[:, :, :i0 + 1])
        assert not torch.equal(a[:, :, i0 + 1:], b[:, :, i0 + 1:])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_window_ge_s_equals_causal(device, dtype):
    import torch
    import transformer_attention_attn_amd as attn

    S = 1000
    _, (q, k, v) = _inputs(device, 1, 4, 2, S, 64, dtype, seed=2)
    a = attn.fwd(q, k, v, mask="causal")
    for w in (S, S + 1, 1 << 30):
        b = attn.fwd(q, k, v, mask="causal_window", window=w)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_identical_keys_mean_of_visible_values(device):
    import torch
    import transformer_attention_attn_amd as attn

    S, D = 777, 128
    inp, (q, _, v) = _inputs(device, 1, 4, 4, S, D, "fp32", seed=3)
    k = torch.randn(1, 4, 1, D, device=device).expand(1, 4, S, D).contiguous()
    o = attn.fwd(q, k, v, mask="causal")
    cm = torch.cumsum(v.double(), dim=2) / torch.arange(1, S + 1, device=device).double()[:, None]
    torch.cuda.synchronize()
    assert float((o.double() - cm).abs().max()) < 1e-5
    o = attn.fwd(q, k, v, mask="causal_window", window=10)
    csum = torch.cumsum(v.double(), dim=2)
    lag = torch.cat([torch.zeros_like(csum[:, :, :10]), csum[:, :, :-10]], dim=2)
    cnt = torch.clamp(torch.arange(1, S + 1, device=device), max=10).double()[:, None]
    torch.cuda.synchronize()
    assert float((o.double() - (csum - lag) / cnt).abs().max()) < 1e-5


@pytest.mark.parametrize("mask", ["causal", "local_global"])
def test_gqa_equals_mha_on_repeated_kv(device, mask):
    import torch
    import transformer_attention_attn_amd as attn

    S, D, Hq, Hkv = 1100, 128, 8, 2
    _, (q, k, v) = _inputs(device, 2, Hq, Hkv, S, D, seed=4)
    g = [5, 600] if mask == "local_global" else None
    a = attn.fwd(q, k, v, mask=mask, window=40, global_idx=g)
    kr = k.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    vr = v.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    b = attn.fwd(q, kr, vr, mask=mask, window=40, global_idx=g)
    torch.cuda.synchronize()
    assert float((a.float() - b.float()).abs().max()) <= 2e-2
    # single key/value head (multi-query attention)
    c = attn.fwd(q, k[:, :1].contiguous(), v[:, :1].contiguous(), mask=mask, window=40,
                 global_idx=g)
    d = attn.fwd(q, k[:, :1].repeat(1, Hq, 1, 1).contiguous(),
                 v[:, :1].repeat(1, Hq, 1, 1).contiguous(), mask=mask, window=40, global_idx=g)
    torch.cuda.synchronize()
    assert float((c.float() - d.float()).abs().max()) <= 2e-2


def test_bitwise_reproducible_and_no_allocation(device):
    import torch
    import transformer_attention_attn_amd as attn

    w = workloads.WORKLOADS["causal_gqa_bf16_s8192"]
    _, (q, k, v) = _inputs(device, w.B, w.Hq, w.Hkv, w.S, w.D, seed=w.seed)
    outs = [torch.empty_like(q) for _ in range(4)]
    attn.fwd(q, k, v, mask="causal", out=outs[0])  # first launch loads the code object
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(device)[0]
    for o in outs:
        attn.fwd(q, k, v, mask="causal", out=o)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info(device)[0]
    # every buffer existed before the first reading: the calls allocate nothing
    assert free0 == free1, free0 - free1
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_non_default_stream(device):
    import torch
    import transformer_attention_attn_amd as attn

    _, (q, k, v) = _inputs(device, 1, 4, 4, 512, 64, seed=7)
    ref = attn.fwd(q, k, v, mask="causal")
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device)
    out = torch.empty_like(q)
    with torch.cuda.stream(s):
        attn.fwd(q, k, v, mask="causal", out=out)
    s.synchronize()
    assert torch.equal(out, ref)
    out2 = torch.zeros_like(q)
    attn.fwd(q, k, v, mask="causal", out=out2, stream=s)
    s.synchronize()
    assert torch.equal(out2, ref)


def test_only_global_rows_see_all(device):
    """With V = one-hot position codes, the weights reach the output: global
    rows spread weight over all S keys, band rows only over band + globals."""
    import torch
    import transformer_attention_attn_amd as attn

    S, D, w, g = 128, 128, 4, [0, 70]
    q = torch.randn(1, 1, S, D, device=device)
    k = torch.randn(1, 1, S, D, device=device)
    v = torch.eye(S, D, device=device)[None, None].contiguous()
    o = attn.fwd(q, k, v, mask="local_global", window=w, global_idx=g)
    torch.cuda.synchronize()
    nz = (o[0, 0] > 0).sum(dim=1).cpu().numpy()
    for i in range(S):
        if i in g:
            assert nz[i] == S
        else:
            band = min(i, w) + min(S - 1 - i, w) + 1
            extra = sum(1 for x in g if abs(x - i) > w)
            assert nz[i] == band + extra
