"""HIP graph capture of the entry points (GPU).

The library allocates nothing, records no memset and reads every per-call
input (lengths, slopes, layouts) from device memory, so one captured launch
can be replayed.  Each test captures a call on a side stream, then replays
the graph several times with eager work and synchronisations between the
replays, changing the device-side inputs between replays, and checks every
replay bit for bit against an eager call on the same inputs.
"""
import numpy as np
import pytest

import workloads

attn = pytest.importorskip("transformer_attention_attn_amd")


def bf16_tensor(bits, device):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def capture(fn):
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up launch outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.gpu
def test_graph_fwd_replays(device):
    import torch

    print("graph: attn_fwd causal GQA S=1000 D=128", flush=True)
    inp = workloads.make_inputs(1, 8, 2, 1000, 128, "bf16", seed=50)
    q, k, v = workloads.to_torch(inp, "bf16", device)
    out = torch.empty_like(q)
    g = capture(lambda: attn.fwd(q, k, v, mask="causal", out=out))
    rng = np.random.default_rng(51)
    for rep in range(3):
        # new inputs in place, some unrelated eager work, then the replay
        q.copy_(torch.from_numpy(rng.standard_normal(q.shape, dtype=np.float32)).to(device))
        junk = torch.randn(1 << 20, device=device).sum()
        g.replay()
        torch.cuda.synchronize()
        ref = attn.fwd(q, k, v, mask="causal")
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
        del junk


@pytest.mark.gpu
def test_graph_decode_replays_with_new_lengths(device):
    import torch

    print("graph: attn_decode B=4 Hq=32 Hkv=8 Smax=4096 D=128 with a workspace", flush=True)
    inp = workloads.make_decode_inputs(4, 32, 8, 1, 4096, 128, seed=52)
    q, k, v = (bf16_tensor(inp[n + "_bits"], device) for n in ("q", "k", "v"))
    lens = torch.tensor([4096, 100, 1, 3000], dtype=torch.int32, device=device)
    n_ws = attn.decode_workspace_bytes(4, 32, 8, 1, 4096, 128)
    ws = torch.empty(max(n_ws, 16), dtype=torch.uint8, device=device)
    out = torch.empty_like(q)
    g = capture(lambda: attn.decode(q, k, v, cache_len=lens, out=out, workspace=ws))
    for rep, new in enumerate(([4096, 100, 1, 3000], [17, 4000, 2048, 0], [1, 1, 1, 1])):
        lens.copy_(torch.tensor(new, dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        ref = attn.decode(q, k, v, cache_len=lens.clone())
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep


@pytest.mark.gpu
def test_graph_fwd_ex_replays_with_new_lengths_and_layout(device):
    import torch

    print("graph: attn_fwd_ex padded ALiBi and block-sparse", flush=True)
    inp = workloads.make_decode_inputs(2, 8, 2, 600, 600, 64, seed=53)
    q, k, v = (bf16_tensor(inp[n + "_bits"], device) for n in ("q", "k", "v"))
    slopes = torch.from_numpy(workloads.make_alibi_slopes(8)).to(device)
    ql = torch.tensor([600, 300], dtype=torch.int32, device=device)
    kl = torch.tensor([600, 300], dtype=torch.int32, device=device)
    out = torch.empty_like(q)
    g = capture(lambda: attn.fwd_ex(q, k, v, mask="causal", out=out, alibi_slopes=slopes,
                                    q_len=ql, kv_len=kl))
    for rep, (a, b) in enumerate(((600, 300), (1, 599), (64, 65))):
        ql.copy_(torch.tensor([a, b], dtype=torch.int32))
        kl.copy_(torch.tensor([a, b], dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        ref = attn.fwd_ex(q, k, v, mask="causal", alibi_slopes=slopes, q_len=ql.clone(),
                          kv_len=kl.clone())
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep

    nb = 10
    lay = torch.from_numpy(attn.layout_strided(nb, 1, 3).view(np.int32)).to(device)
    out2 = torch.empty_like(q)
    g2 = capture(lambda: attn.fwd_ex(q, k, v, mask="causal", out=out2, block_layout=lay))
    for rep, words in enumerate((attn.layout_strided(nb, 1, 3), attn.layout_fixed(nb, 3),
                                 attn.layout_bigbird(nb, 1, 1, np.arange(nb)[:, None] % nb))):
        lay.copy_(torch.from_numpy(words.view(np.int32)))
        g2.replay()
        torch.cuda.synchronize()
        ref = attn.fwd_ex(q, k, v, mask="causal", block_layout=lay.clone())
        torch.cuda.synchronize()
        assert torch.equal(out2.view(torch.int16), ref.view(torch.int16)), rep


@pytest.mark.gpu
def test_graph_distance_bias_replays_with_new_table(device):
    import torch

    print("graph: attn_fwd_ex with a distance-bias table, padded", flush=True)
    B, Hq, Hkv, S, D = 2, 8, 2, 500, 128
    inp = workloads.make_decode_inputs(B, Hq, Hkv, S, S, D, seed=54)
    q, k, v = (bf16_tensor(inp[n + "_bits"], device) for n in ("q", "k", "v"))
    table = torch.from_numpy(workloads.make_distance_bias(Hq, S, S, seed=55)).to(device)
    ql = torch.tensor([500, 200], dtype=torch.int32, device=device)
    out = torch.empty_like(q)
    g = capture(lambda: attn.fwd_ex(q, k, v, mask="causal_window", window=130, out=out,
                                    q_len=ql, kv_len=ql, dist_bias=table))
    for rep in range(3):
        table.copy_(torch.from_numpy(workloads.make_distance_bias(Hq, S, S, seed=56 + rep)))
        ql.copy_(torch.tensor([500 - 100 * rep, 200 + rep], dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        ref = attn.fwd_ex(q, k, v, mask="causal_window", window=130, q_len=ql.clone(),
                          kv_len=ql.clone(), dist_bias=table.clone())
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep


@pytest.mark.gpu
def test_graph_fp8_e5m2_d64_replays(device):
    import torch

    print("graph: attn_fwd FP8 E5M2 D=64 causal", flush=True)
    inp = workloads.make_inputs(1, 8, 2, 700, 64, "fp8_e5m2", seed=57)
    q, k, v = workloads.to_torch(inp, "fp8_e5m2", device)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=device)
    g = capture(lambda: attn.fwd(q, k, v, mask="causal", out=out))
    for rep in range(3):
        new = workloads.make_inputs(1, 8, 2, 700, 64, "fp8_e5m2", seed=58 + rep)
        q.copy_(torch.from_numpy(new["q_codes"]).view(torch.float8_e5m2).to(device))
        g.replay()
        torch.cuda.synchronize()
        ref = attn.fwd(q, k, v, mask="causal")
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep


@pytest.mark.gpu
def test_graph_windowed_decode_replays_with_new_lengths(device):
    import torch

    print("graph: attn_decode causal_window w=1000 B=4 Smax=8192 with a workspace", flush=True)
    inp = workloads.make_decode_inputs(4, 32, 8, 2, 8192, 128, seed=59)
    q, k, v = (bf16_tensor(inp[n + "_bits"], device) for n in ("q", "k", "v"))
    lens = torch.tensor([8192, 1500, 2, 999], dtype=torch.int32, device=device)
    n_ws = attn.decode_workspace_bytes(4, 32, 8, 2, 8192, 128, mask="causal_window", window=1000)
    ws = torch.empty(max(n_ws, 16), dtype=torch.uint8, device=device)
    out = torch.empty_like(q)
    g = capture(lambda: attn.decode(q, k, v, cache_len=lens, mask="causal_window", window=1000,
                                    out=out, workspace=ws))
    for rep, new in enumerate(([8192, 1500, 2, 999], [2, 8000, 1001, 4096], [1000, 1000, 1000, 3])):
        lens.copy_(torch.tensor(new, dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        ref = attn.decode(q, k, v, cache_len=lens.clone(), mask="causal_window", window=1000)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
