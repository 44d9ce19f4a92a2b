"""attn_decode_noalloc (static device scratch, no workspace argument) against
attn_decode (caller's workspace): the same kernels and split plan, so the
outputs must be bitwise equal.  Two calls in a row on one GPU, the second
with a smaller input, so the second reads the shared scratch after the first
left its partials there; plus a many-split MQA cache, a sliding window and a
call that needs no scratch."""
import pytest

torch = pytest.importorskip("torch")

import transformer_attention_attn_amd as attn  # noqa: E402

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, Sq, Smax, lengths, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    dev = torch.device("cuda:0")
    q = torch.randn(B, Hq, Sq, 128, generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn(B, Hkv, Smax, 128, generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn(B, Hkv, Smax, 128, generator=g).to(torch.bfloat16).to(dev)
    lens = torch.tensor(lengths, dtype=torch.int32, device=dev)
    return q, k, v, lens


def _check(q, k, v, lens, mask="causal", window=0):
    ref = attn.decode(q, k, v, cache_len=lens, mask=mask, window=window)
    out = torch.full_like(q, float("nan"))
    got = attn.decode_noalloc(q, k, v, cache_len=lens, mask=mask, out=out, window=window)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_noalloc_two_calls_second_smaller():
    B, Hq, Hkv, Sq, Smax = 16, 32, 8, 1, 4096
    assert attn.decode_workspace_bytes(B, Hq, Hkv, Sq, Smax, 128) > 0  # key splits in use
    lengths = [(97 * i + 13) % Smax + 1 for i in range(B)]
    _check(*_case(B, Hq, Hkv, Sq, Smax, lengths, seed=11))
    B2, Hq2, Hkv2, Sq2, Smax2 = 2, 8, 2, 2, 1500
    assert 0 < attn.decode_workspace_bytes(B2, Hq2, Hkv2, Sq2, Smax2, 128) < \
        attn.decode_workspace_bytes(B, Hq, Hkv, Sq, Smax, 128)
    _check(*_case(B2, Hq2, Hkv2, Sq2, Smax2, [1500, 333], seed=12))


def test_noalloc_many_splits_mqa_and_no_scratch():
    # one key/value head, 50001 of 65536 positions: 196 splits of eight tiles
    q, k, v, lens = _case(1, 8, 1, 1, 65536, [50001], seed=13)
    assert attn.decode_workspace_bytes(1, 8, 1, 1, 65536, 128) > 0
    _check(q, k, v, lens)
    # a sliding window of 1000 positions over ragged caches
    q, k, v, lens = _case(3, 16, 4, 2, 9000, [9000, 1200, 17], seed=16)
    _check(q, k, v, lens, mask="causal_window", window=1000)
    # caches of at most 256 positions: one split each, no scratch used
    q, k, v, lens = _case(64, 16, 4, 1, 256, [(37 * i) % 256 + 1 for i in range(64)], seed=14)
    assert attn.decode_workspace_bytes(64, 16, 4, 1, 256, 128) == 0
    _check(q, k, v, lens, mask="full")


def test_noalloc_allocates_no_torch_memory():
    q, k, v, lens = _case(16, 32, 8, 1, 4096, [4096] * 16, seed=15)
    out = torch.empty_like(q)
    attn.decode_noalloc(q, k, v, cache_len=lens, out=out)  # first call: scratch lookup
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for _ in range(3):
        attn.decode_noalloc(q, k, v, cache_len=lens, out=out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
