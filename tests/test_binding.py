"""Host-side checks of the Python binding (CPU only, no kernel call): tensors
that are not on the GPU, or not on q's GPU, are refused with ValueError
before any launch, so a host address can never reach a kernel."""
from types import SimpleNamespace

import pytest
import torch

attn = pytest.importorskip("transformer_attention_attn_amd")


def fake(dev):
    """A stand-in with a tensor's is_cuda / device attributes."""
    return SimpleNamespace(is_cuda=str(dev).startswith("cuda"), device=torch.device(dev))


def test_check_devices_accepts_one_gpu():
    q = fake("cuda:0")
    attn.check_devices(q, k=fake("cuda:0"), v=fake("cuda:0"), out=fake("cuda:0"), ws=None)


@pytest.mark.parametrize("name", ["k", "v", "out", "workspace"])
@pytest.mark.parametrize("bad", ["cpu", "cuda:1", "meta"])
def test_check_devices_refuses_other_devices(name, bad):
    q = fake("cuda:0")
    args = {n: fake("cuda:0") for n in ("k", "v", "out", "workspace")}
    args[name] = fake(bad)
    with pytest.raises(ValueError, match=name):
        attn.check_devices(q, **args)


def test_check_devices_refuses_host_q():
    with pytest.raises(ValueError):
        attn.check_devices(fake("cpu"), k=fake("cuda:0"))


def test_host_tensors_are_refused_before_any_launch():
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.fwd(q, q, q)
    with pytest.raises(ValueError):
        attn.fwd_ex(q, q, q)
    with pytest.raises(ValueError):
        attn.decode(q, q, q)
