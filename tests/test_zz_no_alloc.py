"""The no-allocation layer call (exmoe_moe_layer_noalloc, workspace = the library's fixed
per-GPU array) against exmoe_moe_layer with a caller workspace: every output bit for bit,
on two calls in a row with the second smaller, on the decode and prefill paths; sizes past
the array and the exactness counters are refused before anything runs."""
import numpy as np
import pytest

from synthetic import OLMOE, TINY
from tests.helpers import Layer, to_dev_bf16, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def exm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_mixture_experts_amd as m
    return m


def _outputs(b, T, k):
    import torch
    torch.cuda.synchronize()
    return [b.logits.view(torch.int16).cpu().numpy(), b.ids.cpu().numpy(), b.weights.cpu().numpy().view(np.int32),
            b.offsets.cpu().numpy(), b.sorted_flat.cpu().numpy()[:T * k], b.flat_to_sorted.cpu().numpy()[:T * k],
            b.y.view(torch.int16).cpu().numpy()]


def _same_as_layer(exm, lay, T, stream, flags=0, bias=None):
    import torch
    s = lay.shape
    x = to_dev_bf16(lay.syn.x(T, stream=stream))
    b = None if bias is None else torch.from_numpy(bias).cuda()
    ref = exm.moe_layer(x, lay.wr, lay.bank, s.I, s.k, bias=b, flags=flags)
    got = exm.LayerBuffers(T, s.H, s.I, s.E, s.k, flags)
    for t in (got.logits, got.y):
        t.view(torch.int16).fill_(0x7FC1)           # poison: every output must be written
    exm.moe_layer_noalloc(x, lay.wr, lay.bank, s.I, s.k, got, bias=b, flags=flags)
    names = ("logits", "ids", "weights", "offsets", "sorted_flat", "flat_to_sorted", "y")
    for n, a, r in zip(names, _outputs(got, T, s.k), _outputs(ref, T, s.k)):
        assert np.array_equal(a, r), f"T={T} flags={flags}: {n} differs from exmoe_moe_layer"


@pytest.mark.parametrize("Ts", [(16, 4), (16, 1)])
def test_no_alloc_olmoe_decode_twice(exm, Ts):
    log(f"no-alloc layer, OLMoE decode T={Ts}")
    lay = Layer(OLMOE, seed=0, oracle_experts=False)
    for i, T in enumerate(Ts):
        _same_as_layer(exm, lay, T, stream=40 + i)


def test_no_alloc_prefill_then_decode(exm):
    log("no-alloc layer, OLMoE Zipf prefill T=512 then T=128, tiny T=37 then T=5 on the grouped GEMM")
    lay = Layer(OLMOE, seed=0, oracle_experts=False)
    bias = lay.syn.zipf_bias()
    _same_as_layer(exm, lay, 512, stream=60, bias=bias)
    _same_as_layer(exm, lay, 128, stream=61, bias=bias)
    tiny = Layer(TINY, seed=0, oracle_experts=False)
    _same_as_layer(exm, tiny, 37, stream=62, flags=exm.PATH_PREFILL)
    _same_as_layer(exm, tiny, 5, stream=63, flags=exm.PATH_PREFILL)


def test_no_alloc_refuses_too_large_and_counters(exm):
    import torch
    s = OLMOE
    T = 1024                                       # needs more than the fixed 64 MiB array
    assert exm.moe_workspace_bytes(T, s.H, s.I, s.E, s.k) > 64 << 20
    x = torch.zeros((T, s.H), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((s.E, s.H), dtype=torch.bfloat16, device="cuda")
    bank = exm.ExpertBank(base=torch.zeros(exm.packed_expert_bytes(s.H, s.I) * s.E, dtype=torch.uint8, device="cuda"),
                          stride=exm.packed_expert_bytes(s.H, s.I))
    b = exm.LayerBuffers(T, s.H, s.I, s.E, s.k)
    b.y.view(torch.int16).fill_(0x1234)
    with pytest.raises(exm.ExmoeError) as ei:
        exm.moe_layer_noalloc(x, wr, bank, s.I, s.k, b)
    assert ei.value.status == exm.ERR_UNSUPPORTED and "67108864" in str(ei.value)
    with pytest.raises(exm.ExmoeError) as ei:
        exm.moe_layer_noalloc(x[:4], wr, bank, s.I, s.k, exm.LayerBuffers(4, s.H, s.I, s.E, s.k),
                              flags=exm.DEBUG_COUNTERS)
    assert ei.value.status == exm.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((b.y.view(torch.int16) == 0x1234).all()), "a refused call wrote its output"
