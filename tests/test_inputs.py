"""CPU checks of the seeded input generator: reproducibility, distribution
and the low-bit storage recipe (decoded by the oracle's own unpacking)."""
import numpy as np
import torch

from moe_inputs import CONFIGS, make_router, make_x, quantize_pack, tensor_to_numpy_storage
from oracle import moe_oracle as O


def test_seeded_and_reproducible():
    c = CONFIGS[1]
    a, b = make_x(c), make_x(c)
    assert torch.equal(a, b)
    assert not torch.equal(make_x(c, batch=1), a)


def test_x_distribution():
    c = CONFIGS[2]
    x = make_x(c).float()
    assert abs(x.mean().item()) < 0.05 and abs(x.std().item() - 1.0) < 0.05


def test_quantizer_roundtrip_error_bound():
    g = torch.Generator().manual_seed(0)
    w = torch.randn(8, 256, generator=g) * 0.02
    for bits in (4, 2):
        packed, s16 = quantize_pack(w, bits)
        deq = O.dequantize(packed.numpy(), tensor_to_numpy_storage(s16), bits, 256)
        s = np.repeat(O.decode_fp16(tensor_to_numpy_storage(s16)), 32, axis=-1)
        qmax = (1 << (bits - 1)) - 1
        codes = O.unpack_codes(packed.numpy(), bits, 256)
        assert codes.min() >= -qmax and codes.max() <= qmax
        # nearest-code error within half a step, except where clamping hit
        # the fp16-rounded scale (at most one step there)
        err = np.abs(deq - w.double().numpy())
        assert (err <= s * 0.5 + 1e-12).mean() > 0.99
        assert (err <= s * 1.0 + 1e-12).all()


def test_zipf_bias_skews_prefill_routes():
    c = CONFIGS[3].with_(T=512)
    wr, bias = make_router(c)
    assert bias is not None and bias.shape == (512,)
    assert bias[0] > bias[1] > bias[-1]
    x = O.decode_bf16(tensor_to_numpy_storage(make_x(c)))
    l = O.router_logits(x, O.decode_bf16(tensor_to_numpy_storage(wr)), bias.double().numpy())
    ids = O.select_topk(l, c.k)
    counts = np.bincount(ids.reshape(-1), minlength=c.E)
    assert counts.max() > 10 * counts.mean()


def test_hotset_repeat_fraction():
    c = CONFIGS[5]
    wr, bias = make_router(c, layer=0)
    assert int((bias > 0).sum()) == c.hot_count
    x = O.decode_bf16(tensor_to_numpy_storage(make_x(c)))
    l = O.router_logits(x, O.decode_bf16(tensor_to_numpy_storage(wr)), bias.double().numpy())
    ids = O.select_topk(l, c.k)
    assert 0.5 < O.repeat_fraction(ids) < 0.8
