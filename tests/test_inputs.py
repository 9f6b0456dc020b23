"""Host checks of the seeded input generators (no GPU): same seed, same
bits; and the structured score shapes the running-maximum tests rely on."""
import numpy as np
import torch

from exact_attention_15_amd.inputs import (WORKLOADS, make_dout_device, make_qkv, make_qkv_device,
                                           make_structured_qkv)


def test_seeded_inputs_repeat_bit_for_bit():
    a = make_qkv(1, 2, 33, 64, torch.bfloat16, seed=3, H_kv=1)
    b = make_qkv(1, 2, 33, 64, torch.bfloat16, seed=3, H_kv=1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert a[0].shape == (1, 2, 33, 64) and a[1].shape == (1, 1, 33, 64)
    c = make_qkv(1, 2, 33, 64, torch.bfloat16, seed=4, H_kv=1)
    assert not torch.equal(a[0], c[0])
    assert all(w.N >= 1 and w.H % w.kv_heads == 0 for w in WORKLOADS.values())


def _tile_maxima(q, k, tiles):
    s = q[0, 0].double() @ k[0, 0].double().T / q.shape[-1] ** 0.5
    row = s[-1].numpy()
    return np.array([row[64 * t:64 * (t + 1)].max() for t in range(tiles)])


def test_structured_rows_have_the_intended_shape():
    n, d = 300, 64
    rising = _tile_maxima(*make_structured_qkv("rising", 1, 1, n, d, torch.float32, 7)[:2], 5)
    # every full key tile raises the last row's maximum by more than 8 log2
    # units (the ragged fifth tile holds 44 keys)
    assert np.all(np.diff(rising[:4]) > 8 * np.log(2)) and rising[4] > rising[3], rising
    falling = _tile_maxima(*make_structured_qkv("falling", 1, 1, n, d, torch.float32, 7)[:2], 5)
    assert falling[0] == falling.max() and np.all(np.diff(falling) < 0), falling
    q, k, _ = make_structured_qkv("wide", 1, 1, n, d, torch.float32, 7)
    s = q[0, 0].double() @ k[0, 0].double().T / d ** 0.5
    assert 3.0 < float(s.std()) < 5.0
    # spikes at keys 78, 153, 228 (tiles 1, 2, 3): the last row's tile
    # maxima climb by more than 128 log2 units from one tile to the next
    spikes = _tile_maxima(*make_structured_qkv("spikes", 1, 1, n, d, torch.float32, 7)[:2], 5)
    assert np.all(np.diff(spikes[:4]) > 128 * np.log(2)), spikes
    assert abs(spikes[3] - 300.0) < 30.0 and spikes[4] < 10.0, spikes


def test_device_draws_repeat_and_follow_the_recipe():
    """The device-side draws (run here on the CPU generator): same seed, same
    bits; Q, K, V and dO of the requested shapes and dtype, K and V with
    H_kv heads; unit variance before rounding."""
    a = make_qkv_device(1, 4, 256, 64, torch.bfloat16, seed=5, H_kv=2, device="cpu")
    b = make_qkv_device(1, 4, 256, 64, torch.bfloat16, seed=5, H_kv=2, device="cpu")
    assert [t.shape for t in a] == [(1, 4, 256, 64), (1, 2, 256, 64), (1, 2, 256, 64)]
    assert all(t.dtype == torch.bfloat16 for t in a)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert not torch.equal(a[1], a[2])
    x = torch.cat([t.float().flatten() for t in a])
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1.0) < 0.02
    g = make_dout_device(1, 4, 256, 64, torch.float32, seed=5, device="cpu")
    assert g.shape == (1, 4, 256, 64) and not torch.equal(g, a[0].float())
