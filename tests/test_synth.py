"""The input generators (CPU): the device and host forms of the closed-form inputs
agree element for element, and their values are the dyadic ones the size-limit
tests rely on."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")


def test_closed_form_x_device_and_host_agree():
    M, K = 300, 384
    dev = synth.cf_x_torch(M, K, torch.device("cpu"), chunk=128).view(torch.int16).numpy().view(np.uint16)
    assert (dev == synth.cf_x(np.arange(M), K)).all()
    v = synth.bf16_bits_to_f32(synth.cf_x(np.arange(M), K)) if hasattr(synth, "bf16_bits_to_f32") else \
        (synth.cf_x(np.arange(M), K).astype(np.uint32) << 16).view(np.float32)
    assert v.min() == -8 and v.max() == 8 and (v == np.round(v)).all()


def test_closed_form_codes_device_and_host_agree():
    N, K = 200, 256
    dev = synth.cf_codes_torch(N, K, torch.device("cpu"), chunk=64).numpy()
    host = synth.cf_codes(np.arange(N), K)
    assert (dev == host).all() and host.max() == 15 and host.min() == 0


def test_closed_form_grid_values():
    z = synth.cf_zeros(np.arange(64), 20)
    assert z.min() == 0 and z.max() == 15
    s = synth.cf_scales(np.arange(8), 4).view(np.float16).astype(np.float64)
    assert set(np.unique(s)) == {2.0 ** -6, 2.0 ** -7, 2.0 ** -8, 2.0 ** -9}
