"""The E4M3 codec of the input generators (CPU): the code table from the OCP
FP8 definition at its landmarks, and the encoder against torch's
float8_e4m3fn conversion (an independent implementation)."""
import numpy as np
import pytest

from exact_attention_online_softmax_amd import inputs


def test_code_table_landmarks():
    t = inputs.E4M3
    assert t[0x00] == 0.0 and t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0            # largest finite
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9     # smallest normal, subnormal
    assert t[0x07] == 7 * 2.0 ** -9
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert not np.isinf(t).any()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                          # codes 0..0x7e increase


def test_encoder_matches_torch():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    g = np.random.default_rng(5)
    x = np.concatenate([g.standard_normal(50000).astype(np.float32) * s for s in (0.003, 1.0, 40.0)]
                       + [inputs.E4M3[:0x7F].astype(np.float32),
                          ((inputs.E4M3[1:0x7F] + inputs.E4M3[:0x7E]) / 2).astype(np.float32)])
    x = np.concatenate([x, -x, np.array([500.0, -1e9], np.float32)])
    mine = inputs.to_e4m3_bits(x)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    assert np.array_equal(inputs.e4m3_bits_to_f32(mine)[np.isfinite(x)],
                          torch.from_numpy(ref).view(torch.float8_e4m3fn).float().numpy()[np.isfinite(x)])
    assert inputs.to_e4m3_bits(np.array([np.nan], np.float32))[0] == 0x7F
