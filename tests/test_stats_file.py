"""Calibration statistics files: a round trip keeps every value and the RoPE settings, and a
file of another setting or shape is refused (CPU only)."""

import numpy as np
import pytest
import torch

import kv_cache_compression_tri_amd as tri


def _stats(n_layer=3, n_qh=5):
    g = torch.Generator().manual_seed(11)
    return torch.randn((n_layer, n_qh, 64, 2), generator=g), torch.rand((n_layer, n_qh, 64), generator=g) + 0.1


def test_round_trip_is_exact(tmp_path):
    c, m = _stats()
    p = tmp_path / "stats.npz"
    tri.save_stats(p, c, m, rope_base=5e5, rope_layout="interleaved")
    c2, m2, base, layout = tri.load_stats(p, device="cpu", rope_base=5e5, rope_layout="interleaved", n_layer=3, n_qh=5)
    assert torch.equal(c2, c) and torch.equal(m2, m)
    assert base == 5e5 and layout == "interleaved"
    assert c2.dtype == torch.float32 and c2.is_contiguous()


@pytest.mark.parametrize("field,value", [("rope_base", 1e6), ("rope_layout", "half"), ("n_layer", 4), ("n_qh", 8)])
def test_mismatched_setting_is_refused(tmp_path, field, value):
    c, m = _stats()
    p = tmp_path / "stats.npz"
    tri.save_stats(p, c, m, rope_base=5e5, rope_layout="interleaved")
    with pytest.raises(ValueError, match=field):
        tri.load_stats(p, device="cpu", **{field: value})


def test_malformed_files_are_refused(tmp_path):
    c, m = _stats()
    with pytest.raises(ValueError):
        tri.save_stats(tmp_path / "x.npz", c, m[:, :, :32], rope_base=1e6)
    with pytest.raises(ValueError):
        tri.save_stats(tmp_path / "x.npz", c, m, rope_base=1e6, rope_layout="diagonal")
    p = tmp_path / "bad.npz"
    np.savez(p, center=np.zeros((2, 3, 64, 2), np.float32), mean_abs=np.zeros((2, 3, 60), np.float32),
             rope_base=np.float64(1e6), head_dim=np.int64(128), rope_layout=np.str_("half"))
    with pytest.raises(ValueError, match="malformed"):
        tri.load_stats(p, device="cpu")
