"""Measured device peaks and the path they select (MI355X only).

gqla_measure_peaks streams a 1 GiB buffer (HBM read bandwidth) and runs dense bf16 MFMA
chains; gqla_select_path then applies the roofline rule of section 2 (Path selection)
of "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM Decoding" with the
measured ridge.  The measured values must lie within the device's published peaks
(8 TB/s HBM3E, 2.5 PFLOP/s dense bf16) and well above a tenth of them; the flagship
shape at s_q = 1 has absorb intensity 242 FLOPs/byte, below any ridge in that range, so
the absorb path must be chosen.
"""
import pytest

from latent_kv_cache_amd import gqla as mod

pytestmark = pytest.mark.gpu


def test_measured_peaks_select_absorb():
    import torch
    assert torch.cuda.is_available()
    mod.load()
    print("[gpu-case] measure peaks", flush=True)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    bw, fl = mod.measure_peaks(scratch)
    print(f"[gpu-case] measured {bw / 1e12:.2f} TB/s, {fl / 1e12:.0f} TFLOP/s, ridge {fl / bw:.0f}", flush=True)
    assert 0.8e12 < bw <= 8.0e12 * 1.02
    assert 0.25e15 < fl <= 2.5e15 * 1.02
    ch = mod.select_path(mod.make_shape(128, 8, 512, 64, 128, 1), 128, 128 * 8192, fl, bw)
    assert ch.path == mod.ABSORB and ch.s_q == 1
    # with the multi-token head the absorb path crosses the ridge (compute-bound) and still leads
    ch2 = mod.select_path(mod.make_shape(128, 8, 512, 64, 128, 2), 128, 128 * 8192, fl, bw)
    assert ch2.path == mod.ABSORB and ch2.tokens_per_s >= ch.tokens_per_s
