"""CPU fp64 oracles of the MuonH step (and of the Muon baseline and AdamW beside it).
Test infrastructure only (see muonh_oracle)."""
from .adamw_oracle import adamw_step
from .bf16_state_oracle import (bf16_bits_to_f64, f32_to_bf16_bits, momentum_update_bf16_state,
                                round_real_to_bf16, round_to_bf16)
from .muonh_oracle import (NS_COEFFS, NS_EPS, frobenius_norm, hyperball_project,
                           init_radius, momentum_update, muon_wd_step, muonh_step,
                           newton_schulz)

__all__ = ["adamw_step", "bf16_bits_to_f64", "f32_to_bf16_bits",
           "momentum_update_bf16_state", "round_real_to_bf16", "round_to_bf16", "NS_COEFFS", "NS_EPS", "frobenius_norm", "hyperball_project", "init_radius",
           "momentum_update", "muon_wd_step", "muonh_step", "newton_schulz"]
