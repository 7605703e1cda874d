"""CPU fp64 oracles of the MuonH step (and of the Muon baseline and AdamW beside it).
Test infrastructure only (see muonh_oracle)."""
from .adamw_oracle import adamw_step
from .muonh_oracle import (NS_COEFFS, NS_EPS, frobenius_norm, hyperball_project,
                           init_radius, momentum_update, muon_wd_step, muonh_step,
                           newton_schulz, trial_norm)

__all__ = ["adamw_step", "NS_COEFFS", "NS_EPS", "frobenius_norm", "hyperball_project", "init_radius",
           "momentum_update", "muon_wd_step", "muonh_step", "newton_schulz", "trial_norm"]
