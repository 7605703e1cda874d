"""CPU fp64 oracle of the MuonH step. Test infrastructure only (see muonh_oracle)."""
from .muonh_oracle import (NS_COEFFS, NS_EPS, frobenius_norm, hyperball_project,
                           init_radius, momentum_update, muon_wd_step, muonh_step,
                           newton_schulz, trial_norm)

__all__ = ["NS_COEFFS", "NS_EPS", "frobenius_norm", "hyperball_project", "init_radius",
           "momentum_update", "muon_wd_step", "muonh_step", "newton_schulz", "trial_norm"]
