"""fp64 CPU oracle of the MuonClip step — test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the HIP library and its binding never do.
"""
from .muonclip_oracle import *  # noqa: F401,F403
from .muonclip_oracle import (NS_A, NS_B, NS_C, NS_EPS, NS_STEPS, adamw_step, attention_forward,
                              clip_factor, clip_factor_global, decoupled_update, f32, max_logits,
                              max_logits_bruteforce, momentum, muonclip_step_matrix,
                              nesterov_direction, newton_schulz, ns_flops, qk_clip_rows, rms_matched,
                              round_to_bf16)
