"""fp64 CPU oracle for QK-Normed MLA decode (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the HIP path never does.  The training / prefill forward and
backward (explicit form, torch fp64 autograd) is in qkmla_train_oracle.
"""
from .qkmla_oracle import (absorb_weights_ref, absorbed_decode, append_ref, default_tau,
                           explicit_decode, explicit_decode_multi, explicit_logits,
                           group_of_head, plain_mla_decode, rms, rmsnorm, rope, rope_inv_freq, rowwise_rel_err)

__all__ = ["absorb_weights_ref", "absorbed_decode", "append_ref", "default_tau",
           "explicit_decode", "explicit_decode_multi", "explicit_logits", "group_of_head", "plain_mla_decode",
           "rms", "rmsnorm", "rope", "rope_inv_freq", "rowwise_rel_err"]
