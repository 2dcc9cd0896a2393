"""fp64 CPU oracle of the GDN token mixer (test infrastructure only; see gdn_oracle.py)."""
from .gdn_oracle import (  # noqa: F401
    FLAG_CONV, FLAG_L2QK, FLAG_NORM, FLAG_GATE, FLAG_ALL, CONV_WIDTH,
    silu, sigmoid, short_conv, l2_normalize, gated_delta_rule, gated_delta_rule_product_form,
    zero_centred_rmsnorm, gdn_chain, chain_inputs, prefill_chain, conv_tail, gdn_prefill, gdn_decode,
    gdn_verify, gdn_commit, softplus, gate_alpha_beta, in_projection, out_projection,
    QSA_BLOCK, QSA_TOPK, partial_rope, qsa_compress, qsa_scores, qsa_select,
    gated_delta_rule_backward, recurrence_layer, recurrence_layer_backward, gdn_chain_backward,
    gdn_prefill_backward,
)
from .pool import run_chains, host_cores, default_workers, cpu_model  # noqa: F401,E402
