"""fp64 CPU oracle for the S3R decode hot path.

TEST INFRASTRUCTURE: imported only by tests/, the smoke check in
__graft_entry__.py and the cpu_baseline leg of bench.py. It shares no code with
the HIP library or its binding.
"""
from .s3r_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    commit,
    dense_verify_attn,
    inverse_cdf,
    num_selected,
    select_budget,
    softmax_row,
    sparse_draft_attn,
    spec_accept,
)
from .enumeration import (  # noqa: F401
    accept_probability,
    corrected_distribution,
    dense_joint,
    joint_first_tokens,
)
