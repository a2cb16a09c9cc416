"""rl_rollout_amd: the S3R decode hot path (sparse self-draft, dense verify, exact
speculative accept) for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library libs3r.so (C ABI declared in include/s3r.h);
`rl_rollout_amd.s3r` is its thin Python binding. Importing this package does not
load the library; importing `rl_rollout_amd.s3r` does, and fails loudly if it is
missing.
"""
__all__ = ["workloads", "synth"]
