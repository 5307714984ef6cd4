"""Seeded synthetic workloads for the speculative-decoding verify step.

This package holds only input generation: the model shapes of the five
workloads, seeded weight / KV-cache / context-length / draft-randomness
generators, draft distributions for the sampled verify, the FastMTP draft
head's weights, and the byte accounting used to price a step.  It contains none
of the verify step's arithmetic; both the HIP library's callers and the CPU
oracle's callers draw their inputs from here.
"""
from .configs import CONFIGS, VerifyConfig, get_config, scaled
from .synth import (
    capacity_for,
    context_lengths,
    draft_randomness,
    kv_cache,
    make_weights,
    committed_tokens,
    mtp_config,
    mtp_model_weights,
    mtp_weights,
    sampled_drafts,
    tensor_seed,
)

__all__ = [
    "CONFIGS",
    "VerifyConfig",
    "get_config",
    "scaled",
    "capacity_for",
    "context_lengths",
    "draft_randomness",
    "kv_cache",
    "make_weights",
    "committed_tokens",
    "mtp_config",
    "mtp_model_weights",
    "mtp_weights",
    "sampled_drafts",
    "tensor_seed",
]
