"""Seeded synthetic workloads for the paged KV-cache attention path.

Shared by the tests, the benchmark and the smoke check.  This package only
draws random numbers and lays out the *structure* of a workload: sequence
lengths, block tables handed out by a toy free-list allocator (with shared,
reference-counted prefix blocks), and which logical token rows exist.  It does
none of the method's arithmetic: it never computes a cache slot, gathers a
block or evaluates attention.  The oracle and the HIP path each derive those
on their own from what is generated here.
"""
from .gen import (  # noqa: F401
    Shape, Fill, DecodeStep, DecodeCase, PrefillCase,
    CONFIG_NAMES, decode_config, prefill_config, build_decode, build_prefill,
    bf16_bits_from_f32, poison_bits, np_storage_dtype, SamplerCase, sampler_case,
)
