"""Paged KV-cache store and paged attention (decode, varlen prefill) for
AMD Instinct MI355X (gfx950).

The computation lives in ``libpkv.so`` (hand-written HIP kernels behind the C
ABI declared in ``include/pkv.h``); this package is a thin ctypes binding with
the same names. Importing the package does not load the library; the first
call does, and raises if it is missing (there is no CPU fallback).
"""

from .binding import (  # noqa: F401
    EXPORTS,
    DecodeGraphs,
    LIB_PATH,
    PkvError,
    SchedStep,
    Scheduler,
    StepMeta,
    StepPrep,
    kv_store,
    last_error,
    load_library,
    paged_attn_decode,
    paged_attn_decode_noalloc,
    paged_attn_decode_workspace_size,
    paged_attn_prefill_varlen,
    paged_attn_prefill_store,
    pkv_prefill_plan,
    pkv_prepare_step,
    pkv_rope_cos_sin,
    rope_kv_store,
    sample_temperature,
    sample_temperature_workspace_size,
    prefill_plan_capacity,
)
