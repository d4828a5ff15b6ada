"""Routed-expert int4/int8 MoE step for MI355X (gfx950): Python binding of libmoe.

The work runs in hand-written HIP kernels behind the C ABI in include/moe.h;
this package only marshals arguments (see _lib.py).
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    MOE_EHIP,
    MOE_EINVAL,
    MOE_ENOMEM,
    MOE_ESTATE,
    MOE_OK,
    FILE_DIRECT,
    KERNELS_FAST,
    KERNELS_SCALAR,
    STORE_DEVICE,
    STORE_FILE,
    STORE_HOST,
    Config,
    GatedAttention,
    GatedDeltaNet,
    Model,
    MoeError,
    Pool,
    blob_offset,
    config_of,
    expert_bytes,
    expert_stride,
    last_error,
    lib,
    make_config,
    pack,
    pool_simulate,
    unpack,
)
