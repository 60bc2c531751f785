"""Float64 CPU oracle of the FLUX-class VAE decoder (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never does.
"""
from .vae_oracle import (  # noqa: F401
    EPS,
    GROUPS,
    TILE,
    TILE_OVERLAP_MIN,
    attention,
    causal_stack,
    conv2d,
    conv2d_at,
    conv3d_causal,
    conv3d_causal_at,
    decode,
    decode_causal3d,
    decode_tiled,
    denormalize,
    group_norm,
    group_norm_silu,
    pointwise_conv,
    resnet,
    resnet_causal3d,
    silu,
    softmax_rows,
    split_tiles,
    upsample_nearest2x,
)
