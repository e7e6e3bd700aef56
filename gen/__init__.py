"""Seeded synthetic inputs for the on-the-fly equivariant attention path.

This package is the only code shared by the CPU oracle and the HIP path.  It
holds no arithmetic of the method itself: it draws positions and irrep
features and projection weights, rounds them to bfloat16 storage when asked,
and builds padded neighbour lists with a k-d tree.  Every array it returns is plain numpy.
"""

from .configs import (  # noqa: F401
    CONFIGS,
    Config,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_config,
    make_micro,
    neighbour_list,
    proj_weights,
)
