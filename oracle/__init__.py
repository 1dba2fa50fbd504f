"""CPU oracle (test infrastructure only; never called by the library)."""

from .kvq_oracle import (  # noqa: F401
    CACHE_KEYS,
    GROUP,
    attention,
    decode_all,
    decode_slab,
    default_scale,
    dequant_slab,
    hadamard_rotate,
    pack_all,
    pack_codes,
    pack_slab,
    pack_value_codes,
    quantize_groups,
    retained_mask,
    rotate_query,
    slab_of,
    split_positions,
    unpack_codes,
    unpack_value_codes,
    value_bit_position,
    upcast,
)
from .kvq_stream import SlabStream  # noqa: F401
from .kvq_headq import (  # noqa: F401
    corrected_keys,
    decode_slab_headq,
    headq_side_slab,
    project_residual,
    side_code,
)
