"""MI355X (gfx950) GPT-2 training step: HIP kernels behind the C ABI in
include/gpt2.h, with a thin ctypes binding (``binding``)."""
from . import binding  # noqa: F401
from .binding import (DTYPE_BF16, DTYPE_F32, MODE_EVAL, MODE_TRAIN, Config, Model, lib,  # noqa: F401
                      make_config, num_params, param_table, query_sizes)
