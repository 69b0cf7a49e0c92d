"""MI355X-native packed low-bit MLA KV cache: fused writer and absorbed-MLA decode.

The compute path is the HIP library ``libmla_lowbit.so`` (C ABI declared in
``include/mla_lowbit.h``); this package only marshals torch tensors (device
memory and streams) into its calls. Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""
from .binding import (  # noqa: F401
    Config, C4R4, C2R4, MlaLowbitError, lib, version, page_bytes, decode_workspace_bytes,
    write, decode, decode_noalloc, decode_mq, write_decode, allocate_cache, LIB_PATH,
    qdq, bf16_page_bytes, bf16_decode_workspace_bytes, allocate_bf16_cache, bf16_write,
    bf16_decode,
)
