"""MI355X-native Dynamic Bifocal RoPE attention (prefill + single-token decode).

The compute runs in the HIP library libbifocal.so (C ABI in include/bifocal.h); this
package only marshals torch tensors (device memory, the current stream) into that ABI.
There is no fallback: if the library is missing, every entry point raises.

Submodules:
  bifocal    -- the binding: bifocal_prefill, bifocal_prefill_chunk, bifocal_decode,
                bifocal_decode_varlen, bifocal_decode_step, the unfused three-pass
                forms, bifocal_positions, ...
  workloads  -- seeded synthetic inputs (no attention arithmetic)
  build      -- compiles the library in-tree with hipcc for gfx950
"""
from .bifocal import (BifocalError, bifocal_decode, bifocal_decode_step, bifocal_decode_varlen, bifocal_decode_varlen_workspace_bytes,  # noqa: F401
                      bifocal_decode_unfused, bifocal_decode_unfused_workspace_bytes, bifocal_decode_workspace_bytes,
                      bifocal_prefill_unfused, bifocal_prefill_unfused_workspace_bytes, decode_unfused, prefill_unfused,
                      bifocal_group_size, bifocal_positions, bifocal_prefill, bifocal_prefill_chunk,
                      bifocal_prefill_workspace_bytes, bifocal_status_string, decode, decode_step, decode_varlen, library_path,
                      load_library, positions, prefill, prefill_chunk)
