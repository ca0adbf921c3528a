"""MI355X-native draft verification through a gated-delta-rule layer.

The C ABI (include/ldv.h, libldv.so) holds the HIP kernels for gfx950; this
package is its Python binding.  Importing the package loads the library and
fails if it has not been built.
"""
from .ldv import (LDV_BF16, LDV_F32, MAX_LONG_T, MAX_T, STATUS_BAD_ACCEPTED, STATUS_BAD_PARENT,  # noqa: F401
                  STATUS_BAD_POSITION, STATUS_BAD_SLOT, LdvError, commit_state, gather_states,
                  gather_states_packed, load, read_block_states, read_block_states_packed, select_accepted,
                  select_accepted_noalloc,
                  select_workspace_bytes, status_string, verify_chain, verify_chain_long, verify_tree, version)

load()
