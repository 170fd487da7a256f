"""MI355X-native MSA (Memory Sparse Attention) routed-layer hot path.

The computation lives in libmsa.so (HIP kernels for gfx950 behind the C ABI
of include/msa.h); ``_lib`` is its ctypes binding, ``memory`` holds the torch
device-memory plumbing, ``interleave`` the host loop of Memory Interleave.
"""
from ._lib import (MSA_BF16, MSA_F32, MsaBank, MsaError, MsaRope, default_scale, msa_abi_version,  # noqa: F401
                   msa_attend_workspace_bytes, msa_bank_layout, msa_device_pointer, msa_last_error, msa_layer_forward,
                   msa_layer_forward_noalloc, msa_layer_forward_reroute,
                   msa_layer_route, msa_layer_select_attend, msa_layer_workspace_bytes, msa_pool_memory,
                   msa_rope_table, msa_route_score, msa_route_workspace_bytes, msa_router_project, msa_scan_read_probe,
                   msa_sparse_attend,
                   msa_topk, msa_topk_workspace_bytes)
