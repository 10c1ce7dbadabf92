"""MI355X-native 3x3x3 submanifold sparse convolution (and its strided sibling).

The compute path is libssc.so (hand-written HIP for gfx950, C ABI in
include/ssc.h); ``binding`` marshals torch tensors into it.  ``workloads``
draws the seeded synthetic inputs.
"""
from .binding import (Plan, SparsePlan, SSCError, build_neighbor_map, build_sparse_map, conv_workspace_bytes,
                      decode_seq, encode_seq, grid_sample, grid_sample_bwd, grid_sample_fwd,
                      grid_sample_workspace_bytes, lib, lib_path, plan_bytes, plan_pair_counts, plan_row_orders,
                      plan_status,
                      seq_code_width, sparse_conv3d, sparse_conv3d_bwd, sparse_conv3d_fwd, sparse_out_coords,
                      sparse_out_shape, sparse_plan_status, sparse_workspace, status_string, subm_conv3d,
                      subm_conv3d_bwd, subm_conv3d_fwd, subm_conv3d_fwd_noalloc, workspace)

__all__ = ["Plan", "SparsePlan", "SSCError", "build_neighbor_map", "build_sparse_map", "sparse_conv3d",
           "sparse_conv3d_bwd", "sparse_conv3d_fwd", "sparse_out_coords", "sparse_out_shape", "sparse_plan_status",
           "sparse_workspace", "conv_workspace_bytes", "decode_seq", "encode_seq",
           "grid_sample", "grid_sample_bwd", "grid_sample_fwd", "grid_sample_workspace_bytes", "lib",
           "lib_path", "plan_bytes", "plan_pair_counts", "plan_row_orders", "plan_status", "seq_code_width", "status_string",
           "subm_conv3d", "subm_conv3d_bwd", "subm_conv3d_fwd", "subm_conv3d_fwd_noalloc", "workspace"]
