"""optimizer_step_dl_amd -- the fused AdamW / AMSGrad optimizer step for
AMD Instinct MI355X (gfx950), as the C-ABI library ``libradamw.so`` and a thin
ctypes binding whose functions carry the C entry points' names.

Build in-tree first: ``python -m optimizer_step_dl_amd.build``.
"""
from ._abi import (  # noqa: F401
    AdamWState, Control, DecisionMismatch, FusedResult, Options, RadamwError, Segment, SegmentList, Stats, TensorList, EXPORTS,
    LIB_PATH,
    bucket_arena, bucket_segment, control, load, options, radamw_bucket_layout,
    radamw_check_decision, radamw_decide, radamw_fused_step_multi, radamw_fused_step_multi_noalloc, radamw_fused_workspace_bytes, radamw_grad_stats,
    radamw_grad_stats_rows, radamw_host_coefficients, radamw_last_hip_error, radamw_launch_count,
    radamw_list_create, radamw_list_destroy, radamw_list_fused_step, radamw_list_step, radamw_lists_fused_step,
    radamw_merge_stats, radamw_options_default, radamw_read_report, radamw_stats_plan,
    radamw_status_string, radamw_step, radamw_step_inplace, radamw_step_multi, radamw_step_multi_writeback,
    radamw_step_staged_inplace, radamw_stream_probe,
    radamw_time_next_update,
)
