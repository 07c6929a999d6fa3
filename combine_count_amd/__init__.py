"""MI355X-native MoE expert-parallel dispatch + combine (one GPU's share).

The compute path is libepdc.so (hand-written HIP for gfx950) behind the C
ABI in include/epdc.h; this package is its Python binding.
"""
from .binding import (EPDC_BF16, EPDC_FP4X2, EPDC_FP8, EPDC_FP32, EPDC_MAX_SCALE_DIM, EPDC_STATUS_ROW_OUTSIDE,
                      EPDC_STATUS_WAIT_TIMEOUT, EPDC_STATUS_WORD, EXPORTS, EpCfg, EpdcError, PreparedCall,
                      dispatch_status, epdc_combine, epdc_combine_push, epdc_combine_reduce, epdc_dispatch,
                      epdc_dispatch_noalloc,
                      epdc_dispatch_scratch_bytes, epdc_landing_rows, epdc_last_error, load_library,
                      prepare_combine, prepare_combine_push, prepare_combine_reduce, prepare_dispatch)
from .buffers import DispatchBuffers, LandingBuffers

__all__ = ["EPDC_BF16", "EPDC_FP32", "EPDC_FP8", "EPDC_FP4X2", "EPDC_MAX_SCALE_DIM", "EPDC_STATUS_WORD",
           "EPDC_STATUS_WAIT_TIMEOUT", "EPDC_STATUS_ROW_OUTSIDE", "EXPORTS", "EpCfg", "EpdcError",
           "dispatch_status", "epdc_combine", "epdc_combine_push", "epdc_dispatch_noalloc",
           "epdc_combine_reduce", "epdc_dispatch", "epdc_dispatch_scratch_bytes", "epdc_landing_rows",
           "epdc_last_error", "load_library", "DispatchBuffers", "LandingBuffers", "PreparedCall",
           "prepare_dispatch", "prepare_combine", "prepare_combine_push", "prepare_combine_reduce"]
