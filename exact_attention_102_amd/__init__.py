"""MI355X-native fused exact attention: hand-written gfx950 HIP kernels behind the
C ABI of include/fa.h (libfa.so), with a thin ctypes binding.

    from exact_attention_102_amd import fa_fwd, fa_bwd, FA_BWD_5GEMM_ATOMIC, FA_BWD_7GEMM
"""
from .binding import (FA_BWD_5GEMM_ATOMIC, FA_BWD_7GEMM, FA_ERR_HIP, FA_ERR_INVALID_ARG,  # noqa: F401
                      FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_OK, PASS_DKDV, PASS_DKDV_ATOMIC, PASS_DQ,
                      PASS_FWD, FAError, fa_bwd, fa_bwd_dkdv, fa_bwd_dq, fa_bwd_dq_delta, fa_bwd_preprocess,
                      fa_bwd_workspace_size, fa_config_name, fa_default_config, fa_fwd, fa_num_configs, fa_status_string, fa_version, lib,
                      fa_fwd_general, fa_bwd_general, fa_fwd_general_workspace_size,
                      fa_bwd_general_workspace_size, FaStrides, FaDropout, fa_fwd_dropout, fa_bwd_dropout,
                      fa_dropout_keep_scale, fa_bwd_noalloc, FA_ERR_TOO_LARGE, FA_NOALLOC_MAX_ROWS)
from .flops import attention_flops, mfa_op_counts, pairs  # noqa: F401
