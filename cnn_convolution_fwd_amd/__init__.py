"""cfwd: forward 2-D convolution for CNN inference on AMD Instinct MI355X (gfx950).

The computation lives in the HIP library ``libcfwd.so`` (C ABI in
``include/cfwd.h``); ``binding`` is its ctypes front end.  Importing this
package does not load the library; the first call does, and fails loudly if it
has not been built (``python -m cnn_convolution_fwd_amd.build``).
"""
from .binding import (Algo, CfwdError, ConvDesc, algo, algo_name, conv2d_fwd, desc_for, fastrun_clear,  # noqa: F401
                      fastrun_load, fastrun_lookup, fastrun_save, fastrun_select, filter_size, list_candidates,
                      make_desc, output_dims, prepare_filter, resolve_algo, version, workspace_size)

__all__ = ["Algo", "CfwdError", "ConvDesc", "algo", "algo_name", "conv2d_fwd", "desc_for", "fastrun_clear",
           "fastrun_load", "fastrun_lookup", "fastrun_save", "fastrun_select", "filter_size", "list_candidates",
           "make_desc", "output_dims", "prepare_filter", "resolve_algo", "version", "workspace_size"]
