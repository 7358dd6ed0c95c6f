"""MI355X-native batch-1 matvec over losslessly compressed BF16 / fp8 weights.

The compute path is the HIP library ``libnwc.so`` (see ``include/nwc.h``);
``decode_matvec_amd.nwc`` is its thin ctypes binding.
"""
