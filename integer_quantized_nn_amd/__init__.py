"""integer_quantized_nn_amd -- integer-quantized convolution and GEMM on MI355X.

The compute path is libiqnn.so (HIP kernels for gfx950 behind the C ABI in
include/iqnn.h); this package is its Python binding.  Importing the package
does not load the library; the first call does, and raises if it is missing.
"""
from .binding import (  # noqa: F401
    EPI_ADD, EPI_ADD_RELU, EPI_NONE, EPI_RAW_INT32, EPI_RELU, INT4, INT8, INT32, UINT4, UINT8,
    ConvDesc, GemmDesc, IqnnError, iqnn_abi_version, iqnn_choose_qparams, iqnn_dequantize, iqnn_maxpool2d, iqnn_qconv_fwd,
    iqnn_qconv_pair_fwd,
    iqnn_qconv_packed_size, iqnn_qconv_prepack, iqnn_qconv_prepack_host, iqnn_qgemm_fwd, iqnn_qgemm_packed_size,
    iqnn_qgemm_prepack, iqnn_qgemm_prepack_host,
    iqnn_quantize, iqnn_quantize_pad,
)
