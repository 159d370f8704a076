"""MI355X-native lossless BF16 MLP-weight codec and reconstructive GEMMs.

The product is the C-ABI library ``libunweight.so`` (include/unweight.h);
``decode_gemm_exp_amd.uw`` is its thin Python binding and
``decode_gemm_exp_amd.synth`` draws the seeded synthetic inputs.
"""
