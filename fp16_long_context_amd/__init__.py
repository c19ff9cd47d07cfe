"""MI355X-native ThriftAttention prefill: quantize -> select -> fused FP16/MXFP4 attention.

The GPU work lives in libthrift.so (HIP for gfx950, C ABI declared in
include/thrift.h); this package only loads it and marshals torch tensors.
Importing the package does not load the library; the first call does, and
fails loudly if it has not been built.
"""
