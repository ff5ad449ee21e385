"""MI355X-native batched K-token verify pass of MTP speculative decoding.

The HIP library (``libvq.so``, C ABI in ``include/vq.h``) holds the three
operations of the verify pass: a skinny quantized matmul, a multi-row decode
attention and exact Leviathan–Chen acceptance. ``speculative_decoding_verify_vq_amd.vq``
is its ctypes binding; importing it loads the library and fails if it is not
built. ``speculative_decoding_verify_vq_amd.stack`` composes the operations into
one verify step of a dense stack.
"""
__version__ = "0.1.0"
