"""layer_streaming_amd: a layer-streamed decoder training step for MI355X.

The compute lives in the C-ABI library ``libmt.so`` built from ``csrc/``
(declared in ``include/mt.h``); ``layer_streaming_amd.mt`` is its ctypes
binding.  Importing this package does not load the library, so the input
generators in ``synth`` stay importable on machines without a build.
"""
