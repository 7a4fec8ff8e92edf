"""cnn_backward_pass_amd: conv-block backward pass for MI355X (gfx950).

The compute lives in the HIP library ``libcbb.so`` (C ABI declared in
``include/cbb.h``); ``cnn_backward_pass_amd.cbb`` is its thin ctypes binding.
``synth`` holds the seeded synthetic inputs of the five workloads.
"""
