"""Layer-streamed transformer training step for MI355X (gfx950).

fp32 master weights and AdamW moments live in host memory; each decoder layer
is streamed into one of two device buffers, run forward, recomputed and run
backward by hand-written HIP kernels, and its gradients are sent back to the
host where a multithreaded AdamW updates the state.

The compute path is the C-ABI library ``libmt.so`` (declared in ``include/mt.h``);
``host_memory_streamed_amd.mt`` is its thin ctypes binding. Importing this
package loads nothing; ``synth`` draws the seeded synthetic inputs.
"""
