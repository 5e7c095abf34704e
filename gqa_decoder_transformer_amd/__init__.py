"""MI355X (gfx950) GQA decoder forward pass: HIP kernels behind the C ABI of
include/ember.h, with a thin ctypes binding (``binding``)."""
