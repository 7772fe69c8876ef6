"""NOSA decode hot path on AMD MI355X (gfx950).

The path (compressed keys -> block selection -> HBM block pool with host
gather -> sparse decode attention) runs in the HIP kernels of libnosa.so,
reached through the C ABI declared in include/nosa.h.  This package holds the
ctypes binding (`binding`), the build step (`build`) and the decode-step
driver that sequences the four calls on device buffers (`runner`).
"""
