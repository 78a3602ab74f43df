"""Output-stationary tiled GEMM for MI355X (gfx950).

The product is the C-ABI library ``libtgemm.so`` (declared in include/tgemm.h);
``tiled_gemm_output_amd.tgemm`` is its thin ctypes binding. Importing this
package loads nothing; the binding loads the library on first use and raises if
it has not been built.
"""
