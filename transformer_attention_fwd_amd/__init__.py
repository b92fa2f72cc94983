"""MI355X (gfx950) attention forward: Python binding of the C-ABI library libfa.so (work in progress)."""
