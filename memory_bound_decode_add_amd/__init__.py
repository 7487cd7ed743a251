"""fdec: fused decode-MLP kernels for MI355X (gfx950), Python binding."""
