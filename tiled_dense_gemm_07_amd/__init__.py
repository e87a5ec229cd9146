"""tilegemm for AMD Instinct MI355X (gfx950): tiled dense GEMM and weight-only
4-bit dequant GEMM as hand-written HIP kernels behind a C ABI (``include/tilegemm.h``).

The Python layer only marshals arguments: ``gemm``, ``dequant_gemm_w4`` and the
config queries live in :mod:`tiled_dense_gemm_07_amd.binding`, which loads
``libtilegemm.so`` on first use and raises if it is missing.
"""

from . import synth  # noqa: F401  (seeded inputs; no GEMM arithmetic)

_BINDING_NAMES = {
    "gemm", "dequant_gemm_w4", "query_config", "list_configs", "gemm_with_config",
    "dequant_gemm_w4_with_config", "load_library", "TileGemmError", "tile_map",
    "status_str", "library_path",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
