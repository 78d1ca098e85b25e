"""Shape and launch-shape tables shared by the GPU parity tests and the host-side plan checks."""
from glu_mlp_gemv_amd import api

# VALU kernel (forced) at small shapes: ragged K, N tails, hidden in registers and in LDS
SMALL = [(1, 1, 8), (1, 3, 8), (1, 65, 64), (1, 3000, 1024), (2, 777, 520), (3, 1000, 4104),
         (5, 129, 2560), (8, 3000, 1024), (8, 640, 8192), (1, 100, 8192), (1, 300, 5128), (2, 257, 6144),
         (4, 1000, 4096)]

# MFMA kernels: shapes x launch-shape overrides (every override must plan on every shape)
MFMA_SHAPES = [(9, 100, 512), (16, 17, 64), (16, 1000, 1032), (17, 333, 2560), (32, 3000, 1024),
               (31, 64, 5120), (33, 200, 520), (70, 1000, 1024), (4, 999, 1024), (1, 2000, 2560),
               (2, 100, 40000), (8, 700, 8)]
MFMA_TUNINGS = [dict(), dict(mfma_segments=2), dict(mfma_segments=8, waves_per_block=2),
                dict(grid=3, waves_per_block=1), dict(mfma_hidden=2), dict(mfma_hidden=3),
                dict(mfma_hidden=3, mfma_segments=2, grid=2), dict(rows_per_wave=8),
                dict(rows_per_wave=8, mfma_segments=4, grid=3)]

# kernels driven through the exhaustive epilogue test
EPILOGUE_PATHS = {"valu": dict(kernel=api.KERNEL_VALU, gemv_dot=1), "generic": dict(kernel=api.KERNEL_GENERIC),
                  "valu_mfma_dot": dict(kernel=api.KERNEL_VALU, gemv_dot=2),
                  "mfma": dict(kernel=api.KERNEL_MFMA),
                  "mfma8": dict(kernel=api.KERNEL_MFMA, rows_per_wave=8),
                  "gemm": dict(kernel=api.KERNEL_GEMM)}

# tiled GEMM (M > 64 by default): shapes x tile overrides, ragged M, N and K tails
GEMM_SHAPES = [(33, 200, 520), (64, 1000, 1024), (70, 333, 2560), (128, 300, 1032), (200, 129, 2048),
               (256, 1000, 1024), (1, 5, 8), (17, 64, 64), (300, 77, 136)]
GEMM_TILES = [dict(), dict(gemm_tile_n=64, gemm_tile_m=64), dict(gemm_tile_n=64, gemm_tile_m=128),
              dict(gemm_tile_n=128, gemm_tile_m=64), dict(gemm_tile_n=128, gemm_tile_m=128),
              dict(mfma_depth=1), dict(gemm_tile_n=64, gemm_tile_m=128, mfma_depth=1),
              dict(gemm_tile_n=128, gemm_tile_m=128, mfma_depth=1), dict(mfma_depth=3), dict(mfma_depth=4),
              dict(gemm_tile_n=64, gemm_tile_m=128, mfma_depth=3), dict(gemm_tile_n=64, gemm_tile_m=128, mfma_depth=4)]
