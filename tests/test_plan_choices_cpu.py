"""The automatic plan for shapes whose choice was settled by measurement on MI355X
(host only: automatic plans need no device). Each row is a shape, the plan the library
picks for it, and what that plan measured against the alternative it replaced (bf16,
microseconds per call, one box); a change of rule that moves one of them should come
with new measurements."""
import pytest

from tiled_gemm_output_amd import tgemm

# (M, N, K) -> (tile_m, tile_n, split_k, stages, tail_split_k)
CHOICES = [
    ((8192, 8192, 8192), (256, 256, 1, 2, 0)),       # the 256x256 tile from one full round on
    ((4096, 4096, 4096), (256, 256, 1, 2, 0)),
    ((16384, 1024, 8192), (256, 256, 1, 3, 0)),      # 4 tile columns: A three K-steps ahead, 203.8 (211.6)
    ((1024, 16384, 8192), (256, 256, 1, 2, 0)),      # 211.8 (224.0 with A three ahead)
    ((6000, 6000, 6000), (256, 256, 1, 2, 3)),       # partly full last round as a split-K tail
    ((128, 8192, 8192), (128, 128, 4, 4, 0)),        # HBM-bound: 4 slices, one per CU, 4 stages (34.7 vs 39.8 with 8)
    ((2048, 1024, 8192), (128, 128, 4, 2, 0)),       # 128 tiles: 44.6 (was 71.7 unsplit)
    ((1536, 1536, 8192), (128, 128, 3, 2, 0)),       # 144 tiles: 53.3 (64.2 with 2 slices)
    ((1280, 1280, 8192), (128, 128, 5, 2, 0)),       # 41.4 (47.9 with 2)
    ((2048, 2048, 8192), (128, 128, 2, 2, 0)),       # 75.4 (81.9 unsplit)
    ((2048, 2048, 4096), (128, 128, 1, 2, 0)),       # 40.8 (44.3 with 4 stages, 46.0 in 2 slices)
    ((6713, 307, 3517), (128, 128, 3, 2, 0)),        # 43.3 (49.8 unsplit)
    ((768, 768, 8192), (128, 128, 7, 4, 0)),         # 24.0 (44.8 as 144 unsplit 64x64 tiles)
    ((768, 768, 2048), (64, 64, 1, 4, 0)),           # 13.5 (17.1 as 128x128 split)
    ((3072, 1536, 8192), (256, 256, 3, 2, 0)),       # 84.5 (102.7 as 128x128; 92.4 against 89.7 with A three ahead)
    ((8954, 586, 5871), (256, 256, 2, 3, 0)),        # 97.1 (108.9 as 128x128); 35 x 3 tiles: A three K-steps ahead
    ((16384, 512, 8192), (256, 256, 2, 3, 0)),       # 64 x 2 tiles in 2 slices: 131.1-132.4 (137.4-139.2 with A two ahead)
    ((1024, 1024, 65536), (256, 256, 16, 2, 0)),     # 154.4 (172.7 as 128x128 in 4; 151 against 140 with A three ahead)
    ((512, 2048, 8192), (128, 128, 4, 4, 0)),        # 32.1 (33.5 with 8 slices, two per CU)
    ((1024, 1024, 1024), (64, 64, 1, 4, 0)),         # short K: 64x64
    ((257, 2440, 3976), (128, 128, 4, 4, 0)),        # 60 tiles: 20.4 (27.2 as 195 unsplit 64x64 tiles)
    ((600, 1400, 4000), (128, 128, 4, 4, 0)),        # 21.2 (27.3 as 220 unsplit 64x64)
    ((251, 2033, 11048), (128, 128, 8, 4, 0)),       # 32 tiles: 29.9 (39.1 as 64x64 in 2 slices)
    ((512, 1024, 8192), (128, 128, 8, 4, 0)),        # 23.5 (27.2 as 64x64 in 2)
    ((1337, 272, 3365), (64, 64, 2, 4, 0)),          # 33 tiles over 53 K-tiles: 16.6 (17.6 as 128x128 in 6)
    ((633, 542, 3251), (64, 64, 2, 4, 0)),           # 16.5 (18.2 as 128x128 in 6)
    ((512, 512, 8192), (64, 64, 4, 4, 0)),           # 16 tiles: 18.1 (20.2 as 128x128 in 12)
    ((2048, 4096, 2048), (256, 128, 1, 2, 0)),       # one round of 256x128: 35.7 (37.7 as 128x128, two per CU)
    ((768, 7936, 4096), (256, 128, 1, 2, 0)),        # 52.9 (58.3 as 128x128)
    ((2560, 2560, 4096), (256, 128, 1, 2, 0)),       # 56.2 (61.0 as 128x128, 74.6 as 256x256)
    ((3072, 3072, 8192), (256, 256, 1, 2, 0)),       # 144 tiles: 143.2 (176.3 as 128x128, 195.8 as 256x128)
    ((3584, 3584, 4096), (256, 256, 1, 2, 0)),       # 196 tiles: 88.8 (106.1 as 256x128)
    ((1536, 1536, 2048), (128, 128, 1, 2, 0)),       # 20.3 (21.0 with 4 stages, 26.0 as 256x128, 24.5 as 64x64)
]


@pytest.mark.parametrize("shape,want", CHOICES, ids=str)
def test_automatic_plan(shape, want):
    M, N, K = shape
    p = tgemm.gemm_plan(None, M, N, K, 1 << 20, K, 1 << 21, N, 1 << 22, N, tgemm.BF16_BF16)
    got = (p["tile_m"], p["tile_n"], p["split_k"], p["stages"], p["tail_split_k"])
    assert got == want, (shape, p)
