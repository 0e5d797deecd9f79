"""The wave-aware token split (TokenWeave, abstract: two wave-aware token subsets).  Hand-derived cases:
256 x 256 output tiles, 256 compute units; a GEMM with N = 8192 has 32 column tiles, so 8 row tiles
(2048 rows) fill one wave."""
import pytest

from tensor_all_reduce_amd.schedule import gemm_waves, wave_aware_split


def test_gemm_waves():
    assert gemm_waves(0, 8192) == 0
    assert gemm_waves(1, 8192) == 1          # one row tile x 32 column tiles
    assert gemm_waves(2048, 8192) == 1       # 8 x 32 = 256 tiles
    assert gemm_waves(2049, 8192) == 2
    assert gemm_waves(4096, 8192) == 2
    assert gemm_waves(8192, 8192) == 4


@pytest.mark.parametrize("T,expect", [
    (8192, 4096),   # the workload's split: 2 + 2 waves, exactly half
    (512, 256),     # the smallest split
    (511, 511),     # fewer than two row tiles: not split
    (768, 256),     # 256 | 512 and 512 | 256 tie in waves and distance to T/2: the lower one
    (5000, 2048),   # 3 waves for 1024..2048 | rest and 3072..4096 | rest (1 + 2); 2048 is nearest to 2500
    (4608, 2048),   # 2304 | 2304 takes 2 + 2 waves, 2048 | 2560 only 1 + 2: wave-aware, not nearest to half
])
def test_wave_aware_split(T, expect):
    assert wave_aware_split(T, 8192) == expect


def test_split_is_a_tile_multiple_and_never_worse_than_halving():
    for T in range(512, 20000, 97):
        t1 = wave_aware_split(T, 8192)
        assert t1 % 256 == 0 and 0 < t1 < T
        half = (T // 2) // 256 * 256
        assert gemm_waves(t1, 8192) + gemm_waves(T - t1, 8192) <= gemm_waves(half, 8192) + gemm_waves(T - half, 8192)
