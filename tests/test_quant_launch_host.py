"""The activation-pass launch shapes that the GPU parity test
test_quantizer_launch_shapes runs cover every wave count (2, 4, 8, 16) and
every number of k-pairs per wave the pass's loop handles differently: none,
one (the step after the loop alone), two, three (a trip and that step) and
four (two trips).  Host only: the K split comes from the library's
activation layout, the rest from the launch rule the GPU test states."""
from tests.test_gpu_parity import QUANT_SHAPES, _quant_waves


def test_quantizer_launch_shapes_cover_the_loop():
    waves, counts = set(), set()
    for M, K, R, norm in QUANT_SHAPES:
        nw, c = _quant_waves(M, K, R, norm)
        waves.add(nw)
        counts |= c
    assert waves == {2, 4, 8, 16} and {0, 1, 2, 3, 4} <= counts, (waves, counts)
