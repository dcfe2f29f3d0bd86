"""The static dealing of logical tiles to positions is a bijection on every
round (CPU; the GPU scheduler tests check the kernel against the same rule)."""
from tests.test_gpu_scheduler import static_position


def test_static_dealing_is_a_bijection_per_round():
    for num_tiles, p in ((12, 4), (560, 256), (1024, 256), (1000, 256), (7, 9), (4096, 256), (300, 250)):
        pos = [static_position(t, num_tiles, p) for t in range(num_tiles)]
        assert sorted(pos) == list(range(num_tiles))
        for base in range(0, num_tiles, p):
            chunk = pos[base:base + p]
            assert sorted(chunk) == list(range(base, min(base + p, num_tiles)))


def test_static_dealing_gives_each_xcd_a_contiguous_run():
    # 256 workers, XCD of worker u = u mod 8: each XCD's 32 tiles of a round are consecutive
    pos = [static_position(t, 1024, 256) for t in range(1024)]
    for rnd in range(4):
        for x in range(8):
            mine = sorted(pos[rnd * 256 + u] for u in range(x, 256, 8))
            assert mine == list(range(mine[0], mine[0] + 32))
