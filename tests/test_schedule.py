"""Workgroup schedule of the tiled kernels (ids 12, 13 and 14), checked on the host through
mpgemm_prefill_schedule: every output tile is computed exactly once -- whole by one
workgroup, or split over P workgroups that take each K part once -- for every tile shape,
with and without the K split of small grids.  The schedule is the same function the
kernels call (x32_work_of), compiled for the host."""
import random

import pytest
import torch

import weight_only_quantized_mpgemm_amd as mp

CONFIGS = (12, 13, 14)
TILES = {12: (128, 256), 13: (256, 128), 14: (256, 256)}


def _padded_n(N):
    return (N + 15) // 16 * 16


def _check(M, N, K, cfg, cus):
    info, work = mp.prefill_schedule(M, N, K, cfg, cus)
    bm, bn = TILES[cfg]
    tm, tn = (M + bm - 1) // bm, (_padded_n(N) + bn - 1) // bn
    assert (info["tile_m"], info["tile_n"], info["tiles_m"], info["tiles_n"]) == (bm, bn, tm, tn)
    tiles, full, P, grid = tm * tn, info["full"], info["parts"], info["grid"]
    loop_k = info["loop_k"]
    assert loop_k % 256 == 0 and loop_k - 256 < (K + 127) // 128 * 128 <= loop_k
    assert grid == full + (tiles - full) * P == work.shape[0]
    # the split rule: only grids of fewer tiles than units, P parts of whole 256-deep
    # blocks, at least 1024 deep each, never with a ragged K
    if P > 1:
        assert cus > 0 and tiles < cus and tiles * P <= cus and full == 0
        assert loop_k % (256 * P) == 0 and loop_k // P >= 1024 and K == loop_k
    else:
        assert full == tiles
    mt, nt, part, sidx = (work[:, i] for i in range(4))
    assert bool(((mt >= 0) & (mt < tm) & (nt >= 0) & (nt < tn)).all())
    cover = torch.zeros(tm, tn, P, dtype=torch.int64)
    cover.index_put_((mt.long(), nt.long(), part.long()), torch.ones(grid, dtype=torch.int64),
                     accumulate=True)
    assert bool((cover == 1).all()), (M, N, K, cfg, cus)
    # whole tiles: part 0, no split index; split tile s: workgroups full + s P + p, part p
    assert bool((part[:full] == 0).all()) and bool((sidx[:full] == -1).all())
    if P > 1:
        b = torch.arange(full, grid)
        assert torch.equal(sidx[full:], ((b - full) // P).int())
        assert torch.equal(part[full:], ((b - full) % P).int())
        # the reduction kernel finds split tile s at tile index full + s: the same tile as
        # that of workgroup full + s of an unsplit launch
        _, flat = mp.prefill_schedule(M, N, K, cfg, 0)
        s = sidx[full::P].long()
        assert torch.equal(mt[full::P], flat[full + s, 0]) and torch.equal(nt[full::P],
                                                                          flat[full + s, 1])
    return info


@pytest.mark.parametrize("cfg", CONFIGS)
def test_schedule_covers_every_tile_once_at_the_workload_shapes(cfg):
    shapes = [(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096), (8192, 10240),
              (8192, 8192), (8192, 57344), (28672, 8192), (5120, 10240), (8192, 5120),
              (5120, 51200), (25600, 5120)]
    for K, N in shapes:
        for M in (65, 128, 512, 1024, 2048, 4096, 8192):
            _check(M, N, K, cfg, 256)


@pytest.mark.parametrize("cfg", CONFIGS)
def test_schedule_covers_every_tile_once_at_random_shapes(cfg):
    rng = random.Random(20 + cfg)
    splits = 0
    for _ in range(1500):
        M = rng.choice([rng.randint(1, 300), rng.randint(1, 5000), rng.randint(1, 20000)])
        N = rng.choice([rng.randint(1, 4000) * 8, rng.randint(1, 700) * 16])
        K = rng.choice([rng.randint(1, 4096) * 8, rng.randint(1, 64) * 256])
        cus = rng.choice([256, 256, 304, 80, 0])
        splits += _check(M, N, K, cfg, cus)["parts"] > 1
    assert splits > 50          # the split path is exercised, not only whole tiles


def test_split_takes_the_largest_part_count_that_fits():
    # 8 x 8192 tiles of 128 x 256 at M = 128, N = 2048: 8 tiles on 256 units, K = 8192
    info = _check(128, 2048, 8192, 12, 256)
    assert (info["grid"], info["parts"]) == (64, 8)
    # 1024-deep parts at least: K = 2048 allows 2
    assert _check(128, 2048, 2048, 12, 256)["parts"] == 2
    # ragged K (not a multiple of 256) never splits
    assert _check(128, 2048, 2048 + 128, 12, 256)["parts"] == 1
    # any part count to 8 that cuts K into whole 256-deep blocks: K = 5120 (20 blocks) at
    # 40 tiles takes five parts (200 workgroups), K = 25600 (100 blocks) at 40 tiles five
    assert _check(128, 10240, 5120, 12, 256)["parts"] == 5
    assert _check(128, 5120, 25600, 13, 256)["parts"] == 5
    # a grid with as many tiles as units runs whole
    assert _check(2048, 4096 * 4, 4096, 12, 256)["parts"] == 1
    # the 256 x 256 tile: 8 x 16 tiles at M = 2048, N = 4096 split K = 14336 (56 blocks) in
    # two; 8 x 112 tiles at N = 28672 run whole
    assert _check(2048, 4096, 14336, 14, 256)["parts"] == 2
    assert _check(2048, 28672, 4096, 14, 256)["parts"] == 1


def test_schedule_rejects_bad_arguments():
    lib = mp.lib()
    info = torch.zeros(8, dtype=torch.int32)
    for args in ((0, 64, 64, 12, 256), (64, 64, 64, 1, 256), (64, 64, 64, 12, -1),
                 (64, -8, 64, 13, 256)):
        assert lib.mpgemm_prefill_schedule(*args, info.data_ptr(), None, 0) == -1
    assert lib.mpgemm_prefill_schedule(64, 64, 64, 12, 256, None, None, 0) == -1
    assert lib.mpgemm_prefill_schedule(64, 64, 68, 12, 256, info.data_ptr(), None, 0) == -2


def test_wide_tile_runs_a_half_empty_last_round_as_narrower_tiles():
    # 8 x 112 = 896 tiles of 256 x 256 on 256 units: three rounds over 24576 columns, the
    # other 4096 as one round of 256 x 128 tiles
    assert mp.prefill_launches(2048, 28672, 4096, 14) == (2, 24576)
    # 16 x 40 = 640 (Llama-3-70B QKV at M = 4096): two rounds over 8192 columns
    assert mp.prefill_launches(4096, 10240, 8192, 14) == (2, 8192)
    # whole rounds, a last round more than half full, or no whole round: one launch
    assert mp.prefill_launches(8192, 28672, 4096, 14) == (1, 28672)     # 14 rounds
    assert mp.prefill_launches(2048, 6144, 4096, 14) == (1, 6144)       # 192 tiles
    assert mp.prefill_launches(1024, 28672, 4096, 14) == (1, 28672)     # 448: 1.75 rounds
    # units that the tile rows do not divide: one launch
    assert mp.prefill_launches(2048, 28672, 4096, 14, cus=304) == (1, 28672)
    # the other tiles always launch once
    for cfg in (12, 13):
        assert mp.prefill_launches(2048, 28672, 4096, cfg) == (1, 28672)
    # the split column falls on whole tiles and leaves whole tile rows for one more round
    rng = random.Random(5)
    for _ in range(2000):
        M, N = rng.randint(1, 20000), rng.randint(1, 4000) * 16
        n, col = mp.prefill_launches(M, N, 4096, 14)
        tm, tn = -(-M // 256), -(-N // 256)
        if n == 2:
            assert col % 256 == 0 and 0 < col < N
            assert tm * (col // 256) % 256 == 0                       # whole rounds
            assert 0 < 2 * tm * (-(-(N - col) // 256)) <= 256         # at most half a round
        else:
            assert col == N
