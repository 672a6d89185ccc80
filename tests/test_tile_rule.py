"""sgemm_run's choice of matrix-core configuration, checked on the host.

sgemm_tile_choice reports, without touching a device, the block tile, K
slice and k sets that sgemm_run and the general form launch for a product on
a given number of compute units.  The tests compare it with the rule as
restated in tests/tile_rule.py (from include/sgemm.h) over a grid of shapes,
batches and CU counts, and pin the configurations of the measured workloads.
The GPU tests (test_gpu_parity.py) check that sgemm_run computes the bits of
the tile the rule names.
"""
import itertools

import pytest

import dense_fp32_matrix_03_amd as sg
from tile_rule import TILE_RULE, _expected_tile

TILE_SIZE = {name: (bm, bn) for name, bm, bn, _ in TILE_RULE}


@pytest.mark.parametrize("cus", [256, 304, 80])
def test_library_choice_matches_the_stated_rule(cus):
    dims = [1, 16, 33, 100, 130, 256, 300, 384, 512, 640, 777, 1000, 1024, 1500, 2048, 3000,
            4096, 8192]
    ks = [1, 32, 64, 100, 256, 512, 777, 1024, 1025, 2048, 4096]
    checked = 0
    for M, N in itertools.product(dims, dims):
        for K in ks:
            for batch in (1, 4):
                if M * N * batch > 1 << 28:
                    continue
                want = TILE_SIZE[_expected_tile(M, N, K, batch, cus)]
                bm, bn, bk, ksets = sg.sgemm_tile_choice(M, N, K, batch, cus)
                assert (bm, bn) == want, f"{M}x{N}x{K} batch {batch} on {cus} CUs"
                assert ksets in (1, 2, 4) and bk % 16 == 0
                checked += 1
    assert checked > 5000


# Configurations of the measured workloads on 256 CUs: (bm, bn, bk, k sets).
WORKLOAD_CONFIGS = [
    ((256, 256, 256, 1), (16, 16, 256, 4)),       # 16 x 16 small-product tile
    ((256, 256, 1024, 1), (16, 16, 1024, 4)),
    ((512, 512, 512, 1), (32, 32, 64, 4)),        # 32 x 32, 64-float slices
    ((768, 768, 768, 1), (32, 32, 32, 4)),        # more work-groups than CUs: 32-float slices
    ((1000, 1500, 777, 1), (64, 96, 32, 2)),      # 256 tiles: one 12-wave work-group per CU
    ((1000, 1700, 777, 1), (32, 32, 32, 4)),      # 288 tiles of 64 x 96: not one round
    ((640, 640, 2048, 1), (32, 64, 64, 2)),
    ((1024, 1024, 1024, 1), (64, 64, 32, 2)),     # two k sets of four waves
    ((1024, 1024, 1152, 1), (64, 64, 32, 2)),
    ((1024, 1024, 1280, 1), (64, 64, 64, 2)),     # 64-float slices from K = 1280
    ((1024, 1024, 1536, 1), (64, 64, 64, 2)),
    ((1024, 1024, 2048, 1), (64, 64, 64, 2)),
    ((3072, 3072, 1024, 1), (64, 64, 32, 1)),     # several work-groups per CU: four waves
    ((2048, 2048, 2048, 1), (128, 128, 32, 1)),
    ((8192, 8192, 8192, 1), (256, 256, 32, 1)),
    ((64, 64, 64, 1024), (64, 64, 32, 1)),        # a batch that fills the CUs
]


@pytest.mark.parametrize("shape,config", WORKLOAD_CONFIGS, ids=lambda v: "x".join(map(str, v)))
def test_workload_configurations(shape, config):
    M, N, K, batch = shape
    assert sg.sgemm_tile_choice(M, N, K, batch, 256) == config


def test_tile_choice_arguments():
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_tile_choice(0, 4, 4)
    assert e.value.status == sg._C["SGEMM_ERR_INVALID_VALUE"]
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_tile_choice(4, 4, 4, 1, 0)
    assert e.value.status == sg._C["SGEMM_ERR_INVALID_VALUE"]
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_tile_choice(1 << 31, 4, 4)
    assert e.value.status == sg._C["SGEMM_ERR_TOO_LARGE"]
