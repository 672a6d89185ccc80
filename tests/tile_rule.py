"""The tile rule of sgemm_run, restated from its description in
include/sgemm.h, for the tests: the CPU tests check it against the library's
own choice (sgemm_tile_choice), the GPU tests check that sgemm_run computes
the bits of the tile it names."""

TILE_RULE = [("mfma_256", 256, 256, 512), ("mfma_128", 128, 128, 512),
             ("mfma_64x96", 64, 96, 768), ("mfma_64", 64, 64, 512),
             ("mfma_32x64", 32, 64, 256), ("mfma_32", 32, 32, 256), ("mfma_16", 16, 16, 256)]


def _small_product(M, N, K, batch, cus):
    """The 16 x 16 tile serves K <= 1024 with at most 8 of its tiles per CU
    and at most 128 KiB of operand reads per CU (128 K bytes per tile)."""
    tiles = -(-M // 16) * -(-N // 16) * batch
    return K <= 1024 and tiles <= 8 * cus and tiles * K * 128 <= 128 * 1024 * cus


def _expected_tile(M, N, K, batch, cus):
    def eff(name, bm, bn, threads):
        if name == "mfma_16":
            return 0.0
        tiles = -(-M // bm) * -(-N // bn) * batch
        if tiles * threads > 2 ** 32 - 1:
            return 0.0
        if name == "mfma_64x96" and tiles > cus:  # one round only
            return 0.0
        rounds = -(-tiles // cus)
        return float(M) * N * batch / (rounds * cus * bm * bn)
    best = max(eff(*t) for t in TILE_RULE)
    tiles16 = -(-M // 16) * -(-N // 16) * batch
    if _small_product(M, N, K, batch, cus) and (tiles16 * K * 128 <= 48 * 1024 * cus
                                                 or best < 0.5):
        return "mfma_16"
    for t in TILE_RULE:
        if eff(*t) >= 0.97 * best:
            return t[0]
    return "mfma_128"
