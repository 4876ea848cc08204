"""Host-side facts the kernels rely on (CPU only)."""


def test_partition_by_multiply_high_is_exact():
    """The layout kernels compute an expert's partition e // Ep as
    (e * ceil(2^32 / Ep)) >> 32; check it for every expert id and every
    experts-per-partition count this build allows (E <= 1024)."""
    for ep in range(1, 1025):
        magic = -(-(1 << 32) // ep)
        for e in range(1024):
            assert (e * magic) >> 32 == e // ep, (e, ep)
