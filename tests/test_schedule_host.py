"""Decode schedule argument checks, which run before any device memory is taken
(so they need no GPU): several queries per sequence and the pool-restricted
Full layer take one query per sequence only where the pages' Reindex does."""
import pytest

from kv_cache_compression_03_amd import schedule as sch


@pytest.mark.parametrize("layers,kw", [
    ("FRUU", dict(Tq=2)),                    # Reindex rescoring takes one query per sequence
    ("FUUU", dict(Tq=3, full_in_pool=True)),  # so does the Full Top-K inside the pool
    ("FUUU", dict(Tq=0)),
    ("UFUU", dict()),                        # Reuse before any selection
    ("RFUU", dict()),                        # Reindex before any Full layer
    ("FXUU", dict()),                        # unknown mode
])
def test_rejected_before_allocation(layers, kw):
    with pytest.raises(ValueError):
        sch.DecodeSchedule(layers, 2, 1000, 512, 8, 128, 64, 128, **kw, device="cpu")
