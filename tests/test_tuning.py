"""Host logic of the start-up autotuner: buckets, the table the entry points
consult, and the saved cache that is ignored when it belongs to another
library build or device."""

from __future__ import annotations

import json

import pytest

import activation_add_rmsnorm_amd as A
from activation_add_rmsnorm_amd import tuning


@pytest.fixture(autouse=True)
def empty_table():
    tuning.clear()
    yield
    tuning.clear()


def test_buckets():
    assert [tuning.bucket(t) for t in (0, 1, 2, 3, 4, 5, 1000, 1024, 1025, 4096)] == \
        [1, 1, 2, 4, 4, 8, 1024, 1024, 2048, 4096]


def test_table_lookup_by_bucket_and_width():
    assert tuning.variant_for("swiglu", 100, 8960) == -1
    tuning.set_variant("swiglu", 100, 8960, 2)
    assert tuning.variant_for("swiglu", 65, 8960) == 2           # same bucket (128)
    assert tuning.variant_for("swiglu", 129, 8960) == -1         # next bucket
    assert tuning.variant_for("swiglu", 100, 8968) == -1         # other width
    assert tuning.variant_for("swiglu_quant_fp8", 100, 8960) == -1
    # the entry points read the same table; an explicit variant always wins
    assert A._variant("swiglu", 100, 8960, -1) == 2
    assert A._variant("swiglu", 100, 8960, 0) == 0
    with pytest.raises(ValueError):
        tuning.set_variant("no_such_op", 1, 8, 0)


def test_variants_fitting_respect_capacity():
    for form in tuning.FORMS:
        for width in (8, 1536, 16384, 65536):
            vs = tuning.variants_fitting(form, width)
            if form == "swiglu_quant_fp8_dynamic" or not form.startswith("swiglu"):
                op, fmt = tuning.FORMS[form]
                assert A.pick_variant(op, 16, width, fmt) in vs
            assert vs


def test_saved_table_round_trip_and_staleness(tmp_path):
    tuning.set_variant("fused_add_rmsnorm", 4096, 1536, 5)
    tuning.set_variant("swiglu_quant_fp8_dynamic", 8192, 28672, 10)
    path = str(tmp_path / "tuned.json")
    tuning.save(path)
    tuning.clear()
    assert tuning.load(path) == 2
    assert tuning.variant_for("fused_add_rmsnorm", 4000, 1536) == 5
    assert tuning.variant_for("swiglu_quant_fp8_dynamic", 8192, 28672) == 10
    # another build of the library: the table is ignored
    data = json.load(open(path))
    data["identity"]["library_sha256"] = "0" * 16
    json.dump(data, open(path, "w"))
    tuning.clear()
    assert tuning.load(path) == 0 and not A._TUNED
    assert tuning.load(str(tmp_path / "missing.json")) == 0
