"""Planted mistakes in the oracle must each turn at least one pin red.

Each case compiles oracle.c with -DQP_PLANT=<n> into a temporary directory
(CPU only) and runs the whole pin battery against that build."""
import os
import shutil
import subprocess

import pytest

import oracle
from oracle.build import build
import pins

NPLANTS = oracle.get()._L.or_plant_count()
NAMES = oracle.get().plant_names()

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")


@pytest.mark.parametrize("plant", range(1, NPLANTS), ids=NAMES[1:])
def test_plant_turns_a_pin_red(plant, tmp_path):
    path = build(plant, outdir=str(tmp_path))
    o = oracle.Oracle(path)
    assert o.plant == plant
    failed = []
    for pin in pins.PINS:
        try:
            pin(o)
        except (AssertionError, ValueError) as e:
            failed.append((pin.__name__, str(e)[:80]))
    assert failed, f"planted fault {NAMES[plant]} passed every pin"
