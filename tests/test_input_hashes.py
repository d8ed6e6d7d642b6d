"""The tiny workload's seeded inputs are reproducible: their SHA-256 hashes match the ones
recorded in tests/golden/tiny_4k_input_sha256.json (written by make_input_hashes.py from the
input generators alone).  A change of seed, shape, dtype, value range or generator shows up
here before it shows up as a parity difference."""

import importlib.util
import json
import os

import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "tiny_4k_input_sha256.json")


def _maker():
    spec = importlib.util.spec_from_file_location(
        "make_input_hashes", os.path.join(HERE, "golden", "make_input_hashes.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _recorded(kind):
    with open(GOLDEN) as fh:
        return json.load(fh)[kind]


def test_tiny_inputs_sha256_cpu():
    assert _maker().tiny_input_hashes(torch.device("cpu")) == _recorded("cpu")


@pytest.mark.gpu
def test_tiny_inputs_sha256_gpu(gpu):
    assert _maker().tiny_input_hashes(gpu) == _recorded("cuda")
