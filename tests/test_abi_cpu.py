"""The C ABI library loads and exports every entry point include/casgd.h
declares; host-only entry points behave as documented.  No GPU needed."""

import os
import re

import pytest

from communication_avoiding_mixed_amd import binding as B
from oracle import casgd_oracle as O

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "casgd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(casgd_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("casgd_create", "casgd_outer_step", "casgd_loss", "casgd_destroy"):
        assert must in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libcasgd.so is not built (run __graft_entry__.build())")
    lib = B.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(B.SIGNATURES)


def test_host_only_entry_points():
    assert B.gram_bytes(16, 64, packed=True) == O.gram_bytes(16, 64, True)
    assert B.gram_bytes(32, 128, packed=False) == O.gram_bytes(32, 128, False)
    assert B.load().casgd_gram_bytes(0, 4, 1) == -1
    for k in range(5):
        assert B.step_seed(0, k) == O.step_seed(0, k)
        assert B.step_seed(2 ** 64 - 1, k) == O.step_seed(2 ** 64 - 1, k)


def test_invalid_arguments_are_rejected_without_a_device():
    lib = B.load()
    assert not lib.casgd_create(None, None, 10, 10, 0, 0)
    assert b"NULL" in lib.casgd_last_error()
    assert lib.casgd_outer_step(None, 1, 1, 0.1, 0, None) == B.EINVAL
    assert lib.casgd_set_stream(None, None) == B.EINVAL
    lib.casgd_destroy(None)
