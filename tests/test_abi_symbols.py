"""libue.so loads without a GPU and exports every function ue.h declares;
the Python binding declares a signature for each of them."""
import ctypes
import os
import re

import pytest

import moe_expert_load_ue_amd as ue

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ue.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(ue_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_parses():
    names = declared_functions()
    assert "ue_load" in names and "ue_plan" in names and "ue_reroute" in names
    assert "ue_weight_sync" in names and "ue_grad_reduce" in names
    assert len(names) >= 13


def test_library_exports_every_declared_symbol():
    if not os.path.exists(ue.LIB_PATH):
        pytest.fail("libue.so is not built (python -m moe_expert_load_ue_amd.build)")
    lib = ctypes.CDLL(ue.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_binding_covers_header():
    assert sorted(ue.SIGNATURES) == declared_functions()
    ue.library()   # sets every restype/argtypes without touching the GPU


def test_status_names():
    lib = ue.library()
    for code, name in ue.STATUS.items():
        assert lib.ue_status_name(code).decode() == name


def test_config_struct_matches_header():
    """The ctypes mirror of ue_config has the header's fields in order."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct ue_config \{(.*?)\} ue_config;", text,
                     flags=re.S).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert [f for f, _ in ue.ue_config._fields_] == fields
    assert ctypes.sizeof(ue.ue_config) == 4 * len(fields)
