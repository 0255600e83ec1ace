"""The C-ABI library loads without a GPU and exports every symbol fg.h declares."""
import ctypes
import os
import re

from ragged_paged_attention_splitfuse_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fg.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(fg_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("fg_plan_pass", "fg_plan_info", "fg_plan_upload", "fg_kv_append",
                 "fg_attention_ragged", "fg_plan_destroy", "fg_status_string", "fg_abi_version"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    assert sorted(binding.SIGNATURES) == declared_functions()


def test_abi_version_and_status_strings():
    assert binding.fg_abi_version() == 1
    assert binding.status_string(0) == "ok"
    assert "twice" in binding.status_string(binding.FG_E_ALIAS)
    assert binding.status_string(12345) == "unknown status"


def test_struct_sizes_match_header_layout():
    # fg_pass_desc: 7 int32 + float, 3 pointers, 4 int32; fg_plan_info_t: 3 int64 + 8 int32
    assert ctypes.sizeof(binding.fg_pass_desc) == 32 + 24 + 16
    assert ctypes.sizeof(binding.fg_plan_info_t) == 24 + 32
