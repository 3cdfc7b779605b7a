"""The C-ABI library loads and exports every entry point include/oxa.h declares (no GPU needed)."""
import ctypes
import os
import re

from tests.lib_loader import ensure_built

import paged_attention_02_amd as oxa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "oxa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oxa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = ensure_built()
    names = declared_functions()
    assert {"oxa_paged_append_rope", "oxa_paged_append", "oxa_paged_decode", "oxa_ragged_prefill",
            "oxa_paged_prefill", "oxa_merge_states", "oxa_merge_state_pair", "oxa_rope_neox",
            "oxa_rope_llama31"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in oxa.SIGNATURES, f"binding lacks a signature for {n}"


def test_abi_version_and_status_strings():
    lib = ensure_built()
    assert lib.oxa_abi_version() == 8
    assert oxa.status_string(0) == "OXA_OK"
    assert oxa.status_string(20) == "OXA_DEV_NOT_EXCLUSIVE"
    assert oxa.status_string(8) == "OXA_ERR_SCRATCH_LIMIT"
    assert oxa.status_string(999) == "unknown"


def test_workspace_queries():
    ensure_built()
    assert oxa.oxa_paged_decode_workspace_bytes(8, 32, 1) == 0
    # the long MQA workload: 8 x 32 rows x 16 partitions x (128 + 1) floats
    assert oxa.oxa_paged_decode_workspace_bytes(8, 32, 16) == 8 * 32 * 16 * 129 * 4 == 2113536
    assert oxa.lib().oxa_ragged_prefill_workspace_bytes(4, 7680, 32, 128) == 0   # too large to split
    # load-balanced decode: partition states, unit starts [units + 1], then
    # (512 + units) piece states of [hq][128] f32 and [hq] f32
    a256 = lambda x: (x + 255) // 256 * 256

    def balanced(b, hq, p):
        units = b * p
        state = b * hq * p * 129 * 4 if p > 1 else 0
        slots = 512 + units
        return a256(state) + a256((units + 1) * 4) + a256(slots * hq * 512) + slots * hq * 4
    assert oxa.oxa_paged_decode_balanced_workspace_bytes(32, 32, 1) == balanced(32, 32, 1) == 8982784
    assert oxa.oxa_paged_decode_balanced_workspace_bytes(8, 32, 16) == balanced(8, 32, 16)
    assert oxa.oxa_paged_decode_balanced_workspace_bytes(1024, 8, 2) == balanced(1024, 8, 2)
    assert oxa.oxa_paged_decode_balanced_workspace_bytes(2049, 8, 1) == 0      # 2048 units at most
    assert oxa.oxa_paged_decode_balanced_workspace_bytes(683, 8, 3) == 0
    assert oxa.oxa_paged_decode_balanced_workspace_bytes(1024, 64, 2) == balanced(1024, 64, 2)
    # small prefill: 8 chunk states of 128 f32 (256-byte aligned) + 8 lse, per (row, head)
    assert oxa.oxa_ragged_prefill_workspace_bytes(2, 96, 32) == 8 * 96 * 32 * (512 + 4)
    assert oxa.oxa_paged_prefill_workspace_bytes(1, 1024, 32) == 8 * 1024 * 32 * (512 + 4)
    assert oxa.oxa_paged_prefill_workspace_bytes(1, 1025, 32) == 0
    assert oxa.oxa_ragged_prefill_workspace_bytes(1, 5, 3) == 8 * 5 * 3 * 516
    # append: one 8-byte record per check work-group (at most 1024 of them)
    assert oxa.oxa_paged_append_rope_workspace_bytes(32768) == 8192
    assert oxa.oxa_paged_append_rope_workspace_bytes(0) == 8192
    assert oxa.oxa_paged_append_workspace_bytes(32768) == 8192
