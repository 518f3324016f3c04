"""The C ABI without a GPU: the library loads, exports every symbol that
include/dflash.h declares, and rejects invalid calls on the host before any
HIP call (so these run on a machine without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def dfl():
    import block_draft_select_amd as m
    return m


def _declared():
    txt = open(os.path.join(ROOT, "include", "dflash.h")).read()
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported(dfl):
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(dfl.lib, n), n
    # and the binding exposes a function of the same name for each entry point
    for n in ("dflash_topk", "dflash_pair_scores", "dflash_trace", "dflash_verify", "dflash_cycle"):
        assert callable(getattr(dfl, n))


def test_version_and_strings(dfl):
    assert dfl.lib.dflash_abi_version() == 1
    assert dfl.lib.dflash_status_string(3) == b"DFLASH_ERR_WORKSPACE"
    assert dfl.lib.dflash_kernel_name(0) == b"topk"
    assert dfl.lib.dflash_kernel_name(99) == b""


def test_workspace_bytes_of_the_five_configs(dfl):
    import synth
    for cid, cfg in synth.CONFIGS.items():
        d = dfl.dims(cfg["B"], cfg["L"], cfg["V"], cfg["K"], cfg["r"], cfg["hidden"],
                     cfg["logit_kind"], cfg["param_kind"])
        n = dfl.workspace_bytes(d)
        R = cfg["B"] * cfg["L"]
        # the chunk statistics alone take B*(L+1)*ceil(V/4096)*16 bytes
        assert n >= cfg["B"] * (cfg["L"] + 1) * (-(-cfg["V"] // 4096)) * 16
        assert n >= R * cfg["r"] * 4
        assert n < 64 << 20


@pytest.mark.parametrize("field,value,status", [
    ("B", 0, 1), ("L", 0, 1), ("L", 17, 1), ("K", 0, 1), ("K", 17, 1), ("V", 8, 1),
    ("V", 4 * 1024 * 1024, 2), ("r", 8, 1), ("r", 264, 1), ("r", 40, 1), ("hidden", 8, 1),
    ("hidden", 100, 1), ("logit_dtype", 7, 1), ("param_dtype", -1, 1), ("V", 1001, 2),
])
def test_bad_dims_rejected(dfl, field, value, status):
    d = dfl.dims(2, 8, 4096, 16, 256, 256, "bf16", "bf16")
    setattr(d, field, value)
    n = ctypes.c_size_t(12345)
    assert dfl.lib.dflash_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == status
    assert n.value == 12345
    assert dfl.lib.dflash_last_error() != b""
    # every entry point refuses the same dims before touching any pointer
    assert dfl.lib.dflash_topk(ctypes.byref(d), None, None, None, None, 0, None) == status
    assert dfl.lib.dflash_cycle(ctypes.byref(d), *([None] * 8), 0, *([None] * 8), None, 0, None) == status


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_vocab_limit(dfl, kind):
    d = dfl.dims(1, 1, dfl.V_MAX, 16, 16, 16, kind, kind)
    assert dfl.lib.dflash_workspace_bytes(ctypes.byref(d), ctypes.byref(ctypes.c_size_t())) == 0
    d = dfl.dims(1, 1, dfl.V_MAX + 8, 16, 16, 16, kind, kind)
    assert dfl.lib.dflash_workspace_bytes(ctypes.byref(d), ctypes.byref(ctypes.c_size_t())) == 2


def test_stream_row_limit(dfl):
    d = dfl.dims(65535 // 9, 8, 4096, 16, 16, 16, "bf16", "bf16")
    assert dfl.lib.dflash_workspace_bytes(ctypes.byref(d), ctypes.byref(ctypes.c_size_t())) == 0
    d = dfl.dims(65535 // 9 + 1, 8, 4096, 16, 16, 16, "bf16", "bf16")
    assert dfl.lib.dflash_workspace_bytes(ctypes.byref(d), ctypes.byref(ctypes.c_size_t())) == 2


def test_null_and_misaligned_pointers_rejected(dfl):
    d = dfl.dims(1, 2, 4096, 4, 16, 16, "bf16", "bf16")
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)
    assert dfl.lib.dflash_topk(ctypes.byref(d), None, fake, fake, fake, 1 << 30, None) == 1
    assert b"U is NULL" in dfl.lib.dflash_last_error()
    assert dfl.lib.dflash_topk(ctypes.byref(d), odd, fake, fake, fake, 1 << 30, None) == 1
    assert b"aligned" in dfl.lib.dflash_last_error()
    # workspace checks come after pointer checks and still launch nothing
    assert dfl.lib.dflash_topk(ctypes.byref(d), fake, fake, fake, None, 1 << 30, None) == 3
    assert dfl.lib.dflash_topk(ctypes.byref(d), fake, fake, fake, fake, 16, None) == 3
    assert b"too small" in dfl.lib.dflash_last_error()
    assert dfl.lib.dflash_read_probe(fake, 17, fake, None) == 1
    assert dfl.lib.dflash_conv2tap(ctypes.byref(d), fake, fake, None, fake, None) == 1
    assert b"Wt is NULL" in dfl.lib.dflash_last_error()
    assert dfl.lib.dflash_conv2tap(ctypes.byref(d), odd, fake, fake, fake, None) == 1
    assert b"aligned" in dfl.lib.dflash_last_error()
    assert dfl.lib.dflash_cycle_maxsum(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, fake, 0, fake,
                                       fake, None, None, None, None, None, None, fake, 1 << 30, None) == 1
    assert b"h is NULL" in dfl.lib.dflash_last_error()
    begins = (ctypes.c_int32 * 2)(0, 2048)
    assert dfl.lib.dflash_topk_merge(ctypes.byref(d), 2, begins, fake, fake, fake, None, None) == 1
    assert b"cand_logit is NULL" in dfl.lib.dflash_last_error()
    assert dfl.lib.dflash_topk_merge(ctypes.byref(d), 0, begins, fake, fake, fake, fake, None) == 1
    bad_begins = (ctypes.c_int32 * 2)(0, 4094)  # last shard narrower than K
    assert dfl.lib.dflash_topk_merge(ctypes.byref(d), 2, bad_begins, fake, fake, fake, fake, None) == 1
    assert b"at least K" in dfl.lib.dflash_last_error()
    assert dfl.lib.dflash_trace_viterbi(ctypes.byref(d), fake, fake, fake, None, fake, None) == 1
    assert b"draft_tok is NULL" in dfl.lib.dflash_last_error()
    bad = dfl.dims(1, 17, 4096, 4, 16, 16, "bf16", "bf16")
    assert dfl.lib.dflash_trace_viterbi(ctypes.byref(bad), fake, fake, fake, fake, fake, None) == 1
    assert dfl.lib.dflash_profile_collect(42, None, None) == 1


def test_static_cycle_rejects_sizes_beyond_its_scratch(dfl):
    # B (L + 1) = 65535 rows of a tiny vocabulary need about 152 MiB of
    # workspace, above the static scratch: rejected on the host, before any
    # HIP call (this runs without a GPU)
    d = dfl.dims(3855, 16, 64, 16, 16, 16, "bf16", "bf16")
    assert dfl.workspace_bytes(d) > dfl.STATIC_SCRATCH_BYTES
    nul = ctypes.c_void_p(0)
    st = dfl.lib.dflash_cycle_static(ctypes.byref(d), *([nul] * 8), 0, *([nul] * 8), nul)
    assert st == dfl.ERR_WORKSPACE
    assert b"static maximum" in dfl.lib.dflash_last_error()
    bad = dfl.dims(0, 8, 1024, 16, 256, 256, "f32", "f32")
    assert dfl.lib.dflash_cycle_static(ctypes.byref(bad), *([nul] * 8), 0, *([nul] * 8), nul) == dfl.ERR_INVALID_ARG
