"""The C-ABI library (CPU only): it loads, exports every entry point that
include/ringattn.h declares, and rejects invalid arguments on the host before any
launch (these calls never reach the GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ringattn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from context_long_sequence_amd import _lib, build

    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    return _lib.load()


def test_header_declares_the_four_entry_points():
    names = _declared()
    for n in ("ring_attn_fwd_step", "lse_merge", "segment_mask_from_pos", "ring_attn_bwd_step"):
        assert n in names
    assert len(names) >= 8


def test_library_exports_every_declared_symbol(lib):
    from context_long_sequence_amd import EXPORTED

    names = _declared()
    assert sorted(EXPORTED) == names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.ra_abi_version() == 3
    assert lib.ra_status_string(0) == b"RA_OK"
    assert lib.ra_status_string(2) == b"RA_ERR_UNSUPPORTED"


def _shape(**kw):
    from context_long_sequence_amd._lib import RaShape

    base = dict(batch=1, q_len=64, kv_len=64, heads_q=4, heads_kv=2, head_dim=128, q_offset=0, kv_offset=0,
                causal=1, softmax_scale=0.088, dtype=1)
    base.update(kw)
    return RaShape(**base)


FAKE = 0x1000  # never dereferenced: every call below fails host-side validation


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 2),
    (dict(heads_q=3), 1),
    (dict(q_len=0), 1),
    (dict(dtype=7), 2),
    (dict(causal=2), 1),
    (dict(q_offset=-1), 1),
    (dict(softmax_scale=0.0), 1),
])
def test_fwd_step_rejects_invalid_shapes(lib, kw, status):
    s = _shape(**kw)
    st = lib.ring_attn_fwd_step(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, None)
    assert st == status
    assert lib.ra_last_error() != b""


def test_null_and_misaligned_pointers_are_rejected(lib):
    s = _shape()
    assert lib.ring_attn_fwd_step(None, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, None) == 1
    assert lib.ring_attn_fwd_step(ctypes.byref(s), None, FAKE, FAKE, None, 0, FAKE, FAKE, None) == 1
    assert lib.ring_attn_fwd_step(ctypes.byref(s), FAKE + 2, FAKE, FAKE, None, 0, FAKE, FAKE, None) == 1
    # segment range past seg_len
    s2 = _shape(q_offset=64)
    assert lib.ring_attn_fwd_step(ctypes.byref(s2), FAKE, FAKE, FAKE, FAKE, 100, FAKE, FAKE, None) == 1
    assert lib.ring_attn_bwd_step(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, FAKE,
                                  FAKE, None) == 1


def test_merge_segment_preprocess_validation(lib):
    assert lib.lse_merge(0, 4, 4, 128, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 1
    assert lib.lse_merge(1, 4, 4, 6, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 2
    assert lib.lse_merge(1, 4, 4, 128, FAKE, FAKE, FAKE, None, None, 0, None) == 1
    assert lib.lse_merge(1, 4, 4, 128, FAKE, FAKE, None, None, None, 0, None) == 1
    assert lib.segment_mask_from_pos(1, 10, None, FAKE, None) == 1
    assert lib.segment_mask_from_pos(1, 0, FAKE, FAKE, None) == 1
    assert lib.segment_mask_from_pos(1, 1 << 40, FAKE, FAKE, None) == 1
    assert lib.ring_attn_bwd_preprocess(1, 4, 4, 96, 1, FAKE, FAKE, FAKE, None) == 2
    assert lib.ring_attn_bwd_preprocess(1, 4, 4, 128, 5, FAKE, FAKE, FAKE, None) == 2


@pytest.mark.parametrize("kw,status", [(dict(head_dim=96), 2), (dict(heads_q=3), 1), (dict(q_len=0), 1)])
def test_fwd_step_merge_rejects_invalid_shapes(lib, kw, status):
    s = _shape(**kw)
    assert lib.ring_attn_fwd_step_merge(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, None, 0, None) == status


def test_fwd_step_merge_validation(lib):
    s = _shape()
    # NULL running result
    assert lib.ring_attn_fwd_step_merge(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, None, FAKE, None, 0, None) == 1
    assert lib.ring_attn_fwd_step_merge(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, FAKE, None, None, 0, None) == 1
    # unknown output dtype; o_out not 8-byte aligned; misaligned running result
    assert lib.ring_attn_fwd_step_merge(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, FAKE, 9, None) == 2
    assert lib.ring_attn_fwd_step_merge(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, FAKE + 4, 1,
                                        None) == 1
    assert lib.ring_attn_fwd_step_merge(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, FAKE + 8, FAKE, None, 0,
                                        None) == 1
    assert b"misaligned" in lib.ra_last_error()


def test_recv_copy_rejects_null_pointers(lib):
    assert lib.ring_recv_copy(None, None, 16, None) == 1  # RA_ERR_INVALID_ARGUMENT
    assert b"non-NULL" in lib.ra_last_error()
    assert lib.ring_recv_copy(None, None, 0, None) == 0  # zero bytes: nothing to do
