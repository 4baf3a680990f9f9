"""Host-side checks of the checkpoint files (lema_checkpoint_save/_load,
include/lema.h): argument validation and the parsing and checking of
safetensors headers, which both happen before any HIP call, so made-up
device addresses are never touched here.

LEMA README, "Features" (interval-based checkpointing of the delta and the
optimizer states) and "Selective Full Fine-Tuning" (a checkpoint holds the
fp32 delta plus the optimizer state; merge_delta reads safetensors files).
Reference files are written by the safetensors library itself, an
implementation independent of this one.
"""
from __future__ import annotations

import ctypes
import json
import os
import struct

import numpy as np
import pytest
from safetensors.numpy import save_file

from optimizer_step_lema_amd import _native as N

FAKE = 0x7F0000001000          # never dereferenced: every case fails or copies nothing


@pytest.fixture(scope="module")
def lib():
    return N.load()


def req(*specs):
    """(name, dtype, numel) triples -> a lema_ckpt_tensor array."""
    arr = (N.CkptTensor * len(specs))()
    for k, (name, dt, n) in enumerate(specs):
        arr[k] = N.CkptTensor(name if isinstance(name, (bytes, type(None))) else name.encode(),
                              dt, 0, FAKE if n else 0, n)
    return arr


def load(lib, path, arr, n=None):
    step = ctypes.c_int64(-99)
    st = lib.lema_checkpoint_load(os.fsencode(str(path)), arr, len(arr) if n is None else n,
                                  ctypes.byref(step), None)
    return st, step.value


def save(lib, path, arr, step=5):
    return lib.lema_checkpoint_save(os.fsencode(str(path)), arr, len(arr), step, None)


@pytest.mark.parametrize("name,dt,n,want", [
    (None, N.LEMA_DT_F32, 4, N.LEMA_ERR_NULL),
    ("a", 7, 4, N.LEMA_ERR_DTYPE),
    ("a", N.LEMA_DT_F32, -1, N.LEMA_ERR_SIZE),
    ("", N.LEMA_DT_F32, 4, N.LEMA_ERR_SIZE),
    ('a"b', N.LEMA_DT_F32, 4, N.LEMA_ERR_SIZE),
    ("a\\b", N.LEMA_DT_F32, 4, N.LEMA_ERR_SIZE),
    ("tab\there", N.LEMA_DT_F32, 4, N.LEMA_ERR_SIZE),
    (b"caf\xc3\xa9", N.LEMA_DT_F32, 4, N.LEMA_ERR_SIZE),
    ("x" * 256, N.LEMA_DT_F32, 4, N.LEMA_ERR_SIZE),
])
def test_request_validation(lib, tmp_path, name, dt, n, want):
    arr = req((name, dt, n))
    assert save(lib, tmp_path / "c.safetensors", arr) == want
    assert load(lib, tmp_path / "c.safetensors", arr)[0] == want
    assert not os.listdir(tmp_path)                 # nothing created


def test_more_validation(lib, tmp_path):
    p = tmp_path / "c.safetensors"
    dup = req(("a", N.LEMA_DT_F32, 4), ("b", N.LEMA_DT_I8, 4), ("a", N.LEMA_DT_BF16, 2))
    assert save(lib, p, dup) == N.LEMA_ERR_SIZE
    arr = req(("a", N.LEMA_DT_F32, 4))
    arr[0].data = None
    assert save(lib, p, arr) == N.LEMA_ERR_NULL
    arr = req(("a", N.LEMA_DT_F32, 4))
    arr[0].reserved = 1
    assert save(lib, p, arr) == N.LEMA_ERR_SIZE
    assert lib.lema_checkpoint_save(None, arr, 1, 0, None) == N.LEMA_ERR_NULL
    assert lib.lema_checkpoint_save(os.fsencode(str(p)), None, 1, 0, None) == N.LEMA_ERR_NULL
    assert lib.lema_checkpoint_save(os.fsencode(str(p)), arr, -1, 0, None) == N.LEMA_ERR_SIZE
    assert lib.lema_checkpoint_load(None, arr, 1, None, None) == N.LEMA_ERR_NULL
    assert not os.listdir(tmp_path)


@pytest.fixture()
def good(tmp_path):
    """A file written by the safetensors library: float32, bfloat16 (as raw
    uint16 bits re-labelled in the header) and int8 tensors with a step."""
    p = tmp_path / "ref.safetensors"
    save_file({"w": np.arange(6, dtype=np.float32), "c": np.arange(5, dtype=np.int8),
               "m2": np.zeros((3, 4), np.float32), "e": np.zeros(0, np.float32)}, str(p),
              metadata={"step": "17"})
    return p


def test_step_only_and_foreign_files(lib, good, tmp_path):
    """n = 0 reads just the step (no device copy, no HIP call); a file without
    an integer step gives -1; tensors the call does not name are ignored."""
    assert load(lib, good, req(), 0) == (N.LEMA_OK, 17)
    p = tmp_path / "nostep.safetensors"
    save_file({"w": np.ones(3, np.float32)}, str(p))
    assert load(lib, p, req(), 0) == (N.LEMA_OK, -1)
    p2 = tmp_path / "badstep.safetensors"
    save_file({"w": np.ones(3, np.float32)}, str(p2), metadata={"step": "ten"})
    assert load(lib, p2, req(), 0) == (N.LEMA_OK, -1)
    # requests of empty tensors copy nothing either
    assert load(lib, good, req(("e", N.LEMA_DT_F32, 0))) == (N.LEMA_OK, 17)


def test_request_mismatches(lib, good):
    """Checked against the header before any copy: a name the file lacks, the
    wrong dtype, the wrong element count (a 2-D tensor counts all its
    elements)."""
    assert load(lib, good, req(("nope", N.LEMA_DT_F32, 6)))[0] == N.LEMA_ERR_NOT_FOUND
    assert load(lib, good, req(("w", N.LEMA_DT_BF16, 6)))[0] == N.LEMA_ERR_DTYPE
    assert load(lib, good, req(("w", N.LEMA_DT_F32, 5)))[0] == N.LEMA_ERR_SIZE
    assert load(lib, good, req(("m2", N.LEMA_DT_F32, 4)))[0] == N.LEMA_ERR_SIZE
    assert load(lib, good, req(("c", N.LEMA_DT_F32, 5)))[0] == N.LEMA_ERR_DTYPE
    # the second request fails: nothing is copied for the first either
    assert load(lib, good, req(("w", N.LEMA_DT_F32, 6), ("nope", N.LEMA_DT_I8, 1)))[0] == \
        N.LEMA_ERR_NOT_FOUND


def raw(path, header, data=b"", hlen=None):
    h = header if isinstance(header, bytes) else json.dumps(header).encode()
    with open(path, "wb") as f:
        f.write(struct.pack("<Q", len(h) if hlen is None else hlen))
        f.write(h)
        f.write(data)


def entry(dtype, shape, b, e):
    return {"dtype": dtype, "shape": shape, "data_offsets": [b, e]}


@pytest.mark.parametrize("case", [
    "missing", "short", "hlen_beyond_file", "hlen_tiny", "not_json", "trailing_garbage",
    "not_object", "entry_not_object", "no_dtype", "bad_shape", "negative_dim",
    "offsets_past_end", "offsets_reversed", "size_mismatch", "float_number", "duplicate_name",
    "bad_escape", "deep_nesting"])
def test_malformed_files(lib, tmp_path, case):
    p = tmp_path / "bad.safetensors"
    data = bytes(24)
    w = entry("F32", [6], 0, 24)
    if case == "missing":
        pass
    elif case == "short":
        p.write_bytes(b"\x05\x00\x00")
    elif case == "hlen_beyond_file":
        raw(p, {"w": w}, data, hlen=1 << 20)
    elif case == "hlen_tiny":
        raw(p, b"{", data, hlen=1)
    elif case == "not_json":
        raw(p, b"{'w': 1}", data)
    elif case == "trailing_garbage":
        raw(p, json.dumps({"w": w}).encode() + b" x", data)
    elif case == "not_object":
        raw(p, b"[1, 2]", data)
    elif case == "entry_not_object":
        raw(p, {"w": [1]}, data)
    elif case == "no_dtype":
        raw(p, {"w": {"shape": [6], "data_offsets": [0, 24]}}, data)
    elif case == "bad_shape":
        raw(p, {"w": entry("F32", "6", 0, 24)}, data)
    elif case == "negative_dim":
        raw(p, {"w": entry("F32", [-6], 0, 24)}, data)
    elif case == "offsets_past_end":
        raw(p, {"w": entry("F32", [6], 0, 24)}, bytes(20))
    elif case == "offsets_reversed":
        raw(p, {"w": entry("F32", [0], 8, 4)}, data)
    elif case == "size_mismatch":
        raw(p, {"w": entry("F32", [5], 0, 24)}, data)
    elif case == "float_number":
        raw(p, b'{"w": {"dtype": "F32", "shape": [6.0], "data_offsets": [0, 24]}}', data)
    elif case == "duplicate_name":
        raw(p, b'{"w": ' + json.dumps(w).encode() + b', "w": ' + json.dumps(w).encode() + b"}",
            data)
    elif case == "bad_escape":
        raw(p, b'{"w\\q": ' + json.dumps(w).encode() + b"}", data)
    elif case == "deep_nesting":
        raw(p, b'{"__metadata__": {"x": ' + b"[" * 40 + b"]" * 40 + b"}}", data)
    assert load(lib, p, req(("w", N.LEMA_DT_F32, 6)))[0] == N.LEMA_ERR_IO


def test_escaped_and_unicode_names_parse(lib, tmp_path):
    """JSON escapes and non-ASCII names in another writer's header parse; a
    request can only name printable ASCII, so it finds the plain entry."""
    p = tmp_path / "esc.safetensors"
    w = entry("F32", [0], 0, 0)
    raw(p, b'{"a\\u00e9\\ud83d\\ude00\\n": ' + json.dumps(w).encode() + b', "plain": ' +
        json.dumps(w).encode() + b', "__metadata__": {"step": "-3"}}')
    assert load(lib, p, req(("plain", N.LEMA_DT_F32, 0))) == (N.LEMA_OK, -3)
    assert load(lib, p, req(("a", N.LEMA_DT_F32, 0)))[0] == N.LEMA_ERR_NOT_FOUND


def test_header_of_a_save_without_device_data(lib, tmp_path):
    """A save whose tensors are all empty writes the header alone (no HIP
    call): the safetensors library opens it and finds the names, dtypes and
    metadata; the header length is a multiple of 8; it loads back."""
    from safetensors import safe_open
    p = tmp_path / "empty.safetensors"
    arr = req(("0.master", N.LEMA_DT_F32, 0), ("0.exp_avg.codes", N.LEMA_DT_I8, 0),
              ("w", N.LEMA_DT_BF16, 0))
    assert save(lib, p, arr, step=123) == N.LEMA_OK
    assert sorted(os.listdir(tmp_path)) == ["empty.safetensors"]     # no temporary left
    with safe_open(str(p), "pt") as f:
        assert f.metadata() == {"format": "lema-checkpoint", "step": "123"}
        assert sorted(f.keys()) == ["0.exp_avg.codes", "0.master", "w"]
    data = p.read_bytes()
    n = struct.unpack("<Q", data[:8])[0]
    assert n % 8 == 0 and len(data) == 8 + n
    header = json.loads(data[8:])
    assert header["w"] == {"dtype": "BF16", "shape": [0], "data_offsets": [0, 0]}
    assert load(lib, p, arr) == (N.LEMA_OK, 123)


def test_save_into_a_missing_directory(lib, tmp_path):
    p = tmp_path / "no" / "such" / "dir.safetensors"
    assert save(lib, p, req(("a", N.LEMA_DT_F32, 0))) == N.LEMA_ERR_IO
    assert not (tmp_path / "no").exists()
