"""The C-ABI library loads and exports every symbol include/mak.h declares;
host-side planning and argument validation work without a GPU (no compute
call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

from transformer_forward_pass_amd import mak, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mak.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mak_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("mak_plan", "mak_load", "mak_prefill", "mak_decode_step", "mak_generate",
              "mak_decode_batch", "mak_batch_max", "mak_free", "mak_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(mak.LIB_PATH), "libmak.so not built"
    out = subprocess.run(["nm", "-D", "--defined-only", mak.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    L = mak.lib()
    for n in _declared():
        assert hasattr(L, n)


def test_plan_sizes_arena_without_gpu():
    s = synth.SHAPES["llama-3.2-1b"]
    n = mak.plan(s)
    weights = s.n_params() * 2
    kv = s.kv_bytes_per_position() * s.max_seq
    assert weights + kv <= n <= weights + kv + 64 * 2 ** 20


@pytest.mark.parametrize("field,value", [("hidden", 100), ("head_dim", 48), ("n_kv_heads", 5),
                                         ("max_batch", 17), ("vocab", 0), ("max_seq", 0)])
def test_plan_rejects_bad_shapes(field, value):
    import dataclasses
    s = dataclasses.replace(synth.SHAPES["tiny"], **{field: value})
    with pytest.raises(mak.MakError) as e:
        mak.plan(s)
    assert e.value.code == mak.MAK_EINVAL


def test_plan_of_4bit_weights():
    import dataclasses
    s16 = synth.SHAPES["llama-3.2-1b"]
    s4 = dataclasses.replace(s16, weight_format="mxfp4")
    n16, n4 = mak.plan(s16), mak.plan(s4)
    # the linear weights shrink from 2 bytes to 17/32 of a byte each
    lin = s16.n_layers * (s16.hidden * (s16.q_dim + 2 * s16.kv_dim) + s16.q_dim * s16.hidden
                          + 3 * s16.hidden * s16.intermediate)
    saved = lin * 2 - (lin // 2 + lin // 32)
    assert abs((n16 - n4) - saved) <= 64 * 2 ** 20
    # 4-bit matrices need K a multiple of the 32-weight block
    for field, value in (("intermediate", 688), ("hidden", 80)):
        s = dataclasses.replace(synth.SHAPES["tiny"], weight_format="mxfp4", **{field: value})
        with pytest.raises(mak.MakError) as e:
            mak.plan(s)
        assert e.value.code == mak.MAK_EINVAL


def test_load_validates_before_touching_the_device():
    L = mak.lib()
    cfg = mak.make_config(synth.SHAPES["tiny"])
    h = ctypes.c_void_p()
    w = mak.mak_weights()
    # arena too small -> ENOMEM, NULL weights -> EINVAL; neither reaches HIP
    assert L.mak_load(ctypes.byref(cfg), None, ctypes.c_void_p(256), 1, None, ctypes.byref(h)) == mak.MAK_EINVAL
    assert L.mak_load(ctypes.byref(cfg), ctypes.byref(w), ctypes.c_void_p(256), 1, None,
                      ctypes.byref(h)) == mak.MAK_EINVAL
    assert b"missing" in L.mak_last_error()


def test_calls_on_null_model_fail_cleanly():
    L = mak.lib()
    assert L.mak_decode_step(None, 0, 0, 0, None, None) == mak.MAK_EINVAL
    assert L.mak_batch_max(None) == mak.MAK_EINVAL
    assert L.mak_slot_length(None, 0) == mak.MAK_EINVAL
    L.mak_free(None)
