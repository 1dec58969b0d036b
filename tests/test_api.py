"""Host-side behaviour of the C ABI, without a GPU: the library loads, exports every
function include/kda.h declares, and rejects bad arguments before touching the device.
Pointers below are never dereferenced: every call fails validation first."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def b():
    from gated_delta_rule_59_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libkda not built")
    binding.lib()
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(b):
    names = declared_functions()
    assert set(names) >= {"kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_workspace_bytes",
                          "kda_check_gates", "kda_status_string", "kda_last_error",
                          "kda_abi_version"}
    for n in names:
        assert hasattr(b.lib(), n), n
    assert b.lib().kda_abi_version() == b.ABI_VERSION == 4


def test_status_strings(b):
    for code, name in b.STATUS.items():
        assert b.lib().kda_status_string(code).decode() == name


FAKE = 1 << 40   # never dereferenced


def base_args(b, **kw):
    a = b.ChunkArgs()
    a.B, a.T, a.H, a.dk, a.dv, a.chunk = 1, 256, 4, 128, 128, 64
    a.act_dtype = a.gate_dtype = b.KDA_BF16
    a.out_dtype = b.KDA_F32
    tok = 256 * 4
    a.q = FAKE
    a.k = FAKE + tok * 128 * 2
    a.v = FAKE + 2 * tok * 128 * 2
    a.g = FAKE + 3 * tok * 128 * 2
    a.beta = FAKE + 4 * tok * 128 * 2
    a.o = FAKE + (1 << 30)
    for key, val in kw.items():
        setattr(a, key, val)
    return a


def call_chunk(b, a):
    return b.lib().kda_chunk_fwd(ctypes.byref(a), None), b.lib().kda_last_error().decode()


@pytest.mark.parametrize("field,value,status", [
    ("dk", 96, 2), ("dv", 256, 2), ("chunk", 48, 2), ("B", 0, 2), ("T", -1, 2), ("H", 0, 2),
    ("act_dtype", 7, 3), ("gate_dtype", 0, 3), ("flags", 16, 4), ("flags", 32, 4), ("segments", 9, 2), ("segments", -1, 2),
])
def test_chunk_rejects_bad_shapes_and_dtypes(b, field, value, status):
    rc, msg = call_chunk(b, base_args(b, **{field: value}))
    assert rc == status, msg
    assert msg


def test_walk_step_flags(b):
    """KDA_FLAG_WALK64 and KDA_FLAG_WALK128 exclude each other; 128-token steps cannot take
    checkpoints that fall between them. Without a flag, few (sequence, head) pairs compose two
    chunks per step (one 163,840-byte block per 128 tokens and head) and many take one (114,688
    bytes per 64-token chunk and head)."""
    rc, msg = call_chunk(b, base_args(b, flags=b.KDA_FLAG_WALK64 | b.KDA_FLAG_WALK128))
    assert rc == 4 and "exclude" in msg
    a = base_args(b, flags=b.KDA_FLAG_WALK128, ckpt=FAKE + (1 << 33), ckpt_every=64, ckpt_slots=4)
    rc, msg = call_chunk(b, a)
    assert rc == 4 and "between" in msg
    q = lambda a: b.lib().kda_chunk_fwd_workspace_bytes(ctypes.byref(a))  # noqa: E731
    assert q(base_args(b, H=8)) == 2 * 8 * 163840                  # 8 pairs: composed
    assert q(base_args(b, H=9)) == 4 * 9 * 114688                  # 9 pairs: one chunk per step
    assert q(base_args(b, H=9, flags=b.KDA_FLAG_WALK128)) == 2 * 9 * 163840
    assert q(base_args(b, H=8, flags=b.KDA_FLAG_WALK64)) == 4 * 8 * 114688


def test_chunk_rejects_null_and_alias(b):
    assert call_chunk(b, base_args(b, q=None))[0] == 1
    assert call_chunk(b, base_args(b, o=None))[0] == 1
    a = base_args(b)
    a.o = a.v   # output on top of an input
    rc, msg = call_chunk(b, a)
    assert rc == 8 and "o overlaps v" in msg
    a = base_args(b, S_T=FAKE + (1 << 31), S0=FAKE + (1 << 31) + 4096)   # partial overlap
    assert call_chunk(b, a)[0] == 8


def test_chunk_varlen_rules(b):
    a = base_args(b, cu_seqlens=FAKE + (1 << 32), N=0)
    assert call_chunk(b, a)[0] == 2
    a = base_args(b, cu_seqlens=FAKE + (1 << 32), N=3, B=2)
    assert call_chunk(b, a)[0] == 2


def test_chunk_checkpoint_rules(b):
    """ckpt_every must be a multiple of the chunk length; a buffer is then required and
    must not overlap anything else; ckpt_every = 0 ignores the other two fields."""
    flags = b.KDA_FLAG_GENERIC   # no workspace needed, so validation reaches the ckpt rules
    ck = FAKE + (1 << 33)
    assert call_chunk(b, base_args(b, flags=flags, ckpt=ck, ckpt_every=96, ckpt_slots=4))[0] == 2
    assert call_chunk(b, base_args(b, flags=flags, ckpt=ck, ckpt_every=-64, ckpt_slots=4))[0] == 2
    assert call_chunk(b, base_args(b, flags=flags, ckpt=ck, ckpt_every=128, ckpt_slots=-1))[0] == 2
    assert call_chunk(b, base_args(b, flags=flags, ckpt=None, ckpt_every=128, ckpt_slots=4))[0] == 1
    a = base_args(b, flags=flags, ckpt_every=128, ckpt_slots=2)
    a.ckpt = a.k   # on top of an input
    rc, msg = call_chunk(b, a)
    assert rc == 8 and "ckpt overlaps k" in msg
    a = base_args(b, flags=flags, ckpt_every=128, ckpt_slots=2)
    a.ckpt = a.o + 64
    assert call_chunk(b, a)[0] == 8


def test_workspace_query(b):
    q = lambda a: b.lib().kda_chunk_fwd_workspace_bytes(ctypes.byref(a))  # noqa: E731
    fast = q(base_args(b))
    # 4 heads compose two chunks per step: one 163,840-byte block per 128 tokens and head;
    # 114,688 bytes per 64-token chunk and head when the walk takes one chunk per step
    assert fast >= 2 * 4 * 163840
    assert q(base_args(b, flags=b.KDA_FLAG_WALK64)) >= 4 * 4 * 114688
    assert q(base_args(b, flags=b.KDA_FLAG_GENERIC)) == 0
    assert q(base_args(b, act_dtype=b.KDA_F32, gate_dtype=b.KDA_F32)) == 0
    assert q(base_args(b, dk=96)) == b.SIZE_MAX and b.lib().kda_last_error()
    assert b.lib().kda_chunk_fwd_workspace_bytes(None) == b.SIZE_MAX
    # the matrix-core path needs scratch and refuses to run without it
    assert call_chunk(b, base_args(b))[0] == 6


def test_noalloc_refuses_sizes_beyond_its_scratch(b):
    """kda_chunk_fwd_noalloc checks its sizes against the fixed scratch before touching a
    device: 820 (128-token block, head) pairs of 163,840 B exceed KDA_NOALLOC_SCRATCH_BYTES."""
    assert b.NOALLOC_SCRATCH_BYTES == 128 << 20
    a = base_args(b, T=128 * 820, H=1)
    tok = 128 * 820
    a.k, a.v, a.g, a.beta = (FAKE + i * tok * 128 * 2 for i in range(1, 5))
    a.o = FAKE + (1 << 34)
    rc = b.lib().kda_chunk_fwd_noalloc(ctypes.byref(a), None)
    assert rc == 6 and "scratch" in b.lib().kda_last_error().decode()
    assert b.lib().kda_chunk_fwd_workspace_bytes(ctypes.byref(a)) > b.NOALLOC_SCRATCH_BYTES


def test_decode_rejects_bad_args(b):
    a = b.DecodeArgs()
    a.N, a.H, a.dk, a.dv = 4, 2, 128, 128
    a.act_dtype = a.gate_dtype = b.KDA_BF16
    a.out_dtype = b.KDA_F32
    a.q, a.k, a.v, a.g, a.beta = (FAKE + i * (1 << 20) for i in range(5))
    a.S = FAKE + (1 << 30)
    a.o = None
    assert b.lib().kda_decode_step(ctypes.byref(a), None) == 1
    a.o = a.S + 16   # inside the state
    assert b.lib().kda_decode_step(ctypes.byref(a), None) == 8
    a.o = FAKE + (1 << 31)
    a.dk = 100
    assert b.lib().kda_decode_step(ctypes.byref(a), None) == 2
    a.dk = 128
    a.gate_dtype = b.KDA_F32
    assert b.lib().kda_decode_step(ctypes.byref(a), None) == 3
    assert b.lib().kda_decode_step(None, None) == 1


def test_sizes_beyond_one_launch_are_refused(b):
    """A launch grid holds at most 2^32 - 1 work-items: larger problems are refused on the host
    with KDA_ERR_BAD_SHAPE instead of reaching the runtime with a truncated grid."""
    a = b.DecodeArgs()
    a.N, a.H, a.dk, a.dv = 1 << 20, 32, 128, 128   # 2^25 pairs of 256 work-items
    a.act_dtype = a.gate_dtype = b.KDA_BF16
    a.out_dtype = b.KDA_F32
    a.q, a.k, a.v, a.g, a.beta = (FAKE + i * (1 << 36) for i in range(5))
    a.S, a.o = FAKE + (6 << 36), FAKE + (7 << 36)
    assert b.lib().kda_decode_step(ctypes.byref(a), None) == 2
    assert "launch" in b.lib().kda_last_error().decode()
    # prefill: 2^24 chunks of one head need 2^32 work-items in the per-chunk kernel
    c = base_args(b, B=1 << 12, T=1 << 18, H=1, flags=b.KDA_FLAG_GENERIC)
    assert b.lib().kda_chunk_fwd_workspace_bytes(ctypes.byref(c)) == b.SIZE_MAX
    assert "launch" in b.lib().kda_last_error().decode()


def test_decode_multi_rejects_bad_args(b):
    a = b.DecodeMultiArgs()
    a.N, a.H, a.dk, a.dv, a.m = 4, 2, 128, 128, 3
    a.act_dtype = a.gate_dtype = b.KDA_BF16
    a.out_dtype = b.KDA_F32
    a.q, a.k, a.v, a.g, a.beta = (FAKE + i * (1 << 20) for i in range(5))
    a.S = FAKE + (1 << 30)
    a.o = FAKE + (1 << 31)
    call = lambda: b.lib().kda_decode_multi(ctypes.byref(a), None)  # noqa: E731
    a.m = 0
    assert call() == 2
    a.m = 3
    a.S = None
    assert call() == 1
    a.S = FAKE + (1 << 30)
    a.o = a.S + 64   # inside the state
    assert call() == 8
    a.o = FAKE + (1 << 31)
    a.accept = a.S   # the accepted counts on top of the state
    assert call() == 8
    a.accept = None
    a.o = None       # nothing asked for: a no-op, accepted without touching the device
    assert call() == 0
    assert b.lib().kda_decode_multi(None, None) == 1


def test_check_gates_rejects_bad_args(b):
    n = ctypes.c_int64(0)
    cnt = FAKE + (1 << 34)
    call = b.lib().kda_check_gates
    assert call(None, 10, None, 0, 1, cnt, 1024, None, ctypes.byref(n)) == 1
    assert call(None, -1, None, 0, 1, cnt, 1024, None, ctypes.byref(n)) == 2
    assert call(None, 0, None, 0, 1, cnt, 1024, None, None) == 1
    assert call(FAKE, 10, None, 0, 1, None, 1024, None, ctypes.byref(n)) == 1   # no counters
    assert call(FAKE, 10, None, 0, 1, cnt, 0, None, ctypes.byref(n)) == 2       # no room
    assert call(FAKE, 10, None, 0, 1, FAKE + 8, 1024, None, ctypes.byref(n)) == 8  # on g


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from gated_delta_rule_59_amd import binding
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.lib()
