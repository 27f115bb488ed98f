"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, rejects invalid arguments before touching the GPU, and sizes
states as the pages' memory accounting says ("How Kimi K3 Engineered Its Way to
the Frontier", section "What the hybrid saves")."""
import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import gated_delta_rule_10_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "page_constants.json")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        pytest.fail("libkda.so is not built (run __graft_entry__.build())")
    return kda.library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"kda_chunk_fwd", "kda_recurrent_step", "kda_state_io"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kda_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in names:
        getattr(lib, n)  # resolvable through ctypes


def test_status_strings_and_version(lib):
    for code, name in [(0, b"KDA_SUCCESS"), (1, b"KDA_ERROR_INVALID_VALUE"),
                       (2, b"KDA_ERROR_UNSUPPORTED"), (3, b"KDA_ERROR_WORKSPACE"),
                       (4, b"KDA_ERROR_LAUNCH")]:
        assert lib.kda_status_string(code) == name
    assert b"gfx950" in lib.kda_version()


def test_state_bytes_match_page_accounting(lib):
    c = json.load(open(GOLDEN))["state_memory"]
    bf16_layer = lib.kda_state_bytes(c["heads"], c["head_dim"], kda.KDA_BF16)
    assert bf16_layer == c["bf16_state_bytes_per_layer"]  # 3 MiB
    per_request = c["kda_layers"] * (bf16_layer + c["conv_cache_bytes_per_layer"]) / 2**20
    assert abs(per_request - c["per_request_mib_printed"]) < 0.005
    assert lib.kda_state_bytes(c["heads"], c["head_dim"], kda.KDA_F32) == 2 * bf16_layer
    assert lib.kda_state_bytes(0, 128, kda.KDA_F32) == 0


def _args(**kw):
    a = kda.ChunkFwdArgs()
    a.num_seqs, a.seq_len, a.num_heads, a.head_dim, a.chunk_size = 1, 64, 2, 128, 64
    a.io_dtype, a.scale = kda.KDA_BF16, 1.0
    fake = 1 << 20  # 16-byte aligned non-null placeholder; never dereferenced on error
    a.q = a.k = a.v = a.g = a.beta = fake
    a.o = fake + 4096
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, 2),
    ("chunk_size", 16, 2),
    ("num_seqs", 0, 1),
    ("num_heads", 0, 1),
    ("seq_len", -1, 1),
    ("io_dtype", 7, 1),
    ("segments", -2, 1),
    ("q", 0, 1),
    ("g", (1 << 20) + 4, 1),  # misaligned
    ("beta", (1 << 20) + 2, 1),  # beta needs 4 bytes
    ("o", 1 << 20, 1),        # aliases q
    ("scale", float("nan"), 1),
])
def test_chunk_fwd_rejects_invalid_arguments(lib, field, value, status):
    a = _args(**{field: value})
    assert lib.kda_chunk_fwd(ctypes.byref(a), None) == status
    size = ctypes.c_size_t(0)
    pointer_field = field in ("q", "g", "beta", "o")  # the size query reads no pointer
    assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(size)) == (
        0 if pointer_field else status)


def test_no_alloc_prefill_validates_on_the_host(lib):
    """The allocation-free prefill checks its arguments as kda_chunk_fwd does and
    refuses, before any GPU work, a plan whose workspace exceeds its buffer."""
    assert lib.kda_chunk_fwd_no_alloc_max_workspace() == 64 << 20
    for field, value, status in (("head_dim", 64, 2), ("num_heads", 0, 1), ("q", 0, 1),
                                 ("g", (1 << 20) + 4, 1)):
        a = _args(**{field: value})
        assert lib.kda_chunk_fwd_no_alloc(ctypes.byref(a), None) == status
    # 96 heads x 64 explicit segments: 3 x 64 states per chain, far beyond 64 MiB
    a = _args(seq_len=8192, num_heads=96, segments=64)
    size = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(size)) == 0
    assert size.value > lib.kda_chunk_fwd_no_alloc_max_workspace()
    assert lib.kda_chunk_fwd_no_alloc(ctypes.byref(a), None) == 3


def test_chunk_fwd_rejects_bad_cu_seqlens(lib):
    for host in ([1, 5, 9], [0, 9, 5]):
        arr = (ctypes.c_int32 * 3)(*host)
        a = _args(num_seqs=2, cu_seqlens=1 << 20)
        a.cu_seqlens_host = arr
        assert lib.kda_chunk_fwd(ctypes.byref(a), None) == 1
    a = _args(num_seqs=2, cu_seqlens=1 << 20)  # device offsets without a host copy
    assert lib.kda_chunk_fwd(ctypes.byref(a), None) == 1


def test_workspace_size_and_shortfall(lib):
    lens = [0, 100, 7, 4096]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    arr = (ctypes.c_int32 * len(cu))(*cu)
    a = _args(num_seqs=len(lens), cu_seqlens=1 << 20)
    a.cu_seqlens_host = arr
    size = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(size)) == 0
    assert size.value >= 4 * len(lens)  # the longest-first sequence order
    a.workspace, a.workspace_bytes = 1 << 20, 0
    assert lib.kda_chunk_fwd(ctypes.byref(a), None) == 3


def test_recurrent_step_rejects_invalid_arguments(lib):
    def args(**kw):
        a = kda.RecurrentStepArgs()
        a.batch, a.num_heads, a.head_dim, a.io_dtype, a.scale = 4, 2, 128, kda.KDA_BF16, 1.0
        fake = 1 << 20
        a.q = a.k = a.v = a.g = a.beta = a.state = a.o = fake
        a.num_slots = 4
        for k_, v_ in kw.items():
            setattr(a, k_, v_)
        return a
    assert lib.kda_recurrent_step(ctypes.byref(args(head_dim=96)), None) == 2
    assert lib.kda_recurrent_step(ctypes.byref(args(batch=-1)), None) == 1
    assert lib.kda_recurrent_step(ctypes.byref(args(num_slots=3)), None) == 1  # identity needs B<=slots
    assert lib.kda_recurrent_step(ctypes.byref(args(state=0)), None) == 1
    assert lib.kda_recurrent_step(ctypes.byref(args(state_indices=(1 << 20) + 2)), None) == 1
    assert lib.kda_recurrent_step(ctypes.byref(args(batch=0, q=0)), None) == 0  # nothing to do
    assert lib.kda_recurrent_step(ctypes.byref(args(state=(1 << 20) + 8)), None) == 1
    assert lib.kda_recurrent_step(ctypes.byref(args(q=(1 << 20) + 1)), None) == 1


def test_state_io_rejects_invalid_arguments(lib):
    f = lib.kda_state_io
    base = 1 << 24
    # op out of range, gather without indices, overlapping ranges, unsupported dim
    assert f(9, base, 0, 2, base * 2, 0, 2, None, 1, 4, 128, None) == 1
    assert f(kda.STATE_GATHER, base, 0, 2, base * 2, 0, 2, None, 1, 4, 128, None) == 1
    assert f(kda.STATE_COPY, base, 0, 2, base + 4096, 0, 2, None, 1, 4, 128, None) == 1
    assert f(kda.STATE_COPY, base, 0, 2, base * 4, 0, 2, None, 1, 4, 64, None) == 2
    assert f(kda.STATE_COPY, base, 0, 1, base * 4, 0, 2, None, 2, 4, 128, None) == 1  # count > src
    assert f(kda.STATE_ZERO, None, 0, 0, base, 0, 2, None, 0, 4, 128, None) == 0  # empty
    # one workgroup per head: count x heads must fit the grid
    assert f(kda.STATE_ZERO, None, 0, 0, base, 0, 1 << 30, None, 1 << 20, 4096, 128, None) == 1


def _gate_args(**gate):
    a = _args()
    a.gate.mode = kda.GATE_LOWER_BOUND
    a.gate.A_log = 1 << 21
    a.gate.lower_bound = -5.0
    for k_, v_ in gate.items():
        setattr(a.gate, k_, v_)
    return a


@pytest.mark.parametrize("field,value,pointer_only", [
    ("mode", 5, False),
    ("A_log", 0, True),
    ("A_log", (1 << 21) + 2, True),    # needs 4 bytes
    ("dt_bias", (1 << 21) + 1, True),
    ("lower_bound", -5.5, False),      # below the floor the exponent bounds assume
    ("lower_bound", 0.25, False),
    ("lower_bound", float("nan"), False),
    ("beta_logits", 2, False),
])
def test_gate_front_end_rejects_invalid_arguments(lib, field, value, pointer_only):
    """The lower-bounded gate's arguments are checked on the host, by both the
    prefill (the size query skips pointers) and the decode step."""
    a = _gate_args(**{field: value})
    assert lib.kda_chunk_fwd(ctypes.byref(a), None) == 1
    size = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(size)) == (
        0 if pointer_only else 1)
    d = kda.RecurrentStepArgs()
    d.batch, d.num_heads, d.head_dim, d.io_dtype, d.scale = 4, 2, 128, kda.KDA_BF16, 1.0
    d.q = d.k = d.v = d.g = d.beta = d.state = d.o = 1 << 20
    d.num_slots = 4
    d.gate = a.gate
    assert lib.kda_recurrent_step(ctypes.byref(d), None) == 1


def test_gate_bounds_accepted_by_the_size_query(lib):
    """lower_bound -5 (the pages' value) and 0 are inside the accepted range."""
    for lb in (-5.0, -1.0, 0.0):
        a = _gate_args(lower_bound=lb, beta_logits=1)
        size = ctypes.c_size_t(0)
        assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(size)) == 0


def test_ctypes_structs_match_the_header(tmp_path):
    """The binding's structure mirrors have the header's field offsets and sizes
    (a C program built against include/kda.h prints them)."""
    import shutil
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    structs = {"kda_chunk_fwd_args": kda.ChunkFwdArgs,
               "kda_recurrent_step_args": kda.RecurrentStepArgs, "kda_gate": kda.Gate,
               "kda_fused_step_args": kda.FusedStepArgs,
               "kda_spec_verify_args": kda.SpecVerifyArgs, "kda_chunk_bwd_args": kda.ChunkBwdArgs}
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "kda.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True,
                               check=True).stdout.splitlines():
        s, f, n = line.split()
        got[(s, f)] = int(n)
    for cname, py in structs.items():
        assert got[(cname, "sizeof")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def test_conv_cache_bytes_match_page_accounting(lib):
    """[P1] "What the hybrid saves": the three ShortConv caches of a 96-head layer
    are 216 KiB in bf16."""
    c = json.load(open(GOLDEN))["state_memory"]
    assert lib.kda_conv_cache_bytes(c["heads"], c["head_dim"], kda.KDA_BF16) == \
        c["conv_cache_bytes_per_layer"]
    assert lib.kda_conv_cache_bytes(c["heads"], c["head_dim"], kda.KDA_F32) == \
        2 * c["conv_cache_bytes_per_layer"]
    assert lib.kda_conv_cache_bytes(0, 128, kda.KDA_BF16) == 0


def test_fused_decode_step_rejects_invalid_arguments(lib):
    def args(**kw):
        a = kda.FusedStepArgs()
        a.batch, a.num_heads, a.head_dim, a.io_dtype, a.scale = 4, 2, 128, kda.KDA_BF16, 1.0
        fake = 1 << 20
        a.q = a.k = a.v = a.g = a.beta = a.state = a.o = a.conv_cache = a.conv_weight = fake
        a.num_slots, a.l2_eps, a.norm_eps, a.out_norm = 4, 1e-6, 1e-6, 1
        for k_, v_ in kw.items():
            setattr(a, k_, v_)
        return a
    f = lambda a: lib.kda_fused_decode_step(ctypes.byref(a), None)
    assert f(args(head_dim=64)) == 2
    assert f(args(batch=-1)) == 1
    assert f(args(num_slots=3)) == 1
    assert f(args(conv_cache=0)) == 1
    assert f(args(conv_weight=(1 << 20) + 4)) == 1  # needs 16 bytes
    assert f(args(conv_cache=(1 << 20) + 1)) == 1
    assert f(args(l2_eps=-1.0)) == 1
    assert f(args(norm_eps=float("inf"))) == 1
    assert f(args(out_norm=2)) == 1
    assert f(args(norm_weight=(1 << 20) + 2)) == 1
    assert f(args(batch=0, q=0, conv_cache=0)) == 0  # nothing to do
    a = args()
    a.gate.mode = 1  # lower-bounded gate without A_log
    assert f(a) == 1


def test_spec_verify_rejects_invalid_arguments(lib):
    def args(**kw):
        va = kda.SpecVerifyArgs()
        a = va.step
        a.batch, a.num_heads, a.head_dim, a.io_dtype, a.scale = 4, 2, 128, kda.KDA_BF16, 1.0
        fake = 1 << 20
        a.q = a.k = a.v = a.g = a.beta = a.state = a.o = a.conv_cache = a.conv_weight = fake
        a.num_slots, a.l2_eps, a.norm_eps, a.out_norm = 4, 1e-6, 1e-6, 1
        va.window, va.replay_window = 3, 3
        va.replay_q = va.replay_k = va.replay_v = va.replay_g = va.replay_beta = fake
        for k_, v_ in kw.items():
            setattr(va, k_, v_)
        return va
    f = lambda va: lib.kda_spec_verify_step(ctypes.byref(va), None)
    assert f(args(window=-1)) == 1
    assert f(args(replay_window=-2)) == 1
    assert f(args(replay_g=0)) == 1
    assert f(args(replay_q=(1 << 20) + 1)) == 1
    assert f(args(num_replay=(1 << 20) + 2)) == 1
    va = args()
    va.step.head_dim = 96
    assert f(va) == 2
    va = args(window=0)  # replay only: the new-window pointers are not read
    va.step.q = 0
    va.step.batch = 0
    assert f(va) == 0


def test_chunk_bwd_rejects_invalid_arguments(lib):
    def args(**kw):
        a = kda.ChunkBwdArgs()
        a.num_seqs, a.seq_len, a.num_heads, a.head_dim = 1, 64, 2, 128
        a.io_dtype, a.scale = kda.KDA_BF16, 1.0
        base = 1 << 20
        a.q, a.k, a.v, a.dO, a.g, a.beta = (base + 4096 * i for i in range(6))
        a.dq, a.dk, a.dv, a.dg, a.dbeta = (base + 4096 * (8 + i) for i in range(5))
        for k_, v_ in kw.items():
            setattr(a, k_, v_)
        return a
    size = ctypes.c_size_t(0)
    assert lib.kda_chunk_bwd_workspace_size(ctypes.byref(args()), ctypes.byref(size)) == 0
    # T / 16 + N + 1 slots of H states and partial records
    assert size.value >= (64 // 16 + 1 + 1) * 2 * 128 * 128 * 4
    f = lambda a: lib.kda_chunk_bwd(ctypes.byref(a), None)
    assert f(args(head_dim=64)) == 2
    assert f(args(num_heads=0)) == 1
    assert f(args(dq=0)) == 1
    assert f(args(dk=(1 << 20) + 4)) == 1          # gradients need 16 bytes
    assert f(args(dv=1 << 20)) == 1                 # output aliases q
    assert f(args()) == 3                           # no workspace


def test_chunk_bwd_minimum_workspace_is_the_largest_sequence(lib):
    """The backward runs in any workspace from the largest single sequence's
    requirement up (groups of sequences in turn); below it KDA_ERROR_WORKSPACE
    comes back before anything is launched."""
    lens = [100, 37, 5000, 0, 64]
    cu = (ctypes.c_int32 * (len(lens) + 1))(*[int(x) for x in np.concatenate([[0], np.cumsum(lens)])])
    a = kda.ChunkBwdArgs()
    a.num_seqs, a.num_heads, a.head_dim = len(lens), 3, 128
    a.cu_seqlens_host, a.cu_seqlens = cu, 16
    a.io_dtype, a.scale = kda.KDA_BF16, 1.0
    full, least = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.kda_chunk_bwd_workspace_size(ctypes.byref(a), ctypes.byref(full)) == 0
    assert lib.kda_chunk_bwd_min_workspace_size(ctypes.byref(a), ctypes.byref(least)) == 0
    assert 0 < least.value < full.value
    one = kda.ChunkBwdArgs()  # the 5000-token sequence alone
    one.num_seqs, one.seq_len, one.num_heads, one.head_dim = 1, 5000, 3, 128
    one.io_dtype, one.scale = kda.KDA_BF16, 1.0
    alone = ctypes.c_size_t(0)
    assert lib.kda_chunk_bwd_workspace_size(ctypes.byref(one), ctypes.byref(alone)) == 0
    assert least.value == alone.value
    base = 1 << 20
    a.q, a.k, a.v, a.dO, a.g, a.beta = (base + 4096 * i for i in range(6))
    a.dq, a.dk, a.dv, a.dg, a.dbeta = (base + 4096 * (8 + i) for i in range(5))
    a.workspace, a.workspace_bytes = 1 << 30, least.value - 1
    assert lib.kda_chunk_bwd(ctypes.byref(a), None) == 3
