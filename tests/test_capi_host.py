"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/spec_verify.h declares, and rejects bad arguments
with the documented status before enqueueing anything."""
import ctypes
import os
import re
import subprocess

import pytest

import speculative_decoding_verify_attn_amd as sv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "spec_verify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_lists_the_calls():
    names = declared_functions()
    for must in ("spec_verify_attn", "spec_verify_sample", "spec_verify_sample_ex", "spec_verify_attn_workspace_size",
                 "spec_verify_sample_workspace_size", "sv_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = sv.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", sv.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_abi_version_and_status_strings():
    L = sv.lib()
    assert L.sv_abi_version() == 1
    assert L.sv_status_string(0) == b"ok"
    assert L.sv_status_string(6) == b"HIP error"


def _attn(**kw):
    L = sv.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 255) & ~255
    a = dict(q=base, k=base, v=base, ks=None, vs=None, table=base, lens=base, out=base,
             B=2, T=5, Hq=32, Hkv=8, d=128, bs=16, maxb=8, nb=16, kv=1, scale=0.088,
             ws=base, wsb=1 << 14, stream=None, algo=0, bps=0, ev=None)
    a.update(kw)
    return L.spec_verify_attn_ex(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["table"], a["lens"], a["out"],
                                 a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["bs"], a["maxb"], a["nb"],
                                 a["kv"], a["scale"], a["ws"], a["wsb"], a["stream"], a["algo"], a["bps"], a["ev"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(B=0), 2),
    (dict(T=17), 2),
    (dict(Hq=30), 2),
    (dict(Hq=256, Hkv=8), 3),     # T*G = 160 > 128
    (dict(d=96), 3),
    (dict(bs=32), 3),
    (dict(kv=7), 3),
    (dict(kv=2), 1),              # E4M3 without scales
    (dict(ks=1 << 20), 2),        # scales given for bf16
    (dict(scale=0.0), 2),
    (dict(algo=2, kv=0), 3),      # matrix cores need bf16/E4M3
    (dict(bps=10), 2),
    (dict(bps=516), 2),
    (dict(bps=-2), 2),
    (dict(bps=-1, kv=0), 3),      # balanced shares need the matrix-core kernel
    (dict(bps=-1, algo=1), 3),
    (dict(bps=-1, B=1025), 3),    # balanced shares: at most 1024 sequences
    (dict(ws=None), 4),
    (dict(wsb=16), 4),
    (dict(q=1 << 20 | 4), 5),     # misaligned
])
def test_attention_argument_checks(kw, status):
    assert _attn(**kw) == status
    assert len(sv.lib().sv_last_error()) > 0


def test_sample_argument_checks():
    L = sv.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = (ctypes.addressof(buf) + 255) & ~255
    assert L.spec_verify_sample(None, p, p, p, p, p, None, 2, 3, 100, p, 1 << 14, None) == 1
    assert L.spec_verify_sample(p, p, p, p, p, p, None, 2, 16, 100, p, 1 << 14, None) == 2
    assert L.spec_verify_sample(p, p, p, p, p, p, None, 0, 3, 100, p, 1 << 14, None) == 2
    assert L.spec_verify_sample(p, p, p, p, p, p, None, 2, 3, 100, p, 8, None) == 4
    assert L.spec_verify_sample(p, p, p, p, p, p, None, 2, 3, 100, None, 1 << 14, None) == 4
    assert L.spec_verify_sample(p + 2, p, p, p, p, p, None, 2, 3, 100, p, 1 << 14, None) == 5
    # the temperature variant: same checks, plus the temperature array's alignment
    ex = L.spec_verify_sample_ex
    assert ex(None, p, p, p, p, None, p, p, None, 2, 3, 100, p, 1 << 14, None) == 1
    assert ex(p, p, p, p, None, None, p, p, None, 2, 16, 100, p, 1 << 14, None) == 2
    assert ex(p, p, p, p, p + 1, None, p, p, None, 2, 3, 100, p, 1 << 14, None) == 5
    assert ex(p, p, p, p, None, p + 2, p, p, None, 2, 3, 100, p, 1 << 14, None) == 5
    assert ex(p, p, p, p, None, p, p, p, None, 2, 3, 1 << 20, p, 1 << 30, None) == 3


def test_typical_argument_checks():
    L = sv.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = (ctypes.addressof(buf) + 255) & ~255
    ty = L.spec_verify_sample_typical
    assert ty(None, p, p, None, 0.1, 0.3, p, p, None, None, 2, 3, 100, p, 1 << 14, None) == 1
    assert ty(p, p, p, None, -0.1, 0.3, p, p, None, None, 2, 3, 100, p, 1 << 14, None) == 2
    assert ty(p, p, p, None, 0.1, float("nan"), p, p, None, None, 2, 3, 100, p, 1 << 14, None) == 2
    assert ty(p, p, p, None, 0.1, 0.3, p, p, None, None, 2, 16, 100, p, 1 << 14, None) == 2
    assert ty(p, p, p, None, 0.1, 0.3, p, p, None, p + 1, 2, 3, 100, p, 1 << 14, None) == 5
    assert ty(p, p, p, None, 0.1, 0.3, p, p, None, None, 2, 3, 100, p, 8, None) == 4


def test_tree_argument_checks():
    L = sv.lib()
    buf = ctypes.create_string_buffer(1 << 20)
    p = (ctypes.addressof(buf) + 255) & ~255
    st = L.spec_verify_sample_tree
    assert st(None, p, p, p, p, p, p, p, None, 2, 4, 100, 2, p, 1 << 18, None) == 1
    assert st(p, p, p, p, p, p, p, p, None, 2, 17, 100, 2, p, 1 << 18, None) == 2     # N > 16
    assert st(p, p, p, p, p, p, p, p, None, 0, 4, 100, 2, p, 1 << 18, None) == 2
    assert st(p, p, p, p, p, p, p, p, None, 2, 4, 100, 4, p, 1 << 18, None) == 2      # max_children > N-1
    assert st(p, p, p + 2, p, p, p, p, p, None, 2, 4, 100, 2, p, 1 << 18, None) == 5
    assert st(p, p, p, p, p, p, p, p, None, 2, 4, 100, 2, p, 8, None) == 4
    assert L.spec_verify_sample_tree_workspace_size(2, 17, 100) == 0
    assert L.spec_verify_sample_tree_workspace_size(2, 16, 100) > 0
    at = L.spec_verify_attn_tree
    # tree_mask NULL is rejected; shape checks as the chain's
    args = [p, p, p, None, None, p, p, None, p, 2, 4, 8, 2, 64, 16, 4, 8, 1, ctypes.c_float(0.125), p, 1 << 18,
            None, 0, 0]
    assert at(*args) == 1
    args[7] = p
    args[10] = 17   # T > 16
    assert at(*args) == 2


def test_tree_commit_argument_checks():
    L = sv.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = (ctypes.addressof(buf) + 255) & ~255
    tc = L.spec_verify_tree_commit
    args = [p, p, p, p, None, None, p, p, None, 2, 6, 2, 64, 16, 4, 8, 1, None]
    a = list(args); a[0] = None
    assert tc(*a) == 1
    a = list(args); a[10] = 17           # N > 16
    assert tc(*a) == 2
    a = list(args); a[12] = 260          # d > 256
    assert tc(*a) == 2
    a = list(args); a[13] = 32           # block size
    assert tc(*a) == 3
    a = list(args); a[16] = 2            # E4M3 without scales
    assert tc(*a) == 1
    a = list(args); a[2] = p + 4         # bf16 cache needs 8-byte alignment
    assert tc(*a) == 5


def test_workspace_queries():
    assert sv.attn_workspace_size(8, 6, 32, 8, 128, 256) > 0
    # balanced shares (blocks_per_split = -1): prefix sums plus one partial
    # slot per unit and per workgroup (at least 256 workgroups)
    L = sv.lib()
    bal = L.spec_verify_attn_workspace_size_ex(8, 6, 32, 8, 128, 256, -1)
    assert bal >= (8 * 8 + 256) * 24 * 128 * 4
    assert L.spec_verify_attn_workspace_size_ex(1025, 6, 32, 8, 128, 256, -1) == 0
    assert L.spec_verify_attn_workspace_size_ex(1024, 6, 32, 8, 128, 256, -1) > 0
    # the planner's choice for large batches is covered by the default size
    big = (64, 8, 32, 8, 128, 1024)
    assert L.spec_verify_attn_workspace_size_ex(*big, 0) >= L.spec_verify_attn_workspace_size_ex(*big, -1)
    assert sv.lib().spec_verify_attn_workspace_size(8, 6, 30, 8, 128, 256) == 0
    assert sv.sample_workspace_size(8, 5, 128256) >= 8 * 6 * 16 * 16
    assert sv.lib().spec_verify_sample_workspace_size(8, 0, 10) == 0


def test_append_and_rollback_argument_checks():
    L = sv.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = (ctypes.addressof(buf) + 255) & ~255
    ok = dict(B=2, T=6, Hkv=8, d=128, bs=16, mb=8, nb=32, kv=1)

    def app(kn=p, vn=p, kc=p, vc=p, ks=None, vs=None, tb=p, cl=p, **over):
        a = dict(ok, **over)
        return L.spec_verify_kv_append(kn, vn, kc, vc, ks, vs, tb, cl, a["B"], a["T"], a["Hkv"], a["d"], a["bs"],
                                       a["mb"], a["nb"], a["kv"], None)

    assert app(kn=None) == 1
    assert app(T=17) == 2
    assert app(T=0) == 2
    assert app(d=130) == 2
    assert app(bs=32) == 3
    assert app(kv=7) == 3
    assert app(kv=2) == 1                       # E4M3 without scales
    assert app(ks=p, vs=p) == 2                 # scales given for bf16
    assert app(kn=p + 4) == 5
    assert app(kc=p + 2) == 5                   # bf16 cache must be 8-byte aligned
    assert L.spec_verify_rollback(None, p, None, 2, 5, None) == 1
    assert L.spec_verify_rollback(p, p, None, 2, 16, None) == 2
    assert L.spec_verify_rollback(p, p, None, 0, 5, None) == 2
    assert L.spec_verify_rollback(p, p + 2, None, 2, 5, None) == 5


def test_check_inputs_argument_checks():
    L = sv.lib()
    buf = ctypes.create_string_buffer(1 << 12)
    base = (ctypes.addressof(buf) + 255) & ~255

    def call(**kw):
        a = dict(table=base, lens=base, T=6, maxb=8, nb=16, tok=base, ntok=5, V=100, u=base, nu=6, B=2, counts=base)
        a.update(kw)
        return L.spec_verify_check_inputs(a["table"], a["lens"], a["T"], a["maxb"], a["nb"], a["tok"], a["ntok"],
                                          a["V"], a["u"], a["nu"], a["B"], a["counts"], None)

    assert call(counts=None) == 1
    assert call(B=0) == 2
    assert call(lens=None) == 1           # the table's visible pages come from the lengths
    assert call(T=0) == 2
    assert call(nb=0) == 2
    assert call(V=0) == 2
    assert call(nu=-1) == 2
    assert call(counts=base + 2) == 5
    assert len(L.sv_last_error()) > 0
