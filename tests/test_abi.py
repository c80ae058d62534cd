"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/kda.h declares, and rejects bad arguments before enqueuing any work
(every call here returns from validation, so no HIP call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    from gated_delta_rule_06_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    from gated_delta_rule_06_amd import kda
    return kda.lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("kda_chunk_fwd", "kda_chunk_fwd_varlen", "kda_decode_step",
                 "kda_recurrent_fwd", "kda_recurrent_fwd_varlen", "kda_gdn_chunk_fwd",
                 "kda_gdn_chunk_fwd_varlen", "kda_gdn_decode_step", "kda_gdn_recurrent_fwd",
                 "kda_gdn_recurrent_fwd_varlen", "kda_chunk_fwd_fused", "kda_recurrent_fwd_fused",
                 "kda_decode_step_fused", "kda_backward", "kda_backward_workspace_size",
                 "kda_backward_noalloc", "kda_noalloc_scratch_bytes",
                 "kda_chunk_fwd_workspace_size", "kda_chunk_fwd_varlen_workspace_size",
                 "kda_status_string", "kda_version"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), "libkda.so does not export %s" % name


def test_status_strings_and_version(lib):
    from gated_delta_rule_06_amd import kda
    assert kda.status_string(0) == "KDA_OK"
    for code in range(-1, -9, -1):
        assert kda.status_string(code).startswith("KDA_ERR_")
    assert "unknown" in kda.status_string(-99)
    assert lib.kda_version() >= 100


def test_workspace_sizes(lib):
    # the balanced schedule's plan (chunk prefix sums, flags) and one fp32
    # hand-over state per slot, min(N * H, 1024) slots
    split = lambda N, H, d: (4352 + (N + 1) * 8 + 255) // 256 * 256 + min(N * H, 1024) * d * d * 4
    assert lib.kda_chunk_fwd_workspace_size(8, 8192, 32, 128, 128, 64, 1) == split(8, 32, 128)
    assert lib.kda_chunk_fwd_varlen_workspace_size(16, 537014, 32, 128, 128, 64, 1) == \
        4608 + 512 * 128 * 128 * 4
    assert lib.kda_chunk_fwd_varlen_workspace_size(300, 9000, 8, 64, 64, 64, 0) == \
        (4352 + 301 * 8 + 255) // 256 * 256 + 1024 * 64 * 64 * 4
    # few long bf16 128x128 chains: the chunk-parallel schedule's factors
    # (74,240 bytes per (chain, chunk) plus a flag each)
    assert lib.kda_chunk_fwd_workspace_size(1, 4096, 16, 128, 128, 64, 1) == 16 * 64 * 74240 + 4096
    assert lib.kda_chunk_fwd_workspace_size(1, 4096, 16, 64, 64, 64, 1) == split(1, 16, 64)
    assert lib.kda_chunk_fwd_workspace_size(1, 511, 16, 128, 128, 64, 1) == split(1, 16, 128)
    # few long packed sequences (bf16 128x128, at most 64 chains, at least 512 tokens
    # per sequence on average): the chunk table, then records for at most
    # H * (ceil(T_total / 64) + N) chunks and a flag each
    rec = 16 * (2048 + 2)
    assert lib.kda_chunk_fwd_varlen_workspace_size(2, 131072, 16, 128, 128, 64, 1) == \
        4608 + rec * 74240 + (rec * 4 + 255) // 256 * 256
    assert lib.kda_chunk_fwd_varlen_workspace_size(4, 1000, 16, 128, 128, 64, 1) == split(4, 16, 128)
    # unsupported sizes: none
    assert lib.kda_chunk_fwd_workspace_size(1, 4096, 16, 128, 128, 64, 0) == 0   # fp32 I/O, d 128
    assert lib.kda_chunk_fwd_workspace_size(4, 100, 2, 96, 128, 64, 1) == 0
    assert lib.kda_chunk_fwd_workspace_size(0, 100, 2, 128, 128, 64, 1) == 0
    assert lib.kda_chunk_fwd_varlen_workspace_size(4, 100, 2, 96, 128, 64, 1) == 0


def test_chunk_parallel_needs_its_workspace(lib):
    P_ = [ctypes.c_void_p(0x100000000 + 0x10000000 * i) for i in range(8)]   # never dereferenced
    need = lib.kda_chunk_fwd_workspace_size(1, 4096, 16, 128, 128, 64, 1)
    call = lambda ws, n: lib.kda_chunk_fwd(P_[0], P_[1], P_[2], P_[3], P_[4], None, P_[5], P_[6],
                                           1, 4096, 16, 128, 128, 0.1, 64, 1, ws, n, None)
    assert call(None, 0) == -4                                        # KDA_ERR_WORKSPACE
    assert call(ctypes.c_void_p(0x200000000), need - 1) == -4
    assert call(ctypes.c_void_p(0x200000000 + 16), need) == -7         # 256-byte alignment
    assert call(P_[5], need) == -6                                      # overlaps out


def test_varlen_workspace_validation(lib):
    """A packed call given a workspace checks its size, alignment and overlap
    before any launch."""
    P_ = [ctypes.c_void_p(0x100000000 + 0x10000000 * i) for i in range(8)]   # never dereferenced
    need = lib.kda_chunk_fwd_varlen_workspace_size(40, 4000, 8, 128, 128, 64, 1)
    call = lambda ws, n: lib.kda_chunk_fwd_varlen(P_[0], P_[1], P_[2], P_[3], P_[4], None, P_[5],
                                                  P_[6], P_[7], 40, 4000, 8, 128, 128, 0.1, 64, 1,
                                                  ws, n, None)
    assert call(ctypes.c_void_p(0x200000000), need - 1) == -4          # KDA_ERR_WORKSPACE
    assert call(ctypes.c_void_p(0x200000000 + 16), need) == -7         # 256-byte alignment
    assert call(P_[5], need) == -6                                      # overlaps out
    assert call(P_[7], need) == -6                                      # overlaps cu_seqlens


P = [ctypes.c_void_p(0x10000000 + 0x1000000 * i) for i in range(12)]   # never dereferenced


def chunk(lib, q=P[0], k=P[1], v=P[2], g=P[3], beta=P[4], S0=None, out=P[5], Sf=P[6], B=1, T=64,
          H=2, dk=128, dv=128, chunk=64, io=1):
    return lib.kda_chunk_fwd(q, k, v, g, beta, S0, out, Sf, B, T, H, dk, dv, 0.1, chunk, io, None,
                             0, None)


def test_chunk_fwd_validation(lib):
    from gated_delta_rule_06_amd import kda
    assert chunk(lib, q=None) == -1                       # KDA_ERR_NULL
    assert chunk(lib, beta=None) == -1
    assert chunk(lib, B=-1) == -2                         # KDA_ERR_DIM
    assert chunk(lib, T=-5) == -2
    assert chunk(lib, H=0) == -2
    assert chunk(lib, chunk=32) == -3                     # KDA_ERR_UNSUPPORTED
    assert chunk(lib, dk=96) == -3
    assert chunk(lib, dv=256) == -3
    assert chunk(lib, io=7) == -3
    assert chunk(lib, io=0) == -3                         # fp32 I/O only for d_k = d_v = 64
    assert chunk(lib, out=P[0]) == -6                     # KDA_ERR_ALIAS: out == q
    assert chunk(lib, Sf=P[5]) == -6                      # S_final == out
    assert chunk(lib, B=0) == 0                           # nothing to do, nothing enqueued
    assert kda.status_string(chunk(lib, q=None)).startswith("KDA_ERR_NULL")


def test_varlen_validation(lib):
    f = lib.kda_chunk_fwd_varlen
    args = lambda **kw: (kw.get("q", P[0]), P[1], P[2], P[3], P[4], None, kw.get("out", P[5]),
                         P[6], kw.get("cu", P[7]), kw.get("N", 3), kw.get("Tt", 100), 2,
                         kw.get("dk", 128), 128, 0.1, kw.get("chunk", 64), 1, None, 0, None)
    assert f(*args(cu=None)) == -1
    assert f(*args(N=-1)) == -2
    assert f(*args(Tt=-1)) == -2
    assert f(*args(dk=32)) == -3
    assert f(*args(chunk=16)) == -3
    assert f(*args(out=P[1])) == -6
    assert f(*args(N=0)) == 0


def test_decode_validation(lib):
    f = lib.kda_decode_step
    args = lambda **kw: (kw.get("q", P[0]), P[1], P[2], P[3], P[4], kw.get("S", P[5]),
                         kw.get("out", P[6]), kw.get("N", 4), 2, kw.get("dk", 128), 128, 0.1,
                         kw.get("io", 1), None)
    assert f(*args(q=None)) == -1
    assert f(*args(S=None)) == -1
    assert f(*args(N=-3)) == -2
    assert f(*args(dk=100)) == -3
    assert f(*args(io=3)) == -3
    assert f(*args(out=P[5])) == -6                       # out overlaps the state
    assert f(*args(N=0)) == 0


def test_recurrent_validation(lib):
    f = lib.kda_recurrent_fwd
    args = lambda **kw: (kw.get("q", P[0]), P[1], P[2], P[3], kw.get("beta", P[4]),
                         kw.get("S0", None), kw.get("out", P[5]), kw.get("Sf", P[6]),
                         kw.get("B", 2), kw.get("T", 4), kw.get("H", 2), kw.get("dk", 128),
                         kw.get("dv", 128), 0.1, kw.get("io", 1), None)
    assert f(*args(q=None)) == -1
    assert f(*args(B=-1)) == -2
    assert f(*args(T=-1)) == -2
    assert f(*args(H=0)) == -2
    assert f(*args(B=1 << 16, T=1 << 16)) == -2            # more tokens than 32-bit indices
    assert f(*args(dk=32)) == -3
    assert f(*args(dv=96)) == -3
    assert f(*args(io=2)) == -3
    assert f(*args(out=P[2])) == -6                         # out == v
    assert f(*args(Sf=P[3])) == -6                          # S_final == log_alpha
    assert f(*args(B=0)) == 0
    assert f(*args(T=0, Sf=None)) == 0                      # nothing to write
    assert f(*args(T=0, S0=P[6])) == 0                      # in place, no tokens: a no-op
    g = lib.kda_recurrent_fwd_varlen
    vargs = lambda **kw: (P[0], P[1], P[2], P[3], P[4], None, kw.get("out", P[5]), P[6],
                          kw.get("cu", P[7]), kw.get("N", 3), kw.get("Tt", 10), 2, 64,
                          kw.get("dv", 64), 0.1, 0, None)
    assert g(*vargs(cu=None)) == -1
    assert g(*vargs(N=-1)) == -2
    assert g(*vargs(Tt=-2)) == -2
    assert g(*vargs(dv=32)) == -3
    assert g(*vargs(out=P[0])) == -6
    assert g(*vargs(N=0)) == 0


def test_gdn_validation(lib):
    """The Gated DeltaNet calls share the KDA validation; their gate array has
    no d_k axis and needs only 4-byte alignment."""
    f = lib.kda_gdn_chunk_fwd
    args = lambda **kw: (P[0], P[1], P[2], kw.get("g", P[3]), P[4], None, kw.get("out", P[5]),
                         P[6], kw.get("B", 1), 64, 2, kw.get("dk", 128), 128, 0.1,
                         kw.get("chunk", 64), 1, None, 0, None)
    assert f(*args(g=None)) == -1
    assert f(*args(B=-1)) == -2
    assert f(*args(dk=32)) == -3
    assert f(*args(chunk=32)) == -3
    assert f(*args(out=P[3])) == -6                         # out == log_alpha
    assert f(*args(g=ctypes.c_void_p(P[3].value + 2))) == -7
    assert f(*args(B=0)) == 0
    d = lib.kda_gdn_decode_step
    assert d(P[0], P[1], P[2], None, P[4], P[5], P[6], 4, 2, 128, 128, 0.1, 1, None) == -1
    assert d(P[0], P[1], P[2], P[3], P[4], P[5], P[6], 4, 2, 96, 128, 0.1, 1, None) == -3
    assert d(P[0], P[1], P[2], P[3], P[4], P[5], P[3], 4, 2, 128, 128, 0.1, 1, None) == -6
    assert d(P[0], P[1], P[2], P[3], P[4], P[5], P[6], 0, 2, 128, 128, 0.1, 1, None) == 0
    r = lib.kda_gdn_recurrent_fwd
    assert r(P[0], P[1], P[2], P[3], P[4], None, P[5], P[6], 2, 4, 2, 64, 64, 0.1, 3, None) == -3
    rv = lib.kda_gdn_recurrent_fwd_varlen
    assert rv(P[0], P[1], P[2], P[3], P[4], None, P[5], P[6], None, 3, 10, 2, 64, 64, 0.1, 0,
              None) == -1
    cv = lib.kda_gdn_chunk_fwd_varlen
    assert cv(P[0], P[1], P[2], P[3], P[4], None, P[5], P[6], P[7], -1, 10, 2, 64, 64, 0.1, 64, 0,
              None, 0, None) == -2


def test_fused_validation(lib):
    """The fused calls validate the prologue before anything else happens."""
    from gated_delta_rule_06_amd.kda import _Prologue
    f = lib.kda_chunk_fwd_fused
    pro = lambda flags, a=P[8], b=P[9]: ctypes.byref(_Prologue(flags, a, b))
    args = lambda **kw: (P[0], P[1], P[2], P[3], P[4], None, kw.get("out", P[5]), P[6],
                         kw.get("cu", None), kw.get("N", 2), 64, 2, 128, 128, 0.1, 64, 1,
                         kw.get("ph", 0), kw.get("pro", None), None, 0, None)
    assert f(*args(pro=pro(8))) == -3                       # unknown flag bit
    assert f(*args(pro=pro(4, a=None))) == -1               # gate without A_log
    assert f(*args(pro=pro(4, a=ctypes.c_void_p(P[8].value + 2)))) == -7
    assert f(*args(pro=pro(4, b=P[5]))) == -6               # gate bias is the output
    assert f(*args(ph=2)) == -3
    assert f(*args(N=0, pro=pro(7))) == 0
    assert f(*args(N=-1)) == -2
    r = lib.kda_recurrent_fwd_fused
    assert r(P[0], P[1], P[2], P[3], P[4], None, P[5], P[6], None, 2, 4, 2, 64, 64, 0.1, 0, 0,
             pro(4, a=None), None) == -1
    d = lib.kda_decode_step_fused
    assert d(P[0], P[1], P[2], P[3], P[4], P[5], P[6], 4, 2, 128, 128, 0.1, 1, 0, pro(16),
             None) == -3
    assert d(P[0], P[1], P[2], P[3], P[4], P[5], P[6], 4, 2, 128, 128, 0.1, 1, 0,
             pro(4, b=P[6]), None) == -6                    # gate bias is the output


def test_alignment_validation(lib):
    odd = lambda p, n: ctypes.c_void_p(p.value + n)
    assert chunk(lib, q=odd(P[0], 2)) == -7                 # KDA_ERR_ALIGN
    assert chunk(lib, g=odd(P[3], 8)) == -7
    assert chunk(lib, Sf=odd(P[6], 4)) == -7
    assert chunk(lib, beta=odd(P[4], 2)) == -7              # beta needs 4 bytes
    f = lib.kda_decode_step
    assert f(odd(P[0], 2), P[1], P[2], P[3], P[4], P[5], P[6], 4, 2, 128, 128, 0.1, 1, None) == -7
    assert f(P[0], P[1], P[2], P[3], odd(P[4], 2), P[5], P[6], 4, 2, 128, 128, 0.1, 1, None) == -7
    r = lib.kda_recurrent_fwd
    assert r(P[0], P[1], odd(P[2], 8), P[3], P[4], None, P[5], P[6], 2, 4, 2, 128, 128, 0.1, 1,
             None) == -7
    from gated_delta_rule_06_amd import kda
    assert kda.status_string(-7).startswith("KDA_ERR_ALIGN")


def test_backward_workspace_and_validation(lib):
    """Sizes and error paths of kda_backward; every call here returns before
    any launch (fake pointers are never dereferenced)."""
    ws = lib.kda_backward_workspace_size
    # one int per chain (256-byte aligned), then one checkpoint slot (d_k x d_v
    # fp32) per head for every 8 tokens, plus one per sequence, then d_v fp32 per
    # head-token
    assert ws(8, 8192, 32, 128, 128, 0) == 1024 + ((8 + 8 * 8192 // 8) * 32 * 128 * 128
                                                   + 8 * 8192 * 32 * 128) * 4
    assert ws(3, 10, 2, 64, 64, 1) == 256 + ((3 + 10 // 8) * 2 * 64 * 64 + 10 * 2 * 64) * 4
    assert ws(1, 4, 2, 96, 64, 0) == 0
    need = ws(2, 4, 2, 64, 64, 0)
    f = lib.kda_backward

    def call(**kw):
        a = dict(q=P[0], k=P[1], v=P[2], g=P[3], beta=P[4], S0=None, do=P[5], dSf=None,
                 dq=P[6], dk=P[7], dv=P[8], dg=P[9], db=P[10], dS0=None, cu=None, N=2, T=4,
                 H=2, d_k=64, d_v=64, io=0, ph=0, ws=P[11], wsb=need)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["do"], a["dSf"], a["dq"],
                 a["dk"], a["dv"], a["dg"], a["db"], a["dS0"], a["cu"], a["N"], a["T"], a["H"],
                 a["d_k"], a["d_v"], 0.125, a["io"], a["ph"], a["ws"], a["wsb"], None)
    assert call(ph=2) == -3
    assert call(d_k=96) == -3
    assert call(io=5) == -3
    assert call(N=-1) == -2
    assert call(dq=None) == -1
    assert call(ws=None) == -4
    assert call(wsb=need - 1) == -4
    assert call(dv=ctypes.c_void_p(P[8].value + 4)) == -7
    assert call(dq=P[0]) == -6                              # dq is q
    assert call(dk=P[6]) == -6                              # two outputs in one array
    assert call(ws=P[3]) == -6                              # workspace is log_alpha
    assert call(N=0) == 0


def test_backward_noalloc_validation(lib):
    """The allocation-free backward validates like kda_backward and rejects a
    problem whose workspace exceeds its static scratch (KDA_ERR_SCRATCH)
    before any HIP call."""
    assert lib.kda_noalloc_scratch_bytes() == 64 << 20

    def call(T=8, H=2, N=1, dk=128, dv=128, q=P[0], per_head=0, io=1):
        return lib.kda_backward_noalloc(q, P[1], P[2], P[3], P[4], None, P[5], None, P[6], P[7],
                                        P[8], P[9], P[10], None, None, N, T, H, dk, dv, 0.1, io,
                                        per_head, None)
    assert call(q=None) == -1
    assert call(T=-1) == -2
    assert call(dk=96) == -3
    assert call(per_head=2) == -3
    assert call(io=5) == -3
    big_T = 4096
    assert lib.kda_backward_workspace_size(1, big_T, 8, 128, 128, 0) > 64 << 20
    assert call(T=big_T, H=8) == -8                        # KDA_ERR_SCRATCH


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The library binding must not import the oracle or compute on the CPU."""
    src = open(os.path.join(ROOT, "gated_delta_rule_06_amd", "kda.py")).read()
    assert "oracle" not in src
    assert "numpy" not in src
