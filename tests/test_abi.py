"""The C ABI without a GPU: the library loads, exports what include/kda.h
declares, and rejects bad arguments on the host before touching HIP."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_kda_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def lib():
    if not os.path.exists(kda.library_path()):
        from gated_delta_rule_kda_amd import build
        build.build()
    return kda._load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == {"kda_abi_version", "kda_last_error", "kda_chunk_fwd",
                          "kda_chunk_fwd_snapshots", "kda_recurrent_fwd", "kda_prefill_prologue",
                          "kda_output_gate", "kda_decode_step", "kda_recurrent_bwd",
                          "kda_recurrent_bwd_workspace_size"}
    L = ctypes.CDLL(kda.library_path())
    for n in names:
        assert hasattr(L, n), n


def test_abi_version():
    assert lib().kda_abi_version() == kda.ABI_VERSION


def test_prologue_struct_layout(tmp_path):
    """The ctypes mirror of kda_decode_prologue has the layout the C compiler
    gives the struct in include/kda.h."""
    import subprocess
    fields = [f[0] for f in kda.DecodePrologue._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"kda.h\"\nint main(void){\n"
                   + 'printf("%zu\\n", sizeof(kda_decode_prologue));\n'
                   + "".join('printf("%%zu\\n", offsetof(kda_decode_prologue, %s));\n' % f for f in fields)
                   + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                           text=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(kda.DecodePrologue)
    for f, off in zip(fields, vals[1:]):
        assert getattr(kda.DecodePrologue, f).offset == off, f


FAKE = 0x100000   # never dereferenced: every call below fails validation first


def chunk(**over):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, beta=FAKE * 5, s0=None, out=FAKE * 6,
             st=None, B=1, T=8, H=2, HV=4, K=32, V=32, scale=0.0, chunk=0, dtype=1)
    a.update(over)
    L = lib()
    rc = L.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["out"], a["st"],
                         a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"], a["scale"], a["chunk"],
                         a["dtype"], None)
    return rc, L.kda_last_error().decode()


# big, disjoint fake ranges so that only the intended overlap triggers
BIG = 1 << 36


@pytest.mark.parametrize("over,code,msg", [
    (dict(HV=3), 1, "multiple"),
    (dict(H=0), 1, ">= 1"),
    (dict(B=-1), 1, ">= 0"),
    (dict(T=-2), 1, ">= 0"),
    (dict(K=16), 2, "32, 64 or 128"),
    (dict(V=256), 2, "32, 64 or 128"),
    (dict(chunk=64), 2, "only 32"),
    (dict(chunk=-1), 1, "chunk"),
    (dict(dtype=7), 2, "dtype"),
    (dict(q=None), 1, "non-NULL"),
    (dict(out=None), 1, "non-NULL"),
    (dict(g=FAKE + 4), 1, "aligned"),
    (dict(scale=float("inf")), 1, "infinite"),
    (dict(q=BIG, k=2 * BIG, v=3 * BIG, g=4 * BIG, beta=5 * BIG, out=3 * BIG + 64), 1, "out overlaps v"),
    (dict(q=BIG, k=2 * BIG, v=3 * BIG, g=4 * BIG, beta=5 * BIG, out=6 * BIG, st=4 * BIG + 16),
     1, "final_state overlaps g"),
    (dict(q=BIG, k=2 * BIG, v=3 * BIG, g=4 * BIG, beta=5 * BIG, out=6 * BIG, s0=7 * BIG,
          st=7 * BIG + 64), 1, "final_state overlaps initial_state"),
    (dict(B=1 << 20, T=1 << 20, H=128, HV=128), 1, "overflow"),
])
def test_chunk_fwd_rejects(over, code, msg):
    rc, err = chunk(**over)
    assert rc == code, err
    assert msg in err, err


def snap_call(snaps, every, **over):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, beta=FAKE * 5, s0=None, out=FAKE * 6,
             st=None, B=1, T=64, H=2, HV=4, K=32, V=32, scale=0.0, chunk=0, dtype=1)
    a.update(over)
    L = lib()
    rc = L.kda_chunk_fwd_snapshots(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["out"],
                                   a["st"], snaps, every, a["B"], a["T"], a["H"], a["HV"], a["K"],
                                   a["V"], a["scale"], a["chunk"], a["dtype"], None)
    return rc, L.kda_last_error().decode()


@pytest.mark.parametrize("snaps,every,over,code,msg", [
    (FAKE * 7, 0, {}, 1, "snapshot_every=0"),
    (FAKE * 7, 48, {}, 1, "multiple of the chunk size"),
    (FAKE * 7, -32, {}, 1, "snapshot_every"),
    (FAKE * 7 + 8, 32, {}, 1, "snapshots is not 16-byte aligned"),
    (3 * BIG + 256, 32, dict(q=BIG, k=2 * BIG, v=3 * BIG, g=4 * BIG, beta=5 * BIG, out=6 * BIG),
     1, "snapshots overlap v"),
    (6 * BIG - 64, 32, dict(q=BIG, k=2 * BIG, v=3 * BIG, g=4 * BIG, beta=5 * BIG, out=6 * BIG),
     1, "snapshots overlap out"),
    (7 * BIG + 64, 32, dict(q=BIG, k=2 * BIG, v=3 * BIG, g=4 * BIG, beta=5 * BIG, out=6 * BIG,
                            st=7 * BIG), 1, "snapshots overlap final_state"),
    (FAKE * 7, 32, dict(HV=3), 1, "kda_chunk_fwd_snapshots: HV=3"),
])
def test_chunk_fwd_snapshots_rejects(snaps, every, over, code, msg):
    rc, err = snap_call(snaps, every, **over)
    assert rc == code, err
    assert msg in err, err


def test_chunk_fwd_snapshots_empty_is_noop():
    # NULL snapshots ignore snapshot_every; no tokens means no HIP call
    rc, err = snap_call(None, 0, T=0, q=None, k=None, v=None, g=None, beta=None, out=None)
    assert rc == 0, err
    rc, err = snap_call(FAKE * 7, 32, B=0, q=None, k=None, v=None, g=None, beta=None, out=None)
    assert rc == 0, err


def test_chunk_fwd_empty_is_noop():
    # B*T == 0 with no final state: nothing to do, no HIP call.
    rc, err = chunk(B=0, q=None, k=None, v=None, g=None, beta=None, out=None)
    assert rc == 0, err
    rc, err = chunk(T=0, q=None, k=None, v=None, g=None, beta=None, out=None)
    assert rc == 0, err


def decode(pro=None, **over):
    a = dict(qkv=FAKE, gate=FAKE * 2, beta=FAKE * 3, state=FAKE * 4, out=FAKE * 5,
             B=2, H=2, HV=4, K=64, V=64, scale=0.0, dtype=0)
    a.update(over)
    L = lib()
    rc = L.kda_decode_step(a["qkv"], a["gate"], a["beta"], a["state"], a["out"],
                           ctypes.byref(pro) if pro is not None else None, a["B"], a["H"], a["HV"],
                           a["K"], a["V"], a["scale"], a["dtype"], None)
    return rc, L.kda_last_error().decode()


def prologue(**kw):
    p = kda.DecodePrologue()
    for k_, v_ in kw.items():
        setattr(p, k_, v_)
    return p


@pytest.mark.parametrize("over,code,msg", [
    (dict(HV=3), 1, "multiple"),
    (dict(K=48), 2, "32, 64 or 128"),
    (dict(dtype=3), 2, "dtype"),
    (dict(state=None), 1, "non-NULL"),
    (dict(out=FAKE + 8), 1, "aligned"),
    (dict(qkv=BIG, gate=2 * BIG, beta=3 * BIG, state=4 * BIG, out=4 * BIG + 4096), 1, "overlaps"),
])
def test_decode_rejects(over, code, msg):
    rc, err = decode(**over)
    assert rc == code, err
    assert msg in err, err


@pytest.mark.parametrize("pro,code,msg", [
    (dict(conv_weight=FAKE * 7, conv_kernel=4), 1, "conv_state"),
    (dict(conv_weight=FAKE * 7, conv_state=FAKE * 8, conv_kernel=0), 1, ">= 1"),
    (dict(conv_weight=FAKE * 7, conv_state=FAKE * 8, conv_kernel=9), 2, "at most 8"),
    (dict(gate_mode=1), 1, "A_log"),
    (dict(gate_mode=5), 1, "gate_mode"),
    (dict(l2norm_qk=1, l2_eps=-1.0), 1, "l2_eps"),
])
def test_decode_prologue_rejects(pro, code, msg):
    rc, err = decode(prologue(**pro))
    assert rc == code, err
    assert msg in err, err


def test_decode_empty_batch_is_noop():
    rc, err = decode(B=0, qkv=None, gate=None, beta=None, state=None, out=None)
    assert rc == 0, err


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 32)
    with pytest.raises(ValueError, match="GPU"):
        kda.chunk_fwd(q, q, q, q, torch.zeros(1, 4, 1))


def prologue_call(pro=None, **over):
    a = dict(x=FAKE, gate=FAKE * 2, beta=FAKE * 3, q=FAKE * 4, k=FAKE * 5, v=FAKE * 6, g=FAKE * 7,
             bo=FAKE * 8, B=1, T=8, H=2, HV=4, K=32, V=32, dtype=1)
    a.update(over)
    L = lib()
    rc = L.kda_prefill_prologue(a["x"], a["gate"], a["beta"], ctypes.byref(pro) if pro else None,
                                a["q"], a["k"], a["v"], a["g"], a["bo"], a["B"], a["T"], a["H"],
                                a["HV"], a["K"], a["V"], a["dtype"], None)
    return rc, L.kda_last_error().decode()


@pytest.mark.parametrize("over,code,msg", [
    (dict(HV=3), 1, "multiple"),
    (dict(K=48), 2, "32, 64 or 128"),
    (dict(dtype=5), 2, "dtype"),
    (dict(T=-1), 1, ">= 0"),
    (dict(x=None), 1, "non-NULL"),
    (dict(g=FAKE * 7 + 4), 1, "g is not 16-byte aligned"),
    (dict(x=BIG, gate=2 * BIG, beta=3 * BIG, q=4 * BIG, k=5 * BIG, v=6 * BIG, g=7 * BIG,
          bo=2 * BIG + 64), 1, "beta_out overlaps gate"),
    (dict(x=BIG, gate=2 * BIG, beta=3 * BIG, q=4 * BIG, k=4 * BIG + 256, v=6 * BIG, g=7 * BIG,
          bo=8 * BIG), 1, "q overlaps k"),
])
def test_prefill_prologue_rejects(over, code, msg):
    rc, err = prologue_call(**over)
    assert rc == code, err
    assert msg in err, err


@pytest.mark.parametrize("pro,code,msg", [
    (dict(conv_weight=FAKE * 9, conv_kernel=0), 1, "conv_kernel=0"),
    (dict(conv_weight=FAKE * 9, conv_kernel=9), 2, "at most 8"),
    (dict(gate_mode=1), 1, "needs A_log"),
    (dict(gate_mode=4), 1, "kda_gate_mode"),
    (dict(l2norm_qk=1, l2_eps=-1.0), 1, "l2_eps"),
])
def test_prefill_prologue_struct_rejects(pro, code, msg):
    p = kda.DecodePrologue()
    for kk, vv in pro.items():
        setattr(p, kk, vv)
    rc, err = prologue_call(pro=p)
    assert rc == code, err
    assert msg in err, err


def test_prefill_prologue_empty_is_noop():
    rc, err = prologue_call(T=0, x=None, gate=None, beta=None, q=None, k=None, v=None, g=None, bo=None)
    assert rc == 0, err


@pytest.mark.parametrize("args,code,msg", [
    (dict(D=48), 2, "head_dim"),
    (dict(rows=-1), 1, "rows"),
    (dict(eps=float("nan")), 1, "eps"),
    (dict(eps=-1.0), 1, "eps"),
    (dict(dtype=3), 2, "dtype"),
    (dict(o=None), 1, "non-NULL"),
    (dict(y=FAKE * 3 + 8), 1, "y is not 16-byte aligned"),
    (dict(y=FAKE * 2 + 64), 1, "y overlaps gate"),
    (dict(y=FAKE + 64), 1, "y overlaps o"),
])
def test_output_gate_rejects(args, code, msg):
    a = dict(o=FAKE, gate=FAKE * 2, y=FAKE * 3, rows=4, D=32, eps=1e-6, dtype=1)
    a.update(args)
    L = lib()
    rc = L.kda_output_gate(a["o"], a["gate"], a["y"], a["rows"], a["D"], a["eps"], a["dtype"], None)
    err = L.kda_last_error().decode()
    assert rc == code, err
    assert msg in err, err


@pytest.mark.parametrize("over,code,msg", [
    (dict(HV=3), 1, "kda_recurrent_fwd: HV=3"),
    (dict(K=16), 2, "32, 64 or 128"),
    (dict(q=None), 1, "non-NULL"),
    (dict(q=BIG, k=2 * BIG, v=3 * BIG, g=4 * BIG, beta=5 * BIG, out=3 * BIG + 64), 1, "out overlaps v"),
])
def test_recurrent_fwd_rejects(over, code, msg):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, beta=FAKE * 5, s0=None, out=FAKE * 6,
             st=None, B=1, T=8, H=2, HV=4, K=32, V=32, scale=0.0, dtype=1)
    a.update(over)
    L = lib()
    rc = L.kda_recurrent_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["out"], a["st"],
                             a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"], a["scale"], a["dtype"], None)
    err = L.kda_last_error().decode()
    assert rc == code, err
    assert msg in err, err


def bwd_call(**over):
    """kda_recurrent_bwd with fake, disjoint pointers (each BIG apart)."""
    a = dict(q=BIG, k=2 * BIG, v=3 * BIG, g=4 * BIG, beta=5 * BIG, s0=None, do=6 * BIG, dst=None,
             dq=7 * BIG, dk=8 * BIG, dv=9 * BIG, dg=10 * BIG, db=11 * BIG, ds0=None, ws=12 * BIG,
             wsb=1 << 40, B=1, T=8, H=2, HV=4, K=32, V=32, scale=0.0, dtype=1)
    a.update(over)
    L = lib()
    rc = L.kda_recurrent_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["do"], a["dst"],
                             a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["ds0"], a["B"], a["T"],
                             a["H"], a["HV"], a["K"], a["V"], a["scale"], a["dtype"], a["ws"], a["wsb"],
                             None)
    return rc, L.kda_last_error().decode()


@pytest.mark.parametrize("over,code,msg", [
    (dict(HV=3), 1, "kda_recurrent_bwd: HV=3"),
    (dict(K=16), 2, "32, 64 or 128"),
    (dict(dtype=5), 2, "dtype"),
    (dict(do=None), 1, "dout must be non-NULL"),
    (dict(dg=None), 1, "dbeta must be non-NULL"),
    (dict(ws=None), 1, "workspace is NULL"),
    (dict(wsb=1000), 1, "needed"),
    (dict(dq=FAKE + 8), 1, "dq is not 16-byte aligned"),
    (dict(dv=3 * BIG + 32), 1, "dv overlaps v"),
    (dict(ws=7 * BIG + 512), 1, "dq overlaps workspace"),
    (dict(ds0=6 * BIG), 1, "dinitial_state overlaps dout"),
    (dict(scale=float("inf")), 1, "infinite"),
])
def test_recurrent_bwd_rejects(over, code, msg):
    rc, err = bwd_call(**over)
    assert rc == code, err
    assert msg in err, err


def test_recurrent_bwd_workspace_size():
    L = lib()
    n = L.kda_recurrent_bwd_workspace_size(2, 100, 2, 4, 64, 128)
    # r, dr [B,T,HV,V]; S_T [B,HV,K,V]; 3 x partials [V/32,B,T,HV,K]; e [B,T,HV,K];
    # block sums and the final-state term [B,HV,K,ceil(T/64)+1] -- fp32, each
    # region rounded up to 256 bytes
    up = lambda floats: (floats * 4 + 255) // 256 * 256
    want = (2 * up(2 * 100 * 4 * 128) + up(2 * 4 * 64 * 128) + 3 * up(4 * 2 * 100 * 4 * 64)
            + up(2 * 100 * 4 * 64) + up(2 * 4 * 64 * 3))
    assert n == want
    assert L.kda_recurrent_bwd_workspace_size(1, 8, 2, 3, 32, 32) == -1
    assert "HV=3" in L.kda_last_error().decode()
    assert L.kda_recurrent_bwd_workspace_size(1, 8, 2, 4, 32, 48) == -1


def test_recurrent_bwd_empty_batch_is_noop():
    rc, err = bwd_call(B=0, q=None, k=None, v=None, g=None, beta=None, do=None, dq=None, dk=None,
                       dv=None, dg=None, db=None, ws=None)
    assert rc == 0, err
