"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, matches the header's struct layout, and rejects bad
arguments on the host before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "plp.h")

abi = pytest.importorskip("rl_policy_gradient_amd._abi")


def _lib():
    if not os.path.exists(abi.LIB_PATH):
        pytest.skip("libplp.so not built")
    return abi.lib()


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"PLP_API\s+[\w\s\*]+?\b(plp_\w+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = _lib()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", abi.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (plp_\w+)", out))
    assert exported == set(names)


def test_struct_layout_matches_header(tmp_path):
    """Compile a probe against include/plp.h with gcc and compare sizeof and
    every offsetof with the ctypes mirror."""
    fields_a = [f for f, _ in abi.PlpArgs._fields_]
    fields_o = [f for f, _ in abi.PlpOutputs._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "plp.h"', "int main(void){"]
    src.append('printf("%zu %zu\\n", sizeof(plp_args), sizeof(plp_outputs));')
    for f in fields_a:
        src.append(f'printf("a {f} %zu\\n", offsetof(plp_args, {f}));')
    for f in fields_o:
        src.append(f'printf("o {f} %zu\\n", offsetof(plp_outputs, {f}));')
    src.append("return 0;}")
    c = tmp_path / "probe.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "probe"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I",
                        "/opt/rocm/include", str(c), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lines = subprocess.run([str(exe)], capture_output=True, text=True).stdout.split("\n")
    sa, so = map(int, lines[0].split())
    assert sa == ctypes.sizeof(abi.PlpArgs) and so == ctypes.sizeof(abi.PlpOutputs)
    for ln in lines[1:]:
        if not ln:
            continue
        kind, name, off = ln.split()
        cls = abi.PlpArgs if kind == "a" else abi.PlpOutputs
        assert getattr(cls, name).offset == int(off), name


def _valid_args():
    a = abi.new_args()
    a.B, a.T, a.H, a.V = 2, 8, 128, 1000
    a.dtype = abi.DTYPE_BF16
    fake = 0x1000  # never dereferenced: every call below fails validation first
    for f in ("hidden", "weight", "targets", "completion_mask", "advantages"):
        setattr(a, f, fake)
    a.epsilon_low = a.epsilon_high = 0.2
    return a


def _call(a, o=None, ws=None, ws_bytes=0):
    L = _lib()
    if o is None:
        o = abi.new_outputs()
        o.loss = o.metrics = 0x2000
    rc = L.plp_fused_lmhead_policy_loss_fwd_bwd(ctypes.byref(a), ctypes.byref(o), ws, ws_bytes, None)
    return rc, L.plp_last_error().decode()


@pytest.mark.parametrize("mutate,code,msg", [
    (lambda a: setattr(a, "top_entropy_quantile", 1.5), abi.PLP_E_INVALID, "top_entropy_quantile"),
    (lambda a: setattr(a, "top_entropy_quantile", -0.1), abi.PLP_E_INVALID, "top_entropy_quantile"),
    (lambda a: setattr(a, "top_entropy_quantile", float("nan")), abi.PLP_E_INVALID, "top_entropy_quantile"),
    (lambda a: setattr(a, "beta", 0.04), abi.PLP_E_INVALID, "ref_logp"),
    (lambda a: setattr(a, "temperature", 0.0), abi.PLP_E_INVALID, "temperature"),
    (lambda a: setattr(a, "B", 0), abi.PLP_E_INVALID, "B and T"),
    (lambda a: setattr(a, "is_level", abi.IS_SEQUENCE), abi.PLP_E_UNSUPPORTED, "sequence-level"),
    (lambda a: (setattr(a, "loss_type", abi.LOSS_GSPO_TOKEN)), abi.PLP_E_UNSUPPORTED, "GSPO_TOKEN"),
    (lambda a: setattr(a, "hidden", None), abi.PLP_E_INVALID, "required"),
    (lambda a: setattr(a, "completion_mask", None), abi.PLP_E_INVALID, "required"),
    (lambda a: setattr(a, "epsilon_low", -0.1), abi.PLP_E_INVALID, "epsilon"),
    (lambda a: setattr(a, "chunk_sequences", -1), abi.PLP_E_INVALID, "chunk_sequences"),
    (lambda a: (setattr(a, "loss_type", abi.LOSS_GRPO), setattr(a, "is_level", abi.IS_SEQUENCE)),
     abi.PLP_E_UNSUPPORTED, "GSPO_TOKEN"),
    (lambda a: (setattr(a, "loss_type", abi.LOSS_DAPO), setattr(a, "global_tokens", -5)),
     abi.PLP_E_INVALID, "global_tokens"),
    (lambda a: setattr(a, "loss_type", 5), abi.PLP_E_INVALID, "loss_type"),
    (lambda a: setattr(a, "weight", 0x1008), abi.PLP_E_INVALID, "16-byte aligned"),
    (lambda a: setattr(a, "token_advantages", 0x4000), abi.PLP_E_UNSUPPORTED, "per-sequence advantages"),
    (lambda a: setattr(a, "advantages", None), abi.PLP_E_INVALID, "advantages"),
    (lambda a: setattr(a, "struct_size", 8), abi.PLP_E_INVALID, "struct_size"),
    (lambda a: setattr(a, "H", 5000), abi.PLP_E_UNSUPPORTED, "H=5000"),
    (lambda a: setattr(a, "dtype", 7), abi.PLP_E_INVALID, "dtype"),
    (lambda a: setattr(a, "weight_prepared", 0x5008), abi.PLP_E_INVALID, "weight_prepared must be 16-byte"),
    (lambda a: (setattr(a, "weight_prepared", 0x5000), setattr(a, "H", 200)), abi.PLP_E_UNSUPPORTED,
     "weight_prepared is for bf16"),
    (lambda a: (setattr(a, "weight_prepared", 0x5000), setattr(a, "dtype", abi.DTYPE_F32)), abi.PLP_E_UNSUPPORTED,
     "weight_prepared is for bf16"),
])
def test_validation_rejects_before_launch(mutate, code, msg):
    a = _valid_args()
    mutate(a)
    rc, err = _call(a)
    assert rc == code, err
    assert msg in err


def test_version_one_args_are_accepted():
    """A caller built against ABI version 1 (struct_size ending before
    global_tokens) passes validation; the field reads as its default."""
    a = _valid_args()
    a.struct_size = abi.PlpArgs.global_tokens.offset
    a.global_tokens = -5  # beyond the caller's struct: must not be read
    a.loss_type = abi.LOSS_DAPO
    rc, err = _call(a, ws=None, ws_bytes=0)
    assert rc == abi.PLP_E_WORKSPACE, err


def test_workspace_checks():
    a = _valid_args()
    rc, err = _call(a, ws=None, ws_bytes=0)
    assert rc == abi.PLP_E_WORKSPACE and "too small" in err
    n = ctypes.c_size_t()
    assert _lib().plp_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    rc, err = _call(a, ws=0x1001, ws_bytes=n.value)
    assert rc == abi.PLP_E_WORKSPACE and "aligned" in err
    o = abi.new_outputs()
    o.loss = o.metrics = 0x2000
    o.grad_bias = 0x3000
    rc, err = _call(a, o=o)
    assert rc == abi.PLP_E_INVALID and "grad_bias" in err


def test_workspace_size_has_no_NV_term():
    """Peak workspace grows with N and with V separately, never with N*V
    (the [N, V] logits are never stored; PR #1320 Summary)."""
    import rl_policy_gradient_amd as plp
    _lib()
    w = {(B, V): plp.workspace_size(B, 1024, 896, V) for B in (1, 8) for V in (32768, 262144)}
    # doubling-style check: the cross term (w(8,big) - w(8,small)) - (w(1,big) - w(1,small)) is ~0
    cross = (w[8, 262144] - w[8, 32768]) - (w[1, 262144] - w[1, 32768])
    assert abs(cross) < 4096, cross
    # and far below what a stored [N, V] fp32 logits tensor would need
    assert w[8, 262144] < 8 * 1024 * 262144 * 4 / 4


def test_other_entry_points_validate():
    L = _lib()
    n = ctypes.c_size_t()
    assert L.plp_selective_entropy_workspace_size(0, 128, 100, 1, ctypes.byref(n)) == abi.PLP_E_INVALID
    assert L.plp_entropy_quantile_mask(None, None, 10, 2.0, None, None, None, 0, None) == abi.PLP_E_INVALID
    assert "q must lie" in L.plp_last_error().decode()
    a = _valid_args()
    assert L.plp_policy_loss_from_logprobs(ctypes.byref(a), None, None, None, None, 0, None) == abi.PLP_E_INVALID
    assert L.plp_abi_version() == 5 == abi.ABI_VERSION


def test_noalloc_quantile_rejects_bad_arguments_on_the_host():
    """The no-allocation entry point checks its arguments before touching the
    device: N outside [0, 2^31), q outside [0, 1], missing pointers."""
    L = _lib()
    assert L.plp_entropy_quantile_mask_noalloc(None, None, -1, 0.5, None, None, None) == abi.PLP_E_INVALID
    assert L.plp_entropy_quantile_mask_noalloc(None, None, 1 << 31, 0.5, None, None, None) == abi.PLP_E_INVALID
    assert b"2^31" in L.plp_last_error()
    assert L.plp_entropy_quantile_mask_noalloc(None, None, 10, 1.5, None, None, None) == abi.PLP_E_INVALID
    assert L.plp_entropy_quantile_mask_noalloc(None, None, 10, 0.5, None, None, None) == abi.PLP_E_INVALID


def test_version_three_args_ignore_weight_prepared():
    """A caller built against ABI version 3 (struct_size ending before
    weight_prepared): the field is not read, so a misaligned value there does
    not fail the call's checks."""
    a = _valid_args()
    a.struct_size = abi.PlpArgs.weight_prepared.offset
    a.weight_prepared = 0x5008
    rc, err = _call(a, ws=None, ws_bytes=0)
    assert rc == abi.PLP_E_WORKSPACE, err


def test_prepared_weight_size_and_checks():
    """The weight's matrix-core copy: V rounded up to 64 rows of H bf16; the
    fused call's workspace shrinks by exactly that much when the caller
    passes it; shapes off the matrix-core path and bad buffers are rejected
    on the host."""
    import rl_policy_gradient_amd as plp
    L = _lib()
    n = ctypes.c_size_t()
    assert L.plp_prepared_weight_size(896, 151936, abi.DTYPE_BF16, ctypes.byref(n)) == 0
    assert n.value == 151936 * 896 * 2  # 151936 is a multiple of 64
    assert L.plp_prepared_weight_size(128, 1000, abi.DTYPE_BF16, ctypes.byref(n)) == 0
    assert n.value == 1024 * 128 * 2
    assert plp.prepared_weight_size(128, 1000) == 1024 * 128 * 2
    assert L.plp_prepared_weight_size(200, 1000, abi.DTYPE_BF16, ctypes.byref(n)) == abi.PLP_E_UNSUPPORTED
    assert L.plp_prepared_weight_size(128, 1000, abi.DTYPE_F32, ctypes.byref(n)) == abi.PLP_E_UNSUPPORTED
    assert L.plp_prepared_weight_size(128, 0, abi.DTYPE_BF16, ctypes.byref(n)) == abi.PLP_E_INVALID
    need = 1024 * 128 * 2
    assert L.plp_prepare_weight(None, 128, 1000, abi.DTYPE_BF16, 0x10000, need, None) == abi.PLP_E_INVALID
    assert L.plp_prepare_weight(0x1000, 128, 1000, abi.DTYPE_BF16, 0x10080, need, None) == abi.PLP_E_INVALID
    assert b"256-byte" in L.plp_last_error()
    assert L.plp_prepare_weight(0x1000, 128, 1000, abi.DTYPE_BF16, 0x10000, need - 1, None) == abi.PLP_E_INVALID
    assert b"too small" in L.plp_last_error()
    for B, V, q, chunk in ((1, 151936, 1.0, 0), (8, 151936, 0.2, 2), (3, 1000, 1.0, 0)):
        full = plp.workspace_size(B, 512, 896, V, top_entropy_quantile=q, chunk_sequences=chunk)
        prep = plp.workspace_size(B, 512, 896, V, top_entropy_quantile=q, chunk_sequences=chunk,
                                  weight_prepared=True)
        assert full - prep == plp.prepared_weight_size(896, V)


def test_selective_entropy_prepared_size_and_checks():
    """The selective-entropy call on a prepared weight: its workspace is the
    plain call's less exactly the weight's copy; shapes off the matrix-core
    path, a NULL or misaligned prepared copy and the plain call's own errors
    are rejected on the host."""
    import rl_policy_gradient_amd as plp
    L = _lib()
    n, m = ctypes.c_size_t(), ctypes.c_size_t()
    for N, H, V in ((512, 896, 151936), (65536, 896, 151936), (37, 128, 1000), (1, 512, 40)):
        assert L.plp_selective_entropy_workspace_size(N, H, V, abi.DTYPE_BF16, ctypes.byref(n)) == 0
        assert L.plp_selective_entropy_prepared_workspace_size(N, H, V, abi.DTYPE_BF16, ctypes.byref(m)) == 0
        assert n.value - m.value == plp.prepared_weight_size(H, V), (N, H, V)
    assert L.plp_selective_entropy_prepared_workspace_size(64, 200, 100, abi.DTYPE_BF16,
                                                           ctypes.byref(m)) == abi.PLP_E_UNSUPPORTED
    assert L.plp_selective_entropy_prepared_workspace_size(64, 128, 100, abi.DTYPE_F32,
                                                           ctypes.byref(m)) == abi.PLP_E_UNSUPPORTED
    assert L.plp_selective_entropy_prepared_workspace_size(0, 128, 100, abi.DTYPE_BF16,
                                                           ctypes.byref(m)) == abi.PLP_E_INVALID
    assert L.plp_selective_entropy_prepared_workspace_size(64, 128, 100, abi.DTYPE_BF16, ctypes.byref(m)) == 0
    ws = m.value

    def call(wprep, h=0x1000, w=0x2000, ent=0x3000, ws_ptr=0x100000, ws_bytes=ws):
        return L.plp_selective_entropy_prepared(h, w, wprep, None, 64, 128, 100, abi.DTYPE_BF16, ctypes.c_float(1.0),
                                                None, ent, None, ws_ptr, ws_bytes, None)

    assert call(None) == abi.PLP_E_INVALID
    assert b"weight_prepared" in L.plp_last_error()
    assert call(0x4008) == abi.PLP_E_INVALID
    assert b"16-byte" in L.plp_last_error()
    assert call(0x4000, ent=None) == abi.PLP_E_INVALID
    assert call(0x4000, ws_bytes=ws - 1) == abi.PLP_E_WORKSPACE
