"""The C ABI without a GPU: the library loads, exports every declared entry
point, its argument structs match the header byte for byte, and every
validation error is returned before anything touches the device."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_deltanet_recurrence_amd as gdr
from gated_deltanet_recurrence_amd import build as gbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gbuild.LIB):
        gbuild.build()
    return gdr.load_library()


def test_exports_every_declared_symbol(lib):
    names = re.findall(r"GDR_API\s+[\w\s\*]+?\b(gdr_\w+)\s*\(", open(HEADER).read())
    assert set(names) == {"gdr_decode", "gdr_chunk", "gdr_chunk_noalloc", "gdr_chunk_workspace_size",
                          "gdr_status_string", "gdr_abi_version", "gdr_conv_prefill", "gdr_conv_decode"}
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", gbuild.LIB], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(names)


def test_abi_version_and_status_strings(lib):
    m = re.search(r"#define GDR_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.gdr_abi_version() == int(m.group(1))
    for code in range(7):
        assert lib.gdr_status_string(code) and lib.gdr_status_string(code) != b"unknown status"
    assert lib.gdr_status_string(99) == b"unknown status"


def _c_layout(tmp_path, struct, fields):
    src = tmp_path / "layout.c"
    body = "".join(f'printf("{f} %zu\\n", offsetof({struct}, {f}));' for f in fields)
    src.write_text(f'#include <stdio.h>\n#include <stddef.h>\n#include "gdr.h"\n'
                   f'int main(void){{printf("sizeof %zu\\n", sizeof({struct}));{body}return 0;}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    return dict((l.split()[0], int(l.split()[1])) for l in lines if l)


@pytest.mark.parametrize("struct,cls", [("gdr_decode_args", gdr.DecodeArgs), ("gdr_chunk_args", gdr.ChunkArgs)])
def test_ctypes_structs_match_header(tmp_path, struct, cls):
    fields = [f for f, _ in cls._fields_]
    c = _c_layout(tmp_path, struct, fields)
    assert c["sizeof"] == ctypes.sizeof(cls)
    for f in fields:
        assert c[f] == getattr(cls, f).offset, f


FAKE = 0x100000   # 16-byte aligned, never dereferenced: validation fails first


def _dec(**kw):
    a = dict(dtype=gdr.GDR_BF16, B=2, Nk=2, Nv=4, S=1, Dk=128, Dv=128, num_slots=4,
             num_state_indices=2, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=None, gk=None,
             state_pool=FAKE, actual_seq_lengths=FAKE, ssm_state_indices=FAKE,
             num_accepted_tokens=None, scale_value=1.0, out=FAKE)
    a.update(kw)
    return gdr.DecodeArgs(**a)


def _chk(**kw):
    a = dict(dtype=gdr.GDR_BF16, B=2, Nk=2, Nv=4, S=100, Dk=128, Dv=128, chunk_size=64,
             q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=None, initial_state=None,
             actual_seq_lengths=None, scale_value=1.0, out=FAKE, final_state=FAKE,
             workspace=FAKE, workspace_bytes=1 << 40)
    a.update(kw)
    return gdr.ChunkArgs(**a)


# Fused gates: the logits, a, A_log and dt_bias come together, in place of beta and g.
_FUSED = dict(beta=None, beta_logits=FAKE, gate_a=FAKE, A_log=FAKE, dt_bias=FAKE)
_OPTION_CASES = [
    (dict(_FUSED, beta=FAKE), gdr.GDR_ERR_SHAPE),
    (dict(_FUSED, g=FAKE), gdr.GDR_ERR_SHAPE),
    (dict(_FUSED, beta_logits=None), gdr.GDR_ERR_NULL),
    (dict(_FUSED, gate_a=None), gdr.GDR_ERR_NULL),
    (dict(_FUSED, A_log=None), gdr.GDR_ERR_NULL),
    (dict(_FUSED, dt_bias=None), gdr.GDR_ERR_NULL),
    (dict(beta_logits=FAKE), gdr.GDR_ERR_SHAPE),
    (dict(_FUSED, Dk=96), gdr.GDR_ERR_UNSUPPORTED),
    (dict(_FUSED, gate_a=FAKE + 2), gdr.GDR_ERR_UNSUPPORTED),
    (dict(_FUSED, beta_logits=FAKE + 2), gdr.GDR_ERR_UNSUPPORTED),
    (dict(beta=FAKE + 2), gdr.GDR_ERR_UNSUPPORTED),
    (dict(_FUSED, B=0, num_state_indices=0, q=None, out=None, workspace=None), gdr.GDR_OK),
]
# Gated RMSNorm epilogue: z and w together, eps a number >= 0, both 16-byte aligned.
_NORM = dict(norm_z=FAKE, norm_w=FAKE, norm_eps=1e-6)
_OPTION_CASES += [
    (dict(norm_z=FAKE), gdr.GDR_ERR_NULL),
    (dict(norm_w=FAKE), gdr.GDR_ERR_NULL),
    (dict(_NORM, norm_eps=-1e-6), gdr.GDR_ERR_SHAPE),
    (dict(_NORM, norm_eps=float("nan")), gdr.GDR_ERR_SHAPE),
    (dict(_NORM, norm_z=FAKE + 4), gdr.GDR_ERR_UNSUPPORTED),
    (dict(_NORM, norm_w=FAKE + 4), gdr.GDR_ERR_UNSUPPORTED),
    (dict(_NORM, Dk=96), gdr.GDR_ERR_UNSUPPORTED),
    (dict(_NORM, B=0, num_state_indices=0, q=None, out=None, workspace=None), gdr.GDR_OK),
]


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), gdr.GDR_ERR_DTYPE),
    (dict(S=0), gdr.GDR_ERR_SHAPE),
    (dict(S=9, num_state_indices=18), gdr.GDR_ERR_SHAPE),
    (dict(Nv=3), gdr.GDR_ERR_SHAPE),
    (dict(B=-1), gdr.GDR_ERR_SHAPE),
    (dict(num_slots=0), gdr.GDR_ERR_SHAPE),
    (dict(num_state_indices=3), gdr.GDR_ERR_SHAPE),
    (dict(Dk=0), gdr.GDR_ERR_SHAPE),
    (dict(q=None), gdr.GDR_ERR_NULL),
    (dict(state_pool=None), gdr.GDR_ERR_NULL),
    (dict(ssm_state_indices=None), gdr.GDR_ERR_NULL),
    (dict(actual_seq_lengths=None), gdr.GDR_ERR_NULL),
    (dict(out=None), gdr.GDR_ERR_NULL),
    (dict(Dk=96), gdr.GDR_ERR_UNSUPPORTED),
    (dict(Dv=256), gdr.GDR_ERR_UNSUPPORTED),
    (dict(v=FAKE + 2), gdr.GDR_ERR_UNSUPPORTED),
    (dict(gk=FAKE + 4), gdr.GDR_ERR_UNSUPPORTED),
    (dict(B=0, num_state_indices=0, q=None, out=None), gdr.GDR_OK),
    (dict(beta=None), gdr.GDR_ERR_NULL),
    (dict(dtype=3), gdr.GDR_ERR_DTYPE),
    (dict(dtype=gdr.GDR_F16, Dk=96), gdr.GDR_ERR_UNSUPPORTED),
] + _OPTION_CASES)
def test_decode_validation(lib, kw, code):
    a = _dec(**kw)
    assert lib.gdr_decode(ctypes.byref(a), None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=-1), gdr.GDR_ERR_DTYPE),
    (dict(S=-1), gdr.GDR_ERR_SHAPE),
    (dict(Nv=5), gdr.GDR_ERR_SHAPE),
    (dict(chunk_size=0), gdr.GDR_ERR_SHAPE),
    (dict(Nk=0), gdr.GDR_ERR_SHAPE),
    (dict(k=None), gdr.GDR_ERR_NULL),
    (dict(final_state=None), gdr.GDR_ERR_NULL),
    (dict(Dk=64, Dv=64), gdr.GDR_ERR_UNSUPPORTED),
    (dict(chunk_size=48), gdr.GDR_ERR_UNSUPPORTED),
    (dict(chunk_size=128), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dtype=gdr.GDR_F32, Dk=128, Dv=128), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dtype=gdr.GDR_F32, Dk=64, Dv=64, chunk_size=64), gdr.GDR_ERR_UNSUPPORTED),
    (dict(initial_state=FAKE + 8), gdr.GDR_ERR_UNSUPPORTED),
    (dict(workspace=None), gdr.GDR_ERR_NULL),
    (dict(workspace_bytes=2 * 4 * 2 * 6144 - 1), gdr.GDR_ERR_SHAPE),
    (dict(workspace=FAKE + 8), gdr.GDR_ERR_UNSUPPORTED),
    (dict(S=1 << 23), gdr.GDR_ERR_UNSUPPORTED),
    (dict(B=0, q=None, out=None, workspace=None), gdr.GDR_OK),
    (dict(beta=None), gdr.GDR_ERR_NULL),
    (dict(dtype=3), gdr.GDR_ERR_DTYPE),
    (dict(dtype=gdr.GDR_F16, chunk_size=48), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dtype=gdr.GDR_F16, Dk=64, Dv=64), gdr.GDR_ERR_UNSUPPORTED),
    (dict(dtype=gdr.GDR_F16, workspace=None), gdr.GDR_ERR_NULL),
] + _OPTION_CASES)
def test_chunk_validation(lib, kw, code):
    a = _chk(**kw)
    assert lib.gdr_chunk(ctypes.byref(a), None) == code


# The allocation-free entry point validates like gdr_chunk, ignores the
# workspace fields, and refuses calls whose scratch exceeds its fixed array
# (B * Nv * ceil(S / 64) chunks of 6 KiB on the 16-bit path) before touching
# the device. Calls that pass validation are GPU tests.
@pytest.mark.parametrize("kw,code", [
    (dict(dtype=-1), gdr.GDR_ERR_DTYPE),
    (dict(Nv=5), gdr.GDR_ERR_SHAPE),
    (dict(k=None), gdr.GDR_ERR_NULL),
    (dict(beta=None), gdr.GDR_ERR_NULL),
    (dict(chunk_size=48), gdr.GDR_ERR_UNSUPPORTED),
    (dict(initial_state=FAKE + 8), gdr.GDR_ERR_UNSUPPORTED),
    (dict(B=0, q=None, out=None), gdr.GDR_OK),
    (dict(B=4, Nk=16, Nv=32, S=4097), gdr.GDR_ERR_SCRATCH_LIMIT),
    (dict(B=4, Nk=16, Nv=32, S=4097, workspace=FAKE + 8, workspace_bytes=0), gdr.GDR_ERR_SCRATCH_LIMIT),
    (dict(B=16, Nk=16, Nv=64, S=16384), gdr.GDR_ERR_SCRATCH_LIMIT),
])
def test_chunk_noalloc_validation(lib, kw, code):
    a = _chk(**kw)
    assert lib.gdr_chunk_noalloc(ctypes.byref(a), None) == code


def test_noalloc_limit_is_the_header_constant(lib):
    m = re.search(r"#define GDR_NOALLOC_SCRATCH_BYTES \((\d+)LL << (\d+)\)", open(HEADER).read())
    limit = int(m.group(1)) << int(m.group(2))
    assert limit == gdr.GDR_NOALLOC_SCRATCH_BYTES
    # the chunked prefill workload's scratch fits exactly; one chunk more does not
    assert lib.gdr_chunk_workspace_size(ctypes.byref(_chk(B=4, Nk=16, Nv=32, S=4096))) == limit
    assert lib.gdr_chunk_workspace_size(ctypes.byref(_chk(B=4, Nk=16, Nv=32, S=4097))) > limit


def test_null_args_struct(lib):
    assert lib.gdr_decode(None, None) == gdr.GDR_ERR_NULL
    assert lib.gdr_chunk(None, None) == gdr.GDR_ERR_NULL
    assert lib.gdr_chunk_noalloc(None, None) == gdr.GDR_ERR_NULL
    assert lib.gdr_conv_prefill(None, None) == gdr.GDR_ERR_NULL
    assert lib.gdr_conv_decode(None, None) == gdr.GDR_ERR_NULL


# Depthwise conv: C = 2*Nk*Dk + Nv*Dv channels, K taps in [1, 8], even head sizes.
def _convp(**kw):
    a = dict(dtype=gdr.GDR_BF16, B=2, S=100, Nk=2, Nv=4, Dk=128, Dv=128, K=4, x=FAKE, weight=FAKE,
             bias=None, initial_state=None, final_state=FAKE, actual_seq_lengths=None, q=FAKE, k=FAKE, v=FAKE)
    a.update(kw)
    return gdr.ConvPrefillArgs(**a)


def _convd(**kw):
    a = dict(dtype=gdr.GDR_BF16, B=2, S=2, Nk=2, Nv=4, Dk=128, Dv=128, K=4, num_slots=4, num_state_indices=4,
             x=FAKE, weight=FAKE, bias=None, state_pool=FAKE, actual_seq_lengths=FAKE, ssm_state_indices=FAKE,
             num_accepted_tokens=None, q=FAKE, k=FAKE, v=FAKE)
    a.update(kw)
    return gdr.ConvDecodeArgs(**a)


_CONV_CASES = [
    (dict(dtype=3), gdr.GDR_ERR_DTYPE),
    (dict(K=0), gdr.GDR_ERR_SHAPE),
    (dict(K=9), gdr.GDR_ERR_SHAPE),
    (dict(Dk=127), gdr.GDR_ERR_SHAPE),
    (dict(Dv=5), gdr.GDR_ERR_SHAPE),
    (dict(Nv=3), gdr.GDR_ERR_SHAPE),
    (dict(B=-1), gdr.GDR_ERR_SHAPE),
    (dict(x=None), gdr.GDR_ERR_NULL),
    (dict(weight=None), gdr.GDR_ERR_NULL),
    (dict(v=None), gdr.GDR_ERR_NULL),
    (dict(x=FAKE + 4), gdr.GDR_ERR_UNSUPPORTED),
    (dict(k=FAKE + 8), gdr.GDR_ERR_UNSUPPORTED),
    (dict(weight=FAKE + 2), gdr.GDR_ERR_UNSUPPORTED),
    (dict(bias=FAKE + 2), gdr.GDR_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,code", _CONV_CASES + [
    (dict(S=0), gdr.GDR_ERR_SHAPE),
    (dict(initial_state=FAKE + 8), gdr.GDR_ERR_UNSUPPORTED),
    (dict(B=0, x=None, q=None), gdr.GDR_OK),
])
def test_conv_prefill_validation(lib, kw, code):
    assert lib.gdr_conv_prefill(ctypes.byref(_convp(**kw)), None) == code


@pytest.mark.parametrize("kw,code", _CONV_CASES + [
    (dict(S=9, num_state_indices=18), gdr.GDR_ERR_SHAPE),
    (dict(num_state_indices=3), gdr.GDR_ERR_SHAPE),
    (dict(num_slots=0), gdr.GDR_ERR_SHAPE),
    (dict(state_pool=None), gdr.GDR_ERR_NULL),
    (dict(ssm_state_indices=None), gdr.GDR_ERR_NULL),
    (dict(actual_seq_lengths=None), gdr.GDR_ERR_NULL),
    (dict(state_pool=FAKE + 8), gdr.GDR_ERR_UNSUPPORTED),
    (dict(B=0, num_state_indices=0, x=None, q=None), gdr.GDR_OK),
])
def test_conv_decode_validation(lib, kw, code):
    assert lib.gdr_conv_decode(ctypes.byref(_convd(**kw)), None) == code


def test_binding_rejects_host_tensors(lib):
    import torch
    x = torch.zeros(1, 1, 1, 16)
    with pytest.raises(RuntimeError):
        gdr.gdr_chunk(x, x, x, torch.zeros(1, 1, 1))
    with pytest.raises(RuntimeError):
        gdr.gdr_decode(x, x, x, torch.zeros(1, 1, 1), torch.zeros(1, 1, 16, 16),
                       torch.zeros(1, dtype=torch.int32), torch.zeros(1, dtype=torch.int32))


def test_binding_maps_status_to_exceptions(lib):
    with pytest.raises(ValueError):
        gdr._check(gdr.GDR_ERR_SHAPE, "x")
    for code in (gdr.GDR_ERR_NULL, gdr.GDR_ERR_DTYPE, gdr.GDR_ERR_UNSUPPORTED, gdr.GDR_ERR_LAUNCH):
        with pytest.raises(RuntimeError):
            gdr._check(code, "x")
    gdr._check(gdr.GDR_OK, "x")


def test_chunk_workspace_size(lib):
    # The matrix-core path needs 6 KB per (sequence, value head, chunk of 64),
    # for chunk sizes 16 and 32 too (it computes in chunks of 64); the float32
    # path needs none.
    assert lib.gdr_chunk_workspace_size(ctypes.byref(_chk())) == 2 * 4 * 2 * 6144
    assert lib.gdr_chunk_workspace_size(ctypes.byref(_chk(S=128))) == 2 * 4 * 2 * 6144
    assert lib.gdr_chunk_workspace_size(ctypes.byref(_chk(S=0))) == 0
    assert lib.gdr_chunk_workspace_size(ctypes.byref(_chk(dtype=gdr.GDR_F32, Dk=32, Dv=32, chunk_size=32))) == 0
    assert lib.gdr_chunk_workspace_size(ctypes.byref(_chk(dtype=gdr.GDR_F16))) == 2 * 4 * 2 * 6144
    for cs in (16, 32):
        assert lib.gdr_chunk_workspace_size(ctypes.byref(_chk(chunk_size=cs))) == 2 * 4 * 2 * 6144
    assert lib.gdr_chunk_workspace_size(ctypes.byref(_chk(chunk_size=48))) == 0
    assert lib.gdr_chunk_workspace_size(None) == -1
