"""GPU test of gdr_chunk_noalloc, the allocation-free entry point: its
outputs and final states equal gdr_chunk's (the same kernels, the scratch
taken from the library's fixed per-GPU array instead of a workspace), on two
calls in a row and more, each smaller than the first, so that whatever an
earlier call left in the array cannot leak into a later call's results."""
import pytest
import torch

import synth
from tests.gpu_util import raw_bits, say, to_dev
import gated_deltanet_recurrence_amd as gdr

pytestmark = pytest.mark.gpu


def _both(c, gates=None):
    args = dict(initial_state=to_dev(c.state), actual_seq_lengths=to_dev(c.lens), g=to_dev(c.g),
                scale_value=c.scale, chunk_size=c.chunk)
    q, k, v, beta = (to_dev(getattr(c, n)) for n in ("q", "k", "v", "beta"))
    say(f"gdr_chunk and gdr_chunk_noalloc {c.dtype} B={c.B} Nk={c.Nk} Nv={c.Nv} S={c.S} C={c.chunk}")
    o1, f1 = gdr.gdr_chunk(q, k, v, beta, **args)
    o2 = torch.empty_like(o1)
    f2 = torch.empty_like(f1)
    gdr.gdr_chunk_noalloc(q, k, v, beta, out=o2, final_state=f2, **args)
    torch.cuda.synchronize()
    assert torch.equal(raw_bits(o1), raw_bits(o2)), "outputs differ"
    assert torch.equal(raw_bits(f1), raw_bits(f2)), "final states differ"


def test_noalloc_equals_chunk_twice_shrinking():
    # first the largest call the array holds (the chunked prefill workload's
    # 8192 chunks), then a smaller ragged one
    _both(synth.config(4, base=471))
    # 512 heads take the whole-head workgroups (2560 chunks)
    _both(synth.config(4, B=8, Nk=16, Nv=64, S=300, lens=[300, 131, 64, 1, 0, 299, 77, 200], base=474))
    _both(synth.config(4, B=2, Nk=2, Nv=4, S=300, lens=[300, 131], base=472))


def test_noalloc_fp32_and_limit():
    # float32 calls need no scratch; a call beyond the array is refused
    _both(synth.prefill_case(B=2, Nk=1, Nv=2, S=100, Dk=32, Dv=32, dtype="f32", base=473, lens=[100, 41],
                             chunk=32, scale=0.3, init_std=0.1))
    q = torch.zeros(4, 16, 4097, 128, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(4, 32, 4097, 128, dtype=torch.bfloat16, device="cuda")
    beta = torch.zeros(4, 32, 4097, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="scratch"):
        gdr.gdr_chunk_noalloc(q, q, v, beta)
