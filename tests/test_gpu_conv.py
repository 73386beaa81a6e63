"""GPU parity of the depthwise causal conv1d + SiLU and its q/k/v split
against the float64 oracle (oracle.conv; the blog post's layer code and
inferencelayer deltanet.rs's conv ring).

Outputs: within the bars of the recurrence (max-abs 2e-2 for bf16 I/O,
1e-4 for float32; the conv sums K float32 products and rounds once), exact
zeros past each length. States: the carried states hold raw inputs, so they
must match bit for bit; untouched pool slots stay bit-identical."""
import numpy as np
import pytest
import torch

import synth
from oracle import conv as oracle_conv
from tests.gpu_util import TOL, raw_bits, say, to_dev, to_f64
import gated_deltanet_recurrence_amd as gdr

pytestmark = pytest.mark.gpu


def _check_qkv(q, k, v, y_ref, heads, L, dtype):
    Nk, Dk, Nv, Dv = heads
    rq, rk, rv = oracle_conv.split(y_ref, Nk, Dk, Nv, Dv)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        g = to_f64(got)
        for b in range(g.shape[0]):
            n = int(L[b])
            if n:
                e = float(np.abs(g[b, :, :n] - ref[b, :, :n]).max())
                assert e <= TOL[dtype], f"{name} b={b} err {e}"
            assert torch.all(raw_bits(got[b, :, n:]) == 0), f"{name} b={b}: nonzero rows past the length"


def _prefill(B, S, heads, K, dtype, base, lens=None, init=True, bias=True, alias=False, poison=True):
    Nk, Dk, Nv, Dv = heads
    C = 2 * Nk * Dk + Nv * Dv
    x, w, bb, st = synth.conv_inputs(base, B, S, C, K, dtype)
    L = np.full(B, S) if lens is None else np.clip(np.asarray(lens), 0, S)
    if poison:
        nanv = synth.BF16_NAN if dtype == "bf16" else np.float32(np.nan)
        for b in range(B):
            x[b, int(L[b]):] = nanv
    say(f"gdr_conv_prefill {dtype} B={B} S={S} heads={heads} K={K} lens={None if lens is None else list(L)} "
        f"init={init} bias={bias} alias={alias}")
    init_d = to_dev(st) if init else None
    q, k, v, fin = gdr.gdr_conv_prefill(to_dev(x), to_dev(w), heads, bias=to_dev(bb) if bias else None,
                                        initial_state=init_d, final_state=init_d if alias else None,
                                        actual_seq_lengths=None if lens is None else to_dev(np.asarray(L, np.int32)))
    torch.cuda.synchronize()
    y_ref, f_ref = oracle_conv.prefill(np.nan_to_num(synth.widen(x, dtype)), w, bb if bias else None,
                                       synth.widen(st, dtype) if init else None, L)
    _check_qkv(q, k, v, y_ref, heads, L, dtype)
    assert np.array_equal(to_f64(fin), f_ref), "final state"


def test_conv_prefill_bf16():
    # several token blocks, ragged tails and an empty sequence; NaN past the lengths
    _prefill(3, 300, (2, 128, 4, 128), 4, "bf16", 811, lens=[300, 129, 0])


def test_conv_prefill_fp32_and_taps():
    _prefill(2, 100, (1, 16, 2, 16), 3, "f32", 812, lens=[100, 37])
    _prefill(2, 70, (1, 16, 1, 32), 1, "f32", 813, init=False)            # K = 1: no state
    _prefill(2, 70, (1, 32, 2, 16), 8, "bf16", 814, lens=[70, 5])          # K = 8, a length below K - 1


def test_conv_prefill_pair_kernel():
    # head sizes even but not multiples of 8: the waves' lanes straddle head
    # boundaries, so one store instruction writes to several planes
    _prefill(2, 150, (1, 10, 2, 6), 3, "f32", 817, lens=[150, 65])
    _prefill(2, 80, (2, 6, 2, 10), 4, "bf16", 818, lens=[80, 1])


def test_conv_prefill_mixed_head_sizes():
    # key and value heads of different sizes, in bf16 and fp16, with K = 4 and 2
    _prefill(2, 97, (1, 12, 3, 20), 4, "bf16", 819, lens=[97, 33])
    _prefill(2, 66, (2, 4, 2, 12), 2, "f16", 820, lens=[3, 66])


def test_conv_prefill_saturated_silu():
    # Inputs and states scaled by 256 (exact in every format): pre-activations
    # reach several hundred, beyond where e^-u is finite in float32, so SiLU
    # must give u for large u and a zero for very negative u. The outputs are
    # large, so the bar adds one rounding of the output (2^-8 |y| for bf16,
    # 2^-24 for float32) and the float32 accumulation of the K taps
    # (K 2^-23 (sum_j |w_j| max|x| + |bias|)) to the absolute bar.
    heads = (1, 16, 2, 16)
    Nk, Dk, Nv, Dv = heads
    C, B, S, K = 2 * Nk * Dk + Nv * Dv, 2, 70, 4
    for dtype, rel in (("bf16", 2.0 ** -8), ("f32", 2.0 ** -24)):
        x, w, bb, st = synth.conv_inputs(831, B, S, C, K, dtype)
        xs, ss = synth.widen(x, dtype) * 256.0, synth.widen(st, dtype) * 256.0
        if dtype == "bf16":
            x, st = synth.bf16_bits(xs), synth.bf16_bits(ss)
        else:
            x, st = xs.astype(np.float32), ss.astype(np.float32)
        L = np.array([S, 41], np.int32)
        say(f"gdr_conv_prefill {dtype} B={B} S={S} heads={heads} K={K}, inputs x256")
        q, k, v, fin = gdr.gdr_conv_prefill(to_dev(x), to_dev(w), heads, bias=to_dev(bb), initial_state=to_dev(st),
                                            actual_seq_lengths=to_dev(L))
        torch.cuda.synchronize()
        y_ref, f_ref = oracle_conv.prefill(synth.widen(x, dtype), w, bb, synth.widen(st, dtype), L)
        m = max(float(np.abs(xs).max()), float(np.abs(ss).max()))
        acc = K * 2.0 ** -23 * (np.abs(w).sum(1) * m + np.abs(bb))   # per channel
        saturated = 0
        for name, got, ref, a in zip(("q", "k", "v"), (q, k, v),
                                     oracle_conv.split(y_ref, Nk, Dk, Nv, Dv),
                                     oracle_conv.split(np.broadcast_to(acc, (1, 1, C)), Nk, Dk, Nv, Dv)):
            g = to_f64(got)
            for b in range(B):
                n = int(L[b])
                r = ref[b, :, :n]
                bound = TOL[dtype] + rel * np.abs(r) + a[0]
                assert np.all(np.abs(g[b, :, :n] - r) <= bound), f"{dtype} {name} b={b}"
                saturated += int((np.abs(r) > 89.0).sum())
                assert torch.all(raw_bits(got[b, :, n:]) == 0), f"{name} b={b}: nonzero rows past the length"
        assert saturated > 0, "no pre-activation beyond the float32 range of e^-u"
        assert np.array_equal(to_f64(fin), f_ref), "final state"


def test_conv_prefill_no_state_no_bias_and_alias():
    _prefill(2, 130, (2, 64, 2, 64), 4, "bf16", 815, init=False, bias=False)
    _prefill(3, 90, (2, 64, 4, 64), 4, "bf16", 816, lens=[90, 2, 64], alias=True)


def _decode(B, S, heads, K, dtype, base, slots, lens, n_acc, idx_mode):
    Nk, Dk, Nv, Dv = heads
    C = 2 * Nk * Dk + Nv * Dv
    x, w, bb, pool = synth.conv_inputs(base, B, S, C, K, dtype, slots=slots)
    rng = np.random.default_rng([base, 7])
    L = np.asarray(lens, np.int32)
    na = None if n_acc is None else np.asarray(n_acc, np.int32)
    if idx_mode == "per_token":
        idx = rng.permutation(slots)[:B * S].astype(np.int32)
    else:   # one slot per sequence, repeated over its positions
        idx = np.repeat(rng.permutation(slots)[:B], S).astype(np.int32)
    say(f"gdr_conv_decode {dtype} B={B} S={S} heads={heads} K={K} slots={slots} idx={idx_mode}")
    pool_d = to_dev(pool)
    q, k, v, pool_out = gdr.gdr_conv_decode(to_dev(x), to_dev(w), heads, pool_d, to_dev(L), to_dev(idx),
                                            bias=to_dev(bb), num_accepted_tokens=None if na is None else to_dev(na))
    torch.cuda.synchronize()
    y_ref, p_ref = oracle_conv.decode(synth.widen(x, dtype), w, bb, synth.widen(pool, dtype), L, idx, na)
    Lc = np.clip(L, 0, S)
    for b in range(B):   # skipped sequences write zeros
        n = int(Lc[b]) if na is None else int(na[b])
        if Lc[b] == 0 or n < 1 or n > S or not 0 <= idx[b * S + n - 1] < slots:
            Lc[b] = 0
    _check_qkv(q, k, v, y_ref, heads, Lc, dtype)
    assert np.array_equal(to_f64(pool_out), p_ref), "pool"


def test_conv_decode_one_token():
    B = 24
    _decode(B, 1, (2, 128, 4, 128), 4, "bf16", 821, slots=32, lens=[1] * (B - 2) + [0, 1], n_acc=None,
            idx_mode="per_seq")


def test_conv_decode_multi_token():
    rng = np.random.default_rng(822)
    B, S = 20, 4
    lens = rng.integers(1, S + 1, B)
    n_acc = np.minimum(rng.integers(1, S + 1, B), lens)
    _decode(B, S, (2, 128, 4, 128), 4, "bf16", 822, slots=B * S + 8, lens=lens, n_acc=n_acc, idx_mode="per_token")
    _decode(B, S, (1, 16, 2, 16), 3, "f32", 823, slots=B + 4, lens=lens, n_acc=None, idx_mode="per_seq")


def test_conv_workloads_full_size():
    # The launch configurations bench.py times: C = 2 Nk Dk + Nv Dv = 8192
    # channels (Nk = 16, Dk = 128, Nv = 32, Dv = 128), K = 4, bf16, bias and
    # carried state; prefill of 4 x 4096 tokens and a one-token step of 64
    # sequences over a 64-slot pool. The conv oracle is cheap enough to run
    # whole at these sizes.
    heads = (16, 128, 32, 128)
    _prefill(4, 4096, heads, 4, "bf16", 505, poison=False)
    _decode(64, 1, heads, 4, "bf16", 505, slots=64, lens=[1] * 64, n_acc=None, idx_mode="per_seq")
