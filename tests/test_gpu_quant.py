"""Bit-exact parity of the HIP quantiser, double quantiser and dequantiser
with the CPU oracle (GPU)."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_22_amd as qn
from tests.gpu_helpers import (bf16_dev, f32_dev, nf4, oracle_quant, synth, to_bits16,
                               weight_dev, weight_f32)

pytestmark = pytest.mark.gpu


def _gpu_quant(W, dtype):
    w = weight_dev(W, dtype).reshape(-1)
    packed, absmax = qn.nf4_quantize(w)
    torch.cuda.synchronize()
    return packed.cpu().numpy(), absmax.cpu().numpy()


def _assert_quant_equal(W, dtype):
    gp, ga = _gpu_quant(W, dtype)
    op, oa = nf4.quantize_nf4(weight_f32(W, dtype))
    assert gp.shape == op.shape and ga.shape == oa.shape
    bad = np.nonzero(gp != op)[0]
    assert bad.size == 0, f"{bad.size} packed bytes differ, first at {bad[:5]}"
    assert np.array_equal(ga.view(np.uint32), oa.view(np.uint32))
    return gp, ga


def test_quantize_tiny_fp32_layer():
    wl = synth.tiny_layer(0)
    _assert_quant_equal(wl.W, "f32")


def test_quantize_decode_weight_bf16():
    wl = synth.decode_layer(1, 4096, 4096, seed=2)
    _assert_quant_equal(wl.W, "bf16")


@pytest.mark.parametrize("shape", [(11008, 4096), (4096, 11008)])
def test_quantize_student_t_training_weights(shape):
    wl = synth.train_linear(*shape, M=16, seed=3)
    _assert_quant_equal(wl.W, "bf16")


def _adversarial_f32(seed=0, nblocks=512):
    """Blocks whose normalised values sit on and around every threshold."""
    rng = np.random.default_rng(seed)
    thr = nf4.nf4_midpoints()
    out = np.zeros((nblocks, 64), np.float32)
    for b in range(nblocks):
        kind = b % 8
        c = np.float32(rng.uniform(0.001, 0.2))
        blk = np.zeros(64, np.float32)
        if kind <= 3:
            for i in range(1, 64):
                t = thr[rng.integers(0, 15)]
                base = np.float32(t * float(c))
                k = int(rng.integers(-6, 7))
                blk[i] = np.float32(base + np.float32(k) * np.spacing(base))
            blk[0] = c if kind % 2 == 0 else -c
        elif kind == 4:  # several elements tied at +-absmax
            blk[:] = rng.uniform(-1, 1, 64).astype(np.float32) * c
            blk[[3, 17, 40]] = [c, -c, c]
        elif kind == 5:  # subnormal block constant
            blk[:] = (rng.uniform(-1, 1, 64) * 1e-39).astype(np.float32)
        elif kind == 6:  # tiny but normal constant (< 2^-100)
            blk[:] = (rng.uniform(-1, 1, 64) * 1e-32).astype(np.float32)
        else:  # zeros and signed zeros, one large block
            blk[:] = 0.0
            if b % 16 == 7:
                blk[::2] = -0.0
            else:
                blk[:] = (rng.standard_normal(64) * 1e30).astype(np.float32)
        out[b] = blk
    return out.reshape(-1)


def test_quantize_adversarial_fp32():
    _assert_quant_equal(_adversarial_f32(0), "f32")


def test_quantize_adversarial_bf16():
    rng = np.random.default_rng(1)
    w = _adversarial_f32(1).reshape(-1, 64)
    bits = synth.bf16_bits(w)
    bits[-8:, :] = rng.integers(0, 0x80, size=(8, 64)).astype(np.uint16)  # bf16 subnormals
    bits[-8:, ::3] |= 0x8000
    _assert_quant_equal(bits.reshape(-1), "bf16")


@pytest.mark.parametrize("numel", [2, 64 * 37 + 10, 4098, 4096 * 3 + 62])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_ragged_tails(numel, dtype):
    rng = np.random.default_rng(numel)
    w = (rng.standard_normal(numel) * 0.02).astype(np.float32)
    W = w if dtype == "f32" else synth.bf16_bits(w)
    _assert_quant_equal(W, dtype)


def test_quantize_is_deterministic():
    wl = synth.decode_layer(1, 4096, 4096, seed=2)
    a = _gpu_quant(wl.W, "bf16")
    b = _gpu_quant(wl.W, "bf16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def _assert_dq_equal(absmax):
    q8, c2 = qn.dq_quantize_scales(f32_dev(absmax))
    torch.cuda.synchronize()
    oq, oc = nf4.double_quantize(absmax)
    assert np.array_equal(q8.cpu().numpy(), oq)
    assert np.array_equal(c2.cpu().numpy().view(np.uint32), oc.view(np.uint32))


def test_dq_on_training_weight_constants():
    wl = synth.train_linear(11008, 4096, M=16, seed=3)
    _, absmax = nf4.quantize_nf4(synth.bf16_to_f32(wl.W))
    _assert_dq_equal(absmax)


def test_dq_crafted_groups():
    rng = np.random.default_rng(5)
    c = np.abs(rng.standard_normal(256 * 6 + 77) * 0.05).astype(np.float32)
    c[256:512] = 0.0                       # zero group
    c[512] = 100.0                         # outlier forces small codes to 0
    lv = nf4.dq_levels().astype(np.float64)
    mids = (lv[:-1] + lv[1:]) / 2
    c[768] = 1.0                           # values on the level mid-points
    for i in range(769, 1024):
        m = mids[rng.integers(0, 255)]
        f = np.float32(m)
        k = int(rng.integers(-2, 3))
        c[i] = np.float32(f + np.float32(k) * np.spacing(f))
    _assert_dq_equal(c)


@pytest.mark.parametrize("double_quant", [True, False])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequant_bit_exact(double_quant, out_dtype):
    wl = synth.train_linear(4096, 11008, M=16, seed=3)
    ref = oracle_quant(wl.W, "bf16", double_quant)
    qw = qn.quantize_weight(bf16_dev(wl.W), double_quant=double_quant)
    out = qn.nf4_dequant(qw, out_dtype)
    torch.cuda.synchronize()
    if out_dtype == torch.float32:
        got = out.cpu().numpy().view(np.uint32)
        want = ref["What"].view(np.uint32)
    else:
        got = to_bits16(out)
        want = nf4.f32_to_bf16_bits(ref["What"])
    bad = np.count_nonzero(got != want)
    assert bad == 0, f"{bad} dequantised elements differ"


def test_dequant_keeps_signed_zeros():
    # A group whose outlier drives q8 = 0 for the other blocks: their
    # negative codes dequantise to -0.0.
    W = (np.random.default_rng(2).standard_normal((64, 256)) * 1e-3).astype(np.float32)
    W[0, 0] = 1e4
    ref = oracle_quant(W, "f32")
    assert np.any(ref["What"].view(np.uint32) == 0x80000000)
    qw = qn.quantize_weight(f32_dev(W))
    out = qn.nf4_dequant(qw, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref["What"].view(np.uint32))


def test_round_trip_is_idempotent_on_device():
    wl = synth.decode_layer(1, 4096, 4096, seed=2)
    qw = qn.quantize_weight(bf16_dev(wl.W))
    w1 = qn.nf4_dequant(qw, torch.float32)
    qw2 = qn.quantize_weight(w1)
    torch.cuda.synchronize()
    assert torch.equal(qw.qscale, qw2.qscale)
    assert torch.equal(qw.gscale, qw2.gscale)
    live = (qw.qscale > 0).repeat_interleave(32)
    assert torch.equal(qw.packed[live], qw2.packed[live])


@pytest.mark.parametrize("numel", [64, 4096 + 64 * 3, 16384, 16384 * 3 + 64 * 5 + 32, 4096 * 4096])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind,scale", [("nf4", "u8"), ("nf4", "fp8"), ("fp4", "u8")])
def test_fused_quantise_dq_equals_the_two_calls(numel, dtype, kind, scale):
    """nf4_quantize_dq (one launch per 256-block group) writes the same codes,
    block constants, level-2 codes and group maxima as the quantiser followed
    by the double quantiser, for sizes with partial blocks and partial groups,
    and both agree with the oracle."""
    rng = np.random.default_rng(numel)
    W = (rng.standard_t(5, numel) * 0.02).astype(np.float32)
    if dtype == "bf16":
        W = synth.bf16_bits(W)
    w = weight_dev(W, dtype).reshape(-1)
    quant = qn.fp4_quantize if kind == "fp4" else qn.nf4_quantize
    p1, a1 = quant(w)
    q1, g1 = qn.dq_quantize_scales(a1, fp8=scale == "fp8")
    a2 = torch.full_like(a1, float("nan"))
    p2, q2, g2 = qn.nf4_quantize_dq(w, kind, scale, absmax=a2)
    p3, q3, g3 = qn.nf4_quantize_dq(w, kind, scale)  # no absmax output
    torch.cuda.synchronize()
    for a, b in ((p1, p2), (q1, q2), (p1, p3), (q1, q3)):
        assert torch.equal(a, b)
    for a, b in ((a1, a2), (g1, g2), (g1, g3)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    if numel <= 16384 * 4:
        from oracle import codebooks
        op, oa = codebooks.quantize_4bit(weight_f32(W, dtype), kind)
        oq, og = (codebooks.double_quantize_fp8(oa) if scale == "fp8"
                  else nf4.double_quantize(oa))
        assert np.array_equal(p2.cpu().numpy(), op)
        assert np.array_equal(q2.cpu().numpy(), oq)
        assert np.array_equal(g2.cpu().numpy().view(np.uint32), og.view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind,scale", [("nf4", "u8"), ("nf4", "fp8"), ("fp4", "u8")])
def test_batched_quantise_dq_equals_one_call_per_weight(dtype, kind, scale):
    """nf4_quantize_dq_batch over eight weights in one launch (sizes with
    partial blocks and groups, one empty, whole-group and multi-group ones)
    writes the bytes of eight nf4_quantize_dq calls, bit for bit, with and
    without block-constant outputs for some entries; the batch of one and
    the small entries also against the oracle."""
    sizes = [64, 4096 + 64 * 3, 0, 16384, 16384 * 3 + 64 * 5 + 32, 1000, 4096 * 1024, 256 * 258]
    ws, Ws = [], []
    for i, n in enumerate(sizes):
        rng = np.random.default_rng(4200 + i)
        W = (rng.standard_t(5, n) * 0.02).astype(np.float32)
        if dtype == "bf16":
            W = synth.bf16_bits(W)
        Ws.append(W)
        ws.append(weight_dev(W, dtype).reshape(-1))
    nb = [-(-n // 64) for n in sizes]
    am = [torch.full((b,), float("nan"), device="cuda:0") if i % 2 == 0 else None
          for i, b in enumerate(nb)]
    got = qn.nf4_quantize_dq_batch(ws, kind, scale, absmax=am)
    one = qn.nf4_quantize_dq_batch(ws[1:2], kind, scale)
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        a1 = torch.full((nb[i],), float("nan"), device="cuda:0")
        p1, q1, g1 = qn.nf4_quantize_dq(w, kind, scale, absmax=a1 if am[i] is not None else None)
        torch.cuda.synchronize()
        p2, q2, g2 = got[i]
        assert torch.equal(p1, p2) and torch.equal(q1, q2), f"entry {i}"
        assert torch.equal(g1.view(torch.int32), g2.view(torch.int32)), f"entry {i}"
        if am[i] is not None:
            assert torch.equal(a1.view(torch.int32), am[i].view(torch.int32)), f"entry {i}"
    from oracle import codebooks
    for i in (0, 1, 5):
        op, oa = codebooks.quantize_4bit(weight_f32(Ws[i], dtype), kind)
        oq, og = (codebooks.double_quantize_fp8(oa) if scale == "fp8"
                  else nf4.double_quantize(oa))
        p, q, g = got[i]
        assert np.array_equal(p.cpu().numpy(), op)
        assert np.array_equal(q.cpu().numpy(), oq)
        assert np.array_equal(g.cpu().numpy().view(np.uint32), og.view(np.uint32))
    for a, b in zip(one[0], got[1]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_quantize_weights_matches_quantize_weight():
    """quantize_weights (batches of up to 8 per launch) gives the weights
    quantize_weight gives one by one: nine 7B-like projections, so two
    launches."""
    rng = np.random.default_rng(77)
    shapes = [(256, 512)] * 4 + [(704, 256)] * 2 + [(256, 704)] * 3
    ws = [weight_dev(synth.bf16_bits((rng.standard_normal(s) * 0.02).astype(np.float32)),
                     "bf16").reshape(s) for s in shapes]
    got = qn.quantize_weights(ws)
    torch.cuda.synchronize()
    for w, g in zip(ws, got):
        want = qn.quantize_weight(w)
        torch.cuda.synchronize()
        assert (g.N, g.K) == (want.N, want.K)
        assert torch.equal(g.packed, want.packed) and torch.equal(g.qscale, want.qscale)
        assert torch.equal(g.gscale.view(torch.int32), want.gscale.view(torch.int32))
