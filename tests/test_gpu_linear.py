"""GPU parity of the training modules on the C ABI (Fp8Linear, Fp8Mlp) and of their fp8 weight cache.

One forward + backward step is compared with the oracle call by call: every library call's inputs
are taken from what the GPU actually fed it (the module keeps its fp8 intermediates when asked), the
oracle computes that call's result from them, and the GPU's output is held to the tolerance of that
call (casts bit-exact, bf16 outputs within the bf16 rule, fp32 within the fp32 rules).  Composing
per call keeps a rounding difference in one call (a bf16 output one ulp off, which moves an fp8
code downstream) from being charged to the next.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import (GELU_CHAIN, GELU_LIP, bf16_host_f64, chain_colsum, chain_gemm, chain_rowsum,
                    check_bf16, check_f32, host, shost)

te = pytest.importorskip("fp8_linear_layer_amd")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    te.load_library()
    global lin
    from fp8_linear_layer_amd import linear as lin


def bits(t):
    return host(t.detach()).view(torch.int16).numpy().view(np.uint16)


def bf16_in(seed, shape, std):
    return torch.from_numpy(W.normal_bf16(np.random.SeedSequence(seed), shape, std)).view(torch.bfloat16).cuda()


def check_cast_transpose(q, s, qt, st, x_bits, fmt, what, pow2=False):
    """The library's cast-transpose of x equals the oracle's cast of x and of x^T, bit for bit."""
    oq, os_, oqt, ost = oracle.cast_per_token_transpose(x_bits, fmt, pow2)
    rows, cols = x_bits.shape
    assert np.array_equal(host(q).numpy(), oq), f"{what}: row-wise codes"
    assert np.array_equal(shost(s, rows).view(np.uint32), os_.view(np.uint32)), f"{what}: row-wise scales"
    assert np.array_equal(host(qt).numpy(), oqt), f"{what}: transposed codes"
    assert np.array_equal(shost(st, cols).view(np.uint32), ost.view(np.uint32)), f"{what}: transposed scales"
    return oq, os_, oqt, ost


def op(q, s, rows):
    return host(q).numpy(), shost(s, rows)


E4, E5 = oracle.E4M3, oracle.E5M2


@pytest.mark.parametrize("pow2", [False, True], ids=["ieee", "pow2"])
def test_fp8_linear_step_matches_oracle_per_call_and_caches_the_weight(pow2):
    """pow2: the forward operands with power-of-two scales and the forward GEMM on FAST (chained)."""
    M, K, N = 256, 384, 256
    g = torch.Generator(device="cuda").manual_seed(5)
    m = lin.Fp8Linear(K, N, bias=True, generator=g, pow2_scales=pow2)
    with torch.no_grad():
        m.bias.copy_(bf16_in(1, (N,), 0.1))
    m.keep = {}
    mg_prev = np.zeros((N, K))
    for step in range(2):                         # two micro-batches: the weight is cast once
        x = bf16_in(10 + step, (M, K), 1.0)
        dy = bf16_in(20 + step, (M, N), 1e-2)
        y = m(x)
        y.backward(dy)
        torch.cuda.synchronize()
        k = m.keep
        qx, sx, qxt, sxt = check_cast_transpose(k["qx"], k["sx"], k["qxt"], k["sxt"], bits(x), E4, "x", pow2)
        qw, sw, qwt, swt = check_cast_transpose(*m.cache.get(m.weight), bits(m.weight), E4, "W", pow2)
        o, d = oracle.gemm_nt(qx, sx, E4, qw, sw, E4)
        yo, _, zm = oracle.fwd_epilogue(o, d, bits(m.bias))
        check_bf16(bf16_host_f64(y), yo, zm, "linear y")
        qdy, sdy, qdyt, sdyt = check_cast_transpose(k["qdy"], k["sdy"], k["qdyt"], k["sdyt"], bits(dy), E5, "dy")
        o, d = oracle.gemm_nt(qdyt, sdyt, E5, qxt, sxt, E4)
        want, mag = oracle.wgrad(o, d, mg_prev.astype(np.float32))
        mg = host(m.weight.main_grad).numpy()
        check_f32(mg, want, mag, "linear dW (main_grad +=)", chain_gemm(M, 1 + step))
        assert m.weight.grad is None
        db, dbm = oracle.operand_row_sums(qdyt, sdyt, E5)
        check_f32(host(k["db32"]).numpy(), db, dbm, "linear db", chain_rowsum(M), mma=False)
        assert torch.equal(host(m.bias.grad).view(torch.int16), host(k["db32"]).to(torch.bfloat16).view(torch.int16))
        mg_prev = mg.astype(np.float64)
        m.bias.grad = None
    assert m.cache.casts == 1, "the weight was re-cast between micro-batches"
    # an in-place update (as an optimizer step makes) bumps the version: the next pass re-casts
    with torch.no_grad():
        m.weight.mul_(0.5)
    m(bf16_in(30, (M, K), 1.0))
    assert m.cache.casts == 2
    check_cast_transpose(*m.cache.get(m.weight), bits(m.weight), E4, "W after update", pow2)


def test_fp8_linear_input_gradient():
    M, K, N = 384, 256, 512
    g = torch.Generator(device="cuda").manual_seed(7)
    m = lin.Fp8Linear(K, N, bias=False, generator=g)
    m.keep = {}
    x = bf16_in(40, (M, K), 1.0).requires_grad_(True)
    dy = bf16_in(41, (M, N), 1e-2)
    m(x).backward(dy)
    torch.cuda.synchronize()
    k = m.keep
    qdy, sdy = op(k["qdy"], k["sdy"], M)
    _, _, qwt, swt = m.cache.get(m.weight)
    o, d = oracle.gemm_nt(qdy, sdy, E5, *op(qwt, swt, K), E4)
    check_bf16(bf16_host_f64(x.grad), o, d, "linear dx")
    o, d = oracle.gemm_nt(*op(k["qdyt"], k["sdyt"], N), E5, *op(k["qxt"], k["sxt"], K), E4)
    want, mag = oracle.wgrad(o, d, np.zeros((N, K), np.float32))
    check_f32(host(m.weight.main_grad).numpy(), want, mag, "linear dW", chain_gemm(M, 1))


@pytest.mark.parametrize("pow2", [False, True], ids=["ieee", "pow2"])
def test_fp8_mlp_step_matches_oracle_per_call(pow2):
    """pow2: x, h, W1 and W2 cast with power-of-two scales, both forward GEMMs on FAST (chained);
    the gradients keep IEEE scales."""
    M, K, H, N = 256, 256, 512, 384
    g = torch.Generator(device="cuda").manual_seed(9)
    m = lin.Fp8Mlp(K, H, N, generator=g, pow2_scales=pow2)
    with torch.no_grad():
        m.b1.copy_(bf16_in(2, (H,), 0.1))
        m.b2.copy_(bf16_in(3, (N,), 0.1))
    m.keep = {}
    x = bf16_in(50, (M, K), 1.0).requires_grad_(True)
    dy = bf16_in(51, (M, N), 1e-2)
    y = m(x)
    y.backward(dy)
    torch.cuda.synchronize()
    k = m.keep
    qx, sx, qxt, sxt = check_cast_transpose(k["qx"], k["sx"], k["qxt"], k["sxt"], bits(x), E4, "x", pow2)
    qw1, sw1, qw1t, sw1t = check_cast_transpose(*m.c1.get(m.w1), bits(m.w1), E4, "W1", pow2)
    qw2, sw2, qw2t, sw2t = check_cast_transpose(*m.c2.get(m.w2), bits(m.w2), E4, "W2", pow2)
    # fc1 forward: h = GELU(z), z saved
    o, d = oracle.gemm_nt(qx, sx, E4, qw1, sw1, E4)
    h, z, zm = oracle.fwd_epilogue(o, d, bits(m.b1), True)
    check_bf16(bf16_host_f64(k["h"]), h, zm * GELU_LIP, "mlp h")
    check_bf16(bf16_host_f64(k["z1"]), z, zm, "mlp z1")
    # fc2 forward on the GPU's own h
    qh, sh, qht, sht = check_cast_transpose(k["qh"], k["sh"], k["qht"], k["sht"], bits(k["h"]), E4, "h", pow2)
    o, d = oracle.gemm_nt(qh, sh, E4, qw2, sw2, E4)
    yo, _, ym = oracle.fwd_epilogue(o, d, bits(m.b2))
    check_bf16(bf16_host_f64(y), yo, ym, "mlp y")
    # backward: fc2 weight and bias gradients
    qdy, sdy, qdyt, sdyt = check_cast_transpose(k["qdy"], k["sdy"], k["qdyt"], k["sdyt"], bits(dy), E5, "dy")
    o, d = oracle.gemm_nt(qdyt, sdyt, E5, qht, sht, E4)
    want, mag = oracle.wgrad(o, d, np.zeros((N, H), np.float32))
    check_f32(host(m.w2.main_grad).numpy(), want, mag, "mlp dW2", chain_gemm(M, 1))
    db2, db2m = oracle.operand_row_sums(qdyt, sdyt, E5)
    check_f32(host(k["db2_32"]).numpy(), db2, db2m, "mlp db2", chain_rowsum(M), mma=False)
    # fc2 data gradient through fc1's GELU (on the GPU's own z1) with fc1's bias gradient
    o, d = oracle.gemm_nt(qdy, sdy, E5, qw2t, sw2t, E4)
    D, Dm, db1, db1m = oracle.dgrad_epilogue(o, d, bits(k["z1"]), bgrad=True)
    check_bf16(bf16_host_f64(k["dz1"]), D, Dm, "mlp dz1")
    check_f32(host(k["db1_32"]).numpy(), db1, db1m, "mlp db1", chain_colsum(N, M, GELU_CHAIN))
    assert torch.equal(host(m.b1.grad).view(torch.int16), host(k["db1_32"]).to(torch.bfloat16).view(torch.int16))
    # fc1 weight gradient and the input gradient, on the GPU's own dz1
    qdz, sdz, qdzt, sdzt = check_cast_transpose(k["qdz"], k["sdz"], k["qdzt"], k["sdzt"], bits(k["dz1"]), E5, "dz1")
    o, d = oracle.gemm_nt(qdzt, sdzt, E5, qxt, sxt, E4)
    want, mag = oracle.wgrad(o, d, np.zeros((H, K), np.float32))
    check_f32(host(m.w1.main_grad).numpy(), want, mag, "mlp dW1", chain_gemm(M, 1))
    o, d = oracle.gemm_nt(qdz, sdz, E5, qw1t, sw1t, E4)
    check_bf16(bf16_host_f64(x.grad), o, d, "mlp dx")
    assert m.c1.casts == 1 and m.c2.casts == 1
