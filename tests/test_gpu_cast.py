"""GPU parity of te_cast_fp8_per_token: fp8 codes and fp32 scales bit-identical to the oracle."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import bf16_dev, host, scale_ld, shost

te = pytest.importorskip("fp8_linear_layer_amd")
pytestmark = pytest.mark.gpu

FMT = {te.TE_DTYPE_E4M3: oracle.E4M3, te.TE_DTYPE_E5M2: oracle.E5M2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    te.load_library()


def gpu_cast(bits, dt, pow2, ld_x=None, ld_q=None):
    rows, cols = bits.shape
    ld_x = ld_x or cols
    ld_q = ld_q or cols
    xb = np.zeros((rows, ld_x), np.uint16)
    xb[:, :cols] = bits
    x = bf16_dev(xb)[:, :cols]
    qfull = torch.full((rows, ld_q), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((cols // 128, scale_ld(rows)), -7.0, dtype=torch.float32, device="cuda")
    te.te_cast_fp8_per_token(x, dt, te.TE_CAST_POW2_SCALE if pow2 else 0, q=qfull[:, :cols], scales=s)
    torch.cuda.synchronize()
    qh = host(qfull).numpy()
    assert (qh[:, cols:] == 0xA5).all(), "cast wrote past cols"
    sh = host(s).numpy()
    assert (sh[:, rows:] == -7.0).all(), "cast wrote into the scale padding"
    return qh[:, :cols], shost(s, rows)


def assert_same(bits, dt, pow2, **kw):
    q, s = gpu_cast(bits, dt, pow2, **kw)
    qo, so = oracle.cast_per_token(bits, FMT[dt], pow2)
    bad = np.argwhere(q != qo)
    assert bad.size == 0, f"{len(bad)} code mismatches, first {bad[0]}: gpu {q[tuple(bad[0])]:#x} oracle {qo[tuple(bad[0])]:#x}"
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), "scale mismatch"


def special_rows(dt):
    """Rows of edge-case groups: zeros, subnormals, tiny amax, huge values, midpoints, signed zeros."""
    fmax = oracle.fp8_max(FMT[dt])
    rows = []
    rows.append(np.zeros(128, np.float32))
    r = np.zeros(128, np.float32); r[5] = -0.0; r[6] = 1e-40; r[7] = -3e-39; rows.append(r)      # subnormal bf16
    rows.append(np.float32(2.0 ** -110) * np.arange(-64, 64, dtype=np.float32))                   # amax below the floor
    rows.append(np.float32(1e-36) * np.linspace(-1, 1, 128, dtype=np.float32))
    rows.append(np.float32(3e38) * np.linspace(-1, 1, 128, dtype=np.float32))                      # near fp32 max
    r = np.full(128, 1.0625, np.float32); r[0] = fmax; rows.append(r)                               # ties at scale 1
    r = np.linspace(-fmax, fmax, 128, dtype=np.float32); rows.append(r)
    r = np.full(128, -0.0, np.float32); r[3] = 2.0 ** -133; rows.append(r)                        # smallest bf16 subnormal
    rng = np.random.default_rng(3)
    r = (rng.standard_normal(128) * 10.0 ** rng.uniform(-30, 30, 128)).astype(np.float32); rows.append(r)
    return W.f32_to_bf16_bits(np.stack(rows))


@pytest.mark.parametrize("dt", [te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2])
@pytest.mark.parametrize("pow2", [False, True])
def test_cast_edge_groups(dt, pow2):
    bits = special_rows(dt)
    # pad to 256 columns with a normal group so rows also span two groups
    extra = W.normal_bf16(np.random.SeedSequence(1), (bits.shape[0], 128))
    assert_same(np.concatenate([bits, extra], axis=1), dt, pow2)


@pytest.mark.parametrize("dt", [te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2])
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("rows,cols,ldx,ldq", [(1, 128, None, None), (5, 384, 392, 400), (37, 1024, 1152, 1040),
                                               (1000, 640, None, None)])
def test_cast_shapes_and_strides(dt, pow2, rows, cols, ldx, ldq):
    bits = W.normal_bf16(np.random.SeedSequence(rows * 7 + cols), (rows, cols), 0.3)
    assert_same(bits, dt, pow2, ld_x=ldx, ld_q=ldq)


@pytest.mark.parametrize("name,shape,std,dt", [
    ("dense-wgrad A", (7168, 4096), 1.0, te.TE_DTYPE_E4M3),
    ("dense-wgrad B", (2112, 4096), 1.0, te.TE_DTYPE_E4M3),
    ("fprop W", (14336, 4096), 0.02, te.TE_DTYPE_E4M3),
    ("dgrad dZ", (8192, 14336), 1e-3, te.TE_DTYPE_E5M2),
])
def test_cast_workload_sizes(name, shape, std, dt):
    bits = W.normal_bf16(np.random.SeedSequence(zlib.crc32(name.encode())), shape, std)
    assert_same(bits, dt, False)
    assert_same(bits[:512], dt, True)


def test_cast_is_deterministic():
    bits = W.normal_bf16(np.random.SeedSequence(9), (256, 1024))
    a = gpu_cast(bits, te.TE_DTYPE_E4M3, False)
    b = gpu_cast(bits, te.TE_DTYPE_E4M3, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------ fused cast-transpose
def gpu_cast_t(bits, dt, pow2, rowwise=True, ld_x=None, ld_q=None, ld_qt=None):
    rows, cols = bits.shape
    ld_x, ld_q, ld_qt = ld_x or cols, ld_q or cols, ld_qt or rows
    xb = np.zeros((rows, ld_x), np.uint16)
    xb[:, :cols] = bits
    x = bf16_dev(xb)[:, :cols]
    qfull = torch.full((rows, ld_q), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((cols // 128, scale_ld(rows)), -7.0, dtype=torch.float32, device="cuda")
    qtfull = torch.full((cols, ld_qt), 0x5A, dtype=torch.uint8, device="cuda")
    st = torch.full((rows // 128, scale_ld(cols)), -9.0, dtype=torch.float32, device="cuda")
    te.te_cast_fp8_per_token_transpose(x, dt, te.TE_CAST_POW2_SCALE if pow2 else 0, rowwise=rowwise,
                                       q=qfull[:, :cols] if rowwise else None, scales=s if rowwise else None,
                                       qt=qtfull[:, :rows], scales_t=st)
    torch.cuda.synchronize()
    qh, sh, qth, sth = host(qfull).numpy(), host(s).numpy(), host(qtfull).numpy(), host(st).numpy()
    assert (qth[:, rows:] == 0x5A).all(), "cast-transpose wrote past rows"
    assert (sth[:, cols:] == -9.0).all(), "cast-transpose wrote into the transposed scale padding"
    if not rowwise:
        assert (qh == 0xA5).all() and (sh == -7.0).all(), "row-wise outputs written although not requested"
        return None, None, qth[:, :rows], shost(st, cols)
    assert (qh[:, cols:] == 0xA5).all() and (sh[:, rows:] == -7.0).all()
    return qh[:, :cols], shost(s, rows), qth[:, :rows], shost(st, cols)


def assert_same_t(bits, dt, pow2, rowwise=True, **kw):
    q, s, qt, st = gpu_cast_t(bits, dt, pow2, rowwise, **kw)
    qo, so, qto, sto = oracle.cast_per_token_transpose(bits, FMT[dt], pow2)
    bad = np.argwhere(qt != qto)
    assert bad.size == 0, f"{len(bad)} transposed code mismatches, first {bad[0]}"
    assert np.array_equal(st.view(np.uint32), sto.view(np.uint32)), "transposed scale mismatch"
    if rowwise:
        bad = np.argwhere(q != qo)
        assert bad.size == 0, f"{len(bad)} row-wise code mismatches, first {bad[0]}"
        assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), "row-wise scale mismatch"


@pytest.mark.parametrize("dt", [te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2])
@pytest.mark.parametrize("pow2", [False, True])
def test_cast_transpose_edge_groups(dt, pow2):
    # the edge-case groups as columns (transposed direction) next to normal data
    sp = special_rows(dt)                                           # [9, 128]
    extra = W.normal_bf16(np.random.SeedSequence(2), (128, 128 - sp.shape[0]))
    assert_same_t(np.ascontiguousarray(np.concatenate([sp.T, extra], axis=1)), dt, pow2)
    # and as rows (row-wise direction)
    sp2 = np.concatenate([sp, W.normal_bf16(np.random.SeedSequence(3), (128 - sp.shape[0], 128))], axis=0)
    assert_same_t(np.ascontiguousarray(np.concatenate([sp2, sp2[::-1]], axis=1)), dt, pow2)


@pytest.mark.parametrize("dt", [te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2])
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("rowwise", [True, False])
@pytest.mark.parametrize("rows,cols,ldx,ldq,ldqt", [(128, 128, None, None, None), (256, 384, None, None, None),
                                                    (384, 1024, 1152, 1040, 400), (1024, 640, 648, None, 1040)])
def test_cast_transpose_shapes_and_strides(dt, pow2, rowwise, rows, cols, ldx, ldq, ldqt):
    bits = W.normal_bf16(np.random.SeedSequence(rows * 11 + cols), (rows, cols), 0.3)
    assert_same_t(bits, dt, pow2, rowwise, ld_x=ldx, ld_q=ldq, ld_qt=ldqt)


@pytest.mark.parametrize("dt", [te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2])
@pytest.mark.parametrize("rows,cols,ldx,ldqt", [(128, 8, None, None), (256, 200, 208, None), (384, 1064, 1072, 400)])
def test_cast_transpose_ragged_columns(dt, rows, cols, ldx, ldqt):
    """Without the row-wise cast the column count needs only be a multiple of 8: the last tile
    column is partial."""
    bits = W.normal_bf16(np.random.SeedSequence(rows * 13 + cols), (rows, cols), 0.3)
    assert_same_t(bits, dt, False, rowwise=False, ld_x=ldx, ld_qt=ldqt)


@pytest.mark.parametrize("name,shape,std,dt", [
    ("dense-wgrad dY (tokens x out)", (4096, 7168), 1.0, te.TE_DTYPE_E4M3),
    ("dense-wgrad X (tokens x in)", (4096, 2112), 1.0, te.TE_DTYPE_E4M3),
    ("fprop X (tokens x in)", (8192, 4096), 1.0, te.TE_DTYPE_E4M3),
])
def test_cast_transpose_workload_sizes(name, shape, std, dt):
    bits = W.normal_bf16(np.random.SeedSequence(zlib.crc32(name.encode())), shape, std)
    assert_same_t(bits, dt, False, rowwise=shape[1] % 128 == 0)


@pytest.mark.parametrize("dt", [te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2])
@pytest.mark.parametrize("pow2", [False, True])
def test_cast_batch_matches_the_oracle_per_operand(dt, pow2):
    """One launch over operands of different shapes and strides: each result bit-identical to the
    oracle's cast of that operand; nothing written outside any of them."""
    shapes = [(37, 384, 392, 400), (300, 128, None, None), (1, 1024, 1152, 1040), (513, 640, None, 656)]
    xs, bufs, ss, bits_all = [], [], [], []
    for i, (rows, cols, ldx, ldq) in enumerate(shapes):
        ldx, ldq = ldx or cols, ldq or cols
        bits = W.normal_bf16(np.random.SeedSequence(500 + i), (rows, cols), 0.3 + i)
        xb = np.zeros((rows, ldx), np.uint16)
        xb[:, :cols] = bits
        xs.append(bf16_dev(xb)[:, :cols])
        bufs.append(torch.full((rows, ldq), 0xA5, dtype=torch.uint8, device="cuda"))
        ss.append(torch.full((cols // 128, scale_ld(rows)), -7.0, dtype=torch.float32, device="cuda"))
        bits_all.append(bits)
    te.te_cast_fp8_per_token_batch(xs, dt, te.TE_CAST_POW2_SCALE if pow2 else 0,
                                   qs=[b[:, :x.shape[1]] for b, x in zip(bufs, xs)], scales=ss)
    torch.cuda.synchronize()
    for (rows, cols, _, _), bits, qb, sb in zip(shapes, bits_all, bufs, ss):
        qh, sh = host(qb).numpy(), host(sb).numpy()
        assert (qh[:, cols:] == 0xA5).all() and (sh[:, rows:] == -7.0).all()
        qo, so = oracle.cast_per_token(bits, FMT[dt], pow2)
        assert np.array_equal(qh[:, :cols], qo)
        assert np.array_equal(shost(sb, rows).view(np.uint32), so.view(np.uint32))


def test_cast_batch_wgrad_operands():
    """The dense weight gradient's two operands (7168 x 4096 and 2112 x 4096) in one launch."""
    a = W.normal_bf16(np.random.SeedSequence(601), (7168, 4096))
    b = W.normal_bf16(np.random.SeedSequence(602), (2112, 4096))
    (qa, sa), (qb, sb) = te.te_cast_fp8_per_token_batch([bf16_dev(a), bf16_dev(b)], te.TE_DTYPE_E4M3)
    for bits, q, s in ((a, qa, sa), (b, qb, sb)):
        qo, so = oracle.cast_per_token(bits, oracle.E4M3)
        assert np.array_equal(host(q).numpy(), qo)
        assert np.array_equal(shost(s, bits.shape[0]).view(np.uint32), so.view(np.uint32))
