"""GPU parity: fp4_gemm against the oracle's exact dequantized product.
|C_gpu - C| <= 1e-4 * sum_k |A_hat B_hat| per element (fp32 C), plus one bf16
rounding of C for bf16 output; bit-exact in the exact-integer case."""
import numpy as np
import pytest
import torch

from fp4_quantized_diffusion_amd import inputs
from oracle import gemm as ogemm, mxfp4, nvfp4
from tests._parity import gemm_within_tol, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def quantize_both(fq, a, b, fmt, dtype=torch.float32):
    qa = fq.quantize(dev(a.astype(np.float32)).to(dtype), fmt)
    qb = fq.quantize(dev(b.astype(np.float32)).to(dtype), fmt)
    return qa, qb


def oracle_c(qa, qb, fmt, rows=None, cols=None):
    k = qa.k
    ac, as_ = to_np(qa.codes)[:, : k // 2], to_np(qa.scales)
    bc, bs = to_np(qb.codes)[:, : k // 2], to_np(qb.scales)
    if rows is not None:
        ac, as_ = ac[rows], as_[rows]
    if cols is not None:
        bc, bs = bc[cols], bs[cols]
    if fmt == "mx":
        return ogemm.gemm_mx(ac, as_, bc, bs)
    return ogemm.gemm_nv(ac, as_, to_np(qa.tensor_scale)[0], bc, bs, to_np(qb.tensor_scale)[0])


@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_tiny_config(gpu_lib, fmt, out):
    x, b = inputs.tiny(0)
    qa, qb = quantize_both(gpu_lib, x, b, fmt)
    c = gpu_lib.gemm(qa, qb, out)
    c_exact, s_abs = oracle_c(qa, qb, fmt)
    ok, worst = gemm_within_tol(to_np(c.float()), c_exact, s_abs, bf16_out=(out == "bf16"))
    assert ok, worst


def test_exact_integer_case_bit_exact(gpu_lib):
    """Scales 2^0 and grid codes: products are multiples of 1/4 and partial
    sums stay below 2^22, so fp32 accumulation is exact and the GPU result
    must equal the oracle bit for bit -- any operand-layout, K-order or
    scale-plumbing slip shows up here."""
    rng = np.random.default_rng(30)
    for (m, n, k) in [(256, 256, 256), (300, 260, 512), (129, 515, 4096), (16, 16, 32)]:
        ac = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
        bc = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        as_ = np.full((m, k // 32), 127, np.uint8)
        bs = np.full((n, k // 32), 127, np.uint8)
        from fp4_quantized_diffusion_amd.binding import QTensor, FMT_MX
        lda = ((k // 2 + 15) // 16) * 16
        acd = torch.zeros((m, lda), dtype=torch.uint8, device=DEV); acd[:, : k // 2] = dev(ac)
        bcd = torch.zeros((n, lda), dtype=torch.uint8, device=DEV); bcd[:, : k // 2] = dev(bc)
        qa = QTensor(acd, dev(as_), None, FMT_MX, k)
        qb = QTensor(bcd, dev(bs), None, FMT_MX, k)
        c = to_np(gpu_lib.gemm(qa, qb, "f32"))
        c_exact, _ = ogemm.gemm_mx(ac, as_, bc, bs)
        np.testing.assert_array_equal(c.astype(np.float64), c_exact)


@pytest.mark.parametrize("k", [5600, 2240, 96])
def test_unaligned_scale_rows(gpu_lib, k):
    """Scale rows of K/32 bytes with no padding (an odd stride for K = 5600):
    the GEMM's byte-wise scale path."""
    rng = np.random.default_rng(k)
    m, n = 300, 272
    ac = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    as_ = rng.integers(120, 134, size=(m, k // 32), dtype=np.uint8)
    bs = rng.integers(120, 134, size=(n, k // 32), dtype=np.uint8)
    from fp4_quantized_diffusion_amd.binding import QTensor, FMT_MX
    lda = ((k // 2 + 15) // 16) * 16
    acd = torch.zeros((m, lda), dtype=torch.uint8, device=DEV); acd[:, : k // 2] = dev(ac)
    bcd = torch.zeros((n, lda), dtype=torch.uint8, device=DEV); bcd[:, : k // 2] = dev(bc)
    qa = QTensor(acd, dev(as_), None, FMT_MX, k)
    qb = QTensor(bcd, dev(bs), None, FMT_MX, k)
    for out in ("f32", "bf16"):
        c = to_np(gpu_lib.gemm(qa, qb, out).float())
        c_exact, s_abs = ogemm.gemm_mx(ac, as_, bc, bs)
        ok, worst = gemm_within_tol(c, c_exact, s_abs, bf16_out=(out == "bf16"))
        assert ok, (out, worst)


def test_padded_scale_rows_with_garbage(gpu_lib):
    """Scale rows padded past K/32 with 0xFF (an E8M0 NaN): the padding must
    never reach the MFMA (K = 2240 ends mid-word)."""
    rng = np.random.default_rng(35)
    m, n, k = 260, 256, 2240
    a = rng.standard_normal((m, k)).astype(np.float32)
    b = rng.standard_normal((n, k)).astype(np.float32)
    qa, qb = quantize_both(gpu_lib, a, b, "mx")
    from fp4_quantized_diffusion_amd.binding import QTensor
    def pad(q):
        s = torch.full((q.scales.shape[0], 72), 0xFF, dtype=torch.uint8, device=DEV)
        s[:, :70] = q.scales
        return QTensor(q.codes, s[:, :70], None, q.fmt, q.k)
    c = to_np(gpu_lib.gemm(pad(qa), pad(qb), "f32"))
    c_exact, s_abs = oracle_c(qa, qb, "mx")
    ok, worst = gemm_within_tol(c, c_exact, s_abs)
    assert ok, worst


def test_varied_scales_exact_rational_small(gpu_lib):
    """Random codes and random E8M0 scales (not from a quantizer) -- exercises
    the per-lane scale selection of every K-block."""
    rng = np.random.default_rng(31)
    m, n, k = 64, 48, 512
    ac = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    as_ = rng.integers(117, 138, size=(m, k // 32), dtype=np.uint8)
    bs = rng.integers(117, 138, size=(n, k // 32), dtype=np.uint8)
    from fp4_quantized_diffusion_amd.binding import QTensor, FMT_MX
    qa = QTensor(dev(ac), dev(as_), None, FMT_MX, k)
    qb = QTensor(dev(bc), dev(bs), None, FMT_MX, k)
    c = to_np(gpu_lib.gemm(qa, qb, "f32"))
    c_exact, s_abs = ogemm.gemm_mx(ac, as_, bc, bs)
    ok, worst = gemm_within_tol(c, c_exact, s_abs)
    assert ok, worst


@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("shape", [(300, 260, 96), (257, 513, 2240), (100, 70, 5600), (33, 2432, 9728), (1, 1, 32)])
def test_ragged_shapes(gpu_lib, fmt, shape):
    m, n, k = shape
    rng = np.random.default_rng(m * 7 + n)
    a = rng.standard_t(4, size=(m, k)).astype(np.float32)
    b = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    qa, qb = quantize_both(gpu_lib, a, b, fmt)
    for out in ("f32", "bf16"):
        c = gpu_lib.gemm(qa, qb, out)
        c_exact, s_abs = oracle_c(qa, qb, fmt)
        ok, worst = gemm_within_tol(to_np(c.float()), c_exact, s_abs, bf16_out=(out == "bf16"))
        assert ok, (out, worst)


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_residual_and_in_place(gpu_lib, fmt):
    rng = np.random.default_rng(32)
    m, n, k = 200, 300, 640
    a = rng.standard_normal((m, k)).astype(np.float32)
    b = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    r = rng.standard_normal((m, n)).astype(np.float32)
    qa, qb = quantize_both(gpu_lib, a, b, fmt)
    c_exact, s_abs = oracle_c(qa, qb, fmt)
    rd = dev(r)
    c = to_np(gpu_lib.gemm(qa, qb, "f32", residual=rd))
    ok, worst = gemm_within_tol(c, c_exact + r, s_abs + np.abs(r) * 1e-3)
    assert ok, worst
    gpu_lib.gemm(qa, qb, "f32", residual=rd, out=rd)   # in place
    ok, worst = gemm_within_tol(to_np(rd), c_exact + r, s_abs + np.abs(r) * 1e-3)
    assert ok, worst


def test_determinism(gpu_lib):
    rng = np.random.default_rng(33)
    a = rng.standard_normal((512, 1024)).astype(np.float32)
    b = rng.standard_normal((768, 1024)).astype(np.float32)
    qa, qb = quantize_both(gpu_lib, a, b, "mx")
    c0 = to_np(gpu_lib.gemm(qa, qb, "f32"))
    for _ in range(5):
        np.testing.assert_array_equal(to_np(gpu_lib.gemm(qa, qb, "f32")), c0)


@pytest.mark.parametrize("cls,which", [("flux", 1), ("flux", 2), ("sana", 1), ("sana", 2), ("sd35", 1)])
def test_full_size_sampled(gpu_lib, cls, which):
    """Workload-class GEMMs at full size, in the launch configuration the
    benchmark uses (bf16 activations, bf16 output): quantized codes of sampled
    rows are bit-exact and sampled outputs are within tolerance."""
    a, w = inputs.class_linear(cls, which)
    qa, qb = quantize_both(gpu_lib, a, w, "mx", torch.bfloat16)
    c = gpu_lib.gemm(qa, qb, "bf16")
    torch.cuda.synchronize()
    rng = np.random.default_rng(34)
    rows = np.sort(rng.choice(a.shape[0], 48, replace=False))
    rows[-1] = a.shape[0] - 1
    cols = np.sort(rng.choice(w.shape[0], 64, replace=False))
    cols[-1] = w.shape[0] - 1
    oc, os_ = mxfp4.quantize(a[rows])
    k = a.shape[1]
    np.testing.assert_array_equal(to_np(qa.codes[rows])[:, : k // 2], oc)
    np.testing.assert_array_equal(to_np(qa.scales[rows]), os_)
    c_exact, s_abs = oracle_c(qa, qb, "mx", rows, cols)
    c_s = to_np(c.float())[np.ix_(rows, cols)]
    ok, worst = gemm_within_tol(c_s, c_exact, s_abs, bf16_out=True)
    assert ok, worst


@pytest.mark.parametrize("cls,which", [("flux", 1), ("flux", 2), ("sd35", 1)])
def test_full_size_sampled_nv(gpu_lib, cls, which):
    """The NVFP4-style pair at full workload size (bf16 activations and
    weights, bf16 output): the tensor scales equal the oracle's over the whole
    operands, the codes and E4M3 scales of sampled rows are bit-exact, and
    sampled outputs are within the GEMM tolerance of the exact dequantized
    product."""
    from oracle import nvfp4
    a, w = inputs.class_linear(cls, which)
    qa, qb = quantize_both(gpu_lib, a, w, "nv", torch.bfloat16)
    c = gpu_lib.gemm(qa, qb, "bf16")
    torch.cuda.synchronize()
    sg_a, sg_b = nvfp4.tensor_scale(a), nvfp4.tensor_scale(w)
    assert to_np(qa.tensor_scale)[0] == sg_a and to_np(qb.tensor_scale)[0] == sg_b
    rng = np.random.default_rng(35)
    rows = np.sort(rng.choice(a.shape[0], 48, replace=False))
    rows[-1] = a.shape[0] - 1
    cols = np.sort(rng.choice(w.shape[0], 64, replace=False))
    cols[-1] = w.shape[0] - 1
    k = a.shape[1]
    oc, os_, _ = nvfp4.quantize(a[rows], s_g=sg_a)
    np.testing.assert_array_equal(to_np(qa.codes[rows])[:, : k // 2], oc)
    np.testing.assert_array_equal(to_np(qa.scales[rows])[:, : k // 16], os_)
    oc, os_, _ = nvfp4.quantize(w[cols], s_g=sg_b)
    np.testing.assert_array_equal(to_np(qb.codes[cols])[:, : k // 2], oc)
    np.testing.assert_array_equal(to_np(qb.scales[cols])[:, : k // 16], os_)
    c_exact, s_abs = oracle_c(qa, qb, "nv", rows, cols)
    c_s = to_np(c.float())[np.ix_(rows, cols)]
    ok, worst = gemm_within_tol(c_s, c_exact, s_abs, bf16_out=True)
    assert ok, worst


def nv_operand(codes, scales, ts, k, code_garbage=None, scale_ld=None, scale_fill=0x7F):
    """An NVFP4-style QTensor from host codes [rows, k/2] and E4M3 scale
    bytes [rows, k/16]. Code rows are padded to a multiple of 16 bytes with
    `code_garbage` (random bytes; zeros if None); scale rows get stride
    `scale_ld` (default k/16 rounded up to 4), the padding filled with
    `scale_fill` (0x7F: an E4M3 NaN)."""
    from fp4_quantized_diffusion_amd.binding import QTensor, FMT_NV
    rows = codes.shape[0]
    lda = ((k // 2 + 15) // 16) * 16
    cbuf = np.zeros((rows, lda), np.uint8) if code_garbage is None else code_garbage.integers(
        0, 256, size=(rows, lda), dtype=np.uint8)
    cbuf[:, : k // 2] = codes
    nb = k // 16
    ld = scale_ld or ((nb + 3) // 4) * 4
    sbuf = np.full((rows, ld), scale_fill, np.uint8)
    sbuf[:, :nb] = scales
    sd = dev(sbuf)[:, :nb]
    return QTensor(dev(cbuf), sd, torch.tensor([ts], dtype=torch.float32, device=DEV), FMT_NV, k)


@pytest.mark.parametrize("m,n,k", [(256, 256, 256), (300, 260, 512), (129, 515, 4096), (16, 16, 48),
                                   (70, 33, 400)])
def test_nv_exact_integer_case_bit_exact(gpu_lib, m, n, k):
    """NVFP4-style operands with every block scale 1.0 (E4M3 0x38) and tensor
    scales 1: products are multiples of 1/4 and partial sums stay below 2^22,
    so the GPU must equal the oracle bit for bit (operand layout, K order,
    K tails that end mid-chunk, row padding holding random bytes)."""
    rng = np.random.default_rng(m + 3 * n + k)
    ac = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    as_ = np.full((m, k // 16), 0x38, np.uint8)
    bs = np.full((n, k // 16), 0x38, np.uint8)
    qa = nv_operand(ac, as_, 1.0, k, code_garbage=rng)
    qb = nv_operand(bc, bs, 1.0, k, code_garbage=rng)
    c = to_np(gpu_lib.gemm(qa, qb, "f32"))
    c_exact, _ = ogemm.gemm_nv(ac, as_, 1.0, bc, bs, 1.0)
    np.testing.assert_array_equal(c.astype(np.float64), c_exact)


@pytest.mark.parametrize("m,n,k", [(300, 260, 400), (257, 513, 2240), (64, 48, 9728), (1, 1, 16)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_nv_random_scales_and_garbage_padding(gpu_lib, m, n, k, out):
    """Random codes with random E4M3 block scales over the whole finite range
    (subnormals included) and arbitrary fp32 tensor scales; code rows padded
    with random bytes and scale rows with 0x7F (NaN): nothing past K may
    reach the sum."""
    rng = np.random.default_rng(7 * m + n + k)
    ac = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    as_ = rng.integers(0, 127, size=(m, k // 16), dtype=np.uint8)
    bs = rng.integers(0, 127, size=(n, k // 16), dtype=np.uint8)
    ta, tb = np.float32(3.7e-3), np.float32(0.0123)
    qa = nv_operand(ac, as_, ta, k, code_garbage=rng, scale_ld=k // 16 + 4)
    qb = nv_operand(bc, bs, tb, k, code_garbage=rng, scale_ld=k // 16 + 4)
    c = to_np(gpu_lib.gemm(qa, qb, out).float())
    c_exact, s_abs = ogemm.gemm_nv(ac, as_, ta, bc, bs, tb)
    ok, worst = gemm_within_tol(c, c_exact, s_abs, bf16_out=(out == "bf16"))
    assert ok, worst


@pytest.mark.parametrize("k", [592, 80])
def test_nv_unaligned_scale_rows(gpu_lib, k):
    """Scale rows of K/16 bytes with no padding (odd stride): the byte-wise
    NVFP4-style kernel."""
    rng = np.random.default_rng(k)
    m, n = 130, 200
    ac = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    as_ = rng.integers(40, 70, size=(m, k // 16), dtype=np.uint8)
    bs = rng.integers(40, 70, size=(n, k // 16), dtype=np.uint8)
    qa = nv_operand(ac, as_, 0.5, k, scale_ld=k // 16)
    qb = nv_operand(bc, bs, 2.0, k, scale_ld=k // 16)
    assert qa.scales.stride(0) % 4 != 0
    c = to_np(gpu_lib.gemm(qa, qb, "f32"))
    c_exact, s_abs = ogemm.gemm_nv(ac, as_, 0.5, bc, bs, 2.0)
    ok, worst = gemm_within_tol(c, c_exact, s_abs)
    assert ok, worst


