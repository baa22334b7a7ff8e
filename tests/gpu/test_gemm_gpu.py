"""GEMM kernel parity: orthrus_gemm_bf16 against an fp64 matmul of the same
bf16 operands (the definition C = A B^T), every epilogue, ragged edges."""

import numpy as np
import pytest
import torch

import heterogeneous_embed_decode_amd as hed
from synth.bf16 import f32_to_bf16_bits, bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale=1.0):
    bits = f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale)
    return bits, bf16_bits_to_f32(bits).astype(np.float64)


def _dev(bits):
    return torch.from_numpy(bits.view(np.int16)).cuda()


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _row_rel_max(a, b):
    # a few wrong elements (one MFMA block's registers, say) hide in the
    # matrix-wide norm; every row must be right on its own
    num = np.linalg.norm(a - b, axis=1)
    den = np.maximum(np.linalg.norm(b, axis=1), 1e-30)
    return float((num / den).max())


SHAPES = [(34, 128, 64), (300, 176, 64), (129, 257, 176), (1, 64, 4096), (4160, 384, 512),
          (64, 1000, 4096), (1040, 2056, 520), (700, 1300, 200), (512, 1024, 64),
          (2000, 1536, 2048),
          # the one-wave-per-SIMD kernel (bf16 outputs, K a multiple of 32):
          # an odd number of K-steps, ragged rows and columns, K = 4096
          (700, 1300, 96), (1030, 1100, 4096),
          # residual grid of one workgroup per CU: 256 whole tiles (plain
          # read-modify-write) plus a stream-K remainder, ragged rows and columns
          (4160, 4096, 256), (4100, 4200, 128),
          # residual grid of one workgroup per tile (the tiles past the last
          # full round of CUs fill at least half of them)
          (2048, 4096, 64), (1800, 4100, 72)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("epi", [hed.EPI_BF16, hed.EPI_F32, hed.EPI_RESID])
def test_gemm_epilogues(M, N, K, epi):
    print(f"gemm M={M} N={N} K={K} epi={epi}", flush=True)
    rng = np.random.default_rng(M * 7 + N + K + epi)
    a_bits, A = _bf16(rng, (M, K))
    b_bits, B = _bf16(rng, (N, K), 0.05)
    ref = A @ B.T
    dA, dB = _dev(a_bits), _dev(b_bits)
    if epi == hed.EPI_BF16:
        C = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    else:
        C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    C0 = None
    if epi == hed.EPI_RESID:
        C0 = rng.standard_normal((M, N)).astype(np.float32)
        C.copy_(torch.from_numpy(C0))
        ref = ref + C0
    st = hed.orthrus_gemm_bf16(dA.data_ptr(), K, dB.data_ptr(), K, C.data_ptr(), N, M, N, K, epi)
    assert st == hed.OK
    torch.cuda.synchronize()
    if epi == hed.EPI_BF16:
        got = bf16_bits_to_f32(C.cpu().numpy().view(np.uint16)).astype(np.float64)
        tol = 8e-3
    else:
        got = C.cpu().numpy().astype(np.float64)
        tol = 1e-5
    assert _rel(got, ref) < tol
    assert _row_rel_max(got, ref) < 2 * tol


@pytest.mark.parametrize("M,F,K", [(34, 176, 64), (257, 200, 128), (1024, 1024, 512), (777, 1160, 264),
                                   # a last tile row of 64 or fewer rows run as a launch of 64-row tiles
                                   (4160, 2048, 256), (2112, 4096, 128), (1040, 8192, 64),
                                   # one-wave-per-SIMD kernel: ragged rows and output columns, an odd
                                   # number of K-steps, K = 4096
                                   (1000, 1100, 96), (600, 2000, 4096)])
def test_gemm_swiglu(M, F, K):
    print(f"swiglu M={M} F={F} K={K}", flush=True)
    rng = np.random.default_rng(M + F)
    a_bits, A = _bf16(rng, (M, K))
    b_bits, B = _bf16(rng, (2 * F, K), 0.1)
    g = A @ B[:F].T
    u = A @ B[F:].T
    ref = g / (1 + np.exp(-g)) * u
    C = torch.zeros((M, F), dtype=torch.int16, device="cuda")
    dA, dB = _dev(a_bits), _dev(b_bits)   # keep both alive across the launch
    st = hed.orthrus_gemm_bf16(dA.data_ptr(), K, dB.data_ptr(), K, C.data_ptr(), F,
                               M, F, K, hed.EPI_SWIGLU, F)
    assert st == hed.OK
    torch.cuda.synchronize()
    got = bf16_bits_to_f32(C.cpu().numpy().view(np.uint16)).astype(np.float64)
    assert _rel(got, ref) < 8e-3
    assert _row_rel_max(got, ref) < 1.6e-2


def test_gemm_rejects_bad_sizes():
    assert hed.orthrus_gemm_bf16(1, 12, 1, 12, 1, 4, 4, 4, 12, 0) == hed.EINVAL
    assert hed.orthrus_gemm_bf16(1, 16, 1, 16, 1, 4, 4, 4, 16, 9) == hed.EINVAL


# Adapter shrink U = bf16(s X A^T) through its own entry point: ragged row
# and column tiles, a row stride wider than K, and scales other than 1 (the
# scale is folded into the GEMM's bf16 epilogue).
SHRINK = [(1, 16, 32, 1.0, 0), (15, 48, 64, 0.5, 0), (17, 24, 96, 2.0, 8), (300, 64, 4096, 1.0, 0),
          (7168, 48, 4096, 1.0, 0), (4096, 16, 4096, 0.25, 0), (129, 1, 160, 1.0, 0), (33, 40, 224, 3.0, 16),
          (200, 80, 256, 1.0, 0), (50, 16, 72, 1.0, 0)]


@pytest.mark.parametrize("ws", [False, True], ids=["one_pass", "k_split"])
@pytest.mark.parametrize("rows,nr,K,scale,pad", SHRINK)
def test_lora_shrink(rows, nr, K, scale, pad, ws):
    """With a workspace the library splits K over several workgroups per
    tile when the tiles are too few to fill the chip (the 300-, 4096- and
    7168-row cases at K = 4096) and adds the fp32 partials in order."""
    print(f"shrink rows={rows} nr={nr} K={K} scale={scale} pad={pad} ws={ws}", flush=True)
    rng = np.random.default_rng(rows * 31 + nr * 7 + K)
    ldx = K + pad
    x_bits, X = _bf16(rng, (rows, ldx))
    a_bits, A = _bf16(rng, (nr, K), 0.02)
    ref = scale * (X[:, :K] @ A.T)
    U = torch.zeros((rows, nr), dtype=torch.int16, device="cuda")
    dX, dA = _dev(x_bits), _dev(a_bits)  # held until the kernel has run
    W = torch.full((8 * rows * nr,), float("nan"), device="cuda") if ws else None
    st = hed.orthrus_lora_shrink_bf16(dX.data_ptr(), ldx, dA.data_ptr(), rows, nr, K, scale, U.data_ptr(),
                                      W.data_ptr() if ws else None, 32 * rows * nr if ws else 0)
    assert st == hed.OK
    torch.cuda.synchronize()
    got = bf16_bits_to_f32(U.cpu().numpy().view(np.uint16)).astype(np.float64)
    # one bf16 rounding of an fp32 sum: 2^-8 relative per element plus the
    # fp32 accumulation error, far below it at these K
    err = np.abs(got - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.sqrt(K)), (float(err.max()), rows, nr, K)

