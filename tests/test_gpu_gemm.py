"""GPU parity of the bf16 MFMA GEMM (mamba_gemm_bf16 through the C ABI) against the plain
definition C = A B evaluated in float64 on the same bf16 values (numpy matmul).

Bound: max_i |c_i - ref_i| / max(|ref_i|, rms(ref)) <= 1e-2 (bf16 output rounding is at most
2^-8 relative; fp32 accumulation adds ~1e-6).
"""
import os

import numpy as np
import pytest
import torch

from selective_state_space_47_amd import _build, binding, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _native():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    binding.lib()


def rel_err(got, ref):
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), rms)))


def bf16(rng, shape, scale=1.0):
    return synth.round_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


# (4112, 2056, 520, 4) is a many-tile shape with ragged M, N and K tails.  With B K-contiguous,
# K a multiple of 32, M >= 256 and N >= 128 the large-tile kernel serves the call:
# (256, 128, 64, 1) one 256 x 256 tile half outside N and a single K step; (272, 136, 128, 2) and
# (1040, 520, 192, 3) ragged M and N on 256 x 128 tiles, the latter with an odd number of K
# steps; (4096, 2048, 512, 4) 256 x 256 tiles; (512, 256, 160, 2) and (272, 136, 96, 1) K a
# multiple of the 32-deep K step but not of 64, with fewer K steps than stages (5 and 3);
# (256, 256, 32, 2) a single K step (the load prologue only).
SHAPES = [(16, 8, 8, 1), (128, 128, 64, 1), (144, 200, 136, 2), (256, 384, 520, 3),
          (192, 264, 5120, 2), (5120, 136, 160, 1), (48, 1000, 72, 2),
          (4096, 2048, 512, 4), (4112, 2056, 520, 4),
          (256, 128, 64, 1), (272, 136, 128, 2), (1040, 520, 192, 3),
          (512, 256, 160, 2), (272, 136, 96, 1), (256, 256, 32, 2)]


@pytest.mark.parametrize("b_kcontig", [True, False])
@pytest.mark.parametrize("c_trans", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_matches_fp64(shape, b_kcontig, c_trans):
    M, N, K, batch = shape
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A = bf16(rng, (M, K), 1.0 / np.sqrt(K))
    Bm = bf16(rng, (batch, K, N))                      # (k, n) per batch
    Bstore = np.ascontiguousarray(Bm.transpose(0, 2, 1)) if b_kcontig else Bm
    tA = torch.from_numpy(A).to(DEV).to(torch.bfloat16)
    tB = torch.from_numpy(Bstore).to(DEV).to(torch.bfloat16)
    print(f"[gemm] M={M} N={N} K={K} batch={batch} b_kcontig={b_kcontig} c_trans={c_trans}",
          flush=True)
    C = binding.mamba_gemm_bf16(tA, tB, b_kcontig=b_kcontig, c_trans=c_trans)
    torch.cuda.synchronize()
    C = C.float().cpu().numpy()
    if c_trans:
        C = C.transpose(0, 2, 1)
    ref = np.matmul(A.astype(np.float64)[None], Bm.astype(np.float64))
    e = rel_err(C, ref)
    print(f"[gemm] rel err {e:.2e}", flush=True)
    assert e <= 1e-2


def test_gemm_validation():
    A = torch.zeros((20, 16), dtype=torch.bfloat16, device=DEV)   # M % 16 != 0
    B = torch.zeros((1, 8, 16), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="-2"):
        binding.mamba_gemm_bf16(A, B)
