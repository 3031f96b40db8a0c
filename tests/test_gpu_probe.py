"""The matrix-core rate probe (chunkattn_mfma_probe) computes what it claims:
every accumulator of every wave of every workgroup equals iters * A_s B_s
exactly, with A_s, B_s decoded from the operand words by the fragment layout
of the 16x16x32 bf16 matrix instruction stated in include/chunkattn.h (row
l % 16 of A and column l % 16 of B hold the lane's eight values at k = 8*(l/16)
.. +7; lane l holds rows 4*(l/16) .. +3 of column l % 16 of the result).  The
expected products are computed here with numpy from the same words; with
entries in {-1, 0, 1} the products are small integers, so the comparison is
exact.  An exact result shows that every instruction the FLOP count assumes
ran."""
import numpy as np
import pytest
import torch

from chunked_spatio_temporal_amd import chunkattn as ca
from chunked_spatio_temporal_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ca.load_library()
    yield


def _bf16_words_to_float(words: np.ndarray) -> np.ndarray:
    """[.., n] uint32 words -> [.., 2n] float32 (low half first)."""
    w = words.astype(np.uint32)
    lo = (w & 0xFFFF) << 16
    hi = w & 0xFFFF0000
    out = np.empty(w.shape[:-1] + (2 * w.shape[-1],), dtype=np.uint32)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out.view(np.float32)


def _expected(words: np.ndarray, iters: int) -> np.ndarray:
    """[8 accumulators][64 lanes][4] of one wave."""
    vals = _bf16_words_to_float(words)  # [64 lanes][64 values]: 4 sets x (A 8, B 8)
    exp = np.zeros((8, 64, 4), dtype=np.float64)
    prods = []
    for s in range(4):
        A = np.zeros((16, 32))
        B = np.zeros((32, 16))
        for lane in range(64):
            r, g = lane % 16, lane // 16
            A[r, 8 * g:8 * g + 8] = vals[lane, 16 * s:16 * s + 8]
            B[8 * g:8 * g + 8, r] = vals[lane, 16 * s + 8:16 * s + 16]
        prods.append(A @ B)
    for a in range(8):
        D = prods[a % 4]
        for lane in range(64):
            n, g = lane % 16, lane // 16
            exp[a, lane, :] = iters * D[4 * g:4 * g + 4, n]
    return exp


@pytest.mark.parametrize("iters,seed", [(1, 3), (777, 4), (1 << 19, 5)])
def test_probe_result_is_exact(iters, seed):
    print("case probe", iters, seed, flush=True)
    ctx = ca.Context(0, 0)
    ops = synth.probe_operands(seed, device=DEV)
    out = torch.full((ctx.cu_count * ca.PROBE_OUT_PER_WORKGROUP,), float("nan"),
                     dtype=torch.float32, device=DEV)
    n_wg, flops = ca.mfma_probe(ops, iters, out, ctx=ctx)
    torch.cuda.synchronize()
    assert n_wg == ctx.cu_count
    assert flops == n_wg * 8 * 8 * iters * 2 * 16 * 16 * 32
    got = out.view(n_wg, 8, 8, 64, 4).cpu().numpy().astype(np.float64)
    exp = _expected(ops.cpu().numpy(), iters)
    assert np.array_equal(got, np.broadcast_to(exp, got.shape))


def test_probe_rejects_bad_arguments():
    ctx = ca.Context(0, 0)
    ops = synth.probe_operands(0, device=DEV)
    out = torch.empty(ctx.cu_count * ca.PROBE_OUT_PER_WORKGROUP, dtype=torch.float32, device=DEV)
    for iters in (0, (1 << 19) + 1):
        with pytest.raises(ca.ChunkAttnError) as e:
            ca.mfma_probe(ops, iters, out, ctx=ctx)
        assert e.value.status == ca.EINVAL
    with pytest.raises(ValueError):
        ca.mfma_probe(ops, 1, out[:100], ctx=ctx)
