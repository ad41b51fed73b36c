"""The accuracy ablation on a small layer: the ordering the pages claim.

"A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
scale", sections "absmax quantization", "inside the MatMul" and "LLM.int8()
summary": vector-wise scales beat one scale per tensor, and moving outlier
columns to 16-bit removes most of the error they cause.  Reported by the
ablation module; here its ordering is checked on seeded data."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_ablation_ordering():
    from int8_quantized_matmul_row_amd import ablation
    rows = ablation.run(M=64, N=512, K=1024, densities=(0.0, 0.01), thresholds=(6.0,))
    print(ablation.table(rows), flush=True)
    by = {(r["density"], r["scheme"]): r for r in rows}
    # no outliers: LLM.int8() at t = 6 is the vector-wise scheme exactly
    assert by[(0.0, "LLM.int8()")]["rel_fro"] == by[(0.0, "vector-wise")]["rel_fro"]
    assert by[(0.0, "LLM.int8()")]["n_out"] == 0
    # with outlier columns: decomposition << vector-wise <= per-tensor
    d = by[(0.01, "LLM.int8()")]
    v = by[(0.01, "vector-wise")]
    p = by[(0.01, "per-tensor absmax")]
    assert d["n_out"] == 10
    assert d["rel_fro"] < 0.25 * v["rel_fro"]
    assert v["rel_fro"] <= 1.05 * p["rel_fro"]


def test_ablation_fp8_rows():
    """The FP8 variant keeps part of the decomposition's benefit: with outlier
    columns, FP8 at threshold 6 is closer to the exact product than FP8
    without outlier columns.  The gain is smaller than int8's (E4M3 keeps a
    relative precision of 2^-4 at every magnitude, so a large absmax costs it
    less), and E4M3 codes are less precise than int8 codes on this data; both
    are reported by the ablation, not gated: the pages give no figure."""
    from int8_quantized_matmul_row_amd import ablation
    rows = ablation.run(M=64, N=512, K=1024, densities=(0.0, 0.01), thresholds=(6.0,))
    by = {(r["density"], r["scheme"]): r for r in rows}
    d = by[(0.01, "FP8 LLM.int8()")]
    v = by[(0.01, "FP8 vector-wise")]
    assert d["n_out"] == 10 and v["n_out"] == 0
    assert d["rel_fro"] < 0.9 * v["rel_fro"]
    assert by[(0.0, "FP8 LLM.int8()")]["rel_fro"] == by[(0.0, "FP8 vector-wise")]["rel_fro"]
