"""CPU check of the random GPU cases: deterministic, and they reach every path, split and
unsplit calls, the split merge kernels for few and many partials, forced widths, the fused
entry point, fp32 and head dim 64."""
from tests import random_cases as R


def test_draws_are_deterministic():
    assert [R.case_id(i) for i in range(R.N_CASES)] == [R.case_id(i) for i in range(R.N_CASES)]


def test_draws_cover_the_space():
    cs = [R.draw(i) for i in range(R.N_CASES)]
    assert {c["path"] for c in cs} == {"vector", "mfma", "valu"}
    assert any(c["parts"] == 1 for c in cs)
    assert any(2 <= c["parts"] <= 16 for c in cs) and any(c["parts"] > 16 for c in cs)
    assert {c["width"] for c in cs} >= {"", "1", "2", "4"}
    assert any(c["fused"] for c in cs) and not all(c["fused"] for c in cs)
    assert any(c["dt"] == "f32" for c in cs) and any(c["D"] == 64 for c in cs)
    assert any((c["ctx"] == 1).any() for c in cs) and any(c["S"] == 1 for c in cs)
    assert {c["B"] for c in cs} == {4, 8, 16, 32, 64, 128}
