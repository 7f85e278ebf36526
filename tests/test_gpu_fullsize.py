"""Full-size parity at every workload the layer is measured on, in the launch
configuration bench.py times: selection maps bit-exact on every head, every
tensor of the sampled heads (whole heads, fwd and bwd) against the oracle."""
import pytest
import torch

from long_context_pretraining_amd import inputs
from long_context_pretraining_amd import lighthouse as lh
from tests.adversarial import make_adversarial
from tests.gpu_support import compare_head, compare_selection, run_layer, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lh.load_library()


def _run(name, heads, mutate=None):
    w = inputs.WORKLOADS[name]
    say(f"[fullsize] {w}")
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_dout(w)
    if mutate:
        mutate(w, q, k, v, log=say)
    r = run_layer(w, q, k, v, dout)
    say(f"  S = {r.plan.S} (formula {r.plan.S_formula}); checking selection on all {w.B * w.H} heads")
    compare_selection(w, q, k, r)
    for b, h in heads:
        compare_head(w, q, k, v, dout, r, b, h)
    del r
    torch.cuda.empty_cache()


def test_headline_98k_k1536():
    """B=1 H=16 N=98304 d=64 bf16, p=4 L=4 k=1536 (S=19968)."""
    _run("llama530m_98k_k1536", [(0, 0), (0, 7), (0, 15)])


def test_98k_k6144_clamped():
    """k=6144 exceeds the coarsest level (1536): that level is fully
    expanded and S = 56832 instead of the formula's 75264."""
    _run("llama530m_98k_k6144", [(0, 5)])


def test_98k_adversarial_ties():
    """Clustered x8 spans, exact-tie subtrees, tie groups straddling every cut."""
    _run("llama530m_98k_adversarial", [(0, 0), (0, 11)], mutate=make_adversarial)


def test_extreme_512k():
    """B=1 H=16 N=524288 d=64 bf16, p=4 L=6 k=1536: the coarsest level (512)
    is below k, so S = 27136 instead of 31232."""
    _run("extreme_512k", [(0, 3)])


def test_98k_ablation_p2_L3():
    """The ablation optimum p=2, L=3, k=1536 on the 98K layer (S=30720)."""
    _run("ablation_p2_L3_98k", [(0, 9)])
