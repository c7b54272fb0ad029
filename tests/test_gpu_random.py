"""Layer parity on seeded random configurations: expert counts 1-40, top-k up
to 4, token counts 1-700, widths with K and N tails, SwiGLU or GELU, softmax
or sigmoid scoring, a shared expert or none, capacity factors from dropping
most assignments to none, fp32 and bf16, and the FP8 forward and data-gradient
variants where the widths allow. Every case is compared with the oracle as the
fixed cases are (tests/test_gpu_layer.py); the draws reach grouped tile counts
and per-XCD remainders that the fixed cases do not."""
import numpy as np
import pytest

from moe_inputs import Workload
from parity_util import run_and_compare

pytestmark = pytest.mark.gpu


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    E = int(rng.choice([1, 2, 3, 5, 8, 13, 32, 40]))
    k = int(rng.integers(1, min(E, 4) + 1))
    T = int(rng.integers(1, 701))
    dtype = "fp32" if rng.random() < 0.2 else "bf16"
    d = int(rng.choice([16, 48, 64, 136, 208, 320]))
    f = int(rng.choice([16, 40, 96, 200, 256, 384]))
    act = str(rng.choice(["swiglu", "gelu"]))
    score = str(rng.choice(["softmax", "sigmoid"]))
    cf = [None, 0.5, 1.0, 1.25, 2.0][int(rng.integers(0, 5))]
    fp8 = dtype == "bf16" and d % 16 == 0 and f % 16 == 0 and rng.random() < 0.8
    return Workload(f"rand{i}", T=T, d=d, E=E, k=k, f=f, dtype=dtype, act=act, score=score,
                    n_shared=int(rng.integers(0, 2)), cf=cf,
                    sel_bias=score == "sigmoid" and rng.random() < 0.5,
                    aux_coef=float(rng.choice([0.0, 0.02])),
                    z_coef=float(rng.choice([0.0, 0.01])) if score == "softmax" else 0.0,
                    fp8=fp8, fp8_bwd=fp8 and rng.random() < 0.6, seed=i)


@pytest.mark.parametrize("i", range(24))
def test_random_layer_parity(i):
    w = _draw(i)
    print(f"[case] random {i} {w}", flush=True)
    rep, flips, _, _ = run_and_compare(w)
    print(rep, flush=True)
