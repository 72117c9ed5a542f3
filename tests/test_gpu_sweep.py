"""A seeded sweep of random shapes through the separate calls, the fused step and the paged
step, each against the CPU oracle.

The hand-picked cases elsewhere pin one feature at a time; here the features are drawn
together: batch, tree size and shape, query heads per K/V head, head size, input type, prefix
lengths (empty, tile multiples and one either side, ragged) and the split-K setting.  Every
output row is compared; the fused step must also equal the separate calls bit for bit.  The
shapes come from a fixed seed, so a failure names a case that runs again the same way.

Short prefixes leave early tree nodes with one to a few keys, so an output row is close to a
single V row and reaches |o| of 4 to 5 even at the default scale: those rows carry the bf16
output rounding and the bf16 rounding of P at that size, and the sweep holds every output to
the sharp-row bar of the dtype's max-abs tolerance plus 2^-7 |o| (bf16).
"""
import numpy as np
import pytest
import torch

from gpu_util import RTOL_SHARP, check_step, run_step, run_step_fused, upload
from synth import make_paged, make_workload

pytestmark = pytest.mark.gpu

T_CHOICES = [1, 2, 7, 31, 32, 33, 60, 63, 64, 65, 96, 127, 128]
L_CHOICES = [0, 1, 63, 64, 65, 127, 128, 129, 500, 1023, 1300]
SPLITS = [0, 0, 64, 128, 320, 100000]


def _draw(i: int, paged: bool = False) -> dict:
    r = np.random.default_rng(np.random.SeedSequence([2024, 1 if paged else 0, i]))
    T = int(r.choice(T_CHOICES)) if r.random() < 0.6 else int(r.integers(1, 129))
    lo, hi = sorted(int(x) for x in r.choice(L_CHOICES, 2))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 3, 4, 5, 8]))
    return dict(B=int(r.integers(1, 7)), T=T, L=(lo, hi), Hkv=Hkv, Hq=Hkv * G,
                D=int(r.choice([64, 128])), dtype="f32" if r.random() < 0.25 else "bf16",
                parent_kind=str(r.choice(["random", "deep", "chain", "star"]))), \
        int(r.choice(SPLITS))


N_CONTIG, N_PAGED = 96, 32


def _draw_groups(i: int) -> tuple[dict, int]:
    """Large query-head groups (multi-query shapes among them): G * T spans one to 16 row
    blocks of 256 rows, with a ragged last block."""
    r = np.random.default_rng(np.random.SeedSequence([2024, 2, i]))
    G = int(r.choice([6, 7, 12, 16, 24, 32, 48, 64]))
    T = int(r.integers(1, min(128, 4096 // G) + 1))
    lo, hi = sorted(int(x) for x in r.choice(L_CHOICES, 2))
    Hkv = int(r.choice([1, 1, 2]))
    return dict(B=int(r.integers(1, 4)), T=T, L=(lo, hi), Hkv=Hkv, Hq=Hkv * G,
                D=int(r.choice([64, 128])), dtype="f32" if r.random() < 0.25 else "bf16",
                parent_kind=str(r.choice(["random", "deep", "chain", "star"]))), \
        int(r.choice(SPLITS))


N_GROUPS = 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_attn_amd as tv

    tv.load_library()


@pytest.mark.parametrize("i", range(N_CONTIG))
def test_sweep_contiguous(i):
    kw, split_keys = _draw(i)
    w = make_workload("batch32_L512-4096_T60", extra_seed=500 + i, **kw)
    print(f"[case] sweep {i}: {kw} split_keys={split_keys}", flush=True)
    a = run_step(upload(w), split_keys=split_keys)
    stats = check_step(w, a, label=f"sweep {i}", rtol=RTOL_SHARP[w.dtype])
    print(f"       max-abs err {stats['err']:.3e}  lse err {stats['lse_err']:.3e}", flush=True)
    b = run_step_fused(upload(w), split_keys=split_keys)
    for k in a:  # bytes: the caches hold NaN-poisoned rows past every prefix
        x, y = np.ascontiguousarray(a[k]), np.ascontiguousarray(b[k])
        assert x.shape == y.shape and np.array_equal(x.view(np.uint8), y.view(np.uint8)), \
            f"sweep {i}: fused {k}"


@pytest.mark.parametrize("i", range(N_GROUPS))
def test_sweep_large_groups(i):
    kw, split_keys = _draw_groups(i)
    w = make_workload("batch32_L512-4096_T60", extra_seed=900 + i, **kw)
    print(f"[case] sweep groups {i}: {kw} split_keys={split_keys}", flush=True)
    a = run_step(upload(w), split_keys=split_keys)
    stats = check_step(w, a, label=f"sweep groups {i}", rtol=RTOL_SHARP[w.dtype])
    print(f"       max-abs err {stats['err']:.3e}  lse err {stats['lse_err']:.3e}", flush=True)
    b = run_step_fused(upload(w), split_keys=split_keys)
    for k in a:
        x, y = np.ascontiguousarray(a[k]), np.ascontiguousarray(b[k])
        assert x.shape == y.shape and np.array_equal(x.view(np.uint8), y.view(np.uint8)), \
            f"sweep groups {i}: fused {k}"


@pytest.mark.parametrize("i", range(N_PAGED))
def test_sweep_paged(i):
    from test_gpu_step_paged import _fused, _oracle_check, _same, _separate

    kw, split_keys = _draw(i, paged=True)
    w = make_workload("batch32_L512-4096_T60", extra_seed=700 + i, **kw)
    pl = make_paged(w, 1, seed=20 + i)
    print(f"[case] sweep paged {i}: {kw} split_keys={split_keys}", flush=True)
    res = _fused(w, pl, split_keys=split_keys, spare_top=1)
    _oracle_check(w, pl, res, spare_top=1, rtol=RTOL_SHARP[w.dtype])
    _same(res, _separate(w, pl, split_keys=split_keys, spare_top=1), spare_top=1)
