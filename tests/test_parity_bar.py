"""The GPU parity bar itself, checked on the CPU: the bracketing bf16 values
come out bf16-representable, enclose the reference, and have no bf16 value
strictly between them (checked against bf16's bit patterns, not against the
formula that computes them)."""
import torch

from gpu_harness import TOL, bf16_brackets, within_bar


def _next_up(x: torch.Tensor) -> torch.Tensor:
    """The next bf16 value above each bf16 value (finite, nonzero inputs), by
    stepping the 16-bit pattern: +1 for positive values, -1 for negative."""
    bits = x.to(torch.bfloat16).view(torch.int16).to(torch.int32)
    step = torch.where(x > 0, 1, -1)
    return (bits + step).to(torch.int16).view(torch.bfloat16).double()


def test_brackets_are_adjacent_bf16_values():
    g = torch.Generator().manual_seed(0)
    mags = torch.exp2(torch.empty(20000, dtype=torch.float64).uniform_(-130, 100, generator=g))
    sign = torch.where(torch.rand(20000, generator=g) < 0.5, -1.0, 1.0).double()
    ref = mags * sign
    ref = torch.cat([ref, torch.tensor([1.0, -4.0, 2.0**-126, 3.0, 0.1, -0.1], dtype=torch.float64)])
    lo, hi = bf16_brackets(ref)
    assert torch.equal(lo.to(torch.bfloat16).double(), lo)
    assert torch.equal(hi.to(torch.bfloat16).double(), hi)
    assert (lo <= ref).all() and (ref <= hi).all()
    exact = lo == hi
    assert torch.equal(exact, ref.to(torch.bfloat16).double() == ref)
    nz = (~exact) & (lo != 0)
    assert torch.equal(_next_up(lo[nz]), hi[nz])


def test_correct_rounding_always_passes_and_two_steps_off_fails():
    g = torch.Generator().manual_seed(1)
    ref = torch.empty(50000, dtype=torch.float64).uniform_(-40, 40, generator=g)
    rounded = ref.to(torch.bfloat16).double()
    assert within_bar(rounded, ref).all()
    lo, hi = bf16_brackets(ref)
    # two bf16 steps above the upper bracket: accepted only if within TOL
    far = _next_up(_next_up(hi[hi > 0]))
    r = ref[hi > 0]
    ok = within_bar(far, r)
    assert torch.equal(ok, (far - r).abs() <= TOL)
    assert (~ok[r.abs() >= 2]).all()


def test_tolerance_clause():
    ref = torch.tensor([0.5, 0.5, 0.5], dtype=torch.float64)
    got = torch.tensor([0.5 + 0.0099, 0.5 - 0.0099, 0.5 + 0.0101], dtype=torch.float64)
    assert within_bar(got, ref).tolist() == [True, True, False]
