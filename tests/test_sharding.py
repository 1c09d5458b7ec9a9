"""Host logic of the sharded step's matrix ownership (no GPU)."""
import pytest

from workloads import CONFIGS, matrix_flops, owner_split


def test_gpt2_124m_on_8_ranks_balanced():
    shapes = CONFIGS["gpt2_124m_matrix_set"].shapes
    owned = owner_split(shapes, 8)
    flat = sorted(i for o in owned for i in o)
    assert flat == list(range(len(shapes)))           # each matrix exactly once
    for o in owned:                                     # 6 square + 3 MLP matrices each
        sq = sum(1 for i in o if shapes[i][0] == shapes[i][1])
        assert (sq, len(o) - sq) == (6, 3)
    loads = [sum(matrix_flops(*shapes[i]) for i in o) for o in owned]
    assert max(loads) == min(loads)                     # equal by construction here


def test_balance_bound_and_determinism():
    shapes = [(768, 768)] * 5 + [(1024, 4096)] * 3 + [(300, 200), (64, 128), (2048, 512)]
    for world in (1, 2, 3, 5, 16):
        owned = owner_split(shapes, world)
        assert owned == owner_split(shapes, world)
        assert sorted(i for o in owned for i in o) == list(range(len(shapes)))
        loads = [sum(matrix_flops(*shapes[i]) for i in o) for o in owned]
        # greedy longest-first: the spread is at most the largest single matrix
        assert max(loads) - min(loads) <= max(matrix_flops(*s) for s in shapes)
    assert owner_split(shapes, 1) == [list(range(len(shapes)))]
    assert sum(1 for o in owner_split(shapes, 16) if not o) == 16 - len(shapes)


def test_matrix_flops_convention():
    # m(m+1)n + m^2(m+1) + 2m^2 n with m = min, n = max; orientation-free
    assert matrix_flops(2, 3) == 2 * 3 * 3 + 4 * 3 + 2 * 4 * 3
    assert matrix_flops(3072, 768) == matrix_flops(768, 3072)
    with pytest.raises(ValueError):
        owner_split([(2, 2)], 0)
