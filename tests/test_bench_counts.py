"""The algorithmic flop counts that bench.py prices the four-stage
Rosenbrock gradient kernels with (Robertson, d = 3), derived here from the
coefficient tables' nonzero patterns under the arithmetic schedule both
sides use: a zero coefficient costs nothing; a sum of coefficient terms is a
product, then multiply-adds (FMA = 2 flops); the stage right-hand side adds
gamma h f(Y_i) last (a product when no other term is present); the error
estimate is a product, then multiply-adds.  The per-stage parts that do not
depend on the table (Jacobian 9, W 13, LU 13, four right-hand sides 4 x 13,
four solves 4 x 15; in reverse four transposed solves 60, Wbar 63, fbar 12,
the vector-Jacobian products at four stages 132, ybar sums 12, Jbar 9 and
the dJ contraction 29) are the same for every four-stage table.

A stage whose row of A equals the previous stage's (the fourth-order method's
a_4j = a_3j) is evaluated at the same point: the algorithmic count gives it
no stage sum and no right-hand side of its own, and in reverse one
vector-Jacobian product of the two stages' summed cotangents (3 additions)
and no a_ij terms of its own in the stage cotangents."""
import importlib.util
import os
from fractions import Fraction as Fr

from test_oracle_pins import ROS4_A, ROS4_C, ROS4_E, ROS4_M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Rodas3's nonzero pattern (gamma = 1/2): a_31 = a_41 = 2, a_43 = 1; c_21 = 4,
# c_31 = 1, c_32 = -1, c_41 = 1, c_42 = -1, c_43 = -8/3; m = (2, 0, 1, 1);
# e = (0, 0, 0, 1).  Indices from 0.
RODAS3_A = {(2, 0): Fr(2), (3, 0): Fr(2), (3, 2): Fr(1)}
RODAS3_C = {(1, 0): Fr(4), (2, 0): Fr(1), (2, 1): Fr(-1), (3, 0): Fr(1), (3, 1): Fr(-1),
            (3, 2): Fr(-8, 3)}
RODAS3_M = [Fr(2), Fr(0), Fr(1), Fr(1)]
RODAS3_E = [Fr(0), Fr(0), Fr(0), Fr(1)]


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _sum_cost(terms):
    return 0 if terms == 0 else 2 * terms - 1


def _shared(A, i):
    """Stage i sits at the previous stage's point: the same row of A."""
    return i >= 2 and all(A.get((i, j), 0) == A.get((i - 1, j), 0) for j in range(i))


def _counts(A, C, M, E, d=3):
    nz = lambda tab, i, j: tab.get((i, j), 0) != 0
    points = [i for i in range(4) if not _shared(A, i)]
    fwd = 9 + 13 + 13 + len(points) * 13 + 4 * 15
    fwd += d * 2 * sum(1 for (i, j), v in A.items() if v != 0 and i in points)  # Y_i sums
    for i in range(4):                                                   # stage rhs
        g = sum(1 for j in range(i) if nz(C, i, j))
        fwd += d * (1 if g == 0 else 2 * g + 1)
    fwd += d * 2 * sum(1 for m in M if m != 0)                           # y+
    fwd += d * _sum_cost(sum(1 for e in E if e != 0))                    # error
    adj = 60 + 63 + 12 + len(points) * 33 + d * (4 - len(points)) + 12 + 9 + 29
    for i in range(4):                                                   # stage cotangents
        terms = (M[i] != 0) + sum((nz(A, l, i) and l in points) + nz(C, l, i)
                                  for l in range(i + 1, 4))
        adj += d * _sum_cost(terms)
    return fwd, adj


def test_shared_stage_point_of_the_fourth_order_method():
    """Only the fourth-order method has a stage at its predecessor's point."""
    assert [i for i in range(4) if _shared(ROS4_A, i)] == [3]
    assert not any(_shared(RODAS3_A, i) for i in range(4))
    assert _counts(ROS4_A, ROS4_C, ROS4_M, ROS4_E) == (239, 353)


def test_rosenbrock4_flop_counts_match_bench():
    b = _bench()
    for name, tab in (("rodas3", (RODAS3_A, RODAS3_C, RODAS3_M, RODAS3_E)),
                      ("ros4", (ROS4_A, ROS4_C, ROS4_M, ROS4_E))):
        fwd, adj = _counts(*tab)
        assert b.fwd_flop_per_step(name, "robertson", 3) == fwd, name
        assert b.flop_per_step(name, "robertson", 3) == fwd + adj, name
