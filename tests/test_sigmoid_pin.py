"""The router's sigmoid is one fixed fp64 evaluation that the oracle and the
HIP kernel each implement (routing ids are integers decided by floating
point, so they must agree bit for bit).  The kernel holds its constants as
hex literals; the oracle derives them at run time from log(2) and k!.  This
pins the two sets equal, bit for bit: a constant mistyped on either side
changes some sigmoid by an ulp, which the id comparisons alone catch only
at rare near-ties."""
import os
import re

import numpy as np

import oracle

ROUTE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "routing_dispatch_grouped_amd", "csrc", "route.hip")


def _kernel_constants():
    src = open(ROUTE).read()
    hexf = r"(0x[0-9a-fA-F]\.[0-9a-fA-F]+p[+-]\d+)"
    one = {}
    for name in ("kLog2e", "kLn2Hi", "kLn2Lo"):
        m = re.search(r"constexpr double %s = %s;" % (name, hexf), src)
        assert m, name
        one[name] = float.fromhex(m.group(1))
    m = re.search(r"constexpr double kInvFact\[14\] = \{([^}]*)\}", src, re.S)
    assert m
    fact = [float.fromhex(v) for v in re.findall(hexf, m.group(1))]
    assert len(fact) == 14
    return np.array([one["kLog2e"], one["kLn2Hi"], one["kLn2Lo"]] + fact)


def test_kernel_sigmoid_constants_equal_the_oracles():
    got = _kernel_constants()
    ref = oracle.sigmoid_constants()
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), (got, ref)


def test_constants_from_their_definitions():
    # independent of both implementations: Python's own double arithmetic
    import math
    c = oracle.sigmoid_constants()
    assert c[0] == 1.0 / math.log(2.0)
    hi, lo = c[1], c[2]
    assert hi + lo == math.log(2.0) and hi == float.fromhex("0x1.62e42fefa38p-1")
    m, e = math.frexp(hi)
    assert (m * 2.0 ** 42) == int(m * 2.0 ** 42)      # 42 significant bits: n * hi is exact for |n| < 2^11
    for k in range(14):
        assert c[3 + k] == 1.0 / math.factorial(k)
