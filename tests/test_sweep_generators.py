"""The random-sweep problem generators (CPU): each one stays inside the shapes
it states, so that a sweep log's claim about what it covered holds."""
import sweep_random_wide as sw


def _common(p):
    assert 1 <= p["Lq"] and 1 <= p["Lkv"] and p["H"] % p["Hkv"] == 0
    assert (not p["causal"]) or p["Lq"] <= p["Lkv"], "causal needs Lq <= Lkv (bottom-right alignment)"
    assert p["d"] in (64, 128) and p["o"] in ("f16", "f32") and p["dt"] in ("f16", "f32")
    if p["outliers"]:
        assert all(0 <= c < p["d"] for c in p["outliers"]) and 1 <= len(p["outliers"]) <= max(1, round(0.02 * p["d"]))


def test_wide_problems():
    for i in range(1, 3001):
        p = sw.problem(i)
        _common(p)
        assert p["Lq"] <= 2000 and p["Lkv"] <= 3000 and p["H"] // p["Hkv"] in (1, 2, 4, 8)


def test_decode_problems_take_the_split_path():
    for i in range(2001):
        p = sw.decode_problem(i)
        _common(p)
        assert (p["H"] // p["Hkv"]) * p["Lq"] <= 16 and p["Lkv"] <= 20000 and p["Lq"] <= 4


def test_index_softmax_problems():
    decode = 0
    for i in range(2001):
        p = sw.lut_problem(i)
        _common(p)
        assert 1 <= p["bits"] <= 8 and 0.5 <= p["clip"] <= 8.0 and p["vmode"] in ("tensor", "head", "channel")
        decode += (p["H"] // p["Hkv"]) * p["Lq"] <= 16
    assert 400 <= decode <= 900          # about 30 % decode shapes


def test_int4_and_hadamard_problems():
    for gen in (sw.int4_problem, sw.hadamard_problem):
        for i in range(2001):
            p = gen(i)
            _common(p)
            assert p["vmode"] in ("tensor", "token", "head", "channel")
