"""Host-side checks of the C-ABI library (no GPU needed, no compute calls):
exported symbols, status strings, argument validation, workspace sizing and
the work schedules of every kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

import muon_newton_schulz_04_amd as mu
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mu.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return mu.load_library()


def header_functions():
    names = set()
    for h in HEADERS:
        src = open(h).read()
        names |= set(re.findall(r"^[A-Za-z_][\w \*]*?\b(muon_\w+)\s*\(", src, re.M))
    return sorted(names)


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) >= 18
    for n in ("muon_adam_plan_create", "muon_plan_step_apply", "muon_plan_set_weights"):
        assert n in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/*.h but not exported"


def test_abi_version_and_status_strings(lib):
    assert mu.muon_abi_version() == 4
    for code in range(10):
        s = mu.muon_status_str(code)
        assert s and s != "unknown status"
    assert mu.muon_status_str(99) == "unknown status"


def arr_of(rows_cols_ld_ptrs):
    arr = (mu.MuonMatrix * max(1, len(rows_cols_ld_ptrs)))()
    for i, t in enumerate(rows_cols_ld_ptrs):
        arr[i] = mu.MuonMatrix(*t)
    return arr


def ws_status(lib, mats, dtype=mu.MUON_BF16, n=None):
    out = ctypes.c_size_t(0)
    return lib.muon_workspace_bytes(arr_of(mats), len(mats) if n is None else n, dtype,
                                    ctypes.byref(out)), out.value


B = 1 << 40


@pytest.mark.parametrize("mats,want", [
    ([(-1, 4, 4, B, B + 4096, B + 8192)], 3),               # negative rows
    ([(4, 8, 4, B, B + 4096, B + 8192)], 3),                # ld < cols
    ([(70000, 8, 8, B, B + 4 << 20, B + 8 << 20)], 3),      # rows > max dim
    ([(40000, 40000, 40000, B, B + (4 << 32), B + (8 << 32))], 3),  # too many elements
    ([(4, 8, 8, 0, B, B + 4096)], 1),                       # NULL grad
    ([(4, 8, 8, B, B + 4096, 0)], 1),                       # NULL out
    ([(4, 8, 8, B + 1, B + 4096, B + 8192)], 4),            # misaligned grad
    ([(4, 8, 8, B, B + 4096, B + 40)], 1),                  # out overlaps grad (not equal)
    ([(4, 8, 8, B, B + 40, B + 8192)], 1),                  # momentum overlaps grad
    ([(4, 8, 8, B, B + 4096, B + 8192), (4, 8, 8, B + 8192, B + 12288, B + 16384)], 1),  # out0 = grad1
])
def test_validation_errors(lib, mats, want):
    st, _ = ws_status(lib, mats)
    assert st == want


def test_validation_accepts_aliasing_out_and_grad_and_empty(lib):
    st, nb = ws_status(lib, [(4, 8, 8, B, B + 4096, B)])
    assert st == 0 and nb > 0
    st, nb = ws_status(lib, [(0, 8, 8, B, B + 4096, B + 8192), (5, 0, 0, 0, 0, 0)])
    assert st == 0 and nb == 0
    st, nb = ws_status(lib, [], n=0)
    assert st == 0 and nb == 0
    assert ws_status(lib, [(4, 8, 8, B, B + 4096, B + 8192)], dtype=7)[0] == 2
    assert ws_status(lib, [(4, 8, 8, B, B + 4096, B + 8192)], n=-1)[0] == 3


def test_config_validation_before_any_device_call(lib):
    mats = arr_of([(4, 8, 8, B, B + 4096, B + 8192)])
    bad = [mu.make_config(1, 0, 0, 65), mu.make_config(1, 0, 0, -1),
           mu.make_config(float("nan"), 0, 0, 1), mu.make_config(1, 0, 0, 1, momentum=1.0),
           mu.make_config(1, 0, 0, 1, momentum=-0.1), mu.make_config(1, 0, 0, 1, eps=-1.0),
           mu.make_config(1, 0, 0, 1, precision=1)]          # only the default operand format
    for cfg in bad:
        assert lib.muon_step(mats, 1, mu.MUON_BF16, ctypes.byref(cfg), None, 0, None) == 1
    cfg = mu.make_config(1, 0, 0, 1, momentum=0.9)
    nomom = arr_of([(4, 8, 8, B, 0, B + 8192)])   # momentum NULL with mu != 0
    assert lib.muon_step(nomom, 1, mu.MUON_BF16, ctypes.byref(cfg), None, 0, None) == 1
    assert lib.muon_step(mats, 1, mu.MUON_BF16, None, None, 0, None) == 1
    assert lib.muon_plan_step(None, ctypes.byref(cfg), None, 0, None) == 1


def test_coefficient_range_check_for_bf16_sets(lib):
    """bf16 sets refuse coefficients that take a point of [0, 1] outside
    [-2, 2] within the configured steps (fp16 operands, the low byte of X),
    or whose B = b A + c A A could leave fp16's range; fp32 sets take any
    finite coefficients. Every coefficient set the workloads use passes."""
    mats = arr_of([(4, 8, 8, B, B + 4096, B + 8192)])
    ok = [mu.make_config(3.4445, -4.7750, 2.0315, 5), mu.make_config(1.5, -0.5, 0.0, 10),
          mu.make_config(3.4445, -4.7750, 2.0315, 64), mu.make_config(1.0, 0.0, 0.0, 64),
          mu.make_config(0.0, 1.0, 0.0, 1), mu.make_config(0.0, 0.0, 1.0, 1),
          mu.make_config(2.0, 0.0, 0.0, 1), mu.make_config(-1.0, 0.0, 0.0, 3)]
    bad = [mu.make_config(2.0, 0.0, 0.0, 2),          # 4 x after two steps
           mu.make_config(3.0, 0.0, 0.0, 1),          # 3 x
           mu.make_config(3.4445, 0.0, 0.0, 1),       # the quintic's linear term alone
           mu.make_config(0.0, 0.0, 300.0, 0),        # 16 |c| > 4096, even with zero steps
           mu.make_config(1.0, 2000.0, -2000.0, 1)]   # 4|b| + 16|c| too large
    # mats has a NULL-free set but no workspace: a config that passes
    # validation then fails on the workspace (5), one that does not fails
    # with MUON_E_INVALID (1), before any device call
    for cfg in ok:
        assert lib.muon_step(mats, 1, mu.MUON_BF16, ctypes.byref(cfg), None, 0, None) == 5
    for cfg in bad:
        assert lib.muon_step(mats, 1, mu.MUON_BF16, ctypes.byref(cfg), None, 0, None) == 1
        assert lib.muon_step(mats, 1, mu.MUON_F32, ctypes.byref(cfg), None, 0, None) == 5


def expected_ws(shapes, dtype):
    def ru(x, m):
        return (x + m - 1) // m * m
    parts = 0
    for r, c in shapes:
        rpi = max(1, 16384 // c)
        parts += (r + rpi - 1) // rpi
    off = ru(parts * 8, 256)        # partial sums of u^2 and their exponents
    if dtype == mu.MUON_BF16:
        # per 64 x 64 tile of each padded matrix: sum of u^2 and largest |u|;
        # per matrix: {sigma, p, p guessed, 0}
        tiles = sum(ru(min(r, c), 256) // 64 * (ru(max(r, c), 256) // 64)
                    for r, c in shapes if r and c)
        if tiles:
            off = ru(off + tiles * 4, 256)
            off = ru(off + tiles * 4, 256)
            off = ru(off + len(shapes) * 16, 256)
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        t = 256 if dtype == mu.MUON_BF16 else 128
        mp, np_ = ru(m, t), ru(n, t)
        sizes = ([mp * np_, mp * np_ * 2, mp * np_ * 2, mp * mp * 2, mp * mp * 2]
                 if dtype == mu.MUON_BF16 else
                 [mp * np_ * 4, mp * np_ * 4, mp * mp * 4, mp * mp * 4])
        for s in sizes:
            off = ru(off + s, 256)
    # split Gram tiles: one 256 x 256 fp32 partial tile per part, at the end
    if dtype == mu.MUON_BF16:
        red = split_reduce_items(shapes)
        nparts = int(red[:, 3].astype(np.int64).__and__(255).sum()) // 4 if len(red) else 0
        if nparts:
            off = ru(off + nparts * 256 * 256 * 4, 256)
        # chained schedule: a ticket counter per XCD and a completion
        # counter per matrix (int32)
        if len(chain_items(shapes)):
            off = ru(off + (8 + len(shapes)) * 4, 256)
    return off


def chain_items(shapes):
    """The chained schedule's lists (schedule kind MUON_K_COUNT + 2)."""
    return mu.muon_schedule_query(shapes, mu.MUON_BF16, 7)


def split_reduce_items(shapes):
    """The reduce items of split Gram tiles (schedule kind MUON_K_COUNT)."""
    s = mu.muon_schedule_query(shapes, mu.MUON_BF16, 5)
    return s[s[:, 0] >= 0] if len(s) else s


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workspace_bytes_formula(lib, name):
    cfg = CONFIGS[name]
    dt = mu.MUON_F32 if cfg.dtype == "fp32" else mu.MUON_BF16
    assert mu.muon_workspace_bytes(list(cfg.shapes), dt) == expected_ws(cfg.shapes, dt)


def test_gram_split_only_where_the_longest_tiles_dominate(lib):
    """Split Gram tiles: the one-block set (two 768 x 3072 matrices among
    four 768^2) splits its 96-stage tiles into 24-stage parts; the full
    GPT-2-124M set (work per CU above half the longest tile) does not split."""
    small = list(CONFIGS["gpt2_small_block"].shapes)
    red = split_reduce_items(small)
    assert len(red) == 4 * 12 and set(red[:, 3] & 255) == {4}
    assert set(max(small[i]) for i in red[:, 0]) == {3072}
    assert len(split_reduce_items(list(CONFIGS["gpt2_124m_matrix_set"].shapes))) == 0
    assert len(mu.muon_schedule_query(small, mu.MUON_F32, 5)) == 0   # fp32 sets never split


SHAPE_SETS = {
    "gpt2_124m": list(CONFIGS["gpt2_124m_matrix_set"].shapes),
    "ragged": [(200, 333), (333, 200), (1, 1), (129, 129), (64, 128), (700, 50)],
    "one_big": [(4096, 1024)],
}


@pytest.mark.parametrize("dtype", [mu.MUON_BF16, mu.MUON_F32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("setname", list(SHAPE_SETS))
def test_schedules_cover_every_tile_exactly_once(lib, setname, dtype):
    check_schedules(SHAPE_SETS[setname], dtype)


def test_schedules_of_random_sets(lib):
    """The same invariants on seeded random sets (1 to 12 matrices, sides 1
    to 9000, some of them split their Gram tiles)."""
    rng = np.random.default_rng(2024)
    for _ in range(25):
        k = int(rng.integers(1, 13))
        shapes = [(int(rng.integers(1, 3000)), int(rng.integers(1, 9000))) for _ in range(k)]
        shapes = [(r, c) if rng.random() < 0.5 else (c, r) for r, c in shapes]
        for dtype in (mu.MUON_BF16, mu.MUON_F32):
            check_schedules(shapes, dtype)
            assert mu.muon_workspace_bytes(shapes, dtype) == expected_ws(shapes, dtype)


def check_schedules(shapes, dtype):
    tm = tn = 256 if dtype == mu.MUON_BF16 else 128
    scheds = [mu.muon_schedule_query(shapes, dtype, k) for k in (0, 1, 2, 3, 4, 6)]
    for k, s in enumerate(scheds):
        assert len(s) % 8 == 0, "grid is a multiple of the XCD count"
        empty = s[:, 0] < 0
        assert np.all(s[empty] == -1)
    mom, nrm, gram, poly, upd, scale = (s[s[:, 0] >= 0] if len(s) else np.zeros((0, 4), int)
                                        for s in scheds)
    slots = mom[:, 3]
    assert len(np.unique(slots)) == len(slots) and slots.min() == 0 and slots.max() == len(slots) - 1
    for i, (r, c) in enumerate(shapes):
        m, n = min(r, c), max(r, c)
        mp, np_ = -(-m // tm) * tm, -(-n // tn) * tn
        mi = mom[mom[:, 0] == i]
        rows = np.zeros(r, int)
        for _, r0, nr, _s in mi:
            rows[r0:r0 + nr] += 1
        assert np.all(rows == 1), "every row summed exactly once"
        ni = nrm[nrm[:, 0] == i]
        assert sorted(map(tuple, ni[:, 1:3])) == [(a, b) for a in range(mp // 64) for b in range(np_ // 64)]
        # tiles that reach the upper triangle, and every upper element in exactly one
        want_tri = [(a, b) for a in range(mp // tm) for b in range(mp // tn)
                    if b * tn + tn - 1 >= a * tm]
        # gram: a tile is one item (c = 0) or S parts (c = pbase << 16 | sp << 8 | S,
        # sp = 0 .. S-1, S dividing the tile's stages / 8) plus one reduce item
        gi = gram[gram[:, 0] == i]
        tiles = {}
        for _, a, b, c in gi:
            tiles.setdefault((a, b), []).append(int(c))
        assert sorted(tiles) == want_tri
        red_i = split_reduce_items(shapes) if dtype == mu.MUON_BF16 else np.zeros((0, 4), int)
        red = {}
        for m_, a, b, c in red_i:
            if m_ == i:
                red.setdefault((int(a), int(b)), []).append(int(c))
        for t, cs in red.items():      # four quarters per split tile, same pbase and S
            assert sorted((c >> 8) & 255 for c in cs) == [0, 1, 2, 3]
            assert len({c & ~0xff00 for c in cs}) == 1
        red = {t: cs[0] & ~0xff00 for t, cs in red.items()}
        for t, cs in tiles.items():
            if cs == [0]:
                assert t not in red
                continue
            S = cs[0] & 255
            assert S >= 2 and (np_ // 32 // 8) % S == 0 and len(cs) == S
            assert sorted((c >> 8) & 255 for c in cs) == list(range(S))
            assert len({c >> 16 for c in cs}) == 1 and red[t] == ((cs[0] >> 16) << 16 | S)
        assert set(red) <= set(tiles)
        for s in (gram, poly):
            si = s[s[:, 0] == i]
            cover = np.zeros((mp, mp), int)
            for _, a, b, c in si:
                if s is gram and (c & 255) >= 2 and (c >> 8) & 255:
                    continue                      # count each split tile once
                cover[a * tm:(a + 1) * tm, b * tn:(b + 1) * tn] += 1
            assert np.all(np.triu(cover) == np.triu(np.ones((mp, mp), int)))
        pi = poly[poly[:, 0] == i]
        assert sorted(map(tuple, pi[:, 1:3])) == want_tri
        ui = upd[upd[:, 0] == i]
        assert sorted(map(tuple, ui[:, 1:3])) == [(a, b) for a in range(mp // tm) for b in range(np_ // tn)]
        # scale pass (bf16): one item {i, 0, 0, 0} per matrix
        si = scale[scale[:, 0] == i]
        if dtype == mu.MUON_BF16 and m > 0:
            assert si.tolist() == [[i, 0, 0, 0]]
        else:
            assert len(si) == 0
    if dtype == mu.MUON_BF16:
        spans = sorted({(c >> 16, (c >> 16) + (c & 255)) for *_, c in split_reduce_items(shapes)})
        assert all(e0 <= b1 for (_, e0), (b1, _) in zip(spans, spans[1:]))   # disjoint partial slots
        check_chain(shapes, gram, poly, upd)


def check_chain(shapes, gram, poly, upd):
    """The chained schedule, where the set has one: every Gram, poly and
    update tile of a step exactly once, all tiles of a matrix on one XCD,
    each tile's wait count the number of its matrix's tiles in the earlier
    kernels of the step, and every tile listed after all tiles it waits for
    (so a workgroup only ever waits for lower tickets)."""
    ch = chain_items(shapes)
    if len(ch) == 0:
        return
    assert len(split_reduce_items(shapes)) == 0, "split Gram tiles are never chained"
    mats, tile, xk, need = ch[:, 0], ch[:, 1], ch[:, 2], ch[:, 3]
    xcd, kind = xk >> 8, xk & 255
    assert np.all(np.diff(xcd) >= 0) and xcd.min() >= 0 and xcd.max() < 8, "lists in XCD order"
    assert set(kind.tolist()) <= {2, 3, 4}
    nonempty = [i for i, (r, c) in enumerate(shapes) if min(r, c) > 0]
    assert sorted(set(mats.tolist())) == nonempty
    for i in nonempty:
        sel = mats == i
        assert len(set(xcd[sel].tolist())) == 1, "one XCD per matrix"
        want = {2: gram, 3: poly, 4: upd}
        counts = {}
        for k, src in want.items():
            got = sorted(((t >> 16) & 0xffff, t & 0xffff) for t in tile[sel & (kind == k)])
            exp = sorted(map(tuple, src[src[:, 0] == i][:, 1:3].tolist()))
            assert got == exp, (i, k)
            counts[k] = len(exp)
        before = {2: 0, 3: counts[2], 4: counts[2] + counts[3]}
        assert all(need[j] == before[kind[j]] for j in np.flatnonzero(sel))
        pos = np.flatnonzero(sel)
        k_of = kind[pos]
        for k in (3, 4):
            if np.any(k_of == k):
                assert pos[k_of < k].max(initial=-1) < pos[k_of == k].min(), "dependencies listed first"


def test_schedule_query_kinds(lib):
    """Kinds 0 .. MUON_K_COUNT + 2 (the split-Gram sums, the scale pass of X0
    and the chained schedule) are queried; anything else is MUON_E_INVALID,
    before any work."""
    shapes = [(200, 333), (768, 768)]
    for kind in range(8):
        mu.muon_schedule_query(shapes, mu.MUON_BF16, kind)
    for kind in (-1, 8, 100):
        with pytest.raises(mu.MuonError) as e:
            mu.muon_schedule_query(shapes, mu.MUON_BF16, kind)
        assert e.value.code == 1
    # the scale pass exists for bf16 sets only, one item per non-empty matrix
    s = mu.muon_schedule_query(shapes + [(0, 64)], mu.MUON_BF16, 6)
    assert sorted(s[s[:, 0] >= 0][:, 0].tolist()) == [0, 1]
    assert len(mu.muon_schedule_query(shapes, mu.MUON_F32, 6)) == 0


def test_chained_schedule_where_the_set_spreads_over_the_xcds(lib):
    """Chained: bf16 sets of at least eight matrices whose work spreads
    evenly over the XCDs and whose update launch is under 24 waves of 256
    tiles (the GPT-2-124M and 350M sets); not: deeper sets (the 2048 x 8192
    set, 64 waves), fp32 sets, sets of fewer matrices, sets that split Gram
    tiles."""
    for name in ("gpt2_124m_matrix_set", "gpt2_350m_matrix_set"):
        ch = chain_items(list(CONFIGS[name].shapes))
        assert len(ch) > 0, name
        per_xcd = np.bincount(ch[:, 2] >> 8, minlength=8)
        assert per_xcd.max() <= 1.25 * per_xcd.mean(), name
    assert len(chain_items(list(CONFIGS["wide_2048x8192_powerlaw"].shapes))) == 0
    assert len(chain_items([(2048, 8192)] * 23)) > 0        # 23 waves
    assert len(chain_items([(2048, 8192)] * 24)) == 0       # 24 waves
    assert len(chain_items(list(CONFIGS["gpt2_small_block"].shapes))) == 0
    assert len(chain_items([(768, 768)] * 7)) == 0
    assert len(mu.muon_schedule_query([(768, 768)] * 16, mu.MUON_F32, 7)) == 0
    # one huge matrix beside small ones cannot spread evenly
    assert len(chain_items([(8192, 8192)] + [(256, 256)] * 8)) == 0


def test_gram_schedule_balances_xcds_and_keeps_matrices_together(lib):
    shapes = SHAPE_SETS["gpt2_124m"]
    s = mu.muon_schedule_query(shapes, mu.MUON_BF16, 2)
    cost = np.zeros(8)
    owner = {}
    split = 0
    for b, (mat, ti, tj, _) in enumerate(s):
        if mat < 0:
            continue
        x = b % 8
        cost[x] += max(shapes[mat])      # all tiles have the same area
        if owner.setdefault(mat, x) != x:
            split += 1
    assert cost.max() / cost.mean() < 1.1
    assert split <= 8


# ------------------------------------------------------------------ Adam branch (host only)

def adam_list(specs):
    """muon_adam_tensor array from (numel, param, grad, m, v) placeholder
    addresses (never dereferenced: only host validation runs)."""
    arr = (mu.MuonAdamTensor * max(len(specs), 1))()
    for i, (n, p, g, m, v) in enumerate(specs):
        arr[i] = mu.MuonAdamTensor(n, p, g, m, v, 1.0, 1.0)
    return arr, len(specs)


B = 1 << 40


@pytest.mark.parametrize("specs,want", [
    ([(100000, B, B + 2 ** 20, B + 2 ** 21, B + 2 ** 22), (7, B + 2 ** 23, B + 2 ** 24,
                                                          B + 2 ** 25, B + 2 ** 26)], 0),
    ([(-1, B, B + 4096, B + 8192, B + 12288)], 3),                         # negative size
    ([(2 ** 31 + 1, B, B + 2 ** 33, B + 2 ** 34, B + 2 ** 35)], 3),         # beyond 2^31
    ([(64, 0, B + 4096, B + 8192, B + 12288)], 1),                          # NULL param
    ([(64, B + 1, B + 4096, B + 8192, B + 12288)], 4),                      # param misaligned
    ([(64, B, B + 4096, B + 8194, B + 12288)], 4),                          # moment not 4-aligned
    ([(64, B, B + 4096, B + 8192, B + 8192 + 128)], 1),                     # m and v overlap
    ([(64, B, B + 4096, B + 8192, B + 12288), (64, B + 64, B + 20000, B + 24000, B + 28000)], 1),
    ([(0, 0, 0, 0, 0)], 0),                                                 # empty: pointers ignored
])
def test_adam_host_validation(lib, specs, want):
    arr, n = adam_list(specs)
    items = ctypes.c_int64(-1)
    assert lib.muon_adam_work_items(arr, n, mu.MUON_BF16, ctypes.byref(items)) == want
    if want == 0:
        exp = sum((s[0] + 16383) // 16384 for s in specs)
        assert items.value == exp


def test_adam_grads_may_alias_each_other(lib):
    """Read-only gradients may overlap each other (shared zero grads)."""
    arr, n = adam_list([(64, B, B + 2 ** 20, B + 8192, B + 12288),
                        (64, B + 2 ** 16, B + 2 ** 20, B + 2 ** 17, B + 2 ** 18)])
    items = ctypes.c_int64(0)
    assert lib.muon_adam_work_items(arr, n, mu.MUON_F32, ctypes.byref(items)) == 0
    assert items.value == 2
