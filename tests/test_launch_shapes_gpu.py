"""Every launch shape of every kernel flavour against the CPU oracle.

The library picks how many 1 KB row groups a wave handles (1, 2 or 4) from
the launch's size and the kernel flavour; each choice is a separate kernel
instantiation.  For each call and flavour these tests run a ladder of sizes
(a few tokens; about 12 k and 24 k row groups, where a small launch doubles
the groups per wave to keep every wave resident; about 80 k row groups,
where large launches start from their streaming choice, which differs
between the GPT-J and NeoX layouts; and large launches whose tokens have
one or three row groups, which cap the choice), read the choice back through
``rkv_last_launch_groups_per_wave`` and hold every launch to the parity bar
of the other GPU tests: bit-identical with RKV_ROUND_EXACT, within one fp16
ulp (one E4M3 code step) in the default mode.  The ladder must reach all
three choices in each mode, so a change of the launch rule that strands an
instantiation fails here instead of going untested.
"""
import pytest

import rope_kv_cache_amd as rkv
import workloads as W
from harness import compare, download, exact_diffs, expected, launch, upload

pytestmark = pytest.mark.gpu

NEOX, GPTJ = W.NEOX, W.GPTJ
MODES = ("fast", "exact")

# name, B, S, Hq, Hkv, D, R, style
CONTIG_LADDER = [
    ("tiny", 2, 16, 9, 2, 128, 128, NEOX),
    ("groups12k", 3, 1000, 9, 2, 128, 64, GPTJ),
    ("groups24k", 4, 1500, 9, 2, 128, 128, GPTJ),
    ("groups80k", 4, 5000, 9, 2, 128, 64, GPTJ),
    ("groups80k_neox", 4, 5000, 9, 2, 128, 128, NEOX),
    ("one_group_70k", 4, 17500, 4, 2, 64, 64, GPTJ),
    ("three_groups_24k", 4, 6000, 8, 2, 128, 128, NEOX),
]

# name, N, batch, Hkv, D, R, maxPagesPerSeq, style (numPages = batch * maxPages)
PAGED_LADDER = [
    ("tiny", 64, 2, 5, 128, 128, 2, NEOX),
    ("groups9k", 3000, 6, 5, 128, 64, 16, GPTJ),
    ("groups18k", 6000, 12, 5, 128, 128, 16, NEOX),
    ("groups75k", 25000, 50, 5, 128, 128, 16, GPTJ),
    ("one_group_70k", 70000, 70, 2, 128, 128, 16, NEOX),
]


def _say(*a):
    print(*a, flush=True)


def _contig(call, name, B, S, Hq, Hkv, D, R, style, seed):
    cap = S + 64
    label = f"{call}_{name}"
    if call == "packed":
        return W.packed(B, S, Hq, Hkv, D, R, cap, style, seed, name=label)
    if call == "continuous":
        return W.continuous(B, S, Hq, Hkv, D, R, cap, style, seed, S, cap, name=label)
    return W.tree(B, S, Hq, Hkv, D, R, cap, style, seed, S, cap, name=label)


def _flavoured(w, flavour, seed):
    if flavour in ("norm", "norm_fp8"):
        W.with_qk_norm(w, seed + 1, scale=2.0)
    if flavour in ("fp8", "norm_fp8"):
        W.with_fp8_cache(w, seed + 2, fill="sentinel")
    return w


def _run_ladder(workloads, flavour):
    """Parity of every workload in both modes; returns {mode: set of G}."""
    seen = {m: set() for m in MODES}
    for w in workloads:
        want = expected(w)
        for mode in MODES:
            t = upload(w)
            launch(w, t, exact=(mode == "exact"))
            g = rkv.last_launch_groups_per_wave()
            got = download(w, t)
            del t
            rep = compare(w, got, want)
            _say(f"[shapes] {w.name} {flavour} {mode}: G={g} {rep}")
            assert g in (1, 2, 4), g
            seen[mode].add(g)
            if mode == "exact":
                assert not exact_diffs(rep), f"exact mode not bit-identical: {rep}"
            else:
                keys = ("_max_ulp_ge_2m6", "_max_code_step") if "norm" in flavour else \
                    ("_max_ulp", "_max_code_step")
                assert all(v <= 1 for k, v in rep.items() if k.endswith(keys)), rep
    return seen


@pytest.mark.parametrize("flavour", ["fp16", "fp8", "norm", "norm_fp8"])
@pytest.mark.parametrize("call", ["packed", "continuous", "tree"])
def test_contig_launch_shapes(call, flavour):
    ws = (_flavoured(_contig(call, *row, 9000 + 10 * k), flavour, 9000 + 10 * k)
          for k, row in enumerate(CONTIG_LADDER))
    seen = _run_ladder(ws, flavour)
    for mode in MODES:
        assert seen[mode] == {1, 2, 4}, (mode, seen)


@pytest.mark.parametrize("flavour", ["fp16", "fp8"])
@pytest.mark.parametrize("gather", [False, True], ids=["table_rows", "gather_fused"])
def test_paged_launch_shapes(gather, flavour):
    def make(k, name, N, batch, Hkv, D, R, max_pages, style):
        seed = 9500 + 10 * k
        label = f"paged_{'gather_' if gather else ''}{name}"
        args = (N, batch, Hkv, D, R, batch * max_pages, max_pages, style, seed)
        w = W.paged_gather(*args, rope_states=2, name=label) if gather else \
            W.paged(*args, name=label)
        return _flavoured(w, flavour, seed)

    seen = _run_ladder((make(k, *row) for k, row in enumerate(PAGED_LADDER)), flavour)
    for mode in MODES:
        assert seen[mode] == {1, 2, 4}, (mode, seen)


# ---------------------------------------------- forced launch shapes ----

def _forced(workloads, flavour, plans=(0,)):
    """Each workload under every forced row-group count (and paged load plan):
    the library reports the forced choice and the result keeps the parity
    bar; the override is reset afterwards."""
    try:
        for w in workloads:
            want = expected(w)
            for plan in plans:
                for g in (1, 2, 4):
                    rkv.set_launch_overrides(g, plan)
                    for mode in MODES:
                        t = upload(w)
                        launch(w, t, exact=(mode == "exact"))
                        got_g = rkv.last_launch_groups_per_wave()
                        got_plan = rkv.last_launch_paged_loads()
                        got = download(w, t)
                        del t
                        rep = compare(w, got, want)
                        _say(f"[forced] {w.name} {flavour} G={g} plan={plan} {mode}: {rep}")
                        assert got_g == g, (got_g, g)
                        if plan:
                            assert got_plan == plan, (got_plan, plan)
                        if mode == "exact":
                            assert not exact_diffs(rep), f"exact mode not bit-identical: {rep}"
                        else:
                            keys = ("_max_ulp_ge_2m6", "_max_code_step") if "norm" in flavour \
                                else ("_max_ulp", "_max_code_step")
                            assert all(v <= 1 for k, v in rep.items() if k.endswith(keys)), rep
    finally:
        rkv.set_launch_overrides(0, 0)


@pytest.mark.parametrize("flavour", ["fp16", "fp8", "norm", "norm_fp8"])
@pytest.mark.parametrize("call", ["packed", "continuous", "tree"])
def test_contig_forced_shapes(call, flavour):
    """Tokens of 12 row groups (the workloads' head counts): every forced
    choice is an instantiation the size ladder reaches only at some sizes."""
    w = _flavoured(_contig(call, "forced", 3, 40, 32, 8, 128, 128, NEOX if call != "packed"
                           else GPTJ, 9800), flavour, 9800)
    _forced([w], flavour)


@pytest.mark.parametrize("flavour", ["fp16", "fp8"])
@pytest.mark.parametrize("gather", [False, True], ids=["table_rows", "gather_fused"])
def test_paged_forced_shapes_and_load_plans(gather, flavour):
    """Both load plans (early, late) under every forced row-group count, on
    a workload with padding rows and unmapped pages."""
    seed = 9900 + gather
    args = (300, 7, 8, 128, 128, 7 * 9, 9, NEOX, seed)
    w = W.paged_gather(*args, rope_states=2, width=43, pad_frac=0.2, bad_frac=0.2,
                       name="paged_gather_forced") if gather else \
        W.paged(*args, width=43, pad_frac=0.2, bad_frac=0.2, name="paged_forced")
    _forced([_flavoured(w, flavour, seed)], flavour, plans=(1, 2))
