"""Randomized host checks of the head-chunk planner and the pool sizes (no GPU).

For arbitrary head counts and chunk sizes: the library accepts exactly the
chunk sizes of the rule (head_chunk divides Hq, and divides or is a multiple of
G = Hq/Hkv), and its chunk table keeps the contract the backward relies on to
sum dK/dV over chunks: the chunks run through the query heads in order, a kv
head's fp32 accumulators start fresh at its first chunk and are loaded at every
later one, each query head of its group is added exactly once, and the
accumulators are finalized at the chunk that adds the group's last head. For
random sizes: the pools match the layout byte for byte, they grow with
head_chunk except where a chunk of a whole kv group drops the fp32 dK/dV
accumulators, the combined workspace is the larger of the two, the chunk-size picker returns the largest chunk that
fits its budget, and the fused backward's pool is the two-kernel pool without
its packed dQ plus one fp32 dQ partial per XCD.
"""

import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from long_context_attention_upipe_amd import _lib as L

ALIGN = 256  # every pool region starts on this boundary
MAX_XCD = 8  # fp32 dQ partials in the fused pool


def rule(Hq, Hkv, hc):
    if Hq < 1 or Hkv < 1 or Hq % Hkv:
        return False
    if hc < 1 or Hq % hc:
        return False
    G = Hq // Hkv
    return G % hc == 0 or hc % G == 0


def valid_chunks(Hq, Hkv):
    return [hc for hc in range(1, Hq + 1) if rule(Hq, Hkv, hc)]


@settings(max_examples=500, deadline=None, derandomize=True)
@given(Hq=st.integers(1, 48), Hkv=st.integers(1, 48), hc=st.integers(0, 50))
def test_plan_accepts_exactly_the_rule_and_keeps_the_accumulation_contract(Hq, Hkv, hc):
    if not rule(Hq, Hkv, hc):
        with pytest.raises(L.UpipeError):
            L.upipe_attn_plan(Hq, Hkv, hc)
        return
    plan = L.upipe_attn_plan(Hq, Hkv, hc)
    G = Hq // Hkv
    assert [c["q_head0"] for c in plan] == list(range(0, Hq, hc))
    assert plan[0]["load_kv"]
    added = {}        # kv head -> query heads summed into its accumulators
    finalized = set()
    pool_kv = None    # kv heads the pool holds
    for c in plan:
        heads = list(range(c["q_head0"], c["q_head0"] + hc))
        kvs = sorted({h // G for h in heads})
        assert kvs == list(range(c["kv_head0"], c["kv_head0"] + c["n_kv"]))
        assert c["load_kv"] == (pool_kv != tuple(kvs))
        pool_kv = tuple(kvs)
        for g in kvs:
            if c["first_for_kv"]:
                assert g not in added, "accumulators started twice"
                added[g] = set()
            else:
                assert g in added and g not in finalized, "accumulators loaded before they were started"
            mine = {h for h in heads if h // G == g}
            assert not (added[g] & mine), "a query head added twice"
            added[g] |= mine
            full = added[g] == set(range(g * G, (g + 1) * G))
            assert c["last_for_kv"] == full
            if full:
                finalized.add(g)
    assert finalized == set(range(Hkv))


@st.composite
def problems(draw):
    Hkv = draw(st.integers(1, 8))
    G = draw(st.integers(1, 8))
    S = draw(st.integers(1, 3_000_000))
    d = draw(st.sampled_from([64, 128]))
    dtype = draw(st.sampled_from([0, 1]))
    return S, Hkv * G, Hkv, d, dtype


def align(n):
    return -(-n // ALIGN) * ALIGN


def layout_pools(S, Hq, Hkv, d, hc, dtype):
    """The pools as the layout defines them, region by region, each region
    starting on an ALIGN boundary. Forward: the chunk's q and out rows, its kv
    heads' k rows and v (bf16: transposed in 64-key blocks, S padded to 64).
    Backward: q, dO and dq rows, k and v, -D and lse*log2(e) per row, and two
    fp32 [S, d] dK/dV accumulators when a kv group spans several chunks."""
    es = 2 if dtype == 0 else 4
    U = S * d * es
    G = Hq // Hkv
    nkv = max(1, hc // G)
    vt = (-(-S // 64) * 64 if dtype == 0 else S) * d * es
    fwd = 2 * align(hc * U) + align(nkv * U) + align(nkv * vt)
    bwd = 3 * align(hc * U) + 2 * align(nkv * U) + 2 * align(hc * S * 4) + (2 * align(S * d * 4) if hc < G else 0)
    return fwd, bwd


@settings(max_examples=300, deadline=None, derandomize=True)
@given(problems())
def test_pools_match_the_layout_and_workspace_is_their_max(p):
    S, Hq, Hkv, d, dtype = p
    for hc in valid_chunks(Hq, Hkv):
        fwd = L.upipe_attn_fwd_workspace_bytes(S, Hq, Hkv, d, hc, dtype)
        bwd = L.upipe_attn_bwd_workspace_bytes(S, Hq, Hkv, d, hc, dtype)
        assert (fwd, bwd) == layout_pools(S, Hq, Hkv, d, hc, dtype), hc
        assert L.upipe_attn_workspace_bytes(S, Hq, Hkv, d, hc, dtype) == max(fwd, bwd)


@settings(max_examples=200, deadline=None, derandomize=True)
@given(problems())
def test_pools_grow_with_head_chunk_except_where_the_accumulators_drop_out(p):
    """Each step up in head_chunk adds per-head buffers; the one saving is the
    fp32 dK/dV accumulators, which vanish once a chunk holds a whole kv group.
    In bf16 they weigh 4 bf16 head tensors, more than the 3 added going from
    head_chunk G/2 to G, so at G = 2 the backward pool is smaller at head_chunk
    2 than at 1; everywhere else it grows, strictly once a head's tensor fills
    an aligned unit (tiny pools can tie)."""
    S, Hq, Hkv, d, dtype = p
    G = Hq // Hkv
    es = 2 if dtype == 0 else 4
    hcs = valid_chunks(Hq, Hkv)
    fwd = [L.upipe_attn_fwd_workspace_bytes(S, Hq, Hkv, d, hc, dtype) for hc in hcs]
    bwd = [L.upipe_attn_bwd_workspace_bytes(S, Hq, Hkv, d, hc, dtype) for hc in hcs]
    big = S * d * es >= ALIGN
    for i in range(1, len(hcs)):
        assert fwd[i] > fwd[i - 1] if big else fwd[i] >= fwd[i - 1]
        if dtype == 0 and G == 2 and (hcs[i - 1], hcs[i]) == (1, 2):
            assert bwd[i] < bwd[i - 1]
        else:
            assert bwd[i] > bwd[i - 1] if big else bwd[i] >= bwd[i - 1], (hcs, bwd)


@settings(max_examples=200, deadline=None, derandomize=True)
@given(problems(), st.floats(0.0, 1.3))
def test_pick_head_chunk_is_the_largest_that_fits(p, frac):
    S, Hq, Hkv, d, dtype = p
    hcs = valid_chunks(Hq, Hkv)
    need = {hc: L.upipe_attn_workspace_bytes(S, Hq, Hkv, d, hc, dtype) for hc in hcs}
    budget = int(frac * need[hcs[-1]])
    fits = [hc for hc in hcs if need[hc] <= budget]
    if not fits:
        with pytest.raises(L.UpipeError) as e:
            L.upipe_attn_pick_head_chunk(S, Hq, Hkv, d, dtype, budget)
        assert e.value.status == -3
        smallest = min(hcs, key=lambda hc: (need[hc], hc))
        assert f"smallest workspace is {need[smallest]} bytes (head_chunk {smallest})" in str(e.value)
        return
    assert L.upipe_attn_pick_head_chunk(S, Hq, Hkv, d, dtype, budget) == max(fits)


@settings(max_examples=200, deadline=None, derandomize=True)
@given(problems())
def test_fused_pool_is_the_two_kernel_pool_without_dq_plus_the_partials(p):
    S, Hq, Hkv, _, _ = p
    d = 128
    n_ktiles = -(-S // 128)
    for hc in valid_chunks(Hq, Hkv):
        two = L.upipe_attn_bwd_workspace_bytes(S, Hq, Hkv, d, hc, 0)
        fused = L.upipe_attn_bwd_fused_workspace_bytes(S, Hq, Hkv, d, hc)
        nkv = max(1, hc // (Hq // Hkv))
        sync_bytes = 4 * (MAX_XCD + 1 + n_ktiles * nkv * 4)  # tickets, error word, progress words
        extra = MAX_XCD * hc * S * d * 4 - hc * S * d * 2 + sync_bytes
        # each region is rounded up to the alignment on its own
        assert abs((fused - two) - extra) < 4 * ALIGN, (hc, fused - two, extra)
