"""Pins for the CPU oracle: each test ties it to something other than itself.

- brute force (pure-Python fp64 loops, correctly rounded dot products via fsum,
  a dense visibility matrix built from the parent array) on tiny inputs;
- a library routine: torch's scaled_dot_product_attention in float64 for the
  chain tree (bottom-right causal mask) and for every root-to-node path of a
  random tree (the tree mask equals per-path causal attention);
- closed forms: zero query, identical keys, a single key, two keys;
- invariants: page-table permutation (scattered vs contiguous layout), masked
  tree rows and unreferenced slots that must not influence the result;
- the bf16 rounding helper against IEEE round-to-nearest-even cases and torch's
  float32 -> bfloat16 conversion;
- the pages' KV byte figures for the byte model used by the benchmark.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from mla_tree_verify_02_amd import inputs as I

HERE = os.path.dirname(os.path.abspath(__file__))


# ------------------------------------------------------------------ helpers

def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (numpy reinterpretation, exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tiny(batch=1, n=3, h=2, prefixes=(7,), slots=64, tree="random", seed=11, **kw):
    return I.make_workload(batch=batch, num_nodes=n, num_heads=h, prefix_lens=list(prefixes),
                           num_slots=slots, tree=tree, config_id=900 + seed, max_depth=3, **kw)


def ancestors_of(parents, i):
    out = []
    j = i
    while j >= 0:
        out.append(j)
        j = int(parents[j])
    return out[::-1]  # root first


def brute_force(wl, visible):
    """Pure-Python fp64 reference: visible(b, i, p, S) decides the mask."""
    q = widen(wl.np_q())
    kv = widen(wl.np_kv())
    table = wl.np_page_table()
    seq = wl.np_seq_lens()
    B, N, H, _ = q.shape
    out = np.zeros((B, N, H, 512))
    lse = np.zeros((B, N, H))
    for b in range(B):
        S = int(seq[b])
        for i in range(N):
            for h in range(H):
                qv = q[b, i, h]
                scores, vals = [], []
                for p in range(S):
                    if not visible(b, i, p, S):
                        continue
                    row = kv[table[b, p]]
                    # products of two bf16 values are exact in double; fsum rounds once
                    scores.append(wl.scale * math.fsum((qv * row).tolist()))
                    vals.append(row[:512])
                if not scores:
                    lse[b, i, h] = -math.inf
                    continue
                mx = max(scores)
                lz = mx + math.log(math.fsum(math.exp(s - mx) for s in scores))
                lse[b, i, h] = lz
                w = [math.exp(s - lz) for s in scores]
                for c in range(512):
                    out[b, i, h, c] = math.fsum(wk * v[c] for wk, v in zip(w, vals))
    return out, lse


def tree_visible(wl):
    anc = [[set(ancestors_of(wl.parents[b], i)) for i in range(wl.num_nodes)]
           for b in range(wl.batch)]

    def vis(b, i, p, S):
        pre = S - wl.num_nodes
        return p < pre or (p - pre) in anc[b][i]
    return vis


def bits_visible(wl):
    m = wl.np_mask()

    def vis(b, i, p, S):
        pre = S - wl.num_nodes
        if p < pre:
            return True
        j = p - pre
        return bool((int(m[b, i, j // 32]) >> (j % 32)) & 1)
    return vis


def close(a, b, rtol, atol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    ok = both_inf | (np.abs(a - b) <= atol + rtol * np.abs(b))
    return bool(ok.all())


# ------------------------------------------------------------ P1 brute force

@pytest.mark.parametrize("case", [
    dict(batch=1, n=3, h=2, prefixes=(7,), tree="chain", seed=1),
    dict(batch=2, n=5, h=2, prefixes=(40, 3), tree="random", seed=2, slots=128),
    dict(batch=1, n=4, h=1, prefixes=(0,), tree="binary", seed=3),
    dict(batch=2, n=5, h=1, prefixes=(11, 29), tree="random", seed=4, slots=128),
])
def test_brute_force_tree_masks(oracle_mod, case):
    wl = tiny(**case)
    out, lse, out64, lse64 = oracle_mod.run_workload(wl, want_f64=True)
    bo, bl = brute_force(wl, tree_visible(wl))
    assert close(lse64, bl, 1e-12, 1e-12)
    assert close(out64, bo, 1e-12, 1e-12)
    # the stored results are the rounded unrounded ones
    assert np.array_equal(lse, lse64.astype(np.float32))
    rounded = np.vectorize(oracle_mod.f64_to_bf16, otypes=[np.uint16])(out64)
    assert np.array_equal(out, rounded)


@pytest.mark.parametrize("n", [31, 32, 33, 64])
def test_brute_force_random_bitmasks_word_boundaries(oracle_mod, n):
    # non-ancestor masks, including bits in the second word for n > 32
    m = I.random_bitmask(n, seed=70 + n, density=0.4)
    m[0, :] = 0  # node 0 sees only the prefix
    wl = I.make_workload(batch=1, num_nodes=n, num_heads=1, prefix_lens=[3], num_slots=128,
                         tree="chain", config_id=950 + n, mask=m)
    out, lse, out64, lse64 = oracle_mod.run_workload(wl, want_f64=True)
    bo, bl = brute_force(wl, bits_visible(wl))
    assert close(lse64, bl, 1e-12, 1e-12)
    assert close(out64, bo, 1e-12, 1e-12)


def test_bits_at_or_above_n_are_ignored(oracle_mod):
    n = 5
    wl = tiny(n=n, h=1, prefixes=(6,), tree="random", seed=20)
    m = wl.np_mask().copy()
    base = oracle_mod.run_workload(wl)
    m[..., 0] |= np.uint32(0xFFFFFFE0)  # bits 5..31 do not name tree nodes
    wl.tree_mask = torch.from_numpy(m.view(np.int32).copy())
    other = oracle_mod.run_workload(wl)
    assert np.array_equal(base[0], other[0]) and np.array_equal(base[1], other[1])


# ---------------------------------------------------- P5 / P4 library routine

def sdpa_reference(qrows, keys, allowed, scale):
    """torch float64 attention: qrows [L,576], keys [S,576], allowed bool [L,S]."""
    qt = torch.from_numpy(qrows)[None, None]
    kt = torch.from_numpy(keys)[None, None]
    vt = torch.from_numpy(np.ascontiguousarray(keys[:, :512]))[None, None]
    am = torch.from_numpy(allowed)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)
    logits = (qt @ kt.transpose(-1, -2)) * scale
    logits = logits.masked_fill(~am, -math.inf)
    return o[0, 0].numpy(), torch.logsumexp(logits, dim=-1)[0, 0].numpy()


def test_chain_equals_library_causal_attention(oracle_mod):
    n, h, ctx = 8, 3, 300
    wl = I.make_workload(batch=1, num_nodes=n, num_heads=h, prefix_lens=[ctx], num_slots=1024,
                         tree="chain", config_id=960)
    out, lse, out64, lse64 = oracle_mod.run_workload(wl, want_f64=True)
    q = widen(wl.np_q())[0]
    S = ctx + n
    keys = widen(wl.np_kv())[wl.np_page_table()[0, :S]]
    # bottom-right aligned causal mask: node i sees the prefix and nodes 0..i
    allowed = np.arange(S)[None, :] < (ctx + 1 + np.arange(n))[:, None]
    for hh in range(h):
        o, l = sdpa_reference(q[:, hh], keys, allowed, wl.scale)
        assert close(out64[0, :, hh], o, 1e-12, 1e-12)
        assert close(lse64[0, :, hh], l, 1e-12, 1e-12)


def test_tree_equals_per_path_causal_attention(oracle_mod):
    n, h, ctx = 24, 2, 50
    wl = I.make_workload(batch=1, num_nodes=n, num_heads=h, prefix_lens=[ctx], num_slots=512,
                         tree="random", max_depth=5, config_id=961)
    out, lse, out64, lse64 = oracle_mod.run_workload(wl, want_f64=True)
    q = widen(wl.np_q())[0]
    kv = widen(wl.np_kv())
    table = wl.np_page_table()[0]
    for i in range(n):
        path = ancestors_of(wl.parents[0], i)
        positions = list(range(ctx)) + [ctx + j for j in path]
        keys = kv[table[positions]]
        allowed = np.ones((1, len(positions)), dtype=bool)  # plain attention over the path
        for hh in range(h):
            o, l = sdpa_reference(q[i:i + 1, hh], keys, allowed, wl.scale)
            assert close(out64[0, i, hh], o[0], 1e-12, 1e-12)
            assert close(lse64[0, i, hh], l[0], 1e-12, 1e-12)


# ------------------------------------------------------------- P2 / P6 closed forms

def test_single_key_returns_its_latent(oracle_mod):
    wl = tiny(n=1, h=2, prefixes=(0,), tree="chain", seed=30)
    out, lse, out64, lse64 = oracle_mod.run_workload(wl, want_f64=True)
    row_bits = wl.np_kv()[wl.np_page_table()[0, 0]]
    for hh in range(2):
        assert np.array_equal(out[0, 0, hh], row_bits[:512])  # bf16 in, same bf16 out
        qv = widen(wl.np_q())[0, 0, hh]
        s = wl.scale * math.fsum((qv * widen(row_bits)).tolist())
        assert abs(lse64[0, 0, hh] - s) <= 1e-13 * max(1.0, abs(s))
        assert lse[0, 0, hh] == np.float32(s)


def test_zero_query_gives_mean_of_visible_latents(oracle_mod):
    wl = tiny(batch=2, n=4, h=1, prefixes=(9, 2), tree="random", seed=31)
    wl.q.zero_()
    out, lse, out64, lse64 = oracle_mod.run_workload(wl, want_f64=True)
    kv = widen(wl.np_kv())
    vis = tree_visible(wl)
    for b in range(2):
        S = int(wl.np_seq_lens()[b])
        for i in range(4):
            ps = [p for p in range(S) if vis(b, i, p, S)]
            rows = kv[wl.np_page_table()[b, ps]][:, :512]
            mean = np.array([math.fsum(rows[:, c].tolist()) / len(ps) for c in range(512)])
            assert close(out64[b, i, 0], mean, 1e-13, 1e-13)
            assert abs(lse64[b, i, 0] - math.log(len(ps))) <= 1e-14


def test_identical_keys(oracle_mod):
    wl = tiny(n=3, h=2, prefixes=(13,), tree="chain", seed=32)
    table = wl.np_page_table()[0]
    S = int(wl.np_seq_lens()[0])
    kvb = wl.kv_pool.view(torch.int16)
    kvb[torch.from_numpy(table[1:S].astype(np.int64))] = kvb[int(table[0])].clone()
    out, lse, out64, lse64 = oracle_mod.run_workload(wl, want_f64=True)
    row_bits = wl.np_kv()[table[0]]
    qv = widen(wl.np_q())[0]
    for i in range(3):
        for hh in range(2):
            assert np.array_equal(out[0, i, hh], row_bits[:512])
            s = wl.scale * math.fsum((qv[i, hh] * widen(row_bits)).tolist())
            nvis = 13 + i + 1
            assert abs(lse64[0, i, hh] - (s + math.log(nvis))) <= 1e-12 * max(1, abs(s))


def test_two_keys_logistic_weights(oracle_mod):
    wl = tiny(n=1, h=2, prefixes=(1,), tree="chain", seed=33)
    out, lse, out64, lse64 = oracle_mod.run_workload(wl, want_f64=True)
    kv = widen(wl.np_kv())
    t = wl.np_page_table()[0]
    k1, k2 = kv[t[0]], kv[t[1]]
    for hh in range(2):
        qv = widen(wl.np_q())[0, 0, hh]
        s1 = wl.scale * math.fsum((qv * k1).tolist())
        s2 = wl.scale * math.fsum((qv * k2).tolist())
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        w2 = 1.0 / (1.0 + math.exp(s1 - s2))
        assert close(out64[0, 0, hh], w1 * k1[:512] + w2 * k2[:512], 1e-13, 1e-13)
        lz = max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2)))
        assert abs(lse64[0, 0, hh] - lz) <= 1e-13 * max(1, abs(lz))


def test_empty_visible_set(oracle_mod):
    m = np.array([[0], [3]], dtype=np.uint32)  # node 0 sees nothing, node 1 sees 0 and 1
    wl = I.make_workload(batch=1, num_nodes=2, num_heads=1, prefix_lens=[0], num_slots=16,
                         tree="chain", config_id=970, mask=m)
    out, lse = oracle_mod.run_workload(wl)
    assert np.all(out[0, 0, 0] == 0) and lse[0, 0, 0] == -np.inf
    assert np.isfinite(lse[0, 1, 0])


# ------------------------------------------------------------- P3 / P7 invariants

def relayout(wl, table_seed, layout):
    """Same logical rows at every position, stored under another page table."""
    other = I.make_workload(batch=wl.batch, num_nodes=wl.num_nodes, num_heads=wl.num_heads,
                            prefix_lens=wl.prefix_lens, num_slots=wl.num_slots, tree="chain",
                            layout=layout, table_seed=table_seed, config_id=980,
                            mask=wl.np_mask())
    other.q = wl.q.clone()
    kv_new = torch.full_like(wl.kv_pool.view(torch.int16), I.BF16_NAN_BITS)
    t_old, t_new = wl.np_page_table(), other.np_page_table()
    for b, S in enumerate(wl.np_seq_lens()):
        src = torch.from_numpy(t_old[b, :S].astype(np.int64))
        dst = torch.from_numpy(t_new[b, :S].astype(np.int64))
        kv_new[dst] = wl.kv_pool.view(torch.int16)[src]
    other.kv_pool = kv_new.view(torch.bfloat16)
    return other


def test_page_table_permutation_invariance(oracle_mod):
    wl = I.make_workload(batch=3, num_nodes=6, num_heads=2, prefix_lens=[70, 5, 130],
                         num_slots=1024, tree="random", max_depth=3, config_id=981)
    ref = oracle_mod.run_workload(wl)
    for seed, layout in [(5, "scattered"), (6, "scattered"), (7, "runs64")]:
        other = relayout(wl, seed, layout)
        assert not np.array_equal(other.np_page_table(), wl.np_page_table())
        got = oracle_mod.run_workload(other)
        assert np.array_equal(got[0], ref[0])
        assert np.array_equal(got[1].view(np.uint32), ref[1].view(np.uint32))


def test_unreferenced_nan_slots_are_not_read(oracle_mod):
    wl = tiny(batch=2, n=4, h=2, prefixes=(20, 33), tree="random", seed=40, slots=256)
    out, lse = oracle_mod.run_workload(wl)
    assert np.isfinite(lse).all()
    assert np.isfinite(widen(out)).all()


def test_masked_tree_rows_do_not_leak(oracle_mod):
    # chain: tree node N-1 is seen by node N-1 only; poison its latent with +-1e4
    n = 8
    wl = I.make_workload(batch=1, num_nodes=n, num_heads=2, prefix_lens=[40], num_slots=256,
                         tree="chain", config_id=982)
    base = oracle_mod.run_workload(wl)
    slot = int(wl.np_page_table()[0, 40 + n - 1])
    poison = torch.tensor([1e4 if c % 2 == 0 else -1e4 for c in range(576)]).to(torch.bfloat16)
    wl.kv_pool[slot] = poison
    got = oracle_mod.run_workload(wl)
    assert np.array_equal(got[0][0, :n - 1], base[0][0, :n - 1])
    assert np.array_equal(got[1][0, :n - 1], base[1][0, :n - 1])
    assert not np.array_equal(got[0][0, n - 1], base[0][0, n - 1])


def test_positions_past_seq_len_are_not_read(oracle_mod):
    wl = I.make_workload(batch=2, num_nodes=3, num_heads=1, prefix_lens=[10, 4], num_slots=64,
                         tree="chain", config_id=983, max_kv=40)
    base = oracle_mod.run_workload(wl)
    t = wl.np_page_table().copy()
    t[0, 13:] = 10 ** 6  # out-of-range junk past S_b must never be dereferenced
    t[1, 7:] = -5
    wl.page_table = torch.from_numpy(t)
    got = oracle_mod.run_workload(wl)
    assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1])


def test_bad_inputs_are_rejected(oracle_mod):
    wl = tiny(n=2, h=1, prefixes=(3,), tree="chain", seed=41)
    t = wl.np_page_table().copy()
    t[0, 1] = wl.num_slots  # referenced index out of range
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.run(wl.np_q(), wl.np_kv(), t, wl.np_seq_lens(), wl.np_mask(), wl.scale)
    s = wl.np_seq_lens().copy()
    s[0] = 1  # shorter than the tree
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.run(wl.np_q(), wl.np_kv(), wl.np_page_table(), s, wl.np_mask(), wl.scale)


def test_row_subset_matches_full_run(oracle_mod):
    wl = tiny(batch=2, n=3, h=2, prefixes=(15, 8), tree="random", seed=42)
    full = oracle_mod.run_workload(wl)
    rows = [0, 5, 7, 11]
    part = oracle_mod.run_workload(wl, rows=rows)
    fo, fl = full[0].reshape(-1, 512), full[1].reshape(-1)
    po, pl = part[0].reshape(-1, 512), part[1].reshape(-1)
    for r in rows:
        assert np.array_equal(po[r], fo[r]) and pl[r] == fl[r]


def test_threading_does_not_change_bits(oracle_mod):
    wl = tiny(batch=2, n=5, h=3, prefixes=(31, 17), tree="random", seed=43, slots=128)
    a = oracle_mod.run_workload(wl, threads=1)
    b = oracle_mod.run_workload(wl, threads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------ bf16 rounding

def test_bf16_widening_all_patterns(oracle_mod):
    pats = np.arange(0, 1 << 16, 97, dtype=np.uint32)
    ref = (pats << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle_mod.bf16_to_f64(int(p)) for p in pats])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_rounding_matches_torch_on_float32_values(oracle_mod):
    g = torch.Generator().manual_seed(5)
    x = torch.cat([torch.randn(3000, generator=g) * 10.0 ** torch.randint(-30, 30, (3000,), generator=g),
                   torch.randn(500, generator=g) * 1e-39,    # float32 subnormals
                   torch.tensor([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1.0e-45])])
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle_mod.f64_to_bf16(float(v)) for v in x.tolist()], dtype=np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("value,bits", [
    (1.0 + 2.0 ** -8, 0x3F80),                      # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),                  # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),         # above the tie: direct rounding goes up
    (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
    ((2.0 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),       # midpoint above the largest finite: inf
    ((2.0 - 2.0 ** -8) * 2.0 ** 127 * (1 - 2.0 ** -30), 0x7F7F),
    (2.0 ** -133, 0x0001),                          # smallest subnormal
    (1.5 * 2.0 ** -133, 0x0002),                    # subnormal tie -> even
    (2.5 * 2.0 ** -133, 0x0002),
    (2.0 ** -140, 0x0000),
    (-(2.0 ** -140), 0x8000),
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
    (float("nan"), 0x7FC0),
])
def test_bf16_rounding_ieee_cases(oracle_mod, value, bits):
    assert oracle_mod.f64_to_bf16(value) == bits


# --------------------------------------------------------------------- P8 bytes

def test_byte_model_reproduces_page_figures():
    with open(os.path.join(HERE, "golden", "page_byte_figures.json")) as f:
        gold = json.load(f)
    tol = gold["tolerance_rel"]
    for fig in gold["figures"]:
        for ctx in (fig["context_tokens"], fig["context_tokens"] * 1024 // 1000):
            per_layer = I.algorithmic_bytes([ctx + 8], 8, 8)
            total = fig["layers"] * per_layer
            assert abs(total - fig["bytes_per_step"]) <= tol * fig["bytes_per_step"], (ctx, total)
            assert I.ROW_BYTES == 1152
