"""GPU parity of the four C-ABI calls against the CPU oracle, on the seeded
workloads at their full sizes and on edge cases (shape sweep, T = 0,
determinism, unwritten-output sentinels)."""
import numpy as np
import pytest
import torch

import oracle
import parity
from sparse_moe_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(L, logits_in=None, token_sample=None, fused_route=False):
    print("case: %s T=%d H=%d E=%d K=%d I=%d act=%s fused_route=%s" % (
        L.spec.name, L.x.shape[0], L.spec.H, L.spec.E, L.spec.K, L.spec.I, L.spec.act, fused_route),
        flush=True)
    g, bufs = parity.run_gpu_layer(L, logits_in, fused_route=fused_route)
    res = parity.check_layer(L, g, logits_in=logits_in, token_sample=token_sample)
    print("  ->", res, flush=True)
    return g, res


@pytest.mark.parametrize("fused", [False, True])
def test_tiny_layer(fused):
    _run(synth.make_layer(synth.SPECS[0]), fused_route=fused)


@pytest.mark.parametrize("fused", [False, True])
def test_decode_1_token(fused):
    _run(synth.make_layer(synth.SPECS[1]), fused_route=fused)


@pytest.mark.parametrize("fused", [False, True])
def test_decode_8_tokens(fused):
    g, res = _run(synth.make_layer(synth.SPECS[2]), fused_route=fused)
    assert 30 <= res["distinct_experts"] <= 64


def test_decode_8_tokens_injected_uniform_logits():
    spec = synth.SPECS[2]
    L = synth.make_layer(spec)
    lg = synth.uniform_logits(spec.T, spec.E, spec.seed)
    _run(L, logits_in=lg)


def tile_covering_tokens(offsets: np.ndarray, sorted_slots: np.ndarray, K: int,
                         tile: int = 128) -> np.ndarray:
    """Tokens whose slots touch every (expert, slot tile) of the grouped GEMM:
    greedily, each uncovered tile contributes the token of its last slot (the
    ragged end of a partial tile), which also covers that token's other slots.
    The tiles are taken `tile` slots at a time, a finer cover than the kernel's
    when it merges an expert's last few slots into a longer last tile: both
    parts of such a tile (its first 128 slots and the rows past them) are then
    sampled."""
    N = sorted_slots.size
    tile_of = np.empty(N, np.int64)
    tiles = []
    for e in range(offsets.size - 1):
        for s0 in range(offsets[e], offsets[e + 1], tile):
            tile_of[s0:min(s0 + tile, offsets[e + 1])] = len(tiles)
            tiles.append((s0, min(s0 + tile, offsets[e + 1])))
    pos_of_slot = np.empty(N, np.int64)
    pos_of_slot[sorted_slots] = np.arange(N)
    covered = np.zeros(len(tiles), bool)
    chosen = []
    for i, (s0, s1) in enumerate(tiles):
        if covered[i]:
            continue
        t = int(sorted_slots[s1 - 1]) // K
        chosen.append(t)
        covered[tile_of[pos_of_slot[t * K:(t + 1) * K]]] = True
    assert covered.all()
    return np.unique(np.array(chosen))


def test_prefill_4096_tokens_every_tile_sampled():
    # every token's routing and permutation are compared; the expert outputs and
    # the combined output on a token sample that touches every (expert, slot
    # tile) of the grouped GEMM, plus the first and last token
    spec = synth.SPECS[3]
    L = synth.make_layer(spec)
    print("case: prefill-4096, GPU run", flush=True)
    g, _ = parity.run_gpu_layer(L)
    sample = tile_covering_tokens(g["offsets"], g["sorted_slots"], spec.K)
    sample = np.unique(np.concatenate([[0, spec.T - 1], sample]))
    ntiles = int(np.sum((np.diff(g["offsets"]) + 127) // 128))
    print("  %d tokens cover all %d slot tiles" % (sample.size, ntiles), flush=True)
    res = parity.check_layer(L, g, token_sample=sample)
    print("  ->", res, flush=True)


@pytest.mark.parametrize("T", [1, 2, 3, 7, 8, 33, 512])
@pytest.mark.parametrize("E,K", [(8, 1), (8, 2), (128, 8), (128, 1)])
def test_shape_sweep(T, E, K):
    base = synth.SPECS[0] if E == 8 else synth.SPECS[2]
    spec = synth.LayerSpec(**{**base.__dict__, "E": E, "K": K, "T": T,
                              "name": "sweep-T%d-E%d-K%d" % (T, E, K)})
    L = synth.make_layer(spec, seed=100 + T)
    sample = None if (E == 8 or T <= 8) else np.arange(0, T, max(1, T // 6))
    _run(L, token_sample=sample, fused_route=(T <= 8))


@pytest.mark.parametrize("H,I,E,K,T,act", [
    (4096, 4096, 16, 16, 3, "f32"),     # largest H, I and K (K = E): GEMV path
    (4096, 4096, 16, 16, 64, "bf16"),   # the same on the bf16 MFMA path
    (256, 128, 256, 16, 40, "bf16"),    # the most experts: GEMV path
    (256, 128, 256, 16, 160, "bf16"),   # the most experts: MFMA path, one-slot tiles
])
def test_maximum_sizes(H, I, E, K, T, act):
    # the library's limits (MOE_MAX_H, MOE_MAX_I, MOE_MAX_E, MOE_MAX_K), on
    # sampled tokens where the oracle is slow
    spec = synth.LayerSpec("max-H%d-I%d-E%d-K%d-T%d" % (H, I, E, K, T), H=H, E=E, K=K, I=I, T=T,
                           act=act, router_std=1 / np.sqrt(H), seed=17)
    L = synth.make_layer(spec)
    sample = None if H < 1024 and T <= 40 else np.unique(np.r_[0, T // 2, T - 1])
    _run(L, token_sample=sample, fused_route=(T * K <= 1024 and T <= 8))


def test_fused_route_repeated_calls_reset_the_counter():
    # the fused routing kernel leaves its completion counter at zero: many calls in a
    # row on one workspace keep giving the oracle's routing
    from sparse_moe_amd import binding
    spec = synth.SPECS[2]
    bufs = None
    for seed in range(5):
        L = synth.make_layer(spec, seed=50 + seed)
        g, bufs = parity.run_gpu_layer(L, bufs=bufs, fused_route=True)
        parity.check_layer(L, g)
    assert int(bufs.ws_route[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("E,K", [(128, 8), (100, 16), (256, 16), (8, 8), (65, 1)])
def test_topk_exact_ties(E, K):
    # Zero router weights make every logit equal its bias exactly; biases drawn
    # from a few values (with -0 and +0) give many exact ties, which must resolve
    # to the lower expert index (descending logit, then ascending index) in the
    # fused few-token kernel and in the one-wave-per-token top-K kernel alike.
    from sparse_moe_amd import binding
    rng = np.random.default_rng(E * 31 + K)
    H, T = 64, 3
    bias = rng.choice(np.array([-1.5, -0.0, 0.0, 0.25, 2.0], np.float32), size=E)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).cuda()
    wr = torch.zeros((E, H), dtype=torch.float32, device="cuda")
    b = torch.from_numpy(bias).cuda()
    logits_ref = np.repeat(bias[None, :].astype(np.float64) + 0.0, T, axis=0)
    ids_ref, w_ref = oracle.topk_softmax(logits_ref, K)
    for fused in (True, False):
        bufs = binding.LayerBuffers(T, H, 64, E, K, torch.float32)
        if fused:
            binding.moe_route(x, wr, bufs.logits, bufs.topk_ids, bufs.topk_w, bufs.offsets,
                              bufs.sorted_slots, bufs.slot_pos, bufs.ws_route, logit_bias=b)
        else:
            binding.moe_router_topk(x, wr, bufs.logits, bufs.topk_ids, bufs.topk_w, logit_bias=b)
        torch.cuda.synchronize()
        assert np.array_equal(bufs.topk_ids.cpu().numpy(), ids_ref), (fused, E, K)
        assert np.max(np.abs(bufs.topk_w.cpu().numpy() - w_ref)) <= 1e-6


def test_odd_block_count_rows():
    # H = 32 * 9 and I = 32 * 3: rows with an odd number of Q4_0 blocks
    spec = synth.LayerSpec("odd-blocks", H=288, E=8, K=2, I=96, T=5, act="f32",
                           router_std=1 / 17, seed=7)
    _run(synth.make_layer(spec))


def test_zero_tokens_is_a_noop():
    from sparse_moe_amd import binding
    L = synth.make_layer(synth.SPECS[0], T=1)
    x = parity.to_dev(L.x)[:0]
    bufs = binding.LayerBuffers(0, 256, 64, 8, 2, torch.float32)
    binding.moe_layer(x, parity.to_dev(L.w_router), parity.to_dev(L.w_gate_up),
                      parity.to_dev(L.w_down), 2, bufs=bufs)
    torch.cuda.synchronize()


def test_deterministic_and_fully_written():
    from sparse_moe_amd import binding
    spec = synth.SPECS[2]
    L = synth.make_layer(spec)
    outs = []
    for rep in range(2):
        bufs = binding.LayerBuffers(spec.T, spec.H, spec.I, spec.E, spec.K, torch.bfloat16)
        for t in (bufs.logits, bufs.topk_w, bufs.y_sorted, bufs.out):
            t.fill_(float("nan"))
        for t in (bufs.topk_ids, bufs.offsets, bufs.sorted_slots, bufs.slot_pos):
            t.fill_(-1)
        g, _ = parity.run_gpu_layer(L, bufs=bufs)
        for k, v in g.items():
            if v.dtype.kind == "f":
                assert np.all(np.isfinite(v)), k
            else:
                assert np.all(v >= 0), k
        outs.append(g)
    for k in outs[0]:
        assert np.array_equal(outs[0][k].view(np.uint8), outs[1][k].view(np.uint8)), k


@pytest.mark.parametrize("H,I,E,K,T,zipf", [
    (288, 96, 8, 2, 70, None),       # odd block counts per row (9 and 3): served by the GEMV path
    (256, 64, 8, 2, 600, None),      # ~150 slots per expert: two slot tiles per expert
    (256, 192, 4, 1, 300, None),     # K = 1, a partial second column tile of the gate/up product
    (256, 128, 8, 2, 200, None),     # ~50 slots per expert: tiles of 33-64 slots
    (2816, 704, 128, 8, 64, None),   # Gemma shape at the smallest token count of the MFMA path
    # Zipf-skewed routing: experts of a few slots (one mostly empty tile) next
    # to experts of several tiles, as in the layer stack
    (512, 128, 32, 4, 256, 1.1),
])
def test_mfma_path_shapes(H, I, E, K, T, zipf):
    # bf16 activations with T >= 64 take the bf16 MFMA grouped GEMM
    spec = synth.LayerSpec("mfma-H%d-I%d-E%d-K%d-T%d" % (H, I, E, K, T), H=H, E=E, K=K, I=I, T=T,
                           act="bf16", router_std=1 / np.sqrt(H), seed=11, zipf_s=zipf)
    L = synth.make_layer(spec)
    if zipf is not None:
        # the routing really mixes experts of at most 16 slots with experts of
        # more than one 128-slot tile
        ids, _ = oracle.topk_softmax(oracle.router_logits(L.x, L.w_router, bias=L.router_bias), K)
        counts = np.bincount(ids.ravel(), minlength=E)
        assert ((counts > 0) & (counts <= 16)).any() and (counts > 128).any(), counts
    sample = None if H < 1024 else np.arange(0, T, 5)
    _run(L, token_sample=sample)


@pytest.mark.parametrize("I", [64, 192])
def test_mfma_tile_size_boundaries(I):
    # Injected logits route exactly 1, 32, 33, 64, 65, 96, 97 and 129 slots to
    # the eight experts: both sides of every slot-tile variant (2, 4, 6 and 8
    # fragments of 16 slots, and a second tile of one slot).  I = 64 gives the
    # down product a single block pair, I = 192 an odd number of pairs.
    counts = [1, 32, 33, 64, 65, 96, 97, 129]
    T, E = sum(counts), len(counts)
    spec = synth.LayerSpec("tile-bounds-I%d" % I, H=256, E=E, K=1, I=I, T=T, act="bf16",
                           router_std=1 / 16, seed=29)
    L = synth.make_layer(spec)
    rng = np.random.default_rng(31)
    owner = rng.permutation(np.repeat(np.arange(E), counts))
    lg = (rng.standard_normal((T, E)) * 0.1).astype(np.float32)
    lg[np.arange(T), owner] += 10.0
    g, res = _run(L, logits_in=lg)
    assert np.array_equal(np.diff(g["offsets"]), np.array(counts)), np.diff(g["offsets"])


@pytest.mark.parametrize("H,I", [(256, 512), (64, 64), (128, 192)])
def test_mfma_tile_boundaries_among_many_experts(H, I):
    # The slot counts above (1, 32, 33, 64, 65, 96, 97, 129) and the bounds of
    # the merged last tile of up to 160 slots (144 and 145: one tile of 9 and
    # of 10 fragments; 160: the largest single tile; 161: 128 + 33; 288:
    # 128 + 160; 289: 128 + 128 + 33) among 128 more experts of 384 slots each
    # (three full tiles): the tile numbering and the XCD runs over a few
    # hundred tiles, with every tile variant present.  The shapes give the
    # two-stage ring 4, 1 and 2 block pairs (gate/up) and 8, 1 and 3 (down),
    # and leave waves without rows in the last column tile.  Injected logits
    # fix every token's expert; outputs are checked on the first and last token
    # of the fourteen boundary experts and of a few others.
    counts = [1, 32, 33, 64, 65, 96, 97, 129, 144, 145, 160, 161, 288, 289] + [384] * 128
    T, E = sum(counts), len(counts)
    spec = synth.LayerSpec("tile-bounds-many-H%d-I%d" % (H, I), H=H, E=E, K=1, I=I, T=T, act="bf16",
                           router_std=1 / 16, seed=37)
    L = synth.make_layer(spec)
    rng = np.random.default_rng(41)
    owner = rng.permutation(np.repeat(np.arange(E), counts))
    lg = (rng.standard_normal((T, E)) * 0.1).astype(np.float32)
    lg[np.arange(T), owner] += 10.0
    sample = np.concatenate([np.nonzero(owner == e)[0][[0, -1]] for e in range(14)] +
                            [np.nonzero(owner == e)[0][[0, -1]] for e in (14, 70, E - 1)])
    g, res = _run(L, logits_in=lg, token_sample=np.unique(sample))
    assert np.array_equal(np.diff(g["offsets"]), np.array(counts))


@pytest.mark.parametrize("I", [512, 704])
def test_mfma_longest_first_numbering(I):
    # A grid of a few dozen tiles, so both grouped-GEMM launches rank the slot
    # tiles longest first: experts with tiles of every size class (1-32, 33-64,
    # 65-96 and 97-128 slots, full tiles, none), every token checked.
    counts = [1, 20, 33, 50, 65, 90, 97, 120, 128, 129, 200, 256, 300, 5, 0, 77]
    T, E = sum(counts), len(counts)
    spec = synth.LayerSpec("longest-first-I%d" % I, H=256, E=E, K=1, I=I, T=T, act="bf16",
                           router_std=1 / 16, seed=43)
    L = synth.make_layer(spec)
    rng = np.random.default_rng(47)
    owner = rng.permutation(np.repeat(np.arange(E), counts))
    lg = (rng.standard_normal((T, E)) * 0.1).astype(np.float32)
    lg[np.arange(T), owner] += 10.0
    g, res = _run(L, logits_in=lg)
    assert np.array_equal(np.diff(g["offsets"]), np.array(counts))
