"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Routing (top-k ids), per-expert counts, offsets and the permutation must be
bit-exact; gate weights within 1e-6; the layer output within
|g - r| <= 2e-2 * max(|r|, rms(r)) element-wise (bf16 output, fp32
accumulation against an unrounded oracle)."""

import dataclasses

import numpy as np
import pytest

import oracle
import synth
from conftest import assert_out_close, weights_kwargs
from gpu_util import GpuLayer, require_gpu, say

pytestmark = pytest.mark.gpu

_cache = {}


def gpu_layer(case, max_tokens=4096):
    key = (case.shape.family(), case.shape.top_k, case.seed, max_tokens)
    if key not in _cache:
        _cache.clear()
        _cache[key] = GpuLayer(case.shape, case.weights, max_tokens=max_tokens)
    return _cache[key]


def check_routing(res, ref):
    np.testing.assert_array_equal(res["topk_idx"], ref["topk_idx"])
    np.testing.assert_allclose(res["topk_w"], ref["topk_w"], rtol=0, atol=1e-6)
    np.testing.assert_array_equal(res["counts"], ref["counts"])
    np.testing.assert_array_equal(res["offsets"], ref["offsets"])
    np.testing.assert_array_equal(res["perm"], ref["perm"])
    np.testing.assert_array_equal(res["inv_perm"], ref["inv"])


def _oracle(case, hidden=None, **over):
    kw = weights_kwargs(case.weights)
    kw.update(over)
    prec = "f64" if case.shape.d_model * case.shape.d_ff <= 128 * 256 else "f32"
    return oracle.forward(case.hidden if hidden is None else hidden, top_k=case.shape.top_k, precision=prec,
                          num_shared=case.shape.num_shared, bits=case.shape.bits, group=case.shape.group, **kw)


@pytest.mark.parametrize("name", ["tiny", "fine_tiny", "mixtral_decode", "phi35_skew", "fine_decode",
                                  "mixtral_prefill", "fine_prefill", "shared_tiny", "fine_shared_tiny",
                                  "shared_decode", "shared_prefill", "tiny_q4g128", "tiny_q8", "tiny_q8g128",
                                  "mixtral_decode_q4g128", "mixtral_decode_q8g128", "phi35_skew_q8",
                                  "mixtral_prefill_q4g128", "mixtral_prefill_q8g128"])
def test_layer_parity(name):
    require_gpu()
    say(f"{name}: generating layer")
    case = synth.make_case(name)
    g = gpu_layer(case)
    say(f"{name}: T={case.shape.T} forward on the GPU")
    res = g.run(case.hidden)
    say(f"{name}: oracle")
    ref = _oracle(case)
    check_routing(res, ref)
    assert res["flags"] == 0
    assert_out_close(res["out"], ref["out"])
    say(f"{name}: ok, active experts {int((ref['counts'] > 0).sum())}, max rows {int(ref['counts'].max())}")


@pytest.mark.parametrize("name,T", [("tiny", 1), ("tiny", 3), ("tiny", 37), ("fine_tiny", 100),
                                    ("fine_tiny", 257), ("tiny", 1000), ("shared_tiny", 1),
                                    ("shared_tiny", 33), ("shared_tiny", 300), ("fine_shared_tiny", 64),
                                    ("fine_shared_tiny", 65), ("tiny_q4g128", 1), ("tiny_q4g128", 33),
                                    ("tiny_q4g128", 65), ("tiny_q4g128", 300), ("tiny_q8", 40), ("tiny_q8", 200),
                                    ("tiny_q8g128", 17), ("tiny_q8g128", 129),
                                    # Mixtral-shaped routed decode: the combine in the down kernel (T <= 8)
                                    # and in a kernel of its own (32-row tiles)
                                    ("mixtral_decode", 8), ("mixtral_decode", 40)])
def test_ragged_token_counts(name, T):
    require_gpu()
    case = synth.make_case(name, T=T)
    say(f"{name}: T={T}")
    res = gpu_layer(case).run(case.hidden)
    ref = _oracle(case)
    check_routing(res, ref)
    assert_out_close(res["out"], ref["out"])


def test_zero_router_ties_go_to_lowest_ids():
    require_gpu()
    case = synth.make_case("fine_tiny")
    E = case.shape.num_experts
    zr, zb = np.zeros((E, case.shape.d_model), np.float32), np.zeros(E, np.float32)
    say("fine_tiny: zero router")
    res = gpu_layer(case).run(case.hidden, router_w=zr, router_b=zb)
    assert np.all(res["topk_idx"] == np.arange(6)[None, :])
    assert np.all(res["topk_w"] == np.float32(1 / 6))
    ref = _oracle(case, router_w=zr, router_b=zb)
    check_routing(res, ref)
    assert_out_close(res["out"], ref["out"])


@pytest.mark.parametrize("E,k,S", [(1, 1, 0), (4, 4, 0), (8, 1, 0), (16, 8, 0), (256, 8, 0), (1, 1, 1),
                                   (8, 6, 2), (255, 1, 1), (4, 1, 7)])
def test_small_special_shapes(E, k, S):
    require_gpu()
    shape = synth.LayerShape(24, 128, 256, E, k, E + S, "identity", 0.0, S)
    w = synth.make_weights(shape, seed=3)
    x = synth.make_hidden(24, 128, seed=3)
    case = synth.Case("special", shape, 3, x, w)
    say(f"special E={E} k={k} shared={S}")
    res = GpuLayer(shape, w).run(x)
    ref = _oracle(case)
    check_routing(res, ref)
    assert_out_close(res["out"], ref["out"])
    if k == E:
        assert np.all(np.sort(res["topk_idx"], axis=1) == np.arange(E + S))


@pytest.mark.parametrize("T,E,k,zero", [(16, 128, 8, False), (16, 128, 8, True), (8, 256, 3, False),
                                         (32, 40, 5, False), (20, 32, 2, False), (20, 32, 4, True),
                                         (64, 64, 6, False), (1, 64, 8, False)])
def test_few_token_topk_shapes(T, E, k, zero):
    """The few-token router's finish at every segment width it uses (16 lanes
    per token up to T = 16, 8 up to 32, 4 up to 64) and both of its round
    forms (at most four experts per lane held sorted in registers, more read
    from LDS each round); `zero`: a zero router, every logit tied."""
    require_gpu()
    shape = synth.LayerShape(T, 128, 256, E, k, E, "identity", 1.0)
    w = synth.make_weights(shape, seed=5)
    x = synth.make_hidden(T, 128, seed=5)
    case = synth.Case("topk", shape, 5, x, w)
    over = {}
    if zero:
        over = dict(router_w=np.zeros((E, 128), np.float32), router_b=np.zeros(E, np.float32))
    say(f"few-token top-k T={T} E={E} k={k} zero={zero}")
    res = GpuLayer(shape, w, max_tokens=T).run(x, **over)
    ref = _oracle(case, **over)
    check_routing(res, ref)
    if zero:
        assert np.all(res["topk_idx"] == np.arange(k)[None, :])
    assert_out_close(res["out"], ref["out"])


@pytest.mark.parametrize("T", [16, 300])
def test_out_of_range_slot_sets_flag_and_contributes_zero(T):
    require_gpu()
    case = synth.make_case("tiny", T=T)
    table = case.weights.slot_table.copy()
    table[2] = 1000
    say(f"tiny: bad slot, T={T}")
    res = gpu_layer(case).run(case.hidden, slot_table=table)
    assert res["flags"] & 1
    ref = _oracle(case, slot_table=table)
    check_routing(res, ref)
    assert_out_close(res["out"], ref["out"])
    clean = gpu_layer(case).run(case.hidden)
    assert clean["flags"] == 0                    # each forward clears the flags


@pytest.mark.parametrize("T", [16, 300])
def test_out_of_range_shared_slot_sets_flag_and_contributes_zero(T):
    require_gpu()
    case = synth.make_case("shared_tiny", T=T)
    table = case.weights.slot_table.copy()
    table[case.shape.num_experts] = -1            # the shared expert's slot
    say(f"shared_tiny: bad shared slot, T={T}")
    res = gpu_layer(case).run(case.hidden, slot_table=table)
    assert res["flags"] & 1
    ref = _oracle(case, slot_table=table)
    check_routing(res, ref)
    assert_out_close(res["out"], ref["out"])
    routed_only = oracle.forward(case.hidden, top_k=1, precision="f64",
                                 **dict(weights_kwargs(case.weights), slot_table=table[:-1]))["out"]
    np.testing.assert_allclose(ref["out"], routed_only, rtol=0, atol=0)


@pytest.mark.parametrize("name,T", [("fine_tiny", 16), ("fine_tiny", 300), ("tiny_q8g128", 300), ("tiny", 16)])
def test_deterministic_and_slot_permutation_invariant(name, T):
    require_gpu()
    case = synth.make_case(name, T=T)
    g = gpu_layer(case)
    say(f"{name}: determinism, T={T}")
    a = g.run(case.hidden)
    b = g.run(case.hidden)
    np.testing.assert_array_equal(a["out_bits"], b["out_bits"])
    # the same experts moved to other slots give the same bits
    w = case.weights
    S = w.w_gate.shape[0]
    pi = np.random.default_rng(5).permutation(S)
    moved = {}
    for f in ("w_gate", "w_up", "w_down", "s_gate", "z_gate", "s_up", "z_up", "s_down", "z_down"):
        arr = np.empty_like(getattr(w, f))
        arr[pi] = getattr(w, f)
        moved[f] = arr
    w2 = dataclasses.replace(w, slot_table=pi[w.slot_table].astype(np.int32), **moved)
    say(f"{name}: permuted pool")
    c = GpuLayer(case.shape, w2, max_tokens=4096).run(case.hidden)
    np.testing.assert_array_equal(a["out_bits"], c["out_bits"])


_GRAPH_CASES = {
    "fine_tiny": synth.case_shape("fine_tiny"),
    # pools with room for a second copy of every expert (shared one included)
    "q8g128_shared": synth.LayerShape(16, 256, 384, 8, 1, 24, "sparse", 1.0, 1, 8, 128),
    "q4g128_prefill": synth.LayerShape(200, 256, 384, 8, 2, 16, "sparse", 1.0, 0, 4, 128),
}


@pytest.mark.parametrize("name", sorted(_GRAPH_CASES))
def test_graph_replay_matches_eager_and_reads_inputs_at_replay(name):
    torch = require_gpu()
    shape = _GRAPH_CASES[name]
    T = shape.T
    case = synth.Case(name, shape, 0, synth.make_hidden(T, shape.d_model, 0), synth.make_weights(shape, 0))
    g = gpu_layer(case)
    T, d = case.shape.T, case.shape.d_model
    x1 = case.hidden
    x2 = synth.make_hidden(T, d, seed=99)
    e1 = g.run(x1)
    e2 = g.run(x2)
    # a pool in which every expert also has a copy in an unused slot
    w = case.weights
    S = w.w_gate.shape[0]
    free = sorted(set(range(S)) - set(w.slot_table.tolist()))
    copy_table = np.array(free[:len(w.slot_table)], np.int32)
    arrays = {}
    for f in ("w_gate", "w_up", "w_down", "s_gate", "z_gate", "s_up", "z_up", "s_down", "z_down"):
        arr = getattr(w, f).copy()
        arr[copy_table] = arr[w.slot_table]
        arrays[f] = arr
    w2 = dataclasses.replace(w, **arrays)
    gl = GpuLayer(case.shape, w2, max_tokens=T)
    stream = torch.cuda.Stream()
    xb = gl.hidden(x1)
    table = gl.to_device(w.slot_table)
    out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    ws = gl.layer.new_workspace(T)
    torch.cuda.synchronize()  # the zero fill runs on the default stream, the replays on `stream`
    say(f"{name}: capture, T={T}")
    with torch.cuda.stream(stream):
        gl.layer.capture(xb, gl.router_w, gl.router_b, table, gl.dw, out, ws, stream)
    from gpu_util import bf16_bits_to_f64
    ref1 = _oracle(case)
    for rep in range(3):
        with torch.cuda.stream(stream):
            gl.layer.replay(stream)
        stream.synchronize()
        got = out.cpu().view(torch.int16).numpy()
        np.testing.assert_array_equal(got, e1["out_bits"], err_msg=f"replay {rep}")
        # the replay against the oracle itself: routing bit-exact, out within 2e-2
        check_routing({k: v.cpu().numpy() for k, v in gl.layer.routing(ws, T).items()}, ref1)
        assert_out_close(bf16_bits_to_f64(out), ref1["out"], what=f"replay {rep}")
        _ = (xb.float() * 2).sum().item()             # eager work between replays
    # new hidden states and a rewritten slot table, read at replay
    xb.copy_(gl.hidden(x2))
    table.copy_(gl.to_device(copy_table))
    torch.cuda.synchronize()
    ref2 = _oracle(case, hidden=x2, **{f: arrays[f] for f in arrays}, slot_table=copy_table)
    for rep in range(2):
        with torch.cuda.stream(stream):
            gl.layer.replay(stream)
        stream.synchronize()
        np.testing.assert_array_equal(out.cpu().view(torch.int16).numpy(), e2["out_bits"], err_msg=f"rep {rep}")
        check_routing({k: v.cpu().numpy() for k, v in gl.layer.routing(ws, T).items()}, ref2)
        assert_out_close(bf16_bits_to_f64(out), ref2["out"], what=f"rewritten inputs, replay {rep}")
        _ = (xb.float() * 3).sum().item()


def test_zero_tokens_is_a_noop():
    torch = require_gpu()
    case = synth.make_case("tiny")
    g = gpu_layer(case)
    x = torch.empty((0, case.shape.d_model), dtype=torch.bfloat16, device="cuda")
    out = g.layer.forward(x, g.router_w, g.router_b, g.slot_table, g.dw)
    torch.cuda.synchronize()
    assert out.shape == (0, case.shape.d_model)


def test_one_workspace_across_token_counts_keeps_control_words_zero():
    """The fused kernels' completion tickets live at the start of the workspace
    (moe_control_bytes of them); every call must leave them zero, whatever T
    the previous call had."""
    torch = require_gpu()
    case0 = synth.make_case("fine_tiny")
    g = gpu_layer(case0)
    ws = g.layer.new_workspace(300)
    for T in (16, 5, 64, 1, 300, 16, 65, 3):
        case = synth.make_case("fine_tiny", T=T)
        say(f"fine_tiny: shared workspace, T={T}")
        x = g.hidden(case.hidden)
        out = g.layer.forward(x, g.router_w, g.router_b, g.slot_table, g.dw, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:g.layer.control_bytes()].abs().sum().item()) == 0, f"control words not cleared after T={T}"
        ref = _oracle(case)
        from gpu_util import bf16_bits_to_f64
        assert_out_close(bf16_bits_to_f64(out), ref["out"])
        idx = g.layer.routing(ws, T)["topk_idx"].cpu().numpy()
        np.testing.assert_array_equal(idx, ref["topk_idx"])


@pytest.mark.parametrize("name,T", [("tiny_q4g128", 16), ("tiny_q4g128", 300), ("tiny_q8g128", 16),
                                    ("tiny_q8g128", 300)])
def test_zero_group_scales(name, T):
    """Groups whose scale is 0 contribute nothing (the codes may be anything);
    the prefill kernels keep their running sums in the previous group's scale."""
    require_gpu()
    case = synth.make_case(name, T=T)
    w = case.weights
    arrays = {f: getattr(w, f).copy() for f in ("s_gate", "s_up", "s_down")}
    for e in range(case.shape.num_experts):
        sl = int(w.slot_table[e])
        arrays["s_gate"][sl, 0, ::3] = 0          # first group of every third gate row
        arrays["s_up"][sl, 1, :] = 0              # the whole second group of up
        arrays["s_down"][sl, 1:, 5] = 0           # all but the first group of down row 5
    w2 = dataclasses.replace(w, **arrays)
    case2 = synth.Case(name, case.shape, case.seed, case.hidden, w2)
    say(f"{name}: zero group scales, T={T}")
    res = GpuLayer(case.shape, w2, max_tokens=T).run(case.hidden)
    ref = _oracle(case2)
    check_routing(res, ref)
    assert_out_close(res["out"], ref["out"])


@pytest.mark.parametrize("name", ["tiny", "fine_tiny", "tiny_q8g128"])
def test_maximum_token_count(name):
    """T = 65536, the largest max_tokens the library accepts (fine_tiny: 393216
    routed rows through the multi-block regroup)."""
    require_gpu()
    T = 65536
    case = synth.make_case(name, T=T)
    say(f"{name}: T={T}")
    res = GpuLayer(case.shape, case.weights, max_tokens=T).run(case.hidden)
    ref = _oracle(case)
    check_routing(res, ref)
    assert res["flags"] == 0
    assert_out_close(res["out"], ref["out"])


@pytest.mark.parametrize("bits,group,T", [(4, 128, 16), (4, 128, 300), (8, 128, 300), (8, 0, 300)])
def test_narrow_layer_formats(bits, group, T):
    """d = 128: one k-group for the gate/up inputs and the narrow (128-column)
    prefill down kernel, for every weight format."""
    require_gpu()
    shape = synth.LayerShape(T, 128, 256, 8, 2, 8, "identity", 0.0, 0, bits, group)
    w = synth.make_weights(shape, seed=5)
    x = synth.make_hidden(T, 128, seed=5)
    case = synth.Case("narrow", shape, 5, x, w)
    say(f"narrow d=128: bits={bits} group={group} T={T}")
    res = GpuLayer(shape, w, max_tokens=T).run(x)
    ref = _oracle(case)
    check_routing(res, ref)
    assert_out_close(res["out"], ref["out"])


@pytest.mark.parametrize("T", [64, 4096])
def test_one_hot_expert_takes_every_token(T):
    """A router bias that sends every token's first choice to expert 5: one
    group of T rows (32 row tiles at T = 4096), the others share the second
    choices."""
    require_gpu()
    case = synth.make_case("fine_tiny", T=T)
    b = np.zeros(case.shape.num_experts, np.float32)
    b[5] = 50.0
    say(f"fine_tiny: one hot expert, T={T}")
    res = gpu_layer(case).run(case.hidden, router_b=b)
    ref = _oracle(case, router_b=b)
    assert np.all(ref["topk_idx"][:, 0] == 5) and ref["counts"][5] == T
    check_routing(res, ref)
    assert_out_close(res["out"], ref["out"])


@pytest.mark.parametrize("T,E,k,slots,kind,zipf,group", [(300, 2, 2, 2, "identity", 0.0, 0),
                                                            (400, 2, 2, 2, "perm", 0.0, 0),
                                                            (513, 2, 2, 2, "identity", 0.0, 0),
                                                            (500, 3, 2, 5, "sparse", 1.0, 0),
                                                            (700, 4, 2, 4, "perm", 1.2, 0),
                                                            (400, 2, 2, 2, "identity", 0.0, 128)])
def test_prefill_ragged_row_tiles(T, E, k, slots, kind, zipf, group):
    """Prefill layers (d = d_ff = 256) whose experts end in ragged 128-row
    tiles: 44 rows after two full tiles (k = E: every token in every group),
    16 rows, a lone row after four full tiles, and Zipf-skewed groups over a
    permuted or sparse slot pool; one grouped-scale case."""
    require_gpu()
    shape = synth.LayerShape(T, 256, 256, E, k, slots, kind, zipf, 0, 4, group)
    w = synth.make_weights(shape, seed=11)
    x = synth.make_hidden(T, 256, seed=11)
    case = synth.Case("ragged_prefill", shape, 11, x, w)
    say(f"ragged prefill tiles: T={T} E={E} k={k} slots={slots}/{kind} zipf={zipf} group={group}")
    res = GpuLayer(shape, w, max_tokens=T).run(x)
    ref = _oracle(case)
    check_routing(res, ref)
    assert res["flags"] == 0
    assert_out_close(res["out"], ref["out"])
    say(f"ragged prefill tiles: ok, rows per expert {ref['counts'].tolist()}")


def test_layers_graph_at_the_benchmarked_decode_shape_matches_the_oracle():
    """The graph bench.py times: several Mixtral-shaped decode layers (T = 16,
    d = 4096, d_ff = 14336, E = 8, top-2) back to back in one HIP graph, each
    with its own handle, its own copy of the weight pool and its own output,
    one shared workspace -- built by bench.py's own graph builder.  Every
    layer's output is checked against the oracle on every replay, and after a
    pool copy is rewritten in place (two experts' weights exchanged) only the
    layer reading that copy changes, to the oracle's new result."""
    torch = require_gpu()
    import bench
    from expert_ffn_layer_router_amd import DeviceWeights, MoeLayer, to_device
    from gpu_util import bf16_bits_to_f64
    case = synth.make_case("mixtral_decode")
    shape, w = case.shape, case.weights
    T, d, nl = shape.T, shape.d_model, 3
    say(f"mixtral_decode: {nl}-layer graph, T={T}")
    x = to_device(case.hidden).view(torch.bfloat16)
    rw, st = to_device(w.router_w), to_device(w.slot_table)
    pools = [DeviceWeights.upload(w)]
    pools += [pools[0].clone() for _ in range(nl - 1)]
    layers = [MoeLayer(d, shape.d_ff, shape.num_experts, shape.top_k, shape.num_slots, T) for _ in range(nl)]
    outs = [torch.empty((T, d), dtype=torch.bfloat16, device="cuda") for _ in range(nl)]
    ws = layers[0].new_workspace(T)
    stream = torch.cuda.Stream()  # (build_layer_graph orders it after the zero fill and pool copies)
    graph = bench.build_layer_graph(layers, pools, outs, x, rw, None, st, ws, stream, torch)
    ref = _oracle(case)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        stream.synchronize()
        for i, o in enumerate(outs):
            assert_out_close(bf16_bits_to_f64(o), ref["out"], what=f"layer {i}, replay {rep}")
        check_routing({k: v.cpu().numpy() for k, v in layers[-1].routing(ws, T).items()}, ref)
        _ = (x.float() * 2).sum().item()             # eager work between replays
    # pool copy 1 now holds another layer: experts 0 and 1 exchange weights
    s0, s1 = int(w.slot_table[0]), int(w.slot_table[1])
    for f, t in pools[1].tensors.items():
        a = t[s0].clone()
        t[s0].copy_(t[s1])
        t[s1].copy_(a)
    swapped = {}
    for f in ("w_gate", "w_up", "w_down", "s_gate", "z_gate", "s_up", "z_up", "s_down", "z_down"):
        arr = getattr(w, f).copy()
        arr[[s0, s1]] = arr[[s1, s0]]
        swapped[f] = arr
    ref_sw = _oracle(case, **swapped)
    assert np.abs(ref_sw["out"] - ref["out"]).max() > 0.1 * np.abs(ref["out"]).max()
    torch.cuda.synchronize()
    before = [o.cpu().view(torch.int16).numpy().copy() for o in outs]
    with torch.cuda.stream(stream):
        graph.replay()
    stream.synchronize()
    for i, o in enumerate(outs):
        if i == 1:
            assert_out_close(bf16_bits_to_f64(o), ref_sw["out"], what="rewritten pool copy")
        else:
            np.testing.assert_array_equal(o.cpu().view(torch.int16).numpy(), before[i], err_msg=f"layer {i}")
            assert_out_close(bf16_bits_to_f64(o), ref["out"], what=f"layer {i} after the rewrite")


@pytest.mark.parametrize("name,T,dense", [("tiny", 14, True), ("tiny", 15, True), ("tiny_q4g128", 16, False),
                                          ("tiny_q8", 16, False), ("tiny_q8g128", 16, False)])
def test_dense_tiles_formats_and_ragged_tokens(name, T, dense):
    """Few tokens with nearly every expert routed to run dense tiles (every
    expert takes all T tokens; the router runs beside the gate/up GEMM), for
    per-row int4 weights: ragged T; the grouped and 8-bit formats at the same
    shapes keep routed tiles (tiny_q8g128 with a shared expert)."""
    require_gpu()
    import bench
    case = synth.make_case(name, T=T)
    assert bench.dense_decode(case.shape) == dense
    say(f"{name}: dense tiles, T={T}")
    res = gpu_layer(case).run(case.hidden)
    ref = _oracle(case)
    check_routing(res, ref)
    assert res["flags"] == 0
    assert_out_close(res["out"], ref["out"])


def test_dense_tiles_with_shared_experts_and_k_equal_e():
    require_gpu()
    import bench
    for shape in (synth.LayerShape(16, 128, 256, 8, 2, 11, "sparse", 0.0, 2),
                  synth.LayerShape(16, 128, 256, 4, 4, 4, "identity", 0.0, 0)):
        w = synth.make_weights(shape, seed=7)
        x = synth.make_hidden(16, 128, seed=7)
        case = synth.Case("dense", shape, 7, x, w)
        assert bench.dense_decode(shape)
        say(f"dense: E={shape.num_experts} k={shape.top_k} shared={shape.num_shared}")
        res = GpuLayer(shape, w).run(x)
        ref = _oracle(case)
        check_routing(res, ref)
        assert_out_close(res["out"], ref["out"])


def test_dense_tiles_flag_only_routed_experts_with_bad_slots():
    """Dense tiles compute every expert's gate/up before the routing is known;
    an expert nobody routes to may have an invalid slot (e.g. not resident in
    the expert cache) without raising the flag, while a routed one raises it
    and contributes zero."""
    require_gpu()
    case = synth.make_case("tiny")
    E = case.shape.num_experts
    bias = np.zeros(E, np.float32)
    bias[7] = -50.0                          # expert 7: never routed to
    table = case.weights.slot_table.copy()
    table[7] = -1
    say("tiny dense: unrouted expert with slot -1")
    res = gpu_layer(case).run(case.hidden, slot_table=table, router_b=bias)
    ref = _oracle(case, slot_table=table, router_b=bias)
    assert ref["counts"][7] == 0
    assert res["flags"] == 0
    check_routing(res, ref)
    assert_out_close(res["out"], ref["out"])
    bias[2] = 50.0                           # expert 2: every token's first choice, at a bad slot
    table[2] = 1000
    say("tiny dense: routed expert at slot 1000")
    res = gpu_layer(case).run(case.hidden, slot_table=table, router_b=bias)
    ref = _oracle(case, slot_table=table, router_b=bias)
    assert ref["counts"][2] == 16
    assert res["flags"] & 1
    check_routing(res, ref)
    assert_out_close(res["out"], ref["out"])


def test_one_workspace_across_dense_and_routed_plans():
    """The same workspace through dense-tile (T = 14..16) and routed-tile
    plans: every call leaves the control words zero and matches the oracle."""
    torch = require_gpu()
    import bench
    from gpu_util import bf16_bits_to_f64
    case0 = synth.make_case("tiny")
    g = gpu_layer(case0)
    ws = g.layer.new_workspace(300)
    kinds = set()
    for T in (16, 5, 14, 64, 16, 300, 15, 1, 16):
        case = synth.make_case("tiny", T=T)
        kinds.add(bench.dense_decode(case.shape))
        say(f"tiny: shared workspace, T={T}")
        out = g.layer.forward(g.hidden(case.hidden), g.router_w, g.router_b, g.slot_table, g.dw, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:g.layer.control_bytes()].abs().sum().item()) == 0, f"control words not cleared after T={T}"
        ref = _oracle(case)
        assert_out_close(bf16_bits_to_f64(out), ref["out"])
        np.testing.assert_array_equal(g.layer.routing(ws, T)["topk_idx"].cpu().numpy(), ref["topk_idx"])
    assert kinds == {True, False}
