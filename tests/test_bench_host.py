"""Host logic of bench.py (no device): the algorithmic work it divides by, and
when a committed counter summary may supply the `traffic` figure."""

import json

import bench
import synth


def test_algorithmic_bytes_of_the_decode_gate_up_launch():
    """8 active Mixtral-shaped int4 experts: gate and up codes (d d_ff / 2 bytes
    each) and fp16 (s, z) per output row of both, plus the 16 x rows read and
    the 32 h rows written in bf16 -- worked out by hand; the router runs in the
    same launch (dense tiles), so its fp32 weights, bias and the slot table
    count too."""
    shape = synth.case_shape("mixtral_decode")
    work = bench.algorithmic_work(shape, [4] * 8)
    per_expert = 2 * 14336 * 4096 // 2 + 2 * 2 * 2 * 14336
    router = 4 * 8 * 4096 + 4 * 8 + 4 * 8
    assert work["gate_up"]["bytes"] == 8 * per_expert + 2 * 16 * 4096 + 2 * 32 * 14336 + router == 471859264
    fine = synth.case_shape("fine_decode")      # routed tiles: the router has a launch of its own
    per_fine = 2 * 2048 * 4096 // 2 + 2 * 2 * 2 * 2048
    assert bench.algorithmic_work(fine, [1] * 64)["gate_up"]["bytes"] == 64 * per_fine + 2 * 16 * 4096 + 2 * 96 * 2048
    assert work["gate_up"]["flops"] == 4 * 32 * 4096 * 14336
    assert work["down"]["flops"] == 2 * 32 * 4096 * 14336


def test_inactive_experts_move_no_weight_bytes():
    shape = synth.case_shape("mixtral_decode")
    full, half = bench.algorithmic_work(shape, [4] * 8), bench.algorithmic_work(shape, [8, 0] * 4)
    per_expert = 2 * 14336 * 4096 // 2 + 2 * 2 * 2 * 14336
    assert full["gate_up"]["bytes"] - half["gate_up"]["bytes"] == 4 * per_expert
    assert half["active"] == 4


def _summary(tmp_path, workload, family_sha, fetch_kib, write_kib):
    prof = tmp_path / "profiles"
    prof.mkdir(exist_ok=True)
    data = {"workload": workload, "family_sha": family_sha, "scale": {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0},
            "kernels": {"void moe::stream_gemm_kernel<true, 1, 2, 4, true, 1, 4, false>(moe::StreamArgs)":
                        {"FETCH_SIZE": fetch_kib, "WRITE_SIZE": write_kib}}}
    (prof / f"stream_gemm_{workload}_pmc.json").write_text(json.dumps(data))


def test_traffic_is_read_while_the_family_sources_are_unchanged(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    shas = {f: bench.family_sha(f) for f in bench.GEMM_FAMILY_SOURCES}
    _summary(tmp_path, "wl", shas, fetch_kib=1000.0, write_kib=10.0)
    assert bench.load_traffic("wl", "stream_gemm_kernel<true") == (1000.0 * 2.0 + 10.0) * 1024.0
    # a change to the other family's sources leaves the summary valid
    _summary(tmp_path, "wl", dict(shas, prefill_gemm="0" * 16), fetch_kib=1000.0, write_kib=10.0)
    assert bench.load_traffic("wl", "stream_gemm_kernel<true") is not None
    # a change to its own family's sources voids it
    _summary(tmp_path, "wl", dict(shas, stream_gemm="0" * 16), fetch_kib=1000.0, write_kib=10.0)
    assert bench.load_traffic("wl", "stream_gemm_kernel<true") is None


def test_family_hash_follows_its_sources(tmp_path, monkeypatch):
    files = []
    for name in ("k.hip", "h.h"):
        p = tmp_path / name
        p.write_text(name)
        files.append(str(p))
    monkeypatch.setattr(bench, "GEMM_FAMILY_SOURCES", {"stream_gemm": files})
    before = bench.family_sha("stream_gemm")
    (tmp_path / "h.h").write_text("h.h changed")
    assert bench.family_sha("stream_gemm") != before


def test_graph_length_divides_the_step_count():
    """The timed region is whole replays of one graph: its length divides the
    step count, with at least two replays when that leaves 4 or more layers
    per graph, and never more layers than the model has."""
    for steps in list(range(1, 70)) + [96, 97, 100, 128, 256, 1000]:
        n = bench.graph_length(steps, 32)
        assert steps % n == 0 and 1 <= n <= max(32, 1)
        if steps >= 8 and any(steps % q == 0 for q in range(4, min(32, steps // 2) + 1)):
            assert steps // n >= 2
    assert bench.graph_length(20) == 10
    assert bench.graph_length(256) == 32
    assert bench.graph_length(5) == 5
    assert bench.graph_length(7) == 7


def test_dense_rule_matches_the_library_plan():
    """bench.py's copy of the library's dense-tile rule: a dense plan keeps h
    rows for every expert and token (2 E T d_ff bytes and more), the routed plan
    only for the T k routed rows, which is less."""
    import ctypes
    from expert_ffn_layer_router_amd import _lib
    lib = _lib.load()
    for name, T in [("mixtral_decode", 16), ("mixtral_decode", 12), ("mixtral_decode", 3), ("mixtral_decode", 1),
                    ("fine_decode", 16), ("phi35_skew", 64), ("phi35_skew", 16), ("shared_decode", 16)]:
        s = synth.case_shape(name, T=T)
        cfg = _lib.MoeConfig(s.d_model, s.d_ff, s.num_experts, s.top_k, s.num_slots, 64, 0, s.num_shared, s.bits,
                             s.group)
        h = ctypes.c_void_p()
        assert lib.moe_create(ctypes.byref(cfg), ctypes.byref(h)) == 0
        n = ctypes.c_size_t()
        assert lib.moe_workspace_size(h, T, ctypes.byref(n)) == 0
        lib.moe_destroy(h)
        dense_h = 2 * (s.num_experts + s.num_shared) * T * s.d_ff
        assert bench.dense_decode(s) == (n.value >= dense_h), (name, T, n.value, dense_h)
    assert bench.dense_decode(synth.case_shape("mixtral_decode"))
    assert not bench.dense_decode(synth.case_shape("fine_decode"))
