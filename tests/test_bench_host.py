"""Host logic of bench.py (no device): the algorithmic work it divides by, and
when a committed counter summary may supply the `traffic` figure."""

import json

import bench
import synth


def test_algorithmic_bytes_of_the_decode_gate_up_launch():
    """8 active Mixtral-shaped int4 experts: gate and up codes (d d_ff / 2 bytes
    each) and fp16 (s, z) per output row of both, plus the 16 x rows read and
    the 32 h rows written in bf16 -- worked out by hand."""
    shape = synth.case_shape("mixtral_decode")
    work = bench.algorithmic_work(shape, [4] * 8)
    per_expert = 2 * 14336 * 4096 // 2 + 2 * 2 * 2 * 14336
    assert work["gate_up"]["bytes"] == 8 * per_expert + 2 * 16 * 4096 + 2 * 32 * 14336 == 471728128
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
