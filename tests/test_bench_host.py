"""Host logic of bench.py, on the CPU: the rows the early-exit window reads per
sequence, the margin rule the bench's parity sample applies, and the pooled
oracle baseline (worker pool, /dev/shm hand-off, parity counting) on a small
batch with a planted mismatch."""
import multiprocessing

import numpy as np

import bench
import oracle
from draft_token_verification_06_amd import synth


def test_early_exit_rows_follow_the_block_schedule():
    # gamma = 8: blocks [0,1), [1,3), [3,9) over target rows, draft rows up to 8
    assert bench.early_exit_rows([0], 8) == 2
    assert bench.early_exit_rows([1], 8) == 2 + 4
    assert bench.early_exit_rows([2], 8) == 2 + 4
    for n in range(3, 9):
        assert bench.early_exit_rows([n], 8) == 2 * 8 + 1
    assert bench.early_exit_rows([0, 1, 8], 8) == 2 + 6 + 17
    for gamma in (1, 2, 5, 17, 64):
        rows = [bench.early_exit_rows([n], gamma) for n in range(gamma + 1)]
        assert rows == sorted(rows) and rows[0] == 2 and rows[-1] == 2 * gamma + 1


def test_margin_rule_looks_only_at_the_point_of_divergence():
    o = {"n": 2, "out": [5, 6, 7], "ratio": [0.9, 0.30001, 0.2], "u": [0.1, 0.3, 0.25],
         "sample": {"tau": 0.5, "Z": 1.0, "C_lo": 0.4, "C_hi": 0.6}}
    # GPU accepted draft 2 where the oracle rejected it: only position 2 counts
    assert not bench._margin_case(o, 3, [5, 6, 7, 9])
    o2 = dict(o, ratio=[0.9, 0.8, 0.250001], u=[0.1, 0.3, 0.25])
    assert bench._margin_case(o2, 3, [5, 6, 7, 9])
    # a near-threshold test at position 1 does not excuse a divergence at 2
    o3 = dict(o, ratio=[0.9, 0.300001, 0.2], u=[0.1, 0.3, 0.25])
    assert not bench._margin_case(o3, 3, [5, 6, 7, 9])
    # same n, different draw: only the draw's CDF margin counts
    assert not bench._margin_case(o, 2, [5, 6, 8])
    o4 = dict(o, sample={"tau": 0.4000001, "Z": 1.0, "C_lo": 0.4, "C_hi": 0.6})
    assert bench._margin_case(o4, 2, [5, 6, 8])
    assert not bench._margin_case(o4, 2, [5, 9, 8])  # accepted drafts must agree


def test_pooled_oracle_baseline_counts_a_planted_mismatch(monkeypatch):
    B = 3
    monkeypatch.setattr(bench, "B", B)
    # a second, timing-only round of the four calls
    monkeypatch.setattr(bench, "CPU_SAMPLE_SECONDS", 1e9)
    monkeypatch.setattr(bench, "CPU_SAMPLE_MAX_ROUNDS", 2)
    data = [synth.window_config5(a, B=B, seed=1005 + k, device="cpu") for k, a in enumerate(bench.ALPHAS)]
    ref = []
    for d in data:
        ns, outs, Ps = [], [], []
        for b in range(B):
            T = oracle.decode(synth.to_host_bits(d["target"][b]), "bf16")
            D = oracle.decode(synth.to_host_bits(d["draft"][b]), "bf16")
            u, v = oracle.window_uniforms(0, 0, b, 0, bench.GAMMA)
            o = oracle.verify_window(T, D, d["tokens"][b].numpy(), bench.GAMMA, u, v)
            ns.append(o["n"])
            outs.append(o["out"] + [-1] * (bench.GAMMA + 1 - len(o["out"])))
            Ps.append(o["P"] + [0.0] * (bench.GAMMA - len(o["P"])))
        ref.append((np.array(ns), np.array(outs), np.array(Ps)))
    n1 = ref[1][0][2]
    ref[1][1][2, n1] = (ref[1][1][2, n1] + 1) % 128256  # a wrong draw
    with multiprocessing.get_context("fork").Pool(2) as pool:
        base, parity = bench.cpu_baseline(pool, data, ref)
    assert parity["sequences"] == len(bench.ALPHAS) * B
    assert parity["mismatches"] == 1 and parity["margin_cases"] == 0
    assert base["cores"] == 2 and base["kind"] == "oracle" and base["value"] > 0
    assert sorted(base["full_call_wall_s"]) == sorted(str(a) for a in bench.ALPHAS)
    assert base["single_core_ms_per_sequence"] > 0
    assert base["calls"] == 2 * len(bench.ALPHAS) and base["sample"].startswith("2 round(s)")
    assert 0 < base["cpu_seconds"] and abs(base["value"] - B * bench.GAMMA * base["calls"] / base["seconds"]) < 1e-6 * base["value"]
    assert len(parity["beta"]) == len(bench.ALPHAS)
    for st in parity["beta"]:
        assert 1.0 <= st["exact_expected_emitted"] <= bench.GAMMA + 1 and 0.0 < st["mean_alpha"] < 1.0
