"""CPU: the benchmark's results file (one JSON line per finished workload; --results / --resume)."""
import bench


def test_results_round_trip_and_resume(tmp_path):
    path = str(tmp_path / "results.jsonl")
    assert bench.load_results(path) == {}
    r3 = {"workload": "block-sparse causal prefill", "value": 1000.0, "unit": "TFLOP/s", "ms": 2.1}
    r5 = {"workload": "vertical-slash", "value": 800.0, "unit": "TFLOP/s", "ms": 25.0}
    bench.append_result(path, 3, r3)
    bench.append_result(path, 5, r5)
    with open(path, "a") as f:
        f.write('{"workload_index": 6, "result": {"va')  # a run cut off mid-write
    got = bench.load_results(path)
    assert got == {3: r3, 5: r5}
    # a later line for the same workload wins
    r3b = dict(r3, ms=2.05)
    with open(path, "a") as f:
        f.write("\n")
    bench.append_result(path, 3, r3b)
    assert bench.load_results(path) == {3: r3b, 5: r5}
