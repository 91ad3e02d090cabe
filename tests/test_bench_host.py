"""Host logic of bench.py (no GPU): when the committed counter traffic is reported, and the
one-GPU guard."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "block_sparse_attention_11_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def test_traffic_reported_only_for_its_workload_and_sources(tmp_path, monkeypatch):
    """A counter record is used only for its own workload and while the kernel's sources
    hash to the value stored with it (the committed record itself may predate the
    current sources; then bench reports traffic as null)."""
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    wl = int(rec["workload_id"])
    fresh = dict(rec, kernels={k: dict(v, sources_sha256=_sources_sha256(v["sources"]))
                               for k, v in rec["kernels"].items()})
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(fresh))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    for kernel, entry in rec["kernels"].items():
        assert bench._measured_traffic(kernel, wl) == entry["bytes_per_launch"], kernel
        assert bench._measured_traffic(kernel, wl + 1) is None, kernel
    assert bench._measured_traffic("no_such_kernel", wl) is None
    # a record whose source hash no longer matches the sources is not used
    stale = dict(rec, kernels={k: dict(v, sources_sha256="0" * 64) for k, v in rec["kernels"].items()})
    path.write_text(json.dumps(stale))
    for kernel in rec["kernels"]:
        assert bench._measured_traffic(kernel, wl) is None, kernel


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_route_pairs_count_group_members_with_the_m128_launch():
    """The per-route split attributes the pairs of blocks that run inside group items to the
    M128 launch; the two routes together hold every useful pair of the plan."""
    import numpy as np
    import block_sparse_attention_11_amd as K
    from workloads import make_workload
    w = make_workload(3, heads=[0])
    plan = K.kpage_plan(w)
    members = K.kpage_plan_export(plan, "group_members")
    members = members[members >= 0]
    assert members.size > 0
    with_groups = bench._route_pairs(w, K, plan)
    plain = bench._route_pairs(w)
    useful = K.kpage_plan_stats(plan)["useful"]
    assert with_groups["q128"] + with_groups["q64"] == useful == plain["q128"] + plain["q64"]
    moved = sum(int(w.q_valid[0, q]) * int(np.asarray(w.kv_valid[0])[w.q2k_idx[w.q2k_ptr[0, q]:w.q2k_ptr[0, q + 1]]].sum())
                for q in members)
    assert with_groups["q128"] - plain["q128"] == moved
