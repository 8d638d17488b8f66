"""bench.py on the host, without a GPU: the one-GPU contract and the profile-summary reader."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                           capture_output=True, text=True, env={**os.environ, **env}, timeout=300)
        assert r.returncode == 2, (argv, r.stderr)
        assert "one GPU" in r.stderr and r.stdout == ""


def test_committed_profiles_are_readable_and_name_their_workload():
    import bench
    for name in ("large_hidden", "training", "fine_grained", "imbalanced"):
        path = os.path.join(ROOT, "profiles", "kernels_%s.md" % name)
        assert os.path.exists(path), path
        meta = [json.loads(l) for l in open(path) if l.strip().startswith("{")]
        assert len(meta) == 1 and meta[0]["workload"] == name
        kernels = meta[0]["kernels"]
        # every GEMM and row kernel of the step is in the table, with calibrated traffic
        fams = {bench._family(k) for k in kernels}
        for k in ("moe_fprop_w13_swiglu", "moe_fprop_w2", "moe_w2_backward", "moe_dgrad_w13",
                  "moe_wgrad_w13", "moe_combine<true>", "moe_combine<false>",
                  "moe_combine_bwd_dscores"):
            assert k in fams, (name, k)
        assert all(v["traffic_bytes"] and v["timed_avg_us"] > 0 for v in kernels.values())
