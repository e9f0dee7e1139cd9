"""Host logic of bench.py (CPU only): the algorithmic bytes behind
roofline.achieved match the oracle's compressed-bytes closed form plus the
query, output and side-output bytes; the committed traffic figure is used only
while the kernel sources match the hash recorded with it; more than one GPU is
refused."""
import json
import os
import shutil
import subprocess
import sys

import pytest

import bench
from oracle import accounting

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name", ["c5", "c4", "c3"])
def test_decode_bytes_match_the_oracle_closed_form(name):
    wl = bench.Workload(name, "cpu")
    w = wl.w
    F = w["n_sink"] + w["recent_window"] + 1
    wl.M = [2048, 0, 17, 1500][: wl.B] + [1024] * max(0, wl.B - 4)
    nbytes, tokens = wl.decode_bytes_and_tokens()
    kv = accounting.compressed_bytes(wl.d, wl.hkv, w["middle_k_bits"], w["middle_v_bits"], 32,
                                     [F] * wl.B, wl.M)
    qo = wl.B * wl.hq * wl.d * 2 * 2
    side = 4 * sum(F + m for m in wl.M) if wl.side else 0
    app = wl.B * wl.hkv * wl.d * 2 * 2           # the new token's fp16 K and V rows written into the cache
    # per sequence one demoted token: fp16 K and V rows read, packed K and V
    # codes and group scales written; with a score policy every live score
    # read and written
    packed = wl.hkv * (wl.d * (w["middle_k_bits"] + w["middle_v_bits"]) // 8 + 4 * (wl.d // 32))
    upd = wl.B * (wl.hkv * wl.d * 4 + packed)
    if wl.policy in ("h2o", "ema"):
        upd += 8 * sum(F + m for m in wl.M)
    assert nbytes == kv + qo + side + app + upd
    assert tokens == sum(F + m for m in wl.M)


def test_traffic_figure_tracks_the_kernel_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    import hashlib
    h = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles").mkdir()
    prof = tmp_path / "profiles" / "decode_attn_cx_hbm.txt"
    prof.write_text(f"traffic_bytes_per_call: 12345\nsources: k.hip\nsource_sha256: {h}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("cx") == 12345
    src.write_text("kernel v2\n")
    assert bench.measured_traffic("cx") is None
    assert bench.measured_traffic("missing") is None


def test_committed_traffic_profile_is_parseable():
    path = os.path.join(ROOT, "profiles", "decode_attn_c5_hbm.txt")
    fields = {}
    for line in open(path):
        k, sep, v = line.partition(":")
        if sep:
            fields[k.strip()] = v.strip()
    assert int(fields["traffic_bytes_per_call"]) > 134_000_000
    for s in fields["sources"].split():
        assert os.path.exists(os.path.join(ROOT, s))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
