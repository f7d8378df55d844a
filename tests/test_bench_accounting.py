"""bench.py's algorithmic work per call against the per-unit figures the
measurement plan fixes for the Flash ratio-4 and ratio-128 layers (4096-token
chunks): GEMM flops 2*T*N*H, and the pool's bytes (every projected kv/score
element read once, the APE table, the rows written, the live frontier rows
written).  The achieved GB/s and TFLOP/s in the bench line are these figures
over measured times, so a mistake here would misstate every roofline."""

import bench
from compressed_kv_attention_compressor_amd import synth

R4, R128 = synth.FLASH_R4, synth.FLASH_R128


def test_gemm_flops():
    assert bench.layer_algorithmic(R4, 0, 4096)[0] == 85_899_345_920
    assert bench.layer_algorithmic(R128, 0, 4096)[0] == 34_359_738_368
    assert bench.layer_algorithmic(R4, 0, 4096)[3] == 2560
    assert bench.layer_algorithmic(R128, 0, 4096)[3] == 1024


def test_pool_bytes_of_the_plain_path():
    # 4096 tokens from position 0 read 41,943,040 B of projection, 20,480 B of
    # APE, write 2,621,440 B of rows and 40,960 B of live frontier (ratio 4);
    # the bench's plain-path call covers tokens 1..4095 (one token's 10,240 B
    # fewer) and counts the ratio-4 frontier write in the separate carry
    # launch (read and written there).
    _, pb, rows, N = bench.layer_algorithmic(R4, 1, 4095)
    assert rows == 2048
    assert pb + N * 4 + bench.carry_bytes(R4, 1, 4095) // 2 == 44_625_920
    # Ratio 128: 16,777,216 + 262,144 + 65,536 B, no live frontier after 4096 tokens.
    _, pb, rows, N = bench.layer_algorithmic(R128, 1, 4095)
    assert rows == 32
    assert pb + N * 4 == 17_104_896


def test_fused_finisher_bytes():
    # Fused ratio-4 call: pooled rows read once and rows written (1024 rows x
    # 640 dims x 4 B, twice), plus the frontier tokens it writes from the
    # staged tokens (4 kept tokens x 1280 columns x 2 tensors, read and written).
    _, pb, _, _ = bench.layer_algorithmic(R4, 0, 4096)
    assert pb == 1024 * 640 * 4 * 2 + 4 * 1280 * 2 * 4 * 2 == 5_324_800


def test_decode_gemv_bytes_per_token():
    # The measurement plan's per-token decode figure for the 30 compressed
    # layers of the Flash stack: 440,401,920 B of bf16 weights (15 ratio-4
    # layers of 2560 x 4096 and 15 ratio-128 layers of 1024 x 4096).
    shapes = [(l, synth.stack_layer_shape(r)) for l, r in
              enumerate([0, 0] + [4 if l % 2 == 0 else 128 for l in range(2, 32)])]
    assert bench.decode_gemv_bytes(shapes) == 440_401_920
    assert bench.decode_gemv_bytes([(0, R4)]) == 20_971_520
    assert bench.decode_gemv_bytes([(0, R128)]) == 8_388_608


def test_more_than_one_gpu_is_refused():
    # One GPU is measured; asking for more exits non-zero with a message and
    # prints no result line.
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert '"metric"' not in r.stdout


def test_counter_summaries_go_stale_with_any_source_they_depend_on(tmp_path, monkeypatch):
    # A summary's counters are used only while its digest matches the kernel
    # source and the shared headers and build script it compiles with.
    import os
    import shutil
    csrc = tmp_path / "compressed_kv_attention_compressor_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    for f in ("proj_gemm.hip", "device_common.h", "kernel_args.h", "launch.h"):
        shutil.copy(os.path.join(bench.ROOT, "compressed_kv_attention_compressor_amd", "csrc", f), csrc / f)
    shutil.copy(os.path.join(bench.ROOT, "compressed_kv_attention_compressor_amd", "build.py"),
                tmp_path / "compressed_kv_attention_compressor_amd" / "build.py")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "GEMM_SOURCE", str(csrc / "proj_gemm.hip"))
    monkeypatch.setattr(bench, "SHARED_SOURCES", [str(csrc / f) for f in ("device_common.h", "kernel_args.h", "launch.h")]
                        + [str(tmp_path / "compressed_kv_attention_compressor_amd" / "build.py")])
    digest = bench.source_digest(bench.GEMM_SOURCE)
    (tmp_path / "profiles" / "traffic_w.txt").write_text(
        f"# comment = ignored\ngemm_hbm_bytes_per_launch = 123\ngemm_sources_sha256 = {digest}\n")
    assert bench.read_traffic("w") == 123.0
    (csrc / "device_common.h").write_text((csrc / "device_common.h").read_text() + "\n// edit\n")
    assert bench.read_traffic("w") is None


def test_indexer_and_attention_counters_follow_their_own_sources(tmp_path, monkeypatch):
    # indexer_* and attention_* figures are keyed to indexer.hip and
    # attention.hip (plus the shared headers), not to the projection source.
    import os
    import shutil
    csrc = tmp_path / "compressed_kv_attention_compressor_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    for f in ("proj_gemm.hip", "indexer.hip", "attention.hip", "device_common.h", "kernel_args.h", "launch.h"):
        shutil.copy(os.path.join(bench.ROOT, "compressed_kv_attention_compressor_amd", "csrc", f), csrc / f)
    shutil.copy(os.path.join(bench.ROOT, "compressed_kv_attention_compressor_amd", "build.py"),
                tmp_path / "compressed_kv_attention_compressor_amd" / "build.py")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for name, f in (("GEMM_SOURCE", "proj_gemm.hip"), ("INDEXER_SOURCE", "indexer.hip"),
                    ("ATTENTION_SOURCE", "attention.hip")):
        monkeypatch.setattr(bench, name, str(csrc / f))
    monkeypatch.setattr(bench, "SHARED_SOURCES", [str(csrc / f) for f in ("device_common.h", "kernel_args.h", "launch.h")]
                        + [str(tmp_path / "compressed_kv_attention_compressor_amd" / "build.py")])
    for kind, src in (("indexer", "indexer.hip"), ("attention", "attention.hip")):
        (tmp_path / "profiles" / f"traffic_{kind}.txt").write_text(
            f"{kind}_hbm_bytes_per_call = 7\n{kind}_sources_sha256 = {bench.source_digest(str(csrc / src))}\n")
        assert bench.read_traffic(kind, f"{kind}_hbm_bytes_per_call") == 7.0
        (csrc / "proj_gemm.hip").write_text((csrc / "proj_gemm.hip").read_text() + "\n// edit\n")
        assert bench.read_traffic(kind, f"{kind}_hbm_bytes_per_call") == 7.0
        (csrc / src).write_text((csrc / src).read_text() + "\n// edit\n")
        assert bench.read_traffic(kind, f"{kind}_hbm_bytes_per_call") is None
