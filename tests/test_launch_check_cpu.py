"""The launch-configuration rule that every kernel launch and every kernel
node of a captured step graph must pass (mak_launch_check in
transformer_forward_pass_amd/csrc/mak_internal.h), compiled on the host with
g++ and exercised case by case: grid, workgroup bound, dynamic-LDS ceiling,
total LDS per workgroup."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "transformer_forward_pass_amd", "csrc", "mak_internal.h")

CASES = [
    # gx, gy, gz, bx, by, bz, max_threads, static, dyn, max_dyn, per_block, expected rule
    (1, 1, 1, 256, 1, 1, 256, 1024, 0, 65536, 163840, 0),
    (4096, 1, 1, 512, 1, 1, 512, 4096, 96 * 1024, 96 * 1024, 163840, 0),
    (0, 1, 1, 256, 1, 1, 256, 0, 0, 65536, 163840, 1),
    (5, 0, 1, 256, 1, 1, 256, 0, 0, 65536, 163840, 1),
    (5, 1, 1, 512, 1, 1, 256, 0, 0, 65536, 163840, 2),
    (5, 1, 1, 16, 16, 4, 512, 0, 0, 65536, 163840, 2),
    (5, 1, 1, 0, 1, 1, 512, 0, 0, 65536, 163840, 2),
    (5, 1, 1, 256, 1, 1, 256, 0, 96 * 1024 + 1, 96 * 1024, 163840, 3),
    (5, 1, 1, 256, 1, 1, 256, 8192, 156 * 1024, 160 * 1024, 163840, 4),
    (5, 1, 1, 256, 1, 1, 256, 4096, 156 * 1024, 160 * 1024, 163840, 0),
]


def test_launch_check_rules(tmp_path):
    src = tmp_path / "t.cpp"
    lines = ['#include "%s"' % HDR, "#include <cstdio>", "int main() {", "  int bad = 0;"]
    for c in CASES:
        *args, want = c
        lines.append("  if (mak_launch_check(%s) != %d) { std::printf(\"case %s\\n\"); bad++; }"
                     % (", ".join("%dLL" % a if i >= 6 else "%du" % a for i, a in enumerate(args)), want,
                        ",".join(map(str, c))))
    lines += ["  return bad;", "}"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "t"
    subprocess.run(["g++", "-std=c++17", "-O1", "-o", str(exe), str(src)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
