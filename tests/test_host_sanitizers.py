"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two host-only builds, each with -fsanitize=address,undefined and no recovery, so
that any out-of-bounds access, use after free, signed overflow, misaligned or null
access in them aborts the test:
  * the managed window's plan (hybrid_linear_block_amd/csrc/hf_window.h), driven over
    the same chunk sequences as tests/test_window_plan.py and replayed on its ring model;
  * the C ABI's host side (csrc/hf_abi.hip: validation, workspace layouts, handle
    lifetime), with the sanitizers on its host pass only, linked with stand-ins for the
    kernel launchers, driven through every entry point with invalid and valid arguments. On a
    host without a GPU a valid call ends at the HIP runtime with HF_ERR_HIP.
No device code is built with a sanitizer.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import test_window_plan as twp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hybrid_linear_block_amd", "csrc")
INC = os.path.join(ROOT, "include")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


@pytest.fixture(scope="module")
def window_driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("window_asan")
    src = d / "drv.cc"
    src.write_text(twp.DRIVER)
    exe = d / "drv"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", *SAN, "-I", CSRC, str(src), "-o", str(exe)],
                   check=True)
    return str(exe)


def _run(exe, text):
    out = subprocess.run([exe], input=text, capture_output=True, text=True, env=ENV)
    assert out.returncode == 0, out.stderr[-3000:]
    return out.stdout.split("\n")[:-1]


def test_window_plan_sanitized(window_driver):
    rng = np.random.default_rng(7)
    cases = [(1560 * 3, 1560 * 9, 2), (1560 * 3, 1560 * 9, 5), (100, 900, 3)]
    for chunk, win, mult in cases:
        cap = mult * win
        ops = []
        for _ in range(40):
            ops += [f"B {chunk}", "A", "A"]
        text = f"{cap} {win} 0 {chunk}\n" + "\n".join(ops) + "\n"
        lines = _run(window_driver, text)
        twp.replay(lines, ops, cap, win, 0, chunk)
    for trial in range(20):  # random chunk sizes, large start indices, rejections
        win = int(rng.integers(5, 200))
        cap = int(rng.integers(2, 5)) * win
        ev0 = int(rng.integers(0, 10 ** 12))
        max_ev = int(rng.integers(1, 2 * win))
        ops = []
        for _ in range(60):
            ops.append(f"B {int(rng.integers(0, win + 3))}")
            ops += ["A"] * int(rng.integers(0, 3))
        text = f"{cap} {win} {ev0} {max_ev}\n" + "\n".join(ops) + "\n"
        lines = _run(window_driver, text)
        twp.replay(lines, ops, cap, win, ev0, max_ev)


# Stand-ins for the device-side launchers (no kernels are built here): each reports that
# no device is present, as the runtime itself does on this host.
STUBS = r"""
#include "hf_launch.h"
namespace hf {
int device_cu_count() { return 256; }
AbsorbPlan absorb_plan(int, int, int, int64_t n) { AbsorbPlan p{(int)(n > 0 ? n : 1), 1}; return p; }
int absorb_items(int, int heads, int, const AbsorbPlan& p) { return heads * p.n_split; }
size_t absorb_partial_floats(int heads, int d) { return (size_t)heads * 24 * (d * d + d); }
hipError_t launch_absorb(int, int, int, const void*, const void*, int64_t, int64_t, float*, float*,
                         float*, uint16_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_absorb_parts(int, int, int, const void*, const void*, int64_t, int64_t, float*,
                               hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_absorb_reduce(int, int, int, int64_t, const float*, float*, float*, uint16_t*,
                                hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_split_state(int, int, const float*, uint16_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_rope_table(float2*, int, int, double, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_block_pool(int, int, int, int, const void*, int64_t, int64_t, const void*, int64_t,
                             int64_t, float*, float*, int, int, hipStream_t, const KeyCache&,
                             const Rope&, const Ragged&) { return hipErrorNoDevice; }
hipError_t launch_absorb_and_pool(int, int, int, int, const void*, const void*, int64_t, int64_t,
                                  float*, const void*, int64_t, int64_t, const void*, int64_t,
                                  int64_t, float*, float*, int, int, hipStream_t, const KeyCache&,
                                  const Rope&) { return hipErrorNoDevice; }
hipError_t launch_score_select(int, int, int, int, int, int, const float*, const float*, float, int,
                               int32_t*, float*, hipStream_t, const Ragged&) {
  return hipErrorNoDevice; }
hipError_t launch_select_and_reduce(int, int, int, int, int, int, int, const float*, const float*,
                                    float, int, int32_t*, const float*, int64_t, float*, float*,
                                    uint16_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_sparse_swa(int, int, int, int, const void*, int64_t, int64_t, const void*,
                             const void*, int64_t, int64_t, const int32_t*, int, const float*,
                             const uint16_t*, const float*, float, float, void*, int64_t,
                             hipStream_t, const Rope&, const Ragged&, const AbsorbAhead&) {
  return hipErrorNoDevice; }
hipError_t launch_attend_backward(int, int, int, const BwdArgs&, int, hipStream_t) {
  return hipErrorNoDevice; }
hipError_t launch_absorb_backward(int, int, int, const void*, const void*, int64_t, int64_t,
                                  const float*, const float*, float*, float*, int64_t,
                                  hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_fill_zero(void*, size_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_copy_rows_kv(const void*, const void*, void*, void*, int, size_t, size_t,
                               hipStream_t) { return hipErrorNoDevice; }
}  // namespace hf
"""

ABI_DRIVER = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "hf.h"
#define EXPECT(x, want) do { int r_ = (int)(x); if (r_ != (int)(want)) { \
  std::printf("line %d: got %d want %d\n", __LINE__, r_, (int)(want)); return 1; } } while (0)
int main() {
  hf_config c = {12, 128, 64, HF_BF16, 1e-6f, 0.f, 4680, 14040, 4680, 55};
  const size_t ws = hf_workspace_bytes(&c);
  if (ws == 0 || hf_backward_workspace_bytes(&c) == 0) return 1;
  hf_config bad = c; bad.head_dim = 96;
  EXPECT(hf_workspace_bytes(&bad), 0);
  bad = c; bad.eps = 0.f;
  EXPECT(hf_workspace_bytes(&bad), 0);
  bad = c; bad.max_n_kv = (int64_t)1 << 40;
  EXPECT(hf_workspace_bytes(&bad), 0);
  EXPECT(hf_workspace_bytes(nullptr), 0);
  // fake, aligned device addresses: never dereferenced on the host
  char* A = reinterpret_cast<char*>((uintptr_t)1 << 20);
  hf_state* st = nullptr;
  EXPECT(hf_state_init(&c, (float*)A, (float*)A, A, ws - 1, 1, 0, nullptr, &st), HF_ERR_INVALID_ARG);
  EXPECT(hf_state_init(&c, (float*)(A + 4), (float*)A, A, ws, 1, 0, nullptr, &st), HF_ERR_INVALID_ARG);
  EXPECT(hf_state_init(&c, (float*)A, (float*)A, A, ws, 1, -1, nullptr, &st), HF_ERR_INVALID_ARG);
  EXPECT(hf_state_init(&c, (float*)A, (float*)A, A, ws, 1, 0, nullptr, nullptr), HF_ERR_INVALID_ARG);
  // a valid init reaches the runtime: no device on this host
  const int r = hf_state_init(&c, (float*)A, (float*)A, A, ws, 1, 0, nullptr, &st);
  if (r == HF_OK) {  // a device is present: exercise the handle's host paths too
    EXPECT(hf_absorb_evicted(st, A, A, 10, 10 * 128, 5, nullptr), HF_ERR_STATE);
    EXPECT(hf_absorb_and_attend_ahead(st, A, 10, 1280, A, A, 100, 12800, -1, 1, A, 1280, nullptr,
                                      A, A, 10, 1280, 5, nullptr), HF_ERR_STATE);
    EXPECT(hf_pending_ev(st), 0);
    EXPECT(hf_attend_chunk(st, A, 10, 1280, A, A, 100, 12800, 3, A, 1280, nullptr, nullptr),
           HF_ERR_INVALID_ARG);
    hf_state_destroy(st);
  } else {
    EXPECT(r, HF_ERR_HIP);
    EXPECT(st == nullptr, 1);
  }
  // null handles and null arguments
  EXPECT(hf_absorb_and_attend_ahead(nullptr, A, 10, 1280, A, A, 10, 1280, -1, 1, A, 1280, nullptr,
                                    A, A, 10, 1280, 0, nullptr), HF_ERR_INVALID_ARG);
  EXPECT(hf_absorb_flush(nullptr, nullptr), HF_ERR_INVALID_ARG);
  EXPECT(hf_pending_ev(nullptr), -1);
  EXPECT(hf_absorb_evicted(nullptr, A, A, 10, 1280, 0, nullptr), HF_ERR_INVALID_ARG);
  EXPECT(hf_attend_chunk(nullptr, A, 10, 1280, A, A, 10, 1280, 1, A, 1280, nullptr, nullptr),
         HF_ERR_INVALID_ARG);
  EXPECT(hf_window_attach(nullptr, A, A, 20, 10), HF_ERR_INVALID_ARG);
  void* ks; void* vs; int64_t hs;
  EXPECT(hf_window_begin_chunk(nullptr, 1, nullptr, &ks, &vs, &hs), HF_ERR_INVALID_ARG);
  int64_t f, n;
  EXPECT(hf_window_range(nullptr, &f, &n), HF_ERR_INVALID_ARG);
  double ms[HF_KERNEL_COUNT]; int32_t cnt[HF_KERNEL_COUNT];
  EXPECT(hf_profile_stop(nullptr, ms, cnt), HF_ERR_INVALID_ARG);
  EXPECT(hf_next_ev_index(nullptr), -1);
  hf_state_destroy(nullptr);
  // the allocation-free call: validation, scratch limit, then the runtime
  EXPECT(hf_attend_chunk_noalloc(&c, nullptr, (float*)A, A, 4680, 4680 * 128, A, A, 14040,
                                 14040 * 128, 55, A, 4680 * 128, nullptr, nullptr), HF_ERR_INVALID_ARG);
  EXPECT(hf_attend_chunk_noalloc(&c, (float*)A, (float*)A, A, 4 * 4680, 4 * 4680 * 128, A, A,
                                 4 * 14040, 4 * 14040 * 128, 220, A, 4 * 4680 * 128, nullptr,
                                 nullptr), HF_ERR_INVALID_ARG);
  const int rn = hf_attend_chunk_noalloc(&c, (float*)A, (float*)A, A, 4680, 4680 * 128, A, A,
                                         14040, 14040 * 128, 55, A, 4680 * 128, nullptr, nullptr);
  if (rn != HF_ERR_HIP && rn != HF_OK) return 1;
  {  // ragged windows: validation only (no handle)
    int64_t off[13] = {0};
    int32_t tk[12];
    for (int h = 0; h < 12; ++h) { off[h + 1] = off[h] + 1000; tk[h] = 4; }
    EXPECT(hf_attend_ragged(nullptr, A, 10, 1280, A, A, off, tk, A, 1280, nullptr, nullptr),
           HF_ERR_INVALID_ARG);
  }
  hf_rope rp = {44, 10000.f, 1560, 8};
  if (hf_rope_workspace_bytes(&c, &rp) == 0) return 1;
  hf_rope bad_rope = rp; bad_rope.rot_dims = 43;
  EXPECT(hf_rope_workspace_bytes(&c, &bad_rope), 0);
  EXPECT(hf_set_rope(nullptr, &rp, A, 1 << 30, nullptr), HF_ERR_INVALID_ARG);
  for (int s = 0; s <= 5; ++s) if (!hf_status_string((hf_status)s)) return 1;
  std::printf("ok\n");
  return 0;
}
"""


@pytest.fixture(scope="module")
def abi_driver(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is needed")
    d = tmp_path_factory.mktemp("abi_asan")
    (d / "stubs.cc").write_text(STUBS)
    (d / "drv.cc").write_text(ABI_DRIVER)
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    hip_inc = os.path.join(rocm, "include")
    # one compiler (ROCm's clang) and its sanitizer runtime for every host object
    cxx = os.path.join(rocm, "llvm", "bin", "clang++")
    host_san = []
    for f in SAN:  # host pass only
        host_san += ["-Xarch_host", f]
    subprocess.run([hipcc, "--offload-arch=gfx950", "-fPIC", "-std=c++17", "-O1", "-g", *host_san,
                    "-Wno-unused-command-line-argument", "-I", INC,
                    "-c", os.path.join(CSRC, "hf_abi.hip"), "-o", str(d / "abi.o")], check=True,
                   capture_output=True)
    for name in ("stubs", "drv"):
        subprocess.run([cxx, "-std=c++17", "-fPIC", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", INC,
                        "-I", CSRC, "-I", hip_inc, "-c", str(d / f"{name}.cc"), "-o",
                        str(d / f"{name}.o")], check=True)
    exe = d / "drv"
    subprocess.run([cxx, *SAN, str(d / "drv.o"), str(d / "abi.o"), str(d / "stubs.o"), "-L",
                    os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}",
                    "-o", str(exe)], check=True)
    return str(exe)


def test_abi_host_side_sanitized(abi_driver):
    out = subprocess.run([abi_driver], capture_output=True, text=True, env=ENV, timeout=300)
    assert out.returncode == 0, (out.stdout + out.stderr)[-3000:]
    assert out.stdout.strip().endswith("ok")
