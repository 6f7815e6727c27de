"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU needed).

The ABI source (api.hip) is rebuilt with the sanitizers on its host pass only
(each -fsanitize= follows -Xarch_host; device code is built as always) and
linked with the library's other objects and a small driver into one
executable.  The driver walks the argument-validation paths of every entry
point -- each returns before its first HIP call -- with NULL pointers,
out-of-range sizes, bad hyper-parameters and long error messages, and checks
the returned codes.  Any out-of-bounds access, use of uninitialised or freed
memory, overflow or misaligned access in those paths aborts the driver.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]

DRIVER = r'''
#include <cmath>
#include <cstdio>
#include <cstring>
#include "iqlher.h"
static int failures = 0;
#define EXPECT(call, code) do { int rc_ = (call); if (rc_ != (code)) { \
    std::printf("line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, rc_, (int)(code), iqlh_last_error()); \
    ++failures; } else if ((code) != IQLH_OK && iqlh_last_error()[0] == 0) { \
    std::printf("line %d: no error message\n", __LINE__); ++failures; } } while (0)
static iqlh_config good() {
    iqlh_config c; std::memset(&c, 0, sizeof(c));
    c.state_dim = 16; c.hidden = 32; c.max_batch = 256; c.num_groups = 1; c.compute_dtype = IQLH_F32;
    c.states_ld = 16; c.tau[0] = c.tau[1] = 0.7f; c.lr = 3e-4f; c.beta1 = 0.9f; c.beta2 = 0.999f; c.eps = 1e-8f;
    c.max_grad_norm = 1.f;
    return c;
}
int main() {
    int64_t cnt = 0;
    EXPECT(iql_num_params(16, 32, &cnt), IQLH_OK);
    if (cnt != 1633) { std::printf("param count %lld\n", (long long)cnt); ++failures; }
    EXPECT(iql_num_params(0, 4, &cnt), IQLH_EINVAL);
    EXPECT(iql_num_params(16, 32, nullptr), IQLH_EINVAL);
    iqlh_config c = good();
    c.hidden2 = 24;
    EXPECT(iql_config_num_params(&c, &cnt), IQLH_OK);
    if (cnt != 16 * 32 + 32 + 24 * 32 + 24 + 24 + 1) { std::printf("two-width count %lld\n", (long long)cnt); ++failures; }
    EXPECT(iql_config_num_params(nullptr, &cnt), IQLH_EINVAL);
    c.hidden2 = -1;
    EXPECT(iql_config_num_params(&c, &cnt), IQLH_EINVAL);
    // iql_create: every config error is caught before any allocation
    float init[4] = {0, 0, 0, 0};
    iql_handle h = nullptr;
    EXPECT(iql_create(nullptr, init, &h), IQLH_EINVAL);
    struct { int field; double value; int code; } bad[] = {
        {0, 3, IQLH_EINVAL}, {1, 0, IQLH_EINVAL}, {2, 5, IQLH_EINVAL}, {3, 7, IQLH_EINVAL}, {4, 5000, IQLH_ESHAPE},
        {5, 0.0, IQLH_EINVAL}, {6, 1.0, IQLH_EINVAL}, {7, 0.0, IQLH_EINVAL}, {8, 1.5, IQLH_EINVAL},
        {9, NAN, IQLH_EINVAL}, {10, -1, IQLH_EINVAL}, {11, 9000, IQLH_ESHAPE}};
    for (auto& b : bad) {
        c = good();
        switch (b.field) {
            case 0: c.num_groups = (int)b.value; break;
            case 1: c.max_batch = (int)b.value; break;
            case 2: c.states_ld = (int64_t)b.value; break;
            case 3: c.compute_dtype = (int)b.value; break;
            case 4: c.hidden = (int)b.value; break;
            case 5: c.max_grad_norm = (float)b.value; break;
            case 6: c.beta2 = (float)b.value; break;
            case 7: c.eps = (float)b.value; break;
            case 8: c.tau[0] = (float)b.value; break;
            case 9: c.lr = (float)b.value; break;
            case 10: c.hidden2 = (int)b.value; break;
            case 11: c.hidden2 = (int)b.value; break;
        }
        EXPECT(iql_create(&c, init, &h), b.code);
    }
    c = good();
    EXPECT(iql_create(&c, nullptr, &h), IQLH_EINVAL);
    EXPECT(iql_create(&c, init, nullptr), IQLH_EINVAL);
    // entry points on a NULL handle
    EXPECT(iql_train_step(nullptr, init, init, 1, nullptr, nullptr, nullptr, nullptr), IQLH_EINVAL);
    EXPECT(iql_train_step_aw(nullptr, init, init, 1, init, 9, 3.f, nullptr, nullptr, nullptr, nullptr, nullptr), IQLH_EINVAL);
    EXPECT(iql_compute_gradients(nullptr, init, init, 1, nullptr, nullptr), IQLH_EINVAL);
    EXPECT(iql_apply_gradients(nullptr, 1, nullptr, nullptr, nullptr), IQLH_EINVAL);
    EXPECT(iql_aux_step(nullptr, nullptr, init, init, 1, nullptr, 0, 0.f, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr), IQLH_EINVAL);
    int32_t rows = 0; int64_t floats = 0;
    EXPECT(iql_partial_layout(nullptr, 1, &rows, &floats), IQLH_EINVAL);
    EXPECT(iql_destroy(nullptr), IQLH_EINVAL);
    if (iql_step_counter(nullptr) != nullptr) { std::printf("step counter of NULL\n"); ++failures; }
    // policy
    float* p16 = (float*)16;
    EXPECT(iql_aw_policy(nullptr, nullptr, 1, 10, 9, 3.f, nullptr, nullptr), IQLH_EINVAL);
    EXPECT(iql_aw_policy(p16, p16, 1, 10, 65, 3.f, p16, nullptr), IQLH_EINVAL);
    EXPECT(iql_aw_policy(p16, p16, 0, 10, 9, 3.f, p16, nullptr), IQLH_EINVAL);
    EXPECT(iql_aw_policy(p16, p16, 1, 10, 9, INFINITY, p16, nullptr), IQLH_EINVAL);
    // HER
    her_config hc; std::memset(&hc, 0, sizeof(hc));
    hc.state_dim = 8; hc.goal_dim = 9; hc.strategy = HER_FUTURE; hc.goal_threshold = 0.01f;
    her_buffer hb; std::memset(&hb, 0, sizeof(hb)); hb.capacity = hb.buffer_size = 10;
    her_out ho; std::memset(&ho, 0, sizeof(ho)); ho.states_ld = 8;
    int32_t src[4] = {0, 1, 2, 3};
    EXPECT(her_relabel(&hc, &hb, src, 4, 1, nullptr, &ho, nullptr), IQLH_EINVAL);   // goal_dim > state_dim
    hc.goal_dim = 2; hc.strategy = 5;
    EXPECT(her_relabel(&hc, &hb, src, 4, 1, nullptr, &ho, nullptr), IQLH_EINVAL);   // unknown strategy
    hc.strategy = HER_RANDOM;
    EXPECT(her_relabel(&hc, &hb, src, -1, 1, nullptr, &ho, nullptr), IQLH_EINVAL);
    EXPECT(her_relabel(&hc, &hb, src, 0, 1, nullptr, &ho, nullptr), IQLH_OK);       // no-op
    hc.strategy = HER_FINAL;
    EXPECT(her_relabel(&hc, &hb, src, 3, 1, nullptr, &ho, nullptr), IQLH_EINVAL);   // no episode ends
    EXPECT(her_relabel(nullptr, &hb, src, 3, 1, nullptr, &ho, nullptr), IQLH_EINVAL);
    // budget (both entry points), a host array of 9 sources
    const float* srcs[9]; float fr[9];
    for (int j = 0; j < 9; ++j) { srcs[j] = p16; fr[j] = 0.1f; }
    size_t ws = 0;
    EXPECT(grad_budget_workspace_bytes(100, 9, &ws), IQLH_EINVAL);
    EXPECT(grad_budget_workspace_bytes(0, 4, &ws), IQLH_EINVAL);
    EXPECT(grad_budget_workspace_bytes(132612, 4, &ws), IQLH_OK);
    EXPECT(grad_budget_accumulate(p16, srcs, fr, fr, 9, 100, 1.f, nullptr, nullptr, p16, 4096, nullptr), IQLH_EINVAL);
    EXPECT(grad_budget_accumulate(p16, srcs, fr, fr, 4, 100, 1.f, nullptr, nullptr, p16, 4, nullptr), IQLH_EINVAL);
    EXPECT(grad_budget_accumulate(p16, srcs, fr, fr, 4, 100, -1.f, nullptr, nullptr, p16, 4096, nullptr), IQLH_EINVAL);
    srcs[2] = nullptr;
    EXPECT(grad_budget_accumulate(p16, srcs, fr, fr, 4, 100, 1.f, nullptr, nullptr, p16, 4096, nullptr), IQLH_EINVAL);
    EXPECT(grad_budget_accumulate_noalloc(p16, srcs, fr, fr, 4, 100, 1.f, nullptr, nullptr, nullptr), IQLH_EINVAL);
    srcs[2] = p16;
    EXPECT(grad_budget_accumulate_noalloc(p16, srcs, fr, fr, 9, 100, 1.f, nullptr, nullptr, nullptr), IQLH_EINVAL);
    EXPECT(grad_budget_accumulate_noalloc(p16, srcs, fr, fr, 4, 0, 1.f, nullptr, nullptr, nullptr), IQLH_EINVAL);
    iqlh_adam ad; std::memset(&ad, 0, sizeof(ad));
    EXPECT(grad_budget_accumulate_noalloc(p16, srcs, fr, fr, 4, 100, 1.f, nullptr, &ad, nullptr), IQLH_EINVAL);
    // prioritized sampling
    EXPECT(per_workspace_bytes(0, &ws), IQLH_EINVAL);
    EXPECT(per_workspace_bytes((int64_t)1 << 40, &ws), IQLH_EINVAL);
    EXPECT(per_workspace_bytes(1000, &ws), IQLH_OK);
    int32_t* i16 = (int32_t*)16;
    EXPECT(per_sample_indices(p16, 1000, 4, 1, nullptr, 0.4f, i16, p16, nullptr, p16, 8, nullptr), IQLH_EINVAL);
    EXPECT(per_sample_indices(p16, 1000, 4, 1, nullptr, -1.f, i16, p16, nullptr, p16, ws, nullptr), IQLH_EINVAL);
    EXPECT(per_sample_indices(p16, 1000, -1, 1, nullptr, 0.4f, i16, p16, nullptr, p16, ws, nullptr), IQLH_EINVAL);
    // sentinel
    const float* bufs[40]; int64_t lens[40];
    for (int s = 0; s < 40; ++s) { bufs[s] = p16; lens[s] = 4; }
    EXPECT(iqlh_nonfinite_check(bufs, lens, 0, i16, nullptr), IQLH_EINVAL);
    EXPECT(iqlh_nonfinite_check(bufs, lens, 33, i16, nullptr), IQLH_EINVAL);
    lens[3] = -1;
    EXPECT(iqlh_nonfinite_check(bufs, lens, 8, i16, nullptr), IQLH_EINVAL);
    // a message longer than the error buffer is truncated, not overrun
    EXPECT(iql_create(nullptr, init, &h), IQLH_EINVAL);
    if (std::strlen(iqlh_last_error()) >= 512) { std::printf("error text not terminated\n"); ++failures; }
    std::printf("%d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
'''


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    objs = sorted(glob.glob(os.path.join(ROOT, "offline_rl_step_amd", "_build", "*.o")))
    objs = [o for o in objs if not o.endswith("api.hip.o")]
    if len(objs) < 5:
        pytest.skip("library objects not built (python offline_rl_step_amd/build.py)")
    d = tmp_path_factory.mktemp("san")
    api_o = str(d / "api_san.o")
    r = subprocess.run([HIPCC, *FLAGS, *SAN, "-c", os.path.join(ROOT, "offline_rl_step_amd", "csrc", "api.hip"),
                        "-o", api_o], capture_output=True, text=True)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    drv = d / "driver.hip"
    drv.write_text(DRIVER)
    drv_o = str(d / "driver.o")
    subprocess.run([HIPCC, *FLAGS, *SAN, "-c", str(drv), "-o", drv_o], check=True, capture_output=True)
    exe = str(d / "driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, drv_o, api_o, *objs, "-o", exe], capture_output=True,
                       text=True)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    return exe


def test_host_validation_paths_are_clean_under_asan_and_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "0 failures" in r.stdout
