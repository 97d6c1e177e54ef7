// Exercises every host-side path of the C ABI that needs no GPU, under the
// address and undefined-behaviour sanitizers: configuration checks (valid and
// invalid), workspace sizing and the schedule for every schedule kind, NULL and
// misaligned arguments of every entry point, creation failing without a device
// (its clean-up path), status strings and error messages.  Exits non-zero on a
// wrong status; the sanitizers abort on a memory or UB error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "kvm.h"

static int failures = 0;
#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);       \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static kvm_config base() {
  kvm_config c;
  std::memset(&c, 0, sizeof c);
  c.batch = 2;
  c.heads = 3;
  c.head_dim = 64;
  c.rope_dims = 32;
  c.chunk = 64;
  c.window = 128;
  c.n_sinks = 4;
  c.sched = KVM_SCHED_SQRT;
  c.alpha = 8;
  c.max_tokens = 4096;
  c.rope_theta = 10000.f;
  c.ln_eps = 1e-5f;
  c.dtype = KVM_BF16;
  c.exponent = 0.5;
  return c;
}

int main() {
  // valid configurations of every schedule, chunk and dtype: sizes and schedules
  const int chunks[] = {32, 64, 128, 256};
  for (int sched = 0; sched < 4; ++sched)
    for (int ci = 0; ci < 4; ++ci)
      for (int dt = 0; dt < 2; ++dt) {
        kvm_config c = base();
        c.sched = sched;
        c.chunk = chunks[ci];
        c.window = 2 * chunks[ci];
        c.max_slots = 300;
        c.dtype = dt;
        c.flags = (sched == 2 ? KVM_FLAG_TRACE : 0u) | (dt ? KVM_FLAG_NO_SINK_PROTECT : 0u);
        size_t bytes = 0;
        EXPECT(kvm_workspace_bytes(&c, &bytes) == KVM_OK && bytes > 0);
        const int64_t n = 40;
        std::vector<int32_t> sk(n), app(n), rows(n);
        EXPECT(kvm_schedule(&c, n, sk.data(), app.data(), rows.data()) == KVM_OK);
        for (int64_t j = 1; j < n; ++j) EXPECT(rows[j] >= rows[j - 1]);
        EXPECT(kvm_schedule(&c, n, nullptr, nullptr, nullptr) == KVM_OK);
        EXPECT(kvm_schedule(&c, -1, sk.data(), nullptr, nullptr) == KVM_E_INVALID_ARG);
      }
  // invalid configurations
  {
    kvm_config bad[16];
    for (auto& b : bad) b = base();
    bad[0].batch = 0;
    bad[1].head_dim = 128;
    bad[2].rope_dims = 16;
    bad[3].chunk = 48;
    bad[4].window = 100;
    bad[5].n_sinks = 65;
    bad[6].alpha = 0;
    bad[7].sched = 9;
    bad[8].max_tokens = 0;
    bad[9].rope_theta = -1.f;
    bad[10].ln_eps = -1.f;
    bad[11].softmax_scale = -2.f;
    bad[12].dtype = 7;
    bad[13].flags = 1u << 30;
    bad[14].sched = KVM_SCHED_POWER;
    bad[14].exponent = 2.0;
    bad[15].sched = KVM_SCHED_FIXED;
    bad[15].max_slots = 4;
    for (auto& b : bad) {
      size_t bytes = 0;
      EXPECT(kvm_workspace_bytes(&b, &bytes) == KVM_E_INVALID_ARG);
      EXPECT(std::strlen(kvm_last_error()) > 0);
    }
  }
  // NULL and misaligned arguments of every entry point
  kvm_config c = base();
  size_t bytes = 0;
  EXPECT(kvm_workspace_bytes(nullptr, &bytes) == KVM_E_INVALID_ARG);
  EXPECT(kvm_workspace_bytes(&c, nullptr) == KVM_E_INVALID_ARG);
  EXPECT(kvm_schedule(nullptr, 4, nullptr, nullptr, nullptr) == KVM_E_INVALID_ARG);
  kvm_state* st = reinterpret_cast<kvm_state*>(0x1);
  EXPECT(kvm_state_create(&c, nullptr, 1 << 20, nullptr, &st) == KVM_E_INVALID_ARG && st == nullptr);
  EXPECT(kvm_state_create(&c, reinterpret_cast<void*>(0x1000), 1 << 20, nullptr, nullptr) == KVM_E_INVALID_ARG);
  EXPECT(kvm_workspace_bytes(&c, &bytes) == KVM_OK);
  EXPECT(kvm_state_create(&c, reinterpret_cast<void*>(0x1008), bytes, nullptr, &st) == KVM_E_WORKSPACE);
  EXPECT(kvm_state_create(&c, reinterpret_cast<void*>(0x1000), bytes - 1, nullptr, &st) == KVM_E_WORKSPACE);
  // Without a GPU a valid creation fails at its first device call: the state is
  // freed and nothing is returned.  (With a GPU present the workspace address
  // below is not device memory, so the case is left out.)
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess || n_dev == 0) {
    st = reinterpret_cast<kvm_state*>(0x1);
    const kvm_status cs = kvm_state_create(&c, reinterpret_cast<void*>(0x10000), bytes, nullptr, &st);
    EXPECT(cs == KVM_E_HIP && st == nullptr);
  }
  EXPECT(kvm_prefill(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, nullptr) == KVM_E_INVALID_ARG);
  EXPECT(kvm_decode_step(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == KVM_E_INVALID_ARG);
  kvm_state_view view;
  std::memset(&view, 0, sizeof view);
  EXPECT(kvm_state_read(nullptr, -1, &view, nullptr) == KVM_E_INVALID_ARG);
  EXPECT(kvm_state_load(nullptr, &view, nullptr) == KVM_E_INVALID_ARG);
  EXPECT(kvm_snapshot_read(nullptr, 0, nullptr, nullptr, nullptr, nullptr) == KVM_E_INVALID_ARG);
  kvm_state_info info;
  EXPECT(kvm_state_get_info(nullptr, &info) == KVM_E_INVALID_ARG);
  EXPECT(kvm_state_check(nullptr, nullptr) == KVM_E_INVALID_ARG);
  EXPECT(kvm_state_reset(nullptr, nullptr) == KVM_E_INVALID_ARG);
  EXPECT(kvm_profile_enable(nullptr, 1) == KVM_E_INVALID_ARG);
  kvm_profile_times pt;
  EXPECT(kvm_profile_read(nullptr, &pt) == KVM_E_INVALID_ARG);
  EXPECT(kvm_state_destroy(nullptr) == KVM_OK);
  EXPECT(kvm_prefill_ragged(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, nullptr) ==
         KVM_E_INVALID_ARG);
  EXPECT(kvm_decode_step_ragged(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
         KVM_E_INVALID_ARG);
  EXPECT(kvm_state_reset_sequence(nullptr, 0, nullptr) == KVM_E_INVALID_ARG);
  EXPECT(kvm_state_positions(nullptr, nullptr) == KVM_E_INVALID_ARG);
  EXPECT(kvm_backward_workspace_bytes(&c, &bytes) == KVM_OK && bytes > 0);
  EXPECT(kvm_backward_workspace_bytes(nullptr, &bytes) == KVM_E_INVALID_ARG);
  EXPECT(kvm_prefill_backward(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              1, nullptr, 0, nullptr) == KVM_E_INVALID_ARG);
  // the entry point that allocates nothing: argument checks come before any device call
  alignas(16) static uint16_t buf[4][2 * 3 * 64 * 64];
  alignas(16) static float gl[2 * 3 * 64];
  kvm_config tr = base();
  tr.flags = KVM_FLAG_TRACE;
  EXPECT(kvm_prefill_noalloc(&tr, buf[0], buf[1], buf[2], gl, buf[3], 64, nullptr) == KVM_E_INVALID_ARG);
  kvm_config pw = base();
  pw.sched = KVM_SCHED_POWER;
  EXPECT(kvm_prefill_noalloc(&pw, buf[0], buf[1], buf[2], gl, buf[3], 64, nullptr) == KVM_E_INVALID_ARG);
  kvm_config big = base();
  big.batch = 64;
  big.heads = 16;
  big.max_tokens = 16384;
  EXPECT(kvm_prefill_noalloc(&big, buf[0], buf[1], buf[2], gl, buf[3], 64, nullptr) == KVM_E_WORKSPACE);
  EXPECT(kvm_prefill_noalloc(&c, nullptr, buf[1], buf[2], gl, buf[3], 64, nullptr) == KVM_E_INVALID_ARG);
  EXPECT(kvm_prefill_noalloc(&c, buf[0], buf[1], buf[2], gl, buf[0], 64, nullptr) == KVM_E_INVALID_ARG);  // aliasing
  EXPECT(kvm_prefill_noalloc(&c, buf[0], buf[1], buf[2], gl, buf[3], 5000, nullptr) == KVM_E_INVALID_ARG);
  EXPECT(kvm_prefill_noalloc(&c, buf[0], buf[1], buf[2], gl, buf[3], 0, nullptr) == KVM_OK);
  // status strings
  for (int s = 0; s <= 6; ++s) EXPECT(kvm_status_str(static_cast<kvm_status>(s)) != nullptr);
  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("sanitized host checks: ok\n");
  return 0;
}
