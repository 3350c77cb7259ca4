// Calls every C-ABI entry point with invalid arguments (and the size and
// status queries with valid ones) so that an AddressSanitizer /
// UndefinedBehaviorSanitizer build of the library's host code reports any
// fault in the argument checks.  Every case returns before the device is
// touched, so no GPU is needed.  Exit status 0 = every call returned what the
// header says.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "glass_amd.h"

namespace {
int failures = 0;
void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d (%s)\n", what, got, want, glass_last_error());
    ++failures;
  }
}
void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }
}  // namespace

int main() {
  void* F = fake(0x100000);
  int* Fi = static_cast<int*>(F);
  // bdmv
  expect(glass_bdmv_batched(nullptr, F, F, 14, 64, 1, GLASS_F32, nullptr), GLASS_EINVAL, "bdmv y");
  expect(glass_bdmv_batched(F, F, fake(0x100002), 14, 64, 1, GLASS_F32, nullptr), GLASS_EINVAL,
         "bdmv misaligned");
  expect(glass_bdmv_batched(F, F, F, 0, 64, 1, GLASS_F32, nullptr), GLASS_EINVAL, "bdmv ss");
  expect(glass_bdmv_batched(F, F, F, 65, 64, 1, GLASS_F32, nullptr), GLASS_EUNSUPPORTED,
         "bdmv ss big");
  expect(glass_bdmv_batched(F, F, F, 14, 64, -1, GLASS_F32, nullptr), GLASS_EINVAL, "bdmv B");
  expect(glass_bdmv_batched(F, F, F, 14, 64, 1, (glass_dtype)7, nullptr), GLASS_EINVAL,
         "bdmv dtype");
  expect(glass_bdmv_batched(nullptr, nullptr, nullptr, 14, 64, 0, GLASS_F32, nullptr), GLASS_OK,
         "bdmv empty");
  // pcg
  expect(glass_pcg_batched(nullptr, F, F, F, 6, 32, 1, 20, 1e-6, 0, Fi, GLASS_F32, nullptr),
         GLASS_EINVAL, "pcg x");
  expect(glass_pcg_batched(F, F, F, F, 6, 32, 1, -1, 1e-6, 0, Fi, GLASS_F32, nullptr),
         GLASS_EINVAL, "pcg iters");
  expect(glass_pcg_batched(F, F, F, F, 6, 32, 1, 20, NAN, 0, Fi, GLASS_F32, nullptr),
         GLASS_EINVAL, "pcg nan tol");
  expect(glass_pcg_batched(F, F, F, F, 6, 32, 1, 20, 1e-6, INFINITY, Fi, GLASS_F32, nullptr),
         GLASS_EINVAL, "pcg inf tol");
  expect(glass_pcg_batched(F, F, F, F, 64, 200, 1, 20, 1e-6, 0, Fi, GLASS_F32, nullptr),
         GLASS_EUNSUPPORTED, "pcg rows");
  expect(glass_pcg_batched(F, F, F, F, 6, 32, 1, 20, 1e-6, 0, nullptr, GLASS_F32, nullptr),
         GLASS_EINVAL, "pcg iters_out");
  expect(glass_pcg_batched_ex(F, F, F, F, 6, 32, 1, 20, 1e-6, 0, Fi, nullptr, nullptr, GLASS_F32,
                              8u, nullptr),
         GLASS_EINVAL, "pcg flags");
  expect(glass_pcg_batched_ex(F, F, F, F, 6, 32, 1, 20, 1e-6, 0, Fi, static_cast<int*>(fake(0x100002)), nullptr,
                              GLASS_F32, 0u, nullptr),
         GLASS_EINVAL, "pcg status misaligned");
  expect(glass_pcg_batched(nullptr, nullptr, nullptr, nullptr, 6, 32, 0, 20, 1e-6, 0, nullptr,
                           GLASS_F32, nullptr),
         GLASS_OK, "pcg empty");
  expect(glass_pcg_batched_placement(0, 32, GLASS_F32, 1, 0), GLASS_EINVAL, "placement ss");
  expect(glass_pcg_batched_placement(64, 200, GLASS_F32, 1, 0), GLASS_EUNSUPPORTED,
         "placement rows");
  expect(glass_pcg_batched_pinned_rows(6, 32, GLASS_F32, 1, 4u), GLASS_EINVAL, "pinned flags");
  expect(glass_pcg_batched_pinv_pass_rows(6, 32, GLASS_F32, 1, 4u, 0), GLASS_EINVAL, "pass rows flags");
  expect(glass_pcg_batched_pinv_pass_rows(6, 32, GLASS_F32, 1, 0u, -1), GLASS_EINVAL, "pass rows pass");
  expect(glass_pcg_batched_pinv_pass_rows(6, 32, (glass_dtype)7, 1, 0u, 0), GLASS_EINVAL, "pass rows dtype");
  // grid
  const size_t ws = glass_pcg_grid_workspace_bytes(12, 8192, GLASS_F64);
  if (ws == 0) {
    std::printf("FAIL grid workspace size 0\n");
    ++failures;
  }
  expect((int)glass_pcg_grid_workspace_bytes(12, 3, GLASS_F64), 0, "grid ws small kp");
  expect(glass_pcg_grid(F, F, F, F, 12, 3, 10, 1e-10, 0, Fi, F, ws, GLASS_F64, nullptr),
         GLASS_EINVAL, "grid kp");
  expect(glass_pcg_grid(F, F, F, F, 12, 8192, 10, 1e-10, 0, Fi, nullptr, ws, GLASS_F64, nullptr),
         GLASS_EINVAL, "grid ws null");
  expect(glass_pcg_grid(F, F, F, F, 12, 8192, 10, 1e-10, 0, Fi, fake(0x100080), ws, GLASS_F64,
                        nullptr),
         GLASS_EINVAL, "grid ws align");
  expect(glass_pcg_grid(F, F, F, F, 12, 8192, 10, 1e-10, 0, Fi, F, ws - 1, GLASS_F64, nullptr),
         GLASS_EINVAL, "grid ws size");
  expect(glass_pcg_grid_ex(F, F, F, F, 12, 8192, 10, 1e-10, 0, Fi, nullptr, nullptr, F, ws,
                           GLASS_F64, 64u, nullptr),
         GLASS_EINVAL, "grid flags");
  expect(glass_pcg_grid_noalloc(F, F, F, F, 12, 8192, -2, 1e-10, 0, Fi, nullptr, nullptr,
                                GLASS_F64, 0u, nullptr),
         GLASS_EINVAL, "noalloc iters");
  expect(glass_pcg_grid_noalloc(nullptr, F, F, F, 12, 8192, 10, 1e-10, 0, Fi, nullptr, nullptr,
                                GLASS_F64, 0u, nullptr),
         GLASS_EINVAL, "noalloc x");
  // bdsv
  const size_t need = glass_bdsv_workspace_bytes(14, 32, 1, GLASS_F32);
  expect((int)glass_bdsv_workspace_bytes(25, 32, 1, GLASS_F32), 0, "bdsv ws ss");
  expect(glass_bdsv_batched(F, F, F, 14, 32, 1, nullptr, F, need - 1, GLASS_F32, nullptr),
         GLASS_EINVAL, "bdsv ws size");
  expect(glass_bdsv_batched(F, F, F, 25, 32, 1, nullptr, nullptr, 0, GLASS_F32, nullptr),
         GLASS_EUNSUPPORTED, "bdsv ss");
  expect(glass_bdsv_batched(F, nullptr, F, 14, 32, 1, nullptr, nullptr, 0, GLASS_F32, nullptr),
         GLASS_EINVAL, "bdsv S");
  // probe
  unsigned sink = 0;
  expect(glass_stream_read(F, 24, &sink, 1, nullptr), GLASS_EINVAL, "stream read size");
  expect(glass_stream_read(nullptr, 32, &sink, 1, nullptr), GLASS_EINVAL, "stream read src");
  int wg = 0;
  expect(glass_lds_read(&sink, 1, 0, 16, &wg, nullptr), GLASS_EINVAL, "lds read rounds");
  expect(glass_lds_read(&sink, 0, 4, 16, &wg, nullptr), GLASS_EINVAL, "lds read sink words");
  expect(glass_lds_read(&sink, 1, 4, 16, nullptr, nullptr), GLASS_EINVAL, "lds read wg out");
  expect(glass_lds_read(&sink, 1, 4, 12, &wg, nullptr), GLASS_EINVAL, "lds read width");
  // status text
  for (int code = -6; code <= 2; ++code)
    if (!glass_status_string(code) || std::strlen(glass_status_string(code)) == 0) ++failures;
  if (glass_version() < 300) ++failures;
  std::printf("capi sanitizer driver: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
