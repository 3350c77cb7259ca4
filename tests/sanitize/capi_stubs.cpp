// Stand-ins for the kernel launchers, so the C ABI's host code (capi.hip)
// links into a sanitizer build without the device code.  The driver only
// exercises calls that return before a launcher is reached; if one is
// reached anyway, it reports GLASS_EHIP.
#include <cstddef>

#include "glass_amd.h"
#include "hip/hip_runtime_api.h"

namespace glass {
int launch_bdmv(glass_dtype, void*, const void*, const void*, int, int, int, hipStream_t) {
  return GLASS_EHIP;
}
int launch_pcg_batched(glass_dtype, void*, const void*, const void*, const void*, int, int, int,
                       int, double, double, int*, int*, void*, bool, bool, hipStream_t) {
  return GLASS_EHIP;
}
int pcg_batched_placement(glass_dtype, int, int, bool, bool, bool) { return GLASS_EHIP; }
int pcg_batched_pinned_rows(glass_dtype, int, int, bool, bool, bool) { return GLASS_EHIP; }
int pcg_batched_pinv_pass_rows(glass_dtype, int, int, bool, bool, bool, int) { return GLASS_EHIP; }
size_t bdsv_workspace_bytes(int ss, int kp, long long n_problems, glass_dtype dt) {
  const size_t es = dt == GLASS_F32 ? 4 : 8;
  return ((size_t)n_problems * kp * ss * (ss + 1) * es + 255) / 256 * 256;
}
int launch_bdsv(glass_dtype, void*, const void*, const void*, int, int, int, int*, void*,
                hipStream_t) {
  return GLASS_EHIP;
}
size_t grid_workspace_bytes(int ss, int kp, glass_dtype dt) {
  const size_t w = dt == GLASS_F32 ? 1 : 2;
  const size_t g = (size_t)(kp / 2 < 2048 ? kp / 2 : 2048);
  return 256 + 2 * g * 2 * w * 8 + 2 * g * 4 * (size_t)ss * w * 8;
}
int launch_pcg_grid(glass_dtype, void*, const void*, const void*, const void*, int, int, int,
                    double, double, int*, int*, void*, void*, size_t, bool, bool, bool,
                    hipStream_t) {
  return GLASS_EHIP;
}
int launch_lds_read(unsigned*, size_t, int, int, int*, hipStream_t) { return GLASS_EHIP; }
int launch_stream_read(const void*, size_t, unsigned*, size_t, hipStream_t) { return GLASS_EHIP; }
}  // namespace glass
