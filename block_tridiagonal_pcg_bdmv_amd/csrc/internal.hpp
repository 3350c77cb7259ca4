// Host-side plumbing shared by the C ABI (capi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <string>

#include "glass_amd.h"

namespace glass {

// Record a failure for glass_last_error() and return `code`.
int fail(int code, const std::string& msg);
int fail_hip(hipError_t e, const char* what);
const char* last_error_text();

struct DeviceInfo {
  int device = -1;
  int cu_count = 0;
  size_t max_lds_per_block = 0;  // bytes of LDS one workgroup may allocate
  int cooperative = 0;
};
// Properties of the current HIP device (queried once per device).
int current_device_info(DeviceInfo* out);

// Per-device caches of launch facts that do not change between calls:
// kernel_occupancy = hipOccupancyMaxActiveBlocksPerMultiprocessor for
// (kernel, block threads, dynamic LDS) on the current device;
// allow_dynamic_lds raises a kernel's dynamic-LDS limit to `bytes` (once per
// device for each larger size; sizes up to 64 KB need nothing).
int kernel_occupancy(const void* kernel, int threads, size_t lds, int* out);
int allow_dynamic_lds(const void* kernel, size_t bytes);

// Tuning and test switches (GLASS_AMD_* variables) are honoured only in a
// process that set GLASS_AMD_TUNING=1 before the library's first call;
// otherwise every switch takes its default, so a user's environment cannot
// change a placement, and no call reads the environment.
// tuning_getenv(name): getenv(name) in such a process, else nullptr.
const char* tuning_getenv(const char* name);
// Optional launch-shape override (tests and tuning sweeps): returns
// `fallback` when `name` is unset or not a positive integer.
int env_int(const char* name, int fallback);
// A 0/1 switch: "0" or "1", else `fallback`.
int env_flag(const char* name, int fallback);

// Kernel launchers.  Arguments are already validated by the C ABI.
int launch_bdmv(glass_dtype dt, void* y, const void* S, const void* v, int ss,
                int kp, int n_problems, hipStream_t stream);

int launch_pcg_batched(glass_dtype dt, void* x, const void* S,
                       const void* Pinv, const void* b, int ss, int kp,
                       int n_problems, int max_iters, double rel_tol,
                       double abs_tol, int* iters, int* status, void* rho,
                       bool pinv_diag, bool pinv_packed, hipStream_t stream);

// Several problems per wave (pcg_multi.hip): whether the shape has that
// placement, and its launcher (arguments validated by the C ABI).
bool pcg_multi_fits(glass_dtype dt, int ss, int kp);
int launch_pcg_multi(glass_dtype dt, void* x, const void* S, const void* Pinv, const void* b,
                     int ss, int kp, int n_problems, int max_iters, double rel_tol,
                     double abs_tol, int* iters, int* status, void* rho, hipStream_t stream);

// Placement glass_pcg_batched_ex would choose (GLASS_PLACEMENT_*), or an error.
// pinv_packed: Pinv given as packed D blocks (implies pinv_diag).
int pcg_batched_placement(glass_dtype dt, int ss, int kp, bool aligned16, bool pinv_diag,
                          bool pinv_packed);
// Pinv rows the S-resident placement keeps pinned in LDS (0 otherwise).
int pcg_batched_pinv_pass_rows(glass_dtype dt, int ss, int kp, bool aligned16, bool pinv_diag,
                               bool pinv_packed, int pass);
int pcg_batched_pinned_rows(glass_dtype dt, int ss, int kp, bool aligned16, bool pinv_diag,
                            bool pinv_packed);

size_t bdsv_workspace_bytes(int ss, int kp, long long n_problems, glass_dtype dt);
int launch_bdsv(glass_dtype dt, void* x, const void* S, const void* b, int ss,
                int kp, int n_problems, int* status, void* workspace,
                hipStream_t stream);

size_t grid_workspace_bytes(int ss, int kp, glass_dtype dt);
// workspace == nullptr: use the device's static scratch (no allocation).
int launch_pcg_grid(glass_dtype dt, void* x, const void* S, const void* Pinv,
                    const void* b, int ss, int kp, int max_iters,
                    double rel_tol, double abs_tol, int* iters, int* status,
                    void* rho, void* workspace, size_t workspace_bytes,
                    bool exclusive, bool single, bool keep, hipStream_t stream);

// Streaming-read probe (measurement aid); arguments validated by the C ABI.
int launch_lds_read(unsigned* sink, size_t sink_words, int rounds, int width, int* workgroups,
                    hipStream_t stream);
int launch_stream_read(const void* src, size_t nbytes, unsigned* sink, size_t sink_words,
                       hipStream_t stream);

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

}  // namespace glass
