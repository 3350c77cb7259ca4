// C ABI of the library (declared in include/glass_amd.h): argument checks,
// error reporting and dispatch to the kernel launchers.  Every check runs on
// the host before anything touches the device, so invalid calls return an
// error code with nothing enqueued.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include "internal.hpp"

namespace glass {

namespace {
thread_local std::string g_last_error;

std::mutex g_dev_mutex;
std::vector<DeviceInfo> g_devices;  // indexed by device ordinal
}  // namespace

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

const char* last_error_text() { return g_last_error.c_str(); }

int fail_hip(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return GLASS_EHIP;
}

int current_device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  if ((int)g_devices.size() <= dev) g_devices.resize(dev + 1);
  DeviceInfo& d = g_devices[dev];
  if (d.device != dev) {
    DeviceInfo q;
    q.device = dev;
    int v = 0;
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return fail_hip(e, "hipDeviceGetAttribute(CU count)");
    q.cu_count = v;
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev)) != hipSuccess)
      return fail_hip(e, "hipDeviceGetAttribute(LDS per block)");
    q.max_lds_per_block = (size_t)v;
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeCooperativeLaunch, dev)) != hipSuccess)
      return fail_hip(e, "hipDeviceGetAttribute(cooperative launch)");
    q.cooperative = v;
    d = q;
  }
  *out = d;
  return GLASS_OK;
}

namespace {
std::mutex g_launch_mutex;
// (device, kernel, threads, lds) -> workgroups per CU
std::map<std::tuple<int, const void*, int, size_t>, int> g_occupancy;
// (device, kernel) -> largest dynamic LDS allowed so far
std::map<std::pair<int, const void*>, size_t> g_lds_allowed;
}  // namespace

int kernel_occupancy(const void* kernel, int threads, size_t lds, int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  const auto key = std::make_tuple(dev, kernel, threads, lds);
  {
    std::lock_guard<std::mutex> lock(g_launch_mutex);
    auto it = g_occupancy.find(key);
    if (it != g_occupancy.end()) {
      *out = it->second;
      return GLASS_OK;
    }
  }
  int v = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, threads, lds);
  if (e != hipSuccess) return fail_hip(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  std::lock_guard<std::mutex> lock(g_launch_mutex);
  g_occupancy[key] = v;
  *out = v;
  return GLASS_OK;
}

int allow_dynamic_lds(const void* kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return GLASS_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  const auto key = std::make_pair(dev, kernel);
  std::lock_guard<std::mutex> lock(g_launch_mutex);
  size_t& have = g_lds_allowed[key];
  if (have >= bytes) return GLASS_OK;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return fail_hip(e, "hipFuncSetAttribute(dynamic LDS)");
  have = bytes;
  return GLASS_OK;
}

const char* tuning_getenv(const char* name) {
  static const bool on = [] {
    const char* t = std::getenv("GLASS_AMD_TUNING");
    return t && t[0] == '1' && t[1] == '\0';
  }();
  return on ? std::getenv(name) : nullptr;
}

int env_int(const char* name, int fallback) {
  const char* s = tuning_getenv(name);
  if (!s || !*s) return fallback;
  char* end = nullptr;
  long v = std::strtol(s, &end, 10);
  if (end == s || *end != '\0' || v <= 0 || v > (1L << 30)) return fallback;
  return (int)v;
}

int env_flag(const char* name, int fallback) {
  const char* s = tuning_getenv(name);
  if (!s) return fallback;
  if (s[0] == '0' && s[1] == '\0') return 0;
  if (s[0] == '1' && s[1] == '\0') return 1;
  return fallback;
}

}  // namespace glass

using glass::fail;

namespace {

size_t elem_size(glass_dtype dt) {
  return dt == GLASS_F32 ? sizeof(float) : sizeof(double);
}

int check_common(glass_dtype dtype, int ss, int kp, long long n_problems) {
  if (dtype != GLASS_F32 && dtype != GLASS_F64) return fail(GLASS_EINVAL, "unknown dtype");
  if (ss < 1) return fail(GLASS_EINVAL, "state_size must be >= 1");
  if (ss > GLASS_MAX_STATE_SIZE) return fail(GLASS_EUNSUPPORTED, "state_size above GLASS_MAX_STATE_SIZE");
  if (kp < 1) return fail(GLASS_EINVAL, "knot_points must be >= 1");
  if (n_problems < 0) return fail(GLASS_EINVAL, "n_problems must be >= 0");
  // keep every element index of one problem inside int range
  if ((long long)kp * ss * 3 * ss > (1LL << 30)) return fail(GLASS_EUNSUPPORTED, "problem too large");
  return GLASS_OK;
}

int check_ptr(const void* p, glass_dtype dt, const char* name) {
  if (!p) return fail(GLASS_EINVAL, std::string(name) + " is NULL");
  if (!glass::aligned(p, elem_size(dt)))
    return fail(GLASS_EINVAL, std::string(name) + " is not aligned to the element size");
  return GLASS_OK;
}

int check_tols(int max_iters, double rel_tol, double abs_tol) {
  if (max_iters < 0) return fail(GLASS_EINVAL, "max_iters must be >= 0");
  if (!(rel_tol >= 0.0) || std::isinf(rel_tol)) return fail(GLASS_EINVAL, "rel_tol must be finite and >= 0");
  if (!(abs_tol >= 0.0) || std::isinf(abs_tol)) return fail(GLASS_EINVAL, "abs_tol must be finite and >= 0");
  return GLASS_OK;
}

}  // namespace

extern "C" {

int glass_bdmv_batched(void* y, const void* S, const void* v, int state_size,
                       int knot_points, int n_problems, glass_dtype dtype,
                       void* hip_stream) {
  if (int rc = check_common(dtype, state_size, knot_points, n_problems)) return rc;
  if (n_problems == 0) return GLASS_OK;  // nothing to do; pointers may be NULL
  if (int rc = check_ptr(y, dtype, "y")) return rc;
  if (int rc = check_ptr(S, dtype, "S")) return rc;
  if (int rc = check_ptr(v, dtype, "v")) return rc;
  return glass::launch_bdmv(dtype, y, S, v, state_size, knot_points, n_problems,
                            (hipStream_t)hip_stream);
}

// Flags of the batched PCG; packed diagonal blocks imply block-diagonal.
constexpr unsigned kPcgFlags = GLASS_PCG_PINV_BLOCK_DIAGONAL | GLASS_PCG_PINV_DIAGONAL_BLOCKS;
constexpr unsigned kPinvDiag = GLASS_PCG_PINV_BLOCK_DIAGONAL | GLASS_PCG_PINV_DIAGONAL_BLOCKS;

int glass_pcg_batched_ex(void* x, const void* S, const void* Pinv,
                         const void* b, int state_size, int knot_points,
                         int n_problems, int max_iters, double rel_tol,
                         double abs_tol, int* iters_out, int* status_out,
                         void* rho_out, glass_dtype dtype, unsigned flags,
                         void* hip_stream) {
  if (int rc = check_common(dtype, state_size, knot_points, n_problems)) return rc;
  if (flags & ~kPcgFlags) return fail(GLASS_EINVAL, "unknown pcg flags");
  if (int rc = check_tols(max_iters, rel_tol, abs_tol)) return rc;
  if ((long long)knot_points * state_size > 8192)
    return fail(GLASS_EUNSUPPORTED, "knot_points*state_size above 8192 (use glass_pcg_grid)");
  if (n_problems == 0) return GLASS_OK;  // nothing to do; pointers may be NULL
  if (int rc = check_ptr(x, dtype, "x")) return rc;
  if (int rc = check_ptr(S, dtype, "S")) return rc;
  if (int rc = check_ptr(Pinv, dtype, "Pinv")) return rc;
  if (int rc = check_ptr(b, dtype, "b")) return rc;
  if (!iters_out) return fail(GLASS_EINVAL, "iters_out is NULL");
  if (!glass::aligned(iters_out, 4)) return fail(GLASS_EINVAL, "iters_out misaligned");
  if (status_out && !glass::aligned(status_out, 4)) return fail(GLASS_EINVAL, "status_out misaligned");
  if (rho_out && !glass::aligned(rho_out, elem_size(dtype))) return fail(GLASS_EINVAL, "rho_out misaligned");
  return glass::launch_pcg_batched(dtype, x, S, Pinv, b, state_size, knot_points,
                                   n_problems, max_iters, rel_tol, abs_tol,
                                   iters_out, status_out, rho_out,
                                   (flags & kPinvDiag) != 0,
                                   (flags & GLASS_PCG_PINV_DIAGONAL_BLOCKS) != 0,
                                   (hipStream_t)hip_stream);
}

int glass_pcg_batched(void* x, const void* S, const void* Pinv, const void* b,
                      int state_size, int knot_points, int n_problems,
                      int max_iters, double rel_tol, double abs_tol,
                      int* iters_out, glass_dtype dtype, void* hip_stream) {
  return glass_pcg_batched_ex(x, S, Pinv, b, state_size, knot_points,
                              n_problems, max_iters, rel_tol, abs_tol,
                              iters_out, nullptr, nullptr, dtype, 0u, hip_stream);
}

int glass_pcg_batched_placement(int state_size, int knot_points,
                                glass_dtype dtype, int aligned16, unsigned flags) {
  if (int rc = check_common(dtype, state_size, knot_points, 1)) return rc;
  if (flags & ~kPcgFlags) return fail(GLASS_EINVAL, "unknown pcg flags");
  if ((long long)knot_points * state_size > 8192)
    return fail(GLASS_EUNSUPPORTED, "knot_points*state_size above 8192 (use glass_pcg_grid)");
  return glass::pcg_batched_placement(dtype, state_size, knot_points, aligned16 != 0,
                                      (flags & kPinvDiag) != 0,
                                      (flags & GLASS_PCG_PINV_DIAGONAL_BLOCKS) != 0);
}

int glass_pcg_batched_pinned_rows(int state_size, int knot_points, glass_dtype dtype,
                                  int aligned16, unsigned flags) {
  if (int rc = check_common(dtype, state_size, knot_points, 1)) return rc;
  if (flags & ~kPcgFlags) return fail(GLASS_EINVAL, "unknown pcg flags");
  if ((long long)knot_points * state_size > 8192)
    return fail(GLASS_EUNSUPPORTED, "knot_points*state_size above 8192 (use glass_pcg_grid)");
  return glass::pcg_batched_pinned_rows(dtype, state_size, knot_points, aligned16 != 0,
                                        (flags & kPinvDiag) != 0,
                                        (flags & GLASS_PCG_PINV_DIAGONAL_BLOCKS) != 0);
}

int glass_pcg_batched_pinv_pass_rows(int state_size, int knot_points, glass_dtype dtype,
                                     int aligned16, unsigned flags, int pass) {
  if (int rc = check_common(dtype, state_size, knot_points, 1)) return rc;
  if (flags & ~kPcgFlags) return fail(GLASS_EINVAL, "unknown pcg flags");
  if (pass < 0) return fail(GLASS_EINVAL, "pass must be >= 0");
  if ((long long)knot_points * state_size > 8192)
    return fail(GLASS_EUNSUPPORTED, "knot_points*state_size above 8192 (use glass_pcg_grid)");
  return glass::pcg_batched_pinv_pass_rows(dtype, state_size, knot_points, aligned16 != 0,
                                           (flags & kPinvDiag) != 0,
                                           (flags & GLASS_PCG_PINV_DIAGONAL_BLOCKS) != 0, pass);
}

size_t glass_bdsv_workspace_bytes(int state_size, int knot_points, int n_problems,
                                  glass_dtype dtype) {
  if (dtype != GLASS_F32 && dtype != GLASS_F64) return 0;
  if (state_size < 1 || state_size > GLASS_BDSV_MAX_STATE_SIZE || knot_points < 1 ||
      n_problems < 0)
    return 0;
  return glass::bdsv_workspace_bytes(state_size, knot_points, n_problems, dtype);
}

int glass_bdsv_batched(void* x, const void* S, const void* b, int state_size,
                       int knot_points, int n_problems, int* status_out,
                       void* workspace, size_t workspace_bytes,
                       glass_dtype dtype, void* hip_stream) {
  if (int rc = check_common(dtype, state_size, knot_points, n_problems)) return rc;
  if (state_size > GLASS_BDSV_MAX_STATE_SIZE)
    return fail(GLASS_EUNSUPPORTED, "bdsv: state_size above GLASS_BDSV_MAX_STATE_SIZE");
  if (n_problems == 0) return GLASS_OK;  // nothing to do; pointers may be NULL
  if (int rc = check_ptr(x, dtype, "x")) return rc;
  if (int rc = check_ptr(S, dtype, "S")) return rc;
  if (int rc = check_ptr(b, dtype, "b")) return rc;
  if (status_out && !glass::aligned(status_out, 4)) return fail(GLASS_EINVAL, "status_out misaligned");
  if (workspace) {
    if (int rc = check_ptr(workspace, dtype, "workspace")) return rc;
    if (workspace_bytes <
        glass::bdsv_workspace_bytes(state_size, knot_points, n_problems, dtype))
      return fail(GLASS_EINVAL, "workspace smaller than glass_bdsv_workspace_bytes()");
  }
  return glass::launch_bdsv(dtype, x, S, b, state_size, knot_points, n_problems,
                            status_out, workspace, (hipStream_t)hip_stream);
}

size_t glass_pcg_grid_workspace_bytes(int state_size, int knot_points,
                                      glass_dtype dtype) {
  if (dtype != GLASS_F32 && dtype != GLASS_F64) return 0;
  if (state_size < 1 || state_size > GLASS_MAX_STATE_SIZE || knot_points < 4) return 0;
  return glass::grid_workspace_bytes(state_size, knot_points, dtype);
}

}  // extern "C"

namespace {

// Argument checks shared by the grid entry points (all but the workspace).
int check_grid(void* x, const void* S, const void* Pinv, const void* b, int state_size,
               int knot_points, int max_iters, double rel_tol, double abs_tol,
               int* iters_out, int* status_out, void* rho_out, glass_dtype dtype,
               unsigned flags) {
  if (int rc = check_common(dtype, state_size, knot_points, 1)) return rc;
  if (flags & ~(unsigned)(GLASS_GRID_EXCLUSIVE | GLASS_GRID_SINGLE_REDUCTION |
                          GLASS_GRID_KEEP_WORKSPACE))
    return fail(GLASS_EINVAL, "unknown grid flags");
  if (knot_points < 4) return fail(GLASS_EINVAL, "grid pcg needs knot_points >= 4");
  if (int rc = check_ptr(x, dtype, "x")) return rc;
  if (int rc = check_ptr(S, dtype, "S")) return rc;
  if (int rc = check_ptr(Pinv, dtype, "Pinv")) return rc;
  if (int rc = check_ptr(b, dtype, "b")) return rc;
  if (!iters_out) return fail(GLASS_EINVAL, "iters_out is NULL");
  if (!glass::aligned(iters_out, 4)) return fail(GLASS_EINVAL, "iters_out misaligned");
  if (status_out && !glass::aligned(status_out, 4)) return fail(GLASS_EINVAL, "status_out misaligned");
  if (rho_out && !glass::aligned(rho_out, elem_size(dtype))) return fail(GLASS_EINVAL, "rho_out misaligned");
  return check_tols(max_iters, rel_tol, abs_tol);
}

}  // namespace

extern "C" {

int glass_pcg_grid_ex(void* x, const void* S, const void* Pinv, const void* b,
                      int state_size, int knot_points, int max_iters,
                      double rel_tol, double abs_tol, int* iters_out,
                      int* status_out, void* rho_out, void* workspace,
                      size_t workspace_bytes, glass_dtype dtype,
                      unsigned flags, void* hip_stream) {
  if (int rc = check_grid(x, S, Pinv, b, state_size, knot_points, max_iters, rel_tol, abs_tol,
                          iters_out, status_out, rho_out, dtype, flags))
    return rc;
  if (!workspace) return fail(GLASS_EINVAL, "workspace is NULL");
  if (!glass::aligned(workspace, 256)) return fail(GLASS_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < glass::grid_workspace_bytes(state_size, knot_points, dtype))
    return fail(GLASS_EINVAL, "workspace smaller than glass_pcg_grid_workspace_bytes()");
  return glass::launch_pcg_grid(dtype, x, S, Pinv, b, state_size, knot_points,
                                max_iters, rel_tol, abs_tol, iters_out,
                                status_out, rho_out, workspace, workspace_bytes,
                                (flags & GLASS_GRID_EXCLUSIVE) != 0,
                                (flags & GLASS_GRID_SINGLE_REDUCTION) != 0,
                                (flags & GLASS_GRID_KEEP_WORKSPACE) != 0,
                                (hipStream_t)hip_stream);
}

int glass_pcg_grid_noalloc(void* x, const void* S, const void* Pinv, const void* b,
                           int state_size, int knot_points, int max_iters,
                           double rel_tol, double abs_tol, int* iters_out,
                           int* status_out, void* rho_out, glass_dtype dtype,
                           unsigned flags, void* hip_stream) {
  if (int rc = check_grid(x, S, Pinv, b, state_size, knot_points, max_iters, rel_tol, abs_tol,
                          iters_out, status_out, rho_out, dtype, flags))
    return rc;
  return glass::launch_pcg_grid(dtype, x, S, Pinv, b, state_size, knot_points,
                                max_iters, rel_tol, abs_tol, iters_out,
                                status_out, rho_out, nullptr, 0,
                                (flags & GLASS_GRID_EXCLUSIVE) != 0,
                                (flags & GLASS_GRID_SINGLE_REDUCTION) != 0,
                                (flags & GLASS_GRID_KEEP_WORKSPACE) != 0,
                                (hipStream_t)hip_stream);
}

int glass_pcg_grid(void* x, const void* S, const void* Pinv, const void* b,
                   int state_size, int knot_points, int max_iters,
                   double rel_tol, double abs_tol, int* iters_out,
                   void* workspace, size_t workspace_bytes, glass_dtype dtype,
                   void* hip_stream) {
  return glass_pcg_grid_ex(x, S, Pinv, b, state_size, knot_points, max_iters,
                           rel_tol, abs_tol, iters_out, nullptr, nullptr,
                           workspace, workspace_bytes, dtype, 0u, hip_stream);
}

int glass_stream_read(const void* src, size_t nbytes, unsigned* sink, size_t sink_words,
                      void* hip_stream) {
  if (!src || !sink) return fail(GLASS_EINVAL, "stream read: NULL pointer");
  if (!glass::aligned(src, 16) || nbytes % 16 != 0 || nbytes == 0)
    return fail(GLASS_EINVAL, "stream read: src must be 16-byte aligned, nbytes a positive multiple of 16");
  if (!glass::aligned(sink, 4) || sink_words == 0)
    return fail(GLASS_EINVAL, "stream read: sink must be 4-byte aligned with at least one word");
  return glass::launch_stream_read(src, nbytes, sink, sink_words, (hipStream_t)hip_stream);
}

int glass_lds_read(unsigned* sink, size_t sink_words, int rounds, int bytes_per_load,
                   int* workgroups_out, void* hip_stream) {
  if (!sink || !workgroups_out) return fail(GLASS_EINVAL, "LDS read: NULL pointer");
  if (!glass::aligned(sink, 4) || sink_words == 0)
    return fail(GLASS_EINVAL, "LDS read: sink must be 4-byte aligned with at least one word");
  if (rounds < 1 || rounds > (1 << 20)) return fail(GLASS_EINVAL, "LDS read: rounds must be 1 .. 2^20");
  if (bytes_per_load != 4 && bytes_per_load != 8 && bytes_per_load != 16)
    return fail(GLASS_EINVAL, "LDS read: bytes_per_load must be 4, 8 or 16");
  return glass::launch_lds_read(sink, sink_words, rounds, bytes_per_load, workgroups_out,
                                (hipStream_t)hip_stream);
}

const char* glass_status_string(int status) {
  switch (status) {
    case GLASS_OK: return "ok";
    case GLASS_EINVAL: return "invalid argument";
    case GLASS_EUNSUPPORTED: return "unsupported size";
    case GLASS_EHIP: return "HIP runtime error";
    case GLASS_ECOOP: return "cooperative grid cannot be co-resident";
    default: return "unknown status";
  }
}

const char* glass_last_error(void) { return glass::last_error_text(); }

int glass_version(void) { return 500; }

}  // extern "C"
