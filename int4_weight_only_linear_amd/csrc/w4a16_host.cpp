// Host side of libw4a16: the C ABI declared in include/w4a16.h -- argument
// validation, packing, a per-device property cache, path selection, and the
// launch of the kernels on the caller's stream.
//
// Validation follows the accept set the pages describe for the kernel's
// `can_implement` (quantisation type, activation dtype, group size and K
// divisibility; "Upstream sync 67/N: merge 382bbd5144 HybridW4A16LinearKernel
// (conflict)", reviewer's item 2), and the zero-point contract of the same
// page's section "Upstream's Python side is kept -- and it does NOT work here".
#include "w4a16.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>

#include "w4a16_internal.h"

namespace w4a16 {

namespace {

Tuning read_tuning() {
  Tuning t{};
  t.m_threshold = -1;
  if (const char* e = std::getenv("W4A16_FORCE_PATH")) {
    if (std::strcmp(e, "gemv") == 0) t.force_path = W4A16_PATH_GEMV;
    if (std::strcmp(e, "gemm") == 0) t.force_path = W4A16_PATH_GEMM;
  }
  if (const char* e = std::getenv("W4A16_M_THRESHOLD")) {
    char* end = nullptr;
    const long v = std::strtol(e, &end, 10);
    if (end != e && v >= 0 && v <= W4A16_GEMV_MAX_M) t.m_threshold = (int)v;
  }
  if (const char* e = std::getenv("W4A16_GEMM_TILE")) {
    const int n = std::sscanf(e, "%d,%d,%d,%d", &t.gemm_tile[0], &t.gemm_tile[1], &t.gemm_tile[2],
                              &t.gemm_tile[3]);
    t.gemm_tile_n = n > 0 ? n : 0;
  }
  if (const char* e = std::getenv("W4A16_GEMV_KPW")) t.gemv_kpw = std::atoi(e);
  if (const char* e = std::getenv("W4A16_GEMV_SPLITS")) t.gemv_splits = std::atoi(e);
  t.gemv_no_wgsz = std::getenv("W4A16_GEMV_NO_WGSZ") != nullptr;
  t.gemv_no_one = std::getenv("W4A16_GEMV_NO_ONE") != nullptr;
  if (const char* e = std::getenv("W4A16_LOG")) t.log = *e && std::strcmp(e, "0") != 0;
  return t;
}

// The current settings.  A reload publishes a new copy and keeps the old one
// (a few dozen bytes per reload), so a reader that still holds it stays valid.
std::atomic<const Tuning*> g_tuning{nullptr};
std::mutex g_tuning_mutex;

}  // namespace

const Tuning& tuning() {
  const Tuning* t = g_tuning.load(std::memory_order_acquire);
  if (t) return *t;
  std::lock_guard<std::mutex> lock(g_tuning_mutex);
  t = g_tuning.load(std::memory_order_acquire);
  if (!t) {
    t = new Tuning(read_tuning());
    g_tuning.store(t, std::memory_order_release);
  }
  return *t;
}

void reload_tuning() {
  std::lock_guard<std::mutex> lock(g_tuning_mutex);
  g_tuning.store(new Tuning(read_tuning()), std::memory_order_release);
}

}  // namespace w4a16

namespace {

thread_local std::string g_last_error;

w4a16_status fail(w4a16_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

w4a16_status ok() {
  g_last_error.clear();
  return W4A16_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [a, a + na) and [b, b + nb) overlap
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// ---- per-device properties, filled once per device ------------------------
struct DeviceInfo {
  bool ready = false;
  hipError_t err = hipSuccess;
  bool gfx950 = false;
  int cu_count = 0;
  char arch[64] = {0};
  // this device's copy of `scratch` (w4a16_linear_noalloc), set up on the
  // entry point's first call on the device
  bool scratch_ready = false;
  void* scratch_ptr = nullptr;
};

constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_device_mutex;

w4a16_status device_info(const DeviceInfo** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(W4A16_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(W4A16_ERR_DEVICE, "device ordinal %d out of range", dev);
  DeviceInfo& d = g_devices[dev];
  {
    std::lock_guard<std::mutex> lock(g_device_mutex);
    if (!d.ready) {
      hipDeviceProp_t prop;
      d.err = hipGetDeviceProperties(&prop, dev);
      if (d.err == hipSuccess) {
        std::snprintf(d.arch, sizeof(d.arch), "%s", prop.gcnArchName);
        d.cu_count = prop.multiProcessorCount;
        d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                   (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
      }
      d.ready = true;
    }
  }
  if (d.err != hipSuccess)
    return fail(W4A16_ERR_DEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(d.err));
  if (!d.gfx950)
    return fail(W4A16_ERR_UNSUPPORTED, "libw4a16 supports gfx950 only; this device is %s", d.arch);
  *out = &d;
  return W4A16_OK;
}

// ---- scratch of the allocation-free entry point ----------------------------
// w4a16_linear_noalloc takes its split-K workspace (completion counters, then
// fp32 partial sums) from this array instead of from the caller.  Every GPU
// the library runs on holds its own copy, from module load until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// copy: the address a kernel needs comes from hipGetSymbolAddress, taken once
// per device with that device current (DeviceInfo::scratch_ptr).
constexpr size_t kScratchBytes = W4A16_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;

// This device's scratch address; on the first call on the device the
// counter region is cleared by a kernel on `stream` (stream-ordered before
// the launch that follows).
w4a16_status scratch_for(DeviceInfo& d, int dev, hipStream_t stream, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!d.scratch_ready) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != dev)
      return fail(W4A16_ERR_DEVICE, "noalloc: device %d is not current", dev);
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(W4A16_ERR_DEVICE, "noalloc: hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    const hipError_t z = w4a16::launch_zero_words(ptr, w4a16::kCounterBytes, stream);
    if (z != hipSuccess)
      return fail(W4A16_ERR_LAUNCH, "noalloc: clearing the scratch counters failed: %s", hipGetErrorString(z));
    d.scratch_ptr = ptr;
    d.scratch_ready = true;
  }
  *out = d.scratch_ptr;
  return W4A16_OK;
}

size_t act_bytes(int64_t n) { return (size_t)n * 2; }

bool valid_group(int32_t g) { return g == 32 || g == 64 || g == 128; }

// Group sizes: the pages' accept set {32, 64, 128}, and per-channel scales
// (group_size == K, one scale and zero point per row) for K a multiple of 32.
bool group_ok(int32_t g, int64_t K) { return valid_group(g) || (g == K && K % 32 == 0); }

// The kernels' group for a group size: itself, or for per-channel scales the
// largest of 128, 64, 32 dividing K, every group of a row then reading the
// row's one scale (gmul = 0, row stride sG = 1).
struct GroupMap {
  int kgroup, sG, gmul;
};
GroupMap group_map(int32_t g, int64_t K) {
  if (valid_group(g)) return {g, (int)(K / g), 1};
  const int kg = K % 128 == 0 ? 128 : (K % 64 == 0 ? 64 : 32);
  return {kg, 1, 0};
}

// Decode-kernel threshold.  The pages route M <= 5 to their skinny kernel
// (tuned on RDNA).  Measured on MI355X (both kernels timed per launch over
// graphs rotating >= 1 GiB of weights; groups 32/64/128, symmetric and
// asymmetric, fp16 and bf16): the decode kernel is faster at every M <= 8
// (at K = 28672 within 1-3 % of the GEMM at M = 8).  Above that it takes one
// k-step per wave and the GEMM (32-token tiles up to M = 32) overtakes it by
// layer size:
//   K = 28672, and K = 14336 / 9728 from 32 M weights (14336 x 4096): the
//                           GEMM from M = 9 (-11 % there at M = 9-12);
//   K = 9728 x 2560:        decode through M = 12, the GEMM from 14;
//   K <= 4096, N >= 14336:  the GEMM from M = 9 at every group;
//   K <= 4096, 4096 x 6144: decode at M = 9, the GEMM 13-16 % faster at
//                           M = 10-14, a tie at 16;
//   K <= 4096, smaller (4096 x 4096, 4096 x 2560, 2560 x 6144): decode
//                           through M = 16.
int64_t gemv_threshold(int64_t N, int64_t K, int32_t group, int32_t dtype, int32_t has_zp) {
  (void)dtype; (void)has_zp;
  const int v = w4a16::tuning().m_threshold;
  if (v >= 0 && v <= W4A16_GEMV_MAX_M) return v;
  const int64_t weights = N * K;
  // K > 16384: from 160 Mi weights on, with groups of 64 or more, the GEMM's
  // 32-token tiles win from M = 7 (28672 x 8192: -7 to -26 % at M = 7 / 8)
  if (K > 16384) return weights >= (int64_t(160) << 20) && group >= 64 ? 6 : 8;
  if (K > 4096) return weights >= (int64_t(32) << 20) ? 8 : 12;
  if (N >= 14336) return 8;
  return weights >= (int64_t(20) << 20) ? 9 : 16;
}

w4a16_path resolve_path(int64_t M, int64_t N, int64_t K, int32_t group, int32_t dtype,
                        int32_t has_zp, int32_t path) {
  if (path == W4A16_PATH_GEMV || path == W4A16_PATH_GEMM) return (w4a16_path)path;
  const int forced = w4a16::tuning().force_path;
  if (forced == W4A16_PATH_GEMV || forced == W4A16_PATH_GEMM) return (w4a16_path)forced;
  return M <= gemv_threshold(N, K, group, dtype, has_zp) ? W4A16_PATH_GEMV : W4A16_PATH_GEMM;
}

constexpr int kPlanningCUs = 256;  // MI355X; the launch plan uses the device's own count

size_t workspace_for(int64_t M, int64_t N, int64_t K, int32_t group, int32_t dtype, bool asym,
                     w4a16_path path, int cu_count) {
  if (M <= 0) return 0;
  if (path == W4A16_PATH_GEMV) {
    const w4a16::GemvPlan plan = w4a16::plan_gemv(M, N, K, group, dtype, cu_count);
    return w4a16::gemv_workspace_bytes(plan, M, N);
  }
  return w4a16::gemm_workspace_bytes(M, N, K, group, dtype, asym, cu_count);
}

bool log_enabled() { return w4a16::tuning().log; }

w4a16_status linear_impl(const void* x, const int32_t* wq, const void* scales, const int32_t* zp,
                         const void* bias, void* y, int64_t M, int64_t N, int64_t K,
                         int32_t group_size, int32_t dtype, void* workspace,
                         size_t workspace_bytes, void* stream, int32_t path) {
  w4a16_status st = w4a16_check_args(x, wq, scales, zp, bias, y, M, N, K, group_size, dtype);
  if (st != W4A16_OK) return st;
  const GroupMap gm = group_map(group_size, K);
  group_size = gm.kgroup;  // from here on, the kernels' group
  if (path < W4A16_PATH_AUTO || path > W4A16_PATH_GEMM)
    return fail(W4A16_ERR_INVALID_ARG, "unknown path %d", (int)path);
  if (M == 0) return ok();
  const DeviceInfo* dev = nullptr;
  st = device_info(&dev);
  if (st != W4A16_OK) return st;
  const w4a16_path p = resolve_path(M, N, K, group_size, dtype, zp != nullptr, path);
  if (p == W4A16_PATH_GEMV && M > W4A16_GEMV_MAX_M)
    return fail(W4A16_ERR_UNSUPPORTED, "the decode kernel takes M <= %d, got M=%lld",
                W4A16_GEMV_MAX_M, (long long)M);
  if (p == W4A16_PATH_GEMV && (uint64_t)N * (uint64_t)K / 2 > 0xFFFFFFFFull)
    return fail(W4A16_ERR_UNSUPPORTED,
                "the decode kernel addresses weights with 32-bit byte offsets: N*K/2 must be "
                "below 4 GiB (N=%lld K=%lld)", (long long)N, (long long)K);
  if (p == W4A16_PATH_GEMM && ((uint64_t)N * (uint64_t)K / 2 > 0xFFFFFFFFull ||
                               (uint64_t)M * (uint64_t)K * 2 > 0xFFFFFFFFull))
    return fail(W4A16_ERR_UNSUPPORTED,
                "the prefill kernel addresses weights and activations with 32-bit byte "
                "offsets: N*K/2 and M*K*2 must be below 4 GiB (M=%lld N=%lld K=%lld)",
                (long long)M, (long long)N, (long long)K);
  const size_t need = workspace_for(M, N, K, group_size, dtype, zp != nullptr, p, dev->cu_count);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(W4A16_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu%s", need,
                workspace_bytes, workspace ? "" : " (NULL)");
  if (need > 0 && !aligned(workspace, 256))
    return fail(W4A16_ERR_ALIGNMENT, "workspace must be 256-byte aligned");

  w4a16::LinearArgs a{x, wq, scales, zp, bias, y, M, N, K, group_size, dtype, gm.sG, gm.gmul};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (p == W4A16_PATH_GEMV) {
    const w4a16::GemvPlan plan = w4a16::plan_gemv(M, N, K, group_size, dtype, dev->cu_count);
    if (log_enabled())
      std::fprintf(stderr,
                   "[w4a16] gemv M=%lld N=%lld K=%lld g=%d %s %s tiles=%d splits=%d waves=%d\n",
                   (long long)M, (long long)N, (long long)K, group_size,
                   dtype == W4A16_F16 ? "f16" : "bf16", zp ? "asym" : "sym", plan.tiles,
                   plan.splits, plan.waves);
    e = w4a16::launch_gemv(a, plan, workspace, s);
  } else {
    if (log_enabled()) {
      const w4a16::GemmPlan plan = w4a16::plan_gemm(M, N, K, group_size, dtype, zp != nullptr, dev->cu_count);
      std::fprintf(stderr,
                   "[w4a16] gemm M=%lld N=%lld K=%lld g=%d %s %s bm=%d bn=%d splits=%d units=%d\n",
                   (long long)M, (long long)N, (long long)K, group_size,
                   dtype == W4A16_F16 ? "f16" : "bf16", zp ? "asym" : "sym", 32 * plan.mb,
                   128 * plan.cb, plan.splits, plan.units);
    }
    e = w4a16::launch_gemm(a, workspace, dev->cu_count, s);
  }
  if (e != hipSuccess) return fail(W4A16_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

void w4a16_reload_tuning(void) { w4a16::reload_tuning(); }

const char* w4a16_last_error(void) { return g_last_error.c_str(); }

// nibble t of a word holds k-offset (0,2,4,6,1,3,5,7)[t]; the inverse map:
static const int kSlotOfKoff[8] = {0, 4, 1, 5, 2, 6, 3, 7};

// The 8-k slice held by stored word j of a row of J words: complete runs of
// 16 words are stored as the 4x4 transpose (word 4r+t <-> slice 4t+r, its own
// inverse); an incomplete last run is stored in order.
static int64_t slice_of_stored_word(int64_t j, int64_t J) {
  const int64_t run = j / 16, p = j % 16;
  if ((run + 1) * 16 > J) return j;
  return run * 16 + 4 * (p % 4) + p / 4;
}

// Where stored word j of row n sits in the packed tensor.  Rows are grouped
// in tiles of 16; a complete tile holds, for each complete run, one block of
// 256 words whose 16-byte piece 16 r + (n mod 16) is the row's run words
// 4r..4r+3, then the 16 rows' incomplete runs row after row.  The rows of a
// final incomplete tile are stored one after another.
static int64_t stored_position(int64_t n, int64_t j, int64_t N, int64_t J) {
  const int64_t tile = n / 16, row = n % 16;
  if ((tile + 1) * 16 > N) return n * J + j;
  const int64_t runs = J / 16, tail = J - 16 * runs;
  const int64_t base = tile * 16 * J;
  if (j < 16 * runs) {
    const int64_t run = j / 16, p = j % 16;
    return base + 256 * run + 4 * (16 * (p / 4) + row) + p % 4;
  }
  return base + 256 * runs + tail * row + (j - 16 * runs);
}

w4a16_status w4a16_pack_weights(const uint8_t* q, int64_t N, int64_t K, int32_t* wq) {
  if (!q || !wq) return fail(W4A16_ERR_INVALID_ARG, "pack_weights: NULL pointer");
  if (N < 0 || K < 0 || K % 8) return fail(W4A16_ERR_INVALID_ARG, "pack_weights: need N >= 0, K >= 0, K %% 8 == 0 (N=%lld K=%lld)", (long long)N, (long long)K);
  for (int64_t i = 0; i < N * K; ++i)
    if (q[i] > 15) return fail(W4A16_ERR_INVALID_ARG, "pack_weights: code %u at %lld exceeds 15", (unsigned)q[i], (long long)i);
  const int64_t J = K / 8;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < J; ++j) {
      const uint8_t* src = q + n * K + slice_of_stored_word(j, J) * 8;
      uint32_t w = 0;
      for (int i = 0; i < 8; ++i) w |= (uint32_t)src[i] << (4 * kSlotOfKoff[i]);
      wq[stored_position(n, j, N, J)] = (int32_t)w;
    }
  return ok();
}

w4a16_status w4a16_unpack_weights(const int32_t* wq, int64_t N, int64_t K, uint8_t* q) {
  if (!q || !wq) return fail(W4A16_ERR_INVALID_ARG, "unpack_weights: NULL pointer");
  if (N < 0 || K < 0 || K % 8) return fail(W4A16_ERR_INVALID_ARG, "unpack_weights: need N >= 0, K >= 0, K %% 8 == 0");
  const int64_t J = K / 8;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < J; ++j) {
      const uint32_t w = (uint32_t)wq[stored_position(n, j, N, J)];
      uint8_t* dst = q + n * K + slice_of_stored_word(j, J) * 8;
      for (int i = 0; i < 8; ++i) dst[i] = (uint8_t)((w >> (4 * kSlotOfKoff[i])) & 0xFu);
    }
  return ok();
}

w4a16_status w4a16_pack_zeros(const uint8_t* z, int64_t N, int64_t G, int32_t* zpk) {
  if (!z || !zpk) return fail(W4A16_ERR_INVALID_ARG, "pack_zeros: NULL pointer");
  if (N < 0 || G < 0 || N % 8) return fail(W4A16_ERR_INVALID_ARG, "pack_zeros: need N >= 0, G >= 0, N %% 8 == 0 (N=%lld)", (long long)N);
  for (int64_t i = 0; i < N * G; ++i)
    if (z[i] > 15) return fail(W4A16_ERR_INVALID_ARG, "pack_zeros: zero point %u at %lld exceeds 15", (unsigned)z[i], (long long)i);
  for (int64_t r = 0; r < N / 8; ++r)
    for (int64_t g = 0; g < G; ++g) {
      uint32_t w = 0;
      for (int i = 0; i < 8; ++i) w |= (uint32_t)z[(r * 8 + i) * G + g] << (4 * i);
      zpk[r * G + g] = (int32_t)w;
    }
  return ok();
}

w4a16_status w4a16_unpack_zeros(const int32_t* zpk, int64_t N, int64_t G, uint8_t* z) {
  if (!z || !zpk) return fail(W4A16_ERR_INVALID_ARG, "unpack_zeros: NULL pointer");
  if (N < 0 || G < 0 || N % 8) return fail(W4A16_ERR_INVALID_ARG, "unpack_zeros: need N >= 0, G >= 0, N %% 8 == 0");
  for (int64_t r = 0; r < N / 8; ++r)
    for (int64_t g = 0; g < G; ++g) {
      const uint32_t w = (uint32_t)zpk[r * G + g];
      for (int i = 0; i < 8; ++i) z[(r * 8 + i) * G + g] = (uint8_t)((w >> (4 * i)) & 0xFu);
    }
  return ok();
}

w4a16_status w4a16_check_args(const void* x, const int32_t* wq, const void* scales,
                              const int32_t* zp, const void* bias, const void* y, int64_t M,
                              int64_t N, int64_t K, int32_t group_size, int32_t dtype) {
  if (dtype != W4A16_F16 && dtype != W4A16_BF16)
    return fail(W4A16_ERR_INVALID_ARG, "activation dtype must be fp16 (0) or bf16 (1), got %d", (int)dtype);
  if (!group_ok(group_size, K))
    return fail(W4A16_ERR_UNSUPPORTED,
                "group size must be 32, 64, 128 or K (per-channel, K %% 32 == 0), got %d (K=%lld)",
                (int)group_size, (long long)K);
  if (M < 0) return fail(W4A16_ERR_INVALID_ARG, "M must be >= 0, got %lld", (long long)M);
  if (N < 1) return fail(W4A16_ERR_INVALID_ARG, "N must be >= 1, got %lld", (long long)N);
  if (K < group_size || K % group_size)
    return fail(W4A16_ERR_INVALID_ARG, "K must be a positive multiple of the group size %d, got K=%lld",
                (int)group_size, (long long)K);
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || M * K > INT64_MAX / 2 || N * K > INT64_MAX / 2)
    return fail(W4A16_ERR_INVALID_ARG, "problem too large");
  if (K > w4a16::kMaxK)
    return fail(W4A16_ERR_UNSUPPORTED, "K above %lld is not supported (the kernels' 32-bit offsets), got K=%lld",
                (long long)w4a16::kMaxK, (long long)K);
  if (zp && N % 8)
    return fail(W4A16_ERR_INVALID_ARG, "packed zero points need N %% 8 == 0, got N=%lld", (long long)N);
  if (M == 0) return ok();
  if (!x || !wq || !scales || !y) return fail(W4A16_ERR_INVALID_ARG, "x, wq, scales and y must not be NULL");
  if (!aligned(x, 16)) return fail(W4A16_ERR_ALIGNMENT, "x must be 16-byte aligned");
  if (!aligned(wq, 16)) return fail(W4A16_ERR_ALIGNMENT, "wq must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(y, 2) || (bias && !aligned(bias, 2)))
    return fail(W4A16_ERR_ALIGNMENT, "scales, bias and y must be 2-byte aligned");
  if (zp && !aligned(zp, 4)) return fail(W4A16_ERR_ALIGNMENT, "zp must be 4-byte aligned");
  const int64_t G = K / group_size;
  const size_t ybytes = act_bytes(M * N);
  if (overlap(y, ybytes, x, act_bytes(M * K)) || overlap(y, ybytes, wq, (size_t)N * (K / 8) * 4) ||
      overlap(y, ybytes, scales, act_bytes(N * G)) ||
      (zp && overlap(y, ybytes, zp, (size_t)(N / 8) * G * 4)) ||
      (bias && overlap(y, ybytes, bias, act_bytes(N))))
    return fail(W4A16_ERR_INVALID_ARG, "y must not overlap any input");
  return ok();
}

w4a16_path w4a16_select_path(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t dtype,
                             int32_t has_zp) {
  return resolve_path(M, N, K, group_size, dtype, has_zp, W4A16_PATH_AUTO);
}

size_t w4a16_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t dtype,
                            int32_t has_zp, int32_t path) {
  if (M <= 0 || N <= 0 || K <= 0 || !group_ok(group_size, K) || K % group_size) return 0;
  const int kgroup = group_map(group_size, K).kgroup;
  const w4a16_path p = resolve_path(M, N, K, kgroup, dtype, has_zp, path);
  int cus = kPlanningCUs;
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
    const DeviceInfo* d = nullptr;
    if (device_info(&d) == W4A16_OK) cus = d->cu_count;
    g_last_error.clear();
  }
  return workspace_for(M, N, K, kgroup, dtype, has_zp != 0, p, cus);
}

w4a16_status w4a16_plan(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t dtype,
                        int32_t has_zp, int32_t path, w4a16_plan_info* out) {
  if (!out) return fail(W4A16_ERR_INVALID_ARG, "plan: out must not be NULL");
  if (dtype != W4A16_F16 && dtype != W4A16_BF16)
    return fail(W4A16_ERR_INVALID_ARG, "activation dtype must be fp16 (0) or bf16 (1), got %d", (int)dtype);
  if (!group_ok(group_size, K))
    return fail(W4A16_ERR_UNSUPPORTED,
                "group size must be 32, 64, 128 or K (per-channel, K %% 32 == 0), got %d (K=%lld)",
                (int)group_size, (long long)K);
  if (M < 1 || N < 1 || K < group_size || K % group_size || M > INT32_MAX || N > INT32_MAX)
    return fail(W4A16_ERR_INVALID_ARG, "plan: need M >= 1, N >= 1 and K a positive multiple of the group");
  if (K > w4a16::kMaxK)
    return fail(W4A16_ERR_UNSUPPORTED, "K above %lld is not supported", (long long)w4a16::kMaxK);
  if (has_zp && N % 8)
    return fail(W4A16_ERR_INVALID_ARG, "packed zero points need N %% 8 == 0, got N=%lld", (long long)N);
  if (path < W4A16_PATH_AUTO || path > W4A16_PATH_GEMM)
    return fail(W4A16_ERR_INVALID_ARG, "unknown path %d", (int)path);
  const GroupMap gm = group_map(group_size, K);
  const w4a16_path p = resolve_path(M, N, K, gm.kgroup, dtype, has_zp, path);
  if (p == W4A16_PATH_GEMV && M > W4A16_GEMV_MAX_M)
    return fail(W4A16_ERR_UNSUPPORTED, "the decode kernel takes M <= %d, got M=%lld",
                W4A16_GEMV_MAX_M, (long long)M);
  int cus = kPlanningCUs;
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
    const DeviceInfo* d = nullptr;
    if (device_info(&d) == W4A16_OK) cus = d->cu_count;
  }
  w4a16_plan_info r{};
  r.path = p;
  if (p == W4A16_PATH_GEMV) {
    const w4a16::GemvPlan g = w4a16::plan_gemv(M, N, K, gm.kgroup, dtype, cus);
    r.tile_features = w4a16::kGemvRowsPerTile;
    r.tile_tokens = w4a16::kGemvMaxM;
    r.tiles = g.tiles;
    if (g.one_kpw && gm.gmul == 1) {
      // the single-token instance (given 16-byte aligned scales and zero points)
      r.kernel = 1;
      r.splits = g.one_splits;
      r.waves = g.one_waves;
      r.launches = 1;
      r.counter_tiles = g.one_splits > 1 ? g.tiles : 0;
    } else {
      r.splits = g.splits;
      r.waves = g.waves;
      r.launches = g.splits > 1 ? (int32_t)((g.tiles + w4a16::kMaxCounters - 1) / w4a16::kMaxCounters) : 1;
      r.counter_tiles = g.splits > 1 ? std::min<int64_t>(g.tiles, w4a16::kMaxCounters) : 0;
    }
  } else {
    const w4a16::GemmPlan g = w4a16::plan_gemm(M, N, K, gm.kgroup, dtype, has_zp != 0, cus);
    r.tile_features = 128 * g.cb;
    r.tile_tokens = 32 * g.mb;
    r.splits = g.splits;
    r.tiles = g.tiles;
    r.waves = 4;
    r.two_pass = g.splits > 1 && g.two_pass;
    r.launches = (r.two_pass ? 2 : 1) + (g.tail_units > 0 ? 1 : 0);
    r.counter_tiles = g.splits > 1 && !g.two_pass ? g.tiles : 0;
    if (g.tail_units > 0) {
      r.tail_tile_tokens = 32 * g.tail_mb;
      r.tail_tile_features = 128 * g.cb;
      r.tail_tiles = g.tail_units;
    }
  }
  r.workspace_bytes = workspace_for(M, N, K, gm.kgroup, dtype, has_zp != 0, p, cus);
  *out = r;
  return ok();
}

w4a16_status w4a16_linear(const void* x, const int32_t* wq, const void* scales, const int32_t* zp,
                          const void* bias, void* y, int64_t M, int64_t N, int64_t K,
                          int32_t group_size, int32_t dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return linear_impl(x, wq, scales, zp, bias, y, M, N, K, group_size, dtype, workspace,
                     workspace_bytes, stream, W4A16_PATH_AUTO);
}

w4a16_status w4a16_linear_path(const void* x, const int32_t* wq, const void* scales,
                               const int32_t* zp, const void* bias, void* y, int64_t M, int64_t N,
                               int64_t K, int32_t group_size, int32_t dtype, void* workspace,
                               size_t workspace_bytes, void* stream, int32_t path) {
  return linear_impl(x, wq, scales, zp, bias, y, M, N, K, group_size, dtype, workspace,
                     workspace_bytes, stream, path);
}

w4a16_status w4a16_linear_noalloc(const void* x, const int32_t* wq, const void* scales,
                                  const int32_t* zp, const void* bias, void* y, int64_t M,
                                  int64_t N, int64_t K, int32_t group_size, int32_t dtype,
                                  void* stream) {
  w4a16_status st = w4a16_check_args(x, wq, scales, zp, bias, y, M, N, K, group_size, dtype);
  if (st != W4A16_OK) return st;
  if (M == 0) return ok();
  const DeviceInfo* dev = nullptr;
  st = device_info(&dev);
  if (st != W4A16_OK) return st;
  const GroupMap gm = group_map(group_size, K);
  const w4a16_path p = resolve_path(M, N, K, gm.kgroup, dtype, zp != nullptr, W4A16_PATH_AUTO);
  const size_t need = workspace_for(M, N, K, gm.kgroup, dtype, zp != nullptr, p, dev->cu_count);
  if (need > kScratchBytes)
    return fail(W4A16_ERR_UNSUPPORTED,
                "w4a16_linear_noalloc: this problem needs %zu bytes of split-K workspace, above the "
                "%zu bytes of scratch it holds; call w4a16_linear with a workspace instead",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int d = -1;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDevices)
      return fail(W4A16_ERR_DEVICE, "noalloc: no current device");
    st = scratch_for(g_devices[d], d, static_cast<hipStream_t>(stream), &ws);
    if (st != W4A16_OK) return st;
  }
  return linear_impl(x, wq, scales, zp, bias, y, M, N, K, group_size, dtype, ws, need, stream,
                     W4A16_PATH_AUTO);
}

w4a16_status w4a16_dequant(const int32_t* wq, const void* scales, const int32_t* zp, void* w,
                           int64_t N, int64_t K, int32_t group_size, int32_t dtype, void* stream) {
  if (dtype != W4A16_F16 && dtype != W4A16_BF16)
    return fail(W4A16_ERR_INVALID_ARG, "activation dtype must be fp16 (0) or bf16 (1), got %d", (int)dtype);
  if (!group_ok(group_size, K))
    return fail(W4A16_ERR_UNSUPPORTED,
                "group size must be 32, 64, 128 or K (per-channel, K %% 32 == 0), got %d (K=%lld)",
                (int)group_size, (long long)K);
  if (N < 1 || K < group_size || K % group_size)
    return fail(W4A16_ERR_INVALID_ARG, "need N >= 1 and K a positive multiple of the group size");
  if (zp && N % 8) return fail(W4A16_ERR_INVALID_ARG, "packed zero points need N %% 8 == 0");
  if (!wq || !scales || !w) return fail(W4A16_ERR_INVALID_ARG, "wq, scales and w must not be NULL");
  if (!aligned(wq, 4) || !aligned(w, 16) || !aligned(scales, 2) || (zp && !aligned(zp, 4)))
    return fail(W4A16_ERR_ALIGNMENT, "w must be 16-byte aligned, wq and zp 4-byte, scales 2-byte");
  const DeviceInfo* dev = nullptr;
  w4a16_status st = device_info(&dev);
  if (st != W4A16_OK) return st;
  const GroupMap gm = group_map(group_size, K);
  hipError_t e = w4a16::launch_dequant(wq, scales, zp, gm.sG, gm.gmul, w, N, K, gm.kgroup, dtype,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(W4A16_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

w4a16_status w4a16_moe_linear(const void* x, const int32_t* wq, const void* scales,
                              const int32_t* zp, const void* bias, const int32_t* topk_ids,
                              const float* topk_weights, void* y, int64_t M, int64_t topk,
                              int64_t E, int64_t N, int64_t K, int32_t group_size, int32_t dtype,
                              int32_t x_per_slot, void* stream) {
  if (dtype != W4A16_F16 && dtype != W4A16_BF16)
    return fail(W4A16_ERR_INVALID_ARG, "activation dtype must be fp16 (0) or bf16 (1), got %d", (int)dtype);
  if (!group_ok(group_size, K))
    return fail(W4A16_ERR_UNSUPPORTED,
                "group size must be 32, 64, 128 or K (per-channel, K %% 32 == 0), got %d (K=%lld)",
                (int)group_size, (long long)K);
  if (M < 0 || topk < 1 || E < 1 || N < 1)
    return fail(W4A16_ERR_INVALID_ARG, "need M >= 0, topk >= 1, E >= 1, N >= 1");
  if (K < group_size || K % group_size)
    return fail(W4A16_ERR_INVALID_ARG, "K must be a positive multiple of the group size %d, got K=%lld",
                (int)group_size, (long long)K);
  if (zp && N % 8)
    return fail(W4A16_ERR_INVALID_ARG, "packed zero points need N %% 8 == 0, got N=%lld", (long long)N);
  if (M * topk > w4a16::kMaxGridZ || N > INT32_MAX || K > INT32_MAX || E > INT32_MAX)
    return fail(W4A16_ERR_UNSUPPORTED, "M * topk must be at most %lld", (long long)w4a16::kMaxGridZ);
  if ((uint64_t)N * (uint64_t)K / 2 > 0xFFFFFFFFull)
    return fail(W4A16_ERR_UNSUPPORTED, "one expert's weights must be below 4 GiB (N*K/2)");
  if (K > w4a16::kMaxK)
    return fail(W4A16_ERR_UNSUPPORTED, "K above %lld is not supported (the kernels' 32-bit offsets), got K=%lld",
                (long long)w4a16::kMaxK, (long long)K);
  if (M == 0) return ok();
  if (!x || !wq || !scales || !topk_ids || !y)
    return fail(W4A16_ERR_INVALID_ARG, "x, wq, scales, topk_ids and y must not be NULL");
  if (!aligned(x, 16) || !aligned(wq, 16))
    return fail(W4A16_ERR_ALIGNMENT, "x and wq must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(y, 2) || (bias && !aligned(bias, 2)) || !aligned(topk_ids, 4) ||
      (topk_weights && !aligned(topk_weights, 4)) || (zp && !aligned(zp, 4)))
    return fail(W4A16_ERR_ALIGNMENT, "scales, bias and y must be 2-byte aligned; zp, topk_ids and "
                "topk_weights 4-byte aligned");
  const int64_t slots = M * topk;
  const int64_t G = K / group_size;
  const size_t ybytes = act_bytes(slots * N);
  if (overlap(y, ybytes, x, act_bytes((x_per_slot ? slots : M) * K)) ||
      overlap(y, ybytes, wq, (size_t)E * N * (K / 8) * 4) || overlap(y, ybytes, scales, act_bytes(E * N * G)) ||
      (zp && overlap(y, ybytes, zp, (size_t)E * (N / 8) * G * 4)) ||
      (bias && overlap(y, ybytes, bias, act_bytes(E * N))) || overlap(y, ybytes, topk_ids, (size_t)slots * 4) ||
      (topk_weights && overlap(y, ybytes, topk_weights, (size_t)slots * 4)))
    return fail(W4A16_ERR_INVALID_ARG, "y must not overlap any input");
  const DeviceInfo* dev = nullptr;
  w4a16_status st = device_info(&dev);
  if (st != W4A16_OK) return st;
  const GroupMap gm = group_map(group_size, K);
  // one K range per slot (the slots fill the device): planned as if for one CU
  const w4a16::GemvPlan plan = w4a16::plan_gemv(1, N, K, gm.kgroup, dtype, 1);
  w4a16::LinearArgs a{x, wq, scales, zp, bias, y, 1, N, K, gm.kgroup, dtype, gm.sG, gm.gmul};
  w4a16::MoeArgs moe{topk_ids, topk_weights, topk, E, slots, x_per_slot != 0};
  if (plan.splits != 1 && !w4a16::gemv_one_runs(a, plan, &moe))
    return fail(W4A16_ERR_UNSUPPORTED, "K=%lld is too large for one decode workgroup per slot",
                (long long)K);
  hipError_t e = w4a16::launch_gemv(a, plan, nullptr, static_cast<hipStream_t>(stream), &moe);
  if (e != hipSuccess) return fail(W4A16_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t w4a16_dense_workspace_size(int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t has_bias) {
  (void)has_bias;
  if (M <= 0 || N <= 0 || K <= 0 || K % 32 || (dtype != W4A16_F16 && dtype != W4A16_BF16)) return 0;
  int cus = kPlanningCUs;
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
    const DeviceInfo* d = nullptr;
    if (device_info(&d) == W4A16_OK) cus = d->cu_count;
    g_last_error.clear();
  }
  return w4a16::gemm_workspace_bytes(M, N, K, 128, dtype, false, cus, true);
}

w4a16_status w4a16_linear_dense(const void* x, const void* w, const void* bias, void* y, int64_t M,
                                int64_t N, int64_t K, int32_t dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (dtype != W4A16_F16 && dtype != W4A16_BF16)
    return fail(W4A16_ERR_INVALID_ARG, "activation dtype must be fp16 (0) or bf16 (1), got %d", (int)dtype);
  if (M < 0 || N < 1 || K < 32 || K % 32)
    return fail(W4A16_ERR_INVALID_ARG, "need M >= 0, N >= 1 and K a positive multiple of 32 (M=%lld N=%lld K=%lld)",
                (long long)M, (long long)N, (long long)K);
  if ((uint64_t)N * (uint64_t)K * 2 > 0xFFFFFFFFull || (uint64_t)M * (uint64_t)K * 2 > 0xFFFFFFFFull ||
      M > INT32_MAX || N > INT32_MAX)
    return fail(W4A16_ERR_UNSUPPORTED,
                "the dense path addresses w and x with 32-bit byte offsets: N*K*2 and M*K*2 must be "
                "below 4 GiB (M=%lld N=%lld K=%lld)", (long long)M, (long long)N, (long long)K);
  if (M == 0) return ok();
  if (!x || !w || !y) return fail(W4A16_ERR_INVALID_ARG, "x, w and y must not be NULL");
  if (!aligned(x, 16) || !aligned(w, 16))
    return fail(W4A16_ERR_ALIGNMENT, "x and w must be 16-byte aligned");
  if (!aligned(y, 2) || (bias && !aligned(bias, 2)))
    return fail(W4A16_ERR_ALIGNMENT, "bias and y must be 2-byte aligned");
  const size_t ny = act_bytes(M * N);
  if (overlap(y, ny, x, act_bytes(M * K)) || overlap(y, ny, w, act_bytes(N * K)) ||
      overlap(y, ny, bias, bias ? act_bytes(N) : 0))
    return fail(W4A16_ERR_INVALID_ARG, "y must not overlap x, w or bias");
  const DeviceInfo* dev = nullptr;
  w4a16_status st = device_info(&dev);
  if (st != W4A16_OK) return st;
  const size_t need = w4a16::gemm_workspace_bytes(M, N, K, 128, dtype, false, dev->cu_count, true);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(W4A16_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu%s", need,
                workspace_bytes, workspace ? "" : " (NULL)");
  if (need > 0 && !aligned(workspace, 256))
    return fail(W4A16_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (need > 0 && (overlap(workspace, need, y, ny) || overlap(workspace, need, x, act_bytes(M * K)) ||
                   overlap(workspace, need, w, act_bytes(N * K))))
    return fail(W4A16_ERR_INVALID_ARG, "the workspace must not overlap x, w or y");
  // the prefill GEMM's dense instances: w in place of the packed codes, no
  // scales or zero points
  w4a16::LinearArgs a{x, static_cast<const int32_t*>(w), nullptr, nullptr, bias, y, M, N, K, 128, dtype, 0, 0};
  a.dense = true;
  const hipError_t e = w4a16::launch_gemm(a, workspace, dev->cu_count, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(W4A16_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

w4a16_status w4a16_unpack_device(const int32_t* wq, uint8_t* q, int64_t N, int64_t K, void* stream) {
  if (N < 0 || K < 0 || K % 8) return fail(W4A16_ERR_INVALID_ARG, "need N >= 0, K >= 0, K %% 8 == 0");
  if (N == 0 || K == 0) return ok();
  if (!wq || !q) return fail(W4A16_ERR_INVALID_ARG, "wq and q must not be NULL");
  if (!aligned(wq, 4) || !aligned(q, 8)) return fail(W4A16_ERR_ALIGNMENT, "wq must be 4-byte and q 8-byte aligned");
  const DeviceInfo* dev = nullptr;
  w4a16_status st = device_info(&dev);
  if (st != W4A16_OK) return st;
  hipError_t e = w4a16::launch_unpack(wq, q, N, K, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(W4A16_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
