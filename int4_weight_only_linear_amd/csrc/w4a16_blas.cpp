// Dense GEMM for the dequantised prefill copy: y = x . w^T with w[N, K] the
// activation-dtype weights w4a16_dequant wrote (the pages' optional
// dequantized prefill cache: "Converge the two W4A16 linear kernels onto the
// upstream shell", "What this does").  A plain dense product, so it goes to
// the vendor BLAS on the matrix cores; rocBLAS is opened at run time on the
// first dense call, so the rest of the library never depends on it and a
// missing rocBLAS is an error of this path only.  The process's own copy is
// used when one is already loaded (same soname).
#include <dlfcn.h>

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>  // types and constants only; functions come from dlsym

#include <cstdio>
#include <mutex>
#include <string>

#include "w4a16.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

struct Blas {
  bool tried = false;
  bool ok = false;
  std::string why;
  decltype(&rocblas_create_handle) create = nullptr;
  decltype(&rocblas_set_stream) set_stream = nullptr;
  decltype(&rocblas_set_workspace) set_workspace = nullptr;
  decltype(&rocblas_gemm_ex) gemm = nullptr;
};

Blas g_blas;
std::mutex g_blas_mutex;
constexpr int kMaxDenseDevices = 64;
rocblas_handle g_handles[kMaxDenseDevices] = {};

const Blas& blas() {
  std::lock_guard<std::mutex> lock(g_blas_mutex);
  if (g_blas.tried) return g_blas;
  g_blas.tried = true;
  void* h = dlopen("librocblas.so.5", RTLD_NOW | RTLD_LOCAL);
  if (!h) h = dlopen("librocblas.so", RTLD_NOW | RTLD_LOCAL);
  if (!h) {
    const char* e = dlerror();
    g_blas.why = std::string("rocBLAS could not be opened: ") + (e ? e : "unknown error");
    return g_blas;
  }
  g_blas.create = reinterpret_cast<decltype(g_blas.create)>(dlsym(h, "rocblas_create_handle"));
  g_blas.set_stream = reinterpret_cast<decltype(g_blas.set_stream)>(dlsym(h, "rocblas_set_stream"));
  g_blas.set_workspace = reinterpret_cast<decltype(g_blas.set_workspace)>(dlsym(h, "rocblas_set_workspace"));
  g_blas.gemm = reinterpret_cast<decltype(g_blas.gemm)>(dlsym(h, "rocblas_gemm_ex"));
  if (!g_blas.create || !g_blas.set_stream || !g_blas.set_workspace || !g_blas.gemm) {
    g_blas.why = "rocBLAS lacks rocblas_create_handle, rocblas_set_stream, rocblas_set_workspace "
                 "or rocblas_gemm_ex";
    return g_blas;
  }
  g_blas.ok = true;
  return g_blas;
}

}  // namespace

bool dense_gemm(const void* x, const void* w, void* d, bool d_f32, int64_t M, int64_t N, int64_t K,
                int dtype, void* blas_ws, size_t blas_ws_bytes, hipStream_t stream,
                std::string* why) {
  const Blas& b = blas();
  if (!b.ok) {
    *why = b.why;
    return false;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDenseDevices) {
    *why = "no current device";
    return false;
  }
  rocblas_handle handle;
  {
    std::lock_guard<std::mutex> lock(g_blas_mutex);
    if (!g_handles[dev] && b.create(&g_handles[dev]) != rocblas_status_success) {
      g_handles[dev] = nullptr;
      *why = "rocblas_create_handle failed";
      return false;
    }
    handle = g_handles[dev];
    // one handle per device: the stream and workspace below are set and used
    // under the lock, so concurrent callers on one device do not mix them
    if (b.set_stream(handle, stream) != rocblas_status_success ||
        b.set_workspace(handle, blas_ws, blas_ws_bytes) != rocblas_status_success) {
      *why = "rocblas_set_stream / rocblas_set_workspace failed";
      return false;
    }
    // column-major view: D[N, M] = W^T(N x K) . X(K x M), W stored K x N
    // (lda = K), X stored K x M (ldb = K), D stored N x M (ldd = N)
    const rocblas_datatype t = dtype == W4A16_F16 ? rocblas_datatype_f16_r : rocblas_datatype_bf16_r;
    const rocblas_datatype td = d_f32 ? rocblas_datatype_f32_r : t;
    const float alpha = 1.0f, beta = 0.0f;
    const rocblas_status st = b.gemm(handle, rocblas_operation_transpose, rocblas_operation_none,
                                     (rocblas_int)N, (rocblas_int)M, (rocblas_int)K, &alpha, w, t,
                                     (rocblas_int)K, x, t, (rocblas_int)K, &beta, d, td,
                                     (rocblas_int)N, d, td, (rocblas_int)N,
                                     rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    if (st != rocblas_status_success) {
      char buf[96];
      std::snprintf(buf, sizeof(buf), "rocblas_gemm_ex failed with status %d", (int)st);
      *why = buf;
      return false;
    }
  }
  return true;
}

}  // namespace w4a16
