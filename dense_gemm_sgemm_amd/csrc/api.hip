// C ABI: argument validation, kernel selection and launch.
#define MI355GEMM_BUILDING 1
#include "mi355gemm.h"

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "internal.h"

using namespace mi355gemm;

namespace {

// K slab depths of the tiled kernels (the granularity of split-K ranges) and
// the automatic split-K rules, measured on MI355X: the 16-bit partials run
// on the full-tile kernel, fastest at 256-400 workgroups with ranges that
// divide K; the fp32 partial kernel is fastest at about 512.
constexpr int kF32Slab = 16;
constexpr int kF16Slab = 64;
constexpr SplitRule kF32Rule{64, 512, 3, false};
constexpr SplitRule kF16Rule{256, 400, 2, true};

bool force_general() {
  const char* v = std::getenv("MI355GEMM_FORCE_PATH");
  return v != nullptr && std::strcmp(v, "general") == 0;
}

// Per-device verdict of the gfx950 check: 0 unknown, -1 not supported, else
// the device's compute-unit count.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];

// Returns the current device's CU count, or GEMM_ERR_UNSUPPORTED_DEVICE.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_ERR_UNSUPPORTED_DEVICE;
  if (dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED_DEVICE;
  int s = g_device_state[dev].load(std::memory_order_acquire);
  if (s == 0) {
    hipDeviceProp_t prop;
    const bool ok = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                    std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                    prop.multiProcessorCount > 0;
    s = ok ? prop.multiProcessorCount : -1;
    g_device_state[dev].store(s, std::memory_order_release);
  }
  return s > 0 ? s : GEMM_ERR_UNSUPPORTED_DEVICE;
}

int f32_select(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb,
               float beta, const float* C, int ldc) {
  (void)beta;
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_NEGATIVE_DIM;
  if (M == 0 || N == 0) return GEMM_PATH_NOOP;
  if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
    return GEMM_ERR_BAD_LD;
  if (C == nullptr) return GEMM_ERR_NULL_POINTER;
  if (K == 0 || alpha == 0.f) return GEMM_PATH_F32_SCALE;
  if (A == nullptr || B == nullptr) return GEMM_ERR_NULL_POINTER;
  if (force_general()) return GEMM_PATH_F32_GENERAL;
  if (splitk_plan(M, N, K, kF32Slab, kF32Rule, 0).splits > 1) return GEMM_PATH_F32_SPLITK;
  if (f32_mfma_fits(M, N, K, A, lda, B, ldb, C, ldc)) return GEMM_PATH_F32_MFMA;
  return GEMM_PATH_F32_GENERAL;
}

int f16_select(int M, int N, int K, const void* A, int lda, const void* B, int ldb, const void* C,
               int ldc) {
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_NEGATIVE_DIM;
  if (M == 0 || N == 0) return GEMM_PATH_NOOP;
  if (lda < (K > 1 ? K : 1) || ldb < (K > 1 ? K : 1) || ldc < (N > 1 ? N : 1))
    return GEMM_ERR_BAD_LD;
  if (C == nullptr) return GEMM_ERR_NULL_POINTER;
  if (K == 0) return GEMM_PATH_F16_ZERO;
  if (A == nullptr || B == nullptr) return GEMM_ERR_NULL_POINTER;
  if (force_general()) return GEMM_PATH_F16_GENERAL;
  if (f16_gemv_fits(M, N)) return GEMM_PATH_F16_GEMV;
  if (splitk_plan(M, N, K, kF16Slab, kF16Rule, 0).splits > 1) return GEMM_PATH_F16_SPLITK;
  if (f16_mfma_fits(M, N, K, A, lda, B, ldb, C, ldc)) return GEMM_PATH_F16_MFMA;
  return GEMM_PATH_F16_GENERAL;
}

// The fused call: the same checks plus its own arguments.  K == 0 runs the
// edge kernel, whose product is then zero, so that C = act(bias) + residual.
int f16_ex_select(int M, int N, int K, const void* A, int lda, const void* B, int ldb,
                  const void* bias, int act, const void* res, int ldr, const void* C, int ldc) {
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_NEGATIVE_DIM;
  if (act != GEMM_ACT_NONE && act != GEMM_ACT_RELU && act != GEMM_ACT_SILU)
    return GEMM_ERR_BAD_ARG;
  if (M == 0 || N == 0) return GEMM_PATH_NOOP;
  if (lda < (K > 1 ? K : 1) || ldb < (K > 1 ? K : 1) || ldc < (N > 1 ? N : 1))
    return GEMM_ERR_BAD_LD;
  if (res != nullptr && ldr < (N > 1 ? N : 1)) return GEMM_ERR_BAD_LD;
  if (C == nullptr) return GEMM_ERR_NULL_POINTER;
  if (K > 0 && (A == nullptr || B == nullptr)) return GEMM_ERR_NULL_POINTER;
  if (K == 0 || force_general()) return GEMM_PATH_F16_GENERAL;
  if (f16_gemv_fits(M, N)) return GEMM_PATH_F16_GEMV;
  if (splitk_plan(M, N, K, kF16Slab, kF16Rule, 0).splits > 1) return GEMM_PATH_F16_SPLITK;
  if (f16_mfma_fits(M, N, K, A, lda, B, ldb, C, ldc) && f16_epi_fits(bias, res, ldr))
    return GEMM_PATH_F16_MFMA;
  return GEMM_PATH_F16_GENERAL;
}

// gemm_ex: the operands the A * B^T kernels read.  An operand that is not
// K-contiguous (A for OP_T, B for OP_N) is read from a transposed copy with
// rows padded to a multiple of 8 elements at a 256-byte aligned address.
struct ExLayout {
  bool copy_a, copy_b;
  int64_t lda, ldb;   // leading dimensions the kernels see
};

int64_t padded_row(int K) { return ((int64_t)(K > 1 ? K : 1) + 7) / 8 * 8; }

ExLayout ex_layout(int op_a, int op_b, int K, int lda, int ldb) {
  ExLayout l;
  l.copy_a = op_a == GEMM_OP_T && K > 0;
  l.copy_b = op_b == GEMM_OP_N && K > 0;
  l.lda = l.copy_a ? padded_row(K) : lda;
  l.ldb = l.copy_b ? padded_row(K) : ldb;
  return l;
}

// Stands for the address of a transposed copy in the path choice.
const void* const kCopyAddress = reinterpret_cast<const void*>(uintptr_t(256));

int ex_select(int type, int op_a, int op_b, int M, int N, int K, const void* A, int lda,
              const void* B, int ldb, const void* bias, int act, const void* res, int ldr,
              const void* C, int ldc) {
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_NEGATIVE_DIM;
  if ((type != GEMM_TYPE_F16 && type != GEMM_TYPE_BF16) ||
      (op_a != GEMM_OP_N && op_a != GEMM_OP_T) || (op_b != GEMM_OP_N && op_b != GEMM_OP_T) ||
      (act != GEMM_ACT_NONE && act != GEMM_ACT_RELU && act != GEMM_ACT_SILU))
    return GEMM_ERR_BAD_ARG;
  if (M == 0 || N == 0) return GEMM_PATH_NOOP;
  const int need_a = op_a == GEMM_OP_N ? K : M, need_b = op_b == GEMM_OP_N ? N : K;
  if (lda < (need_a > 1 ? need_a : 1) || ldb < (need_b > 1 ? need_b : 1) ||
      ldc < (N > 1 ? N : 1))
    return GEMM_ERR_BAD_LD;
  if (res != nullptr && ldr < (N > 1 ? N : 1)) return GEMM_ERR_BAD_LD;
  if (C == nullptr) return GEMM_ERR_NULL_POINTER;
  if (K > 0 && (A == nullptr || B == nullptr)) return GEMM_ERR_NULL_POINTER;
  const bool epi = bias != nullptr || res != nullptr || act != GEMM_ACT_NONE;
  if (K == 0) return epi ? GEMM_PATH_F16_GENERAL : GEMM_PATH_F16_ZERO;
  if (force_general()) return GEMM_PATH_F16_GENERAL;
  if (f16_gemv_fits(M, N)) return GEMM_PATH_F16_GEMV;
  if (splitk_plan(M, N, K, kF16Slab, kF16Rule, 0).splits > 1) return GEMM_PATH_F16_SPLITK;
  const ExLayout l = ex_layout(op_a, op_b, K, lda, ldb);
  if (f16_mfma_fits(M, N, K, l.copy_a ? kCopyAddress : A, l.lda, l.copy_b ? kCopyAddress : B,
                    l.ldb, C, ldc) &&
      (!epi || f16_epi_fits(bias, res, ldr)))
    return GEMM_PATH_F16_MFMA;
  return GEMM_PATH_F16_GENERAL;
}

int to_status(hipError_t e) { return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH; }

// The tiled kernel of a product that takes neither split-K nor the
// matrix-vector kernel.
hipError_t f32_tiled(const F32Args& a, int cus, hipStream_t s) {
  if (!force_general() && f32_mfma_fits(a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc))
    return launch_f32_mfma(a, cus, s);
  return launch_f32_edge(a, cus, s);
}

hipError_t f16_tiled(const Args16& a, bool epi, int cus, hipStream_t s) {
  if (!force_general() && f16_mfma_fits(a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb, a.C, a.ldc) &&
      (!epi || f16_epi_fits(a.bias, a.res, a.ldr)))
    return launch_f16_mfma(a, epi, cus, s);
  return launch_f16_edge(a, epi, s);
}

// Workspaces of the automatic split-K path, one per (device, stream): every
// use of one is ordered on its stream, so calls on different streams never
// share one.  An entry only grows (the old block is returned on the same
// stream, after the work that used it), and lives until the process ends.
struct StreamWorkspace {
  int dev;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
};
std::mutex g_ws_mutex;
std::vector<StreamWorkspace> g_ws;

// A workspace of at least `bytes` for work on `s`, or nullptr; called with
// g_ws_mutex held.  The caller keeps the lock until it has enqueued all the
// work that uses a kept workspace, so that two host threads on one stream
// cannot interleave their partial and reduction kernels.  *owned tells the
// caller to return the workspace after use: so it is under stream capture,
// where the allocation becomes part of the graph and must not be kept.
void* stream_workspace(hipStream_t s, size_t bytes, bool* owned) {
  *owned = false;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = nullptr;
  if (cap != hipStreamCaptureStatusNone) {
    if (hipMallocAsync(&p, bytes, s) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    *owned = true;
    return p;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  for (StreamWorkspace& w : g_ws) {
    if (w.dev != dev || w.stream != s) continue;
    if (w.bytes >= bytes) return w.ptr;
    if (hipMallocAsync(&p, bytes, s) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    (void)hipFreeAsync(w.ptr, s);
    w.ptr = p;
    w.bytes = bytes;
    return p;
  }
  if (hipMallocAsync(&p, bytes, s) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_ws.push_back(StreamWorkspace{dev, s, p, bytes});
  return p;
}

// The split-K path of the plain calls.  If no workspace can be had, the
// tiled kernel runs instead.
hipError_t f32_auto_split(F32Args a, int cus, hipStream_t s) {
  const SplitPlan plan = splitk_plan(a.M, a.N, a.K, kF32Slab, kF32Rule, 0);
  std::unique_lock<std::mutex> lock(g_ws_mutex);
  bool owned = false;
  void* ws = stream_workspace(s, plan.bytes, &owned);
  if (owned || ws == nullptr) lock.unlock();
  if (ws == nullptr) return f32_tiled(a, cus, s);
  a.sk = splitk_args(plan, a.M, a.N, ws);
  const hipError_t e = launch_f32_splitk(a, s);
  const hipError_t f = owned ? hipFreeAsync(ws, s) : hipSuccess;
  return e != hipSuccess ? e : f;
}

hipError_t f16_auto_split(Args16 a, bool epi, int cus, hipStream_t s) {
  const SplitPlan plan = splitk_plan(a.M, a.N, a.K, kF16Slab, kF16Rule, 0);
  std::unique_lock<std::mutex> lock(g_ws_mutex);
  bool owned = false;
  void* ws = stream_workspace(s, plan.bytes, &owned);
  if (owned || ws == nullptr) lock.unlock();
  if (ws == nullptr) return f16_tiled(a, epi, cus, s);
  a.sk = splitk_args(plan, a.M, a.N, ws);
  const hipError_t e = launch_f16_splitk(a, epi, cus, s);
  const hipError_t f = owned ? hipFreeAsync(ws, s) : hipSuccess;
  return e != hipSuccess ? e : f;
}

// Checks a caller's workspace against a plan.
bool workspace_ok(const SplitPlan& plan, const void* ws, unsigned long long bytes) {
  return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 15u) == 0 && bytes >= plan.bytes;
}

}  // namespace

extern "C" {

MI355GEMM_API int gemm_f32(int M, int N, int K, float alpha, const float* A, int lda,
                           const float* B, int ldb, float beta, float* C, int ldc, void* stream) {
  const int path = f32_select(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (path < 0 || path == GEMM_PATH_NOOP) return path < 0 ? path : GEMM_OK;
  const int cus = check_device();
  if (cus < 0) return cus;
  const F32Args a{A, B, C, lda, ldb, ldc, M, N, K, alpha, beta};
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (path) {
    case GEMM_PATH_F32_SCALE: return to_status(launch_f32_scale(a, s));
    case GEMM_PATH_F32_MFMA: return to_status(launch_f32_mfma(a, cus, s));
    case GEMM_PATH_F32_SPLITK: return to_status(f32_auto_split(a, cus, s));
    default: return to_status(launch_f32_edge(a, cus, s));
  }
}

MI355GEMM_API int gemm_f16_nt(int M, int N, int K, const void* A, int lda, const void* B, int ldb,
                              void* C, int ldc, void* stream) {
  const int path = f16_select(M, N, K, A, lda, B, ldb, C, ldc);
  if (path < 0 || path == GEMM_PATH_NOOP) return path < 0 ? path : GEMM_OK;
  const int cus = check_device();
  if (cus < 0) return cus;
  const Args16 a{static_cast<const half_t*>(A), static_cast<const half_t*>(B),
                  static_cast<half_t*>(C), lda, ldb, ldc, M, N, K};
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (path) {
    case GEMM_PATH_F16_ZERO: return to_status(launch_f16_zero(a, s));
    case GEMM_PATH_F16_MFMA: return to_status(launch_f16_mfma(a, false, cus, s));
    case GEMM_PATH_F16_GEMV: return to_status(launch_f16_gemv(a, false, s));
    case GEMM_PATH_F16_SPLITK: return to_status(f16_auto_split(a, false, cus, s));
    default: return to_status(launch_f16_edge(a, false, s));
  }
}

MI355GEMM_API int gemm_f16_nt_ex(int M, int N, int K, const void* A, int lda, const void* B,
                                 int ldb, const void* bias, int act, const void* residual,
                                 int ldr, void* C, int ldc, void* stream) {
  const int path = f16_ex_select(M, N, K, A, lda, B, ldb, bias, act, residual, ldr, C, ldc);
  if (path < 0 || path == GEMM_PATH_NOOP) return path < 0 ? path : GEMM_OK;
  const int cus = check_device();
  if (cus < 0) return cus;
  Args16 a{static_cast<const half_t*>(A), static_cast<const half_t*>(B),
            static_cast<half_t*>(C), lda, ldb, ldc, M, N, K};
  a.bias = static_cast<const half_t*>(bias);
  a.res = static_cast<const half_t*>(residual);
  a.ldr = residual ? ldr : 0;
  a.act = act;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (path == GEMM_PATH_F16_MFMA) return to_status(launch_f16_mfma(a, true, cus, s));
  if (path == GEMM_PATH_F16_GEMV) return to_status(launch_f16_gemv(a, true, s));
  if (path == GEMM_PATH_F16_SPLITK) return to_status(f16_auto_split(a, true, cus, s));
  return to_status(launch_f16_edge(a, true, s));
}

MI355GEMM_API int gemm_ex(int type, int op_a, int op_b, int M, int N, int K, const void* A,
                          int lda, const void* B, int ldb, const void* bias, int act,
                          const void* residual, int ldr, void* C, int ldc, void* stream) {
  const int path = ex_select(type, op_a, op_b, M, N, K, A, lda, B, ldb, bias, act, residual, ldr,
                             C, ldc);
  if (path < 0 || path == GEMM_PATH_NOOP) return path < 0 ? path : GEMM_OK;
  const int cus = check_device();
  if (cus < 0) return cus;
  const bool epi = bias != nullptr || residual != nullptr || act != GEMM_ACT_NONE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ExLayout l = ex_layout(op_a, op_b, K, lda, ldb);
  Args16 a{static_cast<const half_t*>(A), static_cast<const half_t*>(B),
           static_cast<half_t*>(C), l.lda, l.ldb, ldc, M, N, K};
  a.bias = static_cast<const half_t*>(bias);
  a.res = static_cast<const half_t*>(residual);
  a.ldr = residual ? ldr : 0;
  a.act = act;
  a.fmt = type == GEMM_TYPE_BF16 ? kFmtBF16 : kFmtF16;
  if (path == GEMM_PATH_F16_ZERO) return to_status(launch_f16_zero(a, s));

  // Workspace: the transposed copies, then the split-K partial sums.
  auto round256 = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t bytes_a = l.copy_a ? round256((size_t)M * l.lda * 2) : 0;
  const size_t bytes_b = l.copy_b ? round256((size_t)N * l.ldb * 2) : 0;
  const SplitPlan plan = path == GEMM_PATH_F16_SPLITK
                             ? splitk_plan(M, N, K, kF16Slab, kF16Rule, 0)
                             : SplitPlan{};
  const size_t total = bytes_a + bytes_b + (plan.splits > 1 ? plan.bytes : 0);
  std::unique_lock<std::mutex> lock(g_ws_mutex, std::defer_lock);
  bool owned = false;
  char* ws = nullptr;
  if (total > 0) {
    lock.lock();
    ws = static_cast<char*>(stream_workspace(s, total, &owned));
    if (owned) lock.unlock();
    if (ws == nullptr) return GEMM_ERR_WORKSPACE;
  }
  hipError_t e = hipSuccess;
  if (l.copy_a) {   // A is [K][lda]: its transpose is op(A), M x K
    a.A = reinterpret_cast<const half_t*>(ws);
    e = launch_transpose16(static_cast<const half_t*>(A), lda, K, M, reinterpret_cast<half_t*>(ws),
                           l.lda, s);
  }
  if (e == hipSuccess && l.copy_b) {   // B is [K][ldb]: its transpose is B^T stored N x K
    a.B = reinterpret_cast<const half_t*>(ws + bytes_a);
    e = launch_transpose16(static_cast<const half_t*>(B), ldb, K, N,
                           reinterpret_cast<half_t*>(ws + bytes_a), l.ldb, s);
  }
  if (e == hipSuccess) {
    switch (path) {
      case GEMM_PATH_F16_GEMV: e = launch_f16_gemv(a, epi, s); break;
      case GEMM_PATH_F16_SPLITK:
        a.sk = splitk_args(plan, M, N, ws + bytes_a + bytes_b);
        e = launch_f16_splitk(a, epi, cus, s);
        break;
      case GEMM_PATH_F16_MFMA: e = launch_f16_mfma(a, epi, cus, s); break;
      default: e = launch_f16_edge(a, epi, s); break;
    }
  }
  const hipError_t f = owned ? hipFreeAsync(ws, s) : hipSuccess;
  return to_status(e != hipSuccess ? e : f);
}

MI355GEMM_API int gemm_f32_splitk(int M, int N, int K, float alpha, const float* A, int lda,
                                  const float* B, int ldb, float beta, float* C, int ldc,
                                  int splits, void* workspace, unsigned long long workspace_bytes,
                                  void* stream) {
  const int path = f32_select(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (path < 0 || path == GEMM_PATH_NOOP) return path < 0 ? path : GEMM_OK;
  SplitPlan plan;
  if (path != GEMM_PATH_F32_SCALE && (splits > 0 || path == GEMM_PATH_F32_SPLITK))
    plan = splitk_plan(M, N, K, kF32Slab, kF32Rule, splits);
  if (plan.splits > 1 && !workspace_ok(plan, workspace, workspace_bytes))
    return GEMM_ERR_WORKSPACE;
  const int cus = check_device();
  if (cus < 0) return cus;
  F32Args a{A, B, C, lda, ldb, ldc, M, N, K, alpha, beta};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.splits > 1) {
    a.sk = splitk_args(plan, M, N, workspace);
    return to_status(launch_f32_splitk(a, s));
  }
  switch (path) {
    case GEMM_PATH_F32_SCALE: return to_status(launch_f32_scale(a, s));
    case GEMM_PATH_F32_MFMA: return to_status(launch_f32_mfma(a, cus, s));
    case GEMM_PATH_F32_SPLITK: return to_status(f32_tiled(a, cus, s));   // splits == 1
    default: return to_status(launch_f32_edge(a, cus, s));
  }
}

MI355GEMM_API int gemm_f16_nt_splitk(int M, int N, int K, const void* A, int lda, const void* B,
                                     int ldb, void* C, int ldc, int splits, void* workspace,
                                     unsigned long long workspace_bytes, void* stream) {
  const int path = f16_select(M, N, K, A, lda, B, ldb, C, ldc);
  if (path < 0 || path == GEMM_PATH_NOOP) return path < 0 ? path : GEMM_OK;
  SplitPlan plan;
  if (path != GEMM_PATH_F16_ZERO && (splits > 0 || path == GEMM_PATH_F16_SPLITK))
    plan = splitk_plan(M, N, K, kF16Slab, kF16Rule, splits);
  if (plan.splits > 1 && !workspace_ok(plan, workspace, workspace_bytes))
    return GEMM_ERR_WORKSPACE;
  const int cus = check_device();
  if (cus < 0) return cus;
  Args16 a{static_cast<const half_t*>(A), static_cast<const half_t*>(B),
            static_cast<half_t*>(C), lda, ldb, ldc, M, N, K};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.splits > 1) {
    a.sk = splitk_args(plan, M, N, workspace);
    return to_status(launch_f16_splitk(a, false, cus, s));
  }
  switch (path) {
    case GEMM_PATH_F16_ZERO: return to_status(launch_f16_zero(a, s));
    case GEMM_PATH_F16_MFMA: return to_status(launch_f16_mfma(a, false, cus, s));
    case GEMM_PATH_F16_GEMV: return to_status(launch_f16_gemv(a, false, s));
    case GEMM_PATH_F16_SPLITK: return to_status(f16_tiled(a, false, cus, s));   // splits == 1
    default: return to_status(launch_f16_edge(a, false, s));
  }
}

MI355GEMM_API unsigned long long gemm_f32_splitk_workspace(int M, int N, int K, int splits) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return splitk_plan(M, N, K, kF32Slab, kF32Rule, splits).bytes;
}

MI355GEMM_API unsigned long long gemm_f16_nt_splitk_workspace(int M, int N, int K, int splits) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if (splits <= 0 && f16_gemv_fits(M, N)) return 0;
  return splitk_plan(M, N, K, kF16Slab, kF16Rule, splits).bytes;
}

MI355GEMM_API int gemm_f32_path(int M, int N, int K, float alpha, const float* A, int lda,
                                const float* B, int ldb, float beta, const float* C, int ldc) {
  return f32_select(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
}

MI355GEMM_API int gemm_f16_nt_path(int M, int N, int K, const void* A, int lda, const void* B,
                                   int ldb, const void* C, int ldc) {
  return f16_select(M, N, K, A, lda, B, ldb, C, ldc);
}

MI355GEMM_API int gemm_f16_nt_ex_path(int M, int N, int K, const void* A, int lda, const void* B,
                                      int ldb, const void* bias, int act, const void* residual,
                                      int ldr, const void* C, int ldc) {
  return f16_ex_select(M, N, K, A, lda, B, ldb, bias, act, residual, ldr, C, ldc);
}

MI355GEMM_API int gemm_ex_path(int type, int op_a, int op_b, int M, int N, int K, const void* A,
                               int lda, const void* B, int ldb, const void* bias, int act,
                               const void* residual, int ldr, const void* C, int ldc) {
  return ex_select(type, op_a, op_b, M, N, K, A, lda, B, ldb, bias, act, residual, ldr, C, ldc);
}

MI355GEMM_API const char* gemm_status_string(int status) {
  switch (status) {
    case GEMM_OK: return "success";
    case GEMM_ERR_NEGATIVE_DIM: return "a matrix dimension (M, N or K) is negative";
    case GEMM_ERR_BAD_LD: return "a leading dimension is smaller than its row length";
    case GEMM_ERR_NULL_POINTER: return "a matrix pointer that would be accessed is NULL";
    case GEMM_ERR_UNSUPPORTED_DEVICE: return "no HIP device, or the current device is not gfx950";
    case GEMM_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
    case GEMM_ERR_BAD_ARG:
      return "an enumerated argument (type, operation or activation) has no defined meaning";
    case GEMM_ERR_WORKSPACE:
      return "a workspace the call needs is NULL, smaller than the size query reports, not "
             "16-byte aligned, or could not be allocated";
    default: return "unknown status code";
  }
}

MI355GEMM_API const char* gemm_path_name(int path) {
  switch (path) {
    case GEMM_PATH_NOOP: return "noop";
    case GEMM_PATH_F32_SCALE: return "f32_scale";
    case GEMM_PATH_F32_GENERAL: return "f32_general";
    case GEMM_PATH_F32_MFMA: return "f32_mfma";
    case GEMM_PATH_F16_ZERO: return "f16_zero";
    case GEMM_PATH_F16_GENERAL: return "f16_general";
    case GEMM_PATH_F16_MFMA: return "f16_mfma";
    case GEMM_PATH_F16_GEMV: return "f16_gemv";
    case GEMM_PATH_F16_SPLITK: return "f16_splitk";
    case GEMM_PATH_F32_SPLITK: return "f32_splitk";
    default: return "?";
  }
}

}  // extern "C"
