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

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Stands for the address of a workspace copy in the path choice.
const void* const kCopyAddress = reinterpret_cast<const void*>(uintptr_t(256));

// Large enough that copying A and B into padded rows and running the
// full-tile kernel beats the edge kernel (at least 2^30 multiply-adds; the
// copies then cost about a fifth of the product on MI355X).
bool padding_pays(int M, int N, int K) { return (int64_t)M * N * K >= (int64_t(1) << 30); }

// The fp32 path, and for GEMM_PATH_F32_PADDED the extent the streaming
// kernels see: an operand whose rows are not whole tiles, not 16-byte aligned
// or whose K is not a multiple of 64 is copied into zero-padded rows (A:
// Mp x Kp, B: Kp x Np); the other is read in place.  Tiles are 128 x 128
// when the padded product has at least kPadTiles of them, else 64 x 64.
struct Plan32 {
  int path = GEMM_PATH_NOOP;
  bool copy_a = false, copy_b = false;
  int Mp = 0, Np = 0, Kp = 0;
  int64_t lda = 0, ldb = 0;
};
constexpr int64_t kPadTiles = 256;   // the CU count of MI355X

Plan32 plan32(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb,
              float beta, const float* C, int ldc) {
  (void)beta;
  Plan32 pl;
  auto done = [&](int code) {
    pl.path = code;
    return pl;
  };
  if (M < 0 || N < 0 || K < 0) return done(GEMM_ERR_NEGATIVE_DIM);
  if (M == 0 || N == 0) return done(GEMM_PATH_NOOP);
  if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
    return done(GEMM_ERR_BAD_LD);
  if (C == nullptr) return done(GEMM_ERR_NULL_POINTER);
  if (K == 0 || alpha == 0.f) return done(GEMM_PATH_F32_SCALE);
  if (A == nullptr || B == nullptr) return done(GEMM_ERR_NULL_POINTER);
  if (force_general()) return done(GEMM_PATH_F32_GENERAL);
  if (splitk_plan(M, N, K, kF32Slab, kF32Rule, 0).splits > 1) return done(GEMM_PATH_F32_SPLITK);
  const bool tiles = f32_mfma_fits(M, N, K, A, lda, B, ldb, C, ldc);
  if (f32_stream_fits(M, N, K, A, lda, B, ldb, C, ldc) || (tiles && !padding_pays(M, N, K)))
    return done(GEMM_PATH_F32_MFMA);
  if (!padding_pays(M, N, K)) return done(GEMM_PATH_F32_GENERAL);
  const int64_t big = round_up(M, 128) * round_up(N, 128) / (128 * 128);
  const int bt = big >= kPadTiles ? 128 : 64;
  const bool k_ok = K % 64 == 0;
  pl.copy_a = !(k_ok && M % bt == 0 && f32_operand_fits(A, lda));
  pl.copy_b = !(k_ok && N % bt == 0 && f32_operand_fits(B, ldb));
  pl.Kp = (int)round_up(K, 64);
  pl.Mp = pl.copy_a ? (int)round_up(M, bt) : M;
  pl.Np = pl.copy_b ? (int)round_up(N, bt) : N;
  pl.lda = pl.copy_a ? pl.Kp : lda;
  pl.ldb = pl.copy_b ? pl.Np : ldb;
  // the copies' leading dimensions must also suit the kernels' lane offsets
  if (!f32_operand_fits(kCopyAddress, pl.lda) || !f32_operand_fits(kCopyAddress, pl.ldb))
    return done(GEMM_PATH_F32_GENERAL);
  return done(GEMM_PATH_F32_PADDED);
}

int f32_select(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb,
               float beta, const float* C, int ldc) {
  return plan32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc).path;
}

// The 16-bit calls share one selection.  Plan16 records the kernel path and
// which operands the kernels read from a workspace copy instead of in place:
// an operand that is not K-contiguous (gemm_ex's A for OP_T, B for OP_N) is
// copied transposed; on the padded path an operand whose rows are not whole
// tiles, not 16-byte aligned or whose K is not a multiple of the slab is
// copied into zero-padded rows of round64(K) elements, 128-row multiples.
struct Plan16 {
  int path = GEMM_PATH_NOOP;
  bool copy_a = false, copy_b = false;
  bool gemv_kn = false;         // matrix-vector path with the long operand K-major
  int Mp = 0, Np = 0, Kp = 0;   // the extent the kernels see
  int64_t lda = 0, ldb = 0;     // leading dimensions the kernels see
};


// The validated plan of a 16-bit call, or a negative GEMM_ERR_* code in
// plan.path.  K == 0 gives C = act(bias) + residual: zero when there is no
// write-back, else the edge kernel with an empty product.
Plan16 plan16(int type, int op_a, int op_b, int M, int N, int K, const void* A, int lda,
              const void* B, int ldb, const void* bias, int act, const void* res, int ldr,
              const void* C, int ldc) {
  Plan16 pl;
  auto fail = [&](int code) {
    pl.path = code;
    return pl;
  };
  if (M < 0 || N < 0 || K < 0) return fail(GEMM_ERR_NEGATIVE_DIM);
  if ((type != GEMM_TYPE_F16 && type != GEMM_TYPE_BF16) ||
      (op_a != GEMM_OP_N && op_a != GEMM_OP_T) || (op_b != GEMM_OP_N && op_b != GEMM_OP_T) ||
      (act != GEMM_ACT_NONE && act != GEMM_ACT_RELU && act != GEMM_ACT_SILU))
    return fail(GEMM_ERR_BAD_ARG);
  if (M == 0 || N == 0) return fail(GEMM_PATH_NOOP);
  const int need_a = op_a == GEMM_OP_N ? K : M, need_b = op_b == GEMM_OP_N ? N : K;
  if (lda < (need_a > 1 ? need_a : 1) || ldb < (need_b > 1 ? need_b : 1) ||
      ldc < (N > 1 ? N : 1))
    return fail(GEMM_ERR_BAD_LD);
  if (res != nullptr && ldr < (N > 1 ? N : 1)) return fail(GEMM_ERR_BAD_LD);
  if (C == nullptr) return fail(GEMM_ERR_NULL_POINTER);
  if (K > 0 && (A == nullptr || B == nullptr)) return fail(GEMM_ERR_NULL_POINTER);
  const bool epi = bias != nullptr || res != nullptr || act != GEMM_ACT_NONE;
  pl.Mp = M;
  pl.Np = N;
  pl.Kp = K;
  pl.lda = lda;
  pl.ldb = ldb;
  if (K == 0) return fail(epi ? GEMM_PATH_F16_GENERAL : GEMM_PATH_F16_ZERO);
  // Transposed copies (gemm_ex layouts other than A * B^T).
  pl.copy_a = op_a == GEMM_OP_T;
  pl.copy_b = op_b == GEMM_OP_N;
  const int64_t row8 = round_up(K, 8);
  if (pl.copy_a) pl.lda = row8;
  if (pl.copy_b) pl.ldb = row8;
  const void* a_read = pl.copy_a ? kCopyAddress : A;
  const void* b_read = pl.copy_b ? kCopyAddress : B;
  if (force_general()) return fail(GEMM_PATH_F16_GENERAL);
  if (f16_gemv_fits(M, N)) {
    // A long operand stored K-major is read in place by the K-major kernel,
    // which also reads the short one in either layout: no copies.
    const bool wb = f16_gemv_w_is_b(M, N);
    if (wb ? op_b == GEMM_OP_N : op_a == GEMM_OP_T) {
      pl.gemv_kn = true;
      pl.copy_a = pl.copy_b = false;
      pl.lda = lda;
      pl.ldb = ldb;
    }
    return fail(GEMM_PATH_F16_GEMV);
  }
  if (splitk_plan(M, N, K, kF16Slab, kF16Rule, 0).splits > 1) return fail(GEMM_PATH_F16_SPLITK);
  if (f16_mfma_fits(M, N, K, a_read, pl.lda, b_read, pl.ldb, C, ldc) &&
      (!epi || f16_epi_fits(bias, res, ldr)))
    return fail(GEMM_PATH_F16_MFMA);
  // Large products the full tiles cannot take in place (ragged, unaligned
  // rows, odd leading dimensions, C or the write-back operands unaligned):
  // the register-staged kernel reads the operands (or their transposed
  // copies) where they are.
  if (padding_pays(M, N, K) && f16_staged_fits(M, N, K, pl.lda, pl.ldb))
    return fail(GEMM_PATH_F16_STAGED);
  return fail(GEMM_PATH_F16_GENERAL);
}

int f16_select(int M, int N, int K, const void* A, int lda, const void* B, int ldb, const void* C,
               int ldc) {
  return plan16(GEMM_TYPE_F16, GEMM_OP_N, GEMM_OP_T, M, N, K, A, lda, B, ldb, nullptr,
                GEMM_ACT_NONE, nullptr, 0, C, ldc)
      .path;
}

int f16_ex_select(int M, int N, int K, const void* A, int lda, const void* B, int ldb,
                  const void* bias, int act, const void* res, int ldr, const void* C, int ldc) {
  return plan16(GEMM_TYPE_F16, GEMM_OP_N, GEMM_OP_T, M, N, K, A, lda, B, ldb, bias, act, res, ldr,
                C, ldc)
      .path;
}

int ex_select(int type, int op_a, int op_b, int M, int N, int K, const void* A, int lda,
              const void* B, int ldb, const void* bias, int act, const void* res, int ldr,
              const void* C, int ldc) {
  return plan16(type, op_a, op_b, M, N, K, A, lda, B, ldb, bias, act, res, ldr, C, ldc).path;
}

int to_status(hipError_t e) { return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH; }

// As to_status, with a workspace that could not be allocated reported as such.
int run_status(hipError_t e) {
  return e == hipErrorOutOfMemory ? GEMM_ERR_WORKSPACE : to_status(e);
}

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

// The padded fp32 path: zero-padded copies of the operands that need them
// (one launch), then the masked streaming kernel on the padded extent.
// Without a workspace the edge kernel runs instead.
hipError_t run32_padded(const Plan32& pl, F32Args a, int cus, hipStream_t s) {
  auto round256 = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t bytes_a = pl.copy_a ? round256((size_t)pl.Mp * pl.lda * 4) : 0;
  const size_t bytes_b = pl.copy_b ? round256((size_t)pl.Kp * pl.ldb * 4) : 0;
  std::unique_lock<std::mutex> lock(g_ws_mutex, std::defer_lock);
  bool owned = false;
  char* ws = nullptr;
  if (bytes_a + bytes_b > 0) {   // else only C is unaligned: no copies
    lock.lock();
    ws = static_cast<char*>(stream_workspace(s, bytes_a + bytes_b, &owned));
    if (owned || ws == nullptr) lock.unlock();
    if (ws == nullptr) return launch_f32_edge(a, cus, s);
  }
  float* dst_a = reinterpret_cast<float*>(ws);
  float* dst_b = reinterpret_cast<float*>(ws + bytes_a);
  const PadCopy32 pad_a{a.A, dst_a, a.lda, pl.lda, a.M, a.K, pl.Mp, pl.Kp};
  const PadCopy32 pad_b{a.B, dst_b, a.ldb, pl.ldb, a.K, a.N, pl.Kp, pl.Np};
  hipError_t e = hipSuccess;
  if (pl.copy_a || pl.copy_b)
    e = pl.copy_a ? launch_pad32(pad_a, pl.copy_b ? &pad_b : nullptr, s)
                  : launch_pad32(pad_b, nullptr, s);
  if (e == hipSuccess) {
    if (pl.copy_a) a.A = dst_a;
    if (pl.copy_b) a.B = dst_b;
    a.lda = pl.lda;
    a.ldb = pl.ldb;
    a.m_out = a.M;
    a.n_out = a.N;
    a.M = pl.Mp;
    a.N = pl.Np;
    a.K = pl.Kp;
    e = launch_f32_mfma_masked(a, cus, s);
  }
  const hipError_t f = owned ? hipFreeAsync(ws, s) : hipSuccess;
  return e != hipSuccess ? e : f;
}

// Runs a validated 16-bit plan: the operand copies (transposed and/or
// padded) into the workspace, then the kernels of the plan's path.  a holds
// the caller's operands and output; op_a / op_b say how A and B are stored.
hipError_t run16(const Plan16& pl, Args16 a, int op_a, int op_b, bool epi, int cus, hipStream_t s) {
  if (pl.path == GEMM_PATH_F16_ZERO) return launch_f16_zero(a, s);
  auto round256 = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t bytes_a = pl.copy_a ? round256((size_t)pl.Mp * pl.lda * 2) : 0;
  const size_t bytes_b = pl.copy_b ? round256((size_t)pl.Np * pl.ldb * 2) : 0;
  const SplitPlan split = pl.path == GEMM_PATH_F16_SPLITK
                              ? splitk_plan(a.M, a.N, a.K, kF16Slab, kF16Rule, 0)
                          : pl.gemv_kn ? gemv_kn_plan(a.M, a.N, a.K)
                                       : SplitPlan{};
  const size_t total = bytes_a + bytes_b + (split.splits > 1 || pl.gemv_kn ? split.bytes : 0);
  std::unique_lock<std::mutex> lock(g_ws_mutex, std::defer_lock);
  bool owned = false;
  char* ws = nullptr;
  if (total > 0) {
    lock.lock();
    ws = static_cast<char*>(stream_workspace(s, total, &owned));
    if (owned) lock.unlock();
    if (ws == nullptr) {
      // Without a workspace: the plain split-K product runs unsplit; the
      // copies and the K-major matrix-vector partial sums cannot be done.
      if (!pl.copy_a && !pl.copy_b && !pl.gemv_kn) return f16_tiled(a, epi, cus, s);
      return hipErrorOutOfMemory;
    }
  }
  hipError_t e = hipSuccess;
  // Transposed copies: A is [K][lda] (its transpose is op(A), M x K), B is
  // [K][ldb] (its transpose is B^T stored N x K).  The transpositions of both
  // operands share one launch.
  half_t* dst_a = reinterpret_cast<half_t*>(ws);
  half_t* dst_b = reinterpret_cast<half_t*>(ws + bytes_a);
  const PadCopy tr_a{a.A, dst_a, a.lda, pl.lda, a.K, a.M, pl.Kp, pl.Mp};
  const PadCopy tr_b{a.B, dst_b, a.ldb, pl.ldb, a.K, a.N, pl.Kp, pl.Np};
  (void)op_a;
  (void)op_b;
  if (pl.copy_a || pl.copy_b)
    e = pl.copy_a ? launch_transpose16(tr_a, pl.copy_b ? &tr_b : nullptr, s)
                  : launch_transpose16(tr_b, nullptr, s);
  if (pl.copy_a) a.A = dst_a;
  if (pl.copy_b) a.B = dst_b;
  a.lda = pl.lda;
  a.ldb = pl.ldb;
  if (e == hipSuccess) {
    switch (pl.path) {
      case GEMM_PATH_F16_GEMV:
        e = pl.gemv_kn ? launch_f16_gemv_kn(a, op_a, op_b, epi, split, ws + bytes_a + bytes_b, s)
                       : launch_f16_gemv(a, epi, s);
        break;
      case GEMM_PATH_F16_SPLITK:
        a.sk = splitk_args(split, a.M, a.N, ws + bytes_a + bytes_b);
        e = launch_f16_splitk(a, epi, cus, s);
        break;
      case GEMM_PATH_F16_MFMA: e = launch_f16_mfma(a, epi, cus, s); break;
      case GEMM_PATH_F16_STAGED: e = launch_f16_staged(a, epi, cus, s); break;
      default: e = launch_f16_edge(a, epi, s); break;
    }
  }
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
  const Plan32 pl = plan32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  const int path = pl.path;
  if (path < 0 || path == GEMM_PATH_NOOP) return path < 0 ? path : GEMM_OK;
  const int cus = check_device();
  if (cus < 0) return cus;
  const F32Args a{A, B, C, lda, ldb, ldc, M, N, K, alpha, beta};
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (path) {
    case GEMM_PATH_F32_SCALE: return to_status(launch_f32_scale(a, s));
    case GEMM_PATH_F32_MFMA: return to_status(launch_f32_mfma(a, cus, s));
    case GEMM_PATH_F32_SPLITK: return to_status(f32_auto_split(a, cus, s));
    case GEMM_PATH_F32_PADDED: return to_status(run32_padded(pl, a, cus, s));
    default: return to_status(launch_f32_edge(a, cus, s));
  }
}

MI355GEMM_API int gemm_f16_nt(int M, int N, int K, const void* A, int lda, const void* B, int ldb,
                              void* C, int ldc, void* stream) {
  const Plan16 pl = plan16(GEMM_TYPE_F16, GEMM_OP_N, GEMM_OP_T, M, N, K, A, lda, B, ldb, nullptr,
                           GEMM_ACT_NONE, nullptr, 0, C, ldc);
  if (pl.path < 0 || pl.path == GEMM_PATH_NOOP) return pl.path < 0 ? pl.path : GEMM_OK;
  const int cus = check_device();
  if (cus < 0) return cus;
  const Args16 a{static_cast<const half_t*>(A), static_cast<const half_t*>(B),
                 static_cast<half_t*>(C), lda, ldb, ldc, M, N, K};
  return run_status(run16(pl, a, GEMM_OP_N, GEMM_OP_T, false, cus,
                          static_cast<hipStream_t>(stream)));
}

MI355GEMM_API int gemm_f16_nt_ex(int M, int N, int K, const void* A, int lda, const void* B,
                                 int ldb, const void* bias, int act, const void* residual,
                                 int ldr, void* C, int ldc, void* stream) {
  const Plan16 pl = plan16(GEMM_TYPE_F16, GEMM_OP_N, GEMM_OP_T, M, N, K, A, lda, B, ldb, bias, act,
                           residual, ldr, C, ldc);
  if (pl.path < 0 || pl.path == GEMM_PATH_NOOP) return pl.path < 0 ? pl.path : GEMM_OK;
  const int cus = check_device();
  if (cus < 0) return cus;
  Args16 a{static_cast<const half_t*>(A), static_cast<const half_t*>(B),
           static_cast<half_t*>(C), lda, ldb, ldc, M, N, K};
  a.bias = static_cast<const half_t*>(bias);
  a.res = static_cast<const half_t*>(residual);
  a.ldr = residual ? ldr : 0;
  a.act = act;
  return run_status(run16(pl, a, GEMM_OP_N, GEMM_OP_T, true, cus,
                          static_cast<hipStream_t>(stream)));
}

MI355GEMM_API int gemm_ex(int type, int op_a, int op_b, int M, int N, int K, const void* A,
                          int lda, const void* B, int ldb, const void* bias, int act,
                          const void* residual, int ldr, void* C, int ldc, void* stream) {
  const Plan16 pl = plan16(type, op_a, op_b, M, N, K, A, lda, B, ldb, bias, act, residual, ldr, C,
                           ldc);
  if (pl.path < 0 || pl.path == GEMM_PATH_NOOP) return pl.path < 0 ? pl.path : GEMM_OK;
  const int cus = check_device();
  if (cus < 0) return cus;
  const bool epi = bias != nullptr || residual != nullptr || act != GEMM_ACT_NONE;
  Args16 a{static_cast<const half_t*>(A), static_cast<const half_t*>(B),
           static_cast<half_t*>(C), lda, ldb, ldc, M, N, K};
  a.bias = static_cast<const half_t*>(bias);
  a.res = static_cast<const half_t*>(residual);
  a.ldr = residual ? ldr : 0;
  a.act = act;
  a.fmt = type == GEMM_TYPE_BF16 ? kFmtBF16 : kFmtF16;
  return run_status(run16(pl, a, op_a, op_b, epi, cus, static_cast<hipStream_t>(stream)));
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
    case GEMM_PATH_F16_STAGED: return "f16_staged";
    case GEMM_PATH_F32_PADDED: return "f32_padded";
    default: return "?";
  }
}

}  // extern "C"
