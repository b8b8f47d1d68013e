// C ABI: argument validation, kernel selection and launch.
//
// The library allocates nothing and keeps no per-call state: every buffer a
// call touches is the caller's.  The plain calls (gemm_f32, gemm_f16_nt,
// gemm_f16_nt_ex) run kernels that need no scratch memory; the calls whose
// kernels do (split-K partial sums, gemm_ex's transposed copies for small
// products and its K-major matrix-vector partial sums) take a caller-owned
// workspace and report its size through a query.
#define MI355GEMM_BUILDING 1
#include "mi355gemm.h"

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "internal.h"

using namespace mi355gemm;

namespace {

// K slab depths of the tiled kernels (the granularity of split-K ranges) and
// the split-K rules that splits <= 0 selects, measured on MI355X: the 16-bit
// partials run on the full-tile kernel, fastest at 256-400 workgroups with
// ranges that divide K; the fp32 partial kernel is fastest at about 512.
constexpr int kF32Slab = 16;
constexpr int kF16Slab = 64;
constexpr SplitRule kF32Rule{64, 512, 3, false};
constexpr SplitRule kF16Rule{256, 400, 2, true};

bool force_general() {
  const char* v = std::getenv("MI355GEMM_FORCE_PATH");
  return v != nullptr && std::strcmp(v, "general") == 0;
}

// Size of the static scratch area behind gemm_f16_nt_splitk_static.
constexpr size_t kStaticScratchBytes = GEMM_STATIC_SCRATCH_BYTES;

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
size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Stands for the address of a workspace copy in the path choice.
const void* const kCopyAddress = reinterpret_cast<const void*>(uintptr_t(256));

// Large enough for the 16-bit register-staged wide tiles to beat the
// 128 x 128 edge kernel (at least 2^30 multiply-adds).
bool large_product(int M, int N, int K) { return (int64_t)M * N * K >= (int64_t(1) << 30); }

// The fp32 path of gemm_f32 (or a negative GEMM_ERR_* code).
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
  if (f32_stream_fits(M, N, K, A, lda, B, ldb, C, ldc) ||
      f32_mfma_fits(M, N, K, A, lda, B, ldb, C, ldc))
    return GEMM_PATH_F32_MFMA;
  return GEMM_PATH_F32_GENERAL;
}

// The 16-bit calls share one selection.  Plan16 records the kernel path and
// the workspace it needs: an operand that is not K-contiguous (gemm_ex's A
// for OP_T, B for OP_N) is copied transposed into the workspace
// ([rows][round8(K)], 256-byte aligned) for the A * B^T kernels; the
// matrix-vector kernel with its long operand K-major leaves partial sums over
// ranges of K there; gemm_ex's split-K leaves the partial sums of its ranges
// there, after any copies.
struct Plan16 {
  int path = GEMM_PATH_NOOP;
  int lay = 0;                  // F16_MFMA reading B [K][N] (1), A [K][M] (2) or both (3) in place
  bool copy_a = false, copy_b = false;
  bool gemv_kn = false;         // matrix-vector path with the long operand K-major
  int64_t lda = 0, ldb = 0;     // leading dimensions the A * B^T kernels see
  size_t bytes_a = 0, bytes_b = 0, bytes_kn = 0, bytes_split = 0;
  size_t workspace() const { return bytes_a + bytes_b + bytes_kn + bytes_split; }
};

// The validated plan of a 16-bit call, or a negative GEMM_ERR_* code in
// plan.path.  K == 0 gives C = act(bias) + residual: zero when there is no
// write-back, else the edge kernel with an empty product (it reads neither
// operand, whatever their layout).
Plan16 plan16(int type, int op_a, int op_b, int M, int N, int K, const void* A, int lda,
              const void* B, int ldb, const void* bias, int act, const void* res, int ldr,
              const void* C, int ldc, bool allow_split = false, bool in_place = true) {
  Plan16 pl;
  auto done = [&](int code) {
    pl.path = code;
    return pl;
  };
  if (M < 0 || N < 0 || K < 0) return done(GEMM_ERR_NEGATIVE_DIM);
  if ((type != GEMM_TYPE_F16 && type != GEMM_TYPE_BF16) ||
      (op_a != GEMM_OP_N && op_a != GEMM_OP_T) || (op_b != GEMM_OP_N && op_b != GEMM_OP_T) ||
      (act != GEMM_ACT_NONE && act != GEMM_ACT_RELU && act != GEMM_ACT_SILU))
    return done(GEMM_ERR_BAD_ARG);
  if (M == 0 || N == 0) return done(GEMM_PATH_NOOP);
  const int need_a = op_a == GEMM_OP_N ? K : M, need_b = op_b == GEMM_OP_N ? N : K;
  if (lda < (need_a > 1 ? need_a : 1) || ldb < (need_b > 1 ? need_b : 1) ||
      ldc < (N > 1 ? N : 1))
    return done(GEMM_ERR_BAD_LD);
  if (res != nullptr && ldr < (N > 1 ? N : 1)) return done(GEMM_ERR_BAD_LD);
  if (C == nullptr) return done(GEMM_ERR_NULL_POINTER);
  if (K > 0 && (A == nullptr || B == nullptr)) return done(GEMM_ERR_NULL_POINTER);
  const bool epi = bias != nullptr || res != nullptr || act != GEMM_ACT_NONE;
  pl.lda = lda;
  pl.ldb = ldb;
  if (K == 0) return done(epi ? GEMM_PATH_F16_GENERAL : GEMM_PATH_F16_ZERO);
  // Transposed copies of the operands that are not K-contiguous, for the
  // A * B^T kernels (16-byte aligned, rows of round8(K) elements).
  auto copies = [&](bool ca, bool cb) {
    const int64_t row8 = round_up(K, 8);
    pl.copy_a = ca;
    pl.copy_b = cb;
    if (ca) {
      pl.lda = row8;
      pl.bytes_a = round256((size_t)M * row8 * 2);
    }
    if (cb) {
      pl.ldb = row8;
      pl.bytes_b = round256((size_t)N * row8 * 2);
    }
  };
  const bool ca = op_a == GEMM_OP_T, cb = op_b == GEMM_OP_N;
  if (force_general()) {
    copies(ca, cb);
    return done(GEMM_PATH_F16_GENERAL);
  }
  if (f16_gemv_fits(M, N)) {
    // The long operand W stored K-major is read in place by the K-major
    // kernel, which also reads the short one in either layout; its ranges of
    // K leave partial sums in the workspace.  Otherwise only the short
    // operand may need a (small) transposed copy.
    const bool wb = f16_gemv_w_is_b(M, N);
    if (wb ? cb : ca) {
      pl.gemv_kn = true;
      pl.bytes_kn = round256(gemv_kn_plan(M, N, K).bytes);
    } else {
      copies(ca, cb);
    }
    return done(GEMM_PATH_F16_GEMV);
  }
  // gemm_ex: long K over few output tiles splits K into ranges (on the
  // transposed copies in the other layouts).
  if (allow_split) {
    const SplitPlan sp = splitk_plan(M, N, K, kF16Slab, kF16Rule, 0);
    if (sp.splits > 1) {
      copies(ca, cb);
      pl.bytes_split = sp.bytes;
      return done(GEMM_PATH_F16_SPLITK);
    }
  }
  // NN, TT and TN on whole tiles or their ragged form: the full-tile kernels
  // read the K-major operands in place through the transposing LDS reads (no
  // copy, no workspace), unless the A * B^T tiles on copies would cost less.
  const int lay = cb && !ca ? 1 : ca && !cb ? 2 : ca && cb ? 3 : 0;
  if (in_place && lay != 0 && f16_kmajor_fits(lay, M, N, K, A, lda, B, ldb, C, ldc) &&
      (!epi || f16_epi_fits(bias, res, ldr))) {
    pl.lay = lay;
    return done(GEMM_PATH_F16_MFMA);
  }
  // The other layouts and shapes run on transposed copies: on 5376 x 5376 x
  // 2048 TN's copies and the full-tile kernel take 113-122 us, where the
  // register-staged wide tiles reading the K-major operands in place (8 x 8
  // blocks transposed in registers) took 164-481 us.
  copies(ca, cb);
  const void* a_read = ca ? kCopyAddress : A;
  const void* b_read = cb ? kCopyAddress : B;
  if (f16_mfma_fits(M, N, K, a_read, pl.lda, b_read, pl.ldb, C, ldc) &&
      (!epi || f16_epi_fits(bias, res, ldr)))
    return done(GEMM_PATH_F16_MFMA);
  // Large products that are not whole tiles but whose A and B rows start at
  // 16-byte addresses (K % 8 == 0): the full-tile kernels' ragged form.
  if (large_product(M, N, K) && f16_ragged_fits(M, N, K, a_read, pl.lda, b_read, pl.ldb))
    return done(GEMM_PATH_F16_MFMA);
  // Large products the full tiles cannot take (ragged, unaligned rows, odd
  // leading dimensions, C or the write-back operands unaligned): the
  // register-staged wide tiles read the operands (or the copies) in place.
  if (large_product(M, N, K) && f16_staged_fits(M, N, K, pl.lda, pl.ldb))
    return done(GEMM_PATH_F16_STAGED);
  return done(GEMM_PATH_F16_GENERAL);
}

int to_status(hipError_t e) { return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH; }

// A caller's workspace: 16-byte aligned and at least `need` bytes (or not
// needed at all).
bool workspace_ok(size_t need, const void* ws, unsigned long long bytes) {
  return need == 0 ||
         (ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 15u) == 0 && bytes >= need);
}

// Runs a validated 16-bit plan.  a holds the caller's operands (in their
// stored layouts) and output; op_a / op_b say how A and B are stored; ws is
// the caller's workspace (checked against the plan by the caller).
hipError_t run16(const Plan16& pl, Args16 a, int op_a, int op_b, bool epi, int cus, char* ws,
                 hipStream_t s) {
  switch (pl.path) {
    case GEMM_PATH_F16_ZERO: return launch_f16_zero(a, s);
    case GEMM_PATH_F16_GEMV:
      if (pl.gemv_kn)
        return launch_f16_gemv_kn(a, op_a, op_b, epi, gemv_kn_plan(a.M, a.N, a.K), ws, s);
      break;
    default: break;
  }
  // Transposed copies: A is [K][lda] (its transpose is op(A), M x K), B is
  // [K][ldb] (its transpose is B^T stored N x K).  The transpositions of both
  // operands share one launch.
  if (pl.copy_a || pl.copy_b) {
    half_t* dst_a = reinterpret_cast<half_t*>(ws);
    half_t* dst_b = reinterpret_cast<half_t*>(ws + pl.bytes_a);
    const PadCopy tr_a{a.A, dst_a, a.lda, pl.lda, a.K, a.M, a.K, a.M};
    const PadCopy tr_b{a.B, dst_b, a.ldb, pl.ldb, a.K, a.N, a.K, a.N};
    const hipError_t e = pl.copy_a ? launch_transpose16(tr_a, pl.copy_b ? &tr_b : nullptr, s)
                                   : launch_transpose16(tr_b, nullptr, s);
    if (e != hipSuccess) return e;
    if (pl.copy_a) a.A = dst_a;
    if (pl.copy_b) a.B = dst_b;
    a.lda = pl.lda;
    a.ldb = pl.ldb;
  }
  switch (pl.path) {
    case GEMM_PATH_F16_GEMV: return launch_f16_gemv(a, epi, s);
    case GEMM_PATH_F16_SPLITK:
      a.sk = splitk_args(splitk_plan(a.M, a.N, a.K, kF16Slab, kF16Rule, 0), a.M, a.N,
                         ws + pl.bytes_a + pl.bytes_b);
      return launch_f16_splitk(a, epi, cus, s);
    case GEMM_PATH_F16_MFMA:
      return pl.lay ? launch_f16_kmajor(a, pl.lay, epi, cus, s) : launch_f16_mfma(a, epi, cus, s);
    case GEMM_PATH_F16_STAGED: return launch_f16_staged(a, epi, cus, s);
    default: return launch_f16_edge(a, epi, s);
  }
}

// The kernels of a plain fp32 path that is not a quick return.
hipError_t run32(int path, const F32Args& a, int cus, hipStream_t s) {
  switch (path) {
    case GEMM_PATH_F32_SCALE: return launch_f32_scale(a, s);
    case GEMM_PATH_F32_MFMA: return launch_f32_mfma(a, cus, s);
    default: return launch_f32_edge(a, cus, s);
  }
}

// The split count of an explicit split-K call: `splits` ranges if positive,
// else the automatic rule; 1 (no split) for products the split-K kernels do
// not serve (quick returns, the matrix-vector shapes).
SplitPlan f32_split(int path, int M, int N, int K, int splits) {
  if (path < 0 || path == GEMM_PATH_NOOP || path == GEMM_PATH_F32_SCALE) return SplitPlan{};
  return splitk_plan(M, N, K, kF32Slab, kF32Rule, splits);
}

SplitPlan f16_split(int path, int M, int N, int K, int splits) {
  if (path < 0 || path == GEMM_PATH_NOOP || path == GEMM_PATH_F16_ZERO) return SplitPlan{};
  if (splits <= 0 && f16_gemv_fits(M, N)) return SplitPlan{};
  return splitk_plan(M, N, K, kF16Slab, kF16Rule, splits);
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
  return to_status(run32(path, a, cus, static_cast<hipStream_t>(stream)));
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
  return to_status(run16(pl, a, GEMM_OP_N, GEMM_OP_T, false, cus, nullptr,
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
  return to_status(run16(pl, a, GEMM_OP_N, GEMM_OP_T, true, cus, nullptr,
                         static_cast<hipStream_t>(stream)));
}

MI355GEMM_API int gemm_ex(int type, int op_a, int op_b, int M, int N, int K, const void* A,
                          int lda, const void* B, int ldb, const void* bias, int act,
                          const void* residual, int ldr, void* C, int ldc, void* workspace,
                          unsigned long long workspace_bytes, void* stream) {
  Plan16 pl = plan16(type, op_a, op_b, M, N, K, A, lda, B, ldb, bias, act, residual, ldr, C, ldc,
                     true);
  if (pl.path < 0 || pl.path == GEMM_PATH_NOOP) return pl.path < 0 ? pl.path : GEMM_OK;
  // split-K only when the workspace holds its partial sums too
  if (pl.path == GEMM_PATH_F16_SPLITK && !workspace_ok(pl.workspace(), workspace, workspace_bytes))
    pl = plan16(type, op_a, op_b, M, N, K, A, lda, B, ldb, bias, act, residual, ldr, C, ldc);
  if (!workspace_ok(pl.workspace(), workspace, workspace_bytes)) return GEMM_ERR_WORKSPACE;
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
  return to_status(run16(pl, a, op_a, op_b, epi, cus, static_cast<char*>(workspace),
                         static_cast<hipStream_t>(stream)));
}

MI355GEMM_API unsigned long long gemm_ex_workspace(int type, int op_a, int op_b, int M, int N,
                                                   int K, int lda, int ldb) {
  // An upper bound for any pointers: aligned stand-ins, a packed C, and the
  // copies even where aligned NN / TT operands are read in place (those calls
  // use none of it).
  const Plan16 pl = plan16(type, op_a, op_b, M, N, K, kCopyAddress, lda, kCopyAddress, ldb,
                           nullptr, GEMM_ACT_NONE, nullptr, 0, kCopyAddress, N > 1 ? N : 1, true,
                           false);
  return pl.path < 0 ? 0 : pl.workspace();
}

MI355GEMM_API int gemm_f32_splitk(int M, int N, int K, float alpha, const float* A, int lda,
                                  const float* B, int ldb, float beta, float* C, int ldc,
                                  int splits, void* workspace, unsigned long long workspace_bytes,
                                  void* stream) {
  const int path = f32_select(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
  if (path < 0 || path == GEMM_PATH_NOOP) return path < 0 ? path : GEMM_OK;
  const SplitPlan plan = f32_split(path, M, N, K, splits);
  if (plan.splits > 1 && !workspace_ok(plan.bytes, workspace, workspace_bytes))
    return GEMM_ERR_WORKSPACE;
  const int cus = check_device();
  if (cus < 0) return cus;
  F32Args a{A, B, C, lda, ldb, ldc, M, N, K, alpha, beta};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.splits > 1) {
    a.sk = splitk_args(plan, M, N, workspace);
    return to_status(launch_f32_splitk(a, s));
  }
  return to_status(run32(path, a, cus, s));
}

MI355GEMM_API int gemm_f16_nt_splitk(int M, int N, int K, const void* A, int lda, const void* B,
                                     int ldb, void* C, int ldc, int splits, void* workspace,
                                     unsigned long long workspace_bytes, void* stream) {
  const Plan16 pl = plan16(GEMM_TYPE_F16, GEMM_OP_N, GEMM_OP_T, M, N, K, A, lda, B, ldb, nullptr,
                           GEMM_ACT_NONE, nullptr, 0, C, ldc);
  if (pl.path < 0 || pl.path == GEMM_PATH_NOOP) return pl.path < 0 ? pl.path : GEMM_OK;
  const SplitPlan plan = f16_split(pl.path, M, N, K, splits);
  if (plan.splits > 1 && !workspace_ok(plan.bytes, workspace, workspace_bytes))
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
  return to_status(run16(pl, a, GEMM_OP_N, GEMM_OP_T, false, cus, nullptr, s));
}

}  // extern "C"

// ---- gemm_f16_nt_splitk_static: the split-K call with library-held scratch.
//
// The partial sums live in `scratch`, a device array of fixed size in this
// library's code object (one copy per GPU, for the life of the process).  In
// host code the name `scratch` is only a stand-in for the symbol: the kernels
// get its device address, looked up once per device with
// hipGetSymbolAddress while that device is current and kept in
// g_scratch_addr.  The partial kernels store every element of every tile the
// reduction reads, so nothing has to be cleared between calls.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

std::mutex g_scratch_lock;
std::atomic<void*> g_scratch_addr[kMaxDevices];

// The device address of the current device's `scratch`, or nullptr if the
// runtime cannot give it.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  std::lock_guard<std::mutex> guard(g_scratch_lock);
  ptr = g_scratch_addr[dev].load(std::memory_order_relaxed);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_addr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

extern "C" {

MI355GEMM_API int gemm_f16_nt_splitk_static(int M, int N, int K, const void* A, int lda,
                                            const void* B, int ldb, void* C, int ldc, int splits,
                                            void* stream) {
  const Plan16 pl = plan16(GEMM_TYPE_F16, GEMM_OP_N, GEMM_OP_T, M, N, K, A, lda, B, ldb, nullptr,
                           GEMM_ACT_NONE, nullptr, 0, C, ldc);
  if (pl.path < 0 || pl.path == GEMM_PATH_NOOP) return pl.path < 0 ? pl.path : GEMM_OK;
  const SplitPlan plan = f16_split(pl.path, M, N, K, splits);
  if (plan.splits > 1 && plan.bytes > kStaticScratchBytes) return GEMM_ERR_SCRATCH_LIMIT;
  const int cus = check_device();
  if (cus < 0) return cus;
  Args16 a{static_cast<const half_t*>(A), static_cast<const half_t*>(B),
           static_cast<half_t*>(C), lda, ldb, ldc, M, N, K};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.splits > 1) {
    void* ws = scratch_address();
    if (ws == nullptr) return GEMM_ERR_LAUNCH;
    a.sk = splitk_args(plan, M, N, ws);
    return to_status(launch_f16_splitk(a, false, cus, s));
  }
  return to_status(run16(pl, a, GEMM_OP_N, GEMM_OP_T, false, cus, nullptr, s));
}

MI355GEMM_API unsigned long long gemm_f32_splitk_workspace(int M, int N, int K, int splits) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return f32_split(GEMM_PATH_F32_MFMA, M, N, K, splits).bytes;
}

MI355GEMM_API unsigned long long gemm_f16_nt_splitk_workspace(int M, int N, int K, int splits) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return f16_split(GEMM_PATH_F16_MFMA, M, N, K, splits).bytes;
}

MI355GEMM_API int gemm_f32_path(int M, int N, int K, float alpha, const float* A, int lda,
                                const float* B, int ldb, float beta, const float* C, int ldc) {
  return f32_select(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
}

MI355GEMM_API int gemm_f16_nt_path(int M, int N, int K, const void* A, int lda, const void* B,
                                   int ldb, const void* C, int ldc) {
  return plan16(GEMM_TYPE_F16, GEMM_OP_N, GEMM_OP_T, M, N, K, A, lda, B, ldb, nullptr,
                GEMM_ACT_NONE, nullptr, 0, C, ldc)
      .path;
}

MI355GEMM_API int gemm_f16_nt_ex_path(int M, int N, int K, const void* A, int lda, const void* B,
                                      int ldb, const void* bias, int act, const void* residual,
                                      int ldr, const void* C, int ldc) {
  return plan16(GEMM_TYPE_F16, GEMM_OP_N, GEMM_OP_T, M, N, K, A, lda, B, ldb, bias, act, residual,
                ldr, C, ldc)
      .path;
}

MI355GEMM_API int gemm_ex_path(int type, int op_a, int op_b, int M, int N, int K, const void* A,
                               int lda, const void* B, int ldb, const void* bias, int act,
                               const void* residual, int ldr, const void* C, int ldc) {
  return plan16(type, op_a, op_b, M, N, K, A, lda, B, ldb, bias, act, residual, ldr, C, ldc, true)
      .path;
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
      return "the call needs a workspace and the one given is NULL, smaller than the size "
             "query reports, or not 16-byte aligned";
    case GEMM_ERR_SCRATCH_LIMIT:
      return "the split-K partial sums would exceed the library's static scratch area "
             "(GEMM_STATIC_SCRATCH_BYTES, 32 MiB); use fewer splits or gemm_f16_nt_splitk "
             "with a workspace";
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
    case GEMM_PATH_F16_STAGED: return "f16_staged";
    case GEMM_PATH_F16_SPLITK: return "f16_splitk";
    default: return "?";
  }
}

}  // extern "C"
