// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mi355gemm.h"

namespace mi355gemm {

typedef _Float16 half_t;

// Split-K: the K slabs of a product are cut into `splits` ranges of `per`
// slabs; the partial product of range s over output tile (tm, tn) goes to
// ws[s * split_stride + m * ld + n] (fp32, the workspace padded to whole
// tiles), and a second kernel adds the ranges in order s = 0, 1, ... .
struct SplitK {
  float* ws = nullptr;
  int64_t ld = 0, split_stride = 0;
  int splits = 1, per = 0;
};

// Arguments of one fp32 call, as validated by the C-ABI layer.
struct F32Args {
  const float* A;
  const float* B;
  float* C;
  int64_t lda, ldb, ldc;
  int M, N, K;
  float alpha, beta;
  SplitK sk;                      // split-K partial products (partial kernels only)
};

// 16-bit storage formats.  Kernels move both as 16-bit words (half_t
// pointers) and convert through word_to_f32 / f32_to_word.
enum { kFmtF16 = 0, kFmtBF16 = 1 };
typedef __bf16 bf16_t;

// Arguments of one 16-bit A*B^T call (A, B, C, bias and residual all in
// format `fmt`).  bias .. act describe the fused write-back
// C = act(A*B^T + bias) + residual; kernels instantiated without it ignore
// them.
struct Args16 {
  const half_t* A;
  const half_t* B;
  half_t* C;
  int64_t lda, ldb, ldc;
  int M, N, K;
  const half_t* bias = nullptr;   // [N] or null
  const half_t* res = nullptr;    // [M][ldr] or null
  int64_t ldr = 0;
  int act = 0;                    // 0 none, 1 ReLU, 2 SiLU
  SplitK sk;                      // split-K partial products (partial kernels only)
  int fmt = kFmtF16;              // storage format of every 16-bit operand
};

// A 16-bit storage word as fp32, and fp32 rounded to a storage word (nearest,
// ties to even; bfloat16 through the hardware conversion).
template <int FMT>
__device__ __forceinline__ float word_to_f32(half_t w) {
  if constexpr (FMT == kFmtF16) {
    return (float)w;
  } else {
    return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, w) << 16);
  }
}

template <int FMT>
__device__ __forceinline__ half_t f32_to_word(float x) {
  if constexpr (FMT == kFmtF16) {
    return (half_t)x;
  } else {
    return __builtin_bit_cast(half_t, (bf16_t)x);
  }
}

// The fused write-back's activations on an fp32 value.  SiLU x / (1 + e^-x)
// takes the hardware exponential and reciprocal (each within a few fp32 ulps;
// x = -inf gives NaN, as the quotient does).
__device__ __forceinline__ float epi_relu(float x) { return x > 0.f ? x : 0.f; }
__device__ __forceinline__ float epi_silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
}
__device__ __forceinline__ float epi_act(float x, int act) {
  if (act == GEMM_ACT_RELU) return epi_relu(x);
  if (act == GEMM_ACT_SILU) return epi_silu(x);
  return x;
}

// A split-K decision: `splits` K ranges of `per` slabs each and the workspace
// bytes they need; splits == 1 means no split.
struct SplitPlan {
  int splits = 1, per = 0;
  size_t bytes = 0;
};
// The library's choice of a split count: ranges = workgroup budget / tiles
// (tiles of 128 x 128), capped at K / min_range and 64, rounded down to a
// power of two if asked; no split below min_splits ranges.
struct SplitRule {
  int min_range, max_workgroups, min_splits;
  bool power_of_two;
};
// For an M x N x K product walked in slabs of `slab`: `requested` ranges if
// positive (at most one per slab), else the rule's choice.
SplitPlan splitk_plan(int M, int N, int K, int slab, const SplitRule& rule, int requested);
SplitK splitk_args(const SplitPlan& plan, int M, int N, void* workspace);

// Launchers.  Each enqueues its kernel(s) on `stream` and returns the HIP
// runtime's verdict on the launch.
hipError_t launch_f32_scale(const F32Args& a, hipStream_t stream);
hipError_t launch_f32_edge(const F32Args& a, int cus, hipStream_t stream);
hipError_t launch_f32_mfma(const F32Args& a, int cus, hipStream_t stream);
hipError_t launch_f16_zero(const Args16& a, hipStream_t stream);
hipError_t launch_f16_edge(const Args16& a, bool epi, hipStream_t stream);
hipError_t launch_f16_mfma(const Args16& a, bool epi, int cus, hipStream_t stream);
hipError_t launch_f16_gemv(const Args16& a, bool epi, hipStream_t stream);
// The matrix-vector case with the long operand stored K-major (B for
// op_b = N when M is the small side, A for op_a = T when N is): partial sums
// over ranges of K into an fp32 workspace, then the split-K reduction with
// the call's write-back.  gemv_kn_plan gives the ranges and workspace bytes.
SplitPlan gemv_kn_plan(int M, int N, int K);
hipError_t launch_f16_gemv_kn(const Args16& a, int op_a, int op_b, bool epi, const SplitPlan& plan,
                              void* workspace, hipStream_t stream);
// The split-K reduction alone: a.sk names the partial sums.
hipError_t launch_f16_reduce(const Args16& a, bool epi, hipStream_t stream);
// A transposition: dst[c * ldd + r] = src[r * lds + c] for the rows x cols
// source; the destination's rows_p x cols_p extent (source orientation) is
// written, zero outside the source (dst 16-byte aligned, ldd a multiple of
// 8).  launch_transpose16 runs one or two of them in one launch.
struct PadCopy {
  const half_t* src;
  half_t* dst;
  int64_t lds, ldd;
  int rows, cols, rows_p, cols_p;
};
hipError_t launch_transpose16(const PadCopy& first, const PadCopy* second, hipStream_t stream);
// The register-staged wide-tile kernel for A * B^T: any shape (K >= 8),
// leading dimension (below 2^23) and 2-byte alignment, no copies, no
// workspace.
bool f16_staged_fits(int M, int N, int K, int64_t lda, int64_t ldb);
// Few output tiles (at most as many 64 x 64 tiles as CUs) and K a multiple of
// 128 (no fused write-back): 32 x 32 or 16 x 16 tiles with K split across the
// four waves of a workgroup.
bool f16_small_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                    const void* C, int64_t ldc, int cus);
hipError_t launch_f16_small(const Args16& a, int cus, hipStream_t stream);
// The full-tile kernels' ragged form: any M, N >= 128, K > 64 with K % 8 ==
// 0, A and B rows at 16-byte addresses, C anywhere.
bool f16_ragged_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb);
hipError_t launch_f16_staged(const Args16& a, bool epi, int cus, hipStream_t stream);
// The full-tile kernels with K-major operands read in place: lay 1, B
// stored [K][N] (gemm_ex NN); lay 2, A stored [K][M] (gemm_ex TT); lay 3,
// both (gemm_ex TN).  Tiles of 256 x 256 (NN, TT), 224 x 256 (NN) or
// 256 x 224 (TT, TN), 128 x 128 or 128 x 192, where they cost no more than
// the A * B^T tiles on transposed copies: whole tiles with K % 64 == 0 (C
// 16-byte aligned, ldc % 8 == 0), or the ragged form for products of at
// least 2^30 multiply-adds at least 128 wide and tall (C anywhere; K > 64,
// and K % 8 == 0 unless both operands are K-major); A and B 16-byte
// aligned, lda and ldb multiples of 8 (below 2^28).
bool f16_kmajor_fits(int lay, int M, int N, int K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, const void* C, int64_t ldc);
hipError_t launch_f16_kmajor(const Args16& a, int lay, bool epi, int cus, hipStream_t stream);
// Split-K: the partial products (a.sk filled in), then the reduction.
hipError_t launch_f16_partials(const Args16& a, hipStream_t stream);
hipError_t launch_f32_partials(const F32Args& a, hipStream_t stream);
hipError_t launch_f16_splitk(const Args16& a, bool epi, int cus, hipStream_t stream);
// The fast partial-product kernel, and when it applies.
bool f16_partials_fit(const Args16& a);
hipError_t launch_f16_partials_mfma(const Args16& a, int cus, hipStream_t stream);
hipError_t launch_f32_splitk(const F32Args& a, hipStream_t stream);

// Shape and alignment conditions of the fast kernels (checked on the host).
bool f32_mfma_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                   const void* C, int64_t ldc);
// The fp32 streaming kernels apply in place (full tiles, K a multiple of 64,
// leading dimensions within their 32-bit lane offsets).
bool f32_stream_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                     const void* C, int64_t ldc);
// Alignment conditions of the fast kernel's fused write-back.
bool f16_epi_fits(const void* bias, const void* res, int64_t ldr);
bool f16_mfma_fits(int M, int N, int K, const void* A, int64_t lda, const void* B, int64_t ldb,
                   const void* C, int64_t ldc);
// M or N small enough for the matrix-vector kernel.
bool f16_gemv_fits(int M, int N);
// Which operand the matrix-vector kernels stream: B when M is the small side
// (M <= 8 and M <= N), else A.
bool f16_gemv_w_is_b(int M, int N);

// Launches `kernel(args, tile_base)` over `tiles` workgroups, split into
// launches of at most 2^20 workgroups so that no grid exceeds the 32-bit
// work-item count of a dispatch.  Workgroup b of a launch handles tile
// tile_base + b.
template <typename Args>
hipError_t launch_tiles(const void* kernel, const Args& a, int64_t tiles, int threads,
                        unsigned lds_bytes, hipStream_t stream) {
  constexpr int64_t kMaxBlocks = int64_t(1) << 20;
  for (int64_t base = 0; base < tiles; base += kMaxBlocks) {
    const int64_t n = (tiles - base < kMaxBlocks) ? tiles - base : kMaxBlocks;
    Args p = a;
    int64_t b = base;
    void* args[] = {&p, &b};
    const hipError_t e =
        hipLaunchKernel(kernel, dim3((unsigned)n), dim3(threads), args, lds_bytes, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace mi355gemm
