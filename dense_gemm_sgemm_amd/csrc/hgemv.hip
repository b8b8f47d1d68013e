// 16-bit (fp16 or bf16) C = A * B^T when M or N is at most 8: the
// matrix-vector case of decode steps (page "第 6 章 Shared Memory & Tile",
// section 6.5.5).
//
// With M <= 8 each output is C[v][r] = dot(B row r, A row v); with N <= 8 it
// is C[r][v] = dot(A row r, B row v).  Either way one long operand W (B or A)
// is streamed from HBM once, row by row, and V <= 8 short rows X (the other
// operand) are re-read from cache.  A tile of a tiled kernel would be almost
// empty here and the matrix cores idle; the bound is HBM bandwidth for W, so
// the kernel keeps as many W bytes in flight as it can and does its
// arithmetic with v_dot2_f32_f16 / v_dot2_f32_bf16 (two products added into
// an fp32 accumulator):
//
//  * a row group is 4 rows of W and TPR threads (one wave, or the whole
//    workgroup of 4 waves for long rows); thread t of the group takes the
//    chunks of 8 halves t, t + TPR, t + 2 TPR, ... of all 4 rows and of the
//    V vectors, U chunks per row at a time so that 4 U 16-byte loads are in
//    flight per thread before the first product;
//  * rows and vectors may start at any 2-byte address: the 16-byte loads
//    carry only the data's alignment (the target runs with unaligned access
//    enabled) and the K % 8 tail is read element by element;
//  * the 4 V fp32 partial sums of a thread are reduced across the wave by a
//    halving exchange (each step sends half of the remaining sums to the
//    partner lane and keeps the other half), across the waves of a group
//    through LDS, in a fixed order, so results do not vary from run to run;
//  * the EPI instance applies the fused write-back act(acc + bias) +
//    residual before the rounding to half.
#include "internal.h"

namespace mi355gemm {
namespace hgemv {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kRows = 4;       // rows of W per row group
constexpr int kThreads = 256;  // threads per workgroup
constexpr int kMaxV = 8;       // vectors per call

// One GEMV problem: Y[r * y_r + v * y_v] = sum_k W[r * ldw + k] X[v * ldx + k]
// for r < R, v < V (V is the kernel's template argument).  The write-back
// reads bias[r * b_r + v * b_v] and res[r * res_r + v * res_v].
struct GemvArgs {
  const half_t* W;
  const half_t* X;
  half_t* Y;
  int64_t ldw, ldx, y_r, y_v;
  const half_t* bias;
  int64_t b_r, b_v;
  const half_t* res;
  int64_t res_r, res_v;
  int R, K, act;
};

constexpr int pow2_at_least(int n) { return n <= 1 ? 1 : 2 * pow2_at_least((n + 1) / 2); }

// 16 bytes at byte offset `off` of a wave-uniform row base: the uniform base
// stays in scalar registers and each lane supplies a 32-bit offset.
__device__ __forceinline__ h8 load8(const char* base, uint32_t off) {
  h8 v;
  __builtin_memcpy(&v, base + off, 16);
  return v;
}

// The first n (1 <= n < 8) halves at byte offset `off`, zero after them.  The
// loads stay inside the n elements.
__device__ __forceinline__ h8 load_part(const char* base, uint32_t off, int n) {
  const half_t* p = reinterpret_cast<const half_t*>(base + off);
  h8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const half_t x = p[e < n ? e : n - 1];
    v[e] = e < n ? x : (half_t)0;
  }
  return v;
}

typedef __bf16 bh2 __attribute__((ext_vector_type(2)));
typedef __bf16 bh8 __attribute__((ext_vector_type(8)));

// acc + the dot product of 8 16-bit words of format FMT, two products at a
// time into the fp32 accumulator (v_dot2_f32_f16 / v_dot2_f32_bf16).
template <int FMT>
__device__ __forceinline__ float dot8(h8 w, h8 x, float acc) {
  if constexpr (FMT == kFmtF16) {
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      acc = __builtin_amdgcn_fdot2(h2{w[e], w[e + 1]}, h2{x[e], x[e + 1]}, acc, false);
  } else {
    const bh8 wb = __builtin_bit_cast(bh8, w), xb = __builtin_bit_cast(bh8, x);
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      acc = __builtin_amdgcn_fdot2_f32_bf16(bh2{wb[e], wb[e + 1]}, bh2{xb[e], xb[e + 1]}, acc,
                                            false);
  }
  return acc;
}

// Sums a[0..P) over the 64 lanes of the wave.  On return lane l holds the
// total of index l / (64 / P).  The first log2(P) steps halve the number of
// live sums: with partner l ^ m, the lane whose bit m is set keeps the upper
// half and sends the lower one; the remaining steps add the single sum
// across the lanes that share an index.
template <int P>
__device__ __forceinline__ float wave_reduce(float (&a)[P], int lane) {
#pragma unroll
  for (int h = P / 2, m = 32; h >= 1; h /= 2, m /= 2) {
    // A bit mask rather than a select of two array elements, which the
    // compiler would turn into a dynamically indexed (scratch) array.
    const uint32_t up = (lane & m) != 0 ? 0xffffffffu : 0u;
#pragma unroll
    for (int j = 0; j < h; ++j) {
      const uint32_t lo = __float_as_uint(a[j]), hi = __float_as_uint(a[j + h]);
      const float send = __uint_as_float((lo & up) | (hi & ~up));
      const float keep = __uint_as_float((hi & up) | (lo & ~up));
      a[j] = keep + __shfl_xor(send, m);
    }
  }
  float s = a[0];
#pragma unroll
  for (int m = 32 / P; m >= 1; m /= 2) s += __shfl_xor(s, m);
  return s;
}

// U chunk steps of one thread: every load is issued before the first
// product, so that 4 U + V U loads are in flight at once.
template <int U, int V, int FMT>
__device__ __forceinline__ void chunk_steps(const char* const (&w)[kRows],
                                            const char* const (&x)[V], uint32_t off,
                                            uint32_t stride, float* acc) {
  h8 wv[U][kRows], xv[U][V];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) wv[u][r] = load8(w[r], off + u * stride);
#pragma unroll
    for (int v = 0; v < V; ++v) xv[u][v] = load8(x[v], off + u * stride);
  }
  // Keeps the scheduler from sinking the loads next to their first use.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int v = 0; v < V; ++v) acc[r * V + v] = dot8<FMT>(wv[u][r], xv[u][v], acc[r * V + v]);
}

template <int V, int TPR, int U, bool EPI, int FMT>
__global__ __launch_bounds__(kThreads) void hgemv_kernel(GemvArgs p, int64_t wg_base) {
  constexpr int kRV = kRows * V;
  constexpr int P = pow2_at_least(kRV);
  constexpr int kGroups = kThreads / TPR;
  constexpr int kWavesPerGroup = TPR / 64;
  __shared__ float red[kThreads / 64][P];

  const int tid = threadIdx.x, lane = tid & 63;
  const int t = tid % TPR;
  const int group = __builtin_amdgcn_readfirstlane(tid / TPR);
  const int64_t r0 = ((wg_base + blockIdx.x) * kGroups + group) * kRows;

  // Rows past R read row R - 1 (their results are dropped) so that every load
  // stays unconditional.
  const char* w[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int64_t row = r0 + r < p.R ? r0 + r : p.R - 1;
    w[r] = reinterpret_cast<const char*>(p.W + row * p.ldw);
  }
  const char* x[V];
#pragma unroll
  for (int v = 0; v < V; ++v) x[v] = reinterpret_cast<const char*>(p.X + v * p.ldx);

  float acc[P];
#pragma unroll
  for (int i = 0; i < P; ++i) acc[i] = 0.f;

  const int Kc = p.K >> 3;      // whole chunks per row
  const int nfull = Kc / TPR;   // chunk steps in which every thread has a chunk
  // Byte offsets fit in 32 bits: a row holds fewer than 2^31 halves.
  uint32_t off = 16u * t;
  constexpr uint32_t kStride = 16u * TPR;
  int i = 0;
  for (; i + U <= nfull; i += U, off += U * kStride) chunk_steps<U, V, FMT>(w, x, off, kStride, acc);
  for (; i < nfull; ++i, off += kStride) chunk_steps<1, V, FMT>(w, x, off, kStride, acc);
  // The last, partial chunk step: whole chunks below Kc, then the thread
  // whose next chunk is Kc takes the K % 8 tail.
  const int c = t + nfull * TPR;
  const int tail = p.K & 7;
  if (c < Kc) {
    chunk_steps<1, V, FMT>(w, x, off, kStride, acc);
  } else if (c == Kc && tail != 0) {
    h8 wv[kRows], xv[V];
#pragma unroll
    for (int r = 0; r < kRows; ++r) wv[r] = load_part(w[r], off, tail);
#pragma unroll
    for (int v = 0; v < V; ++v) xv[v] = load_part(x[v], off, tail);
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int v = 0; v < V; ++v) acc[r * V + v] = dot8<FMT>(wv[r], xv[v], acc[r * V + v]);
  }

  float s = wave_reduce<P>(acc, lane);
  const int idx = lane / (64 / P);
  const bool owner = (lane % (64 / P)) == 0 && idx < kRV;
  if constexpr (kWavesPerGroup > 1) {
    if (owner) red[tid >> 6][idx] = s;
    __syncthreads();
    if (t >= kRV) return;
    // The group's waves in order, so the sum order is fixed.
    const int w0 = group * kWavesPerGroup;
    s = red[w0][t];
#pragma unroll
    for (int q = 1; q < kWavesPerGroup; ++q) s += red[w0 + q][t];
  } else {
    if (!owner) return;
  }
  const int o = kWavesPerGroup > 1 ? t : idx;
  const int r = o / V, v = o % V;
  const int64_t row = r0 + r;
  if (row >= p.R) return;
  if constexpr (EPI) {
    if (p.bias) s += word_to_f32<FMT>(p.bias[row * p.b_r + v * p.b_v]);
    s = epi_act(s, p.act);
    if (p.res) s += word_to_f32<FMT>(p.res[row * p.res_r + v * p.res_v]);
  }
  p.Y[row * p.y_r + v * p.y_v] = f32_to_word<FMT>(s);
}

typedef void (*KernelFn)(GemvArgs, int64_t);

template <int TPR, int U, bool EPI, int FMT>
KernelFn pick_v(int V) {
  switch (V) {
    case 1: return hgemv_kernel<1, TPR, U, EPI, FMT>;
    case 2: return hgemv_kernel<2, TPR, U, EPI, FMT>;
    case 3: return hgemv_kernel<3, TPR, U, EPI, FMT>;
    case 4: return hgemv_kernel<4, TPR, U, EPI, FMT>;
    case 5: return hgemv_kernel<5, TPR, U, EPI, FMT>;
    case 6: return hgemv_kernel<6, TPR, U, EPI, FMT>;
    case 7: return hgemv_kernel<7, TPR, U, EPI, FMT>;
    default: return hgemv_kernel<8, TPR, U, EPI, FMT>;
  }
}

// Rows of K >= 2048 go to a whole workgroup per row group, with four chunk
// steps in flight for very long rows and one or two vectors; shorter rows to
// one wave per row group.
template <bool EPI, int FMT>
KernelFn pick(int V, int kc, bool& wide) {
  wide = kc >= kThreads;
  if (!wide) return pick_v<64, 2, EPI, FMT>(V);
  if (V <= 2 && kc >= 4 * kThreads)
    return V == 1 ? hgemv_kernel<1, kThreads, 4, EPI, FMT> : hgemv_kernel<2, kThreads, 4, EPI, FMT>;
  return pick_v<kThreads, 2, EPI, FMT>(V);
}

}  // namespace hgemv

bool f16_gemv_fits(int M, int N) { return M <= hgemv::kMaxV || N <= hgemv::kMaxV; }

hipError_t launch_f16_gemv(const Args16& a, bool epi, hipStream_t stream) {
  using namespace hgemv;
  GemvArgs g;
  int V;
  if (a.M <= kMaxV && a.M <= a.N) {
    // C[v][r] = dot(B row r, A row v): the bias follows r, the residual row v.
    g = GemvArgs{a.B, a.A, a.C, a.ldb, a.lda, 1, a.ldc, a.bias, 1, 0, a.res, 1, a.ldr,
                 a.N, a.K, a.act};
    V = a.M;
  } else {
    // C[r][v] = dot(A row r, B row v): the bias follows v, the residual row r.
    g = GemvArgs{a.A, a.B, a.C, a.lda, a.ldb, a.ldc, 1, a.bias, 0, 1, a.res, a.ldr, 1,
                 a.M, a.K, a.act};
    V = a.N;
  }
  const int64_t groups = (g.R + kRows - 1) / kRows;
  // Measured on MI355X: rows of K >= 2048 are split over a whole workgroup
  // (1 x 16384 x 4096: 19.5 us against 22.2 us with one wave per row group),
  // shorter ones over one wave, four row groups per workgroup (K = 768:
  // 4.1 us against 5.7 us).  Very long rows with one or two vectors keep four
  // chunk steps in flight (K = 16384: 83 us against 87 us).
  const int kc = a.K >> 3;
  bool wide = false;
  KernelFn fn;
  if (a.fmt == kFmtBF16)
    fn = epi ? pick<true, kFmtBF16>(V, kc, wide) : pick<false, kFmtBF16>(V, kc, wide);
  else
    fn = epi ? pick<true, kFmtF16>(V, kc, wide) : pick<false, kFmtF16>(V, kc, wide);
  const int tpr = wide ? kThreads : 64;
  const int64_t per_wg = kThreads / tpr;
  const int64_t wgs = (groups + per_wg - 1) / per_wg;
  return launch_tiles(reinterpret_cast<const void*>(fn), g, wgs, kThreads, 0, stream);
}

}  // namespace mi355gemm
