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


// ---------------------------------------------------------------------------
// The long operand stored K-major: W[k][l] with each row (one k) contiguous in
// l, as B is for op_b = N (l = n) and A for op_a = T (l = m).  Then
// Y[v][l] = sum_k X[v][k] W[k][l], and a thread's neighbours in a row hold
// different outputs, so the kernel walks W row by row instead of along K:
//
//  * each lane owns 8 consecutive columns; the workgroups are spread over
//    column blocks and over ranges of `per` rows of K, so that every row of W
//    is read once and enough loads are in flight to stream it from HBM (see
//    kn_wg_cols for how the four waves of a workgroup divide the work);
//  * each 16-byte load brings 8 columns of one row; two rows k, k + 1 are
//    paired column by column into v_dot2 operands (W[k][l], W[k+1][l]) and
//    multiplied with (X[v][k], X[v][k+1]), staged in LDS in that packed form
//    (X may be stored in either layout: it is read with both strides);
//  * each range writes its fp32 partial sums to a workspace laid out as the
//    split-K partials, [range][M][round4(N)], and the split-K reduction adds
//    the ranges in order and applies the write-back.
struct KnArgs {
  const half_t* W;
  const half_t* X;
  float* ws;
  int64_t ldw, x_v, x_k;
  int64_t ws_s, ws_v, ws_l;   // partial (range s, v, l) at ws[s ws_s + v ws_v + l ws_l]
  int L, K, per, colblocks;
};

constexpr int kKnCols = 8;                     // columns per thread
constexpr int kKnMaxPer = 1024;                // rows of K per range (X staging in LDS)

// Columns l .. l + 7 of one row, zero past L.
__device__ __forceinline__ h8 load_cols(const half_t* row, int64_t l, int L) {
  h8 v;
  if (l + kKnCols <= L) {
    __builtin_memcpy(&v, row + l, 16);
  } else {
#pragma unroll
    for (int e = 0; e < kKnCols; ++e) v[e] = l + e < L ? row[l + e] : (half_t)0;
  }
  return v;
}

__device__ __forceinline__ uint32_t word_bits(half_t h) {
  return __builtin_bit_cast(uint16_t, h);
}

// acc + w.lo * x.lo + w.hi * x.hi, both operands two 16-bit words of format FMT.
template <int FMT>
__device__ __forceinline__ float dot2w(uint32_t w, uint32_t x, float acc) {
  if constexpr (FMT == kFmtF16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), __builtin_bit_cast(h2, x), acc,
                                  false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bh2, w), __builtin_bit_cast(bh2, x),
                                           acc, false);
}

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Rows k (w0) and k + 1 (w1) of the thread's 8 columns into the accumulators;
// xp[v] = (X[v][k], X[v][k+1]).
template <int V, int FMT>
__device__ __forceinline__ void kn_pair(h8 w0, h8 w1, const uint32_t* xp, float (&acc)[V][kKnCols]) {
  const u4 a = __builtin_bit_cast(u4, w0), b = __builtin_bit_cast(u4, w1);
  uint32_t pr[kKnCols];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pr[2 * j] = (a[j] & 0xffffu) | (b[j] << 16);            // column 2j: (W[k], W[k+1])
    pr[2 * j + 1] = (a[j] >> 16) | (b[j] & 0xffff0000u);     // column 2j + 1
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const uint32_t x = xp[v];
#pragma unroll
    for (int e = 0; e < kKnCols; ++e) acc[v][e] = dot2w<FMT>(pr[e], x, acc[v][e]);
  }
}

// Columns a workgroup of the K-major kernel owns: with one or two vectors its
// four waves share 512 columns and take every fourth row pair of the range
// (their sums meet in LDS); with more, each wave owns 512 columns of its own
// and walks the whole range (an LDS exchange of 8 V sums per lane would cost
// more than it saves).
constexpr int kn_wg_cols(int V) { return V <= 2 ? 64 * kKnCols : kThreads * kKnCols; }

// U row pairs (2 U 16-byte loads) in flight per thread; sums of the waves
// that share columns are added in wave order.
template <int V, int U, int FMT>
__global__ __launch_bounds__(kThreads) void hgemv_kn_kernel(KnArgs p, int64_t base) {
  constexpr int kWaves = kThreads / 64;
  constexpr bool kShare = V <= 2;            // the waves share their columns
  constexpr int kStep = kShare ? kWaves : 1;  // row-pair stride of one wave
  __shared__ uint32_t xs[kKnMaxPer / 2][V];
  __shared__ float red[kShare ? kWaves - 1 : 1][V][64 * kKnCols];
  const int64_t b = base + blockIdx.x;
  const int s = (int)(b / p.colblocks), cb = (int)(b % p.colblocks);
  const int k0 = s * p.per;
  const int k1 = p.K < k0 + p.per ? p.K : k0 + p.per;
  const int rows = k1 - k0;   // at least 1
  const int pairs = (rows + 1) / 2;
  for (int i = threadIdx.x; i < pairs * V; i += kThreads) {
    const int kp = i / V, v = i % V;
    const int k = k0 + 2 * kp;
    const half_t* x = p.X + v * p.x_v;
    const uint32_t lo = word_bits(x[(int64_t)k * p.x_k]);
    const uint32_t hi = k + 1 < k1 ? word_bits(x[(int64_t)(k + 1) * p.x_k]) : 0u;
    xs[kp][v] = lo | (hi << 16);
  }
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t l =
      (int64_t)cb * kn_wg_cols(V) + (kShare ? lane : (int)threadIdx.x) * (int64_t)kKnCols;
  // Lanes past L load nothing but still reach the barrier below.
  const bool active = l < p.L;

  float acc[V][kKnCols];
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int e = 0; e < kKnCols; ++e) acc[v][e] = 0.f;
  const half_t* w = p.W + (int64_t)k0 * p.ldw;
  const int full = rows / 2;         // pairs whose two rows are both in the range
  const int first = kShare ? wave : 0;
  if (active) {
    int j = first;
    for (; j + kStep * (U - 1) < full; j += kStep * U) {
      h8 w0[U], w1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kp = j + kStep * u;
        w0[u] = load_cols(w + (int64_t)(2 * kp) * p.ldw, l, p.L);
        w1[u] = load_cols(w + (int64_t)(2 * kp + 1) * p.ldw, l, p.L);
      }
      // Keeps the scheduler from sinking the loads next to their first use.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) kn_pair<V, FMT>(w0[u], w1[u], xs[j + kStep * u], acc);
    }
    for (; j < full; j += kStep)
      kn_pair<V, FMT>(load_cols(w + (int64_t)(2 * j) * p.ldw, l, p.L),
                      load_cols(w + (int64_t)(2 * j + 1) * p.ldw, l, p.L), xs[j], acc);
    if ((rows & 1) && full % kStep == first)   // the range's last row alone
      kn_pair<V, FMT>(load_cols(w + (int64_t)(2 * full) * p.ldw, l, p.L), h8{}, xs[full], acc);
  }
  if constexpr (kShare) {
    if (wave > 0) {
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int e = 0; e < kKnCols; ++e) red[wave - 1][v][lane * kKnCols + e] = acc[v][e];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int q = 0; q < kWaves - 1; ++q)
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int e = 0; e < kKnCols; ++e) acc[v][e] += red[q][v][lane * kKnCols + e];
  }
  if (!active) return;
  float* dst = p.ws + s * p.ws_s + l * p.ws_l;
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int e = 0; e < kKnCols; ++e)
      if (l + e < p.L) dst[v * p.ws_v + e * p.ws_l] = acc[v][e];
}

typedef void (*KnKernelFn)(KnArgs, int64_t);

template <int FMT>
KnKernelFn pick_kn(int V) {
  switch (V) {
    case 1: return hgemv_kn_kernel<1, 8, FMT>;
    case 2: return hgemv_kn_kernel<2, 8, FMT>;
    case 3: return hgemv_kn_kernel<3, 8, FMT>;
    case 4: return hgemv_kn_kernel<4, 8, FMT>;
    case 5: return hgemv_kn_kernel<5, 4, FMT>;
    case 6: return hgemv_kn_kernel<6, 4, FMT>;
    case 7: return hgemv_kn_kernel<7, 4, FMT>;
    default: return hgemv_kn_kernel<8, 4, FMT>;
  }
}

// The small side and the long one: B is W when M is the small side.
inline bool w_is_b(int M, int N) { return M <= kMaxV && M <= N; }

}  // namespace hgemv

bool f16_gemv_fits(int M, int N) { return M <= hgemv::kMaxV || N <= hgemv::kMaxV; }
bool f16_gemv_w_is_b(int M, int N) { return hgemv::w_is_b(M, N); }

// Ranges of K for the K-major kernel: about 2048 workgroups in all, at most
// 256 ranges of at least 16 and at most kKnMaxPer rows (an even number), and
// partial sums of at most an eighth of W's bytes (S V L 4 <= K L 2 / 8).
SplitPlan gemv_kn_plan(int M, int N, int K) {
  using namespace hgemv;
  SplitPlan plan;
  const bool wb = w_is_b(M, N);
  const int L = wb ? N : M, V = wb ? M : N;
  const int64_t colblocks = ((int64_t)L + kn_wg_cols(V) - 1) / kn_wg_cols(V);
  int64_t s = 2048 / colblocks;
  if (s > (int64_t)K / (16 * V)) s = (int64_t)K / (16 * V);
  if (s < 1) s = 1;
  if (s > 256) s = 256;
  int64_t per = ((int64_t)K + s - 1) / s;
  per = (per + 1) / 2 * 2;
  if (per < 16) per = 16;
  if (per > kKnMaxPer) per = kKnMaxPer;
  plan.splits = (int)(((int64_t)K + per - 1) / per);
  plan.per = (int)per;
  plan.bytes = (size_t)plan.splits * M * ((N + 3) / 4 * 4) * 4;
  return plan;
}

hipError_t launch_f16_gemv_kn(const Args16& a, int op_a, int op_b, bool epi, const SplitPlan& plan,
                              void* workspace, hipStream_t stream) {
  using namespace hgemv;
  const bool wb = w_is_b(a.M, a.N);
  const int V = wb ? a.M : a.N;
  const int64_t ld = (a.N + 3) / 4 * 4;
  KnArgs k;
  k.ws = static_cast<float*>(workspace);
  k.ws_s = (int64_t)a.M * ld;
  k.K = a.K;
  k.per = plan.per;
  if (wb) {
    // W = B stored [K][ldb] (op_b = N); X = A; partial (v = m, l = n).
    k.W = a.B;
    k.ldw = a.ldb;
    k.X = a.A;
    k.x_v = op_a == GEMM_OP_N ? a.lda : 1;
    k.x_k = op_a == GEMM_OP_N ? 1 : a.lda;
    k.L = a.N;
    k.ws_v = ld;
    k.ws_l = 1;
  } else {
    // W = A stored [K][lda] (op_a = T); X = B; partial (v = n, l = m).
    k.W = a.A;
    k.ldw = a.lda;
    k.X = a.B;
    k.x_v = op_b == GEMM_OP_T ? a.ldb : 1;
    k.x_k = op_b == GEMM_OP_T ? 1 : a.ldb;
    k.L = a.M;
    k.ws_v = 1;
    k.ws_l = ld;
  }
  k.colblocks = (k.L + kn_wg_cols(V) - 1) / kn_wg_cols(V);
  const KnKernelFn fn = a.fmt == kFmtBF16 ? pick_kn<kFmtBF16>(V) : pick_kn<kFmtF16>(V);
  hipError_t e = launch_tiles(reinterpret_cast<const void*>(fn), k,
                              (int64_t)k.colblocks * plan.splits, kThreads, 0, stream);
  if (e != hipSuccess) return e;
  Args16 r = a;
  r.sk.ws = k.ws;
  r.sk.ld = ld;
  r.sk.split_stride = k.ws_s;
  r.sk.splits = plan.splits;
  r.sk.per = plan.per;
  return launch_f16_reduce(r, epi, stream);
}

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
