// Split-K (page "第 6 章 Shared Memory & Tile", section 6.5.6): when an
// M x N x K product has too few output tiles to occupy the GPU and K is long,
// K is cut into ranges, the partial product of every (tile, range) pair is
// computed by its own workgroup into an fp32 workspace, and a second kernel
// adds the ranges and writes C.
//
//  * the partial kernels are the tiled MFMA kernels (128 x 128 tiles) run
//    over a slab range; they store whole tiles into a workspace padded to
//    whole tiles, [splits][Mp][Np] fp32 with Mp, Np rounded up to 128, so
//    their stores need no bounds;
//  * the reduction kernel gives each thread four consecutive outputs of one
//    row and adds the ranges in order 0, 1, ..., splits - 1, so the result
//    does not depend on timing; it then applies the call's write-back (fp32:
//    alpha * sum + beta * C, C not read when beta == 0; fp16 and bf16:
//    rounding to the storage format, or the fused bias / activation /
//    residual);
//  * the split count (measured on MI355X over 1 to 144 tiles of 128 x 128
//    and K from 2048 to 16384): as many ranges as keep tiles x splits within
//    one wave of two workgroups per CU, at most 64, each range at least 256
//    (fp16) or 64 (fp32) deep in K; no split below three ranges or for K
//    under 2048.  A second wave of workgroups, or ranges shallower than
//    that, cost more than the partial sums' traffic saves.
#include "internal.h"

namespace mi355gemm {
namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;
// Workgroup slots of an MI355X: 256 CUs, two partial-product workgroups each.
constexpr int kSlots = 2 * 256;
constexpr int kMaxSplits = 64;
constexpr int kMinSplits = 3;
constexpr int kMinSplitK = 2048;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

int64_t round_tile(int x) { return ((int64_t)x + kTile - 1) / kTile * kTile; }

// The summed partials of outputs (m, n .. n + 3); false past the matrix.
struct Quad {
  int64_t m;
  int n;
  f4 acc;
};

__device__ __forceinline__ bool gather(const SplitK& sk, int M, int N, int64_t base, Quad& q) {
  const int64_t idx = (base + blockIdx.x) * kThreads + threadIdx.x;
  const int64_t qn = (N + 3) / 4;
  q.m = idx / qn;
  if (q.m >= M) return false;
  q.n = (int)(idx - q.m * qn) * 4;
  const float* src = sk.ws + q.m * sk.ld + q.n;
  q.acc = *(const f4*)src;
  // Eight ranges' loads in flight at a time, added in range order.
  int s = 1;
  for (; s + 8 <= sk.splits; s += 8) {
    f4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(const f4*)(src + (s + u) * sk.split_stride);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) q.acc[e] += v[u][e];
  }
  for (; s < sk.splits; ++s) {
    const f4 v = *(const f4*)(src + s * sk.split_stride);
#pragma unroll
    for (int e = 0; e < 4; ++e) q.acc[e] += v[e];
  }
  return true;
}

template <bool EPI, int FMT>
__global__ __launch_bounds__(kThreads) void reduce_f16_kernel(Args16 p, int64_t base) {
  Quad q;
  if (!gather(p.sk, p.M, p.N, base, q)) return;
  h4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x = q.acc[e];
    if constexpr (EPI) {
      const bool in = q.n + e < p.N;
      if (p.bias && in) x += word_to_f32<FMT>(p.bias[q.n + e]);
      x = epi_act(x, p.act);
      if (p.res && in) x += word_to_f32<FMT>(p.res[q.m * p.ldr + q.n + e]);
    }
    o[e] = f32_to_word<FMT>(x);
  }
  half_t* dst = p.C + q.m * p.ldc + q.n;
  if (q.n + 4 <= p.N) {
    __builtin_memcpy(dst, &o, 8);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (q.n + e < p.N) dst[e] = o[e];
  }
}

__global__ __launch_bounds__(kThreads) void reduce_f32_kernel(F32Args p, int64_t base) {
  Quad q;
  if (!gather(p.sk, p.M, p.N, base, q)) return;
  float* dst = p.C + q.m * p.ldc + q.n;
  f4 c = {0.f, 0.f, 0.f, 0.f};
  const bool whole = q.n + 4 <= p.N;
  if (p.beta != 0.f) {
    if (whole) {
      __builtin_memcpy(&c, dst, 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (q.n + e < p.N) c[e] = dst[e];
    }
  }
  f4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = p.alpha * q.acc[e];
    if (p.beta != 0.f) o[e] = fmaf(p.beta, c[e], o[e]);
  }
  if (whole) {
    __builtin_memcpy(dst, &o, 16);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (q.n + e < p.N) dst[e] = o[e];
  }
}

int64_t reduce_blocks(int M, int N) {
  return ((int64_t)M * ((N + 3) / 4) + kThreads - 1) / kThreads;
}

}  // namespace

SplitPlan splitk_plan(int M, int N, int K, int slab, int min_range, int requested) {
  SplitPlan plan;
  const int64_t nk = ((int64_t)K + slab - 1) / slab;
  if (M <= 0 || N <= 0 || K <= 0) return plan;
  int64_t s;
  if (requested > 0) {
    s = requested;
  } else {
    const int64_t tiles = (round_tile(M) / kTile) * (round_tile(N) / kTile);
    if (K < kMinSplitK) return plan;
    s = kSlots / tiles;
    if (s > K / min_range) s = K / min_range;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s < kMinSplits) return plan;
  }
  if (s > nk) s = nk;
  if (s < 2) return plan;
  // Ranges of equal depth; with 2 <= s <= nk there are still at least two.
  const int64_t per = (nk + s - 1) / s;
  plan.splits = (int)((nk + per - 1) / per);
  plan.per = (int)per;
  plan.bytes = (size_t)plan.splits * round_tile(M) * round_tile(N) * 4;
  return plan;
}

SplitK splitk_args(const SplitPlan& plan, int M, int N, void* workspace) {
  SplitK sk;
  sk.ws = static_cast<float*>(workspace);
  sk.ld = round_tile(N);
  sk.split_stride = round_tile(M) * sk.ld;
  sk.splits = plan.splits;
  sk.per = plan.per;
  return sk;
}

hipError_t launch_f16_splitk(const Args16& a, bool epi, hipStream_t stream) {
  const hipError_t e = launch_f16_partials(a, stream);
  if (e != hipSuccess) return e;
  const void* k = a.fmt == kFmtBF16
                      ? (epi ? (const void*)reduce_f16_kernel<true, kFmtBF16>
                             : (const void*)reduce_f16_kernel<false, kFmtBF16>)
                      : (epi ? (const void*)reduce_f16_kernel<true, kFmtF16>
                             : (const void*)reduce_f16_kernel<false, kFmtF16>);
  return launch_tiles(k, a, reduce_blocks(a.M, a.N), kThreads, 0, stream);
}

hipError_t launch_f32_splitk(const F32Args& a, hipStream_t stream) {
  const hipError_t e = launch_f32_partials(a, stream);
  if (e != hipSuccess) return e;
  return launch_tiles((const void*)reduce_f32_kernel, a, reduce_blocks(a.M, a.N), kThreads, 0,
                      stream);
}

}  // namespace mi355gemm
