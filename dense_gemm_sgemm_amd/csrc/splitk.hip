// Split-K (page "第 6 章 Shared Memory & Tile", section 6.5.6): when an
// M x N x K product has too few output tiles to occupy the GPU and K is long,
// K is cut into ranges, the partial product of every (tile, range) pair is
// computed by its own workgroup into an fp32 workspace, and a second kernel
// adds the ranges and writes C.
//
//  * the partial kernels are the tiled MFMA kernels (128 x 128 tiles) run
//    over a slab range -- the 16-bit full-tile kernel where the shape,
//    alignment and an exact division of K into the ranges allow it, the edge
//    kernels otherwise; they store whole tiles into a workspace padded to
//    whole tiles, [splits][Mp][Np] fp32 with Mp, Np rounded up to 128, so
//    their stores need no bounds;
//  * the reduction kernel gives each group of G threads four consecutive
//    outputs of one row; thread g of a group adds a contiguous block of
//    ranges in order, and the G block sums are added in block order, so the
//    result does not depend on timing (G = 1 to 8, about eight ranges per
//    thread); it then applies the call's write-back (fp32:
//    alpha * sum + beta * C, C not read when beta == 0; fp16 and bf16:
//    rounding to the storage format, or the fused bias / activation /
//    residual);
//  * the split count (measured on MI355X over 1 to 144 tiles of 128 x 128
//    and K from 2048 to 16384) follows a SplitRule: as many ranges as keep
//    tiles x splits within a workgroup budget, at most 64, each range at
//    least a minimum depth of K, never for K under 2048.  16-bit: budget
//    400, ranges of at least 256, a power of two (so that the ranges divide
//    K exactly and the full-tile kernel computes the partials), at least
//    two.  fp32: budget 512 (one wave of two workgroups per CU), ranges of
//    at least 64, at least three.  Beyond the budget a second wave of
//    workgroups, and below the depth the partial sums' traffic and the
//    workgroups' startup, cost more than the split gains.
#include "internal.h"

namespace mi355gemm {
namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;
constexpr int kMaxSplits = 64;
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

// Ranges s0 .. s1 - 1 (s0 < s1) of the partial sums at src, added in order
// with eight ranges' loads in flight at a time.
__device__ __forceinline__ f4 sum_ranges(const float* src, int64_t stride, int s0, int s1) {
  f4 acc = *(const f4*)(src + s0 * stride);
  int s = s0 + 1;
  for (; s + 8 <= s1; s += 8) {
    f4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(const f4*)(src + (s + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += v[u][e];
  }
  for (; s < s1; ++s) {
    const f4 v = *(const f4*)(src + s * stride);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
  return acc;
}

// G threads share one quad: thread group g adds ranges [S g / G, S (g+1) / G)
// in order, and the G group sums are added in group order through LDS, so
// the result is the same from run to run.  G > 1 keeps many loads in flight
// when there are few outputs and many ranges.  Returns false for threads
// that write nothing (past the matrix, or not in group 0).
template <int G>
__device__ __forceinline__ bool gather(const SplitK& sk, int M, int N, int64_t base, Quad& q) {
  constexpr int kQuads = kThreads / G;   // quads per workgroup
  const int t = threadIdx.x, g = t / kQuads, ql = t % kQuads;
  const int64_t idx = (base + blockIdx.x) * kQuads + ql;
  const int64_t qn = (N + 3) / 4;
  q.m = idx / qn;
  const bool in = q.m < M;
  q.n = (int)(idx - q.m * qn) * 4;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  const int s0 = (int)((int64_t)sk.splits * g / G), s1 = (int)((int64_t)sk.splits * (g + 1) / G);
  if (in && s0 < s1) acc = sum_ranges(sk.ws + q.m * sk.ld + q.n, sk.split_stride, s0, s1);
  if constexpr (G == 1) {
    q.acc = acc;
    return in;
  } else {
    __shared__ f4 red[G][kQuads];
    red[g][ql] = acc;
    __syncthreads();
    if (g != 0 || !in) return false;
    q.acc = red[0][ql];
#pragma unroll
    for (int h = 1; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) q.acc[e] += red[h][ql][e];
    return true;
  }
}

template <bool EPI, int FMT, int G>
__global__ __launch_bounds__(kThreads) void reduce_f16_kernel(Args16 p, int64_t base) {
  Quad q;
  if (!gather<G>(p.sk, p.M, p.N, base, q)) return;
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

template <int G>
__global__ __launch_bounds__(kThreads) void reduce_f32_kernel(F32Args p, int64_t base) {
  Quad q;
  if (!gather<G>(p.sk, p.M, p.N, base, q)) return;
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

// Threads per quad: about eight ranges per thread (one round of loads).
int reduce_groups(int splits) { return splits >= 64 ? 8 : splits >= 32 ? 4 : splits >= 16 ? 2 : 1; }

int64_t reduce_blocks(int M, int N, int groups) {
  const int64_t quads_per_block = kThreads / groups;
  return ((int64_t)M * ((N + 3) / 4) + quads_per_block - 1) / quads_per_block;
}

template <bool EPI, int FMT>
const void* reduce16(int groups) {
  switch (groups) {
    case 8: return (const void*)reduce_f16_kernel<EPI, FMT, 8>;
    case 4: return (const void*)reduce_f16_kernel<EPI, FMT, 4>;
    case 2: return (const void*)reduce_f16_kernel<EPI, FMT, 2>;
    default: return (const void*)reduce_f16_kernel<EPI, FMT, 1>;
  }
}

}  // namespace

SplitPlan splitk_plan(int M, int N, int K, int slab, const SplitRule& rule, int requested) {
  SplitPlan plan;
  const int64_t nk = ((int64_t)K + slab - 1) / slab;
  if (M <= 0 || N <= 0 || K <= 0) return plan;
  int64_t s;
  if (requested > 0) {
    s = requested;
  } else {
    const int64_t tiles = (round_tile(M) / kTile) * (round_tile(N) / kTile);
    if (K < kMinSplitK) return plan;
    s = rule.max_workgroups / tiles;
    if (s > K / rule.min_range) s = K / rule.min_range;
    if (s > kMaxSplits) s = kMaxSplits;
    if (rule.power_of_two)
      while (s & (s - 1)) s &= s - 1;   // keep the highest set bit
    if (s < rule.min_splits) return plan;
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

hipError_t launch_f16_splitk(const Args16& a, bool epi, int cus, hipStream_t stream) {
  const hipError_t e = f16_partials_fit(a) ? launch_f16_partials_mfma(a, cus, stream)
                                           : launch_f16_partials(a, stream);
  if (e != hipSuccess) return e;
  return launch_f16_reduce(a, epi, stream);
}

hipError_t launch_f16_reduce(const Args16& a, bool epi, hipStream_t stream) {
  const int g = reduce_groups(a.sk.splits);
  const void* k = a.fmt == kFmtBF16
                      ? (epi ? reduce16<true, kFmtBF16>(g) : reduce16<false, kFmtBF16>(g))
                      : (epi ? reduce16<true, kFmtF16>(g) : reduce16<false, kFmtF16>(g));
  return launch_tiles(k, a, reduce_blocks(a.M, a.N, g), kThreads, 0, stream);
}

hipError_t launch_f32_splitk(const F32Args& a, hipStream_t stream) {
  const hipError_t e = launch_f32_partials(a, stream);
  if (e != hipSuccess) return e;
  const int g = reduce_groups(a.sk.splits);
  const void* k = g == 8 ? (const void*)reduce_f32_kernel<8>
                : g == 4 ? (const void*)reduce_f32_kernel<4>
                : g == 2 ? (const void*)reduce_f32_kernel<2>
                         : (const void*)reduce_f32_kernel<1>;
  return launch_tiles(k, a, reduce_blocks(a.M, a.N, g), kThreads, 0, stream);
}

}  // namespace mi355gemm
