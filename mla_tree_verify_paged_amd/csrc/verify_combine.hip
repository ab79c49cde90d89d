// verify_combine.hip - merges the per-split partials of every (token, head) row.
//
// The pages name a split-K flash decode with a fixed split count ("The Glue That Makes
// Kernels Run", section "The Context: A Custom Kernel in Flight"; "The Final Solder Joint",
// section "The Three-Edits Sequence") but give no merge formula. The plain log-sum-exp merge
// is used: with M = max_s lse_s and w_s = exp(lse_s - M),
//   out = sum_s w_s * O_s / sum_s w_s,   lse = M + log(sum_s w_s),
// and the argmax is the argmax of the split holding the largest max score (lowest split,
// hence lowest key position, on ties).
//
// One wavefront per row; lane l owns output dims [8l, 8l+8). The combine also owns output
// validation: a row whose token belongs to no valid request is written empty (out 0,
// lse -inf, argmax -1) and the matching status bit is set, so every output element is
// defined whatever the device-side tables hold.
#include <math.h>

#include "va_internal.h"

namespace va {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ void store_row(const RunArgs &a, int64_t row, int lane, const float v[8]) {
  if (a.out_bf16) {
    uint4 w;
    w.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
    w.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
    w.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
    w.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
    reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.out) + row * kLatent)[lane] = w;
  } else {
    float4 *dst = reinterpret_cast<float4 *>(static_cast<float *>(a.out) + row * kLatent);
    dst[2 * lane] = make_float4(v[0], v[1], v[2], v[3]);
    dst[2 * lane + 1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

__global__ void __launch_bounds__(kThreads) combine_kernel(RunArgs a, Workspace ws) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.num_tokens * a.H) return;
  const int64_t t = row / a.H;

  // the request that owns token t: the last r with qo_indptr[r] <= t
  int lo = 0, hi = a.bs;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.qo_indptr[mid] <= t) lo = mid; else hi = mid;
  }
  uint32_t bad = 0;
  bool ok = a.bs > 0;
  if (ok) {
    Segment seg;
    bad = load_segment(a, lo, seg);
    ok = bad == 0 && t >= seg.q0 && t < seg.q0 + seg.T;
    if (bad == 0 && !ok) bad = 8u;  // VA_DEV_TOKENS
  } else {
    bad = 8u;
  }

  float v[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) v[c] = 0.f;
  if (!ok) {
    if (lane == 0) {
      atomicOr(ws.status, bad);
      if (a.out_lse) a.out_lse[row] = -INFINITY;
      if (a.out_argmax) a.out_argmax[row] = -1;
    }
    store_row(a, row, lane, v);
    return;
  }

  const int S = ws.splits;
  // max over splits of lse and of the max score
  float M = -INFINITY, best = -INFINITY;
  for (int s = lane; s < S; s += 64) {
    M = fmaxf(M, ws.part_lse[int64_t(s) * ws.rows_cap + row]);
    best = fmaxf(best, ws.part_max[int64_t(s) * ws.rows_cap + row]);
  }
  M = wave_max(M);
  best = wave_max(best);

  float W = 0.f;
  int arg = -1;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const int64_t prow = int64_t(s) * ws.rows_cap + row;
      const float ls = ws.part_lse[prow];
      if (ls == -INFINITY) continue;
      const float w = expf(ls - M);
      W += w;
      const float4 *src = reinterpret_cast<const float4 *>(ws.part_o + prow * kLatent);
      const float4 x0 = src[2 * lane], x1 = src[2 * lane + 1];
      v[0] = fmaf(w, x0.x, v[0]); v[1] = fmaf(w, x0.y, v[1]);
      v[2] = fmaf(w, x0.z, v[2]); v[3] = fmaf(w, x0.w, v[3]);
      v[4] = fmaf(w, x1.x, v[4]); v[5] = fmaf(w, x1.y, v[5]);
      v[6] = fmaf(w, x1.z, v[6]); v[7] = fmaf(w, x1.w, v[7]);
      if (arg < 0 && ws.part_max[prow] == best) arg = ws.part_arg[prow];
    }
    const float inv = 1.f / W;
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] *= inv;
  }
  store_row(a, row, lane, v);
  if (lane == 0) {
    if (a.out_lse) a.out_lse[row] = M == -INFINITY ? -INFINITY : M + logf(W);
    if (a.out_argmax) a.out_argmax[row] = arg;
  }
}

}  // namespace

hipError_t launch_combine(const RunArgs &a, const Workspace &ws, hipStream_t st) {
  const int64_t rows = a.num_tokens * a.H;
  if (rows <= 0) return hipSuccess;
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, st, a, ws);
  return hipGetLastError();
}

}  // namespace va
