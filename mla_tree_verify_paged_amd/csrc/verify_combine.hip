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
// One wavefront per row. The per-split scalars are read lane-parallel (lane s holds split s);
// the 2 KB partial rows of the splits with nonzero weight are then streamed with up to eight
// splits in flight, lane l owning output dims [8l, 8l+8). The combine also owns output
// validation: a row whose token belongs to no valid request is written empty (out 0,
// lse -inf, argmax -1) and the matching status bit is set, so every output element is
// defined whatever the device-side tables hold.
#include <math.h>

#include "va_internal.h"

namespace va {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;
constexpr int kBatch = 8;  // splits whose partial rows are in flight at once

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
  const float *plse = ws.part_lse + row;
  const float *pmax = ws.part_max + row;
  const int64_t stride = ws.rows_cap;

  // per-split scalars, lane-parallel
  float M = -INFINITY, best = -INFINITY;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int s = s0 + lane;
    if (s < S) {
      M = fmaxf(M, plse[s * stride]);
      best = fmaxf(best, pmax[s * stride]);
    }
  }
  M = wave_max(M);
  best = wave_max(best);

  float W = 0.f;
  int arg = -1;
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < S; s0 += 64) {
      const int s = s0 + lane;
      const float ls = s < S ? plse[s * stride] : -INFINITY;
      const float w = ls == -INFINITY ? 0.f : expf(ls - M);
      W += wave_sum(w);
      if (arg < 0) {
        const uint64_t hit = __ballot(s < S && pmax[s * stride] == best);
        if (hit) arg = ws.part_arg[(s0 + __builtin_ctzll(hit)) * stride + row];
      }
      uint64_t live = __ballot(w != 0.f);
      while (live) {
        // up to kBatch splits with nonzero weight: issue their loads, then accumulate
        int idx[kBatch];
        float wt[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          idx[k] = -1;
          wt[k] = 0.f;
          if (live) {
            const int j = __builtin_ctzll(live);
            live &= live - 1;
            idx[k] = s0 + j;
            wt[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
          }
        }
        float4 x0[kBatch], x1[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          if (idx[k] >= 0) {
            const float4 *src = reinterpret_cast<const float4 *>(
                ws.part_o + (int64_t(idx[k]) * stride + row) * kLatent);
            x0[k] = src[2 * lane];
            x1[k] = src[2 * lane + 1];
          } else {
            x0[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            x1[k] = x0[k];
          }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          v[0] = fmaf(wt[k], x0[k].x, v[0]); v[1] = fmaf(wt[k], x0[k].y, v[1]);
          v[2] = fmaf(wt[k], x0[k].z, v[2]); v[3] = fmaf(wt[k], x0[k].w, v[3]);
          v[4] = fmaf(wt[k], x1[k].x, v[4]); v[5] = fmaf(wt[k], x1[k].y, v[5]);
          v[6] = fmaf(wt[k], x1[k].z, v[6]); v[7] = fmaf(wt[k], x1[k].w, v[7]);
        }
      }
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
