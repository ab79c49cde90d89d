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
// Two wavefronts per row, each lane owning 4 output dims: the per-split scalars are read
// lane-parallel (lane s holds split s), then the 16-byte slices of up to 32 splits with
// nonzero weight are loaded at once, so the partial rows of every split are in flight
// together. The combine also owns output validation: a row whose token belongs to no valid
// request is written empty (out 0, lse -inf, argmax -1) and the matching status bit is set,
// so every output element is defined whatever the device-side tables hold.
#include <math.h>

#include "va_internal.h"

namespace va {
namespace {

constexpr int kThreads = 256;
constexpr int kThreadsPerRow = 128;                     // 4 dims each
constexpr int kRowsPerBlock = kThreads / kThreadsPerRow;
constexpr int kBatch = 32;                              // splits whose slices are in flight

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

// the 4 output dims [dim0, dim0 + 4) of `row`
__device__ void store4(const RunArgs &a, int64_t row, int dim0, const float4 &v) {
  if (a.out_bf16) {
    uint2 w;
    w.x = f32_to_bf16_rne(v.x) | (f32_to_bf16_rne(v.y) << 16);
    w.y = f32_to_bf16_rne(v.z) | (f32_to_bf16_rne(v.w) << 16);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + row * kLatent + dim0) = w;
  } else {
    *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + row * kLatent + dim0) = v;
  }
}

__global__ void __launch_bounds__(kThreads) combine_kernel(RunArgs a, Workspace ws) {
  const int lane = threadIdx.x & 63;
  const int sub = threadIdx.x % kThreadsPerRow;            // 0..127 within the row
  const bool lead = sub == 0;                              // writes the row's scalars
  const int64_t row = int64_t(blockIdx.x) * kRowsPerBlock + threadIdx.x / kThreadsPerRow;
  if (row >= a.num_tokens * a.H) return;
  const int64_t t = row / a.H;
  const int dim0 = 4 * sub;
  const int S = ws.splits;
  const int64_t stride = ws.rows_cap;
  const float *plse = ws.part_lse + row;
  const float *pmax = ws.part_max + row;

  // Requested before the row is validated, so that one memory round trip serves all of them:
  // the slices of the first kBatch splits and the scalars of the first 64. Every address is
  // inside the workspace (row < num_tokens * H <= rows_cap); an invalid row discards them.
  float4 x[kBatch];
#pragma unroll
  for (int k = 0; k < kBatch; ++k)
    x[k] = k < S ? *reinterpret_cast<const float4 *>(ws.part_o + (int64_t(k) * stride + row) *
                                                                     kLatent + dim0)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
  const float lse0 = lane < S ? plse[lane * stride] : -INFINITY;
  const float max0 = lane < S ? pmax[lane * stride] : -INFINITY;

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

  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (!ok) {
    if (lead) {
      atomicOr(ws.status, bad);
      if (a.out_lse) a.out_lse[row] = -INFINITY;
      if (a.out_argmax) a.out_argmax[row] = -1;
    }
    store4(a, row, dim0, v);
    return;
  }

  // per-split scalars, lane-parallel (lane s holds split s, then s + 64, ...)
  float M = lse0, best = max0;
  for (int s0 = 64; s0 < S; s0 += 64) {
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
    for (int s0 = 0; s0 < S; s0 += kBatch) {
      // lane j < kBatch: the weight of split s0 + j
      const int s = s0 + lane;
      // splits below 64 come from lane s of the speculative read, the rest from memory
      const float lsh = __shfl(lse0, s & 63, 64);
      float ls = -INFINITY;
      if (lane < kBatch && s < S) ls = s < 64 ? lsh : plse[s * stride];
      const float wgt = ls == -INFINITY ? 0.f : expf(ls - M);
      W += wave_sum(wgt);
      if (arg < 0) {  // wave-uniform
        const uint64_t hit = __ballot(lane < kBatch && s < S && pmax[s * stride] == best);
        if (hit) arg = ws.part_arg[(s0 + __builtin_ctzll(hit)) * stride + row];
      }
      const uint32_t live = uint32_t(__ballot(wgt != 0.f));
      if (s0 > 0) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          if ((live >> k) & 1u)
            x[k] = *reinterpret_cast<const float4 *>(
                ws.part_o + (int64_t(s0 + k) * stride + row) * kLatent + dim0);
          else
            x[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        // a split with zero weight contributes nothing (its slice is not read, or is zero)
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), k));
        if ((live >> k) & 1u) {
          v.x = fmaf(wk, x[k].x, v.x); v.y = fmaf(wk, x[k].y, v.y);
          v.z = fmaf(wk, x[k].z, v.z); v.w = fmaf(wk, x[k].w, v.w);
        }
      }
    }
    const float inv = 1.f / W;
    v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
  }
  store4(a, row, dim0, v);
  if (lead) {
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
