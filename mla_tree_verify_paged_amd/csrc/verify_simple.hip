// verify_simple.hip - split-K partial kernel with fp32 arithmetic (fp32 or bf16 inputs).
//
// One workgroup = one (request, tree token, group of 4 heads, key split); one wavefront per
// head. The split's keys are staged through LDS in tiles of 16 rows, converted to fp32, so
// that one gather of a paged latent row serves the group's heads, as in the head-tiled flash
// design of "The Glue That Connects: Wiring a Custom Flash Attention Kernel into the C-ABI
// Layer" (section "Design Decisions and Trade-Offs"). Scores are 64-lane dot products reduced
// with cross-lane shuffles; the softmax is streamed over the split with a running max and
// sum ("The Glue That Makes Kernels Run", section "The Context: A Custom Kernel in Flight").
// Each wave writes its split's normalised output, log-sum-exp, max score and argmax.
//
// This is the fp32-input path (exact argmax on fp32 data) and the reference kernel for the
// bf16 MFMA path; it is not the fast path.
#include <math.h>

#include "va_internal.h"

namespace va {
namespace {

constexpr int kTile = 16;       // keys per LDS tile
constexpr int kThreads = 256;   // 4 waves
constexpr int kQPerLane = kDim / 64;     // 9
constexpr int kOPerLane = kLatent / 64;  // 8

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <bool kFp32In>
__global__ void __launch_bounds__(kThreads)
simple_partial_kernel(RunArgs a, Workspace ws) {
  __shared__ float ktile[kTile][kDim];
  __shared__ int key_ok[kTile];

  const int S = ws.splits;
  const int head_groups = (a.H + kSimpleHeadsPerBlock - 1) / kSimpleHeadsPerBlock;
  int64_t b = blockIdx.x;
  const int s = int(b % S);
  b /= S;
  const int g = int(b % head_groups);
  b /= head_groups;
  const int i = int(b % a.max_q_per_req);
  const int r = int(b / a.max_q_per_req);
  if (r >= a.bs) return;

  Segment seg;
  const uint32_t bad = load_segment(a, r, seg);
  if (bad) {
    if (threadIdx.x == 0 && i == 0 && g == 0 && s == 0) atomicOr(ws.status, bad);
    return;
  }
  if (i >= seg.T) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = g * kSimpleHeadsPerBlock + wave;
  const bool head_ok = h < a.H;
  const int64_t t = seg.q0 + i;
  const int64_t row = t * a.H + (head_ok ? h : 0);

  const int chunk = (seg.L + S - 1) / S;
  const int k0 = min(seg.L, s * chunk);
  const int k1 = min(seg.L, k0 + chunk);

  float qv[kQPerLane];
  if (head_ok) {
#pragma unroll
    for (int k = 0; k < kQPerLane; ++k) {
      const int64_t e = row * kDim + lane + 64 * k;
      qv[k] = kFp32In ? static_cast<const float *>(a.q)[e]
                      : bf16_to_f32(static_cast<const uint16_t *>(a.q)[e]);
    }
  }

  float o[kOPerLane];
#pragma unroll
  for (int k = 0; k < kOPerLane; ++k) o[k] = 0.f;
  float m = -INFINITY, l = 0.f, best = -INFINITY;
  int best_j = -1;
  const uint8_t *mrow = a.mask + seg.m0 + int64_t(i) * seg.L;

  for (int j0 = k0; j0 < k1; j0 += kTile) {
    const int n = min(kTile, k1 - j0);
    __syncthreads();  // previous tile fully consumed
    if (threadIdx.x < kTile) {
      int ok = 0;
      const int j = j0 + threadIdx.x;
      if (threadIdx.x < n) {
        const int64_t slot = segment_slot(a, seg, j);
        const bool in_range = slot >= 0 && slot < a.num_slots;
        if (!in_range) atomicOr(ws.status, 1u);  // VA_DEV_SLOT_RANGE
        const bool vis = j < seg.P || mrow[j] != 0;
        ok = (in_range && vis) ? 1 : 0;
      }
      key_ok[threadIdx.x] = ok;
    }
    __syncthreads();
    // stage: 8 consecutive elements per thread per step
    for (int e = threadIdx.x * 8; e < kTile * kDim; e += kThreads * 8) {
      const int kk = e / kDim, d = e % kDim;
      float v[8];
      if (kk < n && key_ok[kk]) {
        const int64_t slot = segment_slot(a, seg, j0 + kk);
        if (kFp32In) {
          const float4 *src =
              reinterpret_cast<const float4 *>(static_cast<const float *>(a.kv) + slot * kDim + d);
          const float4 x0 = src[0], x1 = src[1];
          v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
          v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
        } else {
          const uint4 x = *reinterpret_cast<const uint4 *>(
              static_cast<const uint16_t *>(a.kv) + slot * kDim + d);
          const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            v[2 * c] = __uint_as_float(w[c] << 16);
            v[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) ktile[kk][d + c] = v[c];
    }
    __syncthreads();
    if (!head_ok) continue;

    float sc[kTile];
    float tmax = -INFINITY;
    int targ = -1;
#pragma unroll
    for (int kk = 0; kk < kTile; ++kk) {
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < kQPerLane; ++k) part = fmaf(qv[k], ktile[kk][lane + 64 * k], part);
      const float dot = wave_sum(part);
      const bool live = kk < n && key_ok[kk];
      sc[kk] = live ? dot * a.scale : -INFINITY;
      if (sc[kk] > tmax) {
        tmax = sc[kk];
        targ = j0 + kk;
      }
    }
    if (tmax > best) {
      best = tmax;
      best_j = targ;
    }
    const float m_new = fmaxf(m, tmax);
    if (m_new == -INFINITY) continue;  // nothing visible yet
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int k = 0; k < kOPerLane; ++k) o[k] *= alpha;
#pragma unroll
    for (int kk = 0; kk < kTile; ++kk) {
      const float p = expf(sc[kk] - m_new);
      l += p;
#pragma unroll
      for (int k = 0; k < kOPerLane; ++k) o[k] = fmaf(p, ktile[kk][lane + 64 * k], o[k]);
    }
    m = m_new;
  }

  if (!head_ok) return;
  // request r's partials: S blocks of its R = T*H rows, after the S * q0 * H rows of the
  // requests before it
  const int64_t R = int64_t(seg.T) * a.H;
  const int64_t x = row - seg.q0 * a.H;
  const int64_t base = int64_t(S) * seg.q0 * a.H + x;
  const int64_t prow = base + int64_t(s) * R;
  if (prow >= ws.part_rows) {  // cannot happen: the workspace is sized for S splits of every row
    if (lane == 0) atomicOr(ws.status, 2u);  // VA_DEV_SEGMENT
    return;
  }
  if (s == 0 && lane == 0) {
    RowInfo ri;
    ri.base = base;
    ri.n = S;
    ri.stride = int32_t(R);
    ws.row_info[row] = ri;
  }
  float *po = static_cast<float *>(ws.part_o) + prow * kLatent;
  if (l > 0.f) {
    const float inv = 1.f / l;
#pragma unroll
    for (int k = 0; k < kOPerLane; ++k) po[lane + 64 * k] = o[k] * inv;
  } else {
#pragma unroll
    for (int k = 0; k < kOPerLane; ++k) po[lane + 64 * k] = 0.f;
  }
  if (lane == 0) {
    ws.part_lse[prow] = l > 0.f ? m + logf(l) : -INFINITY;
    ws.part_max[prow] = best;
    ws.part_arg[prow] = best_j;
  }
}

}  // namespace

hipError_t launch_simple_partial(const RunArgs &a, const Workspace &ws, int in_fp32,
                                 hipStream_t st) {
  const int64_t head_groups = (a.H + kSimpleHeadsPerBlock - 1) / kSimpleHeadsPerBlock;
  const int64_t blocks = int64_t(a.bs) * a.max_q_per_req * head_groups * ws.splits;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (in_fp32)
    hipLaunchKernelGGL(simple_partial_kernel<true>, dim3(unsigned(blocks)), dim3(kThreads), 0,
                       st, a, ws);
  else
    hipLaunchKernelGGL(simple_partial_kernel<false>, dim3(unsigned(blocks)), dim3(kThreads), 0,
                       st, a, ws);
  return hipGetLastError();
}

}  // namespace va
