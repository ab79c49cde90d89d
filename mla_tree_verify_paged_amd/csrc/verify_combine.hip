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
// The partials are fp32 (the fp32-input kernel), or 16-bit signed-normalised codes with one
// scale per 128 dims (the MFMA kernel's format, half the bytes). Three launch shapes, chosen by
// the step's row count (rows with few rows have many splits, and the reverse):
//  - combine_kernel: one workgroup per row (a quarter of a row below 512 rows, fp32 partials).
//    Every wavefront reads the per-split scalars lane-parallel (lane s holds split s) and
//    derives the same max, weights and argmax; the splits' partial rows are dealt to the four
//    wavefronts (split s to wavefront s % 4), each lane owning 8 output dims (2 in a quarter
//    row), and the four partial sums meet in LDS;
//  - combine_few_rows_kernel (16-bit partials, below 512 rows): a quarter row per workgroup,
//    every split's codes in one round trip;
//  - combine_rows_kernel (16-bit partials, over 2048 rows): one wavefront per row.
// The combine also owns output validation: a row whose token belongs to no valid request is
// written empty (out 0, lse -inf, argmax -1) and the matching status bit is set, so every
// output element is defined whatever the device-side tables hold.
#include <math.h>

#include "va_internal.h"

namespace va {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The request that owns token t: the last r < bs with qo_indptr[r] <= t (0 when there is
// none), from one lane-parallel read of the table per 64 requests rather than a binary search
// of dependent reads. Wave-uniform. A table that is not nondecreasing gives some r, whose
// segment the caller checks t against.
__device__ __forceinline__ int owner_request(const RunArgs &a, int64_t t, int lane) {
  int owner = 0;
  for (int r0 = 0; r0 < a.bs; r0 += 64) {
    const int r = r0 + lane;
    const uint64_t le = __ballot(r < a.bs && a.qo_indptr[r] <= t);
    if (le) owner = r0 + 63 - __builtin_clzll(le);
    if (!(le >> 63)) break;  // the rest of a nondecreasing table lies past t
  }
  return owner;
}

// The index-table entries of requests 0..63 (lane l: request l's qo_indptr[l], qo_indptr[l+1],
// kv_indptr[l], kv_indptr[l+1], mask_indptr[l]), requested at a kernel's start beside the
// row's placement, so that validating a row costs no round trip of its own. Batches of more
// than 64 requests read nothing here and validate from the tables (owner_request, then
// load_segment).
struct SegTables {
  int64_t q0, q1, m0;
  int32_t k0, k1;
};
__device__ __forceinline__ SegTables prefetch_tables(const RunArgs &a, int lane) {
  SegTables p;
  p.q0 = p.q1 = p.m0 = 0;
  p.k0 = p.k1 = 0;
  if (a.bs <= 64 && lane < a.bs) {
    p.q0 = a.qo_indptr[lane];
    p.q1 = a.qo_indptr[lane + 1];
    p.k0 = a.kv_indptr[lane];
    p.k1 = a.kv_indptr[lane + 1];
    p.m0 = a.mask_indptr[lane];
  }
  return p;
}
// The segment of the request that owns token t (the same request owner_request picks) and
// its VA_DEV_* bits. Wave-uniform.
__device__ __forceinline__ uint32_t owner_segment(const RunArgs &a, const SegTables &p,
                                                  int64_t t, int lane, Segment &seg) {
  if (a.bs > 64) return load_segment(a, owner_request(a, t, lane), seg);
  const uint64_t le = __ballot(lane < a.bs && p.q0 <= t);
  const int r = le ? 63 - __builtin_clzll(le) : 0;
  return check_segment(a, lane_i64(p.q0, r), lane_i64(p.q1, r),
                       __builtin_amdgcn_readlane(p.k0, r), __builtin_amdgcn_readlane(p.k1, r),
                       lane_i64(p.m0, r), seg);
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

__device__ __forceinline__ void fma8(float4 &lo, float4 &hi, float w, const float4 &x0,
                                     const float4 &x1) {
  lo.x = fmaf(w, x0.x, lo.x); lo.y = fmaf(w, x0.y, lo.y);
  lo.z = fmaf(w, x0.z, lo.z); lo.w = fmaf(w, x0.w, lo.w);
  hi.x = fmaf(w, x1.x, hi.x); hi.y = fmaf(w, x1.y, hi.y);
  hi.z = fmaf(w, x1.z, hi.z); hi.w = fmaf(w, x1.w, hi.w);
}

// the 2 output dims [dim0, dim0 + 2) of `row`
__device__ void store2(const RunArgs &a, int64_t row, int dim0, float x, float y) {
  if (a.out_bf16) {
    *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(a.out) + row * kLatent + dim0) =
        f32_to_bf16_rne(x) | (f32_to_bf16_rne(y) << 16);
  } else {
    *reinterpret_cast<float2 *>(static_cast<float *>(a.out) + row * kLatent + dim0) =
        make_float2(x, y);
  }
}

// A lane's slice of one partial row as loaded: kV fp32 values, or kV int16 codes (two per
// word) and the scale of their 128-dim group. Decoded only where it is used, so that loads
// stay in flight until then.
template <int kV, bool kI16> struct PartSlice;
template <int kV> struct PartSlice<kV, false> {
  float x[kV];
  __device__ __forceinline__ float value(int e) const { return x[e]; }
  __device__ __forceinline__ float scale(int) const { return 1.f; }
};
template <int kV> struct PartSlice<kV, true> {
  uint32_t w[kV / 2];
  float sc[2];  // the scales of the lane's first and second kV/2 dims
  __device__ __forceinline__ float value(int e) const {
    const uint32_t u = w[e / 2];
    return float((e & 1) ? int32_t(u) >> 16 : int32_t(u << 16) >> 16);
  }
  __device__ __forceinline__ float scale(int e) const { return sc[e < kV / 2 ? 0 : 1]; }
};

// One workgroup per (row, dim slice). kSlices = 1: the whole 512-dim row, each lane owning 8
// dims, [4l, 4l+4) and [256+4l, 256+4l+4), so that the output stores are contiguous across
// the wavefront; kSlices = 4 (steps with few rows, whose rows have many splits): a
// quarter of the row per workgroup, each lane owning 2 dims, so a row's splits are read by
// four workgroups on four compute units. kBatch: splits whose slices a wavefront has in
// flight (fewer keep more workgroups resident). kI16: the partials are int16 codes with a
// scale per 128 dims (the MFMA kernel's format), else fp32.
template <int kBatch, int kSlices, bool kI16>
__global__ void __launch_bounds__(kThreads) combine_kernel(RunArgs a, Workspace ws) {
  constexpr int kV = 8 / kSlices;           // dims per lane
  constexpr int kSliceDims = kLatent / kSlices;
  static_assert(kSliceDims % kScaleGroupDims == 0 || kSlices == 1, "a slice in one group");
  __shared__ float red[kWaves - 1][kV][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // the same, in a scalar register
  const int64_t row = blockIdx.x / kSlices;
  const int slice = int(blockIdx.x % kSlices);
  const int64_t t = row / a.H;
  // the lane's dims: kV consecutive ones at dim_a (kSlices > 1), or 4 at dim_a and 4 at
  // dim_a + 256
  const int dim_a = kSlices == 1 ? 4 * lane : slice * kSliceDims + kV * lane;
  // the scale groups of those dims (int16 partials)
  const int group_a = dim_a / kScaleGroupDims;
  const int group_b = kSlices == 1 ? (dim_a + 256) / kScaleGroupDims : group_a;

  // the tables that validate the row, requested before its placement (one round trip for both)
  const SegTables tabs = prefetch_tables(a, lane);
  // where this row's partials are (written by the partial kernel for every row of a valid
  // request; for other rows it is stale or arbitrary, so it is only used once checked to stay
  // inside the workspace, and such rows are discarded below)
  const RowInfo ri = ws.row_info[row];
  int S = ri.n;
  int64_t base = ri.base, stride = ri.stride;
  const bool placed = S >= 1 && S <= (1 << 20) && stride >= 1 && stride <= (1 << 28) &&
                      base >= 0 && base + int64_t(S - 1) * stride < ws.part_rows;
  if (!placed) {
    S = 0;
    base = 0;
    stride = 0;
  }
  const float *plse = ws.part_lse + base;
  const float *pmax = ws.part_max + base;
  const int64_t ostride = stride * kLatent;
  using Slice = PartSlice<kV, kI16>;
  auto load = [&](int sp, Slice &x) __attribute__((always_inline)) {
    if constexpr (kI16) {
      const int16_t *src =
          static_cast<const int16_t *>(ws.part_o) + base * kLatent + dim_a + sp * ostride;
      const float *sc = ws.part_scale + (base + sp * stride) * kScaleGroups;
      if constexpr (kSlices == 1) {
        const uint2 u = *reinterpret_cast<const uint2 *>(src);
        const uint2 v = *reinterpret_cast<const uint2 *>(src + 256);
        x.w[0] = u.x; x.w[1] = u.y; x.w[2] = v.x; x.w[3] = v.y;
        // the split's four scales (one address for the whole wavefront), then the lane's two
        const float4 s4 = *reinterpret_cast<const float4 *>(sc);
        x.sc[0] = group_a == 0 ? s4.x : s4.y;
        x.sc[1] = group_b == 2 ? s4.z : s4.w;
      } else {
        static_assert(kV == 2, "two dims per lane");
        x.w[0] = *reinterpret_cast<const uint32_t *>(src);
        x.sc[0] = x.sc[1] = sc[group_a];
      }
    } else {
      const float *src = static_cast<const float *>(ws.part_o) + base * kLatent + dim_a +
                         sp * ostride;
      if constexpr (kSlices == 1) {
        const float4 u = *reinterpret_cast<const float4 *>(src);
        const float4 v = *reinterpret_cast<const float4 *>(src + 256);
        x.x[0] = u.x; x.x[1] = u.y; x.x[2] = u.z; x.x[3] = u.w;
        x.x[4] = v.x; x.x[5] = v.y; x.x[6] = v.z; x.x[7] = v.w;
      } else {
        static_assert(kV == 2, "two dims per lane");
        const float2 u = *reinterpret_cast<const float2 *>(src);
        x.x[0] = u.x; x.x[1] = u.y;
      }
    }
  };
  auto store = [&](const float *v) __attribute__((always_inline)) {
    if constexpr (kSlices == 1) {
      store4(a, row, dim_a, make_float4(v[0], v[1], v[2], v[3]));
      store4(a, row, dim_a + 256, make_float4(v[4], v[5], v[6], v[7]));
    } else {
      store2(a, row, dim_a, v[0], v[1]);
    }
  };

  // Requested before the row is validated, so that one memory round trip serves all of them:
  // this wavefront's first kBatch splits and the scalars of the first 64 (all inside the
  // workspace, as checked above).
  Slice x[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int sp = wave + kWaves * j;
    if (sp < S) load(sp, x[j]);
  }
  // the scalars of splits lane + 64*i, i < kScal (kSlices > 1: rows with many splits read all
  // of them in this one round trip; otherwise only the first 64 here)
  constexpr int kScal = kSlices > 1 ? 4 : 1;
  // (and, when the argmax is wanted, the split argmax of the same splits, so that picking the
  // row's argmax needs no further round trip)
  const bool want_arg = a.out_argmax != nullptr;
  const int32_t *parg = ws.part_arg + base;
  float lsv[kScal], mxv[kScal];
  int32_t agv[kScal];
#pragma unroll
  for (int i = 0; i < kScal; ++i) {
    const int sp = lane + 64 * i;
    lsv[i] = sp < S ? plse[int64_t(sp) * stride] : -INFINITY;
    mxv[i] = sp < S ? pmax[int64_t(sp) * stride] : -INFINITY;
    agv[i] = sp < S && want_arg ? parg[int64_t(sp) * stride] : -1;
  }

  // the request that owns token t
  uint32_t bad = 0;
  bool ok = a.bs > 0 && row < a.num_tokens * a.H;
  if (ok) {
    Segment seg;
    bad = owner_segment(a, tabs, t, lane, seg);
    ok = bad == 0 && t >= seg.q0 && t < seg.q0 + seg.T;
    if (bad == 0 && !ok) bad = 8u;  // VA_DEV_TOKENS
    if (ok && !placed) {  // cannot happen: the partial kernel places every valid row
      ok = false;
      bad = 2u;
    }
  } else {
    bad = 8u;
  }
  if (!ok) {
    if (threadIdx.x == 0 && slice == 0) {
      atomicOr(ws.status, bad);
      if (a.out_lse) a.out_lse[row] = -INFINITY;
      if (a.out_argmax) a.out_argmax[row] = -1;
    }
    if (wave == 0) {
      const float zero[kV] = {};
      store(zero);
    }
    return;
  }

  // per-split scalars, lane-parallel (lane s holds split s, then s + 64, ...); every
  // wavefront computes the same M, best and W
  float M = lsv[0], best = mxv[0];
#pragma unroll
  for (int i = 1; i < kScal; ++i) {
    M = fmaxf(M, lsv[i]);
    best = fmaxf(best, mxv[i]);
  }
  for (int s0 = 64 * kScal; s0 < S; s0 += 64) {
    const int s = s0 + lane;
    if (s < S) {
      M = fmaxf(M, plse[int64_t(s) * stride]);
      best = fmaxf(best, pmax[int64_t(s) * stride]);
    }
  }
  M = wave_max_f32(M);
  best = wave_max_f32(best);

  float W = 0.f;
  int arg = -1;
  float acc[kV];
#pragma unroll
  for (int e = 0; e < kV; ++e) acc[e] = 0.f;
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < S; s0 += 64) {
      const int s = s0 + lane;
      // the scalars of split s: held since the first round trip, or read now
      float ls = -INFINITY, mx = -INFINITY;
      int32_t ag = -1;
      if (s0 < 64 * kScal) {
#pragma unroll
        for (int i = 0; i < kScal; ++i)
          if (s0 == 64 * i) {
            ls = lsv[i];
            mx = mxv[i];
            ag = agv[i];
          }
      } else if (s < S) {
        ls = plse[int64_t(s) * stride];
        mx = pmax[int64_t(s) * stride];
        if (want_arg) ag = parg[int64_t(s) * stride];
      }
      const float wgt = ls == -INFINITY ? 0.f : expf(ls - M);
      W += wave_sum_f32(wgt);
      if (arg < 0) {  // wave-uniform: the lowest split holding the largest max score
        const uint64_t hit = __ballot(s < S && mx == best);
        if (hit) arg = __builtin_amdgcn_readlane(ag, int(__builtin_ctzll(hit)));
      }
      // this wavefront's splits of the 64: s0 + wave + 4j, in batches of kBatch
#pragma unroll 1
      for (int j0 = 0; j0 < 64 / kWaves; j0 += kBatch) {
        if (s0 + wave + kWaves * j0 >= S) break;
        if (s0 > 0 || j0 > 0) {
#pragma unroll
          for (int j = 0; j < kBatch; ++j) {
            const int sp = s0 + wave + kWaves * (j0 + j);
            if (sp < S) load(sp, x[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int sl = wv + kWaves * (j0 + j);  // lane of this split within the 64
          const float wk = lane_f32(wgt, sl);
          // a split with zero weight contributes nothing (its row may be unwritten)
          if (s0 + sl < S && wk != 0.f) {
            const float f0 = wk * x[j].scale(0), f1 = wk * x[j].scale(kV - 1);
#pragma unroll
            for (int e = 0; e < kV; ++e)
              acc[e] = fmaf(e < kV / 2 ? f0 : f1, x[j].value(e), acc[e]);
          }
        }
      }
    }
  }
  // the four wavefronts' sums meet in LDS; wavefront 0 finishes the row
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < kV; ++e) red[wave - 1][e][lane] = acc[e];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int k = 0; k < kWaves - 1; ++k) {
#pragma unroll
    for (int e = 0; e < kV; ++e) acc[e] += red[k][e][lane];
  }
  const float inv = M == -INFINITY ? 0.f : 1.f / W;
#pragma unroll
  for (int e = 0; e < kV; ++e) acc[e] *= inv;
  store(acc);
  if (lane == 0 && slice == 0) {
    if (a.out_lse) a.out_lse[row] = M == -INFINITY ? -INFINITY : M + logf(W);
    if (a.out_argmax) a.out_argmax[row] = arg;
  }
}

// Steps with fewer than 512 rows, 16-bit partials: a quarter row per workgroup (one 128-dim
// scale group), and every split's codes requested in one round trip. Such rows have many
// splits (tp8: 240). Wavefront w takes splits w + 4k (k < 64); its lane group g = lane / 16
// reads split k = 4j + g with load j (j < 16), lane l owning dims 8 (l % 16) .. + 8 of the
// slice, so a wavefront covers four splits per 16-byte load and a lane has 16 code loads and
// 16 scalar loads in flight (a one-dword load per split took 64 code loads per lane, over the
// 63 a wavefront can count, and serialised the last of them). Lane s holds the scalars of
// splits s, s + 64, s + 128, s + 192 and folds the slice's group scale into the split's
// weight; each wavefront lays its splits' factors out in LDS so that a lane's 16 are
// contiguous. The 16 partial sums of each dim (4 wavefronts x 4 lane groups) meet in LDS.
// A row has at most kMaxSplits = 256 splits (the work list makes at most one item per compute
// unit, capped at kMaxSplits, and a fixed split count is capped there too).
__global__ void __launch_bounds__(kThreads) combine_few_rows_kernel(RunArgs a, Workspace ws) {
  constexpr int kSlices = kScaleGroups;       // one scale group per workgroup
  constexpr int kGroups = 4;                  // lane groups of 16, one split each per load
  constexpr int kJ = kMaxSplits / (kWaves * kGroups);  // code loads per lane
  constexpr int kScal = kMaxSplits / 64;      // split scalars per lane
  constexpr int kDims = 8;                    // dims per lane
  static_assert(kScaleGroupDims == 16 * kDims, "16 lanes cover a scale group");
  // factors: wavefront w's split 4k + w at [w][(k % 4) * kJ + k / 4]; sums: [w][g][q][dim]
  __shared__ __attribute__((aligned(16))) float fac[kWaves][kGroups * kJ];
  __shared__ __attribute__((aligned(16))) float red[kWaves][kGroups][16][kDims];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, q = lane & 15;
  const int64_t row = blockIdx.x / kSlices;
  const int slice = int(blockIdx.x % kSlices);
  const int64_t t = row / a.H;

  const SegTables tabs = prefetch_tables(a, lane);
  // where this row's partials are (checked to stay inside the workspace, as above)
  const RowInfo ri = ws.row_info[row];
  int S = ri.n;
  int64_t base = ri.base, stride = ri.stride;
  const bool placed = S >= 1 && S <= kMaxSplits && stride >= 1 && stride <= (1 << 28) &&
                      base >= 0 && base + int64_t(S - 1) * stride < ws.part_rows;
  if (!placed) {
    S = 0;
    base = 0;
    stride = 0;
  }
  const int16_t *codes = static_cast<const int16_t *>(ws.part_o) + base * kLatent +
                         slice * kScaleGroupDims + kDims * q;
  const int64_t ostride = stride * kLatent;
  const bool want_arg = a.out_argmax != nullptr;

  // every load goes out before the row is validated
  uint4 cw[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int sp = kWaves * (kGroups * j + g) + wave;
    cw[j] = sp < S ? *reinterpret_cast<const uint4 *>(codes + sp * ostride)
                   : make_uint4(0u, 0u, 0u, 0u);
  }
  float lsv[kScal], mxv[kScal], scv[kScal];
  int32_t agv[kScal];
#pragma unroll
  for (int i = 0; i < kScal; ++i) {
    const int sp = lane + 64 * i;
    const bool in = sp < S;
    const int64_t pr = base + int64_t(sp) * stride;
    lsv[i] = in ? ws.part_lse[pr] : -INFINITY;
    mxv[i] = in ? ws.part_max[pr] : -INFINITY;
    agv[i] = in && want_arg ? ws.part_arg[pr] : -1;
    scv[i] = in ? ws.part_scale[pr * kScaleGroups + slice] : 0.f;
  }

  // the request that owns token t
  uint32_t bad = 0;
  bool ok = a.bs > 0 && row < a.num_tokens * a.H;
  if (ok) {
    Segment seg;
    bad = owner_segment(a, tabs, t, lane, seg);
    ok = bad == 0 && t >= seg.q0 && t < seg.q0 + seg.T;
    if (bad == 0 && !ok) bad = 8u;  // VA_DEV_TOKENS
    if (ok && !placed) {  // cannot happen: the partial kernel places every valid row
      ok = false;
      bad = 2u;
    }
  } else {
    bad = 8u;
  }
  // (the same for every wavefront of the workgroup, so all of them return here or none)
  if (!ok) {
    if (threadIdx.x == 0 && slice == 0) {
      atomicOr(ws.status, bad);
      if (a.out_lse) a.out_lse[row] = -INFINITY;
      if (a.out_argmax) a.out_argmax[row] = -1;
    }
    if (wave == 0) store2(a, row, slice * kScaleGroupDims + 2 * lane, 0.f, 0.f);
    return;
  }

  // the row's largest lse and max score (every wavefront computes the same)
  float M = lsv[0], best = mxv[0];
#pragma unroll
  for (int i = 1; i < kScal; ++i) {
    M = fmaxf(M, lsv[i]);
    best = fmaxf(best, mxv[i]);
  }
  M = wave_max_f32(M);
  best = wave_max_f32(best);
  // the argmax: the lowest split holding the largest max score (split lane + 64 i)
  int arg = -1;
#pragma unroll
  for (int i = kScal - 1; i >= 0; --i) {
    const uint64_t hit = __ballot(mxv[i] == best);
    if (hit) arg = __builtin_amdgcn_readlane(agv[i], int(__builtin_ctzll(hit)));
  }
  // per split: its weight, and the weight times the group scale of its codes (zero for a
  // split without visible keys, whose codes and scale may be unwritten; zero for every split
  // when the row sees no key)
  float wsum = 0.f;
#pragma unroll
  for (int i = 0; i < kScal; ++i) {
    const float w = lsv[i] == -INFINITY ? 0.f : expf(lsv[i] - M);
    wsum += w;
    // split lane + 64 i is split k = lane / 4 + 16 i of wavefront lane % 4
    if ((lane & 3) == wave)
      fac[wave][((lane >> 2) & 3) * kJ + (lane >> 4) + 4 * i] = w != 0.f ? w * scv[i] : 0.f;
  }
  const float W = M == -INFINITY ? 0.f : wave_sum_f32(wsum);
  __syncthreads();
  float fk[kJ];
#pragma unroll
  for (int j4 = 0; j4 < kJ / 4; ++j4) {
    const float4 v = *reinterpret_cast<const float4 *>(&fac[wave][g * kJ + 4 * j4]);
    fk[4 * j4] = v.x;
    fk[4 * j4 + 1] = v.y;
    fk[4 * j4 + 2] = v.z;
    fk[4 * j4 + 3] = v.w;
  }
  // (no zero test: a split without weight has a factor of exactly 0 and finite codes)
  float acc[kDims] = {};
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const uint32_t w4[4] = {cw[j].x, cw[j].y, cw[j].z, cw[j].w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc[2 * m] = fmaf(fk[j], float(int32_t(w4[m] << 16) >> 16), acc[2 * m]);
      acc[2 * m + 1] = fmaf(fk[j], float(int32_t(w4[m]) >> 16), acc[2 * m + 1]);
    }
  }
  *reinterpret_cast<float4 *>(&red[wave][g][q][0]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4 *>(&red[wave][g][q][4]) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  if (wave != 0) return;
  // lane l finishes dims 2l, 2l + 1 of the slice: those of lane l / 4 of every group
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
#pragma unroll
    for (int gg = 0; gg < kGroups; ++gg) {
      const float2 v = *reinterpret_cast<const float2 *>(&red[w][gg][lane >> 2][2 * (lane & 3)]);
      o0 += v.x;
      o1 += v.y;
    }
  const float inv = M == -INFINITY ? 0.f : 1.f / W;
  store2(a, row, slice * kScaleGroupDims + 2 * lane, o0 * inv, o1 * inv);
  if (lane == 0 && slice == 0) {
    if (a.out_lse) a.out_lse[row] = M == -INFINITY ? -INFINITY : M + logf(W);
    if (a.out_argmax) a.out_argmax[row] = arg;
  }
}

// Steps with more than 2048 rows, 16-bit partials: one wavefront per row, four rows per
// workgroup, no LDS and no barrier. Such steps have few splits per row (segmented: about 3,
// stress 4), so a row's reads take one round trip; a workgroup per row left three of its four
// wavefronts with little or nothing to read, and every row's latency held a whole workgroup
// slot. Lane l owns dims [4l, 4l+4) and
// [256+4l, 256+4l+4) (groups l/32 and 2 + l/32), so the output stores are contiguous; it reads
// the matching 8-byte code runs and the two group scales of each split, kB splits per round
// trip, and lane s holds the scalars of splits s, s + 64, ...
template <int kB>
__global__ void __launch_bounds__(kThreads) combine_rows_kernel(RunArgs a, Workspace ws) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= a.num_tokens * int64_t(a.H)) return;  // wave-uniform; nothing below synchronises
  const int64_t t = row / a.H;
  const int dim_a = 4 * lane;
  const int ga = dim_a / kScaleGroupDims, gb = (dim_a + 256) / kScaleGroupDims;

  const SegTables tabs = prefetch_tables(a, lane);
  const RowInfo ri = ws.row_info[row];
  int S = ri.n;
  int64_t base = ri.base, stride = ri.stride;
  const bool placed = S >= 1 && S <= (1 << 20) && stride >= 1 && stride <= (1 << 28) &&
                      base >= 0 && base + int64_t(S - 1) * stride < ws.part_rows;
  if (!placed) {
    S = 0;
    base = 0;
    stride = 0;
  }
  const int16_t *codes = static_cast<const int16_t *>(ws.part_o) + base * kLatent + dim_a;
  const int64_t ostride = stride * kLatent;
  const bool want_arg = a.out_argmax != nullptr;

  // kB splits' code runs and group scales
  uint2 ca[kB], cb[kB];
  float sa[kB], sb[kB];
  auto load = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int sp = s0 + j;
      if (sp < S) {
        const int16_t *src = codes + sp * ostride;
        ca[j] = *reinterpret_cast<const uint2 *>(src);
        cb[j] = *reinterpret_cast<const uint2 *>(src + 256);
        const float *sc = ws.part_scale + (base + int64_t(sp) * stride) * kScaleGroups;
        sa[j] = sc[ga];
        sb[j] = sc[gb];
      }
    }
  };
  // the first kB splits and the scalars of the first 64 go out before the row is validated
  load(0);
  const int s_lane = lane;
  const int64_t pr0 = base + int64_t(s_lane) * stride;
  float ls0 = s_lane < S ? ws.part_lse[pr0] : -INFINITY;
  float mx0 = s_lane < S ? ws.part_max[pr0] : -INFINITY;
  int32_t ag0 = s_lane < S && want_arg ? ws.part_arg[pr0] : -1;

  uint32_t bad = 0;
  bool ok = a.bs > 0;
  if (ok) {
    Segment seg;
    bad = owner_segment(a, tabs, t, lane, seg);
    ok = bad == 0 && t >= seg.q0 && t < seg.q0 + seg.T;
    if (bad == 0 && !ok) bad = 8u;  // VA_DEV_TOKENS
    if (ok && !placed) {  // cannot happen: the partial kernel places every valid row
      ok = false;
      bad = 2u;
    }
  } else {
    bad = 8u;
  }
  if (!ok) {
    if (lane == 0) {
      atomicOr(ws.status, bad);
      if (a.out_lse) a.out_lse[row] = -INFINITY;
      if (a.out_argmax) a.out_argmax[row] = -1;
    }
    store4(a, row, dim_a, make_float4(0.f, 0.f, 0.f, 0.f));
    store4(a, row, dim_a + 256, make_float4(0.f, 0.f, 0.f, 0.f));
    return;
  }

  // the row's largest lse and max score over all splits
  float M = ls0, best = mx0;
  for (int s0 = 64; s0 < S; s0 += 64) {
    const int sp = s0 + lane;
    if (sp < S) {
      const int64_t pr = base + int64_t(sp) * stride;
      M = fmaxf(M, ws.part_lse[pr]);
      best = fmaxf(best, ws.part_max[pr]);
    }
  }
  M = wave_max_f32(M);
  best = wave_max_f32(best);

  float W = 0.f;
  int arg = -1;
  float acc[8] = {};
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < S; s0 += 64) {
      const int sp = s0 + lane;
      float ls = ls0, mx = mx0;
      int32_t ag = ag0;
      if (s0 > 0) {
        const int64_t pr = base + int64_t(sp) * stride;
        ls = sp < S ? ws.part_lse[pr] : -INFINITY;
        mx = sp < S ? ws.part_max[pr] : -INFINITY;
        ag = sp < S && want_arg ? ws.part_arg[pr] : -1;
      }
      const float wgt = ls == -INFINITY ? 0.f : expf(ls - M);
      W += wave_sum_f32(wgt);
      if (arg < 0) {  // the lowest split holding the largest max score
        const uint64_t hit = __ballot(sp < S && mx == best);
        if (hit) arg = __builtin_amdgcn_readlane(ag, int(__builtin_ctzll(hit)));
      }
#pragma unroll 1
      for (int j0 = 0; j0 < 64 && s0 + j0 < S; j0 += kB) {
        if (s0 > 0 || j0 > 0) load(s0 + j0);
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          const float wk = lane_f32(wgt, j0 + j);
          // a split with zero weight contributes nothing (its codes may be unwritten)
          if (s0 + j0 + j < S && wk != 0.f) {
            const float fa = wk * sa[j], fb = wk * sb[j];
            const uint32_t w4[4] = {ca[j].x, ca[j].y, cb[j].x, cb[j].y};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t u = w4[e / 2];
              const float v = float((e & 1) ? int32_t(u) >> 16 : int32_t(u << 16) >> 16);
              acc[e] = fmaf(e < 4 ? fa : fb, v, acc[e]);
            }
          }
        }
      }
    }
  }
  const float inv = M == -INFINITY ? 0.f : 1.f / W;
  store4(a, row, dim_a, make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv));
  store4(a, row, dim_a + 256, make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv));
  if (lane == 0) {
    if (a.out_lse) a.out_lse[row] = M == -INFINITY ? -INFINITY : M + logf(W);
    if (a.out_argmax) a.out_argmax[row] = arg;
  }
}

}  // namespace

hipError_t launch_combine(const RunArgs &a, const Workspace &ws, hipStream_t st) {
  const int64_t rows = a.num_tokens * a.H;
  if (rows <= 0) return hipSuccess;
  if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (rows < 512) {
    // few rows: a quarter of a row per workgroup
    if (rows * 4 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (ws.part_i16)
      hipLaunchKernelGGL(combine_few_rows_kernel, dim3(unsigned(rows * 4)), dim3(kThreads), 0,
                         st, a, ws);
    else
      hipLaunchKernelGGL((combine_kernel<16, 4, false>), dim3(unsigned(rows * 4)),
                         dim3(kThreads), 0, st, a, ws);
  } else if (ws.part_i16 && rows > 2048) {
    // many rows, few splits each: a wavefront per row (segmented 28.8 -> 17.7 us, stress
    // 23.8 -> 15.0 us); with up to 2048 rows a row has more splits (long: 32), which the four
    // wavefronts of a workgroup per row read faster (long 11.5 against 13.8 us)
    hipLaunchKernelGGL(combine_rows_kernel<4>, dim3(unsigned((rows + kWaves - 1) / kWaves)),
                       dim3(kThreads), 0, st, a, ws);
  } else if (ws.part_i16) {
    hipLaunchKernelGGL((combine_kernel<2, 1, true>), dim3(unsigned(rows)), dim3(kThreads), 0, st,
                       a, ws);
  } else {
    hipLaunchKernelGGL((combine_kernel<2, 1, false>), dim3(unsigned(rows)), dim3(kThreads), 0,
                       st, a, ws);
  }
  return hipGetLastError();
}

}  // namespace va
