// va_internal.h - declarations shared by the library's translation units (not installed).
//
// Workspace layout (all offsets 256-byte aligned), for a capacity of N partial rows and
// R = max_q_tokens * H output rows:
//   status   uint32 [64]            sticky VA_DEV_* bits in word 0
//   zero_row uint16 [576]           zeros; key rows that must not be read load from here
//   part_o                          per-split normalised output O_s, in one of two formats:
//            float  [N][512]          fp32 (the fp32-input kernel), or
//            int16  [N][512]          16-bit signed-normalised codes (the bf16 MFMA kernel):
//                                     O_s[d] = code[d] * part_scale[4 * p + d / 128]
//   part_scale float [N][4]         the code scale of each 128-dim group (int16 format only)
//   part_lse float  [N]             per-split log-sum-exp (natural log); -inf for an empty split
//   part_max float  [N]             per-split max score (natural-log units)
//   part_arg int32  [N]             per-split argmax key position (-1 when empty)
//   row_info RowInfo [R]            where output row x's partials are (see RowInfo)
// Request r's partials are one block of n_r * R_r rows (R_r = T_r * H): split k of its local
// row x is partial row base_r + k * R_r + x. The partial kernel writes, for every valid
// request, all n_r splits of every row and the row_info of every row.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace va {

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kDim = kLatent + kRope;  // 576
constexpr int kMaxSplits = 256;

// Where the partials of one output row are: split k (k < n) is partial row base + k * stride.
struct RowInfo {
  int64_t base;
  int32_t n;
  int32_t stride;
};

struct Workspace {
  uint32_t *status;
  const uint16_t *zero_row;
  void *part_o;        // float [N][512] or int16 [N][512] (part_i16)
  float *part_scale;   // [N][4], int16 format only
  int32_t part_i16;    // 1: partial outputs are int16 codes with a scale per 128 dims
  float *part_lse;
  float *part_max;
  int32_t *part_arg;
  RowInfo *row_info;
  int64_t part_rows;  // N, the partial rows the workspace holds
  int64_t rows_cap;   // R
  int32_t splits;     // key splits per request; 0: chosen per call on the device (MFMA)
};

// Arguments of one verify step, as the kernels see them.
struct RunArgs {
  const void *q;
  const void *kv;
  int64_t num_slots;
  const int64_t *kv_indices;
  int64_t num_kv_indices;
  const int64_t *out_cache_loc;  // NULL: tree slots end each kv_indices segment
  const int32_t *kv_indptr;
  const int64_t *qo_indptr;
  const uint8_t *mask;
  int64_t mask_len;
  const int64_t *mask_indptr;
  int32_t bs;
  int64_t num_tokens;
  int32_t H;
  int32_t max_q_per_req;
  float scale;  // natural-log units
  void *out;
  float *out_lse;
  int32_t *out_argmax;
  int32_t out_bf16;
  int32_t want_argmax;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The status words and the zero row, set to zero when a context is created.
constexpr size_t kStatusBytes = 64 * sizeof(uint32_t);
constexpr size_t kZeroRowOffset = kStatusBytes;
constexpr size_t kHeaderBytes = kZeroRowOffset + kDim * sizeof(uint16_t);

// Groups of 128 output dims that share one code scale in the int16 partial format.
constexpr int kScaleGroups = 4;
constexpr int kScaleGroupDims = kLatent / kScaleGroups;

// Byte offsets of the workspace regions for N partial rows and R output rows, with partial
// outputs of `elem_bytes` (4: fp32, 2: int16 codes) per dim; returns the total size.
inline size_t workspace_layout(int64_t N, int64_t R, int elem_bytes, size_t off[7]) {
  size_t o = 0;
  off[0] = o; o = align256(o + kHeaderBytes);
  off[1] = o; o = align256(o + size_t(N) * kLatent * size_t(elem_bytes));
  off[2] = o; o = align256(o + size_t(N) * kScaleGroups * sizeof(float));
  off[3] = o; o = align256(o + size_t(N) * sizeof(float));
  off[4] = o; o = align256(o + size_t(N) * sizeof(float));
  off[5] = o; o = align256(o + size_t(N) * sizeof(int32_t));
  off[6] = o; o = align256(o + size_t(R) * sizeof(RowInfo));
  return o;
}

// Per-request segment validation shared by every kernel (device side). Sets *T, *L, bases,
// and returns a VA_DEV_* bit (0 when the segment is usable).
struct Segment {
  int64_t q0;     // first token
  int32_t T;      // tree tokens
  int32_t L;      // keys
  int32_t P;      // prefix keys
  int64_t kv0;    // first kv_indices entry
  int64_t m0;     // first mask byte
  // the slots of the tree keys (key P + k in slot tree[k]) when they come from
  // out_cache_loc, else NULL (they are kv_indices[kv0 + P + k])
  const int64_t *tree;
};

// Request r's segment from its index-table entries qo_indptr[r], qo_indptr[r + 1],
// kv_indptr[r], kv_indptr[r + 1] and mask_indptr[r]; returns the VA_DEV_* bits of an unusable
// segment (then T = L = P = 0), else 0.
__device__ __forceinline__ uint32_t check_segment(const RunArgs &a, int64_t q0, int64_t q1,
                                                  int64_t k0, int64_t k1, int64_t m0,
                                                  Segment &s) {
  s.q0 = q0;
  s.kv0 = k0;
  s.m0 = m0;
  s.tree = nullptr;
  const int64_t T = q1 - q0, n = k1 - k0;
  // the split layout: kv_indices holds the prefix, out_cache_loc[q0 .. q1) the tree slots
  const int64_t L = a.out_cache_loc ? n + T : n;
  s.T = 0; s.L = 0; s.P = 0;
  // (T <= num_tokens < 2^26 and L <= INT32_MAX, so T * L cannot overflow; the mask bound is
  // tested as m0 > mask_len - T * L, which cannot overflow either, whatever m0 holds)
  if (T < 0 || n < 0 || q0 < 0 || q1 > a.num_tokens || k0 < 0 || k1 > a.num_kv_indices ||
      L < T || L > INT32_MAX || m0 < 0 || T * L > INT32_MAX ||
      (T > 0 && m0 > a.mask_len - T * L))
    return 2u;  // VA_DEV_SEGMENT (a request's mask segment must stay under 2 GiB)
  if (T > a.max_q_per_req) return 4u;  // VA_DEV_Q_PER_REQ
  s.T = int32_t(T);
  s.L = int32_t(L);
  s.P = int32_t(L - T);
  if (a.out_cache_loc) s.tree = a.out_cache_loc + q0;
  return 0u;
}

__device__ __forceinline__ uint32_t load_segment(const RunArgs &a, int r, Segment &s) {
  return check_segment(a, a.qo_indptr[r], a.qo_indptr[r + 1], a.kv_indptr[r],
                       a.kv_indptr[r + 1], a.mask_indptr[r], s);
}

// Arguments of the mask build (see include/verify_attn.h).
struct TreeArgs {
  const int64_t *parents;
  const int64_t *qo_indptr;
  const int32_t *kv_indptr;
  int32_t split_layout;  // kv_indptr counts prefix keys only (tree slots in out_cache_loc)
  int32_t bs;
  int64_t num_tokens;
  int32_t max_q_per_req;
  uint8_t *mask;
  int64_t mask_len;
  int64_t *mask_indptr;
  uint32_t *status;
};

// Arguments of the greedy acceptance.
struct AcceptArgs {
  const int64_t *parents;
  const int64_t *draft_tokens;
  const int64_t *target_tokens;
  const int64_t *qo_indptr;
  int32_t bs;
  int64_t num_tokens;
  int32_t max_q_per_req;
  int32_t *accept_len;
  int64_t *accept_path;
  int32_t max_path;
  int64_t *next_token;
  uint32_t *status;
};

// Largest tree the tree kernels stage in LDS.
constexpr int kMaxTreeNodes = 2048;

// Slot of key position j (0 <= j < L) of a validated segment.
__device__ __forceinline__ int64_t segment_slot(const RunArgs &a, const Segment &s, int j) {
  return (s.tree && j >= s.P) ? s.tree[j - s.P] : a.kv_indices[s.kv0 + j];
}

// The allocation-free entry point's workspace: a static device array of this many bytes per
// GPU (static_scratch.hip). static_scratch() returns its device address on the current device,
// setting it up (address lookup, header cleared on `stream`) on the first call there.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(hipStream_t stream, void **base);

// ---- cross-lane work within a wavefront without LDS round trips (a __shfl is an LDS
// permute whose result is waited for, so a chain of them serialises on LDS latency)
//
// DPP operands (kCtrl): quad_perm 0xB1 = lane ^ 1, 0x4E = lane ^ 2; 0x141 and 0x140 = the
// lane mirrored within 8 and within 16 lanes; 0x111..0x118 = the lane 1..8 places lower in
// its 16-lane row (zero, with kBound, where that lies before the row); 0x142 and 0x143 =
// row_bcast:15 and :31 (the last lane of the row before, and lane 31, into the rows kRowMask
// enables; disabled rows read zero).
template <int kCtrl, int kRowMask = 0xf, bool kBound = false>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xf, kBound);
}
template <int kCtrl, int kRowMask = 0xf, bool kBound = false>
__device__ __forceinline__ int64_t dpp_i64(int64_t v) {
  const uint32_t lo = uint32_t(dpp_i32<kCtrl, kRowMask, kBound>(int(uint32_t(uint64_t(v)))));
  const uint32_t hi = uint32_t(dpp_i32<kCtrl, kRowMask, kBound>(int(uint32_t(uint64_t(v) >> 32))));
  return int64_t((uint64_t(hi) << 32) | lo);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_i32<kCtrl>(__builtin_bit_cast(int, v)));
}
// lane l's value (l wave-uniform), in scalar registers
__device__ __forceinline__ int lane_i32(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ int64_t lane_i64(int64_t v, int l) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(uint64_t(v))), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(uint64_t(v) >> 32)), l));
  return int64_t((uint64_t(hi) << 32) | lo);
}
// Wavefront sums, maxima and minima: a butterfly within each 16-lane row (each step leaves
// groups of 2, 4, 8, 16 lanes equal), then the four rows' values. The result is the same in
// every lane, and in every wavefront that holds the same values in the same lanes.
__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
  v += dpp_i64<0xB1>(v);
  v += dpp_i64<0x4E>(v);
  v += dpp_i64<0x141>(v);
  v += dpp_i64<0x140>(v);
  return (lane_i64(v, 0) + lane_i64(v, 16)) + (lane_i64(v, 32) + lane_i64(v, 48));
}
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, dpp_i32<0xB1>(v));
  v = max(v, dpp_i32<0x4E>(v));
  v = max(v, dpp_i32<0x141>(v));
  v = max(v, dpp_i32<0x140>(v));
  return max(max(lane_i32(v, 0), lane_i32(v, 16)), max(lane_i32(v, 32), lane_i32(v, 48)));
}
__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, dpp_i32<0xB1>(v));
  v = min(v, dpp_i32<0x4E>(v));
  v = min(v, dpp_i32<0x141>(v));
  v = min(v, dpp_i32<0x140>(v));
  return min(min(lane_i32(v, 0), lane_i32(v, 16)), min(lane_i32(v, 32), lane_i32(v, 48)));
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}
// Inclusive prefix sum over the lanes: shifts by 1, 2, 4 and 8 within each 16-lane row, then
// the last lane of rows 0 and 2 added to rows 1 and 3, then lane 31's total to rows 2 and 3.
__device__ __forceinline__ int64_t wave_inclusive_scan_i64(int64_t v) {
  v += dpp_i64<0x111, 0xf, true>(v);
  v += dpp_i64<0x112, 0xf, true>(v);
  v += dpp_i64<0x114, 0xf, true>(v);
  v += dpp_i64<0x118, 0xf, true>(v);
  v += dpp_i64<0x142, 0xa, false>(v);
  v += dpp_i64<0x143, 0xc, false>(v);
  return v;
}

// Launchers (each defined next to its kernels).
hipError_t launch_simple_partial(const RunArgs &a, const Workspace &ws, int in_fp32,
                                 hipStream_t st);
hipError_t launch_mfma_partial(const RunArgs &a, const Workspace &ws, int rows_per_block,
                               int grid, hipStream_t st);
hipError_t launch_combine(const RunArgs &a, const Workspace &ws, hipStream_t st);
hipError_t launch_build_mask(const TreeArgs &a, bool write_indptr, hipStream_t st);
hipError_t launch_accept(const AcceptArgs &a, hipStream_t st);

// Rows per workgroup of each partial kernel (fixes the grid).
constexpr int kSimpleHeadsPerBlock = 4;
constexpr int kMfmaRowsPerBlock = 128;
// Wavefronts of an MFMA partial workgroup: with H a multiple of 64 a row tile holds 64 or 128
// rows, never 32 or fewer, and the 8-wavefront (two per SIMD) variant runs; otherwise the
// 4-wavefront one, which also has the path for items of at most 32 rows.
constexpr int mfma_partial_waves(int num_heads) { return num_heads % 64 == 0 ? 8 : 4; }

}  // namespace va
