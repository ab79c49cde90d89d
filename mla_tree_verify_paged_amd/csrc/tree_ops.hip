// tree_ops.hip - the steps around verify attention that work on the draft trees themselves:
// building the verify mask from the parent array, and greedy acceptance.
//
// The library that exposes verify attention also exposes tree building and tree acceptance
// ("The Glue That Connects: Wiring a Custom Flash Attention Kernel into the C-ABI Layer",
// section "What the Edit Actually Does"); the mask is rebuilt from the tree structure rather
// than decoded from a packed format ("The Glue That Binds: Wiring a Custom CUDA Kernel into
// Production via C-ABI", section "The Thinking Process"). The acceptance rule is the plain
// greedy one (no algorithm is given): from the root, follow the lowest-indexed child whose
// draft token equals the target's token at the current node.
//
// Both are small integer kernels: every output is exact.
#include <algorithm>

#include "va_internal.h"

namespace va {
namespace {

constexpr int kMaskThreads = 256;

// (T, L, P) of request r for either slot layout; false if the segment is not usable.
__device__ __forceinline__ bool tree_shape(const TreeArgs &a, int r, int64_t &q0, int32_t &T,
                                           int32_t &L, int32_t &P) {
  q0 = a.qo_indptr[r];
  const int64_t q1 = a.qo_indptr[r + 1];
  const int64_t n = int64_t(a.kv_indptr[r + 1]) - int64_t(a.kv_indptr[r]);
  const int64_t t = q1 - q0;
  const int64_t l = a.split_layout ? n + t : n;
  if (t < 0 || n < 0 || q0 < 0 || q1 > a.num_tokens || l < t || l > INT32_MAX ||
      t > a.max_q_per_req)
    return false;
  T = int32_t(t);
  L = int32_t(l);
  P = int32_t(l - t);
  return true;
}

// Segment length T_r * L_r of request r in the mask (0 for an unusable request).
__device__ __forceinline__ int64_t mask_segment(const TreeArgs &a, int r) {
  int64_t q0;
  int32_t T, L, P;
  return tree_shape(a, r, q0, T, L, P) ? int64_t(T) * L : 0;
}

// Sum of mask_segment over requests [0, r), by all threads of the workgroup.
__device__ int64_t mask_offset(const TreeArgs &a, int r, int64_t *red) {
  int64_t v = 0;
  for (int k = int(threadIdx.x); k < r; k += kMaskThreads) v += mask_segment(a, k);
  v = wave_sum_i64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t s = 0;
#pragma unroll
  for (int w = 0; w < kMaskThreads / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

// mask_indptr[r+1] = sum over requests <= r of T_r * L_r (workgroup 0 of the mask build).
__device__ void write_mask_indptr(const TreeArgs &a, int64_t *part) {
  int64_t carry = 0;
  if (threadIdx.x == 0) a.mask_indptr[0] = 0;
  for (int base = 0; base < a.bs; base += kMaskThreads) {
    const int r = base + int(threadIdx.x);
    part[threadIdx.x] = r < a.bs ? mask_segment(a, r) : 0;
    __syncthreads();
    // inclusive scan (Hillis-Steele)
    for (int o = 1; o < kMaskThreads; o <<= 1) {
      const int64_t x = threadIdx.x >= unsigned(o) ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += x;
      __syncthreads();
    }
    if (r < a.bs) a.mask_indptr[r + 1] = carry + part[threadIdx.x];
    carry += part[kMaskThreads - 1];
    __syncthreads();
  }
}

// The whole mask build in one launch: one workgroup per mask row (tree token t). With
// write_indptr, each workgroup derives its row's segment offset itself (a reduction over the
// requests before its own) and workgroup 0 also writes mask_indptr, so no separate scan
// launch precedes the rows.
template <bool kWriteIndptr>
__global__ void __launch_bounds__(kMaskThreads) build_mask_kernel(TreeArgs a) {
  extern __shared__ int32_t tree_smem[];  // parents [max_q_per_req], then ancestor flags
  __shared__ int64_t scan[kMaskThreads];
  int32_t *par = tree_smem;
  int32_t *anc = tree_smem + a.max_q_per_req;
  const int64_t t = blockIdx.x;
  if (kWriteIndptr && blockIdx.x == 0) write_mask_indptr(a, scan);
  if (t >= a.num_tokens) return;
  // the request that owns token t: the last r with qo_indptr[r] <= t
  int lo = 0, hi = a.bs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.qo_indptr[mid] <= t) lo = mid; else hi = mid;
  }
  int64_t q0;
  int32_t T, L, P;
  bool ok = a.bs > 0 && tree_shape(a, lo, q0, T, L, P) && t >= q0 && t < q0 + T;
  int64_t m0 = 0;
  if (kWriteIndptr) {
    m0 = mask_offset(a, ok ? lo : 0, scan);  // every thread of the workgroup takes part
  } else if (ok) {
    m0 = a.mask_indptr[lo];
  }
  // (T <= 2048 and L <= INT32_MAX: T * L cannot overflow, nor can mask_len - T * L)
  if (ok && (m0 < 0 || m0 > a.mask_len - int64_t(T) * L)) ok = false;
  if (!ok) {
    if (threadIdx.x == 0) atomicOr(a.status, 2u);  // VA_DEV_SEGMENT: row not written
    return;
  }
  const int i = int(t - q0);
  for (int k = threadIdx.x; k < T; k += kMaskThreads) {
    const int64_t p = a.parents[q0 + k];
    par[k] = (p >= -1 && p < k) ? int32_t(p) : -2;  // -2: does not precede its child
    anc[k] = 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int node = i;
    bool bad = false;
    for (int steps = 0; steps <= T && node >= 0; ++steps) {
      anc[node] = 1;
      const int p = par[node];
      if (p == -2) { bad = true; break; }
      node = p;
    }
    if (bad) atomicOr(a.status, 16u);  // VA_DEV_TREE
  }
  __syncthreads();

  uint8_t *row = a.mask + m0 + int64_t(i) * L;
  // prefix columns: ones, 16 bytes per store once the address is aligned
  const int head = min(int((16 - (reinterpret_cast<uintptr_t>(row) & 15)) & 15), P);
  for (int x = threadIdx.x; x < head; x += kMaskThreads) row[x] = 1;
  const int body = (P - head) / 16;
  uint4 *row16 = reinterpret_cast<uint4 *>(row + head);
  for (int x = threadIdx.x; x < body; x += kMaskThreads)
    row16[x] = make_uint4(0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u);
  for (int x = head + 16 * body + int(threadIdx.x); x < P; x += kMaskThreads) row[x] = 1;
  // tree columns: node k is visible iff it is node i or one of its ancestors
  for (int k = threadIdx.x; k < T; k += kMaskThreads) row[P + k] = uint8_t(anc[k]);
}

// One wavefront per request.
__global__ void __launch_bounds__(64) accept_kernel(AcceptArgs a) {
  extern __shared__ int64_t acc_smem[];  // parents, draft and target tokens [max_q_per_req]
  int64_t *par = acc_smem;
  int64_t *drf = acc_smem + a.max_q_per_req;
  int64_t *tgt = acc_smem + 2 * a.max_q_per_req;
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t q0 = a.qo_indptr[r], q1 = a.qo_indptr[r + 1];
  const int64_t tt = q1 - q0;
  int64_t *path = a.accept_path + int64_t(r) * a.max_path;
  const bool ok = tt >= 0 && q0 >= 0 && q1 <= a.num_tokens && tt <= a.max_q_per_req;
  if (!ok || tt == 0) {
    if (!ok && lane == 0) atomicOr(a.status, 2u);  // VA_DEV_SEGMENT
    for (int k = lane; k < a.max_path; k += 64) path[k] = -1;
    if (lane == 0) {
      a.accept_len[r] = 0;
      a.next_token[r] = -1;
    }
    return;
  }
  const int T = int(tt);
  bool bad = false;
  for (int k = lane; k < T; k += 64) {
    const int64_t p = a.parents[q0 + k];
    bad |= p < -1 || p >= k;  // a parent must precede its child
    par[k] = p;
    drf[k] = a.draft_tokens[q0 + k];
    tgt[k] = a.target_tokens[q0 + k];
  }
  if (__ballot(bad) != 0 && lane == 0) atomicOr(a.status, 16u);  // VA_DEV_TREE
  __syncthreads();
  // With parents preceding children every step moves to a higher node, so the walk ends
  // within T steps; the bound also ends it on a malformed tree (whose output is unspecified).
  int cur = 0, len = 0;
  if (lane == 0 && a.max_path > 0) path[0] = 0;
  for (int steps = 0; steps < T; ++steps) {
    const int64_t want = tgt[cur];
    int best = 0x7fffffff;
    for (int c = lane; c < T; c += 64)
      if (par[c] == cur && drf[c] == want) best = min(best, c);
    best = wave_min_i32(best);
    if (best == 0x7fffffff) break;
    cur = best;
    ++len;
    if (lane == 0 && len < a.max_path) path[len] = cur;
  }
  for (int k = len + 1 + lane; k < a.max_path; k += 64) path[k] = -1;
  if (lane == 0) {
    a.accept_len[r] = len;
    a.next_token[r] = tgt[cur];
  }
}

}  // namespace

hipError_t launch_build_mask(const TreeArgs &a, bool write_indptr, hipStream_t st) {
  if (a.num_tokens > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // one workgroup per mask row; at least one to write mask_indptr when asked
  const int64_t grid = std::max<int64_t>(a.num_tokens, write_indptr ? 1 : 0);
  if (grid == 0) return hipSuccess;
  const size_t smem = size_t(2) * a.max_q_per_req * sizeof(int32_t);
  if (write_indptr)
    hipLaunchKernelGGL(build_mask_kernel<true>, dim3(unsigned(grid)), dim3(kMaskThreads), smem,
                       st, a);
  else
    hipLaunchKernelGGL(build_mask_kernel<false>, dim3(unsigned(grid)), dim3(kMaskThreads), smem,
                       st, a);
  return hipGetLastError();
}

hipError_t launch_accept(const AcceptArgs &a, hipStream_t st) {
  if (a.bs <= 0) return hipSuccess;
  const size_t smem = size_t(3) * a.max_q_per_req * sizeof(int64_t);
  hipLaunchKernelGGL(accept_kernel, dim3(unsigned(a.bs)), dim3(64), smem, st, a);
  return hipGetLastError();
}

}  // namespace va
