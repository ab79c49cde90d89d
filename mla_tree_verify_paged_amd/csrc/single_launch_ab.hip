// single_launch_ab.hip - the fixed costs a single-launch (fused) split-K merge would pay.
//
// Not part of the verify library: a separate measurement library (libsingle_launch_ab.so)
// that bench.py loads for its single-launch A/B. A fused merge (every workgroup writes its
// key split's partial, then the workgroups merge the rows) needs all workgroups resident
// at once and a grid-wide barrier between the two phases. On this GPU that means a
// cooperative launch (the only launch that guarantees co-residency, and the pages' final
// interface names a capture-safe cooperative-groups launch: "The Final Solder Joint", section
// "The Three-Edits Sequence") plus one grid barrier. This file measures both on a kernel with
// the partial kernel's shape (one 256-thread workgroup per compute unit, about 150 KB of LDS):
//   * a plain launch and a cooperative launch of a kernel that only touches its LDS;
//   * the same kernel with 1 and with 33 grid barriers (per-barrier cost by difference);
//   * whether the cooperative launch records into a graph and replays correctly.
// The barrier is hierarchical (8 group counters on separate cache lines, then one counter of
// the 8 group winners, then a generation word), polls with relaxed loads and orders memory
// with agent-scope release/acquire fences. Every spin is bounded: a workgroup that polls 2^22
// times gives up and counts a timeout, so every wave ends whatever the residency.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr int kLdsBytes = 150 * 1024;

__device__ void grid_barrier(uint32_t *bar, uint32_t nblocks) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t gen = __hip_atomic_load(&bar[288], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t ng = nblocks < 8 ? nblocks : 8;
    const uint32_t g = blockIdx.x % ng;
    const uint32_t in_g = (nblocks - g + ng - 1) / ng;
    bool last = false;
    if (__hip_atomic_fetch_add(&bar[32 * g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        in_g - 1) {
      __hip_atomic_store(&bar[32 * g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(&bar[256], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
          ng - 1) {
        __hip_atomic_store(&bar[256], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(&bar[288], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        last = true;
      }
    }
    if (!last) {
      uint32_t polls = 0;
      while (__hip_atomic_load(&bar[288], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        if (++polls > (1u << 22)) {
          __hip_atomic_fetch_add(&bar[290], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// Each workgroup writes a word, crosses the barrier, and checks the word another workgroup
// (usually on another XCD) wrote before it: bar[291] counts mismatches.
__global__ void __launch_bounds__(256) barrier_kernel(uint32_t *bar, uint32_t *data, int barriers,
                                                      uint32_t round) {
  __shared__ char lds[kLdsBytes];
  const uint32_t n = gridDim.x, b = blockIdx.x;
  lds[threadIdx.x] = char(b);
  for (int k = 0; k < barriers; ++k) {
    if (threadIdx.x == 0) data[b * 32] = round * 7919u + uint32_t(k) * 131u + b;
    grid_barrier(bar, n);
    const uint32_t o = (b + 1) % n;
    if (threadIdx.x == 0 && data[o * 32] != round * 7919u + uint32_t(k) * 131u + o)
      __hip_atomic_fetch_add(&bar[291], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    grid_barrier(bar, n);  // the next round's writes wait for every check
  }
  if (lds[threadIdx.x] != char(b))
    __hip_atomic_fetch_add(&bar[291], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

double time_us(hipStream_t s, hipEvent_t e0, hipEvent_t e1, int reps, bool coop, dim3 grid,
               uint32_t *bar, uint32_t *data, int barriers, hipError_t *err) {
  uint32_t round = 1;
  void *args[] = {&bar, &data, &barriers, &round};
  *err = hipEventRecord(e0, s);
  for (int i = 0; i < reps && *err == hipSuccess; ++i) {
    round = uint32_t(i + 2);
    if (coop)
      *err = hipLaunchCooperativeKernel((const void *)barrier_kernel, grid, dim3(256), args, 0, s);
    else
      hipLaunchKernelGGL(barrier_kernel, grid, dim3(256), 0, s, bar, data, barriers, round);
    if (*err == hipSuccess) *err = hipGetLastError();
  }
  if (*err == hipSuccess) *err = hipEventRecord(e1, s);
  if (*err == hipSuccess) *err = hipEventSynchronize(e1);
  float ms = 0.f;
  if (*err == hipSuccess) *err = hipEventElapsedTime(&ms, e0, e1);
  return double(ms) * 1e3 / reps;
}

}  // namespace

namespace {

// Owns the measurement's device resources, released on every return path.
struct Resources {
  uint32_t *bar = nullptr, *data = nullptr;
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipGraph_t g = nullptr;
  hipGraphExec_t ge = nullptr;
  ~Resources() {
    if (ge) (void)hipGraphExecDestroy(ge);
    if (g) (void)hipGraphDestroy(g);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (s) (void)hipStreamDestroy(s);
    if (bar) (void)hipFree(bar);
    if (data) (void)hipFree(data);
  }
};

}  // namespace

// Fills out[0..7]: plain launch (no barrier) us, cooperative launch (no barrier) us,
// cooperative with one barrier pair us, cooperative with 33 barrier pairs us, graph replay of a
// captured cooperative launch with one barrier pair us, barrier timeouts, visibility
// mismatches, graph capture worked (1/0). Returns 0 or a hipError_t code.
extern "C" int single_launch_ab(double *out) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return int(e);
  Resources r;
  if ((e = hipMalloc(&r.bar, 4096)) != hipSuccess) return int(e);
  if ((e = hipMalloc(&r.data, size_t(cus) * 128)) != hipSuccess) return int(e);
  if ((e = hipMemset(r.bar, 0, 4096)) != hipSuccess) return int(e);
  if ((e = hipStreamCreate(&r.s)) != hipSuccess) return int(e);
  if ((e = hipEventCreate(&r.e0)) != hipSuccess) return int(e);
  if ((e = hipEventCreate(&r.e1)) != hipSuccess) return int(e);
  const dim3 grid(static_cast<unsigned>(cus), 1, 1);
  time_us(r.s, r.e0, r.e1, 3, true, grid, r.bar, r.data, 1, &e);  // warm-up
  if (e != hipSuccess) return int(e);
  out[0] = time_us(r.s, r.e0, r.e1, 20, false, grid, r.bar, r.data, 0, &e);
  if (e == hipSuccess) out[1] = time_us(r.s, r.e0, r.e1, 20, true, grid, r.bar, r.data, 0, &e);
  if (e == hipSuccess) out[2] = time_us(r.s, r.e0, r.e1, 20, true, grid, r.bar, r.data, 1, &e);
  if (e == hipSuccess) out[3] = time_us(r.s, r.e0, r.e1, 5, true, grid, r.bar, r.data, 33, &e);
  if (e != hipSuccess) return int(e);
  // graph capture of the cooperative launch
  out[7] = 0.0;
  out[4] = -1.0;
  int barriers = 1;
  uint32_t round = 99;
  void *args[] = {&r.bar, &r.data, &barriers, &round};
  if ((e = hipStreamBeginCapture(r.s, hipStreamCaptureModeGlobal)) != hipSuccess) return int(e);
  const hipError_t ce =
      hipLaunchCooperativeKernel((const void *)barrier_kernel, grid, dim3(256), args, 0, r.s);
  e = hipStreamEndCapture(r.s, &r.g);
  if (ce == hipSuccess && e == hipSuccess &&
      hipGraphInstantiate(&r.ge, r.g, nullptr, nullptr, 0) == hipSuccess) {
    bool ok = true;
    for (int i = 0; i < 3 && ok; ++i) ok = hipGraphLaunch(r.ge, r.s) == hipSuccess;
    ok = ok && hipStreamSynchronize(r.s) == hipSuccess;
    if (ok && hipEventRecord(r.e0, r.s) == hipSuccess) {
      for (int i = 0; i < 20 && ok; ++i) ok = hipGraphLaunch(r.ge, r.s) == hipSuccess;
      float ms = 0.f;
      if (ok && hipEventRecord(r.e1, r.s) == hipSuccess && hipEventSynchronize(r.e1) == hipSuccess &&
          hipEventElapsedTime(&ms, r.e0, r.e1) == hipSuccess) {
        out[4] = double(ms) * 1e3 / 20;
        out[7] = 1.0;
      }
    }
  } else {
    (void)hipGetLastError();
  }
  uint32_t h[4] = {0, 0, 0, 0};
  if ((e = hipStreamSynchronize(r.s)) != hipSuccess) return int(e);
  if ((e = hipMemcpy(h, r.bar + 288, 16, hipMemcpyDeviceToHost)) != hipSuccess) return int(e);
  out[5] = h[2];
  out[6] = h[3];
  return 0;
}
