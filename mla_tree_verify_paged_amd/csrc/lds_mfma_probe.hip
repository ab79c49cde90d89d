// lds_mfma_probe.hip - how fast LDS can feed the matrix cores, at one and at two wavefronts
// per SIMD, and what a dependent accumulation chain costs.
//
// Not part of the verify library: a separate measurement library (liblds_mfma_probe.so) that
// bench.py loads for --lds-probe. It backs the partial kernel's design with measurements:
//  * every 32x32x16 bf16 matrix instruction consumes one operand fragment read from LDS D = 4
//    instructions earlier, in the read forms the kernel uses: one ds_read_b128 per
//    instruction (the K-fragment pattern, 1040-byte rows), two ds_read_b64_tr_b16 (the V^T
//    pattern, 1088-byte rows), the two alternating, or both per instruction (2 KB per 32
//    cycles of matrix work, the operand ratio of a 16-row wavefront); and, to tell the two
//    read forms' LDS rates apart where LDS rather than the matrix core sets the pace, 2 KB per
//    instruction of one form only: two b128 reads, or four transposing reads;
//  * one workgroup per compute unit (a 96 KB LDS array forces it) of 256 threads (one
//    wavefront per SIMD) or 512 threads (two);
//  * matrix-core utilisation = matrix cycles per SIMD / the workgroup's elapsed cycles (first
//    wavefront's start to last wavefront's end on the compute unit's cycle counter), the clock
//    taken from the same span on the 100 MHz real-time counter;
//  * a second kernel issues 16 products per iteration into 1, 2 or 4 accumulators with no
//    memory traffic: cycles per product.
// Every LDS address is masked into the 96 KB array; the kernels touch no other memory but
// their small output arrays.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4;
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsBytes = 96 * 1024;
constexpr int kVOff = 40960;  // the V^T-pattern region

enum Form { kB128 = 0, kTr = 1, kAlt = 2, kBoth = 3, kB128x2 = 4, kTrx2 = 5 };
constexpr int kForms = 6;

// The operand of instruction k: K pattern (row lane % 32 at a 1040-byte stride, 16 bytes per
// lane) or V^T pattern (two transposing reads, rows at a 1088-byte stride). Offsets stay
// below 34 KB in each region.
__device__ __forceinline__ u32x4 k_read(const char *lds, int lane, int k) {
  const int row = lane & 31, half = lane >> 5;
  const uint4 v =
      *reinterpret_cast<const uint4 *>(lds + row * 1040 + 16 * half + 32 * (k & 31));
  return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ u32x4 v_read(const char *lds, int lane, int k) {
  const int g = lane & 15, hf = lane >> 5, m0 = 16 * ((lane >> 4) & 1);
  const char *p = lds + kVOff + (4 * hf + (g >> 2)) * 1088 + (m0 + 4 * (g & 3)) * 2 +
                  (k & 1) * 16 * 1088 + 64 * ((k >> 1) & 15);
  const uint2 w0 =
      __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)p));
  const uint2 w1 = __builtin_bit_cast(
      uint2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)(p + 8 * 1088)));
  return u32x4{w0.x, w0.y, w1.x, w1.y};
}
template <int F, int K>
__device__ __forceinline__ u32x4 operand(const char *lds, int lane, int k) {
  if constexpr (F == kB128) return k_read(lds, lane, k);
  else if constexpr (F == kTr) return v_read(lds, lane, k);
  else if constexpr (F == kAlt) return (K & 1) ? v_read(lds, lane, k) : k_read(lds, lane, k);
  else if constexpr (F == kBoth) return k_read(lds, lane, k) ^ v_read(lds, lane, k);
  // the second b128 read: the same pattern in the V region (offsets below kVOff + 34 KB)
  else if constexpr (F == kB128x2) return k_read(lds, lane, k) ^ k_read(lds + kVOff, lane, k + 7);
  else return v_read(lds, lane, k) ^ v_read(lds, lane, k ^ 1);
}

constexpr int kD = 4;  // operand reads in flight

template <int F, int I, int N>
__device__ __forceinline__ void unrolled(const char *lds, int lane, int base, const bf16x8 &b,
                                         u32x4 *a, f32x16 &acc0, f32x16 &acc1) {
  if constexpr (I < N) {
    const bf16x8 av = __builtin_bit_cast(bf16x8, a[I % kD]);
    if constexpr (I & 1) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, acc1, 0, 0, 0);
    else acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, acc0, 0, 0, 0);
    a[I % kD] = operand<F, (I + kD) % 16>(lds, lane, base + I + kD);
    __builtin_amdgcn_sched_barrier(0);
    unrolled<F, I + 1, N>(lds, lane, base, b, a, acc0, acc1);
  }
}

template <int F, int I>
__device__ __forceinline__ void first_reads(const char *lds, int lane, int base, u32x4 *a) {
  if constexpr (I < kD) {
    a[I] = operand<F, I>(lds, lane, base + I);
    first_reads<F, I + 1>(lds, lane, base, a);
  }
}

template <int F>
__global__ void __launch_bounds__(512) feed_kernel(float *sink, unsigned long long *cyc,
                                                   int iters) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kLdsBytes / 16; i += blockDim.x)
    reinterpret_cast<uint4 *>(lds)[i] = make_uint4(i * 3 + 1, i * 5 + 2, i * 7 + 3, i * 11 + 4);
  __syncthreads();
  f32x16 acc0 = {}, acc1 = {};
  const bf16x8 b =
      __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, uint32_t(lane), 0x3e003e00u, 7u});
  u32x4 a[kD];
  first_reads<F, 0>(lds, lane, wave, a);
  const unsigned long long t0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it)
    unrolled<F, 0, 16>(lds, lane, it * 16 + wave, b, a, acc0, acc1);
  const unsigned long long t1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    unsigned long long *c = cyc + 4 * (blockIdx.x * 8 + wave);
    c[0] = t0;
    c[1] = t1;
    c[2] = r0;
    c[3] = r1;
  }
  // keeps the products and the reads alive
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += acc0[e] + acc1[e];
#pragma unroll
  for (int k = 0; k < kD; ++k) s += float(a[k][1] & 1u);
  if (s == 12345.f) sink[blockIdx.x * 512 + threadIdx.x] = s;
}

template <int C>
__global__ void __launch_bounds__(256) chain_kernel(float *sink, unsigned long long *cyc,
                                                    int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x16 acc[4] = {};
  const bf16x8 a =
      __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, uint32_t(lane), 0x3e003e00u, 7u});
  const bf16x8 b =
      __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, uint32_t(wave), 0x3e003e00u, 9u});
  const unsigned long long t0 = __builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      acc[k % C] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k % C], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const unsigned long long t1 = __builtin_readcyclecounter();
  if (lane == 0) cyc[blockIdx.x * 4 + wave] = t1 - t0;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (s == 12345.f) sink[blockIdx.x * 256 + threadIdx.x] = s;
}

constexpr int kBlocks = 256;  // one workgroup per compute unit
constexpr int kIters = 2000;

// One warm-up launch and one measured launch of `launch`; then the cycle words come back.
template <class L>
hipError_t run_twice(L launch, unsigned long long *dcyc, unsigned long long *h, size_t words) {
  hipError_t e = hipSuccess;
  for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {
    launch();
    e = hipGetLastError();
    if (e == hipSuccess) e = hipDeviceSynchronize();
  }
  if (e == hipSuccess)
    e = hipMemcpy(h, dcyc, sizeof(unsigned long long) * words, hipMemcpyDeviceToHost);
  return e;
}

struct Buffers {
  float *sink = nullptr;
  unsigned long long *dcyc = nullptr;
  ~Buffers() {
    if (sink) (void)hipFree(sink);
    if (dcyc) (void)hipFree(dcyc);
  }
};

}  // namespace

// Fills out[0..23] with (matrix-core utilisation %, LDS bytes per clock per compute unit) for
// the forms b128, two tr reads, alternating, b128 + two tr reads, two b128 reads and four tr
// reads per instruction, at one wavefront per SIMD (out[0..11]) and at two (out[12..23]);
// out[24..26]: cycles per product with 1, 2 and 4 accumulation chains; out[27]: the clock in
// GHz during the last feed measurement. Returns 0 or a hipError_t code.
extern "C" int lds_mfma_probe(double *out) {
  Buffers buf;
  hipError_t e = hipMalloc(&buf.sink, size_t(kBlocks) * 512 * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&buf.dcyc, sizeof(unsigned long long) * 4 * kBlocks * 8);
  if (e != hipSuccess) return int(e);
  static unsigned long long h[4 * kBlocks * 8];
  for (int w = 0; w < 2; ++w) {
    const int threads = 256 * (w + 1), waves = threads / 64;
    for (int f = 0; f < kForms; ++f) {
      float *sink = buf.sink;
      unsigned long long *dcyc = buf.dcyc;
      auto launch = [&]() {
        const dim3 g(kBlocks), t(threads);
        if (f == kB128) hipLaunchKernelGGL(feed_kernel<kB128>, g, t, 0, 0, sink, dcyc, kIters);
        else if (f == kTr) hipLaunchKernelGGL(feed_kernel<kTr>, g, t, 0, 0, sink, dcyc, kIters);
        else if (f == kAlt) hipLaunchKernelGGL(feed_kernel<kAlt>, g, t, 0, 0, sink, dcyc, kIters);
        else if (f == kBoth) hipLaunchKernelGGL(feed_kernel<kBoth>, g, t, 0, 0, sink, dcyc, kIters);
        else if (f == kB128x2)
          hipLaunchKernelGGL(feed_kernel<kB128x2>, g, t, 0, 0, sink, dcyc, kIters);
        else hipLaunchKernelGGL(feed_kernel<kTrx2>, g, t, 0, 0, sink, dcyc, kIters);
      };
      if ((e = run_twice(launch, buf.dcyc, h, 4 * kBlocks * 8)) != hipSuccess) return int(e);
      // per workgroup: first start to last end over its wavefronts (one counter per CU)
      double cycles = 0, ticks = 0;
      for (int b = 0; b < kBlocks; ++b) {
        const unsigned long long *c = h + 4 * (b * 8);
        unsigned long long t0 = c[0], t1 = c[1], r0 = c[2], r1 = c[3];
        for (int v = 1; v < waves; ++v) {
          const unsigned long long *cv = h + 4 * (b * 8 + v);
          t0 = cv[0] < t0 ? cv[0] : t0;
          t1 = cv[1] > t1 ? cv[1] : t1;
          r0 = cv[2] < r0 ? cv[2] : r0;
          r1 = cv[3] > r1 ? cv[3] : r1;
        }
        cycles += double(t1 - t0);
        ticks += double(r1 - r0);
      }
      cycles /= kBlocks;
      ticks /= kBlocks;
      out[27] = ticks > 0 ? cycles / (ticks * 10.0) : 0.0;  // the real-time counter is 100 MHz
      const double mfma_cycles = double(waves) / 4 * kIters * 16 * 32;  // per SIMD
      const double kb = f >= kBoth ? 2.0 : 1.0;
      out[2 * kForms * w + 2 * f] = 100.0 * mfma_cycles / cycles;
      out[2 * kForms * w + 2 * f + 1] = kb * 1024.0 * waves * kIters * 16 / cycles;
    }
  }
  for (int c = 0; c < 3; ++c) {
    float *sink = buf.sink;
    unsigned long long *dcyc = buf.dcyc;
    auto launch = [&]() {
      // 96 KB of (unused) dynamic LDS keeps it at one workgroup, one wavefront per SIMD, per CU
      const dim3 g(kBlocks), t(256);
      if (c == 0) hipLaunchKernelGGL(chain_kernel<1>, g, t, kLdsBytes, 0, sink, dcyc, kIters);
      else if (c == 1) hipLaunchKernelGGL(chain_kernel<2>, g, t, kLdsBytes, 0, sink, dcyc, kIters);
      else hipLaunchKernelGGL(chain_kernel<4>, g, t, kLdsBytes, 0, sink, dcyc, kIters);
    };
    if ((e = run_twice(launch, buf.dcyc, h, kBlocks * 4)) != hipSuccess) return int(e);
    double cycles = 0;
    for (int i = 0; i < kBlocks * 4; ++i) cycles += double(h[i]);
    out[4 * kForms + c] = cycles / (kBlocks * 4) / (kIters * 16.0);
  }
  return 0;
}
