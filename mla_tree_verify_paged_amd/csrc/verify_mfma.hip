// verify_mfma.hip - bf16-input split-K partial kernel on gfx950 matrix cores.
//
// What it computes is the split-K flash decode over paged latent rows with a prefix-plus-
// tree mask ("The Glue That Makes Kernels Run: A Study in Architectural Discipline", section
// "The Context: A Custom Kernel in Flight"): for one key split of one request, the normalised
// partial output, log-sum-exp, max score and argmax of every (token, head) row.
//
// The pages' sm_120 kernel tiled 8 heads per block against a shared-memory latent tile so one
// global read served K and V of several heads ("The Glue That Connects", section "Design
// Decisions and Trade-Offs"; "The Quiet Art of Integration", section "The Context: What Led
// Here"). Here the same reuse is taken much further, the gfx950 way:
//  * a workgroup of 4 wavefronts owns 128 (token, head) rows - with H=64 every head of two
//    tree tokens - so one LDS copy of a key tile serves 128 rows;
//  * key tiles (32 paged latent rows) arrive in LDS by direct global->LDS 16-byte loads
//    (global_load_lds_dwordx4), one tile ahead of the compute, without passing through
//    registers: one load instruction moves the 1 KB latent part of one row, so the row and
//    its slot are wave-uniform and the slots come in through scalar loads. Rows are stored
//    XOR-swizzled in 16-byte units so the K-fragment reads are free of LDS bank conflicts;
//  * S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16: A = key rows from LDS, B = the wave's 32
//    query rows held in registers. The accumulator gives each lane one row and 16 keys, so a
//    softmax row reduction is one cross-lane swap;
//  * P is rounded (to nearest even) to fp16 and O^T += V^T P^T runs on v_mfma_f32_32x32x16_f16. V is the first
//    512 dims of the same rows, converted to fp16 by the thread that loaded each unit while
//    the previous tile's products run, and read as V^T fragments with ds_read_b64_tr_b16.
//    The P fragment is the S accumulator itself: key slots are permuted the same way in both
//    operands;
//  * the running max is rescaled lazily (only when it grows by more than 2^8), in place in
//    the accumulation registers, so the 256 fp32 accumulators per lane never leave them;
//  * workgroups are mapped so that all row tiles of one key split run on the same XCD and
//    share its L2; HBM then sees each latent row about once.
#include <math.h>

#include "va_internal.h"

namespace va {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__fp16)))) __fp16 fp16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = kMfmaRowsPerBlock;    // 128 rows = 4 waves x 32
constexpr int kTK = 32;                     // keys per tile
constexpr int kRowsPerWave = kTK / kWaves;  // 8 key rows staged by each wave
constexpr int kLatRow = kLatent * 2;        // 1024 bytes of latent per key row
constexpr int kRopeRow = kRope * 2;         // 128 bytes of rope per key row
constexpr int kLatTile = kTK * kLatRow;     // 32 KB
constexpr int kRawTile = kLatTile + kTK * kRopeRow;  // + 4 KB = 36 KB
constexpr int kVRow = kLatent * 2 + 64;     // fp16 V tile row stride: 1088 bytes
constexpr int kVTile = kTK * kVRow;         // 34,816 bytes
constexpr int kQFrags = kDim / 16;          // 36 bf16x8 B-operand fragments per lane
constexpr int kLatFrags = kLatent / 16;     // the first 32 of them are latent dims
constexpr int kDBlocks = kLatent / 32;      // 16 output dim blocks of 32
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;            // lazy-rescale threshold (log2 units)
constexpr int kKPrefetch = 7;               // K-fragment LDS reads kept in flight per wave
constexpr int kVPrefetch = 8;               // V-fragment (pairs of transposed) reads in flight

static_assert(kRowsPerWave == 8, "one rope load instruction covers 8 rows");

// LDS: two tile buffers, each a raw bf16 tile (latent rows, then rope rows, both swizzled)
// plus its fp16 latent copy; and the usable-key bits of the tiles in flight (a byte per wave).
__shared__ __attribute__((aligned(16))) char g_raw0[kRawTile];
__shared__ __attribute__((aligned(16))) char g_raw1[kRawTile];
__shared__ __attribute__((aligned(16))) char g_v0[kVTile];
__shared__ __attribute__((aligned(16))) char g_v1[kVTile];
__shared__ uint32_t g_okbits[2];

template <int B> __device__ __forceinline__ char *raw_buf() { return B ? g_raw1 : g_raw0; }
template <int B> __device__ __forceinline__ char *v_buf() { return B ? g_v1 : g_v0; }

// Swizzles (16-byte unit index within a row): latent units XOR (row & 15), rope units XOR
// ((row >> 1) & 7). Both keep a unit inside its aligned group.
__device__ __forceinline__ int lat_swz(int row) { return row & 15; }
__device__ __forceinline__ int rope_swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ uint32_t bf16pair_to_f16pair(uint32_t w) {
  const float lo = __uint_as_float(w << 16);
  const float hi = __uint_as_float(w & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ float swap_halves(float v) { return __shfl_xor(v, 32, 64); }
__device__ __forceinline__ int swap_halves(int v) { return __shfl_xor(v, 32, 64); }

// The value lane l ^ 32 holds (v_permlane32_swap, no LDS round trip).
__device__ __forceinline__ int other_half(int v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  // r[0]: lanes 0-31 keep v[lane], lanes 32-63 get v[lane-32]; r[1]: lanes 0-31 get
  // v[lane+32], lanes 32-63 keep v[lane]
  return (__lane_id() < 32) ? int(r[1]) : int(r[0]);
}
__device__ __forceinline__ float other_half(float v) {
  return __int_as_float(other_half(__float_as_int(v)));
}

// Register-class hint: the 256 output accumulators live in AGPRs for the whole kernel.
// (Empty inline assembly with a register-class constraint; it emits no instruction.)
__device__ __forceinline__ void pin_agpr(f32x16 &x) { asm volatile("" : "+a"(x)); }

// acc *= alpha, element by element, without moving the accumulator out of the registers the
// matrix instructions accumulate in.
__device__ __forceinline__ void scale_acc(f32x16 &acc, float alpha) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float x = acc[e];
    float tmp;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32_e32 %1, %2, %1\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(x), "=&v"(tmp)
        : "v"(alpha));
    acc[e] = x;
  }
}

// One global_load_lds_dwordx4: each lane's 16 bytes at `src` land at lds_dst + 16*lane
// (lds_dst wave-uniform). Issued as inline assembly so that the compiler does not track the
// LDS write (it would otherwise wait for these loads before every LDS read of the other tile
// buffer); the kernel waits for them itself before the data is read, and a barrier orders
// them for the other wavefronts.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_dst) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(lds_dst)
      : "memory", "m0");
}

// Waits until this thread's outstanding vector-memory loads (the tile loads among them) are
// done; also a compiler memory barrier.
__device__ __forceinline__ void wait_tile_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Returns v unchanged, but hides its value from the optimiser so that address arithmetic
// derived from it is recomputed where it is used rather than hoisted out of the tile loop
// and kept live (register pressure is the binding constraint of this kernel).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Per-workgroup constants of one split.
struct Ctx {
  const uint16_t *kv;
  const int64_t *kvi;   // kv_indices of the request
  int64_t num_slots;
  uint32_t *status;
  int k0, k1, P;
  int wave;             // wave-uniform
  int lane, half, col;
};

// The slots of the 8 key rows a wave stages for one tile (wave-uniform, in SGPRs).
struct WaveSlots {
  int64_t s[kRowsPerWave];
};

// Lane i < 8 loads the slot of row 8*wave + i of tile t (-1 past the split). A vector-memory
// load on purpose: it completes in order with the tile loads and is consumed after the wait
// for them, so it never stalls anything on its own.
__device__ __forceinline__ int64_t fetch_slots_vec(const Ctx &c, int t) {
  int64_t v = -1;
  const int j = c.k0 + t * kTK + c.wave * kRowsPerWave + c.lane;
  if (c.lane < kRowsPerWave && j < c.k1) v = c.kvi[j];
  return v;
}

__device__ __forceinline__ void slots_to_sgpr(int64_t v, WaveSlots &ws) {
  const int lo = int(uint64_t(v)), hi = int(uint64_t(v) >> 32);
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const uint32_t l = uint32_t(__builtin_amdgcn_readlane(lo, i));
    const uint32_t h = uint32_t(__builtin_amdgcn_readlane(hi, i));
    ws.s[i] = int64_t((uint64_t(h) << 32) | l);
  }
}

// Usable-key bits of the wave's rows: -1 marks a row past the split; a slot out of range is
// flagged and unusable.
__device__ __forceinline__ uint32_t wave_ok_bits(const Ctx &c, int t, const WaveSlots &ws) {
  uint32_t ok = 0;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int j = c.k0 + t * kTK + c.wave * kRowsPerWave + i;
    const bool in = j < c.k1;
    const bool valid = ws.s[i] >= 0 && ws.s[i] < c.num_slots;
    bad |= in && !valid;
    ok |= uint32_t(in && valid) << i;
  }
  if (bad && c.lane == 0) atomicOr(c.status, 1u);  // VA_DEV_SLOT_RANGE
  return ok;
}

// Direct global->LDS loads of the wave's 8 rows of a tile into raw buffer B: per row one
// 64-lane load of the 1 KB latent part (lane = stored unit, loading logical unit
// lane ^ swizzle), and one load for the rope parts of all 8 rows (8 lanes per row).
template <int B>
__device__ __forceinline__ void issue_tile(const Ctx &c, const WaveSlots &ws, uint32_t ok) {
  const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>(raw_buf<B>()));
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int row = c.wave * kRowsPerWave + i;
    const int64_t sl = ((ok >> i) & 1u) ? ws.s[i] : 0;
    const uint16_t *src = c.kv + sl * kDim + 8 * (c.lane ^ lat_swz(row));
    dma16(src, base + row * kLatRow);
  }
  {
    const int q = c.lane & 7, ri = c.lane >> 3;
    const int row = c.wave * kRowsPerWave + ri;
    int64_t sl = 0;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
      if (ri == i && ((ok >> i) & 1u)) sl = ws.s[i];
    const uint16_t *src = c.kv + sl * kDim + kLatent + 8 * (q ^ rope_swz(row));
    dma16(src, base + kLatTile + c.wave * (kRowsPerWave * kRopeRow));
  }
}

// fp16 copy of the latent unit this thread loaded for row i of its wave (zeros if unusable).
template <int B>
__device__ __forceinline__ void convert_unit(const Ctx &c, int i, uint32_t ok) {
  const int row = c.wave * kRowsPerWave + i;
  const uint4 x = *reinterpret_cast<const uint4 *>(raw_buf<B>() + row * kLatRow + 16 * c.lane);
  uint4 h = make_uint4(0, 0, 0, 0);
  if ((ok >> i) & 1u) {
    h.x = bf16pair_to_f16pair(x.x);
    h.y = bf16pair_to_f16pair(x.y);
    h.z = bf16pair_to_f16pair(x.z);
    h.w = bf16pair_to_f16pair(x.w);
  }
  const int unit = c.lane ^ lat_swz(row);
  *reinterpret_cast<uint4 *>(v_buf<B>() + row * kVRow + 16 * unit) = h;
}

// Running per-lane state of the online softmax.
struct RowState {
  float m;      // running (lazy) max, log2 units
  float mx;     // true max, log2 units
  float lsum;   // this lane's share of the denominator (rounded P)
  int best_j;   // argmax key position
};

// One key tile t in buffer B: QK^T, mask, online softmax, PV. Tile t+1 is loaded into buffer
// B^1 meanwhile (issued first, waited for and converted last), and the slots of tile t+2 are
// fetched.
template <int B, bool kArgmax>
__device__ __forceinline__ void tile_step(const Ctx &c0, int t, int ntiles, WaveSlots &slots,
                                          const bf16x8 *qf, f32x16 *o, RowState &st, float c2,
                                          bool row_ok, const uint8_t *mseg, uint32_t moff) {
  constexpr int NB = B ^ 1;
  Ctx c = c0;
  c.lane = opaque(c0.lane);
  c.col = c.lane & 31;
  c.half = c.lane >> 5;

  // ---- tile t+1: usable bits, loads into buffer B^1; then the slots of tile t+2
  const bool have_next = t + 1 < ntiles;
  uint32_t ok_next = 0;
  if (have_next) {
    ok_next = wave_ok_bits(c, t + 1, slots);
    issue_tile<NB>(c, slots, ok_next);
  }
  int64_t slot_vec = -1;
  // Unconditional: past the split every lane yields -1 without a load, and consuming the value
  // on every path keeps the compiler from treating it as pending (and waiting on the DMAs).
  slot_vec = fetch_slots_vec(c, t + 2);
  __builtin_amdgcn_sched_barrier(0);

  // ---- S^T[key][row]: A = key rows (LDS), B = query rows (registers). Logical unit
  // 2*kc + half of row `col` is stored at unit (2*kc + half) ^ swizzle. Even and odd
  // fragments accumulate into two chains so that consecutive MFMAs are independent.
  f32x16 sacc;
  {
    f32x16 sodd;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sacc[e] = 0.f;
      sodd[e] = 0.f;
    }
    const char *lat = raw_buf<B>() + c.col * kLatRow;
    const int y = lat_swz(c.col) ^ c.half;
    const char *rope = raw_buf<B>() + kLatTile + c.col * kRopeRow;
    const int yr = rope_swz(c.col) ^ c.half;
    auto kaddr = [&](int kc) -> const bf16x8 * {
      if (kc < kLatFrags)
        return reinterpret_cast<const bf16x8 *>(lat + 256 * (kc >> 3) +
                                                16 * ((2 * (kc & 7)) ^ y));
      return reinterpret_cast<const bf16x8 *>(rope + 16 * ((2 * (kc - kLatFrags)) ^ yr));
    };
    // kKPrefetch fragment reads in flight: with one wave per SIMD nothing else hides the LDS
    // latency
    bf16x8 kf[kKPrefetch + 1];
#pragma unroll
    for (int kc = 0; kc < kKPrefetch; ++kc) kf[kc] = *kaddr(kc);
#pragma unroll
    for (int kc = 0; kc < kQFrags; ++kc) {
      if (kc + kKPrefetch < kQFrags)
        kf[(kc + kKPrefetch) % (kKPrefetch + 1)] = *kaddr(kc + kKPrefetch);
      if (kc & 1)
        sodd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kc % (kKPrefetch + 1)], qf[kc],
                                                       sodd, 0, 0, 0);
      else
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kc % (kKPrefetch + 1)], qf[kc],
                                                       sacc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] += sodd[e];
  }

  // ---- raw scores; invisible keys -> -inf. Accumulator e holds key kb + 8*(e/4) +
  // 4*half + e%4 of row `col`. Masking is skipped for tiles of usable prefix keys only.
  const int kb = c.k0 + t * kTK;
  const uint32_t okbits = g_okbits[B];
  const bool tail = kb + kTK > c.P;
  if (tail || okbits != 0xffffffffu) {
    uint32_t tree_vis = 0xffffffffu;
    if (tail) {
      // the lane's row's mask bytes (addresses clamped into the row; keys past the split
      // are already unusable in okbits)
      uint8_t mb[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = kb + 8 * (e >> 2) + 4 * c.half + (e & 3);
        mb[e] = mseg[moff + uint32_t(min(j, c.k1 - 1))];
      }
      tree_vis = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = kb + 8 * (e >> 2) + 4 * c.half + (e & 3);
        tree_vis |= uint32_t(j < c.P || (row_ok && mb[e] != 0)) << e;
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kk = 8 * (e >> 2) + 4 * c.half + (e & 3);
      const bool vis = ((okbits >> kk) & 1u) && ((tree_vis >> e) & 1u);
      sacc[e] = vis ? sacc[e] : -INFINITY;
    }
  }
  // max of the raw scores (the scale is positive, so it keeps the order), then the lane
  // pair holding the other 16 keys of the row
  float tmax;
  int targ = 0x7fffffff;
  if (kArgmax) {
    tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kk = 8 * (e >> 2) + 4 * c.half + (e & 3);
      if (sacc[e] > tmax) { tmax = sacc[e]; targ = kb + kk; }
    }
    const float om = other_half(tmax);
    const int oj = other_half(targ);
    if (om > tmax || (om == tmax && oj < targ)) targ = oj;
    tmax = fmaxf(tmax, om);
  } else {
    tmax = sacc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, sacc[e]);
    tmax = fmaxf(tmax, other_half(tmax));
  }
  tmax *= c2;  // log2 units
  if (kArgmax && tmax > st.mx) st.best_j = targ;
  st.mx = fmaxf(st.mx, tmax);

  // ---- lazy rescale of the running max (rare after the first tile)
  const bool need = tmax > st.m + kRescale;
  if (__any(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(st.m - tmax) : 1.f;
    if (need) st.m = tmax;
    st.lsum *= alpha;
#pragma unroll
    for (int d = 0; d < kDBlocks; ++d) scale_acc(o[d], alpha);
  }
  const float negm = st.m == -INFINITY ? 0.f : -st.m;

  // ---- P = exp2(s*c2 - m) rounded to nearest-even fp16 (v_cvt_pk_f16_f32: unbiased, so the
  // denominator summed from the rounded values does not drift); the sum uses v_dot2
  f16x8 pf[2];
  {
    const f16x2v ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        f32x2 p;
        p.x = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * ch + e], c2, negm));
        p.y = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * ch + e + 1], c2, negm));
        const f16x2v h = __builtin_convertvector(p, f16x2v);
        st.lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2, h),
                                         __builtin_bit_cast(fp16x2, ones), st.lsum, false);
        pf[ch][e] = h.x;
        pf[ch][e + 1] = h.y;
      }
    }
  }

  __builtin_amdgcn_sched_barrier(0);

  // ---- O^T[dim][row] += V^T[dim][key] P^T[key][row]. Key slot 8*half + 4*rr + e of chunk ch
  // is key 16*ch + 4*half + 8*rr + e, in the A operand (transposed read) and in pf[ch].
  {
    const char *vt = v_buf<B>();
    const int g = c.lane & 15;
    const int m0 = 16 * ((c.lane >> 4) & 1);
    const char *vbase = vt + (4 * c.half + (g >> 2)) * kVRow + (m0 + 4 * (g & 3)) * 2;
    auto vfrag = [&](int ch, int d) -> f16x8 {
      f16x8 vf;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const fp16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            (lds_fp16x4 *)(vbase + (16 * ch + 8 * rr) * kVRow + 64 * d));
#pragma unroll
        for (int e = 0; e < 4; ++e) vf[4 * rr + e] = (_Float16)x[e];
      }
      return vf;
    };
    f16x8 vq[kVPrefetch + 1];
#pragma unroll
    for (int it = 0; it < kVPrefetch; ++it) vq[it] = vfrag(it / kDBlocks, it % kDBlocks);
#pragma unroll
    for (int it = 0; it < 2 * kDBlocks; ++it) {
      const int ch = it / kDBlocks, d = it % kDBlocks;
      if (it + kVPrefetch < 2 * kDBlocks) {
        const int it2 = it + kVPrefetch;
        vq[it2 % (kVPrefetch + 1)] = vfrag(it2 / kDBlocks, it2 % kDBlocks);
      }
      o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vq[it % (kVPrefetch + 1)], pf[ch], o[d], 0,
                                                    0, 0);
      pin_agpr(o[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- end of the tile: this thread's loads of tile t+1 (and the slots of t+2) have had the
  // whole tile to land; convert them to the fp16 latent tile, then publish with the barrier
  if (have_next) {
    wait_tile_loads();
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) convert_unit<NB>(c, i, ok_next);
  }
  slots_to_sgpr(slot_vec, slots);

  if (have_next && c.lane == 0)
    reinterpret_cast<uint8_t *>(&g_okbits[NB])[c.wave] = uint8_t(ok_next);
  __syncthreads();
}

template <bool kArgmax>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_partial_kernel(RunArgs a, Workspace ws, int tiles_per_req, int n_work) {
  // ---- XCD-aware work mapping: consecutive work items land on one XCD
  const int nb = gridDim.x;  // a multiple of 8
  const int w = (int(blockIdx.x) & 7) * (nb >> 3) + (int(blockIdx.x) >> 3);
  if (w >= n_work) return;
  const int S = ws.splits;
  const int tile = w % tiles_per_req;
  const int s = (w / tiles_per_req) % S;
  const int r = w / (tiles_per_req * S);

  Segment seg;
  const uint32_t bad = load_segment(a, r, seg);
  if (bad) {
    if (threadIdx.x == 0 && tile == 0 && s == 0) atomicOr(ws.status, bad);
    return;
  }
  const int H = a.H;
  const int rows_req = seg.T * H;
  const int row0 = tile * kRows;
  if (row0 >= rows_req) return;

  Ctx c;
  c.kv = static_cast<const uint16_t *>(a.kv);
  c.kvi = a.kv_indices + seg.kv0;
  c.num_slots = a.num_slots;
  c.status = ws.status;
  c.P = seg.P;
  c.wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  c.lane = int(threadIdx.x) & 63;
  c.half = c.lane >> 5;
  c.col = c.lane & 31;
  const int rho = row0 + c.wave * 32 + c.col;  // local row: token rho / H, head rho % H
  const bool row_ok = rho < rows_req;
  const int rho_c = row_ok ? rho : rows_req - 1;  // rows past the end compute, never write
  const int tok = rho_c / H;
  const int64_t grow = (seg.q0 + tok) * int64_t(H) + rho_c % H;

  // this split's keys: whole tiles
  const int per = (seg.L + S - 1) / S;
  const int chunk = (per + kTK - 1) / kTK * kTK;
  c.k0 = min(seg.L, s * chunk);
  c.k1 = min(seg.L, c.k0 + chunk);
  const int ntiles = (c.k1 - c.k0 + kTK - 1) / kTK;

  // ---- prologue: tile 0 loaded and converted, slots of tile 1 fetched
  WaveSlots slots;
  uint32_t ok0 = 0;
  int64_t slot_vec = -1;
  if (ntiles > 0) {
    slots_to_sgpr(fetch_slots_vec(c, 0), slots);
    ok0 = wave_ok_bits(c, 0, slots);
    issue_tile<0>(c, slots, ok0);
    slot_vec = fetch_slots_vec(c, 1);
  }

  // query fragments (B operand): row `col`, dims 16*kc + 8*half .. +8
  bf16x8 qf[kQFrags];
  {
    const uint4 *qrow = reinterpret_cast<const uint4 *>(
        static_cast<const uint16_t *>(a.q) + grow * kDim);
#pragma unroll
    for (int kc = 0; kc < kQFrags; ++kc) {
      u32x4 v = __builtin_bit_cast(u32x4, qrow[2 * kc + c.half]);
      // keep the fragment resident: without this the compiler re-reads q inside the tile loop
      asm volatile("" : "+v"(v));
      qf[kc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 o[kDBlocks];
#pragma unroll
  for (int d = 0; d < kDBlocks; ++d) {
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
    pin_agpr(o[d]);
  }
  RowState st;
  st.m = -INFINITY;
  st.mx = -INFINITY;
  st.lsum = 0.f;
  st.best_j = -1;
  const float c2 = a.scale * kLog2e;
  // the row's mask bytes: a request-uniform base plus a 32-bit lane offset (a request's mask
  // segment is validated to stay under 2 GiB)
  const uint8_t *mseg = a.mask + seg.m0;
  const uint32_t moff = uint32_t(tok) * uint32_t(seg.L);

  if (ntiles > 0) {
    wait_tile_loads();
    slots_to_sgpr(slot_vec, slots);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) convert_unit<0>(c, i, ok0);
    if (c.lane == 0) reinterpret_cast<uint8_t *>(&g_okbits[0])[c.wave] = uint8_t(ok0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; t += 2) {
    tile_step<0, kArgmax>(c, t, ntiles, slots, qf, o, st, c2, row_ok, mseg, moff);
    if (t + 1 < ntiles)
      tile_step<1, kArgmax>(c, t + 1, ntiles, slots, qf, o, st, c2, row_ok, mseg, moff);
  }

  // ---- write the partial of this split
  const float ltot = st.lsum + swap_halves(st.lsum);
  if (!row_ok) return;
  const int64_t prow = int64_t(s) * ws.rows_cap + grow;
  float4 *po = reinterpret_cast<float4 *>(ws.part_o + prow * kLatent);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
#pragma unroll
  for (int d = 0; d < kDBlocks; ++d)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
      po[(32 * d + 8 * gq + 4 * c.half) / 4] =
          make_float4(o[d][4 * gq] * inv, o[d][4 * gq + 1] * inv, o[d][4 * gq + 2] * inv,
                      o[d][4 * gq + 3] * inv);
  if (c.half == 0) {
    const bool any = ltot > 0.f;
    ws.part_lse[prow] = any ? (st.m + log2f(ltot)) * kLn2 : -INFINITY;
    ws.part_max[prow] = any ? st.mx * kLn2 : -INFINITY;
    ws.part_arg[prow] = any && kArgmax ? st.best_j : -1;
  }
}

}  // namespace

hipError_t launch_mfma_partial(const RunArgs &a, const Workspace &ws, int rows_per_block,
                               hipStream_t st) {
  if (rows_per_block != kRows) return hipErrorInvalidValue;
  const int64_t tiles = (int64_t(a.max_q_per_req) * a.H + kRows - 1) / kRows;
  const int64_t n_work = int64_t(a.bs) * ws.splits * tiles;
  if (n_work <= 0) return hipSuccess;
  const int64_t nb = (n_work + 7) / 8 * 8;
  if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.want_argmax)
    hipLaunchKernelGGL(mfma_partial_kernel<true>, dim3(unsigned(nb)), dim3(kThreads), 0, st, a,
                       ws, int(tiles), int(n_work));
  else
    hipLaunchKernelGGL(mfma_partial_kernel<false>, dim3(unsigned(nb)), dim3(kThreads), 0, st, a,
                       ws, int(tiles), int(n_work));
  return hipGetLastError();
}

}  // namespace va
