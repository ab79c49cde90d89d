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
//    (global_load_lds_dwordx4), two tiles ahead of their products, without passing through
//    registers: one load instruction moves the 1 KB latent part of one row from a scalar
//    base address, so a row costs one instruction plus its slot's address. Latent rows sit
//    at a padded 1040-byte stride and rope units are placed by a lane permutation, so every
//    matrix-operand read is bank-conflict free and is one base register plus an immediate;
//  * S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16: A = key rows from LDS, B = the wave's 32
//    query rows held in registers. The accumulator gives each lane one row and 16 keys, so a
//    softmax row reduction is one cross-lane swap;
//  * P is rounded (to nearest even) to fp16 and O^T += V^T P^T runs on
//    v_mfma_f32_32x32x16_f16. V is the first 512 dims of the same rows, converted to fp16 once
//    per tile (each thread converts the units it loaded) and read as V^T fragments with
//    ds_read_b64_tr_b16. The P fragment is the S accumulator itself: key slots are permuted
//    the same way in both operands;
//  * the tile loop is software-pipelined: the P.V products of tile t and the QK^T products of
//    tile t+1 run in one step (so the scores of tile t+1 are ready when tile t's products
//    end), with the fp16 conversion of tile t+1 and the loads of tile t+2 beside them;
//  * two variants share all of the above. With H a multiple of 64 a workgroup runs eight
//    wavefronts, two per SIMD (section "two wavefronts per SIMD" below): four hold the query
//    rows and do the scores and softmax, four hold three quarters of the output accumulators
//    and stage the tiles, so one wavefront's vector and LDS work issues while the other's
//    matrix instructions run. Otherwise four wavefronts of 32 rows each hold all 256 output
//    accumulators per lane, one wavefront per SIMD, and every other instruction issues
//    between their matrix instructions, so that loop is written to issue as few as possible
//    (it also has the path for items of at most 32 rows);
//  * the running max is rescaled lazily (only when it grows by more than 2^8), in place in
//    the accumulation registers, so the 256 fp32 accumulators per lane never leave them;
//  * workgroups are mapped so that all row tiles of one key split run on the same XCD and
//    share its L2; HBM then sees each latent row about once.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "va_internal.h"

namespace va {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__fp16)))) __fp16 fp16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = kMfmaRowsPerBlock;    // 128 rows = 4 waves x 32
constexpr int kTK = 32;                     // keys per tile
constexpr int kRowsPerWave = kTK / kWaves;  // 8 key rows staged by each wave
constexpr int kLatStride = 2 * kLatent + 16;             // 1040-byte latent row (padded)
constexpr int kRopeOff = kTK * kLatStride;               // 33,280: rope block of a raw tile
constexpr int kRawTile = kRopeOff + kTK * 2 * kRope;     // + 4 KB = 37,376
constexpr int kVRow = 2 * kLatent + 64;                  // fp16 V tile row stride: 1088
constexpr int kVTile = kTK * kVRow;                      // 34,816
constexpr int kVOff = 2 * kRawTile;                      // the two fp16 tiles follow
constexpr int kLdsBytes = kVOff + 2 * kVTile;            // 144,384
constexpr int kQFrags = kDim / 16;          // 36 bf16x8 B-operand fragments per lane
constexpr int kLatFrags = kLatent / 16;     // the first 32 of them are latent dims
constexpr int kDBlocks = kLatent / 32;      // 16 output dim blocks of 32
constexpr int kNumPV = 2 * kDBlocks;        // 32 P.V products per tile
constexpr int kDepth = 3;                   // operand fragment reads in flight
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;            // lazy-rescale threshold (log2 units)

static_assert(kRowsPerWave == 8, "one rope load instruction covers 8 rows");
static_assert(kRawTile % 16 == 0 && kVOff % 16 == 0, "16-byte aligned tiles");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

// The narrow path (items of at most 32 rows) adds a 16 KB partial-score exchange buffer:
// [wave][quad][lane] float4.
constexpr int kXOff = kLdsBytes;
constexpr int kXBytes = kWaves * 4 * 64 * 16;
static_assert(kXOff + kXBytes <= 160 * 1024, "LDS budget of the narrow path");

// LDS: raw bf16 tiles 0 and 1 (latent rows at a padded stride, then the rope block), then
// fp16 latent tiles 0 and 1, then the narrow path's exchange buffer; the usable-key bits of
// the two raw tiles (a byte per wave).
__shared__ __attribute__((aligned(16))) char g_lds[kXOff + kXBytes];
__shared__ uint32_t g_okbits[2];
// the narrow path's key slots of two tiles, loaded straight into LDS: [tile parity][wave][8]
__shared__ __attribute__((aligned(16))) int64_t g_slots[2][kWaves][kRowsPerWave];

__device__ __forceinline__ uint32_t lds_addr(const char *p) {
  return uint32_t(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ uint32_t bf16pair_to_f16pair(uint32_t w) {
  const float lo = __uint_as_float(w << 16);
  const float hi = __uint_as_float(w & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

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

// O^T block += A (fp16 V^T fragment) x B (fp16 P^T fragment), accumulating in AGPRs. Written
// as assembly because the library is compiled with matrix instructions in their VGPR form (the
// score accumulator must not take AGPRs, which the 256 output accumulators fill). The compiler
// does not see this as a matrix instruction: its operands arrive through ordinary waits (A
// from LDS reads, B long before from VALU), and every VALU read of acc is preceded by
// matrix_drain().
__device__ __forceinline__ void pv_mfma(f32x16 &acc, const u32x4 &a, const f16x8 &b) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// acc *= alpha, element by element, without moving the accumulator out of the registers the
// matrix instructions accumulate in. The caller separates this from the matrix instructions
// that write acc (the compiler does not see into the assembly).
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

// Wait states around the in-place rescale: enough for the longest matrix instruction to
// retire before its accumulator is read, and for the rewritten values before the next use.
__device__ __forceinline__ void matrix_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Two values in [-1, 1] as packed 16-bit signed-normalised codes (v_cvt_pknorm_i16_f32:
// clamped, scaled by 32767 and rounded), x in the low half.
__device__ __forceinline__ uint32_t snorm16x2(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(x, y));
}

// Stores the int16 codes of output block d (32 dims) of this lane's row, given as two codes per
// word: c[gq][i] holds dims 32d + 8gq + 4half + 2i, +1. Lane pairs (l, l ^ 32) hold the same
// row; two swaps per pair of groups give each lane 8 consecutive dims, so the block goes out
// in two 16-byte stores per lane instead of four 8-byte ones.
__device__ __forceinline__ void store_codes(int16_t *row_codes, int d, int half,
                                            const uint32_t (&c)[4][2]) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    // lanes 0-31 end with dims 32d + 16k + 0..7, lanes 32-63 with 32d + 16k + 8..15
    const auto s0 = __builtin_amdgcn_permlane32_swap(c[2 * k][0], c[2 * k + 1][0], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(c[2 * k][1], c[2 * k + 1][1], false, false);
    *reinterpret_cast<uint4 *>(row_codes + 32 * d + 16 * k + 8 * half) =
        make_uint4(s0[0], s1[0], s0[1], s1[1]);
  }
}

// One global_load_lds_dwordx4 from a scalar base: lane l's 16 bytes at base + voff land at
// lds + 16*l. Inline assembly so that the compiler does not track the LDS write (it would
// otherwise wait for these loads before every LDS read); the kernel waits for them itself
// before the data is read, and a barrier orders them for the other wavefronts.
// The LDS address travels in M0, which the asm takes as an input operand ("{m0}"), so the
// compiler writes M0 itself and knows it is read here. Wait states the compiler cannot see
// through the asm are supplied inside it: the scalar base comes from v_readlane just before,
// and a vector-memory instruction that reads an SGPR written by a VALU instruction needs 5 wait
// states on this generation (the LDS DMA also needs 1 after the M0 write): s_nop 4 gives 5.
__device__ __forceinline__ void dma_row(uint64_t base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "{m0}"(lds)
      : "memory");
}
// The same from a per-lane 64-bit address (1 wait state after the M0 write).
__device__ __forceinline__ void dma_lanes(const void *src, uint32_t lds) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "{m0}"(lds)
      : "memory");
}

// Waits until this thread's outstanding vector-memory loads (the tile loads among them) are
// done; also a compiler memory barrier.
__device__ __forceinline__ void wait_tile_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// The same, but leaving up to 10 loads in flight (a tile's 9 and a slot fetch issued after
// them): vector-memory loads complete in issue order, so everything issued before those 10
// has landed.
__device__ __forceinline__ void wait_loads_but_10() {
  asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
}
// One global_load_lds_dword per lane from a per-lane address: lane l's 4 bytes land at
// lds + 4*l.
__device__ __forceinline__ void dma_dword_lanes(const void *src, uint32_t lds) {
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(src), "{m0}"(lds)
      : "memory");
}

// Per-workgroup constants of one split.
struct Ctx {
  const uint16_t *kv;
  const int64_t *kvi;   // kv_indices of the request
  const int64_t *tree;  // the tree keys' slots when they come from out_cache_loc, else NULL
  const uint16_t *zero; // a row of zeros
  int64_t num_slots;
  uint32_t *status;
  int k0, k1, P;
  int wave;             // wave-uniform
  int lane, half, col;
};

// Lane l fetches the slot of row (l & 7) of its wave's 8 rows of tile t. Consumed a tile
// later, after the wait for the tile loads; plan_tile discards it for keys past the split.
// Those keys read the split's last entry instead (k0 < k1 for every item), so that the load
// is neither under a branch nor followed by a select on its value: either made the compiler
// wait for it (and so for every load before it) right away.
__device__ __forceinline__ int64_t fetch_slot(const Ctx &c, int t) {
  const int j = c.k0 + t * kTK + c.wave * kRowsPerWave + (c.lane & 7);
  const int jc = min(j, c.k1 - 1);
  return (c.tree && jc >= c.P) ? c.tree[jc - c.P] : c.kvi[jc];
}

// The loads of one tile, prepared from the fetched slots: the row address each lane holds
// (row l & 7; the zero row for keys past the split or slots out of range) and the wave's
// usable-row bits.
struct TileLoads {
  uint64_t addr;
  uint32_t ok;   // bit i: row i of this wave is a usable key
};

__device__ __forceinline__ TileLoads plan_tile(const Ctx &c, int t, int64_t slot) {
  const int j = c.k0 + t * kTK + c.wave * kRowsPerWave + (c.lane & 7);
  const bool in = j < c.k1;
  const bool valid = in && slot >= 0 && slot < c.num_slots;
  TileLoads tl;
  tl.ok = uint32_t(__ballot(valid)) & 0xffu;
  if (__ballot(in && !valid) != 0 && c.lane == 0) atomicOr(c.status, 1u);  // VA_DEV_SLOT_RANGE
  const uint64_t row = uint64_t(reinterpret_cast<uintptr_t>(c.kv)) + uint64_t(slot) * (2 * kDim);
  tl.addr = valid ? row : uint64_t(reinterpret_cast<uintptr_t>(c.zero));
  return tl;
}

// Latent row i of the wave: one 64-lane load of its 1 KB into the padded row.
__device__ __forceinline__ void issue_latent(const Ctx &c, const TileLoads &tl, uint32_t raw,
                                             int i) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(tl.addr)), i));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(tl.addr >> 32)), i));
  const uint64_t base = (uint64_t(hi) << 32) | lo;
  dma_row(base, uint32_t(16 * c.lane), raw + (c.wave * kRowsPerWave + i) * kLatStride);
}

// The rope parts of the wave's 8 rows: lane l loads unit u of row l & 7 into position l of
// the wave's 1 KB rope block, with u = 2*(l >> 4) + (((l >> 3) & 1) ^ (wave & 1)).
__device__ __forceinline__ void issue_rope(const Ctx &c, const TileLoads &tl, uint32_t raw) {
  const int u = 2 * (c.lane >> 4) + (((c.lane >> 3) & 1) ^ (c.wave & 1));
  const char *src = reinterpret_cast<const char *>(uintptr_t(tl.addr)) + 2 * kLatent + 16 * u;
  dma_lanes(src, raw + kRopeOff + c.wave * 1024);
}

__device__ __forceinline__ void publish_ok(const Ctx &c, int buf, uint32_t ok) {
  if (c.lane == 0) reinterpret_cast<uint8_t *>(&g_okbits[buf])[c.wave] = uint8_t(ok);
}

// Per-lane byte offsets (relative to a tile buffer) of the operand reads.
struct LaneOffs {
  uint32_t k_lat;   // K fragment kc < 32: + 32*kc
  uint32_t k_rope;  // K fragment 32 + j: + 256*j
  uint32_t v_tr;    // V^T fragment (chunk ch, half rr, dim block d): + (16ch+8rr)*1088 + 64d
  uint32_t cv_rd;   // conversion read of unit `lane` of the wave's row i: + 1040*i
  uint32_t cv_wr;   // conversion write: + 1088*i
};

__device__ __forceinline__ LaneOffs lane_offsets(const Ctx &c) {
  LaneOffs lo;
  const int row = c.col;
  lo.k_lat = row * kLatStride + 16 * c.half;
  lo.k_rope = kRopeOff + 1024 * (row >> 3) + 128 * (c.half ^ ((row >> 3) & 1)) + 16 * (row & 7);
  const int g = c.lane & 15;
  const int m0 = 16 * ((c.lane >> 4) & 1);
  lo.v_tr = (4 * c.half + (g >> 2)) * kVRow + (m0 + 4 * (g & 3)) * 2;
  lo.cv_rd = c.wave * kRowsPerWave * kLatStride + 16 * c.lane;
  lo.cv_wr = c.wave * kRowsPerWave * kVRow + 16 * c.lane;
  return lo;
}

// Running per-lane state of the online softmax.
struct RowState {
  float m;      // running (lazy) max, log2 units
  float mx;     // true max, log2 units
  float lsum;   // this lane's share of the denominator (rounded P)
  int best_j;   // argmax key position
};

// ---- one pipeline step
//
// A step issues the 68 matrix instructions of one tile's worth of work in a fixed order
// (written as a table), and slots the vector work between them:
//  kFirst - QK^T of tile 0 (36 instructions) and the fp16 copy of tile 0;
//  kMain  - phase A: exp/round/sum of P(t) interleaved with QK^T fragments 0..11 of tile t+1,
//           and the loads of tile t+2 (one row every second op from op 1) and the slot fetch
//           of tile t+3;
//           phase B: P(t).V(t) interleaved with QK^T fragments 12..35 of tile t+1 and the fp16
//           copy of tile t+1; the last eight P.V products cover the latency of the final
//           QK^T result;
//  kLast  - exp/round/sum of P(t), then P(t).V(t).
// The 36 QK^T fragments accumulate into one chain: a matrix instruction that accumulates into
// exactly the registers the one before it wrote issues back to back at full rate on this
// generation (32.8 cycles each, against 32.3 with independent accumulators), and one chain
// needs neither the second 16 accumulators nor their merge.
enum StepKind { kFirst = 0, kMain = 1, kLast = 2 };

struct Op {
  int8_t pv;    // 1: P.V product, 0: QK^T fragment
  int8_t idx;   // fragment index (QK^T: 0..35; P.V: 0..31, chunk = idx / 16, dim block = idx % 16)
};
template <int N> struct OpTable { Op op[N]; };

constexpr int kPhaseA = 12;  // QK^T fragments in phase A of a main step

template <int K> struct StepPlan;
template <> struct StepPlan<kFirst> {
  static constexpr int kOps = kQFrags;
  static constexpr OpTable<kOps> table() {
    OpTable<kOps> t{};
    for (int i = 0; i < kOps; ++i) t.op[i] = Op{0, int8_t(i)};
    return t;
  }
  // conversion unit u: read after op rd(u), one pair converted after each of the next four
  // ops, written after op rd(u) + 4
  static constexpr int rd(int u) { return 2 + 4 * u; }
  static constexpr int kCvLag = 0;
};
template <> struct StepPlan<kMain> {
  static constexpr int kOps = kQFrags + kNumPV;
  static constexpr OpTable<kOps> table() {
    OpTable<kOps> t{};
    int p = 0;
    for (int k = 0; k < kPhaseA; ++k) t.op[p++] = Op{0, int8_t(k)};
    int q = kPhaseA, v = 0;
    while (q < kQFrags || v < kNumPV) {
      if (v < kNumPV) t.op[p++] = Op{1, int8_t(v++)};
      if (q < kQFrags) t.op[p++] = Op{0, int8_t(q++)};
    }
    return t;
  }
  // conversion unit u: read after op rd(u); its pairs are converted after ops rd(u) + 2 ..
  // rd(u) + 5 (one matrix instruction more than the read needs to land) and it is written
  // after op rd(u) + 5
  static constexpr int rd(int u) { return kPhaseA + 2 + 6 * u; }
  static constexpr int kCvLag = 1;
  // the loads of tile t+2: one row after every second op from op 1 (rows 0..7 after ops
  // 1, 3, .., 15, the rope block after op 17), so that the four wavefronts' 36 loads reach
  // the address unit spread out rather than back to back; then the slots of tile t+3
  static constexpr int kDmaOp = 1;
  static constexpr int kDmaStride = 2;
  static constexpr int kSlotOp = kDmaOp + kDmaStride * kRowsPerWave + 1;
};
template <> struct StepPlan<kLast> {
  static constexpr int kOps = kNumPV;
  static constexpr OpTable<kOps> table() {
    OpTable<kOps> t{};
    for (int i = 0; i < kOps; ++i) t.op[i] = Op{1, int8_t(i)};
    return t;
  }
};

struct StepIO {
  const char *kraw;   // raw tile read by QK (and by the conversion)
  const char *vrd;    // fp16 tile read by PV
  char *vwr;          // fp16 tile written by the conversion
  uint32_t dma_raw;   // LDS address of the raw tile the loads fill
};

// Calls f(std::integral_constant<int, I>) for I = I0 .. N-1, unrolled at compile time.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// P(t) = exp2(s*c2 - m) rounded to nearest-even fp16 (v_cvt_pk_f16_f32: unbiased, so the
// denominator summed from the rounded values does not drift), in 8 parts of two keys; the
// sum uses v_dot2.
// Split in two halves so that a step can space the exponentials from their rounding:
// p_exp computes the two exponentials of a part, p_round rounds, sums and places them.
__device__ __forceinline__ f32x2 p_exp(int part, const f32x16 &s, float c2, float negm) {
  const int ch = part >> 2, e = 2 * (part & 3);
  f32x2 p;
  p.x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * ch + e], c2, negm));
  p.y = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * ch + e + 1], c2, negm));
  return p;
}
__device__ __forceinline__ void p_round(int part, const f32x2 &p, float &lsum, f16x8 *pf) {
  const int ch = part >> 2, e = 2 * (part & 3);
  const f16x2v h = __builtin_convertvector(p, f16x2v);
  const f16x2v ones = {(_Float16)1.0f, (_Float16)1.0f};
  lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2, h), __builtin_bit_cast(fp16x2, ones),
                                lsum, false);
  pf[ch][e] = h.x;
  pf[ch][e + 1] = h.y;
}

__device__ __forceinline__ void p_part(int part, const f32x16 &s, float c2, float negm,
                                       float &lsum, f16x8 *pf) {
  const int ch = part >> 2, e = 2 * (part & 3);
  f32x2 p;
  p.x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * ch + e], c2, negm));
  p.y = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * ch + e + 1], c2, negm));
  const f16x2v h = __builtin_convertvector(p, f16x2v);
  const f16x2v ones = {(_Float16)1.0f, (_Float16)1.0f};
  lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2, h), __builtin_bit_cast(fp16x2, ones),
                                lsum, false);
  pf[ch][e] = h.x;
  pf[ch][e + 1] = h.y;
}

__device__ __forceinline__ float neg_max(const RowState &st) {
  return st.m == -INFINITY ? 0.f : -st.m;
}

// kCompute = false: a wavefront whose 32 rows all lie past the request's rows only does its
// share of the tile staging (conversion, loads, slot fetch); the others need that share.
template <int K, bool kCompute = true>
__device__ __forceinline__ void step(const Ctx &c, const LaneOffs &lo, const StepIO &io,
                                     const TileLoads &tl, int64_t &slot_vec, int slot_tile,
                                     const bf16x8 *qf, f32x16 *o, f32x16 &snext,
                                     const f32x16 &scur, RowState &st, float c2, f16x8 *pf) {
  using Plan = StepPlan<K>;
  constexpr int N = Plan::kOps;
  constexpr OpTable<N> T = Plan::table();
  constexpr bool kQK = K != kLast;
  const char *klat = io.kraw + lo.k_lat;
  const char *krope = io.kraw + lo.k_rope;
  const char *vtr = io.vrd + lo.v_tr;
  const char *cvr = io.kraw + lo.cv_rd;
  char *cvw = io.vwr + lo.cv_wr;

  u32x4 fr[kDepth + 1];
  u32x4 craw[kRowsPerWave];
  f32x16 sa;      // the scores of the tile QK reads
  f32x2 pexp;     // the exponentials of the part of P(t) not yet rounded
  const float negm = neg_max(st);

  if constexpr (K == kLast && kCompute) {
#pragma unroll
    for (int part = 0; part < 8; ++part) p_part(part, scur, c2, negm, st.lsum, pf);
  }

  // operand fragment of operation p
  auto load = [&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
    if constexpr (p < N && kCompute) {
      constexpr Op op = T.op[p];
      u32x4 r;
      if constexpr (!op.pv) {
        constexpr int kc = op.idx;
        if constexpr (kc < kLatFrags)
          r = *reinterpret_cast<const u32x4 *>(klat + 32 * kc);
        else
          r = *reinterpret_cast<const u32x4 *>(krope + 256 * (kc - kLatFrags));
      } else {
        constexpr int it = op.idx, ch = it / kDBlocks, d = it % kDBlocks;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const fp16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
              (lds_fp16x4 *)(vtr + (16 * ch + 8 * rr) * kVRow + 64 * d));
          const u32x2 w = __builtin_bit_cast(u32x2, x);
          r[2 * rr] = w[0];
          r[2 * rr + 1] = w[1];
        }
      }
      fr[p % (kDepth + 1)] = r;
    }
  };

  static_for<0, kDepth>(load);
  static_for<0, N>([&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
    constexpr Op op = T.op[p];
    load(std::integral_constant<int, p + kDepth>{});
    const u32x4 a = fr[p % (kDepth + 1)];
    if constexpr (!kCompute) {
    } else if constexpr (op.pv) {
      constexpr int ch = op.idx / kDBlocks, d = op.idx % kDBlocks;
      pv_mfma(o[d], a, pf[ch]);
    } else {
      constexpr int kc = op.idx;
      const bf16x8 av = __builtin_bit_cast(bf16x8, a);
      if constexpr (kc == 0) {
        const f32x16 zero = {};
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[kc], zero, 0, 0, 0);
      } else {
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[kc], sa, 0, 0, 0);
      }
    }
    // phase A: P(t), two keys after each of the first eight fragments; each part's
    // exponentials are rounded and summed one fragment later
    if constexpr (K == kMain && kCompute && p >= 1 && p <= 8) p_round(p - 1, pexp, st.lsum, pf);
    if constexpr (K == kMain && kCompute && p < 8) pexp = p_exp(p, scur, c2, negm);
    // the loads of tile t+2 (zero rows past the split), then the slots of tile t+3
    if constexpr (K == kMain) {
      constexpr int dq = p - Plan::kDmaOp;
      constexpr int dp = (dq >= 0 && dq % Plan::kDmaStride == 0) ? dq / Plan::kDmaStride : -1;
      if constexpr (dp >= 0 && dp < kRowsPerWave) issue_latent(c, tl, io.dma_raw, dp);
      if constexpr (dp == kRowsPerWave) issue_rope(c, tl, io.dma_raw);
      if constexpr (p == Plan::kSlotOp) slot_vec = fetch_slot(c, slot_tile);
    }
    // fp16 copy of the latent units this thread loaded for the tile QK reads
    if constexpr (kQK) {
      static_for<0, kRowsPerWave>([&](auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        constexpr int r0 = Plan::rd(u);
        constexpr int c0 = r0 + Plan::kCvLag;  // the first pair converted after op c0 + 1
        if constexpr (p == r0)
          craw[u] = *reinterpret_cast<const u32x4 *>(cvr + kLatStride * u);
        if constexpr (p > c0 && p <= c0 + 4) craw[u][p - c0 - 1] =
            bf16pair_to_f16pair(craw[u][p - c0 - 1]);
        if constexpr (p == c0 + 4) *reinterpret_cast<u32x4 *>(cvw + kVRow * u) = craw[u];
      });
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  if constexpr (K != kLast && kCompute) snext = sa;
}

// ---- the rest of the softmax of one tile's scores: mask, max (and argmax), lazy rescale
// (kAgpr: the output accumulators sit in AGPRs, out of the compiler's sight; kLean: read the
// mask bytes of a tail tile four at a time, in a loop, to keep registers free)
template <bool kArgmax, int kOBlocks = kDBlocks, bool kAgpr = true, bool kLean = false>
__device__ __forceinline__ void score_max(const Ctx &c, int kb, uint32_t okbits, f32x16 &sacc,
                                          f32x16 *o, RowState &st, float c2, bool row_ok,
                                          const uint8_t *mseg, uint32_t moff) {
  // raw scores; invisible keys -> -inf. Accumulator e holds key kb + 8*(e/4) + 4*half + e%4
  // of row `col`. Masking is skipped for tiles of usable prefix keys only.
  const bool tail = kb + kTK > c.P;
  if (tail || okbits != 0xffffffffu) {
    // key of accumulator e: jh + 8*(e/4) + e%4 (the lane-dependent part folded into jh and
    // okh, so that the per-e offsets are constants)
    const int jh = kb + 4 * c.half;
    const uint32_t okh = okbits >> (4 * c.half);
    uint32_t tree_vis = 0xffffffffu;
    if (tail && kLean) {
      tree_vis = 0;
#pragma unroll 1
      for (int q = 0; q < 4; ++q) {
        uint32_t b4 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = jh + 8 * q + i;
          const uint8_t mv = mseg[moff + uint32_t(min(j, c.k1 - 1))];
          b4 |= uint32_t(j < c.P || (row_ok && mv != 0)) << i;
        }
        tree_vis |= b4 << (4 * q);
      }
    } else if (tail) {
      // the lane's row's mask bytes (addresses clamped into the row; keys past the split
      // are already unusable in okbits)
      uint8_t mb[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = jh + 8 * (e >> 2) + (e & 3);
        mb[e] = mseg[moff + uint32_t(min(j, c.k1 - 1))];
      }
      tree_vis = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = jh + 8 * (e >> 2) + (e & 3);
        tree_vis |= uint32_t(j < c.P || (row_ok && mb[e] != 0)) << e;
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const bool vis = ((okh >> (8 * (e >> 2) + (e & 3))) & 1u) && ((tree_vis >> e) & 1u);
      sacc[e] = vis ? sacc[e] : -INFINITY;
    }
  }
  // max of the raw scores (the scale is positive, so it keeps the order), then the lane
  // pair holding the other 16 keys of the row
  float tmax = sacc[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, sacc[e]);
  tmax = fmaxf(tmax, other_half(tmax));
  const float tmax2 = tmax * c2;  // log2 units
  if (kArgmax) {
    // the argmax moves only when the row's max grows, which soon becomes rare: locate it only
    // then (the lowest key position holding the tile max, over both lane halves)
    const bool improve = tmax2 > st.mx;
    if (__any(improve)) {
      int targ = 0x7fffffff;
#pragma unroll
      for (int e = 15; e >= 0; --e) {
        const int kk = 8 * (e >> 2) + 4 * c.half + (e & 3);
        if (sacc[e] == tmax) targ = kb + kk;
      }
      targ = min(targ, other_half(targ));
      if (improve) st.best_j = targ;
    }
  }
  st.mx = fmaxf(st.mx, tmax2);
  tmax = tmax2;

  // lazy rescale of the running max (rare after the first tile). A row whose running max is
  // still -inf has O = 0 and lsum = 0 (every P it has seen was exp2(-inf) = 0), so it only
  // takes the new max: the first tile of a split rescales nothing.
  const bool need = tmax > st.m + kRescale;
  const bool rescale = need && st.m != -INFINITY;
  if (__any(rescale)) {
    const float alpha = rescale ? __builtin_amdgcn_exp2f(st.m - tmax) : 1.f;
    st.lsum *= alpha;
    if constexpr (kAgpr) {
      matrix_drain();
#pragma unroll
      for (int d = 0; d < kOBlocks; ++d) scale_acc(o[d], alpha);
      matrix_drain();
    } else {
#pragma unroll
      for (int d = 0; d < kOBlocks; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
    }
  }
  if (need) st.m = tmax;
}

// ---- the balanced work list
//
// Request r (a usable segment with T_r > 0) has rt_r = ceil(T_r H / 128) row tiles and
// kt_r = ceil(L_r / 32) key tiles. Its keys are cut into n_r = ceil(kt_r / ct_r) splits of
// at most ct_r key tiles, as even as the count allows (split_range), and a work item is one
// (split, row tile) pair. Items are
// numbered request by request, split-major with the row tile fastest, so consecutive items
// (which the launch places on one XCD) read the same key rows. Every workgroup computes the
// same plan from the index tables, with no host involvement:
//  * a fixed split count S: ct_r = ceil(kt_r / S);
//  * otherwise one common ct for every request, the smallest for which the batch has at most
//    G items (G = the grid, one workgroup per compute unit), so each workgroup gets one item
//    and the largest item is as small as the cut allows; when the requests have G row tiles
//    or more, one split per request.
// The launch has a workgroup for every item. Partial rows: request r's n_r * T_r H rows
// follow those of the requests before it.
struct ReqWork {
  Segment seg;
  int32_t rows;  // T_r * H; 0 when the request has nothing to compute
  int32_t rt;    // row tiles
  int32_t kt;    // key tiles
  uint32_t bad;  // VA_DEV_* bits of an unusable segment
};

__device__ __forceinline__ ReqWork req_work(const RunArgs &a, int r) {
  ReqWork q;
  q.rows = q.rt = q.kt = 0;
  q.bad = 0;
  q.seg.T = q.seg.L = q.seg.P = 0;
  q.seg.q0 = q.seg.kv0 = q.seg.m0 = 0;
  q.seg.tree = nullptr;
  if (r < a.bs) {
    q.bad = load_segment(a, r, q.seg);
    if (q.bad == 0 && q.seg.T > 0) {
      q.rows = q.seg.T * a.H;  // T <= 65536, H <= 4096
      q.rt = (q.rows + kRows - 1) / kRows;
      q.kt = (q.seg.L - 1) / kTK + 1;  // L >= T >= 1
    }
  }
  return q;
}

// Key tiles per split, and the split count, of a request under the plan (c, forced).
__device__ __forceinline__ int split_tiles(int kt, int c, int forced) {
  return forced > 0 ? (kt + forced - 1) / forced : min(c, kt);
}
__device__ __forceinline__ int split_count(const ReqWork &q, int c, int forced) {
  if (q.rt == 0) return 0;
  const int ct = split_tiles(q.kt, c, forced);
  return (q.kt + ct - 1) / ct;
}
// Keys [k0, k1) of split k of n over L keys: the kt = ceil(L / 32) key tiles are dealt so
// that the first kt % n splits take one tile more than the others (every split has at least
// one tile, as n <= kt). Uneven splits let the workgroups with fewer tiles write their
// partials while the others still compute, instead of every workgroup writing at once.
__device__ __forceinline__ void split_range(int L, int k, int n, int &k0, int &k1) {
  const int kt = (L - 1) / kTK + 1;
  const int q = kt / n, r = kt % n;
  const int t0 = k * q + min(k, r);
  k0 = t0 * kTK;
  k1 = min(L, (t0 + q + (k < r ? 1 : 0)) * kTK);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

struct WorkPlan {
  int c;          // key tiles per split (common cut)
  int forced;     // splits per request (0: common cut)
  int64_t items;  // work items in all
};

// Request base + lane: chunk 0 comes from the lane's cached request when kCached.
template <bool kCached>
__device__ __forceinline__ ReqWork chunk_request(const RunArgs &a, const ReqWork &mine,
                                                 int base, int lane) {
  if (kCached && base == 0) return mine;
  return req_work(a, base + lane);
}

__device__ int64_t count_items(const RunArgs &a, const ReqWork &mine, int c, int forced,
                               int lane) {
  if (a.bs == 1) {  // one request (lane 0's): no cross-lane sum
    ReqWork q = mine;
    q.rt = uniform(q.rt);
    q.kt = uniform(q.kt);
    return int64_t(q.rt) * split_count(q, c, forced);
  }
  int64_t n = 0;
  for (int base = 0; base < a.bs; base += 64) {
    const ReqWork q = chunk_request<true>(a, mine, base, lane);
    n += wave_sum_i64(int64_t(q.rt) * split_count(q, c, forced));
  }
  return uniform(n);
}

__device__ WorkPlan plan_work(const RunArgs &a, const ReqWork &mine, int G, int forced,
                              uint32_t *status, bool report, int lane) {
  WorkPlan p;
  p.c = 1;
  p.forced = forced;
  int64_t C = 0, RT = 0;
  int ktmax = 0;
  if (a.bs == 1) {  // one request (lane 0's): no cross-lane sums
    if (report && lane == 0 && mine.bad) atomicOr(status, mine.bad);
    const int rt = uniform(mine.rt), kt = uniform(mine.kt);
    C = int64_t(rt) * kt;
    RT = rt;
    ktmax = kt;
  } else {
    for (int base = 0; base < a.bs; base += 64) {
      const ReqWork q = chunk_request<true>(a, mine, base, lane);
      if (report && q.bad) atomicOr(status, q.bad);
      C += wave_sum_i64(int64_t(q.rt) * q.kt);
      RT += wave_sum_i64(int64_t(q.rt));
      ktmax = max(ktmax, wave_max_i32(q.kt));
    }
    C = uniform(C);
    RT = uniform(RT);
    ktmax = uniform(ktmax);
  }
  if (forced > 0 || C == 0) {
    p.items = C == 0 ? 0 : count_items(a, mine, 1, forced, lane);
    return p;
  }
  int64_t c = (C + G - 1) / G;
  if (RT >= G) {
    c = ktmax;
  } else if (count_items(a, mine, int(min(c, int64_t(ktmax))), 0, lane) > G) {
    // items(c) <= C / c + RT, so ceil(C / (G - RT)) tiles per split fit G items; the count
    // does not grow with c: bisect for the smallest c that fits
    int64_t lo = c, hi = (C + (G - RT) - 1) / (G - RT);
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) >> 1;
      if (count_items(a, mine, int(min(mid, int64_t(ktmax))), 0, lane) <= G) hi = mid;
      else lo = mid;
    }
    c = hi;
  }
  p.c = int(min(c, int64_t(ktmax)));
  p.items = count_items(a, mine, p.c, 0, lane);
  return p;
}

struct Item {
  Segment seg;
  int rows;      // T_r * H
  int rt;        // row tile
  int k;         // split
  int n;         // splits of the request
  int64_t prow;  // the request's first partial row
};

__device__ __forceinline__ Segment uniform(const Segment &s) {
  Segment u;
  u.q0 = uniform(s.q0);
  u.T = uniform(s.T);
  u.L = uniform(s.L);
  u.P = uniform(s.P);
  u.kv0 = uniform(s.kv0);
  u.m0 = uniform(s.m0);
  u.tree = s.tree;
  return u;
}

template <bool kCached>
__device__ bool find_item(const RunArgs &a, const ReqWork &mine, const WorkPlan &p, int64_t w,
                          int lane, Item &it) {
  if (kCached && a.bs == 1) {  // one request (lane 0's): item w is its split w / rt, tile w % rt
    ReqWork q = mine;
    q.rows = uniform(q.rows);
    q.rt = uniform(q.rt);
    q.kt = uniform(q.kt);
    const int n = split_count(q, p.c, p.forced);
    if (q.rt == 0 || w >= int64_t(q.rt) * n) return false;
    it.seg = uniform(q.seg);
    it.seg.tree = a.out_cache_loc ? a.out_cache_loc + it.seg.q0 : nullptr;
    it.rows = q.rows;
    it.rt = int(w % q.rt);
    it.k = int(w / q.rt);
    it.n = n;
    it.prow = 0;
    return true;
  }
  // Items are numbered request by request (lane r holds request base + r): the request
  // holding item w is the one whose range [lo, lo + items) of item numbers contains it, from
  // prefix sums over the lanes; its values come to scalar registers by lane reads.
  int64_t first = 0, prow = 0;
  for (int base = 0; base < a.bs; base += 64) {
    const ReqWork q = chunk_request<kCached>(a, mine, base, lane);
    const int n = split_count(q, p.c, p.forced);
    const int64_t items = int64_t(q.rt) * n;
    const int64_t prows = int64_t(n) * q.rows;
    const int64_t si = wave_inclusive_scan_i64(items);
    const int64_t sp = wave_inclusive_scan_i64(prows);
    const int64_t lo = first + si - items;
    const uint64_t hit = __ballot(items > 0 && lo <= w && w < lo + items);
    if (hit) {
      const int r = __builtin_ctzll(hit);
      const int64_t local = w - lane_i64(lo, r);
      it.seg.q0 = lane_i64(q.seg.q0, r);
      it.seg.T = lane_i32(q.seg.T, r);
      it.seg.L = lane_i32(q.seg.L, r);
      it.seg.P = lane_i32(q.seg.P, r);
      it.seg.kv0 = lane_i64(q.seg.kv0, r);
      it.seg.m0 = lane_i64(q.seg.m0, r);
      // rebuilt from the kernel argument rather than moved between lanes, so that the
      // compiler still knows it points to global memory (it would otherwise use flat loads)
      it.seg.tree = a.out_cache_loc ? a.out_cache_loc + it.seg.q0 : nullptr;
      it.rows = lane_i32(q.rows, r);
      const int rt = lane_i32(q.rt, r);
      it.rt = int(local % rt);
      it.k = int(local / rt);
      it.n = lane_i32(n, r);
      it.prow = prow + lane_i64(sp - prows, r);
      return true;
    }
    first += lane_i64(si, 63);
    prow += lane_i64(sp, 63);
  }
  return false;
}

// One work item: split it.k of row tile it.rt of one request.
// The slots of this wavefront's 8 rows of tile t into g_slots[t & 1][wave]: lane l < 16
// loads dword l & 1 of row l >> 1's slot (keys past the split load a valid entry of the split
// instead, and read_slots discards it). One load instruction per call.
__device__ __forceinline__ void load_slots_lds(const Ctx &c, int t) {
  if (c.lane < 2 * kRowsPerWave) {
    const int j = c.k0 + t * kTK + c.wave * kRowsPerWave + (c.lane >> 1);
    const int jc = min(j, c.k1 - 1);
    const int64_t *e = (c.tree && jc >= c.P) ? c.tree + (jc - c.P) : c.kvi + jc;
    dma_dword_lanes(reinterpret_cast<const uint32_t *>(e) + (c.lane & 1),
                    lds_addr(reinterpret_cast<const char *>(&g_slots[t & 1][c.wave][0])));
  }
}
// Lane l's slot of row l & 7 of tile t from g_slots (-1 past the split), once loaded.
__device__ __forceinline__ int64_t read_slots(const Ctx &c, int t) {
  const int j = c.k0 + t * kTK + c.wave * kRowsPerWave + (c.lane & 7);
  // (a plain LDS read: the wait before it is an assembly statement with a memory clobber, so
  // the read is not moved above it)
  const int64_t v = g_slots[t & 1][c.wave][c.lane & 7];
  return j < c.k1 ? v : -1;
}

template <bool kArgmax>
__device__ __forceinline__ void run_item(const RunArgs &a, const Workspace &ws, const Item &it) {
  const Segment &seg = it.seg;
  const int H = a.H;
  const int rows_req = it.rows;
  const int row0 = it.rt * kRows;

  Ctx c;
  c.kv = static_cast<const uint16_t *>(a.kv);
  c.kvi = a.kv_indices + seg.kv0;
  c.tree = seg.tree;
  c.zero = ws.zero_row;
  c.num_slots = a.num_slots;
  c.status = ws.status;
  c.P = seg.P;
  c.wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  c.lane = int(threadIdx.x) & 63;
  c.half = c.lane >> 5;
  c.col = c.lane & 31;
  const int rho = row0 + c.wave * 32 + c.col;  // local row: token rho / H, head rho % H
  const bool row_ok = rho < rows_req;
  // a wavefront past the request's rows only stages its share of each tile
  const bool active = row0 + c.wave * 32 < rows_req;  // wave-uniform
  const int rho_c = row_ok ? rho : rows_req - 1;  // rows past the end compute, never write
  const int tok = rho_c / H;
  const int64_t grow = (seg.q0 + tok) * int64_t(H) + rho_c % H;

  // this split's keys: whole tiles, at least one (k0 < L)
  split_range(seg.L, it.k, it.n, c.k0, c.k1);
  const int ntiles = (c.k1 - c.k0 + kTK - 1) / kTK;

  const LaneOffs lo = lane_offsets(c);
  char *const raw0 = g_lds;
  char *const raw1 = g_lds + kRawTile;
  char *const v0 = g_lds + kVOff;
  char *const v1 = g_lds + kVOff + kVTile;

  // ---- prologue. The query rows are staged through LDS in two halves (dims [0, 288) and
  // [288, 576)), in the region of the two fp16 tiles, while tiles 0 and 1 load into the raw
  // buffers: wavefront w's half block sits at kVOff + w * 32 * kQHStride, row r at
  // r * kQHStride (36 units of 16 bytes and a pad unit, so that the fragment reads fall in
  // distinct banks), and load i fills bytes [1024 i, 1024 i + 1024) of it, consecutive rows of
  // q. Every load here is an assembly LDS load whose completion the code counts itself (the
  // slots of tiles 0 and 1 also travel through LDS): a register result would make the
  // compiler wait for every load before it. Issue order and waits:
  //   slots of tiles 0, 1 (2) | half A (19) -> wait: slots landed
  //   tile 0 rows (9) | tile 1 rows (9) | slots of tile 2 (1) -> wait: half A landed
  //   half B (19) into the same place -> wait: everything
  constexpr int kQHUnits = kQFrags + 1;             // 37
  constexpr int kQHStride = 16 * kQHUnits;          // 592
  constexpr int kQHChunks = 32 * kQHUnits;          // 1184
  constexpr int kQHLoads = (kQHChunks + 63) / 64;   // 19
  static_assert(kVOff + kWaves * 32 * kQHStride <= kXOff + kXBytes, "query halves fit in LDS");
  char *const qblk = g_lds + kVOff + c.wave * 32 * kQHStride;
  // the wavefront's rows, clamped to the request's last row (an idle wavefront stages that
  // row only)
  const int64_t row_first = seg.q0 * H + row0 + c.wave * 32;
  const int64_t row_last = seg.q0 * H + rows_req - 1;
  const int64_t base_row = min(row_first, row_last);
  const int nrows = int(min(int64_t(32), row_last - base_row + 1));
  const uint64_t qbase =
      uint64_t(reinterpret_cast<uintptr_t>(a.q)) + uint64_t(base_row) * (2 * kDim);
  const uint32_t qlim = uint32_t(nrows * (2 * kDim) - 16);
  // chunk ch = 64 i + lane of half h is unit p = ch % 37 of row r = ch / 37, q unit
  // 36 h + p of that row: byte 16 (ch + 35 r) + 576 h past the first row (the pad unit reads
  // the unit after the half, inside the clamped rows)
  auto stage_half = [&](int h) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kQHLoads; ++i) {
      const int ch = 64 * i + c.lane;
      const uint32_t voff = min(uint32_t(16 * (ch + 35 * (ch / kQHUnits)) + 576 * h), qlim);
      if (64 * (i + 1) <= kQHChunks || ch < kQHChunks)
        dma_row(qbase, voff, lds_addr(qblk) + 1024 * i);
    }
  };
  u32x4 qv[kQFrags];
  auto read_half = [&](int h) __attribute__((always_inline)) {
    const char *qr = qblk + c.col * kQHStride + 16 * c.half;
#pragma unroll
    for (int k = 0; k < kQFrags / 2; ++k)
      qv[h * (kQFrags / 2) + k] = *reinterpret_cast<const u32x4 *>(qr + 32 * k);
  };
  // (nothing the plan loaded is still in flight; saying so keeps the compiler from inserting
  // a wait for it below, which would also wait for these loads)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  int64_t slot_vec = -1;
  if (ntiles > 0) {
    load_slots_lds(c, 0);
    load_slots_lds(c, 1);
  }
  stage_half(0);
  asm volatile("s_waitcnt vmcnt(19)" ::: "memory");  // the slots of tiles 0 and 1
  if (ntiles > 0) {
    const TileLoads t0 = plan_tile(c, 0, read_slots(c, 0));
    const TileLoads t1 = plan_tile(c, 1, read_slots(c, 1));
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) issue_latent(c, t0, lds_addr(raw0), i);
    issue_rope(c, t0, lds_addr(raw0));
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) issue_latent(c, t1, lds_addr(raw1), i);
    issue_rope(c, t1, lds_addr(raw1));
    publish_ok(c, 0, t0.ok);
    publish_ok(c, 1, t1.ok);
    slot_vec = fetch_slot(c, 2);
  }
  asm volatile("s_waitcnt vmcnt(19)" ::: "memory");  // half A
  read_half(0);
  // (half B overwrites what was just read: the reads must be complete)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  stage_half(1);
  wait_tile_loads();
  read_half(1);
  // keep the query fragments resident: without this the compiler re-reads them inside the
  // tile loop
  bf16x8 qf[kQFrags];
#pragma unroll
  for (int kc = 0; kc < kQFrags; ++kc) {
    asm volatile("" : "+v"(qv[kc]));
    qf[kc] = __builtin_bit_cast(bf16x8, qv[kc]);
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

  f16x8 pf[2];
  if (ntiles > 0) {
    // q and tile 0 have landed once at most the 9 loads of tile 1 and the slot fetch of tile 2
    // are outstanding; tile 1 is waited for before the barrier that ends step 0
    wait_loads_but_10();
    __syncthreads();
    TileLoads none;
    none.addr = 0;
    none.ok = 0;
    // S(0) and the fp16 copy of tile 0, its max
    f32x16 scur;
    {
      StepIO io;
      io.kraw = raw0;
      io.vrd = v0;
      io.vwr = v0;
      io.dma_raw = 0;
      const f32x16 unused = {};
      if (active) {
        step<kFirst>(c, lo, io, none, slot_vec, 0, qf, o, scur, unused, st, c2, pf);
        score_max<kArgmax>(c, c.k0, g_okbits[0], scur, o, st, c2, row_ok, mseg, moff);
      } else {
        step<kFirst, false>(c, lo, io, none, slot_vec, 0, qf, o, scur, unused, st, c2, pf);
      }
    }
    wait_tile_loads();
    __syncthreads();

    // steady state: step t finishes the softmax of tile t and multiplies P(t) V(t), computes
    // S(t+1) and its max, converts tile t+1 to fp16 and loads tile t+2 (zero rows once past
    // the split)
    for (int t = 0; t + 1 < ntiles; ++t) {
      const int b = t & 1;
      const TileLoads tl = plan_tile(c, t + 2, slot_vec);
      StepIO sio;
      sio.kraw = b ? raw0 : raw1;
      sio.vrd = b ? v1 : v0;
      sio.vwr = b ? v0 : v1;
      sio.dma_raw = lds_addr(b ? raw1 : raw0);
      publish_ok(c, b, tl.ok);
      f32x16 snext;
      if (active) {
        step<kMain>(c, lo, sio, tl, slot_vec, t + 3, qf, o, snext, scur, st, c2, pf);
        score_max<kArgmax>(c, c.k0 + (t + 1) * kTK, g_okbits[b ^ 1], snext, o, st, c2, row_ok,
                           mseg, moff);
        scur = snext;
      } else {
        step<kMain, false>(c, lo, sio, tl, slot_vec, t + 3, qf, o, snext, scur, st, c2, pf);
      }
      wait_tile_loads();
      __syncthreads();
    }

    // P(t) V(t) of the last tile
    StepIO eio;
    eio.kraw = raw0;
    eio.vrd = ((ntiles - 1) & 1) ? v1 : v0;
    eio.vwr = v0;
    eio.dma_raw = 0;
    f32x16 unused2;
    if (active) step<kLast>(c, lo, eio, none, slot_vec, 0, qf, o, unused2, scur, st, c2, pf);
  }

  // ---- write the partial of this split
  if (!active) return;
  matrix_drain();
  const float ltot = st.lsum + other_half(st.lsum);
  if (!row_ok) return;
  const int64_t prow = it.prow + int64_t(it.k) * rows_req + rho;
  if (prow >= ws.part_rows) {  // cannot happen: the workspace is sized for every plan
    atomicOr(ws.status, 2u);   // VA_DEV_SEGMENT
    return;
  }
  if (it.k == 0 && c.half == 0) {
    RowInfo ri;
    ri.base = it.prow + rho;
    ri.n = it.n;
    ri.stride = rows_req;
    ws.row_info[grow] = ri;
  }
  // int16 codes: each 128-dim group g (output blocks 4g .. 4g+3) is coded against its
  // largest magnitude, am, and stored with the scale am / (32767 l). A group's 64
  // accumulators per lane are read out of the matrix registers once and kept in VGPRs (the
  // query fragments are dead by now) for both the maximum and the coding.
  int16_t *pq = static_cast<int16_t *>(ws.part_o) + prow * kLatent;
  float scl[kScaleGroups];
#pragma unroll
  for (int g = 0; g < kScaleGroups; ++g) {
    float v[4][16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) v[i][e] = o[4 * g + i][e];
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[i][e]));
    m = fmaxf(m, other_half(m));
    const float f = m > 0.f ? __builtin_amdgcn_rcpf(m) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t cw[4][2];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        cw[gq][0] = snorm16x2(v[i][4 * gq] * f, v[i][4 * gq + 1] * f);
        cw[gq][1] = snorm16x2(v[i][4 * gq + 2] * f, v[i][4 * gq + 3] * f);
      }
      store_codes(pq, 4 * g + i, c.half, cw);
    }
    scl[g] = m;
  }
  if (c.half == 0) {
    const float sl = ltot > 0.f ? 1.f / (32767.f * ltot) : 0.f;
    *reinterpret_cast<float4 *>(ws.part_scale + kScaleGroups * prow) =
        make_float4(scl[0] * sl, scl[1] * sl, scl[2] * sl, scl[3] * sl);
    const bool any = ltot > 0.f;
    ws.part_lse[prow] = any ? (st.m + log2f(ltot)) * kLn2 : -INFINITY;
    ws.part_max[prow] = any ? st.mx * kLn2 : -INFINITY;
    ws.part_arg[prow] = any && kArgmax ? st.best_j : -1;
  }
}


// ---- one work item of at most 32 rows: the four wavefronts share the rows and split the
// work. Wavefront w computes the scores over dims [144w, 144w + 144) (9 fragments), the four
// partial score tiles are summed through LDS in a fixed order (so every wavefront holds the
// same scores and makes the same softmax decisions), and wavefront w accumulates output dims
// [128w, 128w + 128). Per tile a wavefront issues 17 matrix instructions instead of 68, so a
// workgroup streams key tiles about as fast as its loads arrive. Tiles are staged exactly as
// in the 128-row path (same LDS layout, loads, fp16 conversion); the loads of tile t+2 are
// issued as soon as every wavefront is done with tile t's raw buffer.
constexpr int kNarrowFrags = kQFrags / kWaves;    // 9 score fragments per wavefront
constexpr int kNarrowBlocks = kDBlocks / kWaves;  // 4 output dim blocks per wavefront

template <bool kArgmax>
__device__ __forceinline__ void run_narrow(const RunArgs &a, const Workspace &ws,
                                           const Item &it) {
  const Segment &seg = it.seg;
  const int H = a.H;
  const int rows_req = it.rows;
  const int row0 = it.rt * kRows;

  Ctx c;
  c.kv = static_cast<const uint16_t *>(a.kv);
  c.kvi = a.kv_indices + seg.kv0;
  c.tree = seg.tree;
  c.zero = ws.zero_row;
  c.num_slots = a.num_slots;
  c.status = ws.status;
  c.P = seg.P;
  c.wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  c.lane = int(threadIdx.x) & 63;
  c.half = c.lane >> 5;
  c.col = c.lane & 31;
  const int rho = row0 + c.col;  // every wavefront: the same 32 rows
  const bool row_ok = rho < rows_req;
  const int rho_c = row_ok ? rho : rows_req - 1;
  const int tok = rho_c / H;
  const int64_t grow = (seg.q0 + tok) * int64_t(H) + rho_c % H;

  split_range(seg.L, it.k, it.n, c.k0, c.k1);
  const int ntiles = (c.k1 - c.k0 + kTK - 1) / kTK;

  const LaneOffs lo = lane_offsets(c);
  char *const raw0 = g_lds;
  char *const raw1 = g_lds + kRawTile;
  char *const v0 = g_lds + kVOff;
  char *const v1 = g_lds + kVOff + kVTile;
  float4 *const xbuf = reinterpret_cast<float4 *>(g_lds + kXOff);
  const int kc0 = kNarrowFrags * c.wave;  // this wavefront's first score fragment

  // ---- prologue: slots of tiles 0 and 1, this wavefront's 9 query fragments (straight into
  // registers: 9 loads per lane), the loads of tiles 0 and 1, the slots of tile 2
  int64_t s0 = fetch_slot(c, 0);
  int64_t s1 = fetch_slot(c, 1);
  u32x4 qv[kNarrowFrags];
  {
    const uint4 *qrow = reinterpret_cast<const uint4 *>(
        static_cast<const uint16_t *>(a.q) + grow * kDim);
#pragma unroll
    for (int i = 0; i < kNarrowFrags; ++i)
      qv[i] = __builtin_bit_cast(u32x4, qrow[2 * (kc0 + i) + c.half]);
  }
  // Key slots from tile 2 on travel through LDS (load_slots_lds / read_slots), loaded by one
  // load instruction per tile whose completion the code tracks itself: every wait below is
  // for a known number of newer loads (the compiler does not count these assembly loads, so a
  // register result would be waited for with vmcnt(0), draining the tile loads behind it).
  // Issue order per tile: its slots, then (a tile later) its 9 row loads.
  {
    const TileLoads t0 = plan_tile(c, 0, s0);
    const TileLoads t1 = plan_tile(c, 1, s1);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) issue_latent(c, t0, lds_addr(raw0), i);
    issue_rope(c, t0, lds_addr(raw0));
    load_slots_lds(c, 2);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) issue_latent(c, t1, lds_addr(raw1), i);
    issue_rope(c, t1, lds_addr(raw1));
    publish_ok(c, 0, t0.ok);
    publish_ok(c, 1, t1.ok);
  }
  bf16x8 qf[kNarrowFrags];
#pragma unroll
  for (int i = 0; i < kNarrowFrags; ++i) {
    asm volatile("" : "+v"(qv[i]));
    qf[i] = __builtin_bit_cast(bf16x8, qv[i]);
  }
  // operand offsets of this wavefront's score fragments (latent, or rope for kc >= 32)
  uint32_t koff[kNarrowFrags];
#pragma unroll
  for (int i = 0; i < kNarrowFrags; ++i) {
    const int kc = kc0 + i;
    koff[i] = kc < kLatFrags ? lo.k_lat + 32 * kc : lo.k_rope + 256 * (kc - kLatFrags);
  }

  f32x16 o[kNarrowBlocks];
#pragma unroll
  for (int d = 0; d < kNarrowBlocks; ++d) {
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
  const uint8_t *mseg = a.mask + seg.m0;
  const uint32_t moff = uint32_t(tok) * uint32_t(seg.L);

  for (int t = 0; t < ntiles; ++t) {
    const int b = t & 1;
    const char *kraw = b ? raw1 : raw0;
    char *vbuf = b ? v1 : v0;
    // tile t (and q) landed: the slots of tile t+2 and the 9 loads of tile t+1 are newer
    wait_loads_but_10();
    __syncthreads();
    const uint32_t ok_t = g_okbits[b];

    // this wavefront's partial scores of tile t (one chain) and the fp16 copy of the units
    // this thread loaded. Every LDS read of the phase is issued first: the assembly matrix
    // instructions end the compiler's scheduling regions, so reads placed between them would
    // each wait out a full LDS round trip.
    u32x4 kf[kNarrowFrags], craw[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kNarrowFrags; ++i)
      kf[i] = *reinterpret_cast<const u32x4 *>(kraw + koff[i]);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
      craw[i] = *reinterpret_cast<const u32x4 *>(kraw + lo.cv_rd + kLatStride * i);
    f32x16 part;
    static_for<0, kNarrowFrags>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      const bf16x8 av = __builtin_bit_cast(bf16x8, kf[i]);
      if constexpr (i == 0) {
        const f32x16 zero = {};
        part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[i], zero, 0, 0, 0);
      } else {
        part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[i], part, 0, 0, 0);
      }
      // the fp16 copy of one unit after each matrix instruction, so that the conversion
      // work issues while the matrix core runs
      if constexpr (i < kRowsPerWave) {
#pragma unroll
        for (int q = 0; q < 4; ++q) craw[i][q] = bf16pair_to_f16pair(craw[i][q]);
        *reinterpret_cast<u32x4 *>(vbuf + lo.cv_wr + kVRow * i) = craw[i];
      }
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xbuf[(c.wave * 4 + q) * 64 + c.lane] =
          make_float4(part[4 * q], part[4 * q + 1], part[4 * q + 2], part[4 * q + 3]);
    // every wavefront's partial scores are out, tile t's raw buffer is no longer read and its
    // fp16 copy is complete
    __syncthreads();

    // the four partial scores, requested before the loads below are issued
    float4 xs[4][kWaves];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int w = 0; w < kWaves; ++w) xs[q][w] = xbuf[(w * 4 + q) * 64 + c.lane];
    // the slots of tile t+3, then the loads of tile t+2 into tile t's raw buffer (zero rows
    // past the split) once its slots, older than the 9 loads of tile t+1 and the slot load
    // just issued, have landed
    {
      load_slots_lds(c, t + 3);
      wait_loads_but_10();
      const TileLoads tl = plan_tile(c, t + 2, read_slots(c, t + 2));
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) issue_latent(c, tl, lds_addr(kraw), i);
      issue_rope(c, tl, lds_addr(kraw));
      publish_ok(c, b, tl.ok);
    }

    // the scores: the four partials summed in wavefront order
    f32x16 sc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 x = xs[q][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        const float4 y = xs[q][w];
        x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
      }
      sc[4 * q] = x.x; sc[4 * q + 1] = x.y; sc[4 * q + 2] = x.z; sc[4 * q + 3] = x.w;
    }
    score_max<kArgmax, kNarrowBlocks>(c, c.k0 + t * kTK, ok_t, sc, o, st, c2, row_ok, mseg,
                                      moff);
    f16x8 pf[2];
    const float negm = neg_max(st);
#pragma unroll
    for (int part_i = 0; part_i < 8; ++part_i) p_part(part_i, sc, c2, negm, st.lsum, pf);
    // a matrix instruction that reads a VGPR written by VALU needs 2 wait states; the
    // compiler does not see the assembly matrix instructions below as such
    asm volatile("s_nop 1" : "+v"(pf[0]), "+v"(pf[1]));

    // O[:, 128w .. 128w+128) += P V over the tile's 32 keys (all V^T reads first, as above)
    const char *vtr = vbuf + lo.v_tr;
    u32x4 vf[2][kNarrowBlocks];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
      for (int db = 0; db < kNarrowBlocks; ++db) {
        const int d = kNarrowBlocks * c.wave + db;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const fp16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
              (lds_fp16x4 *)(vtr + (16 * ch + 8 * rr) * kVRow + 64 * d));
          const u32x2 w2 = __builtin_bit_cast(u32x2, x);
          vf[ch][db][2 * rr] = w2[0];
          vf[ch][db][2 * rr + 1] = w2[1];
        }
      }
    }
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
      for (int db = 0; db < kNarrowBlocks; ++db) pv_mfma(o[db], vf[ch][db], pf[ch]);
    }
  }

  // ---- write this wavefront's 128 dims of the split's partial (and, from wavefront 0, the
  // row's scalars and placement)
  matrix_drain();
  const float ltot = st.lsum + other_half(st.lsum);
  if (!row_ok) return;
  const int64_t prow = it.prow + int64_t(it.k) * rows_req + rho;
  if (prow >= ws.part_rows) {  // cannot happen: the workspace is sized for every plan
    atomicOr(ws.status, 2u);   // VA_DEV_SEGMENT
    return;
  }
  // int16 codes: this wavefront's 128 dims are one scale group (see the 128-row path)
  static_assert(kNarrowBlocks * 32 == kScaleGroupDims, "a wavefront's dims are one group");
  float v[kNarrowBlocks][16];
#pragma unroll
  for (int db = 0; db < kNarrowBlocks; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) v[db][e] = o[db][e];
  float am = 0.f;
#pragma unroll
  for (int db = 0; db < kNarrowBlocks; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(v[db][e]));
  am = fmaxf(am, other_half(am));
  const float f = am > 0.f ? __builtin_amdgcn_rcpf(am) : 0.f;
  int16_t *pq = static_cast<int16_t *>(ws.part_o) + prow * kLatent;
#pragma unroll
  for (int db = 0; db < kNarrowBlocks; ++db) {
    const int d = kNarrowBlocks * c.wave + db;
    uint32_t cw[4][2];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      cw[gq][0] = snorm16x2(v[db][4 * gq] * f, v[db][4 * gq + 1] * f);
      cw[gq][1] = snorm16x2(v[db][4 * gq + 2] * f, v[db][4 * gq + 3] * f);
    }
    store_codes(pq, d, c.half, cw);
  }
  if (c.half == 0)
    ws.part_scale[kScaleGroups * prow + c.wave] = ltot > 0.f ? am / (32767.f * ltot) : 0.f;
  if (c.wave == 0 && c.half == 0) {
    if (it.k == 0) {
      RowInfo ri;
      ri.base = it.prow + rho;
      ri.n = it.n;
      ri.stride = rows_req;
      ws.row_info[grow] = ri;
    }
    const bool any = ltot > 0.f;
    ws.part_lse[prow] = any ? (st.m + log2f(ltot)) * kLn2 : -INFINITY;
    ws.part_max[prow] = any ? st.mx * kLn2 : -INFINITY;
    ws.part_arg[prow] = any && kArgmax ? st.best_j : -1;
  }
}

// ---- two wavefronts per SIMD: score and value wavefronts
//
// A variant of the 128-row item for H a multiple of 64 (then no item has 32 rows or fewer).
// One wavefront per SIMD leaves nothing to issue beside a wavefront's matrix instructions;
// this one runs eight, two per SIMD, each within 256 registers:
//  * score wavefront g (g < 4) holds the 32 query rows of row group g (144 registers) and
//    computes S^T = K Q^T of every tile, the mask, max, argmax and lazy rescale, and the
//    fp16 P, which it hands to its value wavefront through LDS; it accumulates output dims
//    [0, 128) (4 of the 16 dim blocks, 64 registers);
//  * value wavefront 4 + g accumulates dims [128, 512) of the same rows (12 blocks, 192
//    registers) from that P, and does all the staging the four wavefronts of the other
//    variant share (slots, tile loads, fp16 copy), as staging wavefront g.
// Both kinds take the same barriers: one per tile as before, so P(t) is written in step t-1
// and read in step t from a buffer of its own parity. The value wavefront mirrors the running
// max: it receives it with P and rescales its accumulators exactly when the score wavefront
// rescales its own (same operands, same instruction).
constexpr int kWsThreads = 2 * kThreads;
constexpr int kABlocks = 4;                   // output dim blocks of a score wavefront
constexpr int kBBlocks = kDBlocks - kABlocks;   // 12 of a value wavefront
constexpr int kSplitG = kABlocks / 4;           // the scale group the two kinds may share
constexpr bool kSplit = kABlocks % 4 != 0;      // whether they share it
constexpr int kDepthA = 2;                      // operand reads in flight, score wavefront
constexpr int kDepthB = 3;                      // and value wavefront
constexpr int kXPair = 2 * 64 * 16 + 64 * 4;  // P (two 16-key chunks) and the running max
constexpr int kWsXOff = kLdsBytes;
constexpr int kWsLds = kWsXOff + 2 * kWaves * kXPair;  // 162,816
static_assert(kWsLds + sizeof(g_slots) + sizeof(g_okbits) <= 160 * 1024, "LDS budget");
static_assert(kVOff + kWaves * 32 * 16 * (kQFrags + 1) <= kWsLds, "query halves fit in LDS");
__shared__ __attribute__((aligned(16))) char g_ldsw[kWsLds];

// The operand fragment of a QK^T fragment (kPv false, kIdx 0..35) or of P.V product kIdx
// (key chunk kIdx / kNBlk, dim block kBlk0 + kIdx % kNBlk).
template <bool kPv, int kIdx, int kBlk0, int kNBlk>
__device__ __forceinline__ u32x4 op_frag(const char *klat, const char *krope, const char *vtr) {
  u32x4 r;
  if constexpr (!kPv) {
    if constexpr (kIdx < kLatFrags)
      r = *reinterpret_cast<const u32x4 *>(klat + 32 * kIdx);
    else
      r = *reinterpret_cast<const u32x4 *>(krope + 256 * (kIdx - kLatFrags));
  } else {
    constexpr int ch = kIdx / kNBlk, d = kBlk0 + kIdx % kNBlk;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const fp16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
          (lds_fp16x4 *)(vtr + (16 * ch + 8 * rr) * kVRow + 64 * d));
      const u32x2 w = __builtin_bit_cast(u32x2, x);
      r[2 * rr] = w[0];
      r[2 * rr + 1] = w[1];
    }
  }
  return r;
}

// Score wavefront, one step: kFirst - QK^T of tile 0; kMain - P(t).V(t) of its dim blocks,
// then QK^T of tile t+1 (P(t) is dead before the score accumulators are live); kLast -
// P(t).V(t).
template <int K>
__device__ __forceinline__ void ws_score_step(const LaneOffs &lo, const char *kraw,
                                              const char *vrd, const bf16x8 *qf, f32x16 *o,
                                              const f16x8 *pf, f32x16 &sa) {
  constexpr int kPV = K == kFirst ? 0 : 2 * kABlocks;
  constexpr int kQK = K == kLast ? 0 : kQFrags;
  constexpr int N = kPV + kQK;
  constexpr OpTable<N> T = [] {
    OpTable<N> t{};
    int p = 0;
    for (int i = 0; i < kPV; ++i) t.op[p++] = Op{1, int8_t(i)};
    for (int i = 0; i < kQK; ++i) t.op[p++] = Op{0, int8_t(i)};
    return t;
  }();
  const char *klat = kraw + lo.k_lat;
  const char *krope = kraw + lo.k_rope;
  const char *vtr = vrd + lo.v_tr;
  u32x4 fr[kDepthA + 1];
  auto load = [&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
    if constexpr (p < N) {
      constexpr Op op = T.op[p];
      fr[p % (kDepthA + 1)] = op_frag<op.pv != 0, op.idx, 0, kABlocks>(klat, krope, vtr);
    }
  };
  static_for<0, kDepthA>(load);
  static_for<0, N>([&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
    constexpr Op op = T.op[p];
    load(std::integral_constant<int, p + kDepthA>{});
    const u32x4 a = fr[p % (kDepthA + 1)];
    if constexpr (op.pv) {
      constexpr int ch = op.idx / kABlocks, d = op.idx % kABlocks;
      o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), pf[ch], o[d],
                                                    0, 0, 0);
    } else {
      const bf16x8 av = __builtin_bit_cast(bf16x8, a);
      if constexpr (op.idx == 0) {
        const f32x16 zero = {};
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[0], zero, 0, 0, 0);
      } else {
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[op.idx], sa, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Value wavefront: takes P(t) and the max it was computed against.
__device__ __forceinline__ float ws_take(const char *x, int lane, f16x8 *pf) {
  pf[0] = *reinterpret_cast<const f16x8 *>(x + 16 * lane);
  pf[1] = *reinterpret_cast<const f16x8 *>(x + 1024 + 16 * lane);
  return *reinterpret_cast<const float *>(x + 2048 + 4 * lane);
}
// ... and rescales its accumulators when the max moved (mb: the max they are relative to).
__device__ __forceinline__ void ws_rescale(float mn, float &mb, f32x16 *o) {
  const bool rescale = mn != mb && mb != -INFINITY;
  if (__any(rescale)) {
    const float alpha = rescale ? __builtin_amdgcn_exp2f(mb - mn) : 1.f;
#pragma unroll
    for (int d = 0; d < kBBlocks; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
  }
  mb = mn;
}

// Value wavefront, one step. With K == kMain it first stages (loads of tile t+2, the slots of
// tile t+3, the fp16 copy of tile t+1), while the score wavefront's QK^T chain holds the
// matrix core: issue is in order, so staging placed after a product would wait for that
// chain too. Then P(t).V(t) of its dim blocks, which runs while the score wavefront does the
// softmax of tile t+1.
template <int K>
__device__ __forceinline__ void ws_value_step(const Ctx &c, const LaneOffs &lo, const StepIO &io,
                                              const TileLoads &tl, int64_t &slot_vec,
                                              int slot_tile, f32x16 *o, const char *xp,
                                              float &mb) {
  constexpr int N = 2 * kBBlocks;
  // the copy's reads first: their latency passes while P is taken and the loads are issued
  u32x4 craw[kRowsPerWave];
  const char *cvr = io.kraw + lo.cv_rd;
  char *cvw = io.vwr + lo.cv_wr;
  if constexpr (K == kMain) {
#pragma unroll
    for (int u = 0; u < kRowsPerWave; ++u)
      craw[u] = *reinterpret_cast<const u32x4 *>(cvr + kLatStride * u);
  }
  f16x8 pf[2];
  const float mn = ws_take(xp, c.lane, pf);
  if constexpr (K == kMain) {
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) issue_latent(c, tl, io.dma_raw, i);
    issue_rope(c, tl, io.dma_raw);
    slot_vec = fetch_slot(c, slot_tile);
#pragma unroll
    for (int u = 0; u < kRowsPerWave; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) craw[u][i] = bf16pair_to_f16pair(craw[u][i]);
      *reinterpret_cast<u32x4 *>(cvw + kVRow * u) = craw[u];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  const char *vtr = io.vrd + lo.v_tr;
  u32x4 fr[kDepthB + 1];
  auto load = [&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
    if constexpr (p < N)
      fr[p % (kDepthB + 1)] = op_frag<true, p, kABlocks, kBBlocks>(nullptr, nullptr, vtr);
  };
  static_for<0, kDepthB>(load);
  ws_rescale(mn, mb, o);
  static_for<0, N>([&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
    load(std::integral_constant<int, p + kDepthB>{});
    constexpr int ch = p / kBBlocks, d = p % kBBlocks;
    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
        __builtin_bit_cast(f16x8, fr[p % (kDepthB + 1)]), pf[ch], o[d], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// The fp16 copy of a whole tile (the units this thread staged), with no products beside it.
__device__ __forceinline__ void ws_convert(const LaneOffs &lo, const char *raw, char *vt) {
  u32x4 u4[kRowsPerWave];
#pragma unroll
  for (int u = 0; u < kRowsPerWave; ++u)
    u4[u] = *reinterpret_cast<const u32x4 *>(raw + lo.cv_rd + kLatStride * u);
#pragma unroll
  for (int u = 0; u < kRowsPerWave; ++u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) u4[u][i] = bf16pair_to_f16pair(u4[u][i]);
    *reinterpret_cast<u32x4 *>(vt + lo.cv_wr + kVRow * u) = u4[u];
  }
}

// The hand-over of P(t) and the running max it was computed against (lane l: its P fragment
// words and its row's max).
__device__ __forceinline__ void ws_put(char *x, int lane, const f16x8 *pf, float m) {
  *reinterpret_cast<f16x8 *>(x + 16 * lane) = pf[0];
  *reinterpret_cast<f16x8 *>(x + 1024 + 16 * lane) = pf[1];
  *reinterpret_cast<float *>(x + 2048 + 4 * lane) = m;
}

// int16 codes of output blocks [d0, d0 + n) of this lane's row against the group maximum m
// (scale factor f = 1 / m, 0 when m is 0); a block's 16 accumulators per lane.
template <int kN>
__device__ __forceinline__ void ws_codes(int16_t *pq, int d0, int half, const f32x16 *o,
                                         float f) {
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    uint32_t cw[4][2];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      cw[gq][0] = snorm16x2(o[i][4 * gq] * f, o[i][4 * gq + 1] * f);
      cw[gq][1] = snorm16x2(o[i][4 * gq + 2] * f, o[i][4 * gq + 3] * f);
    }
    store_codes(pq, d0 + i, half, cw);
  }
}

template <int kN>
__device__ __forceinline__ float lane_absmax(const f32x16 *o) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < kN; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(o[i][e]));
  return m;
}

// What both kinds of wavefront know of the item.
struct WsItem {
  Ctx c;
  LaneOffs lo;
  int ntiles;
  bool active;   // the row group has rows of the request (wave-uniform)
  bool row_ok;   // this lane's row is one of them
  int rho;       // local row
  int tok;
  int64_t grow;
};

// Epilogue exchange (after the last tile): [wave g][lane] floats at x: ltot, the score
// wavefront's and the value wavefront's group-0 maxima.
__device__ __forceinline__ float *ws_ex(int g, int k) {
  return reinterpret_cast<float *>(g_ldsw + kWsXOff) + (3 * g + k) * 64;
}

template <bool kArgmax>
__device__ __forceinline__ void ws_score(const RunArgs &a, const Workspace &ws, const Item &it,
                                         const WsItem &w) {
  const Ctx &c = w.c;
  const Segment &seg = it.seg;
  const int H = a.H;
  const int rows_req = it.rows;
  const int row0 = it.rt * kRows;
  char *const raw0 = g_ldsw;
  char *const raw1 = g_ldsw + kRawTile;
  char *const v0 = g_ldsw + kVOff;
  char *const v1 = g_ldsw + kVOff + kVTile;

  // the query rows, staged through LDS in two halves as in the one-per-SIMD variant
  constexpr int kQHUnits = kQFrags + 1;
  constexpr int kQHStride = 16 * kQHUnits;
  constexpr int kQHChunks = 32 * kQHUnits;
  constexpr int kQHLoads = (kQHChunks + 63) / 64;
  char *const qblk = g_ldsw + kVOff + c.wave * 32 * kQHStride;
  const int64_t row_first = seg.q0 * H + row0 + c.wave * 32;
  const int64_t row_last = seg.q0 * H + rows_req - 1;
  const int64_t base_row = min(row_first, row_last);
  const int nrows = int(min(int64_t(32), row_last - base_row + 1));
  const uint64_t qbase =
      uint64_t(reinterpret_cast<uintptr_t>(a.q)) + uint64_t(base_row) * (2 * kDim);
  const uint32_t qlim = uint32_t(nrows * (2 * kDim) - 16);
  auto stage_half = [&](int h) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kQHLoads; ++i) {
      const int ch = 64 * i + c.lane;
      const uint32_t voff = min(uint32_t(16 * (ch + 35 * (ch / kQHUnits)) + 576 * h), qlim);
      if (64 * (i + 1) <= kQHChunks || ch < kQHChunks)
        dma_row(qbase, voff, lds_addr(qblk) + 1024 * i);
    }
  };
  u32x4 qv[kQFrags];
  auto read_half = [&](int h) __attribute__((always_inline)) {
    const char *qr = qblk + c.col * kQHStride + 16 * c.half;
#pragma unroll
    for (int k = 0; k < kQFrags / 2; ++k)
      qv[h * (kQFrags / 2) + k] = *reinterpret_cast<const u32x4 *>(qr + 32 * k);
  };
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing of the plan is still in flight
  stage_half(0);
  wait_tile_loads();
  read_half(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  stage_half(1);
  wait_tile_loads();
  read_half(1);
  bf16x8 qf[kQFrags];
#pragma unroll
  for (int kc = 0; kc < kQFrags; ++kc) {
    asm volatile("" : "+v"(qv[kc]));
    qf[kc] = __builtin_bit_cast(bf16x8, qv[kc]);
  }

  f32x16 o[kABlocks];
#pragma unroll
  for (int d = 0; d < kABlocks; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  RowState st;
  st.m = -INFINITY;
  st.mx = -INFINITY;
  st.lsum = 0.f;
  st.best_j = -1;
  const float c2 = a.scale * kLog2e;
  const uint8_t *mseg = a.mask + seg.m0;
  const uint32_t moff = uint32_t(w.tok) * uint32_t(seg.L);
  char *const xb = g_ldsw + kWsXOff + c.wave * kXPair;
  constexpr int kXPar = kWaves * kXPair;

  f16x8 pf[2];
  if (w.ntiles > 0) {
    __syncthreads();  // tile 0 has landed; every query half has been read
    f32x16 s;
    if (w.active) {
      ws_score_step<kFirst>(w.lo, raw0, v0, qf, o, pf, s);
      score_max<kArgmax, kABlocks, false, true>(c, c.k0, g_okbits[0], s, o, st, c2, w.row_ok, mseg,
                                          moff);
      const float negm = neg_max(st);
#pragma unroll
      for (int part = 0; part < 8; ++part) p_part(part, s, c2, negm, st.lsum, pf);
      ws_put(xb, c.lane, pf, st.m);
    }
    __syncthreads();
    for (int t = 0; t + 1 < w.ntiles; ++t) {
      const int b = t & 1;
      if (w.active) {
        ws_score_step<kMain>(w.lo, b ? raw0 : raw1, b ? v1 : v0, qf, o, pf, s);
        score_max<kArgmax, kABlocks, false, true>(c, c.k0 + (t + 1) * kTK, g_okbits[b ^ 1], s,
                                                  o, st, c2, w.row_ok, mseg, moff);
        const float negm = neg_max(st);
#pragma unroll
        for (int part = 0; part < 8; ++part) p_part(part, s, c2, negm, st.lsum, pf);
        ws_put(xb + (b ^ 1) * kXPar, c.lane, pf, st.m);
      }
      __syncthreads();
    }
    if (w.active) ws_score_step<kLast>(w.lo, raw0, ((w.ntiles - 1) & 1) ? v1 : v0, qf, o, pf, s);
  }
  __syncthreads();  // every P has been taken: the exchange area is free

  const float ltot = st.lsum + other_half(st.lsum);
  float ma = 0.f;  // this wavefront's part of the shared scale group
  if constexpr (kSplit) ma = lane_absmax<kABlocks - 4 * kSplitG>(o + 4 * kSplitG);
  if (w.active) {
    ws_ex(c.wave, 0)[c.lane] = ltot;
    ws_ex(c.wave, 1)[c.lane] = ma;
  }
  __syncthreads();
  if (!w.active || !w.row_ok) return;
  const int64_t prow = it.prow + int64_t(it.k) * rows_req + w.rho;
  if (prow >= ws.part_rows) {  // cannot happen: the workspace is sized for every plan
    atomicOr(ws.status, 2u);   // VA_DEV_SEGMENT
    return;
  }
  if (it.k == 0 && c.half == 0) {
    RowInfo ri;
    ri.base = it.prow + w.rho;
    ri.n = it.n;
    ri.stride = rows_req;
    ws.row_info[w.grow] = ri;
  }
  int16_t *pq = static_cast<int16_t *>(ws.part_o) + prow * kLatent;
  const float sl = ltot > 0.f ? 1.f / (32767.f * ltot) : 0.f;
  float *ps = ws.part_scale + kScaleGroups * prow;
#pragma unroll
  for (int g = 0; g < kSplitG; ++g) {
    float m = lane_absmax<4>(o + 4 * g);
    m = fmaxf(m, other_half(m));
    ws_codes<4>(pq, 4 * g, c.half, o + 4 * g, m > 0.f ? __builtin_amdgcn_rcpf(m) : 0.f);
    if (c.half == 0) ps[g] = m * sl;
  }
  if constexpr (kSplit) {
    float m = fmaxf(ma, ws_ex(c.wave, 2)[c.lane]);
    m = fmaxf(m, other_half(m));
    ws_codes<kABlocks - 4 * kSplitG>(pq, 4 * kSplitG, c.half, o + 4 * kSplitG,
                                     m > 0.f ? __builtin_amdgcn_rcpf(m) : 0.f);
    if (c.half == 0) ps[kSplitG] = m * sl;
  }
  if (c.half == 0) {
    const bool any = ltot > 0.f;
    ws.part_lse[prow] = any ? (st.m + log2f(ltot)) * kLn2 : -INFINITY;
    ws.part_max[prow] = any ? st.mx * kLn2 : -INFINITY;
    ws.part_arg[prow] = any && kArgmax ? st.best_j : -1;
  }
}

__device__ __forceinline__ void ws_value(const Workspace &ws, const Item &it, const WsItem &w) {
  const Ctx &c = w.c;
  const int rows_req = it.rows;
  char *const raw0 = g_ldsw;
  char *const raw1 = g_ldsw + kRawTile;
  char *const v0 = g_ldsw + kVOff;
  char *const v1 = g_ldsw + kVOff + kVTile;
  const char *const xb = g_ldsw + kWsXOff + c.wave * kXPair;
  constexpr int kXPar = kWaves * kXPair;

  int64_t slot_vec = -1;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing of the plan is still in flight
  if (w.ntiles > 0) {
    load_slots_lds(c, 0);
    load_slots_lds(c, 1);
    wait_tile_loads();
    const TileLoads t0 = plan_tile(c, 0, read_slots(c, 0));
    const TileLoads t1 = plan_tile(c, 1, read_slots(c, 1));
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) issue_latent(c, t0, lds_addr(raw0), i);
    issue_rope(c, t0, lds_addr(raw0));
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) issue_latent(c, t1, lds_addr(raw1), i);
    issue_rope(c, t1, lds_addr(raw1));
    publish_ok(c, 0, t0.ok);
    publish_ok(c, 1, t1.ok);
    slot_vec = fetch_slot(c, 2);
  }

  f32x16 o[kBBlocks];
#pragma unroll
  for (int d = 0; d < kBBlocks; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  float mb = -INFINITY;
  TileLoads none;
  none.addr = 0;
  none.ok = 0;
  if (w.ntiles > 0) {
    wait_loads_but_10();  // tile 0 (tile 1 and the slot fetch of tile 2 may be in flight)
    __syncthreads();
    ws_convert(w.lo, raw0, v0);
    wait_tile_loads();
    __syncthreads();
    for (int t = 0; t + 1 < w.ntiles; ++t) {
      const int b = t & 1;
      const TileLoads tl = plan_tile(c, t + 2, slot_vec);
      StepIO sio;
      sio.kraw = b ? raw0 : raw1;
      sio.vrd = b ? v1 : v0;
      sio.vwr = b ? v0 : v1;
      sio.dma_raw = lds_addr(b ? raw1 : raw0);
      publish_ok(c, b, tl.ok);
      // (a wavefront whose rows lie past the request runs the same code on a P nobody wrote
      // and never stores the result: one code path, so that the compiler's wait counting
      // sees the slot fetch's completion wait rather than a join it must treat as pending)
      ws_value_step<kMain>(c, w.lo, sio, tl, slot_vec, t + 3, o, xb + b * kXPar, mb);
      wait_tile_loads();
      __syncthreads();
    }
    {
      const int b = (w.ntiles - 1) & 1;
      StepIO eio;
      eio.kraw = raw0;
      eio.vrd = b ? v1 : v0;
      eio.vwr = v0;
      eio.dma_raw = 0;
      ws_value_step<kLast>(c, w.lo, eio, none, slot_vec, 0, o, xb + b * kXPar, mb);
    }
  }
  __syncthreads();  // every P has been taken: the exchange area is free

  // this wavefront's part of the scale group it may share with the score wavefront
  constexpr int kOwn0 = kSplit ? 4 * (kSplitG + 1) - kABlocks : 0;  // its blocks in that group
  float mb0 = 0.f;
  if constexpr (kSplit) mb0 = lane_absmax<kOwn0>(o);
  if (w.active) ws_ex(c.wave, 2)[c.lane] = mb0;
  __syncthreads();
  if (!w.active || !w.row_ok) return;
  const int64_t prow = it.prow + int64_t(it.k) * rows_req + w.rho;
  if (prow >= ws.part_rows) return;  // reported by the score wavefront
  const float ltot = ws_ex(c.wave, 0)[c.lane];
  const float sl = ltot > 0.f ? 1.f / (32767.f * ltot) : 0.f;
  int16_t *pq = static_cast<int16_t *>(ws.part_o) + prow * kLatent;
  float *ps = ws.part_scale + kScaleGroups * prow;
  if constexpr (kSplit) {
    float m = fmaxf(ws_ex(c.wave, 1)[c.lane], mb0);
    m = fmaxf(m, other_half(m));
    ws_codes<kOwn0>(pq, kABlocks, c.half, o, m > 0.f ? __builtin_amdgcn_rcpf(m) : 0.f);
    if (c.half == 0) ps[kSplitG] = m * sl;
  }
#pragma unroll
  for (int g = kSplitG + (kSplit ? 1 : 0); g < kScaleGroups; ++g) {
    const f32x16 *og = o + 4 * g - kABlocks;
    float m = lane_absmax<4>(og);
    m = fmaxf(m, other_half(m));
    ws_codes<4>(pq, 4 * g, c.half, og, m > 0.f ? __builtin_amdgcn_rcpf(m) : 0.f);
    if (c.half == 0) ps[g] = m * sl;
  }
}

template <bool kArgmax>
__device__ __forceinline__ void run_item_ws(const RunArgs &a, const Workspace &ws,
                                            const Item &it) {
  const Segment &seg = it.seg;
  const int H = a.H;
  const int rows_req = it.rows;
  const int row0 = it.rt * kRows;
  const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);

  WsItem w;
  Ctx &c = w.c;
  c.kv = static_cast<const uint16_t *>(a.kv);
  c.kvi = a.kv_indices + seg.kv0;
  c.tree = seg.tree;
  c.zero = ws.zero_row;
  c.num_slots = a.num_slots;
  c.status = ws.status;
  c.P = seg.P;
  c.wave = wv & (kWaves - 1);
  c.lane = int(threadIdx.x) & 63;
  c.half = c.lane >> 5;
  c.col = c.lane & 31;
  w.rho = row0 + c.wave * 32 + c.col;
  w.row_ok = w.rho < rows_req;
  w.active = row0 + c.wave * 32 < rows_req;
  const int rho_c = w.row_ok ? w.rho : rows_req - 1;
  w.tok = rho_c / H;
  w.grow = (seg.q0 + w.tok) * int64_t(H) + rho_c % H;
  split_range(seg.L, it.k, it.n, c.k0, c.k1);
  w.ntiles = (c.k1 - c.k0 + kTK - 1) / kTK;
  w.lo = lane_offsets(c);
  if (wv < kWaves)
    ws_score<kArgmax>(a, ws, it, w);
  else
    ws_value(ws, it, w);
}

template <bool kArgmax>
__global__ void __launch_bounds__(kWsThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_partial_ws_kernel(RunArgs a, Workspace ws, int G) {
  const int nb = gridDim.x;
  const int lane = int(threadIdx.x) & 63;
  const int64_t w = (int(blockIdx.x) & 7) * (nb >> 3) + (int(blockIdx.x) >> 3);
  Item it;
  {
    const ReqWork mine = req_work(a, lane);
    const WorkPlan plan = plan_work(a, mine, G, ws.splits, ws.status,
                                    blockIdx.x == 0 && threadIdx.x < 64, lane);
    if (w >= plan.items || !find_item<true>(a, mine, plan, w, lane, it)) return;
  }
  // (an item of 32 rows or fewer cannot occur: the launch takes this kernel only for H a
  // multiple of 64)
  if (it.rows - it.rt * kRows <= 32) {
    if (threadIdx.x == 0) atomicOr(ws.status, 2u);  // VA_DEV_SEGMENT
    return;
  }
  run_item_ws<kArgmax>(a, ws, it);
}

template <bool kArgmax>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_partial_kernel(RunArgs a, Workspace ws, int G) {
  // XCD-aware mapping: the launch deals workgroups to the 8 XCDs in turn, so workgroup b
  // takes item (b % 8) * (nb / 8) + b / 8: consecutive items share an XCD's L2
  const int nb = gridDim.x;  // a multiple of 8, at least G and the batch's row tiles
  const int lane = int(threadIdx.x) & 63;
  const int64_t w = (int(blockIdx.x) & 7) * (nb >> 3) + (int(blockIdx.x) >> 3);
  Item it;
  {
    const ReqWork mine = req_work(a, lane);
    const WorkPlan plan = plan_work(a, mine, G, ws.splits, ws.status,
                                    blockIdx.x == 0 && threadIdx.x < 64, lane);
    if (w >= plan.items || !find_item<true>(a, mine, plan, w, lane, it)) return;
  }
  if (it.rows - it.rt * kRows <= 32)
    run_narrow<kArgmax>(a, ws, it);
  else
    run_item<kArgmax>(a, ws, it);
}
}  // namespace

hipError_t launch_mfma_partial(const RunArgs &a, const Workspace &ws, int rows_per_block,
                               int work_items, hipStream_t st) {
  if (rows_per_block != kRows || work_items <= 0) return hipErrorInvalidValue;
  if (a.bs <= 0) return hipSuccess;
  // one workgroup per item: with a fixed split count S there are at most S items per row
  // tile; otherwise the plan makes at most work_items items, or one per row tile when the
  // batch has more row tiles than that
  const int64_t tiles = (int64_t(a.max_q_per_req) * a.H + kRows - 1) / kRows;
  const int64_t per_tile = ws.splits > 0 ? ws.splits : 1;
  int64_t nb = std::max(int64_t(work_items), int64_t(a.bs) * tiles * per_tile);
  nb = (nb + 7) / 8 * 8;
  if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (mfma_partial_waves(a.H) == 8) {  // no item of 32 rows or fewer: two per SIMD
    if (a.want_argmax)
      hipLaunchKernelGGL(mfma_partial_ws_kernel<true>, dim3(unsigned(nb)), dim3(kWsThreads), 0,
                         st, a, ws, work_items);
    else
      hipLaunchKernelGGL(mfma_partial_ws_kernel<false>, dim3(unsigned(nb)), dim3(kWsThreads), 0,
                         st, a, ws, work_items);
  } else if (a.want_argmax) {
    hipLaunchKernelGGL(mfma_partial_kernel<true>, dim3(unsigned(nb)), dim3(kThreads), 0, st, a,
                       ws, work_items);
  } else {
    hipLaunchKernelGGL(mfma_partial_kernel<false>, dim3(unsigned(nb)), dim3(kThreads), 0, st, a,
                       ws, work_items);
  }
  return hipGetLastError();
}

}  // namespace va
