// Fine-grained-scaled FP8 GEMM kernels for gfx950 (CDNA4).
//
// Method (DeepGEMM project introduction, section Interfaces; "Deepseek
// DeepGEMM technical principles", section "Technical background and core
// principles"): for every 128-wide K slice, form the FP8 partial product on
// the matrix cores, scale it by sa*sb (1x128 activation scale times 128x128
// weight scale) and add it into an fp32 accumulator ("promotion" every
// N_C = 128).  Output bf16.
//
// gfx950 mapping
// * One v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-deep scale slice of
//   a 16x16 output fragment, so a partial product never mixes two slices:
//   P = mfma(b, a, 0) (the B fragment as the first operand), then
//   acc += P * (sa * sb) on the VALU, per lane for its 1 row x 4 columns, so
//   one activation scale serves the lane's four results.
// * Fragment layouts (64-wide wavefronts).  Operand: lane l holds 32 bytes of
//   K for row (l % 16), lane group l / 16 selects which 32 bytes; A and B use
//   the same K assignment, so the contraction is the full 128-term dot product
//   whatever order the matrix core visits the bytes in.  Result of
//   mfma(b, a): lane l holds output row (l % 16) of the A fragment, columns
//   4 * (l / 16) + i, i = 0..3.  The K-grouped GEMM, whose B scales are per
//   column, keeps mfma(a, b): lane l holds column (l % 16), rows
//   4 * (l / 16) + i.
// * Operands are staged HBM -> LDS with global_load_lds_dwordx4 (no register
//   staging), STAGES deep, one barrier per K slice.  A stage holds the A tile
//   [BM][128], the B tile [BN][128] and the BM activation scales of the slice.
//   K-major tiles keep each row's 128-byte slice whole (one LDS-DMA lane
//   octet per row) but place rows and chunks (kmaj_offset) so that every
//   fragment read is an access order gfx950's LDS serves at its full 256
//   bytes per clock.
// * Persistent workgroups (grid sized to the CU count; two per CU for the
//   64x64 tiles) walk the work units; units that run at the same time on one
//   XCD (workgroup id mod 8) are given neighbouring tiles so they share A and
//   B lines in that XCD's L2.
// * Stream-K for shapes with fewer tiles than CUs: a tile's K range is cut
//   into S parts (decode tiles) or all (tile, slice) iterations are divided
//   into equal runs (large tiles).  A run that covers part of a tile writes
//   an fp32 partial; the last one to arrive (arrival counter) sums the
//   partials in K order - a fixed order, so results are bit-identical run to
//   run - and stores bf16.  No workgroup ever waits for another.  The pages
//   fill idle SMs with unaligned block widths (project introduction,
//   Optimisations); dividing K does that here.
// * Layouts: dense, grouped-contiguous (an expert id per row), grouped-masked
//   (valid rows per expert, read on the device) and K-grouped (an expert's
//   tokens are a K range; per-row scales on both operands).
// * Operand majors (dense layout, fp32 or UE8M0 scales): A may also be stored M-major
//   ([K][lda]) and B N-major ([K][ldb]), the TN / NN / TT forms of D = A B^T
//   beside NT.  Such a tile is staged as [128][BM] (K rows of BM bytes) and
//   its fragments are read with ds_read_b64_tr_b8, gfx950's transposing LDS
//   load, which hands each lane the 8 K values of its own row.
// * Scale formats: fp32 (promotion on the VALU), power-of-two UE8M0 (applied
//   inside v_mfma_scale_f32_16x16x128_f8f6f4, no VALU promotion) and fp32 row
//   scales on B (K-grouped).  The epilogue can also quantise the bf16 output
//   per 1x128 tile for the next layer.

#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

namespace {

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16-byte asynchronous copy global -> LDS.  The LDS destination of lane l is
// m0 + 16 * l, so one instruction fills 1 KB of LDS.  Written as inline asm so
// that the compiler does not add a conservative vmcnt(0) before every LDS read
// (it cannot tell which stage a DMA targets); the pipeline waits explicitly.
__device__ __forceinline__ void dma16(uint32_t lds, const void* base, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}

// 4-byte variant: lane l's dword lands at m0 + 4 * l (256 bytes per instruction).
__device__ __forceinline__ void dma4(uint32_t lds, const void* base, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}

// Wait until at most N of this wave's vector memory operations are in flight,
// then barrier.  The "memory" clobber keeps the compiler from moving LDS or
// global accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ void barrier_all() { asm volatile("s_barrier" : : : "memory"); }

// Wait until at most NEWER stages of this wave's DMAs are in flight (the
// stages issued after the one the loop needs next).  Waves issue different
// numbers of DMAs per stage (DmaPlan P::dmas_of_wave), so the count is
// picked per run of waves with equal counts.
template <class P, int NEWER, int W = 0>
__device__ __forceinline__ void wait_stage(int wave) {
  if constexpr (W + 1 >= P::kWaves) {
    wait_vm<NEWER * P::dmas_of_wave(W)>();
  } else if constexpr (P::dmas_of_wave(W + 1) == P::dmas_of_wave(W)) {
    wait_stage<P, NEWER, W + 1>(wave);
  } else {
    if (wave <= W) wait_vm<NEWER * P::dmas_of_wave(W)>();
    else wait_stage<P, NEWER, W + 1>(wave);
  }
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// K-major operand tiles in LDS.  Tile rows come in groups of 16 (2 KB), one
// 1 KB block for the even rows and one for the odd rows of a group; row
// 16 g + t sits in block 2 g + (t % 2) at 128-byte position
// q(t) = 2 ((t / 2) % 4) + t / 8, with its 16-byte chunk c (K bytes
// 16 c .. 16 c + 15 of the slice) at 16 (c ^ (t % 8)).  One LDS-DMA
// instruction fills one block, 8 whole 128-byte row slices.  A fragment read
// (lane l: row t = l % 16, chunk 2 (l / 16) + h) then gives 16-lane set s the
// 16-byte bank groups (l % 16) ^ (2 s + h): within each set, the linear
// order under an XOR of the low three bits.  gfx950's LDS serves
// ds_read_b128 at 256 bytes per clock (64 banks of 4 bytes) only for such
// orders; other conflict-free orders go at 128 bytes per clock (measured:
// 4.4 against 8.0 clocks per 1 KB read per CU).
__device__ __forceinline__ uint32_t kmaj_offset(int row, int chunk) {
  const int t = row & 15;
  return (uint32_t)((row >> 4) * 2048 + (t & 1) * 1024 + (2 * ((t >> 1) & 3) + (t >> 3)) * 128 +
                    ((chunk ^ t) & 7) * 16);
}

// The tile row whose slice lane l of the LDS-DMA instruction filling block b
// loads (the 8 lanes 8 j .. 8 j + 7 take the 8 chunks of one row; lane l
// takes chunk (l % 8) ^ (row % 8), landing at 16 (l % 8) of the row's
// 128-byte position l / 8).
__device__ __forceinline__ int kmaj_dma_row(int b, int lane) {
  const int q = lane >> 3;
  return (b >> 1) * 16 + 8 * (q & 1) + 2 * (q >> 1) + (b & 1);
}

// Pointers that are the same for the whole wave, kept in SGPRs (the DMA takes
// its base address from an SGPR pair).
template <class P>
__device__ __forceinline__ P* uniform_ptr(P* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ v8i make_v8i(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// MN-major operand tiles.  A K slice of an M-major A (or N-major B) tile is
// held in LDS as 128 K rows of L = BM (BN) bytes; the 16-byte chunk c of K
// row k sits at position c ^ mn_swizzle<L>(k), so that the 8 K rows read
// together by one transposing load (same chunk, 8 consecutive rows) fall in
// 8 distinct 16-byte bank groups.
template <int L>
__device__ __forceinline__ int mn_swizzle(int k) {
  static_assert(L % 128 == 0 || L == 64, "MN-major tiles are 64 or a multiple of 128 bytes wide");
  return L >= 128 ? (k & 7) : ((k >> 1) & 3);
}

typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

// The MFMA operand of the 16 rows (MN indices) col .. col + 15 of an MN-major
// tile: lane l gets row col + l % 16, K bytes 32 (l / 16) .. + 31, the same
// layout as a K-major fragment.  ds_read_b64_tr_b8 works on groups of 16
// lanes: lane r of the group names an 8-byte row R_r, and lane i receives
// the bytes R_{2j + i/8}[i % 8], j = 0..7 (measured on gfx950).  So lane r
// points at K row kbase + r / 2, MN bytes col + 8 (r % 2) .. + 7, and lane i
// then holds MN index col + i at K rows kbase .. kbase + 7.  Four loads
// (kbase = 32 (l / 16) + 8 t, immediate offsets 8 t L) give the 32 bytes.
//
// For every K row this lane names, k = 32 kg + 8 t + fr / 2, so its swizzle
// term x = mn_swizzle(fr / 2) is fixed per lane and sits in address bits
// 4..6 of `lane_off` (the tile base is 1 KB aligned and K rows are a
// multiple of 128 bytes, or 64 bytes with a 2-bit term).  The chunk's low
// bits then enter by XOR, col's higher bits by addition, so a fragment
// costs one add and one xor and no per-fragment register stays live.
template <int L>
__device__ __forceinline__ uint32_t mn_lane_off(int fr, int kg) {
  return (uint32_t)((32 * kg + (fr >> 1)) * L + 16 * mn_swizzle<L>(fr >> 1) + 8 * (fr & 1));
}

template <int L>
__device__ __forceinline__ v8i ld_mn_frag(uint32_t tile_lds, uint32_t lane_off, int col) {
  constexpr int kLow = L >= 128 ? 7 : 3;  // chunk bits taken by the swizzle
  const int c = col >> 4;
  const uint32_t addr = (tile_lds + lane_off + 16u * (uint32_t)(c & ~kLow)) ^ (16u * (uint32_t)(c & kLow));
  lds_v2i* p = (lds_v2i*)(uintptr_t)addr;
  v8i r;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(p + t * L);  // + 8 t L bytes
    r[2 * t] = v.x;
    r[2 * t + 1] = v.y;
  }
  return r;
}

// Compile-time loop: f(std::integral_constant<int, 0>) ... f(<N-1>).
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl<0, N>(f); }

__device__ __forceinline__ v4f mfma_fp8_slice(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // Format codes 0/0 = e4m3 for both operands; no block scale (the scales here
  // are arbitrary fp32 values, applied on the VALU).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// SB_BYTES: LDS bytes a stage keeps for the slice's weight scales: 1 KB (one
// 16-byte DMA per lane: the K-grouped layout's per-column scales of B), or
// 256 bytes (one 4-byte DMA per lane: up to 64 weight-scale blocks), which
// lets a third stage of the 256 x 160 tile fit in the 160 KB of LDS.
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int SB_BYTES = 1024>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 fragments per wave
  // DMA instruction i of a stage fills LDS bytes [1024 i, 1024 i + 1024)
  // (how the instructions are split over the waves: DmaPlan below).
  static constexpr int kAInstr = BM / 8;            // 1 KB DMA instructions per slice
  static constexpr int kBInstr = BN / 8;
  // Fragment rows over which a stage's DMA pieces are spread (0: all of
  // them right after the barrier, before any compute).  Spreading pays with
  // two waves per SIMD, where the other wave keeps the SIMD busy while one
  // waits on the address unit; with one wave per SIMD (4-wave tiles) issuing
  // early measured faster.  The 256x256 tile sits at the 256-register limit
  // of two waves per SIMD; keeping DMA addresses live across its rows would
  // spill, so it issues everything after the first row's MFMAs.
  static constexpr int kSpreadRows = kWaves < 8 ? 0 : ((BM * BN >= 256 * 256) ? 1 : FM);
  static constexpr int kSOffInstr = kAInstr + kBInstr;
  static constexpr int kSBOff = (kAInstr + kBInstr + 1) * 1024;  // weight scales of the slice
  static constexpr int kSBBytes = SB_BYTES;
  static constexpr int kStageBytes = (kAInstr + kBInstr + 1) * 1024 + SB_BYTES;
  static constexpr int kBOff = BM * 128;
  static constexpr int kSOff = (BM + BN) * 128;
  static constexpr bool kOneSB = (128 % TN) == 0;   // wave columns inside one 128-block
  // Overlap the MFMAs of fragment row i+1 with the FMAs of row i (needs a
  // second set of result registers; with two waves per SIMD the other wave
  // provides the overlap instead).
  static constexpr bool kPipe = kWaves <= 4;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "bad tile");
  static_assert(SB_BYTES == 1024 || SB_BYTES == 256, "weight-scale slot of 1 KB or 256 bytes");
  static_assert(BM <= 256, "one scale instruction covers 256 rows");
  static_assert(STAGES >= 2, "need two stages");
  static_assert(kWaves >= 2, "waves 0 and 1 load the scales");
  static_assert(STAGES * kStageBytes + 16 <= 160 * 1024, "LDS overflow");
};

// How a stage's A/B DMA instructions are split over a tile's waves: the first
// DW waves issue them, wave w the instructions j * DW + w for j < kAJ while
// that index is below kAInstr (the last round may be partial when the rows
// do not split evenly), then the B instructions the same way; so every
// wave's j-th instruction falls in the same region (A rows, B rows) - a
// compile-time choice.  Waves 0 and 1 also issue the activation- and
// weight-scale DMA.  DW = kWaves spreads the work over every wave; the
// fp32-scale 8-wave 256-row tiles use DW = 4, one issuing wave per SIMD, so
// each SIMD keeps a wave that never waits on the vector-memory address unit
// while a stage goes out (the plan `DP` chosen in gemm_kernel).
template <class T, int DW>
struct DmaPlan {
  static_assert(DW >= 2 && DW <= T::kWaves, "waves 0 and 1 issue the scale DMAs");
  static constexpr int kWaves = T::kWaves;
  static constexpr int kDW = DW;
  static constexpr int kAJ = (T::kAInstr + DW - 1) / DW;
  static constexpr int kBJ = (T::kBInstr + DW - 1) / DW;
  static constexpr int kLPW = kAJ + kBJ;  // A/B DMA rounds per issuing wave per stage
  static constexpr int kIssue = kLPW + 1;  // DMA pieces per wave per stage (the last: scales)
  // DMA instructions wave w issues per stage.
  static constexpr int dmas_of_wave(int w) {
    return (w < DW ? (T::kAInstr / DW + (w < T::kAInstr % DW ? 1 : 0)) + (T::kBInstr / DW + (w < T::kBInstr % DW ? 1 : 0))
                   : 0) +
           (w < 2 ? 1 : 0);
  }
};

// Decode a linear work-unit index into a tile.  XCD-aware: workgroup w runs on
// XCD w % 8, so within a round the units of one XCD (w = x, x+8, ...) are
// remapped onto consecutive tile indices; tiles are then rastered in groups of
// `group_m` M-tiles so that consecutive indices share rows of A and walk N.
__device__ __forceinline__ int xcd_remap(int u, int grid, int units) {
  const int round_base = (u / grid) * grid;
  if (round_base + grid > units || (grid & 7)) return u;  // last partial round: identity
  const int w = u - round_base;
  return round_base + (w & 7) * (grid >> 3) + (w >> 3);
}

__device__ __forceinline__ void raster(int t, int m_tiles, int n_tiles, int group_m, int& mt,
                                       int& nt) {
  const int per_group = group_m * n_tiles;
  const int grp = t / per_group;
  const int first = grp * group_m;
  const int gsize = min(group_m, m_tiles - first);
  const int r = t - grp * per_group;
  mt = first + r % gsize;
  nt = r / gsize;
}

__device__ __forceinline__ int clamp_rows(int v, int hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

// Scale formats.  UE8M0 exponents are bytes; the scale pointers keep the
// fp32 type and group strides count elements of the format in use.
// kScaleRowB (K-grouped layout): fp32 activation-style 1x128 scales on both
// operands, the B scales per row of B: [K/128][ld_sfb].
constexpr int kScaleF32 = 0, kScaleUE8M0 = 1, kScaleRowB = 2;
template <int SF>
__device__ __forceinline__ const float* scale_ptr(const float* base, int64_t offset) {
  if constexpr (SF == kScaleUE8M0)
    return reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(base) + offset);
  return base + offset;
}

// SF: kScaleF32 (fp32 scales, promoted on the VALU) or kScaleUE8M0 (power-of-
// two exponents applied inside the block-scaled MFMA, see below).
// MAJ: operand majors, bit 0 = A stored M-major [K][lda], bit 1 = B stored
// N-major [K][ldb] (dense layout).
constexpr int kAMajorMN = 1, kBMajorMN = 2;
template <class T, int LAYOUT, bool SK, int SF, int MAJ = 0>
__global__ __launch_bounds__(T::kThreads) void gemm_kernel(GemmParams p, Schedule s) {
  static_assert(MAJ == 0 || (LAYOUT == kDense && SF != kScaleRowB), "MN-major operands: dense layout");
  constexpr bool kAT = (MAJ & kAMajorMN) != 0, kBT = (MAJ & kBMajorMN) != 0;
  // Transposed fragments: the MFMA takes the B fragment as its first operand,
  // so a lane's four results are one output row (row fr of the A fragment)
  // and four consecutive columns 4 kg .. 4 kg + 3.  The row's activation
  // scale is then one value per lane and fragment row, and the four bf16
  // results are 8 contiguous bytes.  Per-column B scales (the K-grouped
  // GEMM) keep the untransposed form, where a lane holds one column.
  constexpr bool kTr = SF != kScaleRowB;
  // One 16x16x128 product of fragments a (16 rows of A) and b (16 rows of B).
  auto slice_mma = [](const v8i& a, const v8i& b) { return kTr ? mfma_fp8_slice(b, a) : mfma_fp8_slice(a, b); };
  // The same with power-of-two scales inside the MFMA: ea for a's rows, eb
  // for b's rows (one exponent byte per lane, for its row l mod 16).
  auto scaled_mma = [](const v8i& a, int ea, const v8i& b, int eb, const v4f& c) {
    return kTr ? __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, 0, eb, 0, ea)
               : __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
  };
  // The split of each stage's DMAs over the waves.  With fp32 scales the
  // 8-wave 256-row tiles (256 x 256 and 256 x 160) let only waves 0-3 (one
  // per SIMD) issue them: the SIMD's other wave keeps the matrix core fed
  // while a stage goes out through the address unit (back to back: masked
  // 4x1024x4096x7168 114-116 -> 110-112 us, 4096x32768x512 151 -> 145-146
  // us, contiguous 973 -> 964-970 us, 4096x2112x7168 on 256 x 160 tiles
  // 95-97 -> 90.5-92 us).  The UE8M0 loop spills with that split and keeps
  // all eight; on the 8-wave 128 x 128 decode tile it measured mixed
  // (128x32768x512 11.0 -> 12.1 us, 128x7168x16384 37.2 -> 36.7 us).
  using DP = DmaPlan<T, (SF == kScaleF32 && T::kWaves == 8 && T::BM == 256) ? 4 : T::kWaves>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::STAGES * T::kStageBytes];
  __shared__ int last_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int fr = lane & 15;  // fragment row (A) / column (B) of this lane
  const int kg = lane >> 4;  // which 32 bytes of the slice
  // This lane's two 16-byte reads of a K-major fragment whose 16 rows start
  // at a multiple of 16: chunks 2 kg and 2 kg + 1 of row fr (kmaj_offset).
  const uint32_t kf0 = kmaj_offset(fr, 2 * kg), kf1 = kmaj_offset(fr, 2 * kg + 1);
  // MFMA operands of a stage at sp: A fragment row i, B fragment column j,
  // from K-major tiles (two 16-byte reads) or MN-major ones (transposing loads).
  auto frag_a = [&](const uint8_t* sp, int i) -> v8i {
    if constexpr (kAT) {
      return ld_mn_frag<T::BM>(lds_addr(sp), mn_lane_off<T::BM>(fr, kg), wm * T::TM + i * 16);
    } else {
      const uint8_t* gp = sp + (wm * T::TM + i * 16) * 128;  // the fragment's 16-row group
      return make_v8i(*reinterpret_cast<const uint4*>(gp + kf0), *reinterpret_cast<const uint4*>(gp + kf1));
    }
  };
  auto frag_b = [&](const uint8_t* sp, int j) -> v8i {
    if constexpr (kBT) {
      return ld_mn_frag<T::BN>(lds_addr(sp) + T::kBOff, mn_lane_off<T::BN>(fr, kg), wn * T::TN + j * 16);
    } else {
      const uint8_t* gp = sp + T::kBOff + (wn * T::TN + j * 16) * 128;
      return make_v8i(*reinterpret_cast<const uint4*>(gp + kf0), *reinterpret_cast<const uint4*>(gp + kf1));
    }
  };
  const int nkb_total = p.k / kBlockK;
  const int n_blocks = (p.n + kBlockK - 1) / kBlockK;
  const uint32_t smem_base = lds_addr(smem);

  // Work units.  Masked: the number of valid M tiles is read on the device.
  int m_tiles = s.m_tiles;
  if (LAYOUT == kMasked) {
    m_tiles = 0;
    for (int g = 0; g < p.num_groups; ++g)
      m_tiles += (clamp_rows(p.masked_m[g], p.m) + T::BM - 1) / T::BM;
  }
  // K-grouped: every group has the same M x N tiles.
  const int tiles = (LAYOUT == kKGrouped ? p.num_groups : 1) * m_tiles * s.n_tiles;
  const int G = gridDim.x;
  // Stream-K.  The tiles of the whole waves of G run one per workgroup
  // (data-parallel); the (tile, K slice) iterations of the remaining tiles
  // are divided into runs, each a contiguous range of iterations:
  //   sk_split == 0: sk_groups = min(G, iterations) runs of equal length,
  //     which may cross tile boundaries (long K ranges, few tiles);
  //   sk_split == S: S runs per tile, each 1/S of its K range (one
  //     segment per run; runs beyond G go round again).
  // A run that covers only part of a tile's K range leaves an fp32 partial;
  // the last workgroup of that tile to finish sums the partials in K order.
  const int sk_split = min(s.sk_split, nkb_total);  // no empty runs
  int dp_tiles = tiles, sk_iters = 0, sk_groups = 1;
  if (SK) {
    dp_tiles = sk_split > 0 ? 0 : (tiles / G) * G;
    sk_iters = (tiles - dp_tiles) * nkb_total;
    sk_groups = sk_split > 0 ? (tiles - dp_tiles) * sk_split : max(1, min(G, sk_iters));
  }
  auto sk_start = [&](int w) {
    if (sk_split > 0) {
      const int tt = w / sk_split;
      return tt * nkb_total + ((w - tt * sk_split) * nkb_total) / sk_split;
    }
    return (int)(((int64_t)sk_iters * w) / sk_groups);
  };
  auto sk_owner = [&](int x) {  // the run containing iteration x
    int w = (int)(((int64_t)x * sk_groups) / sk_iters);
    while (w + 1 < sk_groups && sk_start(w + 1) <= x) ++w;
    while (w > 0 && sk_start(w) > x) --w;
    return w;
  };
  // Runs are numbered so that the workgroups of one XCD (id mod 8) take
  // neighbouring runs, i.e. neighbouring tiles.
  const int vw = (SK && (G & 7) == 0) ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  int run = vw, sk_cur = 0, sk_end = 0, run_first = 0;
  if (SK && run < sk_groups) {
    sk_cur = run_first = sk_start(run);
    sk_end = sk_start(run + 1);
  }
  int dp_u = blockIdx.x;

  while (true) {
    // ------------------------------------------------------------ schedule
    int t, kb0, kb1;
    bool partial = false;  // this unit computes part of the tile's K range
    int slot = 0;          // 0: the run's first segment, 1: its last
    if (SK && sk_cur >= sk_end && sk_split > 0 && run + G < sk_groups) {
      run += G;  // aligned runs beyond the grid go round again
      sk_cur = run_first = sk_start(run);
      sk_end = sk_start(run + 1);
    }
    if (sk_cur < sk_end) {
      const int tr = sk_cur / nkb_total;
      kb0 = sk_cur - tr * nkb_total;
      kb1 = min(nkb_total, kb0 + (sk_end - sk_cur));
      slot = sk_cur == run_first ? 0 : 1;
      sk_cur += kb1 - kb0;
      t = dp_tiles + tr;
      partial = !(kb0 == 0 && kb1 == nkb_total);
    } else if (dp_u < dp_tiles) {
      t = xcd_remap(dp_u, G, dp_tiles);
      kb0 = 0;
      kb1 = nkb_total;
      dp_u += G;
    } else {
      break;
    }
    int g = 0;
    if (LAYOUT == kKGrouped) {
      // Group g owns the K range [k_offsets[g], k_offsets[g+1]) (128-aligned
      // by contract; clamped and rounded down here, so any value is safe).
      const int per_group = m_tiles * s.n_tiles;
      g = t / per_group;
      t -= g * per_group;
      const int k_lo = min(max(p.k_offsets[g], 0), p.k);
      const int k_hi = min(max(p.k_offsets[g + 1], 0), p.k);
      kb0 = __builtin_amdgcn_readfirstlane(k_lo >> 7);
      kb1 = __builtin_amdgcn_readfirstlane(max(k_lo >> 7, k_hi >> 7));
    }
    int mt, nt;
    raster(t, m_tiles, s.n_tiles, s.group_m, mt, nt);
    if (LAYOUT == kMasked) {
      int before = 0;
      for (g = 0; g < p.num_groups - 1; ++g) {
        const int gt = (clamp_rows(p.masked_m[g], p.m) + T::BM - 1) / T::BM;
        if (mt < before + gt) break;
        before += gt;
      }
      mt -= before;
    }
    const int m0 = mt * T::BM;
    const int n0 = nt * T::BN;

    int rows_valid = p.m;
    const uint8_t* A = p.a;
    const float* SA = p.sfa;
    uint16_t* D = p.d;
    uint8_t* DQ = p.dq;
    // Output scales: fp32, or UE8M0 exponent bytes (p.dq_ue8m0); addressed
    // in bytes so both formats share the strides counted in elements.
    const int dsf_esize = p.dq_ue8m0 ? 1 : 4;
    uint8_t* DSF = reinterpret_cast<uint8_t*>(p.dsf);
    if (LAYOUT == kKGrouped) D += (int64_t)g * p.d_gstride;
    if (LAYOUT == kMasked) {
      rows_valid = clamp_rows(p.masked_m[g], p.m);
      A += (int64_t)g * p.a_gstride;
      SA = scale_ptr<SF>(SA, (int64_t)g * p.sfa_gstride);
      D += (int64_t)g * p.d_gstride;
      if (DQ) {
        DQ += (int64_t)g * p.dq_gstride;
        DSF += (int64_t)g * p.dsf_gstride * dsf_esize;
      }
    }
    // Contiguous layout: the experts of the tile's 128-row halves.  A tile
    // whose halves belong to two experts is computed once per expert.
    int pass_group[2] = {0, -1};
    int passes = 1;
    if (LAYOUT == kContiguous) {
      int gh[2] = {-1, -1};
#pragma unroll
      for (int h = 0; h < (T::BM + 127) / 128; ++h) {
        int id = -1;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int row = m0 + h * 128 + lane * 2 + q;
          if (row < p.m && row < m0 + T::BM) {
            const int v = p.m_indices[row];
            if (v >= 0 && v < p.num_groups) id = max(id, v);
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) id = max(id, __shfl_xor(id, off, 64));
        gh[h] = __builtin_amdgcn_readfirstlane(id);
      }
      passes = 0;
      if (gh[0] >= 0) pass_group[passes++] = gh[0];
      if (gh[1] >= 0 && gh[1] != gh[0]) pass_group[passes++] = gh[1];
    }

    A = uniform_ptr(A);
    SA = uniform_ptr(SA);
    for (int pass = 0; pass < passes; ++pass) {
      if (LAYOUT == kContiguous) g = __builtin_amdgcn_readfirstlane(pass == 0 ? pass_group[0] : pass_group[1]);
      const uint8_t* B = uniform_ptr(p.b + (int64_t)g * p.b_gstride);
      const float* SB = uniform_ptr(scale_ptr<SF>(p.sfb, (int64_t)g * p.sfb_gstride));
      const int nkb = kb1 - kb0;
      // K walk order.  With k_rotate the tile visits its slices starting at
      // (tile mod slices) and wraps, so workgroups running at the same time
      // read different 128-byte columns of B.  When every tile starts at the
      // same slice, the concurrent requests differ only in their row bits,
      // and for power-of-two row pitches they crowd onto a few HBM channels
      // (measured: 3.7 TB/s streaming rows 16 KiB apart, 5.7 TB/s rotated).
      const int rot = (s.k_rotate && nkb > 1) ? t % nkb : 0;
      auto kb_at = [&](int it) {
        const int x = it + rot;
        return kb0 + (x >= nkb ? x - nkb : x);
      };

      const int cb_first = n0 >> 7;  // the tile's 128-column weight-scale blocks
      const int cb_count = min((n0 + T::BN - 1) >> 7, n_blocks - 1) - cb_first + 1;

      // Stage loader.  DMA instruction i of a stage fills LDS bytes
      // [1024 i, 1024 i + 1024): instructions [0, BM/8) carry A rows,
      // [BM/8, (BM+BN)/8) B rows, then the BM activation scales and the
      // weight scales.  An issuing wave's share of a stage is DP::kLPW A/B
      // instructions plus, for waves 0 and 1, one scale instruction: piece j
      // of DP::kIssue = kLPW + 1 (a compile-time index; the last piece is the
      // scale DMA, empty for waves 2 and up).
      auto issue_piece = [&](int kb, int buf, auto jc) {
        constexpr int j = decltype(jc)::value;
        const uint32_t stage_lds = smem_base + buf * T::kStageBytes;
        if constexpr (j < DP::kAJ) {
          if (DP::kDW < T::kWaves && wave >= DP::kDW) return;  // not an issuing wave
          const int instr = j * DP::kDW + wave;
          if (T::kAInstr % DP::kDW != 0 && instr >= T::kAInstr) return;  // partial last round
          const int q = instr * 64 + lane;
          if constexpr (kAT) {
            // K row kr of the slice, chunk position cp; the chunk holds rows
            // m .. m + 15 (M % 16 == 0, so a chunk is all valid or all past
            // the end, and those are clamped onto the last valid chunk).
            constexpr int C = T::BM / 16;
            const int kr = q / C, c = (q % C) ^ mn_swizzle<T::BM>(q / C);
            const int gm = min(m0 + 16 * c, p.m - 16);
            // The slice's K rows start at A + 128 kb lda (a uniform base), so
            // the per-lane offset stays the same from slice to slice.
            dma16(stage_lds + instr * 1024, A + (size_t)(kb * 128) * (size_t)p.lda,
                  (uint32_t)kr * (uint32_t)p.lda + (uint32_t)gm);
          } else {
            const int r = kmaj_dma_row(instr, lane), c = (lane & 7) ^ (r & 7);
            const int gr = min(m0 + r, rows_valid - 1);
            // The slice advances the uniform base; the per-lane offset is fixed.
            dma16(stage_lds + instr * 1024, A + kb * 128, (uint32_t)gr * (uint32_t)p.lda + c * 16);
          }
        } else if constexpr (j < DP::kLPW) {
          constexpr int jb = j - DP::kAJ;
          if (DP::kDW < T::kWaves && wave >= DP::kDW) return;  // not an issuing wave
          if (T::kBInstr % DP::kDW != 0 && jb * DP::kDW + wave >= T::kBInstr) return;  // partial last round
          const int instr = T::kAInstr + jb * DP::kDW + wave;
          const int q = (jb * DP::kDW + wave) * 64 + lane;
          if constexpr (kBT) {
            constexpr int C = T::BN / 16;
            const int kr = q / C, c = (q % C) ^ mn_swizzle<T::BN>(q / C);
            const int gn = min(n0 + 16 * c, p.n - 16);
            dma16(stage_lds + instr * 1024, B + (size_t)(kb * 128) * (size_t)p.ldb,
                  (uint32_t)kr * (uint32_t)p.ldb + (uint32_t)gn);
          } else {
            const int r = kmaj_dma_row(jb * DP::kDW + wave, lane), c = (lane & 7) ^ (r & 7);
            const int gn = min(n0 + r, p.n - 1);
            dma16(stage_lds + instr * 1024, B + kb * 128, (uint32_t)gn * (uint32_t)p.ldb + c * 16);
          }
        } else {
          if constexpr (SF == kScaleUE8M0) {
            // Exponent bytes, MN-major for both operands (four to a dword).
            if (wave == 0) {
              // rows m0 .. m0 + BM - 1 of the slice: lane l takes rows
              // m0 + 4l .. m0 + 4l + 3 (never clamped for a valid row).
              const int r4 = min(m0 + 4 * lane, (int)p.ld_sfa - 4);
              dma4(stage_lds + T::kSOffInstr * 1024, SA, (uint32_t)(kb * p.ld_sfa + r4));
            } else if (wave == 1) {
              // column blocks (cb_first & ~3) .. + 7 of the slice (lanes 0, 1).
              const int c4 = min((cb_first & ~3) + 4 * min(lane, 1), (int)p.ld_sfb - 4);
              dma4(stage_lds + T::kSBOff, SB, (uint32_t)(kb * p.ld_sfb + c4));
            }
          } else {
            if (wave == 0) {
              // Activation scales of the slice: rows m0 .. m0 + 4*63 + 3.
              const int r4 = min(m0 + 4 * lane, (int)p.ld_sfa - 4);
              dma16(stage_lds + T::kSOffInstr * 1024, SA, (uint32_t)(kb * p.ld_sfa + r4) * 4u);
            } else if (SF == kScaleRowB) {
              // Row scales of B: columns n0 .. n0 + 4*63 + 3 of the slice.
              if constexpr (SF == kScaleRowB) {
                static_assert(T::kSBBytes == 1024, "per-column B scales need a 1 KB slot");
                if (wave == 1) {
                  const int c4 = min(n0 + 4 * lane, (int)p.ld_sfb - 4);
                  dma16(stage_lds + T::kSBOff, SB, (uint32_t)(kb * p.ld_sfb + c4) * 4u);
                }
              }
            } else if (wave == 1) {
              // Weight scales of the slice for the tile's column blocks (lane l:
              // block cb_first + l; lanes past the last block repeat it).
              const int cb = cb_first + min(lane, cb_count - 1);
              dma4(stage_lds + T::kSBOff, SB, (uint32_t)(cb * nkb_total + kb) * 4u);
            }
          }
        }
      };
      auto issue_stage = [&](int kb, int buf) {
        static_for<DP::kIssue>([&](auto jc) { issue_piece(kb, buf, jc); });
      };
      // The pieces that go out after the MFMAs of fragment row i, spreading a
      // stage's DMAs over the compute of the previous one: the vector-memory
      // address unit takes one 1 KB instruction per 16 clocks, so a wave that
      // issued its whole share at once would sit idle behind the queue.
      auto issue_row = [&](int kb, int buf, auto ic) {
        constexpr int i = decltype(ic)::value;
        static_for<DP::kIssue>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          if constexpr (j * T::kSpreadRows / DP::kIssue == i) issue_piece(kb, buf, jc);
        });
      };

      lds_barrier();  // previous unit's readers are done with every LDS buffer

      v4f acc[T::FM][T::FN];
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

      // Two-stage tiles (the 256x256 one) with power-of-two scales place the
      // slice barrier before the last fragment row and prefetch the next
      // slice's operands across it (measured: 9% faster at 4096x4096x7168).
      // With fp32 scales the same loop spills inside the K loop: across the
      // last row the promotion's partial registers, the slice's A fragment
      // and the next slice's B fragments are live together.
      constexpr bool kLate = T::STAGES == 2 && SF == kScaleUE8M0;
      if constexpr (kLate) {
        static_assert(T::FM >= 2 && !T::kPipe, "the late barrier sits between two fragment rows");
        // Two LDS stages, with the barrier of slice `it` placed before its
        // last fragment row instead of at the start of the slice.  At that
        // point every wave has read all of slice it out of LDS (the last A
        // row is prefetched one row ahead; the B fragments and the weight
        // scales are in registers), so buffer it % 2 can take the DMA of
        // slice it + 2; and slice it + 1, whose DMAs every wave has waited
        // for just before, can be read.  Its B fragments, first A row and
        // scales then load during the last row's MFMAs, and the DMA pieces go
        // out between those MFMAs, so the matrix cores do not drain at the
        // barrier while every wave refetches its operands.
        auto ld_a = frag_a;
        auto ld_b = frag_b;
        auto col_block = [&](int j) { return min((n0 + wn * T::TN + j * 16) >> 7, n_blocks - 1); };
        // DMA pieces of the stage issued after the MFMA of column j of the
        // last row: piece q goes out after column q * FN / kIssue.
        auto issue_after = [&](int kb, int buf, auto jc) {
          constexpr int j = decltype(jc)::value;
          static_for<DP::kIssue>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            if constexpr (q * T::FN / DP::kIssue == j) issue_piece(kb, buf, qc);
          });
        };
        static_assert(SF == kScaleUE8M0, "the late-barrier loop is the power-of-two-scale one");
        if (nkb > 0) issue_stage(kb_at(0), 0);
        if (nkb > 1) {
          issue_stage(kb_at(1), 1);
          wait_stage<DP, 1>(wave);
        } else {
          wait_vm<0>();
        }
        barrier_all();
        {
          // Exponent bytes: A rows at kSOff, the weight blocks (cb_first & ~3)
          // onwards at kSBOff.
          auto ld_e = [&](const uint8_t* sp, int i) { return (int)sp[T::kSOff + wm * T::TM + i * 16 + fr]; };
          auto ld_sbe = [&](const uint8_t* sp, int j) {
            return (int)sp[T::kSBOff + col_block(j) - (cb_first & ~3)];
          };
          v8i bfrag[T::FN];
          int sbe[T::FN];
#pragma unroll
          for (int j = 0; j < T::FN; ++j) {
            bfrag[j] = ld_b(smem, j);
            sbe[j] = ld_sbe(smem, j);
          }
          v8i afrag = ld_a(smem, 0);
          int ae = ld_e(smem, 0);
          for (int it = 0; it < nkb; ++it) {
            const uint8_t* st = smem + (it & 1) * T::kStageBytes;
            const uint8_t* sn = smem + ((it + 1) & 1) * T::kStageBytes;
            // The DMA after the barrier loads slice it + 2; in the last two
            // slices it reloads slice it into its own, no longer read, buffer
            // (identical bytes), which keeps the loop free of branches that
            // would let the compiler sink the MFMAs below the barrier.
            const int kb_next = kb_at(it + 2 < nkb ? it + 2 : it);
            static_for<T::FM>([&](auto ic) {
              constexpr int i = decltype(ic)::value;
              if constexpr (i == T::FM - 1) {
                __builtin_amdgcn_sched_barrier(0);
                wait_vm<0>();  // this wave's DMAs of slice it + 1 (none of it + 2 issued yet)
                barrier_all();
              }
              // Row by row: without this fence the compiler hoists every
              // row's A fragment load to the top of the slice and spills.
              __builtin_amdgcn_sched_barrier(0);
              const v8i a_cur = afrag;
              const int e_cur = ae;
              if constexpr (i + 1 < T::FM) {
                afrag = ld_a(st, i + 1);
                ae = ld_e(st, i + 1);
              } else {
                afrag = ld_a(sn, 0);  // unused after the last slice (reads stale LDS)
                ae = ld_e(sn, 0);
              }
              static_for<T::FN>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                acc[i][j] = scaled_mma(a_cur, e_cur, bfrag[j], sbe[j], acc[i][j]);
                if constexpr (i == T::FM - 1) {
                  // Keep the compiler from hoisting the load above the MFMA
                  // that still reads the register it overwrites.
                  __builtin_amdgcn_sched_barrier(0);
                  bfrag[j] = ld_b(sn, j);
                  sbe[j] = ld_sbe(sn, j);
                  issue_after(kb_next, it & 1, jc);
                }
              });
            });
          }
        }
        // The reload issued in the last slice must land before the epilogue
        // or the next unit writes LDS.
        wait_vm<0>();
      } else {

  #pragma unroll
        for (int st = 0; st < T::STAGES - 1; ++st)
          if (st < nkb) issue_stage(kb_at(st), st);

        for (int it = 0; it < nkb; ++it) {
          // Wait for this wave's DMAs of stage `it` (newer stages may stay in
          // flight), then barrier so every wave's part of the stage has landed.
          if (it + T::STAGES - 2 < nkb) {
            wait_stage<DP, T::STAGES - 2>(wave);
          } else {
            wait_vm<0>();
          }
          barrier_all();
          // Stage it + STAGES - 1 reuses the buffer of stage it - 1, which every
          // wave finished reading before the barrier above.
          const bool refill = it + T::STAGES - 1 < nkb;
          const int kb_next = refill ? kb_at(it + T::STAGES - 1) : 0;
          const int buf_next = (it + T::STAGES - 1) % T::STAGES;
          if constexpr (T::kSpreadRows == 0) {
            if (refill) issue_stage(kb_next, buf_next);
          }

          const uint8_t* st = smem + (it % T::STAGES) * T::kStageBytes;
          if constexpr (SF == kScaleUE8M0) {
            // Block-scaled MFMA: lane l supplies the exponent of its A row
            // (l % 16) and of its B column (l % 16) for the 32-deep K block
            // l / 16; all four blocks of a slice share the 128-wide scales, and
            // the products, scaled by 2^(ea + eb - 254), accumulate into acc
            // inside the matrix core.  No promotion on the VALU.
            const uint8_t* sbb = st + T::kSBOff - (cb_first & ~3);
            int sbe[T::FN];
  #pragma unroll
            for (int j = 0; j < T::FN; ++j)
              sbe[j] = sbb[min((n0 + wn * T::TN + j * 16) >> 7, n_blocks - 1)];
            v8i bfrag[T::FN];
  #pragma unroll
            for (int j = 0; j < T::FN; ++j) bfrag[j] = frag_b(st, j);
            auto load_a = [&](int i) { return frag_a(st, i); };
            auto load_e = [&](int i) { return (int)st[T::kSOff + wm * T::TM + i * 16 + fr]; };
            v8i afrag = load_a(0);
            int ae = load_e(0);
            static_for<T::FM>([&](auto ic) {
              constexpr int i = decltype(ic)::value;
              const v8i a_cur = afrag;
              const int e_cur = ae;
              if constexpr (i + 1 < T::FM) {
                afrag = load_a(i + 1);
                ae = load_e(i + 1);
              }
  #pragma unroll
              for (int j = 0; j < T::FN; ++j)
                acc[i][j] = scaled_mma(a_cur, e_cur, bfrag[j], sbe[j], acc[i][j]);
              if constexpr (T::kSpreadRows > 0) {
                if (refill) issue_row(kb_next, buf_next, ic);
              }
            });
          } else {
            // One weight scale for all the wave's columns when they sit in one
            // 128-column block; row scales of B (K-grouped) differ per column.
            constexpr bool kOneSB = T::kOneSB && SF != kScaleRowB;
            float sbw = 0.0f;
            float sbv[T::FN];
            const float* sbs = reinterpret_cast<const float*>(st + T::kSBOff);
            if constexpr (SF == kScaleRowB) {
  #pragma unroll
              for (int j = 0; j < T::FN; ++j) sbv[j] = sbs[wn * T::TN + j * 16 + fr];  // this lane's output column
            } else if (kOneSB) {
              const int cb = min((n0 + wn * T::TN) >> 7, n_blocks - 1);
              sbw = sbs[cb - cb_first];
            } else {
  #pragma unroll
              for (int j = 0; j < T::FN; ++j) {
                const int cb = min((n0 + wn * T::TN + j * 16) >> 7, n_blocks - 1);
                sbv[j] = sbs[cb - cb_first];
              }
            }
            v8i bfrag[T::FN];
  #pragma unroll
            for (int j = 0; j < T::FN; ++j) bfrag[j] = frag_b(st, j);
            // Software pipeline over the fragment rows: the MFMAs of row i+1 are
            // issued into a second set of result registers before the promotion
            // FMAs of row i, so the matrix core and the VALU overlap instead of
            // each FMA waiting on the MFMA just issued.
            auto load_a = [&](int i) { return frag_a(st, i); };
            // Activation scales of fragment row i for this lane: its row fr
            // (transposed fragments) or rows 4 kg .. 4 kg + 3.
            auto load_s = [&](int i) {
              if constexpr (kTr) {
                const float v = *reinterpret_cast<const float*>(st + T::kSOff + (wm * T::TM + i * 16 + fr) * 4);
                return make_float4(v, v, v, v);
              } else {
                return *reinterpret_cast<const float4*>(st + T::kSOff + (wm * T::TM + i * 16 + 4 * kg) * 4);
              }
            };
            v4f part[T::kPipe ? 2 : 1][T::FN];
            v8i afrag = load_a(0);
            float4 s4 = load_s(0);
            if (T::kPipe) {
  #pragma unroll
              for (int j = 0; j < T::FN; ++j) part[0][j] = slice_mma(afrag, bfrag[j]);
            }
            static_for<T::FM>([&](auto ic) {
              constexpr int i = decltype(ic)::value;
              constexpr int cur = T::kPipe ? (i & 1) : 0;
              const float4 s_cur = s4;
              if constexpr (T::kPipe) {
                if constexpr (i + 1 < T::FM) {
                  afrag = load_a(i + 1);
                  s4 = load_s(i + 1);
  #pragma unroll
                  for (int j = 0; j < T::FN; ++j) part[cur ^ 1][j] = slice_mma(afrag, bfrag[j]);
                }
              } else {
                // MFMAs of row i, then the LDS reads of row i + 1, which complete
                // while the promotion FMAs of row i run.
                // 256x256 tiles: the row's MFMAs go out as one block at raised
                // wave priority, so the SIMD's other wave fills the matrix
                // core's busy time with its promotion FMAs instead of
                // competing for issue (prefill 138.3 -> 134.6 us; on the
                // 128-row tiles the same measured 1-4% slower).
                constexpr bool kPrio = T::BM * T::BN >= 256 * 256;
                if constexpr (kPrio) {
                  __builtin_amdgcn_s_setprio(2);
                  __builtin_amdgcn_sched_barrier(0);
                }
  #pragma unroll
                for (int j = 0; j < T::FN; ++j) part[0][j] = slice_mma(afrag, bfrag[j]);
                if constexpr (kPrio) {
                  __builtin_amdgcn_sched_barrier(0);
                  __builtin_amdgcn_s_setprio(0);
                }
                if constexpr (i + 1 < T::FM) {
                  afrag = load_a(i + 1);
                  s4 = load_s(i + 1);
                }
              }
              if constexpr (T::kSpreadRows > 0) {
                if (refill) issue_row(kb_next, buf_next, ic);
              }
              if constexpr (kTr) {
                // One row per lane: one scale for all four results of a fragment.
                const float sc = kOneSB ? s_cur.x * sbw : 0.0f;
  #pragma unroll
                for (int j = 0; j < T::FN; ++j) {
                  const float scj = kOneSB ? sc : s_cur.x * sbv[j];
  #pragma unroll
                  for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(part[cur][j][e], scj, acc[i][j][e]);
                }
              } else {
                const float sa[4] = {s_cur.x, s_cur.y, s_cur.z, s_cur.w};
                float sc[4];
  #pragma unroll
                for (int e = 0; e < 4; ++e) sc[e] = kOneSB ? sa[e] * sbw : 0.0f;
  #pragma unroll
                for (int j = 0; j < T::FN; ++j)
  #pragma unroll
                  for (int e = 0; e < 4; ++e)
                    acc[i][j][e] = fmaf(part[cur][j][e], kOneSB ? sc[e] : sa[e] * sbv[j], acc[i][j][e]);
              }
            });
          }
        }
      }

      // ------------------------------------------------------- split-K fixup
      if (SK && partial) {
        // Partials go through device-scope (sc1) 16-byte buffer stores and
        // loads, which are coherent across XCDs without a cache-wide
        // write-back.  Each thread waits for its stores to complete before the
        // barrier; the arrival counter is bumped after the barrier, so the
        // workgroup that sees the count reach (contributors - 1) reads
        // complete partials.  Slot 2 r + {0, 1} holds run r's first / last
        // segment; a slot is [fragment][thread] float4.
        constexpr int kFrag = T::FM * T::FN;
        constexpr int kPartBytes = kFrag * T::kThreads * 16;  // BM * BN * 4
        constexpr int kCacheSc1 = 16;                         // cache-policy bits: sc1
        // 128x128 decode tiles first look whether every other contributor
        // has already published: then this workgroup is the last one, keeps
        // its own partial in registers and skips the store-and-wait round
        // trip of its 64 KB partial (about 3 us), the usual case for the
        // workgroup on the critical path.  Nobody waits for anybody either
        // way.  (On 64x64 tiles the counter read costs as much as the 16 KB
        // store it can save: measured 2-3% slower there.)
        constexpr bool kEarly = kFrag <= 8 && T::kWaves <= 8 && T::BM * T::BN >= 128 * 128;
        // The partial slots follow the counter region of the workspace.  A
        // run of S parts per tile has one segment and one slot; an equal run
        // may end in one tile and begin in the next, so it has two.
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(reinterpret_cast<char*>(p.workspace) + kStreamKCounterBytes), (short)0,
            s.sk_slots * kPartBytes, 0x00020000);
        const int my_slot = sk_split > 0 ? run : 2 * run + slot;
        const int tr = t - dp_tiles;
        const int it_a = tr * nkb_total;
        const int w_lo = sk_owner(it_a), w_hi = sk_owner(it_a + nkb_total - 1);
        bool early = false;
        if constexpr (kEarly) {
          if (tid == 0)
            last_flag = __hip_atomic_load(&p.counters[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == w_hi - w_lo;
          __syncthreads();
          early = last_flag;
        }
        v4f own[kEarly ? kFrag : 1];
        if (early) {
#pragma unroll
          for (int f = 0; f < (kEarly ? kFrag : 1); ++f) own[f] = acc[f / T::FN][f % T::FN];
        } else {
#pragma unroll
          for (int f = 0; f < kFrag; ++f)
            __builtin_amdgcn_raw_buffer_store_b128(acc[f / T::FN][f % T::FN], rs,
                                                   my_slot * kPartBytes + f * T::kThreads * 16 + tid * 16, 0, kCacheSc1);
          asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
          __syncthreads();
          if (tid == 0) {
            const int old = __hip_atomic_fetch_add(&p.counters[t], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_flag = (old == w_hi - w_lo);
          }
          __syncthreads();
          if (!last_flag) continue;
        }
        // Sum the partials of runs w_lo .. w_hi (ascending K) into acc, in
        // chunks of fragments with up to kG runs' loads in flight; on the
        // early path this workgroup's own run comes from registers.
        const int lo_slot = sk_start(w_lo) < it_a ? 1 : 0;  // run w_lo began in an earlier tile
        // Fragments per chunk: the largest divisor of kFrag up to 8.
        constexpr int kChunk = kFrag % 8 == 0 ? 8 : kFrag % 5 == 0 ? 5 : kFrag % 4 == 0 ? 4 : kFrag % 3 == 0 ? 3 : kFrag % 2 == 0 ? 2 : 1;
        constexpr int kG = T::kWaves >= 16 ? 1 : (kFrag >= 32 ? 2 : 4);
        static_assert(kFrag % kChunk == 0, "fragments must split into whole chunks");
        static_for<kFrag / kChunk>([&](auto cc) {
          constexpr int f0 = decltype(cc)::value * kChunk;
#pragma unroll
          for (int f = 0; f < kChunk; ++f) acc[(f0 + f) / T::FN][(f0 + f) % T::FN] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
          for (int w = w_lo; w <= w_hi; w += kG) {
            v4f v[kG][kChunk];
#pragma unroll
            for (int q = 0; q < kG; ++q) {
              const int src = sk_split > 0 ? w + q : 2 * (w + q) + ((w + q) == w_lo ? lo_slot : 0);
              const bool mine = kEarly && early && (w + q) == run;
#pragma unroll
              for (int f = 0; f < kChunk; ++f)
                v[q][f] = (w + q <= w_hi && !mine)
                              ? __builtin_amdgcn_raw_buffer_load_b128(
                                    rs, src * kPartBytes + (f0 + f) * T::kThreads * 16 + tid * 16, 0, kCacheSc1)
                              : v4f{0.0f, 0.0f, 0.0f, 0.0f};
              if constexpr (kEarly) {
                if (mine) {
#pragma unroll
                  for (int f = 0; f < kChunk; ++f) v[q][f] = own[f0 + f];
                }
              }
            }
#pragma unroll
            for (int q = 0; q < kG; ++q)
              if (w + q <= w_hi) {
#pragma unroll
                for (int f = 0; f < kChunk; ++f) acc[(f0 + f) / T::FN][(f0 + f) % T::FN] += v[q][f];
              }
          }
        });
        if (tid == 0) __hip_atomic_store(&p.counters[t], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }

      // ------------------------------------------------------------ epilogue
      // bf16 (RNE) results, stored from registers or staged through LDS and
      // stored as 16-byte row chunks.  Transposed fragments: a lane holds row
      // fr, columns 4kg..4kg+3 of each fragment, written as one 8-byte word
      // pair.  Otherwise a lane holds column fr of rows 4kg..4kg+3, and lane
      // pairs (fr, fr^1) swap halves so each lane writes two rows of two
      // adjacent columns as 32-bit words.  Staged rows are padded by 16 bytes:
      // the rows of one write instruction then start on different banks, and
      // the whole 256 x 256 tile fits the two stages' 132 KB, so it is written
      // in one pass (with 32 bytes of padding it took two 128-row passes and
      // two more barriers).
      constexpr int kRowBytes = T::BN * 2 + 16;
      constexpr int kER = (T::BM * kRowBytes <= T::STAGES * T::kStageBytes) ? T::BM : T::TM;
      static_assert(kER * kRowBytes <= T::STAGES * T::kStageBytes, "epilogue tile does not fit");
      static_assert(kER == T::BM || kER == T::TM, "epilogue pass must be whole wave rows");
      const bool odd = fr & 1;
      // Round and pair up first: the packed words take half the registers
      // of the fp32 accumulators, which are dead from here on.
      uint32_t packed[T::FM][T::FN][2];
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
          const uint32_t b0 = f32_to_bf16_rne(acc[i][j][0]), b1 = f32_to_bf16_rne(acc[i][j][1]);
          const uint32_t b2 = f32_to_bf16_rne(acc[i][j][2]), b3 = f32_to_bf16_rne(acc[i][j][3]);
          if constexpr (kTr) {  // columns 4kg, 4kg+1 | 4kg+2, 4kg+3 of row fr
            packed[i][j][0] = b0 | (b1 << 16);
            packed[i][j][1] = b2 | (b3 << 16);
            continue;
          }
          const uint32_t send = odd ? (b0 | (b1 << 16)) : (b2 | (b3 << 16));
          const uint32_t recv = (uint32_t)__shfl_xor((int)send, 1, 64);
          if (odd) {  // rows 4kg+2, 4kg+3; columns fr-1, fr
            packed[i][j][0] = (recv & 0xFFFFu) | (b2 << 16);
            packed[i][j][1] = (recv >> 16) | (b3 << 16);
          } else {    // rows 4kg+0, 4kg+1; columns fr, fr+1
            packed[i][j][0] = b0 | ((recv & 0xFFFFu) << 16);
            packed[i][j][1] = b1 | ((recv >> 16) << 16);
          }
        }
      if (LAYOUT != kContiguous && !DQ) {
        // Plain bf16 output: every lane stores its packed words straight from
        // registers (rows r, r + 1 of two adjacent columns, 32-bit stores;
        // the 8 lanes of a row write 32 contiguous bytes and the wave's 4
        // fragments of a row fill whole 128-byte lines).  No LDS staging
        // and no barrier, so the workgroup goes on to its next tile while
        // the stores drain.  (The contiguous layout keeps the LDS-staged
        // stores: its per-row expert checks here pushed the 256 x 256
        // kernel to 69 spilled registers and 8% more time.)
        if constexpr (kTr) {
          // One 8-byte store per fragment: row fr, columns 4kg .. 4kg + 3
          // (the 4 lanes of a row write 32 contiguous bytes, the wave's 4
          // fragments of a row whole 128-byte lines).
#pragma unroll
          for (int i = 0; i < T::FM; ++i) {
            const int row = m0 + wm * T::TM + i * 16 + fr;
            if (row >= rows_valid) continue;
            uint16_t* drow = D + (int64_t)row * p.ldd;
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
              const int col = n0 + wn * T::TN + j * 16 + 4 * kg;
              if (col + 3 < p.n) {
                *reinterpret_cast<uint2*>(drow + col) = make_uint2(packed[i][j][0], packed[i][j][1]);
              } else {
#pragma unroll
                for (int e = 0; e < 3; ++e)
                  if (col + e < p.n) drow[col + e] = (uint16_t)(packed[i][j][e >> 1] >> ((e & 1) * 16));
              }
            }
          }
          continue;  // next work unit (or pass)
        }
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = m0 + wm * T::TM + i * 16 + 4 * kg + (odd ? 2 : 0) + h;
            if (row >= rows_valid) continue;
            uint16_t* drow = D + (int64_t)row * p.ldd;
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
              const int col = n0 + wn * T::TN + j * 16 + (fr & ~1);
              if (col + 1 < p.n) {
                *reinterpret_cast<uint32_t*>(drow + col) = packed[i][j][h];
              } else if (col < p.n) {
                drow[col] = (uint16_t)(packed[i][j][h] & 0xFFFFu);
              }
            }
          }
        continue;  // next work unit (or pass)
      }
#pragma unroll
      for (int er = 0; er < T::BM / kER; ++er) {
        lds_barrier();  // LDS free: the K loop (or previous pass) is done reading
        if (kER == T::BM || wm == er) {
          const int rbase = (kER == T::BM) ? wm * T::TM : 0;
#pragma unroll
          for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
              if constexpr (kTr) {
                const int r = rbase + i * 16 + fr;
                const int c = wn * T::TN + j * 16 + 4 * kg;
                *reinterpret_cast<uint2*>(smem + r * kRowBytes + c * 2) = make_uint2(packed[i][j][0], packed[i][j][1]);
              } else {
                const int r = rbase + i * 16 + 4 * kg + (odd ? 2 : 0);
                const int c = wn * T::TN + j * 16 + (fr & ~1);
                uint8_t* dst = smem + r * kRowBytes + c * 2;
                *reinterpret_cast<uint32_t*>(dst) = packed[i][j][0];
                *reinterpret_cast<uint32_t*>(dst + kRowBytes) = packed[i][j][1];
              }
            }
        }
        lds_barrier();
        constexpr int kChunksPerRow = T::BN / 8;
        for (int idx = tid; idx < kER * kChunksPerRow; idx += T::kThreads) {
          const int rl = idx / kChunksPerRow, ch = idx - rl * kChunksPerRow;
          const int row = m0 + er * kER + rl;
          bool ok = row < rows_valid && row < m0 + T::BM;
          if (LAYOUT == kContiguous && ok) ok = p.m_indices[row] == g;
          if (!ok) continue;
          const int col = n0 + ch * 8;
          if (col >= p.n) continue;
          const uint4 v = *reinterpret_cast<const uint4*>(smem + rl * kRowBytes + ch * 16);
          uint16_t* drow = D + (int64_t)row * p.ldd;
          if (col + 8 <= p.n) {
            *reinterpret_cast<uint4*>(drow + col) = v;
          } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            for (int e = 0; e < p.n - col; ++e) drow[col + e] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
          }
        }
        if constexpr (T::BN % 128 == 0) {
          if (DQ) {
            // Quantised copy of the output rows just staged: every 1x128 tile
            // (a row's 128-column block; the tile's columns are whole blocks)
            // gets s = amax/448 and e4m3(x/s) computed from the bf16 values,
            // as the activation quantiser computes them.  Eight consecutive
            // lanes own one block of a row, 16 values each; every lane runs
            // every iteration so the amax shuffles see all eight.
            constexpr int kQPerRow = T::BN / 16;
            static_assert((kER * kQPerRow) % T::kThreads == 0, "uneven quantisation passes");
            for (int idx = tid; idx < kER * kQPerRow; idx += T::kThreads) {
              const int rl = idx / kQPerRow, qc = idx - rl * kQPerRow;
              const int row = m0 + er * kER + rl;
              const int col = n0 + qc * 16;
              bool ok = row < rows_valid && row < m0 + T::BM && col < p.n;
              if (LAYOUT == kContiguous && ok) ok = p.m_indices[row] == g;
              const uint4 lo = *reinterpret_cast<const uint4*>(smem + rl * kRowBytes + qc * 32);
              const uint4 hi = *reinterpret_cast<const uint4*>(smem + rl * kRowBytes + qc * 32 + 16);
              const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
              float amax = 0.0f;
#pragma unroll
              for (int e = 0; e < 8; ++e)
                amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(w[e] & 0xFFFFu)), fabsf(bf16_bits_to_f32(w[e] >> 16))));
#pragma unroll
              for (int off = 4; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 8));
              uint32_t out[4];
              float s_out = 0.0f;
              uint32_t e_out = 0u;
              if (p.dq_ue8m0) {
                // Power-of-two scale 2^(E - 127), E as the UE8M0 quantiser picks it.
                e_out = ue8m0_exponent(amax);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  out[e] = e4m3_x4(pow2_quotient(w[2 * e] & 0xFFFFu, e_out), pow2_quotient(w[2 * e] >> 16, e_out),
                                   pow2_quotient(w[2 * e + 1] & 0xFFFFu, e_out),
                                   pow2_quotient(w[2 * e + 1] >> 16, e_out));
              } else {
                s_out = amax / 448.0f;
                const double rcp = tile_reciprocal(s_out);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  out[e] = e4m3_x4(quotient(w[2 * e] & 0xFFFFu, rcp), quotient(w[2 * e] >> 16, rcp),
                                   quotient(w[2 * e + 1] & 0xFFFFu, rcp), quotient(w[2 * e + 1] >> 16, rcp));
              }
              if (ok) {
                *reinterpret_cast<uint4*>(DQ + (int64_t)row * p.n + col) = make_uint4(out[0], out[1], out[2], out[3]);
                if ((qc & 7) == 0) {
                  const int64_t at = (int64_t)(col >> 7) * p.ld_dsf + row;
                  if (p.dq_ue8m0) DSF[at] = (uint8_t)e_out;
                  else reinterpret_cast<float*>(DSF)[at] = s_out;
                }
              }
            }
          }
        }
      }
      if constexpr (T::BN % 128 == 0) {
        // Dense layout: the tile holding the last rows also zeroes the scale
        // padding rows [M, ld_dsf) of its column blocks, as the quantiser does.
        if (DQ && LAYOUT == kDense && m0 + T::BM >= p.m) {
          const int pad = (int)(p.ld_dsf - p.m);
          for (int idx = tid; idx < pad * (T::BN / 128); idx += T::kThreads) {
            const int cb = (n0 >> 7) + idx / pad;
            if (cb * 128 < p.n) {
              const int64_t at = (int64_t)cb * p.ld_dsf + p.m + idx % pad;
              if (p.dq_ue8m0) DSF[at] = 0;
              else reinterpret_cast<float*>(DSF)[at] = 0.0f;
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host side

// Kernel instances (tile shape, wave grid, pipeline depth).
using TileP256 = Tile<256, 256, 2, 4, 2>;  // prefill: 8 waves, 128x64 per wave
using TileP128 = Tile<128, 128, 2, 2, 4>;  // mid-size and decode M <= 128: 64x64 per wave
using TileD128 = Tile<128, 64, 2, 2, 4>;   // decode, narrow N tiles: 64x32 per wave
using TileD64 = Tile<64, 256, 1, 4, 3>;    // decode, M <= 64: 64x64 per wave
using TileS64 = Tile<64, 64, 2, 2, 4>;     // decode, small tiles: 32x32 per wave
using TileW128 = Tile<128, 256, 2, 4, 3>;  // decode, M <= 128, wide N: 8 waves, 64x64 per wave
using TileP128w8 = Tile<128, 128, 2, 4, 4>;  // decode: 8 waves (2 per SIMD), 64x32 per wave
using TileS64w8 = Tile<64, 64, 2, 4, 4>;     // decode small tiles: 8 waves, 32x16 per wave
using TileW128w16 = Tile<128, 256, 4, 4, 3>; // decode wide N: 16 waves, 32x64 per wave
using TileV128 = Tile<128, 256, 1, 4, 3>;    // decode: every wave holds all 128 rows, 128x64 per wave
using TileV128w8 = Tile<128, 256, 1, 8, 3>;  // the same with 8 waves, 128x32 per wave
// Non-power-of-two BLOCK_N (DeepGEMM project introduction, Optimisations,
// unaligned block sizes): 256 x 160, 8 waves of 64 x 80, three stages (the
// 256-byte weight-scale slot makes 3 x 54528 bytes fit the 160 KB of LDS).
// 4096 x 2112 gives 224 such tiles, one wave on 256 CUs, against 144 of
// 256 x 256.
using TileP160 = Tile<256, 160, 4, 2, 3, 256>;

struct Variant {
  int bm, bn, threads;
};
constexpr Variant kVariants[] = {
    {TileP256::BM, TileP256::BN, TileP256::kThreads},
    {TileP128::BM, TileP128::BN, TileP128::kThreads},
    {TileD128::BM, TileD128::BN, TileD128::kThreads},
    {TileD64::BM, TileD64::BN, TileD64::kThreads},
    {TileS64::BM, TileS64::BN, TileS64::kThreads},
    {TileW128::BM, TileW128::BN, TileW128::kThreads},
    {TileP128w8::BM, TileP128w8::BN, TileP128w8::kThreads},
    {TileS64w8::BM, TileS64w8::BN, TileS64w8::kThreads},
    {TileW128w16::BM, TileW128w16::BN, TileW128w16::kThreads},
    {TileV128::BM, TileV128::BN, TileV128::kThreads},
    {TileV128w8::BM, TileV128w8::BN, TileV128w8::kThreads},
    {TileP160::BM, TileP160::BN, TileP160::kThreads},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

template <class T, int LAYOUT, int SF>
hipError_t launch_one(const GemmParams& p, const Schedule& s, int grid, hipStream_t stream) {
  if constexpr (LAYOUT != kContiguous) {  // contiguous tiles may take two passes: data-parallel only
    if (s.stream_k) {
      hipLaunchKernelGGL((gemm_kernel<T, LAYOUT, true, SF>), dim3(grid), dim3(T::kThreads), 0, stream, p, s);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<T, LAYOUT, false, SF>), dim3(grid), dim3(T::kThreads), 0, stream, p, s);
  return hipGetLastError();
}

// Dense GEMM with MN-major operands (p.majors: kAMajorMN | kBMajorMN).
template <class T, int MAJ, int SF>
hipError_t launch_majors_one(const GemmParams& p, const Schedule& s, int grid, hipStream_t stream) {
  if (s.stream_k)
    hipLaunchKernelGGL((gemm_kernel<T, kDense, true, SF, MAJ>), dim3(grid), dim3(T::kThreads), 0, stream, p, s);
  else
    hipLaunchKernelGGL((gemm_kernel<T, kDense, false, SF, MAJ>), dim3(grid), dim3(T::kThreads), 0, stream, p, s);
  return hipGetLastError();
}

template <class T, int SF>
hipError_t launch_majors_sf(const GemmParams& p, const Schedule& s, int grid, hipStream_t stream) {
  switch (p.majors) {
    case kAMajorMN: return launch_majors_one<T, kAMajorMN, SF>(p, s, grid, stream);
    case kBMajorMN: return launch_majors_one<T, kBMajorMN, SF>(p, s, grid, stream);
    case kAMajorMN | kBMajorMN: return launch_majors_one<T, kAMajorMN | kBMajorMN, SF>(p, s, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class T>
hipError_t launch_majors(const GemmParams& p, const Schedule& s, int grid, hipStream_t stream) {
  return p.sf_ue8m0 ? launch_majors_sf<T, kScaleUE8M0>(p, s, grid, stream)
                    : launch_majors_sf<T, kScaleF32>(p, s, grid, stream);
}

template <class T, int SF>
hipError_t launch_layout(int layout, const GemmParams& p, const Schedule& s, int grid, hipStream_t stream) {
  switch (layout) {
    case kDense: return launch_one<T, kDense, SF>(p, s, grid, stream);
    case kContiguous: return launch_one<T, kContiguous, SF>(p, s, grid, stream);
    default: return launch_one<T, kMasked, SF>(p, s, grid, stream);
  }
}

// K-grouped layout: data-parallel, row scales on B.
template <class T>
hipError_t launch_kgrouped(const GemmParams& p, const Schedule& s, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_kernel<T, kKGrouped, false, kScaleRowB>), dim3(grid), dim3(T::kThreads), 0, stream, p, s);
  return hipGetLastError();
}

// Ceiling division of a >= 0 by b > 0 that cannot overflow.
int cdiv(int a, int b) { return a / b + (a % b != 0); }
int64_t cdiv64(int64_t a, int64_t b) { return a / b + (a % b != 0); }

constexpr int smallest_tile_dim(bool rows) {
  int v = 1 << 30;
  for (const Variant& t : kVariants) v = std::min(v, rows ? t.bm : t.bn);
  return v;
}

// Stream-K partial slots are addressed with 32-bit offsets: 2 * grid slots of
// at most 256 KB stay below 2^31 bytes with this cap.
constexpr int kMaxStreamKGrid = 1024;

int forced_variant() {
  // DG_FORCE_CONFIG="variant[:division[:k_rotate]]" overrides the heuristic
  // (sweeps and tests); division 0 = data-parallel, 1 = equal stream-K runs,
  // S >= 2 = S parts per tile.
  const char* e = getenv("DG_FORCE_CONFIG");
  if (!e || !*e) return -1;
  return atoi(e);
}

int forced_stream_k() {  // second field, -1 when absent
  const char* e = getenv("DG_FORCE_CONFIG");
  if (!e || !*e) return -1;
  const char* c = strchr(e, ':');
  return c ? std::max(0, atoi(c + 1)) : -1;
}

int forced_rotate() {  // third field: 0 or 1, -1 when absent
  const char* e = getenv("DG_FORCE_CONFIG");
  if (!e || !*e) return -1;
  const char* c = strchr(e, ':');
  if (!c) return -1;
  c = strchr(c + 1, ':');
  return c ? (atoi(c + 1) != 0) : -1;
}

}  // namespace

bool plannable(int layout, int m, int n, int groups) {
  if (m < 0 || n < 0 || groups < 1) return false;
  const int64_t gmul = (layout == kMasked || layout == kKGrouped) ? groups : 1;
  const int64_t tiles = cdiv64(m, smallest_tile_dim(true)) * cdiv64(n, smallest_tile_dim(false));  // < 2^50
  return tiles <= ((1LL << 31) - 1) / gmul;
}

bool variant_quantises_output(int variant) {
  return variant >= 0 && variant < kNumVariants && kVariants[variant].bn % 128 == 0;
}

GemmConfig choose_config(int layout, int m, int n, int k, int groups, int num_cus, int expected_m, bool qout,
                         bool narrow_ok) {
  // m: dense M, contiguous M_total, masked M_max.  The rules below come from
  // sweeps over tile variants on the benchmark shapes.  For the masked
  // layout a host hint of the typical valid rows per group replaces M_max in
  // the choice of tile (the launch itself still covers M_max rows per group,
  // skipping empty tiles on the device).
  const int nkb = k / kBlockK;
  const bool hinted = layout == kMasked && expected_m > 0 && expected_m < m;
  const int rows = hinted ? expected_m : m;
  const int gmul = (layout == kMasked || layout == kKGrouped) ? groups : 1;
  // Tile counts in 64 bits: with plannable() shapes every count fits an int,
  // but the products below (10 x tiles, tiles x parts) need not.
  auto tiles_of = [&](int bm, int bn) { return (int64_t)cdiv(rows, bm) * gmul * cdiv(n, bn); };
  int v;
  if (rows <= 128) {
    // Decode-sized M: the launch streams B once.  128x128 tiles (8 waves)
    // when they alone keep most CUs busy or K is long, else 64x64 tiles.
    const int64_t t128 = tiles_of(128, 128);
    v = (rows > 64 && (10 * t128 >= 7 * num_cus || nkb >= 64)) ? 6 : 4;
  } else if (tiles_of(256, 256) >= num_cus / 2) {
    v = 0;
    // Non-power-of-two BLOCK_N: when 256 x 256 tiles fill under 70% of the
    // CUs but one round of 256 x 160 tiles fills at least 80% of them, the
    // narrower tile runs data-parallel in one wave (measured 4096 x 2112 x
    // 7168: 103.4 us against 113.6 us for 256 x 256 tiles in equal
    // stream-K runs).  Not for the masked layout, whose tile count is only
    // a hint (4 x 1024 x 4096 x 7168 with about 512 valid rows per group:
    // 177 us with 256 x 160 tiles against 133 us with 256 x 256).
    const int64_t t256 = tiles_of(256, 256), t160 = tiles_of(256, 160);
    if (narrow_ok && !qout && (layout == kDense || layout == kContiguous) && 10 * t256 < 7 * (int64_t)num_cus && 5 * t160 >= 4 * (int64_t)num_cus && t160 <= num_cus) v = 11;
  } else {
    // Mid-size M (e.g. 1024 rows in all): 128-row tiles, 256 columns wide
    // unless 128 columns fill the CUs' last round better (measured on the
    // pages' all-valid masked rows: 1024x7168x2048 39.8 -> 31.1 us with
    // 128x256, 1024x4096x7168 58.5 -> 53.1 us with 128x128).
    auto fill = [&](int64_t t) { return (double)t / (double)(cdiv64(t, num_cus) * num_cus); };
    v = fill(tiles_of(128, 256)) >= fill(tiles_of(128, 128)) ? 5 : 6;
  }
  // A quantised output needs whole 128-column blocks per tile: the 64-wide
  // decode tiles give way to the 128x128 one.
  const bool widened = qout && kVariants[v].bn % 128 != 0;
  if (widened) v = 6;
  const int fv = forced_variant();
  if (fv >= 0 && fv < kNumVariants) v = fv;
  GemmConfig c{};
  c.variant = v;
  c.bm = kVariants[v].bm;
  c.bn = kVariants[v].bn;
  const int m_tiles = cdiv(m, c.bm) * gmul;
  const int n_tiles = cdiv(n, c.bn);
  c.tiles = m_tiles * n_tiles;
  // Work division.  Tiles that leave most CUs idle get their K ranges cut:
  // decode-sized tiles into S equal parts (one part per workgroup), larger
  // tiles with long K into equal runs of iterations over all CUs.  The
  // estimate uses the hinted rows for the masked layout.
  const int64_t est = tiles_of(c.bm, c.bn);
  int sk = 0;  // 0: data-parallel, 1: equal runs, S >= 2: S parts per tile
  if (layout != kContiguous && layout != kKGrouped && nkb >= 2 && 10 * est < 7 * num_cus) {
    // K parts for 128-row (or smaller) tiles up to 1024 rows in all; beyond
    // that, or when parts do not pay, equal runs for long K.
    if (c.bm <= 128 && rows <= 1024) {
      // Shorter parts for the 128x128 tiles that stand in for 64-wide ones
      // (quantised output): fewer tiles, so more parts (64x4096x7168 fused:
      // 27.5 -> 24.2 us with 8 parts instead of 3).
      const int min_slices = (c.bm * c.bn >= 128 * 128 && !widened) ? 16 : 8;
      int parts = (int)std::min<int64_t>(num_cus / std::max<int64_t>(est, 1), nkb / min_slices);
      // Two 64x64 workgroups share a CU: at least 4 parts where 2 x CUs hold
      // them (128x4096x7168: 20.4 -> 19.5 us with 4 parts on 512 workgroups
      // instead of 2 on 256; 64x7168x16384: 36.8 -> 33.8 us).
      if (v == 4 || v == 7)
        parts = std::max(parts, (int)std::min<int64_t>({4, 2 * num_cus / std::max<int64_t>(est, 1), nkb / min_slices}));
      if (c.bm * c.bn < 128 * 128) parts = std::min(parts, 6);  // 64x2112x7168: 6 parts 3% faster than 4
      // A fixup costs a few microseconds; short K ranges are not worth
      // cutting (64x7168x2048: 11.6 us in 2 parts, 10.2 us whole).
      if (nkb < 24) parts = 1;
      if (parts >= 2) sk = parts;
    }
    // Equal runs for long K - except the masked layout's 256 x 256 tiles,
    // whose valid count is only known on the device: there one data-parallel
    // round measured faster (4 x 1024 x 4096 x 7168 with 1841 valid rows, 160
    // valid tiles: 116.9 us against 132.5 us in equal runs).
    if (sk == 0 && rows > 128 && est * nkb >= 24LL * num_cus && !(layout == kMasked && c.bm == 256)) sk = 1;
  }
  const int fs = forced_stream_k();
  if (fs >= 0) sk = fs;
  if (layout == kContiguous || layout == kKGrouped || nkb < 2) sk = 0;
  if (sk >= 2) sk = std::min(sk, nkb);
  c.stream_k = sk > 0 ? 1 : 0;
  c.sk_split = sk >= 2 ? sk : 0;
  // Aligned parts: one workgroup per part, the grid a multiple of 8 so that
  // the XCD-contiguous numbering of runs spreads them evenly over the XCDs.
  // The 64x64 tiles take 72 KB of LDS, so two workgroups share a CU; with
  // more tiles than CUs a grid of two per CU gives each SIMD a second wave
  // (measured 64x32768x512: 11.0 -> 9.5 us, 64x24576x1536: 16.0 -> 14.5 us).
  // The same holds for their K parts.
  const int per_cu = (v == 4 || v == 7) ? 2 : 1;
  const int cap = std::min(num_cus * per_cu, kMaxStreamKGrid);
  const int64_t runs = c.sk_split ? (int64_t)c.tiles * c.sk_split : cap;
  const int64_t slots = c.sk_split ? runs : 2 * runs;
  c.grid = !c.stream_k ? std::max(1, std::min(c.tiles, num_cus * per_cu))
           : (int)std::min<int64_t>(cap, cdiv64(runs, 8) * 8);
  // Partial slots must stay 32-bit addressable, and every tile needs an
  // arrival counter in the workspace's fixed counter region.
  if (c.stream_k && (slots * c.bm * c.bn * 4 >= (1LL << 31) || c.tiles > kStreamKCounters)) {
    c.stream_k = c.sk_split = 0;
    c.grid = std::max(1, std::min(c.tiles, num_cus));
  }
  c.sk_slots = c.stream_k ? (int)slots : 0;
  c.group_m = 8;
  // Rotated K walks for the decode-sized tiles when the weight rows are a
  // multiple of 16 KiB apart (see the kernel's K walk).  The 256x256 tile
  // keeps every tile on the same slice: its operands are shared through L2
  // by the tiles of a raster group, and rotation would spread that working
  // set over many slices.
  c.k_rotate = (c.bm * c.bn < 256 * 256 && k % 16384 == 0) ? 1 : 0;
  const int fr = forced_rotate();
  if (fr >= 0) c.k_rotate = fr;
  return c;
}

size_t workspace_bytes_for(const GemmConfig& cfg, int layout, int m, int n, int groups) {
  (void)layout; (void)m; (void)n; (void)groups;
  if (!cfg.stream_k) return 0;
  // The fixed counter region, then the fp32 partial tiles.
  return kStreamKCounterBytes + (size_t)cfg.sk_slots * cfg.bm * cfg.bn * sizeof(float);
}

hipError_t launch_gemm(int layout, const GemmParams& p0, const GemmConfig& cfg,
                       hipStream_t stream) {
  GemmParams p = p0;
  Schedule s{};
  s.n_tiles = cdiv(p.n, cfg.bn);
  s.m_tiles = layout == kKGrouped ? cdiv(p.m, cfg.bm) : cfg.tiles / s.n_tiles;  // K-grouped: per group
  s.tiles = cfg.tiles;
  s.stream_k = cfg.stream_k;
  s.sk_split = cfg.sk_split;
  s.sk_slots = cfg.sk_slots;
  s.group_m = cfg.group_m;
  s.k_rotate = cfg.k_rotate;
  if (cfg.stream_k) p.counters = reinterpret_cast<int*>(p.workspace);
  if (layout == kKGrouped) {
    switch (cfg.variant) {
      case 0: return launch_kgrouped<TileP256>(p, s, cfg.grid, stream);
      case 4: return launch_kgrouped<TileS64>(p, s, cfg.grid, stream);
      case 5: return launch_kgrouped<TileW128>(p, s, cfg.grid, stream);
      case 6: return launch_kgrouped<TileP128w8>(p, s, cfg.grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.majors) {  // MN-major operands: dense layout, the dense heuristic's tiles
    if (layout != kDense) return hipErrorInvalidValue;
    switch (cfg.variant) {
      case 0: return launch_majors<TileP256>(p, s, cfg.grid, stream);
      case 4: return launch_majors<TileS64>(p, s, cfg.grid, stream);
      case 5: return launch_majors<TileW128>(p, s, cfg.grid, stream);
      case 6: return launch_majors<TileP128w8>(p, s, cfg.grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.sf_ue8m0) {  // UE8M0 instances: the tiles the heuristic picks
    switch (cfg.variant) {
      case 0: return launch_layout<TileP256, kScaleUE8M0>(layout, p, s, cfg.grid, stream);
      case 1: return launch_layout<TileP128, kScaleUE8M0>(layout, p, s, cfg.grid, stream);
      case 4: return launch_layout<TileS64, kScaleUE8M0>(layout, p, s, cfg.grid, stream);
      case 6: return launch_layout<TileP128w8, kScaleUE8M0>(layout, p, s, cfg.grid, stream);
      case 5: return launch_layout<TileW128, kScaleUE8M0>(layout, p, s, cfg.grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (cfg.variant) {
    case 0: return launch_layout<TileP256, kScaleF32>(layout, p, s, cfg.grid, stream);
    case 1: return launch_layout<TileP128, kScaleF32>(layout, p, s, cfg.grid, stream);
    case 2: return launch_layout<TileD128, kScaleF32>(layout, p, s, cfg.grid, stream);
    case 3: return launch_layout<TileD64, kScaleF32>(layout, p, s, cfg.grid, stream);
    case 4: return launch_layout<TileS64, kScaleF32>(layout, p, s, cfg.grid, stream);
    case 5: return launch_layout<TileW128, kScaleF32>(layout, p, s, cfg.grid, stream);
    case 6: return launch_layout<TileP128w8, kScaleF32>(layout, p, s, cfg.grid, stream);
    case 7: return launch_layout<TileS64w8, kScaleF32>(layout, p, s, cfg.grid, stream);
    case 8: return launch_layout<TileW128w16, kScaleF32>(layout, p, s, cfg.grid, stream);
    case 9: return launch_layout<TileV128, kScaleF32>(layout, p, s, cfg.grid, stream);
    case 10: return launch_layout<TileV128w8, kScaleF32>(layout, p, s, cfg.grid, stream);
    default: return launch_layout<TileP160, kScaleF32>(layout, p, s, cfg.grid, stream);
  }
}

}  // namespace dg
