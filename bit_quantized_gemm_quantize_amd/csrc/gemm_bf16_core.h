// Main loop of the 16-bit-MFMA GEMMs: the W4A16 path on the bf16 MFMA and the exact
// NVFP4 path on the fp16 MFMA (Loader::kF16 picks the instruction; the operand
// layout is the same).
//
// Tiling: a wave owns G activation sub-tiles of 32 rows and F weight sub-tiles of 32
// columns (32 x 32 tiles of v_mfma_f32_32x32x16_bf16 / _f16); the callers use 256 x
// 256 output tiles on 8 waves (two per SIMD) of 128 x 64 (G = 4, F = 2), half tiles of
// 256 x 128 on the same 8 waves (F = 1) to fill the CUs when tiles are few, and tiles
// of 256 x 96 on 4 waves stacked along M (64 x 96 per wave: G = 2, F = 3).  K advances in tiles of 64
// elements: each operand tile is 256 rows x 64 bf16 (128 bytes per row) in LDS,
// 16-byte chunks XOR-swizzled by row (chunk c of row r at c ^ lds_swz<8>(r), for the
// 64-bank LDS), two stages, one barrier per K-tile.
//
// A loader policy turns global data into 16-bit LDS rows (Loader::kF16: fp16, else
// bf16):
//   Loader::issue_regs(kt)            issue the global reads of K-tile kt that land
//                                    in registers (Loader::kRegLoads instructions)
//   Loader::issue_lds(kt, lds_a, lds_b)  issue those that go straight into LDS
//   Loader::store<P>(lds_a, lds_b)    convert half P (0, 1) of the registers and
//                                    write it
// (the early-store loaders take a register set index as well, see below).
// Pipeline of K-tile kt: the fragments of the next MFMA step are read while the
// current step's MFMAs run; the registers of K-tile kt+1 are converted into the
// other stage during steps 1 and 2 and then reloaded with K-tile kt+1+S (S =
// Loader::kSets register sets, so a register load has about S K-tiles); the barrier
// sits in the middle of step 3, whose MFMAs need no LDS, so the first half covers
// the wait and the second the fragment reads of K-tile kt+1 and the issue of
// K-tile kt+2's direct-to-LDS loads into the stage just freed.
#pragma once

#include "q4_epilogue.h"

namespace q4 {

constexpr int kBf16BM = 256, kBf16BN = 256;
constexpr int kBf16KT = 64;                 // K elements per K-tile
constexpr int kBf16RowBytes = kBf16KT * 2;  // 128 bytes of bf16 per tile row
constexpr int kBf16Threads = 256;
constexpr int kBf16GroupM = 4;
constexpr int kBf16TileBytes = kBf16BM * kBf16RowBytes;      // one operand tile
constexpr int kBf16MainLds = 4 * kBf16TileBytes;             // [A0][A1][B0][B1]

__device__ __forceinline__ int lds_chunk_off(int row, int chunk) {
  return row * kBf16RowBytes + ((chunk ^ lds_swz<8>(row)) << 4);
}

template <int F, int G = 4>
struct Bf16Frags {
  u32x4 a[2][G], b[2][F];
};

// fragments of MFMA step s (16 K) of the tile at la / lb into buffer BUF: the wave's
// G activation sub-tiles start at row 32 G wx, its F weight sub-tiles at 32 F wy.
// Rows 32 g + r32 all have the swizzle lds_swz<8>(r32), so one swizzled chunk offset
// per step serves every sub-tile; the sub-tiles are 4 KB apart.
template <int BUF, int F, int G>
__device__ __forceinline__ void bf16_read_frags(Bf16Frags<F, G>& fr, const uint8_t* la, const uint8_t* lb,
                                                int s, int wx, int wy, int lane) {
  const int r32 = lane & 31, h = lane >> 5;
  const int chunk = ((2 * s + h) ^ lds_swz<8>(r32)) << 4;
  const uint8_t* pa = la + (wx * 32 * G + r32) * kBf16RowBytes + chunk;
  const uint8_t* pb = lb + (wy * 32 * F + r32) * kBf16RowBytes + chunk;
#pragma unroll
  for (int g = 0; g < G; ++g) fr.a[BUF][g] = ld16(pa + g * 32 * kBf16RowBytes);
#pragma unroll
  for (int f = 0; f < F; ++f) fr.b[BUF][f] = ld16(pb + f * 32 * kBf16RowBytes);
}

__device__ __forceinline__ v16f mfma_f16_32x32x16(u32x4 a, u32x4 b, v16f c) {
  typedef _Float16 v8h __attribute__((ext_vector_type(8)));
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0,
                                                0, 0);
}

// acc[f][g] holds D[n][m] (A operand = weight rows, B operand = activation rows);
// weight sub-tiles f in [F0, F1); fp16 operands when F16, else bf16.
template <int BUF, int F, int F0 = 0, int F1 = F, bool F16 = false, int G = 4>
__device__ __forceinline__ void bf16_mma(v16f (&acc)[F][G], const Bf16Frags<F, G>& fr) {
#pragma unroll
  for (int f = F0; f < F1; ++f)
#pragma unroll
    for (int g = 0; g < G; ++g)
      acc[f][g] = F16 ? mfma_f16_32x32x16(fr.b[BUF][f], fr.a[BUF][g], acc[f][g])
                      : mfma_bf16_32x32x16(fr.b[BUF][f], fr.a[BUF][g], acc[f][g]);
}

// Stage st of the operand tiles: A at lds + st * tile, B at lds + (2 + st) * tile,
// so the stage offsets fold into the LDS instructions' immediate offsets.
template <int ST>
__device__ __forceinline__ uint8_t* bf16_a(uint8_t* lds) { return lds + ST * kBf16TileBytes; }
template <int ST>
__device__ __forceinline__ uint8_t* bf16_b(uint8_t* lds) { return lds + (2 + ST) * kBf16TileBytes; }

// One K-tile: multiply stage CUR while K-tile kt+1 is converted into the other.
// The sched group barriers interleave the conversion arithmetic and the loads with
// single MFMAs, so that the in-order wave keeps the matrix pipe fed
// (Loader::kValuPerStore: VALU ops of one store part).
template <int CUR, int F, int G, class Loader>
__device__ __forceinline__ void bf16_ktile(v16f (&acc)[F][G], Bf16Frags<F, G>& fr, Loader& ld, int kt,
                                           uint8_t* lds, int wx, int wy, int lane) {
  constexpr int NXT = CUR ^ 1;
  constexpr int kMma = G * F;                                  // MFMAs per step
  constexpr int kValu = (Loader::kValuPerStore + kMma - 1) / kMma;
  constexpr int kH = F / 2;                                    // sub-tiles of step 3 before the barrier
  constexpr int SET = Loader::kSets == 2 ? NXT : 0;            // registers holding K-tile kt+1
  // step 0
  bf16_read_frags<1, F, G>(fr, bf16_a<CUR>(lds), bf16_b<CUR>(lds), 1, wx, wy, lane);
  bf16_mma<0, F, 0, F, Loader::kF16, G>(acc, fr);
  __builtin_amdgcn_sched_group_barrier(0x100, G + F, 0);       // fragment reads first
  __builtin_amdgcn_sched_group_barrier(0x008, kMma, 0);
  __builtin_amdgcn_sched_barrier(0);
  // step 1: half 0 of K-tile kt+1 into the other stage
  bf16_read_frags<0, F, G>(fr, bf16_a<CUR>(lds), bf16_b<CUR>(lds), 2, wx, wy, lane);
  ld.template store<0, SET>(bf16_a<NXT>(lds), bf16_b<NXT>(lds));
  bf16_mma<1, F, 0, F, Loader::kF16, G>(acc, fr);
  __builtin_amdgcn_sched_group_barrier(0x100, G + F, 0);
  for (int i = 0; i < kMma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);     // conversion arithmetic
  }
  __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);           // LDS writes of the part
  __builtin_amdgcn_sched_barrier(0);
  // step 2: half 1, then the register loads of K-tile kt+1+S into the same set
  bf16_read_frags<1, F, G>(fr, bf16_a<CUR>(lds), bf16_b<CUR>(lds), 3, wx, wy, lane);
  ld.template store<1, SET>(bf16_a<NXT>(lds), bf16_b<NXT>(lds));
  ld.template issue_regs<SET>(kt + 1 + Loader::kSets);
  bf16_mma<0, F, 0, F, Loader::kF16, G>(acc, fr);
  __builtin_amdgcn_sched_group_barrier(0x100, G + F, 0);
  for (int i = 0; i < kMma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);
  __builtin_amdgcn_sched_group_barrier(0x020, Loader::kRegLoads, 0);
  __builtin_amdgcn_sched_barrier(0);
  // step 3
  bf16_mma<1, F, 0, kH, Loader::kF16, G>(acc, fr);
  __builtin_amdgcn_sched_group_barrier(0x008, G * kH, 0);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<Loader::kRegLoads>();           // K-tile kt+1's loads into LDS have landed
  // every wave has written stage NXT and finished reading stage CUR
  lds_barrier();
  bf16_read_frags<0, F, G>(fr, bf16_a<NXT>(lds), bf16_b<NXT>(lds), 0, wx, wy, lane);
  ld.issue_lds(kt + 2, bf16_a<CUR>(lds), bf16_b<CUR>(lds));
  bf16_mma<1, F, kH, F, Loader::kF16, G>(acc, fr);
  __builtin_amdgcn_sched_group_barrier(0x100, G + F, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, G * (F - kH), 0);
  __builtin_amdgcn_sched_barrier(0);
}

// The same K-tile for loaders whose conversion is heavy (Loader::kLateStores): the
// register loads of K-tile kt+S go out in step 0 (S = Loader::kSets register sets),
// the conversion of K-tile kt+1 fills steps 2 and 3, and the barrier closes the
// K-tile.  Converting in steps 1 and 2 instead would leave the heavy arithmetic less
// latency cover for the loads it waits on.
template <int CUR, int F, int G, class Loader>
__device__ __forceinline__ void bf16_ktile_late(v16f (&acc)[F][G], Bf16Frags<F, G>& fr, Loader& ld,
                                                int kt, uint8_t* lds, int wx, int wy, int lane) {
  constexpr int NXT = CUR ^ 1;
  constexpr int kMma = G * F;
  constexpr int kValu = (Loader::kValuPerStore + kMma - 1) / kMma;
  constexpr int SETL = Loader::kSets == 2 ? CUR : 0;           // receives K-tile kt+S
  constexpr int SETC = Loader::kSets == 2 ? NXT : 0;           // holds K-tile kt+1
  // direct loads first: the wait at the end leaves only the register loads in flight
  ld.issue_lds(kt + 1, bf16_a<NXT>(lds), bf16_b<NXT>(lds));
  ld.template issue_regs<SETL>(kt + Loader::kSets);
  bf16_read_frags<1, F, G>(fr, bf16_a<CUR>(lds), bf16_b<CUR>(lds), 1, wx, wy, lane);
  bf16_mma<0, F, 0, F, Loader::kF16, G>(acc, fr);
  __builtin_amdgcn_sched_group_barrier(0x100, G + F, 0);
  for (int i = 0; i < kMma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  bf16_read_frags<0, F, G>(fr, bf16_a<CUR>(lds), bf16_b<CUR>(lds), 2, wx, wy, lane);
  bf16_mma<1, F, 0, F, Loader::kF16, G>(acc, fr);
  __builtin_amdgcn_sched_group_barrier(0x100, G + F, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, kMma, 0);
  __builtin_amdgcn_sched_barrier(0);
  bf16_read_frags<1, F, G>(fr, bf16_a<CUR>(lds), bf16_b<CUR>(lds), 3, wx, wy, lane);
  ld.template store<0, SETC>(bf16_a<NXT>(lds), bf16_b<NXT>(lds));
  bf16_mma<0, F, 0, F, Loader::kF16, G>(acc, fr);
  __builtin_amdgcn_sched_group_barrier(0x100, G + F, 0);
  for (int i = 0; i < kMma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);
  __builtin_amdgcn_sched_barrier(0);
  ld.template store<1, SETC>(bf16_a<NXT>(lds), bf16_b<NXT>(lds));
  bf16_mma<1, F, 0, F, Loader::kF16, G>(acc, fr);
  for (int i = 0; i < kMma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<(Loader::kSets - 1) * Loader::kRegLoads>();     // K-tile kt+S's loads may stay in flight
  lds_barrier();
  bf16_read_frags<0, F, G>(fr, bf16_a<NXT>(lds), bf16_b<NXT>(lds), 0, wx, wy, lane);
}

template <int F, int G, class Loader>
__device__ __forceinline__ void bf16_mainloop(v16f (&acc)[F][G], Loader& ld, int64_t K, uint8_t* lds,
                                              int wx, int wy, int lane) {
  const int nkt = (int)((K + kBf16KT - 1) / kBf16KT);
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[f][g] = v16f{};
  if (nkt == 0) return;
  Bf16Frags<F, G> fr;
  static_assert(Loader::kSets == 1 || Loader::kSets == 2, "one or two register sets");
  if constexpr (Loader::kLateStores) {
    ld.issue_lds(0, bf16_a<0>(lds), bf16_b<0>(lds));
    ld.template issue_regs<0>(0);
    if constexpr (Loader::kSets == 2) ld.template issue_regs<1>(1);
    ld.template store<0, 0>(bf16_a<0>(lds), bf16_b<0>(lds));
    ld.template store<1, 0>(bf16_a<0>(lds), bf16_b<0>(lds));
    wait_vmcnt<(Loader::kSets - 1) * Loader::kRegLoads>();
    lds_barrier();
    bf16_read_frags<0, F, G>(fr, bf16_a<0>(lds), bf16_b<0>(lds), 0, wx, wy, lane);
    int kt = 0;
    for (; kt + 1 < nkt; kt += 2) {
      bf16_ktile_late<0, F, G>(acc, fr, ld, kt, lds, wx, wy, lane);
      bf16_ktile_late<1, F, G>(acc, fr, ld, kt + 1, lds, wx, wy, lane);
    }
    if (kt < nkt) bf16_ktile_late<0, F, G>(acc, fr, ld, kt, lds, wx, wy, lane);
  } else {
    // register set (kt % 2 with two sets) of K-tile kt; K-tile 1 goes into set 1
    // before K-tile 0 is converted, then K-tile S into set 0 (S = kSets)
    ld.issue_lds(0, bf16_a<0>(lds), bf16_b<0>(lds));
    ld.template issue_regs<0>(0);
    if constexpr (Loader::kSets == 2) ld.template issue_regs<1>(1);
    ld.template store<0, 0>(bf16_a<0>(lds), bf16_b<0>(lds));   // waits for the loads issued so far
    ld.template store<1, 0>(bf16_a<0>(lds), bf16_b<0>(lds));
    ld.template issue_regs<0>(Loader::kSets);
    wait_vmcnt<Loader::kRegLoads * Loader::kSets>();
    lds_barrier();
    ld.issue_lds(1, bf16_a<1>(lds), bf16_b<1>(lds));
    bf16_read_frags<0, F, G>(fr, bf16_a<0>(lds), bf16_b<0>(lds), 0, wx, wy, lane);
    // two K-tiles per trip so that the stages (and register sets) are static; reads
    // past K return zeros, which are converted into a stage nobody multiplies
    int kt = 0;
    for (; kt + 1 < nkt; kt += 2) {
      bf16_ktile<0, F, G>(acc, fr, ld, kt, lds, wx, wy, lane);
      bf16_ktile<1, F, G>(acc, fr, ld, kt + 1, lds, wx, wy, lane);
    }
    if (kt < nkt) bf16_ktile<0, F, G>(acc, fr, ld, kt, lds, wx, wy, lane);
  }
  wait_vmem();                               // the loads past K have landed before LDS is reused
}

// compute units of the current device (256 on MI355X)
__host__ inline int bf16_cus() {
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
  }
  return cus;
}

// Output tiles: the 256 x 256 tiles that do not fill a last round over the CUs
// (rem of them) run as two halves of 128 weight rows when that fits: workgroups
// [0, full) take whole tiles, the rest halves (tile full + q/2, half q % 2).
__host__ inline void bf16_tile_split(int tiles, int* full, int* grid) {
  const int cus = bf16_cus();
  const int rem = tiles % cus;
  *full = (rem > 0 && 2 * rem <= cus) ? tiles - rem : tiles;
  *grid = *full + 2 * (tiles - *full);
}

// Byte offset `off` when idx < limit, else an offset past any buffer (top bit set),
// without a branch (idx, limit < 2^31, off < 2^31).
__device__ __forceinline__ uint32_t in_range_or_oob(uint32_t off, uint32_t idx, uint32_t limit) {
  return off | (((limit - 1u - idx) >> 31) << 31);
}

}  // namespace q4
