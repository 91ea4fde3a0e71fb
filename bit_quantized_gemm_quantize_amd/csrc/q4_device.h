// Device-side building blocks shared by the q4lin kernels (gfx950 / CDNA4 only).
//
// MFMA operand layouts used throughout (wave64, verified on the device):
//  * v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands: lane l supplies row l%32
//    of its operand and the 32 consecutive K elements of group l/32 (16 bytes, low
//    nibble first, in the first four dwords of the 8-dword operand), plus one E8M0
//    scale byte for those 32 elements, picked out of a dword by the op_sel index.
//  * v_mfma_f32_32x32x16_bf16: lane l supplies row l%32 and K elements
//    8*(l/32) .. 8*(l/32)+7.
//  * Both write the 32x32 fp32 result so that lane l holds column l%32 and, in
//    register v (0..15), row 8*(v/4) + 4*(l/32) + v%4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFmtFP4 = 4;   // f8f6f4 MFMA operand format code for E2M1

// 2**E as an fp32 value for E in [-127, 127] (2**-127 is an fp32 subnormal).
__device__ __forceinline__ float exp2i(int E) {
  uint32_t bits = (E >= -126) ? (uint32_t)(E + 127) << 23 : 0x00400000u;
  return __uint_as_float(bits);
}

// floor(log2 v) of a positive bf16 magnitude given as its 15-bit pattern.
// Normal: exponent field - 127; subnormal m * 2**-133: floor(log2 m) - 133.
__device__ __forceinline__ int bf16_floor_log2(uint32_t mag) {
  uint32_t e = mag >> 7;
  if (e != 0) return (int)e - 127;
  return (31 - __builtin_clz(mag & 0x7Fu)) - 133;
}

// Largest 15-bit magnitude pattern among the 2*n bf16 values packed in w[0..n).
// For non-negative bf16 patterns the integer order is the value order.
template <int N>
__device__ __forceinline__ uint32_t bf16_amax_bits(const uint32_t* w) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    lo = max(lo, w[i] & 0x7FFFu);
    hi = max(hi, (w[i] >> 16) & 0x7FFFu);
  }
  return max(lo, hi);
}

// MXFP4 shared exponent of a block (OCP MX: floor(log2 amax) - 2, clamped).
__device__ __forceinline__ int mx_block_exponent(uint32_t amax_bits) {
  if (amax_bits == 0) return -127;
  int E = bf16_floor_log2(amax_bits) - 2;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// Encode 8 bf16 values (4 dwords) to one dword of E2M1 codes, dividing by the
// power of two `scale` with the hardware converter (round to nearest even,
// saturating at 6, sign kept).
__device__ __forceinline__ uint32_t fp4_encode8_pow2(const uint32_t* w, float scale) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[0]), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[1]), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[2]), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf, w[3]), scale, 3);
  return r;
}

// bf16 pattern -> fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The FP4 scaled MFMA: four dwords of E2M1 codes per operand.
template <int OPSEL_A, int OPSEL_B>
__device__ __forceinline__ v16f mfma_fp4_32x32x64(u32x4 a, u32x4 b, v16f c, int sa, int sb) {
  v8i A = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  v8i B = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, kFmtFP4, kFmtFP4, OPSEL_A, sa,
                                                          OPSEL_B, sb);
}

__device__ __forceinline__ v16f mfma_bf16_32x32x16(u32x4 a, u32x4 b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                 __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// Two E2M1 codes (byte B of a dword) times an NVFP4 block scale -> a bf16 pair.
// Each product (two significant bits times the four of an E4M3 value) is an exact
// bf16 value, so keeping the upper halves of the fp32 products is exact; one byte
// permute (bytes 2, 3 of lo, then of hi) packs them.
template <int B>
__device__ __forceinline__ uint32_t nv_dequant_pair(uint32_t codes, float s) {
  const v2f v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, B);
  const uint32_t lo = __float_as_uint(v[0] * s), hi = __float_as_uint(v[1] * s);
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// Row index (within the 32x32 MFMA result) of accumulator register v of lane l.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// LDS swizzle.  The gfx950 LDS has 64 banks of 4 bytes: a 16-byte access by 16 lanes
// is served in one pass when the lanes' addresses fall in 16 different 16-byte slots
// of a 256-byte bank row.  A row of C 16-byte chunks (C = 2, 4 or 8) shares its bank
// row with 16 / C - 1 neighbours; storing chunk c of row r at c ^ lds_swz<C>(r) (the
// row's bank-row index modulo C) gives any 16 consecutive rows, read at one logical
// chunk, 16 distinct slots.
template <int C>
__device__ __forceinline__ int lds_swz(int row) {
  static_assert(C == 2 || C == 4 || C == 8, "16-byte chunks per row");
  return (row >> (C == 8 ? 1 : (C == 4 ? 2 : 3))) & (C - 1);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace q4

namespace q4 {

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the 8
// XCDs (each with its own L2), so consecutive tiles are first handed to one XCD
// as a contiguous range, then laid out in groups of `group_m` tile rows so the
// tiles an XCD runs together share operand panels in its L2.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int group_m, int* tm,
                                        int* tn) {
  const int ntiles = tiles_m * tiles_n;
  const int xcd = bid & 7, local = bid >> 3;
  const int q = ntiles >> 3, rem = ntiles & 7;
  const int lid = xcd * q + (xcd < rem ? xcd : rem) + local;
  const int per_group = group_m * tiles_n;
  const int grp = lid / per_group;
  const int first_m = grp * group_m;
  const int gm = min(group_m, tiles_m - first_m);
  const int in = lid - grp * per_group;
  *tm = first_m + in % gm;
  *tn = in / gm;
}

// Work units of a GEMM launch whose leftover tiles (those that do not fill a last
// round over the CUs) run as two halves each: workgroups [0, 2 (tiles - full)) take
// half tiles, the rest whole ones.  Running the halves first puts the CUs that took
// one half a half tile out of step with the others, so the output stores of the two
// sets do not all fall at once.  A whole tile gets the virtual index bid - halves
// for tile_of (whose XCD assignment holds when halves is a multiple of 8).  Half q
// runs on XCD q % 8: when the leftover tiles split evenly over the XCDs, it takes
// one half of a leftover tile that tile_of gives that XCD, so both halves of a tile
// share their activation rows in one L2; else halves q and q+1 split tile full + q/2.
// Returns whether the unit is a half tile (*half: which half).
__device__ __forceinline__ bool tile_unit(int bid, int tiles, int full, int* vt, int* half) {
  const int halves = 2 * (tiles - full);
  if (bid >= halves) {
    *vt = bid - halves;
    *half = 0;
    return false;
  }
  if ((full & 7) == 0 && ((tiles - full) & 7) == 0) {
    const int j = bid >> 3;
    *vt = full + (bid & 7) + 8 * (j >> 1);
    *half = j & 1;
  } else {
    *vt = full + (bid >> 1);
    *half = bid & 1;
  }
  return true;
}

}  // namespace q4

namespace q4 {

// Raw buffer access: loads whose byte offset lies at or beyond `bytes` return 0,
// so tile edges need no branches (an out-of-range chunk gets offset kOOB).
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kBufferFlags = 0x00020000;   // gfx9 buffer resource word 3

// Rows of a tile that lie inside the matrix: total - start clamped to [0, limit]
// (a half tile can start past the last row of a ragged matrix).
__device__ __forceinline__ uint32_t rows_in(int64_t limit, int64_t total, int64_t start) {
  const int64_t r = total - start;
  return (uint32_t)(r < 0 ? 0 : (r > limit ? limit : r));
}

// base and bytes must be the same in every lane; they are moved to scalar registers
// explicitly, since a descriptor the compiler keeps in vector registers turns every
// access through it into a loop over lanes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

}  // namespace q4

namespace q4 {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from a buffer straight into LDS: lane i's bytes land at
// lds_wave_base + 16 i (the base is wave-uniform).  Out-of-range offsets write 0.
__device__ __forceinline__ void buf_ld16_lds(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave_base, 16, (int)off, 0, 0, 0);
}

// Wait until this wave's outstanding vector-memory loads (including loads into
// LDS) have completed: s_waitcnt vmcnt(0), other counters untouched.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace q4

namespace q4 {

// 4 bytes per lane from a buffer straight into LDS (lane i -> lds_wave_base + 4 i).
__device__ __forceinline__ void buf_ld4_lds(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave_base, 4, (int)off, 0, 0, 0);
}

// s_waitcnt vmcnt(N), 0 <= N <= 63 (gfx9 encoding: low 4 bits in [3:0], high 2
// bits in [15:14]), expcnt and lgkmcnt untouched.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

}  // namespace q4

namespace q4 {

// Workgroup barrier ordering LDS accesses only.  __syncthreads() also waits for
// every outstanding global access of the wave (vmcnt(0)), which would drain the
// loads kept in flight several K-tiles ahead; loads into LDS are waited for
// explicitly (wait_vmcnt) before this barrier instead.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier after an explicit wait for loads into LDS.  The compiler counts
// those loads as LDS writes, so lds_barrier() would make it wait for every vector
// memory operation in flight (vmcnt(0)), global stores included.  This one waits
// only for the wave's own LDS accesses; the memory clobber keeps the compiler from
// moving accesses across it.
__device__ __forceinline__ void barrier_after_wait() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace q4

namespace q4 {

// The same loads into LDS written as instructions the compiler does not see as
// LDS writes.  Its automatic waits would otherwise drain every load in flight
// (vmcnt(0)) before any LDS read, since it cannot tell which ring stage a load
// targets; with these, the kernel waits explicitly (wait_vmcnt) for exactly the
// stage it reads next and never reads or reuses a stage a load may still write.
// No register is written by these instructions; M0 carries the wave's LDS base.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_ld16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t off) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :: "v"(off), "s"(base), "s"(r) : "memory", "m0");
}
__device__ __forceinline__ void dma_ld4(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t off) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dword %0, %2, 0 offen lds"
               :: "v"(off), "s"(base), "s"(r) : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace q4

namespace q4 {

// One thread per (row, 32-element block) of a strided bf16 matrix, consecutive
// threads on consecutive blocks of a row (contiguous loads and stores).
//   MXFP8: E = floor(log2 amax) - 8 (emax of E4M3FN) clamped to [-127, 127], codes
//   E4M3_RNE(x * 2**-E) saturated at +-448 (the product is exact in fp32; the clamp
//   comes before the converter, which rounds to nearest even), 32 code bytes, one
//   scale byte E + 127.
//   MXFP4: E = floor(log2 amax) - 2, codes E2M1_RNE(x * 2**-E) by the hardware
//   converter, 16 code bytes, one scale byte.
constexpr int kBlkMXFP4 = 0, kBlkMXFP8 = 2;
template <int KIND>
__device__ __forceinline__ void mx_block(const uint16_t* __restrict__ x, int64_t K, int64_t sr, int64_t sk,
                                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                         int64_t nblk, int64_t q) {
  const int64_t r = q / nblk, b = q % nblk;
  const uint16_t* src = x + r * sr + b * 32 * sk;
  uint32_t w[16];
  if (sk == 1 && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 v = ld16(src + 8 * c);
      w[4 * c] = v[0]; w[4 * c + 1] = v[1]; w[4 * c + 2] = v[2]; w[4 * c + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = (uint32_t)src[2 * j * sk] | ((uint32_t)src[(2 * j + 1) * sk] << 16);
  }
  const uint32_t amax = bf16_amax_bits<16>(w);
  if (KIND == kBlkMXFP4) {
    const int E = mx_block_exponent(amax);
    const float sc = exp2i(E);
    st16(codes + r * (K >> 1) + b * 16, u32x4{fp4_encode8_pow2(w, sc), fp4_encode8_pow2(w + 4, sc),
                                               fp4_encode8_pow2(w + 8, sc), fp4_encode8_pow2(w + 12, sc)});
    scales[r * nblk + b] = (uint8_t)(E + 127);
    return;
  }
  int E = amax == 0 ? -127 : bf16_floor_log2(amax) - 8;
  E = E < -127 ? -127 : (E > 127 ? 127 : E);
  const float down = exp2i(-E);
  uint32_t out[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * d + j;
      const float xv = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
      v[j] = fminf(fmaxf(xv * down, -448.0f), 448.0f);
    }
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
    out[d] = (uint32_t)word;
  }
  uint8_t* dst = codes + r * K + b * 32;
  st16(dst, u32x4{out[0], out[1], out[2], out[3]});
  st16(dst + 16, u32x4{out[4], out[5], out[6], out[7]});
  scales[r * nblk + b] = (uint8_t)(E + 127);
}

}  // namespace q4
