// MXFP4 x MXFP4 GEMM on the CDNA4 block-scaled MFMA with the low-rank branch
// fused in (its bf16 MFMAs seed the accumulators before the K loop) and the bias
// and store in the epilogue.
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves, one per SIMD.  Wave
// (wm, wn) owns m in [128 wm, +128) and n in [128 wn, +128) as 4 x 4 tiles of
// v_mfma_scale_f32_32x32x64_f8f6f4 (FP4 x FP4, one E8M0 scale per 32 K elements
// per row, applied by the MFMA itself); its 256 accumulators per lane live in the
// matrix registers (AGPRs).  A 128 x 128 wave tile reads 0.5 KB of LDS fragments
// per MFMA, against 0.75 KB for 128 x 64.  K advances in tiles of 256 elements
// (128 bytes per row; 8 scale bytes per row).  The wave count is one constant
// (kWaves = 4 or 8; with 8, two per SIMD, a wave owns 128 x 64).
//
// K order inside a K-tile: lane half h (= lane/32) of every fragment owns the
// contiguous blocks 4h .. 4h+3 of the tile, and MFMA step s (0..3) consumes block
// 4h + s from every lane.  A and B use the same assignment, so each MFMA sums
// products of matching K indices; its scale for the step is byte s of the lane's
// 4-byte scale word (the op_sel index), one aligned dword load per fragment.
//
// Tail: when the tiles do not fill the last round over the CUs (864 tiles on 256
// CUs leave 96), the leftover tiles are split in two halves of 128 weight rows,
// so that the extra round is half as long.  The halves are dispatched first (see
// gemm_mx_kernel).
//
// LDS: the two operand tiles (256 rows x 128 bytes each) are stored with 16-byte
// chunks XOR-swizzled by row (chunk c of row r at c ^ lds_swz<8>(r)), so the 16-byte
// fragment reads are free of bank conflicts.  Tiles go from HBM/L2 straight into
// LDS (buffer loads with the LDS destination, no staging registers; rows and
// K blocks past the matrix read as zero).  Two LDS stages, one barrier per K-tile;
// the fragments of the next MFMA step are read from LDS while the current step's
// MFMAs run.
#include <type_traits>

#include "q4_epilogue.h"

namespace q4 {

constexpr int kBM = 256, kBN = 256;
constexpr int kKT = 256;          // K elements per K-tile
constexpr int kKTB = kKT / 2;     // bytes per row per K-tile
constexpr int kWaves = 4;         // one per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupM = 4;
// weight sub-tiles (32 rows each) per wave: whole tiles and half tiles
constexpr int kFFull = 512 / (32 * kWaves), kFHalf = kFFull / 2;

// LDS: (activation, weight) x two stages of tiles of 256 rows x 128 bytes (so the
// stage offset of an operand, 32 KB, folds into the LDS instructions' immediate
// offsets), then two stages x (activation, weight) of scale rows (256 rows x 16
// bytes: the scale bytes of two consecutive K-tiles); the epilogue reuses the space
// for the output
constexpr int kCodeLds = 2 * 2 * kBM * kKTB;          // 131072
constexpr int kScaleLds = 2 * 2 * kBM * 16;           // 16384
constexpr int kMainLds = kCodeLds + kScaleLds;
// epilogue staging rows: 256 bytes wide (one pass for a bf16 tile) with 4 waves and
// bf16 output, else 128
template <bool OUT_F32>
constexpr int mx_stage_row_max() { return kWaves == 4 && !OUT_F32 ? 256 : 128; }
template <bool OUT_F32, int F>
constexpr int mx_stage_wave_bytes() {
  return EpilogueShape<OUT_F32, F, mx_stage_row_max<OUT_F32>()>::kStageWaveBytes;
}
static_assert(kWaves * mx_stage_wave_bytes<true, kFFull>() <= kMainLds &&
                  kWaves * mx_stage_wave_bytes<false, kFFull>() <= kMainLds,
              "the epilogue stages each wave's output in the operand LDS");

// The operand views of one output tile of 256 activation rows x kTN weight rows
// starting at (m0, n0), and the loads into LDS that feed its K loop.
template <int F>
struct MxLoads {
  static constexpr int kTN = 16 * F * kWaves;                   // weight rows of the tile
  static constexpr int kRowsA = kBM / kWaves, kRowsB = kTN / kWaves;   // rows each wave loads
  // codes, global -> LDS: each wave moves 8 rows x 128 bytes per instruction straight
  // into LDS (lane i -> row i/8, stored position i%8, which holds global chunk
  // (i%8) ^ lds_swz<8>(row), the swizzle).  Wave w covers activation rows kRowsA w ..
  // +kRowsA-1 and weight rows kRowsB w .. +kRowsB-1: kNL instructions per K-tile,
  // issued in three parts (instructions [begin(p), begin(p+1))).
  static constexpr int kNA = kRowsA / 8, kNL = kNA + kRowsB / 8;
  static constexpr int kPart0 = kNL / 3, kPart1 = (kNL - kPart0) / 2;
  static constexpr int begin(int p) { return p == 0 ? 0 : p == 1 ? kPart0 : p == 2 ? kPart0 + kPart1 : kNL; }
  static constexpr int kScaleOps = kWaves == 8 ? 1 : 2;        // scale loads per wave per pair

  uint8_t* lds_raw;
  // buffer views of this tile's rows of codes and scales: rows past M / N read as zero
  __amdgpu_buffer_rsrc_t rc_a, rc_b, rs_a, rs_b;
  uint32_t kbytes, nblk, rows_a, rows_b;
  int wave, lane;

  __device__ __forceinline__ MxLoads(uint8_t* lds, const uint8_t* ac, const uint8_t* as,
                                     const uint8_t* bc, const uint8_t* bs, int64_t M, int64_t N,
                                     int64_t K, int64_t m0, int64_t n0)
      : lds_raw(lds) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // opaque: keeps per-tile address math inside the tile loop
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    kbytes = (uint32_t)(K >> 1);
    nblk = (uint32_t)(K >> 5);
    rows_a = rows_in(kBM, M, m0);
    rows_b = rows_in(kTN, N, n0);
    rc_a = make_rsrc(ac + m0 * kbytes, rows_a * kbytes);
    rc_b = make_rsrc(bc + n0 * kbytes, rows_b * kbytes);
    rs_a = make_rsrc(as + m0 * nblk, rows_a * nblk);
    rs_b = make_rsrc(bs + n0 * nblk, rows_b * nblk);
  }

  template <int PART>
  __device__ __forceinline__ void gload(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int kt,
                                        int stage) const {
    auto& lds = *reinterpret_cast<uint8_t(*)[2][2][kBM * kKTB]>(lds_raw);   // [operand][stage]
    const int lr = lane >> 3, lp = lane & 7;
    // row = 16 q + 8 (j % 2) + lr (per * wave is a multiple of 16): its swizzle
    // lds_swz<8>(row) is 4 (j % 2) + lr / 2, so two block offsets serve every row
    uint32_t koff[2];
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const uint32_t blk = (uint32_t)kt * 8 + (lp ^ (4 * jp + (lr >> 1)));
      koff[jp] = blk < nblk ? blk * 16 : kOOB;
    }
#pragma unroll
    for (int idx = begin(PART); idx < begin(PART + 1); ++idx) {
      const int op = idx < kNA ? 0 : 1;
      const int per = op == 0 ? kRowsA : kRowsB;
      const int j = op == 0 ? idx : idx - kNA;
      const uint32_t row = per * wave + 8 * j + lr;
      // koff = kOOB keeps the sum past the buffer size (rows * kbytes < 2^31): no select
      buf_ld16_lds(op == 0 ? ra : rb, &lds[op][stage][(per * wave + 8 * j) * kKTB], row * kbytes + koff[j & 1]);
    }
  }
  template <int PART>
  __device__ __forceinline__ void gload_part(int kt, int stage) const {
    gload<PART>(rc_a, rc_b, kt, stage);
  }
  // Part PART of K-tile kt of this tile, or of K-tile 0 of tile nx when use_next: the
  // tiles have the same shape, so only the buffer views differ (scalar selects).
  template <int PART>
  __device__ __forceinline__ void gload_part_or(const MxLoads& nx, bool use_next, int kt,
                                                int stage) const {
    gload<PART>(use_next ? nx.rc_a : rc_a, use_next ? nx.rc_b : rc_b, use_next ? 0 : kt, stage);
  }

  // scales, global -> LDS, once per pair of K-tiles: 64 rows per instruction (lane i
  // takes row 64 sw + i, 16 bytes = the scale bytes of K-tiles 2p and 2p+1 of pair
  // p) into scale stage p % 2.  With 8 waves, waves 0-3 take the activation rows
  // and waves 4-7 the weight rows; with 4, every wave takes both.
  __device__ __forceinline__ void sload_from(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                             int p) const {
    auto& lsc = *reinterpret_cast<uint8_t(*)[2][2][kBM * 16]>(lds_raw + kCodeLds);
    const int sw = wave & 3;
    const uint32_t b0 = (uint32_t)p * 16;
    const uint32_t koff = b0 < nblk ? b0 : kOOB;
    const uint32_t off = (64 * sw + lane) * nblk + koff;
#pragma unroll
    for (int k = 0; k < kScaleOps; ++k) {
      const int op = kWaves == 8 ? (wave >> 2) : k;
      buf_ld16_lds(op == 0 ? ra : rb, &lsc[p & 1][op][64 * sw * 16], off);
    }
  }
  __device__ __forceinline__ void sload(int p) const { sload_from(rs_a, rs_b, p); }
  // scale pair p of this tile, or pair p - pairs of tile nx when use_next
  __device__ __forceinline__ void sload_or(const MxLoads& nx, bool use_next, int p, int pairs) const {
    sload_from(use_next ? nx.rs_a : rs_a, use_next ? nx.rs_b : rs_b, use_next ? p - pairs : p);
  }

  // The low-rank operands: the tile's t rows and L2^T rows (contiguous in memory), in
  // the second stage of the activation and weight tiles.
  template <int R>
  __device__ __forceinline__ void lowrank_loads(const float* __restrict__ t,
                                                const uint16_t* __restrict__ l2t, int64_t m0,
                                                int64_t n0) const {
    if constexpr (R > 0) {
      auto& lds = *reinterpret_cast<uint8_t(*)[2][2][kBM * kKTB]>(lds_raw);
      const auto rt = make_rsrc(t + m0 * R, rows_a * (uint32_t)(4 * R));
      const auto rl = make_rsrc(l2t + n0 * R, rows_b * (uint32_t)(2 * R));
      uint8_t* lt = &lds[0][1][0];                 // kBM * 4R <= 32 KB
      uint8_t* ll = &lds[1][1][0];                 // kTN * 2R <= 16 KB
      // 1 KB pieces; lane i fills LDS bytes 16 i .. of its piece, which hold the
      // swizzled chunk (lds_swz) of row 16 i / rowbytes
      constexpr int kCT = 4 * R / 16, kCL = 2 * R / 16;   // 16-byte chunks per t / L2^T row
      constexpr int kPiecesT = kBM * 4 * R / 1024;  // kBM * 4R bytes in 1 KB pieces
#pragma unroll
      for (int j = 0; j < kPiecesT / kWaves; ++j) {
        const int piece = wave * (kPiecesT / kWaves) + j;
        const int row = (piece * 64 + lane) / kCT, c = (piece * 64 + lane) % kCT;
        buf_ld16_lds(rt, lt + piece * 1024, row * (4 * R) + ((c ^ lds_swz<kCT>(row)) << 4));
      }
      constexpr int kPieces = kTN * 2 * R / 1024;  // kTN * 2R bytes
#pragma unroll
      for (int j = 0; j < (kPieces + kWaves - 1) / kWaves; ++j) {
        const int piece = j * kWaves + wave;
        const int row = (piece * 64 + lane) / kCL, c = (piece * 64 + lane) % kCL;
        if (piece < kPieces) buf_ld16_lds(rl, ll + piece * 1024, row * (2 * R) + ((c ^ lds_swz<kCL>(row)) << 4));
      }
    }
  }

  // What the tile's K loop needs in LDS before it starts: K-tile 0 (stage 0), the
  // first two scale pairs, and the low-rank operands (stage 1).
  template <int R>
  __device__ __forceinline__ void prologue(int nkt, const float* __restrict__ t,
                                           const uint16_t* __restrict__ l2t, int64_t m0,
                                           int64_t n0) const {
    if (nkt > 0) {
      gload_part<0>(0, 0);
      gload_part<1>(0, 0);
      gload_part<2>(0, 0);
      sload(0);
      sload(1);
    }
    lowrank_loads<R>(t, l2t, m0, n0);
  }
};

// What the epilogue writes: Y (bf16 or fp32), Y as MXFP4 codes and scales for the
// next layer, the SwiGLU of Y's gate and up columns, or Y split into Q, K and V with
// RoPE on Q and K.
constexpr int kOutY = 0, kOutMx = 1, kOutSwiglu = 2, kOutQkv = 3;

// Outputs beyond Y.  kOutMx: codes [M, N/2] and scale bytes [M, N/32] with row
// strides in bytes.  kOutQkv: K and V outputs (Q goes to y), the RoPE table
// (float [M, head_dim/2, 2] of (cos, sin), or null) and the head width.
struct MxQOut {
  uint8_t* qc;
  int64_t ldc;
  uint8_t* qs;
  int64_t lds;
  uint16_t* yk;
  uint16_t* yv;
  const float* cs;
  int head_dim;
};

// Output staging for a tile whose successor's first K-tile already fills stage 0:
// each wave stages 128 rows x 128 bytes at a time in 16 KB of stage 1 (wave w: the
// stage-1 tile of operand w / 2, offset 16 KB (w % 2)), its 16-byte chunks
// XOR-swizzled by row pair (chunk c of row r at c ^ ((r / 2) % 8)): with the 256
// bytes of a bank row holding two 128-byte rows, 16 consecutive rows then cover
// every bank, so neither the transposing writes nor the row reads conflict.  bf16:
// two passes of 64 columns; fp32: four of 32.
template <bool OUT_F32>
struct MxStage1 {
  static constexpr int kElem = OUT_F32 ? 4 : 2;
  static constexpr int kFPerPass = OUT_F32 ? 1 : 2;
  static constexpr int kPasses = kFFull / kFPerPass;
  static constexpr int kCols = 32 * kFPerPass;         // columns per pass
  static constexpr int kReads = 16;                    // 16-byte reads per lane per pass
};
__device__ __forceinline__ uint8_t* mx_stage1_base(uint8_t* lds_raw, int wave) {
  return lds_raw + (2 * (wave >> 1) + 1) * (kBM * kKTB) + (wave & 1) * 16384;
}
template <bool OUT_F32, bool BIAS>
__device__ __forceinline__ void mx_stage1_write(v16f (&acc)[kFFull][4], int pass, int64_t n_base,
                                                int64_t N, const uint16_t* __restrict__ bias,
                                                int lane, uint8_t* stage) {
  using S = MxStage1<OUT_F32>;
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int fp = 0; fp < S::kFPerPass; ++fp) {
    const int f = pass * S::kFPerPass + fp;
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) {
      const int64_t n = n_base + 32 * f + 8 * vq + 4 * h;
      float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (BIAS && bias != nullptr) {           // the edge path adds zeros without a bias
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n + j < N) b[j] = __uint_as_float((uint32_t)bias[n + j] << 16);
      }
      const int col_byte = (32 * fp + 8 * vq + 4 * h) * S::kElem;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = 32 * g + r32;
        uint8_t* dst = stage + row * 128 + ((((col_byte >> 4) ^ (row >> 1)) & 7) << 4) + (col_byte & 15);
        float a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = BIAS ? acc[f][g][4 * vq + j] + b[j] : acc[f][g][4 * vq + j];
        if (OUT_F32) {
          *reinterpret_cast<v4f*>(dst) = v4f{a[0], a[1], a[2], a[3]};
        } else {
          const v2bf p0 = {(__bf16)a[0], (__bf16)a[1]};
          const v2bf p1 = {(__bf16)a[2], (__bf16)a[3]};
          typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
          *reinterpret_cast<u32x2*>(dst) =
              u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
        }
      }
    }
  }
}
// read i of a pass: row 8 i + lane / 8, logical chunk lane % 8
__device__ __forceinline__ u32x4 mx_stage1_read(const uint8_t* stage, int i, int lane) {
  const int row = 8 * i + (lane >> 3), c = lane & 7;
  return ld16(stage + row * 128 + (((c ^ (row >> 1)) & 7) << 4));
}

// SwiGLU of a tile's accumulators (kOutSwiglu).  Weight rows come in groups of 64:
// the first 32 are the gate and the last 32 the up projection of output columns
// 32 j .. 32 j + 31 of group j.  A wave's weight sub-tiles (32 rows each, F of them)
// are F/2 whole groups, so acc[2p] (gate) and acc[2p + 1] (up) hold the same
// outputs.  With each weight row's bias added first, y = gate / (1 + exp(-gate)) * up
// in fp32, the division taken as a product with the hardware reciprocal (within an
// ulp; an IEEE division is about ten instructions per element, and this epilogue
// runs after the K loop with nothing to hide them under), stored as bf16 [M, N/2]
// through the standard staging.
template <int F>
__device__ __forceinline__ void epilogue_store_swiglu(v16f (&acc)[F][4], int64_t n_base, int64_t m_base,
                                                      int64_t M, int64_t N, const uint16_t* __restrict__ bias,
                                                      uint16_t* y, int64_t ldy, int lane, uint8_t* stage) {
  constexpr int P = F / 2;
  const int h = lane >> 5;
  v16f v[P][4];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int vq = 0; vq < 4; ++vq)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t n = n_base + 64 * p + 8 * vq + 4 * h + jj;    // gate row; up row n + 32
        float bg = 0.0f, bu = 0.0f;
        if (bias != nullptr && n + 32 < N) {
          bg = __uint_as_float((uint32_t)bias[n] << 16);
          bu = __uint_as_float((uint32_t)bias[n + 32] << 16);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float gate = acc[2 * p][g][4 * vq + jj] + bg;
          const float up = acc[2 * p + 1][g][4 * vq + jj] + bu;
          v[p][g][4 * vq + jj] = gate * __builtin_amdgcn_rcpf(1.0f + __expf(-gate)) * up;
        }
      }
  epilogue_store<false, P, 128>(v, n_base / 2, m_base, M, N / 2, nullptr, y, ldy, lane, stage);
}

// QKV split and RoPE of a tile (kOutQkv).  N = 3 D with D a multiple of 128, so a
// wave's columns lie in one section: Q [0, D), K [D, 2 D) or V.  Each section goes to
// its own output [M, D] (bf16).  V, or everything without a table, takes the
// standard bf16 staging.  Q and K are staged in fp32 with the bias added (32 columns
// per pass), and each lane's 32-byte read-back (four adjacent column pairs of a row)
// is rotated by that row's (cos, sin) of the pairs' indices inside the head,
// (a, b) -> (a c - b s, a s + b c), in fp32 before the one rounding to bf16, and
// stored as 16 bytes.
template <int F>
__device__ __forceinline__ void epilogue_store_qkv(v16f (&acc)[F][4], int64_t n_base, int64_t m_base,
                                                   int64_t M, int64_t N, const uint16_t* __restrict__ bias,
                                                   uint16_t* yq, int64_t ldy, int lane, uint8_t* stage,
                                                   const MxQOut& qo) {
  if (n_base >= N) return;                               // wave-uniform: past the last column
  const int64_t D = N / 3;
  const int sec = (int)(n_base / D);
  const int64_t col0 = n_base - sec * D;
  const uint16_t* bsec = bias != nullptr ? bias + sec * D : nullptr;
  uint16_t* dst = sec == 0 ? yq : (sec == 1 ? qo.yk : qo.yv);
  if (sec == 2 || qo.cs == nullptr) {
    epilogue_store<false, F, mx_stage_row_max<false>()>(acc, col0, m_base, M, D, bsec, dst, ldy, lane, stage);
    return;
  }
  using S = EpilogueShape<true, F, 128>;
  static_assert(S::kFPerPass == 1, "one 32-column sub-tile per fp32 pass");
  const int hd = qo.head_dim;
  const int cl = lane & 3;                               // 32-byte chunk: columns 8 cl .. 8 cl + 7
  // the table rows of this wave's 128 rows, through a buffer whose bound returns
  // zeros for rows past M (their outputs are not stored); lane row ml = 16 it +
  // lane / 4 sits at byte 4 hd ml, pair i of it at + 8 i
  const auto rcs = make_rsrc(qo.cs + m_base * hd, rows_in(128, M, m_base) * (uint32_t)hd * 4u);
  const uint32_t row_off = (uint32_t)(lane >> 2) * (uint32_t)hd * 4u;
  const uint32_t colm = (uint32_t)(col0 % hd);
  // byte offsets of the lane's four pairs in a pass: pair index ((col + 2 q) mod hd) / 2
  auto pair_offs = [&](int pass, uint32_t (&off)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      off[q] = row_off + (((colm + 32u * pass + 8u * cl + 2u * q) % (uint32_t)hd) >> 1) * 8u;
  };
  auto load_pair = [&](uint32_t off, int it) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rcs, (int)off, 64 * hd * it, 0));
  };
  float2 tcs[8][4];
  {
    uint32_t off[4];
    pair_offs(0, off);
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
      for (int q = 0; q < 4; ++q) tcs[it][q] = load_pair(off[q], it);
  }
#pragma unroll
  for (int pass = 0; pass < S::kPasses; ++pass) {
    const int64_t col = col0 + 32 * pass + 8 * cl;       // pairs (col + 2 q, col + 2 q + 1), q < 4
    // a wave's LDS accesses take effect in order: the writes of a pass need no wait
    // for the reads of the previous one, nor the reads for the writes
    if (pass > 0) __builtin_amdgcn_wave_barrier();
    epilogue_stage_pass<true, F, 128, false, true>(acc, pass, col0, D, bsec, lane, stage, 1.0f);
    __builtin_amdgcn_wave_barrier();
    // the next pass's table pairs are loaded into each row's registers as soon as
    // this pass has used them, so their latency hides behind this pass's stores and
    // the next pass's staging
    uint32_t offn[4];
    pair_offs(pass + 1, offn);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int ml = 16 * it + (lane >> 2);
      const int64_t m = m_base + ml;
      const uint8_t* src = stage + ml * S::kStageRowBytes + cl * 32;
      const v4f va = *reinterpret_cast<const v4f*>(src), vb = *reinterpret_cast<const v4f*>(src + 16);
      const float v[8] = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float2 t = tcs[it][q];
        const v2bf p = {(__bf16)(v[2 * q] * t.x - v[2 * q + 1] * t.y),
                        (__bf16)(v[2 * q] * t.y + v[2 * q + 1] * t.x)};
        w[q] = __builtin_bit_cast(uint32_t, p);
      }
      if (pass + 1 < S::kPasses) {
#pragma unroll
        for (int q = 0; q < 4; ++q) tcs[it][q] = load_pair(offn[q], it);
      }
      if (m < M) st16_stream(dst + m * ldy + col, u32x4{w[0], w[1], w[2], w[3]});
    }
  }
}

// One output tile of 256 activation rows x kTN weight rows starting at (m0, n0),
// whose prologue loads (MxLoads::prologue) are already issued: wave (wm, wn) owns m
// in [128 wm, +128) and n in [32 F wn, +32 F).  `pending` is the number of this
// wave's stores from the previous tile still queued behind those loads.  next_kind
// says what follows (0 nothing, 1 a whole tile at (nm0, nn0), 2 a half tile).  A
// whole tile followed by a whole tile is chained when K is a multiple of 4 K-tiles:
// its last K-tiles load the next tile's first K-tile and scale pairs in place of
// the loads past K, so only the low-rank operands remain for the next prologue.
// Once the tile's LDS is free again, issue_next(chained) queues what remains of the
// next tile's prologue; the return value is the number of stores queued after it.
template <int R, bool OUT_F32, int OUTM, int F, class Next>
__device__ __forceinline__ int mx_tile(
    uint8_t* lds_raw, const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, int64_t M, int64_t N, int64_t K,
    const uint16_t* __restrict__ bias, void* __restrict__ y, int64_t ldy, int64_t m0, int64_t n0,
    int pending, int next_kind, int64_t nm0, int64_t nn0, const MxQOut& qo, Next&& issue_next) {
  using L = MxLoads<F>;
  constexpr int kMma = 4 * F;                    // MFMAs per wave per step
  auto& lds = *reinterpret_cast<uint8_t(*)[2][2][kBM * kKTB]>(lds_raw);   // [operand][stage]
  auto& lsc = *reinterpret_cast<uint8_t(*)[2][2][kBM * 16]>(lds_raw + kCodeLds);
  const L ld(lds_raw, ac, as, bc, bs, M, N, K, m0, n0);

  // opaque thread index: the compiler would otherwise hoist the tile's address math
  // out of the persistent loop, for both tile shapes, and run out of registers
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1, wm = wave & 1;       // wave's n quarter, m half
  const int r32 = lane & 31, h = lane >> 5;
  const uint32_t nblk = (uint32_t)(K >> 5);
  const int nkt = (int)((K + kKT - 1) / kKT);
  constexpr int kPartBegin[4] = {L::begin(0), L::begin(1), L::begin(2), L::begin(3)};
  constexpr int kScaleOps = L::kScaleOps;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  const bool chain = OUTM == kOutY && F == kFFull && next_kind == 1 && (nkt & 3) == 0 && nkt >= 4;
  const L nx(lds_raw, ac, as, bc, bs, M, N, K, chain ? nm0 : m0, chain ? nn0 : n0);
  const int pairs = nkt >> 1;
  auto gload_part = [&](auto part_c, int kt, int stage) {
    ld.template gload_part<decltype(part_c)::value>(kt, stage);
  };
  // in a chained tile, K-tile nkt is the next tile's K-tile 0 and scale pairs
  // pairs, pairs + 1 are the next tile's pairs 0 and 1
  auto gload_part_or_next = [&](auto part_c, int kt, int stage) {
    ld.template gload_part_or<decltype(part_c)::value>(nx, chain && kt == nkt, kt, stage);
  };
  auto sload_or_next = [&](int p) { ld.sload_or(nx, chain && p >= pairs, p, pairs); };
  // the lane's scale word for K-tile kt: bytes for blocks 8kt + 4h .. 8kt + 4h + 3,
  // at byte 8 (kt % 2) + 4h of the row's 16 bytes in scale stage (kt / 2) % 2.
  // Read raw; valid_scales() replaces the words of blocks past K (whose codes are
  // zero) by 2**0, so that bytes beyond the row's last block never reach the MFMA.
  uint32_t sa[4], sb[F], sa_n[4], sb_n[F];
  auto read_scales = [&](int kt) {
    const int stage = (kt >> 1) & 1, byte = 8 * (kt & 1) + 4 * h;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      sa_n[g] = *reinterpret_cast<const uint32_t*>(&lsc[stage][0][(wm * 128 + 32 * g + r32) * 16 + byte]);
#pragma unroll
    for (int f = 0; f < F; ++f)
      sb_n[f] = *reinterpret_cast<const uint32_t*>(&lsc[stage][1][(wn * 32 * F + 32 * f + r32) * 16 + byte]);
  };
  auto valid_scales = [&](int kt) {
    const bool kin = (uint32_t)kt * 8 + 4 * h < nblk;
#pragma unroll
    for (int g = 0; g < 4; ++g) sa[g] = kin ? sa_n[g] : 0x7F7F7F7Fu;
#pragma unroll
    for (int f = 0; f < F; ++f) sb[f] = kin ? sb_n[f] : 0x7F7F7F7Fu;
  };

  // fragment registers, double-buffered across MFMA steps
  u32x4 fa[2][4], fb[2][F];
  auto read_frags = [&](int buf, int stage, int s) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row = wm * 128 + 32 * g + r32;
      fa[buf][g] = ld16(&lds[0][stage][row * kKTB + (((4 * h + s) ^ lds_swz<8>(row)) << 4)]);
    }
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int row = wn * 32 * F + 32 * f + r32;
      fb[buf][f] = ld16(&lds[1][stage][row * kKTB + (((4 * h + s) ^ lds_swz<8>(row)) << 4)]);
    }
  };

  v16f acc[F][4];

#define Q4_MX_MMA(S, BUF) Q4_MX_MMA_F(S, BUF, 0, F)
#define Q4_MX_MMA_F(S, BUF, F0, F1)                                                             \
  _Pragma("unroll") for (int f = F0; f < F1; ++f)                                               \
    _Pragma("unroll") for (int g = 0; g < 4; ++g)                                               \
      acc[f][g] = mfma_fp4_32x32x64<S, S>(fb[BUF][f], fa[BUF][g], acc[f][g], (int)sb[f],       \
                                          (int)sa[g]);
// within a region: the LDS reads for the next step go out first, then the MFMAs
#define Q4_READS_THEN_MMA(NREADS)                          \
  __builtin_amdgcn_sched_group_barrier(0x100, NREADS, 0); \
  __builtin_amdgcn_sched_group_barrier(0x008, kMma, 0);

  const int64_t n_base = n0 + wn * 32 * F, m_base = m0 + wm * 128;
  // Pipeline: the loads of K-tile kt+1 go out from the barrier of K-tile kt-1 (part
  // 0, once that barrier has freed the stage) through steps 0 and 1 of K-tile kt
  // (parts 1 and 2), and are waited for at the barrier inside step 3 of K-tile kt:
  // nearly a whole K-tile of latency cover.  Scale pair q is loaded with part 0 of
  // K-tile 2q-1, and read (for K-tile 2q) in step 1 of K-tile 2q-1.
  //
  // The prologue loads were queued before the previous tile's stores, and vector
  // memory operations complete in order: waiting until only those stores are
  // outstanding waits for the loads alone.
  if (pending == RegEpilogue<kFFull>::kStores) wait_vmcnt<RegEpilogue<kFFull>::kStores>();
  else if (pending == RegEpilogue<kFHalf>::kStores) wait_vmcnt<RegEpilogue<kFHalf>::kStores>();
  else wait_vmem();
  barrier_after_wait();
  // cleared only here, after the wait: clearing at the tile's start made that tile
  // slower
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = v16f{};
  // The low-rank term t L2 goes into the accumulators first (its operands came
  // with the prologue), so the epilogue is left with the bias and the store.
  if constexpr (R > 0) {
    lowrank_accumulate_lds<R>(acc, &lds[0][1][0], &lds[1][1][0], 128 * wm, 32 * F * wn, lane);
    // stage 1 is free again for K-tile 1.  The prologue loads were waited for above;
    // a fenced barrier would also wait for the previous tile's stores.
    barrier_after_wait();
  }
  if (nkt > 0) {
    gload_part(P0{}, 1, 1);
    read_frags(0, 0, 0);
    read_scales(0);
    valid_scales(0);
  }

  // The loop body is one basic block (no branches), so the sched barriers pin the
  // order: each MFMA step runs with the next step's fragment reads in flight, and
  // the loads are slotted between MFMAs (issuing them in a burst would hold the
  // in-order MFMA stream behind them).  The scales of tile kt+1 are read in step 1,
  // from a stage that an earlier barrier made visible.  The barrier sits in the
  // middle of step 3, whose MFMAs need no LDS: the first half covers the wait, the
  // second the fragment reads of the next tile.  Loads past K read zeros.
  constexpr int kF3 = F / 2;                 // weight sub-tiles of step 3 before the barrier
  auto ktile = [&](auto stage_c, int kt) {
    constexpr int st = decltype(stage_c)::value;
    constexpr int vm0 = kPartBegin[2] - kPartBegin[1], vm1 = kPartBegin[3] - kPartBegin[2];
    constexpr int vm3 = kPartBegin[1] + (st == 1 ? kScaleOps : 0);
    read_frags(1, st, 1);
    gload_part_or_next(P1{}, kt + 1, st ^ 1);
    Q4_MX_MMA(0, 0)
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + F, 0);
    for (int i = 0; i < kMma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < vm0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    read_scales(kt + 1);
    read_frags(0, st, 2);
    gload_part_or_next(P2{}, kt + 1, st ^ 1);
    Q4_MX_MMA(1, 1)
    __builtin_amdgcn_sched_group_barrier(0x100, 8 + 2 * F, 0);
    for (int i = 0; i < kMma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < vm1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    read_frags(1, st, 3);
    Q4_MX_MMA(2, 0)
    Q4_READS_THEN_MMA(4 + F)
    __builtin_amdgcn_sched_barrier(0);
    Q4_MX_MMA_F(3, 1, 0, kF3)
    if (kF3 > 0) __builtin_amdgcn_sched_group_barrier(0x008, 4 * kF3, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmem();
    // every wave's tile kt+1 has landed, and every read of tile kt has completed:
    // stage st is free for tile kt+2
    __syncthreads();
    read_frags(0, st ^ 1, 0);
    gload_part_or_next(P0{}, kt + 2, st);
    if (st == 1) sload_or_next((kt + 3) >> 1);         // kt odd: pair (kt+3)/2
    Q4_MX_MMA_F(3, 1, kF3, F)
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + F, 0);
    for (int i = 0; i < 4 * (F - kF3); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < vm3) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    valid_scales(kt + 1);
  };
  // two K-tiles per trip, so that the stages (and the LDS addresses) are static
  int kt = 0;
  for (; kt + 1 < nkt; kt += 2) {
    ktile(std::integral_constant<int, 0>{}, kt);
    ktile(std::integral_constant<int, 1>{}, kt + 1);
  }
  if (kt < nkt) ktile(std::integral_constant<int, 0>{}, kt);
#undef Q4_MX_MMA
#undef Q4_MX_MMA_F
#undef Q4_READS_THEN_MMA

  if constexpr (F == kFFull) {
   if (chain) {
    // The last loads of the K loop are the next tile's scale pair 1 (into a scale
    // stage): wait for everything before them (the zero loads past K into stage 1)
    // but not for them.
    wait_vmcnt<L::kScaleOps>();
    barrier_after_wait();                    // all waves are done with the operand LDS
    // stage 0 and the scale stages hold the next tile's first K-tile and scale pairs:
    // stage in stage 1 only
    using S = MxStage1<OUT_F32>;
    uint8_t* stage = mx_stage1_base(lds_raw, wave);
    auto& accf = acc;
    if (!OUT_F32 && m_base + 128 <= M && n_base + 128 <= N) {
      // inside the output, bf16: both passes into registers, then the next tile's
      // low-rank loads, then the stores
      u32x4 out[S::kPasses * S::kReads];
#pragma unroll
      for (int pass = 0; pass < S::kPasses; ++pass) {
        // a wave's LDS accesses take effect in order: no wait between the writes, the
        // reads and the next pass's writes
        if (bias) mx_stage1_write<OUT_F32, true>(accf, pass, n_base, N, bias, lane, stage);
        else mx_stage1_write<OUT_F32, false>(accf, pass, n_base, N, bias, lane, stage);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < S::kReads; ++i) out[pass * S::kReads + i] = mx_stage1_read(stage, i, lane);
        __builtin_amdgcn_wave_barrier();
      }
      // the next tile's scale pair 1 may still be landing in a scale stage: a
      // fenced barrier would wait for it
      barrier_after_wait();
      issue_next(true);
      uint16_t* dst = static_cast<uint16_t*>(y) + (m_base + (lane >> 3)) * ldy + n_base + (lane & 7) * 8;
#pragma unroll
      for (int pass = 0; pass < S::kPasses; ++pass)
#pragma unroll
        for (int i = 0; i < S::kReads; ++i)
          st16_stream(dst + (int64_t)8 * i * ldy + pass * S::kCols, out[pass * S::kReads + i]);
      return S::kPasses * S::kReads;
    }
    // edges or fp32: each pass stored as it is read back, with the M and N masks
    constexpr int kPer16 = 16 / S::kElem;
#pragma unroll
    for (int pass = 0; pass < S::kPasses; ++pass) {
      // one path with the bias read guarded (a second copy costs registers)
      mx_stage1_write<OUT_F32, true>(accf, pass, n_base, N, bias, lane, stage);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
      const int64_t n = n_base + pass * S::kCols + (lane & 7) * kPer16;
#pragma unroll 4
      for (int i = 0; i < S::kReads; ++i) {
        const u32x4 v = mx_stage1_read(stage, i, lane);
        const int64_t m = m_base + 8 * i + (lane >> 3);
        if (m < M) {
          uint8_t* dst = static_cast<uint8_t*>(y) + (m * ldy + n) * S::kElem;
          if (n + kPer16 <= N) {
            st16_stream(dst, v);
          } else if (n < N) {
            const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
            for (int j = 0; j < kPer16 && n + j < N; ++j) {
              if (OUT_F32) reinterpret_cast<uint32_t*>(dst)[j] = w[j];
              else reinterpret_cast<uint16_t*>(dst)[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
            }
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
    }
    barrier_after_wait();
    issue_next(true);
    return 0;
   }
  }
  wait_vmem();                               // the loads past K have landed
  __syncthreads();                           // all waves are done with the operand LDS
  uint8_t* stage = lds_raw + wave * mx_stage_wave_bytes<OUT_F32, F>();
  if constexpr (OUTM == kOutMx) {
    epilogue_store_mxfp4<F>(acc, n_base, m_base, M, N, bias, static_cast<uint16_t*>(y), ldy, qo.qc,
                            qo.ldc, qo.qs, qo.lds, lane, stage);
    lds_barrier();
    issue_next(false);
    return 0;
  }
  if constexpr (OUTM == kOutSwiglu) {
    epilogue_store_swiglu<F>(acc, n_base, m_base, M, N, bias, static_cast<uint16_t*>(y), ldy, lane, stage);
    lds_barrier();
    issue_next(false);
    return 0;
  }
  if constexpr (OUTM == kOutQkv) {
    epilogue_store_qkv<F>(acc, n_base, m_base, M, N, bias, static_cast<uint16_t*>(y), ldy, lane, stage, qo);
    lds_barrier();
    issue_next(false);
    return 0;
  }
  // A wave region inside the output, bf16: staged into registers, so that the LDS is
  // free for the next tile's loads before the stores go out.  Otherwise (edges, fp32)
  // staged and stored pass by pass.
  const bool regs = !OUT_F32 && m_base + 128 <= M && n_base + 32 * F <= N;
  u32x4 out[RegEpilogue<F>::kStores];
  if (regs) epilogue_stage_to_regs<F>(acc, n_base, N, bias, lane, stage, out);
  else epilogue_store<OUT_F32, F, mx_stage_row_max<OUT_F32>()>(acc, n_base, m_base, M, N, bias, y, ldy,
                                                               lane, stage);
  lds_barrier();
  issue_next(false);
  if (!regs) return 0;
  epilogue_store_regs<F>(out, n_base, m_base, y, ldy, lane);
  return RegEpilogue<F>::kStores;
}

// Work unit u -> its tile: whole tiles, and halves (weight rows 128 h .. +127) of
// the leftover ones (see tile_unit).  False for a half past the last weight row.
__device__ __forceinline__ bool mx_unit(int u, int tiles_m, int tiles_n, int full, int64_t N,
                                        bool* is_half, int64_t* m0, int64_t* n0) {
  int vt, half, tm, tn;
  *is_half = tile_unit(u, tiles_m * tiles_n, full, &vt, &half);
  tile_of(vt, tiles_m, tiles_n, kGroupM, &tm, &tn);
  *m0 = (int64_t)tm * kBM;
  *n0 = (int64_t)tn * kBN + (*is_half ? 128 * half : 0);
  return *n0 < N;
}

// Persistent: workgroup b runs units b, b + G, b + 2G, ... (G = the grid), so unit u
// still runs on XCD u % 8 when G is a multiple of 8.  Each tile queues the next
// one's first loads as soon as its output is staged, ahead of its own stores, so
// the stores drain while the next tile starts.
template <int R, bool OUT_F32, int OUTM>
__global__ __launch_bounds__(kThreads) void gemm_mx_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const uint8_t* __restrict__ bc,
    const uint8_t* __restrict__ bs, int64_t M, int64_t N, int64_t K, const float* __restrict__ t,
    const uint16_t* __restrict__ l2t, const uint16_t* __restrict__ bias, void* __restrict__ y,
    int64_t ldy, int tiles_m, int tiles_n, int full, int units, MxQOut qo) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kMainLds];
  const int nkt = (int)((K + kKT - 1) / kKT);
  const int step = gridDim.x;
  auto find = [&](int v, bool* h, int64_t* mm, int64_t* nn) {
    while (v < units && !mx_unit(v, tiles_m, tiles_n, full, N, h, mm, nn)) v += step;
    return v;
  };
  auto prologue = [&](bool h, int64_t mm, int64_t nn) {
    if (h) MxLoads<kFHalf>(lds_raw, ac, as, bc, bs, M, N, K, mm, nn).template prologue<R>(nkt, t, l2t, mm, nn);
    else MxLoads<kFFull>(lds_raw, ac, as, bc, bs, M, N, K, mm, nn).template prologue<R>(nkt, t, l2t, mm, nn);
  };
  bool half;
  int64_t m0, n0;
  int u = find(blockIdx.x, &half, &m0, &n0);
  if (u >= units) return;
  prologue(half, m0, n0);
  int pending = 0;
  while (u < units) {
    bool nh = false;
    int64_t nm = 0, nn = 0;
    const int nu = find(u + step, &nh, &nm, &nn);
    const int next_kind = nu >= units ? 0 : (nh ? 2 : 1);
    // chained: only the low-rank operands are left to load
    auto issue_next = [&](bool chained) {
      if (nu >= units) return;
      if (chained) MxLoads<kFFull>(lds_raw, ac, as, bc, bs, M, N, K, nm, nn).template lowrank_loads<R>(t, l2t, nm, nn);
      else prologue(nh, nm, nn);
    };
    if (half)
      pending = mx_tile<R, OUT_F32, OUTM, kFHalf>(lds_raw, ac, as, bc, bs, M, N, K, bias, y, ldy, m0,
                                                 n0, pending, next_kind, nm, nn, qo, issue_next);
    else
      pending = mx_tile<R, OUT_F32, OUTM, kFFull>(lds_raw, ac, as, bc, bs, M, N, K, bias, y, ldy, m0,
                                                 n0, pending, next_kind, nm, nn, qo, issue_next);
    u = nu;
    half = nh;
    m0 = nm;
    n0 = nn;
  }
}

template <int R, bool F32, int OUTM = kOutY>
static void queue(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                  int64_t M, int64_t N, int64_t K, const EpilogueArgs& ep, hipStream_t s) {
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  const int tiles = tiles_m * tiles_n;
  // leftover tiles of the last round over the CUs run as halves when that fits
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
  }
  const int rem = tiles % cus;
  const int full = (tiles > cus && rem > 0 && 2 * rem <= cus) ? tiles - rem : tiles;
  const int units = full + 2 * (tiles - full);
  // one workgroup per CU (the LDS allows no more), each looping over its units
  const int grid = units < cus ? units : cus;
  hipLaunchKernelGGL((gemm_mx_kernel<R, F32, OUTM>), dim3(grid), dim3(kThreads), 0, s, ac, as, bc, bs, M,
                     N, K, ep.t, ep.l2t, ep.bias, ep.y, ep.ldy, tiles_m, tiles_n, full, units,
                     MxQOut{ep.qc, ep.ldc, ep.qs, ep.lds, ep.yk, ep.yv, ep.cs, ep.head_dim});
}

hipError_t launch_gemm_mx(const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K,
                          const EpilogueArgs& ep, hipStream_t s) {
  if (ep.qkv) {
    if (ep.r == 0) queue<0, false, kOutQkv>(ac, as, bc, bs, M, N, K, ep, s);
    else if (ep.r == 16) queue<16, false, kOutQkv>(ac, as, bc, bs, M, N, K, ep, s);
    else queue<32, false, kOutQkv>(ac, as, bc, bs, M, N, K, ep, s);
  } else if (ep.swiglu) {
    if (ep.r == 0) queue<0, false, kOutSwiglu>(ac, as, bc, bs, M, N, K, ep, s);
    else if (ep.r == 16) queue<16, false, kOutSwiglu>(ac, as, bc, bs, M, N, K, ep, s);
    else queue<32, false, kOutSwiglu>(ac, as, bc, bs, M, N, K, ep, s);
  } else if (ep.qc != nullptr) {
    if (ep.r == 0) queue<0, false, kOutMx>(ac, as, bc, bs, M, N, K, ep, s);
    else if (ep.r == 16) queue<16, false, kOutMx>(ac, as, bc, bs, M, N, K, ep, s);
    else queue<32, false, kOutMx>(ac, as, bc, bs, M, N, K, ep, s);
  } else if (ep.out_f32) {
    if (ep.r == 0) queue<0, true>(ac, as, bc, bs, M, N, K, ep, s);
    else if (ep.r == 16) queue<16, true>(ac, as, bc, bs, M, N, K, ep, s);
    else queue<32, true>(ac, as, bc, bs, M, N, K, ep, s);
  } else {
    if (ep.r == 0) queue<0, false>(ac, as, bc, bs, M, N, K, ep, s);
    else if (ep.r == 16) queue<16, false>(ac, as, bc, bs, M, N, K, ep, s);
    else queue<32, false>(ac, as, bc, bs, M, N, K, ep, s);
  }
  return hipGetLastError();
}

}  // namespace q4
