// bf16 GEMM for gfx950: C[M,N] = epilogue(A B), bf16 operands on the
// v_mfma_f32_16x16x32_bf16 matrix cores, float32 accumulate, for the three
// operand layouts the MLP shard's forward and backward use (kNN, kNT, kTN).
//
// Workgroup tile BM x BN, WM x WN waves, each wave a (BM/WM) x (BN/WN) block
// of 16x16 MFMA tiles.  K advances 32 per stage (one MFMA deep) through NBUF
// LDS stages with a prefetch distance of NBUF - 1.  Global data goes straight into LDS with
// `buffer_load_dwordx4 ... lds` (lane l of a wave instruction fills bytes
// 16 l .. 16 l + 15 of a 1 KB LDS block, so the LDS swizzle is applied by
// choosing which global 16-byte chunk each lane fetches): no staging
// registers and no LDS store instructions.
//
// Each operand tile is stored in LDS in its global orientation:
//   K-major operand (A in kNN/kNT, B in kNT): [R rows][32 k], 64-byte rows;
//     chunk c (8 k-values) of row r at position c ^ swzK(r).  An MFMA
//     fragment (16 rows by 32 k; each lane 8 consecutive k of one row) is one
//     16-byte LDS read per lane.
//   MN-major operand (B in kNN/kTN, A in kTN): [32 k][R], 2R-byte rows;
//     chunk c (8 row/column indices) of k-row k at position c ^ swzMN(k).  A
//     fragment is two ds_read_b64_tr_b16 transpose reads.
// Both swizzles make the DMA writes and the fragment reads free of LDS bank
// conflicts.
//
// Edges.  Every 16-byte chunk of global memory is either wholly inside or
// wholly outside the matrix (contiguous dimensions are multiples of 8).  A
// lane whose chunk lies outside (rows past M or N, k past K) is given an
// out-of-range buffer offset and the DMA writes zeros, so partial tiles need
// no branches in the K loop; the epilogue skips stores outside C.
//
// MFMA operand order: the B-fragment goes in the instruction's A slot and the
// A-fragment in its B slot, so the instruction computes the transposed tile
// and each lane ends up owning runs of 4 consecutive output columns of one
// row (16-byte fp32 / 8-byte bf16 stores).
//
// One barrier per stage, placed before the MFMAs of the second half of the
// wave's rows, so the next stage's first fragment reads overlap those MFMAs.
// (The 16x16x32 instruction gives the same float32 results as two
// 32x32x16 steps over the same 32 k, bit for bit, measured on every output of
// the MLP's GEMM shapes; it runs at a ~10% higher clock under the power cap.)
// The barrier is a bare s_barrier after an explicit wait for this wave's loads
// of the next stage only (a full workgroup fence would also wait for the
// loads of the stages still in flight).
#pragma once

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "tp_mlp_kernels.h"

namespace tpmlp {

// Per-group operands of a batch of same-shaped GEMMs (the per-shard GEMMs of
// one step launched together); entries may repeat (the shared X).
struct GroupTable {
  const uint16_t* A[kMaxGroups];
  const uint16_t* B[kMaxGroups];
  const uint16_t* B2[kMaxGroups];  // kEpiSwiGLU: the second B operand (up projection)
  const uint16_t* bias[kMaxGroups];
  void* C[kMaxGroups];
  void* aux[kMaxGroups];
};

struct GemmParams {
  GroupTable t;
  int groups;
  int64_t lda, ldb, ldc;
  int M, N, K;
  int tiles_m, tiles_n;
  // K-split (float32 store / accumulate epilogues only): each group's grid
  // holds `slices` copies of the tile grid; slice s covers k in
  // [s k_slice, min(K, (s + 1) k_slice)).  Slice 0 applies the epilogue to
  // C, slice s > 0 stores its partial to part + ((g (slices - 1) + s - 1)
  // part_stride (leading dimension N).  slices == 1: no split.
  int slices, k_slice;
  float* part;
  int64_t part_stride;
  // Every group reads the same A (a column step's X): groups that divide
  // the XCDs are pinned to XCD subsets (see the tile mapping).
  int shared_a;
};

// Workgroup tile configurations (index = tile id used by the picker).
// split = 1: a stage's DMA loads are spread over both halves of a K step
// (the first half of the loads with the first half of the MFMAs, the rest
// after the mid-step barrier) instead of all in the first half, halving the
// burst of load instructions each CU's load path takes per half step.  On
// the 256x256 tile it measured 0-1% faster on long_seq's and llama7b's
// steps and 2-6% on gpt3_175b's (bit-identical).
struct TileCfg {
  int bm, bn, wm, wn, nbuf;
  int split = 0;
};
constexpr TileCfg kTiles[] = {
    {256, 256, 2, 4, 4, 1},  // 0
    {256, 256, 2, 4, 5},  // 1
    {256, 256, 2, 4, 3},  // 2
    {256, 128, 4, 2, 4},  // 3
    {256, 128, 4, 2, 3},  // 4
    {128, 256, 2, 4, 4},  // 5
    {128, 256, 2, 4, 3},  // 6
    {128, 128, 2, 2, 4},  // 7
    {128, 128, 2, 4, 4},  // 8
    {128, 384, 2, 4, 4},  // 9
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// Epilogues each layout is instantiated with.
constexpr bool layout_has_epi(int layout, int epi) {
  return layout == kNN ? (epi == kEpiBiasGelu || epi == kEpiBiasGeluSave || epi == kEpiStoreF32 ||
                          epi == kEpiAccumF32 || epi == kEpiSwiGLU || epi == kEpiBias || epi == kEpiMulAux)
       : layout == kNT ? (epi == kEpiMulAux || epi == kEpiStoreF32 || epi == kEpiAccumF32)
                       : (epi == kEpiStoreF32 || epi == kEpiAccumF32);
}

// LDS chunk swizzles (see the file comment).  K-major rows are 64 bytes
// (four chunks) and a fragment read takes the four chunks of 16 consecutive
// rows (lanes 16 c .. 16 c + 15 take chunk c).  Timing every swizzle that
// XORs the chunk index with two parity bits of row bits 0..3 for this read on
// MI355X (core cycles per read; 16-byte reads spread over 64 four-byte banks)
// splits them into a conflict-free class and classes 1.7x and 3.3x slower.
// swzK, with q = row bits 2..3, XORs with (-q) mod 4 (bit 0: row bit 2; bit
// 1: row bits 2 ^ 3) and is in the conflict-free class; XOR with q itself is
// in the 1.7x one.
// MN-major rows hold >= 16 chunks; swzMN rotates by 4 chunks per k-row so
// that the four k-rows of a transpose read fall in distinct bank groups, and
// by 2 more chunks for k-rows 8..15 of every 16 (a fragment's lanes 16-31
// read the same columns 8 k-rows below lanes 0-15).
__device__ __forceinline__ int swzK(int r) { return (-(r >> 2)) & 3; }
__device__ __forceinline__ int swzMN(int k) { return (4 * (k & 3)) ^ (2 * ((k >> 3) & 1)); }

// One operand's tile: R rows of the operand (rows of A, or columns of B) by
// 32 k per stage, loaded by NW waves.  KTAIL: K may end inside a stage, so the
// chunks of the last stage are masked per lane by their k.
template <int R, bool KMAJ, int NW, bool KTAIL>
struct OperandTile {
  static constexpr int kBytes = R * 64;  // R x 32 x 2 bytes
  static constexpr int kPerWave = kBytes / 1024 / NW;
  static constexpr int kRow = KMAJ ? 64 : 2 * R;  // LDS row bytes
  static constexpr int kLanesPerRow = kRow / 16;
  static_assert(kBytes % (1024 * NW) == 0, "DMA split");
  static_assert(KMAJ || (R % 128 == 0 && R <= 512), "MN-major tiles need 16-chunk row groups");

  // Global address of (tile row 0, first k of the next stage to be issued);
  // stages are issued in order, so it advances by `step` bytes per stage.
  uint64_t cur;
  uint64_t step;
  uint64_t tile_off;  // bytes from the operand's start to tile row 0
  uint32_t src[kPerWave];  // byte offset of the lane's chunk from (tile row 0, stage k 0)
  int kidx[kPerWave];      // first k (within a stage) of the lane's chunk (KTAIL only)

  // r0: first row (K-major) or column (MN-major) of the tile; rtot: the
  // operand's extent in that dimension; ld: leading dimension in elements.
  // A chunk outside the operand gets offset kOob and reads as zeros; every
  // other offset addresses memory inside the operand, so the descriptors
  // need no exact size.
  __device__ __forceinline__ void init(const uint16_t* ptr, int64_t ld, int r0, int rtot, int wave,
                                       int lane) {
    static_assert(sizeof(uint64_t) == sizeof(ptr), "64-bit pointers");
    if constexpr (KMAJ) {
      tile_off = (uint64_t)r0 * (uint64_t)ld * 2u;
      step = 64;  // 32 k x 2 bytes
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int row = (wave * kPerWave + i) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swzK(row);
        src[i] = r0 + row < rtot ? (uint32_t)row * (uint32_t)ld * 2u + (uint32_t)c * 16u : kOob;
        kidx[i] = c * 8;
      }
    } else {
      tile_off = (uint64_t)r0 * 2u;
      step = (uint64_t)ld * 64u;  // 32 k-rows
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        // chunk o of the tile (LDS bytes 16 o ..): k-row o / kLanesPerRow,
        // position o % kLanesPerRow (a 1 KB block may end inside a k-row)
        const int o = (wave * kPerWave + i) * 64 + lane;
        const int row = o / kLanesPerRow;
        const int c = (o % kLanesPerRow) ^ swzMN(row);
        src[i] = r0 + c * 8 < rtot ? (uint32_t)row * (uint32_t)ld * 2u + (uint32_t)c * 16u : kOob;
        kidx[i] = row;
      }
    }
    rebase(ptr);
  }

  // Continue with another operand of the same shape (the next group).
  __device__ __forceinline__ void rebase(const uint16_t* ptr) {
    cur = reinterpret_cast<uint64_t>(ptr) + tile_off;
  }

  // Loads of the next stage (k0 .. k0 + 31) into the LDS block at lds_addr;
  // kleft = K - k0.  A stage past the end (kleft <= 0) gets an empty
  // descriptor: every lane writes zeros and no memory is read.
  __device__ __forceinline__ i32x4_t desc(int kleft) const {
    return buffer_desc(reinterpret_cast<const void*>(cur), kleft > 0 ? 0x7FFFFFF0u : 0u);
  }
  __device__ __forceinline__ void issue_one(const i32x4_t& d, uint32_t lds_addr, int wave, int i, int kleft) const {
    uint32_t off = src[i];
    if constexpr (KTAIL) off = kidx[i] < kleft ? off : kOob;
    lds_dma16(d, lds_addr + (uint32_t)((wave * kPerWave + i) * 1024), off);
  }
  __device__ __forceinline__ void issue(uint32_t lds_addr, int wave, int kleft) {
    const i32x4_t d = desc(kleft);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) issue_one(d, lds_addr, wave, i, kleft);
    cur += step;
  }
};

// Fragment reads of one operand for a wave whose F fragments start at tile
// row `wbase` (K-major: F blocks of 16 rows; MN-major: F blocks of 16
// columns).  A fragment covers 16 rows (or columns) by the stage's 32 k; lane
// l holds k 8 (l / 16) .. + 7 of row l % 16.
template <int R, bool KMAJ, int F>
struct OperandFrags {
  static constexpr int kRow = KMAJ ? 64 : 2 * R;
  int off[KMAJ ? 1 : F];

  __device__ __forceinline__ void init(int wbase, int lane) {
    if constexpr (KMAJ) {
      const int row = wbase + (lane & 15);
      off[0] = row * 64 + ((lane >> 4) ^ swzK(row)) * 16;  // fragment f: + 16 rows of 64 bytes
    } else {
      // ds_read_b64_tr_b16: 16 lanes read 4 k-rows x 16 columns (lane t: k-row
      // t / 4, columns 4 (t % 4) .. + 3) and each gets one column's 4 k; the
      // second read takes the 4 k-rows below.
      const int g = lane >> 4, t = lane & 15;
      const int krow = 8 * g + (t >> 2);
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int col = wbase + 16 * f + 4 * (t & 3);
        off[f] = krow * kRow + (((col >> 3) ^ swzMN(krow)) * 16) + ((col >> 2) & 1) * 8;
      }
    }
  }

  // Fragment f.  swzK(r + 16 f) == swzK(r) and swzMN(k + 4) == swzMN(k).
  __device__ __forceinline__ bf16x8_t get(const char* S, int f) const {
    if constexpr (KMAJ) {
      return *reinterpret_cast<const bf16x8_t*>(S + off[0] + f * 1024);
    } else {
      const char* p = S + off[f];
      return ds_read_tr_pair(p, p + 4 * kRow);
    }
  }
};

// GSUM: the groups are summed instead of launched side by side: each output
// tile runs its K loop through every group in turn with one float32
// accumulator (which starts at zero, or at C itself with kEpiAccumF32), and
// stores once.  This is the GEMM of the groups' A operands side by side with
// their B operands stacked, [A_0 ... A_{n-1}] [B_0; ...; B_{n-1}], accumulated
// in group order; it equals the sum of the groups' products up to float32
// rounding, and a batch run in several launches (accumulating into C) gives
// the same bits as one launch.
//
// DUAL (kEpiSwiGLU): two B operands, the gate B and the up projection B2, of
// the same shape.  The stage holds A and two B sub-tiles of BN / 2 columns
// each (the gate's and the up projection's for the same BN / 2 output
// columns), every wave reads its FN / 2 gate and FN / 2 up fragments at the
// same offsets of the two sub-tiles, and the epilogue stores
// SiLU(gate) * up: a BM x BN / 2 tile of the output.

// Waves per SIMD to ask the register allocator for: as many as the
// workgroups that the tile's LDS stages let share a CU bring (two 8-wave
// workgroups of 72 KB: four waves per SIMD, so at most 128 VGPRs each).  The
// training epilogue keeps a second output and is left to the allocator (at
// 128 VGPRs it would spill, measured slower than one workgroup per CU).
constexpr int gemm_waves_per_eu(int EPI, int BM, int BN, int WM, int WN, int NBUF) {
  if (EPI == kEpiBiasGeluSave) return 1;
  const int per_cu = (160 * 1024) / (NBUF * (BM + BN) * 64);
  const int w = per_cu * WM * WN / 4;
  return w < 1 ? 1 : (w > 4 ? 4 : w);
}

template <int EPI, int LAYOUT, int BM, int BN, int WM, int WN, int NBUF, bool KTAIL, bool GSUM, int SPLIT>
__global__ __launch_bounds__(WM* WN * 64, gemm_waves_per_eu(EPI, BM, BN, WM, WN, NBUF))
void gemm_bf16_kernel(GemmParams p) {
  constexpr bool AK = LAYOUT != kTN;  // A K-major
  constexpr bool BK = LAYOUT == kNT;  // B K-major
  constexpr bool DUAL = EPI == kEpiSwiGLU;
  constexpr int D = NBUF - 1;         // prefetch distance in K steps of 32
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int NB = DUAL ? 2 : 1;              // B sub-tiles per stage
  constexpr int BNO = BN / NB, WTNO = WTN / NB;  // output columns per workgroup / wave
  constexpr int FNO = FN / NB;                  // output fragments per wave row
  using TA = OperandTile<BM, AK, NW, KTAIL>;
  using TB = OperandTile<BNO, BK, NW, KTAIL>;
  using RA = OperandFrags<BM, AK, FM>;
  using RB = OperandFrags<BNO, BK, FNO>;
  constexpr int A_BYTES = TA::kBytes, STAGE = TA::kBytes + NB * TB::kBytes;
  constexpr int L = TA::kPerWave + NB * TB::kPerWave;  // DMA instructions per wave per stage
  static_assert(!DUAL || (LAYOUT == kNN && FN % 2 == 0 && !GSUM), "SwiGLU: kNN, two fragment sets");
  static_assert(WTM % 32 == 0 && WTN % 16 == 0, "wave tile: two halves of 16-row fragments by 16-column ones");
  static_assert(NBUF >= 3 && NBUF <= 6, "stage count");
  static_assert((D - 1) * L <= 63, "vmcnt immediate");
  static_assert(NBUF * STAGE <= 160 * 1024, "LDS");
  static_assert(!GSUM || EPI == kEpiStoreF32 || EPI == kEpiAccumF32, "group sum stores float32");

  // One array per stage: distinct LDS objects get distinct alias scopes, so
  // the compiler can tell that fragment reads of one stage do not depend on
  // the DMA writes in flight into the others (and inserts no vmcnt wait).
  __shared__ __attribute__((aligned(1024))) char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[STAGE];
  __shared__ __attribute__((aligned(1024))) char st3[NBUF > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char st4[NBUF > 4 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char st5[NBUF > 5 ? STAGE : 16];
  auto stage = [&](auto bset) -> char* {
    constexpr int b = decltype(bset)::value;
    if constexpr (b == 0) return st0;
    else if constexpr (b == 1) return st1;
    else if constexpr (b == 2) return st2;
    else if constexpr (b == 3) return st3;
    else if constexpr (b == 4) return st4;
    else return st5;
  };
  auto stage_lds = [&](auto bset) -> uint32_t {
    constexpr int b = decltype(bset)::value;
    if constexpr (b == 0) return lds_offset(st0);
    else if constexpr (b == 1) return lds_offset(st1);
    else if constexpr (b == 2) return lds_offset(st2);
    else if constexpr (b == 3) return lds_offset(st3);
    else if constexpr (b == 4) return lds_offset(st4);
    else return lds_offset(st5);
  };

  int tm, tn;
  const int tiles = p.tiles_m * p.tiles_n;
  int bid = blockIdx.x, slice = 0, grp = 0;
  if (!GSUM && p.slices > 1) {
    // K-split: the whole grid is regrouped so that each XCD runs a contiguous
    // range of (slice, group, tile) in slice-major order, i.e. the workgroups
    // on one XCD share one K slab of the operands in its L2.
    const int sg_tile = xcd_logical(bid, tiles * p.slices * p.groups);
    const int sg = sg_tile / tiles;
    grp = sg % p.groups;
    slice = sg / p.groups;
    strip_coords<8>(sg_tile - sg * tiles, p.tiles_m, p.tiles_n, tm, tn);
  } else if (!GSUM && p.shared_a && p.groups > 1 && kNumXcd % p.groups == 0 &&
             tiles % (kNumXcd / p.groups) == 0) {
    // A batch that shares A, with groups dividing the XCDs: group g runs on
    // XCDs [g per, (g + 1) per) only (workgroup b runs on XCD b % 8), each of
    // them a contiguous range of the group's tiles walked in strips.  At any
    // time the XCDs of different groups then stream the same rows of A (the
    // last-level cache serves all but one of them) and each group's B stays
    // in `per` L2s.  Measured against the group-major order: long_seq's
    // column step 5% faster, llama7b's 2%, gpt3_175b's and gpt2_small's
    // within 1%; on row steps, whose groups share nothing, it was 3-5%
    // slower on the large shapes, so they keep the group-major order.
    const int per = kNumXcd / p.groups;
    const int x = bid % kNumXcd;
    grp = x / per;
    const int local = (bid / kNumXcd) * per + x % per;  // 0 .. tiles - 1 within the group
    strip_coords<8>((local % per) * (tiles / per) + local / per, p.tiles_m, p.tiles_n, tm, tn);
  } else {
    if (!GSUM && p.groups > 1) {
      grp = bid / tiles;
      bid -= grp * tiles;
    }
    // A group sum's K loop runs through every shard, so each A row panel is
    // long (long_seq: 256 rows x 32768 k) and cannot stay in the last-level
    // cache from one column round to the next: strips of 4 tile rows (x 8
    // columns per XCD round) read each A panel half as many times as strips
    // of 8 (x 4), for twice the B panels, which every XCD shares.  Measured
    // with 256 x 256 tiles: long_seq's shard sum 2% faster, llama7b's the same.
    constexpr int kStrip = (GSUM && BM == 256 && BN == 256) ? 4 : 8;
    tile_coords<kStrip>(bid, tiles, p.tiles_m, p.tiles_n, tm, tn);
  }
  // (wave-uniform by construction; said explicitly so that the operand
  // pointers derived from them stay in scalar registers)
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  grp = __builtin_amdgcn_readfirstlane(grp);
  slice = __builtin_amdgcn_readfirstlane(slice);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = tm * BM;
  const int n0 = tn * BNO;
  int K = p.K;
  int kb = 0;  // first k of this workgroup's slice
  if (p.slices > 1) {
    kb = slice * p.k_slice;
    K = min(K - kb, p.k_slice);
  }
  const int nk = (K + 31) / 32;                 // stages per group
  const int ngroups = GSUM ? p.groups : 1;      // groups this workgroup runs through
  const int nstages = nk * ngroups;
  // Start of group g's operands at k = kb.
  auto a_ptr = [&](int g) {
    return p.t.A[g] + (AK ? (int64_t)kb : (int64_t)kb * p.lda);
  };
  auto b_ptr = [&](int g) {
    return p.t.B[g] + (BK ? (int64_t)kb : (int64_t)kb * p.ldb);
  };

  TA ta;
  TB tb, tb2;
  ta.init(a_ptr(grp), p.lda, m0, p.M, wave, lane);
  tb.init(b_ptr(grp), p.ldb, n0, p.N, wave, lane);
  if constexpr (DUAL) tb2.init(p.t.B2[grp] + (int64_t)kb * p.ldb, p.ldb, n0, p.N, wave, lane);
  // Stages are issued in order: (group 0, stage 0 .. nk - 1), (group 1, ...).
  int iss_g = 0, iss_kt = 0;
  auto issue_stage = [&](auto bset) {
    const uint32_t S = stage_lds(bset);
    const int kleft = iss_g < ngroups ? K - iss_kt * 32 : 0;
    ta.issue(S, wave, kleft);
    tb.issue(S + A_BYTES, wave, kleft);
    if constexpr (DUAL) tb2.issue(S + A_BYTES + TB::kBytes, wave, kleft);
    if (++iss_kt == nk) {
      iss_kt = 0;
      if (GSUM && ++iss_g < ngroups) {
        ta.rebase(a_ptr(iss_g));
        tb.rebase(b_ptr(iss_g));
      } else if (!GSUM) {
        iss_g = 1;
      }
    }
  };

  RA ra;
  RB rb;
  ra.init(wm * WTM, lane);
  rb.init(wn * WTNO, lane);

  // Output layout of an MFMA tile (the B fragment goes in the instruction's A
  // slot): lane l holds row l % 16 of the tile, columns 4 (l / 16) .. + 3.
  const int lrow = lane & 15;
  const int hcol = 4 * (lane >> 4);
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Group sum accumulating into C: the accumulator starts at C's values.
  if constexpr (GSUM && EPI == kEpiAccumF32) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = m0 + wm * WTM + i * 16 + lrow;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * WTN + j * 16 + hcol;
        if (m < p.M && n < p.N)
          acc[i][j] = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p.t.C[0]) + (int64_t)m * p.ldc + n);
      }
    }
  }

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // vmcnt((D - 1) L), expcnt(7), lgkmcnt(0): this wave's loads of the next
  // stage (all but the D - 1 younger stages) and all its LDS reads are done.
  // With SPLIT, the first H0 loads of a stage issue in the first part of a
  // step and the rest in the second, so at the mid-step barrier H0 loads of
  // the newest stage are in flight instead of L.
  constexpr int H0 = SPLIT ? L / 2 : L;
  constexpr int kWaitN = (D - 2) * L + H0;
  constexpr int kWaitNext = (kWaitN & 15) | ((kWaitN >> 4) << 14) | (7 << 4);
  constexpr int kWaitPro = (D - 1) * L;
  constexpr int kWaitProlog = (kWaitPro & 15) | ((kWaitPro >> 4) << 14) | (7 << 4);

  [&]<int... b>(std::integer_sequence<int, b...>) {
    (issue_stage(std::integral_constant<int, b>{}), ...);
  }(std::make_integer_sequence<int, D>{});
  __builtin_amdgcn_s_waitcnt(kWaitProlog);
  asm volatile("s_barrier" ::: "memory");

  // The K loop is written out in issue order: each part of a step is MFMA
  // m, then the fragment reads and DMA loads assigned to it, then a
  // scheduling fence.  The fences keep the compiler from hoisting
  // the loads: they are inline assembly, which scheduling-group hints cannot
  // place, and left alone every DMA and fragment read of a part issues ahead
  // of its first MFMA.  A stage's DMA is prepared once (descriptors, then the
  // pointers advance) and its loads are spread over the MFMAs of the first
  // part; the fragment reads are front-loaded.
  struct StageIssue {
    uint32_t S;
    int kleft;
    i32x4_t da, db, db2;
  };
  auto stage_begin = [&](auto bset) {
    StageIssue r;
    r.S = stage_lds(bset);
    r.kleft = iss_g < ngroups ? K - iss_kt * 32 : 0;
    r.da = ta.desc(r.kleft);
    r.db = tb.desc(r.kleft);
    if constexpr (DUAL) r.db2 = tb2.desc(r.kleft);
    ta.cur += ta.step;
    tb.cur += tb.step;
    if constexpr (DUAL) tb2.cur += tb2.step;
    if (++iss_kt == nk) {
      iss_kt = 0;
      if (GSUM && ++iss_g < ngroups) {
        ta.rebase(a_ptr(iss_g));
        tb.rebase(b_ptr(iss_g));
      } else if (!GSUM) {
        iss_g = 1;
      }
    }
    return r;
  };
  auto dma_one = [&](const StageIssue& r, auto lset) {
    constexpr int l = decltype(lset)::value;
    if constexpr (l < TA::kPerWave) ta.issue_one(r.da, r.S, wave, l, r.kleft);
    else if constexpr (l < TA::kPerWave + TB::kPerWave)
      tb.issue_one(r.db, r.S + A_BYTES, wave, l - TA::kPerWave, r.kleft);
    else tb2.issue_one(r.db2, r.S + A_BYTES + TB::kBytes, wave, l - TA::kPerWave - TB::kPerWave, r.kleft);
  };
  // A step of 32 k on stage buffer c runs the wave's FM x FN MFMAs in two
  // parts.  A's fragments are read in two halves (the wave's fragment rows
  // [0, FH) and [FH, FM)), B's into one of two sets by step parity.  Part 0:
  // the MFMAs of A's first half (read in the previous step) while the second
  // half is read and the refill DMA issues; then the barrier; part 1: the
  // MFMAs of the second half while the next stage's first half of A and its
  // B are read, in the order the next step's first MFMAs use them (A fragment
  // 0, every B fragment, the other A fragments).
  constexpr int FH = FM / 2;
  constexpr int kM = FH * FN;  // MFMAs per part
  bf16x8_t fa0[FH], fa1[FH], fb[2][FN];
  auto read_b = [&](const char* S, int f) {
    return f < FNO ? rb.get(S + A_BYTES, f) : rb.get(S + A_BYTES + TB::kBytes, f - FNO);
  };
  {
    const char* S = stage(I0{});
#pragma unroll
    for (int f = 0; f < FH; ++f) fa0[f] = ra.get(S, f);
#pragma unroll
    for (int f = 0; f < FN; ++f) fb[0][f] = read_b(S, f);
  }
  // Part P of a step with B set BP, fragment reads from stage buffer sset:
  // MFMA m, then fragment read m (reads past the last MFMA follow it), then
  // the DMA loads l with l kM / L == m, then a fence.
  auto part = [&](auto pset, auto bpset, auto sset, const StageIssue* dma) {
    constexpr int P = decltype(pset)::value, BP = decltype(bpset)::value;
    constexpr int kOps = P == 0 ? FH : FH + FN;
    const char* S = stage(sset);
    auto op = [&](auto rset) {
      constexpr int r = decltype(rset)::value;
      if constexpr (P == 0) fa1[r] = ra.get(S, FH + r);
      else if constexpr (r == 0) fa0[0] = ra.get(S, 0);
      else if constexpr (r <= FN) fb[1 - BP][r - 1] = read_b(S, r - 1);
      else fa0[r - FN] = ra.get(S, r - FN);
    };
    auto one = [&](auto mset) {
      constexpr int m = decltype(mset)::value, i = m / FN, j = m % FN;
      if constexpr (P == 0)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[BP][j], fa0[i], acc[i][j], 0, 0, 0);
      else
        acc[FH + i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[BP][j], fa1[i], acc[FH + i][j], 0, 0, 0);
      if constexpr (m < kOps) op(std::integral_constant<int, m>{});
      if constexpr (m == kM - 1 && kOps > kM) {
        [&]<int... r>(std::integer_sequence<int, r...>) {
          (op(std::integral_constant<int, kM + r>{}), ...);
        }(std::make_integer_sequence<int, (kOps > kM ? kOps - kM : 0)>{});
      }
      if (dma) {
        // loads [l0, l0 + nl) of the stage, spread over this part's MFMAs
        constexpr int l0 = P == 0 ? 0 : H0, nl = P == 0 ? H0 : L - H0;
        [&]<int... l>(std::integer_sequence<int, l...>) {
          ((l * kM / nl == m ? (dma_one(*dma, std::integral_constant<int, l0 + l>{}), 0) : 0), ...);
        }(std::make_integer_sequence<int, nl>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    [&]<int... m>(std::integer_sequence<int, m...>) {
      (one(std::integral_constant<int, m>{}), ...);
    }(std::make_integer_sequence<int, kM>{});
  };
  // Step b (static: buffer b % NBUF, B set b % 2, so every LDS access names
  // its buffer at compile time).
  auto kstep = [&](auto bset) {
    constexpr int b = decltype(bset)::value, c = b % NBUF;
    using Cur = std::integral_constant<int, c>;
    using BP = std::integral_constant<int, b % 2>;
    using Refill = std::integral_constant<int, (c + D) % NBUF>;
    using Next = std::integral_constant<int, (c + 1) % NBUF>;
    const StageIssue st = stage_begin(Refill{});
    part(I0{}, BP{}, Cur{}, &st);
    __builtin_amdgcn_s_waitcnt(kWaitNext);
    asm volatile("s_barrier" ::: "memory");
    part(I1{}, BP{}, Next{}, SPLIT ? &st : nullptr);
  };
  // The loop body walks U consecutive steps (a multiple of NBUF and of 2);
  // an early exit handles a stage count that is not a multiple of U (uniform
  // across the workgroup).
  constexpr int U = NBUF % 2 == 0 ? NBUF : 2 * NBUF;
  for (int st = 0; st < nstages; st += U) {
    bool more = true;
    [&]<int... b>(std::integer_sequence<int, b...>) {
      ((more = more && (st + b < nstages), more ? (kstep(std::integral_constant<int, b>{}), 0) : 0), ...);
    }(std::make_integer_sequence<int, U>{});
  }
  // The last stages' loads (out of range, writing zeros) must have landed
  // before this workgroup's LDS can be handed to another.
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)

  // Epilogue.  Per 16-row block i, every global load the epilogue needs (the
  // multiplier or the old value of C) is issued before any store, so the
  // loads overlap; each element is read and written by the same lane only,
  // so this order is also correct when C is aux.  The bias is loaded once.
  // Tiles wholly inside C take a path without per-store bounds checks.
  const int M = p.M, N = p.N;
  int64_t ldc = p.ldc;
  void* Cout = p.t.C[grp];
  void* aux = p.t.aux[grp];
  const uint16_t* bias = p.t.bias[grp];
  bool accumulate = EPI == kEpiAccumF32 && !GSUM;  // (a group sum's accumulator started at C)
  if (slice > 0) {  // a K-split partial: plain float32 store
    Cout = p.part + ((int64_t)grp * (p.slices - 1) + slice - 1) * p.part_stride;
    ldc = N;
    accumulate = false;
  }
  constexpr bool kBias = EPI == kEpiBiasGelu || EPI == kEpiBiasGeluSave || EPI == kEpiBias;
  // Output column of lane `lane`'s 4 values in output fragment j.
  auto col = [&](int j) { return n0 + wn * WTNO + j * 16 + hcol; };
  f32x4_t bias4[FN];
  if constexpr (kBias) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = col(j);
      u32x2_t bb = u32x2_t{0u, 0u};
      if (bias && n < N) bb = *reinterpret_cast<const u32x2_t*>(bias + n);
      bias4[j] = f32x4_t{bf16_bits_to_f32(bb[0] & 0xFFFFu), bf16_bits_to_f32(bb[0] >> 16),
                         bf16_bits_to_f32(bb[1] & 0xFFFFu), bf16_bits_to_f32(bb[1] >> 16)};
    }
  }
  // The final value of output fragment (i, j) before rounding: SiLU(gate)
  // times up for SwiGLU, else the accumulator plus the bias.
  auto value = [&](int i, int j) {
    f32x4_t v;
    if constexpr (DUAL) {
      // gate fragment j and up fragment FNO + j hold the same columns
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = silu_f32(acc[i][j][e]) * acc[i][FNO + j][e];
    } else {
      v = acc[i][j];
      if constexpr (kBias) v += bias4[j];
    }
    return v;
  };
  auto epilogue = [&](auto guard) {
    constexpr bool G = decltype(guard)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = m0 + wm * WTM + i * 16 + lrow;
      const bool mrow = !G || m < M;
      const int64_t row = (int64_t)m * ldc;
      u32x2_t aux2[FN];
      f32x4_t old4[FN];
      if constexpr (EPI == kEpiMulAux || EPI == kEpiAccumF32) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = col(j);
          const bool ok = !G || (mrow && n < N);
          if constexpr (EPI == kEpiMulAux) {
            aux2[j] = u32x2_t{0u, 0u};
            if (ok) aux2[j] = *reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(aux) + row + n);
          } else {
            old4[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (ok && accumulate)
              old4[j] = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(Cout) + row + n);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < FNO; ++j) {
        const int n = col(j);
        if (G && (!mrow || n >= N)) continue;
        const int64_t idx = row + n;
        const f32x4_t v = value(i, j);
        if constexpr (DUAL || EPI == kEpiBias) {
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(Cout) + idx) = pack4_bf16(v);
        } else if constexpr (EPI == kEpiBiasGelu) {
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(Cout) + idx) =
              pack4_bf16(f32x4_t{gelu_f32(v[0]), gelu_f32(v[1]), gelu_f32(v[2]), gelu_f32(v[3])});
        } else if constexpr (EPI == kEpiBiasGeluSave) {
          float y[4], g[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) gelu_and_grad_f32(v[e], y[e], g[e]);
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(Cout) + idx) = pack4_bf16(f32x4_t{y[0], y[1], y[2], y[3]});
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(aux) + idx) = pack4_bf16(f32x4_t{g[0], g[1], g[2], g[3]});
        } else if constexpr (EPI == kEpiMulAux) {
          const u32x2_t gg = aux2[j];
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(Cout) + idx) =
              pack4_bf16(f32x4_t{v[0] * bf16_bits_to_f32(gg[0] & 0xFFFFu), v[1] * bf16_bits_to_f32(gg[0] >> 16),
                                 v[2] * bf16_bits_to_f32(gg[1] & 0xFFFFu), v[3] * bf16_bits_to_f32(gg[1] >> 16)});
        } else if constexpr (EPI == kEpiStoreF32) {
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(Cout) + idx) = v;
        } else {
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(Cout) + idx) = accumulate ? old4[j] + v : v;
        }
      }
    }
  };
  // Tiles wholly inside C with a store-only epilogue go through LDS: each
  // wave writes one 16-row block of 128 output bytes per row (two fp32 or
  // four bf16 output fragments) into its own region of the stage buffers,
  // reads it back by rows and stores whole 128-byte row segments, so that
  // every store instruction writes full cache lines (the accumulator layout
  // alone gives 16- or 8-byte pieces of 16 rows per instruction).
  constexpr bool kCanStage = EPI != kEpiMulAux;
  if constexpr (kCanStage) {
    if (m0 + BM <= M && n0 + BNO <= N && !accumulate) {
      constexpr int kElt = (EPI == kEpiStoreF32 || EPI == kEpiAccumF32) ? 4 : 2;
      constexpr int kWant = 128 / (16 * kElt);  // fragments per 128-byte row segment
      constexpr int kFragsPerChunk = FNO % kWant == 0 ? kWant : (FNO % 2 == 0 ? 2 : 1);
      constexpr int kChunkBytes = kFragsPerChunk * 16 * kElt;  // one row of a chunk: 128 bytes or less
      constexpr int kRowStride = kChunkBytes + 16;             // padded (bank spread)
      constexpr int kRegion = 16 * kRowStride;
      constexpr int kRegionsPerStage = STAGE / kRegion;
      static_assert(kRegionsPerStage * NBUF >= NW, "epilogue staging regions");
      constexpr int kLanesPerRow = kChunkBytes / 16;
      constexpr int kRowsPerPass = 64 / kLanesPerRow;
      static_assert(kRowsPerPass <= 16 && 16 % kRowsPerPass == 0, "row passes");
      constexpr int kPasses = 16 / kRowsPerPass;
      constexpr int kNumOut = EPI == kEpiBiasGeluSave ? 2 : 1;
      // Every wave is past its last fragment read and every DMA of the
      // workgroup has landed before the stage buffers are reused.
      asm volatile("s_barrier" ::: "memory");
      const int sidx = wave / kRegionsPerStage;
      uint32_t region = lds_offset(st0);
      if (sidx == 1) region = lds_offset(st1);
      if (sidx == 2) region = lds_offset(st2);
      if (NBUF > 3 && sidx == 3) region = lds_offset(st3);
      if (NBUF > 4 && sidx == 4) region = lds_offset(st4);
      if (NBUF > 5 && sidx == 5) region = lds_offset(st5);
      region += (uint32_t)((wave % kRegionsPerStage) * kRegion);
      using lds_char = __attribute__((address_space(3))) char;
      lds_char* R = (lds_char*)(uintptr_t)region;
      const int rrow = lane / kLanesPerRow, rcol = (lane % kLanesPerRow) * 16;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int c = 0; c < FNO / kFragsPerChunk; ++c) {
          // Each fragment's 4 final values go to LDS as soon as they are
          // computed (lane l: row l % 16, columns 16 f + 4 (l / 16) .. + 3);
          // the second output of the training epilogue waits packed in
          // registers until the first has been read back.
          u32x2_t second[kNumOut - 1 ? kFragsPerChunk : 1];
          auto slot = [&](int f) { return R + lrow * kRowStride + (16 * f + hcol) * kElt; };
          // Rows back from LDS, whole 128-byte (or 64-byte) row segments to C.
          auto drain = [&](void* out) {
            u32x4_t rows[kPasses];
#pragma unroll
            for (int t = 0; t < kPasses; ++t)
              rows[t] = *(__attribute__((address_space(3))) u32x4_t*)(R + (rrow + t * kRowsPerPass) * kRowStride + rcol);
            char* base = static_cast<char*>(out) +
                         ((int64_t)(m0 + wm * WTM + i * 16 + rrow) * ldc + n0 + wn * WTNO + c * kFragsPerChunk * 16) *
                             kElt + rcol;
#pragma unroll
            for (int t = 0; t < kPasses; ++t)
              *reinterpret_cast<u32x4_t*>(base + (int64_t)t * kRowsPerPass * ldc * kElt) = rows[t];
          };
#pragma unroll
          for (int f = 0; f < kFragsPerChunk; ++f) {
            f32x4_t a = value(i, c * kFragsPerChunk + f);
            if constexpr (EPI == kEpiBiasGelu) {
#pragma unroll
              for (int e = 0; e < 4; ++e) a[e] = gelu_f32(a[e]);
            }
            if constexpr (EPI == kEpiBiasGeluSave) {
              float y[4], g[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) gelu_and_grad_f32(a[e], y[e], g[e]);
              a = f32x4_t{y[0], y[1], y[2], y[3]};
              second[f] = pack4_bf16(f32x4_t{g[0], g[1], g[2], g[3]});
            }
            if constexpr (kElt == 4) *(__attribute__((address_space(3))) f32x4_t*)slot(f) = a;
            else *(__attribute__((address_space(3))) u32x2_t*)slot(f) = pack4_bf16(a);
          }
          drain(Cout);
          if constexpr (kNumOut == 2) {
#pragma unroll
            for (int f = 0; f < kFragsPerChunk; ++f) *(__attribute__((address_space(3))) u32x2_t*)slot(f) = second[f];
            drain(aux);
          }
        }
      }
      return;
    }
  }
  if (m0 + BM <= M && n0 + BNO <= N)
    epilogue(std::false_type{});
  else
    epilogue(std::true_type{});
}

// SwiGLU splits a tile's BN columns into a gate and an up sub-tile of BN / 2
// columns each (MN-major sub-tiles need 128, 256 or 512 columns) and every
// wave's fragments into two equal sets.
constexpr bool tile_allows_swiglu(int t) {
  return (kTiles[t].bn / 2 == 128 || kTiles[t].bn / 2 == 256) && (kTiles[t].bn / kTiles[t].wn / 16) % 2 == 0;
}

// Output columns of one workgroup tile.
constexpr int tile_out_cols(int t, int epi) { return epi == kEpiSwiGLU ? kTiles[t].bn / 2 : kTiles[t].bn; }

// K % 32 != 0 runs on a ragged-K variant of one tile only: kTailTile, or
// kTailTileSwiGLU for the SwiGLU epilogue.
constexpr int kTailTile = 8;
constexpr int kTailTileSwiGLU = 6;

// Which (tile, ragged K, group sum, epilogue) combinations a layout is
// compiled for.
constexpr bool instantiated(int layout, int t, bool ktail, bool gsum, int epi) {
  if (!layout_has_epi(layout, epi)) return false;
  if (gsum && (layout == kTN || (epi != kEpiStoreF32 && epi != kEpiAccumF32))) return false;
  if (epi == kEpiSwiGLU) return !gsum && tile_allows_swiglu(t) && (!ktail || t == kTailTileSwiGLU);
  return !ktail || t == kTailTile;
}

// Launch one tile configuration of one layout (p.tiles_m / p.tiles_n set).
template <int LAYOUT, int T, bool KTAIL, bool GSUM>
hipError_t launch_bf16_tile(const GemmParams& p, Epilogue epi, hipStream_t s) {
  constexpr TileCfg c = kTiles[T];
  const unsigned copies = GSUM ? 1u : (unsigned)p.groups * (unsigned)p.slices;
  const dim3 grid((unsigned)p.tiles_m * (unsigned)p.tiles_n * copies), block(c.wm * c.wn * 64);
  bool done = false;
  [&]<int... e>(std::integer_sequence<int, e...>) {
    (([&] {
       if constexpr (instantiated(LAYOUT, T, KTAIL, GSUM, e)) {
         if (epi == e) {
           hipLaunchKernelGGL((gemm_bf16_kernel<e, LAYOUT, c.bm, c.bn, c.wm, c.wn, c.nbuf, KTAIL, GSUM, c.split>),
                              grid, block, 0, s, p);
           done = true;
         }
       }
     }()),
     ...);
  }(std::make_integer_sequence<int, 7>{});
  return done ? hipGetLastError() : hipErrorInvalidValue;
}

// p.tiles_n counts tiles of tile_out_cols(tile, epi) columns.
template <int LAYOUT>
hipError_t launch_bf16_layout_tile(int tile, const GemmParams& p, Epilogue epi, bool gsum,
                                   hipStream_t s) {
  const bool ktail = p.K % 32 != 0;
  hipError_t r = hipErrorInvalidValue;
  [&]<int... t>(std::integer_sequence<int, t...>) {
    (([&] {
       if (tile != t) return;
       if (ktail) {
         if constexpr (t == kTailTile || t == kTailTileSwiGLU) {
           if (gsum) r = launch_bf16_tile<LAYOUT, t, true, true>(p, epi, s);
           else r = launch_bf16_tile<LAYOUT, t, true, false>(p, epi, s);
         }
       } else if (gsum) {
         r = launch_bf16_tile<LAYOUT, t, false, true>(p, epi, s);
       } else {
         r = launch_bf16_tile<LAYOUT, t, false, false>(p, epi, s);
       }
     }()),
     ...);
  }(std::make_integer_sequence<int, kNumTiles>{});
  return r;
}

// Per-layout entry points (one translation unit each).
hipError_t launch_bf16_nn(int tile, const GemmParams& p, Epilogue epi, bool gsum, hipStream_t s);
hipError_t launch_bf16_nt(int tile, const GemmParams& p, Epilogue epi, bool gsum, hipStream_t s);
hipError_t launch_bf16_tn(int tile, const GemmParams& p, Epilogue epi, bool gsum, hipStream_t s);
// Launch with an explicit tile, and the tile the library picks.
hipError_t launch_gemm_bf16_tile(int tile, const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_bf16_batch_tile(int tile, const GemmBatch& b, hipStream_t s);
int pick_bf16_tile(Layout layout, int64_t M, int64_t N, int64_t K, int groups, bool group_sum);

}  // namespace tpmlp
