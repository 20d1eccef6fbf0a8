// gfx950 (MI355X, CDNA4) kernels of the tensor-parallel MLP shard forward.
//
//   gemm_bf16_kernel  C[M,N] = epilogue(A[M,K] B[K,N]), bf16 operands on the
//                     v_mfma_f32_32x32x16_bf16 matrix cores, fp32 accumulate.
//   gemm_f32_kernel   the same contraction with float32 operands on
//                     v_mfma_f32_16x16x4_f32.
//   shard_reduce_kernel  Z = sum_i Z_i over fp32 partials, streaming.
//
// The column-parallel step Y_i = GeLU(X W_i + b_i) is a GEMM with the bias +
// GeLU epilogue; the row-parallel step Z_i = Y_i V_i is a GEMM with an fp32
// store (or, fused, an fp32 read-add-store into Z).  Both weights arrive
// [in, out] row-major, i.e. B is K x N with N contiguous.
#include "tp_mlp_kernels.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tpmlp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kNumXcd = 8;  // MI355X: 8 XCDs of 32 CUs, each XCD with its own L2

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even float -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}

// GeLU(x) = x * Phi(x) with Phi(x) = erfc(-x / sqrt 2) / 2 (the erf form of
// GeLU, not the tanh approximation).
//
// erfc(z), z >= 0, follows Abramowitz & Stegun, Handbook of Mathematical
// Functions (1964), formula 7.1.26 (after Hastings):
//   erfc(z) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2) + e(z),
//   t = 1 / (1 + p z),  |e(z)| <= 1.5e-7,
// with p = 0.3275911, a1..a5 = 0.254829592, -0.284496736, 1.421413741,
// -1.453152027, 1.061405429.  Here z = |x| / sqrt 2, the factor 1/2 of Phi is
// folded into the a_i, h = erfc(z) / 2 = Phi(-|x|), and Phi(x) = h for x < 0,
// 1 - h otherwise.  The reciprocal and exp2 run on the hardware
// transcendental unit; the whole function is branch-free (about 20 VALU
// operations), which matters because it runs once per element of Y_i.
__device__ __forceinline__ float gelu_f32(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  float q = fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
  q = fmaf(t, q, 0.5f * 1.421413741f);
  q = fmaf(t, q, 0.5f * -0.284496736f);
  q = fmaf(t, q, 0.5f * 0.254829592f);
  q *= t;
  const float e = __builtin_amdgcn_exp2f((z * -1.4426950408889634f) * z);  // exp(-z^2)
  const float h = q * e;
  return x * (x < 0.0f ? h : 1.0f - h);
}

// Map the linear workgroup id to a (tile_m, tile_n) pair.  Workgroups are
// dispatched round-robin over the 8 XCDs, so ids are first regrouped so that
// each XCD receives a contiguous range of logical tiles, and logical tiles are
// walked in column strips of `kGroupM` tile rows so that the tiles resident on
// one XCD at a time share rows of A and columns of B in that XCD's L2.
template <int kGroupM>
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int bid = blockIdx.x;
  const int nb = gridDim.x;
  const int full = nb - nb % kNumXcd;
  int logical = bid;
  if (bid < full) logical = (bid % kNumXcd) * (full / kNumXcd) + bid / kNumXcd;
  const int group = kGroupM * tiles_n;
  const int g = logical / group;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int local = logical - g * group;
  tm = first_m + local % gm;
  tn = local / gm;
}

// ---------------------------------------------------------------------------
// bf16 GEMM.
//
// Workgroup tile BM x BN, K step 64, WM x WN waves, each wave a (BM/WM) x
// (BN/WN) block of 32x32 tiles of v_mfma_f32_32x32x16_bf16.  LDS holds two stages (double buffer) of
//   As: [BM rows][64 k]  — rows of A as they are in memory,
//   Bs: [BN rows][64 k]  — B transposed, so that a column of B (one output
//                          column, 64 consecutive k) is contiguous.
// A row of either is eight 16-byte chunks of 8 k-values; chunk c of row r is
// stored at chunk position c ^ swz(r) (see swz), which keeps the LDS stores
// and the MFMA operand reads free of bank conflicts and makes the
// operand-read address of fragment i a constant offset from fragment 0's.
//
// Global loads are raw buffer loads: a lane whose chunk lies outside the
// matrix (partial tiles in M, N or K) is given an out-of-range offset and the
// hardware returns zeros, so edge tiles need no branches in the K loop.
//
// B (K x N, N contiguous) is transposed on the way into LDS: each thread reads
// an 8(k) x 8(n) block as eight 16-byte row segments and shuffles it in
// registers into eight 8(k)-long column segments.  Consecutive lanes take
// consecutive k-blocks of one column block, so each 8-lane group writes one
// LDS row at eight distinct chunk positions; odd column blocks write their
// columns in the order nn ^ 1, so the two 8-lane halves of a 16-lane group
// write rows of opposite parity (the other half of the banks).
//
// MFMA operand order: the B-fragment goes in the instruction's A slot and the
// A-fragment in its B slot, so the instruction computes the transposed tile
// and each lane ends up owning runs of 4 consecutive output columns of one
// row (16-byte fp32 / 8-byte bf16 stores).
// ---------------------------------------------------------------------------
constexpr uint32_t kOob = 0x80000000u;  // buffer offset that is always out of range

// LDS chunk swizzle of row r (rows of 128 bytes, eight 16-byte chunks).  A
// 16-byte access is served per group of 16 lanes over 64 banks, i.e. sixteen
// 16-byte slots = (row parity, chunk position).  f(r) = (r & 7) ^ ((r >> 3) & 1)
// is a permutation of the 8 positions within every 8 aligned rows and makes
// (r & 1, f(r)) distinct over every 16 aligned rows, so the fragment reads
// (16 consecutive rows, one logical chunk) and the row stores (two rows,
// eight chunks per 16 lanes) are conflict-free; f(r + 32 i) = f(r).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // gfx9 raw buffer: stride 0, num_records = bytes, dword3 = 0x00020000.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <int BM, int BN, int WM, int WN, int EPI, bool EDGE>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const uint16_t* __restrict__ bias, void* __restrict__ C, int M, int N, int K, int tiles_m,
    int tiles_n) {
  constexpr int BK = 64;
  constexpr int CH = BK / 8;  // 16-byte chunks per LDS row
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;      // 32x32 MFMA tiles per wave
  constexpr int A_LD = BM * CH / NT;               // A chunks per thread per stage
  constexpr int NBLK = CH * (BN / 8);              // 8x8 B blocks per stage
  constexpr int B_LD = (NBLK + NT - 1) / NT;       // ... per thread (the last round may be partial)
  constexpr int STAGE = (BM + BN) * BK;            // elements per LDS stage
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert((BM * CH) % NT == 0 && NT % CH == 0, "loader shape");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  int tm, tn;
  tile_coords<8>(tiles_m, tiles_n, tm, tn);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(A, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(B, (uint32_t)K * (uint32_t)N * 2u);

  // A loader: chunk c = tid % 8 of rows i * (NT / 8) + tid / 8.
  const int a_c = tid % CH;
  const int a_r = tid / CH;
  // B loader: k-block kb = blk % 8 and column block nb = blk / 8 of blk = i * NT + tid.
  const int b_kb = tid % CH;

  // Two register sets stage global data on its way to LDS: stage j lives in
  // set j & 1 from its load until its LDS store one pipeline step later.
  u32x4_t ra[2][A_LD];
  u32x4_t rb[2][B_LD][8];

  // Interior tiles (EDGE == false: M, N and K are whole multiples of the
  // tile) keep their per-lane buffer offsets in loop-invariant registers and
  // advance along K through the scalar offset, so a global load costs no VALU.
  // Edge tiles compute a masked offset per load.
  const int nk = (K + BK - 1) / BK;
  uint32_t a_voff[A_LD], b_voff[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i)
    a_voff[i] = ((uint32_t)(m0 + i * (NT / CH) + a_r) * (uint32_t)K + (uint32_t)(a_c * 8)) * 2u;
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int blk = i * NT + tid;
    b_voff[i] = blk < NBLK ? ((uint32_t)(b_kb * 8) * (uint32_t)N + (uint32_t)(n0 + (blk / CH) * 8)) * 2u
                           : kOob;
  }

  auto load_stage = [&](auto set, int k0) {
    constexpr int q = decltype(set)::value;
    if constexpr (!EDGE) {
      // Past the last K step, reload the last one (its data is never used).
      const int kc = min(k0, (nk - 1) * BK);
#pragma unroll
      for (int i = 0; i < A_LD; ++i)
        ra[q][i] = __builtin_amdgcn_raw_buffer_load_b128(rsA, (int)a_voff[i], kc * 2, 0);
#pragma unroll
      for (int i = 0; i < B_LD; ++i)
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          rb[q][i][kk] = __builtin_amdgcn_raw_buffer_load_b128(
              rsB, (int)b_voff[i], (int)((uint32_t)(kc + kk) * (uint32_t)N * 2u), 0);
    } else {
      const bool kin = k0 + a_c * 8 < K;
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const int gm = m0 + i * (NT / CH) + a_r;
        const uint32_t off =
            (gm < M && kin) ? ((uint32_t)gm * (uint32_t)K + (uint32_t)(k0 + a_c * 8)) * 2u : kOob;
        ra[q][i] = __builtin_amdgcn_raw_buffer_load_b128(rsA, (int)off, 0, 0);
      }
      const int gk = k0 + b_kb * 8;
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const int blk = i * NT + tid;
        const int gn = n0 + (blk / CH) * 8;
        const bool ok = blk < NBLK && gk < K && gn < N;
        const uint32_t off = ok ? ((uint32_t)gk * (uint32_t)N + (uint32_t)gn) * 2u : kOob;
        const uint32_t step = ok ? (uint32_t)N * 2u : 0u;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          rb[q][i][kk] = __builtin_amdgcn_raw_buffer_load_b128(rsB, (int)(off + kk * step), 0, 0);
      }
    }
  };

  // v_perm selectors: even columns take the low halves of a k-row pair, odd
  // columns the high halves; lanes of odd column blocks swap the two.
  const uint32_t g_odd = (tid >> 3) & 1;
  const uint32_t sel_even = g_odd ? 0x07060302u : 0x05040100u;
  const uint32_t sel_odd = g_odd ? 0x05040100u : 0x07060302u;

  auto store_stage = [&](auto set, int buf) {
    constexpr int q = decltype(set)::value;
    uint16_t* As = smem + buf * STAGE;
    uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int blk = i * NT + tid;
      if (NBLK % NT != 0 && blk >= NBLK) continue;
      const int nb = blk / CH;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int p = t >> 1;
        const uint32_t sel = (t & 1) ? sel_odd : sel_even;
        u32x4_t col;
#pragma unroll
        for (int j = 0; j < 4; ++j)  // k = 2j (low half of the pair), 2j + 1 (high half)
          col[j] = __builtin_amdgcn_perm(rb[q][i][2 * j + 1][p], rb[q][i][2 * j][p], sel);
        const int n = nb * 8 + (t ^ (int)g_odd);
        *reinterpret_cast<u32x4_t*>(Bs + n * BK + ((b_kb ^ swz(n)) * 8)) = col;
      }
    }
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int r = i * (NT / CH) + a_r;
      *reinterpret_cast<u32x4_t*>(As + r * BK + ((a_c ^ swz(r)) * 8)) = ra[q][i];
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Operand-read offsets (elements) of fragment 0 for each 16-wide k step: a
  // 32x32x16 fragment gives lane l row (l & 31) and k-chunk 2 * ks + (l >> 5).
  const int l32 = lane & 31;
  const int a_row = wm * WTM + l32;
  const int b_row = wn * WTN + l32;
  int a_off[BK / 16], b_off[BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int c = ks * 2 + (lane >> 5);
    a_off[ks] = a_row * BK + ((c ^ swz(a_row)) * 8);
    b_off[ks] = BM * BK + b_row * BK + ((c ^ swz(b_row)) * 8);
  }

  // Fragments double-buffered in registers: F[f] holds one k16 step.
  bf16x8_t fa[2][FM], fb[2][FN];
  auto read_frags = [&](auto fset, int buf, int ks) {
    constexpr int f = decltype(fset)::value;
    const uint16_t* S = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[f][i] = *reinterpret_cast<const bf16x8_t*>(S + a_off[ks] + i * 32 * BK);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[f][j] = *reinterpret_cast<const bf16x8_t*>(S + b_off[ks] + j * 32 * BK);
  };
  auto mfmas = [&](auto fset) {
    constexpr int f = decltype(fset)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[f][j], fa[f][i], acc[i][j], 0, 0, 0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // Pipeline over K steps of 64.  In step kt (LDS buffer P = kt & 1 holds
  // stage kt, register set Q = P ^ 1 holds stage kt + 1):
  //   k16 step 0: read fragments of step 1; MFMAs of step 0; store set Q to
  //               LDS buffer Q (stage kt + 1; that buffer was last read in
  //               step kt - 1, before the barrier that ended it);
  //   k16 step 1: read step 2; MFMAs; load stage kt + 3 into set Q;
  //   k16 step 2: read step 3; MFMAs;
  //   k16 step 3: wait for this wave's LDS traffic, barrier (now stage kt + 1
  //               is complete in buffer Q and nobody reads buffer P any more),
  //               read step 0 of stage kt + 1 from buffer Q while the MFMAs of
  //               step 3 run.
  // Loads past the end of K fetch data that is never consumed, so every step
  // runs the same branch-free body.
  load_stage(I0{}, 0);
  load_stage(I1{}, BK);
  store_stage(I0{}, 0);
  load_stage(I0{}, 2 * BK);
  __syncthreads();
  read_frags(I0{}, 0, 0);

  // Instruction interleaving inside each k16 phase (the scheduler would
  // otherwise sink every fragment read down to its first MFMA): the next
  // step's fragment reads go first, then each MFMA is followed by its share of
  // the phase's LDS stores or global loads and the VALU work that feeds them.
  constexpr int kMfma = FM * FN;
  constexpr int kFragReads = FM + FN;
  constexpr int kDsWrites = A_LD + (NBLK >= NT ? B_LD * 8 : 8);
  constexpr int kVmemReads = A_LD + B_LD * 8;
  constexpr int kWritesPerMfma = (kDsWrites + kMfma - 1) / kMfma;
  constexpr int kReadsPerMfma = (kVmemReads + kMfma - 1) / kMfma;
  // Each MFMA is followed by one fragment read of the next k16 step (so the
  // reads never delay the MFMAs that precede them) and by its share of the
  // phase's LDS stores or global loads and the VALU work that feeds them.
  auto order_plain = [&]() {
#pragma unroll
    for (int m = 0; m < kMfma; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // MFMA
      if (m < kFragReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
  };
  auto order_store = [&]() {
#pragma unroll
    for (int m = 0; m < kMfma; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m < kFragReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);               // VALU
      __builtin_amdgcn_sched_group_barrier(0x200, kWritesPerMfma, 0);  // DS writes
    }
  };
  auto order_load = [&]() {
#pragma unroll
    for (int m = 0; m < kMfma; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m < kFragReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, kReadsPerMfma, 0);  // VMEM reads
    }
  };

  auto step = [&](auto pset, int kt) {
    constexpr int P = decltype(pset)::value;
    using Q = std::integral_constant<int, P ^ 1>;
    read_frags(I1{}, P, 1);
    mfmas(I0{});
    store_stage(Q{}, P ^ 1);
    order_store();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(I0{}, P, 2);
    mfmas(I1{});
    load_stage(Q{}, (kt + 3) * BK);
    order_load();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(I1{}, P, 3);
    mfmas(I0{});
    order_plain();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    read_frags(I0{}, P ^ 1, 0);
    mfmas(I1{});
    order_plain();
    __builtin_amdgcn_sched_barrier(0);
  };
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(I0{}, kt);
    step(I1{}, kt + 1);
  }
  if (kt < nk) step(I0{}, kt);

  // Epilogue.  With the operands swapped, lane l owns row (l & 31) of each
  // 32x32 tile and, for g = 0..3, the 4 consecutive columns 8g + 4(l >> 5) .. +3.
  const int hcol = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm * WTM + i * 32 + l32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn * WTN + j * 32 + 8 * g + hcol;
        if (n >= N) continue;
        f32x4_t v = f32x4_t{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                            acc[i][j][4 * g + 3]};
        if constexpr (EPI == kEpiBiasGelu) {
          if (bias) {
            const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(bias + n);
            v[0] += bf16_bits_to_f32(bb[0] & 0xFFFFu);
            v[1] += bf16_bits_to_f32(bb[0] >> 16);
            v[2] += bf16_bits_to_f32(bb[1] & 0xFFFFu);
            v[3] += bf16_bits_to_f32(bb[1] >> 16);
          }
          u32x2_t o;
          o[0] = f32_to_bf16_bits(gelu_f32(v[0])) | (f32_to_bf16_bits(gelu_f32(v[1])) << 16);
          o[1] = f32_to_bf16_bits(gelu_f32(v[2])) | (f32_to_bf16_bits(gelu_f32(v[3])) << 16);
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(C) + m * N + n) = o;
        } else if constexpr (EPI == kEpiStoreF32) {
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(C) + m * N + n) = v;
        } else {
          f32x4_t* p = reinterpret_cast<f32x4_t*>(static_cast<float*>(C) + m * N + n);
          const f32x4_t old = *p;
          *p = old + v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 GEMM, direct-to-LDS pipeline (interior tiles: M, N, K whole multiples
// of BM, BN, 32).
//
// Eight waves per workgroup (two per SIMD, so one wave's MFMAs cover the
// other's stalls), each owning a (BM/WM) x (BN/WN) block of 32x32 tiles.
// K advances 32 per stage through 4 LDS stages with a prefetch distance of 3:
// global data goes straight into LDS with `buffer_load_dwordx4 ... lds`
// (lane l of a wave instruction fills bytes 16 l .. 16 l + 15 of a 1 KB LDS
// block, so the swizzle is applied by choosing which global chunk each lane
// fetches), with no staging registers and no LDS store instructions.
//
// LDS layout of a stage:
//   A: [BM rows][32 k], 64-byte rows; chunk c (8 k-values) of row r at
//      position c ^ swzA4(r).
//   B: [32 k rows][BN n], BN*2-byte rows (row-major, as in memory); chunk c
//      (8 n-values) of row k at position c ^ swzB(k).
// A fragments are 16-byte reads of a row; B fragments are two
// ds_read_b64_tr_b16 transpose reads: within each 16-lane group, lane t
// points at 4 consecutive n of row k0 + t / 4 (columns n0 + 4 (t % 4)) and
// receives column n0 + t for rows k0 .. k0 + 3, i.e. 4 k-values of one
// output column, which is exactly half of a 32x32x16 B fragment.  Both
// swizzles make the fragment reads free of bank conflicts.
//
// One barrier per stage, placed before the MFMAs of the stage's last k16
// step, so the next stage's first fragment reads overlap those MFMAs.  The
// barrier is a bare s_barrier after an explicit wait for this wave's loads
// of the next stage only (a full workgroup fence would also wait for the
// loads of the two stages still in flight).
// ---------------------------------------------------------------------------
typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swzA4(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
__device__ __forceinline__ int swzB(int k) { return 4 * (k & 3); }

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// gfx9 raw buffer descriptor (stride 0, num_records = bytes) as four SGPRs.
__device__ __forceinline__ i32x4_t buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4_t{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}

// 16 bytes per lane from global memory straight into LDS: lane l's data lands
// at LDS byte address `lds + 16 l` (lds is wave-uniform); out-of-range lanes
// write zeros.  Written as inline assembly so that the compiler does not track
// the LDS write itself: its conservative alias tracking of in-flight LDS DMA
// would otherwise insert vmcnt(0) waits before fragment reads of other stage
// buffers.  Completion is waited for explicitly (vmcnt) before the barrier
// that publishes a stage; the "memory" clobber keeps LDS accesses in order
// around it.  M0 is set here for the instruction; no compiler-generated code
// in the kernels that use this relies on M0.
__device__ __forceinline__ void lds_dma16(i32x4_t desc, char* lds, uint32_t voff, uint32_t soff) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(desc), "s"(__builtin_amdgcn_readfirstlane(soff))
      : "memory", "m0");
}

__device__ __forceinline__ bf16x8_t ds_read_tr_pair(const char* p0, const char* p1) {
  const i16x4_t lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p0);
  const i16x4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p1);
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int BM, int BN, int WM, int WN, int NBUF, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_dma_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const uint16_t* __restrict__ bias, void* __restrict__ C, int M, int N, int K, int tiles_m,
    int tiles_n) {
  constexpr int BK = 32;
  constexpr int D = NBUF - 1;  // prefetch distance in K steps
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int A_PER_W = A_BYTES / 1024 / NW, B_PER_W = B_BYTES / 1024 / NW;
  constexpr int L = A_PER_W + B_PER_W;               // DMA instructions per wave per stage
  constexpr int B_ROW = BN * 2;                      // bytes per B row in LDS
  constexpr int B_LANES_PER_ROW = BN / 8;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "DMA split");
  static_assert(BN % 128 == 0 && BN <= 512, "B swizzle needs 16-chunk groups");
  static_assert(NBUF >= 3 && NBUF <= 6, "stage count");
  static_assert((D - 1) * L <= 63, "vmcnt immediate");
  static_assert(NBUF * STAGE <= 160 * 1024, "LDS");

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

  int tm, tn;
  tile_coords<8>(tiles_m, tiles_n, tm, tn);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int nk = K / BK;

  const i32x4_t rsA = buffer_desc(A, (uint32_t)M * (uint32_t)K * 2u);
  const i32x4_t rsB = buffer_desc(B, (uint32_t)K * (uint32_t)N * 2u);

  // Global byte offsets (loop-invariant) of the chunk each lane fetches for
  // its wave's DMA instructions; K advances through the scalar offset.
  uint32_t a_src[A_PER_W], b_src[B_PER_W];
#pragma unroll
  for (int i = 0; i < A_PER_W; ++i) {
    const int row = (wave * A_PER_W + i) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swzA4(row);
    a_src[i] = ((uint32_t)(m0 + row) * (uint32_t)K + (uint32_t)(c * 8)) * 2u;
  }
#pragma unroll
  for (int i = 0; i < B_PER_W; ++i) {
    const int row = (wave * B_PER_W + i) * (1024 / B_ROW) + lane / B_LANES_PER_ROW;
    const int c = (lane % B_LANES_PER_ROW) ^ swzB(row);
    b_src[i] = ((uint32_t)row * (uint32_t)N + (uint32_t)(n0 + c * 8)) * 2u;
  }
  auto issue_stage = [&](auto bset, int kt) {
    const bool live = kt < nk;  // past the end: out-of-range loads (no traffic), never read
    const uint32_t k0 = (uint32_t)(live ? kt : 0) * BK;
    char* base = stage(bset);
#pragma unroll
    for (int i = 0; i < A_PER_W; ++i)
      lds_dma16(rsA, base + (wave * A_PER_W + i) * 1024, live ? a_src[i] : kOob, k0 * 2u);
#pragma unroll
    for (int i = 0; i < B_PER_W; ++i)
      lds_dma16(rsB, base + A_BYTES + (wave * B_PER_W + i) * 1024, live ? b_src[i] : kOob,
                k0 * (uint32_t)N * 2u);
  };

  // Fragment read offsets within a stage (bytes).
  const int l32 = lane & 31;
  const int a_row = wm * WTM + l32;
  int a_off[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    a_off[ks] = a_row * 64 + ((2 * ks + (lane >> 5)) ^ swzA4(a_row)) * 16;
  const int g = lane >> 4, t = lane & 15;
  const int b_krow = 8 * (g >> 1) + (t >> 2);  // + 16 ks + 4 h
  int b_off[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = wn * WTN + 32 * j + 16 * (g & 1) + 4 * (t & 3);
    b_off[j] = A_BYTES + b_krow * B_ROW + (((n >> 3) ^ swzB(b_krow)) * 16) + ((n >> 2) & 1) * 8;
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8_t fa[2][FM], fb[2][FN];
  auto read_frags = [&](auto fset, auto bset, int ks) {
    constexpr int f = decltype(fset)::value;
    const char* S = stage(bset);
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[f][i] = *reinterpret_cast<const bf16x8_t*>(S + a_off[ks] + i * 32 * 64);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const char* p = S + b_off[j] + ks * 16 * B_ROW;
      fb[f][j] = ds_read_tr_pair(p, p + 4 * B_ROW);
    }
  };
  auto mfmas = [&](auto fset) {
    constexpr int f = decltype(fset)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[f][j], fa[f][i], acc[i][j], 0, 0, 0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  constexpr int kMfma = FM * FN;
  constexpr int kReads = FM + 2 * FN;
  // vmcnt((D - 1) L), expcnt(7), lgkmcnt(0): this wave's loads of the next
  // stage (all but the D - 1 younger stages) and all its LDS reads are done.
  constexpr int kWaitN = (D - 1) * L;
  constexpr int kWaitNext = (kWaitN & 15) | ((kWaitN >> 4) << 14) | (7 << 4);
  constexpr int kWaitFirst = kWaitNext;

  using B0 = std::integral_constant<int, 0>;
  [&]<int... b>(std::integer_sequence<int, b...>) {
    (issue_stage(std::integral_constant<int, b>{}, b), ...);
  }(std::make_integer_sequence<int, D>{});
  __builtin_amdgcn_s_waitcnt(kWaitFirst);
  asm volatile("s_barrier" ::: "memory");
  read_frags(I0{}, B0{}, 0);

  // One K step of 32 on stage buffer C (static, so that every LDS access
  // names its buffer at compile time).
  auto kstep = [&](auto cset, int kt) {
    constexpr int c = decltype(cset)::value;
    using Refill = std::integral_constant<int, (c + D) % NBUF>;
    using Next = std::integral_constant<int, (c + 1) % NBUF>;
    // k16 step 0: refill the buffer freed by stage kt - 1 with stage kt + D,
    // read step 1's fragments, MFMAs of step 0.
    issue_stage(Refill{}, kt + D);
    read_frags(I1{}, cset, 1);
    mfmas(I0{});
#pragma unroll
    for (int m = 0; m < kMfma; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (m < L) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // k16 step 1: once stage kt + 1 has landed for every wave, read its step
    // 0 fragments while the MFMAs of step 1 run.
    __builtin_amdgcn_s_waitcnt(kWaitNext);
    asm volatile("s_barrier" ::: "memory");
    read_frags(I0{}, Next{}, 0);
    mfmas(I1{});
#pragma unroll
    for (int m = 0; m < kMfma; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // The loop body walks the NBUF buffers in order; an early exit handles a
  // step count that is not a multiple of NBUF (uniform across the workgroup).
  for (int kt = 0; kt < nk; kt += NBUF) {
    bool more = true;
    [&]<int... b>(std::integer_sequence<int, b...>) {
      ((more = more && (kt + b < nk), more ? (kstep(std::integral_constant<int, b>{}, kt + b), 0) : 0), ...);
    }(std::make_integer_sequence<int, NBUF>{});
  }
  // The last D stages' loads (out of range, writing zeros) must have landed
  // before this workgroup's LDS can be handed to another.
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)

  const int hcol = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm * WTM + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int64_t n = n0 + wn * WTN + j * 32 + 8 * gq + hcol;
        f32x4_t v = f32x4_t{acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                            acc[i][j][4 * gq + 3]};
        if constexpr (EPI == kEpiBiasGelu) {
          if (bias) {
            const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(bias + n);
            v[0] += bf16_bits_to_f32(bb[0] & 0xFFFFu);
            v[1] += bf16_bits_to_f32(bb[0] >> 16);
            v[2] += bf16_bits_to_f32(bb[1] & 0xFFFFu);
            v[3] += bf16_bits_to_f32(bb[1] >> 16);
          }
          u32x2_t o;
          o[0] = f32_to_bf16_bits(gelu_f32(v[0])) | (f32_to_bf16_bits(gelu_f32(v[1])) << 16);
          o[1] = f32_to_bf16_bits(gelu_f32(v[2])) | (f32_to_bf16_bits(gelu_f32(v[3])) << 16);
          *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(C) + m * N + n) = o;
        } else if constexpr (EPI == kEpiStoreF32) {
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(C) + m * N + n) = v;
        } else {
          f32x4_t* p = reinterpret_cast<f32x4_t*>(static_cast<float*>(C) + m * N + n);
          const f32x4_t old = *p;
          *p = old + v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32 GEMM: 64 x 64 workgroup tile, K step 16, 4 waves of 32 x 32, each a
// 2 x 2 block of v_mfma_f32_16x16x4_f32 tiles.  LDS holds A transposed
// ([k][m]) and B as is ([k][n]) so that both MFMA operands are read as
// consecutive words across lanes.
// ---------------------------------------------------------------------------
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B,
                                                       const float* __restrict__ bias,
                                                       void* __restrict__ C, int M, int N, int K,
                                                       int tiles_m, int tiles_n) {
  constexpr int BM = 64, BN = 64, BK = 16, PAD = 4;
  __shared__ __attribute__((aligned(16))) float As[BK][BM + PAD];
  __shared__ __attribute__((aligned(16))) float Bs[BK][BN + PAD];

  int tm, tn;
  tile_coords<8>(tiles_m, tiles_n, tm, tn);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int ar = tid >> 2, ac = (tid & 3) * 4;     // A: row, first k of a float4
  const int bk = tid >> 4, bc = (tid & 15) * 4;    // B: k, first n of a float4
  for (int k0 = 0; k0 < K; k0 += BK) {
    f32x4_t va = f32x4_t{0.f, 0.f, 0.f, 0.f}, vb = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (m0 + ar < M && k0 + ac < K)
      va = *reinterpret_cast<const f32x4_t*>(A + (m0 + ar) * K + k0 + ac);
    if (k0 + bk < K && n0 + bc < N)
      vb = *reinterpret_cast<const f32x4_t*>(B + (int64_t)(k0 + bk) * N + n0 + bc);
#pragma unroll
    for (int j = 0; j < 4; ++j) As[ac + j][ar] = va[j];
    *reinterpret_cast<f32x4_t*>(&Bs[bk][bc]) = vb;
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < BK / 4; ++kq) {
      const int kk = kq * 4 + (lane >> 4);
      float a_op[2], b_op[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) a_op[j] = Bs[kk][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i) b_op[i] = As[kk][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_op[j], b_op[i], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + wm * 32 + i * 16 + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 32 + j * 16 + 4 * (lane >> 4);
      if (n >= N) continue;
      f32x4_t v = acc[i][j];
      if constexpr (EPI == kEpiBiasGelu) {
        if (bias) v += *reinterpret_cast<const f32x4_t*>(bias + n);
        f32x4_t y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = gelu_f32(v[e]);
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(C) + m * N + n) = y;
      } else if constexpr (EPI == kEpiStoreF32) {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(C) + m * N + n) = v;
      } else {
        f32x4_t* p = reinterpret_cast<f32x4_t*>(static_cast<float*>(C) + m * N + n);
        const f32x4_t old = *p;
        *p = old + v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Shard reduce: Z = ((P_0 + P_1) + P_2) + ... in float32, 16-byte vectors,
// grid-stride.  KC > 0 fixes k at compile time so that all k loads of a
// vector are in flight together; KC == 0 reads k at run time.
// ---------------------------------------------------------------------------
struct PartPtrs {
  const float* p[64];
};

// U 16-byte vectors per thread per iteration, all 1 + (k - 1) loads of them
// issued before the adds, so that each thread keeps U * k loads in flight.
template <int KC, int U>
__global__ __launch_bounds__(256) void shard_reduce_kernel(PartPtrs parts, int k,
                                                           float* __restrict__ Z, int64_t n) {
  const int kk = KC > 0 ? KC : k;
  const int64_t n4 = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * U;
  for (int64_t v0 = ((int64_t)blockIdx.x * blockDim.x) * U + threadIdx.x; v0 < n4; v0 += stride) {
    f32x4_t s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + (int64_t)u * blockDim.x;
      s[u] = v < n4 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(parts.p[0]) + v)
                    : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (KC > 0) {
      f32x4_t t[KC > 1 ? KC - 1 : 1][U];
#pragma unroll
      for (int i = 1; i < KC; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + (int64_t)u * blockDim.x;
          t[i - 1][u] = v < n4 ? __builtin_nontemporal_load(
                                     reinterpret_cast<const f32x4_t*>(parts.p[i]) + v)
                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int i = 1; i < KC; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) s[u] = s[u] + t[i - 1][u];
    } else {
      for (int i = 1; i < kk; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + (int64_t)u * blockDim.x;
          if (v < n4)
            s[u] = s[u] + __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(parts.p[i]) + v);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + (int64_t)u * blockDim.x;
      if (v < n4) __builtin_nontemporal_store(s[u], reinterpret_cast<f32x4_t*>(Z) + v);
    }
  }
  // scalar tail (n not a multiple of 4)
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t e = (n4 << 2) + threadIdx.x;
    float s = parts.p[0][e];
    for (int i = 1; i < kk; ++i) s = s + parts.p[i][e];
    Z[e] = s;
  }
}

template <int U>
hipError_t launch_reduce_u(const PartPtrs& pp, int k, float* Z, int64_t n, int64_t max_blocks,
                           hipStream_t s) {
  const int64_t n4 = n >> 2;
  int64_t blocks = (n4 + 256 * U - 1) / (256 * U);
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(256);
  switch (k) {
    case 1: hipLaunchKernelGGL((shard_reduce_kernel<1, U>), grid, block, 0, s, pp, k, Z, n); break;
    case 2: hipLaunchKernelGGL((shard_reduce_kernel<2, U>), grid, block, 0, s, pp, k, Z, n); break;
    case 4: hipLaunchKernelGGL((shard_reduce_kernel<4, U>), grid, block, 0, s, pp, k, Z, n); break;
    case 8: hipLaunchKernelGGL((shard_reduce_kernel<8, U>), grid, block, 0, s, pp, k, Z, n); break;
    default: hipLaunchKernelGGL((shard_reduce_kernel<0, U>), grid, block, 0, s, pp, k, Z, n); break;
  }
  return hipGetLastError();
}

hipError_t launch_shard_reduce_cfg(const float* const* parts, int k, float* Z, int64_t n, int unroll,
                                   int64_t max_blocks, hipStream_t s) {
  PartPtrs pp;
  for (int i = 0; i < 64; ++i) pp.p[i] = i < k ? parts[i] : nullptr;
  switch (unroll) {
    case 1: return launch_reduce_u<1>(pp, k, Z, n, max_blocks, s);
    case 2: return launch_reduce_u<2>(pp, k, Z, n, max_blocks, s);
    default: return launch_reduce_u<4>(pp, k, Z, n, max_blocks, s);
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_bf16_cfg(const uint16_t* A, const uint16_t* B, const uint16_t* bias, void* C,
                           int64_t M, int64_t N, int64_t K, Epilogue epi, hipStream_t s) {
  // Buffer offsets are 32-bit: launch row blocks of A of at most 2^31 bytes.
  const int64_t rows_per_launch = ((int64_t(1) << 31) / (K * 2)) / BM * BM;
  const size_t c_elt = epi == kEpiBiasGelu ? 2 : 4;
  for (int64_t r0 = 0; r0 < M; r0 += rows_per_launch) {
    const int64_t Mc = M - r0 < rows_per_launch ? M - r0 : rows_per_launch;
    const uint16_t* Ac = A + r0 * K;
    void* Cc = static_cast<char*>(C) + size_t(r0) * size_t(N) * c_elt;
    const int tiles_m = (int)((Mc + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid(tiles_m * tiles_n), block(WM * WN * 64);
    const bool edge = (Mc % BM) || (N % BN) || (K % 64);
#define TPMLP_LAUNCH_BF16(E, G)                                                              \
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, E, G>), grid, block, 0, s, Ac, B, bias, \
                     Cc, (int)Mc, (int)N, (int)K, tiles_m, tiles_n)
    switch (epi) {
      case kEpiBiasGelu:
        if (edge) TPMLP_LAUNCH_BF16(kEpiBiasGelu, true); else TPMLP_LAUNCH_BF16(kEpiBiasGelu, false);
        break;
      case kEpiStoreF32:
        if (edge) TPMLP_LAUNCH_BF16(kEpiStoreF32, true); else TPMLP_LAUNCH_BF16(kEpiStoreF32, false);
        break;
      default:
        if (edge) TPMLP_LAUNCH_BF16(kEpiAccumF32, true); else TPMLP_LAUNCH_BF16(kEpiAccumF32, false);
        break;
    }
#undef TPMLP_LAUNCH_BF16
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BM, int BN, int WM, int WN, int NBUF>
hipError_t launch_bf16_dma(const uint16_t* A, const uint16_t* B, const uint16_t* bias, void* C,
                           int64_t M, int64_t N, int64_t K, Epilogue epi, hipStream_t s) {
  // Interior shapes only (M % BM, N % BN, K % 32 all zero: checked by the
  // caller); 32-bit buffer offsets.
  const int64_t rows_per_launch = ((int64_t(1) << 31) / (K * 2)) / BM * BM;
  const size_t c_elt = epi == kEpiBiasGelu ? 2 : 4;
  for (int64_t r0 = 0; r0 < M; r0 += rows_per_launch) {
    const int64_t Mc = M - r0 < rows_per_launch ? M - r0 : rows_per_launch;
    const uint16_t* Ac = A + r0 * K;
    void* Cc = static_cast<char*>(C) + size_t(r0) * size_t(N) * c_elt;
    const int tiles_m = (int)(Mc / BM);
    const int tiles_n = (int)(N / BN);
    const dim3 grid(tiles_m * tiles_n), block(WM * WN * 64);
    switch (epi) {
      case kEpiBiasGelu:
        hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, WM, WN, NBUF, kEpiBiasGelu>), grid, block, 0,
                           s, Ac, B, bias, Cc, (int)Mc, (int)N, (int)K, tiles_m, tiles_n);
        break;
      case kEpiStoreF32:
        hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, WM, WN, NBUF, kEpiStoreF32>), grid, block, 0,
                           s, Ac, B, bias, Cc, (int)Mc, (int)N, (int)K, tiles_m, tiles_n);
        break;
      default:
        hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, WM, WN, NBUF, kEpiAccumF32>), grid, block, 0,
                           s, Ac, B, bias, Cc, (int)Mc, (int)N, (int)K, tiles_m, tiles_n);
        break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The bf16 GEMM configurations: workgroup tile, wave grid, LDS stages, kernel
// variant (direct-to-LDS for interior shapes, register-staged otherwise) and
// a relative per-tile efficiency used by the tile picker.
typedef hipError_t (*Bf16Launch)(const uint16_t*, const uint16_t*, const uint16_t*, void*, int64_t,
                                 int64_t, int64_t, Epilogue, hipStream_t);
struct Bf16Tile {
  int bm, bn;
  bool dma;
  int wgs_per_cu;  // workgroups that fit on one CU (LDS and registers)
  double eff;
  Bf16Launch launch;
};
const Bf16Tile kBf16Tiles[] = {
    {256, 256, false, 1, 1.0, launch_bf16_cfg<256, 256, 2, 2>},
    {256, 192, false, 1, 0.97, launch_bf16_cfg<256, 192, 2, 2>},
    {256, 128, false, 1, 0.88, launch_bf16_cfg<256, 128, 2, 2>},
    {256, 96, false, 1, 0.8, launch_bf16_cfg<256, 96, 4, 1>},
    {128, 128, false, 2, 0.7, launch_bf16_cfg<128, 128, 2, 2>},
    {256, 256, true, 1, 1.4, launch_bf16_dma<256, 256, 2, 4, 4>},
    {256, 256, true, 1, 1.4, launch_bf16_dma<256, 256, 2, 4, 5>},
    {256, 128, true, 1, 1.2, launch_bf16_dma<256, 128, 4, 2, 4>},
    {256, 128, true, 2, 1.2, launch_bf16_dma<256, 128, 4, 2, 3>},
    {256, 128, true, 1, 1.2, launch_bf16_dma<256, 128, 2, 4, 4>},
    {128, 256, true, 1, 1.2, launch_bf16_dma<128, 256, 2, 4, 4>},
    {128, 256, true, 2, 1.2, launch_bf16_dma<128, 256, 2, 4, 3>},
    {128, 128, true, 2, 1.0, launch_bf16_dma<128, 128, 2, 2, 4>},
    {128, 128, true, 2, 1.0, launch_bf16_dma<128, 128, 2, 4, 4>},
    {256, 256, true, 1, 1.4, launch_bf16_dma<256, 256, 2, 2, 4>},
    {256, 256, true, 1, 1.4, launch_bf16_dma<256, 256, 2, 2, 5>},
    {256, 128, true, 1, 1.2, launch_bf16_dma<256, 128, 2, 2, 4>},
    {256, 128, true, 1, 1.2, launch_bf16_dma<256, 128, 2, 2, 6>},
};
constexpr int kNumBf16Tiles = sizeof(kBf16Tiles) / sizeof(kBf16Tiles[0]);

bool tile_fits(const Bf16Tile& t, int64_t M, int64_t N, int64_t K) {
  return !t.dma || (M % t.bm == 0 && N % t.bn == 0 && K % 32 == 0);
}

hipError_t launch_bf16_tile(int tile, const uint16_t* A, const uint16_t* B, const uint16_t* bias,
                            void* C, int64_t M, int64_t N, int64_t K, Epilogue epi,
                            hipStream_t s) {
  if (tile < 0 || tile >= kNumBf16Tiles || !tile_fits(kBf16Tiles[tile], M, N, K))
    return hipErrorInvalidValue;
  return kBf16Tiles[tile].launch(A, B, bias, C, M, N, K, epi, s);
}

// Tile choice.  Interior shapes use the direct-to-LDS kernel; measured on the
// per-shard GEMMs of the five workloads (MI355X, random bf16 data):
//   * 256x256 (8 waves, 4 stages) when it fills at least two rounds of the 256
//     CUs, or 192..255 tiles (a 0.75 round still beats the smaller tiles);
//   * otherwise 128x256 with 3 stages (two workgroups per CU);
//   * otherwise 128x128 (two workgroups per CU).
// Ragged shapes use the register-staged kernel with the tile of least
// estimated time (rounds of resident workgroups x tile work / efficiency).
constexpr int kTileD256 = 5, kTileD128x256 = 11, kTileD128x128 = 13;

int pick_bf16_tile(int64_t M, int64_t N, int64_t K) {
  if (K % 32 == 0) {
    if (M % 256 == 0 && N % 256 == 0) {
      const int64_t t = (M / 256) * (N / 256);
      if (t >= 512 || (t >= 192 && t < 256)) return kTileD256;
    }
    if (M % 128 == 0 && N % 256 == 0) return kTileD128x256;
    if (M % 128 == 0 && N % 128 == 0) return kTileD128x128;
  }
  int best = 4;  // register-staged 128x128: fits every shape
  double best_t = 1e300;
  for (int t = 0; t < kNumBf16Tiles; ++t) {
    const Bf16Tile& c = kBf16Tiles[t];
    if (c.dma) continue;
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const int64_t slots = 256 * c.wgs_per_cu;
    const int64_t rounds = (tiles + slots - 1) / slots;
    const double time = double(rounds) * c.bm * c.bn * c.wgs_per_cu / c.eff;
    if (time < best_t * 0.999) {
      best_t = time;
      best = t;
    }
  }
  return best;
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, const uint16_t* bias, void* C,
                            int64_t M, int64_t N, int64_t K, Epilogue epi, hipStream_t s) {
  return launch_bf16_tile(pick_bf16_tile(M, N, K), A, B, bias, C, M, N, K, epi, s);
}

hipError_t launch_gemm_f32(const float* A, const float* B, const float* bias, void* C, int64_t M,
                           int64_t N, int64_t K, Epilogue epi, hipStream_t s) {
  const int tiles_m = (int)((M + 63) / 64);
  const int tiles_n = (int)((N + 63) / 64);
  const dim3 grid(tiles_m * tiles_n), block(256);
  switch (epi) {
    case kEpiBiasGelu:
      hipLaunchKernelGGL(gemm_f32_kernel<kEpiBiasGelu>, grid, block, 0, s, A, B, bias, C, (int)M,
                         (int)N, (int)K, tiles_m, tiles_n);
      break;
    case kEpiStoreF32:
      hipLaunchKernelGGL(gemm_f32_kernel<kEpiStoreF32>, grid, block, 0, s, A, B, bias, C, (int)M,
                         (int)N, (int)K, tiles_m, tiles_n);
      break;
    default:
      hipLaunchKernelGGL(gemm_f32_kernel<kEpiAccumF32>, grid, block, 0, s, A, B, bias, C, (int)M,
                         (int)N, (int)K, tiles_m, tiles_n);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_shard_reduce(const float* const* parts, int k, float* Z, int64_t n,
                               hipStream_t s) {
  return launch_shard_reduce_cfg(parts, k, Z, n, 4, 65536, s);
}

}  // namespace tpmlp
