// gfx950 (MI355X, CDNA4) kernels of the tensor-parallel MLP shard forward.
//
//   gemm_bf16_kernel  C[M,N] = epilogue(A[M,K] B[K,N]), bf16 operands on the
//                     v_mfma_f32_16x16x32_bf16 matrix cores, fp32 accumulate.
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

namespace tpmlp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kNumXcd = 8;  // MI355X: 8 XCDs of 32 CUs, each XCD with its own L2

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even float -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}

// GeLU(x) = x * Phi(x), Phi(x) = erfc(-x / sqrt 2) / 2 (the erf form of GeLU;
// erfc keeps the relative accuracy of Phi for negative x).
__device__ __forceinline__ float gelu_f32(float x) {
  return 0.5f * x * erfcf(-0.70710678118654752f * x);
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
// (BN/WN) block of 16x16 MFMA tiles.  LDS holds two stages (double buffer) of
//   As: [BM rows][64 k]  — rows of A as they are in memory,
//   Bs: [BN rows][64 k]  — B transposed, so that a column of B (one output
//                          column, 64 consecutive k) is contiguous.
// A row of either holds eight 16-byte chunks of 8 k-values; chunk c of row r
// is stored at chunk position c ^ swz(r), which keeps both the 16-byte stores
// and the 16-byte MFMA operand reads free of bank conflicts.
//
// B (K x N, N contiguous) is transposed on the way into LDS: each thread reads
// an 8(k) x 8(n) block as eight coalesced 16-byte row segments and shuffles it
// in registers into eight 8(k)-long column segments.
//
// MFMA operand order: the B-fragment goes in the instruction's A slot and the
// A-fragment in its B slot, so the instruction computes the transposed tile
// and each lane ends up owning 4 consecutive output columns of one row
// (16-byte fp32 / 8-byte bf16 stores).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const uint16_t* __restrict__ bias, void* __restrict__ C, int M, int N, int K, int tiles_m,
    int tiles_n) {
  constexpr int BK = 64;
  constexpr int CH = BK / 8;  // 16-byte chunks per LDS row
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_LD = BM * CH / NT;               // A chunks per thread per stage
  constexpr int NBLK = (BK / 8) * (BN / 8);        // 8x8 B blocks per stage
  constexpr int B_LD = (NBLK + NT - 1) / NT;        // ... per thread (the last round may be partial)
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert((BM * CH) % NT == 0 && (NBLK % NT == 0 || NBLK < NT), "loader shape");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * BK];

  int tm, tn;
  tile_coords<8>(tiles_m, tiles_n, tm, tn);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;

  u32x4_t ra[A_LD];
  u32x4_t rb[B_LD][8];

  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int q = i * NT + tid;
      const int r = q / CH, c = q % CH;
      const int64_t gm = m0 + r;
      const int gk = k0 + c * 8;
      if (gm < M && gk < K)
        ra[i] = *reinterpret_cast<const u32x4_t*>(A + gm * K + gk);
      else
        ra[i] = u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int blk = i * NT + tid;
      const int nb = blk % (BN / 8), kb = blk / (BN / 8);
      const int64_t gn = n0 + nb * 8;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int64_t gk = k0 + kb * 8 + kk;
        if (blk < NBLK && gk < K && gn < N)
          rb[i][kk] = *reinterpret_cast<const u32x4_t*>(B + gk * N + gn);
        else
          rb[i][kk] = u32x4_t{0, 0, 0, 0};
      }
    }
  };

  auto store_stage = [&](int buf) {
    uint16_t* As = smem + buf * (BM + BN) * BK;
    uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int q = i * NT + tid;
      const int r = q / CH, c = q % CH;
      *reinterpret_cast<u32x4_t*>(As + r * BK + ((c ^ swz(r)) * 8)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int blk = i * NT + tid;
      if (NBLK % NT != 0 && blk >= NBLK) continue;
      const int nb = blk % (BN / 8), kb = blk / (BN / 8);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) {
        const int p = nn >> 1;
        u32x4_t col;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = rb[i][2 * j][p];      // k = 2j
          const uint32_t hi = rb[i][2 * j + 1][p];  // k = 2j + 1
          col[j] = (nn & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        const int n = nb * 8 + nn;
        *reinterpret_cast<u32x4_t*>(Bs + n * BK + ((kb ^ swz(n)) * 8)) = col;
      }
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage((kt + 1) * BK);
    const uint16_t* As = smem + cur * (BM + BN) * BK;
    const uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int c = ks * 4 + (lane >> 4);
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + r * BK + ((c ^ swz(r)) * 8));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * WTN + j * 16 + (lane & 15);
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + n * BK + ((c ^ swz(n)) * 8));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane owns row (lane & 15) and columns 4*(lane >> 4) .. +3 of each 16x16 tile.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm * WTM + i * 16 + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * WTN + j * 16 + 4 * (lane >> 4);
      if (n >= N) continue;
      f32x4_t v = acc[i][j];
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

template <int KC>
__global__ __launch_bounds__(256) void shard_reduce_kernel(PartPtrs parts, int k,
                                                           float* __restrict__ Z, int64_t n) {
  const int kk = KC > 0 ? KC : k;
  const int64_t n4 = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n4; v += stride) {
    f32x4_t s = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(parts.p[0]) + v);
    if constexpr (KC > 0) {
      f32x4_t t[KC > 1 ? KC - 1 : 1];
#pragma unroll
      for (int i = 1; i < KC; ++i)
        t[i - 1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(parts.p[i]) + v);
#pragma unroll
      for (int i = 1; i < KC; ++i) s = s + t[i - 1];
    } else {
      for (int i = 1; i < kk; ++i)
        s = s + __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(parts.p[i]) + v);
    }
    __builtin_nontemporal_store(s, reinterpret_cast<f32x4_t*>(Z) + v);
  }
  // scalar tail (n not a multiple of 4)
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t e = (n4 << 2) + threadIdx.x;
    float s = parts.p[0][e];
    for (int i = 1; i < kk; ++i) s = s + parts.p[i][e];
    Z[e] = s;
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_bf16_cfg(const uint16_t* A, const uint16_t* B, const uint16_t* bias, void* C,
                           int64_t M, int64_t N, int64_t K, Epilogue epi, hipStream_t s) {
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const dim3 grid(tiles_m * tiles_n), block(WM * WN * 64);
  switch (epi) {
    case kEpiBiasGelu:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, kEpiBiasGelu>), grid, block, 0, s, A,
                         B, bias, C, (int)M, (int)N, (int)K, tiles_m, tiles_n);
      break;
    case kEpiStoreF32:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, kEpiStoreF32>), grid, block, 0, s, A,
                         B, bias, C, (int)M, (int)N, (int)K, tiles_m, tiles_n);
      break;
    default:
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, kEpiAccumF32>), grid, block, 0, s, A,
                         B, bias, C, (int)M, (int)N, (int)K, tiles_m, tiles_n);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, const uint16_t* bias, void* C,
                            int64_t M, int64_t N, int64_t K, Epilogue epi, hipStream_t s) {
  return launch_bf16_cfg<128, 128, 2, 2>(A, B, bias, C, M, N, K, epi, s);
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
  PartPtrs pp;
  for (int i = 0; i < 64; ++i) pp.p[i] = i < k ? parts[i] : nullptr;
  const int64_t n4 = n >> 2;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(256);
  switch (k) {
    case 1:
      hipLaunchKernelGGL(shard_reduce_kernel<1>, grid, block, 0, s, pp, k, Z, n);
      break;
    case 2:
      hipLaunchKernelGGL(shard_reduce_kernel<2>, grid, block, 0, s, pp, k, Z, n);
      break;
    case 4:
      hipLaunchKernelGGL(shard_reduce_kernel<4>, grid, block, 0, s, pp, k, Z, n);
      break;
    case 8:
      hipLaunchKernelGGL(shard_reduce_kernel<8>, grid, block, 0, s, pp, k, Z, n);
      break;
    default:
      hipLaunchKernelGGL(shard_reduce_kernel<0>, grid, block, 0, s, pp, k, Z, n);
      break;
  }
  return hipGetLastError();
}

}  // namespace tpmlp
