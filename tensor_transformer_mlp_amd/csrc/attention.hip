// Scaled dot-product attention of one tensor-parallel shard's heads for
// gfx950 (bf16 in, fp32 softmax and accumulation, bf16 out), the per-shard
// step of the tensor-parallel attention block: each shard owns whole heads,
// so its attention needs no communication.
//
// Input: the shard's projection QKV [B S, 3 Hk] (Hk = heads * D): the query of
// head h at columns h D .. h D + D - 1, its key at Hk + h D, its value at
// 2 Hk + h D.  Output: A [B S, Hk], head h at columns h D.
//
// One workgroup = 4 waves = 128 QG queries of one (sequence, head); each wave
// owns QG groups of 32 queries (QG = 1 or 2) and walks the keys in blocks of
// 64 (causal: up to its last query), with the online softmax (a reference
// maximum m, raised when a block's scores exceed it by more than 2^8, and the
// sum l per query).  Every K and V fragment a wave reads from LDS feeds
// the MFMAs of all its query groups, so QG = 2 halves the LDS reads per
// score:
//   S^T = K Q^T    (keys x queries) on v_mfma_f32_32x32x16_bf16, K as the
//                  instruction's row operand, so every lane holds one query's
//                  scores and the softmax is lane-local (the two half-waves
//                  hold the two halves of the keys and exchange one maximum
//                  per block);
//   O^T += V^T P^T (D x queries), with P^T taken straight from the score
//                  registers (rounded to bf16) and V^T read by transpose
//                  reads, whose key order is chosen to match P's.
// K and V blocks go global -> LDS by direct-to-LDS loads into two stage
// buffers ([64 keys][D], 16-byte chunks XOR-swizzled by key), so loading block
// j + 1 overlaps the MFMAs of block j; the query fragments stay in registers.
// Keys past the sequence end read as zeros and are masked, as are keys after
// the query when causal; queries past the end are computed but not stored.
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "tp_mlp_kernels.h"

namespace tpmlp {

namespace {

struct AttnPtrs {
  const uint16_t* qkv[kMaxGroups];
  uint16_t* out[kMaxGroups];
};

struct AttnParams {
  AttnPtrs t;
  int groups;
  int B, S, heads;  // heads of one shard
  int nqb;          // query blocks of kBQ * QG per sequence
};

constexpr int kBQ = 128, kBK = 64;  // queries per workgroup and query group; keys per block

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to two round-to-nearest-even bf16 in one 32-bit word (a low).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Chunk swizzle of a [keys][D] tile: the 16-byte chunk c of key row k sits
// at position c ^ swz(k).  The LDS (64 banks of 4 bytes) serves a 16-byte
// read of a wave in four passes of 16 lanes, lanes {0-7, 16-23}, {8-15,
// 24-31}, {32-39, 48-55}, {40-47, 56-63} (the grouping that separates the
// conflict-free swizzle of the GEMM's K-major fragments, measured, from the
// ones measured 1.7x slower), and an 8-byte transpose read in two passes of
// 32 lanes.  A K fragment read (lane l: key l % 32, chunk 2 j + l / 32) is
// then conflict-free when swz takes 16 distinct values on keys {0-7, 16-23}
// and on {8-15, 24-31}; a V^T transpose read (lanes 0-31: keys 4 m .. 4 m +
// 3, four consecutive chunks each) when the four keys of every aligned
// quad put their chunk quads apart.  D = 128 (256-byte rows, 16 chunks):
// bits 2-3 of swz = key bits 0-1, bit 0 = key bit 2, bit 1 = key bit 4.  D =
// 64 (128-byte rows, two keys per bank row, 8 chunks): bit 2 = key bit 1,
// bit 0 = key bit 2, bit 1 = key bit 4.  Key bit 5 is not used, so keys k and
// k + 32 share a swizzle (the two 32-key halves of a block are one address
// immediate apart); key bit 4 is, so the V^T reads of keys 16 .. 31 of each
// half have their own lane addresses.  (The previous swizzles, key & 15 and
// (key >> 1) & 7, gave 2-way conflicts on the K reads and 2- to 4-way on the
// V^T reads under this model; rocprofv3's SQ_LDS_BANK_CONFLICT for the
// kernel went from 2.6e7 to 0 with these.)
// The value of lane l ^ 32 (the other half-wave), by v_permlane32_swap: a
// swap of the upper half of one register with the lower half of another,
// here both x, leaves x of lanes 0-31 in every lane of one result and x of
// lanes 32-63 in every lane of the other.
__device__ __forceinline__ void half_pair(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  // (the elements are copied out first: a bit cast of an element of the
  // returned vector reads element 0 with this compiler)
  const uint32_t r0 = r[0], r1 = r[1];
  lo = __builtin_bit_cast(float, r0);
  hi = __builtin_bit_cast(float, r1);
}

template <int D>
__device__ __forceinline__ int swz(int key) {
  if constexpr (D == 128) return ((key & 3) << 2) | ((key >> 2) & 1) | (((key >> 4) & 1) << 1);
  else return ((key >> 2) & 1) | (((key >> 4) & 1) << 1) | (((key >> 1) & 1) << 2);
}

template <int D, bool CAUSAL, int QG>
__global__ __launch_bounds__(256) void attention_kernel(AttnParams p) {
  constexpr int ROW = 2 * D;                 // bytes per key row in LDS
  constexpr int TILE = kBK * ROW;            // one K or V block
  constexpr int STAGE = 2 * TILE;
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int ROWS_PER_DMA = 1024 / ROW;   // rows per 1 KB direct-to-LDS load
  constexpr int DMA_PER_WAVE = TILE / 1024 / 4;
  constexpr int KS = D / 16;                 // MFMA k-steps over D (scores)
  constexpr int DT = D / 32;                 // output tiles of 32 along D
  // Two stage buffers of [K tile | V tile] in one array, so that the second
  // stage is a constant offset from the first.
  __shared__ __attribute__((aligned(1024))) char stages[2 * STAGE];

  // Heaviest query blocks (the last ones, under the causal mask) first.
  const int per_qb = p.groups * p.B * p.heads;
  const int id = blockIdx.x;
  const int qb = p.nqb - 1 - id / per_qb;
  int rest = id % per_qb;
  const int g = rest / (p.B * p.heads);
  rest -= g * p.B * p.heads;
  const int b = rest / p.heads;
  const int head = rest - b * p.heads;

  const int S = p.S;
  const int Hk = p.heads * D;
  const int64_t ld = 3 * (int64_t)Hk;
  const uint16_t* qkv = p.t.qkv[g];
  const uint16_t* seq = qkv + (int64_t)b * S * ld;  // row 0 of this sequence
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const int q0 = qb * kBQ * QG;
  const int qw = q0 + 32 * QG * wave;  // this wave's first query
  int qq[QG];                          // this lane's query in each group
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) qq[qg] = qw + 32 * qg + l32;

  // Query fragments (B operand of S^T = K Q^T): dims 16 j + 8 h2 .. + 7.
  bf16x8_t qf[QG][KS];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const bool ok = qq[qg] < S;
    const uint16_t* qrow = seq + (int64_t)(ok ? qq[qg] : 0) * ld + head * D + 8 * h2;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4_t*>(qrow + 16 * j);
      qf[qg][j] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Direct-to-LDS loads of one K and one V block: this wave's rows of the
  // 64-row tiles.  Lane offsets from the block's first key row.
  uint32_t loff[DMA_PER_WAVE];
  int lrow[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int row = (wave * DMA_PER_WAVE + i) * ROWS_PER_DMA + lane / CH;
    const int c = (lane % CH) ^ swz<D>(row);
    lrow[i] = row;
    loff[i] = (uint32_t)row * (uint32_t)(ld * 2) + (uint32_t)c * 16u;
  }
  auto issue = [&](uint32_t lds, int k0) {
    // The descriptors start at the block's first key row (64-bit address
    // arithmetic here, 32-bit offsets inside the block).
    const i32x4_t kd = buffer_desc(seq + (int64_t)k0 * ld + Hk + head * D, 0x7FFFFFF0u);
    const i32x4_t vd = buffer_desc(seq + (int64_t)k0 * ld + 2 * Hk + head * D, 0x7FFFFFF0u);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const uint32_t off = k0 + lrow[i] < S ? loff[i] : kOob;
      lds_dma16(kd, lds + (uint32_t)((wave * DMA_PER_WAVE + i) * 1024), off);
      lds_dma16(vd, lds + TILE + (uint32_t)((wave * DMA_PER_WAVE + i) * 1024), off);
    }
  };

  // LDS read offsets.  K fragment (A operand of S^T) of 32-key tile u and
  // k-step j: key 32 u + l32, chunk 2 j + h2 (swz(key) does not depend on u).
  const uint32_t L0 = lds_offset(stages);
  uint32_t kaddr[KS];  // stage 0's LDS address; + 32 u ROW and + s STAGE are immediates
#pragma unroll
  for (int j = 0; j < KS; ++j) kaddr[j] = L0 + l32 * ROW + (((2 * j + h2) ^ swz<D>(l32)) << 4);
  // V^T fragment (A operand of O^T += V^T P^T) of output tile t, k-step jj
  // (keys 16 jj ..): two transpose reads at keys 16 jj + 4 h2 + 8 r + (q / 4),
  // columns 32 t + 16 ((lane >> 4) & 1) + 4 (q % 4), q = lane % 16; the
  // swizzle depends on jj % 2 only.
  uint32_t vaddr[2][DT][2];  // [jj % 2]: stage 0's LDS address; + 32 (jj / 2) ROW and + s STAGE are immediates
  {
    const int q = lane & 15;
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int key = 16 * par + 4 * h2 + 8 * r + (q >> 2);
          const int col = 32 * t + 16 * ((lane >> 4) & 1) + 4 * (q & 3);
          vaddr[par][t][r] = L0 + TILE + key * ROW + (((col >> 3) ^ swz<D>(key)) << 4) + ((col >> 2) & 1) * 8;
        }
  }

  f32x16_t acc[QG][DT];
  float m_run[QG], l_run[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[qg][t][e] = 0.f;
    m_run[qg] = -1e30f;
    l_run[qg] = 0.f;
  }
  const float c2 = 1.4426950408889634f / __builtin_sqrtf((float)D);  // log2(e) / sqrt(D)
  constexpr float kSlack = 8.f;  // the weights stay below 2^8
  const bf16x2_t kOnes = {(__bf16)1.0f, (__bf16)1.0f};

  const int kend = CAUSAL ? min(q0 + kBQ * QG, S) : S;
  const int nb = (kend + kBK - 1) / kBK;
  // Causal: blocks past this wave's last query are skipped (every score in
  // them would be masked, changing nothing); the wave still joins the loads
  // and barriers of the workgroup.
  const int kwave = CAUSAL ? qw + 32 * QG - 1 : S;

  using lds_frag = const __attribute__((address_space(3))) bf16x8_t;
  using lds_half = __attribute__((address_space(3))) i16x4_t;
  // One 64-key block from stage buffer SB (a compile-time index: every LDS
  // address below is a per-lane register plus an immediate).  All fragment
  // reads of a product are issued before its MFMAs, so their latencies
  // overlap instead of adding up.
  auto block = [&](auto sset, int k0) {
    constexpr int SB = decltype(sset)::value * STAGE;
    // S^T for the 64 keys: two 32-key tiles per query group.
    f32x16_t s[QG][2];
    bf16x8_t kf[2][KS];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < KS; ++j) kf[u][j] = *(lds_frag*)(uintptr_t)(kaddr[j] + SB + u * 32 * ROW);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[qg][u][e] = 0.f;
#pragma unroll
        for (int j = 0; j < KS; ++j)
          s[qg][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[u][j], qf[qg][j], s[qg][u], 0, 0, 0);
      }
    // every K fragment read first, then the score MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS * QG, 0);
    // V^T fragments of the first k-step, read while the softmax runs.
    bf16x8_t vf[2][DT];
    auto read_v = [&](int jj, bf16x8_t* dst) {
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_half*)(uintptr_t)(vaddr[jj & 1][t][0] + SB + (jj >> 1) * 32 * ROW));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_half*)(uintptr_t)(vaddr[jj & 1][t][1] + SB + (jj >> 1) * 32 * ROW));
        dst[t] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    read_v(0, vf[0]);
    // Mask, block maximum of the raw scores (lane pair l, l ^ 32 hold one
    // query); the maximum m is kept in base-2 units (scores times c2).
    const bool edge = k0 + kBK > S || (CAUSAL && k0 + kBK - 1 > qw);
    bf16x8_t pf[QG][4];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      if (edge) {
        // score e of tile u is key k0 + 4 h2 + (32 u + 8 (e / 4) + e % 4),
        // masked past the last key this query sees
        const int last = (CAUSAL ? min(S - 1, qq[qg]) : S - 1) - k0 - 4 * h2;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * u + 8 * (e >> 2) + (e & 3) > last) s[qg][u][e] = -__builtin_inff();
      }
      // four independent chains, then the two half-waves' maxima
      float m4[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        m4[c] = c == 0 ? -1e30f : s[qg][c >> 1][8 * (c & 1)];
#pragma unroll
        for (int e = c == 0 ? 0 : 1; e < 8; ++e) m4[c] = fmaxf(m4[c], s[qg][c >> 1][8 * (c & 1) + e]);
      }
      float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])), mlo, mhi;
      half_pair(mx, mlo, mhi);
      mx = fmaxf(mlo, mhi);
      // The reference maximum m is raised only when some lane's block
      // maximum exceeds it by more than kSlack: the weights p = 2^(s c2 - m)
      // then stay below 2^kSlack, and the accumulators and the sum l are
      // rescaled (by 2^(m_old - m_new), exact 1 for the lanes whose maximum
      // did not grow) only on those blocks.  Raising m at every new maximum
      // would rescale on nearly every block: some lane of 32 queries usually
      // finds a new maximum among the next 64 keys.  The quotient O / l does
      // not depend on m; the weights are rounded to bf16 relative to their
      // size either way.
      const float m_blk = mx * c2;
      if (__any(m_blk > m_run[qg] + kSlack)) {
        const float m_new = fmaxf(m_run[qg], m_blk);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qg] - m_new);
        m_run[qg] = m_new;
        l_run[qg] *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) acc[qg][t] = acc[qg][t] * alpha;
      }
      const float m = m_run[qg];
      // p = 2^(s c2 - m), one fused multiply-add per score (a masked score,
      // -inf, gives 0), rounded to bf16 in pairs; l sums the rounded pairs
      // (the weights the value products use), two chains of dot products
      // with (1, 1).
      float ps[2] = {0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x4_t pk;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e = 8 * (jj & 1) + 2 * e2;
          const float a0 = __builtin_amdgcn_exp2f(fmaf(s[qg][jj >> 1][e], c2, -m));
          const float a1 = __builtin_amdgcn_exp2f(fmaf(s[qg][jj >> 1][e + 1], c2, -m));
          const uint32_t w = pack_bf16x2(a0, a1);  // (a bit cast of pk[e2] would read pk[0])
          pk[e2] = w;
          ps[e2 & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), kOnes, ps[e2 & 1], false);
        }
        pf[qg][jj] = __builtin_bit_cast(bf16x8_t, pk);
      }
      l_run[qg] += ps[0] + ps[1];
    }
    // O^T += V^T P^T over the 64 keys (4 k-steps of 16), the next k-step's
    // V^T fragments read while this one's MFMAs run.
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (jj + 1 < 4) read_v(jj + 1, vf[(jj + 1) & 1]);
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
          acc[qg][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[jj & 1][t], pf[qg][jj], acc[qg][t], 0, 0, 0);
    }
  };

  // Two stage buffers: block j + 1 loads while block j is computed.  At the
  // top of iteration j the only loads in flight are block j's.  The loop is
  // unrolled by two so that each block's stage is a compile-time index.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // vmcnt(0) lgkmcnt(0) before each barrier: this wave's loads of the next
  // block have landed and its reads of the previous block have returned (the
  // compiler may place the MFMAs that consume those reads after the barrier,
  // and the barrier alone does not wait for them).
  constexpr int kWaitAll = 7 << 4;
  issue(L0, 0);
  for (int j = 0; j < nb; j += 2) {
    __builtin_amdgcn_s_waitcnt(kWaitAll);    // block j has landed
    asm volatile("s_barrier" ::: "memory");  // visible to all; block j - 1 done
    if (j + 1 < nb) issue(L0 + STAGE, (j + 1) * kBK);
    if (j * kBK <= kwave) block(I0{}, j * kBK);
    if (j + 1 < nb) {
      __builtin_amdgcn_s_waitcnt(kWaitAll);
      asm volatile("s_barrier" ::: "memory");
      if (j + 2 < nb) issue(L0, (j + 2) * kBK);
      if ((j + 1) * kBK <= kwave) block(I1{}, (j + 1) * kBK);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);

  // O = O^T / l: lane holds query qq, columns 32 t + 8 (e / 4) + 4 h2 + e % 4.
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    float llo, lhi;
    half_pair(l_run[qg], llo, lhi);
    const float l_tot = llo + lhi;
    if (qq[qg] < S) {
      const float inv = __builtin_amdgcn_rcpf(l_tot);
      uint16_t* orow = p.t.out[g] + ((int64_t)b * S + qq[qg]) * Hk + head * D + 4 * h2;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          u32x2_t o;
          o[0] = pack_bf16x2(acc[qg][t][4 * e4] * inv, acc[qg][t][4 * e4 + 1] * inv);
          o[1] = pack_bf16x2(acc[qg][t][4 * e4 + 2] * inv, acc[qg][t][4 * e4 + 3] * inv);
          *reinterpret_cast<u32x2_t*>(orow + 32 * t + 8 * e4) = o;
        }
    }
  }
}

}  // namespace

// Query groups of 32 per wave: two when the grid of 256-query workgroups
// still holds at least 4096 of them (16 rounds of the CUs), else one.  Two
// groups halve the LDS reads per score, but also the workgroups, and for
// d = 128 the second group's registers leave one wave per SIMD.  Measured
// (bit-identical outputs): 10% faster at S = 32768 (8 shards of 8 heads of
// 128, 8192 workgroups), 10-25% slower at S <= 2048 (gpt2_small's and
// llama7b's shards, 384 and 1024 workgroups).
constexpr int64_t kWideGrid = 4096;

static int attention_query_groups(int64_t S, int64_t seqs) {
  return ((S + 2 * kBQ - 1) / (2 * kBQ)) * seqs >= kWideGrid ? 2 : 1;
}

hipError_t launch_attention_bf16_variant(int variant, const void* const* qkv, void* const* out, int groups,
                                         int64_t B, int64_t S, int heads, int d, bool causal, hipStream_t s) {
  if (groups < 1 || groups > kMaxGroups || (d != 64 && d != 128)) return hipErrorInvalidValue;
  if (variant < -1 || variant > 1) return hipErrorInvalidValue;
  if (B <= 0 || S <= 0) return hipSuccess;
  AttnParams p{};
  for (int gi = 0; gi < groups; ++gi) {
    p.t.qkv[gi] = static_cast<const uint16_t*>(qkv[gi]);
    p.t.out[gi] = static_cast<uint16_t*>(out[gi]);
  }
  p.groups = groups;
  p.B = (int)B;
  p.S = (int)S;
  p.heads = heads;
  const int64_t seqs = (int64_t)groups * B * heads;
  if (variant < 0) variant = attention_query_groups(S, seqs) - 1;
  const int qg = variant + 1;
  p.nqb = (int)((S + kBQ * qg - 1) / (kBQ * qg));
  const int64_t blocks = (int64_t)p.nqb * seqs;
  const dim3 grid((unsigned)blocks), block(256);
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  const auto launch = [&](auto dd, auto cc, auto gg) {
    hipLaunchKernelGGL((attention_kernel<decltype(dd)::value, decltype(cc)::value, decltype(gg)::value>), grid,
                       block, 0, s, p);
  };
  using G1 = std::integral_constant<int, 1>;
  using G2 = std::integral_constant<int, 2>;
  if (d == 128) {
    if (qg == 2) causal ? launch(D128{}, std::true_type{}, G2{}) : launch(D128{}, std::false_type{}, G2{});
    else causal ? launch(D128{}, std::true_type{}, G1{}) : launch(D128{}, std::false_type{}, G1{});
  } else {
    if (qg == 2) causal ? launch(D64{}, std::true_type{}, G2{}) : launch(D64{}, std::false_type{}, G2{});
    else causal ? launch(D64{}, std::true_type{}, G1{}) : launch(D64{}, std::false_type{}, G1{});
  }
  return hipGetLastError();
}

hipError_t launch_attention_bf16(const void* const* qkv, void* const* out, int groups, int64_t B,
                                 int64_t S, int heads, int d, bool causal, hipStream_t s) {
  return launch_attention_bf16_variant(-1, qkv, out, groups, B, S, heads, d, causal, s);
}

}  // namespace tpmlp
