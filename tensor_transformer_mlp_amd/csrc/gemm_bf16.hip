// Host side of the bf16 GEMM: tile choice, batches of per-shard GEMMs, the
// group sum, the K-split and launch splitting.
#include "gemm_bf16_impl.h"

namespace tpmlp {

namespace {

// A dispatch packet counts work-items in 32 bits: keep each launch within
// 2^22 workgroups (of at most 512 work-items).
constexpr int64_t kMaxTilesPerLaunch = int64_t(1) << 22;

bool c_is_bf16(Epilogue e) {
  return e == kEpiBiasGelu || e == kEpiBiasGeluSave || e == kEpiMulAux || e == kEpiSwiGLU || e == kEpiBias;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

int64_t tiles_of(int tile, int64_t M, int64_t N, Epilogue epi = kEpiStoreF32) {
  const int64_t cols = tile_out_cols(tile, epi);
  return ((M + kTiles[tile].bm - 1) / kTiles[tile].bm) * ((N + cols - 1) / cols);
}

hipError_t launch_layout(Layout layout, int tile, const GemmParams& p, Epilogue epi, bool gsum,
                         hipStream_t s) {
  switch (layout) {
    case kNN: return launch_bf16_nn(tile, p, epi, gsum, s);
    case kNT: return launch_bf16_nt(tile, p, epi, gsum, s);
    default: return launch_bf16_tn(tile, p, epi, gsum, s);
  }
}

GemmParams base_params(const GemmBatch& b, int tile) {
  GemmParams p{};
  for (int g = 0; g < b.groups; ++g) {
    p.t.A[g] = static_cast<const uint16_t*>(b.A[g]);
    p.t.B[g] = static_cast<const uint16_t*>(b.B[g]);
    p.t.B2[g] = static_cast<const uint16_t*>(b.B2[g]);
    p.t.bias[g] = static_cast<const uint16_t*>(b.bias[g]);
    p.t.C[g] = b.C[g];
    p.t.aux[g] = b.aux[g];
  }
  p.groups = b.groups;
  p.lda = b.lda;
  p.ldb = b.ldb;
  p.ldc = b.ldc;
  p.M = (int)b.M;
  p.N = (int)b.N;
  p.K = (int)b.K;
  p.tiles_m = (int)((b.M + kTiles[tile].bm - 1) / kTiles[tile].bm);
  const int cols = tile_out_cols(tile, b.epi);
  p.tiles_n = (int)((b.N + cols - 1) / cols);
  p.slices = 1;
  p.k_slice = p.K;
  p.part = nullptr;
  p.part_stride = 0;
  p.shared_a = 1;
  for (int g = 1; g < b.groups; ++g) p.shared_a &= b.A[g] == b.A[0];
  return p;
}

}  // namespace

// Tile choice, from the per-shard GEMMs of the five workloads measured on
// MI355X (random bf16 data), counting the workgroups of the whole batch:
//   * 256x256 (8 waves, 4 stages) when it fills at least two rounds of the 256
//     CUs, or 192..255 tiles (a 0.75 round still beats the smaller tiles);
//   * between one and two rounds of 256x256 tiles, with N a multiple of 384
//     and a long K loop (K >= 4096): 128x384 (4 stages, one workgroup per
//     CU), whose grid is half as many tiles again (gpt3_175b's shard sum:
//     384 tiles of 256x256, 1.5 rounds; 512 of 128x384, two whole rounds);
//   * otherwise 128x256 when N > 128: with 4 stages when its tiles fit one
//     round of the CUs (one workgroup per CU, the deeper prefetch pays), else
//     with 3 stages (two workgroups per CU);
//   * otherwise 128x128 (two workgroups per CU);
//   * K % 32 != 0 (K ends inside a 32-deep stage): the ragged-K variant of the
//     128x128 tile.
// A group sum is one GEMM of the output's size (its K runs through every
// group): the same rule with one group.
int pick_bf16_tile(Layout layout, int64_t M, int64_t N, int64_t K, int groups, bool group_sum) {
  (void)layout;
  if (K % 32) return kTailTile;
  const int64_t kloop = group_sum ? K * groups : K;  // the K loop of one tile
  if (group_sum) groups = 1;
  const int64_t t256 = tiles_of(0, M, N) * groups;
  if (t256 >= 512 || (t256 >= 192 && t256 < 256)) return 0;
  if (t256 > 256 && N % 384 == 0 && kloop >= 4096) return 9;
  if (N > 128) return tiles_of(5, M, N) * groups <= 256 ? 5 : 6;
  return 8;
}

// SwiGLU (two B operands, BM x BN/2 output tiles): 256x256 (128 output
// columns) on the same workgroup-count rule as above, else 128x256 with 3
// stages, which is also the ragged-K tile.
int pick_swiglu_tile(int64_t M, int64_t N, int64_t K, int groups) {
  if (K % 32) return kTailTileSwiGLU;
  const int64_t t256 = tiles_of(0, M, N, kEpiSwiGLU) * groups;
  return (t256 >= 512 || (t256 >= 192 && t256 < 256)) ? 0 : 6;
}

hipError_t launch_gemm_bf16_batch_tile(int tile, const GemmBatch& b, hipStream_t s) {
  if (tile < 0 || tile >= kNumTiles || b.groups < 1 || b.groups > kMaxGroups) return hipErrorInvalidValue;
  if (b.epi == kEpiSwiGLU && (b.group_sum || b.layout != kNN || !tile_allows_swiglu(tile)))
    return hipErrorInvalidValue;
  if (b.M <= 0 || b.N <= 0) return hipSuccess;
  const TileCfg& c = kTiles[tile];
  GemmParams p = base_params(b, tile);
  const int64_t per_row = (int64_t)p.tiles_n * (b.group_sum ? 1 : b.groups);
  const int64_t rows_per_launch = (kMaxTilesPerLaunch / per_row) * c.bm;
  const bool a_kmajor = b.layout != kTN;
  const size_t c_elt = c_is_bf16(b.epi) ? 2 : 4;
  for (int64_t r0 = 0; r0 < b.M; r0 += rows_per_launch) {
    const int64_t Mc = b.M - r0 < rows_per_launch ? b.M - r0 : rows_per_launch;
    for (int g = 0; g < b.groups; ++g) {
      const uint16_t* A = static_cast<const uint16_t*>(b.A[g]);
      p.t.A[g] = a_kmajor ? A + r0 * b.lda : A + r0;
      p.t.C[g] = static_cast<char*>(b.C[g]) + size_t(r0) * size_t(b.ldc) * c_elt;
      p.t.aux[g] = b.aux[g] ? static_cast<char*>(b.aux[g]) + size_t(r0) * size_t(b.ldc) * 2 : nullptr;
    }
    p.M = (int)Mc;
    p.tiles_m = (int)((Mc + c.bm - 1) / c.bm);
    const hipError_t e = launch_layout(b.layout, tile, p, b.epi, b.group_sum, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

GemmBatch single_batch(const GemmArgs& g);

int gemm_bf16_batch_tile(const GemmBatch& b) {
  if (b.epi == kEpiSwiGLU) return pick_swiglu_tile(b.M, b.N, b.K, b.groups);
  return pick_bf16_tile(b.layout, b.M, b.N, b.K, b.groups, b.group_sum);
}

hipError_t launch_gemm_bf16_batch(const GemmBatch& b, hipStream_t s) {
  return launch_gemm_bf16_batch_tile(gemm_bf16_batch_tile(b), b, s);
}

int gemm_bf16_tile_count() { return kNumTiles; }

void gemm_bf16_tile_shape(int tile, int info[4]) {
  const TileCfg& c = kTiles[tile];
  info[0] = c.bm;
  info[1] = c.bn;
  info[2] = c.wm * c.wn;
  info[3] = c.nbuf;
}

bool gemm_bf16_tile_can_run(int tile, const GemmBatch& b) {
  return tile >= 0 && tile < kNumTiles && b.groups >= 1 && b.groups <= kMaxGroups &&
         instantiated(b.layout, tile, b.K % 32 != 0, b.group_sum, b.epi);
}

GemmBatch single_batch(const GemmArgs& g) {
  GemmBatch b{};
  b.A[0] = g.A;
  b.B[0] = g.B;
  b.bias[0] = g.bias;
  b.B2[0] = g.B2;
  b.C[0] = g.C;
  b.aux[0] = g.aux;
  b.groups = 1;
  b.group_sum = false;
  b.M = g.M;
  b.N = g.N;
  b.K = g.K;
  b.lda = g.lda;
  b.ldb = g.ldb;
  b.ldc = g.ldc;
  b.layout = g.layout;
  b.epi = g.epi;
  return b;
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  return launch_gemm_bf16_batch(single_batch(g), s);
}

hipError_t launch_gemm_bf16_tile(int tile, const GemmArgs& g, hipStream_t s) {
  return launch_gemm_bf16_batch_tile(tile, single_batch(g), s);
}

// ---------------------------------------------------------------------------
// K-split.  The bf16 slices use the 128x128 tile (two workgroups per CU), the
// float32 ones the 64x64 tile.  The slice count doubles while one group's
// grid has fewer than 256 workgroups and each slice keeps at least 2048 of K,
// or while it has fewer than 128 and each slice keeps at least 1024 (up to
// 16 slices).
// Measured on MI355X for the weight gradients of the MLP shards (for example
// 768 x 768 x 8192: 4 slices 409 TFLOP/s, 8 slices 311, no split 196).
// ---------------------------------------------------------------------------
namespace {

constexpr int kSplitTile = 8;  // 128x128, 2x4 waves

int64_t split_slice_len(int64_t K, int S) { return ((K + S - 1) / S + 31) / 32 * 32; }

// The slice count depends on one group's shape only, so a shard's result
// does not depend on how many shards share the launch.
int64_t split_tiles(bool bf16, int64_t M, int64_t N) {
  return bf16 ? tiles_of(kSplitTile, M, N) : ((M + 63) / 64) * ((N + 63) / 64);
}

}  // namespace

int gemm_k_slices(bool bf16, int64_t tiles, int64_t K) {
  (void)bf16;
  int S = 1;
  while (S < 16 && tiles * S < 256 &&
         (K / (2 * S) >= 2048 || (tiles * S < 128 && K / (2 * S) >= 1024)))
    S *= 2;
  return S;
}

size_t gemm_split_workspace_bytes(bool bf16, int groups, int64_t M, int64_t N, int64_t K) {
  const int S = gemm_k_slices(bf16, split_tiles(bf16, M, N), K);
  return size_t(groups) * size_t(S - 1) * round256(size_t(M) * size_t(N) * 4);
}

hipError_t launch_gemm_split(const GemmBatch& b, bool bf16, void* ws, hipStream_t s) {
  const int S = gemm_k_slices(bf16, split_tiles(bf16, b.M, b.N), b.K);
  if (S == 1) return bf16 ? launch_gemm_bf16_batch(b, s) : launch_gemm_f32_batch(b, s);
  const int64_t ks = split_slice_len(b.K, S);
  const int n = (int)((b.K + ks - 1) / ks);  // slices actually used (<= S)
  const size_t part = round256(size_t(b.M) * size_t(b.N) * 4);
  // group g's partial of slice i > 0 sits at ws + (g (n - 1) + i - 1) part
  auto part_ptr = [&](int g, int i) {
    return reinterpret_cast<float*>(static_cast<char*>(ws) + (size_t(g) * (n - 1) + i - 1) * part);
  };
  if (bf16) {
    // One launch: the grid holds groups x n copies of the tile grid (few
    // tiles by construction, so no launch splitting is needed).
    GemmParams p = base_params(b, kSplitTile);
    p.slices = n;
    p.k_slice = (int)ks;
    p.part = static_cast<float*>(ws);
    p.part_stride = (int64_t)(part / 4);
    const hipError_t e = launch_layout(b.layout, kSplitTile, p, b.epi, false, s);
    if (e != hipSuccess) return e;
  } else {
    for (int g = 0; g < b.groups; ++g) {
      for (int i = 0; i < n; ++i) {
        const int64_t k0 = i * ks;
        const int64_t a_off = b.layout == kTN ? k0 * b.lda : k0;
        const int64_t b_off = b.layout == kNT ? k0 : k0 * b.ldb;
        GemmArgs a{static_cast<const float*>(b.A[g]) + a_off, static_cast<const float*>(b.B[g]) + b_off,
                   nullptr, nullptr, b.C[g], nullptr, b.M, b.N, b.K - k0 < ks ? b.K - k0 : ks,
                   b.lda, b.ldb, b.ldc, b.layout, b.epi};
        if (i > 0) {
          a.C = part_ptr(g, i);
          a.ldc = b.N;
          a.epi = kEpiStoreF32;
        }
        const hipError_t e = launch_gemm_f32(a, s);
        if (e != hipSuccess) return e;
      }
    }
  }
  float* C[kMaxGroups];
  for (int g = 0; g < b.groups; ++g) C[g] = static_cast<float*>(b.C[g]);
  return launch_split_reduce(C, b.groups, static_cast<const float*>(ws), (int64_t)(part / 4), n,
                             b.M * b.N, s);
}

}  // namespace tpmlp
