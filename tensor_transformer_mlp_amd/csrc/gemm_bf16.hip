// Host side of the bf16 GEMM: tile choice and launch splitting.
#include "gemm_bf16_impl.h"

namespace tpmlp {

namespace {

// A dispatch packet counts work-items in 32 bits: keep each launch within
// 2^22 workgroups (of at most 512 work-items).
constexpr int64_t kMaxTilesPerLaunch = int64_t(1) << 22;

bool c_is_bf16(Epilogue e) {
  return e == kEpiBiasGelu || e == kEpiBiasGeluSave || e == kEpiMulAux;
}

}  // namespace

// Tile choice, from the per-shard GEMMs of the five workloads measured on
// MI355X (random bf16 data):
//   * 256x256 (8 waves, 4 stages) when it fills at least two rounds of the 256
//     CUs, or 192..255 tiles (a 0.75 round still beats the smaller tiles);
//   * otherwise 128x256 with 3 stages (two workgroups per CU) when N > 128;
//   * otherwise 128x128 (two workgroups per CU);
//   * K % 32 != 0 (K ends inside a 32-deep stage): the ragged-K variant of the
//     128x128 tile.
int pick_bf16_tile(Layout layout, int64_t M, int64_t N, int64_t K) {
  (void)layout;
  if (K % 32) return kTailTile;
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  if (t256 >= 512 || (t256 >= 192 && t256 < 256)) return 0;
  if (N > 128) return 6;
  return 8;
}

hipError_t launch_gemm_bf16_tile(int tile, const GemmArgs& g, hipStream_t s) {
  if (tile < 0 || tile >= kNumTiles) return hipErrorInvalidValue;
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const TileCfg& c = kTiles[tile];
  const int64_t tiles_n = (g.N + c.bn - 1) / c.bn;
  const int64_t rows_per_launch = (kMaxTilesPerLaunch / tiles_n) * c.bm;
  const bool a_kmajor = g.layout != kTN;
  const size_t c_elt = c_is_bf16(g.epi) ? 2 : 4;
  const uint16_t* A = static_cast<const uint16_t*>(g.A);
  const uint16_t* B = static_cast<const uint16_t*>(g.B);
  GemmParams p;
  p.B = B;
  p.bias = static_cast<const uint16_t*>(g.bias);
  p.lda = g.lda;
  p.ldb = g.ldb;
  p.ldc = g.ldc;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.tiles_n = (int)tiles_n;
  p.slices = 1;
  p.k_slice = p.K;
  p.part = nullptr;
  p.part_stride = 0;
  for (int64_t r0 = 0; r0 < g.M; r0 += rows_per_launch) {
    const int64_t Mc = g.M - r0 < rows_per_launch ? g.M - r0 : rows_per_launch;
    p.A = a_kmajor ? A + r0 * g.lda : A + r0;
    p.C = static_cast<char*>(g.C) + size_t(r0) * size_t(g.ldc) * c_elt;
    p.aux = g.aux ? static_cast<char*>(g.aux) + size_t(r0) * size_t(g.ldc) * 2 : nullptr;
    p.M = (int)Mc;
    p.tiles_m = (int)((Mc + c.bm - 1) / c.bm);
    hipError_t e;
    switch (g.layout) {
      case kNN: e = launch_bf16_nn(tile, p, g.epi, s); break;
      case kNT: e = launch_bf16_nt(tile, p, g.epi, s); break;
      default: e = launch_bf16_tn(tile, p, g.epi, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  return launch_gemm_bf16_tile(pick_bf16_tile(g.layout, g.M, g.N, g.K), g, s);
}

// ---------------------------------------------------------------------------
// K-split.  The bf16 slices use the 128x128 tile (two workgroups per CU), the
// float32 ones the 64x64 tile.  The slice count doubles while the grid has
// fewer than 256 workgroups and each slice keeps at least 2048 of K, or while
// it has fewer than 128 and each slice keeps at least 1024 (up to 16 slices).
// Measured on MI355X for the weight gradients of the MLP shards (for example
// 768 x 768 x 8192: 4 slices 409 TFLOP/s, 8 slices 311, no split 196).
// ---------------------------------------------------------------------------
namespace {

constexpr int kSplitTile = 8;  // 128x128, 2x4 waves

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

int64_t split_slice_len(int64_t K, int S) { return ((K + S - 1) / S + 31) / 32 * 32; }

// The operands of slice [k0, ...): A and B advanced by k0 along K.
GemmArgs slice_args(const GemmArgs& g, bool bf16, int64_t k0, int64_t kn) {
  GemmArgs a = g;
  const size_t e = bf16 ? 2 : 4;
  const int64_t a_off = g.layout == kTN ? k0 * g.lda : k0;
  const int64_t b_off = g.layout == kNT ? k0 : k0 * g.ldb;
  a.A = static_cast<const char*>(g.A) + size_t(a_off) * e;
  a.B = static_cast<const char*>(g.B) + size_t(b_off) * e;
  a.K = kn;
  return a;
}

}  // namespace

int gemm_k_slices(bool bf16, int64_t M, int64_t N, int64_t K) {
  const int64_t t = bf16 ? ((M + 127) / 128) * ((N + 127) / 128) : ((M + 63) / 64) * ((N + 63) / 64);
  int S = 1;
  while (S < 16 && t * S < 256 &&
         (K / (2 * S) >= 2048 || (t * S < 128 && K / (2 * S) >= 1024)))
    S *= 2;
  return S;
}

size_t gemm_split_workspace_bytes(bool bf16, int64_t M, int64_t N, int64_t K) {
  const int S = gemm_k_slices(bf16, M, N, K);
  return size_t(S - 1) * round256(size_t(M) * size_t(N) * 4);
}

hipError_t launch_gemm_split(const GemmArgs& g, bool bf16, void* ws, hipStream_t s) {
  const int S = gemm_k_slices(bf16, g.M, g.N, g.K);
  if (S == 1) return bf16 ? launch_gemm_bf16(g, s) : launch_gemm_f32(g, s);
  const int64_t ks = split_slice_len(g.K, S);
  const int n = (int)((g.K + ks - 1) / ks);  // slices actually used (<= S)
  const size_t part = round256(size_t(g.M) * size_t(g.N) * 4);
  if (bf16) {
    // One launch: the grid holds n copies of the tile grid (few tiles by
    // construction, so no launch splitting is needed).
    const TileCfg& c = kTiles[kSplitTile];
    GemmParams p;
    p.A = static_cast<const uint16_t*>(g.A);
    p.B = static_cast<const uint16_t*>(g.B);
    p.bias = nullptr;
    p.C = g.C;
    p.aux = nullptr;
    p.lda = g.lda;
    p.ldb = g.ldb;
    p.ldc = g.ldc;
    p.M = (int)g.M;
    p.N = (int)g.N;
    p.K = (int)g.K;
    p.tiles_m = (int)((g.M + c.bm - 1) / c.bm);
    p.tiles_n = (int)((g.N + c.bn - 1) / c.bn);
    p.slices = n;
    p.k_slice = (int)ks;
    p.part = static_cast<float*>(ws);
    p.part_stride = (int64_t)(part / 4);
    hipError_t e;
    switch (g.layout) {
      case kNN: e = launch_bf16_nn(kSplitTile, p, g.epi, s); break;
      case kNT: e = launch_bf16_nt(kSplitTile, p, g.epi, s); break;
      default: e = launch_bf16_tn(kSplitTile, p, g.epi, s); break;
    }
    if (e != hipSuccess) return e;
  } else {
    for (int i = 0; i < n; ++i) {
      const int64_t k0 = i * ks;
      GemmArgs a = slice_args(g, bf16, k0, g.K - k0 < ks ? g.K - k0 : ks);
      if (i > 0) {
        a.C = static_cast<char*>(ws) + size_t(i - 1) * part;
        a.ldc = g.N;
        a.epi = kEpiStoreF32;
      }
      const hipError_t e = launch_gemm_f32(a, s);
      if (e != hipSuccess) return e;
    }
  }
  // C must be dense ([M, N] with ldc == N) for the element-wise sum.
  const float* parts[16];
  parts[0] = static_cast<const float*>(g.C);
  for (int i = 1; i < n; ++i)
    parts[i] = reinterpret_cast<const float*>(static_cast<const char*>(ws) + size_t(i - 1) * part);
  return launch_shard_reduce(parts, n, static_cast<float*>(g.C), g.M * g.N, s);
}

}  // namespace tpmlp
