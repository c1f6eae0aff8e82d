// Host-side Tile-COO encoder for the outlier variant (FlashQuant abstract:
// outliers kept in high precision and encoded per tile, "Tile-COO", so the
// sparse path works tile by tile beside the dense one).
//
// Format (16 x 128 tiles over the N x K weight: the tile of the dense layout,
// 16 rows of one quant group):
//   tile t = (row / 16) * KT + col / 128, KT = ceil(K / 128), row-tile-major;
//   tile_ptr[t] .. tile_ptr[t + 1] (exclusive prefix sum) index tile_rec;
//   record = (fp16 value bits << 16) | (local_row << 8) | local_col, sorted by
//   (local_row, local_col) inside a tile.
#include <algorithm>
#include <cstdint>
#include <utility>
#include <vector>

#include "qgemv.h"

namespace {

constexpr int TILE_R = 16, TILE_C = 128;

}  // namespace

extern "C" {

size_t qgemv_tilecoo_ptr_len(int N, int K) {
  if (N < 1 || K < 1) return 0;
  return (size_t)((N + TILE_R - 1) / TILE_R) * (size_t)((K + TILE_C - 1) / TILE_C) + 1;
}

int qgemv_tilecoo_encode(int N, int K, int64_t nnz, const int32_t* rows, const int32_t* cols,
                         const uint16_t* val_bits, uint32_t* tile_ptr, uint32_t* tile_rec) {
  if (N < 1 || K < 1 || nnz < 0 || nnz > (int64_t)N * K || nnz > 0x7fffffff) return QGEMV_ERR_SHAPE;
  if (!tile_ptr || (nnz > 0 && (!rows || !cols || !val_bits || !tile_rec))) return QGEMV_ERR_NULL;
  const int KT = (K + TILE_C - 1) / TILE_C;
  const size_t T = qgemv_tilecoo_ptr_len(N, K) - 1;
  // sort key per outlier: (tile, local row, local col), unique per position,
  // paired with the outlier's index (tile indices may need more than 16 bits,
  // so the key does not share a word with the index)
  std::vector<std::pair<uint64_t, uint32_t>> key((size_t)nnz);
  for (int64_t i = 0; i < nnz; ++i) {
    const int32_t r = rows[i], c = cols[i];
    if (r < 0 || r >= N || c < 0 || c >= K) return QGEMV_ERR_VALUE;
    if ((val_bits[i] & 0x7C00u) == 0x7C00u) return QGEMV_ERR_VALUE;  // inf or NaN
    const uint64_t t = (uint64_t)(r / TILE_R) * KT + (uint64_t)(c / TILE_C);
    key[i] = {(t << 11) | ((uint64_t)(r % TILE_R) << 7) | (uint64_t)(c % TILE_C), (uint32_t)i};
  }
  std::sort(key.begin(), key.end());
  for (int64_t i = 1; i < nnz; ++i)
    if (key[i].first == key[i - 1].first) return QGEMV_ERR_VALUE;  // duplicate position
  std::fill(tile_ptr, tile_ptr + T + 1, 0u);
  for (int64_t i = 0; i < nnz; ++i) tile_ptr[(key[i].first >> 11) + 1] += 1;
  for (size_t t = 0; t < T; ++t) tile_ptr[t + 1] += tile_ptr[t];
  for (int64_t i = 0; i < nnz; ++i) {
    const uint64_t k = key[i].first;
    tile_rec[i] = ((uint32_t)val_bits[key[i].second] << 16) | (uint32_t)(((k >> 7) & 15u) << 8) | (uint32_t)(k & 127u);
  }
  return QGEMV_OK;
}

}  // extern "C"
