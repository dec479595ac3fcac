// Tile verification between the block-pair screen and the sparse half-steps.
#pragma once

#include "internal.h"

namespace sk {

constexpr int32_t kVerifyB = 128;  // verified tiles are 128 x 128 points

// Device scratch of one verification, grown on demand and reused.
struct VerifyScratch {
  uint8_t* keep = nullptr;   // [nnz] keep flag per candidate
  int32_t* colany = nullptr; // [mb] column block keeps some tile
  int64_t* cnt = nullptr;    // [nb + 1] kept tiles per row block
  int32_t* vrow = nullptr;   // [nnz] row block of each kept tile (sort values)
  int32_t* skey = nullptr;   // [nnz] sorted column blocks (sort keys out)
  void* temp = nullptr;      // rocPRIM scan / sort storage
  size_t temp_bytes = 0;
  int64_t nnz_cap = 0, nb_cap = 0, mb_cap = 0;
  ~VerifyScratch();
  void reserve(int64_t nnz, int64_t nb, int64_t mb);
};

// Keep the candidates (ptr [nb + 1], idx [nnz], row-major over the row side's
// blocks) whose exact row or column share at (f, g) exceeds delta_rel, then
// the row and column fallbacks; writes the kept tiles row-major (vptr
// [nb + 1], vidx) and column-major (tptr [mb + 1], tidx: row blocks in
// increasing order per column block). vidx / tidx need nnz entries. Returns
// the kept count (synchronizes the stream). B must be kVerifyB, d <= 3.
int64_t verify_tiles(sinkhorn_problem* p, const Side& rows, const Side& cols, const float* f,
                     const float* g, double eps, double delta_rel, const int64_t* ptr,
                     const int32_t* idx, int64_t nnz, int64_t nb, int64_t mb, int64_t* vptr,
                     int32_t* vidx, int64_t* tptr, int32_t* tidx, VerifyScratch& s);

}  // namespace sk
