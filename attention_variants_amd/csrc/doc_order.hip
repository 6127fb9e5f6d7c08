// Heaviest-first work order of the query tiles under the document mask.
//
// Under the document mask (one of the masked variants of the talk notes,
// "Evaluation: FlexAttention-supported variants") a query tile of 128 rows
// attends to the keys of the documents its rows belong to, so its key range,
// and with it its run time, follows the document lengths: tiles inside long
// documents walk many key tiles, tiles inside short ones a few.  Dispatched in natural order, heavy tiles that
// start late leave a tail.  This pass computes each tile's key-tile count
// from doc_id with the same range rule as the forward kernel and sorts the
// tiles by descending count (ties by ascending index), the
// longest-processing-time order; the forward kernel then visits the tiles in
// that order.  The order changes when each tile runs, never what it computes.
//
// One workgroup: a per-thread binary search per tile, then a bitonic sort of
// 32-bit keys (count complement above, tile index below) in LDS.

#include <hip/hip_runtime.h>

#include "av_kernels.hpp"

namespace av {
namespace {

constexpr int kThreads = 1024;
constexpr int kIdxBits = 14;  // kDocOrderMax = 2^14 tiles

// first index in row[0, n) whose value is > target (rows are non-decreasing)
__device__ int upper_bound_row(const int* row, int n, int target) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] <= target) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) void doc_order_kernel(const int* doc, int B, int S, int* order) {
  __shared__ uint32_t keys[kDocOrderMax];
  const int nM = (S + kDocTileM - 1) / kDocTileM;
  const int nKV = (S + kDocTileN - 1) / kDocTileN;
  const int n = B * nM;
  int P = 1;
  while (P < n) P <<= 1;

  for (int i = threadIdx.x; i < P; i += kThreads) {
    uint32_t key = 0xffffffffu;  // padding sorts last
    if (i < n) {
      const int b = i / nM, mt = i % nM;
      const int* row = doc + (size_t)b * S;
      const int q0 = mt * kDocTileM, qlast = min(q0 + kDocTileM, S) - 1;
      const int kstart = upper_bound_row(row, S, row[q0] - 1);  // first key of the first row's document
      const int kend = upper_bound_row(row, S, row[qlast]);     // one past the last row's document
      const int cost = min(nKV, (kend + kDocTileN - 1) / kDocTileN) - kstart / kDocTileN;
      key = ((uint32_t)(nKV - cost) << kIdxBits) | (uint32_t)i;
    }
    keys[i] = key;
  }
  __syncthreads();

  // bitonic sort, ascending
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += kThreads) {
        const int p = i ^ j;
        if (p > i) {
          const uint32_t x = keys[i], y = keys[p];
          const bool up = (i & k) == 0;
          if (up ? (x > y) : (x < y)) {
            keys[i] = y;
            keys[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }

  for (int i = threadIdx.x; i < n; i += kThreads) order[i] = (int)(keys[i] & ((1u << kIdxBits) - 1));
}

}  // namespace

hipError_t launch_doc_order(const int* doc, int B, int S, int* order, hipStream_t stream) {
  static_assert(kDocOrderMax == 1 << kIdxBits, "index field width");
  hipLaunchKernelGGL(doc_order_kernel, dim3(1), dim3(kThreads), 0, stream, doc, B, S, order);
  return hipGetLastError();
}

}  // namespace av
