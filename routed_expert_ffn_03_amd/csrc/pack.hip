// Row-pair layout of bf16 expert matrices (weight format 2).
//
// The same bf16 values as the plain [rows, cols] matrix, stored so that rows
// 2p and 2p + 1 alternate every 32 columns: element (r, c) of a matrix sits
// at ((r / 2) * (cols / 32) + c / 32) * 64 + (r % 2) * 32 + c % 32.  A
// 32-column piece of two neighbouring rows is then one 128-byte line, so the
// FFN kernels' weight loads, which take 32 or 64 columns of many rows at a
// time, cover whole lines.  No page prescribes a storage layout for the bf16
// experts; this one is a property of how MI355X moves lines, done once when
// the weights are loaded.
//
// With to_fp16 the values are also converted to fp16 the way the FFN kernels
// convert W_down for the fp16 products (toward zero, exact in fp16's normal
// range): weight format 2 stores W_down that way, so its down phase reads
// fp16 directly.
//
// One 16-byte unit (8 values) per thread and step: unit d of the output is
// ((p * (cols / 32) + c) * 2 + h) * 4 + j, the 8 values of row 2p + h from
// column 32 c + 8 j.  Writes are contiguous; reads take 64 contiguous bytes
// of one row per four lanes.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace moe {
namespace {

__global__ __launch_bounds__(256)
void pack_pairs_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t units, int64_t per_mat,
                       int cols, int to_fp16) {
    const int64_t cu = cols / 8;                      // 16-byte units per plain row
    const int64_t kc = cols / 32;                     // 32-column pieces per row
    for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < units;
         d += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = d / per_mat, e = d - m * per_mat;
        const int64_t j = e & 3, h = (e >> 2) & 1, pc = e >> 3;
        const int64_t p = pc / kc, c = pc - p * kc;
        const u32x4 v = src[m * per_mat + (2 * p + h) * cu + 4 * c + j];
        dst[d] = to_fp16 ? bf16x8_to_f16x8(v) : v;
    }
}

}  // namespace

hipError_t launch_pack_pairs(const uint16_t* src, uint16_t* dst, int64_t mats, int rows, int cols, int to_fp16,
                             hipStream_t s) {
    const int64_t per_mat = (int64_t)rows * cols / 8;
    const int64_t units = mats * per_mat;
    const int64_t blocks = std::min<int64_t>((units + 255) / 256, 65536);
    pack_pairs_kernel<<<(unsigned)blocks, 256, 0, s>>>(reinterpret_cast<const u32x4*>(src),
                                                       reinterpret_cast<u32x4*>(dst), units, per_mat, cols, to_fp16);
    return hipGetLastError();
}

}  // namespace moe
