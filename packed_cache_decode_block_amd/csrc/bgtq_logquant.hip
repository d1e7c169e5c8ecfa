// Row reordering of the high-precision store for LogQuant's log-based filter (LogQuant summary,
// Method 2): when a sequence's high-precision set is halved, its store is reordered so that the
// kept rows fill slots [0, 2W) and the leaving rows sit in slots [2W, 3W) in leaving order, from
// where the quantize-append path reads them as consecutive rows.  The order of rows does not
// matter to the decode (Method 4).
#include "bgtq_internal.h"

namespace bgtq {
namespace {

constexpr int D = 128;
constexpr int COLS = 32;  // dims per workgroup

// Grid (D / COLS, kv head, sequence), 256 threads: the workgroup stages its COLS-dim column of
// every store row in LDS, then writes row j from staged row perm[j] (from the arguments, or from
// device memory when the permutations of all sequences exceed them); keys, then values.
__global__ __launch_bounds__(256) void k_hp_permute(const PermuteArgs a) {
    const int c0 = blockIdx.x * COLS, h = blockIdx.y, b = blockIdx.z;
    const int first = a.seq_first[b];
    if (first < 0) return;  // this sequence's store is unchanged
    const int R = a.n_recent;
    __shared__ uint16_t s_col[BGTQ_HP_ROWS_MAX * COLS];
    for (int pass = 0; pass < 2; ++pass) {
        uint16_t* base = (pass ? a.rows_v : a.rows_k) + ((size_t)b * a.Hkv + h) * R * D;
        __syncthreads();  // the previous pass has written its rows
        for (int i = threadIdx.x; i < R * COLS; i += 256) s_col[i] = base[(i / COLS) * D + c0 + i % COLS];
        __syncthreads();
        for (int i = threadIdx.x; i < R * COLS; i += 256) {
            const int r = i / COLS, c = i % COLS;
            base[r * D + c0 + c] = s_col[(a.perm_dev ? a.perm_dev[first + r] : a.perm[first + r]) * COLS + c];
        }
    }
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, int B, hipStream_t s) {
    if (!a.rows_k || !a.rows_v || a.n_recent < 1 || a.n_recent > BGTQ_HP_ROWS_MAX || B < 1 || B > BGTQ_MAXB)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_hp_permute, dim3(D / COLS, a.Hkv, B), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace bgtq
