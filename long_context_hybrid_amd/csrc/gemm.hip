// Dense projections of the RNN layer: D[M][N] = A[M][K] W[N][K]^T with row-major operands (K
// contiguous in both) and fp32 accumulation; D is stored in the activation dtype.
//
// The layer around the mixer ("Hybrid Linear Attention Done Right", Appendix A, Eq. 18) has two
// such products: x [W_q | W_k | W_v | W_z] in front of the mixer and the output projection W_o^T
// behind it.  Both run on the library's own MFMA kernels:
//   * bf16 with more than kSkinnyMaxRows rows, K a multiple of 128 and at least 256, and N a
//     multiple of 8 (the prefill of a long sequence): the persistent 256 x 256-tile kernel of
//     gemm_tile.hip, MFMA-bound;
//   * everything else (decode steps, short prefills, fp32 storage, other K): the skinny kernel
//     of gemv.hip, which streams W once per 32 or 64 rows of A.
#include "lt_internal.h"

namespace lt {

lt_status gemm_xwt(const void* A, const void* W, void* D, int64_t M, int64_t N, int64_t K,
                   int dtype, hipStream_t stream) {
    if (launch_gate() != hipSuccess) return LT_ERR_HIP;
    if (M > 0x7fffffffLL || N > 0x7fffffffLL || K > 0x7fffffffLL) return LT_ERR_UNSUPPORTED;
    hipError_t e;
    if (dtype == LT_BF16 && M > kSkinnyMaxRows && K % 128 == 0 && K >= 256 && K <= (1 << 22) &&
        N % 8 == 0)
        e = launch_tile_gemm(A, W, D, M, (int)N, (int)K, stream);
    else
        e = launch_skinny_gemm(A, W, D, (int)M, (int)N, (int)K, (int)K, (int)K, (int)N, dtype,
                               stream);
    return e == hipSuccess ? LT_OK : LT_ERR_HIP;
}

}  // namespace lt
