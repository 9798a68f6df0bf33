// Per-token absmax int8 quantization of the activations: one block of AQ_T
// threads per token (the row kept in registers for K <= 8192, read twice
// otherwise).  The arithmetic is in act_quant.h.
#include "act_quant.h"

namespace sbn {
namespace {

template <int CH>
__global__ __launch_bounds__(AQ_T) void act_quant_kernel(const uint16_t* __restrict__ X, int64_t K,
                                                         int64_t ldx, int8_t* __restrict__ Xq,
                                                         float* __restrict__ s_x) {
  __shared__ uint32_t red[AQ_T / 64];
  act_quant_token<CH>(true, blockIdx.x, threadIdx.x, red, X, K, ldx, Xq, s_x);
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* X, int64_t T, int64_t K, int64_t ldx, int8_t* Xq,
                            float* s_x, hipStream_t st) {
  const dim3 grid((unsigned)T), block(AQ_T);
  switch (act_quant_ch(K)) {
    case 1: SBN_LAUNCH("act_quant", act_quant_kernel<1>, grid, block, 0, st, X, K, ldx, Xq, s_x); break;
    case 2: SBN_LAUNCH("act_quant", act_quant_kernel<2>, grid, block, 0, st, X, K, ldx, Xq, s_x); break;
    case 4: SBN_LAUNCH("act_quant", act_quant_kernel<4>, grid, block, 0, st, X, K, ldx, Xq, s_x); break;
    default: SBN_LAUNCH("act_quant", act_quant_kernel<0>, grid, block, 0, st, X, K, ldx, Xq, s_x); break;
  }
  return hipGetLastError();
}

}  // namespace sbn
