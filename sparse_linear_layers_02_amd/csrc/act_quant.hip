// Per-token absmax int8 quantization of the activations.
//
// The pages leave the activation path of Sparse-BitLinear open; this is the
// 1.58-bit BitNet convention: a = max(max_k |x|, 1e-5),
// Xq = rint((127*x) / a) (round half to even), s_x = a / 127, all float32.
//
// One block per token.  The row is read once (kept in registers for
// K <= 8192, read twice otherwise).  The quotient is formed as x * fl(127/a)
// (two roundings, error < 2^-15 near 128); only lanes whose estimate lies
// within 2^-12 of a half-integer redo the single correctly rounded division
// (127*x)/a, so the result equals that division's rint bit for bit.
#include "sbn_internal.h"

namespace sbn {
namespace {

constexpr int AT = 256;

__device__ inline uint32_t max_abs_pair(uint32_t u) {
  const uint32_t lo = u & 0x7FFFu, hi = (u >> 16) & 0x7FFFu;
  return lo > hi ? lo : hi;
}

__device__ inline int quant_one(float x, float rcp, float a) {
  const float qt = x * rcp;
  float qr = rintf(qt);
  if (fabsf(qt - qr) > 0.5f - 0x1p-12f) qr = rintf((127.0f * x) / a);   // near a half: exact path
  return (int)qr;
}

__device__ inline uint32_t quant_pair4(uint32_t u0, uint32_t u1, float rcp, float a) {
  const int q0 = quant_one(bf16_to_f32(u0 & 0xFFFFu), rcp, a);
  const int q1 = quant_one(bf16_to_f32(u0 >> 16), rcp, a);
  const int q2 = quant_one(bf16_to_f32(u1 & 0xFFFFu), rcp, a);
  const int q3 = quant_one(bf16_to_f32(u1 >> 16), rcp, a);
  return (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
         ((uint32_t)(q3 & 0xFF) << 24);
}

__device__ inline uint32_t block_max_u32(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t o = __shfl_xor(v, m);
    v = o > v ? o : v;
  }
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < AT / 64; ++i) r = red[i] > r ? red[i] : r;
  return r;
}

// CH: 16-byte chunks per thread held in registers (0 = stream the row twice)
template <int CH>
__global__ __launch_bounds__(AT) void act_quant_kernel(const uint16_t* __restrict__ X, int64_t K,
                                                       int64_t ldx, int8_t* __restrict__ Xq,
                                                       float* __restrict__ s_x) {
  __shared__ uint32_t red[AT / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const uint4* xr = (const uint4*)(X + row * ldx);
  uint2* qr = (uint2*)(Xq + row * K);
  const int kc = (int)(K / 8);
  uint32_t mx = 0;
  uint4 v[CH > 0 ? CH : 1];
  if (CH > 0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + AT * i;
      if (c < kc) {
        v[i] = xr[c];
        uint32_t t = max_abs_pair(v[i].x);
        t = max(t, max_abs_pair(v[i].y));
        t = max(t, max_abs_pair(v[i].z));
        t = max(t, max_abs_pair(v[i].w));
        mx = max(mx, t);
      }
    }
  } else {
    for (int c = tid; c < kc; c += AT) {
      const uint4 w = xr[c];
      mx = max(mx, max(max(max_abs_pair(w.x), max_abs_pair(w.y)), max(max_abs_pair(w.z), max_abs_pair(w.w))));
    }
  }
  mx = block_max_u32(mx, red);
  const float amax = bf16_to_f32(mx);
  const float a = fmaxf(amax, 1e-5f);
  const float rcp = 127.0f / a;
  if (tid == 0) s_x[row] = a / 127.0f;
  if (CH > 0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + AT * i;
      if (c < kc) {
        uint2 o;
        o.x = quant_pair4(v[i].x, v[i].y, rcp, a);
        o.y = quant_pair4(v[i].z, v[i].w, rcp, a);
        qr[c] = o;
      }
    }
  } else {
    for (int c = tid; c < kc; c += AT) {
      const uint4 w = xr[c];
      uint2 o;
      o.x = quant_pair4(w.x, w.y, rcp, a);
      o.y = quant_pair4(w.z, w.w, rcp, a);
      qr[c] = o;
    }
  }
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* X, int64_t T, int64_t K, int64_t ldx, int8_t* Xq,
                            float* s_x, hipStream_t st) {
  const int64_t kc = K / 8;
  const dim3 grid((unsigned)T), block(AT);
  if (kc <= AT)
    SBN_LAUNCH("act_quant", act_quant_kernel<1>, grid, block, 0, st, X, K, ldx, Xq, s_x);
  else if (kc <= 2 * AT)
    SBN_LAUNCH("act_quant", act_quant_kernel<2>, grid, block, 0, st, X, K, ldx, Xq, s_x);
  else if (kc <= 4 * AT)
    SBN_LAUNCH("act_quant", act_quant_kernel<4>, grid, block, 0, st, X, K, ldx, Xq, s_x);
  else
    SBN_LAUNCH("act_quant", act_quant_kernel<0>, grid, block, 0, st, X, K, ldx, Xq, s_x);
  return hipGetLastError();
}

}  // namespace sbn
