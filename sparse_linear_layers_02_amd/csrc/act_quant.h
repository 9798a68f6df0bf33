// Per-token absmax int8 quantization of one token by a group of AQ_T threads;
// shared by the act_quant call and the fused forward.
//
// The pages leave the activation path of Sparse-BitLinear open; this is the
// 1.58-bit BitNet convention: a = max(max_k |x|, 1e-5),
// Xq = rint((127*x) / a) (round half to even), s_x = a / 127, all float32.
// The quotient is formed as x * fl(127/a) (two roundings, error < 2^-15 near
// 128); only lanes whose estimate lies within 2^-12 of a half-integer redo the
// single correctly rounded division (127*x)/a, so the result equals that
// division's rint bit for bit.
#pragma once

#include "sbn_internal.h"

namespace sbn {

constexpr int AQ_T = 256;   // threads per token

__device__ inline uint32_t aq_max_abs_pair(uint32_t u) {
  const uint32_t lo = u & 0x7FFFu, hi = (u >> 16) & 0x7FFFu;
  return lo > hi ? lo : hi;
}

__device__ inline uint32_t aq_max_abs4(uint4 w) {
  return max(max(aq_max_abs_pair(w.x), aq_max_abs_pair(w.y)), max(aq_max_abs_pair(w.z), aq_max_abs_pair(w.w)));
}

__device__ inline int aq_quant_one(float x, float rcp, float a) {
  const float qt = x * rcp;
  float qr = rintf(qt);
  if (fabsf(qt - qr) > 0.5f - 0x1p-12f) qr = rintf((127.0f * x) / a);   // near a half: exact path
  return (int)qr;
}

__device__ inline uint32_t aq_quant_pair4(uint32_t u0, uint32_t u1, float rcp, float a) {
  const int q0 = aq_quant_one(bf16_to_f32(u0 & 0xFFFFu), rcp, a);
  const int q1 = aq_quant_one(bf16_to_f32(u0 >> 16), rcp, a);
  const int q2 = aq_quant_one(bf16_to_f32(u1 & 0xFFFFu), rcp, a);
  const int q3 = aq_quant_one(bf16_to_f32(u1 >> 16), rcp, a);
  return (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
         ((uint32_t)(q3 & 0xFF) << 24);
}

// Token `row` quantized by the AQ_T threads of a group (g = index in the
// group, red = 4 words of LDS for the group).  CH: 16-byte chunks per thread
// held in registers (0 = read the row twice).  Every thread of the block calls
// this once (it holds one block barrier); threads of a group with !valid only
// take part in the barrier.
template <int CH>
__device__ inline void act_quant_token(bool valid, int64_t row, int g, uint32_t* red,
                                       const uint16_t* __restrict__ X, int64_t K, int64_t ldx,
                                       int8_t* __restrict__ Xq, float* __restrict__ s_x) {
  const uint4* xr = (const uint4*)(X + row * ldx);
  uint2* qr = (uint2*)(Xq + row * K);
  const int kc = valid ? (int)(K / 8) : 0;
  uint32_t mx = 0;
  uint4 v[CH > 0 ? CH : 1];
  if (CH > 0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = g + AQ_T * i;
      if (c < kc) {
        v[i] = xr[c];
        mx = max(mx, aq_max_abs4(v[i]));
      }
    }
  } else {
    for (int c = g; c < kc; c += AQ_T) mx = max(mx, aq_max_abs4(xr[c]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t o = __shfl_xor(mx, m);
    mx = o > mx ? o : mx;
  }
  if ((g & 63) == 0) red[g >> 6] = mx;
  __syncthreads();
  if (!valid) return;
  mx = max(max(red[0], red[1]), max(red[2], red[3]));
  const float amax = bf16_to_f32(mx);
  const float a = fmaxf(amax, 1e-5f);
  const float rcp = 127.0f / a;
  if (g == 0) s_x[row] = a / 127.0f;
  if (CH > 0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = g + AQ_T * i;
      if (c < kc) {
        uint2 o;
        o.x = aq_quant_pair4(v[i].x, v[i].y, rcp, a);
        o.y = aq_quant_pair4(v[i].z, v[i].w, rcp, a);
        qr[c] = o;
      }
    }
  } else {
    for (int c = g; c < kc; c += AQ_T) {
      const uint4 w = xr[c];
      uint2 o;
      o.x = aq_quant_pair4(w.x, w.y, rcp, a);
      o.y = aq_quant_pair4(w.z, w.w, rcp, a);
      qr[c] = o;
    }
  }
}

// chunks per thread for a row of K bf16 values (0: stream the row twice)
inline int act_quant_ch(int64_t K) {
  const int64_t kc = K / 8;
  return kc <= AQ_T ? 1 : kc <= 2 * AQ_T ? 2 : kc <= 4 * AQ_T ? 4 : 0;
}

}  // namespace sbn
