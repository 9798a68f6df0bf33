// Decode GEMV (1 <= T <= 16): Y[t,r] = s_w * s_x[t] * sum_k Xq[t,k] * Wt[r,k],
// streaming the packed weight once and unpacking it in registers.
//
// The pages measure decode on a custom sparse kernel ("Sparse-BitNet",
// gist.science Japanese "技術概要" §3.2: B200 decode; Korean "기술 요약" §4).
// Here the sixteen-wide int8 matrix instruction v_mfma_i32_16x16x64_i8 takes
// 16 weight rows against the (up to) 16 tokens, so the arithmetic is never
// the limit; the cost is reading the packed planes and turning them into
// int8 operands.
//
// Unpacking: a 4096-entry table in LDS maps (4 meta bits, the next 8 code
// bits) to the four int8 weights {-1, 0, +1} of those positions (unused code
// bits are ignored).  Every group of four positions is one table read.
//
// Work split: one block (8 waves) per 16 output rows.  K is cut into ranges of
// 512 positions; a wave takes ranges wave, wave+8, ...  Inside a range, lane
// l (row l%16, part g = l/16) owns a contiguous run of 16*S positions, so its
// meta and code bits are contiguous; the matrix instruction only needs A lane
// (r, g) and B lane (t, g) to cover the same positions, which they do.  The
// waves' 16x16 partial sums are added in LDS.  All loads of a wave's first
// range (packed bits and activations) are issued before the block copies the
// unpack table and synchronises, so the three fetches overlap.
#include "sbn_internal.h"

namespace sbn {
namespace {

struct UnpackTable {
  uint32_t v[4096];
  constexpr UnpackTable() : v() {
    for (int nib = 0; nib < 16; ++nib)
      for (int c8 = 0; c8 < 256; ++c8) {
        uint32_t out = 0;
        int cur = 0;
        for (int p = 0; p < 4; ++p)
          if ((nib >> p) & 1) {
            const int c = (c8 >> (2 * cur)) & 3;
            ++cur;
            const uint32_t b = c == 1 ? 0x01u : c == 3 ? 0xFFu : 0u;
            out |= b << (8 * p);
          }
        v[nib | (c8 << 4)] = out;
      }
  }
};

__device__ const UnpackTable kUnpack;

// bits [off, off+nb) of the normalised word array (off, nb compile-time after unrolling)
template <int NW>
__device__ inline uint32_t bits_at(const uint32_t (&w)[NW], int off, int nb) {
  const int i = off >> 5, s = off & 31;
  uint32_t v = w[i] >> s;
  if (s + nb > 32 && i + 1 < NW) v = __builtin_amdgcn_alignbit(w[i + 1], w[i], s);
  return nb >= 32 ? v : (v & ((1u << nb) - 1u));
}

constexpr int GV_WAVES = 8;            // waves per block (one block per 16 output rows)
constexpr int GV_RANGE = 512;          // K positions per wave range: 8 MFMA steps of 64

template <int N, int M, int OUT>
__global__ __launch_bounds__(64 * GV_WAVES) void gemv_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ s_x, int64_t T, int64_t K,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta, const float* __restrict__ s_w,
    int64_t R, void* __restrict__ Y, int64_t ldy) {
  constexpr int SMAX = GV_RANGE / 64;                  // MFMA steps per range
  constexpr int64_t CB_NUM = 2 * N;                    // code bits per group
  constexpr int NWC = (32 * N * SMAX / M) / 32 + 1;    // normalised code words for a full range
  __shared__ uint32_t lut[4096];
  __shared__ int red[GV_WAVES][256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, rl = lane & 15;
  const int64_t r = (int64_t)blockIdx.x * 16 + rl;
  const int64_t rr = r < R ? r : R - 1;               // rows past R: computed on row R-1, discarded
  const bool tvalid = rl < T;
  const int64_t tt = tvalid ? rl : 0;                 // B column of this lane (token)
  const int64_t crow = K * N / (4 * M);
  const uint8_t* mrow = meta ? meta + rr * (K / 8) : nullptr;
  const uint8_t* crw = codes + rr * crow;
  const int8_t* xrow = Xq + tt * K;
  const int64_t nranges = cdiv(K, GV_RANGE);

  v4i acc = (v4i){0, 0, 0, 0};
  bool first = true;
  for (int64_t ri = wave; ri < nranges || first; ri += GV_WAVES) {
    const bool active = ri < nranges;
    const int64_t kbeg = ri * GV_RANGE;
    int S = active ? (int)((K - kbeg) / 64) : 0;
    S = S < SMAX ? S : SMAX;
    const int64_t p0 = kbeg + 16 * (int64_t)g * S;    // this lane's run: 16*S positions

    // ---- issue every load of this range before anything waits
    uint32_t mw[SMAX / 2 + 1];
#pragma unroll
    for (int i = 0; i < SMAX / 2 + 1; ++i) mw[i] = 0;
    if (N < M && active) {
      const uint16_t* mh = (const uint16_t*)(mrow + p0 / 8);
#pragma unroll
      for (int i = 0; i < SMAX; ++i)
        if (i < S) mw[i >> 1] |= (uint32_t)mh[i] << (16 * (i & 1));
    }
    const int64_t cbit = CB_NUM * (p0 / M);
    const uintptr_t ca = (uintptr_t)(crw + (cbit >> 3));
    const uint32_t* cw4 = (const uint32_t*)(ca & ~(uintptr_t)3);
    const int sh = (int)((ca & 3) * 8 + (cbit & 7));
    const int nbits = 32 * N * S / M;
    const int nd = active ? (sh + nbits + 31) >> 5 : 0;
    uint32_t raw[NWC + 1];
#pragma unroll
    for (int i = 0; i < NWC + 1; ++i) raw[i] = (i < nd) ? cw4[i] : 0u;
    v4i bx[SMAX];
#pragma unroll
    for (int j = 0; j < SMAX; ++j)
      bx[j] = (tvalid && j < S) ? *(const v4i*)(xrow + kbeg + 16 * ((int64_t)g * S + j)) : (v4i){0, 0, 0, 0};

    if (first) {                                       // unpack table, fetched while the loads above fly
      for (int i = tid; i < 1024; i += 64 * GV_WAVES) ((uint4*)lut)[i] = ((const uint4*)kUnpack.v)[i];
      __syncthreads();
      first = false;
    }
    if (!active) break;

    uint32_t cw[NWC];
#pragma unroll
    for (int i = 0; i < NWC; ++i) cw[i] = __builtin_amdgcn_alignbit(raw[i + 1], raw[i], sh);

#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
      if (j < S) {
        uint32_t e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int pos = 16 * j + 4 * k;                        // position within the run
          const uint32_t nib = (N < M) ? ((mw[pos >> 5] >> (pos & 31)) & 0xFu) : 0xFu;
          uint32_t c8;
          if (M == 4) {
            c8 = bits_at<NWC>(cw, (int)CB_NUM * (pos / 4), 8);
          } else {
            const int gi = pos / 8;
            const uint32_t gb = bits_at<NWC>(cw, (int)CB_NUM * gi, 24);
            if ((k & 1) == 0) {
              c8 = gb & 0xFFu;
            } else {
              const uint32_t low = (N < M) ? ((mw[(pos - 4) >> 5] >> ((pos - 4) & 31)) & 0xFu) : 0xFu;
              c8 = (gb >> (2 * __builtin_popcount(low))) & 0xFFu;
            }
          }
          e[k] = lut[nib | (c8 << 4)];
        }
        const v4i a = (v4i){(int)e[0], (int)e[1], (int)e[2], (int)e[3]};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bx[j], acc, 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][lane * 4 + v] = acc[v];
  __syncthreads();
  if (tid < 256) {
    const int e = tid;
    int s = 0;
#pragma unroll
    for (int w = 0; w < GV_WAVES; ++w) s += red[w][e];
    const int L = e >> 2, v = e & 3;
    const int64_t row = (int64_t)blockIdx.x * 16 + 4 * (L >> 4) + v;
    const int64_t t = L & 15;
    if (t < T && row < R) {
      if (OUT == 0) {
        ((int*)Y)[t * ldy + row] = s;
      } else {
        const float y = (float)s * (*s_w * s_x[t]);
        if (OUT == 1) ((float*)Y)[t * ldy + row] = y;
        else ((uint16_t*)Y)[t * ldy + row] = f32_to_bf16_rne(y);
      }
    }
  }
}

template <int N, int M>
hipError_t launch_gemv_nm(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                          const uint8_t* codes, const uint8_t* meta, const float* s_w, int64_t R,
                          void* Y, sbn_dtype ydt, int64_t ldy, hipStream_t st) {
  const dim3 grid((unsigned)cdiv(R, 16)), block(64 * GV_WAVES);
  const uint8_t* mp = (N == M) ? nullptr : meta;
  if (ydt == SBN_I32_ACC)
    SBN_LAUNCH("gemv", (gemv_kernel<N, M, 0>), grid, block, 0, st, Xq, s_x, T, K, codes, mp, s_w, R, Y, ldy);
  else if (ydt == SBN_F32)
    SBN_LAUNCH("gemv", (gemv_kernel<N, M, 1>), grid, block, 0, st, Xq, s_x, T, K, codes, mp, s_w, R, Y, ldy);
  else
    SBN_LAUNCH("gemv", (gemv_kernel<N, M, 2>), grid, block, 0, st, Xq, s_x, T, K, codes, mp, s_w, R, Y, ldy);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                       const uint8_t* codes, const uint8_t* meta, const float* s_w, int64_t R,
                       int n, int m, void* Y, sbn_dtype ydt, int64_t ldy, hipStream_t st) {
#define SBN_GEMV_CASE(NN, MM) \
  if (n == NN && m == MM) return launch_gemv_nm<NN, MM>(Xq, s_x, T, K, codes, meta, s_w, R, Y, ydt, ldy, st);
  SBN_GEMV_CASE(1, 4) SBN_GEMV_CASE(2, 4) SBN_GEMV_CASE(3, 4) SBN_GEMV_CASE(4, 4)
  SBN_GEMV_CASE(1, 8) SBN_GEMV_CASE(2, 8) SBN_GEMV_CASE(3, 8) SBN_GEMV_CASE(4, 8)
  SBN_GEMV_CASE(5, 8) SBN_GEMV_CASE(6, 8) SBN_GEMV_CASE(7, 8) SBN_GEMV_CASE(8, 8)
#undef SBN_GEMV_CASE
  return hipErrorInvalidValue;
}

}  // namespace sbn
