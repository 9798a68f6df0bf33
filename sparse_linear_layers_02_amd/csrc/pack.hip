// Mask, ternarize and pack: the weight side of Sparse-BitLinear.
//
// Pass 1 sums |w| exactly and turns the sum into the per-tensor scale
//   s_w = max(fp32(mean |W|), 1e-5)   (correctly rounded, launch-independent).
// Pass 2 computes, per group of M weights along K, the N largest |w| (ties to
// the lower index), ternarizes with the exact test |w| > s_w/2, and writes the
// meta bitmap and the 2-bit survivor codes.
//
// Sources: gist.science summaries of "Sparse-BitNet" -- German "Technische
// Zusammenfassung" §2 (mask from master-weight magnitudes, N largest per
// block of M; quantize, then mask), Japanese "技術概要" §2.1 (mask from the
// continuous weights, recomputed every step), French "Résumé technique" §2.
//
// Exactness of the sum.  Every bf16 magnitude is sig * 2^(e-134) with an
// 8-bit significand.  Magnitudes with exponent field e in [95, 131), i.e.
// 2^-32 <= |w| < 16, are multiples of 2^-39 below 2^4; a float64 running sum
// of at most 1024 of them stays below 2^53 units, so it is exact in any
// order.  Each thread flushes its float64 sum into an int64 counter of
// 2^-39 units after every row (K <= 2^18 keeps a row's share per thread at
// <= 1024 terms).  Everything outside that window (zero, subnormal, tiny
// or >= 16) goes to 256 per-exponent integer bins with atomics: exact too.
// The last block to finish (atomic counter) forms the total as a 320-bit
// integer in units of 2^-133 and rounds total / (R*K) to fp32: a float64
// estimate, then an exact comparison against the two neighbouring midpoints.
#include "sbn_internal.h"

namespace sbn {
namespace {

constexpr int PT = 256;                  // threads per block, both passes
constexpr uint32_t E_LO = 95, E_HI = 131;
constexpr double FAST_SCALE = 549755813888.0;  // 2^39

struct PackHeader {
  unsigned int counter;
  unsigned int pad[63];
  unsigned long long bins[256];
};

// ------------------------------------------------------------------ 320-bit integer
struct Big {
  uint32_t w[10];
};

__device__ inline void big_zero(Big& b) {
#pragma unroll
  for (int j = 0; j < 10; ++j) b.w[j] = 0;
}

// b += v << sh  (0 <= sh <= 250, v < 2^64)
__device__ inline void big_add_shifted(Big& b, unsigned long long v, int sh) {
  const int li = sh >> 5, bs = sh & 31;
  unsigned __int128 x = (unsigned __int128)v << bs;
  const uint32_t p0 = (uint32_t)x, p1 = (uint32_t)(x >> 32), p2 = (uint32_t)(x >> 64);
  unsigned long long carry = 0;
#pragma unroll
  for (int j = 0; j < 10; ++j) {
    uint32_t add = (j == li) ? p0 : (j == li + 1) ? p1 : (j == li + 2) ? p2 : 0u;
    unsigned long long t = (unsigned long long)b.w[j] + add + carry;
    b.w[j] = (uint32_t)t;
    carry = t >> 32;
  }
}

// -1, 0, +1
__device__ inline int big_cmp(const Big& a, const Big& b) {
  int res = 0;
#pragma unroll
  for (int j = 9; j >= 0; --j) {
    if (res == 0) res = (a.w[j] > b.w[j]) ? 1 : (a.w[j] < b.w[j]) ? -1 : 0;
  }
  return res;
}

// midpoint of two adjacent positive floats, times n, times 2^133, as a Big
__device__ inline Big mid_times_n(float a, float b, unsigned long long n) {
  double mid = ((double)a + (double)b) * 0.5;   // exact: 25 significant bits
  int e;
  double f = frexp(mid, &e);                     // mid = f * 2^e, f in [0.5, 1)
  unsigned long long M = (unsigned long long)ldexp(f, 25);
  Big r;
  big_zero(r);
  big_add_shifted(r, M * n, e - 25 + 133);
  return r;
}

__device__ inline float pick_even(float a, float b) {
  return (__float_as_uint(a) & 1u) ? b : a;
}

// s_w = max(RN_f32(total * 2^-133 / n), 1e-5)
__device__ float round_mean(const Big& t, unsigned long long n) {
  int top = -1;
#pragma unroll
  for (int j = 0; j < 10; ++j)
    if (t.w[j]) top = j;
  if (top < 0) return 1e-5f;
  double v = 0.0;
  int base = 0;
#pragma unroll
  for (int j = 0; j < 10; ++j) {
    if (j == top) {
      double hi = (double)t.w[j];
      double mi = j >= 1 ? (double)t.w[j - 1] : 0.0;
      double lo = j >= 2 ? (double)t.w[j - 2] : 0.0;
      v = (hi * 4294967296.0 + mi) * 4294967296.0 + lo;
      base = 32 * (j - 2);
    }
  }
  const double approx = ldexp(v, base - 133) / (double)n;
  if (approx < 0x1p-20) return 1e-5f;            // far below the floor
  const float r0 = (float)approx;
  const float rn = __uint_as_float(__float_as_uint(r0) + 1u);
  const float rp = __uint_as_float(__float_as_uint(r0) - 1u);
  const int c_hi = big_cmp(t, mid_times_n(r0, rn, n));
  const int c_lo = big_cmp(t, mid_times_n(rp, r0, n));
  float r = r0;
  if (c_hi > 0) r = rn;
  else if (c_hi == 0) r = pick_even(r0, rn);
  else if (c_lo < 0) r = rp;
  else if (c_lo == 0) r = pick_even(rp, r0);
  return fmaxf(r, 1e-5f);
}

// ------------------------------------------------------------------ reductions
__device__ inline unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m);
  hi = __shfl_xor(hi, m);
  return ((unsigned long long)hi << 32) | lo;
}

__device__ inline unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_u64(v, m);
  return v;
}

// ------------------------------------------------------------------ pass 1
__device__ inline void slow_add(unsigned long long* bins, uint32_t mag32) {
  const uint32_t e = mag32 >> 23;
  const uint32_t f = (mag32 >> 16) & 0x7Fu;
  const uint32_t sig = e ? (f | 0x80u) : f;
  atomicAdd(&bins[e], (unsigned long long)sig);
}

// |w| of the two bf16 halves of u; window members returned in float64,
// the rest sent to the bins.
__device__ inline double pair_abs(uint32_t u, unsigned long long* bins) {
  const uint32_t lo = (u << 16) & 0x7FFF0000u;
  const uint32_t hi = u & 0x7FFF0000u;
  const bool lo_in = (lo - (E_LO << 23)) < ((E_HI - E_LO) << 23);
  const bool hi_in = (hi - (E_LO << 23)) < ((E_HI - E_LO) << 23);
  double s = (lo_in ? (double)__uint_as_float(lo) : 0.0) + (hi_in ? (double)__uint_as_float(hi) : 0.0);
  if (!(lo_in && hi_in)) {
    if (!lo_in && lo) slow_add(bins, lo);
    if (!hi_in && hi) slow_add(bins, hi);
  }
  return s;
}

__global__ __launch_bounds__(PT) void abs_sum_kernel(const uint16_t* __restrict__ W, int64_t R,
                                                     int64_t K, int64_t ldw, int64_t rows_per_block,
                                                     unsigned char* __restrict__ ws,
                                                     float* __restrict__ s_w) {
  PackHeader* hdr = (PackHeader*)ws;
  long long* partials = (long long*)(ws + sizeof(PackHeader));
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = min(R, r0 + rows_per_block);
  const int kc = (int)(K / 8);
  unsigned long long acc_i = 0;
  for (int64_t r = r0; r < r1; ++r) {
    const uint4* row = (const uint4*)(W + r * ldw);
    double acc = 0.0;
    for (int c = tid; c < kc; c += PT) {
      const uint4 v = row[c];
      acc += pair_abs(v.x, hdr->bins) + pair_abs(v.y, hdr->bins) + pair_abs(v.z, hdr->bins) +
             pair_abs(v.w, hdr->bins);
    }
    acc_i += (unsigned long long)(acc * FAST_SCALE);   // exact integer < 2^53
  }
  __shared__ unsigned long long red[PT / 64];
  __shared__ int is_last;
  unsigned long long s = wave_sum_u64(acc_i);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    unsigned long long b = 0;
    for (int i = 0; i < PT / 64; ++i) b += red[i];
    partials[blockIdx.x] = (long long)b;
    __threadfence();
    is_last = (atomicAdd(&hdr->counter, 1u) == gridDim.x - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // ---- finalize: the last block sums the partials and the bins
  unsigned __int128 f = 0;
  for (int64_t i = tid; i < (int64_t)gridDim.x; i += PT)
    f += (unsigned long long)__atomic_load_n(&partials[i], __ATOMIC_RELAXED);
  __shared__ unsigned long long flo[PT], fhi[PT];
  __shared__ unsigned long long sbins[256];
  __shared__ unsigned long long nzmask[4];
  flo[tid] = (unsigned long long)f;
  fhi[tid] = (unsigned long long)(f >> 64);
  const unsigned long long b = __atomic_load_n(&hdr->bins[tid], __ATOMIC_RELAXED);
  sbins[tid] = b;
  const unsigned long long bal = __ballot(b != 0);
  if ((tid & 63) == 0) nzmask[tid >> 6] = bal;
  __syncthreads();
  for (int sh = PT / 2; sh > 0; sh >>= 1) {      // tree sum of the 128-bit partial sums
    if (tid < sh) {
      unsigned __int128 a = ((unsigned __int128)fhi[tid] << 64) | flo[tid];
      a += ((unsigned __int128)fhi[tid + sh] << 64) | flo[tid + sh];
      flo[tid] = (unsigned long long)a;
      fhi[tid] = (unsigned long long)(a >> 64);
    }
    __syncthreads();
  }
  if (tid == 0) {
    const unsigned __int128 F = ((unsigned __int128)fhi[0] << 64) | flo[0];
    Big t;
    big_zero(t);
    // fast part: F units of 2^-39 = F * 2^94 units of 2^-133
    big_add_shifted(t, (unsigned long long)F, 94);
    big_add_shifted(t, (unsigned long long)(F >> 64), 94 + 64);
    for (int w = 0; w < 4; ++w) {
      unsigned long long mk = nzmask[w];
      while (mk) {
        const int bit = __ffsll((long long)mk) - 1;
        mk &= mk - 1;
        const int e = w * 64 + bit;
        big_add_shifted(t, sbins[e], (e ? e : 1) - 1);
      }
    }
    *s_w = round_mean(t, (unsigned long long)(R * K));
  }
}

// ------------------------------------------------------------------ pass 2
// One thread = 32 consecutive weights of one row (32/M whole groups).
template <int M>
__global__ __launch_bounds__(PT) void mask_pack_kernel(
    const uint16_t* __restrict__ W, int64_t R, int64_t K, int64_t ldw, int n,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ meta, const float* __restrict__ s_w_ptr,
    unsigned char* __restrict__ ws, int64_t total_chunks, int64_t dr, int64_t dch) {
  if (blockIdx.x == 0) {   // leave the pass-1 header zeroed for the next call
    PackHeader* hdr = (PackHeader*)ws;
    hdr->bins[threadIdx.x] = 0;
    if (threadIdx.x == 0) hdr->counter = 0;
  }
  const float h = 0.5f * (*s_w_ptr);
  const uint32_t thr = __float_as_uint(h) >> 16;      // |w| > h  <=>  key > thr
  const int64_t cpr = K / 32;
  const int64_t crow = K * n / (4 * M);               // code bytes per row
  const int cbc = 8 * n / M;                          // code bytes per chunk (M=8: n, M=4: 2n)
  int64_t c = (int64_t)blockIdx.x * PT + threadIdx.x;
  int64_t r = c / cpr, ch = c - r * cpr;
  for (; c < total_chunks; c += (int64_t)gridDim.x * PT) {
    const uint4* src = (const uint4*)(W + r * ldw + ch * 32);
    const uint4 q0 = src[0], q1 = src[1], q2 = src[2], q3 = src[3];
    const uint32_t u[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                            q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
    uint32_t keep = 0;
    unsigned long long cw = 0;
#pragma unroll
    for (int g = 0; g < 32 / M; ++g) {
      uint32_t key[M], code[M];
#pragma unroll
      for (int p = 0; p < M; ++p) {
        const int i = g * M + p;
        const uint32_t w = (u[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        const uint32_t a = w & 0x7FFFu;
        key[p] = (a << 3) | (uint32_t)(7 - p);          // distinct; lower index wins ties
        const uint32_t nz = a > thr ? 1u : 0u;
        code[p] = nz | ((nz & (w >> 15)) << 1);          // 00 = 0, 01 = +1, 11 = -1
      }
      int slot = 0;
#pragma unroll
      for (int p = 0; p < M; ++p) {
        int rank = 0;
#pragma unroll
        for (int q = 0; q < M; ++q)
          if (q != p) rank += key[q] > key[p] ? 1 : 0;
        const bool kp = rank < n;
        keep |= (kp ? 1u : 0u) << (g * M + p);
        cw |= (unsigned long long)(kp ? code[p] : 0u) << (2 * (n * g + slot));
        slot += kp ? 1 : 0;
      }
    }
    if (meta) *(uint32_t*)(meta + r * (K / 8) + ch * 4) = keep;
    uint8_t* dst = codes + r * crow + ch * cbc;
    if (cbc == 8 && ((uintptr_t)dst & 7) == 0) {
      *(unsigned long long*)dst = cw;
    } else if (cbc == 4 && ((uintptr_t)dst & 3) == 0) {
      *(uint32_t*)dst = (uint32_t)cw;
    } else if ((cbc & 1) == 0 && ((uintptr_t)dst & 1) == 0) {
      for (int i = 0; i < cbc / 2; ++i) ((uint16_t*)dst)[i] = (uint16_t)(cw >> (16 * i));
    } else {
      for (int i = 0; i < cbc; ++i) dst[i] = (uint8_t)(cw >> (8 * i));
    }
    ch += dch;
    r += dr;
    if (ch >= cpr) {
      ch -= cpr;
      ++r;
    }
  }
}

}  // namespace

PackPlan pack_plan(int64_t R, int64_t K) {
  PackPlan p;
  int64_t nb = R < 2048 ? R : 2048;
  int64_t rpb = cdiv(R, nb);
  const int64_t max_rows = (int64_t(1) << 20) / K;   // keeps a block's int64 partial < 2^63
  if (rpb > max_rows) rpb = max_rows;
  if (rpb < 1) rpb = 1;
  nb = cdiv(R, rpb);
  p.nblocks = nb;
  p.rows_per_block = rpb;
  p.bytes = align256(sizeof(PackHeader) + (size_t)nb * 8);
  return p;
}

hipError_t launch_pack(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                       uint8_t* codes, uint8_t* meta, float* s_w, void* ws, hipStream_t st) {
  const PackPlan p = pack_plan(R, K);
  SBN_LAUNCH("abs_sum", abs_sum_kernel, dim3((unsigned)p.nblocks), dim3(PT), 0, st, W, R, K, ldw,
                     p.rows_per_block, (unsigned char*)ws, s_w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = R * (K / 32);
  int64_t blocks = cdiv(total, PT);
  if (blocks > 8192) blocks = 8192;
  const int64_t stride = blocks * PT;
  const int64_t cpr = K / 32;
  const int64_t dr = stride / cpr, dch = stride % cpr;
  uint8_t* mp = (n == m) ? nullptr : meta;
  if (m == 4)
    SBN_LAUNCH("mask_pack", mask_pack_kernel<4>, dim3((unsigned)blocks), dim3(PT), 0, st, W, R, K, ldw,
                       n, codes, mp, s_w, (unsigned char*)ws, total, dr, dch);
  else
    SBN_LAUNCH("mask_pack", mask_pack_kernel<8>, dim3((unsigned)blocks), dim3(PT), 0, st, W, R, K, ldw,
                       n, codes, mp, s_w, (unsigned char*)ws, total, dr, dch);
  return hipGetLastError();
}

}  // namespace sbn
