// Mask, ternarize and pack: the weight side of Sparse-BitLinear.
//
// Pass 1 sums |w| exactly; pass 2 turns the sum into the per-tensor scale
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
// Variants.  The ablation of German §4 ("Ablationsstudien") / French §5 takes
// the mask from the ternary weights instead: the key of a position becomes
// |q| in {0, 1} (q = RoundClip(w / s_w)), ties still to the lower index.  The
// optimizer step (Japanese §2.1: BF16 master weights receive the gradients;
// no optimizer is named, plain SGD is used) replaces pass 1: each chunk of W
// is updated in place, w' = bf16(fma(-lr, g, w)) (one float32 rounding, then
// round-half-to-even to bf16), and the exact sum of |w'| is formed from the
// values just written, so the step and the next pack read W once less than
// an update followed by a separate pack.
//
// Exactness of the sum.  Every bf16 magnitude is sig * 2^(e-134) with an
// 8-bit significand.  Magnitudes with exponent field e in [95, 131), i.e.
// 2^-32 <= |w| < 16, are multiples of 2^-39 below 2^4; a float64 running sum
// of at most 1024 of them stays below 2^53 units, so it is exact in any
// order.  Each thread sums at most 8 * U1 of them in float64 (U1 16-byte
// chunks, while the next U1 load) before flushing into an int64 counter of
// 2^-39 units.
// Everything outside that window (zero, subnormal, tiny or >= 16) is added
// to 256 per-exponent integer bins in LDS: exact too.  Each block writes its
// int64 partial, a flag, and its bins only if it had such values.  Pass 2
// starts with every block forming the total from those few hundred partials
// (the kernel boundary makes them visible; no device-scope fence is issued,
// which on this multi-XCD part would write back and invalidate an L2 per
// block) as a 320-bit integer in units of 2^-133, and rounds total / (R*K) to
// fp32: a float64 estimate, and an exact comparison against the two
// neighbouring midpoints whenever the estimate is too close to one of them
// to decide.  The workspace needs no initialisation.
#include <map>
#include <mutex>

#include "act_quant.h"
#include "sbn_decode.h"

namespace sbn {
namespace {

constexpr int PT = 256;                  // threads per block in pass 2
constexpr uint32_t E_LO = 95, E_HI = 131;
constexpr double FAST_SCALE = 549755813888.0;  // 2^39

// workspace: [partials: nb x i64][flags: nb x u32][bins: nb x 256 x u64], each 256-aligned
struct PackWs {
  long long* partials;
  unsigned* flags;
  unsigned long long* bins;
};
__host__ __device__ inline PackWs pack_ws(unsigned char* ws, int64_t nb) {
  PackWs p;
  p.partials = (long long*)ws;
  p.flags = (unsigned*)(ws + align256((size_t)nb * 8));
  p.bins = (unsigned long long*)(ws + align256((size_t)nb * 8) + align256((size_t)nb * 4));
  return p;
}

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

// s_w = max(RN_f32(total * 2^-133 / n), 1e-5).  The float64 estimate
// (top 96 bits of the total, one division) is within 2^-50 of the exact
// mean relative to it, so it already decides the rounding unless it lies
// within 2^-46 (relative) of a midpoint between two floats; only then are the
// exact 320-bit comparisons against those midpoints made.
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
  const double m_hi = ((double)r0 + (double)rn) * 0.5, m_lo = ((double)rp + (double)r0) * 0.5;
  const double tol = approx * 0x1p-46;
  if (fabs(approx - m_hi) > tol && fabs(approx - m_lo) > tol) return fmaxf(r0, 1e-5f);
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

// in-window test of one magnitude given as fp32 bits (low 16 bits zero)
__device__ inline bool in_window(uint32_t mag32) {
  return (mag32 - (E_LO << 23)) < ((E_HI - E_LO) << 23);
}

// |w| of the two bf16 halves of u in float64 if inside the window, else 0;
// `ok` is cleared when either half is outside it.
__device__ inline double pair_abs(uint32_t u, bool& ok) {
  const uint32_t lo = (u << 16) & 0x7FFF0000u;
  const uint32_t hi = u & 0x7FFF0000u;
  const bool lo_in = in_window(lo), hi_in = in_window(hi);
  ok = ok && (lo_in || lo == 0u) && (hi_in || hi == 0u);      // zero adds nothing either way
  return (lo_in ? (double)__uint_as_float(lo) : 0.0) + (hi_in ? (double)__uint_as_float(hi) : 0.0);
}

// the rare out-of-window values of u go to the exponent bins
__device__ inline void pair_slow(uint32_t u, unsigned long long* bins) {
  const uint32_t lo = (u << 16) & 0x7FFF0000u;
  const uint32_t hi = u & 0x7FFF0000u;
  if (!in_window(lo) && lo) slow_add(bins, lo);
  if (!in_window(hi) && hi) slow_add(bins, hi);
}

#ifndef SBN_PACK_U
#define SBN_PACK_U 2
#endif
#ifndef SBN_PACK_U1
#define SBN_PACK_U1 2
#endif
constexpr int U = SBN_PACK_U;    // 16-byte chunks per thread per step in pass 2 (2:4), plus as many prefetched
constexpr int U1 = SBN_PACK_U1;  // the same in pass 1
constexpr int PT1 = 1024; // pass-1 threads per block: 16 waves keep 64 KB of W in flight per CU

template <bool FLAT>
__device__ inline uint4 chunk_at(const uint16_t* __restrict__ W, int64_t c, int64_t kc, int64_t ldw) {
  if (FLAT) return ((const uint4*)W)[c];
  const int64_t r = c / kc;
  return *(const uint4*)(W + r * ldw + (c - r * kc) * 8);
}

// Pass 1: block b sums |w| over 16-byte chunks [b*cpb, (b+1)*cpb) of the
// row-major chunk order (8 weights per chunk).  Each thread sums U1 chunks per
// step while the next U1 load, and flushes its float64 sum (<= 8*U1 terms,
// exact) into int64 units; out-of-window values take one rare branch per
// group into the LDS bins.
// The SGD step on one chunk of 8 bf16 weights and their 8 float32 gradients.
__device__ inline uint4 sgd_chunk(uint4 w, float4 g0, float4 g1, float nlr) {
  const uint32_t in[4] = {w.x, w.y, w.z, w.w};
  const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = f32_to_bf16_rne(__builtin_fmaf(nlr, g[2 * j], __uint_as_float(in[j] << 16)));
    const uint32_t hi = f32_to_bf16_rne(__builtin_fmaf(nlr, g[2 * j + 1], __uint_as_float(in[j] & 0xFFFF0000u)));
    out[j] = lo | (hi << 16);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

template <bool FLAT>
__device__ inline void grad_at(const float* __restrict__ G, int64_t c, int64_t kc, int64_t ldg, float4& g0,
                               float4& g1) {
  const float4* p;
  if (FLAT) {
    p = (const float4*)G + 2 * c;
  } else {
    const int64_t r = c / kc;
    p = (const float4*)(G + r * ldg + (c - r * kc) * 8);
  }
  g0 = p[0];
  g1 = p[1];
}

// The exact sum of the magnitudes of one step's chunks in units of 2^-39.
// Fast path: every magnitude is summed, and one max and one min over the
// step tell whether any nonzero one lies outside the window (m - 1 wraps
// zero to the top, so zeros never count as too small); if one does, the step
// is summed again with the out-of-window values left to the bins (rare).  The
// two bf16 magnitudes of a word are tested side by side as 16-bit lanes.
template <int N>
__device__ inline unsigned long long step_abs_sum(const uint4 (&cv)[N], unsigned long long* bins, int* any_slow) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  double acc = 0.0;
  u16x2 mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
  const u16x2 one = {1, 1};
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const uint32_t q[4] = {cv[u].x, cv[u].y, cv[u].z, cv[u].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m = q[j] & 0x7FFF7FFFu;
      const u16x2 m2 = __builtin_bit_cast(u16x2, m);
      mx = __builtin_elementwise_max(mx, m2);
      mn = __builtin_elementwise_min(mn, m2 - one);
      acc += (double)__uint_as_float(m << 16) + (double)__uint_as_float(m & 0xFFFF0000u);
    }
  }
  const uint32_t mxs = max((uint32_t)mx.x, (uint32_t)mx.y), mns = min((uint32_t)mn.x, (uint32_t)mn.y);
  if (mxs >= (E_HI << 7) || mns < (E_LO << 7) - 1u) {
    *any_slow = 1;
    bool ok = true;
    acc = 0.0;
#pragma unroll
    for (int u = 0; u < N; ++u)
      acc += pair_abs(cv[u].x, ok) + pair_abs(cv[u].y, ok) + pair_abs(cv[u].z, ok) + pair_abs(cv[u].w, ok);
#pragma unroll
    for (int u = 0; u < N; ++u) {
      pair_slow(cv[u].x, bins);
      pair_slow(cv[u].y, bins);
      pair_slow(cv[u].z, bins);
      pair_slow(cv[u].w, bins);
    }
  }
  return (unsigned long long)(acc * FAST_SCALE);   // exact integer < 2^53
}

// UPD: the optimizer step -- chunk c of W is first updated in place with the
// gradient chunk of G (row stride ldg), nlr = -lr; the sum is of the new values.
// Pass 1 as block `blk` of `nb` (the body of abs_sum_kernel and of the fused
// pass-1 + activation-quantizer kernel).
template <bool FLAT, bool UPD>
__device__ inline void abs_sum_body(int64_t blk, int64_t nb, const uint16_t* __restrict__ W, int64_t R,
                                    int64_t K, int64_t ldw, int64_t cpb, unsigned char* __restrict__ ws,
                                    const float* __restrict__ G, int64_t ldg, float nlr) {
  const PackWs pw = pack_ws(ws, nb);
  __shared__ unsigned long long bins[256];
  __shared__ unsigned long long red[PT1 / 64];
  __shared__ int any_slow;
  const int tid = threadIdx.x;
  if (tid < 256) bins[tid] = 0;
  if (tid == 0) any_slow = 0;
  __syncthreads();
  const int64_t kc = K / 8, total = R * kc;
  const int64_t c0 = blk * cpb;
  const int64_t c1 = min(total, c0 + cpb);
  unsigned long long acc_i = 0;
  constexpr int64_t STEP = (int64_t)PT1 * U1;
  uint4 v[U1], nx[U1];
  float4 g[U1][2], ng[U1][2];
  // Every load is issued (past the block's end it rereads the block's last
  // chunk, and that copy is zeroed before use): with no load under a divergent
  // branch the wait before the sums covers only the chunks being summed, not
  // the next ones in flight.
  int64_t base = c0 + tid;
#pragma unroll
  for (int u = 0; u < U1; ++u) {
    const int64_t c = min(base + (int64_t)u * PT1, c1 - 1);
    v[u] = chunk_at<FLAT>(W, c, kc, ldw);
    if (UPD) grad_at<FLAT>(G, c, kc, ldg, g[u][0], g[u][1]);
  }
  for (; base < c1; base += STEP) {
#pragma unroll
    for (int u = 0; u < U1; ++u) {               // next chunks load while these are summed
      const int64_t c = min(base + STEP + (int64_t)u * PT1, c1 - 1);
      nx[u] = chunk_at<FLAT>(W, c, kc, ldw);
      if (UPD) grad_at<FLAT>(G, c, kc, ldg, ng[u][0], ng[u][1]);
    }
#pragma unroll
    for (int u = 0; u < U1; ++u)
      if (base + (int64_t)u * PT1 >= c1) v[u] = make_uint4(0, 0, 0, 0);
    if (UPD) {
#pragma unroll
      for (int u = 0; u < U1; ++u) {
        const int64_t c = base + (int64_t)u * PT1;
        if (c < c1) {
          v[u] = sgd_chunk(v[u], g[u][0], g[u][1], nlr);
          uint16_t* dst;
          if (FLAT) {
            dst = (uint16_t*)W + c * 8;
          } else {
            const int64_t r = c / kc;
            dst = (uint16_t*)W + r * ldw + (c - r * kc) * 8;
          }
          *(uint4*)dst = v[u];
        }
      }
    }
    acc_i += step_abs_sum(v, bins, &any_slow);
#pragma unroll
    for (int u = 0; u < U1; ++u) {
      v[u] = nx[u];
      if (UPD) {
        g[u][0] = ng[u][0];
        g[u][1] = ng[u][1];
      }
    }
  }
  const unsigned long long s = wave_sum_u64(acc_i);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    unsigned long long b = 0;
    for (int i = 0; i < PT1 / 64; ++i) b += red[i];
    pw.partials[blk] = (long long)b;
    pw.flags[blk] = any_slow ? 1u : 0u;
  }
  if (any_slow && tid < 256) pw.bins[blk * 256 + tid] = bins[tid];
}

template <bool FLAT, bool UPD>
__global__ __launch_bounds__(PT1) void abs_sum_kernel(const uint16_t* __restrict__ W, int64_t R,
                                                     int64_t K, int64_t ldw, int64_t cpb,
                                                     unsigned char* __restrict__ ws,
                                                     const float* __restrict__ G, int64_t ldg, float nlr) {
  abs_sum_body<FLAT, UPD>(blockIdx.x, gridDim.x, W, R, K, ldw, cpb, ws, G, ldg, nlr);
}


// Block-wide (256 threads): total = sum of the pass-1 partials (2^-39 units)
// + the flagged blocks' bins (sig * 2^(e-134) each), then
// s_w = max(RN_fp32(total / numel), 1e-5).  Every pass-2 block forms it from
// the <= a few hundred partials (the kernel boundary after pass 1 makes them
// visible, so no device-scope fence is needed); block 0 also stores it.
__device__ float scale_from_partials(const unsigned char* __restrict__ ws, int64_t nb, int64_t numel,
                                     float* __restrict__ s_w_out, bool store) {
  const PackWs pw = pack_ws((unsigned char*)ws, nb);
  const int tid = threadIdx.x;
  __shared__ unsigned long long wlo[PT / 64], whi[PT / 64];
  __shared__ unsigned long long ebin[256];
  __shared__ int nflag;
  __shared__ int flagged[PT];
  __shared__ float s_sh;
  if (tid == 0) nflag = 0;
  __syncthreads();
  // each partial (< 2^63) split into 32-bit halves, summed separately in u64
  unsigned long long lo = 0, hi = 0;
  for (int64_t i = tid; i < nb; i += PT) {
    const unsigned long long p = (unsigned long long)pw.partials[i];
    lo += p & 0xFFFFFFFFull;
    hi += p >> 32;
    if (pw.flags[i]) {
      const int slot = atomicAdd(&nflag, 1);
      if (slot < PT) flagged[slot] = (int)i;
    }
  }
  lo = wave_sum_u64(lo);
  hi = wave_sum_u64(hi);
  if ((tid & 63) == 0) {
    wlo[tid >> 6] = lo;
    whi[tid >> 6] = hi;
  }
  __syncthreads();
  const int nf = nflag;
  unsigned long long eb = 0;                     // exponent bin `tid` over the flagged blocks (rare)
  if (nf > 0 && nf <= PT) {
    for (int j = 0; j < nf; ++j) eb += pw.bins[(int64_t)flagged[j] * 256 + tid];
  } else if (nf > PT) {
    for (int64_t i = 0; i < nb; ++i)
      if (pw.flags[i]) eb += pw.bins[i * 256 + tid];
  }
  if (nf) ebin[tid] = eb;
  __syncthreads();
  if (tid == 0) {
    unsigned __int128 F = 0;
    for (int w = 0; w < PT / 64; ++w) F += (unsigned __int128)wlo[w] + ((unsigned __int128)whi[w] << 32);
    Big t;
    big_zero(t);
    // fast part: F units of 2^-39 = F * 2^94 units of 2^-133
    big_add_shifted(t, (unsigned long long)F, 94);
    big_add_shifted(t, (unsigned long long)(F >> 64), 94 + 64);
    if (nf)
      for (int e = 0; e < 256; ++e)
        if (ebin[e]) big_add_shifted(t, ebin[e], (e ? e : 1) - 1);
    const float sw = round_mean(t, (unsigned long long)numel);
    s_sh = sw;
    if (store) *s_w_out = sw;
  }
  __syncthreads();
  return s_sh;
}

// ------------------------------------------------------------------ pass 2
// One thread = 32 consecutive weights of one row (32/M whole groups).
template <int M, int n>
__device__ inline void mask_pack_body(
    int64_t blk, int64_t nblk, const uint16_t* __restrict__ W, int64_t R, int64_t K, int64_t ldw,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ meta, float* __restrict__ s_w_ptr,
    const unsigned char* __restrict__ ws, int64_t nb, int64_t total_chunks, int64_t dr, int64_t dch,
    int tmask) {
  const float h = 0.5f * scale_from_partials(ws, nb, R * K, s_w_ptr, blk == 0);
  const uint32_t thr = __float_as_uint(h) >> 16;      // |w| > h  <=>  key > thr
  const int64_t cpr = K / 32;
  const int64_t crow = K * n / (4 * M);               // code bytes per row
  const int cbc = 8 * n / M;                          // code bytes per chunk (M=8: n, M=4: 2n)
  int64_t c = blk * PT + threadIdx.x;
  int64_t r = c / cpr, ch = c - r * cpr;
  for (; c < total_chunks; c += nblk * PT) {
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
        const uint32_t nz = a > thr ? 1u : 0u;
        key[p] = ((tmask ? nz : a) << 3) | (uint32_t)(7 - p);   // distinct; lower index wins ties
        code[p] = nz | ((nz & (w >> 15)) << 1);          // 00 = 0, 01 = +1, 11 = -1
      }
      // Survivors: the n largest of M distinct keys.  n = 1, 2, M - 2, M - 1 take
      // the one or two extreme keys from a min/max network (the largest two or
      // the smallest two: from sorted pairs, the two extremes of a union of two
      // sorted pairs are min(x1, y1) and min(max(x1, y1), min(x2, y2)), and
      // likewise with max), which name the kept or dropped positions; other n
      // count each key's rank.
      constexpr int mode = (n == 1 || n == 2) ? 1 : (n == M - 1 || n == M - 2) ? 2 : 0;
      uint32_t e1x = 0, e2x = 0;
      if (mode != 0) {
        const bool big = mode == 1;                      // keep the largest (else drop the smallest)
        const bool two = big ? n == 2 : n == M - 2;
        uint32_t e1[M / 2], e2[M / 2];                   // per pair: extreme, other
#pragma unroll
        for (int i = 0; i < M / 2; ++i) {
          const uint32_t x = key[2 * i], y = key[2 * i + 1];
          e1[i] = big ? max(x, y) : min(x, y);
          e2[i] = big ? min(x, y) : max(x, y);
        }
#pragma unroll
        for (int w2 = M / 2; w2 > 1; w2 >>= 1) {        // merge pairs of (first, second) extremes
#pragma unroll
          for (int i = 0; i < w2 / 2; ++i) {
            const uint32_t x1 = e1[2 * i], x2 = e2[2 * i], y1 = e1[2 * i + 1], y2 = e2[2 * i + 1];
            e1[i] = big ? max(x1, y1) : min(x1, y1);
            e2[i] = big ? max(min(x1, y1), max(x2, y2)) : min(max(x1, y1), min(x2, y2));
          }
        }
        e1x = e1[0];                                     // the largest (big) / smallest key
        e2x = e2[0];                                     // the second largest / second smallest
      }
      if (mode != 0) {
        // the network's extreme keys name the positions directly (key & 7 = 7 - p):
        // mode 1 keeps those positions, mode 2 drops them; the survivors' codes
        // are the group's code word with the dropped 2-bit fields cut out (mode 2)
        // or the kept fields picked (mode 1)
        const bool two = mode == 1 ? n == 2 : n == M - 2;
        const uint32_t pa = 7u - (e1x & 7u), pb = two ? 7u - (e2x & 7u) : pa;
        const uint32_t lo = pa < pb ? pa : pb, hi = pa < pb ? pb : pa;
        const uint32_t sel = (1u << pa) | (1u << pb);
        uint32_t cg = 0;
#pragma unroll
        for (int p = 0; p < M; ++p) cg |= code[p] << (2 * p);
        uint32_t packed;
        if (mode == 1) {
          packed = two ? ((cg >> (2 * lo)) & 3u) | (((cg >> (2 * hi)) & 3u) << 2) : (cg >> (2 * lo)) & 3u;
        } else {
          packed = (cg & ((1u << (2 * hi)) - 1u)) | ((cg >> (2 * hi + 2)) << (2 * hi));    // cut field hi
          if (two) packed = (packed & ((1u << (2 * lo)) - 1u)) | ((packed >> (2 * lo + 2)) << (2 * lo));   // then lo
        }
        const uint32_t keepg = mode == 1 ? sel : (((1u << M) - 1u) ^ sel);
        keep |= keepg << (g * M);
        cw |= (unsigned long long)packed << (2 * n * g);
      } else {
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

// Pass 2 for 2:4 (the common case).  A 16-byte chunk of W (8 weights, two
// groups) yields exactly one meta byte and one codes byte, both at the
// chunk's flat index, so lanes take consecutive chunks (coalesced loads and
// stores) with U loads in flight.  Per group the second-largest of four
// distinct keys (|w| << 2 | 3 - p) is the threshold; the two keys at or above
// it survive and their codes are picked with find-first-bit.
template <bool TMASK>
__device__ inline void group24(uint32_t w01, uint32_t w23, uint32_t thr, uint32_t& keep4, uint32_t& code4) {
  if constexpr (!TMASK) {
    // keys |w| << 2 | (3 - p), built in place from the two words (distinct; a
    // tie in |w| goes to the lower position); the largest and second largest
    // key name the survivors through their low two bits
    const uint32_t k0 = ((w01 << 2) & 0x1FFFCu) | 3u, k1 = ((w01 >> 14) & 0x1FFFCu) | 2u;
    const uint32_t k2 = ((w23 << 2) & 0x1FFFCu) | 1u, k3 = (w23 >> 14) & 0x1FFFCu;
    const uint32_t hi01 = max(k0, k1), lo01 = min(k0, k1), hi23 = max(k2, k3), lo23 = min(k2, k3);
    const uint32_t ka = max(hi01, hi23), kb = max(min(hi01, hi23), max(lo01, lo23));
    const uint32_t ta = ka & 3u, tb = kb & 3u;                 // 3 - position
    keep4 = (8u >> ta) | (8u >> tb);
    // a survivor's code: nonzero where |w| > thr, i.e. key > thr << 2 | 3; its
    // sign is bit 8p + 7 of the four high bytes gathered by one permute
    const uint32_t thr4 = (thr << 2) | 3u;
    const uint32_t sg = __builtin_amdgcn_perm(w23, w01, 0x07050301u);
    const uint32_t na = ka > thr4 ? 1u : 0u, nb = kb > thr4 ? 1u : 0u;
    const uint32_t sa = (sg << (8u * ta)) >> 31, sb = (sg << (8u * tb)) >> 31;
    const uint32_t ca = na | ((na & sa) << 1), cb = nb | ((nb & sb) << 1);
    code4 = ta > tb ? (ca | (cb << 2)) : (cb | (ca << 2));   // the lower position first
    return;
  }
  constexpr int tmask = 1;                       // keys from the ternary magnitude (|q| in {0, 1})
  const uint32_t w[4] = {w01 & 0xFFFFu, w01 >> 16, w23 & 0xFFFFu, w23 >> 16};
  uint32_t k[4], code8 = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t a = w[p] & 0x7FFFu;
    const uint32_t nz = a > thr ? 1u : 0u;
    k[p] = ((tmask ? nz : a) << 2) | (uint32_t)(3 - p);
    code8 |= (nz | ((nz & (w[p] >> 15)) << 1)) << (2 * p);
  }
  const uint32_t hi01 = max(k[0], k[1]), lo01 = min(k[0], k[1]);
  const uint32_t hi23 = max(k[2], k[3]), lo23 = min(k[2], k[3]);
  const uint32_t second = max(min(hi01, hi23), max(lo01, lo23));
  keep4 = (k[0] >= second ? 1u : 0u) | (k[1] >= second ? 2u : 0u) | (k[2] >= second ? 4u : 0u) |
          (k[3] >= second ? 8u : 0u);
  const uint32_t p0 = __builtin_ctz(keep4), p1 = 31u - __builtin_clz(keep4);
  code4 = ((code8 >> (2 * p0)) & 3u) | (((code8 >> (2 * p1)) & 3u) << 2);
}

template <bool FLAT, bool TMASK>
__device__ inline void mask_pack24_loop(int64_t blk, int64_t nblk, const uint16_t* __restrict__ W, int64_t K,
                                        int64_t ldw, int64_t total, uint8_t* __restrict__ codes,
                                        uint8_t* __restrict__ meta, uint32_t thr, int64_t base, uint4 (&v)[U]) {
  const int64_t kc = K / 8;
  const int64_t step = nblk * PT * U;
  uint4 nx[U];
  for (; base < total; base += step) {
    if (base + step < total) {                   // next chunks load while these are packed
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = base + step + (int64_t)u * PT;
        nx[u] = c < total ? chunk_at<FLAT>(W, c, kc, ldw) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = base + (int64_t)u * PT;
      if (c < total) {
        uint32_t k0, c0, k1, c1;
        group24<TMASK>(v[u].x, v[u].y, thr, k0, c0);
        group24<TMASK>(v[u].z, v[u].w, thr, k1, c1);
        meta[c] = (uint8_t)(k0 | (k1 << 4));
        codes[c] = (uint8_t)(c0 | (c1 << 4));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = nx[u];
  }
}

template <bool FLAT>
__device__ inline void mask_pack24_body(
    int64_t blk, int64_t nblk, const uint16_t* __restrict__ W, int64_t R, int64_t K, int64_t ldw,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ meta, float* __restrict__ s_w_ptr,
    const unsigned char* __restrict__ ws, int64_t nb, int tmask) {
  const int64_t kc = K / 8, total = R * kc;
  const int64_t base = blk * PT * U + threadIdx.x;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {                  // first loads fly while the scale is formed
    const int64_t c = base + (int64_t)u * PT;
    v[u] = c < total ? chunk_at<FLAT>(W, c, kc, ldw) : make_uint4(0, 0, 0, 0);
  }
  const float h = 0.5f * scale_from_partials(ws, nb, R * K, s_w_ptr, blk == 0);
  const uint32_t thr = __float_as_uint(h) >> 16;
  if (tmask) mask_pack24_loop<FLAT, true>(blk, nblk, W, K, ldw, total, codes, meta, thr, base, v);
  else mask_pack24_loop<FLAT, false>(blk, nblk, W, K, ldw, total, codes, meta, thr, base, v);
}

struct MaskPackArgs {
  const uint16_t* W;
  int64_t R, K, ldw;
  int n;
  uint8_t* codes;
  uint8_t* meta;
  float* s_w;
  const unsigned char* ws;
  int64_t nb, total_chunks, dr, dch;
  int tmask;
};

// KIND: 0 = 2:4 with ldw == K, 1 = 2:4, 16 m + n = n of a group of m (4 or 8).
template <int KIND>
__device__ inline void mask_pack_dispatch(int64_t blk, int64_t nblk, const MaskPackArgs& a) {
  if constexpr (KIND == 0)
    mask_pack24_body<true>(blk, nblk, a.W, a.R, a.K, a.ldw, a.codes, a.meta, a.s_w, a.ws, a.nb, a.tmask);
  else if constexpr (KIND == 1)
    mask_pack24_body<false>(blk, nblk, a.W, a.R, a.K, a.ldw, a.codes, a.meta, a.s_w, a.ws, a.nb, a.tmask);
  else
    mask_pack_body<KIND / 16, KIND % 16>(blk, nblk, a.W, a.R, a.K, a.ldw, a.codes, a.meta, a.s_w, a.ws, a.nb, a.total_chunks,
                         a.dr, a.dch, a.tmask);
}

template <int KIND>
__global__ __launch_bounds__(PT) void mask_pack_kernel(const MaskPackArgs a) {
  mask_pack_dispatch<KIND>(blockIdx.x, gridDim.x, a);
}

// The forward's pass 2: blocks [0, nblk) mask and pack W, blocks [nblk, nblk + T)
// quantize one token each.  The quantizer does not depend on the pack, so one
// grid runs them side by side (one launch, and the short token blocks fill the
// compute units beside the pack's loop).
struct QuantArgs {
  const uint16_t* X;
  int64_t T, K, ldx;
  int8_t* Xq;
  float* s_x;
};

template <int KIND, int CH>
__global__ __launch_bounds__(PT) void mask_pack_quant_kernel(const MaskPackArgs a, int64_t nblk, const QuantArgs q) {
  const int64_t b = blockIdx.x;
  if (b < nblk) {
    mask_pack_dispatch<KIND>(b, nblk, a);
  } else {
    __shared__ uint32_t qred[PT / 64];
    act_quant_token<CH>(true, b - nblk, threadIdx.x, qred, q.X, q.K, q.ldx, q.Xq, q.s_x);
  }
}

// Pass 2 at 2:4 for the one-call forward whose GEMM reads a prepared weight
// operand: besides the planes it writes the structured-sparse operand of the
// matrix instruction (16 int8 values and one word of 2-bit indices per lane
// and 128-K step), decoded from the planes' words by the same routine as the
// layout launch's expansion, so that launch does not run.  Block (g, kq): the
// 64 rows of index block g (row fragments 4g .. 4g+3, one per wave) over the
// K steps [kqs kq, kqs kq + kqs); lane l of wave q owns row
// 16 (4g + q) + l % 16 and positions 32 (l / 16) .. +32 of each step, i.e.
// its own lane of the operand fragment: a wave stores one whole 1 KB fragment
// per step, and the four waves fill each 16-byte unit of the index block.
constexpr int OP_KQ = 10;                            // at most this many K steps per block
struct OperandArgs {
  uint8_t* vals;                                     // [RB][KBn][64][16 B]
  uint32_t* idx;                                     // [RB/4][KBn][64][4]
  int64_t RB, KBn, nkq, kqs;                         // kqs: K steps per block (the last may hold fewer)
};

__device__ inline void mask_pack24_operand_body(int64_t blk, const MaskPackArgs& a, const OperandArgs& o) {
  const int64_t g = blk / o.nkq, kq = blk - g * o.nkq;
  const int q = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t rb = 4 * g + q, r = rb * 16 + (l & 15);
  const int64_t K = a.K, rowb = K / 8;
  const int64_t kb0 = kq * o.kqs, kb1 = min(kb0 + o.kqs, o.KBn);
  const bool rowin = r < a.R;
  const uint16_t* wrow = a.W + (rowin ? r : 0) * a.ldw;
  // The 64 bytes of W of step kb (always loaded: a row past R or positions past
  // K read the row's start instead, and that copy is not used).
  auto load = [&](int64_t kb, uint4 (&d)[4]) {
    const int64_t k0 = kb * 128 + 32 * (l >> 4);
    const uint4* src = (const uint4*)(wrow + (rowin && k0 < K ? k0 : 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = src[i];
  };
  uint4 v[4], nv[4];
  load(kb0, v);                                      // the first loads fly while the scale is formed
  const float h = 0.5f * scale_from_partials(a.ws, a.nb, a.R * K, a.s_w, blk == 0);
  const uint32_t thr = __float_as_uint(h) >> 16;
  for (int64_t kb = kb0; kb < kb1; ++kb) {
    load(kb + 1 < kb1 ? kb + 1 : kb, nv);
    const int64_t k0 = kb * 128 + 32 * (l >> 4);
    const bool in = rowin && k0 < K;
    uint32_t mb = 0, cb = 0;                         // the planes' words of these 32 positions
#pragma unroll
    for (int c = 0; c < 4; ++c) {                    // chunk c: positions 8c .. 8c+7, two groups
      uint32_t k0c, c0c, k1c, c1c;
      group24<false>(v[c].x, v[c].y, thr, k0c, c0c);
      group24<false>(v[c].z, v[c].w, thr, k1c, c1c);
      mb |= (k0c | (k1c << 4)) << (8 * c);
      cb |= (c0c | (c1c << 4)) << (8 * c);
    }
    v4i av = (v4i){0, 0, 0, 0};
    int ix = 0x44444444;                             // (0,1) in every half: harmless with zero values
    if (in) {
      *(uint32_t*)(a.meta + r * rowb + k0 / 8) = mb;
      *(uint32_t*)(a.codes + r * rowb + k0 / 8) = cb;
      decode24(mb, cb, av, ix);
    }
    *(v4i*)(o.vals + ((rb * o.KBn + kb) * 64 + l) * 16) = av;
    o.idx[((g * o.KBn + kb) * 64 + l) * 4 + q] = (uint32_t)ix;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = nv[i];
  }
}

// Blocks [0, nop) pack W and write the operand, blocks [nop, nop + T) quantize one token each.
template <int CH>
__global__ __launch_bounds__(PT) void mask_pack_quant_operand_kernel(const MaskPackArgs a, const OperandArgs o,
                                                                     int64_t nop, const QuantArgs qa) {
  const int64_t b = blockIdx.x;
  if (b < nop) {
    mask_pack24_operand_body(b, a, o);
  } else {
    __shared__ uint32_t qred[PT / 64];
    act_quant_token<CH>(true, b - nop, threadIdx.x, qred, qa.X, qa.K, qa.ldx, qa.Xq, qa.s_x);
  }
}

}  // namespace

PackPlan pack_plan(int64_t R, int64_t K) {
  PackPlan p;
  const int64_t total = R * (K / 8);                    // 16-byte chunks
  int64_t nb = cdiv(total, (int64_t)PT1 * U1);
  if (nb > 256) nb = 256;                               // pass 2 reduces one partial per thread
  const int64_t max_cpb = (int64_t(1) << 20) / 8;       // a block's int64 partial stays < 2^63
  int64_t cpb = cdiv(total, nb);
  if (cpb > max_cpb) cpb = max_cpb;
  nb = cdiv(total, cpb);
  p.nblocks = nb;
  p.chunks_per_block = cpb;
  p.bytes = align256((size_t)nb * 8) + align256((size_t)nb * 4) + align256((size_t)nb * 256 * 8);
  return p;
}

static MaskPackArgs mask_pack_args(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                                   uint8_t* codes, uint8_t* meta, float* s_w, const void* ws, uint32_t flags,
                                   int64_t nb, int64_t& nblk, int& kind) {
  MaskPackArgs a;
  a.W = W; a.R = R; a.K = K; a.ldw = ldw; a.n = n;
  a.codes = codes; a.meta = (n == m) ? nullptr : meta; a.s_w = s_w;
  a.ws = (const unsigned char*)ws; a.nb = nb;
  a.tmask = (flags & SBN_MASK_FROM_TERNARY) ? 1 : 0;
  a.total_chunks = R * (K / 32);
  if (n == 2 && m == 4) {
    nblk = cdiv(R * (K / 8), (int64_t)PT * U);
    if (nblk > 1024) nblk = 1024;                       // four blocks per CU, looping
    kind = ldw == K ? 0 : 1;
    a.dr = a.dch = 0;
  } else {
    nblk = cdiv(a.total_chunks, PT);
    if (nblk > 1024) nblk = 1024;                       // four blocks per CU, looping: each block forms the scale once
    const int64_t stride = nblk * PT, cpr = K / 32;
    a.dr = stride / cpr;
    a.dch = stride % cpr;
    kind = 16 * m + n;
  }
  return a;
}

static hipError_t launch_mask_pack(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                                   uint8_t* codes, uint8_t* meta, float* s_w, void* ws, uint32_t flags,
                                   int64_t nb, hipStream_t st) {
  int64_t nblk;
  int kind;
  const MaskPackArgs a = mask_pack_args(W, R, K, ldw, n, m, codes, meta, s_w, ws, flags, nb, nblk, kind);
  const dim3 grid((unsigned)nblk), block(PT);
  if (kind == 0) SBN_LAUNCH("mask_pack", mask_pack_kernel<0>, grid, block, 0, st, a);
  else if (kind == 1) SBN_LAUNCH("mask_pack", mask_pack_kernel<1>, grid, block, 0, st, a);
#define SBN_MP_CASE(KD) \
  else if (kind == KD) SBN_LAUNCH("mask_pack", mask_pack_kernel<KD>, grid, block, 0, st, a);
  SBN_MP_CASE(65) SBN_MP_CASE(67) SBN_MP_CASE(68)                  // 1:4, 3:4, 4:4
  SBN_MP_CASE(129) SBN_MP_CASE(130) SBN_MP_CASE(131) SBN_MP_CASE(132)   // 1:8 .. 8:8
  SBN_MP_CASE(133) SBN_MP_CASE(134) SBN_MP_CASE(135) SBN_MP_CASE(136)
#undef SBN_MP_CASE
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                       uint8_t* codes, uint8_t* meta, float* s_w, void* ws, uint32_t flags,
                       const float* G, int64_t ldg, float lr, hipStream_t st) {
  const PackPlan p = pack_plan(R, K);
  const bool flat = ldw == K && (G == nullptr || ldg == K);
  const dim3 g1((unsigned)p.nblocks), b1(PT1);
  const float nlr = -lr;
  if (G == nullptr && flat)
    SBN_LAUNCH("abs_sum", (abs_sum_kernel<true, false>), g1, b1, 0, st, W, R, K, ldw, p.chunks_per_block,
               (unsigned char*)ws, G, ldg, nlr);
  else if (G == nullptr)
    SBN_LAUNCH("abs_sum", (abs_sum_kernel<false, false>), g1, b1, 0, st, W, R, K, ldw, p.chunks_per_block,
               (unsigned char*)ws, G, ldg, nlr);
  else if (flat)
    SBN_LAUNCH("sgd_abs_sum", (abs_sum_kernel<true, true>), g1, b1, 0, st, W, R, K, ldw, p.chunks_per_block,
               (unsigned char*)ws, G, ldg, nlr);
  else
    SBN_LAUNCH("sgd_abs_sum", (abs_sum_kernel<false, true>), g1, b1, 0, st, W, R, K, ldw, p.chunks_per_block,
               (unsigned char*)ws, G, ldg, nlr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_mask_pack(W, R, K, ldw, n, m, codes, meta, s_w, ws, flags, p.nblocks, st);
}

hipError_t launch_pack_quant(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                             uint8_t* codes, uint8_t* meta, float* s_w, void* ws, uint32_t flags,
                             const uint16_t* X, int64_t T, int64_t ldx, int8_t* Xq, float* s_x, hipStream_t st) {
  const PackPlan p = pack_plan(R, K);
  if (ldw == K)
    SBN_LAUNCH("abs_sum", (abs_sum_kernel<true, false>), dim3((unsigned)p.nblocks), dim3(PT1), 0, st, W, R, K, ldw,
               p.chunks_per_block, (unsigned char*)ws, nullptr, 0, 0.0f);
  else
    SBN_LAUNCH("abs_sum", (abs_sum_kernel<false, false>), dim3((unsigned)p.nblocks), dim3(PT1), 0, st, W, R, K, ldw,
               p.chunks_per_block, (unsigned char*)ws, nullptr, 0, 0.0f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t nblk;
  int kind;
  const MaskPackArgs a = mask_pack_args(W, R, K, ldw, n, m, codes, meta, s_w, ws, flags, p.nblocks, nblk, kind);
  if (kind > 1) {
    // the rank-count pass of other ratios fills the chip by itself (up to 8192
    // blocks): the quantizer gains nothing beside it and runs after it
    e = launch_mask_pack(W, R, K, ldw, n, m, codes, meta, s_w, ws, flags, p.nblocks, st);
    return e != hipSuccess ? e : launch_act_quant(X, T, K, ldx, Xq, s_x, st);
  }
  const QuantArgs q{X, T, K, ldx, Xq, s_x};
  const dim3 grid((unsigned)(nblk + T)), block(PT);
  const int ch = act_quant_ch(K);
#define SBN_MPQ(KIND)                                                                                          \
  do {                                                                                                         \
    if (ch == 1) SBN_LAUNCH("mask_pack_quant", (mask_pack_quant_kernel<KIND, 1>), grid, block, 0, st, a, nblk, q); \
    else if (ch == 2) SBN_LAUNCH("mask_pack_quant", (mask_pack_quant_kernel<KIND, 2>), grid, block, 0, st, a, nblk, q); \
    else if (ch == 4) SBN_LAUNCH("mask_pack_quant", (mask_pack_quant_kernel<KIND, 4>), grid, block, 0, st, a, nblk, q); \
    else SBN_LAUNCH("mask_pack_quant", (mask_pack_quant_kernel<KIND, 0>), grid, block, 0, st, a, nblk, q);  \
  } while (0)
  if (kind == 0) SBN_MPQ(0);
  else SBN_MPQ(1);
#undef SBN_MPQ
  return hipGetLastError();
}

hipError_t launch_pack_quant_operand(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, uint8_t* codes,
                                     uint8_t* meta, float* s_w, void* ws, const uint16_t* X, int64_t T, int64_t ldx,
                                     int8_t* Xq, float* s_x, uint8_t* vals, uint32_t* idx, hipStream_t st) {
  const PackPlan p = pack_plan(R, K);
  if (ldw == K)
    SBN_LAUNCH("abs_sum", (abs_sum_kernel<true, false>), dim3((unsigned)p.nblocks), dim3(PT1), 0, st, W, R, K, ldw,
               p.chunks_per_block, (unsigned char*)ws, nullptr, 0, 0.0f);
  else
    SBN_LAUNCH("abs_sum", (abs_sum_kernel<false, false>), dim3((unsigned)p.nblocks), dim3(PT1), 0, st, W, R, K, ldw,
               p.chunks_per_block, (unsigned char*)ws, nullptr, 0, 0.0f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MaskPackArgs a = {};
  a.W = W; a.R = R; a.K = K; a.ldw = ldw; a.n = 2;
  a.codes = codes; a.meta = meta; a.s_w = s_w;
  a.ws = (const unsigned char*)ws; a.nb = p.nblocks;
  a.tmask = 0;
  OperandArgs o;
  o.vals = vals;
  o.idx = idx;
  o.RB = round_up(R, (int64_t)GEMM_TILE_R) / 16;
  o.KBn = cdiv(K, (int64_t)128);
  o.nkq = cdiv(o.KBn, (int64_t)OP_KQ);              // the K steps split evenly over the fewest blocks
  o.kqs = cdiv(o.KBn, o.nkq);                        // of at most OP_KQ steps (fewer, longer blocks
                                                     // measured faster: 10 steps 17.4 us, 5 steps 18.8 us)
  const int64_t nop = (o.RB / 4) * o.nkq;
  const QuantArgs q{X, T, K, ldx, Xq, s_x};
  const dim3 grid((unsigned)(nop + T)), block(PT);
  const int ch = act_quant_ch(K);
  if (ch == 1) SBN_LAUNCH("mask_pack_quant", mask_pack_quant_operand_kernel<1>, grid, block, 0, st, a, o, nop, q);
  else if (ch == 2) SBN_LAUNCH("mask_pack_quant", mask_pack_quant_operand_kernel<2>, grid, block, 0, st, a, o, nop, q);
  else if (ch == 4) SBN_LAUNCH("mask_pack_quant", mask_pack_quant_operand_kernel<4>, grid, block, 0, st, a, o, nop, q);
  else SBN_LAUNCH("mask_pack_quant", mask_pack_quant_operand_kernel<0>, grid, block, 0, st, a, o, nop, q);
  return hipGetLastError();
}

// ----------------------------------------------------------------- allocation-free pack
// Workspace of sbn_mask_ternarize_pack_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  It takes the pack workspace
// (per-block int64 partials, flags and exponent bins), which every call
// writes in full before reading, so nothing in it has to be cleared; up to
// 256 pass-1 blocks fit, i.e. every weight with R*K <= 2^28.  In host code the
// array's name is not a device address: its address on the current device
// comes from hipGetSymbolAddress, once per device, and only that address is
// handed to the kernels.
constexpr size_t NOALLOC_SCRATCH_BYTES = 528 * 1024;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];
namespace {
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;   // device -> address of `scratch` there
}  // namespace

size_t noalloc_scratch_bytes() { return NOALLOC_SCRATCH_BYTES; }

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr[dev] = p;
  *ptr = p;
  return hipSuccess;
}

}  // namespace sbn
