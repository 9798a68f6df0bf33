// Dual-STE backward of Sparse-BitLinear on gfx950 bf16 matrix cores.
//
// "Sparse-BitNet" (gist.science Japanese "技術概要" §2.1, German "Technische
// Zusammenfassung" §2, Korean "기술 요약" §2.2, French "Résumé technique" §2):
// straight-through estimators for the ternary and activation quantizers, and
// the gradient passes the N:M mask densely so pruned master weights keep
// receiving updates.  With identity Jacobians:
//   dX[t,k] = s_w * sum_r dY[t,r] * Wt[r,k]         (sparse ternary weight)
//   dW[r,k] = sum_t (dY[t,r] * s_x[t]) * Xq[t,k]     (every (r,k))
//
// Numerics.  dY (bf16) times a ternary weight is exact in bf16 operands;
// Xq (|q| <= 127) is exact in bf16.  u = dY * s_x is not, so it is split
// u = hi + lo with hi = bf16(u), lo = bf16(u - hi) (relative error <= 2^-17)
// and dW takes two products.  Accumulation is float32 in the matrix cores.
//
// Passes:
//   expand_wt      packed planes -> bf16 Wt fragments, rows k, contraction r
//   prep_gradw     dY, s_x, Xq -> bf16 fragments (u_hi, u_lo rows r; Xq rows k),
//                  contraction t
//   bf16 GEMM x2   dX^T tile = Wt^T dY^T   and   dW^T tile = Xq^T (u_hi + u_lo)
// Fragment = 16 rows x 32 contraction, lane l holds row l%16 and contraction
// entries 8*(l/16) .. +8 (the lane order of v_mfma_f32_16x16x32_bf16).
#include "sbn_internal.h"

namespace sbn {
namespace {

constexpr uint16_t BF16_ONE = 0x3F80, BF16_MONE = 0xBF80;

__device__ inline uint32_t read_bits_b(const uint8_t* p, int64_t off, int nbits) {
  const uint8_t* q = p + (off >> 3);
  const int s = (int)(off & 7);
  uint32_t v = 0;
  const int nb = (s + nbits + 7) >> 3;
  for (int i = 0; i < nb; ++i) v |= (uint32_t)q[i] << (8 * i);
  return (v >> s) & ((1u << nbits) - 1u);
}

// ternary weight at (r, k) from the packed planes, as bf16 bits
__device__ inline uint16_t w_at(const uint8_t* codes, const uint8_t* meta, int64_t K, int n, int m,
                                int64_t r, int64_t k) {
  const int64_t g = k / m;
  const int p = (int)(k - g * m);
  int slot = p;
  if (n < m) {
    const uint32_t gm = read_bits_b(meta + r * (K / 8), g * m, m);
    if (!((gm >> p) & 1u)) return 0;
    slot = __builtin_popcount(gm & ((1u << p) - 1u));
  }
  const int64_t crow = K * n / (4 * m);
  const uint32_t c = read_bits_b(codes + r * crow, 2 * (n * g + slot), 2);
  return c == 1u ? BF16_ONE : c == 3u ? BF16_MONE : (uint16_t)0;
}

// one thread = one lane of fragment (kb, rb): rows k, contraction r
__global__ __launch_bounds__(256) void expand_wt_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ meta, int64_t R,
                                                        int64_t K, int n, int m, int64_t KB16,
                                                        int64_t RB32, uint4* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= KB16 * RB32 * 64) return;
  const int l = (int)(gid & 63);
  const int64_t f = gid >> 6;
  const int64_t kb = f / RB32, rb = f - kb * RB32;
  const int64_t k = kb * 16 + (l & 15);
  const int64_t r0 = rb * 32 + 8 * (l >> 4);
  uint16_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (k < K && r0 + j < R) ? w_at(codes, meta, K, n, m, r0 + j, k) : (uint16_t)0;
  uint4 o;
  o.x = v[0] | ((uint32_t)v[1] << 16);
  o.y = v[2] | ((uint32_t)v[3] << 16);
  o.z = v[4] | ((uint32_t)v[5] << 16);
  o.w = v[6] | ((uint32_t)v[7] << 16);
  out[gid] = o;
}

// fragments for dW: u = dY*s_x split hi/lo (rows r), Xq as bf16 (rows k); contraction t
__global__ __launch_bounds__(256) void prep_u_kernel(const uint16_t* __restrict__ dY,
                                                     const float* __restrict__ s_x, int64_t T,
                                                     int64_t R, int64_t RB16, int64_t TB32,
                                                     uint4* __restrict__ uhi, uint4* __restrict__ ulo) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= RB16 * TB32 * 64) return;
  const int l = (int)(gid & 63);
  const int64_t f = gid >> 6;
  const int64_t rb = f / TB32, tb = f - rb * TB32;
  const int64_t r = rb * 16 + (l & 15);
  const int64_t t0 = tb * 32 + 8 * (l >> 4);
  uint16_t h[8], lo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t t = t0 + j;
    float u = 0.0f;
    if (r < R && t < T) u = bf16_to_f32(dY[t * R + r]) * s_x[t];
    h[j] = f32_to_bf16_rne(u);
    lo[j] = f32_to_bf16_rne(u - bf16_to_f32(h[j]));
  }
  uint4 a, b;
  a.x = h[0] | ((uint32_t)h[1] << 16); a.y = h[2] | ((uint32_t)h[3] << 16);
  a.z = h[4] | ((uint32_t)h[5] << 16); a.w = h[6] | ((uint32_t)h[7] << 16);
  b.x = lo[0] | ((uint32_t)lo[1] << 16); b.y = lo[2] | ((uint32_t)lo[3] << 16);
  b.z = lo[4] | ((uint32_t)lo[5] << 16); b.w = lo[6] | ((uint32_t)lo[7] << 16);
  uhi[gid] = a;
  ulo[gid] = b;
}

__global__ __launch_bounds__(256) void prep_xq_kernel(const int8_t* __restrict__ Xq, int64_t T,
                                                      int64_t K, int64_t KB16, int64_t TB32,
                                                      uint4* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= KB16 * TB32 * 64) return;
  const int l = (int)(gid & 63);
  const int64_t f = gid >> 6;
  const int64_t kb = f / TB32, tb = f - kb * TB32;
  const int64_t k = kb * 16 + (l & 15);
  const int64_t t0 = tb * 32 + 8 * (l >> 4);
  uint16_t h[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t t = t0 + j;
    const float x = (k < K && t < T) ? (float)Xq[t * K + k] : 0.0f;
    h[j] = (uint16_t)(__float_as_uint(x) >> 16);     // |q| <= 127: exact in bf16
  }
  uint4 a;
  a.x = h[0] | ((uint32_t)h[1] << 16); a.y = h[2] | ((uint32_t)h[3] << 16);
  a.z = h[4] | ((uint32_t)h[5] << 16); a.w = h[6] | ((uint32_t)h[7] << 16);
  out[gid] = a;
}

// ---------------------------------------------------------------- bf16 GEMM on fragments
// MODE 0 (dX): A = Wt fragments (rows k, contraction r), B = dY rows read directly.
// MODE 1 (dW): A = Xq fragments (rows k, contraction t), B = u_hi and u_lo fragments (rows r).
// Block tile 256 (A rows) x 256 (B rows), 8 waves, wave tile 128 x 64 (8 x 4
// accumulator tiles of 16 x 16), one contraction step of 32 per LDS stage
// (MODE 1 takes two B fragments per step), stages filled by direct
// global->LDS loads issued NST - 1 steps ahead.  Ping-pong: waves w and w + 4
// share a SIMD and alternate a memory phase (LDS reads of one step, plus the
// loads of a later stage) with a compute phase (32 or 64 matrix instructions),
// so one of them keeps the matrix core busy while the other waits on LDS.
template <int MODE, int OUT>
__global__ __launch_bounds__(512, 1) void bf16_gemm_kernel(
    const uint8_t* __restrict__ Afr, const uint8_t* __restrict__ Bfr_hi,
    const uint8_t* __restrict__ Bfr_lo, const uint16_t* __restrict__ dY, int64_t nB /*B rows*/,
    int64_t nA /*A rows*/, int64_t nsteps, int64_t Rc /*dY cols (MODE 0)*/,
    const float* __restrict__ s_w, void* __restrict__ Out, int64_t ldo) {
  constexpr int NW = 8, MI = 8, MJ = 4;
  constexpr int NBF = MODE == 1 ? 2 : 1;
  constexpr int A_BYTES = 16 * 1024;
  constexpr int B_BYTES = 16 * 1024 * NBF;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int NST = MODE == 1 ? 3 : 4;              // 144 KB / 128 KB of LDS
  constexpr int LPS = 2 + 2 * NBF;                    // loads per stage per wave
  constexpr int WAIT = (NST - 2) * LPS;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int grp = wave >> 2;                           // waves w and w + 4 share a SIMD
  const int wa = wave & 1, wb = wave >> 1;             // A rows 128*wa.., B rows 64*wb..
  const int64_t tile_b = (int64_t)blockIdx.x * 256;
  const int64_t tile_a = (int64_t)blockIdx.y * 256;
  const int64_t ab0 = tile_a / 16, bb0 = tile_b / 16;

  auto load_stage = [&](int s, int64_t step) {
    uint8_t* base = smem + s * STAGE;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int i = wave + NW * q;
      g2lds16(Afr + ((ab0 + i) * nsteps + step) * 1024 + lane * 16, base + i * 1024);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = wave + NW * q;
      if (MODE == 0) {
        int64_t t = tile_b + 16 * j + (lane & 15);
        t = t < nB ? t : nB - 1;
        int64_t r = step * 32 + 8 * (lane >> 4);
        r = r < Rc ? r : Rc - 8;                   // Wt is zero past R
        g2lds16(dY + t * Rc + r, base + A_BYTES + j * 1024);
      } else {
        const int64_t fr = (bb0 + j) * nsteps + step;
        g2lds16(Bfr_hi + fr * 1024 + lane * 16, base + A_BYTES + j * 1024);
        g2lds16(Bfr_lo + fr * 1024 + lane * 16, base + A_BYTES + 16 * 1024 + j * 1024);
      }
    }
  };

  v4f acc[MI][MJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < MJ; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  v8bf a[MI], b[MJ], b2[MJ];

  // memory phase of step s: issue the loads of stage s + NST - 1, read step s's fragments
  auto mem_phase = [&](int64_t s) {
    if (s + NST - 1 < nsteps) load_stage((int)((s + NST - 1) % NST), s + NST - 1);
    const uint8_t* base = smem + (s % NST) * STAGE;
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      const int jj = MJ * wb + j;
      b[j] = __builtin_bit_cast(v8bf, *(const v4i*)(base + A_BYTES + jj * 1024 + lane * 16));
      if (MODE == 1)
        b2[j] = __builtin_bit_cast(v8bf, *(const v4i*)(base + A_BYTES + 16 * 1024 + jj * 1024 + lane * 16));
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
      a[i] = __builtin_bit_cast(v8bf, *(const v4i*)(base + (MI * wa + i) * 1024 + lane * 16));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  auto comp_phase = [&]() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        if (MODE == 1) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b2[j], acc[i][j], 0, 0, 0);
      }
  };
  // this wave's loads of stage s + 1 have landed (later stages may still fly)
  auto vm_wait = [&](int64_t s) {
    __builtin_amdgcn_sched_barrier(0);
    if (s + NST - 1 < nsteps) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(WAIT) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // Barrier schedule (B0, B1, ... in order; both groups pass the same count):
  //   group 0: B0 | mem(s) B(2s+1) comp(s) wait B(2s+2) | ...
  //   group 1: B0 B1 | mem(s) wait B(2s+2) comp(s) B(2s+3) | ... (no barrier after its last comp)
  // so phase (B(2s+1), B(2s+2)) is comp(s) of group 0 beside mem(s) of group 1,
  // and phase (B(2s+2), B(2s+3)) is comp(s) of group 1 beside mem(s+1) of group 0.
  // Stage s is complete before B(2s) and read only between B(2s) and B(2s+2);
  // its buffer is refilled (stage s + NST) from mem(s+1), after B(2s+2).
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nsteps) load_stage(s, s);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  barrier();                                           // B0: stages 0 .. NST-2 visible
  if (grp == 0) {
    for (int64_t s = 0; s < nsteps; ++s) {
      mem_phase(s);
      barrier();
      comp_phase();
      vm_wait(s);
      barrier();
    }
  } else {
    barrier();
    for (int64_t s = 0; s < nsteps; ++s) {
      mem_phase(s);
      vm_wait(s);
      barrier();
      comp_phase();
      if (s + 1 < nsteps) barrier();
    }
  }

  // lane holds A rows (k) a..a+3 of B row (t or r) b
  const float scale = MODE == 0 ? *s_w : 1.0f;
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int64_t brow = tile_b + 16 * (MJ * wb + j) + (lane & 15);
    if (brow >= nB) continue;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int64_t arow = tile_a + 16 * (MI * wa + i) + 4 * (lane >> 4);
      if (arow >= nA) continue;
      const v4f c = acc[i][j] * scale;
      if (OUT == 1) {
        float* y = (float*)Out + brow * ldo + arow;
        if (arow + 3 < nA) *(v4f*)y = c;
        else for (int v = 0; v < 4 && arow + v < nA; ++v) y[v] = c[v];
      } else {
        uint16_t* y = (uint16_t*)Out + brow * ldo + arow;
        const uint16_t o[4] = {f32_to_bf16_rne(c[0]), f32_to_bf16_rne(c[1]), f32_to_bf16_rne(c[2]),
                               f32_to_bf16_rne(c[3])};
        if (arow + 3 < nA) store_u16x4(y, o[0], o[1], o[2], o[3]);
        else for (int v = 0; v < 4 && arow + v < nA; ++v) y[v] = o[v];
      }
    }
  }
}

struct BwdLayout {
  int64_t KB16, RB32, TB32, RB16;
  size_t wt, xq, uhi, ulo, total;
};

BwdLayout bwd_layout(int64_t T, int64_t R, int64_t K) {
  BwdLayout L;
  const int64_t Kp = round_up(K, 256), Rp32 = round_up(R, 32), Tp32 = round_up(T, 32),
                Rp256 = round_up(R, 256);
  L.KB16 = Kp / 16;
  L.RB32 = Rp32 / 32;
  L.TB32 = Tp32 / 32;
  L.RB16 = Rp256 / 16;
  const size_t wt_b = align256((size_t)(Kp * Rp32 * 2));
  const size_t xq_b = align256((size_t)(Kp * Tp32 * 2));
  const size_t u_b = align256((size_t)(Rp256 * Tp32 * 2));
  L.wt = 0;
  L.xq = wt_b;
  L.uhi = wt_b + xq_b;
  L.ulo = L.uhi + u_b;
  L.total = L.ulo + u_b;
  return L;
}

}  // namespace

size_t bwd_ws_bytes(int64_t T, int64_t R, int64_t K, int /*n*/, int /*m*/) {
  return bwd_layout(T, R, K).total;
}

hipError_t launch_backward(const uint16_t* dY, int64_t T, int64_t R, const int8_t* Xq,
                           const float* s_x, int64_t K, const uint8_t* codes, const uint8_t* meta,
                           const float* s_w, int n, int m, void* dX, sbn_dtype dxdt, float* dW,
                           void* ws, hipStream_t st) {
  const BwdLayout L = bwd_layout(T, R, K);
  uint8_t* w = (uint8_t*)ws;
  hipError_t e;
  if (dX) {
    const int64_t thr = L.KB16 * L.RB32 * 64;
    SBN_LAUNCH("expand_wt", expand_wt_kernel, dim3((unsigned)cdiv(thr, 256)), dim3(256), 0, st, codes,
                       (n == m) ? nullptr : meta, R, K, n, m, L.KB16, L.RB32, (uint4*)(w + L.wt));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 grid((unsigned)cdiv(T, 256), (unsigned)cdiv(K, 256));
    if (dxdt == SBN_F32)
      SBN_LAUNCH("gemm_dx", (bf16_gemm_kernel<0, 1>), grid, dim3(512), 0, st, w + L.wt, nullptr, nullptr,
                         dY, T, K, L.RB32, R, s_w, dX, K);
    else
      SBN_LAUNCH("gemm_dx", (bf16_gemm_kernel<0, 2>), grid, dim3(512), 0, st, w + L.wt, nullptr, nullptr,
                         dY, T, K, L.RB32, R, s_w, dX, K);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (dW) {
    const int64_t tu = L.RB16 * L.TB32 * 64;
    SBN_LAUNCH("prep_u", prep_u_kernel, dim3((unsigned)cdiv(tu, 256)), dim3(256), 0, st, dY, s_x, T, R,
                       L.RB16, L.TB32, (uint4*)(w + L.uhi), (uint4*)(w + L.ulo));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t tx = L.KB16 * L.TB32 * 64;
    SBN_LAUNCH("prep_xq", prep_xq_kernel, dim3((unsigned)cdiv(tx, 256)), dim3(256), 0, st, Xq, T, K,
                       L.KB16, L.TB32, (uint4*)(w + L.xq));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 grid((unsigned)cdiv(R, 256), (unsigned)cdiv(K, 256));
    SBN_LAUNCH("gemm_dw", (bf16_gemm_kernel<1, 1>), grid, dim3(512), 0, st, w + L.xq, w + L.uhi,
                       w + L.ulo, nullptr, R, K, L.TB32, (int64_t)0, s_w, (void*)dW, K);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sbn
