// Dual-STE backward of Sparse-BitLinear on gfx950 bf16 matrix cores.
//
// "Sparse-BitNet" (gist.science Japanese "技術概要" §2.1, German "Technische
// Zusammenfassung" §2, Korean "기술 요약" §2.2, French "Résumé technique" §2):
// straight-through estimators for the ternary and activation quantizers, and
// the gradient passes the N:M mask densely so pruned master weights keep
// receiving updates.  With identity Jacobians:
//   dX[t,k] = s_w * sum_r dY[t,r] * Wt[r,k]         (sparse ternary weight)
//   dW[r,k] = sum_t (dY[t,r] * s_x[t]) * Xq[t,k]     (every (r,k))
// The ablation of German §4 ("Ablationsstudien") / French §5 that blocks the
// gradient of pruned weights is a flag: dW is then 0 wherever the meta bit of
// (r, k) is clear (applied in the dW epilogue).
//
// Numerics.  dY (bf16) times a ternary weight is exact in bf16 operands;
// Xq (|q| <= 127) is exact in bf16.  u = dY * s_x is not, so it is split
// u = hi + lo with hi = bf16(u), lo = bf16(u - hi) (relative error <= 2^-17)
// and dW takes two products.  Accumulation is float32 in the matrix cores.
//
// Passes:
//   expand_wt      packed planes -> bf16 Wt fragments, rows k, contraction r
//   prep_u         dY, s_x -> bf16 u_hi, u_lo fragments, rows r, contraction t
//   prep_xq        Xq -> bf16 fragments, rows k, contraction t
//   bf16 GEMM x2   dX^T tile = Wt^T dY^T   and   dW^T tile = Xq^T (u_hi + u_lo)
// Fragment = 16 rows x 32 contraction, lane l holds row l%16 and contraction
// entries 8*(l/16) .. +8 (the lane order of v_mfma_f32_16x16x32_bf16).
#include "sbn_decode.h"

namespace sbn {
namespace {

constexpr uint16_t BF16_ONE = 0x3F80, BF16_MONE = 0xBF80;

// ---------------------------------------------------------------- fragment transposes
// The three operand passes below are transposes: their sources are row-major
// with the contraction index (r or t) as the row, and a fragment wants 8
// consecutive contraction entries of one output row (k or r) per lane.  A block
// takes a tile of 32 contraction entries x 128 rows: it reads the tile's source
// rows with coalesced 16-byte loads, writes them transposed into LDS as bf16
// ([row][contraction], pitch TP entries), and stores the tile's eight 1 KB
// fragments with one 16-byte store per lane.  Entries past the real sizes are 0.
constexpr int TP = 40;                               // LDS pitch in bf16 (80 B: 16-byte aligned rows)

// the eight fragments (rows row0 .. row0 + 127, contraction block cb) of an LDS
// tile [128][TP] into out[(rowblock * CB + cb) * 64 + lane]
__device__ inline void store_tile(const uint16_t* tile, uint4* __restrict__ out, int64_t rb0, int64_t cb,
                                  int64_t CB) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = threadIdx.x + 256 * h;               // fragment q / 64, lane q % 64
    const int f = q >> 6, l = q & 63;
    const int row = 16 * f + (l & 15), c0 = 8 * (l >> 4);
    out[((rb0 + f) * CB + cb) * 64 + l] = *(const uint4*)(tile + row * TP + c0);
  }
}

// one bf16 into tile[row][c]
__device__ inline void tile_put(uint16_t* tile, int row, int c, uint16_t v) { tile[row * TP + c] = v; }

// Wt fragments (rows k, contraction r) from the packed planes.  Thread (r, seg)
// decodes positions 16 seg .. +16 of the tile's 128 k for row r through the
// unpack table; blocks walk the tiles with a grid stride.
template <int M, int n>                                  // n: survivors per group (straight-line decode)
__global__ __launch_bounds__(256) void expand_wt_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ meta, int64_t R, int64_t K,
                                                        int64_t KB16, int64_t RB32, int64_t cplane,
                                                        uint4* __restrict__ out) {
  __shared__ uint32_t lut[4096];
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * TP];
  for (int i = threadIdx.x; i < 4096; i += 256) lut[i] = unpack_entry((uint32_t)i);
  const bool dense = meta == nullptr;
  const int64_t crow = K * n / (4 * M);                // code bytes per row
  const int64_t lastw = (cplane - 4) & ~(int64_t)3;
  const int64_t ntk = KB16 / 8, ntiles = ntk * RB32;
  // lanes of a wave take 32 consecutive rows r of two segments, so each LDS
  // write instruction fills contiguous bf16 entries of two tile rows
  const int rl = threadIdx.x & 31, seg = threadIdx.x >> 5;
  for (int64_t tt = blockIdx.x; tt < ntiles; tt += gridDim.x) {
    const int64_t kt = tt / RB32, rb = tt - kt * RB32;
    const int64_t r = rb * 32 + rl, k0 = kt * 128 + 16 * seg;
    v4i a = (v4i){0, 0, 0, 0};
    __syncthreads();                                   // lut built / previous tile stored
    if (r < R && k0 < K) {
      const uint32_t mw16 = dense ? 0xFFFFu : (uint32_t)*(const uint16_t*)(meta + r * (K / 8) + k0 / 8);
      const int64_t cbit = r * crow * 8 + k0 * 2 * n / M;   // the 16 positions start on a group boundary
      const int64_t a0 = (cbit >> 3) & ~(int64_t)3;
      const int sh = (int)(cbit - a0 * 8);
      const uint32_t w0 = *(const uint32_t*)(codes + (a0 < lastw ? a0 : lastw));
      const uint32_t w1 = *(const uint32_t*)(codes + (a0 + 4 < lastw ? a0 + 4 : lastw));
      const unsigned long long c = (((unsigned long long)w1 << 32) | w0) >> sh;
      a = unpack16<M>(lut, mw16, dense, n, c, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int8_t v = (int8_t)((uint32_t)a[i >> 2] >> (8 * (i & 3)));
      tile_put(tile, 16 * seg + i, rl, v == 1 ? BF16_ONE : v == -1 ? BF16_MONE : (uint16_t)0);
    }
    __syncthreads();
    store_tile(tile, out, kt * 8, rb, RB32);
  }
}

// u = dY * s_x split into bf16 hi and lo fragments (rows r, contraction t)
__global__ __launch_bounds__(256) void prep_u_kernel(const uint16_t* __restrict__ dY,
                                                     const float* __restrict__ s_x, int64_t T,
                                                     int64_t R, int64_t RB16, int64_t TB32,
                                                     uint4* __restrict__ uhi, uint4* __restrict__ ulo) {
  __shared__ __attribute__((aligned(16))) uint16_t th[128 * TP], tl[128 * TP];
  const int64_t rt = blockIdx.x / TB32, tb = blockIdx.x - rt * TB32;
#pragma unroll
  for (int h = 0; h < 2; ++h) {                        // 32 t x 16 chunks of 8 r; lanes run over t
    const int q = threadIdx.x + 256 * h;
    const int tl_ = q & 31, ch = q >> 5;
    const int64_t t = tb * 32 + tl_, r0 = rt * 128 + 8 * ch;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    float sx = 0.0f;
    if (t < T && r0 < R) {
      sx = s_x[t];
      if (r0 + 8 <= R && R % 8 == 0) v = *(const uint4*)(dY + t * R + r0);
      else {
        uint16_t e[8];
        for (int i = 0; i < 8; ++i) e[i] = r0 + i < R ? dY[t * R + r0 + i] : (uint16_t)0;
        v = make_uint4(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16), e[4] | ((uint32_t)e[5] << 16),
                       e[6] | ((uint32_t)e[7] << 16));
      }
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float u = bf16_to_f32((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) * sx;
      const uint16_t hi = f32_to_bf16_rne(u);
      tile_put(th, 8 * ch + i, tl_, hi);
      tile_put(tl, 8 * ch + i, tl_, f32_to_bf16_rne(u - bf16_to_f32(hi)));
    }
  }
  __syncthreads();
  store_tile(th, uhi, rt * 8, tb, TB32);
  store_tile(tl, ulo, rt * 8, tb, TB32);
}

// Xq as bf16 fragments (rows k, contraction t); |q| <= 127 is exact in bf16
__global__ __launch_bounds__(256) void prep_xq_kernel(const int8_t* __restrict__ Xq, int64_t T,
                                                      int64_t K, int64_t KB16, int64_t TB32,
                                                      uint4* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * TP];
  const int64_t kt = blockIdx.x / TB32, tb = blockIdx.x - kt * TB32;
  const int tl_ = threadIdx.x & 31, ch = threadIdx.x >> 5;  // 32 t x 8 chunks of 16 k; lanes run over t
  const int64_t t = tb * 32 + tl_, k0 = kt * 128 + 16 * ch;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (t < T && k0 < K) v = *(const uint4*)(Xq + t * K + k0);   // K % 64 == 0
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float x = (float)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
    tile_put(tile, 16 * ch + i, tl_, (uint16_t)(__float_as_uint(x) >> 16));
  }
  __syncthreads();
  store_tile(tile, out, kt * 8, tb, TB32);
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
    const float* __restrict__ s_w, void* __restrict__ Out, int64_t ldo, const uint8_t* __restrict__ gmask) {
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
      v4f c = acc[i][j] * scale;
      if (MODE == 1 && gmask) {                        // blocked-gradient variant: dW at pruned (r, k) is 0
        const uint32_t nib = (uint32_t)(gmask[brow * (nA / 8) + (arow >> 3)] >> (arow & 7)) & 15u;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (!((nib >> v) & 1u)) c[v] = 0.0f;
      }
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
                           void* ws, uint32_t flags, hipStream_t st) {
  const BwdLayout L = bwd_layout(T, R, K);
  uint8_t* w = (uint8_t*)ws;
  hipError_t e;
  if (dX) {
    int64_t tiles = (L.KB16 / 8) * L.RB32;
    if (tiles > 2048) tiles = 2048;                     // grid stride: the unpack table is built per block
    const int64_t cplane = round_up(R * K * n / (4 * m), 16);
    const uint8_t* mp = (n == m) ? nullptr : meta;
    const dim3 eg((unsigned)tiles), eb(256);
#define SBN_EW_CASE(MM, NN)                                                                                        \
    else if (m == MM && n == NN) SBN_LAUNCH("expand_wt", (expand_wt_kernel<MM, NN>), eg, eb, 0, st, codes, mp, R, K, \
                                            L.KB16, L.RB32, cplane, (uint4*)(w + L.wt));
    if (false) {
    }
    SBN_EW_CASE(4, 1) SBN_EW_CASE(4, 2) SBN_EW_CASE(4, 3) SBN_EW_CASE(4, 4)
    SBN_EW_CASE(8, 1) SBN_EW_CASE(8, 2) SBN_EW_CASE(8, 3) SBN_EW_CASE(8, 4)
    SBN_EW_CASE(8, 5) SBN_EW_CASE(8, 6) SBN_EW_CASE(8, 7) SBN_EW_CASE(8, 8)
#undef SBN_EW_CASE
    else return hipErrorInvalidValue;
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 grid((unsigned)cdiv(T, 256), (unsigned)cdiv(K, 256));
    if (dxdt == SBN_F32)
      SBN_LAUNCH("gemm_dx", (bf16_gemm_kernel<0, 1>), grid, dim3(512), 0, st, w + L.wt, nullptr, nullptr,
                         dY, T, K, L.RB32, R, s_w, dX, K, nullptr);
    else
      SBN_LAUNCH("gemm_dx", (bf16_gemm_kernel<0, 2>), grid, dim3(512), 0, st, w + L.wt, nullptr, nullptr,
                         dY, T, K, L.RB32, R, s_w, dX, K, nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (dW) {
    SBN_LAUNCH("prep_u", prep_u_kernel, dim3((unsigned)((L.RB16 / 8) * L.TB32)), dim3(256), 0, st, dY, s_x, T, R,
               L.RB16, L.TB32, (uint4*)(w + L.uhi), (uint4*)(w + L.ulo));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    SBN_LAUNCH("prep_xq", prep_xq_kernel, dim3((unsigned)((L.KB16 / 8) * L.TB32)), dim3(256), 0, st, Xq, T, K,
               L.KB16, L.TB32, (uint4*)(w + L.xq));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 grid((unsigned)cdiv(R, 256), (unsigned)cdiv(K, 256));
    const uint8_t* gmask = (flags & SBN_GRAD_W_MASKED) && n < m ? meta : nullptr;
    SBN_LAUNCH("gemm_dw", (bf16_gemm_kernel<1, 1>), grid, dim3(512), 0, st, w + L.xq, w + L.uhi,
                       w + L.ulo, nullptr, R, K, L.TB32, (int64_t)0, s_w, (void*)dW, K, gmask);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sbn
