// Sparse ternary GEMM  Y[t,r] = s_w * s_x[t] * sum_k Xq[t,k] * Wt[r,k]  on gfx950 matrix cores.
//
// The pages run this product on a custom 6:8 sparse kernel ("Sparse-BitNet",
// gist.science Japanese "技術概要" §3.2, German "Technische Zusammenfassung"
// §4); on gfx950 the structured-sparse int8 instruction handles at most two
// non-zeros per four K positions, so:
//   * ratios with n <= 2 (2:4, 1:4, 2:8) run on v_smfmac_i32_16x16x128_i8,
//     W as the sparse A operand (16 output rows x 128 K, two values per four
//     positions plus 2-bit position indices), Xq as the dense B operand;
//   * every other ratio (6:8, 4:8, 3:4, the dense 8:8 control, ...) runs on
//     dense v_mfma_i32_16x16x64_i8 with W expanded to int8 {-1, 0, +1}.
//
// Two kernels per call: an expansion pass turns the packed planes into the
// matrix-core operand order (one contiguous 1 KB fragment per 16 rows x K
// block, so each lane later fetches 16 contiguous bytes), then the GEMM.
//
// GEMM tiling: 256 threads (4 waves in 2 x 2), block tile 256 rows x 256
// tokens, wave tile 128 x 128 (8 x 8 accumulator tiles of 16 x 16 int32),
// K step 128, two LDS stages filled with direct global->LDS loads, issued one
// stage ahead.  The LDS image of every fragment is the lane order the matrix
// instruction reads, so fragment reads are contiguous 16-byte LDS reads.
//
// Operand layouts (gfx950, measured with a lane-layout check):
//   16x16x64 i8 : A lane l -> row l%16, K[16*(l/16) .. +16); B lane l -> col l%16,
//                 same K bytes; C lane l -> rows 4*(l/16)+v (v = 0..3), col l%16.
//   16x16x128 i8 sparse: A lane l -> row l%16, compressed slot j (0..15) is K
//                 32*(l/16) + 4*(j/2) + idx_j (idx_j = bits 2j..2j+1 of the index
//                 register); B lane l -> col l%16, bytes 0..15 = K[16*(l/16)..),
//                 bytes 16..31 = K[64 + 16*(l/16)..); C as above.
#include "sbn_internal.h"

namespace sbn {
namespace {

constexpr int GT = 256;

// read nbits (<= 32) of a little-endian bitstream starting at bit `off`
__device__ inline uint32_t read_bits(const uint8_t* p, int64_t off, int nbits) {
  const uint8_t* q = p + (off >> 3);
  const int s = (int)(off & 7);
  unsigned long long v = 0;
  const int nb = (s + nbits + 7) >> 3;
  for (int i = 0; i < nb; ++i) v |= (unsigned long long)q[i] << (8 * i);
  v >>= s;
  return nbits == 32 ? (uint32_t)v : (uint32_t)(v & ((1ull << nbits) - 1));
}

__device__ inline int8_t code_to_i8(uint32_t c) { return c == 1u ? (int8_t)1 : c == 3u ? (int8_t)-1 : (int8_t)0; }

// ---------------------------------------------------------------- expansion: sparse operand
// one thread = one lane of one (16-row, 128-K) fragment: 16 values + 32 index bits
__global__ __launch_bounds__(256) void expand_sparse_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta, int64_t R, int64_t K,
    int n, int m, int64_t RB, int64_t KBn, uint8_t* __restrict__ vals, uint32_t* __restrict__ idx) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= RB * KBn * 64) return;
  const int l = (int)(gid & 63);
  const int64_t f = gid >> 6;                   // fragment = rb * KBn + kb
  const int64_t rb = f / KBn, kb = f - rb * KBn;
  const int64_t r = rb * 16 + (l & 15);
  const int64_t k0 = kb * 128 + 32 * (l >> 4);
  uint32_t v32[4] = {0, 0, 0, 0};
  uint32_t ix = 0x44444444u;                    // (0,1) in every half: harmless with zero values
  if (r < R && k0 < K && n == 2 && m == 4) {
    // 2:4: meta and codes of these 32 positions are one aligned word each
    const uint32_t mb = *(const uint32_t*)(meta + r * (K / 8) + k0 / 8);
    const uint32_t cb = *(const uint32_t*)(codes + r * (K / 8) + k0 / 8);
    // survivor positions per nibble: p0 = lowest set bit, p1 = highest (SWAR over 8 nibbles)
    const uint32_t M1 = 0x11111111u;
    const uint32_t b0 = mb & M1, b1 = (mb >> 1) & M1, b2 = (mb >> 2) & M1, b3 = (mb >> 3) & M1;
    const uint32_t nb0 = b0 ^ M1, nb1 = b1 ^ M1, nb2 = b2 ^ M1;
    ix = (nb0 & b1) | ((nb0 & nb1) << 1) | ((b3 | nb2) << 2) | ((b3 | b2) << 3);
    // values: compressed slot j holds code bits 2j..2j+1; spread each byte's four
    // codes to four bytes and map 01 -> +1, 11 -> -1
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t y = (cb >> (8 * d)) & 0xFFu;
      const uint32_t sp = (((y & 0x33u) * 0x1001u) & 0x00030003u) | (((y & 0xCCu) * 0x40040u) & 0x03000300u);
      v32[d] = sp | ((sp & 0x02020202u) * 0x7Eu);
    }
  } else if (r < R && k0 < K) {
    const uint32_t mb = *(const uint32_t*)(meta + r * (K / 8) + k0 / 8);
    const int64_t crow = K * n / (4 * m);
    const int64_t gbase = k0 / m;               // groups before k0 in this row
    const int ngroups = 32 / m;
    const uint32_t cb = read_bits(codes + r * crow, 2 * n * gbase, 2 * n * ngroups);
    ix = 0;
    int cur = 0;                                // codes consumed so far in this range
#pragma unroll
    for (int h = 0; h < 8; ++h) {               // eight halves of four positions
      int cnt = 0;
      uint32_t pos[2] = {0, 1};
      int8_t val[2] = {0, 0};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int pp = 4 * h + p;
        if ((mb >> pp) & 1u) {
          const uint32_t c = (cb >> (2 * cur)) & 3u;
          ++cur;
          if (cnt < 2) {
            pos[cnt] = (uint32_t)p;
            val[cnt] = code_to_i8(c);
          }
          ++cnt;
        }
      }
      if (cnt == 1) {                           // keep the two indices distinct and ordered
        if (pos[0] == 3) { pos[1] = 3; val[1] = val[0]; pos[0] = 0; val[0] = 0; }
        else { pos[1] = 3; val[1] = 0; }
      }
      ix |= (pos[0] | (pos[1] << 2)) << (4 * h);
      const int j0 = 2 * h;
      v32[j0 >> 2] |= (uint32_t)(uint8_t)val[0] << (8 * (j0 & 3));
      v32[(j0 + 1) >> 2] |= (uint32_t)(uint8_t)val[1] << (8 * ((j0 + 1) & 3));
    }
  }
  uint4 o;
  o.x = v32[0]; o.y = v32[1]; o.z = v32[2]; o.w = v32[3];
  ((uint4*)vals)[gid] = o;
  idx[gid] = ix;
}

// ---------------------------------------------------------------- expansion: dense operand
// one thread = one lane of one (16-row, 64-K) fragment: 16 int8 values
__global__ __launch_bounds__(256) void expand_dense_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta, int64_t R, int64_t K,
    int n, int m, int64_t RB, int64_t KD, uint8_t* __restrict__ vals) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= RB * KD * 64) return;
  const int l = (int)(gid & 63);
  const int64_t f = gid >> 6;
  const int64_t rb = f / KD, kd = f - rb * KD;
  const int64_t r = rb * 16 + (l & 15);
  const int64_t k0 = kd * 64 + 16 * (l >> 4);
  uint32_t v32[4] = {0, 0, 0, 0};
  if (r < R && k0 < K) {
    const uint32_t mb = (n == m) ? 0xFFFFu : (uint32_t)*(const uint16_t*)(meta + r * (K / 8) + k0 / 8);
    const int64_t crow = K * n / (4 * m);
    const uint32_t cb = read_bits(codes + r * crow, 2 * n * (k0 / m), 2 * n * (16 / m));
    int cur = 0;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      if ((mb >> p) & 1u) {
        const uint32_t c = (cb >> (2 * cur)) & 3u;
        ++cur;
        v32[p >> 2] |= (uint32_t)(uint8_t)code_to_i8(c) << (8 * (p & 3));
      }
    }
  }
  uint4 o;
  o.x = v32[0]; o.y = v32[1]; o.z = v32[2]; o.w = v32[3];
  ((uint4*)vals)[gid] = o;
}

// ---------------------------------------------------------------- GEMM
// Tile order: blocks are dealt to the 8 XCDs round-robin; give each XCD a
// contiguous run of tiles, and walk tiles in groups of 8 row tiles (token
// tile major inside a group), so the blocks resident on one XCD share row
// and token operands in that XCD's L2.
__device__ inline void tile_of_block(int64_t b, int64_t ntR, int64_t ntT, int64_t& rt, int64_t& tt) {
  const int64_t ntiles = ntR * ntT;
  const int64_t xcd = b & 7, local = b >> 3;
  const int64_t base = ntiles / 8, rem = ntiles % 8;
  const int64_t t = xcd * base + (xcd < rem ? xcd : rem) + local;   // blocks of XCD x come first
  const int64_t g = t / (8 * ntT);                                  // group of 8 row tiles
  const int64_t gr = (ntR - 8 * g) < 8 ? (ntR - 8 * g) : 8;
  const int64_t j = t - g * 8 * ntT;
  rt = 8 * g + j % gr;
  tt = j / gr;
}

// OUT: 0 = int32 accumulator, 1 = float32, 2 = bf16.  WR x WT waves, wave tile
// (256/WR) rows x (256/WT) tokens.  SPARSE: K step 128 (smfmac), 3 stages;
// dense: K step 64 (mfma 16x16x64), 4 stages.
template <bool SPARSE, int OUT, int WR, int WT>
__global__ __launch_bounds__(64 * WR * WT, 1) void gemm_kernel(
    const uint8_t* __restrict__ Aw, const uint32_t* __restrict__ Ai, const int8_t* __restrict__ Xq,
    const float* __restrict__ s_x, const float* __restrict__ s_w, int64_t T, int64_t K, int64_t R,
    int64_t nks, int64_t fstride, void* __restrict__ Y, int64_t ldy) {
  constexpr int NW = WR * WT;
  constexpr int MI = 256 / WR / 16, MJ = 256 / WT / 16;          // fragments per wave
  constexpr int A_BYTES = 16 * 1024;
  constexpr int I_BYTES = SPARSE ? 16 * 256 : 0;
  constexpr int BH = SPARSE ? 2 : 1;                              // B 1 KB halves per token block
  constexpr int B_BYTES = 16 * BH * 1024;
  constexpr int STAGE = A_BYTES + I_BYTES + B_BYTES;
  constexpr int NST = SPARSE ? 3 : 4;
  constexpr int KS = SPARSE ? 128 : 64;
  constexpr int LPS = (16 / NW) * (SPARSE ? 2 : 1) + (16 * BH) / NW;   // loads per stage per wave
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wr = wave / WT, wt = wave % WT;
  int64_t rtile, ttile;
  tile_of_block(blockIdx.x, cdiv(R, 256), cdiv(T, 256), rtile, ttile);
  const int64_t tile_r = rtile * 256, tile_t = ttile * 256;
  const int64_t rb0 = tile_r / 16;

  auto load_stage = [&](int s, int64_t ks) {
    uint8_t* base = smem + s * STAGE;
#pragma unroll
    for (int q = 0; q < 16 / NW; ++q) {
      const int i = wave + NW * q;
      const int64_t frag = (rb0 + i) * fstride + ks;
      g2lds16(Aw + frag * 1024 + lane * 16, base + i * 1024);
      if (SPARSE) g2lds4(Ai + frag * 64 + lane, base + A_BYTES + i * 256);
    }
#pragma unroll
    for (int q = 0; q < (16 * BH) / NW; ++q) {
      const int hb = wave + NW * q;                                  // half-block index
      const int j = hb / BH, h = hb % BH;
      int64_t t = tile_t + 16 * j + (lane & 15);
      t = t < T ? t : T - 1;                      // rows past T are computed and discarded
      int64_t k = ks * KS + 64 * h + 16 * (lane >> 4);
      k = k < K ? k : K - 16;                     // W is zero past K, any finite bytes do
      g2lds16(Xq + t * K + k, base + A_BYTES + I_BYTES + hb * 1024);
    }
  };

  v4i acc[MI][MJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < MJ; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nks) load_stage(s, s);

  for (int64_t ks = 0; ks < nks; ++ks) {
    if (ks + NST - 2 < nks) wait_vmcnt<(NST - 2) * LPS>();       // stage ks landed, later ones may fly
    else wait_vmcnt<0>();
    lds_barrier();
    if (ks + NST - 1 < nks) load_stage((int)((ks + NST - 1) % NST), ks + NST - 1);
    const uint8_t* base = smem + (ks % NST) * STAGE;
    const uint8_t* bb = base + A_BYTES + I_BYTES;
    v4i blo[MJ], bhi[MJ];
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      const int jj = MJ * wt + j;
      blo[j] = *(const v4i*)(bb + (jj * BH + 0) * 1024 + lane * 16);
      if (SPARSE) bhi[j] = *(const v4i*)(bb + (jj * BH + 1) * 1024 + lane * 16);
    }
    v4i a = *(const v4i*)(base + (MI * wr) * 1024 + lane * 16);
    int ix = SPARSE ? *(const int*)(base + A_BYTES + (MI * wr) * 256 + lane * 4) : 0;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      v4i an = a;
      int ixn = ix;
      if (i + 1 < MI) {                           // next A fragment in flight during these products
        const int ii = MI * wr + i + 1;
        an = *(const v4i*)(base + ii * 1024 + lane * 16);
        if (SPARSE) ixn = *(const int*)(base + A_BYTES + ii * 256 + lane * 4);
      }
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        if (SPARSE) {
          const v8i b = (v8i){blo[j][0], blo[j][1], blo[j][2], blo[j][3],
                              bhi[j][0], bhi[j][1], bhi[j][2], bhi[j][3]};
          acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, acc[i][j], ix, 0, 0);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, blo[j], acc[i][j], 0, 0, 0);
        }
      }
      a = an;
      ix = ixn;
    }
  }

  // epilogue: lane holds rows r..r+3 of token t
  const float sw = (OUT != 0) ? *s_w : 0.0f;
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int64_t t = tile_t + 16 * (MJ * wt + j) + (lane & 15);
    if (t >= T) continue;
    const float sc = (OUT != 0) ? sw * s_x[t] : 0.0f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int64_t r = tile_r + 16 * (MI * wr + i) + 4 * (lane >> 4);
      if (r >= R) continue;
      const v4i c = acc[i][j];
      if (OUT == 0) {
        int* y = (int*)Y + t * ldy + r;
        if (r + 3 < R) *(v4i*)y = c;
        else for (int v = 0; v < 4 && r + v < R; ++v) y[v] = c[v];
      } else if (OUT == 1) {
        float* y = (float*)Y + t * ldy + r;
        const v4f o = (v4f){(float)c[0] * sc, (float)c[1] * sc, (float)c[2] * sc, (float)c[3] * sc};
        if (r + 3 < R) *(v4f*)y = o;
        else for (int v = 0; v < 4 && r + v < R; ++v) y[v] = o[v];
      } else {
        uint16_t* y = (uint16_t*)Y + t * ldy + r;
        const uint16_t o0 = f32_to_bf16_rne((float)c[0] * sc), o1 = f32_to_bf16_rne((float)c[1] * sc);
        const uint16_t o2 = f32_to_bf16_rne((float)c[2] * sc), o3 = f32_to_bf16_rne((float)c[3] * sc);
        if (r + 3 < R) store_u16x4(y, o0, o1, o2, o3);
        else {
          const uint16_t o[4] = {o0, o1, o2, o3};
          for (int v = 0; v < 4 && r + v < R; ++v) y[v] = o[v];
        }
      }
    }
  }
}

// wave layouts: 8 waves of 128 x 64 (default; two waves per SIMD hide LDS latency) or 4 of 128 x 128
#ifndef SBN_GEMM_WT
#define SBN_GEMM_WT 4
#endif

template <bool SPARSE>
hipError_t launch_gemm_t(const uint8_t* Aw, const uint32_t* Ai, const int8_t* Xq, const float* s_x,
                         const float* s_w, int64_t T, int64_t K, int64_t R, int64_t KBn, void* Y,
                         sbn_dtype ydt, int64_t ldy, hipStream_t st) {
  constexpr int WR = 2, WT = SBN_GEMM_WT;
  const int64_t ntiles = cdiv(T, GEMM_TILE_T) * cdiv(R, GEMM_TILE_R);
  const dim3 grid((unsigned)ntiles), block(64 * WR * WT);
  const int64_t nks = SPARSE ? KBn : K / 64;
  const int64_t fstride = SPARSE ? KBn : 2 * KBn;
  const char* name = SPARSE ? "gemm_smfmac" : "gemm_mfma";
  if (ydt == SBN_I32_ACC)
    SBN_LAUNCH(name, (gemm_kernel<SPARSE, 0, WR, WT>), grid, block, 0, st, Aw, Ai, Xq, s_x, s_w, T, K, R, nks, fstride, Y, ldy);
  else if (ydt == SBN_F32)
    SBN_LAUNCH(name, (gemm_kernel<SPARSE, 1, WR, WT>), grid, block, 0, st, Aw, Ai, Xq, s_x, s_w, T, K, R, nks, fstride, Y, ldy);
  else
    SBN_LAUNCH(name, (gemm_kernel<SPARSE, 2, WR, WT>), grid, block, 0, st, Aw, Ai, Xq, s_x, s_w, T, K, R, nks, fstride, Y, ldy);
  return hipGetLastError();
}

}  // namespace

bool gemm_uses_smfmac(int n, int m) { return n <= 2 && (m == 4 || m == 8); }

static int64_t gemm_rb(int64_t R) { return round_up(R, GEMM_TILE_R) / 16; }

size_t gemm_ws_bytes(int64_t /*T*/, int64_t R, int64_t K, int n, int m) {
  const int64_t RB = gemm_rb(R), KBn = cdiv(K, 128);
  if (gemm_uses_smfmac(n, m))
    return align256((size_t)(RB * KBn * 1024)) + align256((size_t)(RB * KBn * 256));
  return align256((size_t)(RB * KBn * 2 * 1024));
}

hipError_t launch_gemm(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                       const uint8_t* codes, const uint8_t* meta, const float* s_w, int64_t R,
                       int n, int m, void* Y, sbn_dtype ydt, int64_t ldy, void* ws, hipStream_t st) {
  const int64_t RB = gemm_rb(R), KBn = cdiv(K, 128);
  uint8_t* w = (uint8_t*)ws;
  if (gemm_uses_smfmac(n, m)) {
    uint8_t* vals = w;
    uint32_t* idx = (uint32_t*)(w + align256((size_t)(RB * KBn * 1024)));
    const int64_t threads = RB * KBn * 64;
    SBN_LAUNCH("expand_sparse", expand_sparse_kernel, dim3((unsigned)cdiv(threads, 256)), dim3(256), 0, st,
                       codes, meta, R, K, n, m, RB, KBn, vals, idx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_gemm_t<true>(vals, idx, Xq, s_x, s_w, T, K, R, KBn, Y, ydt, ldy, st);
  }
  const int64_t KD = 2 * KBn;
  const int64_t threads = RB * KD * 64;
  SBN_LAUNCH("expand_dense", expand_dense_kernel, dim3((unsigned)cdiv(threads, 256)), dim3(256), 0, st,
                     codes, meta, R, K, n, m, RB, KD, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gemm_t<false>(w, nullptr, Xq, s_x, s_w, T, K, R, KBn, Y, ydt, ldy, st);
}

}  // namespace sbn
