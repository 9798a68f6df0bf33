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
// Two kernels per call.  Two layout passes, run side by side in one launch
// (layout_sparse / layout_dense), put both operands in matrix-core fragment
// order (one contiguous 1 KB block per 16 rows x 64 or 128 K, lane l's 16
// bytes at offset 16*l), so every load of the GEMM main loop is a contiguous
// 1 KB global->LDS transfer and every LDS read a contiguous 16-byte read:
//   expand (sparse or dense) : packed codes + meta -> W fragments
//   tile_x                   : Xq [T][K] row-major -> X fragments, zero padded
// then the GEMM.  A weight prepared once (sbn_prepare_gemm_weight: the
// expansion alone, into a caller buffer) serves later calls with no layout
// launch: the GEMM then loads the X fragments straight from row-major Xq.
//
// GEMM: 512 threads (8 waves), block tile 256 rows x 256 tokens, wave tile
// 128 rows x 64 tokens (8 x 4 accumulator tiles of 16 x 16 int32) -- or 128 /
// 64 tokens per block (8 x 2 / 8 x 1 per wave) when the token count leaves
// the 256 x 256 grid too few tiles for the 256 compute units; K step 128
// (sparse, 3 LDS stages of 52 KB; the 64- and 128-token tiles 2 stages of two steps)
// or 64 (dense, 4 stages of 32 KB), stages
// filled with direct global->LDS loads issued two (sparse) or three (dense)
// steps ahead.  The two waves that share a SIMD (w and w + 4) alternate
// between a memory phase (LDS reads of one step's fragments into registers,
// plus the global loads of a later stage) and a compute phase (32 matrix
// instructions), so one of them keeps the SIMD's matrix core busy while the
// other waits on LDS.  Consecutive blocks take tiles that share row and token
// tiles on the same XCD (tile_of_block), so most operand lines come from L2.
//
// Operand layouts (gfx950, measured with a lane-layout check):
//   16x16x64 i8 : A lane l -> row l%16, K[16*(l/16) .. +16); B lane l -> col l%16,
//                 same K bytes; C lane l -> rows 4*(l/16)+v (v = 0..3), col l%16.
//   16x16x128 i8 sparse: A lane l -> row l%16, compressed slot j (0..15) is K
//                 32*(l/16) + 4*(j/2) + idx_j (idx_j = bits 2j..2j+1 of the index
//                 register); B lane l -> col l%16, bytes 0..15 = K[16*(l/16)..),
//                 bytes 16..31 = K[64 + 16*(l/16)..); C as above.
#include <cstdlib>
#include <cstring>

#include "sbn_decode.h"

namespace sbn {
namespace {

constexpr int GT = 256;

// row fragments of the expanded W: R rounded up to the square tile's 256 rows
inline int64_t gemm_rb_dev(int64_t R) { return round_up(R, GEMM_TILE_R) / 16; }

__device__ inline int8_t code_to_i8(uint32_t c) { return c == 1u ? (int8_t)1 : c == 3u ? (int8_t)-1 : (int8_t)0; }

// ---------------------------------------------------------------- expansion: sparse operand
// 1:4, 1:8, 2:8 (2:4 has its own mapping below): one thread = one lane of
// four row-consecutive (16-row, 128-K) fragments: per fragment 16 compressed
// values + 32 index bits.
// vals [RB][KBn][64][16 B]; idx [RB/4][KBn][64][4 x u32] (row fragment 4g+q in
// word q, so a thread's four index words are one 16-byte store)
__device__ inline void expand_sparse_block(
    int64_t blk, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta, int64_t R, int64_t K,
    int n, int m, int64_t RB, int64_t KBn, int64_t cplane, uint8_t* __restrict__ vals,
    uint32_t* __restrict__ idx) {
  const int64_t gid = blk * 256 + threadIdx.x;
  if (gid >= (RB / 4) * KBn * 64) return;
  const int l = (int)(gid & 63);
  const int64_t f = gid >> 6;                   // = g * KBn + kb
  const int64_t g = f / KBn, kb = f - g * KBn;
  const int64_t k0 = kb * 128 + 32 * (l >> 4);
  uint32_t ixs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t rb = 4 * g + q;
    const int64_t r = rb * 16 + (l & 15);
    v4i a = (v4i){0, 0, 0, 0};
    uint32_t ix = 0x44444444u;                  // (0,1) in every half: harmless with zero values
    if (r < R && k0 < K) {
      // 1:4, 1:8, 2:8: at most two survivors per half-group of four positions.
      // The 32 meta bits and the (<= 16) code bits of these positions come from
      // aligned words; each half-group's survivors take the next codes in order.
      const uint32_t mb = *(const uint32_t*)(meta + r * (K / 8) + k0 / 8);
      const int64_t crow = K * n / (4 * m);                 // code bytes per row
      const int64_t cbit = r * crow * 8 + (k0 / m) * 2 * n; // first code bit of these positions
      const int64_t a0 = (cbit >> 3) & ~(int64_t)3;
      const int sh = (int)(cbit - a0 * 8);
      const int64_t lastw = cplane - 4;
      const uint32_t w0 = *(const uint32_t*)(codes + (a0 < lastw ? a0 : lastw));
      const uint32_t w1 = *(const uint32_t*)(codes + (a0 + 4 < lastw ? a0 + 4 : lastw));
      uint32_t cb = (uint32_t)((((unsigned long long)w1 << 32) | w0) >> sh);
      uint32_t v32[4] = {0, 0, 0, 0};
      ix = 0;
#pragma unroll
      for (int h = 0; h < 8; ++h) {             // eight halves of four positions
        const uint32_t nib = (mb >> (4 * h)) & 15u;
        const int cnt = __builtin_popcount(nib);
        const uint32_t p0 = nib ? (uint32_t)__builtin_ctz(nib) : 0u, p1 = nib ? 31u - (uint32_t)__builtin_clz(nib) : 1u;
        const uint32_t v0 = cnt >= 1 ? (uint32_t)(uint8_t)code_to_i8(cb & 3u) : 0u;
        const uint32_t v1 = cnt == 2 ? (uint32_t)(uint8_t)code_to_i8((cb >> 2) & 3u) : 0u;
        cb >>= 2 * cnt;
        // slots (2h, 2h + 1): distinct, ordered positions; a lone survivor at 3 goes second
        uint32_t i0 = p0, i1 = p1, b0 = v0, b1 = v1;
        if (cnt == 0) { i0 = 0; i1 = 1; }
        if (cnt == 1) {
          if (p0 == 3) { i0 = 0; i1 = 3; b0 = 0; b1 = v0; }
          else { i1 = 3; b1 = 0; }
        }
        ix |= (i0 | (i1 << 2)) << (4 * h);
        v32[h >> 1] |= (b0 | (b1 << 8)) << (16 * (h & 1));
      }
      a = (v4i){(int)v32[0], (int)v32[1], (int)v32[2], (int)v32[3]};
    }
    *(v4i*)(vals + ((rb * KBn + kb) * 64 + l) * 16) = a;
    ixs[q] = ix;
  }
  *(uint4*)(idx + ((g * KBn + kb) * 64 + l) * 4) = make_uint4(ixs[0], ixs[1], ixs[2], ixs[3]);
}

// 2:4: one thread = one row of one 128-K step, i.e. the lanes r%16 + 16*j
// (j = 0..3) of row fragment r/16: the row's 16 meta and 16 code bytes of the
// step (positions in order, so four aligned 32-bit words each) come in two
// wide loads, and the 64 threads of a wave (16 rows x 4 row fragments of one
// index block) write whole 256-byte runs of values and of index words.
__device__ inline void expand_sparse24_block(
    int64_t blk, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta, int64_t R, int64_t K,
    int64_t RB, int64_t KBn, uint8_t* __restrict__ vals, uint32_t* __restrict__ idx) {
  const int64_t gid = blk * 256 + threadIdx.x;
  if (gid >= (RB / 4) * KBn * 64) return;
  const int t = (int)(gid & 63), r16 = t & 15, q = t >> 4;
  const int64_t f = gid >> 6;                   // = g * KBn + kb
  const int64_t g = f / KBn, kb = f - g * KBn;
  const int64_t rb = 4 * g + q, r = rb * 16 + r16;
  const int64_t rowb = K / 8;                   // meta (and 2:4 code) bytes per row
  uint32_t mw[4] = {0, 0, 0, 0}, cw[4] = {0, 0, 0, 0};
  if (r < R) {
    const uint8_t* mp = meta + r * rowb + kb * 16;
    const uint8_t* cp = codes + r * rowb + kb * 16;
    if (kb * 128 + 128 <= K && (rowb & 15) == 0) {
      const uint4 m4 = *(const uint4*)mp, c4 = *(const uint4*)cp;
      mw[0] = m4.x; mw[1] = m4.y; mw[2] = m4.z; mw[3] = m4.w;
      cw[0] = c4.x; cw[1] = c4.y; cw[2] = c4.z; cw[3] = c4.w;
    } else {                                    // rows 8-byte aligned; a last step may hold 64 positions
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (kb * 128 + 64 * h < K) {
          const uint2 m2 = *(const uint2*)(mp + 8 * h), c2 = *(const uint2*)(cp + 8 * h);
          mw[2 * h] = m2.x; mw[2 * h + 1] = m2.y;
          cw[2 * h] = c2.x; cw[2 * h + 1] = c2.y;
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int l = r16 + 16 * j;
    v4i a = (v4i){0, 0, 0, 0};
    int ix = 0x44444444;                        // (0,1) in every half: harmless with zero values
    if (r < R && kb * 128 + 32 * j < K) decode24(mw[j], cw[j], a, ix);
    *(v4i*)(vals + ((rb * KBn + kb) * 64 + l) * 16) = a;
    idx[((g * KBn + kb) * 64 + l) * 4 + q] = (uint32_t)ix;
  }
}

// ---------------------------------------------------------------- expansion: dense operand
// One thread = one lane of one (16-row, 64-K) fragment: 16 int8 weights,
// through the unpack table in LDS (built once per block; blocks walk the
// fragments with a grid stride).  vals [RB][KD][64][16 B].
template <int M>
__device__ inline void expand_dense_blocks(
    int64_t blk, int64_t nblk, uint32_t* lut, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta,
    int64_t R, int64_t K, int n, int64_t RB, int64_t KD, int64_t cplane, uint8_t* __restrict__ vals) {
  for (int i = threadIdx.x; i < 4096; i += 256) lut[i] = unpack_entry((uint32_t)i);
  __syncthreads();
  const int64_t total = RB * KD * 64;
  const int64_t crow = K * n / (4 * M);          // code bytes per row
  const int64_t lastw = (cplane - 4) & ~(int64_t)3;
  const bool dense = meta == nullptr;
  for (int64_t gid = blk * 256 + threadIdx.x; gid < total; gid += nblk * 256) {
    const int l = (int)(gid & 63);
    const int64_t f = gid >> 6;
    const int64_t rb = f / KD, kd = f - rb * KD;
    const int64_t r = rb * 16 + (l & 15);
    const int64_t k0 = kd * 64 + 16 * (l >> 4);
    v4i a = (v4i){0, 0, 0, 0};
    if (r < R && k0 < K) {
      const uint32_t mw16 = dense ? 0xFFFFu : (uint32_t)*(const uint16_t*)(meta + r * (K / 8) + k0 / 8);
      // the 16 positions' codes start at bit cbit of the plane (a group boundary)
      const int64_t cbit = r * crow * 8 + k0 * 2 * n / M;
      const int64_t a0 = (cbit >> 3) & ~(int64_t)3;
      const int sh = (int)(cbit - a0 * 8);                        // < 32; sh + 32 bits <= 64
      const uint32_t w0 = *(const uint32_t*)(codes + (a0 < lastw ? a0 : lastw));
      const uint32_t w1 = *(const uint32_t*)(codes + (a0 + 4 < lastw ? a0 + 4 : lastw));
      const unsigned long long c = (((unsigned long long)w1 << 32) | w0) >> sh;
      a = unpack16<M>(lut, mw16, dense, n, c, 0);
    }
    *(v4i*)(vals + gid * 16) = a;
  }
}

// ---------------------------------------------------------------- activation fragments
// Xt [TBp][KC][64][16 B]: block (tb, kc) holds tokens 16*tb.. and K bytes
// 64*kc..; lane l carries token 16*tb + l%16, K bytes 64*kc + 16*(l/16) ..+16.
// Tokens >= T and K >= K are zero.  One 256-thread block covers 16 tokens x
// 256 K bytes (four Xt blocks): thread i reads 16 bytes of token i/16 (so a
// wave reads four 256-byte row runs) and writes them to lane
// i/16 + 16*((i%16)%4) of Xt block (i%16)/4 -- the four blocks are whole
// within the workgroup, so their lines fill in one L2.
__device__ inline void tile_x_block(int64_t blk, const int8_t* __restrict__ Xq, int64_t T, int64_t K,
                                    int64_t TBp, int64_t KC, uint4* __restrict__ Xt) {
  const int64_t spans = (KC + 3) / 4;
  if (blk >= TBp * spans) return;
  const int64_t tb = blk / spans, sp = blk - tb * spans;
  const int i = threadIdx.x, tok = i >> 4, piece = i & 15;
  const int64_t kc = sp * 4 + (piece >> 2);
  if (kc >= KC) return;
  const int64_t t = tb * 16 + tok;
  const int64_t k = sp * 256 + 16 * piece;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (t < T && k < K) v = *(const uint4*)(Xq + t * K + k);
  Xt[(tb * KC + kc) * 64 + tok + 16 * (piece & 3)] = v;
}

// ---------------------------------------------------------------- the two layout passes in one launch
// Blocks [0, nbw) expand W, blocks [nbw, nbw + nbx) tile X: the two passes are
// independent, so one grid runs them side by side (one launch ramp, and the
// short X pass fills the compute units the W pass leaves idle).
struct XTileArgs {
  const int8_t* Xq;
  int64_t T, K, TBp, KC;
  uint4* Xt;
};

__global__ __launch_bounds__(256) void layout_sparse_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta, int64_t R, int64_t K,
    int n, int m, int64_t RB, int64_t KBn, int64_t cplane, uint8_t* __restrict__ vals,
    uint32_t* __restrict__ idx, int64_t nbw, const XTileArgs xa) {
  const int64_t b = blockIdx.x;
  if (b < nbw) {
    if (n == 2 && m == 4)
      expand_sparse24_block(b, codes, meta, R, K, RB, KBn, vals, idx);
    else
      expand_sparse_block(b, codes, meta, R, K, n, m, RB, KBn, cplane, vals, idx);
  } else
    tile_x_block(b - nbw, xa.Xq, xa.T, xa.K, xa.TBp, xa.KC, xa.Xt);
}

// N: survivors per group, a template argument so each ratio's decode is straight-line code.
template <int M, int N>
__global__ __launch_bounds__(256) void layout_dense_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta, int64_t R, int64_t K,
    int64_t RB, int64_t KD, int64_t cplane, uint8_t* __restrict__ vals, int64_t nbw, const XTileArgs xa) {
  __shared__ uint32_t lut[4096];
  const int64_t b = blockIdx.x;
  if (b < nbw)                                       // uniform per block: the table barrier is safe
    expand_dense_blocks<M>(b, nbw, lut, codes, meta, R, K, N, RB, KD, cplane, vals);
  else
    tile_x_block(b - nbw, xa.Xq, xa.T, xa.K, xa.TBp, xa.KC, xa.Xt);
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


__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// workgroup barrier kept in program order with the surrounding waits
__device__ inline void pp_barrier() {
  sched_fence();
  asm volatile("s_barrier" ::: "memory");
  sched_fence();
}

// OUT: 0 = int32 accumulator, 1 = float32, 2 = bf16.
// MJ: token fragments per wave (4: 256-token block tile; 2 and 1: 128 and 64
// tokens, for token counts whose 256 x 256 grid would leave compute units idle).
template <bool SPARSE, int OUT, int MJ, bool DX>
__global__ __launch_bounds__(512, 1) void gemm_kernel(
    const uint8_t* __restrict__ Aw, const uint8_t* __restrict__ Ai, const uint8_t* __restrict__ Xt,
    const float* __restrict__ s_x, const float* __restrict__ s_w, int64_t T, int64_t R,
    int64_t nks, int64_t fstride, int64_t KC, int64_t ldx, void* __restrict__ Y, int64_t ldy) {
  constexpr int NW = 8, MI = 8;                        // 8 waves; wave tile 8 x MJ fragments
  constexpr int TT = 64 * MJ;                          // tokens per block tile
  constexpr int A_BYTES = 16 * 1024;                   // 16 row fragments
  constexpr int I_BYTES = SPARSE ? 4 * 1024 : 0;       // their index words
  constexpr int BH = SPARSE ? 2 : 1;                   // 1 KB X blocks per token block per step
  constexpr int NXB = 4 * MJ * BH;                     // 1 KB X blocks per stage
  static_assert(NXB % NW == 0, "every wave loads the same number of X blocks");
  constexpr int B_BYTES = NXB * 1024;
  // KS K steps per stage: the 64- and 128-token sparse tiles on the tiled X
  // copy take two per stage (two stages of 56 / 72 KB), so each ping-pong
  // phase holds 16 / 32 matrix instructions per wave instead of 8 / 16 and
  // the barriers per step halve (the dense tiles measured no gain from it,
  // and the direct-X tiles lose 0-11%).
  constexpr int KS = (SPARSE && !DX && MJ <= 2) ? 2 : 1;
  constexpr int SUB = A_BYTES + I_BYTES + B_BYTES;     // one K step
  constexpr int STAGE = KS * SUB;
  constexpr int NST = KS == 2 ? 2 : SPARSE ? 3 : 4;
  static_assert(NST * STAGE <= 160 * 1024, "LDS");
  // global loads per wave per stage: 2 W fragments, NXB / 8 X blocks, the
  // index block (waves 0..3, sparse), per K step
  constexpr int LPS0 = KS * (2 + (SPARSE ? 1 : 0) + NXB / NW);
  constexpr int LPS1 = KS * (2 + NXB / NW);
  constexpr int WAIT0 = (NST - 2) * LPS0, WAIT1 = (NST - 2) * LPS1;
  constexpr int EPI_BYTES = NW * 16 * MJ * 272;         // bf16 epilogue staging, 16*MJ x 272 B per wave
  constexpr int SMEM = NST * STAGE > EPI_BYTES ? NST * STAGE : EPI_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int grp = wave >> 2;                           // waves w and w + 4 share a SIMD
  const int wr = wave & 1, wt = wave >> 1;             // rows 128*wr.., tokens 16*MJ*wt..
  int64_t rtile, ttile;
  tile_of_block(blockIdx.x, cdiv(R, 256), cdiv(T, TT), rtile, ttile);
  const int64_t tile_r = rtile * 256, tile_t = ttile * TT;
  const int64_t rb0 = tile_r / 16, tb0 = tile_t / 16;

  // scales for the epilogue, fetched before the main loop
  float sw = 0.0f, sxv[MJ];
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int64_t t = tile_t + 16 * (MJ * wt + j) + (lane & 15);
    sxv[j] = (OUT != 0 && t < T) ? s_x[t] : 0.0f;
  }
  if (OUT != 0) sw = *s_w;

  // DX: X straight from Xq [T][ldx] instead of the tiled copy, into the same
  // LDS layout: lane l of 1 KB block hb reads token 16*(hb/BH) + l%16 of the
  // tile, bytes 16*(l/16).. of 64-byte chunk step*BH + hb%BH of its row.
  // Tokens past T re-read token T - 1 (they feed only outputs never stored);
  // a chunk past K (the upper half of a last 128-K step) re-reads chunk KC - 1
  // (KC = K / 64 here), whose weights are zero.
  const int8_t* xbase = (const int8_t*)Xt + tile_t * ldx;
  uint32_t xoff[NXB / NW];
  if constexpr (DX) {
#pragma unroll
    for (int q = 0; q < NXB / NW; ++q) {
      const int hb = wave + NW * q;
      const int64_t t = tile_t + 16 * (hb / BH) + (lane & 15);
      xoff[q] = (uint32_t)(((t < T ? t : T - 1) - tile_t) * ldx + 16 * (lane >> 4));
    }
  }

  const int64_t nss = cdiv(nks, KS);                   // stages (the last may hold one K step)
  auto load_stage = [&](int s, int64_t ss) {
#pragma unroll
  for (int u = 0; u < KS; ++u) {
    const int64_t ks = ss * KS + u;
    if (KS > 1 && ks >= nks) break;
    uint8_t* base = smem + s * STAGE + u * SUB;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int i = wave + NW * q;
      g2lds16(Aw + ((rb0 + i) * fstride + ks) * 1024 + lane * 16, base + i * 1024);
    }
    if (SPARSE && grp == 0)
      g2lds16(Ai + ((rb0 / 4 + wave) * fstride + ks) * 1024 + lane * 16, base + A_BYTES + wave * 1024);
#pragma unroll
    for (int q = 0; q < NXB / NW; ++q) {
      const int hb = wave + NW * q;                    // 1 KB block: token block hb/BH, half hb%BH
      if constexpr (DX) {
        int64_t kc = ks * BH + hb % BH;
        kc = kc < KC ? kc : KC - 1;
        g2lds16(xbase + kc * 64 + xoff[q], base + A_BYTES + I_BYTES + hb * 1024);
      } else {
        g2lds16(Xt + ((tb0 + hb / BH) * KC + ks * BH + hb % BH) * 1024 + lane * 16,
                base + A_BYTES + I_BYTES + hb * 1024);
      }
    }
  }
  };

  v4i acc[MI][MJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < MJ; ++j) acc[i][j] = (v4i){0, 0, 0, 0};
  v4i a[KS][MI], blo[KS][MJ], bhi[KS][MJ];
  int ix[KS][MI];

  // memory phase of stage s: issue the loads of stage s + NST - 1, read stage s's fragments
  auto mem_phase = [&](int64_t s) {
    if (s + NST - 1 < nss) load_stage((int)((s + NST - 1) % NST), s + NST - 1);
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const uint8_t* base = smem + (s % NST) * STAGE + u * SUB;
      const uint8_t* bb = base + A_BYTES + I_BYTES;
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        const int jj = MJ * wt + j;
        blo[u][j] = *(const v4i*)(bb + (jj * BH + 0) * 1024 + lane * 16);
        if (SPARSE) bhi[u][j] = *(const v4i*)(bb + (jj * BH + 1) * 1024 + lane * 16);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) a[u][i] = *(const v4i*)(base + (MI * wr + i) * 1024 + lane * 16);
      if (SPARSE) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v4i v = *(const v4i*)(base + A_BYTES + (2 * wr + h) * 1024 + lane * 16);
          ix[u][4 * h] = v[0]; ix[u][4 * h + 1] = v[1]; ix[u][4 * h + 2] = v[2]; ix[u][4 * h + 3] = v[3];
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  auto comp_phase = [&](int64_t s) {
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      if (KS > 1 && s * KS + u >= nks) break;          // a last stage with one K step
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
          if (SPARSE) {
            const v8i b = (v8i){blo[u][j][0], blo[u][j][1], blo[u][j][2], blo[u][j][3],
                                bhi[u][j][0], bhi[u][j][1], bhi[u][j][2], bhi[u][j][3]};
            acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a[u][i], b, acc[i][j], ix[u][i], 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][i], blo[u][j], acc[i][j], 0, 0, 0);
          }
        }
    }
  };
  // this wave's loads of stage s + 1 have landed (later stages may still fly)
  auto vm_wait = [&](int64_t s) {
    sched_fence();
    if (s + NST - 1 < nss) {
      if (grp == 0) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(WAIT0) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(WAIT1) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    sched_fence();
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
    if (s < nss) load_stage(s, s);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  pp_barrier();                                        // B0: stages 0 .. NST-2 visible
  if (grp == 0) {
    for (int64_t s = 0; s < nss; ++s) {
      mem_phase(s);
      pp_barrier();
      comp_phase(s);
      vm_wait(s);
      pp_barrier();
    }
  } else {
    pp_barrier();
    for (int64_t s = 0; s < nss; ++s) {
      mem_phase(s);
      vm_wait(s);
      pp_barrier();
      comp_phase(s);
      if (s + 1 < nss) pp_barrier();
    }
  }

  if (OUT == 2) {
    // bf16: stage the wave's 128 x 16*MJ tile through LDS as [token][row] (pitch
    // 272 B keeps the 8-byte writes of 16 tokens on distinct banks), then store
    // four token rows of 256 contiguous bytes per instruction, non-temporal so
    // the output streams past L2 instead of evicting operands other blocks
    // still read.  All LDS stages are free here: every wave passed its last
    // stage read before B(2*nks).
    constexpr int PITCH = 272;
    static_assert(NW * 16 * MJ * PITCH <= SMEM, "epilogue staging fits");
    uint8_t* st = smem + wave * (16 * MJ * PITCH);
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      const float sc = sw * sxv[j];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const v4i c = acc[i][j];
        uint2 v;
        v.x = pack_bf16x2((float)c[0] * sc, (float)c[1] * sc);
        v.y = pack_bf16x2((float)c[2] * sc, (float)c[3] * sc);
        *(uint2*)(st + (16 * j + (lane & 15)) * PITCH + (16 * i + 4 * (lane >> 4)) * 2) = v;
      }
    }
    const int64_t r0 = tile_r + 128 * wr + 8 * (lane & 15);
#pragma unroll
    for (int q = 0; q < 4 * MJ; ++q) {
      const int tl = 4 * q + (lane >> 4);
      const int64_t t = tile_t + 16 * MJ * wt + tl;
      const v4i v = *(const v4i*)(st + tl * PITCH + (lane & 15) * 16);
      if (t >= T || r0 >= R) continue;
      uint16_t* y = (uint16_t*)Y + t * ldy + r0;
      if (r0 + 7 < R) {
        __builtin_nontemporal_store(v, (v4i*)y);
      } else {
        const uint32_t w[4] = {(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
        for (int e = 0; e < 8 && r0 + e < R; ++e) y[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }
    return;
  }
  // int32 / float32 epilogue: lane holds rows r..r+3 of token t, 16 bytes
#pragma unroll
  for (int j = 0; j < MJ; ++j) {
    const int64_t t = tile_t + 16 * (MJ * wt + j) + (lane & 15);
    if (t >= T) continue;
    const float sc = (OUT != 0) ? sw * sxv[j] : 0.0f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int64_t r = tile_r + 16 * (MI * wr + i) + 4 * (lane >> 4);
      if (r >= R) continue;
      const v4i c = acc[i][j];
      if (OUT == 0) {
        int* y = (int*)Y + t * ldy + r;
        if (r + 3 < R) *(v4i*)y = c;
        else for (int v = 0; v < 4 && r + v < R; ++v) y[v] = c[v];
      } else {
        float* y = (float*)Y + t * ldy + r;
        const v4f o = (v4f){(float)c[0] * sc, (float)c[1] * sc, (float)c[2] * sc, (float)c[3] * sc};
        if (r + 3 < R) *(v4f*)y = o;
        else for (int v = 0; v < 4 && r + v < R; ++v) y[v] = o[v];
      }
    }
  }
}

// ---------------------------------------------------------------- GEMM, wide sparse tile
// One block per compute unit, one wave per SIMD: block tile MI row fragments
// (16*MI rows) x 256 tokens; wave w owns tokens 64w..64w+63 of it against all
// MI row fragments (MI x 4 accumulator tiles: 4*MI accumulator registers per
// lane).  A compute unit streams operands from L2 into LDS at about 23 bytes
// per clock whatever the grid (measured; the 256 x 256 kernel's main loop runs
// at exactly that rate with its matrix cores half idle), so this tile is
// shaped for the fewest operand bytes per output: a K step of 16*MI x 256
// outputs loads MI + NG + 32 KB (W fragments, their index blocks, X), against
// 52 KB for 256 x 256 outputs.  It pays where the 256 x 256 grid ends in a
// partial round: 6912 rows x 4096 tokens is 432 square tiles on 256 compute
// units but 256 tiles of 432 x 256.  Two LDS stages of one K step: the next
// step's loads fly while a step's matrix work runs.
// A raw buffer resource over `bytes` bytes at `base` (reads past the end
// return zero), and a 16-byte-per-lane load through it into LDS at `lds`
// (wave-uniform) + 16 * lane: vector offset `voff`, uniform offset `soff`.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
__device__ inline void buf2lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// DX: X straight from row-major Xq [T][K] (K a multiple of 64) instead of the
// tiled copy.  A K step of one token is then one 128-byte line, and the stage
// holds the tile's 256 lines as [token][8 x 16 bytes], the 16-byte pieces of
// token t's line permuted by xswz(t % 16): a load instruction fetches eight
// whole lines (lane l: line l/8, slot l%8 takes piece (l%8) ^ xswz), and the
// fragment reads (lane: token n of 16, pieces g and g+4) fall on distinct
// banks in every group of 8 and of 16 lanes.  Tokens past T and the bytes
// past the end of Xq read as zero through the buffer resource's bound (the
// whole offset travels in the vector operand, which the bound checks); a last
// half step's upper pieces read the next row, against zero weights.
__device__ inline uint32_t xswz(uint32_t n) { return (n ^ (n >> 3)) & 7u; }

template <int OUT, int MI, bool DX>
__global__ __launch_bounds__(256, 1) void gemm_wide_kernel(
    const uint8_t* __restrict__ Aw, const uint8_t* __restrict__ Ai, const uint8_t* __restrict__ Xt,
    const float* __restrict__ s_x, const float* __restrict__ s_w, int64_t T, int64_t R, int64_t RB,
    int64_t nks, int64_t KC, int64_t K, void* __restrict__ Y, int64_t ldy) {
  static_assert(MI % 4 == 0, "tiles start on an index block");
  constexpr int NG = MI / 4;                         // index blocks of the tile's row fragments
  constexpr int NB = MI + NG + 32;                   // 1 KB blocks per K step: W, index words, X (16 x lo/hi)
  constexpr int STAGE = NB * 1024;
  static_assert(2 * STAGE + 1024 <= 160 * 1024, "LDS");
  // two stage buffers as separate objects, each step's reads and fills naming
  // them statically: the compiler then knows a step's LDS reads do not touch
  // the buffer its global->LDS loads are filling, and does not wait for them
  __shared__ __attribute__((aligned(1024))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sm1[STAGE];
  __shared__ float sxs[256];                         // the tile's activation scales

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  int64_t rtile, ttile;
  tile_of_block(blockIdx.x, cdiv(RB, MI), cdiv(T, 256), rtile, ttile);
  const int64_t rb0 = rtile * MI, tb0 = ttile * 16, tile_t = ttile * 256;
  const int64_t g0 = rb0 / 4;                        // row fragment rb0 + i: index block g0 + i / 4, word i % 4
  if (OUT != 0) sxs[tid] = tile_t + tid < T ? s_x[tile_t + tid] : 0.0f;

  // Loads of one K step: wave w takes W fragments w, w+4, .. (MI / 4 slots),
  // index blocks w and w+4 (the last wave's second slot loads block NG - 1
  // again: same bytes to the same place) and X blocks w, w+4, .. (8 slots).
  // The expanded W holds whole wide tiles of row fragments (the rows past R
  // are never stored).  Buffer loads: one resource per operand, the slot's
  // offset uniform, the lane's 16 bytes as the vector offset (every operand is
  // below 2^31 bytes: the launcher checks).  Slot offsets are walked with
  // opaque adds so the compiler keeps two registers per operand, not one per slot.
  const uint32_t fa = (uint32_t)nks * 1024u;          // bytes per row fragment (and per index block) over all K steps
  const int64_t RBw = round_up(RB, MI);               // row fragments of the expanded W
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(Aw, (uint32_t)(RBw * fa));
  const __amdgpu_buffer_rsrc_t rI = make_rsrc(Ai, (uint32_t)((RBw / 4) * fa));
  const __amdgpu_buffer_rsrc_t rX =
      make_rsrc(Xt, DX ? (uint32_t)(T * K) : (uint32_t)(cdiv(T, 256) * 16 * KC * 1024));
  const uint32_t voff = (uint32_t)lane * 16u;
  // DX: lane's line (token tile_t + 8 * wave + lane / 8 in slot 0; each later
  // slot 32 tokens on) and its piece
  const uint32_t xl = (uint32_t)(8 * wave + (lane >> 3));
  const uint32_t voffx = DX ? (uint32_t)((tile_t + xl) * K) + 16u * ((uint32_t)(lane & 7) ^ xswz(xl & 15u)) : voff;
  // DX: the lane's fragment-read offset in the stage's X lines (token 64 * wave + lane % 16, piece lane / 16)
  const uint32_t xlane = (uint32_t)((64 * wave + (lane & 15)) * 128) +
                         16u * ((uint32_t)(lane >> 4) ^ xswz((uint32_t)(lane & 15)));
  const uint32_t offa0 = (uint32_t)(rb0 + wave) * fa, stepa = 4u * fa;
  const int bi1 = wave + 4 < NG ? wave + 4 : NG - 1;
  const uint32_t offi0 = (uint32_t)(g0 + wave) * fa, offi1 = (uint32_t)(g0 + bi1) * fa;
  const uint32_t offx0 = DX ? 0u : (uint32_t)(((tb0 + wave / 2) * KC + wave % 2) * 1024);
  const uint32_t stepx = DX ? (uint32_t)(32 * K) : (uint32_t)(2 * KC * 1024);
  auto load_stage = [&](uint8_t* d, int ks) {
    const uint32_t k1 = (uint32_t)ks * 1024u;
    uint32_t so = offa0 + k1;
#pragma unroll
    for (int q = 0; q < MI / 4; ++q) {
      buf2lds16(rA, voff, so, d + (wave + 4 * q) * 1024);
      so += stepa;
      asm volatile("" : "+s"(so));
    }
    buf2lds16(rI, voff, offi0 + k1, d + (MI + wave) * 1024);
    buf2lds16(rI, voff, offi1 + k1, d + (MI + bi1) * 1024);
    if constexpr (DX) {
      // the whole offset in the vector operand, so the resource's bound checks all of it
      uint32_t vo = voffx + (uint32_t)ks * 128u;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        buf2lds16(rX, vo, 0u, d + (MI + NG + wave + 4 * q) * 1024);
        vo += stepx;
      }
    } else {
      so = offx0 + 2 * k1;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        buf2lds16(rX, voff, so, d + (MI + NG + wave + 4 * q) * 1024);
        so += stepx;
        asm volatile("" : "+s"(so));
      }
    }
  };

  v4i acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

  // One K step from buffer buf: the wave's four X fragments, then the W
  // fragments and index words two row fragments ahead of the matrix
  // instructions that use them; the loads of K step `next` (if any) are
  // issued after the first reads.
  auto step = [&](const uint8_t* st, uint8_t* nst, int next) {
    const uint8_t* ab = st + lane * 16;
    const uint8_t* ib = st + MI * 1024 + lane * 16;
    v8i b[4];
    if constexpr (DX) {
      // token 64 * wave + 16 * j + n (n = lane % 16): pieces g and g + 4 (g =
      // lane / 16); lines start on 128 bytes, so piece g + 4's slot is piece
      // g's with bit 6 flipped.  The lane's offset is rebuilt every step (an
      // opaque copy) rather than kept per stage buffer and half.
      uint32_t xo = xlane;
      asm volatile("" : "+v"(xo));
      const uint8_t* xr = st + (MI + NG) * 1024;
      const uint8_t* xlo = xr + xo;
      const uint8_t* xhi = xr + (xo ^ 64u);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i lo = *(const v4i*)(xlo + j * 2048), hi = *(const v4i*)(xhi + j * 2048);
        b[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    } else {
      const uint8_t* xb = st + (MI + NG + 8 * wave) * 1024 + lane * 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i lo = *(const v4i*)(xb + (2 * j) * 1024), hi = *(const v4i*)(xb + (2 * j + 1) * 1024);
        b[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
    v4i a[MI], ixg[NG];                              // ixg[g]: index words of row fragments 4g .. 4g+3
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = *(const v4i*)(ab + i * 1024);
    ixg[0] = *(const v4i*)ib;
    sched_fence();
    if (next >= 0) load_stage(nst, next);
    sched_fence();
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      // W fragment i + 2 and, two fragments before a group starts, that group's index words
      const bool ra2 = i + 2 < MI, rg = (i + 2) % 4 == 0 && i + 2 < MI;
      if (ra2) a[i + 2] = *(const v4i*)(ab + (i + 2) * 1024);
      if (rg) ixg[(i + 2) / 4] = *(const v4i*)(ib + ((i + 2) / 4) * 1024);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a[i], b[j], acc[i][j], ixg[i / 4][i % 4], 0, 0);
      if (rg) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // the LDS reads above
      else if (ra2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                // then fragment i's matrix instructions
    }
    sched_fence();
  };

  // stage s lives in buffer s % 2; step s loads stage s + 1 into the other
  // buffer (freed by the barrier after step s - 1)
  auto finish = [&]() {
    wait_vmem();                                     // this wave's loads of the next stage have landed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    pp_barrier();                                    // every wave is done with this buffer; the next stage is whole
  };
  load_stage(sm0, 0);
  wait_vmem();
  pp_barrier();
  const int ns = (int)nks;                           // 32-bit step counts keep the loop control scalar
  int s = 0;
  for (; s + 1 < ns; s += 2) {
    step(sm0, sm1, s + 1);
    finish();
    step(sm1, sm0, s + 2 < ns ? s + 2 : -1);
    finish();
  }
  if (s < ns) {
    step(sm0, sm1, -1);
    finish();
  }

  const float sw = OUT != 0 ? *s_w : 0.0f;
  if constexpr (OUT == 2) {
    // bf16: a wave's 64 tokens x 16*MI rows, one 16-token fragment at a time,
    // through LDS as [token][row] (the stage buffers are free: every wave
    // passed the last barrier), then stored as whole token rows of 32*MI
    // contiguous bytes, 16 per lane, non-temporal so the output streams past
    // L2; the stores of one fragment fly while the next is converted
    constexpr int PITCH = MI * 32 + 16;              // bytes per staged token row (16 bytes of padding)
    constexpr int NV = MI * 2;                       // 16-byte pieces per token row
    static_assert(2 * 32 * PITCH <= STAGE, "epilogue staging fits");
    uint8_t* stg = (wave < 2 ? sm0 : sm1) + (wave & 1) * 32 * PITCH;
    const int64_t r0 = rb0 * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sc = sw * sxs[16 * (4 * wave + j) + (lane & 15)];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const v4i c = acc[i][j];
        uint2 v;
        v.x = pack_bf16x2((float)c[0] * sc, (float)c[1] * sc);
        v.y = pack_bf16x2((float)c[2] * sc, (float)c[3] * sc);
        *(uint2*)(stg + (lane & 15) * PITCH + (16 * i + 4 * (lane >> 4)) * 2) = v;
      }
      const int64_t t0 = tile_t + 16 * (4 * wave + j);
#pragma unroll 2
      for (int k = 0; k < 16 * NV / 64; ++k) {
        const int p = lane + 64 * k, tl = p / NV, pc = p - tl * NV;
        const v4i v = *(const v4i*)(stg + tl * PITCH + pc * 16);
        const int64_t t = t0 + tl, r = r0 + 8 * pc;
        if (t >= T || r >= R) continue;
        uint16_t* y = (uint16_t*)Y + t * ldy + r;
        if (r + 7 < R) {
          __builtin_nontemporal_store(v, (v4i*)y);
        } else {
          const uint32_t w[4] = {(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
          for (int e = 0; e < 8 && r + e < R; ++e) y[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this fragment's reads are done before the next one's writes
    }
    return;
  }
  // int32 / float32: lane holds rows r..r+3 of token t of each accumulator tile, 16 bytes
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tl = 16 * (4 * wave + j) + (lane & 15);
    const int64_t t = tile_t + tl;
    if (t >= T) continue;
    const float sc = OUT != 0 ? sw * sxs[tl] : 0.0f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int64_t r = (rb0 + i) * 16 + 4 * (lane >> 4);
      if (r >= R) continue;
      const v4i c = acc[i][j];
      if (OUT == 0) {
        int* y = (int*)Y + t * ldy + r;
        if (r + 3 < R) *(v4i*)y = c;
        else for (int v = 0; v < 4 && r + v < R; ++v) y[v] = c[v];
      } else {
        float* y = (float*)Y + t * ldy + r;
        const v4f o = (v4f){(float)c[0] * sc, (float)c[1] * sc, (float)c[2] * sc, (float)c[3] * sc};
        if (r + 3 < R) *(v4f*)y = o;
        else for (int v = 0; v < 4 && r + v < R; ++v) y[v] = o[v];
      }
    }
  }
}

template <bool SPARSE, int MJ, bool DX>
hipError_t launch_gemm_mj(const uint8_t* Aw, const uint8_t* Ai, const uint8_t* Xt, const float* s_x,
                          const float* s_w, int64_t T, int64_t K, int64_t R, int64_t KBn, void* Y,
                          sbn_dtype ydt, int64_t ldy, hipStream_t st) {
  const int64_t ntiles = cdiv(T, 64 * MJ) * cdiv(R, GEMM_TILE_R);
  const dim3 grid((unsigned)ntiles), block(512);
  const int64_t nks = SPARSE ? KBn : K / 64;
  const int64_t fstride = SPARSE ? KBn : 2 * KBn;
  const int64_t KC = DX ? K / 64 : 2 * KBn, ldx = K;  // 64-byte chunks of an X row (direct) or a tiled row
  const char* name = SPARSE ? "gemm_smfmac" : "gemm_mfma";
  if (ydt == SBN_I32_ACC)
    SBN_LAUNCH(name, (gemm_kernel<SPARSE, 0, MJ, DX>), grid, block, 0, st, Aw, Ai, Xt, s_x, s_w, T, R, nks, fstride, KC,
               ldx, Y, ldy);
  else if (ydt == SBN_F32)
    SBN_LAUNCH(name, (gemm_kernel<SPARSE, 1, MJ, DX>), grid, block, 0, st, Aw, Ai, Xt, s_x, s_w, T, R, nks, fstride, KC,
               ldx, Y, ldy);
  else
    SBN_LAUNCH(name, (gemm_kernel<SPARSE, 2, MJ, DX>), grid, block, 0, st, Aw, Ai, Xt, s_x, s_w, T, R, nks, fstride, KC,
               ldx, Y, ldy);
  return hipGetLastError();
}

// Token fragments per wave: the tile width whose grid finishes first, with one
// block per compute unit -- rounds of 256 tiles times a tile's time, measured
// at about 1 : 1.25 : 1.8 for the 64-, 128- and 256-token tiles (a 256-token
// tile does four times the work of a 64-token one in 1.8 times the time, so
// wide tiles win once the grid fills the chip).  64 tokens: sparse only.
int gemm_mj(bool sparse, int64_t T, int64_t R) {
  const int64_t rt = cdiv(R, GEMM_TILE_R);
  const double cost[3] = {1.0, 1.25, 1.8};            // MJ = 1, 2, 4
  int best = 4;
  double best_t = 1e300;
  for (int i = 2; i >= (sparse ? 0 : 1); --i) {
    const int mj = 1 << i;
    const double t = (double)cdiv(cdiv(T, 64 * mj) * rt, 256) * cost[i];
    if (t < best_t) {
      best_t = t;
      best = mj;
    }
  }
  return best;
}

constexpr int WIDE_MI = 28;                          // 448-row tiles

template <int MI, bool DX>
hipError_t launch_gemm_wide(const uint8_t* Aw, const uint8_t* Ai, const uint8_t* Xt, const float* s_x,
                            const float* s_w, int64_t T, int64_t K, int64_t R, int64_t KBn, void* Y, sbn_dtype ydt,
                            int64_t ldy, hipStream_t st) {
  const int64_t RB = gemm_rb_dev(R);
  const dim3 grid((unsigned)(cdiv(RB, MI) * cdiv(T, 256))), block(256);
  const int64_t KC = 2 * KBn;
  if (ydt == SBN_I32_ACC)
    SBN_LAUNCH("gemm_smfmac_wide", (gemm_wide_kernel<0, MI, DX>), grid, block, 0, st, Aw, Ai, Xt, s_x, s_w, T, R, RB,
               KBn, KC, K, Y, ldy);
  else if (ydt == SBN_F32)
    SBN_LAUNCH("gemm_smfmac_wide", (gemm_wide_kernel<1, MI, DX>), grid, block, 0, st, Aw, Ai, Xt, s_x, s_w, T, R, RB,
               KBn, KC, K, Y, ldy);
  else
    SBN_LAUNCH("gemm_smfmac_wide", (gemm_wide_kernel<2, MI, DX>), grid, block, 0, st, Aw, Ai, Xt, s_x, s_w, T, R, RB,
               KBn, KC, K, Y, ldy);
  return hipGetLastError();
}

// The wide tile where its grid finishes first: both kernels' main loops run
// at the compute unit's operand streaming rate, so a grid costs its rounds
// of 256 tiles times the bytes one tile loads per K step (KB: 256 x 256: 52,
// 256 x 128: 36, 256 x 64: 28; wide: MI + NG + 32).  SBN_GEMM_TILE=wide or
// =square in the environment overrides the choice (read per call; operands
// of 2^31 bytes or more always take the square tiles).
bool gemm_use_wide(int64_t T, int64_t R, int64_t KBn) {
  // the wide kernel addresses each operand with 32-bit offsets
  const int64_t lim = (int64_t)1 << 31;
  if (round_up(gemm_rb_dev(R), WIDE_MI) * KBn * 1024 >= lim || cdiv(T, 256) * 16 * KBn * 2048 >= lim) return false;
  if (const char* e = getenv("SBN_GEMM_TILE")) {
    if (!strcmp(e, "wide")) return true;
    if (!strcmp(e, "square")) return false;
  }
  const int mj = gemm_mj(true, T, R);
  const double sq_bytes = mj == 4 ? 52.0 : mj == 2 ? 36.0 : 28.0;
  const double sq = (double)cdiv(cdiv(T, 64 * mj) * cdiv(R, GEMM_TILE_R), 256) * sq_bytes;
  const double wide_bytes = WIDE_MI + WIDE_MI / 4 + 32;
  const double wd = (double)cdiv(cdiv(gemm_rb_dev(R), WIDE_MI) * cdiv(T, 256), 256) * wide_bytes;
  return wd < 0.9 * sq;
}

template <bool SPARSE, bool DX>
hipError_t launch_gemm_t(const uint8_t* Aw, const uint8_t* Ai, const uint8_t* Xt, const float* s_x,
                         const float* s_w, int64_t T, int64_t K, int64_t R, int64_t KBn, void* Y,
                         sbn_dtype ydt, int64_t ldy, hipStream_t st) {
  if constexpr (SPARSE) {
    if (gemm_use_wide(T, R, KBn))
      return launch_gemm_wide<WIDE_MI, DX>(Aw, Ai, Xt, s_x, s_w, T, K, R, KBn, Y, ydt, ldy, st);
  }
  const int mj = gemm_mj(SPARSE, T, R);
  if (mj == 4) return launch_gemm_mj<SPARSE, 4, DX>(Aw, Ai, Xt, s_x, s_w, T, K, R, KBn, Y, ydt, ldy, st);
  if (mj == 2) return launch_gemm_mj<SPARSE, 2, DX>(Aw, Ai, Xt, s_x, s_w, T, K, R, KBn, Y, ydt, ldy, st);
  if (SPARSE) return launch_gemm_mj<SPARSE, SPARSE ? 1 : 2, DX>(Aw, Ai, Xt, s_x, s_w, T, K, R, KBn, Y, ydt, ldy, st);
  return hipErrorInvalidValue;
}

}  // namespace

bool gemm_uses_smfmac(int n, int m) { return n <= 2 && (m == 4 || m == 8); }


static int64_t gemm_rb(int64_t R) { return round_up(R, GEMM_TILE_R) / 16; }
static int64_t gemm_tbp(int64_t T) { return round_up(T, GEMM_TILE_T) / 16; }

// [W fragments][index blocks (sparse)][X fragments]
struct GemmWs {
  size_t w_bytes, i_bytes, x_bytes;
};
static GemmWs gemm_ws(int64_t T, int64_t R, int64_t K, int n, int m) {
  const int64_t RB = gemm_rb(R), KBn = cdiv(K, 128);
  GemmWs g;
  g.w_bytes = align256((size_t)(RB * KBn * 2048));                 // sparse: vals use the first half
  if (gemm_uses_smfmac(n, m)) {
    // whole wide tiles of row fragments (the wide kernel reads them; the
    // expansion writes the first RB)
    const int64_t RBw = round_up(RB, WIDE_MI);
    g.w_bytes = align256((size_t)(RBw * KBn * 1024));
    g.i_bytes = align256((size_t)(RBw * KBn * 256));
  } else {
    g.i_bytes = 0;
  }
  g.x_bytes = align256((size_t)(gemm_tbp(T) * KBn * 2 * 1024));
  return g;
}

size_t gemm_ws_bytes(int64_t T, int64_t R, int64_t K, int n, int m) {
  const GemmWs g = gemm_ws(T, R, K, n, m);
  return g.w_bytes + g.i_bytes + g.x_bytes;
}

// The GEMM call in parts: the layout launch expands W into `w` (expand_w),
// beside it tiles X into `xt` when the GEMM follows (run_gemm); without the
// expansion (a prepared weight in `w`) the GEMM reads X straight from Xq: no
// layout launch runs then, while the main loop is faster on the tiled copy
// (about 4% for the wide tile, 5-10% for the square ones), which otherwise
// rides beside the expansion for about 1.4 us at the prefill shape.
static hipError_t gemm_parts(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const uint8_t* codes,
                             const uint8_t* meta, const float* s_w, int64_t R, int n, int m, void* Y, sbn_dtype ydt,
                             int64_t ldy, uint8_t* w, uint8_t* xt, bool expand_w, bool run_gemm, hipStream_t st) {
  const bool dx = !expand_w, tile_x = expand_w && run_gemm;
  if (dx) xt = (uint8_t*)Xq;
  const int64_t RB = gemm_rb(R), KBn = cdiv(K, 128), TBp = tile_x ? gemm_tbp(T) : 0, KC = 2 * KBn;
  const GemmWs g = gemm_ws(T, R, K, n, m);
  const XTileArgs xa{Xq, T, K, TBp, KC, (uint4*)xt};
  const int64_t nbx = tile_x ? TBp * cdiv(KC, 4) : 0;          // X tiling blocks (16 tokens x 256 K bytes)
  const int64_t cplane = round_up(R * (K * n / (4 * m)), 16);  // readable bytes of the codes plane
  hipError_t e;
  if (gemm_uses_smfmac(n, m)) {
    uint8_t* vals = w;
    uint32_t* idx = (uint32_t*)(w + g.w_bytes);
    const int64_t nbw = expand_w ? cdiv((RB / 4) * KBn * 64, 256) : 0;
    if (nbw + nbx > 0) {
      SBN_LAUNCH("layout_sparse", layout_sparse_kernel, dim3((unsigned)(nbw + nbx)), dim3(256), 0, st,
                 codes, meta, R, K, n, m, RB, KBn, cplane, vals, idx, nbw, xa);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (!run_gemm) return hipSuccess;
    return dx ? launch_gemm_t<true, true>(vals, (const uint8_t*)idx, xt, s_x, s_w, T, K, R, KBn, Y, ydt, ldy, st)
              : launch_gemm_t<true, false>(vals, (const uint8_t*)idx, xt, s_x, s_w, T, K, R, KBn, Y, ydt, ldy, st);
  }
  const int64_t KD = 2 * KBn;
  int64_t nbw = expand_w ? cdiv(RB * KD * 64, 256) : 0;
  if (nbw > 1024) nbw = 1024;                              // four blocks per CU, each table built once
  const uint8_t* mp = (n == m) ? nullptr : meta;
  if (nbw + nbx > 0) {
    const dim3 lgrid((unsigned)(nbw + nbx)), lblock(256);
#define SBN_LD_CASE(MM, NN)                                                                                  \
  else if (m == MM && n == NN) SBN_LAUNCH("layout_dense", (layout_dense_kernel<MM, NN>), lgrid, lblock, 0, st, \
                                          codes, mp, R, K, RB, KD, cplane, w, nbw, xa);
    if (false) {
    }
    SBN_LD_CASE(4, 3) SBN_LD_CASE(4, 4)
    SBN_LD_CASE(8, 3) SBN_LD_CASE(8, 4) SBN_LD_CASE(8, 5) SBN_LD_CASE(8, 6) SBN_LD_CASE(8, 7) SBN_LD_CASE(8, 8)
#undef SBN_LD_CASE
    else return hipErrorInvalidValue;
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!run_gemm) return hipSuccess;
  return dx ? launch_gemm_t<false, true>(w, nullptr, xt, s_x, s_w, T, K, R, KBn, Y, ydt, ldy, st)
            : launch_gemm_t<false, false>(w, nullptr, xt, s_x, s_w, T, K, R, KBn, Y, ydt, ldy, st);
}

// The one-call forward writes the GEMM's weight operand from pass 2 of the pack
// (and skips the layout launch) where the GEMM then runs on the wide tiles:
// 2:4 without flags; the wide kernel reads the activations in place.
bool forward_writes_operand(int64_t T, int64_t R, int64_t K, int n, int m, uint32_t flags) {
  return n == 2 && m == 4 && flags == 0 && gemm_use_wide(T, R, cdiv(K, (int64_t)128));
}

size_t gemm_operand_idx_offset(int64_t R, int64_t K, int n, int m) { return gemm_ws(1, R, K, n, m).w_bytes; }

size_t gemm_weight_bytes(int64_t R, int64_t K, int n, int m) {
  const GemmWs g = gemm_ws(1, R, K, n, m);
  return g.w_bytes + g.i_bytes;
}

// the GEMM on a prepared weight reads the activations in place
size_t gemm_x_bytes(int64_t, int64_t, int, int) { return 0; }

hipError_t launch_gemm(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                       const uint8_t* codes, const uint8_t* meta, const float* s_w, int64_t R,
                       int n, int m, void* Y, sbn_dtype ydt, int64_t ldy, void* ws, hipStream_t st) {
  const GemmWs g = gemm_ws(T, R, K, n, m);
  uint8_t* w = (uint8_t*)ws;
  return gemm_parts(Xq, s_x, T, K, codes, meta, s_w, R, n, m, Y, ydt, ldy, w, w + g.w_bytes + g.i_bytes, true, true,
                    st);
}

hipError_t launch_prepare_gemm_weight(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, int n, int m,
                                      uint8_t* prepared, hipStream_t st) {
  return gemm_parts(nullptr, nullptr, 0, K, codes, meta, nullptr, R, n, m, nullptr, SBN_BF16, 0, prepared, nullptr,
                    true, false, st);
}

hipError_t launch_gemm_prepared(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const uint8_t* prepared,
                                const float* s_w, int64_t R, int n, int m, void* Y, sbn_dtype ydt, int64_t ldy,
                                void* ws, hipStream_t st) {
  return gemm_parts(Xq, s_x, T, K, nullptr, nullptr, s_w, R, n, m, Y, ydt, ldy, (uint8_t*)prepared, nullptr,
                    false, true, st);
}

}  // namespace sbn
