// Decode GEMV (1 <= T <= 16): Y[t,r] = s_w * s_x[t] * sum_k Xq[t,k] * Wt[r,k],
// streaming the packed weight once and unpacking it in registers.
//
// The pages measure decode on a custom sparse kernel ("Sparse-BitNet",
// gist.science Japanese "技術概要" §3.2: B200 decode; Korean "기술 요약" §4).
// Here a sixteen-wide int8 matrix instruction takes 16 weight rows against
// the (up to) 16 tokens, so the arithmetic is never the limit; the cost is
// reading the packed planes and turning them into int8 operands.
//
// Work split: a block (4 waves) handles groups of 16 output rows, walking the
// row groups with a grid stride (the decode table below is built once per
// block).  K is cut into ranges of 1024 positions; a wave takes ranges wave,
// wave+4, ...  The K order inside a range is free (a dot product does not
// care), so every lane group g = l/16 owns one contiguous run of the range,
// which makes its meta and code bits one contiguous read of up to 64 bytes;
// the matrix instruction only needs A lane (r, g) and B lane (t, g) to name
// the same positions, and the activation bytes of each B lane are picked to
// match.  The waves' 16 x 16 partial sums are added in LDS.
//
//   2:4   v_smfmac_i32_16x16x128_i8: up to eight steps of 128 positions per
//         range; lane group g's run is 32 positions per step.  Each 32-bit
//         meta word (8 groups) and the matching 32-bit code word (2 survivors
//         x 2 bits per group) become the 16 compressed int8 values and the
//         2-bit position indices with a few shifts and masks (no table).
//   other v_mfma_i32_16x16x64_i8: up to sixteen steps of 64 positions per
//         range, W expanded to int8 {-1, 0, +1} through a 4096-entry table in
//         LDS that maps (4 meta bits, the next 8 code bits) to the four weights
//         of those positions (unused code bits are ignored); each block
//         computes the table while its first loads are in flight.
#include "sbn_decode.h"

namespace sbn {
namespace {

#ifndef SBN_GV_WAVES
#define SBN_GV_WAVES 4
#endif
constexpr int GV_WAVES = SBN_GV_WAVES;  // waves per block
constexpr int GV_RANGE = 4096 / GV_WAVES;   // K positions per wave range
static_assert(GV_RANGE % 128 == 0 && GV_WAVES * 256 <= 4096, "GEMV range");
constexpr int GV_MAX_BLOCKS = 2048;    // grid-stride cap (8 blocks per CU)

// add the waves' 16 x 16 partial sums in LDS and write rows x tokens; thread
// tid < 256 writes element tid (token (tid/4)%16), whose scale sxo it loaded early
template <int OUT>
__device__ inline void gemv_finish(int (*red)[256], v4i acc, int tid, int wave, int lane, int64_t row0,
                                   int64_t T, int64_t R, float sc, void* Y, int64_t ldy) {
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][lane * 4 + v] = acc[v];
  __syncthreads();
  if (tid < 256) {
    const int e = tid;
    int s = 0;
#pragma unroll
    for (int w = 0; w < GV_WAVES; ++w) s += red[w][e];
    const int L = e >> 2, v = e & 3;
    const int64_t row = row0 + 4 * (L >> 4) + v;
    const int64_t t = L & 15;
    if (t < T && row < R) {
      if (OUT == 0) {
        ((int*)Y)[t * ldy + row] = s;
      } else {
        const float y = (float)s * sc;
        if (OUT == 1) ((float*)Y)[t * ldy + row] = y;
        else ((uint16_t*)Y)[t * ldy + row] = f32_to_bf16_rne(y);
      }
    }
  }
  __syncthreads();                                     // red is reused by the next row group
}

// s_w * s_x[t] for the output element this thread writes in gemv_finish
template <int OUT>
__device__ inline float gemv_out_scale(int tid, int64_t T, const float* s_x, const float* s_w) {
  const int64_t t = (tid >> 2) & 15;
  return (OUT != 0 && tid < 256 && t < T) ? *s_w * s_x[t] : 0.0f;
}

// ----------------------------------------------------------------------------- 2:4
// Range of 128*S positions (S <= SMAX steps); lane group g's run is positions
// kbeg + 32*S*g + [0, 32*S), i.e. one meta word and one code word per step.
// Step s maps the instruction's logical K index q (0..127) to position
// kbeg + 32*S*(q/32) + 32*s + q%32.
template <int OUT>
__global__ __launch_bounds__(64 * GV_WAVES) void gemv24_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ s_x, int64_t T, int64_t K,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta, const float* __restrict__ s_w,
    int64_t R, void* __restrict__ Y, int64_t ldy) {
  constexpr int SMAX = GV_RANGE / 128;
  __shared__ int red[GV_WAVES][256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, rl = lane & 15;
  const bool tvalid = rl < T;
  const int8_t* xrow = Xq + (tvalid ? rl : 0) * K;
  const int64_t nranges = cdiv(K, GV_RANGE), nrg = cdiv(R, 16);
  const int gb2 = g >> 1, gb1 = g & 1;
  const float sc = gemv_out_scale<OUT>(tid, T, s_x, s_w);

  // packed words of the lane group's run in range ri of row group rg (2:4: the
  // meta and code planes both hold one bit per position)
  auto load_w = [&](int64_t rg, int64_t ri, int S, uint32_t (&mw)[SMAX], uint32_t (&cw)[SMAX]) {
    const int64_t r = rg * 16 + rl;
    const int64_t rr = r < R ? r : R - 1;             // rows past R: computed on row R-1, discarded
    const uint32_t* mrow = (const uint32_t*)(meta + rr * (K / 8));
    const uint32_t* crow = (const uint32_t*)(codes + rr * (K / 8));
    const int64_t w0 = ri * (GV_RANGE / 32) + (int64_t)S * g;
    if (SMAX % 4 == 0 && S == SMAX) {
#pragma unroll
      for (int h = 0; h < SMAX / 4; ++h) {
        const v4i x = *(const v4i*)(mrow + w0 + 4 * h), y = *(const v4i*)(crow + w0 + 4 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) { mw[4 * h + i] = (uint32_t)x[i]; cw[4 * h + i] = (uint32_t)y[i]; }
      }
    } else {
#pragma unroll
      for (int i = 0; i < SMAX; ++i) {
        mw[i] = i < S ? mrow[w0 + i] : 0u;
        cw[i] = i < S ? crow[w0 + i] : 0u;
      }
    }
  };
  auto load_x = [&](int64_t ri, int S, v4i (&blo)[SMAX], v4i (&bhi)[SMAX]) {
    const int64_t kbeg = ri * GV_RANGE;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const int64_t lo = kbeg + 32 * (int64_t)S * gb2 + 32 * s + 16 * gb1;
      const bool ok = tvalid && s < S;
      blo[s] = ok ? *(const v4i*)(xrow + lo) : (v4i){0, 0, 0, 0};
      bhi[s] = ok ? *(const v4i*)(xrow + lo + 64 * (int64_t)S) : (v4i){0, 0, 0, 0};
    }
  };
  auto steps = [&](int S, const uint32_t (&mw)[SMAX], const uint32_t (&cw)[SMAX], const v4i (&blo)[SMAX],
                   const v4i (&bhi)[SMAX], v4i acc) {
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      if (s < S) {
        v4i a;
        int ix;
        decode24(mw[s], cw[s], a, ix);
        const v8i b = (v8i){blo[s][0], blo[s][1], blo[s][2], blo[s][3], bhi[s][0], bhi[s][1], bhi[s][2], bhi[s][3]};
        acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, acc, ix, 0, 0);
      }
    }
    return acc;
  };
  auto range_steps = [&](int64_t ri) {
    const int S = (int)((K - ri * GV_RANGE) / 128 < SMAX ? (K - ri * GV_RANGE) / 128 : SMAX);
    return S;
  };

  if (nranges <= GV_WAVES) {
    // K fits one range per wave: the activations stay in registers for every
    // row group, and the next row group's packed words load during this one's math
    const bool has = wave < nranges;
    const int S = has ? range_steps(wave) : 0;
    v4i blo[SMAX], bhi[SMAX];
    load_x(wave, S, blo, bhi);
    uint32_t mw[SMAX], cw[SMAX];
    int64_t rg = blockIdx.x;
    if (has) load_w(rg, wave, S, mw, cw);
    for (; rg < nrg; rg += gridDim.x) {
      uint32_t m0[SMAX], c0[SMAX];
#pragma unroll
      for (int i = 0; i < SMAX; ++i) { m0[i] = mw[i]; c0[i] = cw[i]; }
      if (has && rg + gridDim.x < nrg) load_w(rg + gridDim.x, wave, S, mw, cw);
      const v4i acc = steps(S, m0, c0, blo, bhi, (v4i){0, 0, 0, 0});
      gemv_finish<OUT>(red, acc, tid, wave, lane, rg * 16, T, R, sc, Y, ldy);
    }
  } else {
    for (int64_t rg = blockIdx.x; rg < nrg; rg += gridDim.x) {
      v4i acc = (v4i){0, 0, 0, 0};
      for (int64_t ri = wave; ri < nranges; ri += GV_WAVES) {
        const int S = range_steps(ri);
        uint32_t mw[SMAX], cw[SMAX];
        v4i blo[SMAX], bhi[SMAX];
        load_w(rg, ri, S, mw, cw);
        load_x(ri, S, blo, bhi);
        acc = steps(S, mw, cw, blo, bhi, acc);
      }
      gemv_finish<OUT>(red, acc, tid, wave, lane, rg * 16, T, R, sc, Y, ldy);
    }
  }
}

// ----------------------------------------------------------------------------- 2:4, streamed
// K a multiple of 1024, at most 4096: wave w owns positions [1024w, 1024w + 1024)
// of every row (eight steps of 128, lane group g's run = meta and code words
// 8g .. 8g + 7 of the range) and walks the block's row groups.  The packed
// words of the next GV_RING - 1 row groups stream into a ring in LDS that only
// this wave uses, by direct global->LDS loads: several row groups are in
// flight per wave without holding registers, and no load waits behind the math.
// Ring slot: 16 rows x 128 B of meta, then the same of codes; 16-byte chunk c
// of row r sits at chunk position c ^ (r & 7), so the eight lanes that read one
// chunk position of eight rows touch eight different banks, and each 1 KB load
// instruction still reads whole 128-byte row segments.  Survivor values are
// decoded as 64 * w, so the partial sums are 64 times the accumulator.
#ifndef SBN_GV_RING
#define SBN_GV_RING 3
#endif
constexpr int GV_RING = SBN_GV_RING;
#ifndef SBN_GV_STREAM
#define SBN_GV_STREAM 1
#endif
constexpr int GV_STREAM_BLOCKS = 512;  // two blocks per CU

template <int OUT>
__global__ __launch_bounds__(256, 2) void gemv24s_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ s_x, int64_t T, int64_t K,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ meta, const float* __restrict__ s_w,
    int64_t R, void* __restrict__ Y, int64_t ldy) {
  // one LDS array: [4 waves][GV_RING slots][4096 B] ring, then red[2][4][256] ints
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * GV_RING * 4096 + 2 * 4 * 256 * 4];
  uint8_t (*ring)[GV_RING][4096] = (uint8_t (*)[GV_RING][4096])lds;
  int (*red)[4][256] = (int (*)[4][256])(lds + 4 * GV_RING * 4096);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, rl = lane & 15;
  const int64_t nrg = cdiv(R, 16), rowb = K / 8;
  const bool has = wave < K / 1024;                    // wave-uniform
  // scales of the output element this thread writes (token (tid / 4) % 16); the
  // loads are unconditional so nothing waits for them before the loop
  const int64_t tq = (tid >> 2) & 15;
  const float sxv = OUT != 0 ? s_x[tq < T ? tq : 0] : 0.0f;
  const float swv = OUT != 0 ? *s_w : 0.0f;
  uint8_t* myring = &ring[wave][0][0];

  // direct loads of one row group into ring slot `slot`: instruction q of a
  // plane fills chunk positions 64q + lane (row (64q + lane) / 8)
  auto issue = [&](int64_t rg, int slot) {
    uint8_t* dst = myring + slot * 4096;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int sp = 64 * q + lane, rr = sp >> 3, ch = (sp & 7) ^ (rr & 7);
      int64_t r = rg * 16 + rr;
      r = r < R ? r : R - 1;                           // rows past R: row R-1, discarded
      const int64_t off = r * rowb + 128 * wave + 16 * ch;
      g2lds16(meta + off, dst + 1024 * q);
      g2lds16(codes + off, dst + 2048 + 1024 * q);
    }
  };

  int64_t rg = blockIdx.x;
  const int64_t gs = gridDim.x;
  if (has) {
#pragma unroll
    for (int i = 0; i < GV_RING - 1; ++i)
      if (rg + i * gs < nrg) issue(rg + i * gs, i);
  }
  // activations of this wave's range, kept in registers (as gemv24 with S = 8)
  const bool tvalid = rl < T;
  const int8_t* xrow = Xq + (tvalid ? rl : 0) * K;
  v4i blo[8], bhi[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int64_t lo = 1024 * wave + 256 * (g >> 1) + 32 * s + 16 * (g & 1);
    const bool ok = has && tvalid;
    blo[s] = ok ? *(const v4i*)(xrow + lo) : (v4i){0, 0, 0, 0};
    bhi[s] = ok ? *(const v4i*)(xrow + lo + 512) : (v4i){0, 0, 0, 0};
  }
  // make the activations (and with them the first ring slots) resident before
  // the loop, whose only global loads are the counted ring loads
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(blo[s]), "v"(bhi[s]));

  // row groups of this block: rg = blockIdx.x + i * gs, i < nit
  const int nit = rg < nrg ? (int)((nrg - 1 - rg) / gs) + 1 : 0;
  int slot = 0, par = 0;
  for (int it = 0; it < nit; ++it, rg += gs) {
    v4i acc = (v4i){0, 0, 0, 0};
    if (has) {
      if (it + GV_RING - 1 < nit) issue(rg + (GV_RING - 1) * gs, (slot + GV_RING - 1) % GV_RING);
      // this slot's loads are done once at most 4 per later row group remain
      const int later = nit - 1 - it;
      if (later >= GV_RING - 1) wait_vmcnt<4 * (GV_RING - 1)>();
      else if (GV_RING > 3 && later == 2) wait_vmcnt<8>();
      else if (later == 1) wait_vmcnt<4>();
      else wait_vmcnt<0>();
      const uint8_t* sl = myring + slot * 4096 + rl * 128;
      const int c0 = (2 * g) ^ (rl & 7), c1 = (2 * g + 1) ^ (rl & 7);
      const v4i m0 = *(const v4i*)(sl + 16 * c0), m1 = *(const v4i*)(sl + 16 * c1);
      const v4i k0 = *(const v4i*)(sl + 2048 + 16 * c0), k1 = *(const v4i*)(sl + 2048 + 16 * c1);
      const uint32_t mw[8] = {(uint32_t)m0[0], (uint32_t)m0[1], (uint32_t)m0[2], (uint32_t)m0[3],
                              (uint32_t)m1[0], (uint32_t)m1[1], (uint32_t)m1[2], (uint32_t)m1[3]};
      const uint32_t cw[8] = {(uint32_t)k0[0], (uint32_t)k0[1], (uint32_t)k0[2], (uint32_t)k0[3],
                              (uint32_t)k1[0], (uint32_t)k1[1], (uint32_t)k1[2], (uint32_t)k1[3]};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        v4i a;
        int ix;
        decode24_x64(mw[s], cw[s], a, ix);
        const v8i b = (v8i){blo[s][0], blo[s][1], blo[s][2], blo[s][3], bhi[s][0], bhi[s][1], bhi[s][2], bhi[s][3]};
        acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, acc, ix, 0, 0);
      }
      slot = slot + 1 == GV_RING ? 0 : slot + 1;
    }
    // partial sums of the four waves, double-buffered so one barrier per row group suffices
    *(v4i*)&red[par][wave][lane * 4] = acc;
    lds_barrier();
    {
      const int e = tid;
      const int s64 = red[par][0][e] + red[par][1][e] + red[par][2][e] + red[par][3][e];
      const int sum = s64 >> 6;                        // exact: every partial is a multiple of 64
      const int L = e >> 2, v = e & 3;
      const int64_t row = rg * 16 + 4 * (L >> 4) + v;
      const int64_t t = L & 15;
      if (t < T && row < R) {
        if (OUT == 0) {
          ((int*)Y)[t * ldy + row] = sum;
        } else {
          const float y = (float)sum * (swv * sxv);
          if (OUT == 1) ((float*)Y)[t * ldy + row] = y;
          else ((uint16_t*)Y)[t * ldy + row] = f32_to_bf16_rne(y);
        }
      }
    }
    par ^= 1;
  }
}

// ----------------------------------------------------------------------------- table path
// Range of 64*S positions (S <= SMAX steps); lane group g's run is positions
// p0 = kbeg + 16*S*g + [0, 16*S); step j takes positions p0 + 16*j .. +16 as
// A lane (r, g) and the same activation bytes as B lane (t, g).
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
  const bool tvalid = rl < T;
  const int8_t* xrow = Xq + (tvalid ? rl : 0) * K;
  const int64_t crow_bytes = K * N / (4 * M);
  const int64_t nranges = cdiv(K, GV_RANGE), nrg = cdiv(R, 16);
  const float sc = gemv_out_scale<OUT>(tid, T, s_x, s_w);

  // packed bits of the lane group's run in range ri of row group rg: meta
  // words (16 bits per step) and the code words that cover the run, as read
  // (aligned down to 4 bytes; `sh` is the bit offset of the run in raw[0])
  struct Packed {
    uint32_t mw[SMAX / 2];
    uint32_t raw[NWC + 1];
    int sh;
  };
  auto load_w = [&](int64_t rg, int64_t ri, int S, Packed& P) {
    const int64_t r = rg * 16 + rl;
    const int64_t rr = r < R ? r : R - 1;             // rows past R: computed on row R-1, discarded
    const int64_t p0 = ri * GV_RANGE + 16 * (int64_t)g * S;
#pragma unroll
    for (int i = 0; i < SMAX / 2; ++i) P.mw[i] = 0;
    if (N < M && S > 0) {
      const uint8_t* mrow = meta + rr * (K / 8);
      if ((S & 1) == 0) {                              // run starts on a 4-byte boundary
        const uint32_t* mp = (const uint32_t*)(mrow + p0 / 8);
#pragma unroll
        for (int i = 0; i < SMAX / 2; ++i)
          if (2 * i < S) P.mw[i] = mp[i];
      } else {
        const uint16_t* mh = (const uint16_t*)(mrow + p0 / 8);
#pragma unroll
        for (int i = 0; i < SMAX; ++i)
          if (i < S) P.mw[i >> 1] |= (uint32_t)mh[i] << (16 * (i & 1));
      }
    }
    const int64_t cbit = CB_NUM * (p0 / M);
    const uintptr_t ca = (uintptr_t)(codes + rr * crow_bytes + (cbit >> 3));
    const uint32_t* cw4 = (const uint32_t*)(ca & ~(uintptr_t)3);
    P.sh = (int)((ca & 3) * 8 + (cbit & 7));
    const int nbits = 32 * N * S / M;
    const int nd = S > 0 ? (P.sh + nbits + 31) >> 5 : 0;
#pragma unroll
    for (int i = 0; i < NWC + 1; ++i) P.raw[i] = (i < nd) ? cw4[i] : 0u;
  };
  auto load_x = [&](int64_t ri, int S, v4i (&bx)[SMAX]) {
    const int64_t p0 = ri * GV_RANGE + 16 * (int64_t)g * S;
#pragma unroll
    for (int j = 0; j < SMAX; ++j)
      bx[j] = (tvalid && j < S) ? *(const v4i*)(xrow + p0 + 16 * j) : (v4i){0, 0, 0, 0};
  };
  auto steps = [&](int S, const Packed& P, const v4i (&bx)[SMAX], v4i acc) {
    uint32_t cw[NWC];
#pragma unroll
    for (int i = 0; i < NWC; ++i) cw[i] = __builtin_amdgcn_alignbit(P.raw[i + 1], P.raw[i], P.sh);
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
      if (j < S) {
        uint32_t e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int pos = 16 * j + 4 * k;                        // position within the run
          const uint32_t nib = (N < M) ? ((P.mw[pos >> 5] >> (pos & 31)) & 0xFu) : 0xFu;
          uint32_t c8;
          if (M == 4) {
            c8 = bits_at<NWC>(cw, (int)CB_NUM * (pos / 4), 8);
          } else {
            const int gi = pos / 8;
            const uint32_t gb = bits_at<NWC>(cw, (int)CB_NUM * gi, 24);
            if ((k & 1) == 0) {
              c8 = gb & 0xFFu;
            } else {
              const uint32_t low = (N < M) ? ((P.mw[(pos - 4) >> 5] >> ((pos - 4) & 31)) & 0xFu) : 0xFu;
              c8 = (gb >> (2 * __builtin_popcount(low))) & 0xFFu;
            }
          }
          e[k] = lut[nib | (c8 << 4)];
        }
        const v4i a = (v4i){(int)e[0], (int)e[1], (int)e[2], (int)e[3]};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bx[j], acc, 0, 0, 0);
      }
    }
    return acc;
  };
  auto range_steps = [&](int64_t ri) {
    const int64_t left = (K - ri * GV_RANGE) / 64;
    return (int)(left < SMAX ? left : SMAX);
  };

  if (nranges <= GV_WAVES) {
    // one range per wave: activations stay in registers for every row group,
    // and the next row group's packed bits load during this one's math
    const bool has = wave < nranges;
    const int S = has ? range_steps(wave) : 0;
    v4i bx[SMAX];
    load_x(wave, S, bx);
    Packed P;
    int64_t rg = blockIdx.x;
    load_w(rg, wave, S, P);
    for (int i = tid; i < 4096; i += 64 * GV_WAVES) lut[i] = unpack_entry((uint32_t)i);   // while loads fly
    __syncthreads();
    for (; rg < nrg; rg += gridDim.x) {
      const Packed cur = P;
      if (rg + gridDim.x < nrg) load_w(rg + gridDim.x, wave, S, P);
      const v4i acc = steps(S, cur, bx, (v4i){0, 0, 0, 0});
      gemv_finish<OUT>(red, acc, tid, wave, lane, rg * 16, T, R, sc, Y, ldy);
    }
  } else {
    for (int i = tid; i < 4096; i += 64 * GV_WAVES) lut[i] = unpack_entry((uint32_t)i);
    __syncthreads();
    for (int64_t rg = blockIdx.x; rg < nrg; rg += gridDim.x) {
      v4i acc = (v4i){0, 0, 0, 0};
      for (int64_t ri = wave; ri < nranges; ri += GV_WAVES) {
        const int S = range_steps(ri);
        Packed P;
        v4i bx[SMAX];
        load_w(rg, ri, S, P);
        load_x(ri, S, bx);
        acc = steps(S, P, bx, acc);
      }
      gemv_finish<OUT>(red, acc, tid, wave, lane, rg * 16, T, R, sc, Y, ldy);
    }
  }
}

template <int N, int M>
hipError_t launch_gemv_nm(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                          const uint8_t* codes, const uint8_t* meta, const float* s_w, int64_t R,
                          void* Y, sbn_dtype ydt, int64_t ldy, hipStream_t st) {
  const int64_t nrg = cdiv(R, 16);
  const dim3 grid((unsigned)(nrg < GV_MAX_BLOCKS ? nrg : GV_MAX_BLOCKS)), block(64 * GV_WAVES);
  const uint8_t* mp = (N == M) ? nullptr : meta;
  if (SBN_GV_STREAM && N == 2 && M == 4 && K % 1024 == 0 && K <= 4096) {
    const dim3 sgrid((unsigned)(nrg < GV_STREAM_BLOCKS ? nrg : GV_STREAM_BLOCKS)), sblock(256);
    if (ydt == SBN_I32_ACC)
      SBN_LAUNCH("gemv", gemv24s_kernel<0>, sgrid, sblock, 0, st, Xq, s_x, T, K, codes, mp, s_w, R, Y, ldy);
    else if (ydt == SBN_F32)
      SBN_LAUNCH("gemv", gemv24s_kernel<1>, sgrid, sblock, 0, st, Xq, s_x, T, K, codes, mp, s_w, R, Y, ldy);
    else
      SBN_LAUNCH("gemv", gemv24s_kernel<2>, sgrid, sblock, 0, st, Xq, s_x, T, K, codes, mp, s_w, R, Y, ldy);
    return hipGetLastError();
  }
  if (N == 2 && M == 4 && K % 128 == 0) {
    if (ydt == SBN_I32_ACC)
      SBN_LAUNCH("gemv", gemv24_kernel<0>, grid, block, 0, st, Xq, s_x, T, K, codes, mp, s_w, R, Y, ldy);
    else if (ydt == SBN_F32)
      SBN_LAUNCH("gemv", gemv24_kernel<1>, grid, block, 0, st, Xq, s_x, T, K, codes, mp, s_w, R, Y, ldy);
    else
      SBN_LAUNCH("gemv", gemv24_kernel<2>, grid, block, 0, st, Xq, s_x, T, K, codes, mp, s_w, R, Y, ldy);
    return hipGetLastError();
  }
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
