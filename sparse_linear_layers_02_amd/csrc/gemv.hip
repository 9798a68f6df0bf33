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
#include <type_traits>
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

// ----------------------------------------------------------------------------- streamed decode
// For 2:4 and 6:8 with K a multiple of 1024, at most 4096.  Wave w of a block
// owns positions [1024w, 1024w + 1024) of every row and keeps the activations
// of that range in registers; a block walks consecutive row groups (16 rows)
// of one or more weights that share the activations.  The packed words of the
// next GV_RING - 1 row groups stream into a ring in LDS that only this wave
// uses, by direct global->LDS loads: several row groups are in flight per wave
// without holding registers, and no load waits behind the math.  Survivor
// values are decoded as 64 * w (the code in the top two bits of its byte), so
// the partial sums are 64 times the accumulator.
#ifndef SBN_GV_RING
#define SBN_GV_RING 2
#endif
constexpr int GV_RING = SBN_GV_RING;
#ifndef SBN_GV_STREAM
#define SBN_GV_STREAM 1
#endif

// The weights of one streamed launch: either up to GV_MAX_BATCH entries by
// value in the kernel argument, or a table of any length in device memory
// that the caller fills once and reuses.  Both index as P.e[w]; the kernel
// reads an entry with wave-uniform (scalar) loads.
static_assert(sizeof(GvEntry) == 32 && alignof(GvEntry) == 8, "GvEntry: four device pointers");
struct GemvBatch {
  GvEntry e[GV_MAX_BATCH];
};
struct GemvTable {
  const GvEntry* e;
};
// Entry w and a weight's scale, read through the constant address space: the
// table and the scales stay unchanged while the kernel runs, so the loads are
// scalar (the scalar cache; no wait on the ring's vector loads).
typedef const __attribute__((address_space(4))) uint64_t* U64C;
typedef const __attribute__((address_space(4))) float* FloatC;
__device__ inline GvEntry gv_entry(const GemvBatch& P, int64_t w) { return P.e[w]; }
__device__ inline GvEntry gv_entry(const GemvTable& P, int64_t w) {
  const U64C q = (U64C)(P.e + w);
  return GvEntry{(const uint8_t*)q[0], (const uint8_t*)q[1], (const float*)q[2], (void*)q[3]};
}
__device__ inline float gv_scale(const float* s_w) { return *(FloatC)s_w; }

// Sum of the four 16-byte words at p, p + 1 KB, p + 2 KB and p + 3 KB of LDS,
// read in one asm block that also waits for them.  Through the compiler's own
// LDS reads, each sum waited for every direct global->LDS load in flight
// (the compiler cannot tell the ring's loads from these reads), which drained
// the ring once per row group.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ inline v4i lds_sum4_1k(const int* p) {
  const uint32_t a = lds_addr(p);
  v4i x0, x1, x2, x3;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "ds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
      : "v"(a)
      : "memory");
  return x0 + x1 + x2 + x3;
}

// A ring slot's words into registers, the same way: four or five 16-byte
// reads at the given LDS addresses, waited for in the block, so the slot can
// be refilled right after.
__device__ inline void lds_read4(v4i& x0, v4i& x1, v4i& x2, v4i& x3, uint32_t a0, uint32_t a1, uint32_t a2,
                                 uint32_t a3) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}
__device__ inline void lds_read3(v4i& x0, v4i& x1, v4i& x2, uint32_t a0, uint32_t a1, uint32_t a2) {
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %4\n\t"
      "ds_read_b128 %2, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2)
      : "v"(a0), "v"(a1), "v"(a2)
      : "memory");
}
__device__ inline void lds_read5(v4i& x0, v4i& x1, v4i& x2, v4i& x3, v4i& x4, uint32_t a0, uint32_t a1,
                                 uint32_t a2, uint32_t a3, uint32_t a4) {
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %6\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %8\n\t"
      "ds_read_b128 %4, %9\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(x4)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(a4)
      : "memory");
}

// Output side.  Row groups 4k .. 4k + 3 of a weight (64 rows) form one output
// group.  Per row group the four waves' 16 x 16 partial sums go through red
// (one of two buffers, alternating per row group, so one barrier per row group
// suffices).  Thread (r = tid / 16, t = tid % 16) owns rows 4r .. 4r + 3 of
// its output group for token t: it sums them (16 contiguous bytes of each
// wave's partials) after row group r / 4 of the group and keeps them in
// registers; once the group is complete they are stored together.  Row group
// j of a group is summed by wave j (threads 64j .. 64j + 63), so the four
// waves share the summing whatever the number of tokens, and each wave stores
// one 32- or 64-byte run (16 rows) per token.
template <int OUT>
struct StreamOut {
  v4i v;                                               // this lane's four outputs (bf16: v[0..1] packed)
  int64_t prow = -1;                                   // first row of a pending store (-1: none)
  void* pY = nullptr;
  // j: place of the row group in its output group; j0: the first place this
  // block fills in that group; done: the group is complete for this block.
  // The stores are only recorded here and issued by commit(), which the kernel
  // calls right after its next wait for ring loads (stores count in the same
  // vmcnt as the ring loads).
  __device__ inline void row_group(int (*red)[256], v4i acc, int tid, int wave, int lane, int j, int j0, bool done,
                                   int64_t grp_row0, int64_t T, float swv, float sxv, void* Y) {
    *(v4i*)&red[wave][lane * 4] = acc;
    lds_barrier();
    const int r = tid >> 4, t = tid & 15;
    if ((r >> 2) == j && t < T) {
      // rows 4 (r % 4) .. +3 of this row group: entries 64 (r % 4) + 4 t + 0..3 of every wave's partials
      const int e = 64 * (r & 3) + 4 * t;
      const v4i a = lds_sum4_1k(&red[0][e]);
      const v4i sum = a >> 6;                          // exact: every partial is a multiple of 64
      if (OUT == 0) {
        v = sum;
      } else {
        const float sc = swv * sxv;
        float y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) y[q] = (float)sum[q] * sc;
        if (OUT == 1) {
          v = (v4i){(int)__float_as_uint(y[0]), (int)__float_as_uint(y[1]), (int)__float_as_uint(y[2]), (int)__float_as_uint(y[3])};
        } else {
          v[0] = (int)((uint32_t)f32_to_bf16_rne(y[0]) | ((uint32_t)f32_to_bf16_rne(y[1]) << 16));
          v[1] = (int)((uint32_t)f32_to_bf16_rne(y[2]) | ((uint32_t)f32_to_bf16_rne(y[3]) << 16));
        }
      }
    }
    if (done && (r >> 2) >= j0 && (r >> 2) <= j && t < T) {
      prow = grp_row0 + 4 * r;
      pY = Y;
    }
  }
  // Y through global-space pointers: a generic (flat) store would have to
  // wait for the ring's in-flight loads into LDS, which it might alias.
  typedef __attribute__((address_space(1))) uint16_t* GU16;
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(1))) v2u* GU2;
  typedef __attribute__((address_space(1))) int* GI32;
  typedef __attribute__((address_space(1))) v4i* GV4;
  __device__ inline void commit(int tid, int64_t R, int64_t ldy) {
    if (prow < 0) return;
    const int64_t row = prow, t = tid & 15;
    prow = -1;
    if (OUT == 2) {
      const GU16 y = (GU16)pY + t * ldy + row;
      if (row + 4 <= R) {
        *(GU2)y = (v2u){(uint32_t)v[0], (uint32_t)v[1]};
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (row + q < R) y[q] = (uint16_t)((uint32_t)v[q >> 1] >> (16 * (q & 1)));
      }
    } else {
      const GI32 y = (GI32)pY + t * ldy + row;
      if (row + 4 <= R) {
        *(GV4)y = v;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (row + q < R) y[q] = v[q];
      }
    }
  }
};

// 2:4 decoder.  Range of 1024 positions = eight steps of v_smfmac_i32_16x16x128_i8;
// lane group g's run is meta and code words 8g .. 8g + 7 of the range; step s
// maps the instruction's logical K index q (0..127) to position
// 256 (q / 32) + 32 s + q % 32 of the range.  Ring slot: 16 rows x 128 B of
// meta, then the same of codes; 16-byte chunk c of row r sits at chunk
// position c ^ (r & 7), so the eight lanes that read one chunk position of
// eight rows touch eight different banks, and each 1 KB load instruction
// still reads whole 128-byte row segments.
struct Dec24 {
  static constexpr int SLOT = 4096, NDMA = 4, LUT = 0, BPC = 4;   // BPC: resident blocks per CU (40 KB LDS each)
  __host__ __device__ static int64_t meta_row(int64_t K) { return K / 8; }
  __host__ __device__ static int64_t code_row(int64_t K) { return K / 8; }
  int rowq[2], colq[2];
  v4i blo[8], bhi[8];
  __device__ inline void init(int wave, int lane) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int sp = 64 * q + lane, rr = sp >> 3;
      rowq[q] = rr;
      colq[q] = 128 * wave + 16 * ((sp & 7) ^ (rr & 7));
    }
  }
  // row group at planes (m, c); rows of the group from `valid` on read row valid - 1
  __device__ inline void issue(uint8_t* dst, const uint8_t* m, const uint8_t* c, int valid, int64_t K) {
    const int rowb = (int)(K / 8);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = rowq[q] < valid ? rowq[q] : valid - 1;
      const int off = r * rowb + colq[q];
      g2lds16(m + off, dst + 1024 * q);
      g2lds16(c + off, dst + 2048 + 1024 * q);
    }
  }
  __device__ inline void load_x(const int8_t* xrow, bool ok, int wave, int g) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int64_t lo = 1024 * wave + 256 * (g >> 1) + 32 * s + 16 * (g & 1);
      blo[s] = ok ? *(const v4i*)(xrow + lo) : (v4i){0, 0, 0, 0};
      bhi[s] = ok ? *(const v4i*)(xrow + lo + 512) : (v4i){0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(blo[s]), "v"(bhi[s]));
  }
  __device__ inline void build_lut(uint8_t*, int) {}
  struct Frag {
    v4i m0, m1, k0, k1;
  };
  // this lane's words of the slot (row rl, lane group g) into registers
  __device__ inline Frag read(const uint8_t* slot, int rl, int g) const {
    const uint32_t sl = lds_addr(slot + rl * 128);
    const uint32_t c0 = 16 * ((2 * g) ^ (rl & 7)), c1 = 16 * ((2 * g + 1) ^ (rl & 7));
    Frag f;
    lds_read4(f.m0, f.m1, f.k0, f.k1, sl + c0, sl + c1, sl + 2048 + c0, sl + 2048 + c1);
    return f;
  }
  __device__ inline v4i compute(const Frag& f, const uint8_t*) const {
    const v4i m0 = f.m0, m1 = f.m1, k0 = f.k0, k1 = f.k1;
    const uint32_t mw[8] = {(uint32_t)m0[0], (uint32_t)m0[1], (uint32_t)m0[2], (uint32_t)m0[3],
                            (uint32_t)m1[0], (uint32_t)m1[1], (uint32_t)m1[2], (uint32_t)m1[3]};
    const uint32_t cw[8] = {(uint32_t)k0[0], (uint32_t)k0[1], (uint32_t)k0[2], (uint32_t)k0[3],
                            (uint32_t)k1[0], (uint32_t)k1[1], (uint32_t)k1[2], (uint32_t)k1[3]};
    v4i acc = (v4i){0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      v4i a;
      int ix;
      decode24_x64(mw[s], cw[s], a, ix);
      const v8i b = (v8i){blo[s][0], blo[s][1], blo[s][2], blo[s][3], bhi[s][0], bhi[s][1], bhi[s][2], bhi[s][3]};
      acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, acc, ix, 0, 0);
    }
    return acc;
  }
};

// 6:8 decoder, dense v_mfma_i32_16x16x64_i8: sixteen steps of 64; lane group
// g's run is positions 256g .. 256g + 255 of the range (meta words 8g .. 8g+7,
// code words 12g .. 12g+11), step s takes positions 256g + 16s .. +16 as A lane
// (r, g) and the same activation bytes as B lane (t, g).  Ring slot: 16 rows x
// 128 B of meta (chunk c of row r at chunk position c ^ (r & 7)), then 16 rows x
// 192 B of codes (chunk c at position (c + (r & 7)) mod 12).
// Decode of one step (two groups: 16 meta bits, twelve 2-bit codes f0..f11):
// planes P_q = (codes << (6 - 2q)) & 0xC0C0C0C0 hold f_{4b+q} in byte b as
// 64 * w; one round of byte permutes gives
//   A = [f0 f1 f4 f5]  B = [f2 f3 f6 f7]  C = [f8 f9 . .]  D = [f10 f11 . .]
// and each output word (four positions) is one permute of a pair of those,
// with a selector taken from a 256-entry table indexed by the group's meta
// byte (0x0C selects a zero byte at a pruned position).
__device__ inline v4i lut68_entry(uint32_t mb) {
  // survivor rank -> byte of the permute window, per output word, one nibble
  // per rank (rank 0 lowest), so no table in memory is indexed:
  //   words 0, 1: window (lo A, hi B): 0 1 4 5 2 3
  //   word 2:     window (lo B, hi C): 2 3 4 5 12 12
  //   word 3:     window (lo C, hi D): 12 12 0 1 4 5
  constexpr uint32_t M0 = 0x325410u, M2 = 0xCC5432u, M3 = 0x5410CCu;
  uint32_t w[4] = {0, 0, 0, 0};
  uint32_t r = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const bool on = (mb >> p) & 1u;
    const uint32_t rr = r < 6 ? r : 5;
    const uint32_t a = on ? (M0 >> (4 * rr)) & 15u : 12u, b = on ? ((p < 4 ? M2 : M3) >> (4 * rr)) & 15u : 12u;
    w[p >> 2] |= a << (8 * (p & 3));
    w[2 + (p >> 2)] |= b << (8 * (p & 3));
    r += on ? 1u : 0u;
  }
  return (v4i){(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
}

struct Dec68 {
  static constexpr int SLOT = 2048 + 3072, NDMA = 5, LUT = 4096, BPC = 3;   // 52 KB LDS per block
  __host__ __device__ static int64_t meta_row(int64_t K) { return K / 8; }
  __host__ __device__ static int64_t code_row(int64_t K) { return K * 3 / 16; }
  int rowA[5], colA[5];
  v4i bx[16];
  __device__ inline void init(int wave, int lane) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {                        // meta: chunk positions 64q + lane
      const int sp = 64 * q + lane, rr = sp >> 3;
      rowA[q] = rr;
      colA[q] = 128 * wave + 16 * ((sp & 7) ^ (rr & 7));
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {                        // codes: chunk positions 64q + lane
      const int sp = 64 * q + lane, rr = sp / 12, pos = sp - 12 * rr;
      const int c = pos - (rr & 7) < 0 ? pos - (rr & 7) + 12 : pos - (rr & 7);
      rowA[2 + q] = rr;
      colA[2 + q] = 192 * wave + 16 * c;
    }
  }
  __device__ inline void issue(uint8_t* dst, const uint8_t* m, const uint8_t* c, int valid, int64_t K) {
    const int rowm = (int)(K / 8), rowc = (int)(K * 3 / 16);
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int r = rowA[q] < valid ? rowA[q] : valid - 1;
      if (q < 2) g2lds16(m + r * rowm + colA[q], dst + 1024 * q);
      else g2lds16(c + r * rowc + colA[q], dst + 2048 + 1024 * (q - 2));
    }
  }
  __device__ inline void load_x(const int8_t* xrow, bool ok, int wave, int g) {
#pragma unroll
    for (int s = 0; s < 16; ++s)
      bx[s] = ok ? *(const v4i*)(xrow + 1024 * wave + 256 * g + 16 * s) : (v4i){0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 16; ++s) asm volatile("" ::"v"(bx[s]));
  }
  __device__ inline void build_lut(uint8_t* lut, int tid) { *(v4i*)(lut + 16 * tid) = lut68_entry((uint32_t)tid); }
  struct Frag {
    v4i m0, m1, c[3];
  };
  __device__ inline Frag read(const uint8_t* slot, int rl, int g) const {
    const uint32_t sm = lds_addr(slot + rl * 128);
    const uint32_t sc = lds_addr(slot + 2048 + rl * 192);
    const int r7 = rl & 7;
    uint32_t ac[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int c = 3 * g + i + r7;
      ac[i] = sc + 16 * (c < 12 ? c : c - 12);
    }
    Frag f;
    lds_read5(f.m0, f.m1, f.c[0], f.c[1], f.c[2], sm + 16 * ((2 * g) ^ r7), sm + 16 * ((2 * g + 1) ^ r7), ac[0],
              ac[1], ac[2]);
    return f;
  }
  __device__ inline v4i compute(const Frag& f, const uint8_t* lut) const {
    const v4i m0 = f.m0, m1 = f.m1;
    uint32_t cw[12];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const v4i v = f.c[i];
      cw[4 * i] = (uint32_t)v[0]; cw[4 * i + 1] = (uint32_t)v[1]; cw[4 * i + 2] = (uint32_t)v[2]; cw[4 * i + 3] = (uint32_t)v[3];
    }
    const uint32_t mw[8] = {(uint32_t)m0[0], (uint32_t)m0[1], (uint32_t)m0[2], (uint32_t)m0[3],
                            (uint32_t)m1[0], (uint32_t)m1[1], (uint32_t)m1[2], (uint32_t)m1[3]};
    v4i acc = (v4i){0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint32_t m16 = mw[s >> 1] >> (16 * (s & 1));
      const int bo = 24 * s, wi = bo >> 5, sh = bo & 31;
      const uint32_t c = sh == 0 ? cw[wi] : __builtin_amdgcn_alignbit(cw[wi + 1 < 12 ? wi + 1 : 11], cw[wi], sh);
      const uint32_t p0 = (c << 6) & 0xC0C0C0C0u, p1 = (c << 4) & 0xC0C0C0C0u;
      const uint32_t p2 = (c << 2) & 0xC0C0C0C0u, p3 = c & 0xC0C0C0C0u;
      const uint32_t A = __builtin_amdgcn_perm(p1, p0, 0x05010400u);   // [f0 f1 f4 f5]
      const uint32_t B = __builtin_amdgcn_perm(p3, p2, 0x05010400u);   // [f2 f3 f6 f7]
      const uint32_t C = __builtin_amdgcn_perm(p1, p0, 0x07030602u);   // [f8 f9 . .]
      const uint32_t D = __builtin_amdgcn_perm(p3, p2, 0x07030602u);   // [f10 f11 . .]
      const uint2 s01 = *(const uint2*)(lut + 16 * (m16 & 0xFFu));
      const uint2 s23 = *(const uint2*)(lut + 16 * ((m16 >> 8) & 0xFFu) + 8);
      const v4i a = (v4i){(int)__builtin_amdgcn_perm(B, A, s01.x), (int)__builtin_amdgcn_perm(B, A, s01.y),
                          (int)__builtin_amdgcn_perm(C, B, s23.x), (int)__builtin_amdgcn_perm(D, C, s23.y)};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bx[s], acc, 0, 0, 0);
    }
    return acc;
  }
};

// Decode-plane decoder (any ratio, the effective ternary weights at one 2-bit
// code per position), dense v_mfma_i32_16x16x64_i8: sixteen steps of 64 as in
// the 6:8 decoder; lane group g's run is the 64 plane bytes of positions
// 256g .. 256g + 255 (plane words 16g .. 16g + 15 of the range), step s takes
// word 16g + s.  The plane's bit order makes the decode four shift-and-masks:
// (word << 2k) & 0xC0C0C0C0 are positions 4k .. 4k + 3 of the word as 64 * w.
// Ring slot: 16 rows x 256 B; chunk c of row r sits at chunk position
// c ^ (r & 15), so the 16 lanes that read one chunk of 16 rows touch 16
// different 16-byte bank groups.
#ifndef SBN_GV_D2_BPC
#define SBN_GV_D2_BPC 4
#endif
struct Dec2 {
  static constexpr int SLOT = 4096, NDMA = 4, LUT = 0, BPC = SBN_GV_D2_BPC;   // 40 KB LDS per block (ring of 2)
  __host__ __device__ static int64_t meta_row(int64_t) { return 0; }
  __host__ __device__ static int64_t code_row(int64_t K) { return K / 4; }
  int rowq[4], colq[4];
  v4i bx[16];
  __device__ inline void init(int wave, int lane) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {                        // LDS chunk position 64q + lane
      const int sp = 64 * q + lane, rr = sp >> 4;
      rowq[q] = rr;
      colq[q] = 256 * wave + 16 * ((sp & 15) ^ (rr & 15));
    }
  }
  __device__ inline void issue(uint8_t* dst, const uint8_t*, const uint8_t* c, int valid, int64_t K) {
    const int64_t rowc = K / 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = rowq[q] < valid ? rowq[q] : valid - 1;
      g2lds16(c + r * rowc + colq[q], dst + 1024 * q);
    }
  }
  __device__ inline void load_x(const int8_t* xrow, bool ok, int wave, int g) {
#pragma unroll
    for (int s = 0; s < 16; ++s)
      bx[s] = ok ? *(const v4i*)(xrow + 1024 * wave + 256 * g + 16 * s) : (v4i){0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 16; ++s) asm volatile("" ::"v"(bx[s]));
  }
  __device__ inline void build_lut(uint8_t*, int) {}
  struct Frag {
    v4i w[4];
  };
  __device__ inline Frag read(const uint8_t* slot, int rl, int g) const {
    const uint32_t sr = lds_addr(slot + rl * 256);
    Frag f;
    lds_read4(f.w[0], f.w[1], f.w[2], f.w[3], sr + 16 * ((4 * g) ^ rl), sr + 16 * ((4 * g + 1) ^ rl),
              sr + 16 * ((4 * g + 2) ^ rl), sr + 16 * ((4 * g + 3) ^ rl));
    return f;
  }
  __device__ inline v4i compute(const Frag& f, const uint8_t*) const {
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v4i v = f.w[i];
      w[4 * i] = (uint32_t)v[0]; w[4 * i + 1] = (uint32_t)v[1]; w[4 * i + 2] = (uint32_t)v[2]; w[4 * i + 3] = (uint32_t)v[3];
    }
    constexpr uint32_t MK = 0xC0C0C0C0u;
    v4i acc = (v4i){0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const v4i a = (v4i){(int)(w[s] & MK), (int)((w[s] << 2) & MK), (int)((w[s] << 4) & MK), (int)((w[s] << 6) & MK)};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bx[s], acc, 0, 0, 0);
    }
    return acc;
  }
};

// Joint 2:4 code decoder, v_smfmac_i32_16x16x128_i8 with the lane mapping of
// Dec24 (step s, lane group g: groups 64g + 8s .. 64g + 8s + 7 of the range,
// 32 positions).  A group's 6-bit code is its nibble nib = i1 | i2 << 2 (the
// positions of its two slots) and a 2-bit h; the nibble plane's 32-bit word
// for those 8 groups is the instruction's index word as it stands, and the
// slot values come from a 64-entry table of byte pairs (v1, v2 as 64 * w)
// indexed by h | nib << 2, built in LDS by each block.  The table indices of
// four groups are formed at once, one per byte, twice the index (the byte
// offset of a 2-byte entry): h to bits 1-2, nib to bits 3-6.
// Ring slot: 16 rows x 128 B of nibbles (chunk c of row r at c ^ (r & 7)),
// then 16 rows x 64 B of h (chunk c of row r at c ^ ((r >> 2) & 3)); the h
// word u of a row range holds groups 16u .. 16u + 15, group 16u + 8b + 2k + o
// in byte k at bits 2(2b + o).
struct Dec24j {
  static constexpr int SLOT = 3072, NDMA = 3, LUT = 128, BPC = 4;   // 32.1 KB LDS per block
  __host__ __device__ static int64_t meta_row(int64_t K) { return K / 16; }   // h plane (entry.meta)
  __host__ __device__ static int64_t code_row(int64_t K) { return K / 8; }    // nibble plane (entry.codes)
  int rowq[3], colq[3];
  v4i blo[8], bhi[8];
  __device__ inline void init(int wave, int lane) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {                        // nibbles: chunk positions 64q + lane
      const int sp = 64 * q + lane, rr = sp >> 3;
      rowq[q] = rr;
      colq[q] = 128 * wave + 16 * ((sp & 7) ^ (rr & 7));
    }
    const int rr = lane >> 2;                            // h: chunk positions lane
    rowq[2] = rr;
    colq[2] = 64 * wave + 16 * ((lane & 3) ^ ((rr >> 2) & 3));
  }
  __device__ inline void issue(uint8_t* dst, const uint8_t* hp, const uint8_t* np, int valid, int64_t K) {
    const int rown = (int)(K / 8), rowh = (int)(K / 16);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = rowq[q] < valid ? rowq[q] : valid - 1;
      g2lds16(np + r * rown + colq[q], dst + 1024 * q);
    }
    const int r = rowq[2] < valid ? rowq[2] : valid - 1;
    g2lds16(hp + r * rowh + colq[2], dst + 2048);
  }
  __device__ inline void load_x(const int8_t* xrow, bool ok, int wave, int g) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int64_t lo = 1024 * wave + 256 * (g >> 1) + 32 * s + 16 * (g & 1);
      blo[s] = ok ? *(const v4i*)(xrow + lo) : (v4i){0, 0, 0, 0};
      bhi[s] = ok ? *(const v4i*)(xrow + lo + 512) : (v4i){0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(blo[s]), "v"(bhi[s]));
  }
  // entry e = h | nib << 2: (v1, v2) as 64 * w; i1 != i2: the signs in h; i1 == i2:
  // v1 = 0, +1, -1 for h = 0, 1, 3 and v2 = 0 (h = 2 is not a code: zeros)
  __device__ inline void build_lut(uint8_t* lut, int tid) {
    if (tid < 64) {
      const uint32_t h = tid & 3, i1 = (tid >> 2) & 3, i2 = tid >> 4;
      uint32_t v1, v2;
      if (i1 != i2) {
        v1 = (h & 1) ? 0xC0u : 0x40u;
        v2 = (h & 2) ? 0xC0u : 0x40u;
      } else {
        v1 = h == 1 ? 0x40u : (h == 3 ? 0xC0u : 0u);
        v2 = 0u;
      }
      *(uint16_t*)(lut + 2 * tid) = (uint16_t)(v1 | v2 << 8);
    }
  }
  struct Frag {
    v4i n0, n1, h;
  };
  __device__ inline Frag read(const uint8_t* slot, int rl, int g) const {
    const uint32_t sn = lds_addr(slot + rl * 128);
    const uint32_t sh = lds_addr(slot + 2048 + rl * 64) + 16 * (g ^ ((rl >> 2) & 3));
    Frag f;
    lds_read3(f.n0, f.n1, f.h, sn + 16 * ((2 * g) ^ (rl & 7)), sn + 16 * ((2 * g + 1) ^ (rl & 7)), sh);
    return f;
  }
  __device__ inline v4i compute(const Frag& f, const uint8_t* lut) const {
    const uint32_t nw[8] = {(uint32_t)f.n0[0], (uint32_t)f.n0[1], (uint32_t)f.n0[2], (uint32_t)f.n0[3],
                            (uint32_t)f.n1[0], (uint32_t)f.n1[1], (uint32_t)f.n1[2], (uint32_t)f.n1[3]};
    v4i acc = (v4i){0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t N = nw[s], Hw = (uint32_t)f.h[s >> 1];
      const int fe = 2 * (s & 1);                      // h field of the even groups; fe + 1 of the odd ones
      const uint32_t he = fe == 0 ? Hw << 1 : Hw >> 3, ho = fe == 0 ? Hw >> 1 : Hw >> 5;
      const uint32_t E0 = ((N << 3) & 0x78787878u) | (he & 0x06060606u);   // groups 0, 2, 4, 6
      const uint32_t E1 = ((N >> 1) & 0x78787878u) | (ho & 0x06060606u);   // groups 1, 3, 5, 7
      v4i a;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = *(const uint16_t*)(lut + ((E0 >> (8 * k)) & 0xFFu));
        const uint32_t hi = *(const uint16_t*)(lut + ((E1 >> (8 * k)) & 0xFFu));
        a[k] = (int)(lo | hi << 16);
      }
      const v8i b = (v8i){blo[s][0], blo[s][1], blo[s][2], blo[s][3], bhi[s][0], bhi[s][1], bhi[s][2], bhi[s][3]};
      acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, acc, (int)N, 0, 0);
    }
    return acc;
  }
};

// The row groups one block walks, in order: chunks of `chunk` consecutive
// global row groups q = w * nrg + lr (over the count * nrg of the launch),
// chunk b, b + G, b + 2G, ... for block b of G.  Small chunks keep the blocks
// of the chip reading neighbouring addresses at any moment.
struct RgWalk {
  int64_t kc, q, qend, w, lr;
  __device__ inline void seek(int64_t c, int64_t chunk, int64_t total, int64_t nrg) {
    kc = c;
    q = c * chunk;
    qend = q + chunk < total ? q + chunk : total;
    w = q / nrg;
    lr = q - w * nrg;
  }
  __device__ inline bool last_in_chunk() const { return q + 1 == qend; }
  __device__ inline void next(int64_t G, int64_t chunk, int64_t total, int64_t nrg) {
    if (++q == qend) {
      seek(kc + G, chunk, total, nrg);
    } else if (++lr == nrg) {
      lr = 0;
      ++w;
    }
  }
};

// One launch over `count` weights of R rows each: global row group q = w * nrg + lr.
template <int OUT, typename Dec, typename Tab>
__global__ __launch_bounds__(256, Dec::BPC) void gemv_stream_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ s_x, int64_t T, int64_t K, const Tab P,
    int64_t count, int64_t R, int64_t ldy, int64_t chunk) {
  // LDS: the [4 waves][GV_RING][SLOT] ring, the decode table and red[2][4][256]
  // as three objects (the table's reads then do not wait for the ring's
  // in-flight loads)
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * GV_RING * Dec::SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t lut[Dec::LUT > 0 ? Dec::LUT : 16];
  __shared__ __attribute__((aligned(16))) int red[2][4][256];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, rl = lane & 15;
  const int64_t nrg = cdiv(R, 16);
  const int64_t rowm = Dec::meta_row(K), rowc = Dec::code_row(K);      // plane bytes per row
  const bool has = wave < K / 1024;                    // wave-uniform
  const int64_t tq = tid & 15;                         // token of the outputs this thread writes
  const float sxv = OUT != 0 ? s_x[tq < T ? tq : 0] : 0.0f;
  uint8_t* myring = lds + wave * GV_RING * Dec::SLOT;
  Dec dec;
  dec.init(wave, lane);

  // this block's chunks and its number of row groups
  const int64_t total = nrg * count, G = gridDim.x, b = blockIdx.x;
  const int64_t nch = cdiv(total, chunk);
  const int64_t mine = (nch - 1 - b) / G + 1;          // chunks b, b + G, ... below nch (b < nch)
  const bool has_tail = (nch - 1 - b) % G == 0;        // the last, possibly short, chunk is this block's
  const int nit = (int)(mine * chunk - (has_tail ? nch * chunk - total : 0));
  RgWalk iss, cur;                                     // next row group to load / to compute
  iss.seek(b, chunk, total, nrg);
  cur.seek(b, chunk, total, nrg);
  auto issue_next = [&](int slot) {
    const int valid = (int)(R - iss.lr * 16 < 16 ? R - iss.lr * 16 : 16);
    const GvEntry ew = gv_entry(P, iss.w);
    const uint8_t* mp = rowm ? ew.meta + iss.lr * 16 * rowm : nullptr;
    dec.issue(myring + slot * Dec::SLOT, mp, ew.codes + iss.lr * 16 * rowc, valid, K);
    iss.next(G, chunk, total, nrg);
  };
  // GV_RING row groups in flight from the start: a slot is refilled as soon
  // as its words are in registers, so every slot is loading while the wave
  // computes
  if (has) {
#pragma unroll
    for (int i = 0; i < GV_RING; ++i)
      if (i < nit) issue_next(i);
  }
  dec.build_lut(lut, tid);
  const bool tvalid = rl < T;
  dec.load_x(Xq + (tvalid ? rl : 0) * K, has && tvalid, wave, g);
  lds_barrier();                                       // decode table complete

  StreamOut<OUT> out;
  int j0 = (int)(cur.lr & 3);
  int slot = 0, par = 0;
  for (int it = 0; it < nit; ++it) {
    v4i acc = (v4i){0, 0, 0, 0};
    float swv = 0.0f;
    const GvEntry ec = gv_entry(P, cur.w);
    if (OUT != 0) swv = gv_scale(ec.s_w);
    if (has) {
      // row groups it + 1 .. it + GV_RING - 1 (those that exist) were issued
      // after this one: its loads are done once at most NDMA per later row
      // group remain (the stores committed since sit between them and are
      // waited for too)
      const int later = nit - 1 - it;
      if (later >= GV_RING - 1) wait_vmcnt<Dec::NDMA * (GV_RING - 1)>();
      else if (GV_RING > 3 && later == 2) wait_vmcnt<Dec::NDMA * 2>();
      else if (later == 1) wait_vmcnt<Dec::NDMA>();
      else wait_vmcnt<0>();
      out.commit(tid, R, ldy);
      // the slot's words into registers (waited for in the read), then refill it
      const typename Dec::Frag f = dec.read(myring + slot * Dec::SLOT, rl, g);
      if (it + GV_RING < nit) issue_next(slot);
      acc = dec.compute(f, lut);
      slot = slot + 1 == GV_RING ? 0 : slot + 1;
    }
    // output group of four row groups: this block fills places j0 .. j of it
    const int j = (int)(cur.lr & 3);
    if (j == 0) j0 = 0;
    const bool done = j == 3 || cur.lr == nrg - 1 || cur.last_in_chunk();
    out.row_group(red[par], acc, tid, wave, lane, j, j0, done, (cur.lr & ~(int64_t)3) * 16, T, swv, sxv, ec.Y);
    par ^= 1;
    if (!has) out.commit(tid, R, ldy);
    const bool new_chunk = cur.last_in_chunk();
    cur.next(G, chunk, total, nrg);
    if (new_chunk) j0 = (int)(cur.lr & 3);
  }
  out.commit(tid, R, ldy);
}

// ----------------------------------------------------------------------------- one-token streamed decode (2:4)
// For one token the activations are at most 4 KB: they sit in LDS, and each
// wave takes whole row groups over the full contraction (the K / 1024 ranges
// of the 2:4 decoder in turn), so no partial sums cross waves and, after the
// activations are in place, no barrier is needed.  A wave's packed words
// stream through its own ring of NS range slots (direct global->LDS loads,
// as in gemv_stream_kernel); the activations of a range are read from LDS
// into the B fragments of the token's lanes (the other lanes hold zeros).
// Wave gw of the grid's GW waves takes row groups gw, gw + GW, ...
#ifndef SBN_GV_TOK1
#define SBN_GV_TOK1 1
#endif
#ifndef SBN_T1_NS
#define SBN_T1_NS 3
#define SBN_T1_BPC 3
#endif
constexpr int T1_NS = SBN_T1_NS, T1_BPC = SBN_T1_BPC;    // ring slots per wave, resident blocks per CU (52 KB LDS each)

// Wait until the ring slot of this iteration is loaded: at most NDMA loads per
// later range in flight (up to NS - 1 of them) remain, plus the store issued
// after the latest refill (vmcnt counts loads and stores in issue order; a
// ragged group's stores may take more than one instruction, and counting one
// for them only waits for the rest too).
template <int NDMA, int NS>
__device__ inline void wait_ring(int later, bool kst) {
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  if (NS > 3 && later >= 3) {
    if (kst) wait_vmcnt<NDMA * 3 + 1>();
    else wait_vmcnt<NDMA * 3>();
  } else if (NS > 2 && later >= 2) {
    if (kst) wait_vmcnt<NDMA * 2 + 1>();
    else wait_vmcnt<NDMA * 2>();
  } else if (later >= 1) {
    if (kst) wait_vmcnt<NDMA + 1>();
    else wait_vmcnt<NDMA>();
  } else {
    wait_vmcnt<0>();
  }
}

template <int OUT, typename Dec, typename Tab, int NS, int BPC>
__global__ __launch_bounds__(256, BPC) void gemv_tok1_kernel(const int8_t* __restrict__ Xq,
                                                             const float* __restrict__ s_x, int64_t K,
                                                             const Tab P, int64_t count, int64_t R) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * NS * Dec::SLOT];
  __shared__ __attribute__((aligned(16))) int8_t xs[4096];
  __shared__ __attribute__((aligned(16))) uint8_t lut[Dec::LUT > 0 ? Dec::LUT : 16];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, rl = lane & 15;
  const int nr = (int)(K >> 10);                       // ranges of 1024 positions per row
  const int64_t nrg = cdiv(R, 16), total = nrg * count;
  const int64_t rowm = Dec::meta_row(K), rowc = Dec::code_row(K);      // plane bytes per row
  Dec dec;
  for (int64_t i = tid * 16; i < K; i += 256 * 16) *(v4i*)(xs + i) = *(const v4i*)(Xq + i);
  dec.build_lut(lut, tid);
  __syncthreads();
  const int64_t GW = (int64_t)gridDim.x * 4, gw = (int64_t)blockIdx.x * 4 + wave;
  if (gw >= total) return;                             // wave-uniform; no barrier follows
  const float sxv = OUT != 0 ? s_x[0] : 0.0f;
  uint8_t* myring = lds + wave * NS * Dec::SLOT;
  const int nit = (int)(((total - 1 - gw) / GW + 1) * nr);
#pragma unroll
  for (int s = 0; s < 8; ++s) dec.blo[s] = dec.bhi[s] = (v4i){0, 0, 0, 0};

  int64_t iq = gw;                                     // next range to load: range ir of row group iq
  int ir = 0;
  auto issue_next = [&](int slot) {
    const int64_t w = iq / nrg, lr = iq - w * nrg;
    const int valid = (int)(R - lr * 16 < 16 ? R - lr * 16 : 16);
    const GvEntry e = gv_entry(P, w);
    dec.init(ir, lane);                                // the range takes the place of the wave
    dec.issue(myring + slot * Dec::SLOT, e.meta + lr * 16 * rowm, e.codes + lr * 16 * rowc, valid, K);
    if (++ir == nr) {
      ir = 0;
      iq += GW;
    }
  };
#pragma unroll
  for (int i = 0; i < NS; ++i)
    if (i < nit) issue_next(i);

  typedef __attribute__((address_space(1))) uint16_t* GU16;
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(1))) v2u* GU2;
  typedef __attribute__((address_space(1))) int* GI32;
  typedef __attribute__((address_space(1))) v4i* GV4;
  v4i tot = (v4i){0, 0, 0, 0}, pv = (v4i){0, 0, 0, 0};
  int64_t cq = gw, prow = 0;                           // row group being computed; first row of the pending store
  void* pY = nullptr;
  bool pend = false, kst = false;                      // a store is pending / was issued after the latest refill
  // lanes of token 0 (rl == 0) store rows prow .. prow + 3 of the pending group
  auto store = [&]() {
    if (rl == 0) {
      if (OUT == 2) {
        const GU16 y = (GU16)pY + prow;
        if (prow + 4 <= R) {
          *(GU2)y = (v2u){(uint32_t)pv[0], (uint32_t)pv[1]};
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (prow + q < R) y[q] = (uint16_t)((uint32_t)pv[q >> 1] >> (16 * (q & 1)));
        }
      } else {
        const GI32 y = (GI32)pY + prow;
        if (prow + 4 <= R) {
          *(GV4)y = pv;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (prow + q < R) y[q] = pv[q];
        }
      }
    }
  };
  int slot = 0, cr = 0;
  for (int it = 0; it < nit; ++it) {
    // the range's activations (token 0's lanes), read while the ring loads land
    if (rl == 0) {
      const int8_t* xr = xs + 1024 * cr + 256 * (g >> 1) + 16 * (g & 1);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        dec.blo[s] = *(const v4i*)(xr + 32 * s);
        dec.bhi[s] = *(const v4i*)(xr + 32 * s + 512);
      }
    }
    wait_ring<Dec::NDMA, NS>(nit - 1 - it, kst);
    // the slot's words into registers (waited for in the read), refill it,
    // then the previous group's store
    const typename Dec::Frag f = dec.read(myring + slot * Dec::SLOT, rl, g);
    if (it + NS < nit) issue_next(slot);
    kst = pend;
    if (pend) {
      store();
      pend = false;
    }
    tot += dec.compute(f, lut);
    if (++cr == nr) {
      const int64_t w = cq / nrg, lr = cq - w * nrg;
      const GvEntry e = gv_entry(P, w);
      const v4i sum = tot >> 6;                        // exact: every partial is a multiple of 64
      if (OUT == 0) {
        pv = sum;
      } else {
        const float sc = gv_scale(e.s_w) * sxv;
        float y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) y[q] = (float)sum[q] * sc;
        if (OUT == 1) {
          pv = (v4i){(int)__float_as_uint(y[0]), (int)__float_as_uint(y[1]), (int)__float_as_uint(y[2]),
                     (int)__float_as_uint(y[3])};
        } else {
          pv[0] = (int)((uint32_t)f32_to_bf16_rne(y[0]) | ((uint32_t)f32_to_bf16_rne(y[1]) << 16));
          pv[1] = (int)((uint32_t)f32_to_bf16_rne(y[2]) | ((uint32_t)f32_to_bf16_rne(y[3]) << 16));
        }
      }
      prow = lr * 16 + 4 * g;
      pY = e.Y;
      pend = true;
      tot = (v4i){0, 0, 0, 0};
      cr = 0;
      cq += GW;
    }
    slot = slot + 1 == NS ? 0 : slot + 1;
  }
  if (pend) store();
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

// Row groups per chunk: up to 8 (128 rows), fewer when the launch has fewer
// row groups than 8 per resident block, so that small launches still spread
// over the chip (measured on the 128-weight decode pools: chunks of 8 beat one
// contiguous run per block by 1-4%, 6:8 the most).
int64_t stream_chunk(int64_t total, int64_t blocks) {
#ifdef SBN_GV_CHUNK
  if (SBN_GV_CHUNK > 0) return SBN_GV_CHUNK;
#endif
  const int64_t even = cdiv(total, blocks);
  return even < 8 ? even : 8;
}

template <typename Dec, typename Tab>
hipError_t launch_tok1(const char* name, const int8_t* Xq, const float* s_x, int64_t K, const Tab& P, int64_t count,
                       int64_t R, sbn_dtype ydt, hipStream_t st) {
  const int64_t waves = cdiv(R, 16) * count, blocks = 256 * T1_BPC;
  const int64_t nb = cdiv(waves, 4);
  const dim3 grid((unsigned)(nb < blocks ? nb : blocks)), block(256);
  if (ydt == SBN_I32_ACC)
    SBN_LAUNCH(name, (gemv_tok1_kernel<0, Dec, Tab, T1_NS, T1_BPC>), grid, block, 0, st, Xq, s_x, K, P, count, R);
  else if (ydt == SBN_F32)
    SBN_LAUNCH(name, (gemv_tok1_kernel<1, Dec, Tab, T1_NS, T1_BPC>), grid, block, 0, st, Xq, s_x, K, P, count, R);
  else
    SBN_LAUNCH(name, (gemv_tok1_kernel<2, Dec, Tab, T1_NS, T1_BPC>), grid, block, 0, st, Xq, s_x, K, P, count, R);
  return hipGetLastError();
}

template <typename Dec, typename Tab>
hipError_t launch_stream(const char* name, const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                         const Tab& P, int64_t count, int64_t R, sbn_dtype ydt, int64_t ldy, hipStream_t st) {
  const int64_t total = cdiv(R, 16) * count;
  // one token with at least a row group for every resident wave of the
  // one-token kernel; fewer row groups keep four waves on each (K split)
  // (the joint 2:4 code on the one-token kernel measured slower than K-split:
  // 94.1-94.3 against 92.1-92.7 us on the 128-weight pool)
  if constexpr (std::is_same<Dec, Dec24>::value)
    if (SBN_GV_TOK1 && T == 1 && total >= 256 * T1_BPC * 4)
      return launch_tok1<Dec>("gemv_tok1_24", Xq, s_x, K, P, count, R, ydt, st);
  const int64_t blocks = 256 * Dec::BPC;   // one wave of resident blocks over the 256 CUs
  const int64_t chunk = stream_chunk(total, blocks), nch = cdiv(total, chunk);
  const dim3 grid((unsigned)(nch < blocks ? nch : blocks)), block(256);
  if (ydt == SBN_I32_ACC)
    SBN_LAUNCH(name, (gemv_stream_kernel<0, Dec, Tab>), grid, block, 0, st, Xq, s_x, T, K, P, count, R, ldy, chunk);
  else if (ydt == SBN_F32)
    SBN_LAUNCH(name, (gemv_stream_kernel<1, Dec, Tab>), grid, block, 0, st, Xq, s_x, T, K, P, count, R, ldy, chunk);
  else
    SBN_LAUNCH(name, (gemv_stream_kernel<2, Dec, Tab>), grid, block, 0, st, Xq, s_x, T, K, P, count, R, ldy, chunk);
  return hipGetLastError();
}

hipError_t launch_gemv_one(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
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

}  // namespace

hipError_t launch_gemv_batched(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                               const uint8_t* const* codes, const uint8_t* const* meta,
                               const float* const* s_w, int64_t R, int n, int m, void* const* Y,
                               sbn_dtype ydt, int64_t ldy, int count, hipStream_t st) {
  const bool stream_ok = SBN_GV_STREAM && K % 1024 == 0 && K <= 4096 && ((n == 2 && m == 4) || (n == 6 && m == 8));
  if (stream_ok) {
    GemvBatch P;
    for (int b = 0; b < GV_MAX_BATCH; ++b)
      P.e[b] = b < count ? GvEntry{codes[b], meta[b], s_w[b], Y[b]} : GvEntry{nullptr, nullptr, nullptr, nullptr};
    if (n == 2) return launch_stream<Dec24>("gemv_stream_24", Xq, s_x, T, K, P, count, R, ydt, ldy, st);
    return launch_stream<Dec68>("gemv_stream_68", Xq, s_x, T, K, P, count, R, ydt, ldy, st);
  }
  for (int b = 0; b < count; ++b) {
    const hipError_t e = launch_gemv_one(Xq, s_x, T, K, codes[b], meta ? meta[b] : nullptr, s_w[b], R, n, m, Y[b],
                                         ydt, ldy, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

bool gemv_table_shape_ok(int64_t K, int n, int m) {
  return SBN_GV_STREAM && K % 1024 == 0 && K <= 4096 && ((n == 2 && m == 4) || (n == 6 && m == 8));
}

hipError_t launch_gemv_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const GvEntry* table,
                             int64_t count, int64_t R, int n, int m, sbn_dtype ydt, int64_t ldy, hipStream_t st) {
  if (!gemv_table_shape_ok(K, n, m)) return hipErrorInvalidValue;
  const GemvTable P{table};
  if (n == 2) return launch_stream<Dec24>("gemv_stream_24", Xq, s_x, T, K, P, count, R, ydt, ldy, st);
  return launch_stream<Dec68>("gemv_stream_68", Xq, s_x, T, K, P, count, R, ydt, ldy, st);
}

hipError_t launch_gemv(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                       const uint8_t* codes, const uint8_t* meta, const float* s_w, int64_t R,
                       int n, int m, void* Y, sbn_dtype ydt, int64_t ldy, hipStream_t st) {
  return launch_gemv_batched(Xq, s_x, T, K, &codes, &meta, &s_w, R, n, m, &Y, ydt, ldy, 1, st);
}

// ----------------------------------------------------------------------------- decode plane
namespace {

// Packed planes -> decode plane: one thread per plane word (16 positions),
// through the unpack table (blocks walk the words with a grid stride).
template <int M>
__global__ __launch_bounds__(256) void repack_d2_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ meta, int64_t R, int64_t K,
                                                        int n, int64_t cplane, uint32_t* __restrict__ d2) {
  __shared__ uint32_t lut[4096];
  for (int i = threadIdx.x; i < 4096; i += 256) lut[i] = unpack_entry((uint32_t)i);
  __syncthreads();
  const int64_t wpr = K / 16, total = R * wpr;
  const int64_t crow = K * n / (4 * M);                // code bytes per row
  const int64_t lastw = (cplane - 4) & ~(int64_t)3;
  const bool dense = meta == nullptr;
  for (int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x; gid < total; gid += (int64_t)gridDim.x * 256) {
    const int64_t r = gid / wpr, k0 = (gid - r * wpr) * 16;
    const uint32_t mw16 = dense ? 0xFFFFu : (uint32_t)*(const uint16_t*)(meta + r * (K / 8) + k0 / 8);
    const int64_t cbit = r * crow * 8 + k0 * 2 * n / M;
    const int64_t a0 = (cbit >> 3) & ~(int64_t)3;
    const int sh = (int)(cbit - a0 * 8);
    const uint32_t w0 = *(const uint32_t*)(codes + (a0 < lastw ? a0 : lastw));
    const uint32_t w1 = *(const uint32_t*)(codes + (a0 + 4 < lastw ? a0 + 4 : lastw));
    const unsigned long long c = (((unsigned long long)w1 << 32) | w0) >> sh;
    const v4i a = unpack16<M>(lut, mw16, dense, n, c, 0);   // positions 4k .. 4k + 3 in word k, int8
    uint32_t out = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) out |= ((uint32_t)a[k] & 0x03030303u) << (6 - 2 * k);   // +1 -> 01, -1 -> 11
    d2[gid] = out;
  }
}

// Decode-plane GEMV for any K (a multiple of 64): one thread per (row, token),
// four sdot4 per plane word.
template <int OUT>
__global__ __launch_bounds__(256) void gemv_d2_kernel(const int8_t* __restrict__ Xq, const float* __restrict__ s_x,
                                                      int64_t T, int64_t K, const uint32_t* __restrict__ d2,
                                                      const float* __restrict__ s_w, int64_t R, void* __restrict__ Y,
                                                      int64_t ldy) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int t = threadIdx.x & 15;
  if (row >= R || t >= T) return;
  const uint32_t* wr = d2 + row * (K / 16);
  const int* xr = (const int*)(Xq + t * K);
  int acc = 0;
  for (int64_t w = 0; w < K / 16; ++w) {
    const uint32_t word = wr[w];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc = __builtin_amdgcn_sdot4((int)((word << (2 * k)) & 0xC0C0C0C0u), xr[4 * w + k], acc, false);
  }
  const int sum = acc >> 6;                           // exact: every product is a multiple of 64
  if (OUT == 0) {
    ((int*)Y)[t * ldy + row] = sum;
  } else {
    const float y = (float)sum * (*s_w * s_x[t]);
    if (OUT == 1) ((float*)Y)[t * ldy + row] = y;
    else ((uint16_t*)Y)[t * ldy + row] = f32_to_bf16_rne(y);
  }
}

}  // namespace

hipError_t launch_repack_d2(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, int n, int m,
                            uint8_t* d2, hipStream_t st) {
  int64_t blocks = cdiv(R * (K / 16), 256);
  if (blocks > 1024) blocks = 1024;
  const int64_t cplane = round_up(R * (K * n / (4 * m)), 16);
  const uint8_t* mp = (n == m) ? nullptr : meta;
  if (m == 4)
    SBN_LAUNCH("repack_d2", repack_d2_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st, codes, mp, R, K, n, cplane,
               (uint32_t*)d2);
  else
    SBN_LAUNCH("repack_d2", repack_d2_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, st, codes, mp, R, K, n, cplane,
               (uint32_t*)d2);
  return hipGetLastError();
}

namespace {

// 2:4 packed planes -> joint code planes: one thread per 16 groups (64
// positions: 8 meta bytes, 8 code bytes -> 8 nibble bytes, one h word).
__global__ __launch_bounds__(256) void repack_j6_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ meta, int64_t R, int64_t K,
                                                        uint8_t* __restrict__ nib, uint8_t* __restrict__ hpl) {
  const int64_t wpr = K / 64, total = R * wpr;
  for (int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x; gid < total; gid += (int64_t)gridDim.x * 256) {
    const int64_t r = gid / wpr, u = gid - r * wpr;
    const uint64_t mw = *(const uint64_t*)(meta + r * (K / 8) + 8 * u);    // group g: bits 4g .. 4g + 3
    const uint64_t cw = *(const uint64_t*)(codes + r * (K / 8) + 8 * u);   // group g: survivors at bits 4g, 4g + 2
    uint64_t nibs = 0;
    uint32_t hw = 0;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const uint32_t m4 = (uint32_t)(mw >> (4 * g)) & 15u;
      const uint32_t c0 = (uint32_t)(cw >> (4 * g)) & 3u, c1 = (uint32_t)(cw >> (4 * g + 2)) & 3u;
      const uint32_t p0 = m4 ? (uint32_t)__builtin_ctz(m4) : 0u, p1 = m4 ? 31u - (uint32_t)__builtin_clz(m4) : 0u;
      uint32_t i1 = 0, i2 = 0, h = 0;
      if (c0 && c1) {                                  // two nonzeros: their positions and signs
        i1 = p0;
        i2 = p1;
        h = (c0 == 3u ? 1u : 0u) | (c1 == 3u ? 2u : 0u);
      } else if (c0 || c1) {                           // one nonzero: its position twice, its code
        i1 = i2 = c0 ? p0 : p1;
        h = c0 ? c0 : c1;
      }
      nibs |= (uint64_t)(i1 | i2 << 2) << (4 * g);
      const int b = g >> 3, k = (g & 7) >> 1, o = g & 1;
      hw |= h << (8 * k + 2 * (2 * b + o));
    }
    *(uint64_t*)(nib + r * (K / 8) + 8 * u) = nibs;
    *(uint32_t*)(hpl + r * (K / 16) + 4 * u) = hw;
  }
}

}  // namespace

hipError_t launch_repack_j6(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, uint8_t* nib,
                            uint8_t* hpl, hipStream_t st) {
  const int64_t total = R * (K / 64);
  const int64_t blocks = cdiv(total, 256) < 4096 ? cdiv(total, 256) : 4096;
  SBN_LAUNCH("repack_j6", repack_j6_kernel, dim3((unsigned)blocks), dim3(256), 0, st, codes, meta, R, K, nib, hpl);
  return hipGetLastError();
}

hipError_t launch_gemv_j6_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const GvEntry* table,
                                int64_t count, int64_t R, sbn_dtype ydt, int64_t ldy, hipStream_t st) {
  if (!gemv_d2_table_shape_ok(K)) return hipErrorInvalidValue;
  return launch_stream<Dec24j>("gemv_stream_j6", Xq, s_x, T, K, GemvTable{table}, count, R, ydt, ldy, st);
}

hipError_t launch_gemv_j6(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const uint8_t* nib,
                          const uint8_t* hpl, const float* s_w, int64_t R, void* Y, sbn_dtype ydt, int64_t ldy,
                          hipStream_t st) {
  if (!gemv_d2_table_shape_ok(K)) return hipErrorInvalidValue;
  GemvBatch P;
  for (int b = 0; b < GV_MAX_BATCH; ++b)
    P.e[b] = b == 0 ? GvEntry{nib, hpl, s_w, Y} : GvEntry{nullptr, nullptr, nullptr, nullptr};
  return launch_stream<Dec24j>("gemv_stream_j6", Xq, s_x, T, K, P, 1, R, ydt, ldy, st);
}

bool gemv_d2_table_shape_ok(int64_t K) { return SBN_GV_STREAM && K % 1024 == 0 && K <= 4096; }

hipError_t launch_gemv_d2_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const GvEntry* table,
                                int64_t count, int64_t R, sbn_dtype ydt, int64_t ldy, hipStream_t st) {
  if (!gemv_d2_table_shape_ok(K)) return hipErrorInvalidValue;
  return launch_stream<Dec2>("gemv_stream_d2", Xq, s_x, T, K, GemvTable{table}, count, R, ydt, ldy, st);
}

hipError_t launch_gemv_d2_batched(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                  const uint8_t* const* d2, const float* const* s_w, int64_t R, void* const* Y,
                                  sbn_dtype ydt, int64_t ldy, int count, hipStream_t st) {
  if (SBN_GV_STREAM && K % 1024 == 0 && K <= 4096) {
    GemvBatch P;
    for (int b = 0; b < GV_MAX_BATCH; ++b)
      P.e[b] = b < count ? GvEntry{d2[b], nullptr, s_w[b], Y[b]} : GvEntry{nullptr, nullptr, nullptr, nullptr};
    return launch_stream<Dec2>("gemv_stream_d2", Xq, s_x, T, K, P, count, R, ydt, ldy, st);
  }
  const dim3 grid((unsigned)cdiv(R, 16)), block(256);
  for (int b = 0; b < count; ++b) {
    const uint32_t* p = (const uint32_t*)d2[b];
    if (ydt == SBN_I32_ACC)
      SBN_LAUNCH("gemv_d2", gemv_d2_kernel<0>, grid, block, 0, st, Xq, s_x, T, K, p, s_w[b], R, Y[b], ldy);
    else if (ydt == SBN_F32)
      SBN_LAUNCH("gemv_d2", gemv_d2_kernel<1>, grid, block, 0, st, Xq, s_x, T, K, p, s_w[b], R, Y[b], ldy);
    else
      SBN_LAUNCH("gemv_d2", gemv_d2_kernel<2>, grid, block, 0, st, Xq, s_x, T, K, p, s_w[b], R, Y[b], ldy);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sbn
