// Internal declarations shared by the HIP translation units of libsbn.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sbn.h"

namespace sbn {

// ----------------------------------------------------------------- vector types
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ----------------------------------------------------------------- small helpers
__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }
__host__ __device__ inline size_t align256(size_t a) { return (a + 255) & ~size_t(255); }

// float32 -> bf16 bits, round to nearest even (inputs here are finite)
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
// two float32 -> packed bf16 bits (a in the low half), rounded to nearest even
// by the conversion instruction (one instruction per pair; equal to
// f32_to_bf16_rne on finite inputs)
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t h = (bf16x2_t){(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Write-once global stores through the vector path.
__device__ inline void store_u16x4(uint16_t* p, uint16_t a, uint16_t b, uint16_t c, uint16_t d) {
  uint2 v;
  v.x = (uint32_t)a | ((uint32_t)b << 16);
  v.y = (uint32_t)c | ((uint32_t)d << 16);
  *(uint2*)p = v;
}

// ----------------------------------------------------------------- direct-to-LDS loads
// 16 bytes per lane from `g` into LDS at `lds_base + 16*lane` (wave-uniform base).
__device__ inline void g2lds16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ inline void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt with vmcnt = N (gfx9 encoding; expcnt and lgkmcnt left at "no wait")
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS hand-offs that leaves global loads in flight.
// __syncthreads() carries a memory fence that waits for every outstanding
// vector memory operation, which would drain the loads of later pipeline
// stages; here each wave first waits for exactly the loads it must see
// (wait_vmcnt) and for its own LDS reads, then meets the others.  The empty
// asm statements keep the compiler from moving memory operations across.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ----------------------------------------------------------------- workspace layouts
// Pack: [counter + pad: 256 B][bins: 256 x u64][partials: nblocks x i64]
struct PackPlan {
  int64_t nblocks;
  int64_t chunks_per_block;   // 16-byte chunks of W summed by one pass-1 block
  size_t bytes;
};
PackPlan pack_plan(int64_t R, int64_t K);
// The allocation-free pack's device scratch: its size, and its address on the
// current device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);

// Sparse (smfmac) expansion: values [RB][KB128][64][16 B] + idx [RB][KB128][64][4 B]
// Dense expansion: [RB][KB64][64][16 B]; RB covers R rounded up to the GEMM row tile.
constexpr int GEMM_TILE_R = 256;
constexpr int GEMM_TILE_T = 256;
bool gemm_uses_smfmac(int n, int m);
// The optional input check: *found = any NaN / Inf among the first `cols`
// elements (2- or 4-byte floats) of `rows` rows at stride `ld` elements.
// Synchronizes `st`.
hipError_t scan_nonfinite(const void* x, int64_t rows, int64_t cols, int64_t ld, int elem_bytes, hipStream_t st,
                          bool* found);
size_t gemm_ws_bytes(int64_t T, int64_t R, int64_t K, int n, int m);
size_t gemm_weight_bytes(int64_t R, int64_t K, int n, int m);   // the prepared (expanded) weight operand
size_t gemm_x_bytes(int64_t T, int64_t K, int n, int m);         // tiled activations of a prepared-weight GEMM
size_t bwd_ws_bytes(int64_t T, int64_t R, int64_t K, int n, int m);

// ----------------------------------------------------------------- kernel timing
// prof_begin returns -1 when timing is off (one relaxed load); otherwise it
// records a start event on `st` and returns a slot closed by prof_end.
int prof_begin(hipStream_t st, const char* name);
void prof_end(int slot, hipStream_t st);

// launch `kernel` on `st`, bracketed by timing events when timing is on
// Test hook: with SBN_TEST_INJECT_LAUNCH_FAILURE=1 in the environment at the
// first launch, no kernel is launched and the entry point reports SBN_ERR_HIP
// (so the error path is testable on any machine, without touching memory).
bool inject_launch_failure();
void note_injected_failure();

#define SBN_LAUNCH(name, kernel, grid, block, shmem, st, ...)            \
  do {                                                                   \
    if (::sbn::inject_launch_failure()) {                                \
      ::sbn::note_injected_failure();                                    \
    } else {                                                             \
      const int sbn_p_ = ::sbn::prof_begin((st), (name));                \
      hipLaunchKernelGGL(kernel, grid, block, shmem, st, __VA_ARGS__);   \
      ::sbn::prof_end(sbn_p_, (st));                                     \
    }                                                                    \
  } while (0)

// ----------------------------------------------------------------- launchers
// G != nullptr: the optimizer step W <- bf16(fma(-lr, G, W)) runs first, in place.
hipError_t launch_pack(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                       uint8_t* codes, uint8_t* meta, float* s_w, void* ws, uint32_t flags,
                       const float* G, int64_t ldg, float lr, hipStream_t st);
hipError_t launch_act_quant(const uint16_t* X, int64_t T, int64_t K, int64_t ldx, int8_t* Xq,
                            float* s_x, hipStream_t st);
// The pack and the activation quantizer of one forward, with pass 1 of the pack
// and the quantizer in one launch (same results as launch_pack + launch_act_quant).
hipError_t launch_pack_quant(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                             uint8_t* codes, uint8_t* meta, float* s_w, void* ws, uint32_t flags,
                             const uint16_t* X, int64_t T, int64_t ldx, int8_t* Xq, float* s_x, hipStream_t st);
// The one-call forward at 2:4 on the wide GEMM tiles: pass 2 of the pack also
// writes the GEMM's weight operand in the prepared-weight layout (values, then
// the index words at gemm_operand_idx_offset), and the GEMM on it reads the
// activations in place, so no layout launch runs.
bool forward_writes_operand(int64_t T, int64_t R, int64_t K, int n, int m, uint32_t flags);
size_t gemm_operand_idx_offset(int64_t R, int64_t K, int n, int m);
hipError_t launch_pack_quant_operand(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, uint8_t* codes,
                                     uint8_t* meta, float* s_w, void* ws, const uint16_t* X, int64_t T, int64_t ldx,
                                     int8_t* Xq, float* s_x, uint8_t* vals, uint32_t* idx, hipStream_t st);
// The weight operand of the GEMM expanded once (for weights used by many calls),
// and the GEMM on it (the activations are tiled into ws, gemm_x_bytes).
hipError_t launch_prepare_gemm_weight(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, int n, int m,
                                      uint8_t* prepared, hipStream_t st);
hipError_t launch_gemm_prepared(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const uint8_t* prepared,
                                const float* s_w, int64_t R, int n, int m, void* Y, sbn_dtype ydt, int64_t ldy,
                                void* ws, hipStream_t st);
hipError_t launch_gemm(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                       const uint8_t* codes, const uint8_t* meta, const float* s_w, int64_t R,
                       int n, int m, void* Y, sbn_dtype ydt, int64_t ldy, void* ws, hipStream_t st);
// Decode GEMV over `count` (<= GV_MAX_BATCH) weights sharing Xq; host arrays of device pointers.
constexpr int GV_MAX_BATCH = SBN_GEMV_MAX_BATCH;
hipError_t launch_gemv_batched(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                               const uint8_t* const* codes, const uint8_t* const* meta,
                               const float* const* s_w, int64_t R, int n, int m, void* const* Y,
                               sbn_dtype ydt, int64_t ldy, int count, hipStream_t st);
// Decode GEMV over a table of `count` weights in device memory; one launch.  The shapes it covers (K a multiple of 1024 up
// to 4096; 2:4 and 6:8 packed weights, or decode planes of any ratio):
using GvEntry = sbn_gemv_entry;
bool gemv_table_shape_ok(int64_t K, int n, int m);
bool gemv_d2_table_shape_ok(int64_t K);
hipError_t launch_gemv_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const GvEntry* table,
                             int64_t count, int64_t R, int n, int m, sbn_dtype ydt, int64_t ldy, hipStream_t st);
hipError_t launch_gemv_d2_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const GvEntry* table,
                                int64_t count, int64_t R, sbn_dtype ydt, int64_t ldy, hipStream_t st);
// Joint 2:4 code: repack of 2:4 packed planes (K a multiple of 64), and the
// streamed GEMV on it (one weight, or a device table: codes = nibble plane,
// meta = h plane; K a multiple of 1024 up to 4096).
hipError_t launch_repack_j6(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, uint8_t* nib,
                            uint8_t* hpl, hipStream_t st);
hipError_t launch_gemv_j6(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const uint8_t* nib,
                          const uint8_t* hpl, const float* s_w, int64_t R, void* Y, sbn_dtype ydt, int64_t ldy,
                          hipStream_t st);
hipError_t launch_gemv_j6_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const GvEntry* table,
                                int64_t count, int64_t R, sbn_dtype ydt, int64_t ldy, hipStream_t st);
// Decode plane: repack of the packed planes, and the GEMV over up to GV_MAX_BATCH planes.
hipError_t launch_repack_d2(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, int n, int m,
                            uint8_t* d2, hipStream_t st);
hipError_t launch_gemv_d2_batched(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                  const uint8_t* const* d2, const float* const* s_w, int64_t R, void* const* Y,
                                  sbn_dtype ydt, int64_t ldy, int count, hipStream_t st);
hipError_t launch_gemv(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                       const uint8_t* codes, const uint8_t* meta, const float* s_w, int64_t R,
                       int n, int m, void* Y, sbn_dtype ydt, int64_t ldy, hipStream_t st);
hipError_t launch_backward(const uint16_t* dY, int64_t T, int64_t R, const int8_t* Xq,
                           const float* s_x, int64_t K, const uint8_t* codes, const uint8_t* meta,
                           const float* s_w, int n, int m, void* dX, sbn_dtype dxdt, float* dW,
                           void* ws, uint32_t flags, hipStream_t st);

}  // namespace sbn
