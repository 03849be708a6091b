// Device-side helpers shared by the gfx950 kernels of the hybrid attention layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] * B[16x32], fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) .. +8) and B[8*(l/32) .. +8)[l%32]; it gets
// back C[8*(r/4) + 4*(l/32) + r%4][l%32] in element r.
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 -> one dword of two bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element e (0..7) of eight packed bf16, as its 16-bit pattern.
__device__ __forceinline__ uint32_t bf16_elem(const u32x4& v, int e) {
  uint32_t w = v[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// max over the two lanes l and l^32 that hold the same MFMA output column.
__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 ld_global_16B(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st_global_8B(void* p, u32x2 v) {
  *reinterpret_cast<u32x2*>(p) = v;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ lds_ptr_t lds_ptr(void* p) { return (lds_ptr_t)p; }

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer descriptor word 3, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kRsrcWord3);
}

// Eight bytes per lane from LDS with a 16-bit transpose inside each group of
// 16 lanes: lanes that read a 4-row x 16-column bf16 block row-wise (4 lanes
// per row, 8 bytes each) receive one column each, its 4 rows in order.
__device__ __forceinline__ u32x2 ds_read_tr16(const unsigned char* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(lds_ptr((void*)p)));
  return __builtin_bit_cast(u32x2, r);
}

// Global (buffer) -> LDS without passing through VGPRs: lane l writes LDS bytes
// [lds + n*l, lds + n*l + n) for n = 16 or 4 bytes. The descriptor's range check covers
// voff + soff; out-of-range lanes write zeros. The builtin is only compiled in
// the device pass: clang's host pass drops the host handle of a kernel
// template whose body names it.
// AUX: the cache policy bits (16: sc1, device scope).
template <int AUX = 0>
__device__ __forceinline__ void dma16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(lds), 16, voff, soff, 0, AUX);
#endif
}
__device__ __forceinline__ void dma4_to_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(lds), 4, voff, soff, 0, 0);
#endif
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// Row-major [rows][D] bf16 tiles read with ds_read_tr16: 32 lanes (one 256-byte
// LDS cycle) read 4 consecutive rows x 64 bytes; XOR-ing the 16-byte chunk index
// with this value puts the four rows on disjoint bank groups (conflict-free on
// gfx950 as measured with the bank-conflict counter).
template <int NCH>
__device__ __forceinline__ int tr_swz(int row) {
  if constexpr (NCH >= 16) return 4 * (row & 3) + 2 * ((row >> 3) & 1);
  else return 2 * (row & 3);
}

// Work-group barrier that orders LDS only. __syncthreads() also waits for every
// outstanding global load of the wave (its release fence), which would drain
// register prefetches issued for later steps; this waits for the wave's LDS
// operations (lgkmcnt = 0; vmcnt and expcnt left at their maxima) and keeps
// the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Work-group index -> work item, so that consecutive work items land on the
// same XCD (work-groups are dealt to the 8 XCDs round-robin, and each XCD has
// its own L2). Requires gridDim.x % 8 == 0; items >= n_items are padding.
__device__ __forceinline__ int xcd_major_item(int n_groups) {
  const int g = blockIdx.x;
  const int per_xcd = n_groups >> 3;
  return (g & 7) * per_xcd + (g >> 3);
}

// Index checks of the debug build (compiled with -DHA_DEBUG; empty otherwise).
// A failed check ORs its bit into this translation unit's debug word with a
// vector atomic and the kernel goes on (no trap); the entry point reads and
// clears the words after its launches and reports the bits. Each kernel file
// defines its reader with HA_DEBUG_READER.
#if defined(HA_DEBUG)
static __device__ unsigned int g_debug_word;
#define HA_CHECK(cond, bit)                                                       \
  do {                                                                            \
    if (!(cond)) atomicOr(&::ha::g_debug_word, (unsigned)(bit));                  \
  } while (0)
#define HA_DEBUG_READER(fn)                                                       \
  unsigned fn() {                                                                 \
    unsigned v = 0, z = 0;                                                        \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(::ha::g_debug_word), sizeof v) != hipSuccess) return ~0u; \
    if (hipMemcpyToSymbol(HIP_SYMBOL(::ha::g_debug_word), &z, sizeof z) != hipSuccess) return ~0u;   \
    return v;                                                                     \
  }
#else
#define HA_CHECK(cond, bit) \
  do {                      \
  } while (0)
#define HA_DEBUG_READER(fn)
#endif

}  // namespace ha
