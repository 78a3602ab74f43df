// device_common.h -- gfx950 building blocks shared by the GEMM kernels of this
// library (not by the oracle): vector types, buffer descriptors, direct
// global->LDS loads, LDS transpose reads, MFMA wrappers and the workgroup ->
// C-tile schedule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define TG_LDS __attribute__((address_space(3)))

namespace tg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// Element formats of A/B (16-bit floats) and C.
enum InKind { IN_F16 = 0, IN_BF16 = 1 };
enum OutKind { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

// Byte offset that lies beyond every buffer's num_records: a buffer load at this
// offset reads nothing from memory and returns zeros (raw-buffer range check,
// per dword).
constexpr uint32_t kOutOfRange = 0x80000000u;
// Largest num_records used; valid offsets of one tile stay below it (checked on the host).
constexpr uint32_t kMaxRecords = 0x7FFFFFF0u;

// Buffer descriptor over [base, base + bytes) (bytes clamped to kMaxRecords).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  uint32_t n = bytes <= 0 ? 0u : (bytes >= (int64_t)kMaxRecords ? kMaxRecords : (uint32_t)bytes);
  // dword3 = 0x00020000: raw (untyped) 32-bit data format for gfx9-family buffers.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// 16 bytes per lane from rsrc + voffset, written straight into LDS at
// lds_base + 16 * lane (gfx950 buffer_load_dwordx4 ... lds). lds_base must be
// wave-uniform; it lands in M0.
__device__ __forceinline__ void load_lds_x4(__amdgpu_buffer_rsrc_t r, TG_LDS void* lds_base, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, (int)voffset, 0, 0, 0);
}

// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i
// receives element e (e = 0..3) from the 8 bytes addressed by lane 4e + i/4 of
// its group, position i % 4. If lane j of a group addresses row j/4, column
// 4*(j%4) of a 4 x 16 block of 16-bit values, lane i receives column i (rows 0..3).
__device__ __forceinline__ s16x4 lds_read_tr(uint32_t lds_byte_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS s16x4*)(uintptr_t)lds_byte_addr);
}

__device__ __forceinline__ i32x4 lds_read_b128(uint32_t lds_byte_addr) {
  return *(TG_LDS i32x4*)(uintptr_t)lds_byte_addr;
}

__device__ __forceinline__ void lds_write_b128(uint32_t lds_byte_addr, i32x4 v) {
  *(TG_LDS i32x4*)(uintptr_t)lds_byte_addr = v;
}

// One 32x32x16 MFMA step: acc += A(32x16) * B(16x32). Operand lane layout: lane l
// holds row (A) / column (B) l % 32 and reduction indices 8*(l/32) .. 8*(l/32)+7.
template <int IN>
__device__ __forceinline__ f32x16 mfma32(i32x4 a, i32x4 b, f32x16 acc) {
  if constexpr (IN == IN_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0,
                                                  0, 0);
}

// One 16x16x32 MFMA step: lane l holds row/column l % 16 and reduction indices
// 8*(l/16) .. 8*(l/16)+7.
template <int IN>
__device__ __forceinline__ f32x4 mfma16(i32x4 a, i32x4 b, f32x4 acc) {
  if constexpr (IN == IN_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0,
                                                  0, 0);
}

// fp32 -> bfloat16 bits, round to nearest even (hardware conversion,
// v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 -> two bfloat16 in one 32-bit word (a in the low half), round to nearest
// even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// fp32 -> binary16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Workgroup -> C tile. The hardware hands consecutive workgroup ids to the 8
// XCDs in turn, and each XCD has its own L2. Renumber so that the workgroups
// resident on one XCD get consecutive ids, then walk the C tiles in groups of
// `group_m` tile rows (column by column inside a group), so that tiles running
// at the same time on one XCD share A row panels and B column panels in its L2.
// group_m = 0 keeps the hardware's order (tile = workgroup id, M fastest): with a
// single tile row or column there is no panel to share, and consecutive tiles on
// different XCDs spread each XCD's requests over the whole streamed operand.
__device__ __forceinline__ void schedule_tile(int wg, int num_wg, int tiles_m, int group_m, int& tile_m,
                                              int& tile_n) {
  if (group_m == 0) {
    tile_m = wg % tiles_m;
    tile_n = wg / tiles_m;
    return;
  }
  constexpr int kXcds = 8;
  const int q = num_wg / kXcds, r = num_wg % kXcds;
  const int x = wg % kXcds, i = wg / kXcds;
  const int id = x * q + (x < r ? x : r) + i;
  const int tiles_n = num_wg / tiles_m;
  const int per_group = group_m * tiles_n;
  const int g = id / per_group;
  const int first_m = g * group_m;
  const int rows = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int local = id - g * per_group;
  tile_m = first_m + local % rows;
  tile_n = local / rows;
}

}  // namespace tg
