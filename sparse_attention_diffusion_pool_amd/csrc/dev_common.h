// Device-side building blocks for the gfx950 kernels of libpisa: vector types, MFMA wrappers,
// buffer-resource loads (out-of-range bytes read as zero), direct global->LDS copies, the LDS
// transpose read, and the LDS tile swizzles.
//
// Lane layouts used throughout (checked on gfx950 with an in-bounds probe):
//   v_mfma_f32_32x32x16_bf16: A[i][k] -> lane i + 32*(k/8), element k%8; B[k][j] -> lane
//   j + 32*(k/8), element k%8; D[i][j] -> lane j + 32*((i/4)%2), accumulator (i%4) + 4*(i/8).
//   ds_read_b64_tr_b16: within each 16-lane group, lane r supplies the address of 4 consecutive
//   16-bit values M[r][0..3]; lane i receives {M[4e + i/4][i%4] : e = 0..3}.
//   Direct global->LDS 16-byte loads write lane l's data at (wave-uniform base) + 16*l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pisa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// 16-byte global load through a buffer resource: bytes past the resource's range read as 0.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}

// Direct copy global -> LDS of 16 bytes per lane: lane l's bytes land at lds_base + 16*l
// (lds_base must be wave-uniform). Bytes past the resource's range are written as 0.
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima), through the builtin so that the
// compiler's wait-count bookkeeping knows every earlier vector-memory load has completed.
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __asm__ __volatile__("" ::: "memory");
}

// LDS byte address of a __shared__ object. Applied to the object itself it folds to a constant;
// kept as a 32-bit address afterwards, the copies need no generic-to-LDS pointer conversion
// (with its null check) per instruction.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Buffer resource words for copy_chunk_async (same format as make_rsrc).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, kRsrcWord3};
}

__device__ __forceinline__ i16x4 lds_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}

__device__ __forceinline__ bf16x8 join_tr(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS tiles of R rows x 128 bf16 (256 bytes = 16 chunks of 16 bytes per row).
// "row-read" tiles are read 16 bytes per lane along a row by 32 consecutive rows (MFMA operand
// whose contiguous dimension is the reduction): chunk c of row r is stored at c ^ (r & 15).
// "transpose-read" tiles are read with ds_read_b64_tr_b16 over 4 consecutive rows x 32 bytes
// per 16-lane group: chunk c of row r is stored at c ^ ((r & 3) << 2).
__device__ __forceinline__ uint32_t swz_row(uint32_t r, uint32_t c) { return c ^ (r & 15u); }
__device__ __forceinline__ uint32_t swz_tr(uint32_t r, uint32_t c) { return c ^ ((r & 3u) << 2); }

// Copy a tile of `rows` x 256 B (row stride `stride` bytes in global memory) into LDS at `lds`
// with the given swizzle, using nwaves waves. Rows past the resource range arrive as zeros.
template <bool TR>
__device__ __forceinline__ void tile_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t stride, char* lds,
                                            int rows, int wave, int nwaves, int lane) {
  // one wave instruction covers 4 rows (1 KB); lane -> row 4n + lane/16, stored chunk lane%16
  for (int n = wave; n < rows / 4; n += nwaves) {
    uint32_t row = 4 * n + (lane >> 4);
    uint32_t pos = lane & 15;
    uint32_t src_chunk = TR ? swz_tr(row, pos) : swz_row(row, pos);
    buf_load_lds16(r, lds + 1024 * n, row * stride + src_chunk * 16);
  }
}

// Direct copy of a ROWS x 256 B tile by NWAVES waves, with the per-lane part of the global
// offset precomputed (vbase = copy_vbase<TR>(wave, lane)); instruction m of wave w covers tile
// rows 4 (m NWAVES + w) .. +3. The swizzle only depends on (row & 15), which is the same for every
// m when NWAVES is a multiple of 4, so one vbase serves all m (m NWAVES KB goes in soffset).
// With NWAVES = 2, even and odd m differ by 8 in (row & 15): vbase2 is the offset for odd m.
template <int ROWS, int NWAVES>
__device__ __forceinline__ void copy_tile(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t vbase, int wave,
                                          uint32_t vbase2 = 0) {
  static_assert((NWAVES % 4 == 0 || NWAVES == 2) && ROWS % (4 * NWAVES) == 0, "copy_tile layout");
#pragma unroll
  for (int m = 0; m < ROWS / 4 / NWAVES; ++m)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + 1024 * (m * NWAVES + wave)), 16,
                                             (NWAVES == 2 && (m & 1)) ? vbase2 : vbase,
                                             (NWAVES == 2 ? (m & ~1) : m) * NWAVES * 1024, 0, 0);
}

// Per-lane global offset of a 16-row chunk copy. Instruction m (0..3) of a chunk covers chunk rows
// 4 m .. 4 m + 3: lane l reads row 4 m + l / 16 at the swizzle's source chunk for stored chunk l % 16.
// The row's 1024 m bytes are not included: the instruction offset adds them (it counts in the
// buffer range check, which compares vector plus instruction offset with num_records), and on a
// direct-to-LDS load it moves the LDS destination by the same amount (checked on gfx950 with an
// in-bounds probe).
// What remains depends on m only through the swizzle. Transpose-read tiles swizzle by row & 3 =
// l / 16, the same for every m. Row-read tiles swizzle by row & 15 = 4 m | l / 16, and XOR-ing the
// chunk with 4 m flips bits 6..7 of the byte offset: instruction m's offset is m = 0's XOR 64 m.
template <bool TR>
__device__ __forceinline__ uint32_t chunk_lane(int lane) {
  const uint32_t row = lane >> 4, pos = lane & 15;
  const uint32_t chunk = TR ? swz_tr(row, pos) : swz_row(row, pos);
  return row * 256 + chunk * 16;
}

// Direct copy of one 16-row chunk (4 KB) global -> LDS from inline assembly: one m0 write, four
// loads. lds = the chunk's LDS byte address, soff = a scalar byte offset added to every address
// (0 where rows past the data must read as zeros: the range check then needs no assumption about
// the scalar offset), v0 = chunk_lane<TR>(lane). Bytes past the resource's range are written as 0.
// Issued from assembly because the compiler's wait-count insertion cannot tell direct-to-LDS copies
// into one buffer from reads of another: after a copy through the builtin it makes every later LDS
// read wait for the copy. From assembly it does not see the copy at all, so the caller waits for
// completion itself (wait_vmem) before reading the destination. The instructions have no register
// results; their address operands are read when they issue. The row layout's other three offsets
// are formed inside the block in scratch registers (kept out of the loop, they would hold three
// registers for the whole kernel).
// NT (transpose-read tiles only) sets the non-temporal cache policy on the loads: for streams read
// once per kernel, whose lines would only displace others from L2.
template <bool TR, bool NT = false>
__device__ __forceinline__ void copy_chunk_async(const u32x4& rsrc, uint32_t lds, uint32_t v0, uint32_t soff) {
  static_assert(TR || !NT, "non-temporal copies are provided for transpose-read tiles");
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  const u32x4 r = {(uint32_t)__builtin_amdgcn_readfirstlane(rsrc[0]), (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[1]),
                   (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[2]), (uint32_t)__builtin_amdgcn_readfirstlane(rsrc[3])};
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  if constexpr (TR && NT) {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen nt lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:1024 nt lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:2048 nt lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:3072 nt lds"
        :
        : "s"(m0v), "v"(v0), "s"(r), "s"(so)
        : "memory", "m0");
  } else if constexpr (TR) {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:3072 lds"
        :
        : "s"(m0v), "v"(v0), "s"(r), "s"(so)
        : "memory", "m0");
  } else {
    uint32_t t1, t2, t3;
    asm volatile(
        "s_mov_b32 m0, %3\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %4, %5, %6 offen lds\n\t"
        "v_xor_b32 %0, 64, %4\n\t"
        "v_xor_b32 %1, 0x80, %4\n\t"
        "v_xor_b32 %2, 0xc0, %4\n\t"
        "buffer_load_dwordx4 %0, %5, %6 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %1, %5, %6 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %2, %5, %6 offen offset:3072 lds"
        : "=&v"(t1), "=&v"(t2), "=&v"(t3)
        : "s"(m0v), "v"(v0), "s"(r), "s"(so)
        : "memory", "m0");
  }
}

// Direct copy of a ROWS x 256 B tile whose first `bytes` bytes at `base` are valid, by NWAVES waves
// in 16-row chunks: wave w copies chunks w, w + NWAVES, ...; v0 = chunk_lane<TR>(lane). Each chunk
// gets a buffer resource of its own that starts at the chunk and ends where the valid bytes end
// (zero bytes past them), so the rows past the end are zeros by the buffer range check on the
// vector and instruction offsets alone: a raw buffer (stride 0) returns 0 for every load whose
// offset lies at or beyond num_records (CDNA4 ISA, buffer instructions, range checking).
template <int ROWS, int NWAVES, bool TR, bool NT = false>
__device__ __forceinline__ void copy_tile_chunks(const void* base, uint32_t bytes, uint32_t lds, uint32_t v0,
                                                 int wave) {
  static_assert(ROWS % (16 * NWAVES) == 0, "tile rows must split into 16-row chunks over the waves");
#pragma unroll
  for (int n = 0; n < ROWS / 16 / NWAVES; ++n) {
    const uint32_t c = n * NWAVES + wave;
    const uint32_t start = 4096u * c;
    copy_chunk_async<TR, NT>(rsrc_words(static_cast<const char*>(base) + start, bytes > start ? bytes - start : 0u),
                             lds + start, v0, 0u);
  }
}

// extra_rows: 0, or 8 for the odd instructions of a 2-wave copy
template <bool TR>
__device__ __forceinline__ uint32_t copy_vbase(int wave, int lane, int extra_rows = 0) {
  const uint32_t row = 4 * wave + extra_rows + (lane >> 4);  // (row & 15) as in the instruction
  const uint32_t pos = lane & 15;
  const uint32_t chunk = TR ? swz_tr(row, pos) : swz_row(row, pos);
  return row * 256 + chunk * 16;
}

// Address for ds_read_b64_tr_b16 on a transpose-read tile: logical element (row r, column col),
// col a multiple of 4.
__device__ __forceinline__ const char* tr_addr(const char* tile, uint32_t r, uint32_t col) {
  uint32_t byte = col * 2;
  return tile + r * 256 + swz_tr(r, byte >> 4) * 16 + (byte & 15);
}

// 32x32x16 operand "transposed" from a row-major [key][col] transpose-read tile: the lane gets
// X[key_lo + 0..3][col] in elements 0..3 and X[key_hi + 0..3][col] in elements 4..7, where
// col = c0 + (lane % 16 within the 16-lane group) and the caller passes the per-half key bases.
// Lane r of a 16-lane group addresses row key + r/4, columns c0 + 4*(r%4) .. +3.
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, uint32_t key_lo, uint32_t key_hi,
                                             uint32_t c0, uint32_t lane16) {
  uint32_t dr = lane16 >> 2, dc = 4 * (lane16 & 3);
  i16x4 a = lds_tr16(tr_addr(tile, key_lo + dr, c0 + dc));
  i16x4 b = lds_tr16(tr_addr(tile, key_hi + dr, c0 + dc));
  return join_tr(a, b);
}

// max(x[l], x[l ^ 32]) in every lane, through v_permlane32_swap (no LDS round trip): the swap of
// x with itself hands each lane the other half's value in one of the two results.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ uint32_t float_order_key(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace pisa
