// Tile-layout helpers shared by the prefill and backward kernels: swizzled
// row-major K / V (and Q / dO) tiles in LDS, the A-operand row permutation that
// makes 32x32 MFMA accumulators directly usable as the next MFMA's operand,
// buffer descriptors whose range check zero-fills sequence tails, and the LDS
// DMA.  gfx950 only.
#pragma once

#include "device_common.h"

namespace exattn {

// K tile: row `key` is D*2 bytes; 16-byte chunk c is stored at c ^ kswz(key).
// ds_read_b128 serves 16 lanes per clock (256 bytes over the 64 banks), and the
// 16 lanes of an A-operand read read keys k0..k0+15 of one chunk column, so
// their stored chunks must fall in 16 distinct 16-byte bank groups: rows of 256
// bytes or more need 16 distinct positions; two 128-byte rows share one bank
// width, so for d = 64 even and odd keys each need 8.
template <int D>
__device__ __forceinline__ int kswz(int key) {
  if constexpr (D == 64)
    return (key >> 1) & 7;
  else
    return key & 15;
}

// V tile, stored row-major like K: chunk c of row `key` is stored at
// c ^ vswz(key).  A transposing read takes 8 bytes from each of 4 consecutive
// keys x 2 adjacent chunks per 16 lanes, and LDS serves 32 lanes (256 bytes)
// per pass, so the 32 lanes of a pass (keys k..k+3, 4 adjacent chunks) must
// cover all 64 banks: with rows of 256 bytes or more the offset 4 (key & 3)
// puts the 4 keys in 4 distinct 64-byte quarters.  (The earlier 2 (key & 7)
// kept each pass on 32 banks: two cycles per pass, measured as 28% of the LDS
// busy cycles being bank conflicts.)  Rows of 128 bytes alternate bank halves
// by themselves; 2 (key & 3) keeps the chunk pairs apart within a half.
template <int D>
__device__ __forceinline__ int vswz(int key) {
  if constexpr (D >= 128)
    return 4 * (key & 3);
  else
    return 2 * (key & 3);
}

// A-operand row m of a 32-key tile -> key: row 8J + 4H + I is key 16(J/2) + 8H + 4(J%2) + I.
__device__ __forceinline__ int row_key(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// max / sum over the two 32-lane halves, broadcast to all lanes.
__device__ __forceinline__ float halves_max(float x) { return fmaxf(x, xor32(x)); }
__device__ __forceinline__ float halves_sum(float x) { return x + xor32(x); }

// Buffer descriptor for the rows kb .. min(sk, kb + rows) - 1 of one head (row
// stride ss elements): loads past the last valid element return zeros (the
// hardware range check of raw buffer loads is per dword).  Word 3 is the gfx9
// default.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t* g, int64_t ss, int kb,
                                                             int sk, int rows) {
  const int64_t last = (int64_t)min(sk - 1 - kb, rows - 1) * ss + D;  // elements to the end of the last row
  return __builtin_amdgcn_make_buffer_rsrc((void*)(g + (int64_t)kb * ss), 0, (int)(last * 2),
                                           0x00020000);
}

// 16 bytes per lane from a buffer into LDS at lds + 16 * lane (lds must be
// wave-uniform), and 16 bytes per lane into registers.  Kept out of lambdas:
// the host pass of the compiler drops the kernel stub when these builtins sit
// in a lambda body.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds,
                                                  uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, 0, 0, 0);
}
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voffset) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voffset, 0, 0));
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace exattn
