// Device-side helpers shared by the attention kernels (forward and backward).
// Internal header: included only by the kernel sources of libattn.so.
#ifndef ATTN_DEVICE_H_
#define ATTN_DEVICE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per work-group
constexpr int kXcds = 8;          // MI355X: 8 accelerator complex dies, one L2 each

__device__ __forceinline__ float wave_max_pair(float x) {
  return fmaxf(x, __shfl_xor(x, 32, 64));
}

// Lanes l and l ^ 32 hold the two halves of one query row: after
// v_permlane32_swap the two results hold x of lane l and of lane l ^ 32 (in
// some order), so their max / sum is the pair's.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer resource over [base, base + bytes): loads at or past `bytes`
// return zero (hardware range check), which zero-fills keys past the valid
// length without a branch.  Word 3 = 0x00020000: the gfx9 data-format field
// for untyped dword loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Work-group id -> (b*h + head, query tile).  The hardware hands consecutive
// work-group ids to the 8 XCDs in turn; remap so each XCD receives a
// contiguous range of logical ids, i.e. all query tiles of a (b, head) land on
// the same XCD and share K/V through its L2.  Causal tiles run longest first.
__device__ __forceinline__ void tile_of_block(int n_qtiles, bool causal, int& bh, int& qt) {
  const int pid = blockIdx.x;
  const int G = gridDim.x;
  const int xcd = pid % kXcds, idx = pid / kXcds;
  const int per = G / kXcds, rem = G % kXcds;
  const int wg = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  bh = wg / n_qtiles;
  qt = wg - bh * n_qtiles;
  if (causal) qt = n_qtiles - 1 - qt;
}

__device__ __forceinline__ int clamp_len(const int32_t* key_lens, int b, int Tk) {
  int L = key_lens[b];
  return L < 0 ? 0 : (L > Tk ? Tk : L);
}

// Running-max update threshold (log2 units).  The accumulator is rescaled only
// when some row's tile maximum exceeds the reference maximum by more than
// this; otherwise the stale reference is kept and the probabilities are at
// most 2^8 (exact softmax either way: the reference cancels in O / l).
constexpr float kRescaleThreshold = 8.0f;

// key slot order: slot s of a 32-key slice holds key sigma(s) (bits 2 and 3 swapped)
__device__ __forceinline__ int sigma32(int s) { return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1); }

// LDS tiles of K and V are D*2-byte rows of 16-byte chunks, written by
// direct-to-LDS buffer loads (lane l of a load fills bytes 16 l of a 1 KB
// block) and stored XOR-swizzled: physical chunk = logical chunk ^ swz(row).
// K rows are in key-slot order (row 32 hh + s holds key 32 hh + sigma(s)), so
// the A-operand read of S^T is row c for lane c; the swizzle spreads the 16
// lanes that read one chunk column over 16 different chunks.  V rows are in
// key order; the swizzle makes the transposed reads (4 rows x 4 chunks per 16
// lanes) hit distinct chunks.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  r &= 31;
  return D == 128 ? (r & 15) : ((r ^ (r >> 3)) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return D == 128 ? 2 * (r & 3) : 2 * ((r >> 1) & 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from buffer offset `off` straight into LDS at dst + 16 * lane
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
}
// 4 bytes per lane from buffer offset `off` into LDS at dst + 4 * lane
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, off, 0, 0, 0);
}

// Swizzle for tiles read both ways -- 16-byte fragment reads of rows in
// sigma order (ds_read_b128) and transposed reads of 4 consecutive rows
// (ds_read_b64_tr_b16): a permutation of the row's low bits onto the chunk
// index that keeps both patterns free of LDS bank conflicts.
template <int D>
__device__ __forceinline__ int dual_swz(int r) {
  r &= 15;
  if constexpr (D == 128) return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8);
  return (((r >> 1) & 1) << 1) | ((r >> 2) & 1) | ((r >> 1) & 4);
}

// Work-group barrier for the K/V pipeline: first wait until at most N of
// this wave's vector-memory operations (the direct-to-LDS prefetches issued
// last) are outstanding and all its LDS reads have returned, then s_barrier.
// A plain __syncthreads() would also wait for the newest prefetch (its
// release fence covers the LDS writes those loads make).
template <int N>
__device__ __forceinline__ void pipeline_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));   // vmcnt N, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
}

// calls f(integral_constant<int, U>) for U = U0 .. UN-1
template <int U0, int UN, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (U0 < UN) {
    f(std::integral_constant<int, U0>{});
    static_for<U0 + 1, UN>(f);
  }
}

}  // namespace attn

#endif  // ATTN_DEVICE_H_
