// Device-side building blocks for the gfx950 attention kernels: vector
// types, the bf16 MFMA, raw buffer loads with hardware bounds checking,
// exp2, cross-half wave reductions and the XCD-aware block remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace av {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Word 3 of a raw (stride 0) buffer resource on gfx9-family GPUs.
constexpr uint32_t kBufferWord3 = 0x00020000u;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Buffer resource over [base, base + bytes).  Loads at offsets >= bytes
// return zero, which is how ragged tails are read without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

__device__ __forceinline__ i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).  Output layout used by the
// kernels: lane l holds column n = l % 32 and rows
//   m = 8 * (j / 4) + 4 * (l / 32) + (j % 4),  j = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane r supplies the address of 4 consecutive 16-bit values (row r of a
// 16 x 4 block M); lane i receives M[i/4][i%4], M[4+i/4][i%4], M[8+i/4][i%4],
// M[12+i/4][i%4].  Pointing lane r at V[k0 + r/4][c0 + 4*(r%4)] of a
// row-major tile therefore hands lane i the four values V[k0..k0+3][c0 + i]:
// a column of V, which is what a B-transposed MFMA operand needs.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Sum of two bf16 values accumulated in fp32 (v_dot2_f32_bf16 against 1, 1).
__device__ __forceinline__ float add_bf16_pair(bf16x2 p, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
}

__device__ __forceinline__ float uniform_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
__device__ __forceinline__ bool any_lane(bool b) { return __builtin_amdgcn_ballot_w64(b) != 0; }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// max / sum of a value with the value held by lane l ^ 32 (one
// v_permlane32_swap plus one ALU op), result in every lane.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// sum over all 64 lanes (butterfly), result in every lane
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Workgroups are handed to the 8 XCDs round-robin by block id.  Remap so
// that XCD x processes one contiguous range of logical tiles: neighbouring
// logical tiles (the same batch and head, hence the same K/V) then share
// that XCD's L2.  Bijective on [0, total).
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = pid & 7, i = pid >> 3;
  return x * q + (x < r ? x : r) + i;
}

// Logical tile of workgroup pid for grids whose query tiles differ in cost
// (causal and PrefixLM masks; mt_lin = 0 is the heaviest tile of a head).
// When the (batch, head) count is a multiple of 8, XCD x owns heads
// [x*G, (x+1)*G) as under xcd_remap, but receives their tiles heaviest first
// across all G heads: its CUs then take work in longest-first order, where
// head after head (heavy to light within each) leaves a long tail of heavy
// tiles that start late.  Otherwise the order of xcd_remap.
struct TileIdx {
  int bh, mt_lin;
};
__device__ __forceinline__ TileIdx weighted_tile(int pid, int total, int nM) {
  const int BH = total / nM;
  if ((BH & 7) == 0) {
    const int G = BH >> 3, x = pid & 7, i = pid >> 3;
    return {x * G + i % G, i / G};
  }
  const int L = xcd_remap(pid, total);
  return {L / nM, L % nM};
}

// First index in [0, n) whose value exceeds `target` in a non-decreasing
// int row (n when none).  All 64 lanes of the wave cooperate: each round
// probes 64 evenly spaced positions and keeps the gap where the predicate
// flips, so a 16k row needs three dependent loads.
__device__ __forceinline__ int wave_upper_bound(const int* row, int n, int target) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n;
  while (lo < hi) {
    const long long len = hi - lo;
    const int pos = lo + (int)((len * lane) >> 6);
    const bool le = row[pos] <= target;
    const unsigned long long bal = __ballot(le);
    const int c = __popcll(bal);
    if (c == 0) {
      hi = lo;
      break;
    }
    const int p_prev = lo + (int)((len * (c - 1)) >> 6);
    const int p_next = c < 64 ? lo + (int)((len * c) >> 6) : hi;
    lo = p_prev + 1;
    hi = p_next;
  }
  return hi;
}

__device__ __forceinline__ int wave_lower_bound(const int* row, int n, int target) {
  return wave_upper_bound(row, n, target - 1);
}

}  // namespace av
