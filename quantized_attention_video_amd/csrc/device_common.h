// Device-side helpers shared by the quantization and attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sattn {

constexpr int kD = 128;           // head dimension
constexpr int kBlk = 64;          // tokens per quantization block and keys per softmax epoch
constexpr int kTileBytes = 8192;  // one 64-token x 128-channel INT8/E4M3 tile

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Where one sequence (segment) lives.  Dense problems have nseg equal-length segments;
// packed (varlen) problems take their bounds from device prefix sums.
struct SegGeom {
  const int32_t* cu;  // device [nseg+1] prefix sums, or nullptr for dense
  int nseg;
  int64_t L;          // dense: tokens per segment; varlen: tokens held by the tensor view
  int64_t stride_b;   // dense only: elements between segments of the BF16 view
};

struct SegInfo {
  int64_t len;        // valid tokens
  int64_t tok_base;   // dense: 0; varlen: first packed token of the segment
  int64_t elem_base;  // element offset of token 0 in the BF16 view (before head/channel)
  int64_t blk0;       // first 64-token block of the segment in the quantized buffers
};

__device__ __forceinline__ int64_t ceil_blocks(int64_t n) { return (n + kBlk - 1) / kBlk; }

// Segment s, clipped to the tokens the view actually holds.
__device__ __forceinline__ SegInfo seg_info(const SegGeom& g, int s, int64_t stride_t) {
  SegInfo r;
  if (g.cu == nullptr) {
    r.len = g.L;
    r.tok_base = (int64_t)s * g.L;
    r.elem_base = (int64_t)s * g.stride_b;
    r.blk0 = (int64_t)s * ceil_blocks(g.L);
  } else {
    int64_t a = g.cu[s], b = g.cu[s + 1];
    a = a < 0 ? 0 : (a > g.L ? g.L : a);
    b = b < a ? a : (b > g.L ? g.L : b);
    r.len = b - a;
    r.tok_base = a;
    r.elem_base = a * stride_t;
    r.blk0 = a / kBlk + s;
  }
  return r;
}

// Segment holding quantized block `blk`, or -1 for a block in a gap between segments.
__device__ __forceinline__ int seg_of_block(const SegGeom& g, int64_t blk, int64_t stride_t, SegInfo* out) {
  int s;
  if (g.cu == nullptr) {
    int64_t nb = ceil_blocks(g.L);
    if (nb == 0) return -1;
    s = (int)(blk / nb);
    if (s >= g.nseg) return -1;
  } else {
    int lo = 0, hi = g.nseg - 1;  // largest s with cu[s]/64 + s <= blk
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      int64_t c = g.cu[mid];
      c = c < 0 ? 0 : (c > g.L ? g.L : c);
      if (c / kBlk + mid <= blk) lo = mid; else hi = mid - 1;
    }
    s = lo;
  }
  *out = seg_info(g, s, stride_t);
  if (blk < out->blk0 || blk >= out->blk0 + ceil_blocks(out->len)) return -1;
  return s;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight BF16 values (16 bytes) → float.
__device__ __forceinline__ void unpack8(const uint4& raw, float x[8]) {
  x[0] = bf16_lo(raw.x); x[1] = bf16_hi(raw.x);
  x[2] = bf16_lo(raw.y); x[3] = bf16_hi(raw.y);
  x[4] = bf16_lo(raw.z); x[5] = bf16_hi(raw.z);
  x[6] = bf16_lo(raw.w); x[7] = bf16_hi(raw.w);
}

// Two FP32 values rounded to BF16 (nearest, ties to even), packed low | high << 16: one
// v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace sattn
