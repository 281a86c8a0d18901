// Host-side launch descriptors shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"

namespace sattn {

struct QuantLaunch {
  const uint16_t *q, *k, *v;  // BF16 bits
  SegGeom gq, gk, gv;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;
  int nseg, H;
  int64_t q_blocks, k_blocks;  // grid extents over quantized blocks
  int8_t* q8;
  float* q_scale;
  int8_t* k8;
  float* k_scale;
  float* k_mean;
  uint8_t* v8;
  float* v_scale;
  int64_t qblk_cap, kblk_cap;
  int q_scale_shift;  // Q scales per 64-token block: 1 << q_scale_shift
  void* workspace;
  size_t ws_sums_bytes, ws_vmax_bytes;
};

// Checkpoint dump of one (segment, head) (sattn_debug_scores): sampled query rows
// q0, q0 + qstep, ... < q1 of the segment; row i of every buffer is the i-th sampled row.
struct DumpParams {
  int32_t* acc;  // [rows][ld] INT32 accumulators
  float* s;      // [rows][ld] FP32 scores
  int64_t ld;
  float *m, *d, *alpha;  // [rows][nep]
  uint8_t* p8;           // [rows][nep][64]
  float* ro;             // [rows][nep][128]
  int64_t nep;
  float* rcp;            // [rows]: the epilogue's 1 / (448 d)
  int seg, head;
  int64_t q0, q1, qstep;
  int64_t tile0;  // first query tile of the launch (workgroup b takes tile tile0 + b)
};

constexpr int kMaxPieces = 4;  // most workgroups one split tile's keys are shared by

struct AttnParams {
  const int8_t* q8;
  const float* q_scale;
  const int8_t* k8;
  const float* k_scale;
  const uint8_t* v8;
  const float* v_scale;
  int64_t qblk_cap, kblk_cap;
  int H, nseg;
  SegGeom gq;  // query side; stride_b is the output's batch stride
  SegGeom gk;  // key side
  const int32_t* order;  // varlen: segments by decreasing key blocks (nullptr: dense)
  const int32_t* tpref;  // varlen: prefix sums of query tiles in that order
  float c32;             // fl32(sm_scale * log2 e)
  uint16_t* o;
  int64_t o_st, o_sh;
  DumpParams dump;       // used by the checkpoint instantiation only
  int64_t max_kblocks;  // bound on any segment's key blocks (selects the K-scale path)
  int q_scale_shift;    // Q scales per 64-token block: 1 << q_scale_shift (1 or 2)
  const uint16_t* qbf;  // BF16 Q view quantized in the kernel (sattn_fwd_fused), else nullptr
  int64_t qb_sb, qb_st, qb_sh;  // its batch, token and head element strides
  // Key split (dense problems whose grid leaves CUs idle): the epochs of each split tile
  // are shared by `split` workgroups (pieces), which merge their partial results; 1 = no
  // split.  Piece q takes epochs [split_e[q], split_e[q + 1]) (split_e[0] = 0, the last
  // piece runs to the segment's end, the partial last epoch included).
  int split;
  int split_e[kMaxPieces];
  // Per-XCD work index from which tiles are split (0: every tile); the pieces of split tile
  // j are the blocks 8 * (split_from + split * j + q) + xcd, and the tile uses the counter
  // and partials at index min(H, 8) j + xcd.
  int64_t split_from;
  float* part;   // [tile][piece][wave][17][lane] float4: partial O (16) and (m, d) of each piece
  int32_t* cnt;  // [tile]: finished pieces; zero between calls
};

// One piece of a split tile: per wave and lane, 16 float4 of O accumulators and one (m, d).
constexpr int kSplitPieceBytes = 4 * 17 * 64 * 16;
// Bytes of the key-split workspace for `tiles` query tiles of `pieces` pieces each
// (counters, then partials).
inline size_t split_ws_bytes(int64_t tiles, int pieces) {
  const size_t cnt = ((size_t)tiles * 4 + 255) / 256 * 256;
  return cnt + (size_t)tiles * pieces * kSplitPieceBytes;
}

int stats_chunks(int nseg, int H);
hipError_t launch_quantize(const QuantLaunch& a, hipStream_t stream);

// Queries per workgroup of the attention kernel and its grid extent.
int attn_queries_per_wg();
hipError_t launch_plan(const int32_t* cu_q, const int32_t* cu_k, int nseg, int64_t Lq_clip, int64_t Lk_clip,
                       int32_t* order, int32_t* tpref, hipStream_t stream);
hipError_t launch_attention(const AttnParams& p, int64_t grid, bool dump, hipStream_t stream);

}  // namespace sattn
