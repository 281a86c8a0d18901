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
  int32_t* dump_acc;
  float* dump_s;
  int dump_seg, dump_head;
  int64_t dump_lk;
  int64_t max_kblocks;  // bound on any segment's key blocks (selects the K-scale path)
  int q_scale_shift;    // Q scales per 64-token block: 1 << q_scale_shift (1 or 2)
  const uint16_t* qbf;  // BF16 Q view quantized in the kernel (sattn_fwd_fused), else nullptr
  int64_t qb_sb, qb_st, qb_sh;  // its batch, token and head element strides
};

int stats_chunks(int nseg, int H);
hipError_t launch_quantize(const QuantLaunch& a, hipStream_t stream);

// Queries per workgroup of the attention kernel and its grid extent.
int attn_queries_per_wg();
hipError_t launch_plan(const int32_t* cu_q, const int32_t* cu_k, int nseg, int64_t Lq_clip, int64_t Lk_clip,
                       int32_t* order, int32_t* tpref, hipStream_t stream);
hipError_t launch_attention(const AttnParams& p, int64_t grid, bool dump, hipStream_t stream);

}  // namespace sattn
