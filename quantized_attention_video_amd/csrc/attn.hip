// Fused INT8-QK / FP8-PV attention forward for gfx950.
//
// Numerical program: "research/vortex_exact_attention/PHASE2B_ALIGNED_REPORT.md",
// sections "Decision" and "Exactness" (INT32 scores converted to FP32, online softmax
// with per-epoch m and d over increasing 64-key epochs, E4M3 probability words, FP32
// rescale values, P.V accumulated into an FP32 running output, final reciprocal, BF16
// output), and the fused-mainloop description of "h3-blackwell-runtime/
// PERFORMANCE_ROADMAP.md" (QK and PV alternate on separate tensor sub-pipelines while the
// softmax occupies the vector pipes).  The pages' GB10 kernel is warp-specialised with
// mbarriers; this one is designed for CDNA4 instead:
//
//  * One workgroup = 8 waves = 256 queries of one (segment, head); each wave owns 32
//    queries, so two waves share a SIMD and the hardware overlaps one wave's softmax
//    (VALU) with the other's MFMAs.  Per wave the working set stays under 256 VGPRs.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_i32_32x32x32_i8: each lane
//    owns one query column and 32 of the epoch's 64 keys, so the row max and row sum are
//    in-lane plus one v_permlane32_swap between the two half-waves.
//  * The row max is taken on the INT32 accumulators (sigma > 0, and rounding is
//    monotone, so max_j fl32(acc_j*sigma) = fl32(max_j acc_j * sigma) exactly).  Each
//    accumulator is converted exactly to FP32 and one FMA, acc*sigma - (m' - log2 448),
//    gives the base-2 exponent of 448*P with a single rounding.  (Folding a large
//    constant into that FMA to skip the conversion perturbs P by ~1e-4..1e-3 per epoch,
//    enough to flip E4M3 roundings of the dominant keys in peaked rows.)
//  * The lane's 32 probabilities are packed with v_cvt_pk_fp8_f32 directly into the B
//    operand of v_mfma_f32_32x32x64_f8f6f4 (O^T += V^T P^T).  The V tile is stored by the
//    quantizer with its keys permuted to match, so no probability goes through LDS.
//  * K and V tiles (8 KiB each per epoch) are streamed into double-buffered LDS with
//    global_load_lds_dwordx4 (no VGPR staging); one barrier per epoch.
//  * The O rescale by alpha is skipped when no row of the wave changed its max (alpha is
//    then exactly 1, so skipping is bit-identical).
//  * Work items (segment, head, 256-query tile) are ordered so that consecutive
//    workgroups dispatched to one XCD take the same head and neighbouring query tiles,
//    so the 32 CUs of an XCD stream the same K/V tiles through their shared L2; packed
//    batches are ordered longest-first.
#include <limits.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace sattn {

constexpr int kWaves = 8;                  // waves per workgroup
constexpr int kQPerWG = kWaves * 32;       // queries per workgroup
constexpr int kQBlocksPerWG = kWaves / 2;  // 64-query blocks per workgroup
constexpr float kLog2_448 = 8.8073549220576041f;

int attn_queries_per_wg() { return kQPerWG; }

__device__ __forceinline__ int xhalf_max(int x) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float((int)r[0]) + __int_as_float((int)r[1]);
}

template <bool DUMP>
__global__ __launch_bounds__(kWaves * 64) void attn_fwd_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];  // [stage][K, V]
  __shared__ float s_vscale[kD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---------------------------------------------------------------- work item
  const int xcd = blockIdx.x & 7;
  const int64_t kk = blockIdx.x >> 3;
  const int nh = xcd < p.H ? (p.H - xcd + 7) / 8 : 0;
  if (nh == 0) return;
  int s;
  int64_t hl, qt;
  if (p.order == nullptr) {
    const int64_t ntile = (ceil_blocks(p.gq.L) + kQBlocksPerWG - 1) / kQBlocksPerWG;
    const int64_t per_seg = (int64_t)nh * ntile;
    if (per_seg == 0 || kk >= per_seg * p.nseg) return;
    s = (int)(kk / per_seg);
    const int64_t rem = kk - (int64_t)s * per_seg;
    hl = rem / ntile;
    qt = rem - hl * ntile;
  } else {
    if (kk >= (int64_t)p.tpref[p.nseg] * nh) return;
    int lo = 0, hi = p.nseg - 1;  // the sorted position whose tile range holds kk
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)p.tpref[mid] * nh <= kk) lo = mid; else hi = mid - 1;
    }
    const int64_t ntile = p.tpref[lo + 1] - p.tpref[lo];
    const int64_t rem = kk - (int64_t)p.tpref[lo] * nh;
    hl = rem / ntile;
    qt = rem - hl * ntile;
    s = p.order[lo];
  }
  const int h = xcd + 8 * (int)hl;
  const SegInfo qi = seg_info(p.gq, s, p.o_st);
  const SegInfo ki = seg_info(p.gk, s, 0);
  const int64_t nkb = ceil_blocks(ki.len);
  const int64_t qb = qt * kQBlocksPerWG + (wave >> 1);  // this wave's 64-query block
  const int hq = wave & 1;                              // and which 32 of its queries
  const bool active = qb < ceil_blocks(qi.len);
  const int g = lane >> 5, jq = lane & 31;

  if (tid < kD) s_vscale[tid] = p.v_scale[((int64_t)s * p.H + h) * kD + tid];

  // ---------------------------------------------------------------- Q operand (registers)
  v4i qop[4];
  float sig_q = 0.f;
  if (active) {
    const int8_t* qt_ptr = p.q8 + ((int64_t)h * p.qblk_cap + qi.blk0 + qb) * kTileBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) qop[u] = *reinterpret_cast<const v4i*>(qt_ptr + ((hq * 4 + u) * 64 + lane) * 16);
    sig_q = p.q_scale[(int64_t)h * p.qblk_cap + qi.blk0 + qb] * p.c32;  // fl32(q_scale * c)
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) qop[u] = v4i{0, 0, 0, 0};
  }

  const int64_t ktile0 = (int64_t)h * p.kblk_cap + ki.blk0;
  const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k8) + ktile0 * kTileBytes;
  const uint8_t* vg = p.v8 + ktile0 * kTileBytes;
  const float* ksc = p.k_scale + ktile0;

  // Each epoch moves 1024 16-byte chunks (K tile, then V tile); wave w, step j covers
  // chunks j*512 + w*64 + lane, which lie in one tile, so the LDS base is wave-uniform.
  auto issue = [&](int64_t e, int stage) {
#pragma unroll
    for (int j = 0; j < 1024 / (kWaves * 64); ++j) {
      const int c0 = j * kWaves * 64 + wave * 64;
      const int which = c0 >> 9, cw = c0 & 511;
      const uint8_t* src = (which ? vg : kg) + e * kTileBytes + (int64_t)(cw + lane) * 16;
      __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)&lds[stage][which][cw * 16], 16, 0, 0);
    }
  };

  float m = -INFINITY, dpart = 0.f;
  v16f oacc[4];
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[w][i] = 0.f;

  if (nkb > 0) issue(0, 0);
  __syncthreads();  // s_vscale visible even when there are no epochs
  for (int64_t e = 0; e < nkb; ++e) {
    const int st = (int)(e & 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // epoch e landed for every wave; every wave is done with epoch e-1
    if (e + 1 < nkb) issue(e + 1, st ^ 1);
    if (!active) continue;

    // ---------------- S^T = K Q^T (exact INT32)
    const uint8_t* Kl = lds[st][0];
    const uint8_t* Vl = lds[st][1];
    v16i acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v4i a = *reinterpret_cast<const v4i*>(Kl + ((t * 4 + u) * 64 + lane) * 16);
        acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qop[u], acc[t], 0, 0, 0);
      }
    }
    const float sig = sig_q * ksc[e];  // fl32(fl32(q_scale * c) * k_scale)
    const int64_t kvalid = ki.len - e * kBlk;
    const bool tail = kvalid < kBlk;

    if constexpr (DUMP) {
      if (s == p.dump_seg && h == p.dump_head) {
        const int64_t row = qb * kBlk + hq * 32 + jq;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
            if (row < qi.len && key < kvalid) {
              const int a = acc[t][r];
              p.dump_acc[row * p.dump_lk + e * kBlk + key] = a;
              p.dump_s[row * p.dump_lk + e * kBlk + key] = (float)a * sig;
            }
          }
      }
    }

    // ---------------- online softmax (base 2), row max on the integer accumulators
    int mx = INT_MIN;  // masked keys never win
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
        const int a = (tail && key >= kvalid) ? INT_MIN : acc[t][r];
        mx = max(mx, a);
      }
    mx = xhalf_max(mx);
    const float smax = (float)mx * sig;  // = max_j fl32(acc_j * sig)
    const float m_new = fmaxf(m, smax);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first epoch
    const float mm = m_new - kLog2_448;
    float psum = 0.f;
    v8i pb;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float pv[4];
#pragma unroll
        for (int r3 = 0; r3 < 4; ++r3) {
          const int r = 4 * q4 + r3;
          const int key = 32 * t + 8 * q4 + 4 * g + r3;
          float arg = __builtin_fmaf((float)acc[t][r], sig, -mm);
          if (tail && key >= kvalid) arg = -INFINITY;
          pv[r3] = __builtin_amdgcn_exp2f(arg);  // 448 * P
          psum += pv[r3];
        }
        int w01 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);
        w01 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], w01, true);
        pb[4 * t + q4] = w01;
      }
    dpart = dpart * alpha + psum;
    m = m_new;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[w][i] *= alpha;
    }

    // ---------------- O^T += V^T P^T (FP8 x FP8 -> FP32)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const v4i lo = *reinterpret_cast<const v4i*>(Vl + ((w * 2 + 0) * 64 + lane) * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(Vl + ((w * 2 + 1) * 64 + lane) * 16);
      const v8i a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      oacc[w] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, oacc[w], 0, 0, 0, 0, 0, 0);
    }
  }

  // ---------------------------------------------------------------- epilogue
  if (!active) return;
  const float dtot = xhalf_sum(dpart);  // = 448 * d
  const float inv = dtot > 0.f ? 1.0f / dtot : 0.f;
  const int64_t row = qb * kBlk + hq * 32 + jq;
  if (row >= qi.len) return;
  uint16_t* orow = p.o + qi.elem_base + row * p.o_st + (int64_t)h * p.o_sh;
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int c0 = 32 * w + 8 * q4 + 4 * g;
      uint32_t b[4];
#pragma unroll
      for (int r3 = 0; r3 < 4; ++r3) b[r3] = f32_to_bf16_bits((oacc[w][4 * q4 + r3] * inv) * s_vscale[c0 + r3]);
      *reinterpret_cast<uint2*>(orow + c0) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
    }
}

// ---------------------------------------------------------------------------- plan
// One workgroup orders packed segments by decreasing number of key blocks (the work of
// each of their query tiles; ties keep segment order) and writes the prefix sums of
// query tiles in that order.  Above 4096 segments the input order is kept.
constexpr int kPlanMax = 4096;
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                                                    int nseg, int64_t Lq_clip, int64_t Lk_clip,
                                                    int32_t* __restrict__ order, int32_t* __restrict__ tpref) {
  __shared__ int key[kPlanMax];
  __shared__ int ord[kPlanMax];
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const bool sorted = nseg <= kPlanMax;
  auto clip = [](int64_t x, int64_t L) { return x < 0 ? (int64_t)0 : (x > L ? L : x); };
  auto qtiles = [&](int sgm) {
    const int64_t a = clip(cu_q[sgm], Lq_clip), b = clip(cu_q[sgm + 1], Lq_clip);
    const int64_t n = b > a ? b - a : 0;
    return (int)((ceil_blocks(n) + kQBlocksPerWG - 1) / kQBlocksPerWG);
  };
  if (sorted) {
    for (int i = tid; i < nseg; i += 1024) {
      const int64_t a = clip(cu_k[i], Lk_clip), b = clip(cu_k[i + 1], Lk_clip);
      key[i] = (int)ceil_blocks(b > a ? b - a : 0);
    }
    __syncthreads();
    for (int i = tid; i < nseg; i += 1024) {
      int rank = 0;
      const int ki = key[i];
      for (int j = 0; j < nseg; ++j) rank += (key[j] > ki) || (key[j] == ki && j < i);
      ord[rank] = i;
    }
    __syncthreads();
  }
  const int per = (nseg + 1023) / 1024;
  const int lo = tid * per, hi = min(lo + per, nseg);
  int sum = 0;
  for (int j = lo; j < hi; ++j) sum += qtiles(sorted ? ord[j] : j);
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int j = lo; j < hi; ++j) {
    const int sgm = sorted ? ord[j] : j;
    order[j] = sgm;
    tpref[j] = run;
    run += qtiles(sgm);
  }
  if (tid == 1023) tpref[nseg] = part[1023];
}

hipError_t launch_plan(const int32_t* cu_q, const int32_t* cu_k, int nseg, int64_t Lq_clip, int64_t Lk_clip,
                       int32_t* order, int32_t* tpref, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, cu_q, cu_k, nseg, Lq_clip, Lk_clip, order, tpref);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, int64_t grid, bool dump, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (dump)
    hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sattn
