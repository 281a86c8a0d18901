// Quantization of Q, K, V for the INT8-QK / FP8-PV attention forward (gfx950).
//
// Follows the preparation phases that the pages "h3-blackwell-runtime/
// PERFORMANCE_ROADMAP.md" separate out for SageAttention 2.2.0 (K smoothing, Q/K INT8
// quantization, V transpose + FP8 quantization; the Sage2 decomposition paragraph and
// "Phase 4: Dense Sage-Compatible Attention").  All three passes are HBM-bound streams:
//
//   stats    : per (segment, head, chunk of tokens) FP64 sums of K and max|V| per channel
//   finalize : per (segment, head) fixed-order reduction -> k_mean, v_scale, 448/amax
//   quant_qk : per (64-token block, head) amax -> FP32 scale -> INT8 operand tile
//   quant_v  : per (64-token block, head) V * (448/amax) -> E4M3, transposed through LDS
//              into the channel-major operand tile of the P.V contraction
//
// Every rounding decision is a single correctly rounded IEEE operation (the library is
// built with -ffp-contract=off), and every reduction has a fixed order, so the outputs
// are deterministic and independent of the launch geometry.
#include "device_common.h"
#include "launch.h"

namespace sattn {

// ---------------------------------------------------------------------------- stats
// Grid (nchunk, nseg, H), 256 threads.  Thread (r = tid/16, c8 = tid%16) walks tokens
// r, r+16, ... of its chunk over channels 8*c8 .. 8*c8+7; the 16 partial rows are then
// summed in LDS in a fixed order.
__global__ __launch_bounds__(256) void stats_kernel(const uint16_t* __restrict__ k, SegGeom gk, int64_t k_st,
                                                    int64_t k_sh, const uint16_t* __restrict__ v, SegGeom gv,
                                                    int64_t v_st, int64_t v_sh, int H, int nchunk,
                                                    double* __restrict__ sums, float* __restrict__ vmax) {
  __shared__ double red_sum[16][kD];
  __shared__ float red_max[16][kD];
  const int tid = threadIdx.x, r = tid >> 4, c8 = tid & 15;
  const int chunk = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const SegInfo ki = seg_info(gk, s, k_st);
  const SegInfo vi = seg_info(gv, s, v_st);
  const int64_t t0 = ki.len * chunk / nchunk, t1 = ki.len * (chunk + 1) / nchunk;
  double acc[8];
  float mx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { acc[j] = 0.0; mx[j] = 0.f; }
  const uint16_t* kp = k + ki.elem_base + h * k_sh + 8 * c8;
  const uint16_t* vp = v + vi.elem_base + h * v_sh + 8 * c8;
  for (int64_t t = t0 + r; t < t1; t += 16) {
    float xk[8], xv[8];
    unpack8(*reinterpret_cast<const uint4*>(kp + t * k_st), xk);
    unpack8(*reinterpret_cast<const uint4*>(vp + t * v_st), xv);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[j] += (double)xk[j];
      mx[j] = fmaxf(mx[j], fabsf(xv[j]));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    red_sum[r][8 * c8 + j] = acc[j];
    red_max[r][8 * c8 + j] = mx[j];
  }
  __syncthreads();
  if (tid < kD) {
    double sacc = 0.0;
    float m = 0.f;
    for (int i = 0; i < 16; ++i) {
      sacc += red_sum[i][tid];
      m = fmaxf(m, red_max[i][tid]);
    }
    const int64_t o = (((int64_t)s * H + h) * nchunk + chunk) * kD + tid;
    sums[o] = sacc;
    vmax[o] = m;
  }
}

// ---------------------------------------------------------------------------- finalize
// Grid (nseg, H), 128 threads (one per channel).
__global__ __launch_bounds__(kD) void finalize_kernel(SegGeom gk, int H, int nchunk, const double* __restrict__ sums,
                                                      const float* __restrict__ vmax, float* __restrict__ k_mean,
                                                      float* __restrict__ v_scale, float* __restrict__ v_inv) {
  const int c = threadIdx.x, s = blockIdx.x, h = blockIdx.y;
  const SegInfo ki = seg_info(gk, s, 0);
  const int64_t base = ((int64_t)s * H + h) * nchunk * kD + c;
  double sum = 0.0;
  float amax = 0.f;
  for (int i = 0; i < nchunk; ++i) {
    sum += sums[base + (int64_t)i * kD];
    amax = fmaxf(amax, vmax[base + (int64_t)i * kD]);
  }
  const int64_t o = ((int64_t)s * H + h) * kD + c;
  k_mean[o] = ki.len > 0 ? (float)(sum / (double)ki.len) : 0.f;
  v_scale[o] = amax > 0.f ? amax / 448.0f : 0.f;
  v_inv[o] = amax > 0.f ? 448.0f / amax : 0.f;
}

// ---------------------------------------------------------------------------- Q / K
// Grid (blocks, H), 256 threads.  Thread tid handles rows r = tid/16 + 16*i (i < 4) and
// channels 8*(tid%16) .. +7 of the 64-token block: one 16-byte load per row.  Rows 0..31
// are i = 0, 1 and rows 32..63 are i = 2, 3, so with halves = 2 each 32-row half gets its
// own amax and scale (scale_out then holds two scales per block).
__global__ __launch_bounds__(256) void quant_qk_kernel(const uint16_t* __restrict__ x, SegGeom g, int64_t st,
                                                       int64_t sh, int H, const float* __restrict__ mean,
                                                       int8_t* __restrict__ out, float* __restrict__ scale_out,
                                                       int64_t blk_cap, int halves) {
  __shared__ float wmax[2][4];
  const int tid = threadIdx.x, c8 = tid & 15, h = blockIdx.y;
  const int64_t blk = blockIdx.x;
  SegInfo si;
  const int s = seg_of_block(g, blk, st, &si);
  if (s < 0) return;
  const int64_t t0 = (blk - si.blk0) * kBlk;
  const int64_t nvalid = si.len - t0 < kBlk ? si.len - t0 : kBlk;
  float mu[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mu[j] = mean ? mean[((int64_t)s * H + h) * kD + 8 * c8 + j] : 0.f;
  float xs[4][8];
  float am[2] = {0.f, 0.f};  // per 32-row half
  const uint16_t* base = x + si.elem_base + h * sh + 8 * c8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 4) + 16 * i;
    if (r < nvalid) {
      float raw[8];
      unpack8(*reinterpret_cast<const uint4*>(base + (t0 + r) * st), raw);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xs[i][j] = raw[j] - mu[j];  // K smoothing: one correctly rounded FP32 subtraction
        am[i >> 1] = fmaxf(am[i >> 1], fabsf(xs[i][j]));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[i][j] = 0.f;
    }
  }
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const float m = wave_max(am[f]);
    if ((tid & 63) == 0) wmax[f][tid >> 6] = m;
  }
  __syncthreads();
#pragma unroll
  for (int f = 0; f < 2; ++f) am[f] = fmaxf(fmaxf(wmax[f][0], wmax[f][1]), fmaxf(wmax[f][2], wmax[f][3]));
  if (halves == 1) am[0] = am[1] = fmaxf(am[0], am[1]);
  float scale[2], inv[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    scale[f] = am[f] > 0.f ? am[f] / 127.0f : 0.f;
    inv[f] = am[f] > 0.f ? 127.0f / am[f] : 0.f;
  }
  int8_t* tile = out + ((int64_t)h * blk_cap + blk) * kTileBytes;
  const int cbase = 8 * c8, g2 = cbase >> 6, u = (cbase & 63) >> 4, s0 = cbase & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 4) + 16 * i, t = r >> 5, ri = r & 31;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float qv = rintf(xs[i][j] * inv[i >> 1]);  // round half to even
      qv = fminf(fmaxf(qv, -127.f), 127.f);
      w[j >> 2] |= ((uint32_t)((int)qv) & 0xffu) << (8 * (j & 3));
    }
    const int off = ((t * 4 + u) * 64 + g2 * 32 + ri) * 16 + s0;
    *reinterpret_cast<uint2*>(tile + off) = make_uint2(w[0], w[1]);
  }
  if (tid < halves) scale_out[((int64_t)h * blk_cap + blk) * halves + tid] = scale[tid];
}

// ---------------------------------------------------------------------------- V
// Grid (blocks, H), 256 threads.  E4M3 codes are staged channel-major in LDS (rows padded
// to 68 bytes), then each thread emits two 16-byte chunks of the operand tile: chunk
// ((w*2 + f)*64 + g*32 + i) holds channel 32w+i, keys 32f + 8q + 4g + {0..3} (q = 0..3).
__global__ __launch_bounds__(256) void quant_v_kernel(const uint16_t* __restrict__ x, SegGeom g, int64_t st,
                                                      int64_t sh, int H, const float* __restrict__ v_inv,
                                                      uint8_t* __restrict__ out, int64_t blk_cap) {
  constexpr int kRow = 68;
  __shared__ __attribute__((aligned(16))) uint8_t tr[kD * kRow];
  const int tid = threadIdx.x, c8 = tid & 15, h = blockIdx.y;
  const int64_t blk = blockIdx.x;
  SegInfo si;
  const int s = seg_of_block(g, blk, st, &si);
  if (s < 0) return;
  const int64_t t0 = (blk - si.blk0) * kBlk;
  const int64_t nvalid = si.len - t0 < kBlk ? si.len - t0 : kBlk;
  float inv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) inv[j] = v_inv[((int64_t)s * H + h) * kD + 8 * c8 + j];
  const uint16_t* base = x + si.elem_base + h * sh + 8 * c8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 4) + 16 * i;
    float y[8];
    if (r < nvalid) {
      float raw[8];
      unpack8(*reinterpret_cast<const uint4*>(base + (t0 + r) * st), raw);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = raw[j] * inv[j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[j], y[j + 1], 0, false);  // OCP E4M3, RNE
      tr[(8 * c8 + j) * kRow + r] = (uint8_t)(pk & 0xff);
      tr[(8 * c8 + j + 1) * kRow + r] = (uint8_t)((pk >> 8) & 0xff);
    }
  }
  __syncthreads();
  uint8_t* tile = out + ((int64_t)h * blk_cap + blk) * kTileBytes;
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int chunk = tid + 256 * k2;
    const int w = chunk >> 7, f = (chunk >> 6) & 1, gg = (chunk >> 5) & 1, i = chunk & 31;
    const uint8_t* row = tr + (32 * w + i) * kRow + 32 * f + 4 * gg;
    uint4 o;
    o.x = *reinterpret_cast<const uint32_t*>(row + 0);
    o.y = *reinterpret_cast<const uint32_t*>(row + 8);
    o.z = *reinterpret_cast<const uint32_t*>(row + 16);
    o.w = *reinterpret_cast<const uint32_t*>(row + 24);
    *reinterpret_cast<uint4*>(tile + chunk * 16) = o;
  }
}

// ---------------------------------------------------------------------------- launchers
int stats_chunks(int nseg, int H) {
  const int64_t want = (4096 + (int64_t)nseg * H - 1) / ((int64_t)nseg * H);
  return (int)(want < 1 ? 1 : (want > 64 ? 64 : want));
}

hipError_t launch_quantize(const QuantLaunch& a, hipStream_t stream) {
  const int nchunk = stats_chunks(a.nseg, a.H);
  double* sums = reinterpret_cast<double*>(a.workspace);
  float* vmax = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + a.ws_sums_bytes);
  float* vinv = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + a.ws_sums_bytes + a.ws_vmax_bytes);
  hipLaunchKernelGGL(stats_kernel, dim3(nchunk, a.nseg, a.H), dim3(256), 0, stream, a.k, a.gk, a.k_st, a.k_sh, a.v,
                     a.gv, a.v_st, a.v_sh, a.H, nchunk, sums, vmax);
  hipLaunchKernelGGL(finalize_kernel, dim3(a.nseg, a.H), dim3(kD), 0, stream, a.gk, a.H, nchunk, sums, vmax,
                     a.k_mean, a.v_scale, vinv);
  if (a.q_blocks > 0)
    hipLaunchKernelGGL(quant_qk_kernel, dim3(a.q_blocks, a.H), dim3(256), 0, stream, a.q, a.gq, a.q_st, a.q_sh, a.H,
                       (const float*)nullptr, a.q8, a.q_scale, a.qblk_cap, 1 << a.q_scale_shift);
  if (a.k_blocks > 0) {
    hipLaunchKernelGGL(quant_qk_kernel, dim3(a.k_blocks, a.H), dim3(256), 0, stream, a.k, a.gk, a.k_st, a.k_sh, a.H,
                       (const float*)a.k_mean, a.k8, a.k_scale, a.kblk_cap, 1);
    hipLaunchKernelGGL(quant_v_kernel, dim3(a.k_blocks, a.H), dim3(256), 0, stream, a.v, a.gv, a.v_st, a.v_sh, a.H,
                       (const float*)vinv, a.v8, a.kblk_cap);
  }
  return hipGetLastError();
}

}  // namespace sattn
