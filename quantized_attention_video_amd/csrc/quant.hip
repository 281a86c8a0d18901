// Quantization of Q, K, V for the INT8-QK / FP8-PV attention forward (gfx950).
//
// Follows the preparation phases that the "H3 Performance Roadmap" page separates out
// for SageAttention 2.2.0 (K smoothing, Q/K INT8 quantization, V transpose + FP8
// quantization; the Sage2 decomposition paragraph and "Phase 4: Dense Sage-Compatible
// Attention").  All three passes are HBM-bound streams:
//
//   stats_q  : per (segment, head, chunk of tokens) FP64 sums of K and max|V| per channel;
//              in the same launch, per (64-token Q block, head) amax -> FP32 scale(s) ->
//              INT8 operand tile
//   finalize : per (segment, head) fixed-order reduction -> k_mean, v_scale, 448/amax
//   quant_kv : per (64-token block, head) K - k_mean -> amax -> FP32 scale -> INT8 tile,
//              and V * (448/amax) -> E4M3, transposed through LDS into the channel-major
//              operand tile of the P.V contraction
//
// Every rounding decision is a single correctly rounded IEEE operation (the library is
// built with -ffp-contract=off), and every reduction has a fixed order, so the outputs
// are deterministic and independent of the launch geometry.
#include "device_common.h"
#include "launch.h"

namespace sattn {

// ------------------------------------------------------------------ one 64-token block
// 256 threads.  Thread tid holds rows r = tid/16 + 16*i (i < 4), channels 8*(tid%16) .. +7
// of the block: one 16-byte load per row (rows past the segment's end read as absent).
struct BlockRows {
  uint4 raw[4];
  int64_t nvalid;
};

__device__ __forceinline__ BlockRows load_block(const uint16_t* base, int64_t st, int64_t t0, int64_t nvalid,
                                                int tid) {
  BlockRows b;
  b.nvalid = nvalid;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 4) + 16 * i;
    b.raw[i] = r < nvalid ? *reinterpret_cast<const uint4*>(base + (t0 + r) * st) : make_uint4(0, 0, 0, 0);
  }
  return b;
}

// Q or K: x - mean (K smoothing; mean = nullptr for Q), amax per 32-row half -> FP32 scale
// -> INT8 codes into the tile.  Rows 0..31 are i = 0, 1 and rows 32..63 are i = 2, 3, so
// with halves = 2 each 32-row half gets its own amax and scale (two scales per block).
__device__ __forceinline__ void emit_qk(const BlockRows& b, const float* mu, int8_t* tile, float* scale_out,
                                        int halves, int tid, float (*wmax)[4]) {
  const int c8 = tid & 15;
  float xs[4][8];
  float am[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 4) + 16 * i;
    if (r < b.nvalid) {
      float raw[8];
      unpack8(b.raw[i], raw);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xs[i][j] = raw[j] - mu[j];  // one correctly rounded FP32 subtraction (0 for Q)
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
    inv[f] = 127.0f / am[f];
    // amax 0, or so small that the reciprocal overflows: a zero block (scale 0, codes 0)
    const bool zero = !(am[f] > 0.f) || isinf(inv[f]);
    scale[f] = zero ? 0.f : am[f] / 127.0f;
    inv[f] = zero ? 0.f : inv[f];
  }
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
  if (tid < halves) scale_out[tid] = scale[tid];
}

// V: x * (448 / amax_channel) -> E4M3 codes, staged channel-major in LDS (rows padded to
// 68 bytes); then each thread emits two 16-byte chunks of the operand tile: chunk
// ((w*2 + f)*64 + g*32 + i) holds channel 32w+i, keys 32f + 8q + 4g + {0..3} (q = 0..3).
constexpr int kVRow = 68;
__device__ __forceinline__ void emit_v(const BlockRows& b, const float* inv, uint8_t* tile, int tid, uint8_t* tr) {
  const int c8 = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 4) + 16 * i;
    float y[8];
    if (r < b.nvalid) {
      float raw[8];
      unpack8(b.raw[i], raw);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = raw[j] * inv[j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[j], y[j + 1], 0, false);  // OCP E4M3, RNE
      tr[(8 * c8 + j) * kVRow + r] = (uint8_t)(pk & 0xff);
      tr[(8 * c8 + j + 1) * kVRow + r] = (uint8_t)((pk >> 8) & 0xff);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int chunk = tid + 256 * k2;
    const int w = chunk >> 7, f = (chunk >> 6) & 1, gg = (chunk >> 5) & 1, i = chunk & 31;
    const uint8_t* row = tr + (32 * w + i) * kVRow + 32 * f + 4 * gg;
    uint4 o;
    o.x = *reinterpret_cast<const uint32_t*>(row + 0);
    o.y = *reinterpret_cast<const uint32_t*>(row + 8);
    o.z = *reinterpret_cast<const uint32_t*>(row + 16);
    o.w = *reinterpret_cast<const uint32_t*>(row + 24);
    *reinterpret_cast<uint4*>(tile + chunk * 16) = o;
  }
}

// ------------------------------------------------------------------ statistics and Q
// Statistics of one (chunk of tokens, segment, head), 256 threads: thread (r = tid/16,
// c8 = tid%16) walks tokens r, r+16, ... of the chunk over channels 8*c8 .. 8*c8+7,
// summing K in FP64 and taking max|V|; the 16 partial rows are then combined in LDS in a
// fixed order into one FP64 sum and one maximum per channel.
__device__ __forceinline__ void stats_chunk(const uint16_t* __restrict__ k, const SegGeom& gk, int64_t k_st,
                                            int64_t k_sh, const uint16_t* __restrict__ v, const SegGeom& gv,
                                            int64_t v_st, int64_t v_sh, int H, int nchunk, int chunk, int s, int h,
                                            double* __restrict__ sums, float* __restrict__ vmax,
                                            double (*red_sum)[kD], float (*red_max)[kD]) {
  const int tid = threadIdx.x, r = tid >> 4, c8 = tid & 15;
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

// One launch does the K/V statistics and all of Q (which needs no statistics), so the two
// streams share the memory system.  1-D grid of 256-thread blocks: blocks [0, n_stats)
// are (chunk, segment, head) with the chunk fastest; the rest are (Q block, head) with the
// block fastest.
struct StatsQArgs {
  const uint16_t *k, *v, *q;
  SegGeom gk, gv, gq;
  int64_t k_st, k_sh, v_st, v_sh, q_st, q_sh;
  int H, nchunk;
  int64_t n_stats, q_blocks;
  double* sums;
  float* vmax;
  int8_t* q8;
  float* q_scale;
  int64_t qblk_cap;
  int halves;  // Q scales per 64-token block
};

__global__ __launch_bounds__(256) void stats_q_kernel(StatsQArgs a) {
  __shared__ double red_sum[16][kD];
  __shared__ float red_max[16][kD];
  __shared__ float wmax[2][4];
  const int64_t b = blockIdx.x;
  if (b < a.n_stats) {
    const int chunk = (int)(b % a.nchunk);
    const int s = (int)((b / a.nchunk) % a.gk.nseg), h = (int)(b / a.nchunk / a.gk.nseg);
    stats_chunk(a.k, a.gk, a.k_st, a.k_sh, a.v, a.gv, a.v_st, a.v_sh, a.H, a.nchunk, chunk, s, h, a.sums, a.vmax,
                red_sum, red_max);
    return;
  }
  const int tid = threadIdx.x;
  const int64_t blk = (b - a.n_stats) % a.q_blocks;
  const int h = (int)((b - a.n_stats) / a.q_blocks);
  SegInfo si;
  if (seg_of_block(a.gq, blk, a.q_st, &si) < 0) return;
  const int64_t t0 = (blk - si.blk0) * kBlk;
  const int64_t nvalid = si.len - t0 < kBlk ? si.len - t0 : kBlk;
  const BlockRows rows = load_block(a.q + si.elem_base + h * a.q_sh + 8 * (tid & 15), a.q_st, t0, nvalid, tid);
  const float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int64_t tb = (int64_t)h * a.qblk_cap + blk;
  emit_qk(rows, zero, a.q8 + tb * kTileBytes, a.q_scale + tb * a.halves, a.halves, tid, wmax);
}

// ---------------------------------------------------------------------------- finalize
// Grid (nseg, H), 1024 threads: channel c = tid % 128 and part p = tid / 128 reduce
// chunks p, p+8, ...; the eight parts are then combined in order.
constexpr int kFinParts = 8;
__global__ __launch_bounds__(kD * kFinParts) void finalize_kernel(SegGeom gk, int H, int nchunk,
                                                                  const double* __restrict__ sums,
                                                                  const float* __restrict__ vmax,
                                                                  float* __restrict__ k_mean,
                                                                  float* __restrict__ v_scale,
                                                                  float* __restrict__ v_inv) {
  __shared__ double red_sum[kFinParts][kD];
  __shared__ float red_max[kFinParts][kD];
  const int c = threadIdx.x & (kD - 1), part = threadIdx.x / kD, s = blockIdx.x, h = blockIdx.y;
  const int64_t base = ((int64_t)s * H + h) * nchunk * kD + c;
  double sum = 0.0;
  float amax = 0.f;
  for (int i0 = part; i0 < nchunk; i0 += kFinParts * 8) {  // eight loads in flight, summed in order
    double sv[8];
    float mv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + kFinParts * u;
      sv[u] = i < nchunk ? sums[base + (int64_t)i * kD] : 0.0;
      mv[u] = i < nchunk ? vmax[base + (int64_t)i * kD] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sum += sv[u];
      amax = fmaxf(amax, mv[u]);
    }
  }
  red_sum[part][c] = sum;
  red_max[part][c] = amax;
  __syncthreads();
  if (part != 0) return;
  for (int i = 1; i < kFinParts; ++i) {
    sum += red_sum[i][c];
    amax = fmaxf(amax, red_max[i][c]);
  }
  const SegInfo ki = seg_info(gk, s, 0);
  const int64_t o = ((int64_t)s * H + h) * kD + c;
  k_mean[o] = ki.len > 0 ? (float)(sum / (double)ki.len) : 0.f;
  const float inv = 448.0f / amax;
  const bool zero = !(amax > 0.f) || isinf(inv);  // as for INT8 blocks: a zero channel
  v_scale[o] = zero ? 0.f : amax / 448.0f;
  v_inv[o] = zero ? 0.f : inv;
}

// ---------------------------------------------------------------------------- K and V
// Grid (blocks, H), 256 threads.  The K and V rows of the block are both requested
// before either is converted.
__global__ __launch_bounds__(256) void quant_kv_kernel(const uint16_t* __restrict__ k, SegGeom gk, int64_t k_st,
                                                       int64_t k_sh, const uint16_t* __restrict__ v, SegGeom gv,
                                                       int64_t v_st, int64_t v_sh, int H,
                                                       const float* __restrict__ mean,
                                                       const float* __restrict__ v_inv, int8_t* __restrict__ k8,
                                                       float* __restrict__ k_scale, uint8_t* __restrict__ v8,
                                                       int64_t blk_cap) {
  __shared__ float wmax[2][4];
  __shared__ __attribute__((aligned(16))) uint8_t tr[kD * kVRow];
  const int tid = threadIdx.x, c8 = tid & 15, h = blockIdx.y;
  const int64_t blk = blockIdx.x;
  SegInfo ki, vi;
  const int s = seg_of_block(gk, blk, k_st, &ki);
  if (s < 0) return;
  vi = seg_info(gv, s, v_st);
  const int64_t t0 = (blk - ki.blk0) * kBlk;
  const int64_t nvalid = ki.len - t0 < kBlk ? ki.len - t0 : kBlk;
  const BlockRows bk = load_block(k + ki.elem_base + h * k_sh + 8 * c8, k_st, t0, nvalid, tid);
  const BlockRows bv = load_block(v + vi.elem_base + h * v_sh + 8 * c8, v_st, t0, nvalid, tid);
  const int64_t sh = ((int64_t)s * H + h) * kD + 8 * c8;
  float mu[8], inv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mu[j] = mean[sh + j];
    inv[j] = v_inv[sh + j];
  }
  const int64_t tb = (int64_t)h * blk_cap + blk;
  emit_qk(bk, mu, k8 + tb * kTileBytes, k_scale + tb, 1, tid, wmax);
  emit_v(bv, inv, v8 + tb * kTileBytes, tid, tr);
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
  StatsQArgs s;
  s.k = a.k; s.v = a.v; s.q = a.q;
  s.gk = a.gk; s.gv = a.gv; s.gq = a.gq;
  s.k_st = a.k_st; s.k_sh = a.k_sh; s.v_st = a.v_st; s.v_sh = a.v_sh; s.q_st = a.q_st; s.q_sh = a.q_sh;
  s.H = a.H;
  s.nchunk = nchunk;
  s.n_stats = (int64_t)nchunk * a.nseg * a.H;
  s.q_blocks = a.q_blocks;
  s.sums = sums;
  s.vmax = vmax;
  s.q8 = a.q8;
  s.q_scale = a.q_scale;
  s.qblk_cap = a.qblk_cap;
  s.halves = 1 << a.q_scale_shift;
  hipLaunchKernelGGL(stats_q_kernel, dim3((uint32_t)(s.n_stats + a.q_blocks * a.H)), dim3(256), 0, stream, s);
  hipLaunchKernelGGL(finalize_kernel, dim3(a.nseg, a.H), dim3(kD * kFinParts), 0, stream, a.gk, a.H, nchunk, sums,
                     vmax, a.k_mean, a.v_scale, vinv);
  if (a.k_blocks > 0)
    hipLaunchKernelGGL(quant_kv_kernel, dim3(a.k_blocks, a.H), dim3(256), 0, stream, a.k, a.gk, a.k_st, a.k_sh, a.v,
                       a.gv, a.v_st, a.v_sh, a.H, (const float*)a.k_mean, (const float*)vinv, a.k8, a.k_scale, a.v8,
                       a.kblk_cap);
  return hipGetLastError();
}

}  // namespace sattn
