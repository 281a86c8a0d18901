// Fused INT8-QK / FP8-PV attention forward for gfx950.
//
// Numerical program: the "Phase 2B Aligned Numerical Prototype" report, sections
// "Decision" and "Exactness" (INT32 scores converted to FP32, online softmax with
// per-epoch m and d over increasing 64-key epochs, E4M3 probability words, FP32 rescale
// values, P.V accumulated into an FP32 running output, final reciprocal, BF16 output), and
// the fused-mainloop description of the "H3 Performance Roadmap" (QK and PV alternate on
// separate tensor sub-pipelines while the softmax occupies the vector pipes).  The pages' GB10 kernel is warp-specialised with
// mbarriers; this one is designed for CDNA4 instead:
//
//  * One workgroup = 4 waves = 128 queries of one (segment, head); two workgroups share a
//    CU, so each SIMD runs two waves of up to 256 VGPRs.  Each wave owns 32 queries end to
//    end: Q operand, scores, running max and denominator, and the FP32 O accumulators.
//    The softmax's vector work (about five VALU instructions per score: a subtraction,
//    an FMA, an exponential, an add, half an FP8 pack and half a three-input max) is the
//    binding resource; the MFMA work runs beside it.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_i32_32x32x32_i8: each lane
//    owns one query column and 32 of the epoch's 64 keys, so the row max and row sum are
//    in-lane plus one v_permlane32_swap between the two half-waves.
//  * The row max is taken on the INT32 accumulators (sigma > 0, and rounding is
//    monotone, so max_j fl32(acc_j*sigma) = fl32(max_j acc_j * sigma) exactly).  The
//    accumulators start at the bit pattern of 1.5 * 2^23, so each one read as FP32 minus
//    1.5 * 2^23 is the exact accumulator value (one subtraction, no conversion), and one
//    FMA, acc*sigma - (m' - log2 448), gives the base-2 exponent of 448*P with a single
//    rounding.  (Folding the 1.5 * 2^23 * sigma term into that FMA instead perturbs P by
//    ~1e-4..1e-3, enough to flip E4M3 roundings of the dominant keys in peaked rows.)
//  * The lane's 32 probabilities are packed with v_cvt_pk_fp8_f32 directly into the B
//    operand of v_mfma_f32_32x32x64_f8f6f4 (O^T += V^T P^T).  The V tile is stored by the
//    quantizer with its keys permuted to match, so no probability goes through LDS.
//  * K and V tiles (8 KiB each per epoch) stream into three-slot LDS rings with
//    global_load_lds_dwordx4 (no VGPR staging), two epochs ahead of their use; one
//    barrier per epoch.  The softmax of epoch e runs in eight groups of four
//    probabilities, each led by one MFMA: the P.V MFMAs of epoch e-1, then, once a score
//    tile of epoch e is consumed, the QK MFMAs of epoch e+1 into the same registers.  No
//    MFMA result is waited for inside a step, and matrix cores and vector ALUs work at
//    the same time.
//  * The segment's K block scales and the head's V channel scales are copied to LDS in
//    the prologue, whose first requests are the K/V tiles (no scalar load in flight
//    during a step, no global load in the epilogue).  With sattn_fwd_fused the workgroup
//    also quantizes its own queries from the BF16 view, with the quantizer's arithmetic.
//  * The O rescale by alpha runs only in the lanes whose row max changed, and not at all
//    when no row of the wave changed (alpha is then exactly 1, so skipping is
//    bit-identical).
//  * Key split (a workspace given; the tiles of a short last dispatch round, whose halves
//    then run on CUs of their own): two workgroups share a tile's keys; the second first
//    takes the running max over the first half's scores, so every probability word is
//    the sequential recurrence's, and the one that finishes second merges the other's
//    partial O, m and d.
//  * Work items (segment, head, 128-query tile) are ordered so that consecutive
//    workgroups dispatched to one XCD (workgroup b runs on XCD b mod 8) take the same
//    head and neighbouring query tiles, so the CUs of an XCD stream the same K/V tiles
//    through their shared L2; packed batches are ordered longest-first.
#include <limits.h>
#include <math.h>

#include <utility>

#include "device_common.h"
#include "launch.h"

namespace sattn {

constexpr int kWaves = 4;                  // waves per workgroup: two workgroups per CU
constexpr int kLoaderWaves = 4;            // waves that stream the K/V tiles
constexpr int kWavesPerSimd = kWaves > 4 ? kWaves / 4 : 2;
constexpr int kQPerWG = kWaves * 32;       // queries per workgroup
constexpr int kQBlocksPerWG = kWaves / 2;  // 64-query blocks per workgroup
constexpr float kLog2_448 = 8.8073549220576041f;
// The QK accumulators start at kAccBias instead of 0: read as FP32, kAccBias + acc is
// exactly 12582912 + acc for |acc| < 2^22 (INT8 products over 128 channels stay below
// 127^2 * 128 < 2^21), so one exact subtraction replaces the integer conversion, and the
// biased words still order like the accumulators for the integer row max.
constexpr int kAccBias = 0x4B400000;
constexpr float kAccBiasF = 12582912.0f;

int attn_queries_per_wg() { return kQPerWG; }

__device__ __forceinline__ int xhalf_max(int x) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float((int)r[0]) + __int_as_float((int)r[1]);
}

// LDS operands of one PV tile w (V^T rows 32w..32w+31, 64 keys) and one QK step u of
// score tile t (K rows 32t.., channels 64g + 16u ..).
__device__ __forceinline__ v8i load_v(const uint8_t* Vl, int lane, int w) {
  const v4i lo = *reinterpret_cast<const v4i*>(Vl + ((w * 2 + 0) * 64 + lane) * 16);
  const v4i hi = *reinterpret_cast<const v4i*>(Vl + ((w * 2 + 1) * 64 + lane) * 16);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ v4i load_k(const uint8_t* Kl, int lane, int t, int u) {
  return *reinterpret_cast<const v4i*>(Kl + ((t * 4 + u) * 64 + lane) * 16);
}
__device__ __forceinline__ void pv_mfma(v16f& o, const v8i& a, const v8i& pb) {
  o = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, o, 0, 0, 0, 0, 0, 0);
}
// O^T += V^T P^T for one 32-channel tile w (operands read here).
__device__ __forceinline__ void pv_tile(v16f& o, const uint8_t* Vl, const v8i& pb, int lane, int w) {
  pv_mfma(o, load_v(Vl, lane, w), pb);
}

// K and V tiles live in two three-slot LDS rings: epoch e's K tile in k slot e % 3, its V
// tile in v slot e % 3.  Step e reads K(e+1) (QK of the next epoch) and V(e-1) (the
// deferred PV) and requests K(e+3) and V(e+1), so every tile has two epochs to land.  Each
// slot is its own array, so every LDS address in the unrolled loop is a constant.
constexpr int kRing = 3;
constexpr int kUnroll = 6;  // lcm of the ring length and the probability double buffer
__shared__ __attribute__((aligned(16))) uint8_t g_k0[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_k1[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_k2[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_v0[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_v1[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_v2[kTileBytes];
// K block scales of the workgroup's segment, copied to LDS at the start (segments of at
// most kKsLds key blocks; longer ones read them through the scalar cache).  A scalar load
// in flight would make every LDS wait of the step a full lgkmcnt(0) wait: SMEM results
// return out of order on the counter that LDS reads share.
constexpr int kKsLds = 2048;
__shared__ float g_ks[kKsLds];
__shared__ float g_qamax[kWaves];  // fused Q preparation: each wave's 32-row amax
__shared__ __attribute__((aligned(16))) float g_vs[kD];  // this head's V channel scales, for the epilogue
__shared__ int g_split_order;      // key split: how many halves of the tile had finished before this one
constexpr int kChunksPerTile = kTileBytes / 16 / (kLoaderWaves * 64);  // per loader lane
static_assert(kChunksPerTile * kLoaderWaves * 64 * 16 == kTileBytes, "tile split");

template <int I>
__device__ __forceinline__ uint8_t* kslot() {
  static_assert(I >= 0 && I < kRing, "slot");
  if constexpr (I == 0) return g_k0;
  if constexpr (I == 1) return g_k1;
  return g_k2;
}
template <int I>
__device__ __forceinline__ uint8_t* vslot() {
  static_assert(I >= 0 && I < kRing, "slot");
  if constexpr (I == 0) return g_v0;
  if constexpr (I == 1) return g_v1;
  return g_v2;
}

// Per-wave state of the epoch pipeline.
typedef __attribute__((address_space(4))) const float const_f32;

// Workgroup barrier without the memory fence of __syncthreads(): that fence makes a wave
// wait for all of its LDS-DMA requests, which would cap the tile prefetch at one epoch.
// LDS accesses of this wave are completed here (lgkmcnt(0)); tile requests are waited for
// with explicit vmcnt counts before it.
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One 16-byte chunk per lane from global memory into LDS (global_load_lds_dwordx4; lane l
// writes LDS address lds + 16 l).  Written as inline asm so that the compiler's wait-count
// bookkeeping does not see an LDS-DMA write: it would otherwise make LDS reads that it
// cannot prove disjoint wait for every outstanding tile request (vmcnt(0)).  Tile requests
// are waited for explicitly and ordered against their readers by the workgroup barrier.
// The instruction takes its LDS base from m0, a register the compiler reserves: the asm
// saves m0, sets it, issues the load and restores it, so whatever the compiler keeps in
// m0 is unchanged across the statement (two scalar moves per load).
__device__ __forceinline__ void dma_chunk(const uint8_t* base, uint32_t lane_off, const uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const lds_void_t*)lds;  // LDS byte address
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(lane_off), "s"(base), "s"(m0)
      : "memory");
}

struct Pipe {
  v16f oacc[4];  // O^T, 32 channels x 32 queries per tile
  v4i qop[4];            // this wave's Q operand (register copy)
  v16i bias;             // kAccBias in every element: the start value of the QK accumulators
  v8i pb[2];     // E4M3 probabilities of even / odd epochs (PV deferred one step)
  float alpha_prev;  // its rescale factor, applied to O just before its PV is accumulated
  float m, dpart, sig_q;
  const_f32* ksc;   // K block scales, read through the scalar cache
  float ks_next;    // scale of the next epoch, loaded one step ahead
  const uint8_t *kg, *vg;
  uint32_t loff[kChunksPerTile];  // DMA lane offsets: this lane's 16 bytes of each chunk
  int lane, wave, g, nkb;
  bool active;
};

// Checkpoint dump (sattn_debug_scores): the parameters, and this lane's sampled-row index
// (-1 if its query row is not sampled).
struct Dump {
  DumpParams p;
  int64_t idx;
};

// A tile (8 KiB = 512 16-byte chunks) moves into an LDS slot; loader wave w, step j covers
// chunks (j * kLoaderWaves + w) * 64 + lane (a wave-uniform LDS base per instruction).
__device__ __forceinline__ void issue_tile(const Pipe& c, const uint8_t* src_tiles, int e, uint8_t* slot) {
  if (c.wave >= kLoaderWaves) return;
  const uint8_t* tile = src_tiles + (int64_t)e * kTileBytes;  // wave-uniform
#pragma unroll
  for (int j = 0; j < kChunksPerTile; ++j) dma_chunk(tile, c.loff[j], slot + (j * kLoaderWaves + c.wave) * 1024);
}

// The steady steps' K tile and V tile in one statement: m0 saved once, set before each of the
// four loads, restored once (the per-load save and restore of dma_chunk costs ~1.5 % of the
// kernel's time when it runs in every step).
__device__ __forceinline__ void issue_kv(const Pipe& c, const uint8_t* ktile, uint8_t* kdst, const uint8_t* vtile,
                                         uint8_t* vdst) {
  static_assert(kChunksPerTile == 2 && kLoaderWaves == kWaves, "two loads per lane and tile");
  const uint32_t k0 = (uint32_t)(uintptr_t)(const lds_void_t*)(kdst + c.wave * 1024);
  const uint32_t k1 = (uint32_t)(uintptr_t)(const lds_void_t*)(kdst + (kLoaderWaves + c.wave) * 1024);
  const uint32_t v0 = (uint32_t)(uintptr_t)(const lds_void_t*)(vdst + c.wave * 1024);
  const uint32_t v1 = (uint32_t)(uintptr_t)(const lds_void_t*)(vdst + (kLoaderWaves + c.wave) * 1024);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %3\n\t"
      "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %4\n\t"
      "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %4\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(c.loff[0]), "v"(c.loff[1]), "s"(ktile), "s"(vtile), "s"(k0), "s"(k1), "s"(v0), "s"(v1)
      : "memory");
}

// One S^T tile t of the first epoch: acc_t = K(keys 32t..32t+31) . Q^T over 128 channels,
// started at kAccBias (later epochs run these MFMAs inside the softmax of the step before).
__device__ __forceinline__ void qk_tile(v16i& acc_t, const uint8_t* Kl, const v4i (&qop)[4], int lane, int t) {
#pragma unroll
  for (int i = 0; i < 16; ++i) acc_t[i] = kAccBias;
#pragma unroll
  for (int u = 0; u < 4; ++u) acc_t = __builtin_amdgcn_mfma_i32_32x32x32_i8(load_k(Kl, lane, t, u), qop[u], acc_t, 0, 0, 0);
}

// The requests before the first step: K of epochs 0-2 and V of epoch 0.
__device__ __forceinline__ void issue_first_tiles(const Pipe& c, int nkb) {
  if (nkb > 0) issue_tile(c, c.kg, 0, kslot<0>());
  if (nkb > 1) issue_tile(c, c.kg, 1, kslot<1>());
  if (nkb > 2) issue_tile(c, c.kg, 2, kslot<2>());
  if (nkb > 0) issue_tile(c, c.vg, 0, vslot<0>());
}

// Fused Q preparation, second part: the INT8 operands and fl32(q_scale * c) of this wave's
// 32 rows from their BF16 values, with the quantizer's arithmetic (fl32 scale, RNE codes in
// [-127, 127], the zero-block rule); the 64-row block amax combines the sibling wave's,
// which must be visible in LDS.
__device__ __forceinline__ void fused_q_operands(Pipe& c, const uint4 (&qraw)[8], float qamax, const AttnParams& p,
                                                 int wave) {
  const float amax = p.q_scale_shift ? qamax : fmaxf(qamax, g_qamax[wave ^ 1]);
  const float rcp = 127.0f / amax;
  const bool zero = !(amax > 0.f) || isinf(rcp);  // the quantizer's zero-block rule
  const float scale = zero ? 0.f : amax / 127.0f;
  const float inv = zero ? 0.f : rcp;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // word w of operand u: channels 64g + 16u + 4w .. +3
      float x[8];
      unpack8(qraw[2 * u + (w >> 1)], x);
      uint32_t word = 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float qv = rintf(x[4 * (w & 1) + b] * inv);
        qv = fminf(fmaxf(qv, -127.f), 127.f);
        word |= ((uint32_t)((int)qv) & 0xffu) << (8 * b);
      }
      c.qop[u][w] = (int)word;
    }
  }
  c.sig_q = scale * p.c32;
}

// Device-coherent 16-byte store and load through a buffer resource (cache policy SC1: device
// scope, past the caches that are not coherent across the XCDs).
constexpr int kBufWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
constexpr int kCoherentAgent = 16;     // the SC1 bit of the instruction's cache policy
__device__ __forceinline__ void st_coherent16(__amdgpu_buffer_rsrc_t r, int off, float a, float b, float c,
                                              float d) {
  const v4f x = {a, b, c, d};
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, x), r, off, 0, kCoherentAgent);
}
__device__ __forceinline__ v4f ld_coherent16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentAgent));
}

// Key split, a later piece: the running max over the first np epochs of the segment (the
// keys of the earlier pieces), exactly as the sequential recurrence has it when it reaches
// this piece: m = max(m, fl32(max_j acc_j * sigma_e)) per epoch.  QK MFMAs and the row max
// only; the K tiles pass through a three-slot ring with two epochs of prefetch.
__device__ __forceinline__ float prefix_max(const Pipe& c, const uint8_t* kg0, const_f32* ksc0, int np) {
  float m = -INFINITY;
  if (np <= 0) return m;
  issue_tile(c, kg0, 0, kslot<0>());
  if (np > 1) issue_tile(c, kg0, 1, kslot<1>());
  for (int e = 0; e < np; ++e) {
    if (e + 1 < np) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kChunksPerTile) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier();  // K(e) visible; every wave is done with the slot K(e+2) goes to
    const int sl = e % kRing;
    if (e + 2 < np) {
      const int sn = (e + 2) % kRing;
      issue_tile(c, kg0, e + 2, sn == 0 ? kslot<0>() : sn == 1 ? kslot<1>() : kslot<2>());
    }
    const uint8_t* Kl = sl == 0 ? kslot<0>() : sl == 1 ? kslot<1>() : kslot<2>();
    v16i a0, a1;
    qk_tile(a0, Kl, c.qop, c.lane, 0);
    qk_tile(a1, Kl, c.qop, c.lane, 1);
    int mx = INT_MIN;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = max(max(mx, a0[r]), a1[r]);
    mx = xhalf_max(mx);
    m = fmaxf(m, (float)(mx - kAccBias) * (c.sig_q * ksc0[e]));
  }
  barrier();  // every wave is done with the ring before the epoch pipeline reuses it
  return m;
}

// Online softmax of epoch e for this lane's query (32 of the 64 keys; the other 32 are in
// lane ^ 32).  Interleaved with it, on the matrix cores: PV of epoch e-1 and, once a
// score tile has been consumed, QK of epoch e+1 into the same registers (NEXT).  Updates
// m and the lane's partial denominator (in units of 448*P), packs the E4M3 probabilities
// into pb and returns alpha.  TAIL masks keys >= kvalid.
//
// The step is cut into eight groups of four probabilities (scheduling barriers between
// them).  Each group first issues one MFMA, so this wave never asks the matrix core for
// two in a row: groups 0-3 the PV(e-1) tiles 0-3, groups 4-7 the four k-steps of QK(e+1)
// score tile 0 (whose scores groups 0-3 consumed); score tile 1 follows group 7.  The LDS
// operands of each MFMA are read one to two groups ahead of it.
template <bool TAIL, bool NEXT>
__device__ __forceinline__ float softmax_pv(Pipe& c, v16i (&acc)[2], float sig, int kvalid, v8i& pb,
                                            const v8i& pb_prev, const uint8_t* Vprev, const uint8_t* Knext) {
  const int g = c.g;
  v8i va = load_v(Vprev, c.lane, 0), vb = load_v(Vprev, c.lane, 1);
  __builtin_amdgcn_sched_barrier(0);  // the reads go out first; the row max hides them
  int v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int t = i >> 4, r = i & 15;
    const int key = 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
    v[i] = (TAIL && key >= kvalid) ? INT_MIN : acc[t][r];
  }
  int m1[12];  // a three-input max tree: 10 + 4 + 1 v_max3 and one v_max
#pragma unroll
  for (int i = 0; i < 10; ++i) m1[i] = max(max(v[3 * i], v[3 * i + 1]), v[3 * i + 2]);
  m1[10] = v[30];
  m1[11] = v[31];
  int m2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) m2[i] = max(max(m1[3 * i], m1[3 * i + 1]), m1[3 * i + 2]);
  int mx = max(max(max(m2[0], m2[1]), m2[2]), m2[3]);
  mx = xhalf_max(mx);
  const float smax = (float)(mx - kAccBias) * sig;  // = max_j fl32(acc_j * sig)
  const float m_new = fmaxf(c.m, smax);
  const float alpha = __builtin_amdgcn_exp2f(c.m - m_new);  // 0 on the first epoch
  const float mm = m_new - kLog2_448;
  float ps[4] = {0.f, 0.f, 0.f, 0.f};
  v4i ka[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    __builtin_amdgcn_sched_barrier(0);
    if (j < 4) {
      pv_mfma(c.oacc[j], (j & 1) ? vb : va, pb_prev);
      if (j == 0) va = load_v(Vprev, c.lane, 2);
      if (j == 1) vb = load_v(Vprev, c.lane, 3);
      if constexpr (NEXT) {
        if (j >= 2) {
          ka[2 * (j - 2)] = load_k(Knext, c.lane, 0, 2 * (j - 2));
          ka[2 * (j - 2) + 1] = load_k(Knext, c.lane, 0, 2 * (j - 2) + 1);
        }
      }
    } else if constexpr (NEXT) {
      const int u = j - 4;
      acc[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[u], c.qop[u], u == 0 ? c.bias : acc[0], 0, 0, 0);
      ka[u] = load_k(Knext, c.lane, 1, u);
    }
    const int t = j >> 2, q4 = j & 3;
    float pv[4];
#pragma unroll
    for (int r3 = 0; r3 < 4; ++r3) {
      float arg = __builtin_fmaf(__int_as_float(acc[t][4 * q4 + r3]) - kAccBiasF, sig, -mm);
      if (TAIL && 32 * t + 8 * q4 + 4 * g + r3 >= kvalid) arg = -INFINITY;
      pv[r3] = __builtin_amdgcn_exp2f(arg);  // 448 * P
      ps[r3] = j == 0 ? pv[r3] : ps[r3] + pv[r3];
    }
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wuninitialized"
    int old;  // both halves of the word are written below; no register needs zeroing
    int w01 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], old, false);
#pragma clang diagnostic pop
    w01 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], w01, true);
    pb[j] = w01;
    // keep the row-sum adds in their group, between the exponentials (left to itself the
    // compiler sinks all 32 to the end of the step, where they issue back to back)
    asm volatile("" : "+v"(ps[0]), "+v"(ps[1]), "+v"(ps[2]), "+v"(ps[3]));
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NEXT) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[u], c.qop[u], u == 0 ? c.bias : acc[1], 0, 0, 0);
  }
  c.dpart = c.dpart * alpha + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
  c.m = m_new;
  return alpha;
}

// O *= alpha of the epoch whose PV is about to be accumulated, only in the lanes (query
// rows) whose max changed: elsewhere alpha is exactly 1.  The whole block is skipped when
// no row of the wave changed; masked lanes cost the same issue slots but no ALU switching,
// which counts on a power-capped part.
__device__ __forceinline__ void rescale(Pipe& c) {
  const float a = c.alpha_prev;
  if (a != 1.0f) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int i = 0; i < 16; ++i) c.oacc[w][i] *= a;
  }
}

// ---------------------------------------------------------------- checkpoint dump
// The checkpoint quantities of the Phase 2B report's "Exactness" section for the sampled
// query rows, written from the registers of this instantiation (the production kernel with
// stores added): INT32 accumulators and FP32 scores per key, and per epoch the running max,
// the denominator, the rescale factor, the E4M3 probability bytes and the running output.
__device__ __forceinline__ void dump_scores(const Pipe& c, const Dump& dump, int e, int kvalid, const v16i (&acc)[2],
                                            float sig) {
  if (dump.idx < 0) return;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * t + 8 * (r >> 2) + 4 * c.g + (r & 3);
      const int64_t j = (int64_t)e * kBlk + key;
      if (key < kvalid && j < dump.p.ld) {
        const int64_t o = dump.idx * dump.p.ld + j;
        const int32_t a = acc[t][r] - kAccBias;
        if (dump.p.acc) dump.p.acc[o] = a;
        if (dump.p.s) dump.p.s[o] = (float)a * sig;  // fl32(acc * sigma)
      }
    }
}

// Epoch e's running max m, rescale factor alpha and denominator d (both half-waves' partial
// sums, in units of 448 P), and its E4M3 probability bytes in key order.
__device__ __forceinline__ void dump_epoch(const Pipe& c, const Dump& dump, int e, float alpha, const v8i& pb) {
  const float dsum = xhalf_sum(c.dpart);  // cross-lane: every lane of the wave takes part
  if (dump.idx < 0 || e >= dump.p.nep) return;
  const int64_t o = dump.idx * dump.p.nep + e;
  if (dump.p.m) dump.p.m[o] = c.m;
  if (dump.p.alpha) dump.p.alpha[o] = alpha;
  if (dump.p.d) dump.p.d[o] = dsum;
  if (dump.p.p8) {
    uint8_t* row = dump.p.p8 + o * kBlk;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r3 = 0; r3 < 4; ++r3)
        row[32 * (j >> 2) + 8 * (j & 3) + 4 * c.g + r3] = (uint8_t)(((uint32_t)pb[j] >> (8 * r3)) & 0xffu);
  }
}

// The running output RO after epoch e (this lane's 64 of the row's 128 channels).
__device__ __forceinline__ void dump_ro(const Pipe& c, const Dump& dump, int e) {
  if (dump.idx < 0 || e < 0 || e >= dump.p.nep || dump.p.ro == nullptr) return;
  float* row = dump.p.ro + (dump.idx * dump.p.nep + e) * kD;
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int i = 0; i < 16; ++i) row[32 * w + 8 * (i >> 2) + 4 * c.g + (i & 3)] = c.oacc[w][i];
}

// Pipeline step for epoch e (ST = e % kUnroll).  Its scores are already in acc (QK issued
// during the previous step).  Wait until K(e+1) and V(e-1) have landed (the requests of
// step e-1 may stay in flight), barrier, request K(e+3) and V(e+1), then rescale O by
// alpha(e-1) and run the softmax of e with PV(e-1) and QK(e+1) interleaved.  LAST marks
// the final epoch (TAIL masks its keys), which also accumulates its own PV.  STEADY steps
// have e + 3 < nkb: every tile request and scale load is in range, so they run without
// tests or branches.
template <int ST, bool LAST, bool TAIL, bool DUMP, bool KSL, bool STEADY = false>
__device__ __forceinline__ void pipe_step(Pipe& c, int e, int kvalid, const Dump& dump, v16i (&acc)[2]) {
  constexpr int KS = ST % kRing, KN = (ST + 1) % kRing, VP = (ST + 2) % kRing;
  if constexpr (LAST || DUMP) {
    // LAST: V(e) too, its PV runs in this step.  DUMP: the score dump's stores (and any
    // scratch traffic) share the counter, so the counts below would not hold.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (STEADY || e + 2 < c.nkb) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kChunksPerTile) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kChunksPerTile) : "memory");
  }
  barrier();  // K(e+1), V(e-1) visible to every wave; every wave is done with step e-1
  // K(e+3) into the slot of K(e) and V(e+1) into the slot of V(e-2), both read in step e-1
  if constexpr (STEADY) {
    issue_kv(c, c.kg + (int64_t)(e + 3) * kTileBytes, kslot<KS>(), c.vg + (int64_t)(e + 1) * kTileBytes, vslot<KN>());
  } else {
    if (e + 3 < c.nkb) issue_tile(c, c.kg, e + 3, kslot<KS>());
    if (e + 1 < c.nkb) issue_tile(c, c.vg, e + 1, vslot<KN>());
  }
  if (!c.active) return;
  rescale(c);  // O = RO(e-2) * alpha(e-1), so PV(e-1) below completes RO(e-1)
  const float sig = c.sig_q * c.ks_next;  // fl32(fl32(q_scale * c) * k_scale)
  if (STEADY || e + 1 < c.nkb) c.ks_next = KSL ? g_ks[e + 1] : c.ksc[e + 1];
  if constexpr (DUMP) dump_scores(c, dump, e, kvalid, acc, sig);
  c.alpha_prev = softmax_pv<TAIL, !LAST>(c, acc, sig, kvalid, c.pb[ST & 1], c.pb[(ST + 1) & 1], vslot<VP>(),
                                         kslot<KN>());
  if constexpr (DUMP) {
    dump_epoch(c, dump, e, c.alpha_prev, c.pb[ST & 1]);
    dump_ro(c, dump, e - 1);  // the P.V of epoch e-1 has just been accumulated
  }
  if constexpr (LAST) {
    rescale(c);
#pragma unroll
    for (int w = 0; w < 4; ++w) pv_tile(c.oacc[w], vslot<KS>(), c.pb[ST & 1], c.lane, w);
    if constexpr (DUMP) dump_ro(c, dump, e);
  }
}

template <int ST, bool DUMP, bool KSL>
__device__ __forceinline__ void last_step(Pipe& c, int e, int kvalid, const Dump& dump, v16i (&acc)[2]) {
  if (kvalid == kBlk) pipe_step<ST, true, false, DUMP, KSL>(c, e, kBlk, dump, acc);
  else pipe_step<ST, true, true, DUMP, KSL>(c, e, kvalid, dump, acc);
}

// kUnroll full steps e .. e+kUnroll-1 (e a multiple of kUnroll).
template <bool DUMP, bool KSL, bool STEADY, int... STs>
__device__ __forceinline__ void steps_all(Pipe& c, int e, const Dump& dump, v16i (&acc)[2],
                                          std::integer_sequence<int, STs...>) {
  (pipe_step<STs, false, false, DUMP, KSL, STEADY>(c, e + STs, kBlk, dump, acc), ...);
}
// The remaining full steps e + ST < nfull (e a multiple of kUnroll).
template <bool DUMP, bool KSL, int... STs>
__device__ __forceinline__ void steps_rest(Pipe& c, int e, int nfull, const Dump& dump, v16i (&acc)[2],
                                           std::integer_sequence<int, STs...>) {
  ((e + STs < nfull ? pipe_step<STs, false, false, DUMP, KSL>(c, e + STs, kBlk, dump, acc) : void()), ...);
}
// The last epoch nfull (ST = nfull % kUnroll).
template <bool DUMP, bool KSL, int... STs>
__device__ __forceinline__ void step_last(Pipe& c, int nfull, int kvalid, const Dump& dump, v16i (&acc)[2],
                                          std::integer_sequence<int, STs...>) {
  const int st = nfull % kUnroll;
  ((st == STs ? last_step<STs, DUMP, KSL>(c, nfull, kvalid, dump, acc) : void()), ...);
}

template <bool DUMP, bool KSL>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd))) void attn_fwd_kernel(AttnParams p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level addressing in SGPRs

  // ---------------------------------------------------------------- work item
  int s, h, piece = 0;
  int64_t qt;
  bool split_tile = false;  // this tile's keys are shared with a second workgroup
  int64_t split_idx = 0;    // its counter and partials in the workspace
  if constexpr (DUMP) {  // the query tiles of one (segment, head) that hold sampled rows
    s = p.dump.seg;
    h = p.dump.head;
    qt = p.dump.tile0 + blockIdx.x;
  } else {
  const int xcd = blockIdx.x & 7;
  int64_t kk = blockIdx.x >> 3;
  if (p.split > 1 && kk >= p.split_from) {  // the pieces of a tile: neighbours on one XCD
    const int64_t j = (kk - p.split_from) / p.split;
    piece = (int)(kk - p.split_from - j * p.split);
    kk = p.split_from + j;
    split_tile = true;
    split_idx = (p.H < 8 ? p.H : 8) * j + xcd;  // XCDs without a head return below
  }
  const int nh = xcd < p.H ? (p.H - xcd + 7) / 8 : 0;
  if (nh == 0) return;
  int64_t hl;
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
  h = xcd + 8 * (int)hl;
  }
  const SegInfo qi = seg_info(p.gq, s, p.o_st);
  const SegInfo ki = seg_info(p.gk, s, 0);
  const int nkb_seg = (int)ceil_blocks(ki.len);
  // key split: piece q takes epochs [e0, e1) (the last piece the partial last one too)
  const bool last_piece = !split_tile || piece == p.split - 1;
  const int e0 = piece ? min(p.split_e[piece], nkb_seg - 1) : 0;
  const int e1 = last_piece ? nkb_seg : max(e0, min(p.split_e[piece + 1], nkb_seg - 1));
  const int nkb = e1 - e0;
  const int last_valid = last_piece ? (int)(ki.len - (int64_t)(nkb_seg - 1) * kBlk) : kBlk;
  const int64_t qb = qt * kQBlocksPerWG + (wave >> 1);  // this wave's 64-query block
  const int hq = wave & 1;                              // and which 32 of its queries
  if constexpr (DUMP) {  // no sampled row in this tile (uniform over the workgroup): done
    const int64_t lo = max(qt * kQPerWG, p.dump.q0);
    const int64_t hi = min(min(qt * kQPerWG + kQPerWG, p.dump.q1), qi.len);
    const int64_t first = p.dump.q0 + (lo - p.dump.q0 + p.dump.qstep - 1) / p.dump.qstep * p.dump.qstep;
    if (first >= hi) return;
  }


  Pipe c;
  c.lane = lane;
  c.wave = wave;
  c.g = lane >> 5;
  c.nkb = nkb;
  c.active = qb < ceil_blocks(qi.len);
#pragma unroll
  for (int j = 0; j < kChunksPerTile; ++j) c.loff[j] = (uint32_t)(((j * kLoaderWaves + wave) * 64 + lane) * 16);
  c.m = -INFINITY;
  c.dpart = 0.f;
  c.sig_q = 0.f;
  c.alpha_prev = 1.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) c.bias[i] = kAccBias;
  asm volatile("" : "+v"(c.bias));  // kept in registers rather than rematerialised per use
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int i = 0; i < 16; ++i) c.oacc[w][i] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) c.pb[0][i] = c.pb[1][i] = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) c.qop[u] = v4i{0, 0, 0, 0};
  // Fused Q preparation (sattn_fwd_fused): lane g*32 + i holds token 32*hq + i of the
  // wave's 64-row block, channels 64g .. 64g+63, as BF16; the block amax goes through LDS
  // to the sibling wave (one 64-row scale) unless each wave has its own 32-row scale.
  // The first K/V tiles are requested before anything else, so that their latency overlaps
  // the Q and scale loads (the second half of a split tile first runs its running-max pass
  // through the same ring and requests them after it).
  const int64_t ktile0 = (int64_t)h * p.kblk_cap + ki.blk0;
  c.kg = reinterpret_cast<const uint8_t*>(p.k8) + (ktile0 + e0) * kTileBytes;
  c.vg = p.v8 + (ktile0 + e0) * kTileBytes;
  c.ksc = (const_f32*)(p.k_scale + ktile0 + e0);
  const bool dma_first = piece == 0;
  if (dma_first) issue_first_tiles(c, nkb);
  const bool fused_q = p.qbf != nullptr;
  uint4 qraw[8];
  float qamax = 0.f;
  if (fused_q) {
    SegGeom gqin = p.gq;
    gqin.stride_b = p.qb_sb;
    const SegInfo qin = seg_info(gqin, s, p.qb_st);
    const int64_t row = qb * kBlk + hq * 32 + (lane & 31);
    const uint16_t* src = p.qbf + qin.elem_base + row * p.qb_st + (int64_t)h * p.qb_sh + 64 * c.g;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qraw[j] = make_uint4(0u, 0u, 0u, 0u);
      if (c.active && row < qin.len) qraw[j] = *reinterpret_cast<const uint4*>(src + 8 * j);
      float x[8];
      unpack8(qraw[j], x);
#pragma unroll
      for (int i = 0; i < 8; ++i) qamax = fmaxf(qamax, fabsf(x[i]));
    }
    qamax = wave_max(qamax);  // the wave's 32 rows
    if (lane == 0) g_qamax[wave] = qamax;
  } else if (c.active) {
    const int8_t* qt_ptr = p.q8 + ((int64_t)h * p.qblk_cap + qi.blk0 + qb) * kTileBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int8_t* src = qt_ptr + ((hq * 4 + u) * 64 + lane) * 16;
      c.qop[u] = *reinterpret_cast<const v4i*>(src);
    }
    // fl32(q_scale * c) of this wave's 32 rows: the scale of their 64-row block, or of
    // their own half of it with 32-row Q scales
    const int64_t qsi = (((int64_t)h * p.qblk_cap + qi.blk0 + qb) << p.q_scale_shift) + (p.q_scale_shift ? hq : 0);
    c.sig_q = p.q_scale[qsi] * p.c32;
  }
  constexpr int kKsPerThread = kKsLds / (kWaves * 64);
  float ksr[kKsPerThread];
  if constexpr (KSL) {  // this epoch range's K scales, staged through LDS below
#pragma unroll
    for (int j = 0; j < kKsPerThread; ++j) {
      const int i = tid + j * kWaves * 64;
      ksr[j] = i < nkb ? c.ksc[i] : 0.f;
    }
  } else {
    c.ks_next = nkb > 0 ? c.ksc[0] : 0.f;
  }
  float4 vs4 = make_float4(0.f, 0.f, 0.f, 0.f);  // V channel scales, staged in LDS for the epilogue
  if (tid < kD / 4) vs4 = reinterpret_cast<const float4*>(p.v_scale + ((int64_t)s * p.H + h) * kD)[tid];
  // Retire the Q and scale loads here (the tile requests ahead of them too), with a wait the
  // compiler sees: otherwise its wait-count bookkeeping keeps them pending into the epoch
  // loop and waits on vmcnt before the QK MFMAs there, which would also wait for the tile
  // requests in flight.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (piece) {  // a later piece of a split tile: the running max over the earlier keys
    if (fused_q) {  // which needs this wave's Q operands first
      barrier();    // the sibling wave's row maximum in LDS
      if (c.active) fused_q_operands(c, qraw, qamax, p, wave);
    }
    c.m = prefix_max(c, reinterpret_cast<const uint8_t*>(p.k8) + ktile0 * kTileBytes,
                     (const_f32*)(p.k_scale + ktile0), e0);
  }
  if constexpr (KSL) {  // landed by the barrier before the first step
#pragma unroll
    for (int j = 0; j < kKsPerThread; ++j) {
      const int i = tid + j * kWaves * 64;
      if (i < nkb) g_ks[i] = ksr[j];
    }
  }
  if (tid < kD / 4) reinterpret_cast<float4*>(g_vs)[tid] = vs4;

  Dump dump;
  dump.idx = -1;
  if constexpr (DUMP) {
    dump.p = p.dump;
    const int64_t row = qb * kBlk + hq * 32 + (lane & 31), off = row - p.dump.q0;
    if (off >= 0 && row < p.dump.q1 && row < qi.len && off % p.dump.qstep == 0) dump.idx = off / p.dump.qstep;
  }

  // ---------------------------------------------------------------- epoch pipeline
  // Step e reads K(e+1) and V(e-1).  Step 0's deferred PV multiplies the V slot of epoch
  // -1 (slot 2, zeroed here) by all-zero probabilities.
#pragma unroll
  for (int i = tid; i < kTileBytes / 16; i += kWaves * 64) reinterpret_cast<v4i*>(g_v2)[i] = v4i{0, 0, 0, 0};
  v16i acc[2];
  if (!dma_first) issue_first_tiles(c, nkb);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  barrier();  // Q, K(0), the K scales, the Q row maxima and the zeroed V slot visible
  if constexpr (KSL) c.ks_next = nkb > 0 ? g_ks[0] : 0.f;
  if (fused_q && !piece && c.active) fused_q_operands(c, qraw, qamax, p, wave);
  if (nkb > 0) {
    qk_tile(acc[0], kslot<0>(), c.qop, lane, 0);
    qk_tile(acc[1], kslot<0>(), c.qop, lane, 1);
  }
  const int nfull = nkb - 1;  // epochs before the last one
  int e = 0;
  for (; e + kUnroll + 2 < nkb; e += kUnroll)  // every request of these steps is in range
    steps_all<DUMP, KSL, true>(c, e, dump, acc, std::make_integer_sequence<int, kUnroll>{});
  if (e + kUnroll <= nfull) {
    steps_all<DUMP, KSL, false>(c, e, dump, acc, std::make_integer_sequence<int, kUnroll>{});
    e += kUnroll;
  }
  steps_rest<DUMP, KSL>(c, e, nfull, dump, acc, std::make_integer_sequence<int, kUnroll - 1>{});
  if (nkb > 0) step_last<DUMP, KSL>(c, nfull, last_valid, dump, acc, std::make_integer_sequence<int, kUnroll>{});

  // ---------------------------------------------------------------- epilogue
  float dtot = xhalf_sum(c.dpart);  // = 448 * d
  if (split_tile) {
    // Every piece stores m, d and O of its rows; the piece that finishes last merges them in
    // piece order whichever piece that is: m = max_q m_q, O = sum_q O_q 2^(m_q - m) (the
    // first term a product, then one FMA per piece), d likewise.  The partials move through
    // device-coherent 16-byte stores and loads, lane-major so that each instruction covers
    // 1 KiB (they bypass the caches that are not coherent across the XCDs, so the pieces may
    // sit on different XCDs); the stores are complete before this workgroup's arrival is
    // counted, and the merging piece reads only after it saw every other's count.
    // Agent-scope fences would write back and invalidate the whole L2 of the XCD at every
    // tile's end instead.
    const int np = p.split;
    const __amdgpu_buffer_rsrc_t tile_ws = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<char*>(p.part) + split_idx * np * kSplitPieceBytes, 0, np * kSplitPieceBytes, kBufWord3);
    const int lane_off = wave * (kSplitPieceBytes / 4) + lane * 16;
    const int mine = piece * kSplitPieceBytes + lane_off;
    if (c.active) {  // uniform over the wave
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          st_coherent16(tile_ws, mine + (4 * w + q4) * 1024, c.oacc[w][4 * q4], c.oacc[w][4 * q4 + 1],
                        c.oacc[w][4 * q4 + 2], c.oacc[w][4 * q4 + 3]);
      st_coherent16(tile_ws, mine + 16 * 1024, c.m, dtot, 0.f, 0.f);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partials are stored
    __syncthreads();
    if (tid == 0) g_split_order = __hip_atomic_fetch_add(p.cnt + split_idx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (g_split_order != np - 1) return;  // a later piece merges
    if (tid == 0) __hip_atomic_store(p.cnt + split_idx, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // zero for the next call
    if (!c.active) return;
    float mq[kMaxPieces], dq[kMaxPieces];
#pragma unroll
    for (int q = 0; q < kMaxPieces; ++q) {
      mq[q] = -INFINITY;
      dq[q] = 0.f;
      if (q < np) {
        const v4f md = q == piece ? v4f{c.m, dtot, 0.f, 0.f}
                                  : ld_coherent16(tile_ws, q * kSplitPieceBytes + lane_off + 16 * 1024);
        mq[q] = md[0];
        dq[q] = md[1];
      }
    }
    float m = mq[0];
#pragma unroll
    for (int q = 1; q < kMaxPieces; ++q) m = fmaxf(m, mq[q]);
    float aq[kMaxPieces];
#pragma unroll
    for (int q = 0; q < kMaxPieces; ++q) aq[q] = __builtin_amdgcn_exp2f(mq[q] - m);  // 0 past np
    dtot = dq[0] * aq[0];
#pragma unroll
    for (int q = 1; q < kMaxPieces; ++q)
      if (q < np) dtot = __builtin_fmaf(dq[q], aq[q], dtot);
    float acc_o[4][16];
#pragma unroll
    for (int q = 0; q < kMaxPieces; ++q) {
      if (q >= np) break;
      v4f po[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        po[j] = q == piece ? v4f{c.oacc[j >> 2][4 * (j & 3)], c.oacc[j >> 2][4 * (j & 3) + 1],
                                 c.oacc[j >> 2][4 * (j & 3) + 2], c.oacc[j >> 2][4 * (j & 3) + 3]}
                           : ld_coherent16(tile_ws, q * kSplitPieceBytes + lane_off + j * 1024);
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = po[4 * w + (i >> 2)][i & 3];
          acc_o[w][i] = q == 0 ? x * aq[0] : __builtin_fmaf(x, aq[q], acc_o[w][i]);
        }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int i = 0; i < 16; ++i) c.oacc[w][i] = acc_o[w][i];
  }
  if (!c.active) return;
  const float inv = dtot > 0.f ? 1.0f / dtot : 0.f;
  const int64_t row = qb * kBlk + hq * 32 + (lane & 31);
  if (row >= qi.len) return;
  if (DUMP && dump.idx < 0) return;  // the checkpoint run writes the sampled rows only
  if (DUMP && p.dump.rcp != nullptr && c.g == 0) p.dump.rcp[dump.idx] = inv;
  uint16_t* orow = p.o + qi.elem_base + row * p.o_st + (int64_t)h * p.o_sh;
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int c0 = 32 * w + 8 * q4 + 4 * c.g;
      const float4 vs = *reinterpret_cast<const float4*>(g_vs + c0);
      const float vsa[4] = {vs.x, vs.y, vs.z, vs.w};
      float y[4];
#pragma unroll
      for (int r3 = 0; r3 < 4; ++r3) y[r3] = (c.oacc[w][4 * q4 + r3] * inv) * vsa[r3];
      *reinterpret_cast<uint2*>(orow + c0) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
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
  const bool ksl = p.max_kblocks <= kKsLds;  // the same K-scale path with and without the dump
  if (dump && ksl)
    hipLaunchKernelGGL((attn_fwd_kernel<true, true>), dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, p);
  else if (dump)
    hipLaunchKernelGGL((attn_fwd_kernel<true, false>), dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, p);
  else if (ksl)
    hipLaunchKernelGGL((attn_fwd_kernel<false, true>), dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<false, false>), dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sattn
