// C ABI of the library (declared in include/sattn.h): argument validation, buffer
// geometry and kernel launches.  Validation happens before any HIP call, so a call that
// fails it has enqueued nothing; this part runs (and is tested) without a GPU.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "launch.h"
#include "sattn.h"

using namespace sattn;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool view_ok(const void* ptr, int64_t sb, int64_t st, int64_t sh, bool dense) {
  if (ptr == nullptr || !aligned16(ptr)) return false;
  if (st < 0 || sh < 0 || (st % 8) || (sh % 8)) return false;
  if (dense && (sb < 0 || (sb % 8))) return false;
  return true;
}

struct QuantWs {
  size_t sums, vmax, vinv, total;
};

QuantWs quant_ws(int nseg, int H) {
  const size_t n = (size_t)nseg * H * stats_chunks(nseg, H) * kD;
  QuantWs w;
  w.sums = align_up(n * sizeof(double));
  w.vmax = align_up(n * sizeof(float));
  w.vinv = align_up((size_t)nseg * H * kD * sizeof(float));
  w.total = w.sums + w.vmax + w.vinv;
  return w;
}

size_t fwd_ws(int nseg) { return align_up((size_t)nseg * 4) + align_up(((size_t)nseg + 1) * 4); }

// Key split of the dense forward.  Workgroups are dispatched round-robin over the 8 XCDs,
// two per CU at a time; when the last round of an XCD holds few enough tiles that each can
// be shared by 2 or 4 workgroups (pieces) with a CU of their own (at most an eighth, resp. a
// quarter, of the XCD's CUs' worth of tiles), those tiles are split — all of them when the
// whole grid is that small.  One workgroup alone on a CU already keeps its SIMDs most of
// the way busy, so pieces that share a CU gain less than their running-max passes cost.
// A piece needs kSplitMinEpochs / 2 epochs of its own on average.  The piece boundaries
// balance the pieces: piece q runs a pass over the keys before it (QK and the max, about
// 0.4 of a full epoch per epoch) and then its own epochs, so piece q gets a share of the
// epochs proportional to 0.6^q.
constexpr int64_t kSplitMaxTiles = 128;   // 2 pieces: 16 tiles per XCD on 256 CUs
constexpr int64_t kSplitMaxTiles4 = 64;   // 4 pieces: 8 tiles per XCD
constexpr int kSplitMinEpochs = 16;
// Cumulative shares (per mille) of the epochs before piece q, for 2 and 4 pieces.
constexpr int kSplitShare2[2] = {0, 625};
constexpr int kSplitShare4[4] = {0, 460, 735, 901};

// need_q: the Q buffers take part (false for the fused-Q forward and K/V-only quantization).
bool quant_bufs_ok(const sattn_qkv_quant* b, bool need_q = true) {
  if (b == nullptr) return false;
  if (need_q && (b->q == nullptr || b->q_scale == nullptr || !aligned16(b->q) || b->qblk_cap < 0)) return false;
  return b->k && b->k_scale && b->k_mean && b->v && b->v_scale && aligned16(b->k) && aligned16(b->v) &&
         b->kblk_cap >= 0 && (b->q_scale_rows == 0 || b->q_scale_rows == 32 || b->q_scale_rows == 64);
}

// log2(64 / q_scale_rows): Q scales per 64-token block, as a shift.
int q_scale_shift(const sattn_qkv_quant* b) { return b->q_scale_rows == 32 ? 1 : 0; }

int64_t ceil64(int64_t n) { return (n + 63) / 64; }

// Largest grid of 256-thread workgroups one dispatch takes (it counts work-items in 32 bits).
constexpr int64_t kMaxGroups256 = 0xffffffffLL / 256;

// Largest token count whose blocks fit a capacity (cap = floor(T/64) + nseg).
int64_t clip_for_cap(int64_t cap, int nseg) { return cap >= nseg ? (cap - nseg) * 64 + 63 : 0; }

// Quantizer workspace of sattn_quantize_qkv_noalloc: a file-scope device array, one copy on
// every GPU the library runs on, held until the process ends.  Host code never uses the
// name itself (on the host it is only a stand-in for the symbol): its device address is
// looked up once per device, with that device current, and kept in scratch_ptr.
constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

int cu_cache[kMaxDevices] = {};

// Compute units of the current device (asked once per device).
sattn_status cu_count(int* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SATTN_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SATTN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (cu_cache[dev] == 0 &&
      hipDeviceGetAttribute(&cu_cache[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    cu_cache[dev] = 0;
    return SATTN_EHIP;
  }
  *out = cu_cache[dev];
  return SATTN_OK;
}

sattn_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SATTN_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SATTN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SATTN_EHIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return SATTN_OK;
}

}  // namespace

extern "C" {

const char* sattn_status_string(sattn_status s) {
  switch (s) {
    case SATTN_OK: return "ok";
    case SATTN_EINVAL: return "invalid argument";
    case SATTN_EUNSUPPORTED: return "unsupported configuration";
    case SATTN_ENOSPACE: return "buffer or workspace too small";
    case SATTN_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

sattn_status sattn_quant_query(int nseg, int64_t total_q, int64_t total_k, int H, int D, sattn_sizes* out) {
  if (out == nullptr || nseg < 1 || H < 1 || total_q < 0 || total_k < 0) return SATTN_EINVAL;
  if (D != kD) return SATTN_EUNSUPPORTED;
  memset(out, 0, sizeof(*out));
  out->qblk_cap = total_q / 64 + nseg;
  out->kblk_cap = total_k / 64 + nseg;
  out->q_bytes = (size_t)H * out->qblk_cap * kTileBytes;
  out->q_scale_bytes = (size_t)H * out->qblk_cap * 2 * sizeof(float);  // room for 32-row scales
  out->k_bytes = (size_t)H * out->kblk_cap * kTileBytes;
  out->k_scale_bytes = (size_t)H * out->kblk_cap * sizeof(float);
  out->k_mean_bytes = (size_t)nseg * H * kD * sizeof(float);
  out->v_bytes = out->k_bytes;
  out->v_scale_bytes = out->k_mean_bytes;
  out->quant_workspace_bytes = quant_ws(nseg, H).total;
  // room for the key split's partials: at most kSplitMaxTiles tiles (the last dispatch
  // round's, or the whole grid's), and never more than the problem has
  const int64_t qpw = attn_queries_per_wg();
  const int64_t tiles_hi = (int64_t)H * (total_q / qpw + nseg);
  const size_t split = std::max(split_ws_bytes(std::min(tiles_hi, kSplitMaxTiles), 2),
                                split_ws_bytes(std::min(tiles_hi, kSplitMaxTiles4), 4));
  out->fwd_workspace_bytes = fwd_ws(nseg) > split ? fwd_ws(nseg) : split;
  return SATTN_OK;
}

// sattn_quantize_qkv; with workspace == nullptr the device's scratch array is used instead
// (sattn_quantize_qkv_noalloc), after every other argument has been validated.
static sattn_status quantize_impl(sattn_bf16_in q, sattn_bf16_in k, sattn_bf16_in v, int nseg, int H, int D, int64_t Lq,
                                  int64_t Lk, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                  const sattn_qkv_quant* out, void* workspace, size_t workspace_bytes, bool use_scratch,
                                  void* stream) {
  if (nseg < 1 || H < 1 || Lq < 0 || Lk < 0) return SATTN_EINVAL;
  if (D != kD || nseg > 65535 || H > 65535) return SATTN_EUNSUPPORTED;  // grid y/z extents
  const bool varlen = cu_seqlens_q != nullptr;
  if ((cu_seqlens_k != nullptr) != varlen) return SATTN_EINVAL;
  // Q buffers both NULL: K and V only (for sattn_fwd_fused, which quantizes Q itself)
  const bool do_q = out == nullptr || out->q != nullptr || out->q_scale != nullptr;
  if ((do_q && !view_ok(q.ptr, q.stride_b, q.stride_t, q.stride_h, !varlen)) ||
      !view_ok(k.ptr, k.stride_b, k.stride_t, k.stride_h, !varlen) ||
      !view_ok(v.ptr, v.stride_b, v.stride_t, v.stride_h, !varlen))
    return SATTN_EINVAL;
  if (!quant_bufs_ok(out, do_q) || (!use_scratch && (workspace == nullptr || !aligned16(workspace))))
    return SATTN_EINVAL;
  const int64_t total_q = varlen ? Lq : (int64_t)nseg * Lq;
  const int64_t total_k = varlen ? Lk : (int64_t)nseg * Lk;
  if ((do_q && out->qblk_cap < total_q / 64 + nseg) || out->kblk_cap < total_k / 64 + nseg) return SATTN_ENOSPACE;
  const QuantWs ws = quant_ws(nseg, H);
  if (use_scratch) workspace_bytes = kScratchBytes;
  if (workspace_bytes < ws.total) return SATTN_ENOSPACE;

  QuantLaunch a;
  a.q = static_cast<const uint16_t*>(q.ptr);
  a.k = static_cast<const uint16_t*>(k.ptr);
  a.v = static_cast<const uint16_t*>(v.ptr);
  a.gq = SegGeom{cu_seqlens_q, nseg, Lq, q.stride_b};
  a.gk = SegGeom{cu_seqlens_k, nseg, Lk, k.stride_b};
  a.gv = SegGeom{cu_seqlens_k, nseg, Lk, v.stride_b};
  a.q_st = q.stride_t; a.q_sh = q.stride_h;
  a.k_st = k.stride_t; a.k_sh = k.stride_h;
  a.v_st = v.stride_t; a.v_sh = v.stride_h;
  a.nseg = nseg;
  a.H = H;
  a.q_blocks = !do_q ? 0 : varlen ? out->qblk_cap : nseg * ceil64(Lq);
  a.k_blocks = varlen ? out->kblk_cap : nseg * ceil64(Lk);
  a.q8 = out->q; a.q_scale = out->q_scale;
  a.k8 = out->k; a.k_scale = out->k_scale; a.k_mean = out->k_mean;
  a.v8 = out->v; a.v_scale = out->v_scale;
  a.qblk_cap = out->qblk_cap; a.kblk_cap = out->kblk_cap;
  a.q_scale_shift = q_scale_shift(out);
  a.workspace = workspace;
  a.ws_sums_bytes = ws.sums;
  a.ws_vmax_bytes = ws.vmax;
  // the statistics and the Q blocks share one 1-D grid; K/V blocks are the x extent of another
  if (a.q_blocks > kMaxGroups256 || a.k_blocks > kMaxGroups256 ||
      (int64_t)stats_chunks(nseg, H) * nseg * H + a.q_blocks * H > kMaxGroups256)
    return SATTN_EUNSUPPORTED;
  if (use_scratch) {
    const sattn_status st = scratch_for_current_device(&a.workspace);
    if (st != SATTN_OK) return st;
  }
  return launch_quantize(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SATTN_OK : SATTN_EHIP;
}

sattn_status sattn_quantize_qkv(sattn_bf16_in q, sattn_bf16_in k, sattn_bf16_in v, int nseg, int H, int D, int64_t Lq,
                                int64_t Lk, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                const sattn_qkv_quant* out, void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_impl(q, k, v, nseg, H, D, Lq, Lk, cu_seqlens_q, cu_seqlens_k, out, workspace, workspace_bytes, false,
                       stream);
}

sattn_status sattn_quantize_qkv_noalloc(sattn_bf16_in q, sattn_bf16_in k, sattn_bf16_in v, int nseg, int H, int D,
                                        int64_t Lq, int64_t Lk, const int32_t* cu_seqlens_q,
                                        const int32_t* cu_seqlens_k, const sattn_qkv_quant* out, void* stream) {
  return quantize_impl(q, k, v, nseg, H, D, Lq, Lk, cu_seqlens_q, cu_seqlens_k, out, nullptr, 0, true, stream);
}

size_t sattn_noalloc_scratch_bytes(void) { return kScratchBytes; }

static sattn_status fwd_common(const sattn_qkv_quant* qkv, int H, int D, float sm_scale, sattn_bf16_out o,
                               bool dense, bool need_q = true) {
  if (H < 1) return SATTN_EINVAL;
  if (D != kD) return SATTN_EUNSUPPORTED;
  if (!quant_bufs_ok(qkv, need_q)) return SATTN_EINVAL;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return SATTN_EINVAL;
  if (!view_ok(o.ptr, o.stride_b, o.stride_t, o.stride_h, dense)) return SATTN_EINVAL;
  return SATTN_OK;
}

static float log2e_scale(float sm_scale) { return (float)((double)sm_scale * 1.4426950408889634); }

// The key split of a dense forward (p.split = pieces per split tile, their blocks added to
// the grid, the workspace's counters and partials wired in) when the workspace is given and
// large enough, the keys span enough epochs and the tiles of the last dispatch round can
// each have 2 or 4 CUs; else no split.  `grid` = 8 blocks per work index (one per XCD).
static sattn_status plan_split(AttnParams& p, int64_t& grid, int64_t Lk, void* workspace, size_t workspace_bytes) {
  p.split = 1;
  if (workspace == nullptr || ceil64(Lk) < kSplitMinEpochs) return SATTN_OK;
  int cus = 0;
  if (cu_count(&cus) != SATTN_OK) return SATTN_EHIP;
  const int64_t per_xcd = grid / 8;            // work items per XCD
  const int64_t slots = (int64_t)cus / 4;      // two workgroups per CU, cus / 8 CUs per XCD
  const int64_t last = per_xcd % slots;        // the last round's items (all of them in a short grid)
  if (last == 0) return SATTN_OK;
  const int64_t tiles = (p.H < 8 ? p.H : 8) * last;  // XCDs with heads x last-round items
  int np = 0;
  for (int k = kMaxPieces; k >= 2 && np == 0; k /= 2)
    if (k * last <= cus / 8 && ceil64(Lk) >= kSplitMinEpochs * k / 2 &&
        tiles <= (k == 2 ? kSplitMaxTiles : kSplitMaxTiles4) && workspace_bytes >= split_ws_bytes(tiles, k))
      np = k;
  if (np == 0) return SATTN_OK;
  p.split = np;
  p.split_from = per_xcd - last;
  for (int q = 0; q < np; ++q)
    p.split_e[q] = (int)(ceil64(Lk) * (np == 2 ? kSplitShare2[q] : kSplitShare4[q]) / 1000);
  p.cnt = static_cast<int32_t*>(workspace);
  p.part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    (split_ws_bytes(tiles, np) - (size_t)tiles * np * kSplitPieceBytes));
  grid += 8 * last * (np - 1);
  return SATTN_OK;
}

static sattn_status fwd_dense(const sattn_qkv_quant* qkv, int B, int H, int Lq, int Lk, int D, float sm_scale,
                              sattn_bf16_out o, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1 || Lq < 0 || Lk < 0) return SATTN_EINVAL;
  sattn_status st = fwd_common(qkv, H, D, sm_scale, o, true);
  if (st != SATTN_OK) return st;
  if (qkv->qblk_cap < (int64_t)B * ceil64(Lq) || qkv->kblk_cap < (int64_t)B * ceil64(Lk)) return SATTN_ENOSPACE;
  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.q8 = qkv->q; p.q_scale = qkv->q_scale;
  p.k8 = qkv->k; p.k_scale = qkv->k_scale;
  p.v8 = qkv->v; p.v_scale = qkv->v_scale;
  p.qblk_cap = qkv->qblk_cap; p.kblk_cap = qkv->kblk_cap;
  p.H = H; p.nseg = B;
  p.gq = SegGeom{nullptr, B, Lq, o.stride_b};
  p.gk = SegGeom{nullptr, B, Lk, 0};
  p.c32 = log2e_scale(sm_scale);
  p.o = static_cast<uint16_t*>(o.ptr);
  p.o_st = o.stride_t; p.o_sh = o.stride_h;
  p.q_scale_shift = q_scale_shift(qkv);
  p.max_kblocks = ceil64(Lk);
  const int qpw = attn_queries_per_wg();
  const int64_t ntile = ceil64(Lq) * 64 / qpw + (ceil64(Lq) * 64 % qpw != 0);
  int64_t grid = 8 * (int64_t)((H + 7) / 8) * B * ntile;
  if (grid > kMaxGroups256) return SATTN_EUNSUPPORTED;
  st = plan_split(p, grid, Lk, workspace, workspace_bytes);
  if (st != SATTN_OK) return st;
  return launch_attention(p, grid, false, static_cast<hipStream_t>(stream)) == hipSuccess ? SATTN_OK : SATTN_EHIP;
}

sattn_status sattn_fwd(const sattn_qkv_quant* qkv, int B, int H, int Lq, int Lk, int D, float sm_scale,
                       sattn_bf16_out o, void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace != nullptr && !aligned16(workspace)) return SATTN_EINVAL;
  return fwd_dense(qkv, B, H, Lq, Lk, D, sm_scale, o, workspace, workspace_bytes, stream);
}

sattn_status sattn_debug_scores(const sattn_qkv_quant* qkv, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int nseg, int64_t Lq, int64_t Lk, int H, int D, float sm_scale, int seg, int head,
                                int64_t q_begin, int64_t q_end, int64_t q_step, const sattn_checkpoints* ck,
                                sattn_bf16_out o, void* stream) {
  if (nseg < 1 || Lq < 0 || Lk < 0 || ck == nullptr) return SATTN_EINVAL;
  const bool varlen = cu_seqlens_q != nullptr;
  if ((cu_seqlens_k != nullptr) != varlen) return SATTN_EINVAL;
  sattn_status st = fwd_common(qkv, H, D, sm_scale, o, !varlen);
  if (st != SATTN_OK) return st;
  if (seg < 0 || seg >= nseg || head < 0 || head >= H || q_begin < 0 || q_end <= q_begin || q_step < 1 ||
      ck->ld < 0 || ck->nep < 0 || ((ck->acc || ck->s) && ck->ld < 1) ||
      ((ck->m || ck->d || ck->alpha || ck->p8 || ck->ro) && ck->nep < 1))
    return SATTN_EINVAL;
  int64_t q_clip, k_clip;
  if (varlen) {
    if (qkv->qblk_cap < nseg || qkv->kblk_cap < nseg) return SATTN_ENOSPACE;
    q_clip = Lq < clip_for_cap(qkv->qblk_cap, nseg) ? Lq : clip_for_cap(qkv->qblk_cap, nseg);
    k_clip = Lk < clip_for_cap(qkv->kblk_cap, nseg) ? Lk : clip_for_cap(qkv->kblk_cap, nseg);
  } else {
    if (qkv->qblk_cap < (int64_t)nseg * ceil64(Lq) || qkv->kblk_cap < (int64_t)nseg * ceil64(Lk))
      return SATTN_ENOSPACE;
    q_clip = Lq;
    k_clip = Lk;
  }
  if (q_end > q_clip) q_end = q_clip;  // no segment holds more queries than the view
  if (q_end <= q_begin) return SATTN_OK;
  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.q8 = qkv->q; p.q_scale = qkv->q_scale;
  p.k8 = qkv->k; p.k_scale = qkv->k_scale;
  p.v8 = qkv->v; p.v_scale = qkv->v_scale;
  p.qblk_cap = qkv->qblk_cap; p.kblk_cap = qkv->kblk_cap;
  p.H = H; p.nseg = nseg;
  p.gq = SegGeom{cu_seqlens_q, nseg, q_clip, varlen ? 0 : o.stride_b};
  p.gk = SegGeom{cu_seqlens_k, nseg, k_clip, 0};
  p.c32 = log2e_scale(sm_scale);
  p.o = static_cast<uint16_t*>(o.ptr);
  p.o_st = o.stride_t; p.o_sh = o.stride_h;
  p.q_scale_shift = q_scale_shift(qkv);
  p.max_kblocks = ceil64(k_clip);  // selects the K-scale path exactly as the forward does
  DumpParams& d = p.dump;
  d.acc = ck->acc; d.s = ck->s; d.ld = ck->ld;
  d.m = ck->m; d.d = ck->d; d.alpha = ck->alpha; d.p8 = ck->p8; d.ro = ck->ro; d.nep = ck->nep;
  d.rcp = ck->rcp;
  d.seg = seg; d.head = head;
  d.q0 = q_begin; d.q1 = q_end; d.qstep = q_step;
  const int qpw = attn_queries_per_wg();
  d.tile0 = q_begin / qpw;
  const int64_t grid = (q_end - 1) / qpw - d.tile0 + 1;
  if (grid > kMaxGroups256) return SATTN_EUNSUPPORTED;
  return launch_attention(p, grid, true, static_cast<hipStream_t>(stream)) == hipSuccess ? SATTN_OK : SATTN_EHIP;
}

sattn_status sattn_fwd_varlen(const sattn_qkv_quant* qkv, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int nseg, int64_t total_q, int64_t total_k, int H, int D, float sm_scale,
                              sattn_bf16_out o, void* workspace, size_t workspace_bytes, void* stream) {
  if (nseg < 1 || total_q < 0 || total_k < 0 || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)
    return SATTN_EINVAL;
  sattn_status st = fwd_common(qkv, H, D, sm_scale, o, false);
  if (st != SATTN_OK) return st;
  if (workspace == nullptr || !aligned16(workspace)) return SATTN_EINVAL;
  if (workspace_bytes < fwd_ws(nseg)) return SATTN_ENOSPACE;
  if (qkv->qblk_cap < nseg || qkv->kblk_cap < nseg) return SATTN_ENOSPACE;
  int32_t* order = static_cast<int32_t*>(workspace);
  int32_t* tpref = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align_up((size_t)nseg * 4));
  const int64_t q_clip = total_q < clip_for_cap(qkv->qblk_cap, nseg) ? total_q : clip_for_cap(qkv->qblk_cap, nseg);
  // the quantizer's clipping: keys past the K/V views' total_k tokens were never quantized
  const int64_t k_clip = total_k < clip_for_cap(qkv->kblk_cap, nseg) ? total_k : clip_for_cap(qkv->kblk_cap, nseg);
  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.q8 = qkv->q; p.q_scale = qkv->q_scale;
  p.k8 = qkv->k; p.k_scale = qkv->k_scale;
  p.v8 = qkv->v; p.v_scale = qkv->v_scale;
  p.qblk_cap = qkv->qblk_cap; p.kblk_cap = qkv->kblk_cap;
  p.H = H; p.nseg = nseg;
  p.gq = SegGeom{cu_seqlens_q, nseg, q_clip, 0};
  p.gk = SegGeom{cu_seqlens_k, nseg, k_clip, 0};
  p.order = order; p.tpref = tpref;
  p.c32 = log2e_scale(sm_scale);
  p.o = static_cast<uint16_t*>(o.ptr);
  p.o_st = o.stride_t; p.o_sh = o.stride_h;
  p.q_scale_shift = q_scale_shift(qkv);
  p.max_kblocks = ceil64(k_clip);
  const int64_t tiles_bound = q_clip / attn_queries_per_wg() + nseg + 1;
  const int64_t grid = 8 * (int64_t)((H + 7) / 8) * tiles_bound;
  if (grid > kMaxGroups256) return SATTN_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_plan(cu_seqlens_q, cu_seqlens_k, nseg, q_clip, k_clip, order, tpref, s) != hipSuccess) return SATTN_EHIP;
  return launch_attention(p, grid, false, s) == hipSuccess ? SATTN_OK : SATTN_EHIP;
}

sattn_status sattn_fwd_fused(const sattn_qkv_quant* kv, sattn_bf16_in q, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k, int nseg, int H, int64_t Lq, int64_t Lk, int D,
                             float sm_scale, sattn_bf16_out o, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (nseg < 1 || Lq < 0 || Lk < 0) return SATTN_EINVAL;
  const bool varlen = cu_seqlens_q != nullptr;
  if ((cu_seqlens_k != nullptr) != varlen) return SATTN_EINVAL;
  sattn_status st = fwd_common(kv, H, D, sm_scale, o, !varlen, false);
  if (st != SATTN_OK) return st;
  if (!view_ok(q.ptr, q.stride_b, q.stride_t, q.stride_h, !varlen)) return SATTN_EINVAL;
  if (varlen && workspace == nullptr) return SATTN_EINVAL;
  if (workspace != nullptr && !aligned16(workspace)) return SATTN_EINVAL;
  if (varlen && workspace_bytes < fwd_ws(nseg)) return SATTN_ENOSPACE;
  if (kv->kblk_cap < nseg || (!varlen && kv->kblk_cap < (int64_t)nseg * ceil64(Lk))) return SATTN_ENOSPACE;
  const int64_t k_clip = varlen ? (Lk < clip_for_cap(kv->kblk_cap, nseg) ? Lk : clip_for_cap(kv->kblk_cap, nseg))
                                : Lk;
  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.k8 = kv->k; p.k_scale = kv->k_scale;
  p.v8 = kv->v; p.v_scale = kv->v_scale;
  p.kblk_cap = kv->kblk_cap;
  p.H = H; p.nseg = nseg;
  p.gq = SegGeom{cu_seqlens_q, nseg, Lq, varlen ? 0 : o.stride_b};
  p.gk = SegGeom{cu_seqlens_k, nseg, k_clip, 0};
  p.c32 = log2e_scale(sm_scale);
  p.o = static_cast<uint16_t*>(o.ptr);
  p.o_st = o.stride_t; p.o_sh = o.stride_h;
  p.q_scale_shift = q_scale_shift(kv);
  p.max_kblocks = ceil64(k_clip);
  p.qbf = static_cast<const uint16_t*>(q.ptr);
  p.qb_sb = q.stride_b; p.qb_st = q.stride_t; p.qb_sh = q.stride_h;
  const int qpw = attn_queries_per_wg();
  const int64_t ntile = (ceil64(Lq) * 64 + qpw - 1) / qpw;
  int64_t grid = varlen ? 8 * (int64_t)((H + 7) / 8) * (Lq / qpw + nseg + 1) : 8 * (int64_t)((H + 7) / 8) * nseg * ntile;
  if (grid > kMaxGroups256) return SATTN_EUNSUPPORTED;
  if (!varlen) {  // dense: the key split, as in sattn_fwd
    st = plan_split(p, grid, Lk, workspace, workspace_bytes);
    if (st != SATTN_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (varlen) {
    p.order = static_cast<int32_t*>(workspace);
    p.tpref = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align_up((size_t)nseg * 4));
    if (launch_plan(cu_seqlens_q, cu_seqlens_k, nseg, Lq, k_clip, const_cast<int32_t*>(p.order),
                    const_cast<int32_t*>(p.tpref), s) != hipSuccess)
      return SATTN_EHIP;
  }
  return launch_attention(p, grid, false, s) == hipSuccess ? SATTN_OK : SATTN_EHIP;
}

}  // extern "C"
