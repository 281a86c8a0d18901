// A consumer of the C ABI that uses neither Python nor PyTorch: it reads one problem from a
// file, sizes and allocates every buffer itself (hipMalloc) from sattn_quant_query, runs
// sattn_quantize_qkv and sattn_fwd / sattn_fwd_varlen on a stream of its own, and writes the
// BF16 output.  Built next to the library by the package's build step; driven by
// tests/test_gpu_c_abi.py.
//
// Input file, little-endian: int32 mode (0 dense, 1 packed), nseg, H, Lq, Lk (dense: tokens
// per segment; packed: total tokens), float32 sm_scale; packed only: int32 cu_q[nseg + 1],
// cu_k[nseg + 1]; then the BF16 bits of Q, K and V, contiguous ([nseg, L, H, 128] dense,
// [T, H, 128] packed).  Output file: the BF16 bits of O, shaped like Q.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "sattn.h"

namespace {

constexpr int kD = 128;

bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

bool sattn_ok(sattn_status s, const char* what) {
  if (s == SATTN_OK) return true;
  std::fprintf(stderr, "%s: %s\n", what, sattn_status_string(s));
  return false;
}

template <typename T>
bool read_all(std::FILE* f, T* dst, size_t n) {
  return std::fread(dst, sizeof(T), n, f) == n;
}

// Device buffers released on every exit path.
struct DeviceBuffers {
  std::vector<void*> ptrs;
  bool failed = false;
  void* get(size_t bytes) {
    void* p = nullptr;
    if (hipMalloc(&p, bytes > 0 ? bytes : 16) != hipSuccess) {
      failed = true;
      return nullptr;
    }
    ptrs.push_back(p);
    return p;
  }
  ~DeviceBuffers() {
    for (void* p : ptrs) (void)hipFree(p);
  }
};

int run(const char* in_path, const char* out_path) {
  std::FILE* f = std::fopen(in_path, "rb");
  if (!f) {
    std::fprintf(stderr, "cannot open %s\n", in_path);
    return 1;
  }
  int32_t hdr[5];
  float sm_scale = 0.f;
  if (!read_all(f, hdr, 5) || !read_all(f, &sm_scale, 1)) {
    std::fclose(f);
    std::fprintf(stderr, "short header\n");
    return 1;
  }
  const bool packed = hdr[0] == 1;
  const int nseg = hdr[1], H = hdr[2];
  const int64_t Lq = hdr[3], Lk = hdr[4];
  std::vector<int32_t> cu_q, cu_k;
  if (packed) {
    cu_q.resize(nseg + 1);
    cu_k.resize(nseg + 1);
    if (!read_all(f, cu_q.data(), cu_q.size()) || !read_all(f, cu_k.data(), cu_k.size())) {
      std::fclose(f);
      std::fprintf(stderr, "short cu_seqlens\n");
      return 1;
    }
  }
  const int64_t tq = packed ? Lq : nseg * Lq, tk = packed ? Lk : nseg * Lk;
  std::vector<uint16_t> q(tq * H * kD), k(tk * H * kD), v(tk * H * kD);
  const bool ok = read_all(f, q.data(), q.size()) && read_all(f, k.data(), k.size()) &&
                  read_all(f, v.data(), v.size());
  std::fclose(f);
  if (!ok) {
    std::fprintf(stderr, "short tensor data\n");
    return 1;
  }

  sattn_sizes sz;
  if (!sattn_ok(sattn_quant_query(nseg, tq, tk, H, kD, &sz), "sattn_quant_query")) return 1;
  DeviceBuffers mem;
  void* dq = mem.get(q.size() * 2);
  void* dk = mem.get(k.size() * 2);
  void* dv = mem.get(v.size() * 2);
  void* dout = mem.get(q.size() * 2);
  sattn_qkv_quant quant;
  quant.q = static_cast<int8_t*>(mem.get(sz.q_bytes));
  quant.q_scale = static_cast<float*>(mem.get(sz.q_scale_bytes));
  quant.k = static_cast<int8_t*>(mem.get(sz.k_bytes));
  quant.k_scale = static_cast<float*>(mem.get(sz.k_scale_bytes));
  quant.k_mean = static_cast<float*>(mem.get(sz.k_mean_bytes));
  quant.v = static_cast<uint8_t*>(mem.get(sz.v_bytes));
  quant.v_scale = static_cast<float*>(mem.get(sz.v_scale_bytes));
  quant.qblk_cap = sz.qblk_cap;
  quant.kblk_cap = sz.kblk_cap;
  quant.q_scale_rows = 64;
  void* qws = mem.get(sz.quant_workspace_bytes);
  void* fws = mem.get(sz.fwd_workspace_bytes);
  int32_t* dcq = packed ? static_cast<int32_t*>(mem.get(cu_q.size() * 4)) : nullptr;
  int32_t* dck = packed ? static_cast<int32_t*>(mem.get(cu_k.size() * 4)) : nullptr;
  if (mem.failed) {
    std::fprintf(stderr, "hipMalloc failed\n");
    return 1;
  }
  if (!hip_ok(hipMemcpy(dq, q.data(), q.size() * 2, hipMemcpyHostToDevice), "copy q") ||
      !hip_ok(hipMemcpy(dk, k.data(), k.size() * 2, hipMemcpyHostToDevice), "copy k") ||
      !hip_ok(hipMemcpy(dv, v.data(), v.size() * 2, hipMemcpyHostToDevice), "copy v"))
    return 1;
  if (packed && (!hip_ok(hipMemcpy(dcq, cu_q.data(), cu_q.size() * 4, hipMemcpyHostToDevice), "copy cu_q") ||
                 !hip_ok(hipMemcpy(dck, cu_k.data(), cu_k.size() * 4, hipMemcpyHostToDevice), "copy cu_k")))
    return 1;

  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;
  // element strides of contiguous [seg, L, H, D] (dense) or [T, H, D] (packed) tensors
  const int64_t st = (int64_t)H * kD, sh = kD;
  const sattn_bf16_in qin{dq, packed ? 0 : Lq * st, st, sh};
  const sattn_bf16_in kin{dk, packed ? 0 : Lk * st, st, sh};
  const sattn_bf16_in vin{dv, packed ? 0 : Lk * st, st, sh};
  const sattn_bf16_out o{dout, packed ? 0 : Lq * st, st, sh};
  bool good = sattn_ok(sattn_quantize_qkv(qin, kin, vin, nseg, H, kD, Lq, Lk, dcq, dck, &quant, qws,
                                          sz.quant_workspace_bytes, stream),
                       "sattn_quantize_qkv");
  if (good && packed)
    good = sattn_ok(sattn_fwd_varlen(&quant, dcq, dck, nseg, tq, tk, H, kD, sm_scale, o, fws, sz.fwd_workspace_bytes,
                                     stream),
                    "sattn_fwd_varlen");
  else if (good)
    good = sattn_ok(sattn_fwd(&quant, nseg, H, (int)Lq, (int)Lk, kD, sm_scale, o, nullptr, 0, stream), "sattn_fwd");
  good = hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize") && good;
  (void)hipStreamDestroy(stream);
  if (!good) return 1;

  std::vector<uint16_t> out(q.size());
  if (!hip_ok(hipMemcpy(out.data(), dout, out.size() * 2, hipMemcpyDeviceToHost), "copy out")) return 1;
  std::FILE* g = std::fopen(out_path, "wb");
  if (!g || std::fwrite(out.data(), 2, out.size(), g) != out.size()) {
    std::fprintf(stderr, "cannot write %s\n", out_path);
    if (g) std::fclose(g);
    return 1;
  }
  std::fclose(g);
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s problem.bin output.bin\n", argv[0]);
    return 2;
  }
  return run(argv[1], argv[2]);
}
