// nvq_api.cpp -- the C ABI of libnvq (declared in include/nvq.h).
//
// Every entry validates its arguments on the host first (pointers, shapes,
// alignment) and returns a negative status before touching the HIP runtime, so a
// rejected call enqueues nothing and leaves outputs untouched.  Only then is the
// current device's architecture checked (gfx950 only; there is no other code
// path) and the kernel enqueued on the caller's stream.
#include "nvq.h"
#include "nvq_probe.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "nvq_launch.h"

namespace {

thread_local char g_err[512] = "";

nvq_status fail(nvq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shapes are bounded so that every byte offset fits comfortably in int64 and every
// grid dimension in 32 bits.
constexpr int64_t kMaxDim = int64_t(1) << 31;
constexpr int64_t kMaxElems = int64_t(1) << 40;
// Largest M of the tiled entries (grid dimension y counts 16-token tiles).
constexpr int64_t kMaxM = int64_t(1) << 20;

nvq_status check_dims(int64_t M, int64_t N, int64_t K, int64_t kmul, int64_t mmin, int64_t mmax) {
  if (K < kmul || K % kmul != 0) return fail(NVQ_ERR_SHAPE, "K=%lld must be a positive multiple of %lld", (long long)K, (long long)kmul);
  if (K >= kMaxDim) return fail(NVQ_ERR_SHAPE, "K=%lld too large", (long long)K);
  if (N < 1 || N >= kMaxDim) return fail(NVQ_ERR_SHAPE, "N=%lld out of range", (long long)N);
  if (M < mmin || M > mmax) return fail(NVQ_ERR_SHAPE, "M=%lld outside [%lld, %lld] for this entry", (long long)M, (long long)mmin, (long long)mmax);
  if (M > kMaxElems / K || N > kMaxElems / K || M > kMaxElems / N)
    return fail(NVQ_ERR_SHAPE, "M*K, N*K or M*N too large");
  return NVQ_OK;
}

// Per-device result of the architecture check: 0 unknown, 1 gfx950, -1 other.
// Written once per device; the only state the library keeps.
std::atomic<int> g_arch_ok[64];

nvq_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(NVQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(NVQ_ERR_DEVICE, "device index %d unsupported", dev);
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(NVQ_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(NVQ_ERR_DEVICE, "device %d is not gfx950", dev);
  return NVQ_OK;
}

nvq_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(NVQ_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return NVQ_OK;
}

#define NVQ_TRY(x)                  \
  do {                              \
    nvq_status s_ = (x);            \
    if (s_ != NVQ_OK) return s_;    \
  } while (0)

}  // namespace

extern "C" {

const char* nvq_status_str(nvq_status s) {
  switch (s) {
    case NVQ_OK: return "NVQ_OK";
    case NVQ_ERR_NULL: return "NVQ_ERR_NULL";
    case NVQ_ERR_SHAPE: return "NVQ_ERR_SHAPE";
    case NVQ_ERR_RANGE: return "NVQ_ERR_RANGE";
    case NVQ_ERR_ALIGN: return "NVQ_ERR_ALIGN";
    case NVQ_ERR_DEVICE: return "NVQ_ERR_DEVICE";
    case NVQ_ERR_HIP: return "NVQ_ERR_HIP";
    case NVQ_ERR_WORKSPACE: return "NVQ_ERR_WORKSPACE";
    default: return "NVQ_ERR_UNKNOWN";
  }
}

const char* nvq_last_error(void) { return g_err; }

size_t nvq_nvfp4_weight_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 64 || K % 64 != 0 || N >= kMaxDim || K >= kMaxDim || N > kMaxElems / K) return 0;
  const int64_t np = (N + 15) / 16 * 16, kp = (K + 127) / 128 * 128;
  return (size_t)(np * kp / 2 + np * kp / 16);
}

size_t nvq_q4_1_weight_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 32 || K % 32 != 0 || N >= kMaxDim || K >= kMaxDim || N > kMaxElems / K) return 0;
  return (size_t)(N * K / 2 + N * K / 8);
}

size_t nvq_q4_k_weight_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 256 || K % 256 != 0 || N >= kMaxDim || K >= kMaxDim || N > kMaxElems / K) return 0;
  return (size_t)(N * K / 2 + N * (K / 256) * 16);
}

size_t nvq_q5_k_weight_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 256 || K % 256 != 0 || N >= kMaxDim || K >= kMaxDim || N > kMaxElems / K) return 0;
  return (size_t)(N * (K / 256) * 176);
}

size_t nvq_q6_k_weight_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 256 || K % 256 != 0 || N >= kMaxDim || K >= kMaxDim || N > kMaxElems / K) return 0;
  return (size_t)(N * (K / 256) * 210);
}

size_t nvq_iq4_xs_weight_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 256 || K % 256 != 0 || N >= kMaxDim || K >= kMaxDim || N > kMaxElems / K) return 0;
  return (size_t)(N * K / 2 + N * (K / 256) * 8);
}

size_t nvq_gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
  // fp32 partial tiles of the K-split work items that fill the last round over the
  // compute units (the two-term and integer-MFMA GEMM kernels).
  if (M < 1 || N < 1 || K < 64 || K % 64 != 0) return 0;
  if (fmt == NVQ_FMT_NVFP4) return nvq::gemm_nvfp4_workspace(M, N, K);
  if (fmt == NVQ_FMT_Q4_1) return nvq::gemm_q4_1_workspace(M, N, K);
  if ((fmt == NVQ_FMT_Q4_K || fmt == NVQ_FMT_IQ4_XS || fmt == NVQ_FMT_Q5_K || fmt == NVQ_FMT_Q6_K) && K % 256 == 0)
    return nvq::gemm_q4_k_workspace(M, N, K, fmt == NVQ_FMT_Q6_K);
  return 0;
}

nvq_status nvq_pack_nvfp4(const uint8_t* codes, const uint8_t* ue4m3, int64_t N, int64_t K,
                          void* dst_host) {
  if (!codes || !ue4m3 || !dst_host) return fail(NVQ_ERR_NULL, "nvq_pack_nvfp4: NULL pointer");
  if (nvq_nvfp4_weight_bytes(N, K) == 0) return fail(NVQ_ERR_SHAPE, "nvq_pack_nvfp4: N=%lld K=%lld (K %% 64 == 0 required)", (long long)N, (long long)K);
  for (int64_t i = 0; i < N * K; ++i)
    if (codes[i] > 15) return fail(NVQ_ERR_RANGE, "nvq_pack_nvfp4: code > 15 at weight %lld", (long long)i);
  for (int64_t i = 0; i < N * K / 16; ++i)
    if ((ue4m3[i] & 0x80) || ue4m3[i] == 0x7F) return fail(NVQ_ERR_RANGE, "nvq_pack_nvfp4: invalid UE4M3 byte 0x%02x at scale %lld", ue4m3[i], (long long)i);
  // Tile-interleaved layout: 16-row x 128-k tile-chunks; codes of lane l = 16*g + n
  // (row n, k = 32g .. 32g+31 of the chunk) at 16*l, scales (subblocks 2g, 2g+1)
  // at 2*l of the chunk's 128-byte scale block.  Padding rows / k are zero.
  uint8_t* dst = static_cast<uint8_t*>(dst_host);
  const int64_t ntiles = (N + 15) / 16, nch = (K + 127) / 128, ns = K / 16;
  uint8_t* sc = dst + ntiles * nch * 1024;
  for (int64_t t = 0; t < ntiles; ++t)
    for (int64_t c = 0; c < nch; ++c) {
      uint8_t* blk = dst + (t * nch + c) * 1024;
      uint8_t* sblk = sc + (t * nch + c) * 128;
      for (int l = 0; l < 64; ++l) {
        const int64_t row = t * 16 + (l & 15);
        const int64_t k0 = c * 128 + 32 * (l >> 4);
        const bool live = row < N && k0 < K;
        const uint8_t* cr = codes + row * K + k0;
        for (int b = 0; b < 16; ++b)
          blk[16 * l + b] = live ? (uint8_t)(cr[2 * b] | (cr[2 * b + 1] << 4)) : 0;
        for (int j = 0; j < 2; ++j) {
          const int64_t s = k0 / 16 + j;
          sblk[2 * l + j] = (live && s < ns) ? ue4m3[row * ns + s] : 0;
        }
      }
    }
  g_err[0] = '\0';
  return NVQ_OK;
}

}  // extern "C"

namespace {

// The packers check every input before writing any byte of dst.
nvq_status check_max(const uint8_t* v, int64_t n, unsigned maxv, const char* who, const char* what) {
  for (int64_t i = 0; i < n; ++i)
    if (v[i] > maxv) return fail(NVQ_ERR_RANGE, "%s: %s > %u at index %lld", who, what, maxv, (long long)i);
  return NVQ_OK;
}

// codes (their low four bits) two per byte: code 2i in bits 0..3, 2i+1 in bits 4..7
void pack_nibbles(const uint8_t* q, int64_t n, uint8_t* dst) {
  for (int64_t i = 0; i < n / 2; ++i) dst[i] = (uint8_t)((q[2 * i] & 15) | ((q[2 * i + 1] & 15) << 4));
}

// 16-byte K-quant header per 256 weights: d, dmin, then sc_0..7, mn_0..7 as 6-bit
// fields of a little-endian 96-bit number
void pack_kq_headers(const uint8_t* sc, const uint8_t* mn, const uint16_t* d, const uint16_t* dmin, int64_t nsb,
                     uint8_t* dst) {
  for (int64_t i = 0; i < nsb; ++i) {
    uint8_t h[16] = {};
    std::memcpy(h, &d[i], 2);
    std::memcpy(h + 2, &dmin[i], 2);
    for (int f = 0; f < 16; ++f) {
      const uint8_t v = f < 8 ? sc[8 * i + f] : mn[8 * i + f - 8];
      for (int bit = 0; bit < 6; ++bit)
        if ((v >> bit) & 1) h[4 + (6 * f + bit) / 8] |= (uint8_t)(1u << ((6 * f + bit) % 8));
    }
    std::memcpy(dst + 16 * i, h, 16);
  }
}

// bit `bit` of 32 codes as one word: even codes k = 2e at bit e, odd codes k = 2e + 1 at
// bit 16 + e (the arrangement the kernels' even / odd code planes read)
uint32_t pack_code_bits(const uint8_t* q32, int bit) {
  uint32_t w = 0;
  for (int e = 0; e < 16; ++e) {
    w |= (uint32_t)((q32[2 * e] >> bit) & 1) << e;
    w |= (uint32_t)((q32[2 * e + 1] >> bit) & 1) << (16 + e);
  }
  return w;
}

}  // namespace

extern "C" {

nvq_status nvq_pack_q4_1(const uint8_t* q, const uint16_t* d_f16, const uint16_t* m_f16,
                         int64_t N, int64_t K, void* dst_host) {
  if (!q || !d_f16 || !m_f16 || !dst_host) return fail(NVQ_ERR_NULL, "nvq_pack_q4_1: NULL pointer");
  if (nvq_q4_1_weight_bytes(N, K) == 0) return fail(NVQ_ERR_SHAPE, "nvq_pack_q4_1: N=%lld K=%lld (K %% 32 == 0 required)", (long long)N, (long long)K);
  NVQ_TRY(check_max(q, N * K, 15, "nvq_pack_q4_1", "code"));
  uint8_t* dst = static_cast<uint8_t*>(dst_host);
  const int64_t nc = N * K / 2;
  pack_nibbles(q, N * K, dst);
  const int64_t nb = N * K / 32;
  for (int64_t i = 0; i < nb; ++i) {
    const uint32_t pair = (uint32_t)d_f16[i] | ((uint32_t)m_f16[i] << 16);
    std::memcpy(dst + nc + 4 * i, &pair, 4);
  }
  g_err[0] = '\0';
  return NVQ_OK;
}

nvq_status nvq_pack_q4_k(const uint8_t* q, const uint8_t* sc, const uint8_t* mn, const uint16_t* d_f16,
                         const uint16_t* dmin_f16, int64_t N, int64_t K, void* dst_host) {
  if (!q || !sc || !mn || !d_f16 || !dmin_f16 || !dst_host) return fail(NVQ_ERR_NULL, "nvq_pack_q4_k: NULL pointer");
  if (nvq_q4_k_weight_bytes(N, K) == 0) return fail(NVQ_ERR_SHAPE, "nvq_pack_q4_k: N=%lld K=%lld (K %% 256 == 0 required)", (long long)N, (long long)K);
  NVQ_TRY(check_max(q, N * K, 15, "nvq_pack_q4_k", "code"));
  NVQ_TRY(check_max(sc, N * K / 32, 63, "nvq_pack_q4_k", "scale"));
  NVQ_TRY(check_max(mn, N * K / 32, 63, "nvq_pack_q4_k", "min"));
  uint8_t* dst = static_cast<uint8_t*>(dst_host);
  pack_nibbles(q, N * K, dst);
  pack_kq_headers(sc, mn, d_f16, dmin_f16, N * K / 256, dst + N * K / 2);
  g_err[0] = '\0';
  return NVQ_OK;
}

nvq_status nvq_pack_q5_k(const uint8_t* q, const uint8_t* sc, const uint8_t* mn, const uint16_t* d_f16,
                         const uint16_t* dmin_f16, int64_t N, int64_t K, void* dst_host) {
  if (!q || !sc || !mn || !d_f16 || !dmin_f16 || !dst_host) return fail(NVQ_ERR_NULL, "nvq_pack_q5_k: NULL pointer");
  if (nvq_q5_k_weight_bytes(N, K) == 0) return fail(NVQ_ERR_SHAPE, "nvq_pack_q5_k: N=%lld K=%lld (K %% 256 == 0 required)", (long long)N, (long long)K);
  NVQ_TRY(check_max(q, N * K, 31, "nvq_pack_q5_k", "code"));
  NVQ_TRY(check_max(sc, N * K / 32, 63, "nvq_pack_q5_k", "scale"));
  NVQ_TRY(check_max(mn, N * K / 32, 63, "nvq_pack_q5_k", "min"));
  uint8_t* dst = static_cast<uint8_t*>(dst_host);
  pack_nibbles(q, N * K, dst);
  pack_kq_headers(sc, mn, d_f16, dmin_f16, N * K / 256, dst + N * K / 2);
  uint8_t* hb = dst + N * K / 2 + N * K / 16;
  for (int64_t b = 0; b < N * K / 32; ++b) {
    const uint32_t w4 = pack_code_bits(q + 32 * b, 4);
    std::memcpy(hb + 4 * b, &w4, 4);
  }
  g_err[0] = '\0';
  return NVQ_OK;
}

nvq_status nvq_pack_q6_k(const uint8_t* q, const int8_t* sc, const uint16_t* d_f16, int64_t N, int64_t K,
                         void* dst_host) {
  if (!q || !sc || !d_f16 || !dst_host) return fail(NVQ_ERR_NULL, "nvq_pack_q6_k: NULL pointer");
  if (nvq_q6_k_weight_bytes(N, K) == 0) return fail(NVQ_ERR_SHAPE, "nvq_pack_q6_k: N=%lld K=%lld (K %% 256 == 0 required)", (long long)N, (long long)K);
  NVQ_TRY(check_max(q, N * K, 63, "nvq_pack_q6_k", "code"));
  uint8_t* dst = static_cast<uint8_t*>(dst_host);
  pack_nibbles(q, N * K, dst);
  std::memcpy(dst + N * K / 2, sc, (size_t)(N * K / 16));
  uint8_t* hb = dst + N * K / 2 + N * K / 16;
  for (int64_t b = 0; b < N * K / 32; ++b) {
    const uint32_t w[2] = {pack_code_bits(q + 32 * b, 4), pack_code_bits(q + 32 * b, 5)};
    std::memcpy(hb + 8 * b, w, 8);
  }
  std::memcpy(dst + N * K / 2 + N * K / 16 + N * K / 4, d_f16, (size_t)(N * K / 256) * 2);
  g_err[0] = '\0';
  return NVQ_OK;
}

nvq_status nvq_pack_iq4_xs(const uint8_t* q, const uint8_t* ls, const uint16_t* d_f16, int64_t N, int64_t K,
                           void* dst_host) {
  if (!q || !ls || !d_f16 || !dst_host) return fail(NVQ_ERR_NULL, "nvq_pack_iq4_xs: NULL pointer");
  if (nvq_iq4_xs_weight_bytes(N, K) == 0) return fail(NVQ_ERR_SHAPE, "nvq_pack_iq4_xs: N=%lld K=%lld (K %% 256 == 0 required)", (long long)N, (long long)K);
  NVQ_TRY(check_max(q, N * K, 15, "nvq_pack_iq4_xs", "code"));
  NVQ_TRY(check_max(ls, N * K / 32, 63, "nvq_pack_iq4_xs", "scale"));
  uint8_t* dst = static_cast<uint8_t*>(dst_host);
  const int64_t nc = N * K / 2;
  pack_nibbles(q, N * K, dst);
  // one 8-byte header per (row, 256 weights): d, then ls_0..7 as 6-bit fields of a
  // little-endian 48-bit number
  const int64_t nsb = N * K / 256;
  for (int64_t i = 0; i < nsb; ++i) {
    uint64_t f = 0;
    for (int j = 0; j < 8; ++j) f |= (uint64_t)ls[8 * i + j] << (6 * j);
    uint8_t h[8];
    std::memcpy(h, &d_f16[i], 2);
    for (int b = 0; b < 6; ++b) h[2 + b] = (uint8_t)(f >> (8 * b));
    std::memcpy(dst + nc + 8 * i, h, 8);
  }
  g_err[0] = '\0';
  return NVQ_OK;
}

nvq_status nvq_quantize_act_q8_0(const float* x, int64_t M, int64_t K, int8_t* q,
                                 uint16_t* d_f16, int16_t* bsum16, void* stream) {
  if (!x || !q || !d_f16) return fail(NVQ_ERR_NULL, "nvq_quantize_act_q8_0: NULL pointer");
  if (K < 32 || K % 32 != 0 || K >= kMaxDim) return fail(NVQ_ERR_SHAPE, "nvq_quantize_act_q8_0: K=%lld must be a positive multiple of 32", (long long)K);
  if (M < 1 || M > kMaxElems / K) return fail(NVQ_ERR_SHAPE, "nvq_quantize_act_q8_0: M=%lld out of range", (long long)M);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(d_f16, 2) || (bsum16 && !aligned(bsum16, 2)))
    return fail(NVQ_ERR_ALIGN, "nvq_quantize_act_q8_0: x and q must be 16-byte aligned, d_f16/bsum16 2-byte");
  NVQ_TRY(check_device());
  return launched(nvq::launch_act_quant(x, M, K, q, d_f16, bsum16, (hipStream_t)stream), "act_quant");
}

static nvq_status check_common(const void* w, const int8_t* q, const uint16_t* d_f16, const void* y, const char* who) {
  if (!w || !q || !d_f16 || !y) return fail(NVQ_ERR_NULL, "%s: NULL pointer", who);
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(y, 16) || !aligned(d_f16, 2))
    return fail(NVQ_ERR_ALIGN, "%s: w, q and y must be 16-byte aligned, d_f16 2-byte", who);
  return NVQ_OK;
}

// The decode GEMV kernels keep the whole activation table of a row in LDS.
static bool gemv_fits_lds(int64_t K) { return nvq::gemv_lds_bytes(K) <= 160 * 1024 - 1024; }

nvq_status nvq_gemv_nvfp4(const void* w, float w_scale, const int8_t* q, const uint16_t* d_f16,
                          int64_t M, int64_t N, int64_t K, float* y, void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemv_nvfp4"));
  NVQ_TRY(check_dims(M, N, K, 64, 1, NVQ_GEMV_MAX_M));
  if (M > 1 && M * K >= (int64_t(1) << 32))  // the batched kernel indexes activations in 32 bits
    return fail(NVQ_ERR_SHAPE, "nvq_gemv_nvfp4: M*K=%lld too large for the batched kernel (< 2^32)", (long long)(M * K));
  NVQ_TRY(check_device());
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  if (M == 1 && gemv_fits_lds(K))
    return launched(nvq::launch_gemv_nvfp4_m1(wb, w_scale, q, d_f16, N, K, y, nullptr, 0, (hipStream_t)stream), "gemv_nvfp4");
  if (M > 1)
    return launched(nvq::launch_gemv_nvfp4_batch_f16(wb, w_scale, q, d_f16, M, N, K, y, nullptr, (hipStream_t)stream), "gemv_nvfp4 (batched)");
  return launched(nvq::launch_gemm_nvfp4(wb, w_scale, q, d_f16, M, N, K, y, nullptr, nullptr, (hipStream_t)stream), "gemv_nvfp4 (tiled)");
}

nvq_status nvq_gemv_nvfp4_fused(const void* w, float w_scale, const float* x, int64_t N, int64_t K, float* y,
                                int8_t* q_out, uint16_t* d_out, void* stream) {
  if (!w || !x || !y) return fail(NVQ_ERR_NULL, "nvq_gemv_nvfp4_fused: NULL pointer");
  if ((q_out == nullptr) != (d_out == nullptr))
    return fail(NVQ_ERR_NULL, "nvq_gemv_nvfp4_fused: q_out and d_out are given together or not at all");
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 16) || (q_out && !aligned(q_out, 16)) ||
      (d_out && !aligned(d_out, 2)))
    return fail(NVQ_ERR_ALIGN, "nvq_gemv_nvfp4_fused: w, x, y and q_out must be 16-byte aligned, d_out 2-byte");
  NVQ_TRY(check_dims(1, N, K, 64, 1, 1));
  if (!gemv_fits_lds(K)) return fail(NVQ_ERR_SHAPE, "nvq_gemv_nvfp4_fused: K=%lld too large for the LDS activation table", (long long)K);
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemv_nvfp4_fused(static_cast<const uint8_t*>(w), w_scale, x, N, K, y, q_out, d_out,
                                               (hipStream_t)stream), "gemv_nvfp4_fused");
}

nvq_status nvq_gemv_nvfp4_routed(const void* w, const float* w_scales, const int32_t* ids, int64_t n_experts,
                                 int64_t n_active, const int8_t* q, const uint16_t* d_f16, int64_t M, int64_t N,
                                 int64_t K, float* y, void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemv_nvfp4_routed"));
  if (!w_scales || !ids) return fail(NVQ_ERR_NULL, "nvq_gemv_nvfp4_routed: NULL pointer");
  if (!aligned(w_scales, 4) || !aligned(ids, 4))
    return fail(NVQ_ERR_ALIGN, "nvq_gemv_nvfp4_routed: w_scales and ids must be 4-byte aligned");
  if (n_experts < 1 || n_experts >= kMaxDim || n_active < 1 || n_active > 65535)
    return fail(NVQ_ERR_SHAPE, "nvq_gemv_nvfp4_routed: n_experts=%lld n_active=%lld out of range", (long long)n_experts,
                (long long)n_active);
  NVQ_TRY(check_dims(M, N, K, 64, 1, 65535 / n_active));
  if (!gemv_fits_lds(K)) return fail(NVQ_ERR_SHAPE, "nvq_gemv_nvfp4_routed: K=%lld too large for the LDS activation table", (long long)K);
  if ((int64_t)nvq_nvfp4_weight_bytes(N, K) > (int64_t)INT64_MAX / n_experts)
    return fail(NVQ_ERR_SHAPE, "nvq_gemv_nvfp4_routed: expert table too large");
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemv_nvfp4_routed(static_cast<const uint8_t*>(w), w_scales, ids, n_experts, n_active, M, q,
                                                d_f16, N, K, y, (hipStream_t)stream),
                  "gemv_nvfp4_routed");
}

nvq_status nvq_gemv_nvfp4_dot4(const void* w, float w_scale, const int8_t* q, const uint16_t* d_f16,
                               int64_t M, int64_t N, int64_t K, float* y, void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemv_nvfp4_dot4"));
  NVQ_TRY(check_dims(M, N, K, 64, 1, NVQ_GEMV_MAX_M));
  if (!gemv_fits_lds(K)) return fail(NVQ_ERR_SHAPE, "nvq_gemv_nvfp4_dot4: K=%lld too large for the LDS activation table", (long long)K);
  NVQ_TRY(check_device());
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  for (int64_t m = 0; m < M; ++m) {
    hipError_t e = nvq::launch_gemv_nvfp4_m1(wb, w_scale, q + m * K, d_f16 + m * (K / 32), N, K, y + m * N,
                                             nullptr, 1, (hipStream_t)stream);
    if (e != hipSuccess) return fail(NVQ_ERR_HIP, "gemv_nvfp4_dot4 launch: %s", hipGetErrorString(e));
  }
  g_err[0] = '\0';
  return NVQ_OK;
}

static nvq_status check_gemm_nvfp4(const void* w, const int8_t* q, const uint16_t* d_f16, const void* y, int64_t M,
                                    int64_t N, int64_t K, const char* who) {
  NVQ_TRY(check_common(w, q, d_f16, y, who));
  NVQ_TRY(check_dims(M, N, K, 64, 16, kMaxM));
  if ((M + 255) / 256 > (int64_t)1 << 31 || (N + 255) / 256 > (((int64_t)1 << 31) - 1) / ((M + 255) / 256))
    return fail(NVQ_ERR_SHAPE, "%s: M=%lld x N=%lld has too many 256 x 256 tiles for one launch", who, (long long)M, (long long)N);
  return NVQ_OK;
}

nvq_status nvq_gemm_nvfp4(const void* w, float w_scale, const int8_t* q, const uint16_t* d_f16,
                          int64_t M, int64_t N, int64_t K, float* y, void* workspace,
                          size_t ws_bytes, void* stream) {
  NVQ_TRY(check_gemm_nvfp4(w, q, d_f16, y, M, N, K, "nvq_gemm_nvfp4"));
  const size_t need = nvq_gemm_workspace_bytes(NVQ_FMT_NVFP4, M, N, K);
  if (ws_bytes < need || (need && !workspace)) return fail(NVQ_ERR_WORKSPACE, "nvq_gemm_nvfp4: workspace of %zu bytes required", need);
  if (need && !aligned(workspace, 16)) return fail(NVQ_ERR_ALIGN, "nvq_gemm_nvfp4: workspace must be 16-byte aligned");
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemm_nvfp4(static_cast<const uint8_t*>(w), w_scale, q, d_f16, M, N, K, y, nullptr,
                                         static_cast<float*>(workspace), (hipStream_t)stream), "gemm_nvfp4");
}

nvq_status nvq_gemm_nvfp4_noalloc(const void* w, float w_scale, const int8_t* q, const uint16_t* d_f16,
                                  int64_t M, int64_t N, int64_t K, float* y, void* stream) {
  NVQ_TRY(check_gemm_nvfp4(w, q, d_f16, y, M, N, K, "nvq_gemm_nvfp4_noalloc"));
  const size_t need = nvq_gemm_workspace_bytes(NVQ_FMT_NVFP4, M, N, K);
  if (need > nvq::gemm_nvfp4_noalloc_scratch_bytes() || need > NVQ_NOALLOC_SCRATCH_BYTES)
    return fail(NVQ_ERR_WORKSPACE, "nvq_gemm_nvfp4_noalloc: shape needs %zu bytes of scratch, more than the static %zu",
                need, (size_t)NVQ_NOALLOC_SCRATCH_BYTES);
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemm_nvfp4_noalloc(static_cast<const uint8_t*>(w), w_scale, q, d_f16, M, N, K, y,
                                                 (hipStream_t)stream), "gemm_nvfp4_noalloc");
}

nvq_status nvq_gemv_q4_1(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemv_q4_1"));
  if (!bsum16) return fail(NVQ_ERR_NULL, "nvq_gemv_q4_1: bsum16 is required");
  if (!aligned(bsum16, 2)) return fail(NVQ_ERR_ALIGN, "nvq_gemv_q4_1: bsum16 must be 2-byte aligned");
  NVQ_TRY(check_dims(M, N, K, 32, 1, NVQ_GEMV_MAX_M));
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemv_q4_1(static_cast<const uint8_t*>(w), q, d_f16, bsum16, M, N, K, y, nullptr,
                                        (hipStream_t)stream), "gemv_q4_1");
}

nvq_status nvq_gemm_q4_1(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* workspace, size_t ws_bytes, void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemm_q4_1"));
  if (!bsum16) return fail(NVQ_ERR_NULL, "nvq_gemm_q4_1: bsum16 is required");
  if (!aligned(bsum16, 2)) return fail(NVQ_ERR_ALIGN, "nvq_gemm_q4_1: bsum16 must be 2-byte aligned");
  NVQ_TRY(check_dims(M, N, K, 32, 16, kMaxM));
  const size_t need = nvq_gemm_workspace_bytes(NVQ_FMT_Q4_1, M, N, K);
  if (ws_bytes < need || (need && !workspace)) return fail(NVQ_ERR_WORKSPACE, "nvq_gemm_q4_1: workspace of %zu bytes required", need);
  if (need && !aligned(workspace, 16)) return fail(NVQ_ERR_ALIGN, "nvq_gemm_q4_1: workspace must be 16-byte aligned");
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemm_q4_1(static_cast<const uint8_t*>(w), q, d_f16, bsum16, M, N, K, y, nullptr,
                                        static_cast<float*>(workspace), (hipStream_t)stream), "gemm_q4_1");
}

nvq_status nvq_gemv_q4_k(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemv_q4_k"));
  if (!bsum16) return fail(NVQ_ERR_NULL, "nvq_gemv_q4_k: bsum16 is required");
  if (!aligned(bsum16, 2)) return fail(NVQ_ERR_ALIGN, "nvq_gemv_q4_k: bsum16 must be 2-byte aligned");
  NVQ_TRY(check_dims(M, N, K, 256, 1, NVQ_GEMV_MAX_M));
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemv_q4_k(static_cast<const uint8_t*>(w), q, d_f16, bsum16, M, N, K, y, nullptr,
                                        (hipStream_t)stream), "gemv_q4_k");
}

nvq_status nvq_gemm_q4_k(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* workspace, size_t ws_bytes, void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemm_q4_k"));
  if (!bsum16) return fail(NVQ_ERR_NULL, "nvq_gemm_q4_k: bsum16 is required");
  if (!aligned(bsum16, 2)) return fail(NVQ_ERR_ALIGN, "nvq_gemm_q4_k: bsum16 must be 2-byte aligned");
  NVQ_TRY(check_dims(M, N, K, 256, 16, kMaxM));
  const size_t need = nvq_gemm_workspace_bytes(NVQ_FMT_Q4_K, M, N, K);
  if (ws_bytes < need || (need && !workspace)) return fail(NVQ_ERR_WORKSPACE, "nvq_gemm_q4_k: workspace of %zu bytes required", need);
  if (need && !aligned(workspace, 16)) return fail(NVQ_ERR_ALIGN, "nvq_gemm_q4_k: workspace must be 16-byte aligned");
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemm_q4_k(static_cast<const uint8_t*>(w), q, d_f16, bsum16, M, N, K, y, nullptr,
                                        static_cast<float*>(workspace), (hipStream_t)stream), "gemm_q4_k");
}

nvq_status nvq_gemv_q5_k(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemv_q5_k"));
  if (!bsum16) return fail(NVQ_ERR_NULL, "nvq_gemv_q5_k: bsum16 is required");
  if (!aligned(bsum16, 2)) return fail(NVQ_ERR_ALIGN, "nvq_gemv_q5_k: bsum16 must be 2-byte aligned");
  NVQ_TRY(check_dims(M, N, K, 256, 1, NVQ_GEMV_MAX_M));
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemv_q5_k(static_cast<const uint8_t*>(w), q, d_f16, bsum16, M, N, K, y, nullptr,
                                        (hipStream_t)stream), "gemv_q5_k");
}

nvq_status nvq_gemm_q5_k(const void* w, const int8_t* q, const uint16_t* d_f16,
                         const int16_t* bsum16, int64_t M, int64_t N, int64_t K, float* y,
                         void* workspace, size_t ws_bytes, void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemm_q5_k"));
  if (!bsum16) return fail(NVQ_ERR_NULL, "nvq_gemm_q5_k: bsum16 is required");
  if (!aligned(bsum16, 2)) return fail(NVQ_ERR_ALIGN, "nvq_gemm_q5_k: bsum16 must be 2-byte aligned");
  NVQ_TRY(check_dims(M, N, K, 256, 16, kMaxM));
  const size_t need = nvq_gemm_workspace_bytes(NVQ_FMT_Q5_K, M, N, K);
  if (ws_bytes < need || (need && !workspace)) return fail(NVQ_ERR_WORKSPACE, "nvq_gemm_q5_k: workspace of %zu bytes required", need);
  if (need && !aligned(workspace, 16)) return fail(NVQ_ERR_ALIGN, "nvq_gemm_q5_k: workspace must be 16-byte aligned");
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemm_q5_k(static_cast<const uint8_t*>(w), q, d_f16, bsum16, M, N, K, y, nullptr,
                                        static_cast<float*>(workspace), (hipStream_t)stream), "gemm_q5_k");
}

nvq_status nvq_gemv_q6_k(const void* w, const int8_t* q, const uint16_t* d_f16, int64_t M, int64_t N, int64_t K,
                         float* y, void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemv_q6_k"));
  NVQ_TRY(check_dims(M, N, K, 256, 1, NVQ_GEMV_MAX_M));
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemv_q6_k(static_cast<const uint8_t*>(w), q, d_f16, M, N, K, y, nullptr,
                                        (hipStream_t)stream), "gemv_q6_k");
}

nvq_status nvq_gemm_q6_k(const void* w, const int8_t* q, const uint16_t* d_f16, int64_t M, int64_t N, int64_t K,
                         float* y, void* workspace, size_t ws_bytes, void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemm_q6_k"));
  NVQ_TRY(check_dims(M, N, K, 256, 16, kMaxM));
  const size_t need = nvq_gemm_workspace_bytes(NVQ_FMT_Q6_K, M, N, K);
  if (ws_bytes < need || (need && !workspace)) return fail(NVQ_ERR_WORKSPACE, "nvq_gemm_q6_k: workspace of %zu bytes required", need);
  if (need && !aligned(workspace, 16)) return fail(NVQ_ERR_ALIGN, "nvq_gemm_q6_k: workspace must be 16-byte aligned");
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemm_q6_k(static_cast<const uint8_t*>(w), q, d_f16, M, N, K, y, nullptr,
                                        static_cast<float*>(workspace), (hipStream_t)stream), "gemm_q6_k");
}

nvq_status nvq_gemv_iq4_xs(const void* w, const int8_t* table, const int8_t* q, const uint16_t* d_f16, int64_t M,
                           int64_t N, int64_t K, float* y, void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemv_iq4_xs"));
  if (!table) return fail(NVQ_ERR_NULL, "nvq_gemv_iq4_xs: table is required");
  NVQ_TRY(check_dims(M, N, K, 256, 1, NVQ_GEMV_MAX_M));
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemv_iq4_xs(static_cast<const uint8_t*>(w), table, q, d_f16, M, N, K, y, nullptr,
                                          (hipStream_t)stream), "gemv_iq4_xs");
}

nvq_status nvq_gemm_iq4_xs(const void* w, const int8_t* table, const int8_t* q, const uint16_t* d_f16, int64_t M,
                           int64_t N, int64_t K, float* y, void* workspace, size_t ws_bytes, void* stream) {
  NVQ_TRY(check_common(w, q, d_f16, y, "nvq_gemm_iq4_xs"));
  if (!table) return fail(NVQ_ERR_NULL, "nvq_gemm_iq4_xs: table is required");
  NVQ_TRY(check_dims(M, N, K, 256, 16, kMaxM));
  const size_t need = nvq_gemm_workspace_bytes(NVQ_FMT_IQ4_XS, M, N, K);
  if (ws_bytes < need || (need && !workspace)) return fail(NVQ_ERR_WORKSPACE, "nvq_gemm_iq4_xs: workspace of %zu bytes required", need);
  if (need && !aligned(workspace, 16)) return fail(NVQ_ERR_ALIGN, "nvq_gemm_iq4_xs: workspace must be 16-byte aligned");
  NVQ_TRY(check_device());
  return launched(nvq::launch_gemm_iq4_xs(static_cast<const uint8_t*>(w), table, q, d_f16, M, N, K, y, nullptr,
                                          static_cast<float*>(workspace), (hipStream_t)stream), "gemm_iq4_xs");
}

nvq_status nvq_debug_isums_iq4_xs(const int8_t* table, int path, const void* w, const int8_t* q, int64_t M,
                                  int64_t N, int64_t K, int32_t* isums, void* stream) {
  if (path != NVQ_PATH_GEMV && path != NVQ_PATH_GEMM) return fail(NVQ_ERR_RANGE, "nvq_debug_isums_iq4_xs: path=%d", path);
  if (!table || !w || !q || !isums) return fail(NVQ_ERR_NULL, "nvq_debug_isums_iq4_xs: NULL pointer");
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(isums, 4)) return fail(NVQ_ERR_ALIGN, "nvq_debug_isums_iq4_xs: w and q must be 16-byte aligned, isums 4-byte");
  NVQ_TRY(check_dims(M, N, K, 256, 1, kMaxM));
  if (M > kMaxElems / (N * (K / 16))) return fail(NVQ_ERR_SHAPE, "nvq_debug_isums_iq4_xs: output too large");
  NVQ_TRY(check_device());
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  hipStream_t st = (hipStream_t)stream;
  if (path == NVQ_PATH_GEMM)
    return launched(nvq::launch_gemm_iq4_xs(wb, table, q, nullptr, M, N, K, nullptr, isums, nullptr, st), "debug gemm_iq4_xs");
  return launched(nvq::launch_gemv_iq4_xs(wb, table, q, nullptr, M, N, K, nullptr, isums, st), "debug gemv_iq4_xs");
}

nvq_status nvq_debug_isums(int fmt, int path, const void* w, const int8_t* q, int64_t M,
                           int64_t N, int64_t K, int32_t* isums, void* stream) {
  if (fmt != NVQ_FMT_NVFP4 && fmt != NVQ_FMT_Q4_1 && fmt != NVQ_FMT_Q4_K && fmt != NVQ_FMT_Q5_K && fmt != NVQ_FMT_Q6_K)
    return fail(NVQ_ERR_RANGE, "nvq_debug_isums: fmt=%d (IQ4_XS sums need its value table: nvq_debug_isums_iq4_xs)", fmt);
  const bool kq = fmt == NVQ_FMT_Q4_K || fmt == NVQ_FMT_Q5_K || fmt == NVQ_FMT_Q6_K;
  if (path != NVQ_PATH_GEMV && path != NVQ_PATH_GEMM && !(path == NVQ_PATH_GEMV_DOT4 && fmt == NVQ_FMT_NVFP4))
    return fail(NVQ_ERR_RANGE, "nvq_debug_isums: path=%d", path);
  if (!w || !q || !isums) return fail(NVQ_ERR_NULL, "nvq_debug_isums: NULL pointer");
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(isums, 4)) return fail(NVQ_ERR_ALIGN, "nvq_debug_isums: w and q must be 16-byte aligned, isums 4-byte");
  NVQ_TRY(check_dims(M, N, K, fmt == NVQ_FMT_NVFP4 ? 64 : (kq ? 256 : 32), 1, kMaxM));
  if (M > kMaxElems / (N * (K / 16))) return fail(NVQ_ERR_SHAPE, "nvq_debug_isums: output too large");
  if (fmt == NVQ_FMT_NVFP4 && path == NVQ_PATH_GEMV && M > 1 && (M < 16 ? M : 16) * K >= (int64_t(1) << 32))
    return fail(NVQ_ERR_SHAPE, "nvq_debug_isums: K=%lld too large for the batched kernel (16 * K < 2^32)", (long long)K);
  if (path == NVQ_PATH_GEMV_DOT4 && !gemv_fits_lds(K))
    return fail(NVQ_ERR_SHAPE, "nvq_debug_isums: K=%lld too large for the v_dot4 decode kernel", (long long)K);
  NVQ_TRY(check_device());
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  hipStream_t st = (hipStream_t)stream;
  // The sums come from the kernel the product entry would run for this shape: the GEMM
  // dispatch (tiled at M = 1, batched up to 16, two-term above) or the GEMV dispatch
  // (the M = 1 decode kernel, or the tiled one for rows past its LDS table; the
  // batched kernel for M >= 2, 16 tokens per launch).
  if (path == NVQ_PATH_GEMM) {
    if (fmt == NVQ_FMT_NVFP4) return launched(nvq::launch_gemm_nvfp4(wb, 1.0f, q, nullptr, M, N, K, nullptr, isums, nullptr, st), "debug gemm_nvfp4");
    if (fmt == NVQ_FMT_Q4_K) return launched(nvq::launch_gemm_q4_k(wb, q, nullptr, nullptr, M, N, K, nullptr, isums, nullptr, st), "debug gemm_q4_k");
    if (fmt == NVQ_FMT_Q5_K) return launched(nvq::launch_gemm_q5_k(wb, q, nullptr, nullptr, M, N, K, nullptr, isums, nullptr, st), "debug gemm_q5_k");
    if (fmt == NVQ_FMT_Q6_K) return launched(nvq::launch_gemm_q6_k(wb, q, nullptr, M, N, K, nullptr, isums, nullptr, st), "debug gemm_q6_k");
    return launched(nvq::launch_gemm_q4_1(wb, q, nullptr, nullptr, M, N, K, nullptr, isums, nullptr, st), "debug gemm_q4_1");
  }
  if (fmt == NVQ_FMT_Q4_1) return launched(nvq::launch_gemv_q4_1(wb, q, nullptr, nullptr, M, N, K, nullptr, isums, st), "debug gemv_q4_1");
  if (fmt == NVQ_FMT_Q4_K) return launched(nvq::launch_gemv_q4_k(wb, q, nullptr, nullptr, M, N, K, nullptr, isums, st), "debug gemv_q4_k");
  if (fmt == NVQ_FMT_Q5_K) return launched(nvq::launch_gemv_q5_k(wb, q, nullptr, nullptr, M, N, K, nullptr, isums, st), "debug gemv_q5_k");
  if (fmt == NVQ_FMT_Q6_K) return launched(nvq::launch_gemv_q6_k(wb, q, nullptr, M, N, K, nullptr, isums, st), "debug gemv_q6_k");
  if (path == NVQ_PATH_GEMV) {
    if (M > 1) return launched(nvq::launch_gemv_nvfp4_batch_f16(wb, 1.0f, q, nullptr, M, N, K, nullptr, isums, st), "debug gemv_nvfp4 (batched)");
    if (!gemv_fits_lds(K)) return launched(nvq::launch_gemm_nvfp4(wb, 1.0f, q, nullptr, M, N, K, nullptr, isums, nullptr, st), "debug gemv_nvfp4 (tiled)");
  }
  const int64_t per_m = N * (K / 16);
  for (int64_t m = 0; m < M; ++m) {
    hipError_t e = nvq::launch_gemv_nvfp4_m1(wb, 1.0f, q + m * K, nullptr, N, K, nullptr, isums + m * per_m,
                                             path == NVQ_PATH_GEMV_DOT4 ? 1 : 0, st);
    if (e != hipSuccess) return fail(NVQ_ERR_HIP, "debug gemv launch: %s", hipGetErrorString(e));
  }
  g_err[0] = '\0';
  return NVQ_OK;
}

// ---- measurement probes (include/nvq_probe.h) ----

nvq_status nvq_probe_read(const void* src, size_t bytes, int blocks, uint32_t* sink, void* stream) {
  if (!src || !sink) return fail(NVQ_ERR_NULL, "nvq_probe_read: NULL pointer");
  if (!aligned(src, 16) || !aligned(sink, 4))
    return fail(NVQ_ERR_ALIGN, "nvq_probe_read: src must be 16-byte aligned, sink 4-byte");
  if (bytes == 0 || bytes % 16 != 0 || bytes >= (size_t(1) << 46))
    return fail(NVQ_ERR_SHAPE, "nvq_probe_read: bytes=%zu must be a positive multiple of 16", bytes);
  if (blocks < 1 || blocks > 65536) return fail(NVQ_ERR_SHAPE, "nvq_probe_read: blocks=%d outside [1, 65536]", blocks);
  NVQ_TRY(check_device());
  return launched(nvq::launch_probe_read(src, (int64_t)(bytes / 16), blocks, sink, (hipStream_t)stream), "probe_read");
}

nvq_status nvq_probe_gemv_loads(const void* w, int64_t N, int64_t K, int splits, int waves, int batch,
                                uint32_t* sink, void* stream) {
  if (!w || !sink) return fail(NVQ_ERR_NULL, "nvq_probe_gemv_loads: NULL pointer");
  if (!aligned(w, 16) || !aligned(sink, 4))
    return fail(NVQ_ERR_ALIGN, "nvq_probe_gemv_loads: w must be 16-byte aligned, sink 4-byte");
  NVQ_TRY(check_dims(1, N, K, 64, 1, 1));
  const int64_t nch = (K + 127) / 128;
  if (splits < 1 || splits > 8 || splits > nch)
    return fail(NVQ_ERR_RANGE, "nvq_probe_gemv_loads: splits=%d outside [1, min(8, %lld)]", splits, (long long)nch);
  if ((waves != 4 && waves != 8 && waves != 16) || (batch != 3 && batch != 5))
    return fail(NVQ_ERR_RANGE, "nvq_probe_gemv_loads: waves=%d, batch=%d not in {4, 8, 16} x {3, 5}", waves, batch);
  if (((N + 15) / 16) * splits >= (int64_t(1) << 31))
    return fail(NVQ_ERR_SHAPE, "nvq_probe_gemv_loads: grid too large");
  NVQ_TRY(check_device());
  return launched(nvq::launch_probe_gemv_loads(static_cast<const uint8_t*>(w), N, K, splits, waves, batch, sink,
                                               (hipStream_t)stream), "probe_gemv_loads");
}

nvq_status nvq_probe_mfma(int blocks, int64_t iters, int random_operands, float* out, void* stream) {
  if (!out) return fail(NVQ_ERR_NULL, "nvq_probe_mfma: NULL pointer");
  if (!aligned(out, 4)) return fail(NVQ_ERR_ALIGN, "nvq_probe_mfma: out must be 4-byte aligned");
  if (blocks < 1 || blocks > 65536) return fail(NVQ_ERR_SHAPE, "nvq_probe_mfma: blocks=%d outside [1, 65536]", blocks);
  if (iters < 1 || iters > (int64_t(1) << 31)) return fail(NVQ_ERR_SHAPE, "nvq_probe_mfma: iters=%lld outside [1, 2^31]", (long long)iters);
  NVQ_TRY(check_device());
  return launched(nvq::launch_probe_mfma(blocks, iters, random_operands, out, (hipStream_t)stream), "probe_mfma");
}

}  // extern "C"
