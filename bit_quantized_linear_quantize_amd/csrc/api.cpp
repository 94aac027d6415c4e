// C-ABI host layer: argument validation, workspace carve-up, launches and
// error reporting for the entry points declared in include/svdq_w4a4.h.
//
// Validation rules (the pages: only the (precision, group size) pairs of the
// "Supported quantization types" table exist; a quantized checkpoint must
// match its model exactly, "Load a quantized pipeline" note; unsupported GPUs
// are rejected at load time, news article's hardware section):
//   (int4, 64) and (nvfp4, 16) only; AWQ group 64      -> SVDQ_EUNSUPPORTED
//   rank in 0..128, multiple of 16                      -> SVDQ_EUNSUPPORTED
//   M >= 1, K % 128 == 0, 128 <= K <= 16384, N % 64 == 0 -> SVDQ_EINVAL
//   svdq: at most 2^23 - 1 output tiles of 256 x 192     -> SVDQ_EINVAL
//   null / non-16-byte-aligned pointers, out overlapping an input or the
//   workspace, wtscale != 1 for int4                      -> SVDQ_EINVAL
//   workspace too small                                 -> SVDQ_EWORKSPACE
//   device not gfx950                                   -> SVDQ_EARCH
// Everything is checked before the first launch, so on error nothing is
// written.  The library is stateless apart from a per-device architecture
// cache and a thread-local error message.

#include "../../include/svdq_w4a4.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>

#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

constexpr int64_t kMaxM = int64_t(1) << 24;
constexpr int64_t kMaxK = 16384;
constexpr int64_t kMaxPrepRows = int64_t(1) << 22;  // calibration rows and weight rows of the smoothing call
constexpr size_t kAlign = 16;

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

size_t round_up(size_t v) { return (v + 255) & ~size_t(255); }

struct Range {
  const void* p;
  size_t bytes;
};

bool overlaps(const Range& a, const Range& b) {
  if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool arch_is_gfx950(const char* arch) { return arch && std::strncmp(arch, "gfx950", 6) == 0; }

// Lazy, per-device architecture check (first call on a device queries it).
int check_device_arch() {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SVDQ_EDEVICE, std::string("hipGetDevice failed: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(SVDQ_EDEVICE, "device index out of range");
  int c = cache[dev].load(std::memory_order_acquire);
  if (c == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(SVDQ_EDEVICE, std::string("hipGetDeviceProperties failed: ") + hipGetErrorString(e));
    c = arch_is_gfx950(prop.gcnArchName) ? 1 : -1;
    cache[dev].store(c, std::memory_order_release);
    if (c < 0) g_last_error = std::string("device architecture is ") + prop.gcnArchName + ", not gfx950";
  }
  if (c < 0) return fail(SVDQ_EARCH, "device architecture is not gfx950");
  return SVDQ_OK;
}

int check_shape(int64_t M, int64_t K, int64_t N) {
  if (M < 1 || M > kMaxM) return fail(SVDQ_EINVAL, "M must be in [1, 2^24]");
  if (K < 128 || K > kMaxK || K % 128) return fail(SVDQ_EINVAL, "K must be a multiple of 128 in [128, 16384]");
  if (N < 64 || N % 64 || N > (int64_t(1) << 24)) return fail(SVDQ_EINVAL, "N must be a positive multiple of 64");
  return SVDQ_OK;
}

// The product kernel launches one 512-thread workgroup per 256 x 192 output
// tile: the grid must stay below 2^32 work-items.
constexpr int64_t kMaxGemmTiles = (int64_t(1) << 23) - 1;

int check_gemm_tiles(int64_t M, int64_t N) {
  if (((M + 255) / 256) * ((N + 191) / 192) > kMaxGemmTiles)
    return fail(SVDQ_EINVAL, "M x N too large: more than 2^23 - 1 output tiles of 256 x 192");
  return SVDQ_OK;
}

int check_svdq_kind(int precision, int group_size, int rank) {
  if (precision == SVDQ_INT4) {
    if (group_size != 64) return fail(SVDQ_EUNSUPPORTED, "int4 requires group_size 64");
  } else if (precision == SVDQ_NVFP4) {
    if (group_size != 16) return fail(SVDQ_EUNSUPPORTED, "nvfp4 requires group_size 16");
  } else {
    return fail(SVDQ_EUNSUPPORTED, "precision must be SVDQ_INT4 or SVDQ_NVFP4");
  }
  if (rank < 0 || rank > 128 || rank % 16) return fail(SVDQ_EUNSUPPORTED, "rank must be a multiple of 16 in [0, 128]");
  return SVDQ_OK;
}

size_t w_scale_bytes(int64_t N, int64_t K, int precision) {
  return precision == SVDQ_INT4 ? size_t(N) * size_t(K / 64) * 2 : size_t(N) * size_t(K / 16);
}

// Base workspace of one layer (each part 256-byte aligned):
//   act_f16    f16 [M, K]   dequantized activations, the product operand
//   row_scale  int4 only: f32 [M], the power of two factored out of each row
//   lora_act   f32 [M, rank]
size_t workspace_bytes(int64_t M, int64_t K, int precision, int rank) {
  size_t b = round_up(size_t(M) * size_t(K) * 2);
  if (precision == SVDQ_INT4) b += round_up(size_t(M) * 4);
  return b + round_up(size_t(M) * size_t(rank) * 4);
}

// Split K for the plain linear: when the 256 x 192 tiles would occupy less
// than half of the 256 compute units, each tile's stages are shared by up to
// 8 workgroups (at least 2 stages each) that write fp32 partials, summed in a
// fixed order by a second kernel.
int choose_ksplit(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 191) / 192);
  const int nst = int(K / 64);
  if (tiles >= 128) return 1;
  int s = int(std::min<int64_t>(8, 256 / tiles));
  s = std::min(s, nst / 2);
  s = std::max(s, 1);
  while (s > 1 && ((nst + s - 1) / s) * (s - 1) >= nst) --s;  // every split gets stages
  return s;
}

size_t split_bytes(int64_t M, int64_t K, int64_t N) {
  const int s = choose_ksplit(M, N, K);
  return s > 1 ? round_up(size_t(s) * size_t(M) * size_t(N) * 4) : 0;
}

// Workspace of svdq_w4a4_linear / svdq_w4a4_gemm: workspace_bytes, then the
// split-K partials fp32 [ksplit, M, N] when K is split.
size_t linear_workspace_bytes(int64_t M, int64_t K, int64_t N, int precision, int rank) {
  return workspace_bytes(M, K, precision, rank) + split_bytes(M, K, N);
}

int validate_svdq(const void* x, int64_t M, int64_t K, int64_t N, const void* packed_w,
                  const void* wscales, float wtscale, const void* smooth, const void* lora_down,
                  const void* lora_up, const void* bias, int precision, int group_size, int rank,
                  const void* out, const void* workspace, size_t workspace_bytes_given) {
  int rc = check_svdq_kind(precision, group_size, rank);
  if (rc) return rc;
  rc = check_shape(M, K, N);
  if (rc) return rc;
  rc = check_gemm_tiles(M, N);
  if (rc) return rc;
  if (!x || !packed_w || !wscales || !smooth || !out || !workspace)
    return fail(SVDQ_EINVAL, "null pointer argument");
  if ((rank > 0) != (lora_down != nullptr) || (rank > 0) != (lora_up != nullptr))
    return fail(SVDQ_EINVAL, "lora_down / lora_up must be non-null exactly when rank > 0");
  const void* ptrs[] = {x, packed_w, wscales, smooth, lora_down, lora_up, bias, out, workspace};
  for (const void* p : ptrs)
    if (p && !aligned(p)) return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  if (precision == SVDQ_INT4 && wtscale != 1.0f) return fail(SVDQ_EINVAL, "wtscale must be 1.0 for int4");
  if (precision == SVDQ_NVFP4 && !(std::isfinite(wtscale) && wtscale > 0.f))
    return fail(SVDQ_EINVAL, "wtscale must be finite and positive");
  const size_t need = linear_workspace_bytes(M, K, N, precision, rank);
  const Range o{out, size_t(M) * size_t(N) * 2};
  const Range ins[] = {{x, size_t(M) * size_t(K) * 2},
                       {packed_w, size_t(N) * size_t(K / 2)},
                       {wscales, w_scale_bytes(N, K, precision)},
                       {smooth, size_t(K) * 2},
                       {lora_down, size_t(rank) * size_t(K) * 2},
                       {lora_up, size_t(N) * size_t(rank) * 2},
                       {bias, size_t(N) * 2},
                       {workspace, need}};
  for (const Range& r : ins)
    if (overlaps(o, r)) return fail(SVDQ_EINVAL, "out overlaps an input or the workspace");
  if (overlaps(Range{x, size_t(M) * size_t(K) * 2}, Range{workspace, need}))
    return fail(SVDQ_EINVAL, "workspace overlaps x");
  if (workspace_bytes_given < need) return fail(SVDQ_EWORKSPACE, "workspace too small");
  return SVDQ_OK;
}

int validate_awq(const void* x, int64_t M, int64_t K, int64_t N, const void* packed_w,
                 const void* wscales, const void* wzeros, const void* bias, int group_size,
                 const void* out) {
  if (group_size != 64) return fail(SVDQ_EUNSUPPORTED, "awq_w4a16 requires group_size 64");
  int rc = check_shape(M, K, N);
  if (rc) return rc;
  if (!x || !packed_w || !wscales || !wzeros || !out) return fail(SVDQ_EINVAL, "null pointer argument");
  const void* ptrs[] = {x, packed_w, wscales, wzeros, bias, out};
  for (const void* p : ptrs)
    if (p && !aligned(p)) return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  const Range o{out, size_t(M) * size_t(N) * 2};
  const Range ins[] = {{x, size_t(M) * size_t(K) * 2},
                       {packed_w, size_t(N) * size_t(K / 2)},
                       {wscales, size_t(N) * size_t(K / 64) * 2},
                       {wzeros, size_t(N) * size_t(K / 64) * 2},
                       {bias, size_t(N) * 2}};
  for (const Range& r : ins)
    if (overlaps(o, r)) return fail(SVDQ_EINVAL, "out overlaps an input");
  return SVDQ_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SVDQ_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
  return SVDQ_OK;
}

struct Carve {
  uint8_t* act_f16;   // f16 [M, K]
  float* row_scale;   // int4: f32 [M]; else null
  float* lora_act;    // f32 [M, rank]
};

Carve carve(void* workspace, int64_t M, int64_t K, int precision) {
  uint8_t* p = static_cast<uint8_t*>(workspace);
  Carve c{};
  c.act_f16 = p;
  p += round_up(size_t(M) * size_t(K) * 2);
  if (precision == SVDQ_INT4) {
    c.row_scale = reinterpret_cast<float*>(p);
    p += round_up(size_t(M) * 4);
  }
  c.lora_act = reinterpret_cast<float*>(p);
  return c;
}

// Kernel 1 into the workspace; `clear` (clear_n floats, optional) is set to
// zero by the same launch.
int launch_quantize(const void* x, int64_t M, int64_t K, const void* smooth, const void* lora_down,
                    int precision, int rank, void* workspace, hipStream_t s, float* clear = nullptr,
                    int64_t clear_n = 0) {
  const Carve c = carve(workspace, M, K, precision);
  svdq::QuantActArgs qa{x, smooth, lora_down, nullptr, nullptr, c.lora_act, c.act_f16, c.row_scale,
                        M, K, precision, rank, clear, clear_n};
  return launch_status(svdq::launch_quantize_act(qa, s), "quantize_act_lora_down launch");
}

// Kernel 2 (plain store) from a linear workspace (linear_workspace_bytes).
int launch_gemm(const void* workspace, int64_t M, int64_t K, int64_t N, const void* packed_w,
                const void* wscales, float wtscale, const void* lora_up, const void* bias, int precision,
                int rank, void* out, hipStream_t s) {
  const Carve c = carve(const_cast<void*>(workspace), M, K, precision);
  svdq::GemmArgs ga{c.act_f16, c.row_scale, c.lora_act, packed_w, wscales, lora_up, bias, out, nullptr,
                    wtscale, M, K, N, precision, rank};
  ga.ksplit = choose_ksplit(M, N, K);
  if (ga.ksplit > 1)
    ga.partial = reinterpret_cast<float*>(static_cast<uint8_t*>(const_cast<void*>(workspace)) +
                                          workspace_bytes(M, K, precision, rank));
  int rc = launch_status(svdq::launch_gemm_w4a4(ga, s), "gemm_w4a4_lora_up launch");
  if (rc || ga.ksplit == 1) return rc;
  return launch_status(svdq::launch_splitk_reduce(ga.partial, ga.ksplit, M, N, bias, out, s), "split-K sum launch");
}

// ---- fused GELU MLP ----------------------------------------------------------

// One layer of svdq_w4a4_mlp_gelu: the svdq_w4a4_linear rules for its own
// tensors (M rows of input), without the input and output buffers.
int validate_layer(int64_t M, const svdq_w4a4_layer* L, const char* which) {
  const std::string w(which);
  if (!L) return fail(SVDQ_EINVAL, w + " layer is null");
  int rc = check_svdq_kind(L->precision, L->group_size, L->rank);
  if (rc) return rc;
  rc = check_shape(M, L->K, L->N);
  if (rc) return rc;
  rc = check_gemm_tiles(M, L->N);
  if (rc) return rc;
  if (!L->packed_w || !L->wscales || !L->smooth) return fail(SVDQ_EINVAL, w + " layer: null pointer");
  if ((L->rank > 0) != (L->lora_down != nullptr) || (L->rank > 0) != (L->lora_up != nullptr))
    return fail(SVDQ_EINVAL, w + " layer: lora_down / lora_up must be non-null exactly when rank > 0");
  const void* ptrs[] = {L->packed_w, L->wscales, L->smooth, L->lora_down, L->lora_up, L->bias};
  for (const void* p : ptrs)
    if (p && !aligned(p)) return fail(SVDQ_EINVAL, w + " layer: pointers must be 16-byte aligned");
  if (L->precision == SVDQ_INT4 && L->wtscale != 1.0f) return fail(SVDQ_EINVAL, w + " layer: wtscale must be 1.0 for int4");
  if (L->precision == SVDQ_NVFP4 && !(std::isfinite(L->wtscale) && L->wtscale > 0.f))
    return fail(SVDQ_EINVAL, w + " layer: wtscale must be finite and positive");
  return SVDQ_OK;
}

size_t mlp_workspace_bytes(int64_t M, const svdq_w4a4_layer* up, const svdq_w4a4_layer* down) {
  return workspace_bytes(M, up->K, up->precision, up->rank) +
         linear_workspace_bytes(M, down->K, down->N, SVDQ_NVFP4, down->rank);
}

int validate_mlp(const void* x, int64_t M, const svdq_w4a4_layer* up, const svdq_w4a4_layer* down,
                 const void* out, const void* workspace, size_t ws_bytes) {
  int rc = validate_layer(M, up, "up");
  if (rc) return rc;
  rc = validate_layer(M, down, "down");
  if (rc) return rc;
  if (up->N != down->K) return fail(SVDQ_EINVAL, "up->N must equal down->K");
  if (down->precision != SVDQ_NVFP4)
    return fail(SVDQ_EUNSUPPORTED, "the fused MLP quantizes the hidden activations as nvfp4: down must be nvfp4");
  if (!x || !out || !workspace) return fail(SVDQ_EINVAL, "null pointer argument");
  if (!aligned(x) || !aligned(out) || !aligned(workspace))
    return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  const size_t need = mlp_workspace_bytes(M, up, down);
  const Range o{out, size_t(M) * size_t(down->N) * 2};
  const Range ins[] = {{x, size_t(M) * size_t(up->K) * 2},
                       {workspace, need},
                       {up->packed_w, size_t(up->N) * size_t(up->K / 2)},
                       {up->wscales, w_scale_bytes(up->N, up->K, up->precision)},
                       {up->smooth, size_t(up->K) * 2},
                       {up->lora_down, size_t(up->rank) * size_t(up->K) * 2},
                       {up->lora_up, size_t(up->N) * size_t(up->rank) * 2},
                       {up->bias, size_t(up->N) * 2},
                       {down->packed_w, size_t(down->N) * size_t(down->K / 2)},
                       {down->wscales, w_scale_bytes(down->N, down->K, down->precision)},
                       {down->smooth, size_t(down->K) * 2},
                       {down->lora_down, size_t(down->rank) * size_t(down->K) * 2},
                       {down->lora_up, size_t(down->N) * size_t(down->rank) * 2},
                       {down->bias, size_t(down->N) * 2}};
  for (const Range& r : ins)
    if (overlaps(o, r)) return fail(SVDQ_EINVAL, "out overlaps an input or the workspace");
  if (overlaps(Range{x, size_t(M) * size_t(up->K) * 2}, Range{workspace, need}))
    return fail(SVDQ_EINVAL, "workspace overlaps x");
  if (ws_bytes < need) return fail(SVDQ_EWORKSPACE, "workspace too small");
  return SVDQ_OK;
}

// QKV fusion: heads of 128 columns (the epilogue's column order needs two
// heads' v columns per head: 2 * (192 - 128) == 128)
constexpr int kQkvHeadDim = 128;
constexpr int kQkvMaxHeads = 256;

int validate_qkv(const void* x, int64_t M, const svdq_w4a4_layer* qkv, int heads, int head_dim,
                 const void* q_norm, const void* k_norm, float eps, const float* rope_cos,
                 const float* rope_sin, const void* out, const void* workspace, size_t ws_bytes) {
  int rc = validate_layer(M, qkv, "qkv");
  if (rc) return rc;
  if (head_dim != kQkvHeadDim) return fail(SVDQ_EUNSUPPORTED, "head_dim must be 128");
  if (heads < 1 || heads > kQkvMaxHeads) return fail(SVDQ_EINVAL, "heads must be in [1, 256]");
  if (qkv->N != int64_t(3) * heads * head_dim) return fail(SVDQ_EINVAL, "qkv->N must equal 3 * heads * head_dim");
  if (!(std::isfinite(eps) && eps > 0.f)) return fail(SVDQ_EINVAL, "eps must be finite and positive");
  if (!x || !out || !workspace || !q_norm || !k_norm || !rope_cos || !rope_sin)
    return fail(SVDQ_EINVAL, "null pointer argument");
  const void* ptrs[] = {x, out, workspace, q_norm, k_norm, rope_cos, rope_sin};
  for (const void* p : ptrs)
    if (!aligned(p)) return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  const int64_t K = qkv->K, N = qkv->N;
  const size_t need = workspace_bytes(M, K, qkv->precision, qkv->rank);
  const size_t table = size_t(M) * size_t(head_dim / 2) * 4;
  const Range o{out, size_t(M) * size_t(N) * 2};
  const Range ins[] = {{x, size_t(M) * size_t(K) * 2},
                       {workspace, need},
                       {qkv->packed_w, size_t(N) * size_t(K / 2)},
                       {qkv->wscales, w_scale_bytes(N, K, qkv->precision)},
                       {qkv->smooth, size_t(K) * 2},
                       {qkv->lora_down, size_t(qkv->rank) * size_t(K) * 2},
                       {qkv->lora_up, size_t(N) * size_t(qkv->rank) * 2},
                       {qkv->bias, size_t(N) * 2},
                       {q_norm, size_t(head_dim) * 2},
                       {k_norm, size_t(head_dim) * 2},
                       {rope_cos, table},
                       {rope_sin, table}};
  for (const Range& r : ins)
    if (overlaps(o, r)) return fail(SVDQ_EINVAL, "out overlaps an input or the workspace");
  if (overlaps(Range{x, size_t(M) * size_t(K) * 2}, Range{workspace, need}))
    return fail(SVDQ_EINVAL, "workspace overlaps x");
  if (ws_bytes < need) return fail(SVDQ_EWORKSPACE, "workspace too small");
  return SVDQ_OK;
}

}  // namespace

extern "C" {

const char* svdq_last_error(void) { return g_last_error.c_str(); }

size_t svdq_w4a4_workspace_bytes(int64_t M, int64_t K, int64_t N, int precision, int group_size,
                                 int rank) {
  const std::string saved = g_last_error;
  const bool ok = check_svdq_kind(precision, group_size, rank) == SVDQ_OK && check_shape(M, K, N) == SVDQ_OK &&
                  check_gemm_tiles(M, N) == SVDQ_OK;
  g_last_error = saved;
  return ok ? linear_workspace_bytes(M, K, N, precision, rank) : 0;
}

int svdq_w4a4_check(const void* x, int64_t M, int64_t K, int64_t N, const void* packed_w,
                    const void* wscales, float wtscale, const void* smooth, const void* lora_down,
                    const void* lora_up, const void* bias, int precision, int group_size, int rank,
                    const void* out, const void* workspace, size_t ws_bytes, const char* arch) {
  g_last_error.clear();
  int rc = validate_svdq(x, M, K, N, packed_w, wscales, wtscale, smooth, lora_down, lora_up, bias,
                         precision, group_size, rank, out, workspace, ws_bytes);
  if (rc) return rc;
  if (!arch_is_gfx950(arch)) return fail(SVDQ_EARCH, "device architecture is not gfx950");
  return SVDQ_OK;
}

int awq_w4a16_check(const void* x, int64_t M, int64_t K, int64_t N, const void* packed_w,
                    const void* wscales, const void* wzeros, const void* bias, int group_size,
                    const void* out, const char* arch) {
  g_last_error.clear();
  int rc = validate_awq(x, M, K, N, packed_w, wscales, wzeros, bias, group_size, out);
  if (rc) return rc;
  if (!arch_is_gfx950(arch)) return fail(SVDQ_EARCH, "device architecture is not gfx950");
  return SVDQ_OK;
}

int svdq_w4a4_quantize(const void* x, int64_t M, int64_t K, const void* smooth, const void* lora_down,
                       int precision, int group_size, int rank, void* workspace, size_t ws_bytes,
                       void* stream) {
  g_last_error.clear();
  int rc = check_svdq_kind(precision, group_size, rank);
  if (rc) return rc;
  rc = check_shape(M, K, 64);
  if (rc) return rc;
  if (!x || !smooth || !workspace) return fail(SVDQ_EINVAL, "null pointer argument");
  if ((rank > 0) != (lora_down != nullptr))
    return fail(SVDQ_EINVAL, "lora_down must be non-null exactly when rank > 0");
  const void* ptrs[] = {x, smooth, lora_down, workspace};
  for (const void* p : ptrs)
    if (p && !aligned(p)) return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  const size_t need = workspace_bytes(M, K, precision, rank);
  if (overlaps(Range{x, size_t(M) * size_t(K) * 2}, Range{workspace, need}))
    return fail(SVDQ_EINVAL, "workspace overlaps x");
  if (ws_bytes < need) return fail(SVDQ_EWORKSPACE, "workspace too small");
  rc = check_device_arch();
  if (rc) return rc;
  return launch_quantize(x, M, K, smooth, lora_down, precision, rank, workspace,
                         static_cast<hipStream_t>(stream));
}

int svdq_w4a4_gemm(const void* workspace, size_t ws_bytes, int64_t M, int64_t K, int64_t N,
                   const void* packed_w, const void* wscales, float wtscale, const void* lora_up,
                   const void* bias, int precision, int group_size, int rank, void* out, void* stream) {
  g_last_error.clear();
  int rc = check_svdq_kind(precision, group_size, rank);
  if (rc) return rc;
  rc = check_shape(M, K, N);
  if (rc) return rc;
  rc = check_gemm_tiles(M, N);
  if (rc) return rc;
  if (!workspace || !packed_w || !wscales || !out) return fail(SVDQ_EINVAL, "null pointer argument");
  if ((rank > 0) != (lora_up != nullptr))
    return fail(SVDQ_EINVAL, "lora_up must be non-null exactly when rank > 0");
  const void* ptrs[] = {workspace, packed_w, wscales, lora_up, bias, out};
  for (const void* p : ptrs)
    if (p && !aligned(p)) return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  if (precision == SVDQ_INT4 && wtscale != 1.0f) return fail(SVDQ_EINVAL, "wtscale must be 1.0 for int4");
  if (precision == SVDQ_NVFP4 && !(std::isfinite(wtscale) && wtscale > 0.f))
    return fail(SVDQ_EINVAL, "wtscale must be finite and positive");
  const size_t need = linear_workspace_bytes(M, K, N, precision, rank);
  const Range o{out, size_t(M) * size_t(N) * 2};
  const Range ins[] = {{workspace, need},
                       {packed_w, size_t(N) * size_t(K / 2)},
                       {wscales, w_scale_bytes(N, K, precision)},
                       {lora_up, size_t(N) * size_t(rank) * 2},
                       {bias, size_t(N) * 2}};
  for (const Range& r : ins)
    if (overlaps(o, r)) return fail(SVDQ_EINVAL, "out overlaps an input or the workspace");
  if (ws_bytes < need) return fail(SVDQ_EWORKSPACE, "workspace too small");
  rc = check_device_arch();
  if (rc) return rc;
  return launch_gemm(workspace, M, K, N, packed_w, wscales, wtscale, lora_up, bias, precision, rank, out,
                     static_cast<hipStream_t>(stream));
}

int svdq_w4a4_linear(const void* x, int64_t M, int64_t K, int64_t N, const void* packed_w,
                     const void* wscales, float wtscale, const void* smooth, const void* lora_down,
                     const void* lora_up, const void* bias, int precision, int group_size, int rank,
                     void* out, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  int rc = validate_svdq(x, M, K, N, packed_w, wscales, wtscale, smooth, lora_down, lora_up, bias,
                         precision, group_size, rank, out, workspace, ws_bytes);
  if (rc) return rc;
  rc = check_device_arch();
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = launch_quantize(x, M, K, smooth, lora_down, precision, rank, workspace, s);
  if (rc) return rc;
  return launch_gemm(workspace, M, K, N, packed_w, wscales, wtscale, lora_up, bias, precision, rank, out, s);
}

int awq_w4a16_linear(const void* x, int64_t M, int64_t K, int64_t N, const void* packed_w,
                     const void* wscales, const void* wzeros, const void* bias, int group_size,
                     void* out, void* stream) {
  g_last_error.clear();
  int rc = validate_awq(x, M, K, N, packed_w, wscales, wzeros, bias, group_size, out);
  if (rc) return rc;
  rc = check_device_arch();
  if (rc) return rc;
  svdq::AwqArgs a{x, packed_w, wscales, wzeros, bias, out, M, K, N};
  return launch_status(svdq::launch_awq_gemv(a, static_cast<hipStream_t>(stream)), "awq_w4a16 launch");
}

int svdq_w4a4_quantize_act(const void* x, int64_t M, int64_t K, const void* smooth,
                           const void* lora_down, int precision, int group_size, int rank,
                           void* codes_out, void* scales_out, float* lora_act_out, void* stream) {
  g_last_error.clear();
  int rc = check_svdq_kind(precision, group_size, rank);
  if (rc) return rc;
  rc = check_shape(M, K, 64);
  if (rc) return rc;
  if (!x || !smooth || !codes_out || !scales_out) return fail(SVDQ_EINVAL, "null pointer argument");
  if ((rank > 0) != (lora_down != nullptr) || (rank > 0) != (lora_act_out != nullptr))
    return fail(SVDQ_EINVAL, "lora_down / lora_act_out must be non-null exactly when rank > 0");
  const void* ptrs[] = {x, smooth, lora_down, codes_out, scales_out, lora_act_out};
  for (const void* p : ptrs)
    if (p && !aligned(p)) return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  rc = check_device_arch();
  if (rc) return rc;
  svdq::QuantActArgs qa{x, smooth, lora_down, codes_out, scales_out, lora_act_out, nullptr, nullptr, M, K,
                        precision, rank};
  return launch_status(svdq::launch_quantize_act(qa, static_cast<hipStream_t>(stream)),
                       "quantize_act_lora_down launch");
}

int svdq_w4a4_gemm_partials(const void* act_codes, const void* w_codes, int64_t M, int64_t K,
                            int64_t N, int precision, int group_size, int32_t* partials_out,
                            void* stream) {
  g_last_error.clear();
  int rc = check_svdq_kind(precision, group_size, 0);
  if (rc) return rc;
  rc = check_shape(M, K, N);
  if (rc) return rc;
  rc = check_gemm_tiles(M, N);
  if (rc) return rc;
  if (!act_codes || !w_codes || !partials_out) return fail(SVDQ_EINVAL, "null pointer argument");
  const void* ptrs[] = {act_codes, w_codes, partials_out};
  for (const void* p : ptrs)
    if (!aligned(p)) return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  rc = check_device_arch();
  if (rc) return rc;
  svdq::GemmArgs ga{act_codes, nullptr, nullptr, w_codes, nullptr, nullptr, nullptr, nullptr,
                    partials_out, 1.0f, M, K, N, precision, 0};
  return launch_status(svdq::launch_gemm_w4a4(ga, static_cast<hipStream_t>(stream)),
                       "gemm_w4a4 partials launch");
}

size_t svdq_w4a4_mlp_workspace_bytes(int64_t M, const svdq_w4a4_layer* up, const svdq_w4a4_layer* down) {
  const std::string saved = g_last_error;
  const bool ok = validate_layer(M, up, "up") == SVDQ_OK && validate_layer(M, down, "down") == SVDQ_OK &&
                  up->N == down->K && down->precision == SVDQ_NVFP4;
  g_last_error = saved;
  return ok ? mlp_workspace_bytes(M, up, down) : 0;
}

int svdq_w4a4_mlp_gelu_check(const void* x, int64_t M, const svdq_w4a4_layer* up, const svdq_w4a4_layer* down,
                             const void* out, const void* workspace, size_t ws_bytes, const char* arch) {
  g_last_error.clear();
  int rc = validate_mlp(x, M, up, down, out, workspace, ws_bytes);
  if (rc) return rc;
  if (!arch_is_gfx950(arch)) return fail(SVDQ_EARCH, "device architecture is not gfx950");
  return SVDQ_OK;
}

int svdq_w4a4_mlp_gelu(const void* x, int64_t M, const svdq_w4a4_layer* up, const svdq_w4a4_layer* down,
                       void* out, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  int rc = validate_mlp(x, M, up, down, out, workspace, ws_bytes);
  if (rc) return rc;
  rc = check_device_arch();
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t H = up->N;
  const Carve cu = carve(workspace, M, up->K, up->precision);
  void* ws_down = static_cast<uint8_t*>(workspace) + workspace_bytes(M, up->K, up->precision, up->rank);
  const Carve cd = carve(ws_down, M, H, SVDQ_NVFP4);
  // up layer: kernel 1 into the first part of the workspace; the same launch
  // clears the down layer's low-rank accumulator
  rc = launch_quantize(x, M, up->K, up->smooth, up->lora_down, up->precision, up->rank, workspace, s,
                       cd.lora_act, M * down->rank);
  if (rc) return rc;
  // up layer: kernel 2 with the GELU + nvfp4 epilogue writing the down
  // layer's workspace (its bf16 output is not stored)
  svdq::GemmArgs ga{cu.act_f16, cu.row_scale, cu.lora_act, up->packed_w, up->wscales, up->lora_up, up->bias,
                    nullptr, nullptr, up->wtscale, M, up->K, H, up->precision, up->rank,
                    down->smooth, down->lora_down, cd.act_f16, cd.lora_act, down->rank};
  rc = launch_status(svdq::launch_gemm_w4a4(ga, s), "gemm_w4a4_lora_up (GELU epilogue) launch");
  if (rc) return rc;
  // down layer: kernel 2 from its workspace
  return launch_gemm(ws_down, M, H, down->N, down->packed_w, down->wscales, down->wtscale, down->lora_up,
                     down->bias, SVDQ_NVFP4, down->rank, out, s);
}

int svdq_w4a4_qkv_rmsnorm_rope_check(const void* x, int64_t M, const svdq_w4a4_layer* qkv, int heads,
                                     int head_dim, const void* q_norm, const void* k_norm, float eps,
                                     const float* rope_cos, const float* rope_sin, const void* out,
                                     const void* workspace, size_t ws_bytes, const char* arch) {
  g_last_error.clear();
  int rc = validate_qkv(x, M, qkv, heads, head_dim, q_norm, k_norm, eps, rope_cos, rope_sin, out, workspace,
                        ws_bytes);
  if (rc) return rc;
  if (!arch_is_gfx950(arch)) return fail(SVDQ_EARCH, "device architecture is not gfx950");
  return SVDQ_OK;
}

int svdq_w4a4_qkv_rmsnorm_rope(const void* x, int64_t M, const svdq_w4a4_layer* qkv, int heads, int head_dim,
                               const void* q_norm, const void* k_norm, float eps, const float* rope_cos,
                               const float* rope_sin, void* out, void* workspace, size_t ws_bytes,
                               void* stream) {
  g_last_error.clear();
  int rc = validate_qkv(x, M, qkv, heads, head_dim, q_norm, k_norm, eps, rope_cos, rope_sin, out, workspace,
                        ws_bytes);
  if (rc) return rc;
  rc = check_device_arch();
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = launch_quantize(x, M, qkv->K, qkv->smooth, qkv->lora_down, qkv->precision, qkv->rank, workspace, s);
  if (rc) return rc;
  const Carve c = carve(workspace, M, qkv->K, qkv->precision);
  svdq::GemmArgs ga{c.act_f16, c.row_scale, c.lora_act, qkv->packed_w, qkv->wscales, qkv->lora_up, qkv->bias,
                    out, nullptr, qkv->wtscale, M, qkv->K, qkv->N, qkv->precision, qkv->rank};
  ga.q_norm = q_norm;
  ga.k_norm = k_norm;
  ga.rope_cos = rope_cos;
  ga.rope_sin = rope_sin;
  ga.eps = eps;
  ga.heads = heads;
  return launch_status(svdq::launch_gemm_w4a4(ga, s), "gemm_w4a4_lora_up (RMSNorm + RoPE epilogue) launch");
}

// ---- offline weight preparation ------------------------------------------------
size_t svdq_w4a4_prep_workspace_bytes(int64_t K) {
  if (K < 1 || K > kMaxK) return 0;
  return round_up(size_t(K) * 8);
}

int svdq_w4a4_smooth_factors(const void* x_calib, int64_t M, const float* w, int64_t N, int64_t K,
                             void* smooth_out, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (M < 1 || M > kMaxPrepRows || N < 1 || N > kMaxPrepRows)
    return fail(SVDQ_EINVAL, "M and N must be in [1, 2^22]");
  if (K < 128 || K > kMaxK || K % 128) return fail(SVDQ_EINVAL, "K must be a multiple of 128 in [128, 16384]");
  if (!x_calib || !w || !smooth_out || !workspace) return fail(SVDQ_EINVAL, "null pointer argument");
  const void* ptrs[] = {x_calib, w, smooth_out, workspace};
  for (const void* p : ptrs)
    if (!aligned(p)) return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  const size_t need = svdq_w4a4_prep_workspace_bytes(K);
  const Range o{smooth_out, size_t(K) * 2};
  const Range ins[] = {{x_calib, size_t(M) * size_t(K) * 2}, {w, size_t(N) * size_t(K) * 4}, {workspace, need}};
  for (const Range& r : ins)
    if (overlaps(o, r)) return fail(SVDQ_EINVAL, "smooth_out overlaps an input or the workspace");
  if (ws_bytes < need) return fail(SVDQ_EWORKSPACE, "workspace too small");
  int rc = check_device_arch();
  if (rc) return rc;
  svdq::SmoothArgs a{x_calib, w, smooth_out, static_cast<uint32_t*>(workspace), M, N, K};
  return launch_status(svdq::launch_smooth_factors(a, static_cast<hipStream_t>(stream)), "smooth factors launch");
}

int svdq_w4a4_pack_weight(const float* resid, int64_t N, int64_t K, int precision, int group_size,
                          void* packed_w_out, void* wscales_out, float* wtscale_out, void* workspace,
                          size_t ws_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_svdq_kind(precision, group_size, 0);
  if (rc) return rc;
  if (N < 1 || N > (int64_t(1) << 24)) return fail(SVDQ_EINVAL, "N must be in [1, 2^24]");
  if (K < 128 || K > kMaxK || K % 128) return fail(SVDQ_EINVAL, "K must be a multiple of 128 in [128, 16384]");
  if (!resid || !packed_w_out || !wscales_out || !workspace) return fail(SVDQ_EINVAL, "null pointer argument");
  if (precision == SVDQ_NVFP4 && !wtscale_out) return fail(SVDQ_EINVAL, "nvfp4 needs wtscale_out");
  const void* ptrs[] = {resid, packed_w_out, wscales_out, workspace};
  for (const void* p : ptrs)
    if (!aligned(p)) return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(wtscale_out) % 4) return fail(SVDQ_EINVAL, "wtscale_out must be 4-byte aligned");
  const size_t need = svdq_w4a4_prep_workspace_bytes(K);
  const Range outs[] = {{packed_w_out, size_t(N) * size_t(K / 2)},
                        {wscales_out, w_scale_bytes(N, K, precision)},
                        {wtscale_out, 4}};
  const Range ins[] = {{resid, size_t(N) * size_t(K) * 4}, {workspace, need}};
  for (const Range& o : outs)
    for (const Range& r : ins)
      if (overlaps(o, r)) return fail(SVDQ_EINVAL, "an output overlaps the residual or the workspace");
  if (overlaps(outs[0], outs[1]) || overlaps(outs[0], outs[2]) || overlaps(outs[1], outs[2]))
    return fail(SVDQ_EINVAL, "outputs overlap");
  if (ws_bytes < need) return fail(SVDQ_EWORKSPACE, "workspace too small");
  rc = check_device_arch();
  if (rc) return rc;
  svdq::PackArgs a{resid, packed_w_out, wscales_out, wtscale_out, static_cast<uint32_t*>(workspace), N, K,
                   precision};
  return launch_status(svdq::launch_pack_weight(a, static_cast<hipStream_t>(stream)), "pack weight launch");
}

int svdq_w4a4_gelu_table(void* out, void* stream) {
  g_last_error.clear();
  if (!out) return fail(SVDQ_EINVAL, "null pointer argument");
  if (!aligned(out)) return fail(SVDQ_EINVAL, "out must be 16-byte aligned");
  int rc = check_device_arch();
  if (rc) return rc;
  return launch_status(svdq::launch_gelu_table_copy(static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)),
                       "GELU table copy launch");
}

}  // extern "C"
