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

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"

// Scratch of svdq_w4a4_linear_noalloc: a static array in device memory, one
// copy on every GPU the library runs on, held until the process ends.  Host
// code never takes the array's name as an address (on the host it is only a
// stand-in): the per-device address comes from hipGetSymbolAddress, taken
// once per device with that device current (noalloc_scratch below).
constexpr size_t kNoallocScratchBytes = SVDQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

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

// Kernel 1 of the linear splits K over S workgroups per 16 rows (S = 1, 2,
// 4 or 8, dividing the K/64 chunks) while the row blocks alone would leave
// more than half of the 256 compute units idle; its low-rank sums are then
// S fp32 partials, added in order by a second kernel.
int k1_slices(int64_t M, int64_t K) {
  const int64_t blocks = (M + 15) / 16;
  const int64_t chunks = K / 64;
  int s = 1;
  while (s < 8 && blocks * s * 2 <= 256 && chunks % (s * 2) == 0) s *= 2;
  return s;
}

// Base workspace of one layer (each part 256-byte aligned):
//   act_op     the product operand [M, K]: int4 codes as fp8 E4M3 bytes,
//              nvfp4 the dequantized values as fp16
//   act_scale  int4 only: bf16 [M, K/64], the group scales
//   lora_act   f32 [M, rank]
//   lora_part  f32 [S, M, rank] when kernel 1 splits K (S = k1_slices > 1)
size_t workspace_bytes(int64_t M, int64_t K, int precision, int rank) {
  size_t b = round_up(size_t(M) * size_t(K) * (precision == SVDQ_INT4 ? 1 : 2));
  if (precision == SVDQ_INT4) b += round_up(size_t(M) * size_t(K / 64) * 2);
  b += round_up(size_t(M) * size_t(rank) * 4);
  const int S = k1_slices(M, K);
  if (S > 1) b += round_up(size_t(S) * size_t(M) * size_t(rank) * 4);
  return b;
}

// Split K for the plain linear: when the 256 x 192 tiles would occupy at
// most half of the 256 compute units, each tile's stages (128 values of K for
// int4, 64 for nvfp4) are shared by up to 8 workgroups that write fp32
// partials, summed in a fixed order by a second kernel.  A split takes about
// five stages or more (at least 2 splits where there are 4 stages): fewer
// stages per workgroup leave its fixed cost and the partials' traffic
// unamortized (measured at M = 128..512, K = 1152..6144, N = 3072).
int choose_ksplit(int64_t M, int64_t N, int64_t K, int precision) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 191) / 192);
  const int nst = int(K / (precision == SVDQ_INT4 ? 128 : 64));
  if (tiles > 128) return 1;
  int s = int(std::min<int64_t>(8, 256 / tiles));
  s = std::min(s, nst / 2);
  s = std::min(s, std::max(2, nst / 5));
  s = std::max(s, 1);
  while (s > 1 && ((nst + s - 1) / s) * (s - 1) >= nst) --s;  // every split gets stages
  return s;
}

size_t split_bytes(int64_t M, int64_t K, int64_t N, int precision) {
  const int s = choose_ksplit(M, N, K, precision);
  return s > 1 ? round_up(size_t(s) * size_t(M) * size_t(N) * 4) : 0;
}

// Workspace of svdq_w4a4_linear / svdq_w4a4_gemm: workspace_bytes, then the
// split-K partials fp32 [ksplit, M, N] when K is split.
size_t linear_workspace_bytes(int64_t M, int64_t K, int64_t N, int precision, int rank) {
  return workspace_bytes(M, K, precision, rank) + split_bytes(M, K, N, precision);
}

// with_workspace false: the caller's workspace is not checked (the
// allocation-free entry brings its own)
int validate_svdq(const void* x, int64_t M, int64_t K, int64_t N, const void* packed_w,
                  const void* wscales, float wtscale, const void* smooth, const void* lora_down,
                  const void* lora_up, const void* bias, int precision, int group_size, int rank,
                  const void* out, const void* workspace, size_t workspace_bytes_given,
                  bool with_workspace = true) {
  int rc = check_svdq_kind(precision, group_size, rank);
  if (rc) return rc;
  rc = check_shape(M, K, N);
  if (rc) return rc;
  rc = check_gemm_tiles(M, N);
  if (rc) return rc;
  if (!x || !packed_w || !wscales || !smooth || !out || (with_workspace && !workspace))
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
  if (!with_workspace) return SVDQ_OK;
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
  uint8_t* act_op;    // int4: E4M3 bytes [M, K]; nvfp4: f16 [M, K]
  uint16_t* act_scale;  // int4: bf16 [M, K/64]; else null
  float* lora_act;    // f32 [M, rank]
  float* lora_part;   // f32 [k1_slices, M, rank] (when kernel 1 splits K)
};

Carve carve(void* workspace, int64_t M, int64_t K, int precision, int rank) {
  uint8_t* p = static_cast<uint8_t*>(workspace);
  Carve c{};
  c.act_op = p;
  p += round_up(size_t(M) * size_t(K) * (precision == SVDQ_INT4 ? 1 : 2));
  if (precision == SVDQ_INT4) {
    c.act_scale = reinterpret_cast<uint16_t*>(p);
    p += round_up(size_t(M) * size_t(K / 64) * 2);
  }
  c.lora_act = reinterpret_cast<float*>(p);
  c.lora_part = c.lora_act + round_up(size_t(M) * size_t(rank) * 4) / 4;
  return c;
}

// Kernel 1 into the workspace.
int launch_quantize(const void* x, int64_t M, int64_t K, const void* smooth, const void* lora_down,
                    int precision, int rank, void* workspace, hipStream_t s) {
  const Carve c = carve(workspace, M, K, precision, rank);
  svdq::QuantActArgs qa{x, smooth, lora_down, nullptr, nullptr, c.lora_act, c.act_op,
                        reinterpret_cast<float*>(c.act_scale), M, K, precision, rank};
  qa.scale_bf16 = true;
  qa.k_slices = k1_slices(M, K);
  qa.lora_part = c.lora_part;
  int rc = launch_status(svdq::launch_quantize_act(qa, s), "quantize_act_lora_down launch");
  if (rc || qa.k_slices == 1 || rank == 0) return rc;
  // the slices' low-rank partials, added in slice order
  return launch_status(svdq::launch_tile_partial_sum(c.lora_part, qa.k_slices, M * rank, c.lora_act, s),
                       "low-rank slice sum launch");
}

// Kernel 2 (plain store) from a linear workspace (linear_workspace_bytes).
int launch_gemm(const void* workspace, int64_t M, int64_t K, int64_t N, const void* packed_w,
                const void* wscales, float wtscale, const void* lora_up, const void* bias, int precision,
                int rank, void* out, hipStream_t s) {
  const Carve c = carve(const_cast<void*>(workspace), M, K, precision, rank);
  svdq::GemmArgs ga{c.act_op, c.act_scale, c.lora_act, packed_w, wscales, lora_up, bias, out, nullptr,
                    wtscale, M, K, N, precision, rank};
  ga.ksplit = choose_ksplit(M, N, K, precision);
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

// The fused MLP's workspace: the up layer's (no split partials), the down
// layer's linear workspace, then the down layer's low-rank partials of the up
// projection's column tiles, fp32 [ceil(H / 192), M, down rank].
size_t mlp_tiles(const svdq_w4a4_layer* up) { return size_t((up->N + 191) / 192); }

size_t mlp_workspace_bytes(int64_t M, const svdq_w4a4_layer* up, const svdq_w4a4_layer* down) {
  return workspace_bytes(M, up->K, up->precision, up->rank) +
         linear_workspace_bytes(M, down->K, down->N, SVDQ_NVFP4, down->rank) +
         round_up(mlp_tiles(up) * size_t(M) * size_t(down->rank) * 4);
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

// QKV fusion: heads of 32, 64 or 128 columns (a column tile holds 128 q | k
// columns, whole heads, and 64 v columns, so heads * head_dim must be a
// multiple of 64)
constexpr int kQkvMaxHeads = 256;

int validate_qkv(const void* x, int64_t M, const svdq_w4a4_layer* qkv, int heads, int head_dim,
                 const void* q_norm, const void* k_norm, float eps, const float* rope_cos,
                 const float* rope_sin, const void* out, const void* workspace, size_t ws_bytes) {
  int rc = validate_layer(M, qkv, "qkv");
  if (rc) return rc;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(SVDQ_EUNSUPPORTED, "head_dim must be 32, 64 or 128");
  if (heads < 1 || heads > kQkvMaxHeads) return fail(SVDQ_EINVAL, "heads must be in [1, 256]");
  if ((heads * head_dim) % 64 != 0)
    return fail(SVDQ_EUNSUPPORTED, "heads * head_dim must be a multiple of 64 (head_dim 32: an even head count)");
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


// ---- allocation-free linear ----------------------------------------------------
std::mutex g_scratch_mu;
void* g_scratch[64];

// This device's address of `scratch`, looked up on the first call on the
// device (with it current) and kept.
int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SVDQ_EDEVICE, std::string("hipGetDevice failed: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(SVDQ_EDEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SVDQ_EDEVICE, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SVDQ_OK;
}

// ---- offline preparation: the rank-r split -------------------------------------
// A randomized range finder with subspace iteration (Halko, Martinsson and
// Tropp, "Finding structure with randomness", 2011, Algorithms 4.3 / 4.4):
// the products with the weight run on the GPU (prep_svd.hip); the l x l
// factorizations (l = rank + oversampling) run here in fp64, after a copy of
// the l x l Gram matrix to the host.

constexpr int64_t kMaxPrepN = int64_t(1) << 20;
constexpr int kMaxOversample = 32;
constexpr int kMaxPowerIters = 16;

// row slices of an A^T B product with C columns (about 512 workgroups)
int prep_slices(int64_t R, int64_t C) {
  const int64_t chunks = (C + 63) / 64;
  int64_t s = std::max<int64_t>(1, 512 / chunks);
  s = std::min<int64_t>(s, 32);
  s = std::min<int64_t>(s, std::max<int64_t>(1, R / 32));
  return int(s);
}

// Workspace of svdq_w4a4_prepare_weight, each part 256-byte aligned.
struct PrepCarve {
  uint32_t* amax;   // u32 [2K]  column / tensor maxima
  double* omega;    // [K, l]    Gaussian test matrix
  double* y;        // [N, l]
  double* q;        // [N, l]
  double* tmp;      // [max(N, K), l]
  double* z;        // [K, l]
  double* zq;       // [K, l]
  double* part;     // [slices, C, l] partial sums of A^T B
  double* g;        // [l, l]
  double* small;    // [l, l]      small right factors uploaded from the host
  double* up64;     // [N, rank]
  double* dt64;     // [K, rank]
  float* resid;     // [N, K]
};

size_t prep_part_elems(int64_t N, int64_t K, int l) {
  const int64_t R = std::max(N, K);
  const int64_t a = int64_t(prep_slices(N, K)) * K, b = int64_t(prep_slices(K, N)) * N;
  const int64_t c = int64_t(prep_slices(R, l)) * l;
  return size_t(std::max(std::max(a, b), c)) * size_t(l);
}

size_t prep_carve(void* base, int64_t N, int64_t K, int rank, int l, PrepCarve* c) {
  uint8_t* p = static_cast<uint8_t*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? p + off : nullptr;
    off += round_up(bytes);
    return r;
  };
  const size_t d = sizeof(double);
  PrepCarve t{};
  t.amax = static_cast<uint32_t*>(take(size_t(K) * 8));
  if (rank > 0) {
    t.omega = static_cast<double*>(take(size_t(K) * l * d));
    t.y = static_cast<double*>(take(size_t(N) * l * d));
    t.q = static_cast<double*>(take(size_t(N) * l * d));
    t.tmp = static_cast<double*>(take(size_t(std::max(N, K)) * l * d));
    t.z = static_cast<double*>(take(size_t(K) * l * d));
    t.zq = static_cast<double*>(take(size_t(K) * l * d));
    t.part = static_cast<double*>(take(prep_part_elems(N, K, l) * d));
    t.g = static_cast<double*>(take(size_t(l) * l * d));
    t.small = static_cast<double*>(take(size_t(l) * l * d));
    t.up64 = static_cast<double*>(take(size_t(N) * rank * d));
    t.dt64 = static_cast<double*>(take(size_t(K) * rank * d));
  }
  t.resid = static_cast<float*>(take(size_t(N) * size_t(K) * 4));
  if (c) *c = t;
  return off;
}

// Upper Cholesky factor Rm (l x l, row-major) of G + shift I.  A pivot not
// above 1e-13 of its diagonal entry marks a column that depends on the
// earlier ones: it is dropped (keep = 0, its row of Rm zero).
void chol_upper(const std::vector<double>& G, int l, double shift, std::vector<double>& Rm,
                std::vector<char>& keep) {
  Rm.assign(size_t(l) * l, 0.0);
  keep.assign(l, 0);
  for (int i = 0; i < l; ++i) {
    const double gii = G[size_t(i) * l + i] + shift;
    double d = gii;
    for (int m = 0; m < i; ++m)
      if (keep[m]) d -= Rm[size_t(m) * l + i] * Rm[size_t(m) * l + i];
    if (!(gii > 0.0) || !(d > 1e-13 * gii)) continue;
    keep[i] = 1;
    const double rii = std::sqrt(d);
    Rm[size_t(i) * l + i] = rii;
    for (int j = i + 1; j < l; ++j) {
      double v = G[size_t(i) * l + j];
      for (int m = 0; m < i; ++m)
        if (keep[m]) v -= Rm[size_t(m) * l + i] * Rm[size_t(m) * l + j];
      Rm[size_t(i) * l + j] = v / rii;
    }
  }
}

// T = Rm^-1 on the kept rows and columns (upper triangular), zero elsewhere
void inv_upper(const std::vector<double>& Rm, const std::vector<char>& keep, int l, std::vector<double>& T) {
  T.assign(size_t(l) * l, 0.0);
  for (int j = 0; j < l; ++j) {
    if (!keep[j]) continue;
    T[size_t(j) * l + j] = 1.0 / Rm[size_t(j) * l + j];
    for (int i = j - 1; i >= 0; --i) {
      if (!keep[i]) continue;
      double v = 0.0;
      for (int m = i + 1; m <= j; ++m)
        if (keep[m]) v += Rm[size_t(i) * l + m] * T[size_t(m) * l + j];
      T[size_t(i) * l + j] = -v / Rm[size_t(i) * l + i];
    }
  }
}

struct PrepCtx {
  hipStream_t s;
  int l;
  PrepCarve c;
};

int prep_status(hipError_t e, const char* what) {
  return e == hipSuccess ? SVDQ_OK : fail(SVDQ_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

// Device X [R, l] -> Qo [R, l] with orthonormal columns (dependent columns
// zero) and, if Rf is given, the upper triangular Rf [l, l] with X = Qo Rf:
// shifted CholeskyQR followed by two CholeskyQR passes (Fukaya, Kannan,
// Nakatsukasa, Yamamoto and Yanagisawa, "Shifted Cholesky QR for computing
// the QR factorization of ill-conditioned matrices", 2020).  X may not be Qo
// or the context's tmp buffer.
int prep_orth(PrepCtx& x, const double* X, int64_t R, double* Qo, std::vector<double>* Rf) {
  const int l = x.l;
  std::vector<double> G(size_t(l) * l), Rm, T, acc;
  std::vector<char> keep;
  if (Rf) {
    acc.assign(size_t(l) * l, 0.0);
    for (int i = 0; i < l; ++i) acc[size_t(i) * l + i] = 1.0;
  }
  const double* cur = X;
  double* const dst[3] = {Qo, x.c.tmp, Qo};
  svdq::PrepSrc src;
  for (int pass = 0; pass < 3; ++pass) {
    src.dense = cur;
    int rc = prep_status(svdq::launch_prep_atb(src, R, l, cur, l, prep_slices(R, l), x.c.part, x.c.g, x.s),
                         "Gram matrix launch");
    if (rc) return rc;
    rc = prep_status(hipMemcpyAsync(G.data(), x.c.g, G.size() * sizeof(double), hipMemcpyDeviceToHost, x.s),
                     "Gram matrix copy");
    if (rc) return rc;
    rc = prep_status(hipStreamSynchronize(x.s), "stream synchronize");
    if (rc) return rc;
    double shift = 0.0;
    if (pass == 0) {
      double tr = 0.0;
      for (int i = 0; i < l; ++i) tr += G[size_t(i) * l + i];
      shift = 11.0 * (double(R) * l + double(l) * (l + 1)) * 0x1p-53 * tr;
    }
    chol_upper(G, l, shift, Rm, keep);
    inv_upper(Rm, keep, l, T);
    rc = prep_status(hipMemcpyAsync(x.c.small, T.data(), T.size() * sizeof(double), hipMemcpyHostToDevice, x.s),
                     "factor copy");
    if (rc) return rc;
    rc = prep_status(svdq::launch_prep_ab(src, R, l, x.c.small, l, dst[pass], x.s), "CholeskyQR product launch");
    if (rc) return rc;
    // the host T must outlive its copy
    rc = prep_status(hipStreamSynchronize(x.s), "stream synchronize");
    if (rc) return rc;
    if (Rf) {  // acc = Rm acc
      std::vector<double> nxt(size_t(l) * l, 0.0);
      for (int i = 0; i < l; ++i)
        for (int m = i; m < l; ++m) {
          const double r = Rm[size_t(i) * l + m];
          if (r == 0.0) continue;
          for (int j = 0; j < l; ++j) nxt[size_t(i) * l + j] += r * acc[size_t(m) * l + j];
        }
      acc.swap(nxt);
    }
    cur = dst[pass];
  }
  if (Rf) Rf->swap(acc);
  return SVDQ_OK;
}

// One-sided Jacobi SVD (Hestenes) of the l x l row-major A: A = U diag(sig)
// V^T, singular values in descending order.  Columns of A are rotated in
// pairs until every pair is orthogonal to 1e-15 of the product of their norms.
void jacobi_svd(std::vector<double> A, int l, std::vector<double>& U, std::vector<double>& sig,
                std::vector<double>& V) {
  V.assign(size_t(l) * l, 0.0);
  for (int i = 0; i < l; ++i) V[size_t(i) * l + i] = 1.0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    bool rotated = false;
    for (int p = 0; p < l - 1; ++p)
      for (int q = p + 1; q < l; ++q) {
        double a = 0.0, b = 0.0, g = 0.0;
        for (int i = 0; i < l; ++i) {
          const double xp = A[size_t(i) * l + p], xq = A[size_t(i) * l + q];
          a += xp * xp;
          b += xq * xq;
          g += xp * xq;
        }
        if (g == 0.0 || std::fabs(g) <= 1e-15 * std::sqrt(a * b)) continue;
        rotated = true;
        const double zeta = (b - a) / (2.0 * g);
        const double t = std::copysign(1.0, zeta) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        const double cs = 1.0 / std::sqrt(1.0 + t * t), sn = cs * t;
        for (int i = 0; i < l; ++i) {
          double& xp = A[size_t(i) * l + p];
          double& xq = A[size_t(i) * l + q];
          const double np = cs * xp - sn * xq, nq = sn * xp + cs * xq;
          xp = np;
          xq = nq;
          double& vp = V[size_t(i) * l + p];
          double& vq = V[size_t(i) * l + q];
          const double mp = cs * vp - sn * vq, mq = sn * vp + cs * vq;
          vp = mp;
          vq = mq;
        }
      }
    if (!rotated) break;
  }
  std::vector<double> s(l);
  for (int j = 0; j < l; ++j) {
    double n2 = 0.0;
    for (int i = 0; i < l; ++i) n2 += A[size_t(i) * l + j] * A[size_t(i) * l + j];
    s[j] = std::sqrt(n2);
  }
  std::vector<int> order(l);
  for (int j = 0; j < l; ++j) order[j] = j;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return s[a] > s[b]; });
  U.assign(size_t(l) * l, 0.0);
  sig.assign(l, 0.0);
  std::vector<double> Vs(size_t(l) * l);
  for (int jj = 0; jj < l; ++jj) {
    const int j = order[jj];
    sig[jj] = s[j];
    for (int i = 0; i < l; ++i) {
      U[size_t(i) * l + jj] = s[j] > 0.0 ? A[size_t(i) * l + j] / s[j] : 0.0;
      Vs[size_t(i) * l + jj] = V[size_t(i) * l + j];
    }
  }
  V.swap(Vs);
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

int svdq_w4a4_linear_noalloc(const void* x, int64_t M, int64_t K, int64_t N, const void* packed_w,
                             const void* wscales, float wtscale, const void* smooth, const void* lora_down,
                             const void* lora_up, const void* bias, int precision, int group_size, int rank,
                             void* out, void* stream) {
  g_last_error.clear();
  int rc = validate_svdq(x, M, K, N, packed_w, wscales, wtscale, smooth, lora_down, lora_up, bias, precision,
                         group_size, rank, out, nullptr, 0, false);
  if (rc) return rc;
  const size_t need = linear_workspace_bytes(M, K, N, precision, rank);
  if (need > kNoallocScratchBytes)
    return fail(SVDQ_EWORKSPACE, "svdq_w4a4_linear_noalloc: this call needs " + std::to_string(need) +
                                     " bytes of scratch, more than the " + std::to_string(kNoallocScratchBytes) +
                                     " of the static scratch (use svdq_w4a4_linear with a workspace)");
  rc = check_device_arch();
  if (rc) return rc;
  void* ws = nullptr;
  rc = noalloc_scratch(&ws);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = launch_quantize(x, M, K, smooth, lora_down, precision, rank, ws, s);
  if (rc) return rc;
  return launch_gemm(ws, M, K, N, packed_w, wscales, wtscale, lora_up, bias, precision, rank, out, s);
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

int svdq_w4a4_quantize_operand(const void* x, int64_t M, int64_t K, const void* smooth,
                               const void* lora_down, int precision, int group_size, int rank,
                               void* operand_out, float* scale_out, float* lora_act_out,
                               void* stream) {
  g_last_error.clear();
  int rc = check_svdq_kind(precision, group_size, rank);
  if (rc) return rc;
  rc = check_shape(M, K, 64);
  if (rc) return rc;
  if (!x || !smooth || !operand_out) return fail(SVDQ_EINVAL, "null pointer argument");
  if ((precision == SVDQ_INT4) != (scale_out != nullptr))
    return fail(SVDQ_EINVAL, "scale_out must be non-null exactly for int4");
  if ((rank > 0) != (lora_down != nullptr) || (rank > 0) != (lora_act_out != nullptr))
    return fail(SVDQ_EINVAL, "lora_down / lora_act_out must be non-null exactly when rank > 0");
  const void* ptrs[] = {x, smooth, lora_down, operand_out, scale_out, lora_act_out};
  for (const void* p : ptrs)
    if (p && !aligned(p)) return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  const Range outs[] = {{operand_out, size_t(M) * size_t(K) * (precision == SVDQ_INT4 ? 1 : 2)},
                        {scale_out, size_t(M) * size_t(K / 64) * 4},
                        {lora_act_out, size_t(M) * size_t(rank) * 4}};
  const Range xr{x, size_t(M) * size_t(K) * 2};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], xr)) return fail(SVDQ_EINVAL, "an output overlaps x");
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outs[j])) return fail(SVDQ_EINVAL, "outputs overlap");
  }
  rc = check_device_arch();
  if (rc) return rc;
  svdq::QuantActArgs qa{x, smooth, lora_down, nullptr, nullptr, lora_act_out, operand_out, scale_out, M, K,
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
  const Carve cu = carve(workspace, M, up->K, up->precision, up->rank);
  void* ws_down = static_cast<uint8_t*>(workspace) + workspace_bytes(M, up->K, up->precision, up->rank);
  const Carve cd = carve(ws_down, M, H, SVDQ_NVFP4, down->rank);
  float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws_down) +
                                        linear_workspace_bytes(M, H, down->N, SVDQ_NVFP4, down->rank));
  // up layer: kernel 1 into the first part of the workspace
  rc = launch_quantize(x, M, up->K, up->smooth, up->lora_down, up->precision, up->rank, workspace, s);
  if (rc) return rc;
  // up layer: kernel 2 with the GELU + nvfp4 epilogue writing the down
  // layer's operand and its column tiles' low-rank partials (the up layer's
  // bf16 output is not stored)
  svdq::GemmArgs ga{cu.act_op, cu.act_scale, cu.lora_act, up->packed_w, up->wscales, up->lora_up, up->bias,
                    nullptr, nullptr, up->wtscale, M, up->K, H, up->precision, up->rank,
                    down->smooth, down->lora_down, cd.act_op, part, down->rank};
  rc = launch_status(svdq::launch_gemm_w4a4(ga, s), "gemm_w4a4_lora_up (GELU epilogue) launch");
  if (rc) return rc;
  // the down layer's low-rank activations: the tiles' partials added in order
  if (down->rank > 0) {
    rc = launch_status(svdq::launch_tile_partial_sum(part, int(mlp_tiles(up)), M * down->rank, cd.lora_act, s),
                       "low-rank partial sum launch");
    if (rc) return rc;
  }
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
  const Carve c = carve(workspace, M, qkv->K, qkv->precision, qkv->rank);
  svdq::GemmArgs ga{c.act_op, c.act_scale, c.lora_act, qkv->packed_w, qkv->wscales, qkv->lora_up, qkv->bias,
                    out, nullptr, qkv->wtscale, M, qkv->K, qkv->N, qkv->precision, qkv->rank};
  ga.q_norm = q_norm;
  ga.k_norm = k_norm;
  ga.rope_cos = rope_cos;
  ga.rope_sin = rope_sin;
  ga.eps = eps;
  ga.heads = heads;
  ga.head_dim = head_dim;
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

size_t svdq_w4a4_prepare_workspace_bytes(int64_t N, int64_t K, int rank, int oversample) {
  if (N < 1 || N > kMaxPrepN || K < 128 || K > kMaxK || K % 128) return 0;
  if (rank < 0 || rank > 128 || rank % 16 || rank > std::min(N, K)) return 0;
  if (oversample < 0 || oversample > kMaxOversample) return 0;
  return prep_carve(nullptr, N, K, rank, rank + oversample, nullptr);
}

int svdq_w4a4_prepare_weight(const float* w, const void* x_calib, int64_t Mc, int64_t N, int64_t K,
                             int precision, int group_size, int rank, int oversample, int power_iters,
                             uint64_t seed, void* smooth_out, void* lora_down_out, void* lora_up_out,
                             void* packed_w_out, void* wscales_out, float* wtscale_out, double* sigma_out,
                             void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_svdq_kind(precision, group_size, rank);
  if (rc) return rc;
  if (N < 1 || N > kMaxPrepN) return fail(SVDQ_EINVAL, "N must be in [1, 2^20]");
  if (Mc < 1 || Mc > kMaxPrepRows) return fail(SVDQ_EINVAL, "the calibration rows must be in [1, 2^22]");
  if (K < 128 || K > kMaxK || K % 128) return fail(SVDQ_EINVAL, "K must be a multiple of 128 in [128, 16384]");
  if (rank > std::min(N, K)) return fail(SVDQ_EINVAL, "rank exceeds min(N, K)");
  if (oversample < 0 || oversample > kMaxOversample) return fail(SVDQ_EINVAL, "oversample must be in [0, 32]");
  if (power_iters < 0 || power_iters > kMaxPowerIters) return fail(SVDQ_EINVAL, "power_iters must be in [0, 16]");
  if (!w || !x_calib || !smooth_out || !packed_w_out || !wscales_out || !wtscale_out || !workspace)
    return fail(SVDQ_EINVAL, "null pointer argument");
  if ((rank > 0) != (lora_down_out != nullptr) || (rank > 0) != (lora_up_out != nullptr))
    return fail(SVDQ_EINVAL, "lora_down_out / lora_up_out must be non-null exactly when rank > 0");
  const void* ptrs[] = {w, x_calib, smooth_out, lora_down_out, lora_up_out, packed_w_out, wscales_out, workspace};
  for (const void* p : ptrs)
    if (p && !aligned(p)) return fail(SVDQ_EINVAL, "pointer arguments must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(wtscale_out) % 4) return fail(SVDQ_EINVAL, "wtscale_out must be 4-byte aligned");
  const int l = rank + oversample;
  const size_t need = prep_carve(nullptr, N, K, rank, l, nullptr);
  const Range outs[] = {{smooth_out, size_t(K) * 2},
                        {lora_down_out, size_t(rank) * size_t(K) * 2},
                        {lora_up_out, size_t(N) * size_t(rank) * 2},
                        {packed_w_out, size_t(N) * size_t(K / 2)},
                        {wscales_out, w_scale_bytes(N, K, precision)},
                        {wtscale_out, 4}};
  const Range ins[] = {{w, size_t(N) * size_t(K) * 4}, {x_calib, size_t(Mc) * size_t(K) * 2}, {workspace, need}};
  for (size_t i = 0; i < 6; ++i) {
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return fail(SVDQ_EINVAL, "an output overlaps an input or the workspace");
    for (size_t j = i + 1; j < 6; ++j)
      if (overlaps(outs[i], outs[j])) return fail(SVDQ_EINVAL, "outputs overlap");
  }
  if (ws_bytes < need) return fail(SVDQ_EWORKSPACE, "workspace too small");
  rc = check_device_arch();
  if (rc) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  PrepCtx x{s, l, {}};
  prep_carve(workspace, N, K, rank, l, &x.c);
  // 1. smoothing factors from the calibration activations
  svdq::SmoothArgs sa{x_calib, w, smooth_out, x.c.amax, Mc, N, K};
  rc = launch_status(svdq::launch_smooth_factors(sa, s), "smooth factors launch");
  if (rc) return rc;
  if (rank > 0) {
    svdq::PrepSrc W;
    W.w = w;
    W.smooth = smooth_out;
    // 2. range finder: Y = W_hat Omega, Q = orth(Y); subspace iteration
    rc = launch_status(svdq::launch_prep_gauss(x.c.omega, K * l, seed, s), "test matrix launch");
    if (rc) return rc;
    rc = launch_status(svdq::launch_prep_ab(W, N, K, x.c.omega, l, x.c.y, s), "range product launch");
    if (rc) return rc;
    rc = prep_orth(x, x.c.y, N, x.c.q, nullptr);
    if (rc) return rc;
    for (int it = 0; it < power_iters; ++it) {
      rc = launch_status(svdq::launch_prep_atb(W, N, K, x.c.q, l, prep_slices(N, K), x.c.part, x.c.z, s),
                         "transposed product launch");
      if (rc) return rc;
      rc = prep_orth(x, x.c.z, K, x.c.zq, nullptr);
      if (rc) return rc;
      rc = launch_status(svdq::launch_prep_ab(W, N, K, x.c.zq, l, x.c.y, s), "range product launch");
      if (rc) return rc;
      rc = prep_orth(x, x.c.y, N, x.c.q, nullptr);
      if (rc) return rc;
    }
    // 3. Z = W_hat^T Q = Zq Rz, so W_hat ~ Q Rz^T Zq^T; SVD of the l x l Rz^T
    rc = launch_status(svdq::launch_prep_atb(W, N, K, x.c.q, l, prep_slices(N, K), x.c.part, x.c.z, s),
                       "transposed product launch");
    if (rc) return rc;
    std::vector<double> Rz;
    rc = prep_orth(x, x.c.z, K, x.c.zq, &Rz);
    if (rc) return rc;
    std::vector<double> At(size_t(l) * l), U, sig, V;
    for (int i = 0; i < l; ++i)
      for (int j = 0; j < l; ++j) At[size_t(i) * l + j] = Rz[size_t(j) * l + i];
    jacobi_svd(At, l, U, sig, V);
    if (sigma_out)
      for (int i = 0; i < rank; ++i) sigma_out[i] = sig[i];
    // 4. lora_up = (Q U)[:, :rank]; lora_down = ((Zq V)[:, :rank] diag(sig))^T, both rounded to bf16
    std::vector<double> B(size_t(l) * rank);
    for (int i = 0; i < l; ++i)
      for (int j = 0; j < rank; ++j) B[size_t(i) * rank + j] = U[size_t(i) * l + j];
    svdq::PrepSrc D;
    D.dense = x.c.q;
    rc = prep_status(hipMemcpyAsync(x.c.small, B.data(), B.size() * sizeof(double), hipMemcpyHostToDevice, s),
                     "factor copy");
    if (rc) return rc;
    rc = launch_status(svdq::launch_prep_ab(D, N, l, x.c.small, rank, x.c.up64, s), "factor product launch");
    if (rc) return rc;
    rc = prep_status(hipStreamSynchronize(s), "stream synchronize");
    if (rc) return rc;
    for (int i = 0; i < l; ++i)
      for (int j = 0; j < rank; ++j) B[size_t(i) * rank + j] = V[size_t(i) * l + j] * sig[j];
    D.dense = x.c.zq;
    rc = prep_status(hipMemcpyAsync(x.c.small, B.data(), B.size() * sizeof(double), hipMemcpyHostToDevice, s),
                     "factor copy");
    if (rc) return rc;
    rc = launch_status(svdq::launch_prep_ab(D, K, l, x.c.small, rank, x.c.dt64, s), "factor product launch");
    if (rc) return rc;
    rc = launch_status(svdq::launch_prep_to_bf16(x.c.up64, N, rank, rank, false, static_cast<uint16_t*>(lora_up_out),
                                                 s), "factor rounding launch");
    if (rc) return rc;
    rc = launch_status(svdq::launch_prep_to_bf16(x.c.dt64, K, rank, rank, true,
                                                 static_cast<uint16_t*>(lora_down_out), s), "factor rounding launch");
    if (rc) return rc;
  }
  // 5. residual from the bf16 factors, then quantization and packing
  rc = launch_status(svdq::launch_prep_residual(w, smooth_out, lora_up_out, lora_down_out, N, K, rank, x.c.resid, s),
                     "residual launch");
  if (rc) return rc;
  svdq::PackArgs pa{x.c.resid, packed_w_out, wscales_out, wtscale_out, x.c.amax, N, K, precision};
  rc = launch_status(svdq::launch_pack_weight(pa, s), "pack weight launch");
  if (rc) return rc;
  return prep_status(hipStreamSynchronize(s), "stream synchronize");
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
