// C ABI of the H-BitLinear forward: argument validation, workspace layout and
// kernel dispatch.  Every check runs before any HIP call, so invalid calls
// return without touching the device.
#include "../../include/hbl.h"
#include "../../include/hbl_attn.h"

#include <hip/hip_runtime.h>
#include <mutex>
#include <string.h>

#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];   // 1 = gfx950, 0 = not supported
int g_dev_cus[kMaxDevices];  // compute units

hbl_status check_device(int* cus = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HBL_ERR_DEVICE;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t p;
    g_dev_ok[dev] = hipGetDeviceProperties(&p, dev) == hipSuccess && strncmp(p.gcnArchName, "gfx950", 6) == 0;
    g_dev_cus[dev] = g_dev_ok[dev] ? p.multiProcessorCount : 0;
  });
  if (cus) *cus = g_dev_cus[dev];
  return g_dev_ok[dev] ? HBL_OK : HBL_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int log2_exact(int64_t k) {
  if (k <= 0 || (k & (k - 1)) != 0) return -1;
  int l = 0;
  while ((int64_t(1) << l) < k) ++l;
  return l;
}

constexpr int64_t kMinK = 64, kMaxK = 32768;

hbl_status check_shape(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || M >= (int64_t(1) << 31)) return HBL_ERR_SHAPE;
  if (log2_exact(K) < 0 || K < kMinK || K > kMaxK) return HBL_ERR_SHAPE;
  if (N <= 0 || N % 16 != 0 || N >= (int64_t(1) << 31)) return HBL_ERR_SHAPE;
  if (M * (K > N ? K : N) >= (int64_t(1) << 40)) return HBL_ERR_SHAPE;
  return HBL_OK;
}

bool valid_dtype(hbl_dtype d) { return d == HBL_F32 || d == HBL_BF16; }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Forward workspace: [codes][scales][matmul scratch].  The INT4 prefill
// (M > kFp6MinM) keeps its codes in the six-bit operand layout of the fp6 x
// fp4 matrix instruction.
bool fp6_path(int bits, int64_t M, int64_t K) { return bits == 4 && M > hbl::kFp6MinM && K >= hbl::kFp6MinK; }
// 5..64 tokens (not the few-token and short-row kernels): the decode matmul
// reads the codes in the decode-blocked layout, 16-token groups
bool blocked_path(int bits, int64_t M, int64_t K) { return !fp6_path(bits, M, K) && M >= 5 && M <= 64 && K >= 512; }
size_t codes_bytes(int bits, int64_t M, int64_t K) {
  const int64_t rows = blocked_path(bits, M, K) ? (M + 15) / 16 * 16 : M;
  return align256((size_t)rows * K * (fp6_path(bits, M, K) ? 6 : bits) / 8);
}
size_t scales_bytes(int64_t M) { return align256((size_t)M * 4); }

hbl_status launched(hipError_t e) { return e == hipSuccess ? HBL_OK : HBL_ERR_LAUNCH; }

// Backward workspace: [dxh fp32 M*K][dy^T bf16 N*Mp][xh^T bf16 K*Mp][gain partials fp32 rows*K],
// Mp = M rounded up to 64 (zero columns).  The transform kernel runs on a
// fixed grid of up to 512 workgroups (two per CU of a 256-CU part).
struct BwdLayout {
  int64_t Mp;
  int grid, rows;
  size_t dxh, dyt, xht, dgp, total;
};
BwdLayout bwd_layout(int64_t M, int64_t K, int64_t N) {
  BwdLayout L{};
  L.Mp = (M + 63) / 64 * 64;
  const int tpb = hbl::bwd_prep_tpb(log2_exact(K));
  const int64_t need = tpb > 0 ? (M + tpb - 1) / tpb : 0;
  L.grid = (int)(need < 512 ? need : 512);
  L.rows = L.grid * tpb;
  L.dxh = align256((size_t)M * K * 4);
  L.dyt = align256((size_t)N * L.Mp * 2);
  L.xht = align256((size_t)K * L.Mp * 2);
  L.dgp = align256((size_t)L.rows * K * 4);
  L.total = L.dxh + L.dyt + L.xht + L.dgp;
  return L;
}

}  // namespace

// Every check of the forward's arguments except the workspace's (host only).
hbl_status hbl::forward_check(int bits, const void* x, hbl_dtype x_dtype, const float* gain,
                              const uint8_t* w_packed, const float* w_alpha, int64_t M, int64_t K, int64_t N,
                              const void* y, hbl_dtype y_dtype) {
  if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype) || (bits != 8 && bits != 4)) return HBL_ERR_DTYPE;
  if (hbl_status s = check_shape(M, K, N)) return s;
  if (M == 0) return HBL_OK;
  if (!x || !w_packed || !w_alpha || !y) return HBL_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_packed) || !aligned16(w_alpha) || !aligned16(y) || (gain && !aligned16(gain)))
    return HBL_ERR_ALIGN;
  return HBL_OK;
}

namespace {

// H-BitLinear forward (rotate) or BitLinear without the transform.
hbl_status forward(int bits, bool rotate, const void* x, hbl_dtype x_dtype, const float* gain,
                   const uint8_t* w_packed, const float* w_alpha, int64_t M, int64_t K, int64_t N, void* y,
                   hbl_dtype y_dtype, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (hbl_status s = hbl::forward_check(bits, x, x_dtype, gain, w_packed, w_alpha, M, K, N, y, y_dtype)) return s;
  if (M == 0) return HBL_OK;
  if (!workspace) return HBL_ERR_NULL;
  if (!aligned16(workspace)) return HBL_ERR_ALIGN;
  if (ws_bytes < hbl_workspace_bytes(bits == 8 ? HBL_OP_FORWARD_INT8 : HBL_OP_FORWARD_INT4, M, K, N))
    return HBL_ERR_WORKSPACE;
  int cus = 0;
  if (hbl_status s = check_device(&cus)) return s;

  if (hbl::decode_fused_supported((int)M, log2_exact(K), rotate)) {
    hbl::FusedDecodeArgs f{};
    f.x = x; f.x_bf16 = x_dtype == HBL_BF16; f.gain = gain; f.wpack = w_packed; f.walpha = w_alpha; f.out = y;
    f.out_kind = y_dtype == HBL_BF16 ? hbl::OUT_BF16 : hbl::OUT_F32;
    f.M = (int)M; f.N = (int)N; f.logk = log2_exact(K); f.bits = bits; f.rotate = rotate; f.stream = stream;
    return launched(hbl::launch_decode_fused(f));
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* codes = ws;
  float* dscale = reinterpret_cast<float*>(ws + codes_bytes(bits, M, K));
  void* gws = ws + codes_bytes(bits, M, K) + scales_bytes(M);
  const bool blocked = blocked_path(bits, M, K);
  const size_t gws_bytes = hbl::gemm_workspace_bytes(M, K, N, blocked);

  // split-K decode shapes: prep clears the matmul's arrival counters, so the
  // matmul's last workgroup per tile reduces (no separate reduction launch)
  const bool fp6 = fp6_path(bits, M, K);
  uint32_t* counts = hbl::gemm_tile_counter_ptr(gws, M, K, N, blocked);

  hbl::PrepArgs p{};
  p.x = x; p.x_bf16 = x_dtype == HBL_BF16; p.gain = gain; p.M = (int)M; p.cus = cus; p.logk = log2_exact(K);
  p.bits = bits; p.mode = fp6 ? 2 : 0; p.rotate = rotate; p.codes = codes; p.dscale = dscale; p.blocked = blocked;
  p.xt = nullptr; p.zero = counts; p.nzero = counts ? hbl::gemm_tile_counters(M, K, N, blocked) : 0; p.stream = stream;
  if (hipError_t e = hbl::launch_prep(p)) return launched(e);

  hbl::GemmArgs g{};
  g.codes = codes; g.bits = bits; g.wpack = w_packed; g.dscale = dscale; g.walpha = w_alpha; g.out = y;
  g.out_kind = y_dtype == HBL_BF16 ? hbl::OUT_BF16 : hbl::OUT_F32;
  g.M = (int)M; g.N = (int)N; g.K = (int)K; g.ws = gws; g.ws_bytes = gws_bytes; g.tile_count = counts;
  g.codes_blocked = blocked; g.stream = stream;
  return launched(fp6 ? hbl::launch_gemm_fp6(g) : hbl::launch_gemm(g));
}

}  // namespace

extern "C" {

const char* hbl_status_string(hbl_status s) {
  switch (s) {
    case HBL_OK: return "ok";
    case HBL_ERR_NULL: return "null pointer";
    case HBL_ERR_SHAPE: return "unsupported shape";
    case HBL_ERR_DTYPE: return "unsupported dtype or bit width";
    case HBL_ERR_ALIGN: return "pointer not 16-byte aligned";
    case HBL_ERR_WORKSPACE: return "workspace too small";
    case HBL_ERR_LAUNCH: return "kernel launch failed";
    case HBL_ERR_DEVICE: return "no gfx950 device";
    case HBL_ERR_SCRATCH: return "problem needs more scratch than the no-alloc forward's static array";
    default: break;
  }
  return "unknown status";
}

size_t hbl_workspace_bytes(int op, int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K <= 0 || N <= 0) return 0;
  switch (op) {
    case HBL_OP_QUANTIZE_WEIGHTS: return align256((size_t)N * 8);
    case HBL_OP_QUANTIZE_WEIGHTS_ROTATED: return align256((size_t)N * 8) + align256((size_t)N * K * 4);
    case HBL_OP_MATMUL: return align256(hbl::gemm_workspace_bytes(M, K, N, false));
    case HBL_OP_BACKWARD: return M > 0 && log2_exact(K) > 0 ? bwd_layout(M, K, N).total : 0;
    case HBL_OP_FORWARD_INT8:
    case HBL_OP_FORWARD_INT4: {
      const int bits = op == HBL_OP_FORWARD_INT8 ? 8 : 4;
      return codes_bytes(bits, M, K) + scales_bytes(M) +
             align256(hbl::gemm_workspace_bytes(M, K, N, blocked_path(bits, M, K)));
    }
    default: return 0;
  }
}

hbl_status hbl_quantize_weights(const float* w, int64_t N, int64_t K, uint8_t* w_packed, float* w_alpha,
                                void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!w || !w_packed || !w_alpha || !workspace) return HBL_ERR_NULL;
  if (hbl_status s = check_shape(0, K, N)) return s;
  if (!aligned16(w) || !aligned16(w_packed) || !aligned16(w_alpha) || !aligned16(workspace)) return HBL_ERR_ALIGN;
  if (ws_bytes < hbl_workspace_bytes(HBL_OP_QUANTIZE_WEIGHTS, 0, K, N)) return HBL_ERR_WORKSPACE;
  if (hbl_status s = check_device()) return s;
  hbl::WquantArgs a{w, (int)N, (int)K, w_packed, w_alpha, static_cast<double*>(workspace), stream};
  return launched(hbl::launch_wquant(a));
}

hbl_status hbl_quantize_weights_rotated(const float* w, int64_t N, int64_t K, uint8_t* w_packed, float* w_alpha,
                                        void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!w || !w_packed || !w_alpha || !workspace) return HBL_ERR_NULL;
  if (hbl_status s = check_shape(0, K, N)) return s;
  if (!aligned16(w) || !aligned16(w_packed) || !aligned16(w_alpha) || !aligned16(workspace)) return HBL_ERR_ALIGN;
  if (ws_bytes < hbl_workspace_bytes(HBL_OP_QUANTIZE_WEIGHTS_ROTATED, 0, K, N)) return HBL_ERR_WORKSPACE;
  int cus = 0;
  if (hbl_status s = check_device(&cus)) return s;
  // workspace: [row sums, fp64][rotated rows, fp32 [N][K]]
  float* wr = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + align256((size_t)N * 8));
  hbl::PrepArgs p{};
  p.x = w; p.x_bf16 = false; p.gain = nullptr; p.M = (int)N; p.cus = cus; p.logk = log2_exact(K);
  p.bits = 8; p.mode = 3; p.rotate = true; p.xt = wr; p.stream = stream;
  if (hipError_t e = hbl::launch_prep(p)) return launched(e);
  hbl::WquantArgs a{wr, (int)N, (int)K, w_packed, w_alpha, static_cast<double*>(workspace), stream};
  return launched(hbl::launch_wquant(a));
}

hbl_status hbl_forward_int8(const void* x, hbl_dtype x_dtype, const float* gain, const uint8_t* w_packed,
                            const float* w_alpha, int64_t M, int64_t K, int64_t N, void* y, hbl_dtype y_dtype,
                            void* workspace, size_t ws_bytes, hipStream_t stream) {
  return forward(8, true, x, x_dtype, gain, w_packed, w_alpha, M, K, N, y, y_dtype, workspace, ws_bytes, stream);
}

hbl_status hbl_forward_int4(const void* x, hbl_dtype x_dtype, const float* gain, const uint8_t* w_packed,
                            const float* w_alpha, int64_t M, int64_t K, int64_t N, void* y, hbl_dtype y_dtype,
                            void* workspace, size_t ws_bytes, hipStream_t stream) {
  return forward(4, true, x, x_dtype, gain, w_packed, w_alpha, M, K, N, y, y_dtype, workspace, ws_bytes, stream);
}

static hbl_status quantize_act(bool rotate, const void* x, hbl_dtype x_dtype, const float* gain, int64_t M,
                               int64_t K, int bits, void* codes, float* dscale, hipStream_t stream) {
  if (!valid_dtype(x_dtype) || (bits != 8 && bits != 4 && bits != HBL_BITS_INT4_FP6)) return HBL_ERR_DTYPE;
  if (hbl_status s = check_shape(M, K, 16)) return s;
  if (bits == HBL_BITS_INT4_FP6 && K < hbl::kFp6MinK) return HBL_ERR_SHAPE;
  if (M == 0) return HBL_OK;
  if (!x || !codes || !dscale) return HBL_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(dscale) || (gain && !aligned16(gain))) return HBL_ERR_ALIGN;
  int cus = 0;
  if (hbl_status s = check_device(&cus)) return s;
  hbl::PrepArgs p{};
  p.x = x; p.x_bf16 = x_dtype == HBL_BF16; p.gain = gain; p.M = (int)M; p.cus = cus; p.logk = log2_exact(K);
  p.bits = bits == 8 ? 8 : 4; p.mode = bits == HBL_BITS_INT4_FP6 ? 2 : 0; p.rotate = rotate;
  p.codes = static_cast<uint8_t*>(codes); p.dscale = dscale; p.stream = stream;
  return launched(hbl::launch_prep(p));
}

hbl_status hbl_quantize_act(const void* x, hbl_dtype x_dtype, const float* gain, int64_t M, int64_t K, int bits,
                            void* codes, float* dscale, hipStream_t stream) {
  return quantize_act(true, x, x_dtype, gain, M, K, bits, codes, dscale, stream);
}

hbl_status hbl_quantize_act_unrotated(const void* x, hbl_dtype x_dtype, const float* gain, int64_t M, int64_t K,
                                      int bits, void* codes, float* dscale, hipStream_t stream) {
  return quantize_act(false, x, x_dtype, gain, M, K, bits, codes, dscale, stream);
}

hbl_status hbl_quantize_rotated(const float* xt, int64_t M, int64_t K, int bits, void* codes, float* dscale,
                                hipStream_t stream) {
  if (bits != 8 && bits != 4 && bits != HBL_BITS_INT4_FP6) return HBL_ERR_DTYPE;
  if (hbl_status s = check_shape(M, K, 16)) return s;
  if (bits == HBL_BITS_INT4_FP6 && K < hbl::kFp6MinK) return HBL_ERR_SHAPE;
  if (M == 0) return HBL_OK;
  if (!xt || !codes || !dscale) return HBL_ERR_NULL;
  if (!aligned16(xt) || !aligned16(codes) || !aligned16(dscale)) return HBL_ERR_ALIGN;
  int cus = 0;
  if (hbl_status s = check_device(&cus)) return s;
  hbl::PrepArgs p{};
  p.x = xt; p.x_bf16 = false; p.gain = nullptr; p.M = (int)M; p.cus = cus; p.logk = log2_exact(K);
  p.bits = bits == 8 ? 8 : 4; p.mode = bits == HBL_BITS_INT4_FP6 ? 2 : 0; p.rotate = false; p.as_given = true;
  p.codes = static_cast<uint8_t*>(codes); p.dscale = dscale; p.stream = stream;
  return launched(hbl::launch_prep(p));
}

hbl_status hbl_bitlinear_forward(const void* x, hbl_dtype x_dtype, const float* gain, const uint8_t* w_packed,
                                 const float* w_alpha, int64_t M, int64_t K, int64_t N, int bits, void* y,
                                 hbl_dtype y_dtype, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return forward(bits, false, x, x_dtype, gain, w_packed, w_alpha, M, K, N, y, y_dtype, workspace, ws_bytes, stream);
}

hbl_status hbl_rmsnorm_fwht(const void* x, hbl_dtype x_dtype, const float* gain, int64_t M, int64_t K, float* xt,
                            hipStream_t stream) {
  if (!valid_dtype(x_dtype)) return HBL_ERR_DTYPE;
  if (hbl_status s = check_shape(M, K, 16)) return s;
  if (M == 0) return HBL_OK;
  if (!x || !xt) return HBL_ERR_NULL;
  if (!aligned16(x) || !aligned16(xt) || (gain && !aligned16(gain))) return HBL_ERR_ALIGN;
  int cus = 0;
  if (hbl_status s = check_device(&cus)) return s;
  hbl::PrepArgs p{};
  p.x = x; p.x_bf16 = x_dtype == HBL_BF16; p.gain = gain; p.M = (int)M; p.cus = cus; p.logk = log2_exact(K);
  p.bits = 8; p.mode = 1; p.rotate = true; p.xt = xt; p.stream = stream;
  return launched(hbl::launch_prep(p));
}

static hbl_status matmul(const void* codes, int bits, const float* dscale, const uint8_t* w_packed,
                         const float* w_alpha, int64_t M, int64_t K, int64_t N, void* out, int out_kind,
                         void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (bits != 8 && bits != 4 && bits != HBL_BITS_INT4_FP6) return HBL_ERR_DTYPE;
  if (hbl_status s = check_shape(M, K, N)) return s;
  if (bits == HBL_BITS_INT4_FP6 && K < hbl::kFp6MinK) return HBL_ERR_SHAPE;
  if (M == 0) return HBL_OK;
  if (!codes || !w_packed || !out) return HBL_ERR_NULL;
  if (out_kind != hbl::OUT_ACC_I32 && (!dscale || !w_alpha)) return HBL_ERR_NULL;
  const bool fp6 = bits == HBL_BITS_INT4_FP6;
  const size_t need = align256(hbl::gemm_workspace_bytes(M, K, N, false));
  if (need && !workspace) return HBL_ERR_NULL;
  if (!aligned16(codes) || !aligned16(w_packed) || !aligned16(out) || (dscale && !aligned16(dscale)) ||
      (w_alpha && !aligned16(w_alpha)) || (workspace && !aligned16(workspace)))
    return HBL_ERR_ALIGN;
  if (ws_bytes < need) return HBL_ERR_WORKSPACE;
  if (hbl_status s = check_device()) return s;
  hbl::GemmArgs g{};
  g.codes = static_cast<const uint8_t*>(codes); g.bits = bits; g.wpack = w_packed; g.dscale = dscale;
  g.walpha = w_alpha; g.out = out; g.out_kind = out_kind; g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.ws = workspace; g.ws_bytes = ws_bytes; g.stream = stream;
  return launched(fp6 ? hbl::launch_gemm_fp6(g) : hbl::launch_gemm(g));
}

hbl_status hbl_matmul_dequant(const void* codes, int bits, const float* dscale, const uint8_t* w_packed,
                              const float* w_alpha, int64_t M, int64_t K, int64_t N, void* y, hbl_dtype y_dtype,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(y_dtype)) return HBL_ERR_DTYPE;
  return matmul(codes, bits, dscale, w_packed, w_alpha, M, K, N, y,
                y_dtype == HBL_BF16 ? hbl::OUT_BF16 : hbl::OUT_F32, workspace, ws_bytes, stream);
}

hbl_status hbl_gemm_ternary(const void* codes, int bits, const uint8_t* w_packed, int64_t M, int64_t K, int64_t N,
                            int32_t* acc, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return matmul(codes, bits, nullptr, w_packed, nullptr, M, K, N, acc, hbl::OUT_ACC_I32, workspace, ws_bytes,
                stream);
}

hbl_status hbl_unpack_weights(const uint8_t* w_packed, int64_t N, int64_t K, int8_t* w_t, hipStream_t stream) {
  if (!w_packed || !w_t) return HBL_ERR_NULL;
  if (hbl_status s = check_shape(0, K, N)) return s;
  if (!aligned16(w_packed) || !aligned16(w_t)) return HBL_ERR_ALIGN;
  if (hbl_status s = check_device()) return s;
  return launched(hbl::launch_unpack(w_packed, (int)N, (int)K, w_t, stream));
}


// ---------------------------------------------------------------------------
// Low-bit attention states.

static bool heads_d_ok(int64_t d) { return d == 64 || d == 128 || d == 256; }
static constexpr int64_t kCount = int64_t(1) << 31;

static size_t attn_part_bytes(int64_t B, int64_t Hq, int64_t d, int64_t Tmax) {
  int ct = 0, nchunk = 0;
  hbl::attn_plan(B, Hq, (int)d, Tmax, &ct, &nchunk);
  if (nchunk == 1) return 0;                 // one workgroup per head writes the output itself
  return align256((size_t)B * Hq * nchunk * hbl::attn_part_stride((int)d) * sizeof(float));
}

hbl_status hbl_quantize_heads(const void* x, int64_t R, int64_t d, int bits, uint8_t* codes, float* scale,
                              hipStream_t stream) {
  if (!hbl::heads_bits_supported(bits)) return HBL_ERR_DTYPE;
  if (!heads_d_ok(d) || R < 0 || R >= kCount || R * d >= (int64_t(1) << 40)) return HBL_ERR_SHAPE;
  if (R == 0) return HBL_OK;
  if (!x || !codes || !scale) return HBL_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scale)) return HBL_ERR_ALIGN;
  if (hbl_status s = check_device()) return s;
  hbl::QuantHeadsArgs a{};
  a.x0 = x; a.codes0 = codes; a.scale0 = scale; a.B = 1; a.H = 1; a.Tn = R; a.Tmax = R; a.pos = nullptr;
  a.d = (int)d; a.bits = bits; a.stream = stream;
  return launched(hbl::launch_quant_heads(a));
}

hbl_status hbl_dequantize_heads(const uint8_t* codes, const float* scale, int64_t R, int64_t d, int bits, void* y,
                                hbl_dtype y_dtype, hipStream_t stream) {
  if (!hbl::heads_bits_supported(bits) || !valid_dtype(y_dtype)) return HBL_ERR_DTYPE;
  if (!heads_d_ok(d) || R < 0 || R >= kCount || R * d >= (int64_t(1) << 40)) return HBL_ERR_SHAPE;
  if (R == 0) return HBL_OK;
  if (!codes || !scale || !y) return HBL_ERR_NULL;
  if (!aligned16(codes) || !aligned16(scale) || !aligned16(y)) return HBL_ERR_ALIGN;
  if (hbl_status s = check_device()) return s;
  return launched(hbl::launch_dequant_heads(codes, scale, R, (int)d, bits, y, y_dtype == HBL_BF16, stream));
}

hbl_status hbl_kv_cache_append(const void* k, const void* v, int64_t B, int64_t Tn, int64_t Hkv, int64_t d,
                               int bits, const int32_t* pos, int64_t Tmax, uint8_t* k_codes, float* k_scale,
                               uint8_t* v_codes, float* v_scale, hipStream_t stream) {
  if (!hbl::heads_bits_supported(bits)) return HBL_ERR_DTYPE;
  if (!heads_d_ok(d) || B < 0 || B >= kCount || Tn < 0 || Tn >= kCount || Hkv <= 0 || Hkv >= kCount ||
      Tmax <= 0 || Tmax >= kCount || B * Hkv * Tn >= kCount || B * Hkv * Tmax > (int64_t(1) << 34))
    return HBL_ERR_SHAPE;
  if (B == 0 || Tn == 0) return HBL_OK;
  if (!k || !v || !k_codes || !k_scale || !v_codes || !v_scale) return HBL_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_codes) || !aligned16(k_scale) || !aligned16(v_codes) ||
      !aligned16(v_scale) || (pos && !aligned16(pos)))
    return HBL_ERR_ALIGN;
  if (hbl_status s = check_device()) return s;
  hbl::QuantHeadsArgs a{};
  a.x0 = k; a.x1 = v; a.codes0 = k_codes; a.codes1 = v_codes; a.scale0 = k_scale; a.scale1 = v_scale;
  a.B = B; a.H = Hkv; a.Tn = Tn; a.Tmax = Tmax; a.pos = pos; a.d = (int)d; a.bits = bits; a.stream = stream;
  return launched(hbl::launch_quant_heads(a));
}

size_t hbl_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t d, int64_t Tmax) {
  if (!heads_d_ok(d) || B <= 0 || Hq <= 0 || Tmax <= 0) return 0;
  return attn_part_bytes(B, Hq, d, Tmax);
}

hbl_status hbl_attention_prefill(const void* q, int q_bits, const uint8_t* k_codes, const float* k_scale,
                                 const uint8_t* v_codes, const float* v_scale, int kv_bits, const int32_t* start,
                                 int64_t B, int64_t Tn, int64_t Hq, int64_t Hkv, int64_t d, int64_t Tmax, void* out,
                                 hbl_dtype out_dtype, hipStream_t stream) {
  if (!hbl::heads_bits_supported(kv_bits) || q_bits < 2 || q_bits > 8 || !valid_dtype(out_dtype))
    return HBL_ERR_DTYPE;
  if (!heads_d_ok(d) || B < 0 || B >= kCount || Tn < 0 || Tn >= kCount || Hkv <= 0 || Hq <= 0 || Hq >= kCount ||
      Hq % Hkv != 0 || Tmax <= 0 || Tmax >= kCount || B * Hkv * Tmax > (int64_t(1) << 34) ||
      B * Hq * ((Tn + 63) / 64) >= kCount || Tmax * (d * kv_bits / 8) >= kCount || Tmax + Tn >= kCount - 512)
    return HBL_ERR_SHAPE;
  if (B == 0 || Tn == 0) return HBL_OK;
  if (!q || !k_codes || !k_scale || !v_codes || !v_scale || !start || !out) return HBL_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(k_scale) || !aligned16(v_codes) || !aligned16(v_scale) ||
      !aligned16(start) || !aligned16(out))
    return HBL_ERR_ALIGN;
  if (hbl_status st = check_device()) return st;
  hbl::PrefillArgs a{};
  a.q = q; a.qbits = q_bits; a.kc = k_codes; a.ks = k_scale; a.vc = v_codes; a.vs = v_scale; a.kvbits = kv_bits;
  a.start = start; a.B = (int)B; a.Tn = (int)Tn; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.d = (int)d; a.Tmax = Tmax;
  a.out = out; a.out_bf16 = out_dtype == HBL_BF16; a.stream = stream;
  return launched(hbl::launch_attention_prefill(a));
}

hbl_status hbl_attention_decode(const void* q, int q_bits, const uint8_t* k_codes, const float* k_scale,
                                const uint8_t* v_codes, const float* v_scale, int kv_bits, const int32_t* lens,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t Tmax, void* out,
                                hbl_dtype out_dtype, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!hbl::heads_bits_supported(kv_bits) || q_bits < 2 || q_bits > 8 || !valid_dtype(out_dtype))
    return HBL_ERR_DTYPE;
  if (!heads_d_ok(d) || B < 0 || B >= kCount || Hkv <= 0 || Hq <= 0 || Hq >= kCount || Hq % Hkv != 0 ||
      Tmax <= 0 || Tmax >= kCount || B * Hkv * Tmax > (int64_t(1) << 34))
    return HBL_ERR_SHAPE;
  if (B == 0) return HBL_OK;
  int ct = 0, nchunk = 0;
  hbl::attn_plan(B, Hq, (int)d, Tmax, &ct, &nchunk);
  if (B * Hq * nchunk >= kCount - 8 * Hq) return HBL_ERR_SHAPE;
  if (Tmax * (d * kv_bits / 8) >= kCount) return HBL_ERR_SHAPE;   // one head's codes addressed in 32 bits
  const size_t need = attn_part_bytes(B, Hq, d, Tmax);
  if (!q || !k_codes || !k_scale || !v_codes || !v_scale || !lens || !out || (need && !workspace))
    return HBL_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(k_scale) || !aligned16(v_codes) || !aligned16(v_scale) ||
      !aligned16(lens) || !aligned16(out) || (workspace && !aligned16(workspace)))
    return HBL_ERR_ALIGN;
  if (ws_bytes < need) return HBL_ERR_WORKSPACE;
  if (hbl_status s = check_device()) return s;
  hbl::AttnArgs a{};
  a.q = q; a.qbits = q_bits; a.kc = k_codes; a.ks = k_scale; a.vc = v_codes; a.vs = v_scale; a.kvbits = kv_bits;
  a.lens = lens; a.B = (int)B; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.d = (int)d; a.Tmax = Tmax;
  a.ct = ct; a.nchunk = nchunk; a.part = static_cast<float*>(workspace); a.out = out;
  a.out_bf16 = out_dtype == HBL_BF16; a.stream = stream;
  return launched(hbl::launch_attention_decode(a));
}


// ---------------------------------------------------------------------------
// Backward pass.

hbl_status hbl_backward_weights(const uint8_t* w_packed, int64_t N, int64_t K, void* w_bf16_t, hipStream_t stream) {
  if (hbl_status st = check_shape(0, K, N)) return st;
  if (N % 32 != 0) return HBL_ERR_SHAPE;
  if (!w_packed || !w_bf16_t) return HBL_ERR_NULL;
  if (!aligned16(w_packed) || !aligned16(w_bf16_t)) return HBL_ERR_ALIGN;
  if (hbl_status st = check_device()) return st;
  return launched(hbl::launch_wbt(w_packed, (int)N, (int)K, static_cast<uint16_t*>(w_bf16_t), stream));
}

hbl_status hbl_backward(const void* x, hbl_dtype x_dtype, const float* gain, const void* codes, int bits,
                        const float* d, const void* w_bf16_t, const float* w_alpha, const void* dy, int64_t M,
                        int64_t K, int64_t N, int rotate, void* dx, hbl_dtype dx_dtype, float* dw, float* dgain,
                        void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(x_dtype) || !valid_dtype(dx_dtype) || (bits != 8 && bits != 4)) return HBL_ERR_DTYPE;
  if (hbl_status st = check_shape(M, K, N)) return st;
  if (M < 1 || N % 32 != 0) return HBL_ERR_SHAPE;
  if (!x || !codes || !d || !w_bf16_t || !w_alpha || !dy || !dx || !dw || !workspace || (dgain && !gain))
    return HBL_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(d) || !aligned16(w_bf16_t) || !aligned16(w_alpha) ||
      !aligned16(dy) || !aligned16(dx) || !aligned16(dw) || !aligned16(workspace) || (gain && !aligned16(gain)) ||
      (dgain && !aligned16(dgain)))
    return HBL_ERR_ALIGN;
  const BwdLayout L = bwd_layout(M, K, N);
  if (ws_bytes < L.total) return HBL_ERR_WORKSPACE;
  if (hbl_status st = check_device()) return st;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* dxh = reinterpret_cast<float*>(ws);
  uint16_t* dyt = reinterpret_cast<uint16_t*>(ws + L.dxh);
  uint16_t* xht = reinterpret_cast<uint16_t*>(ws + L.dxh + L.dyt);
  float* dgp = reinterpret_cast<float*>(ws + L.dxh + L.dyt + L.xht);
  // input gradient: dxh = dy . (W_t^T)^T * a, then transform + RMSNorm backward
  if (hipError_t e = hbl::launch_gemm_bf16_nt(static_cast<const uint16_t*>(dy),
                                              static_cast<const uint16_t*>(w_bf16_t), w_alpha, dxh, (int)M, (int)K,
                                              (int)N, stream))
    return launched(e);
  hbl::BwdArgs b{};
  b.dxh = dxh; b.x = x; b.x_bf16 = x_dtype == HBL_BF16; b.gain = gain; b.M = (int)M; b.logk = log2_exact(K);
  b.dx = dx; b.dx_bf16 = dx_dtype == HBL_BF16; b.rotate = rotate != 0; b.stream = stream;
  if (hipError_t e = hbl::launch_bwd_prep(b, L.grid, dgain ? dgp : nullptr)) return launched(e);
  if (dgain)
    if (hipError_t e = hbl::launch_dg_reduce(dgp, L.rows, (int)K, dgain, stream)) return launched(e);
  // weight gradient: dw = dy^T . xh over the tokens (token-last copies)
  if (hipError_t e = hbl::launch_transpose_tokens(0, dy, nullptr, (int)M, (int)N, (int)L.Mp, dyt, stream))
    return launched(e);
  if (hipError_t e = hbl::launch_transpose_tokens(bits, codes, d, (int)M, (int)K, (int)L.Mp, xht, stream))
    return launched(e);
  return launched(hbl::launch_gemm_bf16_nt(dyt, xht, nullptr, dw, (int)N, (int)K, (int)L.Mp, stream));
}

}  // extern "C"
